// nsa_launch.h -- host-side launch functions of the gfx950 kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

// Shape of one call, resolved on the host.
struct Shape {
  int B, T, Hq, Hkv, D, G, topk, W;
  int nc;      // complete compressed blocks = T / 64
  int ncp;     // nc rounded up to a multiple of 64 (padded transposed copies)
  float scale; // tau
  uint32_t flags;
};

// K1: mean-pool.  kc/vc [B][nc][Hkv][D] (nullable); vct [B][Hkv][D][ncp]
// (nullable); kvimg [B][Hkv][nc][KvImage<T, D>::BYTES] staged block images
// (nullable); knorm [B][Hkv][nc] fp32, largest
// key norm per block (nullable); kc_lo [B][nc][Hkv][D] residual of the
// rounded kc (bf16 only, nullable).
hipError_t launch_pool(bool is_bf16, const Shape& s, const void* k, const void* v, void* kc,
                       void* vc, void* vct, void* kvimg, float* knorm, void* kc_lo,
                       hipStream_t st);

// K2: compressed attention + importance + top-k.
//   o_cmp [B][T][Hq][D] (nullable), ubound [B][Hq][T] (nullable; log2 units),
//   indices [B][Hkv][T][topk] (written unless do_topk == false).
hipError_t launch_cmp_select(bool is_bf16, const Shape& s, const void* q, const void* kc,
                             const void* kc_lo, const void* vct, const float* radius,
                             void* o_cmp, float* ubound, int32_t* indices, bool do_topk,
                             hipStream_t st);

// K3: selection + window + gated combine.  knorm from K1 (required).
hipError_t launch_sel_win(bool is_bf16, const Shape& s, const void* q, const void* k,
                          const void* kvimg, const void* gates, const void* o_cmp,
                          const float* knorm, const int32_t* indices, void* out, float* lse,
                          void* o_sel, hipStream_t st);

// Backward (selection branch).
//   prep: bimg [B][Hkv][T/64][BwdImage<T, D>::BYTES] (K, V, K^T fragments of
//   each key block), delta [B][Hq][T] fp32, dos [B][T][Hq][D].
hipError_t launch_bwd_prep(bool is_bf16, const Shape& s, const void* k, const void* v,
                           const void* gates, const void* o_sel, const void* dout, void* bimg,
                           float* delta, void* dos, hipStream_t st);
hipError_t launch_bwd_revmap(const Shape& s, const int32_t* indices, uint64_t* revmap,
                             hipStream_t st);
hipError_t launch_bwd_dq(bool is_bf16, const Shape& s, const void* q, const void* bimg,
                         const int32_t* indices, const float* lse, const float* delta,
                         const void* dos, void* dq, hipStream_t st);
// Planning and partial-sum buffers of the dk/dv pass (all in the workspace):
//   lists [B][Hkv][nblk][T] u16 positions that selected each block, counts
//   [B][Hkv][nblk], items (bwd_items_bytes), slot_base / slot_cnt
//   [B][Hkv][nblk], nitems (1 int), part (bwd_part_floats fp32).
struct BwdPlanWs {
  void* items;
  uint16_t* lists;
  int* counts;
  int* slot_base;
  int* slot_cnt;
  int* nitems;
  float* part;
};
hipError_t launch_bwd_dkdv(bool is_bf16, const Shape& s, const void* q, const void* bimg,
                           const float* lse, const float* delta, const void* dos,
                           const uint64_t* revmap, void* dk, void* dv, const BwdPlanWs& ws,
                           hipStream_t st);
size_t bwd_items_bytes(const Shape& s);
size_t bwd_part_floats(const Shape& s);

}  // namespace nsa
