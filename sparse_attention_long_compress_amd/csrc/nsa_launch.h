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
//   o_cmp [B][T][Hq][D] (nullable), lse_cmp [B][Hq][T] fp32 natural log, -inf
//   where no compressed block is visible (nullable), indices
//   [B][Hkv][T][topk] (written unless do_topk == false).
hipError_t launch_cmp_select(bool is_bf16, const Shape& s, const void* q, const void* kc,
                             const void* kc_lo, const void* vct, void* o_cmp, float* lse_cmp,
                             int32_t* indices, bool do_topk, hipStream_t st);

// K3: selection + window + gated combine.  knorm from K1 (required).
//   lse / o_sel: selection branch log-sum-exp [B][Hq][T] and output (nullable);
//   lse_win / o_win: the same for the window branch (nullable).
// arguments of the selection / window kernels (K3)
struct SelWinArgs {
  const void* q;
  const void* k;
  const void* kvimg;   // [B][Hkv][nc] staged K / V^T images of the blocks (KvImage)
  const void* gates;
  const void* o_cmp;
  const float* knorm;  // [B][Hkv][nc] largest key norm of each block
  const int32_t* indices;
  void* out;
  float* lse;
  void* o_sel;
  float* lse_win;
  void* o_win;
};
// K3 with packed selection items (sel_compact.hip): bf16, head_dim 64, four
// query heads per KV group, window range within 32 blocks, LDS within 160 KB
bool sel_compact_eligible(bool is_bf16, const Shape& s);
hipError_t launch_sel_compact(const Shape& s, const SelWinArgs& args, hipStream_t st);

// decode.hip: one new query per sequence over a KV cache
size_t decode_lds_bytes(bool is_bf16, const Shape& s);
hipError_t launch_decode(bool is_bf16, const Shape& s, const void* q, const void* kcache,
                         const void* vcache, const void* kcmp, const void* vcmp,
                         const int32_t* lens, const void* gates, void* out, int32_t* indices,
                         hipStream_t st);

// name of the kernel launch_sel_win runs for this shape
const char* sel_win_kernel_name(bool is_bf16, const Shape& s);
hipError_t launch_sel_win(bool is_bf16, const Shape& s, const void* q, const void* k,
                          const void* kvimg, const void* gates, const void* o_cmp,
                          const float* knorm, const int32_t* indices, void* out, float* lse,
                          void* o_sel, float* lse_win, void* o_win, hipStream_t st);

// Backward (selection branch).
//   prep: bimg [B][Hkv][T/64][BwdImage<T, D>::BYTES] (K, V, K^T fragments of
//   each key block), delta [B][Hq][T] fp32, dos [B][T][Hq][D].
// Extra outputs of the preparation kernel for the full backward (all
// [B][T][Hq][D] in the input dtype or [B][Hq][T] fp32; dgates [B][T][Hq][3]).
struct PrepFullArgs {
  const void* o_win;
  const void* o_cmp;
  void* dos_w;
  void* dos_c;
  float* delta_w;
  float* delta_c;
  void* dgates;
};
hipError_t launch_bwd_prep(bool is_bf16, const Shape& s, const void* k, const void* v,
                           const void* gates, const void* o_sel, const void* dout, void* bimg,
                           float* delta, void* dos, const PrepFullArgs* full, hipStream_t st);
// pooled-key images [B][Hkv][ceil(nc / 64)][BwdImage<T, D>::BYTES] from the
// pooled keys / values kc, vc [B][nc][Hkv][D]
hipError_t launch_bwd_pool_image(bool is_bf16, const Shape& s, const void* kc, const void* vc,
                                 void* pimg, hipStream_t st);
hipError_t launch_bwd_revmap(const Shape& s, const int32_t* indices, uint64_t* revmap,
                             hipStream_t st);
// dq pass of one branch (mode 0 selection, 1 window, 2 compression over the
// pooled-key images).  img: block images (modes 0, 1) or pooled-key images
// (mode 2); indices only for mode 0; lse / delta [B][Hq][T] and dos
// [B][T][Hq][D] of that branch.  The pass adds tau * its gradient to acc_in
// (fp32 [B][T][Hq][D], nullable) and writes the sum to acc_out (fp32,
// nullable) and / or dq (input dtype, nullable).
struct DqArgs {
  const void* q;
  const void* img;
  const int32_t* indices;
  const float* lse;
  const float* delta;
  const void* dos;
  const float* acc_in;
  float* acc_out;
  void* dq;
};
hipError_t launch_bwd_dq(bool is_bf16, const Shape& s, int mode, const DqArgs& args, hipStream_t st);

// Planning and partial-sum buffers of the dk/dv pass (all in the workspace):
//   lists [B][Hkv][nblk][T] u16 positions that selected each block, counts
//   [B][Hkv][nblk], items (bwd_items_bytes), slot_base / slot_cnt
//   [B][Hkv][nblk], slot_base_c / slot_cnt_c [B][Hkv][ceil(nc / 64)] (full
//   backward only), nitems (1 int), part (bwd_part_floats fp32).
struct BwdPlanWs {
  void* items;
  uint16_t* lists;
  int* counts;
  int* slot_base;
  int* slot_cnt;
  int* slot_base_c;
  int* slot_cnt_c;
  int* nitems;
  float* part;
};
// The branches a dk/dv pass covers: selection only (full == false; index 0 of
// lse / delta / dos) or selection, window and compression (indices 0, 1, 2).
// img: block images; pimg: pooled-key images (full only).
struct KvBranches {
  bool full;
  const void* q;
  const void* img;
  const void* pimg;
  const float* lse[3];
  const float* delta[3];
  const void* dos[3];
};
hipError_t launch_bwd_dkdv(bool is_bf16, const Shape& s, const KvBranches& br, const uint64_t* revmap,
                           void* dk, void* dv, const BwdPlanWs& ws, hipStream_t st);
size_t bwd_items_bytes(const Shape& s, bool full);
size_t bwd_part_floats(const Shape& s, bool full);

// Single-pass selection backward with atomics (bf16): dq written directly;
// dk, dv accumulated in fp32 (dk32, dv32 [B][T][Hkv][D], zeroed here) by
// atomic adds, then rounded into dk (x tau) and dv.
hipError_t launch_bwd_single(const Shape& s, const void* q, const void* bimg, const int32_t* indices,
                             const float* lse, const float* delta, const void* dos, void* dq, void* dk,
                             void* dv, float* dk32, float* dv32, hipStream_t st);

}  // namespace nsa
