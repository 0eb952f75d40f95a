// bwd.hip -- gradient of the selection branch, two passes, no atomics.
//
// [SIC] "Sparsity is Cool", Method (NSA implementation): every query attends a
// subset of keys of its own, so the key/value-stationary backward of dense
// attention does not apply directly; the two-pass scheme -- a query-stationary
// pass for dQ and a key/value-stationary pass for dK/dV over a reconstructed
// reverse key->query map -- avoids atomic contention.  The selection and the
// gates are held fixed; the branch receives g_sel * dO.  With P_s the
// selection softmax (recomputed from the saved log-sum-exp), dP_s = dOs . v_s,
// Delta = dOs . o_sel and dS_s = P_s (dP_s - Delta):
//   dq = tau sum_s dS_s k_s,   dk_s = tau sum dS_s q,   dv_s = sum P_s dOs.
//
// B0 prep    : dOs = g_sel dO (element type), Delta (fp32, from that dOs), block images
//              (K, V, K^T fragments) for B2 and B3.
// B1 revmap  : M[b][g][j][c] = 64-bit mask of the positions of tile c (64
//              positions) that selected block j -- one wave per (tile, group),
//              one lane per position, a bit-matrix transpose by lane
//              exchanges; no atomics.
// B2 dq      : query-stationary, the block walk of the forward's selection
//              kernel (bwd_dq.hip).
// B3 dk/dv   : key/value-stationary over the rows of M (bwd_dkdv.hip); blocks
//              read by many queries are split into items whose partial sums
//              B4 adds in a fixed order, so the result is bitwise reproducible.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

template <typename T> struct V16b;
template <> struct V16b<bf16> { typedef bf16x8 type; };
template <> struct V16b<float> { typedef f32x4 type; };

// ============================================================ B0: preparation
// Backward image of one 64-key block from its K and V rows staged in LDS
// (kt, vt: [64][D + 8]): K and V fragments in K3's A-operand order, then K^T.
template <typename T, int D>
__device__ void write_bwd_image(const T (*kt)[D + 8], const T (*vt)[D + 8], unsigned char* img) {
  typedef BwdImage<T, D> I;
  constexpr int EPV = 16 / sizeof(T);
  for (int w = threadIdx.x; w < I::PIECES * 64; w += 256) {
    const int pc = w / 64, l = w % 64;
    const int f = pc / I::NV, vv = pc % I::NV;
    const int a = l / 16, rho = l % 16;
    T piece[EPV];
    if (f < 2 * I::NFRAG) {  // K or V, key rows
      const int ff = f % I::NFRAG;
      const int u = I::K::k_u(ff), ks = I::K::k_ks(ff);
      const T* src = (f < I::NFRAG ? &kt[0][0] : &vt[0][0]) +
                     (size_t)I::K::krow(u, rho) * (D + 8) + ks * 32 + 8 * a + vv * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) piece[e] = src[e];
    } else {                 // K^T: channel rows, 8 consecutive keys per lane
      const int f2 = f - 2 * I::NFRAG, mt = I::K::v_mt(f2), hf = I::K::v_h(f2);
      const int ch = mt * 16 + rho, key0 = 32 * hf + 8 * a + vv * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) piece[e] = kt[key0 + e][ch];
    }
    *reinterpret_cast<f32x4*>(img + (size_t)pc * 1024 + 16 * l) = *reinterpret_cast<const f32x4*>(piece);
  }
}

// grid (nblk, Hkv, B), 256 threads: block j of positions / keys, KV group g.
// Writes the block's backward image and, for the G heads of the group at
// these positions, dOs = g_sel dO and Delta = dOs . o_sel.  With `full`
// (dgates != nullptr) also the window and compression branches' dOs and
// Delta and the gate gradients dgates = (dO . o_cmp, dO . o_sel, dO . o_win).
struct PrepFull {
  const void* o_win;
  const void* o_cmp;
  void* dos_w;
  void* dos_c;
  float* delta_w;
  float* delta_c;
  void* dgates;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Shape s, const T* __restrict__ k,
                                                       const T* __restrict__ v,
                                                       const T* __restrict__ gates,
                                                       const T* __restrict__ o_sel,
                                                       const T* __restrict__ dout,
                                                       unsigned char* __restrict__ bimg,
                                                       float* __restrict__ delta,
                                                       T* __restrict__ dos, PrepFull fx) {
  typedef BwdImage<T, D> I;
  constexpr int EPV = 16 / sizeof(T);
  typedef typename V16b<T>::type Vec;
  __shared__ __align__(16) T kt[kBlock][D + 8];
  __shared__ __align__(16) T vt[kBlock][D + 8];
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = s.G;
  const size_t k_row = (size_t)s.Hkv * D;
  for (int i = threadIdx.x; i < kBlock * (D / EPV); i += 256) {
    const int r = i / (D / EPV), c8 = i % (D / EPV);
    const size_t src = ((size_t)b * s.T + j * kBlock + r) * k_row + (size_t)g * D + c8 * EPV;
    *reinterpret_cast<Vec*>(&kt[r][c8 * EPV]) = *reinterpret_cast<const Vec*>(k + src);
    *reinterpret_cast<Vec*>(&vt[r][c8 * EPV]) = *reinterpret_cast<const Vec*>(v + src);
  }
  __syncthreads();
  write_bwd_image<T, D>(kt, vt, bimg + (((size_t)b * s.Hkv + g) * (s.T / kBlock) + j) * (size_t)I::BYTES);
  // dOs and Delta for the G heads of the group: D / EPV consecutive lanes per
  // (position, head) row, 16-byte accesses
  constexpr int TPR = D / EPV;
  static_assert((kBlock * TPR) % 256 == 0, "whole passes");
  const bool full = fx.dgates != nullptr;
  for (int i = threadIdx.x; i < kBlock * G * TPR; i += 256) {
    const int row = i / TPR, c = i % TPR;
    const int t = j * kBlock + row / G, h = g * G + row % G;
    const size_t base = (((size_t)b * s.T + t) * s.Hq + h) * D + c * EPV;
    const T* grow = gates + (((size_t)b * s.T + t) * s.Hq + h) * 3;
    const float gs = (float)grow[1];
    const Vec dv = *reinterpret_cast<const Vec*>(dout + base);
    const Vec ov = *reinterpret_cast<const Vec*>(o_sel + base);
    Vec outv;
    float acc = 0.f, dg[3] = {0.f, 0.f, 0.f};
    // Delta is taken from the dOs values the dP products use (rounded to the
    // element type), so that dP - Delta is exactly zero where one key holds a
    // row's whole probability and the rows of dS keep summing to ~0
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      outv[e] = (T)(gs * (float)dv[e]);
      acc += (float)outv[e] * (float)ov[e];
      dg[1] += (float)dv[e] * (float)ov[e];
    }
    *reinterpret_cast<Vec*>(dos + base) = outv;
    float accw = 0.f, accc = 0.f;
    if (full) {
      const float gc = (float)grow[0], gw = (float)grow[2];
      const Vec wv = *reinterpret_cast<const Vec*>((const T*)fx.o_win + base);
      const Vec cv = *reinterpret_cast<const Vec*>((const T*)fx.o_cmp + base);
      Vec ow_, oc_;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float d0 = (float)dv[e];
        ow_[e] = (T)(gw * d0);
        oc_[e] = (T)(gc * d0);
        accw += (float)ow_[e] * (float)wv[e];
        accc += (float)oc_[e] * (float)cv[e];
        dg[0] += d0 * (float)cv[e];
        dg[2] += d0 * (float)wv[e];
      }
      *reinterpret_cast<Vec*>((T*)fx.dos_w + base) = ow_;
      *reinterpret_cast<Vec*>((T*)fx.dos_c + base) = oc_;
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) {
      acc += __shfl_xor(acc, off);
      if (full) {
        accw += __shfl_xor(accw, off);
        accc += __shfl_xor(accc, off);
#pragma unroll
        for (int z = 0; z < 3; ++z) dg[z] += __shfl_xor(dg[z], off);
      }
    }
    if (c == 0) {
      const size_t r = ((size_t)b * s.Hq + h) * s.T + t;
      delta[r] = acc;
      if (full) {
        fx.delta_w[r] = accw;
        fx.delta_c[r] = accc;
        T* dgo = (T*)fx.dgates + (((size_t)b * s.T + t) * s.Hq + h) * 3;
#pragma unroll
        for (int z = 0; z < 3; ++z) dgo[z] = (T)dg[z];
      }
    }
  }
}

// Backward image of the pooled keys: grid (ceil(nc / 64), Hkv, B), 256
// threads; pooled "block" J holds the pooled keys / values 64 J .. 64 J + 63
// (kc, vc [B][nc][Hkv][D] from the pooling kernel; zero past the last
// complete block) in the BwdImage layout, so the backward kernels treat the
// compressed branch's keys like a key block.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pool_image_kernel(Shape s, const T* __restrict__ kc,
                                                             const T* __restrict__ vc,
                                                             unsigned char* __restrict__ pimg) {
  typedef BwdImage<T, D> I;
  constexpr int EPV = 16 / sizeof(T);
  typedef typename V16b<T>::type Vec;
  __shared__ __align__(16) T kt[kBlock][D + 8];
  __shared__ __align__(16) T vt[kBlock][D + 8];
  const int J = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const size_t k_row = (size_t)s.Hkv * D;
  for (int i = threadIdx.x; i < kBlock * (D / EPV); i += 256) {
    const int r = i / (D / EPV), c8 = i % (D / EPV);
    const int jj = J * kBlock + r;
    Vec kv_, vv_;
    if (jj < s.nc) {
      const size_t src = ((size_t)b * s.nc + jj) * k_row + (size_t)g * D + c8 * EPV;
      kv_ = *reinterpret_cast<const Vec*>(kc + src);
      vv_ = *reinterpret_cast<const Vec*>(vc + src);
    } else {
#pragma unroll
      for (int e = 0; e < EPV; ++e) { kv_[e] = (T)0.f; vv_[e] = (T)0.f; }
    }
    *reinterpret_cast<Vec*>(&kt[r][c8 * EPV]) = kv_;
    *reinterpret_cast<Vec*>(&vt[r][c8 * EPV]) = vv_;
  }
  __syncthreads();
  const int NJc = (s.nc + kBlock - 1) / kBlock;
  write_bwd_image<T, D>(kt, vt, pimg + (((size_t)b * s.Hkv + g) * NJc + J) * (size_t)I::BYTES);
}

// ============================================================ B1: reverse map
// grid (nblk tiles c, Hkv, B), 64 threads (lane = position of the tile).
// revmap[b][g][j][c] for j <= c, per 64-block chunk q: lane l builds its
// position's row of a 64 x 64 bit matrix (bit i: block 64 q + i chosen), and a
// transpose of that matrix by six butterfly stages of lane exchanges (shuffles,
// no LDS table, no atomics) leaves in lane l the positions that chose block
// 64 q + l.
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t x, int m) {
  const unsigned lo = (unsigned)__shfl_xor((int)(unsigned)x, m);
  const unsigned hi = (unsigned)__shfl_xor((int)(unsigned)(x >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}
__global__ __launch_bounds__(64) void bwd_revmap_kernel(Shape s, const int32_t* __restrict__ idx,
                                                        uint64_t* __restrict__ revmap) {
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nblk = s.T / kBlock;
  const int l = threadIdx.x;
  const int t = c * kBlock + l;
  const int32_t* row = idx + (((size_t)b * s.Hkv + g) * s.T + t) * s.topk;
  // (the row's loads all go out before the first is used: top-k <= 32)
  int jv[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) jv[e] = e < s.topk ? row[e] : -1;
  uint64_t* dst = revmap + (((size_t)b * s.Hkv + g) * nblk) * nblk + c;
  // two chunks at a time: their transposes are independent chains
  for (int q = 0; 64 * q <= c; q += 2) {
    uint64_t r[2] = {0ull, 0ull};  // indices outside 0 .. c are ignored
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int j = jv[e];
      const bool in = j >= 0 && j <= c;
#pragma unroll
      for (int x = 0; x < 2; ++x) r[x] |= (in && (j >> 6) == q + x) ? 1ull << (j & 63) : 0ull;
    }
    // transpose: at stage h, lanes l and l ^ h exchange the h-bit halves of
    // every 2h-bit group that the other one needs
#pragma unroll
    for (int h = 32; h >= 1; h >>= 1) {
      const uint64_t lo = h == 32 ? 0x00000000FFFFFFFFull : h == 16 ? 0x0000FFFF0000FFFFull
                        : h == 8 ? 0x00FF00FF00FF00FFull : h == 4 ? 0x0F0F0F0F0F0F0F0Full
                        : h == 2 ? 0x3333333333333333ull : 0x5555555555555555ull;
      uint64_t p[2];
#pragma unroll
      for (int x = 0; x < 2; ++x) p[x] = shfl_xor64(r[x], h);
#pragma unroll
      for (int x = 0; x < 2; ++x)
        r[x] = (l & h) ? ((r[x] & ~lo) | ((p[x] & ~lo) >> h)) : ((r[x] & lo) | ((p[x] & lo) << h));
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int j = 64 * (q + x) + l;
      if (j <= c) dst[(size_t)j * nblk] = r[x];
    }
  }
}

// ============================================================ launchers
hipError_t launch_bwd_prep(bool is_bf16, const Shape& s, const void* k, const void* v,
                           const void* gates, const void* o_sel, const void* dout, void* bimg,
                           float* delta, void* dos, const PrepFullArgs* full, hipStream_t st) {
  dim3 grid(s.T / kBlock, s.Hkv, s.B);
  unsigned char* im = (unsigned char*)bimg;
  PrepFull fx{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  if (full) fx = PrepFull{full->o_win, full->o_cmp, full->dos_w, full->dos_c, full->delta_w,
                          full->delta_c, full->dgates};
  if (is_bf16) {
    if (s.D == 64)
      hipLaunchKernelGGL((bwd_prep_kernel<bf16, 64>), grid, dim3(256), 0, st, s, (const bf16*)k,
                         (const bf16*)v, (const bf16*)gates, (const bf16*)o_sel, (const bf16*)dout,
                         im, delta, (bf16*)dos, fx);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<bf16, 128>), grid, dim3(256), 0, st, s, (const bf16*)k,
                         (const bf16*)v, (const bf16*)gates, (const bf16*)o_sel, (const bf16*)dout,
                         im, delta, (bf16*)dos, fx);
  } else {
    hipLaunchKernelGGL((bwd_prep_kernel<float, 64>), grid, dim3(256), 0, st, s, (const float*)k,
                       (const float*)v, (const float*)gates, (const float*)o_sel,
                       (const float*)dout, im, delta, (float*)dos, fx);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_pool_image(bool is_bf16, const Shape& s, const void* kc, const void* vc,
                                 void* pimg, hipStream_t st) {
  dim3 grid((s.nc + kBlock - 1) / kBlock, s.Hkv, s.B);
  unsigned char* im = (unsigned char*)pimg;
  if (is_bf16) {
    if (s.D == 64)
      hipLaunchKernelGGL((bwd_pool_image_kernel<bf16, 64>), grid, dim3(256), 0, st, s,
                         (const bf16*)kc, (const bf16*)vc, im);
    else
      hipLaunchKernelGGL((bwd_pool_image_kernel<bf16, 128>), grid, dim3(256), 0, st, s,
                         (const bf16*)kc, (const bf16*)vc, im);
  } else {
    hipLaunchKernelGGL((bwd_pool_image_kernel<float, 64>), grid, dim3(256), 0, st, s,
                       (const float*)kc, (const float*)vc, im);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_revmap(const Shape& s, const int32_t* indices, uint64_t* revmap,
                             hipStream_t st) {
  const int nblk = s.T / kBlock;
  dim3 grid(nblk, s.Hkv, s.B);
  hipLaunchKernelGGL(bwd_revmap_kernel, grid, dim3(64), 0, st, s, indices, revmap);
  return hipGetLastError();
}

}  // namespace nsa
