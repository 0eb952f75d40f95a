// pool.hip -- K1: mean-pool compression of K and V.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work? / COMPRESSION:
// the tokens of each block are summarised into one key and one value;
// [SIC] "Sparsity is Cool", Method: the summary is a mean-pool, block 64.
//
// One workgroup per (64-token block j, KV head g, batch b).  The block's K and
// V tiles (64 x D) are read once, coalesced (each thread owns 8 consecutive
// channels of a few rows), summed in fp32 and divided by 64; the mean is
// rounded once to the element type.  The same pass also emits what the
// attention kernels want to read as MFMA operands:
//   vt     [B][Hkv][D][T]   V transposed (rows of 64 keys are contiguous per
//                           channel, so a lane's 8 consecutive keys are one
//                           16-byte load);
//   vct    [B][Hkv][D][ncp] the pooled V transposed, zero-padded to ncp;
//   radius [B][Hkv][ncp]    max_i |k_i - Kc_j| over the block (fp32), the
//                           block's key radius around its mean, used to
//                           bound the block's largest logit;
//   kc_lo  [B][nc][Hkv][D]  (bf16 only) Kc - round(Kc), so that the block
//                           scores can use hi + lo (about 16 more bits) and
//                           the top-k decisions are not moved by the rounding
//                           of the pooled keys.
// HBM-bound: reads 2*64*D elements per (j, g, b), writes about the same once
// more (vt) plus 2*D pooled values.
#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(Shape s, const T* __restrict__ k,
                                                   const T* __restrict__ v, T* __restrict__ kc,
                                                   T* __restrict__ vc, T* __restrict__ vct,
                                                   T* __restrict__ vt, float* __restrict__ radius,
                                                   T* __restrict__ kc_lo) {
  constexpr int CH = D / 8;            // 8-channel chunks per row
  constexpr int RG = 256 / CH;         // row groups
  constexpr int RPT = kBlock / RG;     // rows per thread
  __shared__ float part[RG][D + 4];
  __shared__ float mean_s[D];
  __shared__ float dist_s[kBlock];
  __shared__ T tr[D][kBlock + 8];      // transposed V tile

  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int ch = tid % CH, rg = tid / CH;
  const size_t row_stride = (size_t)s.Hkv * D;
  const size_t base = ((size_t)b * s.T + (size_t)j * kBlock) * row_stride + (size_t)g * D;

  // ---- K: load 8 channels x RPT rows, partial sums --------------------------
  float kr[RPT][8];
  float acc[8];
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    typename Frag<T>::type x = Frag<T>::load(k + base + (size_t)row * row_stride + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) { kr[i][e] = (float)x[e]; acc[e] += kr[i][e]; }
  }
  for (int e = 0; e < 8; ++e) part[rg][ch * 8 + e] = acc[e];
  __syncthreads();
  const size_t cbase = (((size_t)b * s.nc + j) * s.Hkv + g) * D;
  if (tid < D) {
    float m = 0.f;
    for (int r = 0; r < RG; ++r) m += part[r][tid];
    const float mf = m * (1.0f / kBlock);
    T mr = from_f32<T>(mf);
    if (kc) kc[cbase + tid] = mr;
    // residual of the rounded mean, so that hi + lo carries ~16 more bits
    if (kc_lo) kc_lo[cbase + tid] = from_f32<T>(mf - (float)mr);
    mean_s[tid] = mf;
  }
  __syncthreads();
  if (radius) {
    // squared distance of each row to the rounded mean
    float dsq[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float df = kr[i][e] - mean_s[ch * 8 + e];
        sum += df * df;
      }
      dsq[i] = sum;
    }
    // reduce over the CH chunks of a row: stage through part[]
#pragma unroll
    for (int i = 0; i < RPT; ++i) part[rg][ch + i * CH] = dsq[i];  // RPT*CH <= D+4 slots
    __syncthreads();
    if (tid < kBlock) {
      const int r = tid / RPT, i = tid % RPT;
      float sum = 0.f;
      for (int c = 0; c < CH; ++c) sum += part[r][c + i * CH];
      dist_s[tid] = sum;
    }
    __syncthreads();
    if (tid == 0) {
      float mx = 0.f;
      for (int r = 0; r < kBlock; ++r) mx = fmaxf(mx, dist_s[r]);
      // small relative slack covers fp32 rounding of the distance itself
      radius[((size_t)b * s.Hkv + g) * s.ncp + j] = sqrtf(mx) * (1.0f + 1e-5f) + 1e-30f;
      if (j == s.nc - 1)
        for (int jj = s.nc; jj < s.ncp; ++jj) radius[((size_t)b * s.Hkv + g) * s.ncp + jj] = 0.f;
    }
    __syncthreads();
  }

  // ---- V: same mean, plus the transposed copies -------------------------------
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int row = rg * RPT + i;
    typename Frag<T>::type x = Frag<T>::load(v + base + (size_t)row * row_stride + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[e] += (float)x[e];
      tr[ch * 8 + e][row] = x[e];
    }
  }
  for (int e = 0; e < 8; ++e) part[rg][ch * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float m = 0.f;
    for (int r = 0; r < RG; ++r) m += part[r][tid];
    T mr = from_f32<T>(m * (1.0f / kBlock));
    if (vc) vc[cbase + tid] = mr;
    if (vct) {
      T* col = vct + (((size_t)b * s.Hkv + g) * D + tid) * s.ncp;
      col[j] = mr;
      if (j == s.nc - 1)
        for (int jj = s.nc; jj < s.ncp; ++jj) col[jj] = from_f32<T>(0.f);
    }
  }
  if (vt) {
    // D rows of 64 contiguous keys; 16-byte pieces
    constexpr int PIECES = kBlock * sizeof(T) / 16;  // per channel row
    for (int w = tid; w < D * PIECES; w += 256) {
      const int d = w / PIECES, pc = w % PIECES;
      constexpr int EPP = 16 / sizeof(T);
      T* dst = vt + (((size_t)b * s.Hkv + g) * D + d) * s.T + (size_t)j * kBlock + pc * EPP;
      // EPP elements (8 bf16 or 4 fp32) per aligned 16-byte store
      if constexpr (sizeof(T) == 2) {
        bf16x8 r;
        for (int e = 0; e < 8; ++e) r[e] = tr[d][pc * 8 + e];
        *reinterpret_cast<bf16x8*>(dst) = r;
      } else {
        f32x4 r;
        for (int e = 0; e < 4; ++e) r[e] = tr[d][pc * 4 + e];
        *reinterpret_cast<f32x4*>(dst) = r;
      }
    }
  }
}

template <typename T, int D>
static hipError_t launch_pool_t(const Shape& s, const void* k, const void* v, void* kc, void* vc,
                                void* vct, void* vt, float* radius, void* kc_lo, hipStream_t st) {
  dim3 grid(s.nc, s.Hkv, s.B);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, s, (const T*)k, (const T*)v,
                     (T*)kc, (T*)vc, (T*)vct, (T*)vt, radius, (T*)kc_lo);
  return hipGetLastError();
}

hipError_t launch_pool(bool is_bf16, const Shape& s, const void* k, const void* v, void* kc,
                       void* vc, void* vct, void* vt, float* radius, void* kc_lo,
                       hipStream_t st) {
  if (s.nc == 0) return hipSuccess;
  if (is_bf16) {
    if (s.D == 64) return launch_pool_t<bf16, 64>(s, k, v, kc, vc, vct, vt, radius, kc_lo, st);
    return launch_pool_t<bf16, 128>(s, k, v, kc, vc, vct, vt, radius, kc_lo, st);
  }
  return launch_pool_t<float, 64>(s, k, v, kc, vc, vct, vt, radius, nullptr, st);
}

}  // namespace nsa
