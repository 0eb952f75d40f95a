// pool.hip -- K1: mean-pool compression of K and V.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work? / COMPRESSION:
// the tokens of each block are summarised into one key and one value;
// [SIC] "Sparsity is Cool", Method: the summary is a mean-pool, block 64.
//
// Two workgroups per (64-token block j, KV head g, batch b): one for the K
// tile, one for the V tile, so that each is a single memory round trip deep.
// A tile (64 x D) is read once, coalesced (each thread owns 8 consecutive
// channels of a few rows), summed in fp32 and divided by 64; the mean is
// rounded once to the element type.  The same pass also emits what the
// attention kernels want to read as MFMA operands (the K workgroup the K half
// of the block image, the V workgroup the V^T half):
//   kvimg  [B][Hkv][nc][KvImage bytes]  each block's K and V^T in MFMA
//                           fragment order (see KvImage), the image the
//                           selection / window kernel copies into LDS with
//                           contiguous 1 KB loads;
//   vct    [B][Hkv][D][ncp] the pooled V transposed, zero-padded to ncp;
//   knorm  [B][Hkv][nc]     max_i |k_i| over the block (fp32), which bounds
//                           every logit against the block by Cauchy-Schwarz;
//   kc_lo  [B][nc][Hkv][D]  (bf16 only) Kc - round(Kc), so that the block
//                           scores can use hi + lo (about 16 more bits) and
//                           the top-k decisions are not moved by the rounding
//                           of the pooled keys.
// HBM-bound: reads 2*64*D elements per (j, g, b), writes the same once more
// (kvimg) plus 2*D pooled values.
#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(Shape s, const T* __restrict__ k,
                                                   const T* __restrict__ v, T* __restrict__ kc,
                                                   T* __restrict__ vc, T* __restrict__ vct,
                                                   T* __restrict__ kvimg, float* __restrict__ knorm,
                                                   T* __restrict__ kc_lo) {
  constexpr int CH = D / 8;            // 8-channel chunks per row
  constexpr int RG = 256 / CH;         // row groups
  constexpr int RPT = kBlock / RG;     // rows per thread
  typedef KvImage<T, D> I;
  __shared__ float part[RG][D + 4];
  __shared__ float dist_s[kBlock];
  // the K tile (64 x D + pad) or, in a V workgroup, the V tile transposed (D x 64 + pad)
  constexpr int TILE = kBlock * (D + 8) > D * (kBlock + 8) ? kBlock * (D + 8) : D * (kBlock + 8);
  __shared__ __align__(16) T tile_raw[TILE];
  T (*tile)[D + 8] = reinterpret_cast<T (*)[D + 8]>(tile_raw);
  T (*tr)[kBlock + 8] = reinterpret_cast<T (*)[kBlock + 8]>(tile_raw);

  // z = 2 b + (0: K, 1: V): the two halves of a block are independent
  // workgroups, each one memory round trip deep
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z >> 1;
  const bool vpart = (blockIdx.z & 1) != 0;
  const int tid = threadIdx.x;
  const int ch = tid % CH, rg = tid / CH;
  const size_t row_stride = (size_t)s.Hkv * D;
  const size_t base = ((size_t)b * s.T + (size_t)j * kBlock) * row_stride + (size_t)g * D;
  const size_t cbase = (((size_t)b * s.nc + j) * s.Hkv + g) * D;
  unsigned char* img = kvimg ? reinterpret_cast<unsigned char*>(kvimg) +
                                   (((size_t)b * s.Hkv + g) * s.nc + j) * (size_t)I::BYTES
                             : nullptr;

  if (!vpart) {
    // ---- K: load 8 channels x RPT rows, partial sums ------------------------
    float kr[RPT][8];
    float acc[8];
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int row = rg * RPT + i;
      typename Frag<T>::type x = Frag<T>::load(k + base + (size_t)row * row_stride + ch * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) { kr[i][e] = (float)x[e]; acc[e] += kr[i][e]; tile[row][ch * 8 + e] = x[e]; }
    }
    for (int e = 0; e < 8; ++e) part[rg][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
      float m = 0.f;
      for (int r = 0; r < RG; ++r) m += part[r][tid];
      const float mf = m * (1.0f / kBlock);
      T mr = from_f32<T>(mf);
      if (kc) kc[cbase + tid] = mr;
      // residual of the rounded mean, so that hi + lo carries ~16 more bits
      if (kc_lo) kc_lo[cbase + tid] = from_f32<T>(mf - (float)mr);
    }
    __syncthreads();
    if (knorm) {
      // squared norm of each row (fp32, from the exact input values)
      float nsq[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += kr[i][e] * kr[i][e];
        nsq[i] = sum;
      }
      // reduce over the CH chunks of a row: stage through part[]
#pragma unroll
      for (int i = 0; i < RPT; ++i) part[rg][ch + i * CH] = nsq[i];  // RPT*CH <= D+4 slots
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
        // small relative slack covers fp32 rounding of the norm itself
        knorm[((size_t)b * s.Hkv + g) * s.nc + j] = sqrtf(mx) * (1.0f + 1e-5f);
      }
    }
    if (img) {
      __syncthreads();  // the K tile is complete
      // the K fragments: the first half of the image
      for (int w = tid; w < I::PIECES / 2 * 64; w += 256) {
        const int pc = w / 64, l = w % 64;
        const int f = pc / I::NV, vv = pc % I::NV;
        const int a = l / 16, rho = l % 16;
        const T* src = &tile[I::krow(I::k_u(f), rho)][I::k_ks(f) * 32 + 8 * a + vv * I::EPV];
        T piece[I::EPV];
#pragma unroll
        for (int e = 0; e < I::EPV; ++e) piece[e] = src[e];
        *reinterpret_cast<f32x4*>(img + (size_t)pc * 1024 + 16 * l) = *reinterpret_cast<const f32x4*>(piece);
      }
    }
  } else {
    // ---- V: the same mean, plus the transposed copies ------------------------
    float acc[8];
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
    __syncthreads();  // also completes the transposed tile
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
    if (img) {
      // the V^T fragments: the second half of the image
      for (int w = tid; w < I::PIECES / 2 * 64; w += 256) {
        const int pc = I::PIECES / 2 + w / 64, l = w % 64;
        const int f2 = pc / I::NV - I::NFRAG, vv = pc % I::NV;
        const int a = l / 16, rho = l % 16;
        const T* src = &tr[I::v_mt(f2) * 16 + rho][32 * I::v_h(f2) + 8 * a + vv * I::EPV];
        T piece[I::EPV];
#pragma unroll
        for (int e = 0; e < I::EPV; ++e) piece[e] = src[e];
        *reinterpret_cast<f32x4*>(img + (size_t)pc * 1024 + 16 * l) = *reinterpret_cast<const f32x4*>(piece);
      }
    }
  }
}

template <typename T, int D>
static hipError_t launch_pool_t(const Shape& s, const void* k, const void* v, void* kc, void* vc,
                                void* vct, void* kvimg, float* knorm, void* kc_lo, hipStream_t st) {
  dim3 grid(s.nc, s.Hkv, 2 * s.B);  // z: batch and K / V half
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, st, s, (const T*)k, (const T*)v,
                     (T*)kc, (T*)vc, (T*)vct, (T*)kvimg, knorm, (T*)kc_lo);
  return hipGetLastError();
}

hipError_t launch_pool(bool is_bf16, const Shape& s, const void* k, const void* v, void* kc,
                       void* vc, void* vct, void* kvimg, float* knorm, void* kc_lo,
                       hipStream_t st) {
  if (s.nc == 0) return hipSuccess;
  if (is_bf16) {
    if (s.D == 64) return launch_pool_t<bf16, 64>(s, k, v, kc, vc, vct, kvimg, knorm, kc_lo, st);
    return launch_pool_t<bf16, 128>(s, k, v, kc, vc, vct, kvimg, knorm, kc_lo, st);
  }
  return launch_pool_t<float, 64>(s, k, v, kc, vc, vct, kvimg, knorm, nullptr, st);
}

}  // namespace nsa
