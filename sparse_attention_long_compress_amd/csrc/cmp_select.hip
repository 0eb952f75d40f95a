// cmp_select.hip -- K2: compressed attention, block importance and top-k.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work?:
//   COMPRESSION -- attention over the block summaries (the pooled keys);
//   SELECTION   -- block importance reuses the compression attention scores;
// [SIC] "Sparsity is Cool", Method: top-k 16 over 64-token blocks; Key claims:
//   the first block is always read.  Readings used here: the importance of
//   block j for (t, g) is the compressed-attention probability summed over the
//   query heads of KV group g; block 0 and the query's own block are always
//   selected and count toward k; ties go to the lower block index.
//
// One workgroup (4 waves) per (tile of P query positions, KV group g, batch b);
// every position of a tile lies in the same 64-token block c, so they share the
// candidate set 1..c-1.  Query rows are ordered (position, head), 16 rows form
// one MFMA column group, each wave owns R/4 rows.
//   Pass 1: S^T = Kc Q^T on bf16/fp32 MFMA, online softmax, o_cmp = P Vc, and
//           U = max_j (tau q.Kc_j + tau |q| radius_j) over blocks 0 .. own, an
//           upper bound of every logit the row's selected blocks can produce
//           (log2 units).
//   Pass 2: recompute S^T, p = exp(s - lse), sum p over the G heads of each
//           position with DPP (adjacent lanes), stage S[position][block] in LDS
//           64 candidates at a time; one lane per position keeps its top-m
//           list in registers.  Each candidate is a 32-bit key: the score in
//           fixed point (21 bits over [0, G], resolution G / 2^21) above the
//           field 2047 - j, so "higher score, then lower index" is one unsigned
//           compare and inserting into the sorted list is one v_med3_u32 per
//           entry.
// For bf16 inputs the scores use the pooled keys as hi + lo (the rounded mean
// plus its bf16 residual, two MFMAs), so rounding Kc to bf16 does not move the
// importance by more than ~1e-6.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

constexpr uint32_t kIdxMask = 2047u;  // block index field of a top-k key

// score in [0, G] -> 21-bit fixed point (qscale = 2^21 / G) above the index field
__device__ __forceinline__ uint32_t topk_key(float score, float qscale, int j) {
  const float f = fminf(fmaxf(score * qscale, 0.f), 2097151.f);
  return ((uint32_t)f << 11) | (kIdxMask - (uint32_t)j);
}
__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

template <typename T, int D, int G, int LMAX>
__global__ __launch_bounds__(256) void cmp_select_kernel(
    Shape s, const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ kcl,
    const T* __restrict__ vct,
    const float* __restrict__ radius, T* __restrict__ o_cmp, float* __restrict__ ubound,
    int32_t* __restrict__ indices, int do_topk) {
  constexpr int P = (256 / G) < 64 ? (256 / G) : 64;  // positions per tile
  constexpr int R = P * G;                            // rows per tile
  constexpr int CGW = (R / 4) / 16 > 0 ? (R / 4) / 16 : 1;  // column groups per wave
  constexpr int KS = D / 32;                          // k-steps over the head dim
  constexpr int MT = D / 16;                          // 16-row tiles over the head dim
  constexpr int CHK = 64;                             // candidates staged per round
  typedef typename Frag<T>::type FragT;

  __shared__ float S_l[P][CHK + 1];

  const int tile = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int t0 = tile * P;
  const int c = t0 / kBlock;  // own block of every position in the tile
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const float c1 = s.scale * kLog2e;
  const int nvis = min(s.nc, c + 1);  // compressed blocks any row of the tile may see
  const int m_free = s.topk - (c == 0 ? 1 : 2);
  const bool need_scores = do_topk && (c - 1 > m_free);

  const size_t kc_row = (size_t)s.Hkv * D;
  const T* kc_b = kc + (size_t)b * s.nc * kc_row + (size_t)g * D;
  const T* kcl_b = kcl ? kcl + (size_t)b * s.nc * kc_row + (size_t)g * D : nullptr;
  const T* vct_b = vct + ((size_t)b * s.Hkv + g) * (size_t)D * s.ncp;
  const float* rad_b = radius ? radius + ((size_t)b * s.Hkv + g) * s.ncp : nullptr;

  float lse2[CGW];

  // ------------------------------------------------------------------ pass 1
  for (int cg = 0; cg < CGW; ++cg) {
    const int row = w * (R / 4) + cg * 16 + col;
    const bool row_ok = row < R;
    const int p = (row_ok ? row : 0) / G, hh = (row_ok ? row : 0) % G;
    const int t = t0 + p, h = g * G + hh;
    const T* qrow = q + (((size_t)b * s.T + t) * s.Hq + h) * D;
    FragT qf[KS];
    float qn2 = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = Frag<T>::load(qrow + ks * 32 + a * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) qn2 += (float)qf[ks][e] * (float)qf[ks][e];
    }
    const float qnorm = sqrtf(colsum4(qn2));
    float m = -INFINITY, lsum = 0.f, ub = -INFINITY;
    f32x4 o[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] = zero4();

    for (int j0 = 0; j0 < nvis; j0 += 32) {
      f32x4 st[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int key = j0 + 8 * (col / 4) + 4 * u + (col % 4);
        key = min(key, s.nc - 1);
        const T* krow = kc_b + (size_t)key * kc_row;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = mma(acc, Frag<T>::load(krow + ks * 32 + a * 8), qf[ks]);
        if (kcl_b) {
          const T* lrow = kcl_b + (size_t)key * kc_row;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mma(acc, Frag<T>::load(lrow + ks * 32 + a * 8), qf[ks]);
        }
        st[u] = acc;
      }
      float x[8], pv[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int jj = j0 + 8 * a + 4 * u + r;
          const bool vis = row_ok && (jj * kBlock + kBlock - 1 <= t) && jj < s.nc;
          const float xv = st[u][r] * c1;
          x[4 * u + r] = vis ? xv : -INFINITY;
          // bound over every block the row may select: 0 .. own (complete
          // or not, the block's keys are all within radius of its mean)
          if (row_ok && rad_b && jj <= c && jj < s.nc)
            ub = fmaxf(ub, xv + qnorm * c1 * rad_b[jj]);
        }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
      mx = colmax4(mx);
      const float mn = fmaxf(m, mx);
      float alpha = 1.f, psum = 0.f;
      if (mn == -INFINITY) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = 0.f;
      } else {
        alpha = fast_exp2(m - mn);
#pragma unroll
        for (int e = 0; e < 8; ++e) { pv[e] = fast_exp2(x[e] - mn); psum += pv[e]; }
      }
      lsum = lsum * alpha + colsum4(psum);
      m = mn;
      const FragT pf = Frag<T>::from_f32(pv);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const FragT vf = Frag<T>::load(vct_b + (size_t)(mt * 16 + col) * s.ncp + j0 + 8 * a);
        o[mt] = mma(o[mt] * alpha, vf, pf);
      }
    }
    lse2[cg] = (lsum > 0.f) ? m + __log2f(lsum) : -INFINITY;
    if (o_cmp && row_ok) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      T* orow = o_cmp + (((size_t)b * s.T + t) * s.Hq + h) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store4(orow + mt * 16 + 4 * a, o[mt] * inv);
    }
    if (ubound && row_ok) {
      ub = colmax4(ub);
      if (a == 0) ubound[((size_t)b * s.Hq + h) * s.T + t] = ub;
    }
  }

  if (!do_topk) return;

  // ------------------------------------------------------------------ pass 2
  uint32_t list[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) list[i] = 0u;

  if (need_scores) {
    for (int jb = 1; jb <= c - 1; jb += CHK) {
      for (int cg = 0; cg < CGW; ++cg) {
        const int row = w * (R / 4) + cg * 16 + col;
        const bool row_ok = row < R;
        const int p = (row_ok ? row : 0) / G, hh = (row_ok ? row : 0) % G;
        const int t = t0 + p, h = g * G + hh;
        const T* qrow = q + (((size_t)b * s.T + t) * s.Hq + h) * D;
        FragT qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = Frag<T>::load(qrow + ks * 32 + a * 8);
        for (int j0 = jb; j0 < jb + CHK && j0 <= c - 1; j0 += 32) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            int key = j0 + 8 * (col / 4) + 4 * u + (col % 4);
            key = min(key, s.nc - 1);
            const T* krow = kc_b + (size_t)key * kc_row;
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) acc = mma(acc, Frag<T>::load(krow + ks * 32 + a * 8), qf[ks]);
            if (kcl_b) {
              const T* lrow = kcl_b + (size_t)key * kc_row;
#pragma unroll
              for (int ks = 0; ks < KS; ++ks)
                acc = mma(acc, Frag<T>::load(lrow + ks * 32 + a * 8), qf[ks]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = j0 + 8 * a + 4 * u + r;
              float pr = row_ok ? fast_exp2(acc[r] * c1 - lse2[cg]) : 0.f;
              pr = group_sum<G>(pr);
              if (row_ok && (col % G) == 0 && jj <= c - 1) S_l[p][jj - jb] = pr;
            }
          }
        }
      }
      __syncthreads();
      if (threadIdx.x < P) {
        const int jend = min(jb + CHK, c);
        const float qscale = 2097152.f / (float)G;
        for (int jj = jb; jj < jend; ++jj) {
          const uint32_t x = topk_key(S_l[threadIdx.x][jj - jb], qscale, jj);
#pragma unroll
          for (int i = LMAX - 1; i >= 1; --i) list[i] = umed3(list[i], list[i - 1], x);
          list[0] = max(list[0], x);
        }
      }
      __syncthreads();
    }
  }

  if (threadIdx.x < P) {
    const int t = t0 + threadIdx.x;
    constexpr int KMAX = LMAX + 2;
    int sel[KMAX];
#pragma unroll
    for (int i = 0; i < KMAX; ++i) sel[i] = 0x7fffffff;
    int n = 0;
    auto ins = [&](int x) {
#pragma unroll
      for (int i = KMAX - 1; i >= 1; --i) sel[i] = max(min(sel[i], x), min(max(sel[i], x), sel[i - 1]));
      sel[0] = min(sel[0], x);
      ++n;
    };
    ins(0);
    if (c > 0) ins(c);
    if (!need_scores) {
      for (int j = 1; j <= c - 1; ++j) ins(j);
    } else {
#pragma unroll
      for (int i = 0; i < LMAX; ++i)
        if (i < m_free) ins((int)(kIdxMask - (list[i] & kIdxMask)));
    }
    int32_t* dst = indices + (((size_t)b * s.Hkv + g) * s.T + t) * s.topk;
#pragma unroll
    for (int i = 0; i < KMAX; ++i)
      if (i < s.topk) dst[i] = i < n ? sel[i] : -1;
  }
}

template <typename T, int D, int G>
static hipError_t launch_cs(const Shape& s, const void* q, const void* kc, const void* kcl,
                            const void* vct, const float* radius, void* o_cmp, float* ubound,
                            int32_t* indices, bool do_topk, hipStream_t st) {
  constexpr int P = (256 / G) < 64 ? (256 / G) : 64;
  dim3 grid(s.T / P, s.Hkv, s.B);
  if (s.topk - 2 <= 16)
    hipLaunchKernelGGL((cmp_select_kernel<T, D, G, 16>), grid, dim3(256), 0, st, s, (const T*)q,
                       (const T*)kc, (const T*)kcl, (const T*)vct, radius, (T*)o_cmp, ubound,
                       indices, do_topk ? 1 : 0);
  else
    hipLaunchKernelGGL((cmp_select_kernel<T, D, G, 32>), grid, dim3(256), 0, st, s, (const T*)q,
                       (const T*)kc, (const T*)kcl, (const T*)vct, radius, (T*)o_cmp, ubound,
                       indices, do_topk ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_cs_g(const Shape& s, const void* q, const void* kc, const void* kcl,
                              const void* vct, const float* radius, void* o_cmp, float* ubound,
                              int32_t* indices, bool do_topk, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_cs<T, D, 1>(s, q, kc, kcl, vct, radius, o_cmp, ubound, indices, do_topk, st);
    case 2: return launch_cs<T, D, 2>(s, q, kc, kcl, vct, radius, o_cmp, ubound, indices, do_topk, st);
    case 4: return launch_cs<T, D, 4>(s, q, kc, kcl, vct, radius, o_cmp, ubound, indices, do_topk, st);
    case 8: return launch_cs<T, D, 8>(s, q, kc, kcl, vct, radius, o_cmp, ubound, indices, do_topk, st);
    default: return launch_cs<T, D, 16>(s, q, kc, kcl, vct, radius, o_cmp, ubound, indices, do_topk, st);
  }
}

hipError_t launch_cmp_select(bool is_bf16, const Shape& s, const void* q, const void* kc,
                             const void* kc_lo, const void* vct, const float* radius,
                             void* o_cmp, float* ubound, int32_t* indices, bool do_topk,
                             hipStream_t st) {
  if (is_bf16) {
    if (s.D == 64)
      return launch_cs_g<bf16, 64>(s, q, kc, kc_lo, vct, radius, o_cmp, ubound, indices, do_topk, st);
    return launch_cs_g<bf16, 128>(s, q, kc, kc_lo, vct, radius, o_cmp, ubound, indices, do_topk, st);
  }
  return launch_cs_g<float, 64>(s, q, kc, nullptr, vct, radius, o_cmp, ubound, indices, do_topk, st);
}

}  // namespace nsa
