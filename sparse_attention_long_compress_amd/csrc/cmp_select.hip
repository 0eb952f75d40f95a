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
// One workgroup (up to 8 waves) per (tile of P query positions, KV group g, batch b);
// every position of a tile lies in the same 64-token block c, so they share the
// candidate set 1..c-1.  Query rows are ordered (position, head), 16 rows form
// one MFMA column group, each wave owns R/NW rows.  Pooled keys and values are
// staged in LDS 64 blocks at a time (shared by all waves).
//   Pass 1: S^T = Kc Q^T on MFMA, online softmax, o_cmp = P Vc and the
//           row's log-sum-exp (natural log; -inf when no block is visible).
//   Pass 2: recompute S^T, p = exp(s - lse), sum p over the G heads of each
//           position with DPP (adjacent lanes), stage S[position][block] in LDS
//           64 candidates at a time; each wave scans its share of them with
//           one lane per position keeping a sorted top-m list in registers
//           (each wave's candidates of a chunk are sorted by a bitonic network
//           and merged in), and the waves' lists are merged pairwise at the
//           end.  A candidate is a 32-bit key: the score in fixed point (21
//           bits over [0, G], resolution G / 2^21) above the field 2047 - j,
//           so "higher score, then lower index" is one unsigned compare.
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
// Top N of two descending lists a, b (N a power of two), into a: the pairwise
// maxima of a and b reversed are the N largest of the union as a bitonic
// sequence, which log2(N) compare-exchange stages sort descending.
template <int N>
__device__ __forceinline__ void merge_desc(uint32_t (&a)[N], const uint32_t (&b)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = max(a[i], b[N - 1 - i]);
#pragma unroll
  for (int d = N / 2; d >= 1; d >>= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if ((i & d) == 0) {
        const uint32_t hi = max(a[i], a[i + d]), lo = min(a[i], a[i + d]);
        a[i] = hi;
        a[i + d] = lo;
      }
}

// sort N keys descending (N a power of two; bitonic network of min / max)
template <int N>
__device__ __forceinline__ void sort_desc(uint32_t (&a)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int d = k / 2; d >= 1; d >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int p = i ^ d;
        if (p > i) {
          const bool desc = (i & k) == 0;
          const uint32_t hi = max(a[i], a[p]), lo = min(a[i], a[p]);
          a[i] = desc ? hi : lo;
          a[p] = desc ? lo : hi;
        }
      }
}

template <typename T, int D, int G>
struct K2Cfg {
  // positions per tile: 256 rows at head_dim 64, 128 at 128 (capped at one block)
  static constexpr int P = ((D == 64 ? 256 : 128) / G) < 64 ? ((D == 64 ? 256 : 128) / G) : 64;
  static constexpr int R = P * G;                            // rows per tile
  static constexpr int NW = (R / 16) < 8 ? (R / 16) : 8;     // waves (at least one column group each)
  static constexpr int NT = NW * 64;
  static constexpr int RWV = R / NW;                         // rows per wave
  static constexpr int CGW = RWV / 16;                       // column groups per wave
  static constexpr int CPW = 64 / NW;                        // top-k candidates per wave and chunk
  static constexpr int KS = D / 32, MT = D / 16;
  // minimum waves per SIMD (launch bound): 4 with 8 waves -- two workgroups
  // per CU, at most 128 VGPRs (at head_dim 128 the tile has half as many
  // positions, one column group per wave, so that it fits); fp32 fragments
  // are twice as wide and would spill under that bound
  static constexpr int MIN_WAVES_EU = (NW == 8 && sizeof(T) == 2) ? 4 : 1;
  static constexpr int KST = D + 8;   // LDS row stride of the pooled-key chunk
  static constexpr int VST = 64 + 8;  // LDS row stride of the pooled-value chunk
};

template <typename T, int D, int G, int LMAX>
__global__ __launch_bounds__((K2Cfg<T, D, G>::NT), (K2Cfg<T, D, G>::MIN_WAVES_EU)) void cmp_select_kernel(
    Shape s, const T* __restrict__ q, const T* __restrict__ kc, const T* __restrict__ kcl,
    const T* __restrict__ vct, T* __restrict__ o_cmp, float* __restrict__ lse_cmp,
    int32_t* __restrict__ indices, int do_topk) {
  typedef K2Cfg<T, D, G> C;
  constexpr int P = C::P, CGW = C::CGW, KS = C::KS, MT = C::MT, KST = C::KST, VST = C::VST;
  constexpr int NW = C::NW, NT = C::NT, CPW = C::CPW;
  typedef typename Frag<T>::type FragT;
  constexpr int EPV = 16 / sizeof(T);

  // the pooled-key tiles (and their residuals) share storage with the lists
  // the waves hand over when merging their top-k lists, which happens after
  // the last chunk (keeps head_dim 128 at two workgroups per CU)
  constexpr size_t KL_BYTES = 2 * 64 * KST * sizeof(T);
  constexpr size_t ML_BYTES = (size_t)((NW + 1) / 2) * P * (LMAX + 1) * 4;
  __shared__ __align__(16) unsigned char kl_raw[KL_BYTES > ML_BYTES ? KL_BYTES : ML_BYTES];
  T* Ks = reinterpret_cast<T*>(kl_raw);
  T* Ls = Ks + 64 * KST;
  auto mlist = reinterpret_cast<uint32_t(*)[P][LMAX + 1]>(kl_raw);  // [(NW + 1) / 2][P][LMAX + 1]
  __shared__ __align__(16) T Vs[D * VST];
  __shared__ float S_l[P][65];

  const int NTL = s.T / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, s.B * s.Hkv, NTL, bg, tile);
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int c = t0 / kBlock;  // own block of every position in the tile
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const float c1 = s.scale * kLog2e;
  const int nvis = min(s.nc, c + 1);  // compressed blocks any row of the tile may see
  const int m_free = s.topk - (c == 0 ? 1 : 2);
  const bool need_scores = do_topk && (c - 1 > m_free);
  const bool has_lo = kcl != nullptr;

  const size_t kc_row = (size_t)s.Hkv * D;
  const T* kc_b = kc + (size_t)b * s.nc * kc_row + (size_t)g * D;
  const T* kcl_b = has_lo ? kcl + (size_t)b * s.nc * kc_row + (size_t)g * D : nullptr;
  const T* vct_b = vct + ((size_t)b * s.Hkv + g) * (size_t)D * s.ncp;

  // 16-byte chunk c of pooled-key row r in LDS: rows 16..31 (mod 32) are
  // rotated by four chunks so that the 16 rows one MFMA fragment read touches
  // (r and r + 16 among them) fall in distinct bank groups
  auto kchunk = [](int r, int c) { return c ^ (((r >> 4) & 1) << 2); };
  // stage pooled keys (and the residual) of blocks jb .. jb+63, and optionally
  // the pooled values; rows past the last complete block are clamped (masked)
  auto stage = [&](int jb, bool with_v) {
    for (int i = threadIdx.x; i < 64 * (D / EPV); i += NT) {
      const int r = i / (D / EPV), c8 = i % (D / EPV);
      const int key = min(jb + r, s.nc - 1);
      const int cs = kchunk(r, c8);
      *reinterpret_cast<int4*>(Ks + r * KST + cs * EPV) =
          *reinterpret_cast<const int4*>(kc_b + (size_t)key * kc_row + c8 * EPV);
      if (has_lo)
        *reinterpret_cast<int4*>(Ls + r * KST + cs * EPV) =
            *reinterpret_cast<const int4*>(kcl_b + (size_t)key * kc_row + c8 * EPV);
    }
    if (with_v)
      for (int i = threadIdx.x; i < D * (64 / EPV); i += NT) {
        const int r = i / (64 / EPV), c8 = i % (64 / EPV);
        *reinterpret_cast<int4*>(Vs + r * VST + c8 * EPV) =
            *reinterpret_cast<const int4*>(vct_b + (size_t)r * s.ncp + jb + c8 * EPV);
      }
  };
  // S^T tile u of the 32-key half h of the staged chunk (keys h*32 + 8a + 4u + r)
  auto scores = [&](int h, int u, const FragT (&qf)[KS]) -> f32x4 {
    const int kr = h * 32 + 8 * (col / 4) + 4 * u + (col % 4);
    f32x4 acc = zero4();
    // elements ks * 32 + 8 a .. + 7 of the row: chunk (ks * 32 + 8 a) / EPV
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mma(acc, Frag<T>::load(Ks + kr * KST + kchunk(kr, (ks * 32 + a * 8) / EPV) * EPV), qf[ks]);
    if (has_lo) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = mma(acc, Frag<T>::load(Ls + kr * KST + kchunk(kr, (ks * 32 + a * 8) / EPV) * EPV), qf[ks]);
    }
    return acc;
  };

  // rows of this wave: (position, head) with lane column col in group cg
  FragT qf[CGW][KS];
  int tpos[CGW], hidx[CGW], ppos[CGW];
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    const int row = w * C::RWV + cg * 16 + col;
    ppos[cg] = row / G;
    tpos[cg] = t0 + ppos[cg];
    hidx[cg] = g * G + row % G;
    const T* qrow = q + (((size_t)b * s.T + tpos[cg]) * s.Hq + hidx[cg]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[cg][ks] = Frag<T>::load(qrow + ks * 32 + a * 8);
  }

  // ------------------------------------------------------------------ pass 1
  float m[CGW], lsum[CGW], lse2[CGW];
  f32x4 o[CGW][MT];
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    m[cg] = -INFINITY;
    lsum[cg] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[cg][mt] = zero4();
  }
  for (int jb = 0; jb < nvis; jb += 64) {
    __syncthreads();
    stage(jb, true);
    __syncthreads();
    for (int h = 0; h < 2 && jb + h * 32 < nvis; ++h) {
      // blocks below the tile's own block are visible to every row of it (and
      // complete): only a half that reaches block c needs the per-element mask
      const bool full = jb + h * 32 + 31 < c;
#pragma unroll
      for (int cg = 0; cg < CGW; ++cg) {
        float x[8], pv[8];  // raw scores (the scale c1 > 0 is applied in the exponent)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const f32x4 st = scores(h, u, qf[cg]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (full) {
              x[4 * u + r] = st[r];
            } else {
              const int jj = jb + h * 32 + 8 * a + 4 * u + r;
              const bool vis = (jj * kBlock + kBlock - 1 <= tpos[cg]) && jj < s.nc;
              x[4 * u + r] = vis ? st[r] : -INFINITY;
            }
          }
        }
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
        mx = xmax4(mx) * c1;
        const float mn = fmaxf(m[cg], mx);
        float alpha = 1.f, psum = 0.f;
        if (mn == -INFINITY) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = 0.f;
        } else {
          alpha = fast_exp2(m[cg] - mn);
#pragma unroll
          for (int e = 0; e < 8; ++e) { pv[e] = fast_exp2(fmaf(x[e], c1, -mn)); psum += pv[e]; }
        }
        lsum[cg] = lsum[cg] * alpha + xsum4(psum);
        m[cg] = mn;
        const FragT pf = Frag<T>::from_f32(pv);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          o[cg][mt] = mma(o[cg][mt] * alpha,
                          Frag<T>::load(Vs + (mt * 16 + col) * VST + h * 32 + 8 * a), pf);
      }
    }
  }
#pragma unroll
  for (int cg = 0; cg < CGW; ++cg) {
    lse2[cg] = (lsum[cg] > 0.f) ? m[cg] + __log2f(lsum[cg]) : -INFINITY;
    // (the row coordinates pass through an opaque copy, so the Q loads'
    // addresses are recomputed here rather than kept alive, in scratch,
    // across pass 1)
    int tq = tpos[cg], hq = hidx[cg];
    asm volatile("" : "+v"(tq), "+v"(hq));
    if (o_cmp) {
      const float inv = lsum[cg] > 0.f ? 1.f / lsum[cg] : 0.f;
      T* orow = o_cmp + (((size_t)b * s.T + tq) * s.Hq + hq) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) store4(orow + mt * 16 + 4 * a, o[cg][mt] * inv);
    }
    if (lse_cmp && a == 0) lse_cmp[((size_t)b * s.Hq + hq) * s.T + tq] = lse2[cg] * kLn2;
  }

  if (!do_topk) return;

  // ------------------------------------------------------------------ pass 2
  uint32_t list[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) list[i] = 0u;
  const float qscale = 2097152.f / (float)G;

  if (need_scores) {
    // candidates 1 .. c - 1 in the 64-block chunks of pass 1, last chunk first:
    // when it is pass 1's last chunk its keys are still in LDS
    const int jb_last1 = (nvis - 1) / 64 * 64;  // pass 1's last chunk
    const int jb_top = (c - 1) / 64 * 64;
    for (int jb = jb_top; jb >= 0; jb -= 64) {
      if (jb != jb_last1) {
        __syncthreads();
        stage(jb, false);
      }
      __syncthreads();
      for (int h = 0; h < 2 && jb + h * 32 <= c - 1; ++h) {
#pragma unroll
        for (int cg = 0; cg < CGW; ++cg) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const f32x4 st = scores(h, u, qf[cg]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int jj = jb + h * 32 + 8 * a + 4 * u + r;
              float pr = fast_exp2(st[r] * c1 - lse2[cg]);
              pr = group_sum<G>(pr);
              if ((col % G) == 0 && jj >= 1 && jj <= c - 1) S_l[ppos[cg]][jj - jb] = pr;
            }
          }
        }
      }
      __syncthreads();
      // wave w takes candidates jb + CPW w .. jb + CPW (w + 1) - 1, one lane per
      // position: all read at once, sorted by a network, merged into the list
      // (a missing candidate is key 0)
      if (l < P) {
        const int j0 = max(jb + CPW * w, 1), j1 = min(jb + CPW * w + CPW, c);
        uint32_t cand[LMAX];
#pragma unroll
        for (int k = 0; k < LMAX; ++k)
          cand[k] = (k < CPW && j0 + k < j1) ? topk_key(S_l[l][j0 + k - jb], qscale, j0 + k) : 0u;
        static_assert(CPW <= LMAX && (CPW & (CPW - 1)) == 0, "candidates per wave");
        uint32_t (&c8)[CPW] = *reinterpret_cast<uint32_t(*)[CPW]>(cand);
        sort_desc(c8);
        merge_desc(list, cand);
      }
    }
    // merge the per-wave lists pairwise into wave 0's: in the round of stride
    // st, wave w + st hands its list to wave w (w a multiple of 2 st)
#pragma unroll
    for (int st = 1; st < NW; st <<= 1) {
      __syncthreads();
      if (w % (2 * st) == st && l < P) {
#pragma unroll
        for (int i = 0; i < LMAX; ++i) mlist[w / (2 * st)][l][i] = list[i];
      }
      __syncthreads();
      if (w % (2 * st) == 0 && w + st < NW && l < P) {
        uint32_t other[LMAX];
#pragma unroll
        for (int i = 0; i < LMAX; ++i) other[i] = mlist[w / (2 * st)][l][i];
        merge_desc(list, other);
      }
    }
  }

  // The row's selection in increasing block order: block 0, the picks (all in
  // 1 .. c - 1) sorted, the own block c.  Without scores every block 0 .. c
  // is selected.
  if (w == 0 && l < P) {
    const int t = t0 + l;
    int32_t* dst = indices + (((size_t)b * s.Hkv + g) * s.T + t) * s.topk;
    if (!need_scores) {
      for (int i = 0; i < s.topk; ++i) dst[i] = i <= c ? i : -1;
    } else {
      // block indices of the picks (list is sorted by score), unused slots
      // last, sorted ascending
      uint32_t pk[LMAX];
#pragma unroll
      for (int i = 0; i < LMAX; ++i) pk[i] = i < m_free ? ~(kIdxMask - (list[i] & kIdxMask)) : 0u;
      sort_desc(pk);  // descending in ~j: ascending in j
      dst[0] = 0;
#pragma unroll
      for (int i = 0; i < LMAX; ++i)
        if (i < m_free) dst[1 + i] = (int32_t)~pk[i];
      dst[1 + m_free] = c;
      for (int i = m_free + 2; i < s.topk; ++i) dst[i] = -1;
    }
  }
}

template <typename T, int D, int G>
static hipError_t launch_cs(const Shape& s, const void* q, const void* kc, const void* kcl,
                            const void* vct, void* o_cmp, float* lse_cmp,
                            int32_t* indices, bool do_topk, hipStream_t st) {
  constexpr int P = K2Cfg<T, D, G>::P, NT = K2Cfg<T, D, G>::NT;
  dim3 grid(s.T / P * s.Hkv * s.B);
  if (s.topk - 2 <= 16)
    hipLaunchKernelGGL((cmp_select_kernel<T, D, G, 16>), grid, dim3(NT), 0, st, s, (const T*)q,
                       (const T*)kc, (const T*)kcl, (const T*)vct, (T*)o_cmp, lse_cmp,
                       indices, do_topk ? 1 : 0);
  else
    hipLaunchKernelGGL((cmp_select_kernel<T, D, G, 32>), grid, dim3(NT), 0, st, s, (const T*)q,
                       (const T*)kc, (const T*)kcl, (const T*)vct, (T*)o_cmp, lse_cmp,
                       indices, do_topk ? 1 : 0);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_cs_g(const Shape& s, const void* q, const void* kc, const void* kcl,
                              const void* vct, void* o_cmp, float* lse_cmp,
                              int32_t* indices, bool do_topk, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_cs<T, D, 1>(s, q, kc, kcl, vct, o_cmp, lse_cmp, indices, do_topk, st);
    case 2: return launch_cs<T, D, 2>(s, q, kc, kcl, vct, o_cmp, lse_cmp, indices, do_topk, st);
    case 4: return launch_cs<T, D, 4>(s, q, kc, kcl, vct, o_cmp, lse_cmp, indices, do_topk, st);
    case 8: return launch_cs<T, D, 8>(s, q, kc, kcl, vct, o_cmp, lse_cmp, indices, do_topk, st);
    default: return launch_cs<T, D, 16>(s, q, kc, kcl, vct, o_cmp, lse_cmp, indices, do_topk, st);
  }
}

hipError_t launch_cmp_select(bool is_bf16, const Shape& s, const void* q, const void* kc,
                             const void* kc_lo, const void* vct, void* o_cmp, float* lse_cmp,
                             int32_t* indices, bool do_topk, hipStream_t st) {
  if (is_bf16) {
    if (s.D == 64)
      return launch_cs_g<bf16, 64>(s, q, kc, kc_lo, vct, o_cmp, lse_cmp, indices, do_topk, st);
    return launch_cs_g<bf16, 128>(s, q, kc, kc_lo, vct, o_cmp, lse_cmp, indices, do_topk, st);
  }
  return launch_cs_g<float, 64>(s, q, kc, nullptr, vct, o_cmp, lse_cmp, indices, do_topk, st);
}

}  // namespace nsa
