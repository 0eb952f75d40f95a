// decode.hip -- NSA for one new query position per sequence over a KV cache.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work?: the three
// branches (compression over block summaries, selection of the top blocks by
// the compression scores, sliding window) and their gates; [SIC] "Sparsity is
// Cool", Method: block 64, top-k 16, window 512.  A decode step is the prefill
// computation restricted to the last row: for a sequence of length L whose
// newest key and value are already in the cache, the query sits at
// t = L - 1 and sees the complete blocks j < L / 64 (compression), the blocks
// {0, t / 64} plus the top (k - |forced|) of 1 .. t/64 - 1 by the group-summed
// compressed probabilities (selection, ties to the lower index), and the keys
// t - W < s <= t (window).
//
// One workgroup (4 waves) per (sequence b, KV group g), G query heads:
//   1. Q of the G heads into LDS (fp32);
//   2. compressed scores, one pooled key per thread; per-head log-sum-exp;
//      probabilities; o_cmp per (head, channel); importance per block;
//   3. top-k by wave 0: 64-bit keys (fp32 importance bits above the inverted
//      block index: one unsigned compare orders by score, then lower index),
//      iterated wave maxima;
//   4. the blocks to read: the selected ones below the window, then the
//      window's blocks; the waves take them round-robin.  Per block a lane
//      owns a key for Q K (G dot products against Q in LDS), each branch keeps
//      a running maximum and sum per head (wave-uniform), and the lanes then
//      own channels for P V (the probabilities pass through LDS).  Keys past
//      t are never read;
//   5. the waves' partial results are combined, gated and written.
// The computation is small per sequence; a batch of sequences is bound by the
// HBM reads of the selected and window blocks.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

namespace {
// waves per workgroup: 8 for bf16 at head_dim 64, 4 otherwise (each wave
// stages one 64-key V tile in LDS)
template <typename T, int D>
struct DecCfg {
  static constexpr int NW = (sizeof(T) == 2 && D == 64) ? 8 : 4;
  static constexpr int NT = NW * kWave;
};

struct DecLds {
  // float offsets into the dynamic LDS block
  int qs, sc, imp, lse, vb, mrg, ml, ints, total_floats;
};

__host__ __device__ inline DecLds dec_lds(int G, int D, int es, int NW, int ncap, int topk,
                                          int wmax_blocks) {
  DecLds o;
  o.qs = 0;
  const int r0 = G * D;
  // phase A: scores / probabilities [G][ncap] and importance [ncap]
  o.sc = r0;
  o.imp = r0 + G * ncap;
  const int endA = o.imp + ncap;
  // phase B (same region): per-wave V tiles [NW][64][D] (input type), per-wave
  // partial outputs [NW][2][G][D] and their (max, sum) [NW][2][G][2]
  o.vb = r0;
  o.mrg = o.vb + NW * 64 * D * es / 4;
  o.ml = o.mrg + NW * 2 * G * D;
  const int endB = o.ml + NW * 2 * G * 2;
  o.lse = (endA > endB ? endA : endB);
  o.ints = o.lse + G;
  // ints: selected blocks [32], count, walk list [topk + wmax_blocks], its
  // selection flags [same], count
  o.total_floats = o.ints + 32 + 1 + 2 * (topk + wmax_blocks) + 1;
  return o;
}

// Wave-wide reductions with in-register lane exchanges: DPP within each
// 16-lane row (quad swaps, half-row and row mirrors), then the gfx950
// permlane16 / permlane32 swaps across rows; no LDS crossbar round trips.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  auto dpp = [](float x, int ctrl) -> float {
    switch (ctrl) {
      case 0xB1: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
      case 0x4E: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
      case 0x141: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, true));
      default: return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, true));
    }
  };
  v = op(v, dpp(v, 0xB1));   // lane ^ 1
  v = op(v, dpp(v, 0x4E));   // lane ^ 2
  v = op(v, dpp(v, 0x141));  // the other quad of 8
  v = op(v, dpp(v, 0x140));  // the other half of 16
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
// largest 64-bit key of the wave (the same exchanges on both halves)
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  auto mx = [](unsigned long long x, unsigned long long y) { return x > y ? x : y; };
  auto dpp64 = [](unsigned long long x, int ctrl) -> unsigned long long {
    int lo = (int)(unsigned)x, hi = (int)(unsigned)(x >> 32);
    switch (ctrl) {
      case 0xB1: lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xF, 0xF, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xF, 0xF, true); break;
      case 0x4E: lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xF, 0xF, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xF, 0xF, true); break;
      case 0x141: lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xF, 0xF, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xF, 0xF, true); break;
      default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xF, 0xF, true); hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xF, 0xF, true); break;
    }
    return ((unsigned long long)(unsigned)hi << 32) | (unsigned)lo;
  };
  v = mx(v, dpp64(v, 0xB1));
  v = mx(v, dpp64(v, 0x4E));
  v = mx(v, dpp64(v, 0x141));
  v = mx(v, dpp64(v, 0x140));
  auto swap = [](unsigned long long x, bool p32) -> unsigned long long {
    const unsigned lo = (unsigned)x, hi = (unsigned)(x >> 32);
    if (p32) {
      auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
      auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
      const unsigned long long u = ((unsigned long long)b[0] << 32) | a[0];
      const unsigned long long w = ((unsigned long long)b[1] << 32) | a[1];
      return u > w ? u : w;
    }
    auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const unsigned long long u = ((unsigned long long)b[0] << 32) | a[0];
    const unsigned long long w = ((unsigned long long)b[1] << 32) | a[1];
    return u > w ? u : w;
  };
  v = swap(v, false);
  return swap(v, true);
}
}  // namespace

struct DecodeArgs {
  const void* q;        // [B][Hq][D]
  const void* kcache;   // [B][Lmax][Hkv][D]
  const void* vcache;   // [B][Lmax][Hkv][D]
  const void* kcmp;     // [B][Lmax/64][Hkv][D]
  const void* vcmp;     // [B][Lmax/64][Hkv][D]
  const int32_t* lens;  // [B]
  const void* gates;    // [B][Hq][3]
  void* out;            // [B][Hq][D]
  int32_t* indices;     // [B][Hkv][topk] or null
};

template <typename T, int D, int G>
__global__ __launch_bounds__((DecCfg<T, D>::NT)) void decode_kernel(Shape s, DecodeArgs a) {
  constexpr int NT = DecCfg<T, D>::NT, NW = DecCfg<T, D>::NW;
  typedef typename Frag<T>::type FragT;
  constexpr int CPL = D / kWave;  // channels per lane in P V
  const float NINF = -__builtin_inff();
  const int bg = blockIdx.x;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave;
  const int Lmax = s.T, ncap = Lmax / kBlock;
  const int L = min(max(a.lens[b], 1), Lmax);  // lengths outside [1, Lmax] are clamped
  const int t = L - 1, own = t / kBlock, nc = L / kBlock;
  const float c1 = s.scale * kLog2e;
  const bool sel_on = !(s.flags & 2u), cmp_on = !(s.flags & 1u), win_on = !(s.flags & 4u);
  const bool need_topk = sel_on || a.indices != nullptr;
  const bool need_cmp = cmp_on || need_topk;
  const int topk = s.topk, W = s.W;
  const int jw_lo = win_on ? max(0, t - W + 1) / kBlock : own + 1;
  const int wmax_blocks = (W - 1) / kBlock + 2 < ncap ? (W - 1) / kBlock + 2 : ncap;
  const DecLds lay = dec_lds(G, D, (int)sizeof(T), NW, ncap, topk, wmax_blocks);

  extern __shared__ __align__(16) float sm[];
  float* qs = sm + lay.qs;
  float* sc = sm + lay.sc;
  float* imp = sm + lay.imp;
  float* lse = sm + lay.lse;
  int* ints = reinterpret_cast<int*>(sm + lay.ints);
  int* selv = ints;                 // [32]
  int* nsel = ints + 32;            // [1]
  int* blist = ints + 33;           // [topk + wmax_blocks]
  int* bsel = blist + topk + wmax_blocks;
  int* nbl = bsel + topk + wmax_blocks;

  const T* q = (const T*)a.q + ((size_t)b * s.Hq + (size_t)g * G) * D;
  const size_t row = (size_t)s.Hkv * D;  // elements between consecutive positions
  const T* kc = (const T*)a.kcache + (size_t)b * Lmax * row + (size_t)g * D;
  const T* vc = (const T*)a.vcache + (size_t)b * Lmax * row + (size_t)g * D;
  const T* kp = (const T*)a.kcmp + (size_t)b * ncap * row + (size_t)g * D;
  const T* vp = (const T*)a.vcmp + (size_t)b * ncap * row + (size_t)g * D;

  // ---- 1. Q (fp32) into LDS
  for (int i = tid; i < G * D; i += NT) qs[i] = to_f32(q[i]);
  __syncthreads();

  // dot products of one key row (in 8-element pieces) with the G queries
  auto qk = [&](const T* krow, float (&x)[G]) {
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = 0.f;
#pragma unroll 2
    for (int d0 = 0; d0 < D; d0 += 8) {
      const typename Frag<T>::type kv = Frag<T>::load(krow + d0);
      float kf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[e] = (float)kv[e];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(qs + h * D + d0);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(qs + h * D + d0 + 4);
        x[h] += q0[0] * kf[0] + q0[1] * kf[1] + q0[2] * kf[2] + q0[3] * kf[3] +
                q1[0] * kf[4] + q1[1] * kf[5] + q1[2] * kf[6] + q1[3] * kf[7];
      }
    }
  };

  // ---- 2. compressed attention and block importance
  float ocmp[(G * D + NT - 1) / NT];
#pragma unroll
  for (int i = 0; i < (G * D + NT - 1) / NT; ++i) ocmp[i] = 0.f;
  if (need_cmp && nc > 0) {
    for (int j = tid; j < nc; j += NT) {
      float x[G];
      qk(kp + (size_t)j * row, x);
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h * ncap + j] = x[h] * c1;
    }
    __syncthreads();
    for (int h = w; h < G; h += NW) {  // log-sum-exp per head (log2 units)
      float m = NINF;
      for (int j = l; j < nc; j += kWave) m = fmaxf(m, sc[h * ncap + j]);
      m = wave_max(m);
      float sum = 0.f;
      for (int j = l; j < nc; j += kWave) sum += fast_exp2(sc[h * ncap + j] - m);
      sum = wave_sum(sum);
      if (l == 0) lse[h] = m + __log2f(sum);
    }
    __syncthreads();
    for (int i = tid; i < G * nc; i += NT) {
      const int h = i / nc, j = i % nc;
      sc[h * ncap + j] = fast_exp2(sc[h * ncap + j] - lse[h]);
    }
    __syncthreads();
    for (int j = tid; j < nc; j += NT) {
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) sum += sc[h * ncap + j];
      imp[j] = sum;
    }
    if (cmp_on) {
#pragma unroll
      for (int i = 0; i < (G * D + NT - 1) / NT; ++i) {
        const int e = tid + i * NT;
        if (e < G * D) {
          const int h = e / D, d = e % D;
          float acc = 0.f;
#pragma unroll 32
          for (int j = 0; j < nc; ++j) acc += sc[h * ncap + j] * to_f32(vp[(size_t)j * row + d]);
          ocmp[i] = acc;
        }
      }
    }
    __syncthreads();
  }

  // ---- 3. top-k (wave 0)
  if (w == 0) {
    const int ncand = max(own - 1, 0);              // candidates 1 .. own-1
    const int m_free = topk - (own == 0 ? 1 : 2);
    int n = 0;
    if (l == 0) {
      selv[n++] = 0;
      if (own > 0) selv[n++] = own;
    }
    n = __shfl(n, 0);
    if (need_topk) {
      if (ncand <= m_free) {
        for (int j = 1 + l; j <= ncand; j += kWave) selv[n + j - 1] = j;
        n += ncand;
      } else {
        constexpr int PER = 16;  // candidates per lane (ncand <= 1022)
        unsigned long long key[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int j = 1 + l + i * kWave;
          key[i] = j <= ncand ? ((unsigned long long)__float_as_uint(imp[j]) << 32) | (0xffffffffu - (unsigned)j)
                              : 0ull;
        }
        for (int r = 0; r < m_free; ++r) {
          unsigned long long best = 0ull;
#pragma unroll
          for (int i = 0; i < PER; ++i) best = key[i] > best ? key[i] : best;
          best = wave_max_u64(best);
#pragma unroll
          for (int i = 0; i < PER; ++i)
            if (key[i] == best) key[i] = 0ull;  // keys are unique (the index field)
          if (l == 0) selv[n + r] = (int)(0xffffffffu - (unsigned)best);
        }
        n += m_free;
      }
    }
    // ascending order: lane i < n takes selv[i] and writes it at its rank
    int v = l < n ? selv[l] : 0x7fffffff;
    int rank = 0;
    for (int i = 0; i < n; ++i) rank += __shfl(v, i) < v;
    if (l < n) selv[rank] = v;  // all reads above precede (shuffles of registers)
    if (l == 0) *nsel = n;
  }
  __syncthreads();
  // indices written in ascending order once selv is sorted
  if (a.indices != nullptr && w == 0 && l < topk) {
    const int n = *nsel;
    a.indices[((size_t)b * s.Hkv + g) * topk + l] = l < n ? selv[l] : -1;
  }

  // ---- 4. blocks to read: selected blocks below the window, then the window
  if (tid == 0) {
    const int n = *nsel;
    int k = 0;
    if (need_topk) {
      for (int i = 0; i < n; ++i)
        if (selv[i] < jw_lo) { blist[k] = selv[i]; bsel[k] = 1; ++k; }
    }
    int ip = 0;
    while (ip < n && selv[ip] < jw_lo) ++ip;
    for (int j = jw_lo; j <= own && win_on; ++j) {
      while (ip < n && selv[ip] < j) ++ip;
      blist[k] = j;
      bsel[k] = (ip < n && selv[ip] == j) ? 1 : 0;
      ++k;
    }
    *nbl = k;
  }
  __syncthreads();

  // ---- 5. selection and window attention; wave w takes blocks w, w + NW, ...
  T* vb = reinterpret_cast<T*>(sm + lay.vb) + (size_t)w * 64 * D;  // this wave's V tile [64][D]
  float ms[G], ls[G], mw[G], lw[G];
  float os[G][CPL], ow[G][CPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    ms[h] = NINF; mw[h] = NINF; ls[h] = 0.f; lw[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) { os[h][c] = 0.f; ow[h][c] = 0.f; }
  }
  const bool need_sel = need_topk;  // o_sel is computed whenever the top-k is
  const int nblk = *nbl;
  for (int k = w; k < nblk; k += NW) {
    const int j = blist[k];
    const bool is_sel = need_sel && bsel[k];
    const int key = j * kBlock + l;
    const bool valid = key <= t;
    const bool ins = is_sel && valid;
    const bool inw = win_on && valid && key > t - W;
    // the V row of this lane's key: its 16-byte loads issued first, in
    // flight during Q K
    FragT vr[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i)
      vr[i] = valid ? Frag<T>::load(vc + (size_t)key * row + 8 * i) : Frag<T>::zero();
    float x[G];
    if (valid) {
      qk(kc + (size_t)key * row, x);
    } else {
#pragma unroll
      for (int h = 0; h < G; ++h) x[h] = 0.f;
    }
    // the V row into row l of the wave's tile (zeros past t)
#pragma unroll
    for (int i = 0; i < D / 8; ++i) *reinterpret_cast<FragT*>(vb + l * D + 8 * i) = vr[i];
    const bool any_s = __builtin_amdgcn_ballot_w64(ins) != 0;
    const bool any_w = __builtin_amdgcn_ballot_w64(inw) != 0;
    float ps[G], pw[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float xv = x[h] * c1;
      ps[h] = 0.f;
      pw[h] = 0.f;
      if (any_s) {
        const float bm = wave_max(ins ? xv : NINF);
        const float mn = fmaxf(ms[h], bm);
        const float al = fast_exp2(ms[h] - mn);  // ms = -inf at first: 0
        ls[h] *= al;
#pragma unroll
        for (int c = 0; c < CPL; ++c) os[h][c] *= al;
        ms[h] = mn;
        ps[h] = ins ? fast_exp2(xv - mn) : 0.f;
        ls[h] += wave_sum(ps[h]);
      }
      if (any_w) {
        const float bm = wave_max(inw ? xv : NINF);
        const float mn = fmaxf(mw[h], bm);
        const float al = fast_exp2(mw[h] - mn);
        lw[h] *= al;
#pragma unroll
        for (int c = 0; c < CPL; ++c) ow[h][c] *= al;
        mw[h] = mn;
        pw[h] = inw ? fast_exp2(xv - mn) : 0.f;
        lw[h] += wave_sum(pw[h]);
      }
    }
    // P V: lane l now owns channels l, l + 64, ...; a key's probabilities come
    // from its lane by readlane, its V row from the tile
    const int nk = min(kBlock, t - j * kBlock + 1);
#pragma unroll 4
    for (int kk = 0; kk < nk; ++kk) {
      float vv[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) vv[c] = to_f32(vb[kk * D + l + c * kWave]);
      if (any_s) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ps[h]), kk));
#pragma unroll
          for (int c = 0; c < CPL; ++c) os[h][c] += p1 * vv[c];
        }
      }
      if (any_w) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float p2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pw[h]), kk));
#pragma unroll
          for (int c = 0; c < CPL; ++c) ow[h][c] += p2 * vv[c];
        }
      }
    }
  }
  __syncthreads();  // all waves past their last use of the V tiles

  // ---- 6. combine the waves, gate, write
  float* mrg = sm + lay.mrg;  // [NW][2][G][D]
  float* ml = sm + lay.ml;    // [NW][2][G][2]
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      mrg[((w * 2 + 0) * G + h) * D + l + c * kWave] = os[h][c];
      mrg[((w * 2 + 1) * G + h) * D + l + c * kWave] = ow[h][c];
    }
    if (l == 0) {
      ml[((w * 2 + 0) * G + h) * 2 + 0] = ms[h];
      ml[((w * 2 + 0) * G + h) * 2 + 1] = ls[h];
      ml[((w * 2 + 1) * G + h) * 2 + 0] = mw[h];
      ml[((w * 2 + 1) * G + h) * 2 + 1] = lw[h];
    }
  }
  __syncthreads();
  const T* gates = (const T*)a.gates + ((size_t)b * s.Hq + (size_t)g * G) * 3;
  T* out = (T*)a.out + ((size_t)b * s.Hq + (size_t)g * G) * D;
#pragma unroll
  for (int i = 0; i < (G * D + NT - 1) / NT; ++i) {
    const int e = tid + i * NT;
    if (e >= G * D) break;
    const int h = e / D, d = e % D;
    float res = 0.f;
    for (int br = 0; br < 2; ++br) {
      if (br == 0 && !sel_on) continue;
      if (br == 1 && !win_on) continue;
      float M = NINF;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) M = fmaxf(M, ml[((ww * 2 + br) * G + h) * 2]);
      if (M == NINF) continue;  // no key of this branch (cannot happen for a valid row)
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float sc_w = fast_exp2(ml[((ww * 2 + br) * G + h) * 2] - M);
        den += sc_w * ml[((ww * 2 + br) * G + h) * 2 + 1];
        num += sc_w * mrg[((ww * 2 + br) * G + h) * D + d];
      }
      res += to_f32(gates[h * 3 + 1 + br]) * (num / den);
    }
    if (cmp_on && nc > 0) res += to_f32(gates[h * 3]) * ocmp[i];
    out[e] = from_f32<T>(res);
  }
}

size_t decode_lds_bytes(bool is_bf16, const Shape& s) {
  const int ncap = s.T / kBlock;
  const int wmax = (s.W - 1) / kBlock + 2 < ncap ? (s.W - 1) / kBlock + 2 : ncap;
  const int es = is_bf16 ? 2 : 4;
  const int NW = (is_bf16 && s.D == 64) ? DecCfg<bf16, 64>::NW : DecCfg<float, 64>::NW;
  return (size_t)dec_lds(s.G, s.D, es, NW, ncap, s.topk, wmax).total_floats * 4;
}

template <typename T, int D, int G>
static hipError_t launch_dec(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  const size_t lds = decode_lds_bytes(sizeof(T) == 2, s);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<T, D, G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_kernel<T, D, G>), dim3(s.B * s.Hkv), dim3(DecCfg<T, D>::NT), lds, st, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_dec_g(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_dec<T, D, 1>(s, a, st);
    case 2: return launch_dec<T, D, 2>(s, a, st);
    case 4: return launch_dec<T, D, 4>(s, a, st);
    case 8: return launch_dec<T, D, 8>(s, a, st);
    default: return launch_dec<T, D, 16>(s, a, st);
  }
}

hipError_t launch_decode(bool is_bf16, const Shape& s, const void* q, const void* kcache,
                         const void* vcache, const void* kcmp, const void* vcmp,
                         const int32_t* lens, const void* gates, void* out, int32_t* indices,
                         hipStream_t st) {
  DecodeArgs a{q, kcache, vcache, kcmp, vcmp, lens, gates, out, indices};
  if (is_bf16) {
    if (s.D == 64) return launch_dec_g<bf16, 64>(s, a, st);
    return launch_dec_g<bf16, 128>(s, a, st);
  }
  return launch_dec_g<float, 64>(s, a, st);
}

}  // namespace nsa
