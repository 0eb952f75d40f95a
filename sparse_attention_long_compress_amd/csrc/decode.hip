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
// fp32 caches: one workgroup (4 waves) per (sequence b, KV group g), G query
// heads (the bf16 kernel further below does the same on MFMA tiles):
//   1. Q of the G heads into LDS (fp32);
//   2. compressed scores, one pooled key per thread; per-head log-sum-exp;
//      probabilities; o_cmp per (head, channel); importance per block;
//   3. top-k by wave 0 (topk_wave: radix select over unique keys made of the
//      importance bits and the inverted block index);
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

__host__ __device__ inline int al4(int x) { return (x + 3) & ~3; }  // 16-byte multiple

__host__ __device__ inline DecLds dec_lds(int G, int D, int es, int NW, int ncap, int topk,
                                          int wmax_blocks) {
  DecLds o;
  o.qs = 0;
  const int r0 = G * D;
  // phase A: scores / probabilities [G][ncap] and importance [ncap]
  o.sc = r0;
  o.imp = al4(r0 + G * ncap);  // 16-byte aligned: the top-k reads it four at a time
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

// Radix select over PER key slots per lane (empty slots hold 0): writes the
// chosen candidates (keys >= the m-th largest) to selv[1 ..] in ascending
// block order (slot i of lane l is block 1 + l + 64 i) and returns 1 + m.
template <int PER>
__device__ __forceinline__ int radix_pick(const float* imp, int ncand, int m, int l, int* selv) {
  unsigned long long key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = 1 + l + i * kWave;
    key[i] = j <= ncand ? ((unsigned long long)__float_as_uint(imp[j]) << 10) | (unsigned)(1023 - j) : 0ull;
  }
  // every trial has a bit set, so the empty slots (0) never count
  unsigned long long prefix = 0ull;
  for (int bit = 41; bit >= 0; --bit) {
    const unsigned long long trial = prefix | (1ull << bit);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) cnt += __popcll(__builtin_amdgcn_ballot_w64(key[i] >= trial));
    if (cnt >= m) prefix = trial;
  }
  // exactly m keys are >= prefix (the keys are unique, prefix >= 1)
  const unsigned long long below = l == 0 ? 0ull : (~0ull >> (kWave - l));
  int base = 1;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const bool ch = key[i] >= prefix;
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(ch);
    if (ch) selv[base + __popcll(bal & below)] = 1 + l + i * kWave;
    base += __popcll(bal);
  }
  return base;
}


// Top-k of one (sequence, group), run by one wave (lane l): the forced blocks
// 0 and own, then the m_free largest importances among blocks 1 .. own-1
// (ties to the lower index), or every candidate when there are no more than
// m_free.  selv[] receives the blocks in ascending order and *nsel their
// count.
//
// Candidate j gets the key (fp32 importance bits << 10) | (1023 - j): keys
// are unique, a larger key is a higher importance or an equal one at a lower
// index (the importances are sums of exponentials, never negative, so their
// bit patterns order like their values), and every candidate's key is >= 1.
// The m_free-th largest key is found bit by bit from the top (radix select:
// keep a bit when at least m_free keys reach the prefix with it set), with
// one 64-bit compare and a ballot count per key slot and bit; the chosen
// candidates are the keys at or above it, placed in ascending block order by
// ballot prefix counts.
__device__ void topk_wave(const float* imp, int own, int topk, bool need_topk, int l, int* selv,
                          int* nsel) {
  const int ncand = max(own - 1, 0);              // candidates 1 .. own-1
  const int m_free = topk - (own == 0 ? 1 : 2);
  if (!need_topk || ncand > m_free) {
    // block 0 first, the own block last (every candidate lies between)
    int n = 1;
    if (l == 0) selv[0] = 0;
    if (need_topk && m_free > 0) {
      // key slots per lane: ncand <= 1022 (caches of at most 65536 positions)
      if (ncand <= 2 * kWave) n = radix_pick<2>(imp, ncand, m_free, l, selv);
      else if (ncand <= 4 * kWave) n = radix_pick<4>(imp, ncand, m_free, l, selv);
      else if (ncand <= 8 * kWave) n = radix_pick<8>(imp, ncand, m_free, l, selv);
      else n = radix_pick<16>(imp, ncand, m_free, l, selv);
    }
    if (l == 0 && own > 0) selv[n] = own;
    if (l == 0) *nsel = n + (own > 0 ? 1 : 0);
    return;
  }
  // every candidate is taken: 0, 1 .. own-1, own
  for (int j = l; j <= own; j += kWave) selv[j] = j;
  if (l == 0) *nsel = own + 1;
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
  if (w == 0) topk_wave(imp, own, topk, need_topk, l, selv, nsel);
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


// ---------------------------------------------------------------------------
// bf16: the same step on 16x16x32 MFMA tiles.  Per 64-key block a wave
// computes S^T = K Q^T (16 keys x 16 head columns per tile; the G query
// heads of the group fill the first G columns, the rest are zero) and then
// O^T += V^T P^T for each branch (16 channels x 16 head columns per tile).
// The keys of the four score tiles are permuted (dkey) so that a lane's four
// scores of tiles 2h and 2h+1 are the eight consecutive keys 32h + 8a ..
// +7 that the P V step contracts in its k step h: the bf16 probabilities
// become the P^T operand without any lane exchange, and each head's running
// maximum, sum and output live in the lanes of its column.  The V rows are
// transposed through a per-wave LDS tile (64 keys per channel row).
//
// Work split: wave 0 computes the compressed scores (pooled keys in chunks
// of 64, the same score tiles), their log-sum-exp, the importance and the
// top-k while the other waves walk the window's blocks (the own block and
// block 0, which are always selected, also feed the selection branch there);
// after one barrier all waves walk the remaining selected blocks and wave 0
// also the compressed output (P V over the pooled values).
namespace {
template <int D>
struct DecM {
  static constexpr int KS = D / 32;       // k steps of Q K
  static constexpr int MT = D / 16;       // channel tiles of P V
  static constexpr int VST = kBlock + 8;  // elements per channel row of a V^T tile
  static constexpr int VQ = D / 32;       // (key quad, 8-channel chunk) units per lane
};

struct DecMLds {
  // float offsets into the dynamic LDS block
  int vt, mrg, ml, sc, imp, ocmp, ints, total_floats;
};

__host__ __device__ inline DecMLds dec_mfma_lds(int G, int D, int NW, int ncap) {
  DecMLds o;
  const int vt_f = NW * D * (kBlock + 8) / 2;  // per-wave bf16 V^T tiles [D][VST]
  const int mrg_f = NW * 2 * G * D;            // per-wave partial outputs [NW][2][G][D]
  const int ml_f = NW * 2 * G * 2;             // their (max, sum) [NW][2][G][2]
  o.vt = 0;
  o.mrg = 0;  // the merge reuses the tiles after the last block
  o.ml = mrg_f;
  const int end = al4(vt_f > mrg_f + ml_f ? vt_f : mrg_f + ml_f);
  o.sc = end;                       // scaled compressed scores [G][ncap]
  o.imp = al4(o.sc + G * ncap);     // importance [ncap]
  o.ocmp = al4(o.imp + ncap);       // normalised o_cmp [G][D]
  o.ints = al4(o.ocmp + G * D);     // selv [32], nsel, blist [32], nbl
  o.total_floats = o.ints + 66;
  return o;
}

// Waves per workgroup of the bf16 kernel.  Head dim 64: eight (wave 0 on the
// compressed scores, seven on the window's up to nine blocks).  Head dim 128:
// six when their V^T tiles and the per-cache score arrays fit in 160 KB of
// LDS, else four; six walk the window in two rounds instead of three
// (4 -> 6 waves: 44.0 -> 42.2 us per step at 64 sequences x 8192, Hkv 4, G 4;
// 10, 12 or 16 waves at head dim 64 were slower than 8).
inline int dec_mfma_waves(int G, int D, int ncap) {
  if (D == 64) return 8;
  return dec_mfma_lds(G, D, 6, ncap).total_floats * 4 <= 160 * 1024 ? 6 : 4;
}

// row of score tile u (0..3) at tile row i (0..15) -> key within the block
__device__ __forceinline__ int dkey(int u, int i) {
  return 32 * (u >> 1) + 8 * (i >> 2) + 4 * (u & 1) + (i & 3);
}

__device__ __forceinline__ unsigned pack_bf16x2(bf16 lo, bf16 hi) {
  return (unsigned)__builtin_bit_cast(unsigned short, lo) |
         ((unsigned)__builtin_bit_cast(unsigned short, hi) << 16);
}

// hand-off of LDS data between the lanes of one wave: the wave's LDS
// accesses execute in program order, so only the compiler must be kept from
// moving accesses across this point
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}
}  // namespace

template <int D, int G, int NW>
__global__ __launch_bounds__(NW * kWave) void decode_mfma_kernel(Shape s, DecodeArgs a) {
  typedef bf16 T;
  constexpr int NT = NW * kWave, KS = DecM<D>::KS, MT = DecM<D>::MT;
  constexpr int VST = DecM<D>::VST, VQ = DecM<D>::VQ;
  static_assert(G <= 16, "the heads of a group fill at most one 16-column tile");
  const float NINF = -__builtin_inff();
  const int bg = blockIdx.x;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave), l = tid % kWave;
  const int col = l & 15, a4 = l >> 4;
  const int Lmax = s.T, ncap = Lmax / kBlock;
  const int L = min(max(a.lens[b], 1), Lmax);  // lengths outside [1, Lmax] are clamped
  const int t = L - 1, own = t / kBlock, nc = L / kBlock;
  const float c1 = s.scale * kLog2e;
  const bool sel_on = !(s.flags & 2u), cmp_on = !(s.flags & 1u), win_on = !(s.flags & 4u);
  const bool need_topk = sel_on || a.indices != nullptr;
  const bool need_cmp = cmp_on || need_topk;
  const int topk = s.topk, W = s.W;
  const int jw_lo = win_on ? max(0, t - W + 1) / kBlock : own + 1;
  const DecMLds lay = dec_mfma_lds(G, D, NW, ncap);

  extern __shared__ __align__(16) float sm[];
  T* vt = reinterpret_cast<T*>(sm + lay.vt) + (size_t)w * D * VST;  // this wave's V^T tile
  float* sc = sm + lay.sc;
  float* imp = sm + lay.imp;
  float* ocmp = sm + lay.ocmp;
  int* ints = reinterpret_cast<int*>(sm + lay.ints);
  int* selv = ints;       // [32]
  int* nsel = ints + 32;  // [1]
  int* blist = ints + 33; // [32]
  int* nbl = ints + 65;   // [1]

  const size_t row = (size_t)s.Hkv * D;  // elements between consecutive positions
  const T* kc = (const T*)a.kcache + (size_t)b * Lmax * row + (size_t)g * D;
  const T* vc = (const T*)a.vcache + (size_t)b * Lmax * row + (size_t)g * D;
  const T* kp = (const T*)a.kcmp + (size_t)b * ncap * row + (size_t)g * D;
  const T* vp = (const T*)a.vcmp + (size_t)b * ncap * row + (size_t)g * D;

  // Q^T as the B operand: lane (column col, group a4) holds Q[col][32 ks + 8 a4 ..]
  const T* q = (const T*)a.q + ((size_t)b * s.Hq + (size_t)g * G) * D;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = col < G ? Frag<T>::load(q + (size_t)col * D + 32 * ks + 8 * a4) : Frag<T>::zero();

  // per branch (0: selection, 1: window): running maximum (log2 units) and
  // this lane's part of the sum, per head column; O^T tiles (lane: channels
  // 16 mt + 4 a4 + r of head col)
  float m[2], ls[2];
  f32x4 acc[2][MT];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    m[br] = NINF;
    ls[br] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[br][mt] = zero4();
  }

  // ---- pieces of one 64-key block
  // loads of the block's V rows (unit: key quad l % 16, chunk (l / 16) + 4 v)
  auto load_v = [&](bf16x8 (&vr)[VQ][4], const T* vb, int kvalid) {
#pragma unroll
    for (int v = 0; v < VQ; ++v)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = 4 * col + kk;
        vr[v][kk] = key < kvalid ? Frag<T>::load(vb + (size_t)key * row + 8 * (a4 + 4 * v)) : Frag<T>::zero();
      }
  };
  // loads of K as the A operand of the four score tiles
  auto load_k = [&](bf16x8 (&kf)[4][KS], const T* kb, int kvalid) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int key = dkey(u, col);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[u][ks] = key < kvalid ? Frag<T>::load(kb + (size_t)key * row + 32 * ks + 8 * a4) : Frag<T>::zero();
    }
  };
  // scaled scores: x[u][r] for key dkey(u, 4 a4 + r), head col (log2 units)
  auto scores = [&](f32x4 (&x)[4], const bf16x8 (&kf)[4][KS]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f32x4 c = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) c = mma(c, kf[u][ks], qf[ks]);
      x[u] = c * c1;
    }
  };
  // V^T tile: channel row 8 c + e, keys 4 quad .. 4 quad + 3 in one 8-byte
  // store; then the tile is read back by other lanes of the wave
  auto stage_vt = [&](const bf16x8 (&vr)[VQ][4]) {
#pragma unroll
    for (int v = 0; v < VQ; ++v) {
      const int c = a4 + 4 * v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint2 pr;
        pr.x = pack_bf16x2(vr[v][0][e], vr[v][1][e]);
        pr.y = pack_bf16x2(vr[v][2][e], vr[v][3][e]);
        *reinterpret_cast<uint2*>(vt + (8 * c + e) * VST + 4 * col) = pr;
      }
    }
    wave_lds_sync();
  };
  // O^T += V^T P^T from the staged tile: lane (channel 16 mt + col, group a4)
  // holds keys 32 h + 8 a4 .. +7 of the A operand; pf[h] is the P^T operand
  auto pv = [&](f32x4 (&o)[MT], const bf16x8 (&pf)[2], float al) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 c = o[mt] * al;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        c = mma(c, *reinterpret_cast<const bf16x8*>(vt + (16 * mt + col) * VST + 32 * h + 8 * a4), pf[h]);
      o[mt] = c;
    }
  };
  // one key block of the selection (br 0) and / or window (br 1) branch;
  // keys with block index >= kvalid are not read, window keys are those at
  // block index >= wkey0
  auto attend_block = [&](const T* kb, const T* vb, int kvalid, int wkey0, bool do_s, bool do_w) {
    bf16x8 vr[VQ][4];
    bf16x8 kf[4][KS];
    load_v(vr, vb, kvalid);
    load_k(kf, kb, kvalid);
    f32x4 x[4];
    scores(x, kf);
    stage_vt(vr);
#pragma unroll
    for (int br = 0; br < 2; ++br) {
      if (br == 0 ? !do_s : !do_w) continue;
      const int klo = br == 0 ? 0 : wkey0;  // first key of the branch in this block
      float bm = NINF;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kidx = dkey(u, 4 * a4 + r);
          if (kidx < kvalid && kidx >= klo) bm = fmaxf(bm, x[u][r]);
        }
      bm = xmax4(bm);
      const float mn = fmaxf(m[br], bm);
      const float al = m[br] == NINF ? 0.f : fast_exp2(m[br] - mn);
      // probabilities straight into the P^T operand of k step u / 2,
      // element 4 (u % 2) + r
      bf16x8 pf[2];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kidx = dkey(u, 4 * a4 + r);
          const float pvl = (kidx < kvalid && kidx >= klo) ? fast_exp2(x[u][r] - mn) : 0.f;
          psum += pvl;
          pf[u >> 1][4 * (u & 1) + r] = (bf16)pvl;
        }
      ls[br] = ls[br] * al + psum;
      m[br] = mn;
      pv(acc[br], pf, al);
    }
    wave_lds_sync();  // tile reads done before the next block's stores
  };

  if (!need_cmp && tid == 0) *nbl = 0;

  // ---- window blocks (waves 1 .. NW-1; every wave when wave 0 has no
  // compressed work)
  const int wfirst = need_cmp ? 1 : 0;
  if (win_on && w >= wfirst) {
    for (int j = jw_lo + (w - wfirst); j <= own; j += NW - wfirst) {
      const size_t off = (size_t)j * kBlock * row;
      attend_block(kc + off, vc + off, min(kBlock, t - j * kBlock + 1), t - W + 1 - j * kBlock,
                   sel_on && (j == 0 || j == own), true);
    }
  }

  // ---- wave 0: compressed scores (two chunks of 64 pooled keys in flight
  // at a time), their log-sum-exp per head, the importance, the top-k and the
  // list of selected blocks still to walk.  The compressed output (P V over
  // the pooled values) is left for after the barrier: the top-k does not
  // need it.
  const int nchunk = (nc + kBlock - 1) / kBlock;
  float lse = 0.f;  // per head column, log2 units
  if (w == 0 && need_cmp) {
    float mc = NINF, lc = 0.f;
    auto chunk_stats = [&](const bf16x8 (&kf)[4][KS], int ci) {
      const int kvalid = min(kBlock, nc - ci * kBlock);
      f32x4 x[4];
      scores(x, kf);
      float bm = NINF;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kidx = dkey(u, 4 * a4 + r);
          if (kidx < kvalid) {
            bm = fmaxf(bm, x[u][r]);
            if (col < G) sc[col * ncap + ci * kBlock + kidx] = x[u][r];
          }
        }
      bm = xmax4(bm);
      const float mn = fmaxf(mc, bm);
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (dkey(u, 4 * a4 + r) < kvalid) psum += fast_exp2(x[u][r] - mn);
      lc = (mc == NINF ? 0.f : lc * fast_exp2(mc - mn)) + psum;
      mc = mn;
    };
    for (int ci = 0; ci < nchunk; ci += 2) {
      bf16x8 kA[4][KS], kB[4][KS];
      load_k(kA, kp + (size_t)ci * kBlock * row, min(kBlock, nc - ci * kBlock));
      if (ci + 1 < nchunk) load_k(kB, kp + (size_t)(ci + 1) * kBlock * row, min(kBlock, nc - (ci + 1) * kBlock));
      chunk_stats(kA, ci);
      if (ci + 1 < nchunk) chunk_stats(kB, ci + 1);
    }
    if (nc > 0) {
      lse = mc + __log2f(xsum4(lc));
      float lse_h[G];
#pragma unroll
      for (int h = 0; h < G; ++h)
        lse_h[h] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lse), h));
      wave_lds_sync();  // scores from every lane are in LDS
      for (int j = l; j < nc; j += kWave) {
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) sum += fast_exp2(sc[h * ncap + j] - lse_h[h]);
        imp[j] = sum;
      }
      wave_lds_sync();
    }
    topk_wave(imp, own, topk, need_topk, l, selv, nsel);
    wave_lds_sync();
    const int n = *nsel;
    if (a.indices != nullptr && l < topk) a.indices[((size_t)b * s.Hkv + g) * topk + l] = l < n ? selv[l] : -1;
    {
      // the selected blocks still to walk (block 0 and the own block of the
      // window range were walked above), ascending, compacted by ballot
      const int j = l < n ? selv[l] : 0;
      const bool keep = sel_on && l < n && !(win_on && j >= jw_lo && (j == 0 || j == own));
      const unsigned long long bal = __builtin_amdgcn_ballot_w64(keep);
      const unsigned long long below = l == 0 ? 0ull : (~0ull >> (kWave - l));
      if (keep) blist[__popcll(bal & below)] = j;
      if (l == 0) *nbl = __popcll(bal);
    }
  }
  __syncthreads();

  // ---- the remaining selected blocks, every wave (from the last wave down)
  const int nb = *nbl;
  for (int k = NW - 1 - w; k < nb; k += NW) {
    const int j = blist[k];
    const size_t off = (size_t)j * kBlock * row;
    attend_block(kc + off, vc + off, min(kBlock, t - j * kBlock + 1), 0, true, false);
  }
  // ---- wave 0: the compressed output, o_cmp = sum_j p_j Vc_j with
  // p_j = 2^(score - lse) from the stored scores
  if (w == 0 && cmp_on && nc > 0) {
    f32x4 oc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oc[mt] = zero4();
    for (int ci = 0; ci < nchunk; ++ci) {
      const int kvalid = min(kBlock, nc - ci * kBlock);
      bf16x8 vr[VQ][4];
      load_v(vr, vp + (size_t)ci * kBlock * row, kvalid);
      // P^T operand: lane (head col, group a4), k step h: keys 32 h + 8 a4 + e
      bf16x8 pf[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kidx = 32 * h + 8 * a4 + e;
          const float pvl = (col < G && kidx < kvalid) ? fast_exp2(sc[col * ncap + ci * kBlock + kidx] - lse) : 0.f;
          pf[h][e] = (bf16)pvl;
        }
      stage_vt(vr);
      pv(oc, pf, 1.f);
      wave_lds_sync();
    }
    if (col < G) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(ocmp + col * D + 16 * mt + 4 * a4) = oc[mt];
    }
  }
  __syncthreads();  // all waves past their last use of the V^T tiles

  // ---- combine the waves, gate, write
  float* mrg = sm + lay.mrg;  // [NW][2][G][D]
  float* ml = sm + lay.ml;    // [NW][2][G][2]
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    const float lt = xsum4(ls[br]);
    if (col < G) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *reinterpret_cast<f32x4*>(mrg + ((w * 2 + br) * G + col) * D + 16 * mt + 4 * a4) = acc[br][mt];
      if (a4 == 0) {
        ml[((w * 2 + br) * G + col) * 2 + 0] = m[br];
        ml[((w * 2 + br) * G + col) * 2 + 1] = lt;
      }
    }
  }
  __syncthreads();
  const T* gates = (const T*)a.gates + ((size_t)b * s.Hq + (size_t)g * G) * 3;
  T* out = (T*)a.out + ((size_t)b * s.Hq + (size_t)g * G) * D;
  for (int e = tid; e < G * D; e += NT) {
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
        const float mw = ml[((ww * 2 + br) * G + h) * 2];
        if (mw == NINF) continue;  // this wave saw no key of the branch
        const float sc_w = fast_exp2(mw - M);
        den += sc_w * ml[((ww * 2 + br) * G + h) * 2 + 1];
        num += sc_w * mrg[((ww * 2 + br) * G + h) * D + d];
      }
      res += to_f32(gates[h * 3 + 1 + br]) * (num / den);
    }
    if (cmp_on && nc > 0) res += to_f32(gates[h * 3]) * ocmp[e];
    out[e] = from_f32<T>(res);
  }
}

size_t decode_lds_bytes(bool is_bf16, const Shape& s) {
  const int ncap = s.T / kBlock;
  if (is_bf16) {
    return (size_t)dec_mfma_lds(s.G, s.D, dec_mfma_waves(s.G, s.D, ncap), ncap).total_floats * 4;
  }
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

template <int D, int G, int NW>
static hipError_t launch_dec_mfma_nw(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  const size_t lds = decode_lds_bytes(true, s);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_mfma_kernel<D, G, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_mfma_kernel<D, G, NW>), dim3(s.B * s.Hkv), dim3(NW * kWave), lds, st, s, a);
  return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_dec_mfma(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  if constexpr (D == 64) {
    return launch_dec_mfma_nw<D, G, 8>(s, a, st);
  } else {
    if (dec_mfma_waves(G, D, s.T / kBlock) == 6) return launch_dec_mfma_nw<D, G, 6>(s, a, st);
    return launch_dec_mfma_nw<D, G, 4>(s, a, st);
  }
}

template <int D>
static hipError_t launch_dec_mfma_g(const Shape& s, const DecodeArgs& a, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_dec_mfma<D, 1>(s, a, st);
    case 2: return launch_dec_mfma<D, 2>(s, a, st);
    case 4: return launch_dec_mfma<D, 4>(s, a, st);
    case 8: return launch_dec_mfma<D, 8>(s, a, st);
    default: return launch_dec_mfma<D, 16>(s, a, st);
  }
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
    if (s.D == 64) return launch_dec_mfma_g<64>(s, a, st);
    return launch_dec_mfma_g<128>(s, a, st);
  }
  return launch_dec_g<float, 64>(s, a, st);
}

}  // namespace nsa
