// sel_win.hip -- K3: selection attention + sliding-window attention + gated
// combination, fused in one kernel.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work?: SELECTION
// attends over the original tokens of the selected blocks, SLIDING WINDOW over
// the most recent tokens, and the three branch outputs are mixed by gates.
// [SIC] "Sparsity is Cool", Method: window 512; Key claims: the first block is
// always read.  Reading: one joint softmax over all selected tokens s <= t.
//
// One workgroup per (tile of P positions, KV group g, batch b).  Rows are
// (position, head); each wave owns RW rows as NCG column groups of 16 lane
// slots, and a row never leaves its (group, slot): both branch accumulators
// live in registers (MFMA C layout of O^T: lane = row, registers = channels).
//
// The kernel walks the key blocks 0 .. last (the own block of the tile's last
// position) once.  Each block's K (64 x D) and V^T (D x 64) are staged in LDS
// by the whole workgroup, double-buffered (the next block's global loads are in
// flight while the current one is computed).  For every staged block:
//   window     rows whose window t-W < s <= t meets the block: dense 16-row
//              MFMA tiles, online softmax per row;
//   selection  rows whose position selected the block (block 0, the own block
//              and the top-k picks alike): a wave packs, per MFMA tile, at most
//              one row per lane slot -- the positions sharing a slot are its
//              NCG groups -- so a tile needs no data movement between lanes and
//              each lane adds the tile's O^T into the accumulator of the group
//              its row belongs to.  Probabilities use a fixed per-row reference
//              m_ref = max(tau q.k_t, U - 64) (log2 units) where U (from K2)
//              bounds every logit of the row's candidate blocks: terms never
//              exceed 2^64 and the own key's term never underflows unless
//              U - tau q.k_t > 164; a tile holding such a row first takes the
//              exact maximum over its selected blocks (slower, exact path).
// Results are deterministic (no atomics).  At the end
//   out = g_cmp o_cmp + g_sel acc_sel / l_sel + g_win acc_win / l_win
// rounded once.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

struct SelWinArgs {
  const void* q;
  const void* k;
  const void* vt;
  const void* gates;
  const void* o_cmp;
  const float* ubound;
  const int32_t* indices;
  void* out;
  float* lse;
  void* o_sel;
};

template <typename T, int D, int G>
struct K3Cfg {
  // waves per workgroup and target rows per wave: both accumulators (selection
  // and window, 2 * rows/16 * D/4 fp32 registers per lane) must fit in registers
  static constexpr int NW = (sizeof(T) == 2 && D == 128) ? 8 : 4;
  static constexpr int NT = NW * 64;
  static constexpr int RWT = (sizeof(T) == 2 && D == 128) ? 32 : 64;
  static constexpr int P = (NW * RWT / G) < 128 ? (NW * RWT / G) : 128;  // positions per tile
  static constexpr int R = P * G;                 // rows per tile
  static constexpr int RW = R / NW;               // rows per wave
  static constexpr int NCG = RW / 16;             // column groups per wave (1, 2 or 4)
  static constexpr int NSG = 16 / G;              // lane-slot groups (one position each)
  static constexpr int PW = RW / G;               // positions per wave = NCG * NSG
  static constexpr int KS = D / 32;               // k-steps over the head dim
  static constexpr int MT = D / 16;               // 16-channel tiles
  static constexpr int QST = D + 8;               // LDS row stride (elements), Q and K tiles
  static constexpr int VST = 64 + 8;              // LDS row stride (elements), V^T tile
  static constexpr int KCH = 64 * D * (int)sizeof(T) / 16;  // 16-byte chunks per K block
  static constexpr int CPT = KCH / NT > 0 ? KCH / NT : 1;   // chunks per thread (K and V each)
  static_assert(RW % 16 == 0, "rows per wave");
  static_assert(KCH % NT == 0, "staging split");
};

template <typename T, int D, int G>
static size_t k3_lds_bytes(int topk) {
  typedef K3Cfg<T, D, G> C;
  return sizeof(T) * ((size_t)2 * 64 * C::QST + (size_t)2 * D * C::VST + (size_t)C::R * C::QST) +
         (size_t)C::P * topk * 2 + 16;
}

// 16-byte vector of T
template <typename T> struct V16;
template <> struct V16<bf16> { typedef bf16x8 type; };
template <> struct V16<float> { typedef f32x4 type; };

template <typename T, int D, int G>
__global__ __launch_bounds__((K3Cfg<T, D, G>::NT)) void sel_win_kernel(Shape s, SelWinArgs args) {
  typedef K3Cfg<T, D, G> C;
  constexpr int NT = C::NT, P = C::P, R = C::R, NCG = C::NCG, NSG = C::NSG;
  constexpr int PW = C::PW, KS = C::KS, MT = C::MT, QST = C::QST, VST = C::VST, CPT = C::CPT;
  typedef typename Frag<T>::type FragT;
  typedef typename V16<T>::type Vec;
  constexpr int EPV = 16 / sizeof(T);  // elements per 16-byte vector

  const T* __restrict__ q = (const T*)args.q;
  const T* __restrict__ k = (const T*)args.k;
  const T* __restrict__ vt = (const T*)args.vt;

  const int NTL = (s.T + P - 1) / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, s.B * s.Hkv, NTL, bg, tile);
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int nvalid = min(P, s.T - t0);  // the last tile may be ragged (T % P != 0)
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const int sg = col / G, hh = col % G;  // lane slot -> slot group, head
  const float c1 = s.scale * kLog2e;
  const bool sel_on = !(s.flags & 2u);
  const bool cmp_on = !(s.flags & 1u);
  const bool win_on = !(s.flags & 4u);
  const bool need_sel = sel_on || args.lse != nullptr || args.o_sel != nullptr;
  const int topk = s.topk;

  const size_t k_row = (size_t)s.Hkv * D;
  const T* k_b = k + (size_t)b * s.T * k_row + (size_t)g * D;
  const T* vt_b = vt + ((size_t)b * s.Hkv + g) * (size_t)D * s.T;
  const size_t q_row = (size_t)s.Hq * D;

  extern __shared__ __align__(16) unsigned char smem[];
  T* Kl = reinterpret_cast<T*>(smem);             // [2][64][QST]
  T* Vl = Kl + 2 * 64 * QST;                      // [2][D][VST]
  T* Ql = Vl + 2 * D * VST;                       // [R][QST]
  int16_t* lists = reinterpret_cast<int16_t*>(Ql + (size_t)R * QST);  // [P][topk]
  int* flag = reinterpret_cast<int*>(lists + P * topk);

  // ---------------------------------------------------------------- setup
  // Q tile (rows (p, hh), positions t0 .. t0+P-1) -> LDS
  {
    constexpr int QCH = R * D / EPV;
    for (int i = threadIdx.x; i < QCH; i += NT) {
      const int r = i / (D / EPV), c8 = i % (D / EPV);
      const int p = r / G, h2 = r % G;
      Vec v;
      if (p < nvalid) {
        v = *reinterpret_cast<const Vec*>(q + ((size_t)b * s.T + t0 + p) * q_row +
                                          (size_t)(g * G + h2) * D + c8 * EPV);
      } else {
        for (int e = 0; e < EPV; ++e) v[e] = (T)0.f;
      }
      *reinterpret_cast<Vec*>(Ql + (size_t)r * QST + c8 * EPV) = v;
    }
  }
  if (need_sel) {
    for (int i = threadIdx.x; i < P * topk; i += NT) {
      const int p = i / topk, e = i % topk;
      const int j =
          p < nvalid ? args.indices[(((size_t)b * s.Hkv + g) * s.T + t0 + p) * topk + e] : -1;
      lists[i] = (int16_t)(j < 0 ? 0x7fff : j);  // block indices are < 1024
    }
  }
  if (threadIdx.x == 0) *flag = 0;

  // staging of block j: global -> registers (fetch), registers -> LDS (commit)
  Vec kreg[CPT], vreg[CPT];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = threadIdx.x + i * NT;
      const int kr = ci / (D / EPV), kc = ci % (D / EPV);
      kreg[i] = *reinterpret_cast<const Vec*>(k_b + (size_t)(j * kBlock + kr) * k_row + kc * EPV);
      const int vr = ci / (kBlock / EPV), vc = ci % (kBlock / EPV);
      vreg[i] = *reinterpret_cast<const Vec*>(vt_b + (size_t)vr * s.T + j * kBlock + vc * EPV);
    }
  };
  auto commit = [&](int bf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = threadIdx.x + i * NT;
      const int kr = ci / (D / EPV), kc = ci % (D / EPV);
      *reinterpret_cast<Vec*>(Kl + (size_t)(bf * 64 + kr) * QST + kc * EPV) = kreg[i];
      const int vr = ci / (kBlock / EPV), vc = ci % (kBlock / EPV);
      *reinterpret_cast<Vec*>(Vl + (size_t)(bf * D + vr) * VST + vc * EPV) = vreg[i];
    }
  };

  const int c_last = (t0 + nvalid - 1) / kBlock;
  const int j_win0 = win_on ? max(0, t0 - s.W + 1) / kBlock : c_last + 1;
  const int j_begin = need_sel ? 0 : j_win0;

  __syncthreads();

  // per-lane row bookkeeping: lane slot col, group cg -> position / row
  float m_ref[NCG], l_sel[NCG], m_w[NCG], l_w[NCG];
  int ptr[NCG], nxt[NCG];
  f32x4 acc_sel[NCG][MT], acc_win[NCG][MT];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    m_ref[cg] = 0.f;
    l_sel[cg] = 0.f;
    m_w[cg] = -INFINITY;
    l_w[cg] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { acc_sel[cg][mt] = zero4(); acc_win[cg][mt] = zero4(); }
    const int p = w * PW + cg * NSG + sg;
    ptr[cg] = 0;
    nxt[cg] = need_sel ? lists[p * topk] : 0x7fff;
  }

  auto qfrag = [&](int row, int ks) -> FragT {
    return Frag<T>::load(Ql + (size_t)row * QST + ks * 32 + a * 8);
  };

  // reference maximum per row: tau q.k_t (the own key, always selected), U - 64
  if (need_sel) {
    int any_flag = 0;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const int p = w * PW + cg * NSG + sg;
      if (p >= nvalid) continue;
      const int t = t0 + p, h = g * G + hh;
      const T* krow = k_b + (size_t)t * k_row;
      float d = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FragT qv = qfrag(p * G + hh, ks);
        const FragT kv = Frag<T>::load(krow + ks * 32 + a * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) d += (float)qv[e] * (float)kv[e];
      }
      const float mdiag = xsum4(d) * c1;
      const float ub = args.ubound[((size_t)b * s.Hq + h) * s.T + t];
      m_ref[cg] = fmaxf(mdiag, ub - 64.f);
      any_flag |= (ub - mdiag > 164.f) ? 1 : 0;
    }
    if (any_flag) atomicOr(flag, 1);
  }
  __syncthreads();
  const bool exact_pass = need_sel && (*flag != 0);

  // ------------------------------------------------- exact maxima (rare path)
  if (exact_pass) {
    float m_ex[NCG];
    int eptr[NCG], enx[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) { m_ex[cg] = -INFINITY; eptr[cg] = 0; enx[cg] = nxt[cg]; }
    for (int j = 0; j <= c_last; ++j) {
      fetch(j);
      commit(0);
      __syncthreads();
      int gm = 0;
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        if (enx[cg] == j) {
          gm |= 1 << cg;
          ++eptr[cg];
          const int p = w * PW + cg * NSG + sg;
          enx[cg] = eptr[cg] < topk ? lists[p * topk + eptr[cg]] : 0x7fff;
        }
      }
      const int cnt = __popc(gm);
      for (int tt = 0; __builtin_amdgcn_ballot_w64(tt < cnt) != 0; ++tt) {
        int rem = gm;
        for (int z = 0; z < tt; ++z) rem &= rem - 1;
        const int cgt = rem ? __ffs(rem) - 1 : 0;
        const bool valid = tt < cnt;
        const int p = w * PW + cgt * NSG + sg;
        const int t = t0 + p;
        FragT qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = qfrag(p * G + hh, ks);
        float mx = -INFINITY;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int krow = cc * 32 + 8 * (col / 4) + 4 * u + (col % 4);
            f32x4 st = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              st = mma(st, Frag<T>::load(Kl + (size_t)krow * QST + ks * 32 + a * 8), qf[ks]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * kBlock + cc * 32 + 8 * a + 4 * u + r;
              if (key <= t) mx = fmaxf(mx, st[r] * c1);
            }
          }
        mx = xmax4(mx);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          if (valid && cg == cgt) m_ex[cg] = fmaxf(m_ex[cg], mx);
      }
      __syncthreads();
    }
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) m_ref[cg] = m_ex[cg];
  }

  // ------------------------------------------------------------ main walk
  if (j_begin <= c_last) {
    fetch(j_begin);
    commit(0);
  }
  __syncthreads();
  for (int j = j_begin; j <= c_last; ++j) {
    const int bf = (j - j_begin) & 1;
    const bool more = j < c_last;
    if (more) fetch(j + 1);
    const T* Kb = Kl + (size_t)bf * 64 * QST;
    const T* Vb = Vl + (size_t)bf * D * VST;

    // ---------------- window: dense tiles over this wave's rows
    if (j >= j_win0) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const int p = w * PW + cg * NSG + sg;
        const int t = t0 + p;
        if (__builtin_amdgcn_ballot_w64(j * kBlock <= t && j * kBlock + kBlock - 1 > t - s.W) == 0)
          continue;  // block outside every window of this column group
        FragT qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = qfrag(p * G + hh, ks);
        float x[2][8];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int krow = cc * 32 + 8 * (col / 4) + 4 * u + (col % 4);
            f32x4 st = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              st = mma(st, Frag<T>::load(Kb + (size_t)krow * QST + ks * 32 + a * 8), qf[ks]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * kBlock + cc * 32 + 8 * a + 4 * u + r;
              x[cc][4 * u + r] = (key <= t && key > t - s.W) ? st[r] * c1 : -INFINITY;
            }
          }
        float mx = x[0][0];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, x[cc][e]);
        mx = xmax4(mx);
        const float mn = fmaxf(m_w[cg], mx);
        float alpha = 1.f, psum = 0.f;
        float pv[2][8];
        if (mn == -INFINITY) {
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[cc][e] = 0.f;
        } else {
          alpha = fast_exp2(m_w[cg] - mn);
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) { pv[cc][e] = fast_exp2(x[cc][e] - mn); psum += pv[cc][e]; }
        }
        l_w[cg] = l_w[cg] * alpha + xsum4(psum);
        m_w[cg] = mn;
        const FragT pf0 = Frag<T>::from_f32(pv[0]);
        const FragT pf1 = Frag<T>::from_f32(pv[1]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const T* vrow = Vb + (size_t)(mt * 16 + col) * VST + 8 * a;
          f32x4 o = acc_win[cg][mt] * alpha;
          o = mma(o, Frag<T>::load(vrow), pf0);
          acc_win[cg][mt] = mma(o, Frag<T>::load(vrow + 32), pf1);
        }
      }
    }

    // ---------------- selection: slot-packed tiles of the rows that chose j
    if (need_sel) {
      int gm = 0;
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        if (nxt[cg] == j) {
          gm |= 1 << cg;
          ++ptr[cg];
          const int p = w * PW + cg * NSG + sg;
          nxt[cg] = ptr[cg] < topk ? lists[p * topk + ptr[cg]] : 0x7fff;
        }
      }
      const int cnt = __popc(gm);
      for (int tt = 0; __builtin_amdgcn_ballot_w64(tt < cnt) != 0; ++tt) {
        int rem = gm;
        for (int z = 0; z < tt; ++z) rem &= rem - 1;
        const int cgt = rem ? __ffs(rem) - 1 : 0;
        const bool valid = tt < cnt;
        const int p = w * PW + cgt * NSG + sg;
        const int t = t0 + p;
        float mr = m_ref[0];
#pragma unroll
        for (int cg = 1; cg < NCG; ++cg) mr = (cg == cgt) ? m_ref[cg] : mr;
        FragT qf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = qfrag(p * G + hh, ks);
        float pv[2][8];
        float psum = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int krow = cc * 32 + 8 * (col / 4) + 4 * u + (col % 4);
            f32x4 st = zero4();
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              st = mma(st, Frag<T>::load(Kb + (size_t)krow * QST + ks * 32 + a * 8), qf[ks]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int key = j * kBlock + cc * 32 + 8 * a + 4 * u + r;
              const float e = (valid && key <= t) ? fast_exp2(st[r] * c1 - mr) : 0.f;
              pv[cc][4 * u + r] = e;
              psum += e;
            }
          }
        psum = xsum4(psum);
        const FragT pf0 = Frag<T>::from_f32(pv[0]);
        const FragT pf1 = Frag<T>::from_f32(pv[1]);
        float msk[NCG];
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          msk[cg] = (valid && cg == cgt) ? 1.f : 0.f;
          l_sel[cg] += msk[cg] * psum;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const T* vrow = Vb + (size_t)(mt * 16 + col) * VST + 8 * a;
          f32x4 o = zero4();
          o = mma(o, Frag<T>::load(vrow), pf0);
          o = mma(o, Frag<T>::load(vrow + 32), pf1);
#pragma unroll
          for (int cg = 0; cg < NCG; ++cg) acc_sel[cg][mt] += o * msk[cg];
        }
      }
    }

    // the other buffer held block j - 1, which every wave finished before the
    // barrier that ended the previous iteration
    if (more) commit(bf ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------ combine
  const T* gates = (const T*)args.gates;
  T* out = (T*)args.out;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int p = w * PW + cg * NSG + sg;
    if (p >= nvalid) continue;
    const int t = t0 + p, h = g * G + hh;
    const T* grow = gates + (((size_t)b * s.T + t) * s.Hq + h) * 3;
    const float gc = cmp_on ? to_f32(grow[0]) : 0.f;
    const float gs = sel_on ? to_f32(grow[1]) : 0.f;
    const float gw = win_on ? to_f32(grow[2]) : 0.f;
    const float iw = win_on ? gw / l_w[cg] : 0.f;
    const float il = need_sel ? 1.f / l_sel[cg] : 0.f;
    const size_t obase = ((size_t)b * s.T + t) * q_row + (size_t)h * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int d0 = mt * 16 + 4 * a;
      f32x4 res = acc_win[cg][mt] * iw;
      if (need_sel) {
        const f32x4 os = acc_sel[cg][mt] * il;
        if (sel_on) res += os * gs;
        if (args.o_sel) store4((T*)args.o_sel + obase + d0, os);
      }
      if (cmp_on && t >= kBlock - 1) res += load4((const T*)args.o_cmp + obase + d0) * gc;
      store4(out + obase + d0, res);
    }
    if (args.lse && a == 0)
      args.lse[((size_t)b * s.Hq + h) * s.T + t] = (m_ref[cg] + __log2f(l_sel[cg])) * kLn2;
  }
}

template <typename T, int D, int G>
static hipError_t launch_sw(const Shape& s, const SelWinArgs& args, hipStream_t st) {
  typedef K3Cfg<T, D, G> C;
  const size_t lds = k3_lds_bytes<T, D, G>(s.topk);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)sel_win_kernel<T, D, G>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((s.T + C::P - 1) / C::P * s.Hkv * s.B);
  hipLaunchKernelGGL((sel_win_kernel<T, D, G>), grid, dim3(C::NT), lds, st, s, args);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_sw_g(const Shape& s, const SelWinArgs& a, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_sw<T, D, 1>(s, a, st);
    case 2: return launch_sw<T, D, 2>(s, a, st);
    case 4: return launch_sw<T, D, 4>(s, a, st);
    case 8: return launch_sw<T, D, 8>(s, a, st);
    default: return launch_sw<T, D, 16>(s, a, st);
  }
}

hipError_t launch_sel_win(bool is_bf16, const Shape& s, const void* q, const void* k,
                          const void* vt, const void* gates, const void* o_cmp,
                          const float* ubound, const int32_t* indices, void* out, float* lse,
                          void* o_sel, hipStream_t st) {
  SelWinArgs a{q, k, vt, gates, o_cmp, ubound, indices, out, lse, o_sel};
  if (is_bf16) {
    if (s.D == 64) return launch_sw_g<bf16, 64>(s, a, st);
    return launch_sw_g<bf16, 128>(s, a, st);
  }
  return launch_sw_g<float, 64>(s, a, st);  // fp32 is supported at head_dim 64 only
}

}  // namespace nsa
