// sel_win.hip -- K3: selection attention + sliding-window attention + gated
// combination, fused in one kernel.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work?: SELECTION
// attends over the original tokens of the selected blocks, SLIDING WINDOW over
// the most recent tokens, and the three branch outputs are mixed by gates.
// [SIC] "Sparsity is Cool", Method: window 512; Key claims: the first block is
// always read.  Reading: one joint softmax over all selected tokens s <= t.
//
// Work decomposition.  One workgroup per (tile of P positions, KV group g,
// batch b); eight waves.  A row is one (position, head).  A column group is 16
// rows: 16/G consecutive positions times the G heads of the group, i.e. one
// MFMA column tile.  Each wave owns NCG column groups for the whole kernel:
// their Q fragments and both branch accumulators (MFMA C layout of O^T: lane =
// row, registers = channels) stay in registers.
//
// One reference per row for both softmaxes.  Every logit of row (t, h) obeys
//   tau q.k_s * log2(e) <= U = tau log2(e) |q| max_s |k_s|      (Cauchy-Schwarz)
// with the maximum over the keys of blocks 0 .. own (K1 stores each block's
// largest key norm).  Both branches subtract m = max(tau log2(e) q.k_t, U - 64)
// (log2 units): no term exceeds 2^64 and the own key -- attended by both
// branches -- keeps a term >= 2^-100 unless U - tau log2(e) q.k_t > 164.  A
// wave holding such a row first takes the exact maxima, one per branch, over
// the keys each branch attends (slower path, rare).  Because the reference is
// fixed, the accumulation over blocks is a plain sum: a block's QK^T product
// and its exponentials serve both branches, and rows that do not attend a
// block get a reference of +inf (probability exactly 0) instead of a mask.
//
// Key blocks j = first .. own(last position) are walked once.  Each block's
// image -- its K (64 x D) and V^T (D x 64) in MFMA fragment order, written by
// the pooling kernel (KvImage) -- is copied global -> LDS with contiguous 1 KB
// global_load_lds pieces (no register staging; fragment reads from LDS are
// contiguous 16 bytes per lane, so bank-conflict free) through a ring of two
// groups of GB blocks: the next group's loads are in flight while a group is
// computed, with one barrier per group.  A wave skips a block's math when none
// of its column groups attends it.  The key order inside the image makes the C layout of S^T the
// B-operand layout of P^T (no data movement between QK^T and PV).
// Results are deterministic (no atomics).  At the end
//   out = g_cmp o_cmp + g_sel acc_sel / l_sel + g_win acc_win / l_win
// rounded once.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

// Per-shape tuning (waves per workgroup, column groups per wave, K / V^T
// fragments per LDS read batch): overridable for experiments.
#ifndef NSA_K3_W64
#define NSA_K3_W64 16
#endif
#ifndef NSA_K3_NCG64
#define NSA_K3_NCG64 1
#endif
#ifndef NSA_K3_FCH64
#define NSA_K3_FCH64 2
#endif
#ifndef NSA_K3_W128
#define NSA_K3_W128 12
#endif
#ifndef NSA_K3_NCG128
#define NSA_K3_NCG128 1
#endif
#ifndef NSA_K3_FCH128
#define NSA_K3_FCH128 2
#endif
// (one query head per KV group: the column group is 16 positions, and wider
// read batches measured faster at sequence 8192)
#ifndef NSA_K3_FCH128_G1
#define NSA_K3_FCH128_G1 4
#endif
// packed selection items for the shapes sel_compact.hip covers (0: general kernel)
#ifndef NSA_K3_COMPACT
#define NSA_K3_COMPACT 1
#endif
// LDS budget of the staging ring (bytes); the ring takes as many stages as fit
#ifndef NSA_K3_RING_BYTES
#define NSA_K3_RING_BYTES (144 * 1024)
#endif

namespace nsa {

template <typename T, int D, int G>
struct K3Cfg {
  static constexpr bool WIDE = D == 128 || sizeof(T) == 4;
  static constexpr int NW = WIDE ? NSA_K3_W128 : NSA_K3_W64;  // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int WGPC = NW >= 8 ? 1 : 8 / NW;  // workgroups per CU aimed at (launch bound)
  // column groups per wave: more share every K / V^T fragment read but cost
  // registers (occupancy)
  static constexpr int NCG = WIDE ? NSA_K3_NCG128 : NSA_K3_NCG64;
  static constexpr int NSG = 16 / G;              // positions per column group
  static constexpr int PW = NCG * NSG;            // positions per wave
  static constexpr int P = NW * PW;               // positions per workgroup
  static constexpr int KS = D / 32;               // 32-element k steps over the head dim
  static constexpr int MT = D / 16;               // 16-channel output tiles
  typedef KvImage<T, D> Img;
  static constexpr int NV = Img::NV;              // 16-byte pieces per lane fragment
  static constexpr int EPV = Img::EPV;            // elements per piece and lane
  static constexpr int NFRAG = Img::NFRAG;        // fragments per operand and block (4 KS = 2 MT)
  static constexpr int FCH_ = WIDE ? (G == 1 ? NSA_K3_FCH128_G1 : NSA_K3_FCH128) : NSA_K3_FCH64;
  static constexpr int FCH = (NFRAG < FCH_ ? NFRAG : FCH_) / NV;  // fragments per LDS read batch
  static constexpr int FRAG_BYTES = NV * 1024;
  static constexpr int STAGE = Img::BYTES;        // one block's image: K fragments, then V^T
  // blocks per barrier group; the ring holds two groups (about 128 KB)
  static constexpr int GB = (NSA_K3_RING_BYTES / STAGE / 2) < 4 ? (NSA_K3_RING_BYTES / STAGE / 2) : 4;
  static constexpr int NBUF = 2 * GB;
  static_assert(GB >= 1, "ring too small");
  static constexpr int LOADS = 2 * NFRAG * NV;    // 1 KB global->LDS loads per stage
  static_assert(NSG * G == 16, "column group = 16 rows");
};

template <typename T, int D, int G>
static size_t k3_lds_bytes(int topk) {
  typedef K3Cfg<T, D, G> C;
  return (size_t)C::NBUF * C::STAGE + (size_t)C::P * topk * 2;
}

template <typename T, int D, int G>
__global__ __launch_bounds__((K3Cfg<T, D, G>::NT), (K3Cfg<T, D, G>::WGPC)) void sel_win_kernel(Shape s, SelWinArgs args) {
  typedef K3Cfg<T, D, G> C;
  constexpr int NT = C::NT, P = C::P, NCG = C::NCG, NSG = C::NSG, PW = C::PW;
  constexpr int KS = C::KS, MT = C::MT, NV = C::NV, EPV = C::EPV, NFRAG = C::NFRAG, FCH = C::FCH;
  constexpr int FRAG_BYTES = C::FRAG_BYTES, STAGE = C::STAGE, NBUF = C::NBUF, GB = C::GB, LOADS = C::LOADS;
  typedef typename Frag<T>::type FragT;
  typedef typename C::Img Img;
  const float INF = __builtin_inff();

  const T* __restrict__ q = (const T*)args.q;
  const T* __restrict__ k = (const T*)args.k;

  const int NTL = (s.T + P - 1) / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, s.B * s.Hkv, NTL, bg, tile);
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int nvalid = min(P, s.T - t0);  // the last tile may be ragged
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const int sg = col / G, hh = col % G;
  const int h = g * G + hh;
  const float c1 = s.scale * kLog2e;
  const bool sel_on = !(s.flags & 2u);
  const bool cmp_on = !(s.flags & 1u);
  const bool win_on = !(s.flags & 4u);
  const bool need_sel = sel_on || args.lse != nullptr || args.o_sel != nullptr;
  const int topk = s.topk;
  const int W = s.W;

  const size_t k_row = (size_t)s.Hkv * D;
  const T* k_b = k + (size_t)b * s.T * k_row + (size_t)g * D;
  const unsigned char* img_b =
      (const unsigned char*)args.kvimg + ((size_t)b * s.Hkv + g) * s.nc * (size_t)STAGE;
  const size_t q_row = (size_t)s.Hq * D;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;                                          // [NBUF][STAGE]
  int16_t* lists = reinterpret_cast<int16_t*>(smem + (size_t)NBUF * STAGE);  // [P][topk]

  // ------------------------------------------------------------ setup
  if (need_sel) {
    for (int i = threadIdx.x; i < P * topk; i += NT) {
      const int p = i / topk, e = i % topk;
      const int j = p < nvalid ? args.indices[(((size_t)b * s.Hkv + g) * s.T + t0 + p) * topk + e] : -1;
      lists[i] = (int16_t)(j < 0 ? 0x7fff : j);  // block indices are < 1024
    }
  }

  const int c_last = (t0 + nvalid - 1) / kBlock;
  // largest key norm over blocks 0 .. c_last (every wave reduces it itself)
  float mk = 0.f;
  {
    const float* kn = args.knorm + ((size_t)b * s.Hkv + g) * s.nc;
    for (int j = l; j <= c_last; j += kWave) mk = fmaxf(mk, kn[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mk = fmaxf(mk, __shfl_xor(mk, o));
  }

  // per column group: this lane's row
  int tpos[NCG], own[NCG], nxt[NCG], ptr[NCG];
  bool valid[NCG];
  FragT qf[NCG][KS];
  float mr_s[NCG], mr_w[NCG];  // references (log2 units) of the two softmaxes
  bool any_exact = false;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int p0 = w * PW + cg * NSG;
    const int p = p0 + sg;
    tpos[cg] = t0 + p;
    own[cg] = (t0 + p0) / kBlock;  // NSG divides 64: one own block per column group
    valid[cg] = p < nvalid;
    ptr[cg] = 0;
    // every load of the row is issued before the first is used; rows past
    // the ragged end read the last row and are zeroed afterwards
    const int tr = min(tpos[cg], s.T - 1);
    FragT kv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[cg][ks] = Frag<T>::load(q + ((size_t)b * s.T + tr) * q_row + (size_t)h * D + ks * 32 + 8 * a);
      kv[ks] = Frag<T>::load(k_b + (size_t)tr * k_row + ks * 32 + 8 * a);
    }
    float qq = 0.f, d = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (!valid[cg]) qf[cg][ks] = Frag<T>::zero();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qf[cg][ks][e];
        qq += x * x;
        d += x * (float)kv[ks][e];
      }
    }
    qq = xsum4(qq);
    d = xsum4(d);
    const float mdiag = d * c1;
    const float ub = c1 * sqrtf(qq) * mk * (1.0f + 1e-6f);
    const float m = fmaxf(mdiag, ub - 64.f);
    mr_s[cg] = valid[cg] ? m : INF;
    mr_w[cg] = mr_s[cg];
    any_exact |= valid[cg] && (ub - mdiag > 164.f);
  }
  __syncthreads();  // lists visible
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int p = w * PW + cg * NSG + sg;
    nxt[cg] = (need_sel && valid[cg]) ? lists[p * topk] : 0x7fff;
  }
  // Wave-uniform activity of each column group (lanes 0..15 hold its 16 rows):
  //   nsel   next block any of its rows selected (0x7fff: none left);
  //   window blocks jw_lo .. jw_hi meet some row's window; blocks <= jw_edge
  //          hold keys at or below t - W for some row (partial window block).
  int nsel[NCG], jw_lo[NCG], jw_hi[NCG], jw_edge[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    nsel[cg] = __builtin_amdgcn_readfirstlane(row_min16(nxt[cg]));
    const int pf = w * PW + cg * NSG;  // first position of the column group
    const int nv = min(max(nvalid - pf, 0), NSG);
    const int tf = t0 + pf, tl = tf + nv - 1;
    if (win_on && nv > 0) {
      jw_lo[cg] = max(0, tf - W + 1) / kBlock;
      jw_hi[cg] = tf / kBlock;
      jw_edge[cg] = tl >= W ? (tl - W) / kBlock : -1;
    } else {
      jw_lo[cg] = 1;
      jw_hi[cg] = 0;
      jw_edge[cg] = -1;
    }
  }

  // ------------------------------------------ exact maxima (rare; per wave)
  // The wave reads the K fragments straight from global memory; no barriers.
  const bool exact = __builtin_amdgcn_ballot_w64(any_exact) != 0;
  if (exact) {
    float ms[NCG], mw[NCG];
    int ep[NCG], en[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) { ms[cg] = -INF; mw[cg] = -INF; ep[cg] = 0; en[cg] = nxt[cg]; }
    const int jw0 = win_on ? max(0, t0 - W + 1) / kBlock : c_last + 1;
    for (int j = need_sel ? 0 : jw0; j <= c_last; ++j) {
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        const int t = tpos[cg];
        const bool sl = en[cg] == j;
        if (sl) {
          ++ep[cg];
          const int p = w * PW + cg * NSG + sg;
          en[cg] = ep[cg] < topk ? lists[p * topk + ep[cg]] : 0x7fff;
        }
        const bool wl = win_on && valid[cg] && j * kBlock <= t && j * kBlock + kBlock - 1 > t - W;
        if (__builtin_amdgcn_ballot_w64(sl || wl) == 0) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int krow = KvImage<T, D>::krow(u, col);
          f32x4 st = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            st = mma(st, Frag<T>::load(k_b + (size_t)(j * kBlock + krow) * k_row + ks * 32 + 8 * a),
                     qf[cg][ks]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = j * kBlock + key_of(u, a, r);
            const float x = st[r] * c1;
            if (sl && key <= t) ms[cg] = fmaxf(ms[cg], x);
            if (wl && key <= t && key > t - W) mw[cg] = fmaxf(mw[cg], x);
          }
        }
      }
    }
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float a1 = xmax4(ms[cg]), a2 = xmax4(mw[cg]);
      if (valid[cg]) {
        if (need_sel) mr_s[cg] = a1;
        if (win_on) mr_w[cg] = a2;
      }
    }
  }

  // ------------------------------------------------------------ main walk
  const int j_win0 = win_on ? max(0, t0 - W + 1) / kBlock : c_last + 1;
  const int j_begin = need_sel ? 0 : j_win0;
  const int nblk = c_last - j_begin + 1;

  // stage loads of block j's image into ring slot bf; lane l copies its 16
  // bytes of a piece
  // waves 0 .. LOADS / 4 - 1 copy four consecutive 1 KB pieces each (fewer
  // waves spending scalar issue slots on the copies)
  static_assert(LOADS % 4 == 0 && LOADS / 4 <= C::NW, "loader waves");
  auto issue = [&](int j, int bf) {
    if (w < LOADS / 4) {
      unsigned char* stage = ring + (size_t)bf * STAGE + (size_t)w * 4096;
      const unsigned char* src = img_b + (size_t)j * STAGE + (size_t)w * 4096 + 16 * l;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
        __builtin_amdgcn_global_load_lds((const void*)(src + q2 * 1024), (void*)(stage + q2 * 1024), 16, 0, 0);
    }
  };

  float l_s[NCG], l_w[NCG];
  f32x4 acc_s[NCG][MT], acc_w[NCG][MT];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    l_s[cg] = 0.f;
    l_w[cg] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { acc_s[cg][mt] = zero4(); acc_w[cg][mt] = zero4(); }
  }

  // The ring holds two groups of GB blocks: while one group is computed the
  // next one is in flight.  One barrier per group (not per block) lets each
  // wave's uneven per-block work average out over the group.
  const int ngrp = (nblk + GB - 1) / GB;
  auto issue_group = [&](int gi) {
#pragma unroll
    for (int q = 0; q < GB; ++q)
      if (gi * GB + q < nblk) issue(j_begin + gi * GB + q, (gi & 1) * GB + q);
  };
  issue_group(0);

  for (int gi = 0; gi < ngrp; ++gi) {
    wait_vmcnt<0>();       // this wave's loads of group gi (the only ones in flight)
    barrier_keep_loads();  // all of group gi is in LDS; group gi-1's slots are free
    if (gi + 1 < ngrp) issue_group(gi + 1);
  for (int q = 0; q < GB; ++q) {
    const int r = gi * GB + q;
    if (r >= nblk) break;
    const int j = j_begin + r;
    const unsigned char* stage = ring + (size_t)((gi & 1) * GB + q) * STAGE;

    // which rows attend block j: scalar tests per column group, per-lane
    // tests only for the groups that attend it
    bool sl[NCG], wl[NCG], act_s[NCG], act_w[NCG], act[NCG], wlow[NCG];
    bool any = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      act_s[cg] = j == nsel[cg];
      act_w[cg] = j >= jw_lo[cg] && j <= jw_hi[cg];
      wlow[cg] = act_w[cg] && j <= jw_edge[cg];
      act[cg] = act_s[cg] || act_w[cg];
      any |= act[cg];
      sl[cg] = false;
      wl[cg] = false;
      if (act_s[cg]) {
        sl[cg] = nxt[cg] == j;
        if (sl[cg]) {
          ++ptr[cg];
          const int p = w * PW + cg * NSG + sg;
          nxt[cg] = ptr[cg] < topk ? lists[p * topk + ptr[cg]] : 0x7fff;
        }
        nsel[cg] = __builtin_amdgcn_readfirstlane(row_min16(nxt[cg]));
      }
      if (act_w[cg]) {
        const int t = tpos[cg];
        wl[cg] = valid[cg] && j * kBlock <= t && j * kBlock + kBlock - 1 > t - W;
      }
    }
    if (!any) continue;

    // S^T = K Q^T for the active column groups.  The K fragments are read from
    // LDS in chunks of up to 8, all loads of a chunk issued before the first
    // MFMA, and each fragment serves every active column group.
    f32x4 st[NCG][4];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int u = 0; u < 4; ++u) st[cg][u] = zero4();
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
      FragT kf[FCH];
#pragma unroll
      for (int i = 0; i < FCH; ++i) kf[i] = lds_frag<T>(stage + (size_t)(f0 + i) * FRAG_BYTES, l);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        if (!act[cg]) continue;
#pragma unroll
        for (int i = 0; i < FCH; ++i) {
          const int u = Img::k_u(f0 + i), ks = Img::k_ks(f0 + i);
          st[cg][u] = mma(st[cg][u], kf[i], qf[cg][ks]);
        }
      }
    }

    // first chunk of V^T fragments: issued now, in flight during the softmax
    FragT vf0[FCH];
#pragma unroll
    for (int i = 0; i < FCH; ++i) vf0[i] = lds_frag<T>(stage + (size_t)(NFRAG + i) * FRAG_BYTES, l);

    // probabilities, per branch, as PV B fragments (one per 32-key half).
    // Blocks strictly inside every row's range (no causal diagonal, no window
    // edge) take a mask-free path; rows that do not attend get reference +inf.
    FragT ps[NCG][2], pw[NCG][2];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      if (!act[cg]) continue;
      const int t = tpos[cg];
      const bool diag = j == own[cg];
      // after the exact pass the two branches have different references:
      // every block the window attends takes the two-reference path
      const bool dual = exact && act_w[cg];
      if (!diag && !wlow[cg] && !dual) {
        const bool both = act_s[cg] && act_w[cg];
        const bool att = act_s[cg] ? sl[cg] : wl[cg];
        const float mr = (both ? (sl[cg] || wl[cg]) : att) ? mr_s[cg] : INF;  // mr_s == mr_w unless exact
        FragT pf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(st[cg][2 * hf + e / 4][e % 4] * c1 - mr);
          pf[hf] = Frag<T>::from_f32(pv);
        }
        if (both) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            ps[cg][hf] = frag_keep(pf[hf], sl[cg]);
            pw[cg][hf] = frag_keep(pf[hf], wl[cg]);
          }
          l_s[cg] += frag_sum(ps[cg][0]) + frag_sum(ps[cg][1]);
          l_w[cg] += frag_sum(pw[cg][0]) + frag_sum(pw[cg][1]);
        } else if (act_s[cg]) {
          ps[cg][0] = pf[0];
          ps[cg][1] = pf[1];
          l_s[cg] += frag_sum(pf[0]) + frag_sum(pf[1]);
        } else {
          pw[cg][0] = pf[0];
          pw[cg][1] = pf[1];
          l_w[cg] += frag_sum(pf[0]) + frag_sum(pf[1]);
        }
      } else {
        // causal diagonal, window edge, or rows with two exact references
        const float ms = sl[cg] ? mr_s[cg] : INF, mw = wl[cg] ? mr_w[cg] : INF;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8], qw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 2 * hf + e / 4, rr = e % 4;
            const float x = st[cg][u][rr] * c1;
            const int key = j * kBlock + key_of(u, a, rr);
            const bool caus = key <= t;
            pv[e] = caus ? fast_exp2(x - ms) : 0.f;
            qw[e] = (caus && key > t - W) ? fast_exp2(x - mw) : 0.f;
          }
          ps[cg][hf] = Frag<T>::from_f32(pv);
          pw[cg][hf] = Frag<T>::from_f32(qw);
        }
        if (act_s[cg]) l_s[cg] += frag_sum(ps[cg][0]) + frag_sum(ps[cg][1]);
        if (act_w[cg]) l_w[cg] += frag_sum(pw[cg][0]) + frag_sum(pw[cg][1]);
      }
    }

    // O^T += V^T P^T; V^T fragments in chunks as above, each read once
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
      FragT vf[FCH];
#pragma unroll
      for (int i = 0; i < FCH; ++i)
        vf[i] = f0 == 0 ? vf0[i] : lds_frag<T>(stage + (size_t)(NFRAG + f0 + i) * FRAG_BYTES, l);
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) {
        if (act_s[cg]) {
#pragma unroll
          for (int i = 0; i < FCH; ++i) {
            const int mt = Img::v_mt(f0 + i), hf = Img::v_h(f0 + i);
            acc_s[cg][mt] = mma(acc_s[cg][mt], vf[i], ps[cg][hf]);
          }
        }
        if (act_w[cg]) {
#pragma unroll
          for (int i = 0; i < FCH; ++i) {
            const int mt = Img::v_mt(f0 + i), hf = Img::v_h(f0 + i);
            acc_w[cg][mt] = mma(acc_w[cg][mt], vf[i], pw[cg][hf]);
          }
        }
      }
    }
  }
  }

  // ------------------------------------------------------------ combine
  // Gates and the compressed output of every row are loaded before the first
  // store so that the loads overlap; rows past the ragged end read the last
  // row and store nothing.
  const T* gates = (const T*)args.gates;
  T* out = (T*)args.out;
  float g3[NCG][3];
  f32x4 oc[NCG][MT];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int tr = min(tpos[cg], s.T - 1);
    const T* grow = gates + (((size_t)b * s.T + tr) * s.Hq + h) * 3;
#pragma unroll
    for (int e = 0; e < 3; ++e) g3[cg][e] = to_f32(grow[e]);
    const size_t rb = ((size_t)b * s.T + tr) * q_row + (size_t)h * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oc[cg][mt] = load4((const T*)args.o_cmp + rb + mt * 16 + 4 * a);
  }
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const float ls = xsum4(l_s[cg]), lw = xsum4(l_w[cg]);
    if (!valid[cg]) continue;
    const int t = tpos[cg];
    // the compressed branch has no block for the first 63 positions; its
    // buffer is then left unwritten, so it is selected, not scaled by zero
    const bool use_c = cmp_on && t >= kBlock - 1;
    const float gc = g3[cg][0];
    const float gs = sel_on ? g3[cg][1] : 0.f;
    const float gw = win_on ? g3[cg][2] : 0.f;
    const float iw = win_on ? gw / lw : 0.f;
    const float ilw = win_on ? 1.f / lw : 0.f;
    const float il = need_sel ? 1.f / ls : 0.f;
    const size_t obase = ((size_t)b * s.T + t) * q_row + (size_t)h * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int d0 = mt * 16 + 4 * a;
      f32x4 res = acc_w[cg][mt] * iw;
      if (args.o_win) store4((T*)args.o_win + obase + d0, acc_w[cg][mt] * ilw);
      if (need_sel) {
        const f32x4 os = acc_s[cg][mt] * il;
        if (sel_on) res += os * gs;
        if (args.o_sel) store4((T*)args.o_sel + obase + d0, os);
      }
      if (use_c) res += oc[cg][mt] * gc;
      store4(out + obase + d0, res);
    }
    if (args.lse && a == 0) args.lse[((size_t)b * s.Hq + h) * s.T + t] = (mr_s[cg] + __log2f(ls)) * kLn2;
    if (args.lse_win && a == 0)
      args.lse_win[((size_t)b * s.Hq + h) * s.T + t] = win_on ? (mr_w[cg] + __log2f(lw)) * kLn2 : -INF;
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

const char* sel_win_kernel_name(bool is_bf16, const Shape& s) {
  return NSA_K3_COMPACT && sel_compact_eligible(is_bf16, s) ? "sel_compact_kernel" : "sel_win_kernel";
}

hipError_t launch_sel_win(bool is_bf16, const Shape& s, const void* q, const void* k,
                          const void* kvimg, const void* gates, const void* o_cmp,
                          const float* knorm, const int32_t* indices, void* out, float* lse,
                          void* o_sel, float* lse_win, void* o_win, hipStream_t st) {
  SelWinArgs a{q, k, kvimg, gates, o_cmp, knorm, indices, out, lse, o_sel, lse_win, o_win};
  if (NSA_K3_COMPACT && sel_compact_eligible(is_bf16, s)) return launch_sel_compact(s, a, st);
  if (is_bf16) {
    if (s.D == 64) return launch_sw_g<bf16, 64>(s, a, st);
    return launch_sw_g<bf16, 128>(s, a, st);
  }
  return launch_sw_g<float, 64>(s, a, st);  // fp32 is supported at head_dim 64 only
}

}  // namespace nsa
