// sel_compact.hip -- K3 for bf16, head_dim 64, four query heads per KV group:
// selection + sliding-window attention + gated combination with the selected
// blocks packed per block.
//
// [DSA] "DeepSeek's Native Sparse Attention", How Does NSA Work?: the heads of
// a GQA group share one block selection per query position, and a selected
// block is attended over its original tokens; the window covers the most
// recent tokens.  [SIC] "Sparsity is Cool", Method: window 512.
//
// Why a second kernel.  An MFMA column tile is 16 rows, so with four heads per
// group one column group is four positions.  Their block selections differ,
// and in the general kernel a column group computes every block that any of
// its four positions chose: with top-k 16 at sequence 8192 about 43% of the
// QK^T / PV columns and exponentials go to rows that did not choose the block.
// Here the selection work is packed instead:
//   * each wave still owns one column group (4 positions x 4 heads) and its
//     register range -- the blocks of the group's sliding window (or only the
//     own block when the window branch is off) -- and handles there, as the
//     general kernel does, the window branch and the selections that fall in
//     the range (one exponential serves both branches);
//   * every other selected block j is an item list: the positions of the tile
//     that chose j, four to an item (16 full columns).  Items go to the waves
//     round-robin in walk order; a wave that takes an item reads the rows' Q
//     from LDS, and adds the item's partial P V and row sums into fp32 row
//     accumulators in LDS (ds_add_f32).
// Both parts use the row's fixed softmax reference (the Cauchy-Schwarz bound
// of the general kernel), so a row's sum over its blocks is a plain sum and
// the order of the additions only changes rounding.
//
// The K / V^T block images are staged global -> LDS as in the general kernel,
// through a ring of four one-block slots with one barrier per block (LDS also
// holds the tile's Q and the row accumulators).  An item's P V and its
// accumulator update are deferred to the next block's period, so that the
// updates of one period all come from one block's items -- their rows are
// distinct -- and need no atomics; the two halves of consecutive items run in
// different waves at the same time.  60 positions per workgroup, 15 waves.
#include <math.h>
#include <stdint.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

namespace {
constexpr int kcNW = 15;               // waves per workgroup
constexpr int kcNT = kcNW * kWave;
constexpr int kcG = 4;                 // query heads per KV group
constexpr int kcNSG = 16 / kcG;        // positions per column group / item
constexpr int kcP = kcNW * kcNSG;      // positions per workgroup
constexpr int kcROWS = kcNW * 16;      // rows (position, head) per workgroup
constexpr int kcD = 64;
constexpr int kcNBUF = 4;              // staging ring: one-block slots
typedef KvImage<bf16, kcD> kcImg;
constexpr int kcSTAGE = kcImg::BYTES;  // 16 KB
constexpr int kcQROW = kcD * 2;        // bytes per Q row in LDS
constexpr int kcMAXR = 32;             // register range of at most 32 blocks (bit set)
// LDS layout
constexpr int kcOFF_Q = kcNBUF * kcSTAGE;               // [ROWS][64] bf16, 16-byte chunks swizzled
constexpr int kcACC = kcD + 4;                          // accumulator row: 64 channels, row sum,
                                                        // window reference, pad
constexpr int kcOFF_ACC = kcOFF_Q + kcROWS * kcQROW;    // [ROWS][68] fp32 (16-byte aligned rows)
constexpr int kcOFF_M = kcOFF_ACC + kcROWS * kcACC * 4; // [ROWS] selection reference (log2)
constexpr int kcOFF_SB = kcOFF_M + kcROWS * 4;          // [P] register-range selection bits
constexpr int kcOFF_MASK = kcOFF_SB + kcP * 4;          // [nblk] u64 item masks (positions)
static_assert(kcOFF_MASK % 8 == 0, "mask alignment");

// Q row r, 16-byte chunk c
__device__ __forceinline__ int q_off(int r, int c) { return r * kcQROW + ((c ^ (r & 7)) << 4); }
}  // namespace

size_t sel_compact_lds_bytes(int T) { return (size_t)kcOFF_MASK + (size_t)((T + kBlock - 1) / kBlock) * 8; }

bool sel_compact_eligible(bool is_bf16, const Shape& s) {
  return is_bf16 && s.D == kcD && s.G == kcG && (s.W - 1) / kBlock + 2 <= kcMAXR &&
         sel_compact_lds_bytes(s.T) <= 160 * 1024;
}

// compile-time tag of the walk's two period bodies
template <bool B>
struct RangeTag {
  static constexpr bool value = B;
};

__global__ __launch_bounds__(kcNT, 1) void sel_compact_kernel(Shape s, SelWinArgs args) {
  typedef bf16 T;
  typedef bf16x8 FragT;
  typedef kcImg Img;
  constexpr int G = kcG, NSG = kcNSG, P = kcP, NW = kcNW, NT = kcNT;
  constexpr int KS = kcD / 32, MT = kcD / 16, NFRAG = Img::NFRAG, FCH = 2, STAGE = kcSTAGE;
  constexpr int LOADS = Img::PIECES;
  const float INF = __builtin_inff();

  const T* __restrict__ q = (const T*)args.q;
  const T* __restrict__ k = (const T*)args.k;

  const int NBG = s.B * s.Hkv;
  const int NTL = (s.T + P - 1) / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, NBG, NTL, bg, tile);
  if (tile < 0 || bg >= NBG) return;  // padding of the grid to whole XCD rounds
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int nvalid = min(P, s.T - t0);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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

  const size_t k_row = (size_t)s.Hkv * kcD;
  const T* k_b = k + (size_t)b * s.T * k_row + (size_t)g * kcD;
  const unsigned char* img_b =
      (const unsigned char*)args.kvimg + ((size_t)b * s.Hkv + g) * s.nc * (size_t)STAGE;
  const size_t q_row = (size_t)s.Hq * kcD;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;
  unsigned char* qs = smem + kcOFF_Q;
  float* accL = reinterpret_cast<float*>(smem + kcOFF_ACC);
  float* mref = reinterpret_cast<float*>(smem + kcOFF_M);
  unsigned* selbits = reinterpret_cast<unsigned*>(smem + kcOFF_SB);
  unsigned long long* masks = reinterpret_cast<unsigned long long*>(smem + kcOFF_MASK);

  const int c_last = (t0 + nvalid - 1) / kBlock;
  const int nb = c_last + 1;

  const int j_win0 = win_on ? max(0, t0 - W + 1) / kBlock : c_last + 1;
  const int j_begin = need_sel ? 0 : j_win0;
  const int nblk = c_last - j_begin + 1;

  // stage loads: waves 0 .. 3 copy the block image, four 1 KB pieces each
  // (lane l copies its 16 bytes of a piece); the other waves issue nothing
  static_assert(LOADS == 16, "four loader waves x four pieces");
  constexpr int NLD = 4;
  auto issue = [&](int j, int bf) {
    if (w < NLD) {
      unsigned char* stage = ring + (size_t)bf * STAGE + (size_t)w * 4096;
      const unsigned char* src = img_b + (size_t)j * STAGE + (size_t)w * 4096 + 16 * l;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2)
        __builtin_amdgcn_global_load_lds((const void*)(src + q2 * 1024), (void*)(stage + q2 * 1024), 16, 0, 0);
    }
  };

  // The first two blocks are copied while the setup below runs (their loads
  // are in flight behind the setup's own global loads).
  if (nblk > 0) issue(j_begin, 0);
  if (nblk > 1) issue(j_begin + 1, 1);
  // the walk's copies of blocks j_begin + 2, + 3, ... (loader waves): the
  // lane's source address advances by one block image per call
  const unsigned char* src_next = img_b + (size_t)(j_begin + 2) * STAGE + (size_t)w * 4096 + 16 * l;
  auto issue_next = [&](int bf) __attribute__((always_inline)) {
    unsigned char* stage = ring + (size_t)bf * STAGE + (size_t)w * 4096;
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2)
      __builtin_amdgcn_global_load_lds((const void*)(src_next + q2 * 1024), (void*)(stage + q2 * 1024), 16, 0, 0);
    src_next += STAGE;
  };


  // ------------------------------------------------------------ setup
  {
    f32x4* acc4 = reinterpret_cast<f32x4*>(accL);
    for (int i = threadIdx.x; i < kcROWS * kcACC / 4; i += NT) acc4[i] = zero4();
    for (int i = threadIdx.x; i < P; i += NT) selbits[i] = 0u;
    for (int i = threadIdx.x; i < nb; i += NT) masks[i] = 0ull;
  }

  // the wave's column group: positions p0 .. p0 + 3; this lane's row is
  // position p0 + sg, head hh (row index 16 w + col = 4 p + hh)
  const int p0 = w * NSG;
  const int p = p0 + sg;
  const int tpos = t0 + p;
  const int own = (t0 + p0) / kBlock;  // NSG divides 64 and t0: one own block
  const bool valid = p < nvalid;
  const int nv = min(max(nvalid - p0, 0), NSG);
  const int tf = t0 + p0, tl = tf + nv - 1;
  int jw_lo = 1, jw_hi = 0, jw_edge = -1;
  if (win_on && nv > 0) {
    jw_lo = max(0, tf - W + 1) / kBlock;
    jw_hi = own;
    jw_edge = tl >= W ? (tl - W) / kBlock : -1;
  }
  // register range: the window blocks, or the own block alone
  const int jr_lo = nv > 0 ? (win_on ? jw_lo : own) : 1;
  const int jr_hi = nv > 0 ? own : 0;

  // largest key norm over blocks 0 .. c_last
  float mk = 0.f;
  {
    const float* kn = args.knorm + ((size_t)b * s.Hkv + g) * s.nc;
    for (int j = l; j <= c_last; j += kWave) mk = fmaxf(mk, kn[j]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mk = fmaxf(mk, __shfl_xor(mk, o));
  }

  // Q fragments (registers, and the tile's copy in LDS), fixed reference
  FragT qf[KS];
  float mr_s;
  bool any_exact;
  {
    float qq = 0.f, d = 0.f;
    const int r = 16 * w + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (valid) {
        qf[ks] = Frag<T>::load(q + ((size_t)b * s.T + tpos) * q_row + (size_t)h * kcD + ks * 32 + 8 * a);
        const FragT kv = Frag<T>::load(k_b + (size_t)tpos * k_row + ks * 32 + 8 * a);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qf[ks][e];
          qq += x * x;
          d += x * (float)kv[e];
        }
      } else {
        qf[ks] = Frag<T>::zero();
      }
      *reinterpret_cast<FragT*>(qs + q_off(r, 4 * ks + a)) = qf[ks];
    }
    qq = xsum4(qq);
    d = xsum4(d);
    const float mdiag = d * c1;
    const float ub = c1 * sqrtf(qq) * mk * (1.0f + 1e-6f);
    const float m = fmaxf(mdiag, ub - 64.f);
    mr_s = valid ? m : INF;
    any_exact = valid && (ub - mdiag > 164.f);
  }
  __syncthreads();  // zeroed bits, masks and accumulators

  // selection table of the tile -> register-range bits per position, item
  // masks per block
  if (need_sel) {
    for (int i = threadIdx.x; i < P * topk; i += NT) {
      const int pp = i / topk, e = i % topk;
      if (pp >= nvalid) continue;
      const int j = args.indices[(((size_t)b * s.Hkv + g) * s.T + t0 + pp) * topk + e];
      if (j < 0) continue;
      const int tq = t0 + (pp / NSG) * NSG;  // first position of its column group
      const int lo = win_on ? max(0, tq - W + 1) / kBlock : tq / kBlock;
      if (j >= lo) {
        if (j - lo < kcMAXR) atomicOr(&selbits[pp], 1u << (j - lo));  // else not causal: never read
      } else {
        atomicOr(&masks[j], 1ull << pp);
      }
    }
  }
  __syncthreads();
  const unsigned sb = valid ? selbits[p] : 0u;
  __syncthreads();  // the selection-bit area is reused below

  // Item dealing, fixed once: block j has nitem_j = ceil(chosen positions / 4)
  // items, dealt to the waves round-robin in block order; deal[j] holds the
  // wave of its first item (the running count mod NW) and nitem_j << 4.
  unsigned char* deal = reinterpret_cast<unsigned char*>(selbits);  // [nb] (nb <= 4 P)
  if (w == 0 && need_sel) {
    int run = 0;
    for (int c0 = 0; c0 < nb; c0 += kWave) {
      const int j = c0 + l;
      const int ni = j < nb ? (__builtin_popcountll(masks[j]) + NSG - 1) / NSG : 0;
      int x = ni;  // inclusive prefix sum over the lanes
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (l >= o) x += y;
      }
      if (j < nb) deal[j] = (unsigned char)(((run + x - ni) % NW) | (ni << 4));
      run += __shfl(x, kWave - 1);
    }
  }
  __syncthreads();

  // ------------------------------------------ exact maxima (rare; per wave)
  const bool exact = __builtin_amdgcn_ballot_w64(any_exact) != 0;
  if (exact) {
    float ms = -INF, mw = -INF;
    const int jw0 = win_on ? max(0, t0 - W + 1) / kBlock : c_last + 1;
    for (int j = need_sel ? 0 : jw0; j <= c_last; ++j) {
      bool sl = false;
      if (need_sel && valid) {
        if (j >= jr_lo && j <= jr_hi) sl = (sb >> (j - jr_lo)) & 1u;
        else if (j < jr_lo) sl = (masks[j] >> p) & 1ull;
      }
      const bool wl = win_on && valid && j * kBlock <= tpos && j * kBlock + kBlock - 1 > tpos - W;
      if (__builtin_amdgcn_ballot_w64(sl || wl) == 0) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int krow = Img::krow(u, col);
        f32x4 st = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          st = mma(st, Frag<T>::load(k_b + (size_t)(j * kBlock + krow) * k_row + ks * 32 + 8 * a), qf[ks]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = j * kBlock + key_of(u, a, r);
          const float x = st[r] * c1;
          if (sl && key <= tpos) ms = fmaxf(ms, x);
          if (wl && key <= tpos && key > tpos - W) mw = fmaxf(mw, x);
        }
      }
    }
    const float a1 = xmax4(ms), a2 = xmax4(mw);
    float mr_w = mr_s;
    if (valid) {
      if (need_sel) mr_s = a1;
      if (win_on) mr_w = a2;
    }
    // the window reference differs from mr_s only here: kept in LDS (the
    // row's accumulator padding), not in a register across the walk
    if (a == 0) accL[(16 * w + col) * kcACC + kcD + 1] = mr_w;
  }
  if (a == 0) mref[16 * w + col] = mr_s;  // visible after the first ring barrier

  // ------------------------------------------------------------ main walk
  float l_s = 0.f, l_w = 0.f;
  f32x4 acc_s[MT], acc_w[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) { acc_s[mt] = zero4(); acc_w[mt] = zero4(); }

  // Ring of four one-block slots.  In period i the wave's item of the
  // previous block (slot (i - 1) % 4, still resident) first gets its P V and
  // its accumulator update, then block j_begin + i (slot i % 4) is computed;
  // block i + 1 is in flight and block i + 2 goes into the slot of block i - 2.
  // The accumulator updates of a period all come from one block's items,
  // whose rows are distinct, so plain read-modify-writes are race free.
  // (the first two blocks were issued at the start of the kernel)

  // the wave's deferred item: P^T fragments, row, column validity, row sum
  int pend = 0;  // wave-uniform: this wave has a deferred item (an int, so it stays a scalar)
  int dv = 0;  // per lane: the deferred item's column is a real row (an int, kept in a VGPR)
  FragT dp[2];
  int dr = 0;
  float dl = 0.f;
  auto finish_item = [&](const unsigned char* pstage) {
    f32x4 o1[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o1[mt] = zero4();
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
      FragT vf[FCH];
#pragma unroll
      for (int i2 = 0; i2 < FCH; ++i2) vf[i2] = lds_frag<T>(pstage + (size_t)(NFRAG + f0 + i2) * 1024, l);
#pragma unroll
      for (int i2 = 0; i2 < FCH; ++i2) o1[Img::v_mt(f0 + i2)] = mma(o1[Img::v_mt(f0 + i2)], vf[i2], dp[Img::v_h(f0 + i2)]);
    }
    if (dv) {
      float* rowp = accL + dr * kcACC;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4* cp = reinterpret_cast<f32x4*>(rowp + 16 * mt + 4 * a);
        *cp = *cp + o1[mt];
      }
      if (a == 0) rowp[kcD] += dl;
    }
  };

  // blocks where this wave has an item: refreshed every 64 blocks, bit 0 is
  // the current block
  unsigned long long ev = 0ull;
  // One block period.  A wave's blocks before its register range run a
  // body without the register-range part (scalar issue, shared by the
  // 15 waves of a CU, bounds the walk); each period has one barrier on
  // either path, so every wave meets the same barriers.
  // the item mask of blocks bi .. bi + 63 (bi a multiple of 64)
  auto refresh = [&](int bi) __attribute__((always_inline)) {
    const int jj = j_begin + bi + l;
    bool e = false;
    if (need_sel && jj <= c_last) {
      const int d = deal[jj];
      e = (w - (d & 15) + NW) % NW < (d >> 4);
    }
    ev = __builtin_amdgcn_ballot_w64(e);
  };
  auto period = [&](int bi, auto range_tag, auto loader_tag) __attribute__((always_inline)) {
    constexpr bool RANGE = decltype(range_tag)::value;    // blocks of the register range possible
    constexpr bool LOADER = decltype(loader_tag)::value;  // one of the NLD loader waves
    if (LOADER) {  // the loaders' pieces of block bi have landed (block bi + 1 may be in flight)
      if (bi + 1 < nblk) wait_vmcnt<4>();
      else wait_vmcnt<0>();
    }
    barrier_keep_loads();  // block bi in LDS; every wave is done with block bi - 2
    if (LOADER && bi + 2 < nblk) issue_next((bi + 2) & 3);
    const int j = j_begin + bi;
    const unsigned char* stage = ring + (size_t)(bi & 3) * STAGE;

    // ---- the deferred item of the previous block: P V, accumulator update
    if (pend) {
      finish_item(ring + (size_t)((bi - 1) & 3) * STAGE);
      pend = 0;
    }

    // (the second loop of the walk starts at the register range: j >= jr_lo)
    if (RANGE && j <= jr_hi) {
      // register range of the wave's own column group; when the window is
      // on, the register range is exactly the window's blocks
      const bool act_w = win_on;
      const bool sl = valid && ((sb >> (j - jr_lo)) & 1u);
      const bool act_s = __builtin_amdgcn_ballot_w64(sl) != 0;
      const bool wl = act_w && valid && j * kBlock <= tpos && j * kBlock + kBlock - 1 > tpos - W;
      const bool wlow = act_w && j <= jw_edge;
      const bool act0 = act_s || act_w;

      if (act0) {
        // ---- own column group: window branch and in-range selections
        FragT qo[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qo[ks] = *reinterpret_cast<const FragT*>(qs + q_off(16 * w + col, 4 * ks + a));
        f32x4 st[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) st[u] = zero4();
#pragma unroll
        for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
          FragT kf[FCH];
#pragma unroll
          for (int i = 0; i < FCH; ++i) kf[i] = lds_frag<T>(stage + (size_t)(f0 + i) * 1024, l);
#pragma unroll
          for (int i = 0; i < FCH; ++i) st[Img::k_u(f0 + i)] = mma(st[Img::k_u(f0 + i)], kf[i], qo[Img::k_ks(f0 + i)]);
        }
        FragT vf0[FCH];
#pragma unroll
        for (int i = 0; i < FCH; ++i) vf0[i] = lds_frag<T>(stage + (size_t)(NFRAG + i) * 1024, l);

        FragT ps[2], pw[2];
        const bool diag = j == own;
        // with exact references the window's maximum differs from the
        // selection's: every block the window attends takes the
        // two-reference path (also where no row selected the block)
        const bool dual = exact && act_w;
        if (!diag && !wlow && !dual) {
          const bool both = act_s && act_w;
          const bool att = act_s ? sl : wl;
          const float mr = (both ? (sl || wl) : att) ? mr_s : INF;  // mr_s == mr_w unless exact
          FragT pf[2];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(st[2 * hf + e / 4][e % 4] * c1 - mr);
            pf[hf] = Frag<T>::from_f32(pv);
          }
          if (both) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              ps[hf] = frag_keep(pf[hf], sl);
              pw[hf] = frag_keep(pf[hf], wl);
            }
            l_s += frag_sum(ps[0]) + frag_sum(ps[1]);
            l_w += frag_sum(pw[0]) + frag_sum(pw[1]);
          } else if (act_s) {
            ps[0] = pf[0];
            ps[1] = pf[1];
            l_s += frag_sum(pf[0]) + frag_sum(pf[1]);
          } else {
            pw[0] = pf[0];
            pw[1] = pf[1];
            l_w += frag_sum(pf[0]) + frag_sum(pf[1]);
          }
        } else {
          // causal diagonal, window edge, or rows with two exact references
          const float mrw = exact ? accL[(16 * w + col) * kcACC + kcD + 1] : mr_s;
          const float ms = sl ? mr_s : INF, mw = wl ? mrw : INF;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            float pv[8], qw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int u = 2 * hf + e / 4, rr = e % 4;
              const float x = st[u][rr] * c1;
              const int key = j * kBlock + key_of(u, a, rr);
              const bool caus = key <= tpos;
              pv[e] = caus ? fast_exp2(x - ms) : 0.f;
              qw[e] = (caus && key > tpos - W) ? fast_exp2(x - mw) : 0.f;
            }
            ps[hf] = Frag<T>::from_f32(pv);
            pw[hf] = Frag<T>::from_f32(qw);
          }
          if (act_s) l_s += frag_sum(ps[0]) + frag_sum(ps[1]);
          if (act_w) l_w += frag_sum(pw[0]) + frag_sum(pw[1]);
        }
#pragma unroll
        for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
          FragT vf[FCH];
#pragma unroll
          for (int i = 0; i < FCH; ++i)
            vf[i] = f0 == 0 ? vf0[i] : lds_frag<T>(stage + (size_t)(NFRAG + f0 + i) * 1024, l);
#pragma unroll
          for (int i = 0; i < FCH; ++i) {
            const int mt = Img::v_mt(f0 + i), hf = Img::v_h(f0 + i);
            if (act_s) acc_s[mt] = mma(acc_s[mt], vf[i], ps[hf]);
            if (act_w) acc_w[mt] = mma(acc_w[mt], vf[i], pw[hf]);
          }
        }
      }

    }

      // ---- this wave's item of the block (at most one: items <= NW)
      const bool has_item = (unsigned)ev & 1u;  // bit 0 is block bi (shifted once per period)
      ev >>= 1;
      if (has_item) {
        const unsigned long long mm = masks[j];
        const unsigned long long m =
            ((unsigned long long)__builtin_amdgcn_readfirstlane((unsigned)(mm >> 32)) << 32) |
            (unsigned)__builtin_amdgcn_readfirstlane((unsigned)mm);
        const int npos = __builtin_popcountll(m);
        const int it = (w - (__builtin_amdgcn_readfirstlane(deal[j]) & 15) + NW) % NW;
        // slot it * NSG + sg -> position (ds_permute pushes each chosen
        // position to the lane of its rank; ds_bpermute pulls the slot)
        const bool bit = (m >> l) & 1ull;
        const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
        const int slot2pos = __builtin_amdgcn_ds_permute((bit ? rank : 63) * 4, l);
        const int slot = it * NSG + sg;
        const int pos = __builtin_amdgcn_ds_bpermute((slot & 63) * 4, slot2pos);
        dv = slot < npos ? 1 : 0;
        dr = dv ? G * pos + hh : hh;         // unused columns read rows 0 .. 3 (finite)
        const float m1 = dv ? mref[dr] : INF;  // reference +inf: probability 0
        FragT qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = *reinterpret_cast<const FragT*>(qs + q_off(dr, 4 * ks + a));
        f32x4 st[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) st[u] = zero4();
#pragma unroll
        for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
          FragT kf[FCH];
#pragma unroll
          for (int i2 = 0; i2 < FCH; ++i2) kf[i2] = lds_frag<T>(stage + (size_t)(f0 + i2) * 1024, l);
#pragma unroll
          for (int i2 = 0; i2 < FCH; ++i2) st[Img::k_u(f0 + i2)] = mma(st[Img::k_u(f0 + i2)], kf[i2], qa[Img::k_ks(f0 + i2)]);
        }
        // every key of the block is causal for the item's rows: the block
        // precedes their register range
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(st[2 * hf + e / 4][e % 4] * c1 - m1);
          dp[hf] = Frag<T>::from_f32(pv);
        }
        dl = xsum4(frag_sum(dp[0]) + frag_sum(dp[1]));
        pend = 1;
      }
  };
  const int split = jr_hi >= jr_lo ? min(max(jr_lo - j_begin, 0), nblk) : nblk;
  // the periods in runs that end at multiples of 64: the item mask is
  // refreshed at the start of each 64 blocks, not tested every period
  int bi = 0;
  if (w < NLD) {
    while (bi < split) {
      if ((bi & (kWave - 1)) == 0) refresh(bi);
      const int stop = min(split, (bi | (kWave - 1)) + 1);
      for (; bi < stop; ++bi) period(bi, RangeTag<false>{}, RangeTag<true>{});
    }
    while (bi < nblk) {
      if ((bi & (kWave - 1)) == 0) refresh(bi);
      const int stop = min(nblk, (bi | (kWave - 1)) + 1);
      for (; bi < stop; ++bi) period(bi, RangeTag<true>{}, RangeTag<true>{});
    }
  } else {
    while (bi < split) {
      if ((bi & (kWave - 1)) == 0) refresh(bi);
      const int stop = min(split, (bi | (kWave - 1)) + 1);
      for (; bi < stop; ++bi) period(bi, RangeTag<false>{}, RangeTag<false>{});
    }
    while (bi < nblk) {
      if ((bi & (kWave - 1)) == 0) refresh(bi);
      const int stop = min(nblk, (bi | (kWave - 1)) + 1);
      for (; bi < stop; ++bi) period(bi, RangeTag<true>{}, RangeTag<false>{});
    }
  }
  // the last block's items: after every wave has finished the previous
  // block's updates
  barrier_keep_loads();
  if (pend) finish_item(ring + (size_t)((nblk - 1) & 3) * STAGE);
  __syncthreads();  // every accumulator update is in LDS

  // ------------------------------------------------------------ combine
  const T* gates = (const T*)args.gates;
  T* out = (T*)args.out;
  const int r0 = 16 * w + col;
  const float* arow = accL + r0 * kcACC;
  const float ls = xsum4(l_s) + (need_sel ? arow[kcD] : 0.f);
  const float lw = xsum4(l_w);
  if (!valid) return;
  // the position again, opaque to the compiler: the row offsets below are
  // recomputed here instead of being held in registers across the walk
  int te = tpos;
  asm volatile("" : "+v"(te));
  const T* grow = gates + (((size_t)b * s.T + te) * s.Hq + h) * 3;
  const float gc = cmp_on ? to_f32(grow[0]) : 0.f;
  const float gs = sel_on ? to_f32(grow[1]) : 0.f;
  const float gw = win_on ? to_f32(grow[2]) : 0.f;
  const float iw = win_on ? gw / lw : 0.f;
  const float ilw = win_on ? 1.f / lw : 0.f;
  const float il = need_sel ? 1.f / ls : 0.f;
  const size_t obase = ((size_t)b * s.T + te) * q_row + (size_t)h * kcD;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int d0 = mt * 16 + 4 * a;
    f32x4 res = acc_w[mt] * iw;
    if (args.o_win) store4((T*)args.o_win + obase + d0, acc_w[mt] * ilw);
    if (need_sel) {
      f32x4 sacc = acc_s[mt];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) sacc[rr] += arow[d0 + rr];
      const f32x4 os = sacc * il;
      if (sel_on) res += os * gs;
      if (args.o_sel) store4((T*)args.o_sel + obase + d0, os);
    }
    if (cmp_on && tpos >= kBlock - 1) res += load4((const T*)args.o_cmp + obase + d0) * gc;
    store4(out + obase + d0, res);
  }
  if (args.lse && a == 0) args.lse[((size_t)b * s.Hq + h) * s.T + tpos] = (mr_s + __log2f(ls)) * kLn2;
  if (args.lse_win && a == 0)
    args.lse_win[((size_t)b * s.Hq + h) * s.T + tpos] = win_on ? ((exact ? arow[kcD + 1] : mr_s) + __log2f(lw)) * kLn2 : -INF;
}

hipError_t launch_sel_compact(const Shape& s, const SelWinArgs& args, hipStream_t st) {
  const size_t lds = sel_compact_lds_bytes(s.T);
  hipError_t e = hipFuncSetAttribute((const void*)sel_compact_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int NBG = s.B * s.Hkv;
  const int NTL = (s.T + kcP - 1) / kcP;
  int n = NTL * NBG;
  if (8 % NBG == 0) n = (n + 7) / 8 * 8;  // whole XCD rounds; the padding returns at once
  hipLaunchKernelGGL(sel_compact_kernel, dim3(n), dim3(kcNT), lds, st, s, args);
  return hipGetLastError();
}

}  // namespace nsa
