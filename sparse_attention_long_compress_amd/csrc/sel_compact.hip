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
// Here the selection work is packed instead.
//
// Work decomposition.  One workgroup per (64 positions = one key block, KV
// group, batch): sixteen waves, each owning one column group (4 positions x 4
// heads), 128 registers per lane (a build option gives eight waves with two
// column groups each and 256 registers).
//   * Register range: the window blocks of the tile's first position (or
//     only the own block when the window branch is off), the same for every
//     column group.  There the wave computes, as the general kernel does, the
//     window branch and the selections that fall in the range, with both
//     accumulators in registers and one exponential per element serving both
//     branches.  The range is software-pipelined: a period issues Q K^T of
//     its block, then P V of the previous range block, then takes the
//     exponentials.
//   * Items: every selected block j before the range is a list of the tile's
//     positions that chose it, four to an item (16 full MFMA columns).  The
//     items of a block are dealt to the waves round-robin (a wave takes at
//     most one of a block, two with eight waves); an item's P V is added into
//     fp32 row accumulators in LDS.
// Both parts use the row's fixed softmax reference (a Cauchy-Schwarz bound,
// or the exact per-branch maxima in the rare rows where the bound is loose),
// so a row's sum over its blocks is a plain sum: the order of the additions
// only changes rounding.
//
// The walk.  Blocks j_begin .. own are walked once, one barrier per block.
// Each block's image (K and V^T in MFMA fragment order, written by the pooling
// kernel) is copied global -> LDS with 1 KB global_load_lds pieces, one per
// wave, into a ring of three K slots and four V^T slots; the copy of block
// i + 2 is issued in period i.  An item is two-stage: in the period of its
// block the wave issues Q K^T (Q rows from the tile's copy in LDS, the item's
// four positions looked up once per 48 blocks); in the next period, with the
// MFMA results long complete, it takes the exponentials, issues P V (the
// block's V^T still in its slot) and adds the result to the rows'
// accumulators.  All accumulator updates of one period therefore come from
// one block's items, whose rows are distinct: plain read-modify-writes, no
// atomics, deterministic results.
#include <math.h>
#include <stdint.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

namespace {
#ifndef NSA_K3C_NW
#define NSA_K3C_NW 16
#endif
constexpr int kcNW = NSA_K3C_NW;            // waves per workgroup (8 or 16)
constexpr int kcNT = kcNW * kWave;
constexpr int kcNCG = 16 / kcNW;            // column groups per wave
constexpr int kcNX = (16 + kcNW - 1) / kcNW; // items a wave may take of one block (<= 16 items)
constexpr int kcPPW = 16 / kcNW;            // 1 KB pieces of a block image each wave copies
constexpr int kcG = 4;                      // query heads per KV group
constexpr int kcNSG = 16 / kcG;             // positions per column group / item
constexpr int kcP = kcNW * kcNCG * kcNSG;   // positions per workgroup: one key block
constexpr int kcROWS = kcP * kcG;           // rows (position, head) per workgroup
constexpr int kcD = 64;
typedef KvImage<bf16, kcD> kcImg;
constexpr int kcHALF = kcImg::BYTES / 2;    // 8 KB: the K (or the V^T) fragments of a block
constexpr int kcKSLOTS = 3;                 // K ring: blocks i, i + 1, i + 2
constexpr int kcVSLOTS = 4;                 // V^T ring: blocks i - 1 (items), i, i + 1, i + 2
constexpr int kcQROW = kcD * 2;             // bytes per Q row in LDS
constexpr int kcMAXR = 32;                  // register range of at most 32 blocks (bit set)
constexpr int kcMAXW = 4;                   // chosen-block bitmap words: sequences up to 16384
constexpr int kcACC = kcD + 4;              // accumulator row: 64 channels, item row sum, pad
constexpr int kcCHUNK = 48;                 // blocks per item-table refresh: a multiple of the ring
                                            // phases (12), at most one per lane
// LDS layout
constexpr int kcOFF_V = kcKSLOTS * kcHALF;
constexpr int kcOFF_Q = kcOFF_V + kcVSLOTS * kcHALF;     // [ROWS][64] bf16, 16-byte chunks swizzled
constexpr int kcOFF_ACC = kcOFF_Q + kcROWS * kcQROW;     // [ROWS][68] fp32 (16-byte aligned rows)
constexpr int kcOFF_SB = kcOFF_ACC + kcROWS * kcACC * 4; // [P] register-range selection bits
constexpr int kcOFF_MASK = kcOFF_SB + kcP * 4;           // [nb] u64 item masks, [nb] deal bytes,
                                                         // [ROWS] selection references
static_assert(kcOFF_MASK % 8 == 0, "mask alignment");
static_assert(kcP == kBlock, "one workgroup per key block of positions");

// Q row r, 16-byte chunk c
__device__ __forceinline__ int q_off(int r, int c) { return r * kcQROW + ((c ^ (r & 7)) << 4); }

// The four positions (bytes; 0xFF: none) of item `r` of a block whose choosing
// positions are the set bits of m: the set bits of rank 4 r .. 4 r + 3.
__device__ __forceinline__ unsigned item_positions(unsigned long long m, int r) {
  for (int i = 0; i < 4 * r; ++i) m &= m - 1;
  unsigned res = 0;
#pragma unroll
  for (int k2 = 0; k2 < 4; ++k2) {
    const unsigned p = m ? (unsigned)__builtin_ctzll(m) : 0xFFu;
    res |= p << (8 * k2);
    m &= m - 1;
  }
  return res;
}
}  // namespace

size_t sel_compact_lds_bytes(int T) {
  const size_t nb = (size_t)(T + kBlock - 1) / kBlock;
  return (size_t)kcOFF_MASK + nb * 8 + (nb + 7) / 8 * 16 + kcROWS * 4;
}

bool sel_compact_eligible(bool is_bf16, const Shape& s) {
  return is_bf16 && s.D == kcD && s.G == kcG && s.T % kcP == 0 && s.T <= kcMAXW * 64 * kBlock &&
         (s.W - 1) / kBlock + 2 <= kcMAXR && sel_compact_lds_bytes(s.T) <= 160 * 1024;
}

// compile-time tags of the walk's period bodies
template <bool B>
struct RangeTag {
  static constexpr bool value = B;
};
template <int V>
struct ItemsTag {
  static constexpr int value = V;
};

__global__ __launch_bounds__(kcNT, 1) void sel_compact_kernel(Shape s, SelWinArgs args) {
  typedef bf16 T;
  typedef bf16x8 FragT;
  typedef kcImg Img;
  constexpr int G = kcG, NSG = kcNSG, P = kcP, NW = kcNW, NT = kcNT, NCG = kcNCG;
  constexpr int KS = kcD / 32, MT = kcD / 16, NFRAG = Img::NFRAG;
  // K / V^T fragments per LDS read batch: all of them (reads first, a
  // scheduling fence, then the MFMAs) when registers allow, else pairs
  constexpr int KF = kcNW == 8 ? NFRAG : 2;
  constexpr int KFR = KF;  // the item stages' batch in periods with the register range
  constexpr int ACC = kcACC;
  const float INF = __builtin_inff();

  const T* __restrict__ q = (const T*)args.q;
  const T* __restrict__ k = (const T*)args.k;

  const int NBG = s.B * s.Hkv;
  const int NTL = s.T / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, NBG, NTL, bg, tile);
  if (tile < 0 || bg >= NBG) return;  // padding of the grid to whole XCD rounds
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int own = tile;  // the key block of every position of the tile
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
      (const unsigned char*)args.kvimg + ((size_t)b * s.Hkv + g) * s.nc * (size_t)Img::BYTES;
  const size_t q_row = (size_t)s.Hq * kcD;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kring = smem;
  unsigned char* vring = smem + kcOFF_V;
  unsigned char* qs = smem + kcOFF_Q;
  float* accL = reinterpret_cast<float*>(smem + kcOFF_ACC);
  unsigned* selbits = reinterpret_cast<unsigned*>(smem + kcOFF_SB);
  unsigned long long* masks = reinterpret_cast<unsigned long long*>(smem + kcOFF_MASK);

  const int c_last = own;
  const int nb = c_last + 1;
  unsigned short* deal = reinterpret_cast<unsigned short*>(masks + nb);  // [nb]
  float* mref = reinterpret_cast<float*>(deal + (nb + 7) / 8 * 8);  // [ROWS] selection references

  const int j_win0 = win_on ? max(0, t0 - W + 1) / kBlock : c_last + 1;
  // Every column group's register range starts at the first window block of
  // the tile's first position (the own block when the window is off), so no
  // block of the range has items.  Where a group's window starts later, its
  // leading range blocks are window-edge blocks, masked per element.
  const int jr_tile = win_on ? j_win0 : own;
  const int j_begin = need_sel ? 0 : j_win0;
  const int nblk = c_last - j_begin + 1;

  // Stage loads: wave w copies pieces kcPPW w .. kcPPW w + kcPPW - 1 of the block image
  // (pieces 0 .. 7 are the K fragments, 8 .. 15 the V^T fragments); lane l
  // copies its 16 bytes of each piece.
  static_assert(Img::PIECES == kcPPW * NW, "pieces per wave");
  const unsigned char* src_next = img_b + (size_t)j_begin * Img::BYTES + (size_t)(kcPPW * w) * 1024 + 16 * l;
  unsigned char* const dst_base = w < NW / 2 ? kring + (size_t)(kcPPW * w) * 1024
                                             : vring + (size_t)(kcPPW * w - 8) * 1024;
  const int slots = w < NW / 2 ? kcKSLOTS : kcVSLOTS;
  int islot = 0;  // the wave's slot of the next copy (copies go out in block order)
  auto issue = [&]() __attribute__((always_inline)) {
    unsigned char* dst = dst_base + (size_t)islot * kcHALF;
#pragma unroll
    for (int pc = 0; pc < kcPPW; ++pc)
      __builtin_amdgcn_global_load_lds((const void*)(src_next + pc * 1024), (void*)(dst + pc * 1024), 16, 0, 0);
    src_next += Img::BYTES;
    islot = islot + 1 == slots ? 0 : islot + 1;
  };
  // the same with the slot known at compile time: the copy of block i goes to
  // slot i mod 3 (K loaders) or i mod 4 (V^T loaders); PH = i mod 12.  The
  // runtime slot is left as it was: twelve copies bring it back to itself.
  const bool k_loader = w < NW / 2;
  auto issue_c = [&](auto ph_tag) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_tag)::value;
    unsigned char* dst = dst_base + (size_t)(k_loader ? PH % kcKSLOTS : PH % kcVSLOTS) * kcHALF;
#pragma unroll
    for (int pc = 0; pc < kcPPW; ++pc)
      __builtin_amdgcn_global_load_lds((const void*)(src_next + pc * 1024), (void*)(dst + pc * 1024), 16, 0, 0);
    src_next += Img::BYTES;
  };
  static_assert(12 % kcKSLOTS == 0 && 12 % kcVSLOTS == 0, "ring phases divide 12");
  // the first two blocks are copied while the setup runs
  if (nblk > 0) issue();
  if (nblk > 1) issue();

  // ------------------------------------------------------------ setup
  // Every global load of the setup goes out before the first use (one memory
  // round trip): the tile's index rows (contiguous [64][topk] int32, loaded
  // coalesced by all threads), the block key norms, Q and the own keys.
  constexpr int IPT = 32 * P / NT;  // index entries per thread (top-k <= 32)
  int iv[IPT];
  {
    const int32_t* itile = args.indices + (((size_t)b * s.Hkv + g) * s.T + t0) * topk;
    const int nidx = P * topk;
#pragma unroll
    for (int i = 0; i < IPT; ++i) iv[i] = itile[min((int)threadIdx.x + i * NT, nidx - 1)];  // in bounds
  }
  float kn4[kcMAXW];
  {
    const float* kn = args.knorm + ((size_t)b * s.Hkv + g) * s.nc;
#pragma unroll
    for (int x = 0; x < kcMAXW; ++x) kn4[x] = kn[min(l + kWave * x, c_last)];  // in bounds
  }
  // The wave's column groups cg (index C = NCG w + cg): positions
  // 4 C .. 4 C + 3; this lane's row is position 4 C + sg, head hh (row
  // 16 C + col).  Q fragments stay in registers (and are copied to LDS for the
  // items); fixed references of both softmaxes.
  int tpos[NCG], jr_lo[NCG], jw_edge[NCG];
  FragT qf[NCG][KS], kd[NCG][KS];
  float mr_s[NCG], mr_w[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int C = NCG * w + cg;
    tpos[cg] = t0 + C * NSG + sg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[cg][ks] = Frag<T>::load(q + ((size_t)b * s.T + tpos[cg]) * q_row + (size_t)h * kcD + ks * 32 + 8 * a);
      kd[cg][ks] = Frag<T>::load(k_b + (size_t)tpos[cg] * k_row + ks * 32 + 8 * a);
    }
  }
  for (int i = threadIdx.x; i < P; i += NT) selbits[i] = 0u;
  for (int i = threadIdx.x; i < nb; i += NT) masks[i] = 0ull;
  // largest key norm over blocks 0 .. c_last
  float mk = 0.f;
#pragma unroll
  for (int x = 0; x < kcMAXW; ++x) mk = fmaxf(mk, kn4[x]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mk = fmaxf(mk, __shfl_xor(mk, o));
  bool any_exact = false;
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int C = NCG * w + cg;
    const int tf = t0 + C * NSG, tl = tf + NSG - 1;
    jr_lo[cg] = jr_tile;
    jw_edge[cg] = (win_on && tl >= W) ? (tl - W) / kBlock : -1;
    float qq = 0.f, d = 0.f;
    const int r = 16 * C + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (float)qf[cg][ks][e];
        qq += x * x;
        d += x * (float)kd[cg][ks][e];
      }
      *reinterpret_cast<FragT*>(qs + q_off(r, 4 * ks + a)) = qf[cg][ks];
    }
    qq = xsum4(qq);
    d = xsum4(d);
    const float mdiag = d * c1;
    const float ub = c1 * sqrtf(qq) * mk * (1.0f + 1e-6f);
    mr_s[cg] = fmaxf(mdiag, ub - 64.f);
    mr_w[cg] = mr_s[cg];
    any_exact |= ub - mdiag > 164.f;
  }
  __syncthreads();  // zeroed bits and masks, Q copy

  // Selection table of the tile -> register-range bits per position, and per
  // block j outside a position's range a 64-bit mask of the positions that
  // chose it (bitwise ORs into LDS: the result does not depend on their order).
  if (need_sel) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int e = threadIdx.x + i * NT;
      if (e >= P * topk) continue;
      const int pp = e / topk, j = iv[i];
      if (j < 0) continue;
      const int lo = jr_tile;
      if (j >= lo) {
        if (j - lo < kcMAXR) atomicOr(&selbits[pp], 1u << (j - lo));  // else not causal: never read
      } else {
        atomicOr(&masks[j], 1ull << pp);
      }
    }
  }
  __syncthreads();  // bits, masks
  {
    f32x4* acc4 = reinterpret_cast<f32x4*>(accL);
    for (int i = threadIdx.x; i < kcROWS * ACC / 4; i += NT) acc4[i] = zero4();
  }

  unsigned sb[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) sb[cg] = need_sel ? selbits[(NCG * w + cg) * NSG + sg] : 0u;

  // Item dealing, fixed once: block j has nitem_j = ceil(chosen positions / 4)
  // items, dealt to the waves round-robin in block order; deal[j] holds the
  // wave of its first item (the running count mod NW) and nitem_j << 5.
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
      if (j < nb) deal[j] = (unsigned short)(((run + x - ni) % NW) | (ni << 5));
      run += __shfl(x, kWave - 1);
    }
  }

  // ------------------------------------------ exact maxima (rare; per wave)
  const bool exact = __builtin_amdgcn_ballot_w64(any_exact) != 0;
  if (exact) {
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      float ms = -INF, mw = -INF;
      const int tp = tpos[cg];
      for (int j = j_begin; j <= c_last; ++j) {
        bool sl = false;
        if (need_sel) {
          if (j >= jr_lo[cg]) sl = (sb[cg] >> (j - jr_lo[cg])) & 1u;
          else sl = (masks[j] >> ((NCG * w + cg) * NSG + sg)) & 1ull;
        }
        const bool wl = win_on && j * kBlock <= tp && j * kBlock + kBlock - 1 > tp - W;
        if (__builtin_amdgcn_ballot_w64(sl || wl) == 0) continue;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int krow = Img::krow(u, col);
          f32x4 st = zero4();
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            st = mma(st, Frag<T>::load(k_b + (size_t)(j * kBlock + krow) * k_row + ks * 32 + 8 * a), qf[cg][ks]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = j * kBlock + key_of(u, a, r);
            const float x = st[r] * c1;
            if (sl && key <= tp) ms = fmaxf(ms, x);
            if (wl && key <= tp && key > tp - W) mw = fmaxf(mw, x);
          }
        }
      }
      const float a1 = xmax4(ms), a2 = xmax4(mw);
      if (need_sel) mr_s[cg] = a1;
      if (win_on) mr_w[cg] = a2;
    }
  }
  // the selection reference of every row, for the items that cover it
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg)
    if (a == 0) mref[16 * (NCG * w + cg) + col] = mr_s[cg];
  __syncthreads();  // deal table, references

  // ------------------------------------------------------------ main walk
  float l_s[NCG], l_w[NCG];
  f32x4 acc_s[NCG][MT], acc_w[NCG][MT];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    l_s[cg] = 0.f;
    l_w[cg] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { acc_s[cg][mt] = zero4(); acc_w[cg][mt] = zero4(); }
  }

  // The wave's items of blocks cs .. cs + kcCHUNK - 1 (cs: the chunk's first
  // block, a multiple of kcCHUNK): bit i of ev[x] is block j_begin + cs + i
  // (x: the wave's x-th item of the block, when the block has more than NW
  // items); lane i of ipos[x] holds that item's four positions.
  constexpr int NX = kcNX;
  unsigned long long ev[NX];
  unsigned ipos[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) { ev[x] = 0ull; ipos[x] = 0xFFFFFFFFu; }
  auto refresh = [&](int bi) __attribute__((always_inline)) {
    const int jj = j_begin + bi + l;
    int d = 0;
    if (need_sel && jj <= c_last) d = deal[jj];
    const int ni = d >> 5;
    const int r = (w - (d & 31) + NW) % NW;
    const unsigned long long m = (need_sel && jj <= c_last && r < ni) ? masks[jj] : 0ull;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const bool e = r + x * NW < ni;
      ev[x] = __builtin_amdgcn_ballot_w64(e);
      ipos[x] = e ? item_positions(m, r + x * NW) : 0xFFFFFFFFu;
    }
  };

  // Items whose Q K^T was issued in the previous period (stage B pending):
  // S^T, the lane's row, whether it is a real row, its reference.
  int pend[NX];  // wave-uniform (ints, so they stay scalars)
  f32x4 sB[NX][4];
  int rB[NX], vB[NX];
  float mB[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    pend[x] = 0;
    rB[x] = 0;
    vB[x] = 0;
    mB[x] = INF;
#pragma unroll
    for (int u = 0; u < 4; ++u) sB[x][u] = zero4();
  }
  auto any_pend = [&]() __attribute__((always_inline)) {
    int e = 0;
#pragma unroll
    for (int x = 0; x < NX; ++x) e |= pend[x];
    return e;
  };

  FragT ones;  // all-ones MFMA operand (row sums)
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (T)1.0f;
  // stage B of the pending items: exponentials, P V over the block's V^T
  // (vst), row sums, then the rows' accumulator update
  auto finish_items = [&](const unsigned char* vst, auto wide_tag) __attribute__((always_inline)) {
    constexpr int KF = decltype(wide_tag)::value ? NFRAG : KFR;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (!pend[x]) continue;
      pend[x] = 0;
      // the period waits for the longest item chain, which is stage B's: its
      // wave issues ahead of the other waves of its SIMD until the update is out
      __builtin_amdgcn_s_setprio(3);
      float* rowp = accL + rB[x] * ACC;
      // every LDS read of the stage (the rows' current sums, the block's V^T
      // fragments) is issued first; the exponentials overlap their latency
      f32x4 cur[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) cur[mt] = *reinterpret_cast<const f32x4*>(rowp + 16 * mt + 4 * a);
      const float cur_l = rowp[kcD];
      FragT vf[KF];
      if constexpr (KF == NFRAG) {
#pragma unroll
        for (int f = 0; f < NFRAG; ++f) vf[f] = lds_frag<T>(vst + (size_t)f * 1024, l);
        __builtin_amdgcn_sched_barrier(0);
      }
      FragT dp[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(sB[x][2 * hf + e / 4][e % 4] * c1 - mB[x]);
        dp[hf] = Frag<T>::from_f32(pv);
      }
      // P V is accumulated onto the rows' current sums (the MFMA's C operand),
      // and the row sum of P (the bf16 values P V uses) is an MFMA against an
      // all-ones A operand: both on the matrix unit, not the VALU
      f32x4 rs = zero4();
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) rs = mma(rs, ones, dp[hf]);
      const float dl = rs[0];
      f32x4 o1[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o1[mt] = cur[mt];
#pragma unroll
      for (int f0 = 0; f0 < NFRAG; f0 += KF) {
        if constexpr (KF != NFRAG) {
#pragma unroll
          for (int i2 = 0; i2 < KF; ++i2) vf[i2] = lds_frag<T>(vst + (size_t)(f0 + i2) * 1024, l);
        }
#pragma unroll
        for (int i2 = 0; i2 < KF; ++i2)
          o1[Img::v_mt(f0 + i2)] = mma(o1[Img::v_mt(f0 + i2)], vf[i2], dp[Img::v_h(f0 + i2)]);
      }
      if (vB[x]) {  // (unused columns read rows 0 .. 3 and must not write them)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *reinterpret_cast<f32x4*>(rowp + 16 * mt + 4 * a) = o1[mt];
        if (a == 0) rowp[kcD] = cur_l + dl;
      }
      __builtin_amdgcn_s_setprio(0);
    }
  };

  // stage A of this wave's items of block bi (K fragments in kst): Q K^T
  // (evb: the event masks shifted so that bit `bit` is this block's; lane:
  // the block's lane of ipos)
  auto start_items = [&](const unsigned long long (&evb)[NX], int bit, int lane, const unsigned char* kst,
                         auto wide_tag) __attribute__((always_inline)) {
    constexpr int KF = decltype(wide_tag)::value ? NFRAG : KFR;
    int has[NX], any = 0;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      has[x] = (int)((evb[x] >> bit) & 1ull);
      any |= has[x];
    }
    if (!any) return;
    FragT qa[NX][KS];
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      if (NX > 1 && !has[x]) continue;  // (one item slot: has == any)
      const unsigned pos4 = __builtin_amdgcn_readlane(ipos[x], lane);
      const unsigned p8 = (pos4 >> (8 * sg)) & 0xFFu;
      vB[x] = p8 != 0xFFu ? 1 : 0;
      rB[x] = vB[x] ? G * (int)p8 + hh : hh;  // unused columns read rows 0 .. 3 (finite)
      mB[x] = vB[x] ? mref[rB[x]] : INF;  // reference +inf: probability 0
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qa[x][ks] = *reinterpret_cast<const FragT*>(qs + q_off(rB[x], 4 * ks + a));
#pragma unroll
      for (int u = 0; u < 4; ++u) sB[x][u] = zero4();
      pend[x] = 1;
    }
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += KF) {
      FragT kf[KF];
#pragma unroll
      for (int i2 = 0; i2 < KF; ++i2) kf[i2] = lds_frag<T>(kst + (size_t)(f0 + i2) * 1024, l);
      if constexpr (KF == NFRAG) __builtin_amdgcn_sched_barrier(0);  // every read in flight first
#pragma unroll
      for (int i2 = 0; i2 < KF; ++i2)
#pragma unroll
        for (int x = 0; x < NX; ++x)
          if (NX == 1 || has[x]) sB[x][Img::k_u(f0 + i2)] = mma(sB[x][Img::k_u(f0 + i2)], kf[i2], qa[x][Img::k_ks(f0 + i2)]);
    }
  };

  // Register-range work, software-pipelined over the range's blocks: in the
  // period of block j the wave issues Q K^T of block j, then P V of block
  // j - 1 (its P kept in registers, the block's V^T still in its ring slot),
  // then takes the exponentials of block j while those products run, so the
  // matrix unit and the VALU work side by side.
  FragT psc[NCG][2], pwc[NCG][2];  // P of the previous range block (both branches)
  int pvs[NCG], pvw[NCG];          // wave-uniform: that block's branches are active
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) { pvs[cg] = 0; pvw[cg] = 0; }
  auto range_pv = [&](const unsigned char* vst) __attribute__((always_inline)) {
    int any = 0;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) any |= pvs[cg] | pvw[cg];
    if (!any) return;
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += KF) {
      FragT vf[KF];
#pragma unroll
      for (int i = 0; i < KF; ++i) vf[i] = lds_frag<T>(vst + (size_t)(f0 + i) * 1024, l);
#pragma unroll
      for (int i = 0; i < KF; ++i) {
        const int mt = Img::v_mt(f0 + i), hf = Img::v_h(f0 + i);
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          if (pvs[cg]) acc_s[cg][mt] = mma(acc_s[cg][mt], vf[i], psc[cg][hf]);
          if (pvw[cg]) acc_w[cg][mt] = mma(acc_w[cg][mt], vf[i], pwc[cg][hf]);
        }
      }
    }
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) { pvs[cg] = 0; pvw[cg] = 0; }
  };
  // block j (K fragments in kst); vprev: the V^T of block j - 1
  auto range_block = [&](int j, const unsigned char* kst, const unsigned char* vprev) __attribute__((always_inline)) {
    bool sl[NCG], wl[NCG], act_s[NCG], act_w[NCG], act[NCG], wlow[NCG];
    bool any = false;
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const bool in = j >= jr_lo[cg];  // (every column group's range ends at the own block)
      sl[cg] = in && ((sb[cg] >> (j - jr_lo[cg])) & 1u);
      act_s[cg] = __builtin_amdgcn_ballot_w64(sl[cg]) != 0;
      act_w[cg] = in && win_on;  // when the window is on, the range holds its blocks (and edge blocks)
      const int tp = tpos[cg];
      wl[cg] = act_w[cg] && j * kBlock <= tp && j * kBlock + kBlock - 1 > tp - W;
      wlow[cg] = act_w[cg] && j <= jw_edge[cg];
      act[cg] = act_s[cg] || act_w[cg];
      any |= act[cg];
    }
    if (!any) {
      range_pv(vprev);
      return;
    }
    f32x4 st[NCG][4];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int u = 0; u < 4; ++u) st[cg][u] = zero4();
    // the column groups' own Q: registers when they allow (8 waves), else
    // the tile's copy in LDS (16 waves)
    FragT qo[NCG][KS];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qo[cg][ks] = kcNW == 8 ? qf[cg][ks]
                               : *reinterpret_cast<const FragT*>(qs + q_off(16 * (NCG * w + cg) + col, 4 * ks + a));
#pragma unroll
    for (int f0 = 0; f0 < NFRAG; f0 += KF) {
      FragT kf[KF];
#pragma unroll
      for (int i = 0; i < KF; ++i) kf[i] = lds_frag<T>(kst + (size_t)(f0 + i) * 1024, l);
      if constexpr (KF == NFRAG) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < KF; ++i)
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg)
          st[cg][Img::k_u(f0 + i)] = mma(st[cg][Img::k_u(f0 + i)], kf[i], qo[cg][Img::k_ks(f0 + i)]);  // (unused when inactive)
    }
    range_pv(vprev);

#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      if (!act[cg]) continue;
      const int tp = tpos[cg];
      const bool diag = j == own;
      // with exact references the window's maximum differs from the
      // selection's: every block the window attends takes the two-reference
      // path (also where no row selected the block)
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
            psc[cg][hf] = frag_keep(pf[hf], sl[cg]);
            pwc[cg][hf] = frag_keep(pf[hf], wl[cg]);
          }
          l_s[cg] += frag_sum(psc[cg][0]) + frag_sum(psc[cg][1]);
          l_w[cg] += frag_sum(pwc[cg][0]) + frag_sum(pwc[cg][1]);
        } else {
          // one branch only: both sums are updated (the other by 0), so
          // neither accumulator is addressed through a selected pointer
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            psc[cg][hf] = pf[hf];
            pwc[cg][hf] = pf[hf];
          }
          const float sp = frag_sum(pf[0]) + frag_sum(pf[1]);
          l_s[cg] += act_s[cg] ? sp : 0.f;
          l_w[cg] += act_s[cg] ? 0.f : sp;
        }
      } else {
        // causal diagonal, window edge, or rows with two exact references
        // (one exponential per element serves both branches unless the exact
        // references differ)
        const float ms = sl[cg] ? mr_s[cg] : INF, mw = wl[cg] ? mr_w[cg] : INF;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8], qw[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 2 * hf + e / 4, rr = e % 4;
            const float x = st[cg][u][rr] * c1;
            const int key = j * kBlock + key_of(u, a, rr);
            const bool caus = key <= tp;
            const bool inw = caus && key > tp - W;
            if (!exact) {
              const float ex = fast_exp2(x - mr_s[cg]);  // mr_s == mr_w
              pv[e] = caus && sl[cg] ? ex : 0.f;
              qw[e] = inw && wl[cg] ? ex : 0.f;
            } else {
              pv[e] = caus ? fast_exp2(x - ms) : 0.f;
              qw[e] = inw ? fast_exp2(x - mw) : 0.f;
            }
          }
          psc[cg][hf] = Frag<T>::from_f32(pv);
          pwc[cg][hf] = Frag<T>::from_f32(qw);
        }
        if (act_s[cg]) l_s[cg] += frag_sum(psc[cg][0]) + frag_sum(psc[cg][1]);
        if (act_w[cg]) l_w[cg] += frag_sum(pwc[cg][0]) + frag_sum(pwc[cg][1]);
      }
      pvs[cg] = act_s[cg];
      pvw[cg] = act_w[cg];
    }
  };

  // One block period: the loads of block bi have landed (block bi + 1 may be
  // in flight), barrier, the copy of block bi + 2, then stage B of the items
  // of block bi - 1, the register range, stage A of the items of block bi.
  // Every path has exactly one barrier per block.
  int kslot = 0, vslot = 0;  // ring slots of block bi
  int cs = 0;                // first block of the item-table chunk
  // (FULL: blocks bi + 1 and bi + 2 exist, so the wait and the copy need no
  // test: most periods before the register range)
  auto period = [&](int bi, auto range_tag, auto items_tag, auto full_tag) __attribute__((always_inline)) {
    constexpr bool RANGE = decltype(range_tag)::value;
    constexpr int ITEMS = decltype(items_tag)::value;  // 0 none, 1 stage B only, 2 both stages
    constexpr bool FULL = decltype(full_tag)::value;
    if (FULL || bi + 1 < nblk) wait_vmcnt<kcPPW>();
    else wait_vmcnt<0>();
    barrier_keep_loads();  // block bi in LDS; every wave is done with block bi - 1's K and bi - 2's V^T
    if (FULL || bi + 2 < nblk) issue();
    const unsigned char* kst = kring + (size_t)kslot * kcHALF;
    const unsigned char* vprev = vring + (size_t)((vslot + kcVSLOTS - 1) & (kcVSLOTS - 1)) * kcHALF;
    if (ITEMS >= 1 && any_pend()) finish_items(vprev, RangeTag<!RANGE>{});
    if (RANGE) range_block(j_begin + bi, kst, vprev);
    if (ITEMS == 2) start_items(ev, bi - cs, bi - cs, kst, RangeTag<!RANGE>{});
    kslot = kslot + 1 == kcKSLOTS ? 0 : kslot + 1;
    vslot = (vslot + 1) & (kcVSLOTS - 1);
  };
  // a full period before the register range whose ring phase bi mod 12 = PH is
  // known at compile time (evg: the event masks shifted by lane0 = bi - PH - cs)
  auto period_c = [&](auto ph_tag, int lane0, const unsigned long long (&evg)[NX]) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_tag)::value;
    wait_vmcnt<kcPPW>();
    barrier_keep_loads();
    issue_c(ItemsTag<(PH + 2) % 12>{});
    const unsigned char* kst = kring + (size_t)(PH % kcKSLOTS) * kcHALF;
    const unsigned char* vprev = vring + (size_t)((PH + kcVSLOTS - 1) % kcVSLOTS) * kcHALF;
    if (any_pend()) finish_items(vprev, RangeTag<true>{});
    start_items(evg, PH, lane0 + PH, kst, RangeTag<true>{});
  };
  static_assert((kcVSLOTS & (kcVSLOTS - 1)) == 0, "V^T slots: a power of two");

  // Blocks before the register range run a body without the range part; the
  // range's first period still finishes the items of the block before it,
  // and its other periods have no item work.
  const int split = max(jr_tile - j_begin, 0);
  int bi = 0;
  // (the range has at least one block, so every period before it has block
  // bi + 1; all but possibly the last have bi + 2)
  const int split_full = min(split, nblk - 2);
  while (bi < split) {
    cs = bi;  // a multiple of kcCHUNK, so of 12
    refresh(bi);
    const int stop = min(split, bi + kcCHUNK);
    const int stop_full = min(stop, split_full);
    // twelve periods at a time with their ring slots known at compile time
    for (; bi + 12 <= stop_full; bi += 12) {
      const int lane0 = bi - cs;
      unsigned long long evg[NX];
#pragma unroll
      for (int x = 0; x < NX; ++x) evg[x] = ev[x] >> lane0;
      period_c(ItemsTag<0>{}, lane0, evg);
      period_c(ItemsTag<1>{}, lane0, evg);
      period_c(ItemsTag<2>{}, lane0, evg);
      period_c(ItemsTag<3>{}, lane0, evg);
      period_c(ItemsTag<4>{}, lane0, evg);
      period_c(ItemsTag<5>{}, lane0, evg);
      period_c(ItemsTag<6>{}, lane0, evg);
      period_c(ItemsTag<7>{}, lane0, evg);
      period_c(ItemsTag<8>{}, lane0, evg);
      period_c(ItemsTag<9>{}, lane0, evg);
      period_c(ItemsTag<10>{}, lane0, evg);
      period_c(ItemsTag<11>{}, lane0, evg);
    }
    for (; bi < stop_full; ++bi) period(bi, RangeTag<false>{}, ItemsTag<2>{}, RangeTag<true>{});
    for (; bi < stop; ++bi) period(bi, RangeTag<false>{}, ItemsTag<2>{}, RangeTag<false>{});
  }
  if (bi < nblk) period(bi++, RangeTag<true>{}, ItemsTag<1>{}, RangeTag<false>{});
  for (; bi < nblk; ++bi) period(bi, RangeTag<true>{}, ItemsTag<0>{}, RangeTag<false>{});
  // P V of the last range block, then stage B of the last block's items,
  // after every wave has finished the previous block's updates
  range_pv(vring + (size_t)((vslot + kcVSLOTS - 1) & (kcVSLOTS - 1)) * kcHALF);
  barrier_keep_loads();
  if (any_pend()) finish_items(vring + (size_t)((vslot + kcVSLOTS - 1) & (kcVSLOTS - 1)) * kcHALF, RangeTag<false>{});
  __syncthreads();  // every accumulator update is in LDS

  // ------------------------------------------------------------ combine
  // Every global load of the epilogue (gates, compressed-branch output of both
  // column groups) is issued before the first store: the stores may alias
  // them as far as the compiler knows, so loads placed after a store would
  // each wait a full memory round trip.
  const T* gates = (const T*)args.gates;
  T* out = (T*)args.out;
  // The epilogue's row coordinates are recomputed here from values the
  // compiler cannot see through, so the addresses of the setup's loads are not
  // kept alive (in scratch) across the walk for reuse.
  int tpe[NCG], he = h, cle = col, ae = a;
  asm volatile("" : "+v"(he), "+v"(cle), "+v"(ae));
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    tpe[cg] = tpos[cg];
    asm volatile("" : "+v"(tpe[cg]));
  }
  float gcv[NCG], gsv[NCG], gwv[NCG];
  f32x4 ocv[NCG][MT];
  // (unconditional loads, selected afterwards: the compressed output's buffer
  // always exists, unwritten where unused, so it is never multiplied in)
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int te = tpe[cg];
    const T* grow = gates + (((size_t)b * s.T + te) * s.Hq + he) * 3;
    gcv[cg] = to_f32(grow[0]);
    gsv[cg] = to_f32(grow[1]);
    gwv[cg] = to_f32(grow[2]);
    const size_t obase = ((size_t)b * s.T + te) * q_row + (size_t)he * kcD;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ocv[cg][mt] = load4((const T*)args.o_cmp + obase + mt * 16 + 4 * ae);
  }
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const bool ld = cmp_on && tpe[cg] >= kBlock - 1;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) ocv[cg][mt][rr] = ld ? ocv[cg][mt][rr] : 0.f;
    gcv[cg] = cmp_on ? gcv[cg] : 0.f;
    gsv[cg] = sel_on ? gsv[cg] : 0.f;
    gwv[cg] = win_on ? gwv[cg] : 0.f;
  }
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int r0 = 16 * (NCG * w + cg) + cle;
    const float* arow = accL + r0 * ACC;
    const float ls = xsum4(l_s[cg]) + (need_sel ? arow[kcD] : 0.f);
    const float lw = xsum4(l_w[cg]);
    const int te = tpe[cg];
    const float iw = win_on ? gwv[cg] / lw : 0.f;
    const float ilw = win_on ? 1.f / lw : 0.f;
    const float il = need_sel ? 1.f / ls : 0.f;
    const size_t obase = ((size_t)b * s.T + te) * q_row + (size_t)he * kcD;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int d0 = mt * 16 + 4 * ae;
      f32x4 res = acc_w[cg][mt] * iw + ocv[cg][mt] * gcv[cg];
      if (args.o_win) store4((T*)args.o_win + obase + d0, acc_w[cg][mt] * ilw);
      if (need_sel) {
        f32x4 sacc = acc_s[cg][mt];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) sacc[rr] += arow[d0 + rr];
        const f32x4 os = sacc * il;
        if (sel_on) res += os * gsv[cg];
        if (args.o_sel) store4((T*)args.o_sel + obase + d0, os);
      }
      store4(out + obase + d0, res);
    }
    if (args.lse && ae == 0) args.lse[((size_t)b * s.Hq + he) * s.T + te] = (mr_s[cg] + __log2f(ls)) * kLn2;
    if (args.lse_win && ae == 0)
      args.lse_win[((size_t)b * s.Hq + he) * s.T + te] = win_on ? (mr_w[cg] + __log2f(lw)) * kLn2 : -INF;
  }
}

hipError_t launch_sel_compact(const Shape& s, const SelWinArgs& args, hipStream_t st) {
  const size_t lds = sel_compact_lds_bytes(s.T);
  hipError_t e = hipFuncSetAttribute((const void*)sel_compact_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int NBG = s.B * s.Hkv;
  const int NTL = s.T / kcP;
  int n = NTL * NBG;
  if (8 % NBG == 0) n = (n + 7) / 8 * 8;  // whole XCD rounds; the padding returns at once
  hipLaunchKernelGGL(sel_compact_kernel, dim3(n), dim3(kcNT), lds, st, s, args);
  return hipGetLastError();
}

}  // namespace nsa
