// bwd_dkdv.hip -- B3: dk and dv of the selection branch, key-stationary, and
// B4: the deterministic reduction of the partial sums.
//
// [SIC] "Sparsity is Cool", Method (NSA implementation): the selection-branch
// backward as two passes; this key/value-stationary pass gives dk and dv with
// no atomics.  With P_s = exp(tau q.k_s - lse), dP_s = dOs.v_s, Delta =
// dOs.o_sel and dS_s = P_s (dP_s - Delta), summed over the (position, head)
// rows whose position selected the key's block and is causally after it:
//   dk_s = tau sum dS_s q,   dv_s = sum P_s dOs.
//
// Work item: (key block j, range of query tiles, KV group g, batch b).  The
// item's rows come from the reverse map (per 64-position tile, the mask of
// positions that selected j), compacted into an ascending position list in
// LDS.  Its G heads make G consecutive rows; the rows are cut into chunks of
// 32 that the waves of the workgroup take round-robin.  Every wave owns all
// 64 keys (dk and dv accumulate in MFMA registers) and stages its own chunks
// (q, dOs, lse, Delta) with global_load_lds into a private LDS ring, so the
// chunk loop has no workgroup barrier.  Rows sit in LDS row-major with a
// 16-byte-slot XOR swizzle; the 32-row x 16-channel operands of the row
// contractions come from the transposing LDS read.  Per chunk and 16-key
// subtile v (K and V fragments of the backward block image, staged once):
//   S = Q K^T, dP = dOs V^T  (rows permuted so that the C layout is the A
//                             layout of P^T and dS^T)
//   P = exp2(tau log2(e) S - lse2), dS = P (dP - Delta)
//   dV += P^T dOs, dK += dS^T Q    (32-row contractions)
// At the end the waves' accumulators are summed through LDS; an item that is
// the only one of its block writes dk / dv, the others write fp32 partials
// (MFMA fragment order) that B4 adds in item order.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

// ------------------------------------------------------------------ items
// The rows of block j are the positions that selected it (ascending, from the
// reverse map) times the G heads of the group.  A block's position list is
// cut into items of about kItemRows rows (at most kMaxItemPos positions, the
// LDS list of the dk/dv kernel); blocks with several items get one partial
// slot per item.
struct Item {
  int bg, j, lo, hi, slot;  // (batch, group) index, block, rows [lo, hi), partial slot or -1
  int mode;                 // KV_SEL: [lo, hi) indexes the block's position list;
                            // KV_WIN, KV_CMP: positions lo .. hi - 1 themselves
};

// Branch of a dk/dv item: selection rows (position lists), window rows
// (positions 64 j .. 64 j + 62 + W) or compression rows (positions from
// 64 (64 j + 1) - 1 on) against the pooled-key block j (pooled keys 64 j ..).
enum { KV_SEL = 0, KV_WIN = 1, KV_CMP = 2 };

// key (a token index, or a pooled-key index for KV_CMP) visible to row position t
__device__ __forceinline__ bool kv_allowed(int mode, int key, int t, int W) {
  if (mode == KV_SEL) return key <= t;
  if (mode == KV_WIN) return key <= t && key > t - W;
  return key < (t + 1) / kBlock;
}
// whether a chunk of rows with positions first .. last (ascending) needs the
// element mask against block j
__device__ __forceinline__ bool kv_chunk_masked(int mode, int j, int first, int last, int W) {
  if (mode == KV_SEL) return first < j * kBlock + kBlock - 1;
  if (mode == KV_WIN) return first < j * kBlock + kBlock - 1 || last >= j * kBlock + W;
  return (first + 1) / kBlock < j * kBlock + kBlock;
}

// Arguments of the dk/dv kernels: per-branch log-sum-exp, Delta and dOs
// (indexed by the item's mode), the block images and the pooled-key images.
struct KvArgs {
  const void* q;
  const unsigned char* img;
  const unsigned char* pimg;
  const uint16_t* lists;
  const float* lse[3];
  const float* delta[3];
  const void* dos[3];
  const int* nitems;
  void* dk;
  void* dv;
  float* part;
};

constexpr int kItemRows = 2048;
constexpr int kMaxItemPos = 2048;

__host__ __device__ inline int items_of(int npos, int G) {
  int n = (npos * G + kItemRows - 1) / kItemRows;
  const int m = (npos + kMaxItemPos - 1) / kMaxItemPos;
  n = n > m ? n : m;
  return n > 1 ? n : 1;
}

// rows of the window and compression items of block j (positions)
__host__ __device__ inline int win_positions(int j, int T, int W) {
  const int hi = j * kBlock + kBlock - 1 + W < T ? j * kBlock + kBlock - 1 + W : T;
  return hi - j * kBlock;
}
__host__ __device__ inline int cmp_first_position(int J) { return kBlock * (kBlock * J + 1) - 1; }

// Upper bound on the item count (grid size; workspace): a selection block has
// at most 1 + rows / kItemRows items and every position selects at most top_k
// blocks; window and compression items are counted exactly.
int bwd_item_bound(const Shape& s, bool full) {
  const long nblk = s.T / kBlock;
  const long rows = (long)s.T * s.topk * s.G;
  long n = nblk + (rows + kItemRows - 1) / kItemRows;
  if (full) {
    for (int j = 0; j < nblk; ++j) n += items_of(win_positions(j, s.T, s.W), s.G);
    for (int J = 0; J * kBlock < s.nc; ++J) {
      const int pc = s.T - cmp_first_position(J);
      if (pc > 0) n += items_of(pc, s.G);
    }
  }
  return (int)((long)s.B * s.Hkv * n);
}

// B1b: grid (nblk, Hkv, B), 256 threads.  Ascending positions that selected
// block j -> lists[b][g][j][0 .. P_j) (capacity T), counts[b][g][j] = P_j.
__global__ __launch_bounds__(256) void bwd_lists_kernel(Shape s, const uint64_t* __restrict__ revmap,
                                                        uint16_t* __restrict__ lists,
                                                        int* __restrict__ counts) {
  __shared__ uint64_t msk[256];
  __shared__ int off[256];
  __shared__ int wsum[4];
  __shared__ int carry;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nblk = s.T / kBlock;
  const size_t e = ((size_t)b * s.Hkv + g) * nblk + j;
  const uint64_t* rm = revmap + e * nblk;
  uint16_t* out = lists + e * (size_t)s.T;
  const int x = threadIdx.x, w = x / 64, l = x % 64;
  if (x == 0) carry = 0;
  __syncthreads();
  for (int c0 = j; c0 < nblk; c0 += 256) {
    const uint64_t m = c0 + x < nblk ? rm[c0 + x] : 0ull;
    const int n = __popcll(m);
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (l >= o) incl += y;
    }
    if (l == 63) wsum[w] = incl;
    msk[x] = m;
    __syncthreads();
    int pre = carry;
    for (int k = 0; k < w; ++k) pre += wsum[k];
    off[x] = pre + incl - n;
    __syncthreads();
    if (x == 255) carry = pre + incl;
    const int nt = min(256, nblk - c0);
    for (int ti = w; ti < nt; ti += 4) {
      const uint64_t mm = msk[ti];
      if ((mm >> l) & 1ull) out[off[ti] + __popcll(mm & ((1ull << l) - 1ull))] = (uint16_t)((c0 + ti) * kBlock + l);
    }
    __syncthreads();
  }
  if (x == 0) counts[e] = carry;
}

// B1c: one workgroup.  Items of every (batch, group, block) in natural order
// (block-major): the block's selection items, then (full) its window items
// and, for j a multiple of 64, the compression items of pooled-key block j / 64.
// slot_base / slot_cnt per block (selection-only: -1 / 1 for a single item,
// written directly); slot_base_c / slot_cnt_c per pooled-key block (full).
__global__ __launch_bounds__(1024) void bwd_items_kernel(int NJ, int nblk, int G, int T, int W, int full,
                                                        const int* __restrict__ counts,
                                                        Item* __restrict__ items, int* __restrict__ slot_base,
                                                        int* __restrict__ slot_cnt, int* __restrict__ slot_base_c,
                                                        int* __restrict__ slot_cnt_c, int* __restrict__ nitems) {
  __shared__ int wtot[2][16];
  __shared__ int carry[2];
  const int x = threadIdx.x, w = x / 64, l = x % 64;
  const int NJc = (nblk + kBlock - 1) / kBlock;
  if (x == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int e0 = 0; e0 < NJ; e0 += 1024) {
    const int e = e0 + x;
    const int j = e % nblk;
    const int P = e < NJ ? counts[e] : 0;
    const int ns = e < NJ ? items_of(P, G) : 0;
    const int pw = full ? win_positions(j, T, W) : 0;
    const int nw = e < NJ && full ? items_of(pw, G) : 0;
    const int pc = full && j % kBlock == 0 ? T - cmp_first_position(j / kBlock) : 0;
    const int nc = e < NJ && pc > 0 ? items_of(pc, G) : 0;
    const int n = ns + nw + nc;
    const int sl = full ? n : (ns > 1 ? ns : 0);
    int in = n, is = sl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(in, o), z = __shfl_up(is, o);
      if (l >= o) { in += y; is += z; }
    }
    if (l == 63) { wtot[0][w] = in; wtot[1][w] = is; }
    __syncthreads();
    int pi = carry[0], ps = carry[1];
    for (int k = 0; k < w; ++k) { pi += wtot[0][k]; ps += wtot[1][k]; }
    const int io = pi + in - n, so = ps + is - sl;
    if (e < NJ) {
      const int bg = e / nblk;
      slot_base[e] = sl > 0 ? so : -1;
      slot_cnt[e] = ns + nw;
      if (full && j % kBlock == 0) {
        slot_base_c[bg * NJc + j / kBlock] = so + ns + nw;
        slot_cnt_c[bg * NJc + j / kBlock] = nc;
      }
      int k = io;
      for (int i = 0; i < ns; ++i, ++k) {
        Item it;
        it.bg = bg; it.j = j; it.mode = KV_SEL;
        it.lo = P * i / ns;  // P <= 65536, n <= P: no overflow
        it.hi = P * (i + 1) / ns;
        it.slot = sl > 0 ? so + i : -1;
        items[k] = it;
      }
      for (int i = 0; i < nw; ++i, ++k) {
        Item it;
        it.bg = bg; it.j = j; it.mode = KV_WIN;
        it.lo = j * kBlock + pw * i / nw;
        it.hi = j * kBlock + pw * (i + 1) / nw;
        it.slot = so + ns + i;
        items[k] = it;
      }
      for (int i = 0; i < nc; ++i, ++k) {
        Item it;
        it.bg = bg; it.j = j / kBlock; it.mode = KV_CMP;
        it.lo = cmp_first_position(j / kBlock) + pc * i / nc;
        it.hi = cmp_first_position(j / kBlock) + pc * (i + 1) / nc;
        it.slot = so + ns + nw + i;
        items[k] = it;
      }
    }
    __syncthreads();
    if (x == 1023) { carry[0] = pi + in; carry[1] = ps + is; }
    __syncthreads();
  }
  if (x == 0) *nitems = carry[0];
}

// ------------------------------------------------------------------ B3
template <typename T, int D, int G>
struct KvCfg {
  typedef BwdImage<T, D> Img;
  static constexpr bool WIDE = D == 128 || sizeof(T) == 4;
  static constexpr int NW = WIDE ? 3 : 4;             // waves per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int CR = 32;                       // rows per chunk
  static constexpr int CP = CR / G;                   // positions per chunk
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES;                 // bytes of one row
  static constexpr int SLOTS = ROWB / 16;             // 16-byte slots per row
  static constexpr int TB = CR * ROWB;                // bytes of one tensor's chunk
  static constexpr int NLD = TB / 1024;               // 1 KB loads per tensor and chunk
  static constexpr int RPI = 1024 / ROWB;             // rows per 1 KB load
  static constexpr int LQ = 2 * NLD + 1;              // loads per chunk (q, dOs, lse | Delta)
  static constexpr int STAGE = 2 * TB + 256;
  static constexpr int NR = WIDE ? 2 : 3;             // ring stages per wave
  static constexpr int NFRAG = Img::NFRAG, NV = Img::NV;
  static constexpr int FRAG_BYTES = NV * 1024;
  static constexpr int KVB = 2 * NFRAG * FRAG_BYTES;  // K and V fragments of the block image
  static constexpr int KS = D / 32, MT = D / 16;
  static constexpr int NFR = 4 * MT;                  // accumulator fragments per tensor
  static constexpr int MAXPOS = kMaxItemPos;
  static constexpr size_t RING = (size_t)NW * NR * STAGE;
  static constexpr size_t LDS = KVB + RING + MAXPOS * 2;
  static_assert(CP >= 1 && CP * G == CR, "a chunk holds whole positions");
  static_assert(RING >= (size_t)NW * NFR * 1024, "reduction fits in the ring");
  static_assert((NR - 1) * LQ < 64, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

// swizzle of the 16-byte slots of chunk row R (low three slot bits)
__device__ __forceinline__ int row_swz(int R) { return (R & 7) ^ (((R >> 3) & 1) << 2); }

// 8 consecutive elements (channel ch, a multiple of 8) of chunk row R
template <typename T, int ROWB>
__device__ __forceinline__ typename Frag<T>::type row_frag(const unsigned char* base, int R, int ch);
template <>
__device__ __forceinline__ bf16x8 row_frag<bf16, 128>(const unsigned char* base, int R, int ch) {
  const int c = ch >> 3;
  return *reinterpret_cast<const bf16x8*>(base + R * 128 + ((c ^ row_swz(R)) << 4));
}
template <>
__device__ __forceinline__ bf16x8 row_frag<bf16, 256>(const unsigned char* base, int R, int ch) {
  const int c = ch >> 3;
  return *reinterpret_cast<const bf16x8*>(base + R * 256 + (((c & 8) | ((c & 7) ^ row_swz(R))) << 4));
}
template <>
__device__ __forceinline__ f32x8 row_frag<float, 256>(const unsigned char* base, int R, int ch) {
  const int c0 = ch >> 2, c1 = c0 + 1;
  const f32x4 x = *reinterpret_cast<const f32x4*>(base + R * 256 + (((c0 & 8) | ((c0 & 7) ^ row_swz(R))) << 4));
  const f32x4 y = *reinterpret_cast<const f32x4*>(base + R * 256 + (((c1 & 8) | ((c1 & 7) ^ row_swz(R))) << 4));
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = x[i]; r[4 + i] = y[i]; }
  return r;
}

// B fragment of a 32-row x 16-channel tile (channels 16 m ..): lane (a, col)
// gets rows 8a + e, channel 16 m + col.  bf16: two transposing LDS reads (in
// each 16-lane group, lane i receives element i % 4 of the 8 bytes addressed
// by lanes 4e + i / 4, e = 0..3); fp32: element loads.
template <typename T, int ROWB>
__device__ __forceinline__ typename Frag<T>::type col_frag(const unsigned char* base, int l, int m);
template <int ROWB>
__device__ __forceinline__ bf16x8 col_frag_bf16(const unsigned char* base, int l, int m) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int a = l >> 4, L = l & 15;
  const int c = 2 * m + ((L & 3) >> 1);
  s16x4 h[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int R = 8 * a + 4 * hh + (L >> 2);
    const int slot = ROWB == 128 ? (c ^ row_swz(R)) : ((c & 8) | ((c & 7) ^ row_swz(R)));
    const unsigned char* p = base + R * ROWB + (slot << 4) + ((L & 1) << 3);
    h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) unsigned char*)(p)));
  }
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  s16x8 r = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, r);
}
template <>
__device__ __forceinline__ bf16x8 col_frag<bf16, 128>(const unsigned char* base, int l, int m) {
  return col_frag_bf16<128>(base, l, m);
}
template <>
__device__ __forceinline__ bf16x8 col_frag<bf16, 256>(const unsigned char* base, int l, int m) {
  return col_frag_bf16<256>(base, l, m);
}
template <>
__device__ __forceinline__ f32x8 col_frag<float, 256>(const unsigned char* base, int l, int m) {
  const int a = l >> 4, col = l & 15;
  const int ch = 16 * m + col, c = ch >> 2;
  f32x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int R = 8 * a + e;
    r[e] = *reinterpret_cast<const float*>(base + R * 256 + (((c & 8) | ((c & 7) ^ row_swz(R))) << 4) +
                                           ((ch & 3) << 2));
  }
  return r;
}

// B fragment (32 rows x 16 channels, bf16) by two transposing reads at the
// precomputed lane offsets of its two 4-row halves
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* base, const int (&off)[2]) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) unsigned char*)(base + off[0])));
  const s16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) unsigned char*)(base + off[1])));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 r = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <typename T, int D, int G>
__global__ __launch_bounds__((KvCfg<T, D, G>::NT), 1) void bwd_dkdv_kernel(
    Shape s, const Item* __restrict__ items, KvArgs args) {
  typedef KvCfg<T, D, G> C;
  constexpr int NW = C::NW, NT = C::NT, CP = C::CP, TB = C::TB, NLD = C::NLD, RPI = C::RPI;
  constexpr int SLOTS = C::SLOTS, LQ = C::LQ, STAGE = C::STAGE, NR = C::NR;
  constexpr int NFRAG = C::NFRAG, FRAG_BYTES = C::FRAG_BYTES, KVB = C::KVB;
  constexpr int KS = C::KS, MT = C::MT, NFR = C::NFR, ROWB = C::ROWB;
  typedef typename Frag<T>::type FragT;
  typedef typename BwdImage<T, D>::K KI;
  const float INF = __builtin_inff();

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kv = smem;                                    // [KVB]
  unsigned char* ring = smem + KVB;                            // [NW][NR][STAGE]
  uint16_t* plist = reinterpret_cast<uint16_t*>(ring + C::RING);  // [MAXPOS]

  // items in block-major order (an XCD-interleaved order measured slower)
  if ((int)blockIdx.x >= *args.nitems) return;
  const Item it = items[blockIdx.x];
  const int mode = it.mode;
  const T* __restrict__ q = (const T*)args.q;
  const float* __restrict__ lse = args.lse[mode];
  const float* __restrict__ delta = args.delta[mode];
  const T* __restrict__ dos = (const T*)args.dos[mode];
  T* __restrict__ dk = (T*)args.dk;
  T* __restrict__ dv = (T*)args.dv;
  float* __restrict__ part = args.part;
  const int Wn = s.W;
  const int nblk = s.T / kBlock;
  const int g = it.bg % s.Hkv, b = it.bg / s.Hkv;
  const int j = it.j;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = threadIdx.x % kWave;
  const int a = l >> 4, col = l & 15;
  const float c1 = s.scale * kLog2e;
  const size_t q_row = (size_t)s.Hq * D;

  // K and V fragments of block j (first 2 NFRAG fragments of its backward image)
  {
    const unsigned char* src =
        (mode == KV_CMP ? args.pimg + ((size_t)it.bg * ((s.nc + kBlock - 1) / kBlock) + j) * (size_t)BwdImage<T, D>::BYTES
                        : args.img + ((size_t)it.bg * nblk + j) * (size_t)BwdImage<T, D>::BYTES) + 16 * l;
    for (int pc = w; pc < KVB / 1024; pc += NW)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)pc * 1024), (void*)(kv + (size_t)pc * 1024),
                                       16, 0, 0);
  }
  // the item's slice of the block's ascending position list
  const int npos = it.hi - it.lo;
  {
    if (mode == KV_SEL) {
      const uint16_t* src = args.lists + ((size_t)it.bg * nblk + j) * (size_t)s.T + it.lo;
      for (int i = threadIdx.x; i < npos; i += NT) plist[i] = src[i];
    } else {
      for (int i = threadIdx.x; i < npos; i += NT) plist[i] = (uint16_t)(it.lo + i);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  f32x4 adk[NFR], adv[NFR];
#pragma unroll
  for (int i = 0; i < NFR; ++i) { adk[i] = zero4(); adv[i] = zero4(); }

  const int nch = (npos + CP - 1) / CP;
  const int my_n = nch > w ? (nch - w + NW - 1) / NW : 0;
  unsigned char* wring = ring + (size_t)w * NR * STAGE;

  auto issue_chunk = [&](int ck, int stage) {
    unsigned char* st = wring + (size_t)stage * STAGE;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int R = n * RPI + l / SLOTS, sl = l % SLOTS;
      const int qi = ck * CP + R / G;
      const int t = plist[qi < npos ? qi : 0];
      const int h = g * G + R % G;
      const int c = (sl & ~7) | ((sl & 7) ^ row_swz(R));
      const size_t off = ((size_t)b * s.T + t) * q_row + (size_t)h * D + c * (16 / sizeof(T));
      __builtin_amdgcn_global_load_lds((const void*)(q + off), (void*)(st + n * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(dos + off), (void*)(st + TB + n * 1024), 16, 0, 0);
    }
    {
      const int R = l & 31;
      const int qi = ck * CP + R / G;
      const int t = plist[qi < npos ? qi : 0];
      const int h = g * G + R % G;
      const float* src = (l < 32 ? lse : delta) + ((size_t)b * s.Hq + h) * s.T + t;
      __builtin_amdgcn_global_load_lds((const void*)src, (void*)(st + 2 * TB), 4, 0, 0);
    }
  };

  for (int i = 0; i < NR - 1 && i < my_n; ++i) issue_chunk(w + i * NW, i);
  for (int i = 0; i < my_n; ++i) {
    const int ck = w + i * NW;
    if (i + NR - 1 < my_n) {
      lds_fence();
      issue_chunk(w + (i + NR - 1) * NW, (i + NR - 1) % NR);
      wait_vmcnt<(NR - 1) * LQ>();
    } else {
      wait_vmcnt<0>();
    }
    lds_fence();
    const unsigned char* st = wring + (size_t)(i % NR) * STAGE;
    const unsigned char* qs = st;
    const unsigned char* ds = st + TB;
    const float* meta = reinterpret_cast<const float*>(st + 2 * TB);

    // rows 8a + e of this lane: log2-domain lse (+inf for rows past the list) and Delta
    float lr[8], dl[8];
    {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(meta + 8 * a);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(meta + 8 * a + 4);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(meta + 32 + 8 * a);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(meta + 32 + 8 * a + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lr[e] = l0[e] * kLog2e;
        lr[4 + e] = l1[e] * kLog2e;
        dl[e] = d0[e];
        dl[4 + e] = d1[e];
      }
    }
    const bool full = (ck + 1) * CP <= npos;
    if (!full) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ck * CP + (8 * a + e) / G >= npos) lr[e] = INF;
    }
    const bool masked = kv_chunk_masked(mode, j, __builtin_amdgcn_readfirstlane(plist[ck * CP]),
                                        __builtin_amdgcn_readfirstlane(plist[min(ck * CP + CP, npos) - 1]), Wn);

    // A fragments of Q and dOs for the two row subtiles (row 8(rho/4) + 4u + rho%4)
    FragT qa[2][KS], da[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int R = 8 * (col >> 2) + 4 * u + (col & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[u][ks] = row_frag<T, ROWB>(qs, R, ks * 32 + 8 * a);
        da[u][ks] = row_frag<T, ROWB>(ds, R, ks * 32 + 8 * a);
      }
    }
    FragT pf[4], sf[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      // dP accumulates onto -Delta of each element's row: dP - Delta comes out of the MFMA
      f32x4 sv[2] = {zero4(), zero4()};
      f32x4 dp[2] = {f32x4{-dl[0], -dl[1], -dl[2], -dl[3]}, f32x4{-dl[4], -dl[5], -dl[6], -dl[7]}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FragT kf = lds_frag<T>(kv + (size_t)(4 * ks + v) * FRAG_BYTES, l);
        const FragT vf = lds_frag<T>(kv + (size_t)(NFRAG + 4 * ks + v) * FRAG_BYTES, l);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          sv[u] = mma(sv[u], qa[u][ks], kf);
          dp[u] = mma(dp[u], da[u][ks], vf);
        }
      }
      float p[8], x[8];
      if (!masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(sv[e >> 2][e & 3] * c1 - lr[e]);
          x[e] = p[e] * dp[e >> 2][e & 3];
        }
      } else {
        const int key = j * kBlock + KI::krow(v, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qi = ck * CP + (8 * a + e) / G;
          const int t = plist[qi < npos ? qi : 0];
          p[e] = kv_allowed(mode, key, t, Wn) ? fast_exp2(sv[e >> 2][e & 3] * c1 - lr[e]) : 0.f;
          x[e] = p[e] * dp[e >> 2][e & 3];
        }
      }
      pf[v] = Frag<T>::from_f32(p);
      sf[v] = Frag<T>::from_f32(x);
    }
    // dV += P^T dOs, dK += dS^T Q over the chunk's 32 rows
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const FragT dt = col_frag<T, ROWB>(ds, l, m);
      const FragT qt = col_frag<T, ROWB>(qs, l, m);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        adv[v * MT + m] = mma(adv[v * MT + m], pf[v], dt);
        adk[v * MT + m] = mma(adk[v * MT + m], sf[v], qt);
      }
    }
  }

  // sum the waves' accumulators through LDS (the rings are free now) and write:
  // the only item of a block writes dk / dv (rows staged in LDS for 16-byte
  // stores), the others their fp32 partial in fragment order
  __syncthreads();
  float* red = reinterpret_cast<float*>(ring);
  constexpr int OWN = (NFR + NW - 1) / NW;  // fragments summed per wave
  const size_t k_row = (size_t)s.Hkv * D;
#pragma unroll
  for (int tns = 0; tns < 2; ++tns) {
#pragma unroll
    for (int fi = 0; fi < NFR; ++fi)
      *reinterpret_cast<f32x4*>(red + ((size_t)(w * NFR + fi) * 64 + l) * 4) = tns == 0 ? adk[fi] : adv[fi];
    __syncthreads();
    f32x4 sum[OWN];
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int fi = w + o * NW;
      sum[o] = zero4();
      if (fi < NFR)
        for (int w2 = 0; w2 < NW; ++w2) sum[o] += *reinterpret_cast<const f32x4*>(red + ((size_t)(w2 * NFR + fi) * 64 + l) * 4);
    }
    __syncthreads();
    if (it.slot >= 0) {
      float* ps = part + ((size_t)it.slot * 2 + tns) * (size_t)NFR * 256;
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int fi = w + o * NW;
        if (fi < NFR) *reinterpret_cast<f32x4*>(ps + ((size_t)fi * 64 + l) * 4) = sum[o];
      }
    } else {
      const float sc = tns == 0 ? s.scale : 1.f;
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int fi = w + o * NW;
        if (fi < NFR) {
          const int v = fi / MT, m = fi % MT;
#pragma unroll
          for (int r = 0; r < 4; ++r) red[KI::krow(v, 4 * a + r) * D + 16 * m + col] = sum[o][r] * sc;
        }
      }
      __syncthreads();
      T* dst = (tns == 0 ? dk : dv) + ((size_t)b * s.T + j * kBlock) * k_row + (size_t)g * D;
      for (int i = threadIdx.x; i < kBlock * D / 8; i += NT) {
        const int kk = i / (D / 8), c8 = (i % (D / 8)) * 8;
        store8(dst + (size_t)kk * k_row + c8, red + kk * D + c8);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ B3, paired waves
// bf16 at head_dim 64: eight waves, two per SIMD.  Waves w and w + 4 form pair
// p = w % 4 (same SIMD) and split the block's keys: wave half kh = w / 4 owns
// the 16-key subtiles 2 kh and 2 kh + 1 (dK, dV accumulators: 64 fp32 per
// lane).  Pair p takes chunks p, p + 4, ... (one per round); its two waves
// stage each chunk together (q + lse | Delta by the first, dOs by the second)
// into the pair's LDS ring, and one workgroup barrier per round publishes the
// round's chunks and frees the previous round's stages.
template <typename T, int D, int G>
struct KvPairCfg {
  typedef BwdImage<T, D> Img;
  static constexpr int NW = 8, NT = NW * 64, NP = 4;   // waves, pairs
  static constexpr int CR = 32, CP = CR / G;
  static constexpr int ES = sizeof(T);
  static constexpr int ROWB = D * ES, SLOTS = ROWB / 16, TB = CR * ROWB;
  static constexpr int NLD = TB / 1024, RPI = 1024 / ROWB;
  static constexpr int STAGE = 2 * TB + 256;
  static constexpr int NR = 4;                          // ring stages per pair
  static constexpr int L0 = NLD + 1, L1 = NLD;          // loads per chunk of key halves 0 and 1
  static constexpr int NFRAG = Img::NFRAG, NV = Img::NV;
  static constexpr int FRAG_BYTES = NV * 1024;
  static constexpr int KVB = 2 * NFRAG * FRAG_BYTES;
  static constexpr int KS = D / 32, MT = D / 16;
  static constexpr int NFW = 2 * MT;                    // accumulator fragments per tensor and wave
  static constexpr int NFR = 4 * MT;                    // accumulator fragments per tensor and block
  static constexpr int MAXPOS = kMaxItemPos;
  static constexpr size_t RING = (size_t)NP * NR * STAGE;
  static constexpr size_t LDS = KVB + RING + MAXPOS * 2;
  static_assert(CP >= 1 && CP * G == CR, "a chunk holds whole positions");
  static_assert(RING >= (size_t)NW * NFW * 1024 && RING >= (size_t)kBlock * D * 4, "reduction fits in the ring");
  static_assert((NR - 2) * L0 < 64, "vmcnt range");
  static_assert(LDS <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int G>
__global__ __launch_bounds__((KvPairCfg<T, D, G>::NT)) void bwd_dkdv_pair_kernel(
    Shape s, const Item* __restrict__ items, KvArgs args) {
  typedef KvPairCfg<T, D, G> C;
  constexpr int NT = C::NT, NP = C::NP, CP = C::CP, TB = C::TB, NLD = C::NLD, RPI = C::RPI;
  constexpr int SLOTS = C::SLOTS, STAGE = C::STAGE, NR = C::NR, L0 = C::L0, L1 = C::L1;
  constexpr int NFRAG = C::NFRAG, FRAG_BYTES = C::FRAG_BYTES, KVB = C::KVB;
  constexpr int KS = C::KS, MT = C::MT, NFW = C::NFW, NFR = C::NFR, ROWB = C::ROWB;
  typedef typename Frag<T>::type FragT;
  typedef typename BwdImage<T, D>::K KI;
  const float INF = __builtin_inff();

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* kv = smem;                                        // [KVB]
  unsigned char* ring = smem + KVB;                                // [NP][NR][STAGE]
  uint16_t* plist = reinterpret_cast<uint16_t*>(ring + C::RING);  // [MAXPOS]

  if ((int)blockIdx.x >= *args.nitems) return;
  const Item it = items[blockIdx.x];
  const int mode = it.mode;
  const T* __restrict__ q = (const T*)args.q;
  const float* __restrict__ lse = args.lse[mode];
  const float* __restrict__ delta = args.delta[mode];
  const T* __restrict__ dos = (const T*)args.dos[mode];
  T* __restrict__ dk = (T*)args.dk;
  T* __restrict__ dv = (T*)args.dv;
  float* __restrict__ part = args.part;
  const int Wn = s.W;
  const int nblk = s.T / kBlock;
  const int g = it.bg % s.Hkv, b = it.bg / s.Hkv;
  const int j = it.j;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int pr = w % NP, kh = w / NP;
  const int l = threadIdx.x % kWave;
  const int a = l >> 4, col = l & 15;
  const float c1 = s.scale * kLog2e;
  const size_t q_row = (size_t)s.Hq * D;

  {
    const unsigned char* src =
        (mode == KV_CMP ? args.pimg + ((size_t)it.bg * ((s.nc + kBlock - 1) / kBlock) + j) * (size_t)BwdImage<T, D>::BYTES
                        : args.img + ((size_t)it.bg * nblk + j) * (size_t)BwdImage<T, D>::BYTES) + 16 * l;
    for (int pc = w; pc < KVB / 1024; pc += C::NW)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)pc * 1024), (void*)(kv + (size_t)pc * 1024),
                                       16, 0, 0);
  }
  const int npos = it.hi - it.lo;
  {
    if (mode == KV_SEL) {
      const uint16_t* src = args.lists + ((size_t)it.bg * nblk + j) * (size_t)s.T + it.lo;
      for (int i = threadIdx.x; i < npos; i += NT) plist[i] = src[i];
    } else {
      for (int i = threadIdx.x; i < npos; i += NT) plist[i] = (uint16_t)(it.lo + i);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  f32x4 adk[NFW], adv[NFW];
#pragma unroll
  for (int i = 0; i < NFW; ++i) { adk[i] = zero4(); adv[i] = zero4(); }

  const int nch = (npos + CP - 1) / CP;
  const int rounds = (nch + NP - 1) / NP;
  unsigned char* pring = ring + (size_t)pr * NR * STAGE;
  auto has = [&](int r) { return r * NP + pr < nch; };

  // lane-constant byte offsets inside a staged chunk (row-major, swizzled):
  // A fragments of the row subtiles, transposing reads of the 16-channel tiles
  static_assert(ROWB == 128, "paired kernel: bf16, head_dim 64");
  auto slot_off = [](int R, int c) { return R * 128 + ((c ^ row_swz(R)) << 4); };
  int roff[2][KS], troff[MT][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) roff[u][ks] = slot_off(8 * (col >> 2) + 4 * u + (col & 3), ks * 4 + a);
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      troff[m][hh] = slot_off(8 * a + 4 * hh + (col >> 2), 2 * m + ((col & 3) >> 1)) + ((col & 1) << 3);
  // staging: per 1 KB load n, this lane's row (position index in the chunk,
  // head) and the byte offset of its 16 bytes inside the (position, group) rows
  int ld_pi[NLD], ld_off[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int R = n * RPI + l / SLOTS, sl = l % SLOTS;
    ld_pi[n] = R / G;
    ld_off[n] = ((R % G) * D + ((sl & ~7) | ((sl & 7) ^ row_swz(R))) * (16 / (int)sizeof(T))) * (int)sizeof(T);
  }
  const int mt_pi = (l & 31) / G;
  const float* mt_src = (l < 32 ? lse : delta) + ((size_t)b * s.Hq + g * G + (l & 31) % G) * s.T;
  const unsigned char* grp_q = (const unsigned char*)(q + (size_t)b * s.T * q_row + (size_t)g * G * D);
  const unsigned char* grp_d = (const unsigned char*)(dos + (size_t)b * s.T * q_row + (size_t)g * G * D);

  // this wave's share of the loads of its pair's chunk of round r
  auto issue = [&](int r) {
    if (!has(r)) return;
    const int ck = r * NP + pr;
    unsigned char* st = pring + (size_t)(r % NR) * STAGE;
    const unsigned char* src_t = kh == 0 ? grp_q : grp_d;
    unsigned char* dst_t = st + (kh == 0 ? 0 : TB);
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      const int qi = ck * CP + ld_pi[n];
      const int t = plist[qi < npos ? qi : 0];
      __builtin_amdgcn_global_load_lds((const void*)(src_t + (size_t)t * (q_row * sizeof(T)) + ld_off[n]),
                                       (void*)(dst_t + n * 1024), 16, 0, 0);
    }
    if (kh == 0) {
      const int qi = ck * CP + mt_pi;
      const int t = plist[qi < npos ? qi : 0];
      __builtin_amdgcn_global_load_lds((const void*)(mt_src + t), (void*)(st + 2 * TB), 4, 0, 0);
    }
  };

  for (int r = 0; r < NR - 1; ++r) issue(r);
  for (int r = 0; r < rounds; ++r) {
    // this wave's loads of round r are done when at most the later rounds' remain
    if (has(r + NR - 2)) {
      if (kh == 0) wait_vmcnt<(NR - 2) * L0>();
      else wait_vmcnt<(NR - 2) * L1>();
    } else {
      wait_vmcnt<0>();
    }
    barrier_keep_loads();  // round r's chunks are in LDS; round r-1's stages are free
    issue(r + NR - 1);
    if (!has(r)) continue;
    const int ck = r * NP + pr;
    const unsigned char* st = pring + (size_t)(r % NR) * STAGE;
    const unsigned char* qs = st;
    const unsigned char* ds = st + TB;
    const float* meta = reinterpret_cast<const float*>(st + 2 * TB);

    float lr[8], dl[8];
    {
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(meta + 8 * a);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(meta + 8 * a + 4);
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(meta + 32 + 8 * a);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(meta + 32 + 8 * a + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lr[e] = l0[e] * kLog2e;
        lr[4 + e] = l1[e] * kLog2e;
        dl[e] = d0[e];
        dl[4 + e] = d1[e];
      }
    }
    if ((ck + 1) * CP > npos) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (ck * CP + (8 * a + e) / G >= npos) lr[e] = INF;
    }
    const bool masked = kv_chunk_masked(mode, j, __builtin_amdgcn_readfirstlane(plist[ck * CP]),
                                        __builtin_amdgcn_readfirstlane(plist[min(ck * CP + CP, npos) - 1]), Wn);

    FragT qa[2][KS], da[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qa[u][ks] = *reinterpret_cast<const FragT*>(qs + roff[u][ks]);
        da[u][ks] = *reinterpret_cast<const FragT*>(ds + roff[u][ks]);
      }
    FragT pf[2], sf[2];
#pragma unroll
    for (int vv = 0; vv < 2; ++vv) {
      const int v = 2 * kh + vv;
      // dP accumulates onto -Delta of each element's row: dP - Delta comes out of the MFMA
      f32x4 sv[2] = {zero4(), zero4()};
      f32x4 dp[2] = {f32x4{-dl[0], -dl[1], -dl[2], -dl[3]}, f32x4{-dl[4], -dl[5], -dl[6], -dl[7]}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const FragT kf = lds_frag<T>(kv + (size_t)(4 * ks + v) * FRAG_BYTES, l);
        const FragT vf = lds_frag<T>(kv + (size_t)(NFRAG + 4 * ks + v) * FRAG_BYTES, l);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          sv[u] = mma(sv[u], qa[u][ks], kf);
          dp[u] = mma(dp[u], da[u][ks], vf);
        }
      }
      float p[8], x[8];
      if (!masked) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(sv[e >> 2][e & 3] * c1 - lr[e]);
          x[e] = p[e] * dp[e >> 2][e & 3];
        }
      } else {
        const int key = j * kBlock + KI::krow(v, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qi = ck * CP + (8 * a + e) / G;
          const int t = plist[qi < npos ? qi : 0];
          p[e] = kv_allowed(mode, key, t, Wn) ? fast_exp2(sv[e >> 2][e & 3] * c1 - lr[e]) : 0.f;
          x[e] = p[e] * dp[e >> 2][e & 3];
        }
      }
      pf[vv] = Frag<T>::from_f32(p);
      sf[vv] = Frag<T>::from_f32(x);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const FragT dt = tr_frag(ds, troff[m]);
      const FragT qt = tr_frag(qs, troff[m]);
#pragma unroll
      for (int vv = 0; vv < 2; ++vv) {
        adv[vv * MT + m] = mma(adv[vv * MT + m], pf[vv], dt);
        adk[vv * MT + m] = mma(adk[vv * MT + m], sf[vv], qt);
      }
    }
  }

  // sum the four pairs' accumulators through LDS and write (as the 4-wave kernel)
  __syncthreads();
  float* red = reinterpret_cast<float*>(ring);
  const size_t k_row = (size_t)s.Hkv * D;
#pragma unroll
  for (int tns = 0; tns < 2; ++tns) {
#pragma unroll
    for (int fi = 0; fi < NFW; ++fi)
      *reinterpret_cast<f32x4*>(red + ((size_t)(w * NFW + fi) * 64 + l) * 4) = tns == 0 ? adk[fi] : adv[fi];
    __syncthreads();
    // output fragment of = w, w + 8 (of NFR): key half kh2 = of / NFW, local fragment fl = of % NFW
    f32x4 sum[2];
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int of = w + o * C::NW;
      const int kh2 = of / NFW, fl = of % NFW;
      sum[o] = zero4();
      for (int p2 = 0; p2 < NP; ++p2)
        sum[o] += *reinterpret_cast<const f32x4*>(red + ((size_t)((kh2 * NP + p2) * NFW + fl) * 64 + l) * 4);
    }
    __syncthreads();
#pragma unroll
    for (int o = 0; o < 2; ++o) {
      const int of = w + o * C::NW;
      const int kh2 = of / NFW, fl = of % NFW;
      const int v = 2 * kh2 + fl / MT, m = fl % MT;
      const int fi = v * MT + m;  // fragment index of the 4-wave kernel's partial layout
      if (it.slot >= 0) {
        float* ps = part + ((size_t)it.slot * 2 + tns) * (size_t)NFR * 256;
        *reinterpret_cast<f32x4*>(ps + ((size_t)fi * 64 + l) * 4) = sum[o];
      } else {
        const float sc = tns == 0 ? s.scale : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) red[KI::krow(v, 4 * a + r) * D + 16 * m + col] = sum[o][r] * sc;
      }
    }
    if (it.slot < 0) {
      __syncthreads();
      T* dst = (tns == 0 ? dk : dv) + ((size_t)b * s.T + j * kBlock) * k_row + (size_t)g * D;
      for (int i = threadIdx.x; i < kBlock * D / 8; i += NT) {
        const int kk = i / (D / 8), c8 = (i % (D / 8)) * 8;
        store8(dst + (size_t)kk * k_row + c8, red + kk * D + c8);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ B4
// grid (B Hkv nblk): the partial sums of a block's items, added in item order,
// rows staged in LDS for 16-byte stores.  With the compression branch
// (slot_base_c != nullptr) the pooled key j of pooled-key block j / 64 adds
// its gradient (the sum of that block's compression partials, row j % 64)
// divided by 64 to every key of block j: the gradient of the mean-pool.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Shape s, const int* __restrict__ slot_base,
                                                         const int* __restrict__ slot_cnt,
                                                         const int* __restrict__ slot_base_c,
                                                         const int* __restrict__ slot_cnt_c,
                                                         const float* __restrict__ part,
                                                         T* __restrict__ dk, T* __restrict__ dv) {
  typedef typename BwdImage<T, D>::K KI;
  constexpr int MT = D / 16, NFR = 4 * MT;
  constexpr int PER = 2 * NFR * 64 / 256;  // fragment entries (4 floats) per thread
  __shared__ __align__(16) float ot[2][kBlock * D];
  __shared__ float pooled[2][D];
  const int e = blockIdx.x;
  const int base = slot_base[e];
  if (base < 0) return;
  const int ns = slot_cnt[e];
  const int nblk = s.T / kBlock;
  const int bg = e / nblk, j = e % nblk;
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const bool full = slot_base_c != nullptr;
  if (full) {
    // row jj = j % 64 of the pooled-key block's partials: fragment v, lane group
    // a, register r hold key jj (inverse of the image's key order), lane col channel
    const int NJc = (s.nc + kBlock - 1) / kBlock;
    const int ec = bg * NJc + j / kBlock, jj = j % kBlock;
    const int cb = slot_base_c[ec], cn = slot_cnt_c[ec];
    const int v = 2 * (jj / 32) + (jj % 8) / 4, a = (jj % 32) / 8, r = jj % 4;
    for (int i = threadIdx.x; i < 2 * D; i += 256) {
      const int tns = i / D, ch = i % D, m = ch / 16, col = ch % 16;
      float acc = 0.f;
      for (int z = 0; z < cn; ++z)
        acc += part[((size_t)(cb + z) * 2 + tns) * NFR * 256 + ((size_t)(v * MT + m) * 64 + 16 * a + col) * 4 + r];
      pooled[tns][ch] = acc * (1.f / kBlock);
    }
  }
  const float* pb = part + (size_t)base * 2 * NFR * 256;
  f32x4 sum[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) sum[k] = *reinterpret_cast<const f32x4*>(pb + ((size_t)threadIdx.x + 256 * k) * 4);
  for (int z = 1; z < ns; ++z) {
    const float* pz = pb + (size_t)z * 2 * NFR * 256;
#pragma unroll
    for (int k = 0; k < PER; ++k) sum[k] += *reinterpret_cast<const f32x4*>(pz + ((size_t)threadIdx.x + 256 * k) * 4);
  }
  __syncthreads();  // pooled row visible
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + 256 * k;
    const int tns = i / (NFR * 64), fi = (i / 64) % NFR, l = i % 64;
    const int v = fi / MT, m = fi % MT, a = l >> 4, col = l & 15;
    const float sc = tns == 0 ? s.scale : 1.f;
    const float add = full ? pooled[tns][16 * m + col] : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) ot[tns][KI::krow(v, 4 * a + r) * D + 16 * m + col] = (sum[k][r] + add) * sc;
  }
  __syncthreads();
  const size_t k_row = (size_t)s.Hkv * D;
  for (int i = threadIdx.x; i < 2 * kBlock * D / 8; i += 256) {
    const int tns = i / (kBlock * D / 8), i2 = i % (kBlock * D / 8);
    const int kk = i2 / (D / 8), c8 = (i2 % (D / 8)) * 8;
    T* dst = (tns == 0 ? dk : dv) + ((size_t)b * s.T + j * kBlock + kk) * k_row + (size_t)g * D + c8;
    store8(dst, &ot[tns][kk * D + c8]);
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int D, int G>
static hipError_t launch_kv_t(const Shape& s, const Item* items, int grid_items, const KvArgs& a,
                              hipStream_t st) {
  typedef KvCfg<T, D, G> C;
  hipError_t e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<T, D, G>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, G>), dim3(grid_items), dim3(C::NT), C::LDS, st, s, items, a);
  return hipGetLastError();
}
template <int G>
static hipError_t launch_kv_pair(const Shape& s, const Item* items, int grid_items, const KvArgs& a,
                                 hipStream_t st) {
  typedef KvPairCfg<bf16, 64, G> C;
  hipError_t e = hipFuncSetAttribute((const void*)bwd_dkdv_pair_kernel<bf16, 64, G>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_pair_kernel<bf16, 64, G>), dim3(grid_items), dim3(C::NT), C::LDS, st, s,
                     items, a);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t launch_kv_g(const Shape& s, const Item* items, int grid_items, const KvArgs& a,
                              hipStream_t st) {
  switch (s.G) {
    case 1: return launch_kv_t<T, D, 1>(s, items, grid_items, a, st);
    case 2: return launch_kv_t<T, D, 2>(s, items, grid_items, a, st);
    case 4: return launch_kv_t<T, D, 4>(s, items, grid_items, a, st);
    case 8: return launch_kv_t<T, D, 8>(s, items, grid_items, a, st);
    default: return launch_kv_t<T, D, 16>(s, items, grid_items, a, st);
  }
}

hipError_t launch_bwd_dkdv(bool is_bf16, const Shape& s, const KvBranches& br, const uint64_t* revmap,
                           void* dk, void* dv, const BwdPlanWs& ws, hipStream_t st) {
  const int nblk = s.T / kBlock;
  const int NJ = s.B * s.Hkv * nblk;
  const bool full = br.full;
  Item* items = (Item*)ws.items;
  hipLaunchKernelGGL(bwd_lists_kernel, dim3(nblk, s.Hkv, s.B), dim3(256), 0, st, s, revmap, ws.lists,
                     ws.counts);
  hipLaunchKernelGGL(bwd_items_kernel, dim3(1), dim3(1024), 0, st, NJ, nblk, s.G, s.T, s.W, full ? 1 : 0,
                     ws.counts, items, ws.slot_base, ws.slot_cnt, ws.slot_base_c, ws.slot_cnt_c, ws.nitems);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  KvArgs a;
  a.q = br.q;
  a.img = (const unsigned char*)br.img;
  a.pimg = (const unsigned char*)br.pimg;
  a.lists = ws.lists;
  for (int m = 0; m < 3; ++m) {
    a.lse[m] = br.lse[m];
    a.delta[m] = br.delta[m];
    a.dos[m] = br.dos[m];
  }
  a.nitems = ws.nitems;
  a.dk = dk;
  a.dv = dv;
  a.part = ws.part;
  const int grid_items = bwd_item_bound(s, full);
  if (is_bf16) {
    if (s.D == 64) {
      switch (s.G) {
        case 1: e = launch_kv_pair<1>(s, items, grid_items, a, st); break;
        case 2: e = launch_kv_pair<2>(s, items, grid_items, a, st); break;
        case 4: e = launch_kv_pair<4>(s, items, grid_items, a, st); break;
        case 8: e = launch_kv_pair<8>(s, items, grid_items, a, st); break;
        default: e = launch_kv_pair<16>(s, items, grid_items, a, st); break;
      }
    } else {
      e = launch_kv_g<bf16, 128>(s, items, grid_items, a, st);
    }
  } else {
    e = launch_kv_g<float, 64>(s, items, grid_items, a, st);
  }
  if (e != hipSuccess) return e;
  const int* sbc = full ? ws.slot_base_c : nullptr;
  const int* scc = full ? ws.slot_cnt_c : nullptr;
  if (is_bf16) {
    if (s.D == 64)
      hipLaunchKernelGGL((bwd_reduce_kernel<bf16, 64>), dim3(NJ), dim3(256), 0, st, s, ws.slot_base,
                         ws.slot_cnt, sbc, scc, ws.part, (bf16*)dk, (bf16*)dv);
    else
      hipLaunchKernelGGL((bwd_reduce_kernel<bf16, 128>), dim3(NJ), dim3(256), 0, st, s, ws.slot_base,
                         ws.slot_cnt, sbc, scc, ws.part, (bf16*)dk, (bf16*)dv);
  } else {
    hipLaunchKernelGGL((bwd_reduce_kernel<float, 64>), dim3(NJ), dim3(256), 0, st, s, ws.slot_base,
                       ws.slot_cnt, sbc, scc, ws.part, (float*)dk, (float*)dv);
  }
  return hipGetLastError();
}

size_t bwd_items_bytes(const Shape& s, bool full) { return (size_t)bwd_item_bound(s, full) * sizeof(Item); }
size_t bwd_part_floats(const Shape& s, bool full) {
  return (size_t)bwd_item_bound(s, full) * 2 * kBlock * s.D;
}

}  // namespace nsa
