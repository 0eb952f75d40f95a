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
struct Item {
  int j, c_lo, c_hi, slot;
};

constexpr int kMaxSegTiles = 32;  // query tiles per item at most (bounds the LDS position list)

// Query tiles that can read block j are c >= j.  Block 0, read by every
// position, is cut into runs of 8 tiles; block j >= 1 into the geometric runs
// [j, 2j), [2j, 4j), ... (each holds about the same expected number of
// selecting rows when the selection probability falls like 1 / position),
// each run cut further into pieces of at most kMaxSegTiles tiles.  The same
// functions run on the host (sizing) and on the device (item table).
__host__ __device__ inline int segments_of(int j, int nblk) {
  if (j == 0) return (nblk + 7) / 8;
  int n = 0;
  for (long lo = j; lo < nblk; lo *= 2) {
    const long hi = lo * 2 < nblk ? lo * 2 : nblk;
    n += (int)((hi - lo + kMaxSegTiles - 1) / kMaxSegTiles);
  }
  return n;
}
__host__ __device__ inline void segment_range(int j, int i, int nblk, int& lo_out, int& hi_out) {
  if (j == 0) {
    lo_out = 8 * i;
    hi_out = 8 * i + 8 < nblk ? 8 * i + 8 : nblk;
    return;
  }
  for (long lo = j; lo < nblk; lo *= 2) {
    const long hi = lo * 2 < nblk ? lo * 2 : nblk;
    const int np = (int)((hi - lo + kMaxSegTiles - 1) / kMaxSegTiles);
    if (i < np) {
      const long len = hi - lo;
      lo_out = (int)(lo + len * i / np);
      hi_out = (int)(lo + len * (i + 1) / np);
      return;
    }
    i -= np;
  }
  lo_out = hi_out = nblk;
}

int bwd_item_count(int nblk) {
  int n = 0;
  for (int j = 0; j < nblk; ++j) n += segments_of(j, nblk);
  return n;
}
int bwd_slot_count(int nblk) {
  int n = 0;
  for (int j = 0; j < nblk; ++j) {
    const int ns = segments_of(j, nblk);
    if (ns > 1) n += ns;
  }
  return n;
}

// Item table and the first partial slot of every block (-1: one item, no
// partials).  One workgroup; exclusive scans over the blocks, 1024 at a time.
__global__ __launch_bounds__(1024) void bwd_items_kernel(int nblk, Item* __restrict__ items,
                                                        int* __restrict__ slot_base) {
  __shared__ int sc[1024], ss[1024];
  __shared__ int carry[2];
  const int x = threadIdx.x;
  if (x == 0) carry[0] = carry[1] = 0;
  __syncthreads();
  for (int j0 = 0; j0 < nblk; j0 += 1024) {
    const int j = j0 + x;
    const int ns = j < nblk ? segments_of(j, nblk) : 0;
    const int sl = ns > 1 ? ns : 0;
    sc[x] = ns;
    ss[x] = sl;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int a = x >= off ? sc[x - off] : 0;
      const int c = x >= off ? ss[x - off] : 0;
      __syncthreads();
      sc[x] += a;
      ss[x] += c;
      __syncthreads();
    }
    const int io = carry[0] + sc[x] - ns, so = carry[1] + ss[x] - sl;
    if (j < nblk) {
      slot_base[j] = ns > 1 ? so : -1;
      for (int i = 0; i < ns; ++i) {
        Item it;
        it.j = j;
        segment_range(j, i, nblk, it.c_lo, it.c_hi);
        it.slot = ns > 1 ? so + i : -1;
        items[io + i] = it;
      }
    }
    __syncthreads();
    if (x == 1023) {
      carry[0] += sc[1023];
      carry[1] += ss[1023];
    }
    __syncthreads();
  }
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
  static constexpr int MAXPOS = kMaxSegTiles * kBlock;
  static constexpr size_t RING = (size_t)NW * NR * STAGE;
  static constexpr size_t LDS = KVB + RING + MAXPOS * 2 + 64 * 4;
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

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

template <typename T, int D, int G>
__global__ __launch_bounds__((KvCfg<T, D, G>::NT), 1) void bwd_dkdv_kernel(
    Shape s, const Item* __restrict__ items, const T* __restrict__ q,
    const unsigned char* __restrict__ bimg, const float* __restrict__ lse,
    const float* __restrict__ delta, const T* __restrict__ dos, const uint64_t* __restrict__ revmap,
    T* __restrict__ dk, T* __restrict__ dv, float* __restrict__ part, int nslots) {
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
  int* toff = reinterpret_cast<int*>(plist + C::MAXPOS);          // [64]

  const int nblk = s.T / kBlock;
  const Item it = items[blockIdx.x];
  const int g = blockIdx.y, b = blockIdx.z;
  const int j = it.j;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = threadIdx.x % kWave;
  const int a = l >> 4, col = l & 15;
  const float c1 = s.scale * kLog2e;
  const size_t q_row = (size_t)s.Hq * D;

  // K and V fragments of block j (first 2 NFRAG fragments of its backward image)
  {
    const unsigned char* src = bimg + (((size_t)b * s.Hkv + g) * nblk + j) * (size_t)BwdImage<T, D>::BYTES + 16 * l;
    for (int pc = w; pc < KVB / 1024; pc += NW)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)pc * 1024), (void*)(kv + (size_t)pc * 1024),
                                       16, 0, 0);
  }
  // ascending list of the positions of tiles [c_lo, c_hi) that selected block j
  const uint64_t* rm = revmap + (((size_t)b * s.Hkv + g) * nblk + j) * nblk;
  const int ntile = it.c_hi - it.c_lo;
  if (w == 0) {
    const uint64_t msk = l < ntile ? rm[it.c_lo + l] : 0ull;
    int n = __popcll(msk), incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (l >= off) incl += y;
    }
    toff[l] = incl - n;
    if (l == 63) toff[63] = incl;  // total (tiles never fill all 64 lanes: ntile <= 32)
  }
  __syncthreads();
  const int npos = toff[63];
  for (int ti = w; ti < ntile; ti += NW) {
    const uint64_t msk = rm[it.c_lo + ti];
    if ((msk >> l) & 1ull)
      plist[toff[ti] + __popcll(msk & ((1ull << l) - 1ull))] = (uint16_t)((it.c_lo + ti) * kBlock + l);
  }
  wait_vmcnt<0>();
  __syncthreads();

  f32x4 adk[NFR], adv[NFR];
#pragma unroll
  for (int i = 0; i < NFR; ++i) { adk[i] = zero4(); adv[i] = zero4(); }

  const int nch = (npos + CP - 1) / CP;
  const int my_n = nch > w ? (nch - w + NW - 1) / NW : 0;
  unsigned char* wring = ring + (size_t)w * NR * STAGE;
  const int last_key_mask = j * kBlock + kBlock - 1;  // rows before this position need the causal mask

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
    const bool masked = plist[ck * CP] < last_key_mask;

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
      f32x4 sv[2] = {zero4(), zero4()}, dp[2] = {zero4(), zero4()};
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
          x[e] = p[e] * (dp[e >> 2][e & 3] - dl[e]);
        }
      } else {
        const int key = j * kBlock + KI::krow(v, col);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int qi = ck * CP + (8 * a + e) / G;
          const int t = plist[qi < npos ? qi : 0];
          p[e] = key <= t ? fast_exp2(sv[e >> 2][e & 3] * c1 - lr[e]) : 0.f;
          x[e] = p[e] * (dp[e >> 2][e & 3] - dl[e]);
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

  // sum the waves' accumulators through LDS (the rings are free now) and write
  __syncthreads();
  float* red = reinterpret_cast<float*>(ring);
  const size_t k_row = (size_t)s.Hkv * D;
#pragma unroll
  for (int tns = 0; tns < 2; ++tns) {
#pragma unroll
    for (int fi = 0; fi < NFR; ++fi)
      *reinterpret_cast<f32x4*>(red + ((size_t)(w * NFR + fi) * 64 + l) * 4) = tns == 0 ? adk[fi] : adv[fi];
    __syncthreads();
    for (int fi = w; fi < NFR; fi += NW) {
      f32x4 sum = *reinterpret_cast<const f32x4*>(red + ((size_t)fi * 64 + l) * 4);
      for (int w2 = 1; w2 < NW; ++w2) sum += *reinterpret_cast<const f32x4*>(red + ((size_t)(w2 * NFR + fi) * 64 + l) * 4);
      if (it.slot < 0) {
        const int v = fi / MT, m = fi % MT;
        T* dst = tns == 0 ? dk : dv;
        const float sc = tns == 0 ? s.scale : 1.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = j * kBlock + KI::krow(v, 4 * a + r);
          dst[((size_t)b * s.T + kk) * k_row + (size_t)g * D + 16 * m + col] = (T)(sum[r] * sc);
        }
      } else {
        float* ps = part + ((((size_t)b * s.Hkv + g) * (size_t)nslots + it.slot) * 2 + tns) * (size_t)NFR * 256;
        *reinterpret_cast<f32x4*>(ps + ((size_t)fi * 64 + l) * 4) = sum;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ B4
// grid (nblk, Hkv, B): the partial sums of a block's items, in item order.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Shape s, const int* __restrict__ slot_base,
                                                         const float* __restrict__ part, int nslots,
                                                         T* __restrict__ dk, T* __restrict__ dv) {
  typedef typename BwdImage<T, D>::K KI;
  constexpr int MT = D / 16, NFR = 4 * MT;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nblk = s.T / kBlock;
  const int base = slot_base[j];
  if (base < 0) return;
  const int ns = segments_of(j, nblk);
  const size_t k_row = (size_t)s.Hkv * D;
  const float* pb = part + (((size_t)b * s.Hkv + g) * (size_t)nslots + base) * 2 * (size_t)NFR * 256;
  for (int i = threadIdx.x; i < 2 * NFR * 64; i += 256) {
    const int tns = i / (NFR * 64), fi = (i / 64) % NFR, l = i % 64;
    f32x4 sum = *reinterpret_cast<const f32x4*>(pb + (size_t)i * 4);
    for (int z = 1; z < ns; ++z) sum += *reinterpret_cast<const f32x4*>(pb + ((size_t)z * 2 * NFR * 64 + i) * 4);
    const int v = fi / MT, m = fi % MT, a = l >> 4, col = l & 15;
    T* dst = tns == 0 ? dk : dv;
    const float sc = tns == 0 ? s.scale : 1.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = j * kBlock + KI::krow(v, 4 * a + r);
      dst[((size_t)b * s.T + kk) * k_row + (size_t)g * D + 16 * m + col] = (T)(sum[r] * sc);
    }
  }
}

// ------------------------------------------------------------------ launchers
template <typename T, int D, int G>
static hipError_t launch_kv_t(const Shape& s, const Item* items, int nitems, int nslots, const void* q,
                              const void* bimg, const float* lse, const float* delta, const void* dos,
                              const uint64_t* revmap, void* dk, void* dv, float* part, hipStream_t st) {
  typedef KvCfg<T, D, G> C;
  hipError_t e = hipFuncSetAttribute((const void*)bwd_dkdv_kernel<T, D, G>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return e;
  dim3 grid(nitems, s.Hkv, s.B);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, G>), grid, dim3(C::NT), C::LDS, st, s, items, (const T*)q,
                     (const unsigned char*)bimg, lse, delta, (const T*)dos, revmap, (T*)dk, (T*)dv,
                     part, nslots);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t launch_kv_g(const Shape& s, const Item* items, int nitems, int nslots, const void* q,
                              const void* bimg, const float* lse, const float* delta, const void* dos,
                              const uint64_t* revmap, void* dk, void* dv, float* part, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_kv_t<T, D, 1>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
    case 2: return launch_kv_t<T, D, 2>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
    case 4: return launch_kv_t<T, D, 4>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
    case 8: return launch_kv_t<T, D, 8>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
    default: return launch_kv_t<T, D, 16>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
  }
}

hipError_t launch_bwd_dkdv(bool is_bf16, const Shape& s, const void* q, const void* bimg,
                           const float* lse, const float* delta, const void* dos,
                           const uint64_t* revmap, void* dk, void* dv, void* items_ws,
                           int* slot_base, float* part, hipStream_t st) {
  const int nblk = s.T / kBlock;
  const int nitems = bwd_item_count(nblk), nslots = bwd_slot_count(nblk);
  Item* items = (Item*)items_ws;
  hipLaunchKernelGGL(bwd_items_kernel, dim3(1), dim3(1024), 0, st, nblk, items, slot_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (is_bf16) {
    if (s.D == 64)
      e = launch_kv_g<bf16, 64>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
    else
      e = launch_kv_g<bf16, 128>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
  } else {
    e = launch_kv_g<float, 64>(s, items, nitems, nslots, q, bimg, lse, delta, dos, revmap, dk, dv, part, st);
  }
  if (e != hipSuccess) return e;
  if (nslots == 0) return hipSuccess;
  dim3 grid(nblk, s.Hkv, s.B);
  if (is_bf16) {
    if (s.D == 64)
      hipLaunchKernelGGL((bwd_reduce_kernel<bf16, 64>), grid, dim3(256), 0, st, s, slot_base, part,
                         nslots, (bf16*)dk, (bf16*)dv);
    else
      hipLaunchKernelGGL((bwd_reduce_kernel<bf16, 128>), grid, dim3(256), 0, st, s, slot_base, part,
                         nslots, (bf16*)dk, (bf16*)dv);
  } else {
    hipLaunchKernelGGL((bwd_reduce_kernel<float, 64>), grid, dim3(256), 0, st, s, slot_base, part,
                       nslots, (float*)dk, (float*)dv);
  }
  return hipGetLastError();
}

size_t bwd_items_bytes(int nblk) { return (size_t)bwd_item_count(nblk) * sizeof(Item); }
size_t bwd_part_floats(const Shape& s) {
  return (size_t)s.B * s.Hkv * bwd_slot_count(s.T / kBlock) * 2 * kBlock * s.D;
}

}  // namespace nsa
