// bwd.hip -- gradient of the selection branch, two passes, no atomics.
//
// [SIC] "Sparsity is Cool", Method (NSA implementation): every query attends a
// subset of keys of its own, so the key/value-stationary backward of dense
// attention does not apply directly; the two-pass scheme -- a query-stationary
// pass for dQ and a key/value-stationary pass for dK/dV over a reconstructed
// reverse key->query map -- avoids atomic contention.  The selection and the
// gates are held fixed; the branch receives g_sel * dO.  With P_s the
// selection softmax (recomputed from the saved log-sum-exp), dP_s = dOs . v_s,
// Delta = dOs . o_sel and dS_s = P_s (dP_s - Delta):
//   dq = tau sum_s dS_s k_s,   dk_s = tau sum dS_s q,   dv_s = sum P_s dOs.
//
// B0 prep    : dOs = g_sel dO (element type), Delta (fp32), block images
//              (K, V, K^T fragments) for B2.
// B1 revmap  : M[b][g][j][c] = 64-bit mask of the positions of tile c (64
//              positions) that selected block j -- one wave per (tile, group),
//              one lane per position, a ballot per block; no atomics.
// B2 dq      : query-stationary, the block walk of the forward's selection
//              kernel (bwd_dq.hip).
// B3 dk/dv   : key/value-stationary: a workgroup owns one key block (each wave
//              16 keys, accumulators in registers) and a range of query tiles;
//              the rows that selected the block (from M) are compacted into
//              32-row chunks staged in LDS (row-major and transposed copies of
//              Q and dOs).  Blocks read by many queries (block 0, early blocks)
//              are split into segments whose partial sums are added in a fixed
//              order by B4, so the result is bitwise reproducible.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

template <typename T> struct V16b;
template <> struct V16b<bf16> { typedef bf16x8 type; };
template <> struct V16b<float> { typedef f32x4 type; };

// ============================================================ B0: preparation
// grid (nblk, Hkv, B), 256 threads: block j of positions / keys, KV group g.
// Writes the block's backward image (K, V, K^T fragments, BwdImage) and, for
// the G heads of the group at these positions, dOs = g_sel dO and Delta.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(Shape s, const T* __restrict__ k,
                                                       const T* __restrict__ v,
                                                       const T* __restrict__ gates,
                                                       const T* __restrict__ o_sel,
                                                       const T* __restrict__ dout,
                                                       unsigned char* __restrict__ bimg,
                                                       float* __restrict__ delta,
                                                       T* __restrict__ dos) {
  typedef BwdImage<T, D> I;
  constexpr int EPV = 16 / sizeof(T);
  typedef typename V16b<T>::type Vec;
  __shared__ __align__(16) T kt[kBlock][D + 8];
  __shared__ __align__(16) T vt[kBlock][D + 8];
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = s.G;
  const size_t k_row = (size_t)s.Hkv * D;
  for (int i = threadIdx.x; i < kBlock * (D / EPV); i += 256) {
    const int r = i / (D / EPV), c8 = i % (D / EPV);
    const size_t src = ((size_t)b * s.T + j * kBlock + r) * k_row + (size_t)g * D + c8 * EPV;
    *reinterpret_cast<Vec*>(&kt[r][c8 * EPV]) = *reinterpret_cast<const Vec*>(k + src);
    *reinterpret_cast<Vec*>(&vt[r][c8 * EPV]) = *reinterpret_cast<const Vec*>(v + src);
  }
  __syncthreads();
  unsigned char* img = bimg + (((size_t)b * s.Hkv + g) * (s.T / kBlock) + j) * (size_t)I::BYTES;
  for (int w = threadIdx.x; w < I::PIECES * 64; w += 256) {
    const int pc = w / 64, l = w % 64;
    const int f = pc / I::NV, vv = pc % I::NV;
    const int a = l / 16, rho = l % 16;
    T piece[EPV];
    if (f < 2 * I::NFRAG) {  // K or V, key rows
      const int ff = f % I::NFRAG;
      const int u = I::K::k_u(ff), ks = I::K::k_ks(ff);
      const T* src = (f < I::NFRAG ? &kt[0][0] : &vt[0][0]) +
                     (size_t)I::K::krow(u, rho) * (D + 8) + ks * 32 + 8 * a + vv * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) piece[e] = src[e];
    } else {                 // K^T: channel rows, 8 consecutive keys per lane
      const int f2 = f - 2 * I::NFRAG, mt = I::K::v_mt(f2), hf = I::K::v_h(f2);
      const int ch = mt * 16 + rho, key0 = 32 * hf + 8 * a + vv * EPV;
#pragma unroll
      for (int e = 0; e < EPV; ++e) piece[e] = kt[key0 + e][ch];
    }
    *reinterpret_cast<f32x4*>(img + (size_t)pc * 1024 + 16 * l) = *reinterpret_cast<const f32x4*>(piece);
  }
  // dOs and Delta for the G heads of the group: one wave per (position, head) row
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  for (int row = w; row < kBlock * G; row += 4) {
    const int t = j * kBlock + row / G, h = g * G + row % G;
    const size_t base = (((size_t)b * s.T + t) * s.Hq + h) * D;
    const float gs = (float)gates[(((size_t)b * s.T + t) * s.Hq + h) * 3 + 1];
    float acc = 0.f;
    for (int d = l; d < D; d += kWave) {
      const float v_ = gs * (float)dout[base + d];
      dos[base + d] = (T)v_;
      acc += v_ * (float)o_sel[base + d];
    }
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (l == 0) delta[((size_t)b * s.Hq + h) * s.T + t] = acc;
  }
}

// ============================================================ B1: reverse map
// grid (nblk tiles c, Hkv, B), 64 threads.  revmap[b][g][j][c] for j <= c.
__global__ __launch_bounds__(64) void bwd_revmap_kernel(Shape s, const int32_t* __restrict__ idx,
                                                        uint64_t* __restrict__ revmap) {
  extern __shared__ unsigned char bits[];  // [c+1][64]
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nblk = s.T / kBlock;
  const int l = threadIdx.x;
  for (int i = l; i < (c + 1) * 64; i += 64) bits[i] = 0;
  __syncthreads();
  const int t = c * kBlock + l;
  const int32_t* row = idx + (((size_t)b * s.Hkv + g) * s.T + t) * s.topk;
  for (int e = 0; e < s.topk; ++e) {
    const int j = row[e];
    if (j >= 0 && j <= c) bits[j * 64 + l] = 1;
  }
  __syncthreads();
  uint64_t* dst = revmap + (((size_t)b * s.Hkv + g) * nblk) * nblk;
  for (int j = 0; j <= c; ++j) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(bits[j * 64 + l] != 0);
    if (l == 0) dst[(size_t)j * nblk + c] = m;
  }
}

// ============================================================ B3: dk / dv
// Work items: (block j, query-tile range [c_lo, c_hi), partial slot or -1).
struct Item {
  int j, c_lo, c_hi, slot;
};

// Segments of the query tiles that can read block j (tiles c >= j): block 0,
// read by every query, in runs of 8 tiles; block j >= 1 in geometric runs
// [j, 2j), [2j, 4j), ... (each holds about the same expected number of
// selecting rows).  The same function runs on the host (sizing) and on the
// device (table building).
__host__ __device__ inline int segments_of(int j, int nblk) {
  if (j == 0) return (nblk + 7) / 8;
  int n = 0;
  for (long lo = j; lo < nblk; lo *= 2) ++n;
  return n;
}
__host__ __device__ inline void segment_range(int j, int i, int nblk, int& lo, int& hi) {
  if (j == 0) {
    lo = 8 * i;
    hi = min(nblk, 8 * i + 8);
    return;
  }
  long a = j;
  for (int z = 0; z < i; ++z) a *= 2;
  lo = (int)a;
  hi = (int)min((long)nblk, 2 * a);
}

__global__ void bwd_items_kernel(int nblk, Item* items, int* slot_base) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int n = 0, slots = 0;
  for (int j = 0; j < nblk; ++j) {
    const int ns = segments_of(j, nblk);
    slot_base[j] = ns > 1 ? slots : -1;
    for (int i = 0; i < ns; ++i) {
      Item it;
      it.j = j;
      segment_range(j, i, nblk, it.c_lo, it.c_hi);
      it.slot = ns > 1 ? slots + i : -1;
      items[n++] = it;
    }
    if (ns > 1) slots += ns;
  }
}

template <typename T, int D, int G>
struct KvCfg {
  static constexpr int CR = 32;         // rows (queries) per chunk
  static constexpr int CP = CR / G >= 1 ? CR / G : 1;  // positions per chunk
  static constexpr int KS = D / 32, MT = D / 16;
  static constexpr int QST = D + 8;      // row-major stride
  static constexpr int TST = CR + 8;     // transposed stride
};

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    Shape s, const Item* __restrict__ items, const T* __restrict__ q, const T* __restrict__ k,
    const T* __restrict__ v, const float* __restrict__ lse, const float* __restrict__ delta,
    const T* __restrict__ dos, const uint64_t* __restrict__ revmap, T* __restrict__ dk,
    T* __restrict__ dv, float* __restrict__ part, int nslots) {
  typedef KvCfg<T, D, G> C;
  constexpr int CR = C::CR, CP = C::CP, KS = C::KS, MT = C::MT, QST = C::QST, TST = C::TST;
  typedef typename Frag<T>::type FragT;
  static_assert(G <= CR, "a chunk holds whole positions");

  __shared__ __align__(16) T Qr[CR * QST];
  __shared__ __align__(16) T Dr[CR * QST];
  __shared__ __align__(16) T Qt[D * TST];
  __shared__ __align__(16) T Dt[D * TST];
  __shared__ float lse_s[CR], del_s[CR];
  __shared__ int tpos_s[CR];
  __shared__ uint8_t plist[64];

  const int nblk = s.T / kBlock;
  const Item it = items[blockIdx.x];
  const int g = blockIdx.y, b = blockIdx.z;
  const int j = it.j;
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const float c1 = s.scale * kLog2e;
  const size_t k_row = (size_t)s.Hkv * D, q_row = (size_t)s.Hq * D;
  const int key_l = w * 16 + col;  // this lane's key column within the block
  const int key = j * kBlock + key_l;

  // B operands: K and V rows of this wave's 16 keys
  FragT kf[KS], vf[KS];
  {
    const T* kr = k + ((size_t)b * s.T + key) * k_row + (size_t)g * D;
    const T* vr = v + ((size_t)b * s.T + key) * k_row + (size_t)g * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = Frag<T>::load(kr + ks * 32 + a * 8);
      vf[ks] = Frag<T>::load(vr + ks * 32 + a * 8);
    }
  }
  f32x4 adk[MT], adv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) { adk[mt] = zero4(); adv[mt] = zero4(); }

  const uint64_t* rm = revmap + (((size_t)b * s.Hkv + g) * nblk + j) * nblk;
  for (int c = it.c_lo; c < it.c_hi; ++c) {
    const uint64_t mask = rm[c];
    if (mask == 0ull) continue;
    const int n = __popcll(mask);
    // positions of the tile that selected j, ascending
    __syncthreads();
    if (w == 0 && ((mask >> l) & 1ull)) plist[__popcll(mask & ((1ull << l) - 1ull))] = (uint8_t)l;
    __syncthreads();
    for (int p0 = 0; p0 < n; p0 += CP) {
      // stage the chunk: rows (position, head), row-major and transposed
      for (int i = threadIdx.x; i < CR * D; i += 256) {
        const int r = i / D, d = i % D;
        const int pi = p0 + r / G;
        T qv = (T)0.f, dv_ = (T)0.f;
        if (pi < n) {
          const int t = c * kBlock + plist[pi], h = g * G + r % G;
          const size_t src = ((size_t)b * s.T + t) * q_row + (size_t)h * D + d;
          qv = q[src];
          dv_ = dos[src];
        }
        Qr[r * QST + d] = qv;
        Dr[r * QST + d] = dv_;
        Qt[d * TST + r] = qv;
        Dt[d * TST + r] = dv_;
      }
      if (threadIdx.x < CR) {
        const int r = threadIdx.x;
        const int pi = p0 + r / G;
        if (pi < n) {
          const int t = c * kBlock + plist[pi], h = g * G + r % G;
          lse_s[r] = lse[((size_t)b * s.Hq + h) * s.T + t] * kLog2e;
          del_s[r] = delta[((size_t)b * s.Hq + h) * s.T + t];
          tpos_s[r] = t;
        } else {
          lse_s[r] = INFINITY;  // P = 0
          del_s[r] = 0.f;
          tpos_s[r] = -1;
        }
      }
      __syncthreads();
      // S = Q K^T and dP = dOs V^T for the chunk's 32 rows x this wave's 16 keys;
      // tile u holds rows 8(rho/4) + 4u + rho%4 so that lane (a, col) owns rows
      // 8a + e (e = 4u + r) of key column col -- the A layout of P^T / dS^T.
      float pv[8], dsv[8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int qr = 8 * (col / 4) + 4 * u + (col % 4);
        f32x4 st = zero4(), dp = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          st = mma(st, Frag<T>::load(Qr + qr * QST + ks * 32 + a * 8), kf[ks]);
          dp = mma(dp, Frag<T>::load(Dr + qr * QST + ks * 32 + a * 8), vf[ks]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 8 * a + 4 * u + r;
          const bool ok = key <= tpos_s[row];
          const float pr = ok ? fast_exp2(st[r] * c1 - lse_s[row]) : 0.f;
          pv[4 * u + r] = pr;
          dsv[4 * u + r] = pr * (dp[r] - del_s[row]);
        }
      }
      const FragT pf = Frag<T>::from_f32(pv);
      const FragT sf = Frag<T>::from_f32(dsv);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        adv[mt] = mma(adv[mt], pf, Frag<T>::load(Dt + (mt * 16 + col) * TST + 8 * a));
        adk[mt] = mma(adk[mt], sf, Frag<T>::load(Qt + (mt * 16 + col) * TST + 8 * a));
      }
      __syncthreads();
    }
  }

  // C layout: lane holds keys (rows) 4a + r of the wave's 16, channel 16 mt + col
  if (it.slot < 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kk = j * kBlock + w * 16 + 4 * a + r;
        const size_t o = ((size_t)b * s.T + kk) * k_row + (size_t)g * D + mt * 16 + col;
        dk[o] = (T)(adk[mt][r] * s.scale);
        dv[o] = (T)adv[mt][r];
      }
  } else {
    // partial sums of this segment: part[b][g][slot][dk | dv][64 keys][D]
    float* ps = part + (((size_t)b * s.Hkv + g) * (size_t)nslots + it.slot) * 2 * kBlock * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kl = w * 16 + 4 * a + r;
        ps[(size_t)kl * D + mt * 16 + col] = adk[mt][r];
        ps[(size_t)(kBlock + kl) * D + mt * 16 + col] = adv[mt][r];
      }
  }
}

// ============================================================ B4: reduction
// grid (nblk, Hkv, B): blocks split into several segments add their partial
// sums in segment order (deterministic).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(Shape s, const int* __restrict__ slot_base,
                                                         const float* __restrict__ part, int nslots,
                                                         T* __restrict__ dk, T* __restrict__ dv) {
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int nblk = s.T / kBlock;
  const int base = slot_base[j];
  if (base < 0) return;
  const int ns = segments_of(j, nblk);
  const float* pb = part + (((size_t)b * s.Hkv + g) * (size_t)nslots + base) * 2 * kBlock * D;
  const size_t k_row = (size_t)s.Hkv * D;
  for (int i = threadIdx.x; i < kBlock * D; i += 256) {
    float sk = 0.f, sv = 0.f;
    for (int z = 0; z < ns; ++z) {
      sk += pb[(size_t)z * 2 * kBlock * D + i];
      sv += pb[(size_t)z * 2 * kBlock * D + kBlock * D + i];
    }
    const int kl = i / D, d = i % D;
    const size_t o = ((size_t)b * s.T + j * kBlock + kl) * k_row + (size_t)g * D + d;
    dk[o] = (T)(sk * s.scale);
    dv[o] = (T)sv;
  }
}

// ============================================================ launchers
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

hipError_t launch_bwd_prep(bool is_bf16, const Shape& s, const void* k, const void* v,
                           const void* gates, const void* o_sel, const void* dout, void* bimg,
                           float* delta, void* dos, hipStream_t st) {
  dim3 grid(s.T / kBlock, s.Hkv, s.B);
  unsigned char* im = (unsigned char*)bimg;
  if (is_bf16) {
    if (s.D == 64)
      hipLaunchKernelGGL((bwd_prep_kernel<bf16, 64>), grid, dim3(256), 0, st, s, (const bf16*)k,
                         (const bf16*)v, (const bf16*)gates, (const bf16*)o_sel, (const bf16*)dout,
                         im, delta, (bf16*)dos);
    else
      hipLaunchKernelGGL((bwd_prep_kernel<bf16, 128>), grid, dim3(256), 0, st, s, (const bf16*)k,
                         (const bf16*)v, (const bf16*)gates, (const bf16*)o_sel, (const bf16*)dout,
                         im, delta, (bf16*)dos);
  } else {
    hipLaunchKernelGGL((bwd_prep_kernel<float, 64>), grid, dim3(256), 0, st, s, (const float*)k,
                       (const float*)v, (const float*)gates, (const float*)o_sel,
                       (const float*)dout, im, delta, (float*)dos);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_revmap(const Shape& s, const int32_t* indices, uint64_t* revmap,
                             hipStream_t st) {
  const int nblk = s.T / kBlock;
  dim3 grid(nblk, s.Hkv, s.B);
  hipLaunchKernelGGL(bwd_revmap_kernel, grid, dim3(64), (size_t)nblk * 64, st, s, indices, revmap);
  return hipGetLastError();
}

template <typename T, int D, int G>
static hipError_t launch_kv_t(const Shape& s, const Item* items, int nitems, int nslots,
                              const void* q, const void* k, const void* v, const float* lse,
                              const float* delta, const void* dos, const uint64_t* revmap,
                              void* dk, void* dv, float* part, hipStream_t st) {
  dim3 grid(nitems, s.Hkv, s.B);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, G>), grid, dim3(256), 0, st, s, items, (const T*)q,
                     (const T*)k, (const T*)v, lse, delta, (const T*)dos, revmap, (T*)dk, (T*)dv,
                     part, nslots);
  return hipGetLastError();
}
template <typename T, int D>
static hipError_t launch_kv_g(const Shape& s, const Item* items, int nitems, int nslots,
                              const void* q, const void* k, const void* v, const float* lse,
                              const float* delta, const void* dos, const uint64_t* revmap,
                              void* dk, void* dv, float* part, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_kv_t<T, D, 1>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
    case 2: return launch_kv_t<T, D, 2>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
    case 4: return launch_kv_t<T, D, 4>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
    case 8: return launch_kv_t<T, D, 8>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
    default: return launch_kv_t<T, D, 16>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
  }
}

hipError_t launch_bwd_dkdv(bool is_bf16, const Shape& s, const void* q, const void* k,
                           const void* v, const float* lse, const float* delta, const void* dos,
                           const uint64_t* revmap, void* dk, void* dv, void* items_ws,
                           int* slot_base, float* part, hipStream_t st) {
  const int nblk = s.T / kBlock;
  const int nitems = bwd_item_count(nblk), nslots = bwd_slot_count(nblk);
  Item* items = (Item*)items_ws;
  hipLaunchKernelGGL(bwd_items_kernel, dim3(1), dim3(64), 0, st, nblk, items, slot_base);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (is_bf16) {
    if (s.D == 64)
      e = launch_kv_g<bf16, 64>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
    else
      e = launch_kv_g<bf16, 128>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
  } else {
    e = launch_kv_g<float, 64>(s, items, nitems, nslots, q, k, v, lse, delta, dos, revmap, dk, dv, part, st);
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
