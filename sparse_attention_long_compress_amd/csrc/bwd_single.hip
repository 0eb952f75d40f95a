// bwd_single.hip -- single-pass selection backward with atomics (the
// alternative the two-pass scheme is measured against).
//
// [SIC] "Sparsity is Cool", Method (NSA implementation): a query-stationary
// backward computes dq, dk and dv in one walk over each query's selected
// blocks, adding dk and dv with atomics; because many queries select the same
// block, those atomics contend -- the reason for the two-pass scheme of
// bwd_dq.hip / bwd_dkdv.hip.  This kernel is that single pass on gfx950:
// the dq walk of bwd_dq.hip (block images in a two-group LDS ring, one 16-row
// column group per wave) plus, per attended block, P and dS in the row-major
// orientation (a second S / dP product with the operands swapped, so the C
// layout is the A layout of P^T and dS^T over the group's 16 rows), the
// 16-row contractions dV_j += P^T dOs and dK_j += dS^T Q on
// v_mfma_f32_16x16x16_bf16, and fp32 atomic adds of the 64 x D results into
// dk / dv accumulators; a last kernel scales and rounds them.  bf16 only.
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

namespace nsa {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

template <int D, int G>
struct SingleCfg {
  typedef BwdImage<bf16, D> Img;
  static constexpr int NW = 8, NT = NW * 64;   // one 16-row column group per wave
  static constexpr int NSG = 16 / G, P = NW * NSG;
  static constexpr int KS = D / 32, MT = D / 16, NFRAG = Img::NFRAG;
  static constexpr int STAGE = Img::BYTES;
  static constexpr int GB = D == 128 ? 1 : 2, NBUF = 2 * GB;
  static constexpr int LOADS = Img::PIECES;
  static_assert(NSG * G == 16, "column group = 16 rows");
  static_assert((size_t)NBUF * STAGE >= (size_t)NW * 2 * 16 * D * 2, "transpose scratch fits in the ring");
};

template <int D, int G>
__global__ __launch_bounds__((SingleCfg<D, G>::NT)) void bwd_single_kernel(
    Shape s, const bf16* __restrict__ q, const unsigned char* __restrict__ bimg,
    const int32_t* __restrict__ indices, const float* __restrict__ lse,
    const float* __restrict__ delta, const bf16* __restrict__ dos, bf16* __restrict__ dq,
    float* __restrict__ dk32, float* __restrict__ dv32) {
  typedef SingleCfg<D, G> C;
  constexpr int NT = C::NT, P = C::P, NSG = C::NSG, KS = C::KS, MT = C::MT, NFRAG = C::NFRAG;
  constexpr int STAGE = C::STAGE, GB = C::GB, LOADS = C::LOADS;
  typedef typename C::Img::K KI;
  const float INF = __builtin_inff();

  const int nblk_all = s.T / kBlock;
  const int NTL = (s.T + P - 1) / P;
  int bg, tile;
  xcd_order(blockIdx.x, gridDim.x, s.B * s.Hkv, NTL, bg, tile);
  const int g = bg % s.Hkv, b = bg / s.Hkv;
  const int t0 = tile * P;
  const int nvalid = min(P, s.T - t0);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int l = threadIdx.x % kWave;
  const int a = l / 16, col = l % 16;
  const int sg = col / G, hh = col % G;
  const int h = g * G + hh;
  const float c1 = s.scale * kLog2e;
  const int topk = s.topk;
  const size_t q_row = (size_t)s.Hq * D, k_row = (size_t)s.Hkv * D;
  const unsigned char* img_b = bimg + ((size_t)b * s.Hkv + g) * nblk_all * (size_t)STAGE;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;
  int16_t* lists = reinterpret_cast<int16_t*>(smem + (size_t)C::NBUF * STAGE);
  for (int i = threadIdx.x; i < P * topk; i += NT) {
    const int p = i / topk, e = i % topk;
    const int j = p < nvalid ? indices[(((size_t)b * s.Hkv + g) * s.T + t0 + p) * topk + e] : -1;
    lists[i] = (int16_t)(j < 0 ? 0x7fff : j);
  }

  // this lane's row (lane col of the column group) and, for the row-major
  // products, the rows 4a + r of the group
  const int pf = w * NSG;
  const int p = pf + sg;
  const int t = t0 + p;
  const bool valid = p < nvalid;
  const int own = (t0 + pf) / kBlock;
  bf16x8 qf[KS], df[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (valid) {
      const size_t o = ((size_t)b * s.T + t) * q_row + (size_t)h * D + ks * 32 + 8 * a;
      qf[ks] = Frag<bf16>::load(q + o);
      df[ks] = Frag<bf16>::load(dos + o);
    } else {
      qf[ks] = Frag<bf16>::zero();
      df[ks] = Frag<bf16>::zero();
    }
  }
  float lse2 = INF, dl = 0.f;
  if (valid) {
    lse2 = lse[((size_t)b * s.Hq + h) * s.T + t] * kLog2e;
    dl = delta[((size_t)b * s.Hq + h) * s.T + t];
  }
  float lr4[4], dl4[4];
  int t4[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * a + r;  // row of the group
    const int pr = pf + rr / G, hr = g * G + rr % G;
    t4[r] = t0 + pr;
    const bool vr = pr < nvalid;
    lr4[r] = vr ? lse[((size_t)b * s.Hq + hr) * s.T + t4[r]] * kLog2e : INF;
    dl4[r] = vr ? delta[((size_t)b * s.Hq + hr) * s.T + t4[r]] : 0.f;
  }
  // Q^T and dOs^T of the group's 16 rows as 16x16x16 B operands (lane (a, col):
  // rows 4a .. 4a + 3 of channel 16 m + col), transposed through LDS
  s16x4 qT[MT], dT[MT];
  {
    bf16* scr = reinterpret_cast<bf16*>(ring) + (size_t)w * 2 * 16 * D;  // [2][16 rows][D]
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      *reinterpret_cast<bf16x8*>(scr + col * D + ks * 32 + 8 * a) = qf[ks];
      *reinterpret_cast<bf16x8*>(scr + 16 * D + col * D + ks * 32 + 8 * a) = df[ks];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qT[m][e] = __builtin_bit_cast(short, scr[(4 * a + e) * D + 16 * m + col]);
        dT[m][e] = __builtin_bit_cast(short, scr[16 * D + (4 * a + e) * D + 16 * m + col]);
      }
    __syncthreads();  // the ring is reused for the block images
  }

  int ptr = 0;
  int nxt = valid ? lists[p * topk] : 0x7fff;
  int nsel = __builtin_amdgcn_readfirstlane(row_min16(nxt));
  const int c_last = (t0 + nvalid - 1) / kBlock;
  const int nblk = c_last + 1;

  auto issue = [&](int j, int bf) {
    unsigned char* stage = ring + (size_t)bf * STAGE;
    const unsigned char* src = img_b + (size_t)j * STAGE + 16 * l;
    for (int pc = w; pc < LOADS; pc += C::NW)
      __builtin_amdgcn_global_load_lds((const void*)(src + (size_t)pc * 1024),
                                       (void*)(stage + (size_t)pc * 1024), 16, 0, 0);
  };
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = zero4();
  const int ngrp = (nblk + GB - 1) / GB;
  auto issue_group = [&](int gi) {
#pragma unroll
    for (int qq = 0; qq < GB; ++qq)
      if (gi * GB + qq < nblk) issue(gi * GB + qq, (gi & 1) * GB + qq);
  };
  issue_group(0);

  for (int gi = 0; gi < ngrp; ++gi) {
    wait_vmcnt<0>();
    barrier_keep_loads();
    if (gi + 1 < ngrp) issue_group(gi + 1);
    for (int qq = 0; qq < GB; ++qq) {
      const int j = gi * GB + qq;
      if (j >= nblk) break;
      if (j != nsel) continue;
      const bool sl = nxt == j;
      // selected rows of the group: lanes 0..15 hold the rows' flags
      const uint64_t selmask = __builtin_amdgcn_ballot_w64(sl);
      if (sl) {
        ++ptr;
        nxt = ptr < topk ? lists[p * topk + ptr] : 0x7fff;
      }
      nsel = __builtin_amdgcn_readfirstlane(row_min16(nxt));
      const unsigned char* stage = ring + (size_t)((gi & 1) * GB + qq) * STAGE;
      const bool diag = j == own;

      // ---- dq part (as in the two-pass dq kernel)
      f32x4 st[4], dp[4], sr[4], dr[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) { st[u] = zero4(); dp[u] = zero4(); sr[u] = zero4(); dr[u] = zero4(); }
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const bf16x8 kf = lds_frag<bf16>(stage + (size_t)f * 1024, l);
        const bf16x8 vf = lds_frag<bf16>(stage + (size_t)(NFRAG + f) * 1024, l);
        const int u = KI::k_u(f), ks = KI::k_ks(f);
        st[u] = mma(st[u], kf, qf[ks]);   // S^T  (C: key rows, lane = group row)
        dp[u] = mma(dp[u], vf, df[ks]);
        sr[u] = mma(sr[u], qf[ks], kf);   // S    (C: group rows 4a + r, lane col = key)
        dr[u] = mma(dr[u], df[ks], vf);
      }
      const float lr = sl ? lse2 : INF;
      bf16x8 dsf[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int u = 2 * hf + e / 4, rr = e % 4;
          const int key = j * kBlock + key_of(u, a, rr);
          const float pr = (!diag || key <= t) ? fast_exp2(st[u][rr] * c1 - lr) : 0.f;
          x[e] = pr * (dp[u][rr] - dl);
        }
        dsf[hf] = Frag<bf16>::from_f32(x);
      }
#pragma unroll
      for (int f = 0; f < NFRAG; ++f) {
        const bf16x8 tf = lds_frag<bf16>(stage + (size_t)(2 * NFRAG + f) * 1024, l);
        acc[KI::v_mt(f)] = mma(acc[KI::v_mt(f)], tf, dsf[KI::v_h(f)]);
      }

      // ---- dk / dv part: P^T and dS^T over the group's rows 4a + r
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int kl = KI::krow(u, col);  // key of lane column col in subtile u
        s16x4 pa, sa;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 4 * a + r;
          const bool on = ((selmask >> rr) & 1ull) && (!diag || j * kBlock + kl <= t4[r]);
          const float pr = on ? fast_exp2(sr[u][r] * c1 - lr4[r]) : 0.f;
          pa[r] = __builtin_bit_cast(short, (bf16)pr);
          sa[r] = __builtin_bit_cast(short, (bf16)(pr * (dr[u][r] - dl4[r])));
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const f32x4 cv = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, dT[m], zero4(), 0, 0, 0);
          const f32x4 ck = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(sa, qT[m], zero4(), 0, 0, 0);
          // C layout: lane (a, col) holds keys krow(u, 4a + r), channel 16 m + col
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const size_t o = ((size_t)b * s.T + j * kBlock + KI::krow(u, 4 * a + r)) * k_row +
                             (size_t)g * D + 16 * m + col;
            atomicAdd(dv32 + o, cv[r]);
            atomicAdd(dk32 + o, ck[r]);
          }
        }
      }
    }
  }

  if (valid) {
    bf16* dst = dq + ((size_t)b * s.T + t) * q_row + (size_t)h * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) store4(dst + mt * 16 + 4 * a, acc[mt] * s.scale);
  }
}

// zero the fp32 accumulators / round them into dk (x tau) and dv
__global__ __launch_bounds__(256) void single_zero_kernel(float* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0.f;
}
__global__ __launch_bounds__(256) void single_round_kernel(const float* __restrict__ dk32,
                                                           const float* __restrict__ dv32,
                                                           bf16* __restrict__ dk, bf16* __restrict__ dv,
                                                           size_t n, float scale) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    dk[i] = (bf16)(dk32[i] * scale);
    dv[i] = (bf16)dv32[i];
  }
}

template <int D, int G>
static hipError_t launch_single_t(const Shape& s, const void* q, const void* bimg, const int32_t* idx,
                                  const float* lse, const float* delta, const void* dos, void* dq,
                                  float* dk32, float* dv32, hipStream_t st) {
  typedef SingleCfg<D, G> C;
  const size_t lds = (size_t)C::NBUF * C::STAGE + (size_t)C::P * s.topk * 2;
  hipError_t e = hipFuncSetAttribute((const void*)bwd_single_kernel<D, G>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((s.T + C::P - 1) / C::P * s.Hkv * s.B);
  hipLaunchKernelGGL((bwd_single_kernel<D, G>), grid, dim3(C::NT), lds, st, s, (const bf16*)q,
                     (const unsigned char*)bimg, idx, lse, delta, (const bf16*)dos, (bf16*)dq, dk32, dv32);
  return hipGetLastError();
}
template <int D>
static hipError_t launch_single_g(const Shape& s, const void* q, const void* bimg, const int32_t* idx,
                                  const float* lse, const float* delta, const void* dos, void* dq,
                                  float* dk32, float* dv32, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_single_t<D, 1>(s, q, bimg, idx, lse, delta, dos, dq, dk32, dv32, st);
    case 2: return launch_single_t<D, 2>(s, q, bimg, idx, lse, delta, dos, dq, dk32, dv32, st);
    case 4: return launch_single_t<D, 4>(s, q, bimg, idx, lse, delta, dos, dq, dk32, dv32, st);
    case 8: return launch_single_t<D, 8>(s, q, bimg, idx, lse, delta, dos, dq, dk32, dv32, st);
    default: return launch_single_t<D, 16>(s, q, bimg, idx, lse, delta, dos, dq, dk32, dv32, st);
  }
}

hipError_t launch_bwd_single(const Shape& s, const void* q, const void* bimg, const int32_t* indices,
                             const float* lse, const float* delta, const void* dos, void* dq, void* dk,
                             void* dv, float* dk32, float* dv32, hipStream_t st) {
  const size_t n = (size_t)s.B * s.T * s.Hkv * s.D;
  hipLaunchKernelGGL(single_zero_kernel, dim3(1024), dim3(256), 0, st, dk32, n);
  hipLaunchKernelGGL(single_zero_kernel, dim3(1024), dim3(256), 0, st, dv32, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = s.D == 64 ? launch_single_g<64>(s, q, bimg, indices, lse, delta, dos, dq, dk32, dv32, st)
                : launch_single_g<128>(s, q, bimg, indices, lse, delta, dos, dq, dk32, dv32, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(single_round_kernel, dim3(1024), dim3(256), 0, st, dk32, dv32, (bf16*)dk, (bf16*)dv,
                     n, s.scale);
  return hipGetLastError();
}

}  // namespace nsa
