// bwd_dq.hip -- B2: dq of the selection branch, query-stationary.
//
// [SIC] "Sparsity is Cool", Method (NSA implementation): the selection-branch
// backward as two passes -- this query-stationary pass computes dq, the
// key/value-stationary pass (bwd.hip) dk and dv, so neither needs atomics.
// With P_s = exp(tau q.k_s - lse) (the forward's log-sum-exp), dP_s = dOs.v_s,
// Delta = dOs.o_sel and dS_s = P_s (dP_s - Delta):  dq = tau sum_s dS_s k_s
// over the keys s <= t of the blocks the row's position selected.
//
// The walk is the one of the forward's selection / window kernel: one
// workgroup per (tile of P positions, KV group g, batch b); each wave owns one
// 16-row column group (16/G positions x G heads) with its q and dOs fragments
// and its dq accumulator (MFMA C layout of dq^T: lane = row) in registers.
// Key blocks 0 .. own(last position) are walked once; each block's backward
// image (K, V and K^T fragments, written by the preparation kernel) is copied
// global -> LDS by global_load_lds into a ring of two groups of blocks (one
// barrier per group).  Per block and column group that attends it (scalar
// test on the next selected block of its rows):
//   S^T = K Q^T, dP^T = V dOs^T          (16-key subtiles, key order of the
//                                          image: C layout = B layout of dS^T)
//   P = exp2(tau log2(e) s - lse2),       rows that did not select the block
//                                          get lse2 = +inf (P = 0)
//   dS = P (dP - Delta) -> bf16,  dq^T += K^T dS^T.
// Deterministic (no atomics).
#include <math.h>

#include "nsa_device.h"
#include "nsa_launch.h"

#ifndef NSA_DQ_RING_BYTES
#define NSA_DQ_RING_BYTES (144 * 1024)
#endif

namespace nsa {

template <typename T, int D, int G>
struct DqCfg {
  typedef BwdImage<T, D> Img;
  static constexpr bool WIDE = D == 128 || sizeof(T) == 4;
  static constexpr int NW = WIDE ? 12 : 16;       // waves per workgroup (one column group each)
  static constexpr int NT = NW * 64;
  static constexpr int NSG = 16 / G;              // positions per column group
  static constexpr int P = NW * NSG;              // positions per workgroup
  static constexpr int KS = D / 32, MT = D / 16;
  static constexpr int NV = Img::NV, NFRAG = Img::NFRAG;
  static constexpr int FCH = (NFRAG < 2 ? NFRAG : 2) / NV > 0 ? (NFRAG < 2 ? NFRAG : 2) / NV : 1;
  static constexpr int FRAG_BYTES = NV * 1024;
  static constexpr int STAGE = Img::BYTES;
  static constexpr int GB = (NSA_DQ_RING_BYTES / STAGE / 2) < 4 ? (NSA_DQ_RING_BYTES / STAGE / 2) : 4;
  static constexpr int NBUF = 2 * GB;
  static constexpr int LOADS = Img::PIECES;
  static_assert(GB >= 1, "ring too small");
  static_assert(NSG * G == 16, "column group = 16 rows");
};

template <typename T, int D, int G>
static size_t dq_lds_bytes(int topk) {
  typedef DqCfg<T, D, G> C;
  return (size_t)C::NBUF * C::STAGE + (size_t)C::P * topk * 2;
}

// Branch of a dq pass.  SEL: the selected blocks (rows that did not select a
// block get lse2 = +inf); WIN: the blocks meeting a row's window, keys
// t - W < s <= t; CMP: "blocks" of 64 pooled keys (the pooled-key images),
// pooled key jj visible to t when 64 (jj + 1) - 1 <= t.
enum { DQ_SEL = 0, DQ_WIN = 1, DQ_CMP = 2 };

template <typename T, int D, int G, int MODE>
__global__ __launch_bounds__((DqCfg<T, D, G>::NT)) void bwd_dq_kernel(
    Shape s, const T* __restrict__ q, const unsigned char* __restrict__ bimg,
    const int32_t* __restrict__ indices, const float* __restrict__ lse,
    const float* __restrict__ delta, const T* __restrict__ dos, const float* __restrict__ acc_in,
    float* __restrict__ acc_out, T* __restrict__ dq) {
  typedef DqCfg<T, D, G> C;
  constexpr int NT = C::NT, P = C::P, NSG = C::NSG, KS = C::KS, MT = C::MT;
  constexpr int NFRAG = C::NFRAG, FCH = C::FCH, FRAG_BYTES = C::FRAG_BYTES, STAGE = C::STAGE;
  constexpr int GB = C::GB, LOADS = C::LOADS;
  typedef typename Frag<T>::type FragT;
  typedef typename C::Img::K KI;  // fragment index helpers of the image
  const float INF = __builtin_inff();

  const int nimg = MODE == DQ_CMP ? (s.nc + kBlock - 1) / kBlock : s.T / kBlock;  // images per (b, g)
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
  const int W = s.W;
  const size_t q_row = (size_t)s.Hq * D;
  const unsigned char* img_b = bimg + ((size_t)b * s.Hkv + g) * nimg * (size_t)STAGE;

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;                                                  // [NBUF][STAGE]
  int16_t* lists = reinterpret_cast<int16_t*>(smem + (size_t)C::NBUF * STAGE);  // [P][topk]

  if constexpr (MODE == DQ_SEL) {
    for (int i = threadIdx.x; i < P * topk; i += NT) {
      const int p = i / topk, e = i % topk;
      const int j = p < nvalid ? indices[(((size_t)b * s.Hkv + g) * s.T + t0 + p) * topk + e] : -1;
      lists[i] = (int16_t)(j < 0 ? 0x7fff : j);
    }
  }

  // this lane's row: position p, head h
  const int pf = w * NSG;  // first position of the column group
  const int p = pf + sg;
  const int t = t0 + p;
  const bool valid = p < nvalid;
  const int own = (t0 + pf) / kBlock;
  const int nvf = min(max(nvalid - pf, 0), NSG);  // valid positions of the column group
  const int tf = t0 + pf, tl = tf + max(nvf, 1) - 1;
  FragT qf[KS], df[KS];
  float lse2 = INF, dl = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (valid) {
      const size_t o = ((size_t)b * s.T + t) * q_row + (size_t)h * D + ks * 32 + 8 * a;
      qf[ks] = Frag<T>::load(q + o);
      df[ks] = Frag<T>::load(dos + o);
    } else {
      qf[ks] = Frag<T>::zero();
      df[ks] = Frag<T>::zero();
    }
  }
  if (valid) {
    lse2 = lse[((size_t)b * s.Hq + h) * s.T + t] * kLog2e;
    dl = delta[((size_t)b * s.Hq + h) * s.T + t];
  }
  __syncthreads();  // lists visible
  int ptr = 0;
  int nxt = 0x7fff, nsel = 0x7fff;
  if constexpr (MODE == DQ_SEL) {
    nxt = valid ? lists[p * topk] : 0x7fff;
    nsel = __builtin_amdgcn_readfirstlane(row_min16(nxt));
  }
  // per column group (scalar): the window blocks and the edge block; the
  // pooled blocks with a key visible to the group's last / first position
  const int jw_lo = max(0, tf - W + 1) / kBlock;
  const int jw_edge = tl >= W ? (tl - W) / kBlock : -1;
  const int nvis_l = (tl + 1) / kBlock, nvis_f = (tf + 1) / kBlock;  // pooled keys visible
  const int nvis = (t + 1) / kBlock;

  const int t_last = t0 + nvalid - 1;
  int j_begin = 0, j_end = 0;  // walk [j_begin, j_end)
  if constexpr (MODE == DQ_SEL) { j_begin = 0; j_end = t_last / kBlock + 1; }
  if constexpr (MODE == DQ_WIN) { j_begin = max(0, t0 - W + 1) / kBlock; j_end = t_last / kBlock + 1; }
  if constexpr (MODE == DQ_CMP) { j_begin = 0; j_end = ((t_last + 1) / kBlock + kBlock - 1) / kBlock; }
  const int nblk = max(j_end - j_begin, 0);

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

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = zero4();

  const int ngrp = (nblk + GB - 1) / GB;
  auto issue_group = [&](int gi) {
#pragma unroll
    for (int qq = 0; qq < GB; ++qq)
      if (gi * GB + qq < nblk) issue(j_begin + gi * GB + qq, (gi & 1) * GB + qq);
  };
  if (ngrp > 0) issue_group(0);

  for (int gi = 0; gi < ngrp; ++gi) {
    wait_vmcnt<0>();       // this wave's loads of group gi (the only ones in flight)
    barrier_keep_loads();  // all of group gi is in LDS; group gi-1's slots are free
    if (gi + 1 < ngrp) issue_group(gi + 1);
    // the group's blocks this column group attends, visited directly (the
    // scalar tests of blocks it skips cost issue slots every wave pays):
    // selection -- from one selected block of its rows to the next;
    // window / compression -- the group's part of a contiguous range
    const int jg0 = j_begin + gi * GB, jg1 = min(jg0 + GB, j_begin + nblk);
    int jl = jg0, jh = jg1;
    if constexpr (MODE == DQ_WIN) {
      jl = max(jg0, jw_lo);
      jh = nvf > 0 ? min(jg1, own + 1) : jl;
    } else if constexpr (MODE == DQ_CMP) {
      jh = nvf > 0 ? min(jg1, (nvis_l + kBlock - 1) / kBlock) : jl;
    }
    for (int j = MODE == DQ_SEL ? nsel : jl; j < (MODE == DQ_SEL ? jg1 : jh);
         j = MODE == DQ_SEL ? nsel : j + 1) {
      const int qq = j - jg0;
      // does the block need the element mask; the row's reference
      bool masked;
      float lr;
      if constexpr (MODE == DQ_SEL) {
        const bool sl = nxt == j;
        if (sl) {
          ++ptr;
          nxt = ptr < topk ? lists[p * topk + ptr] : 0x7fff;
        }
        nsel = __builtin_amdgcn_readfirstlane(row_min16(nxt));  // > j: the lists ascend
        masked = j == own;
        lr = sl ? lse2 : INF;
      } else if constexpr (MODE == DQ_WIN) {
        masked = j == own || j <= jw_edge;
        lr = lse2;
      } else {
        masked = j * kBlock + kBlock > nvis_f;
        lr = lse2;
      }
      const unsigned char* stage = ring + (size_t)((gi & 1) * GB + qq) * STAGE;

      // S^T = K Q^T and dP^T = V dOs^T (K and V fragments in batches of FCH)
      f32x4 st[4], dp[4];
#pragma unroll
      // dP^T accumulates onto -Delta (the row's, in every element of the lane's
      // column), so dP - Delta comes out of the MFMA
      for (int u = 0; u < 4; ++u) { st[u] = zero4(); dp[u] = f32x4{-dl, -dl, -dl, -dl}; }
#pragma unroll
      for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
        FragT kf[FCH], vf[FCH];
#pragma unroll
        for (int i = 0; i < FCH; ++i) {
          kf[i] = lds_frag<T>(stage + (size_t)(f0 + i) * FRAG_BYTES, l);
          vf[i] = lds_frag<T>(stage + (size_t)(NFRAG + f0 + i) * FRAG_BYTES, l);
        }
#pragma unroll
        for (int i = 0; i < FCH; ++i) {
          const int u = KI::k_u(f0 + i), ks = KI::k_ks(f0 + i);
          st[u] = mma(st[u], kf[i], qf[ks]);
          dp[u] = mma(dp[u], vf[i], df[ks]);
        }
      }

      // dS = P (dP - Delta), P from the saved log-sum-exp; element mask on
      // the causal diagonal / window edge / pooled-key visibility boundary
      FragT dsf[2];
      if (!masked) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 2 * hf + e / 4, rr = e % 4;
            const float pr = fast_exp2(st[u][rr] * c1 - lr);
            x[e] = pr * dp[u][rr];
          }
          dsf[hf] = Frag<T>::from_f32(x);
        }
      } else {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = 2 * hf + e / 4, rr = e % 4;
            const int key = j * kBlock + key_of(u, a, rr);
            bool ok;
            if constexpr (MODE == DQ_SEL) ok = key <= t;
            else if constexpr (MODE == DQ_WIN) ok = key <= t && key > t - W;
            else ok = key < nvis;
            const float pr = ok ? fast_exp2(st[u][rr] * c1 - lr) : 0.f;
            x[e] = pr * dp[u][rr];
          }
          dsf[hf] = Frag<T>::from_f32(x);
        }
      }

      // dq^T += K^T dS^T (K^T fragments in batches)
#pragma unroll
      for (int f0 = 0; f0 < NFRAG; f0 += FCH) {
        FragT tf_[FCH];
#pragma unroll
        for (int i = 0; i < FCH; ++i) tf_[i] = lds_frag<T>(stage + (size_t)(2 * NFRAG + f0 + i) * FRAG_BYTES, l);
#pragma unroll
        for (int i = 0; i < FCH; ++i)
          acc[KI::v_mt(f0 + i)] = mma(acc[KI::v_mt(f0 + i)], tf_[i], dsf[KI::v_h(f0 + i)]);
      }
    }
  }

  if (valid) {
    const size_t o = ((size_t)b * s.T + t) * q_row + (size_t)h * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 r = acc[mt] * s.scale;
      if (acc_in) r += *reinterpret_cast<const f32x4*>(acc_in + o + mt * 16 + 4 * a);
      if (acc_out) *reinterpret_cast<f32x4*>(acc_out + o + mt * 16 + 4 * a) = r;
      if (dq) store4(dq + o + mt * 16 + 4 * a, r);
    }
  }
}

template <typename T, int D, int G, int MODE>
static hipError_t launch_dq_t(const Shape& s, const DqArgs& x, hipStream_t st) {
  typedef DqCfg<T, D, G> C;
  const size_t lds = dq_lds_bytes<T, D, G>(s.topk);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)bwd_dq_kernel<T, D, G, MODE>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid((s.T + C::P - 1) / C::P * s.Hkv * s.B);
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, G, MODE>), grid, dim3(C::NT), lds, st, s, (const T*)x.q,
                     (const unsigned char*)x.img, x.indices, x.lse, x.delta, (const T*)x.dos,
                     x.acc_in, x.acc_out, (T*)x.dq);
  return hipGetLastError();
}
template <typename T, int D, int MODE>
static hipError_t launch_dq_g(const Shape& s, const DqArgs& x, hipStream_t st) {
  switch (s.G) {
    case 1: return launch_dq_t<T, D, 1, MODE>(s, x, st);
    case 2: return launch_dq_t<T, D, 2, MODE>(s, x, st);
    case 4: return launch_dq_t<T, D, 4, MODE>(s, x, st);
    case 8: return launch_dq_t<T, D, 8, MODE>(s, x, st);
    default: return launch_dq_t<T, D, 16, MODE>(s, x, st);
  }
}
template <int MODE>
static hipError_t launch_dq_m(bool is_bf16, const Shape& s, const DqArgs& x, hipStream_t st) {
  if (is_bf16) {
    if (s.D == 64) return launch_dq_g<bf16, 64, MODE>(s, x, st);
    return launch_dq_g<bf16, 128, MODE>(s, x, st);
  }
  return launch_dq_g<float, 64, MODE>(s, x, st);
}

hipError_t launch_bwd_dq(bool is_bf16, const Shape& s, int mode, const DqArgs& x, hipStream_t st) {
  if (mode == DQ_WIN) return launch_dq_m<DQ_WIN>(is_bf16, s, x, st);
  if (mode == DQ_CMP) return launch_dq_m<DQ_CMP>(is_bf16, s, x, st);
  return launch_dq_m<DQ_SEL>(is_bf16, s, x, st);
}

}  // namespace nsa
