// nsa_device.h -- device-side building blocks shared by the gfx950 kernels:
// 16x16 MFMA fragments (bf16 and fp32 element types), cross-lane reductions,
// conversions and small load/store helpers.
//
// Fragment conventions (one wavefront = 64 lanes, lane l, a = l / 16):
//   A fragment of a 16 x 32 tile A[m][k] : lane l holds A[l % 16][8a + e], e = 0..7
//   B fragment of a 32 x 16 tile B[k][n] : lane l holds B[8a + e][l % 16]
//   C tile 16 x 16, fp32                 : lane l holds C[4a + r][l % 16], r = 0..3
// The hardware pairs A and B elements by (lane / 16, element), so the product
// is exact whatever physical k order the instruction uses.  bf16 fragments
// feed one v_mfma_f32_16x16x32_bf16; fp32 fragments feed eight
// v_mfma_f32_16x16x4_f32 (instruction e contracts the logical k = 8a + e).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nsa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(float)))) float f32x8;

constexpr int kBlock = 64;  // compression block = selection block
constexpr int kWave = 64;

// Element-type traits: the fragment type holding 8 consecutive k elements.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
  typedef bf16x8 type;
  static __device__ __forceinline__ type load(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
  }
  static __device__ __forceinline__ type zero() {
    type z;
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
  }
  static __device__ __forceinline__ type from_f32(const float* x) {
    type r;
    for (int i = 0; i < 8; ++i) r[i] = (bf16)x[i];
    return r;
  }
};
template <> struct Frag<float> {
  typedef f32x8 type;
  static __device__ __forceinline__ type load(const float* p) {
    const f32x4* q = reinterpret_cast<const f32x4*>(p);
    f32x4 a = q[0], b = q[1];
    type r;
    for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
    return r;
  }
  static __device__ __forceinline__ type zero() {
    type z;
    for (int i = 0; i < 8; ++i) z[i] = 0.0f;
    return z;
  }
  static __device__ __forceinline__ type from_f32(const float* x) {
    type r;
    for (int i = 0; i < 8; ++i) r[i] = x[i];
    return r;
  }
};

__device__ __forceinline__ f32x4 mma(f32x4 c, const bf16x8& a, const bf16x8& b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 zero4() {
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Reductions across the four lane groups (a = l / 16) that share a column.
__device__ __forceinline__ float colmax4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float colsum4(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// DPP move inside 16-lane rows (ctrl is a DPP control code).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
// Sum over aligned groups of G adjacent lanes inside each 16-lane row
// (G in {1, 2, 4, 8, 16}); every lane of a group receives the group sum.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (G >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (G >= 8) v += dpp<0x141>(v);  // row_half_mirror: other quad of the 8
  if constexpr (G >= 16) v += dpp<0x140>(v); // row_mirror: other half of the row
  return v;
}

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

// Store 4 consecutive elements (fp32 values, converted to T).
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
  bf16x4 r;
  for (int i = 0; i < 4; ++i) r[i] = (bf16)v[i];
  *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  bf16x4 r = *reinterpret_cast<const bf16x4*>(p);
  f32x4 o;
  for (int i = 0; i < 4; ++i) o[i] = (float)r[i];
  return o;
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
// Store 8 consecutive fp32 values (16-byte aligned source) as T.
__device__ __forceinline__ void store8(bf16* p, const float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(x), b = *reinterpret_cast<const f32x4*>(x + 4);
  bf16x8 r;
  for (int i = 0; i < 4; ++i) { r[i] = (bf16)a[i]; r[4 + i] = (bf16)b[i]; }
  *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
  reinterpret_cast<f32x4*>(p)[0] = *reinterpret_cast<const f32x4*>(x);
  reinterpret_cast<f32x4*>(p)[1] = *reinterpret_cast<const f32x4*>(x + 4);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum over the four lane groups (l / 16) that hold one MFMA column,
// with the gfx950 lane-swap instructions (VALU; no LDS crossbar traffic)
__device__ __forceinline__ float xmax4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Staged image of one 64-key block of one KV group, the unit the selection /
// window kernel copies global -> LDS.  It is the block's K and V^T as MFMA
// fragments, K fragments first: fragment f < NFRAG is K subtile u = f % 4
// (16 keys) at k step ks = f / 4; fragment NFRAG + h (D / 16) + mt is V^T
// channel tile mt (16 channels) over keys 32 h .. 32 h + 31.  Consecutive
// fragments therefore feed different accumulators (no dependent MFMA pairs
// inside a batch of fragments).  A fragment is NV pieces
// of 64 lanes x 16 bytes (lane l holds its 8 elements; fp32 needs two
// pieces), so every piece is one contiguous 1 KB copy.  Inside a 32-key half,
// MFMA row rho of K subtile u holds key 8 (rho / 4) + 4 (u % 2) + rho % 4: the
// C layout of the two S^T subtiles of a half is then the B-operand layout of
// P^T for that half.
template <typename T, int D>
struct KvImage {
  static constexpr int NV = (int)sizeof(T) * 8 / 16;   // 16-byte pieces per lane fragment
  static constexpr int EPV = 16 / (int)sizeof(T);      // elements per piece and lane
  static constexpr int KS = D / 32;
  static constexpr int NFRAG = D / 8;                  // fragments per operand (4 KS = 2 (D/16))
  static constexpr int MT = D / 16;                    // 16-channel tiles of V^T
  static __device__ __forceinline__ int k_u(int f) { return f & 3; }     // K fragment -> subtile
  static __device__ __forceinline__ int k_ks(int f) { return f >> 2; }   // K fragment -> k step
  static __device__ __forceinline__ int v_mt(int f2) { return f2 % MT; } // V fragment -> channel tile
  static __device__ __forceinline__ int v_h(int f2) { return f2 / MT; }  // V fragment -> key half
  static constexpr int PIECES = 2 * NFRAG * NV;
  static constexpr int BYTES = PIECES * 1024;
  // key (0..63 within the block) in K fragment row rho (= lane % 16) of subtile u
  static __device__ __forceinline__ int krow(int u, int rho) {
    return 32 * (u >> 1) + 8 * (rho >> 2) + 4 * (u & 1) + (rho & 3);
  }
};

// Staged image of one 64-key block for the query-stationary backward (dq):
// K, V and K^T as MFMA fragments, one after the other.  Fragment f < NFRAG
// is K subtile u = f % 4 at k step ks = f / 4 (as in KvImage); fragment
// NFRAG + f is the same for V; fragment 2 NFRAG + h (D / 16) + mt is K^T
// channel tile mt over keys 32 h .. 32 h + 31 (the A operand of dq^T =
// K^T dS^T).  Pieces of 64 lanes x 16 bytes, as in KvImage.
template <typename T, int D>
struct BwdImage {
  typedef KvImage<T, D> K;
  static constexpr int NV = K::NV, EPV = K::EPV, KS = K::KS, NFRAG = K::NFRAG, MT = K::MT;
  static constexpr int PIECES = 3 * NFRAG * NV;
  static constexpr int BYTES = PIECES * 1024;
};

// ---- helpers of the block-walking kernels (selection/window forward, dq) ----
// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Workgroup barrier that is also a compiler memory barrier but, unlike
// __syncthreads, does not drain the outstanding global->LDS loads.
__device__ __forceinline__ void barrier_keep_loads() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// lane fragment (8 elements) stored as [NV][64 lanes][16 bytes] in LDS
template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const unsigned char* base, int l);
template <>
__device__ __forceinline__ bf16x8 lds_frag<bf16>(const unsigned char* base, int l) {
  return *reinterpret_cast<const bf16x8*>(base + 16 * l);
}
template <>
__device__ __forceinline__ f32x8 lds_frag<float>(const unsigned char* base, int l) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(base + 16 * l);
  const f32x4 b = *reinterpret_cast<const f32x4*>(base + 1024 + 16 * l);
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) { r[i] = a[i]; r[4 + i] = b[i]; }
  return r;
}

// Sum of the 8 probabilities of a B fragment (the values the PV MFMA uses).
__device__ __forceinline__ float frag_sum(const bf16x8& p) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {p[2 * i], p[2 * i + 1]};
    s = __builtin_amdgcn_fdot2_f32_bf16(pr, one, s, false);
  }
  return s;
}
__device__ __forceinline__ float frag_sum(const f32x8& p) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += p[i];
  return s;
}
// lanes whose condition is false get an all-zero fragment
__device__ __forceinline__ bf16x8 frag_keep(const bf16x8& p, bool keep) {
  typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
  u32x4 u = __builtin_bit_cast(u32x4, p);
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = keep ? u[i] : 0u;
  return __builtin_bit_cast(bf16x8, u);
}
__device__ __forceinline__ f32x8 frag_keep(const f32x8& p, bool keep) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = keep ? p[i] : 0.f;
  return r;
}

// minimum over each 16-lane row (DPP butterfly; every lane gets its row's minimum)
__device__ __forceinline__ int row_min16(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true));   // lane ^ 1
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true));   // lane ^ 2
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, true));  // other quad of 8
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, true));  // other half of 16
  return v;
}

// key (0..63 within the block) of C-layout element (subtile u, register r) in lane group a
__device__ __forceinline__ int key_of(int u, int a, int r) { return 32 * (u >> 1) + 8 * a + 4 * (u & 1) + r; }

// Work order for a 1-D grid over (batch * kv-group) x tiles.  Workgroups are
// dealt to the 8 XCDs round-robin (XCD = id % 8), each XCD with its own L2.
// When the number of (batch, group) pairs NBG divides 8 or is a multiple of
// it, every XCD is given whole (batch, group) pairs -- their K/V stay in that
// XCD's L2 -- and within an XCD tiles go out largest-first (the tile cost
// grows with its position), so the last wave of workgroups is short.
__device__ __forceinline__ void xcd_order(int L, int N, int NBG, int NTL, int& bg, int& tile) {
  constexpr int X = 8;
  const int x = L % X, sl = L / X;
  if (N % X == 0 && X % NBG == 0) {
    const int share = X / NBG;  // XCDs per (batch, group)
    bg = x / share;
    const int r = sl * share + x % share;
    tile = NTL - 1 - r;
  } else if (N % X == 0 && NBG % X == 0) {
    const int per = NBG / X;    // (batch, group) pairs per XCD
    bg = x + X * (sl / NTL);
    (void)per;
    tile = NTL - 1 - sl % NTL;
  } else {
    bg = L / NTL;
    tile = NTL - 1 - L % NTL;
  }
}

}  // namespace nsa
