// api.hip -- the C ABI declared in include/nsa.h: parameter checks, workspace
// carving and launch sequencing.  Nothing here computes; every step of the
// path runs in the gfx950 kernels (pool.hip, cmp_select.hip, sel_win.hip,
// bwd.hip, bwd_dq.hip, bwd_dkdv.hip).  No allocation, no synchronisation, no global mutable state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/nsa.h"
#include "nsa_launch.h"

using nsa::Shape;

namespace {

constexpr size_t kAlign = 256;
inline size_t up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

nsa_status_t check(const nsa_params_t* p) {
  if (!p) return NSA_ERR_NULL;
  if (p->batch < 1 || p->seq_len < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 ||
      p->head_dim < 1 || p->block < 1 || p->top_k < 2 || p->window < 1)
    return NSA_ERR_SHAPE;
  if (p->n_q_heads % p->n_kv_heads != 0) return NSA_ERR_SHAPE;
  if (p->dtype != NSA_BF16 && p->dtype != NSA_FP32) return NSA_ERR_DTYPE;
  const int G = p->n_q_heads / p->n_kv_heads;
  if (p->head_dim != 64 && p->head_dim != 128) return NSA_ERR_UNSUPPORTED;
  if (p->dtype == NSA_FP32 && p->head_dim != 64) return NSA_ERR_UNSUPPORTED;
  if (p->block != 64) return NSA_ERR_UNSUPPORTED;
  if (p->seq_len % 64 != 0 || p->seq_len > 65536) return NSA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return NSA_ERR_UNSUPPORTED;
  if (p->top_k > 32) return NSA_ERR_UNSUPPORTED;
  if (p->flags & ~0xFu) return NSA_ERR_UNSUPPORTED;
  return NSA_OK;
}

Shape make_shape(const nsa_params_t* p) {
  Shape s;
  s.B = p->batch;
  s.T = p->seq_len;
  s.Hq = p->n_q_heads;
  s.Hkv = p->n_kv_heads;
  s.D = p->head_dim;
  s.G = s.Hq / s.Hkv;
  s.topk = p->top_k;
  s.W = p->window;
  s.nc = s.T / 64;
  s.ncp = (s.nc + 63) / 64 * 64;
  s.scale = p->scale > 0.f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  s.flags = p->flags;
  return s;
}

// Forward workspace regions (byte offsets from the workspace base).
struct FwdLayout {
  size_t kc, kcl, vc, vct, kvimg, knorm, o_cmp, indices, total;
};
FwdLayout fwd_layout(const Shape& s, size_t es) {
  FwdLayout L;
  size_t o = 0;
  L.kc = o;      o += up((size_t)s.B * s.nc * s.Hkv * s.D * es, kAlign);
  L.kcl = o;     o += up((size_t)s.B * s.nc * s.Hkv * s.D * es, kAlign);
  L.vc = o;      o += up((size_t)s.B * s.nc * s.Hkv * s.D * es, kAlign);
  L.vct = o;     o += up((size_t)s.B * s.Hkv * s.D * s.ncp * es, kAlign);
  L.kvimg = o;   o += up((size_t)s.B * s.Hkv * s.nc * 2 * 64 * s.D * es, kAlign);
  L.knorm = o;   o += up((size_t)s.B * s.Hkv * s.nc * 4, kAlign);
  L.o_cmp = o;   o += up((size_t)s.B * s.T * s.Hq * s.D * es, kAlign);
  L.indices = o; o += up((size_t)s.B * s.Hkv * s.T * s.topk * 4, kAlign);
  L.total = o;
  return L;
}

// Backward workspace regions (full: all three branches, nsa_backward).
struct BwdLayout {
  size_t bimg, delta, dos, revmap, lists, counts, items, slot_base, slot_cnt, nitems, part;
  size_t pimg, kc, vc, dos_w, dos_c, delta_w, delta_c, dq32, slot_base_c, slot_cnt_c, total;
};
BwdLayout bwd_layout(const Shape& s, size_t es, bool full) {
  BwdLayout L;
  size_t o = 0;
  const size_t nblk = s.T / 64, NJ = (size_t)s.B * s.Hkv * nblk;
  const size_t NJc = (size_t)s.B * s.Hkv * ((s.nc + 63) / 64);
  const size_t rows = (size_t)s.B * s.Hq * s.T, elems = rows * s.D;
  L.bimg = o;      o += up(NJ * 3 * 64 * s.D * es, kAlign);
  L.delta = o;     o += up(rows * 4, kAlign);
  L.dos = o;       o += up(elems * es, kAlign);
  L.revmap = o;    o += up(NJ * nblk * 8, kAlign);
  L.lists = o;     o += up(NJ * s.T * 2, kAlign);
  L.counts = o;    o += up(NJ * 4, kAlign);
  L.items = o;     o += up(nsa::bwd_items_bytes(s, full), kAlign);
  L.slot_base = o; o += up(NJ * 4, kAlign);
  L.slot_cnt = o;  o += up(NJ * 4, kAlign);
  L.nitems = o;    o += up(4, kAlign);
  L.part = o;      o += up(nsa::bwd_part_floats(s, full) * 4, kAlign);
  L.pimg = L.kc = L.vc = L.dos_w = L.dos_c = L.delta_w = L.delta_c = L.dq32 = 0;
  L.slot_base_c = L.slot_cnt_c = 0;
  if (full) {
    L.pimg = o;        o += up(NJc * 3 * 64 * s.D * es, kAlign);
    L.kc = o;          o += up((size_t)s.B * s.nc * s.Hkv * s.D * es, kAlign);
    L.vc = o;          o += up((size_t)s.B * s.nc * s.Hkv * s.D * es, kAlign);
    L.dos_w = o;       o += up(elems * es, kAlign);
    L.dos_c = o;       o += up(elems * es, kAlign);
    L.delta_w = o;     o += up(rows * 4, kAlign);
    L.delta_c = o;     o += up(rows * 4, kAlign);
    L.dq32 = o;        o += up(elems * 4, kAlign);
    L.slot_base_c = o; o += up(NJc * 4, kAlign);
    L.slot_cnt_c = o;  o += up(NJc * 4, kAlign);
  }
  L.total = o;
  return L;
}

nsa::BwdPlanWs plan_ws(char* ws, const BwdLayout& L) {
  nsa::BwdPlanWs pw;
  pw.items = ws + L.items;
  pw.lists = (uint16_t*)(ws + L.lists);
  pw.counts = (int*)(ws + L.counts);
  pw.slot_base = (int*)(ws + L.slot_base);
  pw.slot_cnt = (int*)(ws + L.slot_cnt);
  pw.slot_base_c = L.slot_base_c ? (int*)(ws + L.slot_base_c) : nullptr;
  pw.slot_cnt_c = L.slot_cnt_c ? (int*)(ws + L.slot_cnt_c) : nullptr;
  pw.nitems = (int*)(ws + L.nitems);
  pw.part = (float*)(ws + L.part);
  return pw;
}

inline size_t esize(const nsa_params_t* p) { return p->dtype == NSA_BF16 ? 2 : 4; }

nsa_status_t launched(hipError_t e) { return e == hipSuccess ? NSA_OK : NSA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int nsa_abi_version(void) { return NSA_ABI_VERSION; }

const char* nsa_status_string(nsa_status_t st) {
  switch (st) {
    case NSA_OK: return "NSA_OK";
    case NSA_ERR_NULL: return "NSA_ERR_NULL: a required pointer is NULL";
    case NSA_ERR_SHAPE: return "NSA_ERR_SHAPE: inconsistent or out-of-range sizes";
    case NSA_ERR_DTYPE: return "NSA_ERR_DTYPE: unknown dtype";
    case NSA_ERR_UNSUPPORTED: return "NSA_ERR_UNSUPPORTED: outside the GPU support envelope";
    case NSA_ERR_WORKSPACE: return "NSA_ERR_WORKSPACE: workspace missing or too small";
    case NSA_ERR_ALIGN: return "NSA_ERR_ALIGN: device pointer not 16-byte aligned";
    case NSA_ERR_LAUNCH: return "NSA_ERR_LAUNCH: kernel launch failed";
  }
  return "NSA_ERR_UNKNOWN";
}

nsa_status_t nsa_check_params(const nsa_params_t* p) { return check(p); }

const char* nsa_forward_kernel(const nsa_params_t* p) {
  if (check(p) != NSA_OK) return nullptr;
  return nsa::sel_win_kernel_name(p->dtype == NSA_BF16, make_shape(p));
}

size_t nsa_workspace_size(const nsa_params_t* p, int for_backward) {
  if (check(p) != NSA_OK) return 0;
  const Shape s = make_shape(p);
  if (for_backward == 2) return bwd_layout(s, esize(p), true).total;
  if (for_backward == 3)  // single-pass selection backward: + fp32 dk, dv accumulators
    return bwd_layout(s, esize(p), false).total + 2 * up((size_t)s.B * s.T * s.Hkv * s.D * 4, kAlign);
  return for_backward ? bwd_layout(s, esize(p), false).total : fwd_layout(s, esize(p)).total;
}

nsa_status_t nsa_pool(const void* k, const void* v, const nsa_params_t* p, void* k_cmp,
                      void* v_cmp, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!k || !v || !k_cmp || !v_cmp) return NSA_ERR_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cmp) || !aligned16(v_cmp)) return NSA_ERR_ALIGN;
  const Shape s = make_shape(p);
  return launched(nsa::launch_pool(p->dtype == NSA_BF16, s, k, v, k_cmp, v_cmp, nullptr, nullptr,
                                   nullptr, nullptr, (hipStream_t)stream));
}

nsa_status_t nsa_compress_select(const void* q, const void* k, const void* v,
                                 const nsa_params_t* p, void* o_cmp, int32_t* indices,
                                 void* workspace, size_t ws_bytes, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !o_cmp || !indices) return NSA_ERR_NULL;
  if (!workspace) return NSA_ERR_WORKSPACE;
  const Shape s = make_shape(p);
  const size_t es = esize(p);
  const FwdLayout L = fwd_layout(s, es);
  if (ws_bytes < L.total) return NSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_cmp) || !aligned16(indices) ||
      ((uintptr_t)workspace % kAlign) != 0)
    return NSA_ERR_ALIGN;
  char* ws = (char*)workspace;
  const bool bf = p->dtype == NSA_BF16;
  hipStream_t hs = (hipStream_t)stream;
  void* kcl = bf ? ws + L.kcl : nullptr;
  hipError_t e = nsa::launch_pool(bf, s, k, v, ws + L.kc, ws + L.vc, ws + L.vct, nullptr,
                                  nullptr, kcl, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_cmp_select(bf, s, q, ws + L.kc, kcl, ws + L.vct, o_cmp, nullptr, indices, true, hs);
  return launched(e);
}

}  // extern "C"

namespace {

// The forward with every optional output: indices (output, or input with
// NSA_INDICES_IN), the selection / window / compression log-sum-exps and
// ungated branch outputs (each nullable; o_cmp_out replaces the workspace copy).
nsa_status_t forward_impl(const void* q, const void* k, const void* v, const void* gates,
                          const nsa_params_t* p, void* out, int32_t* indices, float* lse_sel,
                          void* o_sel, float* lse_win, void* o_win, float* lse_cmp, void* o_cmp_out,
                          void* workspace, size_t ws_bytes, void* stream, void* const* events) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !gates || !out) return NSA_ERR_NULL;
  const bool idx_in = (p->flags & NSA_INDICES_IN) != 0;
  if (idx_in && !indices) return NSA_ERR_NULL;
  if (!workspace) return NSA_ERR_WORKSPACE;
  const Shape s = make_shape(p);
  const size_t es = esize(p);
  const FwdLayout L = fwd_layout(s, es);
  if (ws_bytes < L.total) return NSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gates) || !aligned16(out) ||
      (indices && !aligned16(indices)) || (lse_sel && !aligned16(lse_sel)) ||
      (o_sel && !aligned16(o_sel)) || (lse_win && !aligned16(lse_win)) ||
      (o_win && !aligned16(o_win)) || (lse_cmp && !aligned16(lse_cmp)) ||
      (o_cmp_out && !aligned16(o_cmp_out)) || ((uintptr_t)workspace % kAlign) != 0)
    return NSA_ERR_ALIGN;

  char* ws = (char*)workspace;
  const bool bf = p->dtype == NSA_BF16;
  hipStream_t hs = (hipStream_t)stream;
  const bool cmp_out = !(p->flags & NSA_SKIP_CMP_OUT);
  const bool sel_out = !(p->flags & NSA_SKIP_SEL);
  const bool need_sel = sel_out || lse_sel || o_sel;
  const bool need_topk = !idx_in && (need_sel || indices);
  const bool need_k2 = cmp_out || need_topk || lse_cmp || o_cmp_out;
  int32_t* idx = indices ? indices : (int32_t*)(ws + L.indices);
  void* o_cmp = o_cmp_out ? o_cmp_out : ws + L.o_cmp;

  void* kcl = bf ? ws + L.kcl : nullptr;
  auto mark = [&](int i) {
    if (events && events[i]) (void)hipEventRecord((hipEvent_t)events[i], hs);
  };
  mark(0);
  hipError_t e = nsa::launch_pool(bf, s, k, v, ws + L.kc, ws + L.vc, ws + L.vct, ws + L.kvimg,
                                  (float*)(ws + L.knorm), kcl, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  mark(1);
  if (need_k2) {
    e = nsa::launch_cmp_select(bf, s, q, ws + L.kc, kcl, ws + L.vct,
                               (cmp_out || o_cmp_out) ? o_cmp : nullptr, lse_cmp, idx, need_topk, hs);
    if (e != hipSuccess) return NSA_ERR_LAUNCH;
  }
  mark(2);
  e = nsa::launch_sel_win(bf, s, q, k, ws + L.kvimg, gates, o_cmp, (const float*)(ws + L.knorm), idx,
                          out, lse_sel, o_sel, lse_win, o_win, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  mark(3);
  return NSA_OK;
}

}  // namespace

extern "C" {

nsa_status_t nsa_forward_profile(const void* q, const void* k, const void* v, const void* gates,
                                 const nsa_params_t* p, void* out, int32_t* indices,
                                 float* lse_sel, void* o_sel, void* workspace, size_t ws_bytes,
                                 void* stream, void* const* events) {
  return forward_impl(q, k, v, gates, p, out, indices, lse_sel, o_sel, nullptr, nullptr, nullptr,
                      nullptr, workspace, ws_bytes, stream, events);
}

nsa_status_t nsa_forward_train(const void* q, const void* k, const void* v, const void* gates,
                               const nsa_params_t* p, void* out, const nsa_saved_t* sv,
                               void* workspace, size_t ws_bytes, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!sv || !sv->indices || !sv->lse_sel || !sv->lse_win || !sv->lse_cmp || !sv->o_sel ||
      !sv->o_win || !sv->o_cmp)
    return NSA_ERR_NULL;
  if (p->flags & ~(uint32_t)NSA_INDICES_IN) return NSA_ERR_UNSUPPORTED;
  return forward_impl(q, k, v, gates, p, out, sv->indices, sv->lse_sel, sv->o_sel, sv->lse_win,
                      sv->o_win, sv->lse_cmp, sv->o_cmp, workspace, ws_bytes, stream, nullptr);
}

nsa_status_t nsa_forward(const void* q, const void* k, const void* v, const void* gates,
                         const nsa_params_t* p, void* out, int32_t* indices, float* lse_sel,
                         void* o_sel, void* workspace, size_t ws_bytes, void* stream) {
  return nsa_forward_profile(q, k, v, gates, p, out, indices, lse_sel, o_sel, workspace, ws_bytes,
                             stream, nullptr);
}

}  // extern "C"

// Workspace of nsa_forward_noalloc: one fixed device array per GPU, held from
// the library's load until the process ends.  In host code `scratch` only
// names the symbol; its device address (per device) comes from
// hipGetSymbolAddress and is the only form ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[NSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (nullptr: not yet)

// Device address of this device's scratch array (looked up once per device,
// with that device current).  nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

nsa_status_t nsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gates,
                                 const nsa_params_t* p, void* out, int32_t* indices,
                                 float* lse_sel, void* o_sel, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !gates || !out) return NSA_ERR_NULL;
  if ((p->flags & NSA_INDICES_IN) && !indices) return NSA_ERR_NULL;
  const Shape s = make_shape(p);
  if (fwd_layout(s, esize(p)).total > (size_t)NSA_NOALLOC_SCRATCH_BYTES) return NSA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return NSA_ERR_LAUNCH;
  return forward_impl(q, k, v, gates, p, out, indices, lse_sel, o_sel, nullptr, nullptr, nullptr,
                      nullptr, ws, (size_t)NSA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

nsa_status_t nsa_select_bwd(const void* q, const void* k, const void* v, const void* gates,
                            const int32_t* indices, const float* lse_sel, const void* o_sel,
                            const void* dout, const nsa_params_t* p, void* dq, void* dk,
                            void* dv, void* workspace, size_t ws_bytes, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !gates || !indices || !lse_sel || !o_sel || !dout || !dq || !dk || !dv)
    return NSA_ERR_NULL;
  if (!workspace) return NSA_ERR_WORKSPACE;
  const Shape s = make_shape(p);
  const size_t es = esize(p);
  const BwdLayout L = bwd_layout(s, es, false);
  if (ws_bytes < L.total) return NSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gates) || !aligned16(indices) ||
      !aligned16(lse_sel) || !aligned16(o_sel) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || ((uintptr_t)workspace % kAlign) != 0)
    return NSA_ERR_ALIGN;
  char* ws = (char*)workspace;
  const bool bf = p->dtype == NSA_BF16;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = nsa::launch_bwd_prep(bf, s, k, v, gates, o_sel, dout, ws + L.bimg,
                                      (float*)(ws + L.delta), ws + L.dos, nullptr, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_bwd_revmap(s, indices, (uint64_t*)(ws + L.revmap), hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  nsa::DqArgs da{q, ws + L.bimg, indices, lse_sel, (const float*)(ws + L.delta), ws + L.dos,
                 nullptr, nullptr, dq};
  e = nsa::launch_bwd_dq(bf, s, 0, da, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  nsa::KvBranches br{false, q, ws + L.bimg, nullptr,
                     {lse_sel, nullptr, nullptr},
                     {(const float*)(ws + L.delta), nullptr, nullptr},
                     {ws + L.dos, nullptr, nullptr}};
  e = nsa::launch_bwd_dkdv(bf, s, br, (const uint64_t*)(ws + L.revmap), dk, dv, plan_ws(ws, L), hs);
  return launched(e);
}

nsa_status_t nsa_select_bwd_single(const void* q, const void* k, const void* v, const void* gates,
                                   const int32_t* indices, const float* lse_sel, const void* o_sel,
                                   const void* dout, const nsa_params_t* p, void* dq, void* dk,
                                   void* dv, void* workspace, size_t ws_bytes, void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (p->dtype != NSA_BF16) return NSA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !gates || !indices || !lse_sel || !o_sel || !dout || !dq || !dk || !dv)
    return NSA_ERR_NULL;
  if (!workspace) return NSA_ERR_WORKSPACE;
  const Shape s = make_shape(p);
  const size_t es = esize(p);
  const BwdLayout L = bwd_layout(s, es, false);
  const size_t acc = up((size_t)s.B * s.T * s.Hkv * s.D * 4, kAlign);
  if (ws_bytes < L.total + 2 * acc) return NSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gates) || !aligned16(indices) ||
      !aligned16(lse_sel) || !aligned16(o_sel) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || ((uintptr_t)workspace % kAlign) != 0)
    return NSA_ERR_ALIGN;
  char* ws = (char*)workspace;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = nsa::launch_bwd_prep(true, s, k, v, gates, o_sel, dout, ws + L.bimg,
                                      (float*)(ws + L.delta), ws + L.dos, nullptr, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_bwd_single(s, q, ws + L.bimg, indices, lse_sel, (const float*)(ws + L.delta),
                             ws + L.dos, dq, dk, dv, (float*)(ws + L.total),
                             (float*)(ws + L.total + acc), hs);
  return launched(e);
}

nsa_status_t nsa_backward(const void* q, const void* k, const void* v, const void* gates,
                          const nsa_saved_t* sv, const void* dout, const nsa_params_t* p, void* dq,
                          void* dk, void* dv, void* dgates, void* workspace, size_t ws_bytes,
                          void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (!q || !k || !v || !gates || !sv || !dout || !dq || !dk || !dv || !dgates) return NSA_ERR_NULL;
  if (!sv->indices || !sv->lse_sel || !sv->lse_win || !sv->lse_cmp || !sv->o_sel || !sv->o_win ||
      !sv->o_cmp)
    return NSA_ERR_NULL;
  if (p->flags & ~(uint32_t)NSA_INDICES_IN) return NSA_ERR_UNSUPPORTED;
  if (!workspace) return NSA_ERR_WORKSPACE;
  const Shape s = make_shape(p);
  const size_t es = esize(p);
  const BwdLayout L = bwd_layout(s, es, true);
  if (ws_bytes < L.total) return NSA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(gates) || !aligned16(dout) ||
      !aligned16(sv->indices) || !aligned16(sv->lse_sel) || !aligned16(sv->lse_win) ||
      !aligned16(sv->lse_cmp) || !aligned16(sv->o_sel) || !aligned16(sv->o_win) ||
      !aligned16(sv->o_cmp) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dgates) || ((uintptr_t)workspace % kAlign) != 0)
    return NSA_ERR_ALIGN;
  char* ws = (char*)workspace;
  const bool bf = p->dtype == NSA_BF16;
  hipStream_t hs = (hipStream_t)stream;
  nsa::PrepFullArgs fx{sv->o_win, sv->o_cmp, ws + L.dos_w, ws + L.dos_c, (float*)(ws + L.delta_w),
                       (float*)(ws + L.delta_c), dgates};
  hipError_t e = nsa::launch_bwd_prep(bf, s, k, v, gates, sv->o_sel, dout, ws + L.bimg,
                                      (float*)(ws + L.delta), ws + L.dos, &fx, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_pool(bf, s, k, v, ws + L.kc, ws + L.vc, nullptr, nullptr, nullptr, nullptr, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_bwd_pool_image(bf, s, ws + L.kc, ws + L.vc, ws + L.pimg, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  e = nsa::launch_bwd_revmap(s, sv->indices, (uint64_t*)(ws + L.revmap), hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  // dq: selection, window and compression passes accumulate in fp32; the last
  // one rounds once
  float* dq32 = (float*)(ws + L.dq32);
  nsa::DqArgs d0{q, ws + L.bimg, sv->indices, sv->lse_sel, (const float*)(ws + L.delta), ws + L.dos,
                 nullptr, dq32, nullptr};
  nsa::DqArgs d1{q, ws + L.bimg, nullptr, sv->lse_win, (const float*)(ws + L.delta_w), ws + L.dos_w,
                 dq32, dq32, nullptr};
  nsa::DqArgs d2{q, ws + L.pimg, nullptr, sv->lse_cmp, (const float*)(ws + L.delta_c), ws + L.dos_c,
                 dq32, nullptr, dq};
  e = nsa::launch_bwd_dq(bf, s, 0, d0, hs);
  if (e == hipSuccess) e = nsa::launch_bwd_dq(bf, s, 1, d1, hs);
  if (e == hipSuccess) e = nsa::launch_bwd_dq(bf, s, 2, d2, hs);
  if (e != hipSuccess) return NSA_ERR_LAUNCH;
  nsa::KvBranches br{true, q, ws + L.bimg, ws + L.pimg,
                     {sv->lse_sel, sv->lse_win, sv->lse_cmp},
                     {(const float*)(ws + L.delta), (const float*)(ws + L.delta_w),
                      (const float*)(ws + L.delta_c)},
                     {ws + L.dos, ws + L.dos_w, ws + L.dos_c}};
  e = nsa::launch_bwd_dkdv(bf, s, br, (const uint64_t*)(ws + L.revmap), dk, dv, plan_ws(ws, L), hs);
  return launched(e);
}

}  // extern "C"

nsa_status_t nsa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const void* k_cmp, const void* v_cmp, const int32_t* seq_lens,
                        const void* gates, const nsa_params_t* p, void* out, int32_t* indices,
                        void* stream) {
  nsa_status_t st = check(p);
  if (st != NSA_OK) return st;
  if (p->flags & NSA_INDICES_IN) return NSA_ERR_UNSUPPORTED;
  if (!q || !k_cache || !v_cache || !k_cmp || !v_cmp || !seq_lens || !gates || !out) return NSA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_cmp) ||
      !aligned16(v_cmp) || !aligned16(gates) || !aligned16(out) || ((uintptr_t)seq_lens & 3u) ||
      (indices && ((uintptr_t)indices & 3u)))
    return NSA_ERR_ALIGN;
  const Shape s = make_shape(p);
  if (nsa::decode_lds_bytes(p->dtype == NSA_BF16, s) > 160 * 1024) return NSA_ERR_UNSUPPORTED;
  return launched(nsa::launch_decode(p->dtype == NSA_BF16, s, q, k_cache, v_cache, k_cmp, v_cmp,
                                     seq_lens, gates, out, indices, (hipStream_t)stream));
}
