/*
 * nsa.h -- C ABI of the MI355X (gfx950) Native Sparse Attention library.
 *
 * The operation: causal GQA prefill attention with three branches mixed by
 * per-head gates, as described on the pages
 *   [DSA] "DeepSeek's Native Sparse Attention" (newsletter #44), section
 *         "How Does Native Sparse Attention Work?": COMPRESSION, SELECTION and
 *         SLIDING WINDOW bullets and the gate paragraph that follows them;
 *   [SIC] "Sparsity is Cool: Reverse-Engineering MoBA and NSA" (wiki summary),
 *         section Method (mean-pool compression, block 64, top-k 16, window
 *         512) and Key claims (the first block is always selected; the
 *         two-pass query- plus key/value-stationary selection backward).
 *
 * For query position t (0-based), query head h, KV group g = h / (Hq/Hkv):
 *   compression : Kc_j, Vc_j = mean of the 64 keys/values of block j
 *                 (non-overlapping, complete blocks only);
 *                 o_cmp = softmax_j(tau q.Kc_j) Vc over j < floor((t+1)/64),
 *                 o_cmp = 0 when no block is complete yet;
 *   importance  : S_j(t,g) = sum over the heads of g of the compressed
 *                 attention probabilities;
 *   selection   : I(t,g) = {0, own = t/64} plus the (top_k - |forced|) blocks
 *                 of 1..own-1 with the largest S (ties: lower index); all of
 *                 them when there are no more than that; o_sel = softmax
 *                 attention over the tokens s <= t of the blocks in I;
 *   window      : o_win = softmax attention over t-W < s <= t;
 *   output      : out = g_cmp o_cmp + g_sel o_sel + g_win o_win.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *   - Layouts are row-major and contiguous:
 *       q, out, o_sel, dout, dq : [B][T][Hq][D]
 *       k, v, dk, dv            : [B][T][Hkv][D]
 *       gates                   : [B][T][Hq][3]   (g_cmp, g_sel, g_win)
 *       indices                 : int32 [B][Hkv][T][top_k], ascending, -1 pad
 *       lse_sel                 : float [B][Hq][T], natural log
 *       k_cmp, v_cmp            : [B][T/64][Hkv][D]
 *     Element type of q/k/v/gates/out/o_sel/dout/dq/dk/dv/k_cmp/v_cmp is
 *     params->dtype (bf16 or fp32); accumulation is always fp32.
 *   - Device pointers must be 16-byte aligned (NSA_ERR_ALIGN otherwise).
 *   - Every check happens before the first enqueue: an error status means
 *     nothing was launched.  NSA_ERR_LAUNCH reports a failed kernel launch;
 *     work enqueued before it may have run.
 *   - Calls on different streams may overlap only if each has its own
 *     workspace and outputs.
 *
 * GPU support envelope: head_dim in {64, 128} for bf16, 64 for fp32; block
 * 64; seq_len a multiple of 64 (at most 65536); Hq/Hkv in {1, 2, 4, 8, 16};
 * 2 <= top_k <= 32; window >= 1.  Anything else returns NSA_ERR_UNSUPPORTED.
 */
#ifndef NSA_MI355X_H
#define NSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSA_ABI_VERSION 1

typedef enum {
  NSA_OK = 0,
  NSA_ERR_NULL = -1,        /* a required pointer is NULL                      */
  NSA_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes              */
  NSA_ERR_DTYPE = -3,       /* unknown dtype                                   */
  NSA_ERR_UNSUPPORTED = -4, /* valid NSA problem outside the GPU envelope      */
  NSA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required         */
  NSA_ERR_ALIGN = -6,       /* a device pointer is not 16-byte aligned         */
  NSA_ERR_LAUNCH = -7       /* hipGetLastError reported a failed launch        */
} nsa_status_t;

typedef enum { NSA_BF16 = 0, NSA_FP32 = 1 } nsa_dtype_t;

enum {
  /* The compression branch is left out of `out` (as if g_cmp = 0); it is
   * still computed because selection needs its scores. */
  NSA_SKIP_CMP_OUT = 1,
  /* The selection branch is left out of `out` (as if g_sel = 0); with
   * NSA_SKIP_CMP_OUT as well, compression and selection are not computed at
   * all (sliding-window-only, the pruned-branch layer of [SIC] Key claims). */
  NSA_SKIP_SEL = 2,
  /* The window branch is left out of `out` (as if g_win = 0). */
  NSA_SKIP_WIN = 4,
  /* `indices` is an INPUT: the given table (same layout and rules as the
   * one the library writes) replaces the top-k step. */
  NSA_INDICES_IN = 8
};

typedef struct {
  int32_t batch;      /* B >= 1                                              */
  int32_t seq_len;    /* T >= 1                                              */
  int32_t n_q_heads;  /* Hq, a multiple of Hkv                               */
  int32_t n_kv_heads; /* Hkv >= 1                                            */
  int32_t head_dim;   /* D                                                   */
  int32_t block;      /* compression block = selection block; 64 on the GPU  */
  int32_t top_k;      /* selected blocks per (t, g) INCLUDING block 0 and
                         the own block                                       */
  int32_t window;     /* W: keys t-W < s <= t                                */
  float scale;        /* tau; <= 0 selects 1/sqrt(head_dim)                   */
  int32_t dtype;      /* nsa_dtype_t                                          */
  uint32_t flags;     /* NSA_SKIP_* | NSA_INDICES_IN                          */
} nsa_params_t;

/* Version of this ABI (NSA_ABI_VERSION). */
int nsa_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* nsa_status_string(nsa_status_t status);

/* Checks params against the rules above without touching any device.
 * Returns NSA_OK, NSA_ERR_SHAPE, NSA_ERR_DTYPE or NSA_ERR_UNSUPPORTED. */
nsa_status_t nsa_check_params(const nsa_params_t* p);

/* Bytes of device workspace needed by nsa_forward / nsa_forward_train
 * (for_backward = 0), by nsa_select_bwd (for_backward = 1), by nsa_backward
 * (for_backward = 2) or by nsa_select_bwd_single (for_backward = 3).  Returns 0 for invalid params.  The size is monotone in
 * seq_len and batch. */
size_t nsa_workspace_size(const nsa_params_t* p, int for_backward);

/* Compression step alone ([DSA] COMPRESSION; [SIC] Method: mean-pool over
 * non-overlapping 64-token blocks).  Writes k_cmp and v_cmp
 * [B][T/64][Hkv][D] in params->dtype: the fp32 mean rounded once (RNE for
 * bf16).  No workspace. */
nsa_status_t nsa_pool(const void* k, const void* v, const nsa_params_t* p,
                      void* k_cmp, void* v_cmp, void* stream);

/* Compression, compressed attention, block importance and top-k selection
 * ([DSA] COMPRESSION and SELECTION; [SIC] Method and Key claims).
 *   o_cmp   : [B][T][Hq][D], the UNGATED compressed-branch output, in
 *             params->dtype (0 for t < 63).  Required.
 *   indices : int32 [B][Hkv][T][top_k] selected blocks.  Required; ignored
 *             flags: all.
 * workspace: at least nsa_workspace_size(p, 0) bytes. */
nsa_status_t nsa_compress_select(const void* q, const void* k, const void* v,
                                 const nsa_params_t* p, void* o_cmp, int32_t* indices,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Name of the selection / window / combine kernel that nsa_forward launches
 * for these params (a static string: "sel_compact_kernel" or
 * "sel_win_kernel"), or NULL when nsa_check_params rejects them.  Touches no
 * device; for measurement tools that attribute kernel time. */
const char* nsa_forward_kernel(const nsa_params_t* p);

/* Full NSA forward (all three branches and the gated combination).
 *   out      : required, [B][T][Hq][D] in params->dtype.
 *   indices  : nullable output (or required input with NSA_INDICES_IN).
 *   lse_sel  : nullable output, selection-branch log-sum-exp (for the
 *              backward).
 *   o_sel    : nullable output, ungated selection-branch output in
 *              params->dtype (for the backward).
 * workspace: at least nsa_workspace_size(p, 0) bytes. */
nsa_status_t nsa_forward(const void* q, const void* k, const void* v, const void* gates,
                         const nsa_params_t* p, void* out, int32_t* indices, float* lse_sel,
                         void* o_sel, void* workspace, size_t ws_bytes, void* stream);

/* Bytes of the fixed per-GPU scratch array that nsa_forward_noalloc uses as
 * its workspace (32 MiB; a forward whose nsa_workspace_size(p, 0) exceeds it,
 * e.g. batch 1 at seq 8192 with 16 heads of 64 needs about 26 MiB, is
 * rejected). */
#define NSA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* nsa_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, checks, kernels and results, but no workspace argument --
 * it uses a fixed static device array of NSA_NOALLOC_SCRATCH_BYTES per GPU,
 * which the library holds from load until the process ends.  Nothing is
 * allocated or freed.  Returns NSA_ERR_WORKSPACE (before any launch) when
 * nsa_workspace_size(p, 0) > NSA_NOALLOC_SCRATCH_BYTES, NSA_ERR_LAUNCH if the
 * array's device address cannot be looked up.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and must be serialised by the
 * caller.  The array keeps the previous call's contents; the forward rewrites
 * everything it reads. */
nsa_status_t nsa_forward_noalloc(const void* q, const void* k, const void* v, const void* gates,
                                 const nsa_params_t* p, void* out, int32_t* indices,
                                 float* lse_sel, void* o_sel, void* stream);

/* nsa_forward, plus stage timing for measurement: `events` points to four
 * caller-created hipEvent_t handles (passed as void*; any may be NULL), which
 * are recorded on `stream` before the compression kernel, after it, after the
 * compressed-attention/top-k kernel and after the selection/window/combine
 * kernel.  Otherwise identical to nsa_forward (same checks, same results). */
nsa_status_t nsa_forward_profile(const void* q, const void* k, const void* v, const void* gates,
                                 const nsa_params_t* p, void* out, int32_t* indices,
                                 float* lse_sel, void* o_sel, void* workspace, size_t ws_bytes,
                                 void* stream, void* const* events);

/* Gradient of the selection branch with the selection and the gates held
 * fixed ([SIC] Method: two-pass backward -- a query-stationary pass for dq and
 * a key/value-stationary pass for dk/dv over the reverse block->query map;
 * no atomics, so the result is bitwise reproducible).
 *   dout            : gradient of `out`; the branch receives g_sel * dout.
 *   indices, lse_sel, o_sel : as written by nsa_forward for the same inputs.
 *   dq [B][T][Hq][D], dk, dv [B][T][Hkv][D] : outputs, overwritten.
 * workspace: at least nsa_workspace_size(p, 1) bytes. */
nsa_status_t nsa_select_bwd(const void* q, const void* k, const void* v, const void* gates,
                            const int32_t* indices, const float* lse_sel, const void* o_sel,
                            const void* dout, const nsa_params_t* p, void* dq, void* dk,
                            void* dv, void* workspace, size_t ws_bytes, void* stream);

/* The same gradient as nsa_select_bwd in ONE query-stationary pass that adds
 * dk and dv with fp32 atomics ([SIC] Method: the single-pass kernel whose
 * atomic contention motivates the two-pass scheme; kept for that A/B
 * comparison).  Same arguments and results up to the order of the fp32
 * additions (not bitwise reproducible).  bf16 only (NSA_ERR_UNSUPPORTED
 * otherwise).  workspace: at least nsa_workspace_size(p, 3) bytes. */
nsa_status_t nsa_select_bwd_single(const void* q, const void* k, const void* v, const void* gates,
                                   const int32_t* indices, const float* lse_sel, const void* o_sel,
                                   const void* dout, const nsa_params_t* p, void* dq, void* dk,
                                   void* dv, void* workspace, size_t ws_bytes, void* stream);

/* Tensors the full backward reads, written by nsa_forward_train.  All device
 * pointers, 16-byte aligned, owned by the caller:
 *   indices          int32 [B][Hkv][T][top_k]  (output, or input with
 *                    NSA_INDICES_IN)
 *   lse_sel, lse_win, lse_cmp   fp32 [B][Hq][T]: log-sum-exp (natural log) of
 *                    the selection, window and compressed softmaxes; lse_cmp
 *                    is -inf where no compressed block is visible (t < 63)
 *   o_sel, o_win, o_cmp         [B][T][Hq][D] in params->dtype: the UNGATED
 *                    branch outputs (o_cmp is 0 for t < 63) */
typedef struct {
  int32_t* indices;
  float* lse_sel;
  float* lse_win;
  float* lse_cmp;
  void* o_sel;
  void* o_win;
  void* o_cmp;
} nsa_saved_t;

/* nsa_forward that also writes every tensor of `saved` (all seven required)
 * for nsa_backward.  Same checks and the same `out` as nsa_forward.  flags:
 * only NSA_INDICES_IN is allowed (training runs all three branches).
 * workspace: at least nsa_workspace_size(p, 0) bytes. */
nsa_status_t nsa_forward_train(const void* q, const void* k, const void* v, const void* gates,
                               const nsa_params_t* p, void* out, const nsa_saved_t* saved,
                               void* workspace, size_t ws_bytes, void* stream);

/* Gradient of the whole NSA output ([DSA] How Does NSA Work?: the three
 * branches and the gate mix; [SIC] Method: mean-pool compression), with the
 * selection held fixed (top-k is piecewise constant; no gradient flows
 * through the importance scores):
 *   dgates[t,h] = (dout.o_cmp, dout.o_sel, dout.o_win)          [B][T][Hq][3]
 *   dq, dk, dv  = the softmax-Jacobian gradients of the selection branch
 *                 (tokens of the selected blocks, s <= t), the window branch
 *                 (t - W < s <= t) and the compression branch (pooled keys of
 *                 the complete blocks visible to t, whose gradients flow back
 *                 through the mean-pool as 1/64 per token of the block),
 *                 each branch receiving g_branch * dout.
 * Same two-pass scheme as nsa_select_bwd (query-stationary dq, key-stationary
 * dk/dv over per-block row lists, partial sums added in a fixed order): no
 * atomics, bitwise reproducible.
 *   saved : as written by nsa_forward_train for the same inputs (read only).
 *   dout  : gradient of `out`.
 *   dq [B][T][Hq][D], dk, dv [B][T][Hkv][D], dgates [B][T][Hq][3] in
 *   params->dtype: outputs, overwritten.
 * flags: only NSA_INDICES_IN may be set (ignored here).
 * workspace: at least nsa_workspace_size(p, 2) bytes. */
nsa_status_t nsa_backward(const void* q, const void* k, const void* v, const void* gates,
                          const nsa_saved_t* saved, const void* dout, const nsa_params_t* p,
                          void* dq, void* dk, void* dv, void* dgates, void* workspace,
                          size_t ws_bytes, void* stream);

/* One decode step: NSA for the newest position of each sequence over its KV
 * cache ([DSA] How Does NSA Work?: the three branches and the gate mix,
 * evaluated for a single query; [SIC] Method).  Sequence b has length
 * L_b = seq_lens[b] and its newest key and value are already in the cache, so
 * its query sits at t = L_b - 1 and the result is the prefill output row t of
 * that prefix (compressed blocks j < L_b / 64, selection among 1 .. t/64 - 1
 * plus blocks 0 and t/64, window t - W < s <= t).
 *   q        : [B][Hq][D], the new queries.
 *   k_cache, v_cache : [B][Lmax][Hkv][D]; positions >= L_b are never read.
 *   k_cmp, v_cmp     : [B][Lmax/64][Hkv][D], the mean-pooled complete blocks
 *              of the cache (nsa_pool of the cache, or kept up to date by the
 *              caller as blocks complete); blocks >= L_b / 64 are never read.
 *   seq_lens : int32 [B] on the device, 1 <= L_b <= Lmax; values outside are
 *              clamped to that range (the kernel cannot report them).
 *   gates    : [B][Hq][3] (g_cmp, g_sel, g_win).
 *   params   : batch = B, seq_len = Lmax (the cache capacity, a multiple of
 *              64), heads, head_dim, top_k, window, scale, dtype as for the
 *              prefill; flags: NSA_SKIP_* only (NSA_INDICES_IN is
 *              NSA_ERR_UNSUPPORTED).
 *   out      : [B][Hq][D], overwritten.
 *   indices  : optional int32 [B][Hkv][top_k]: the selected blocks,
 *              ascending, -1 padded.
 * No workspace; the kernel's on-chip memory grows with Lmax and the query
 * heads per group (for fp32 also with the window): NSA_ERR_UNSUPPORTED when it
 * would exceed 160 KB. */
nsa_status_t nsa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const void* k_cmp, const void* v_cmp, const int32_t* seq_lens,
                        const void* gates, const nsa_params_t* p, void* out, int32_t* indices,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NSA_MI355X_H */
