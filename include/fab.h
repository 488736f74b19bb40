/*
 * fab -- FlashAttention-2 backward (and its supporting forward) for AMD MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a plain device pointer to dense, row-major memory; no
 * PyTorch (or any other framework) type appears here.  The caller owns and allocates all
 * memory, including the backward workspace; the library never allocates or frees device
 * memory and keeps no pointer after a call returns.  (The one exception is the static scratch
 * array of fab_bwd_noalloc, loaded with the library's code on each GPU it runs on.)
 *
 * Operation (boostr 0.1.0, src/ops/cuda/attention/flash_bwd.rs, doc comment of
 * flash_attention_bwd_impl): the backward runs in two steps -- a preprocessing step that
 * forms D = rowsum(dO * O) per query row, then a main step that produces dQ, dK and dV,
 * recomputing P = exp(scale * Q K^T - LSE) tile by tile instead of storing it.  The
 * autograd glue on boostr's src/ops/autograd_attention.rs page fixes what the backward
 * consumes (q, k, v, the forward's output and its lse, and dO) and what the forward
 * returns (output, lse).
 *
 * Layouts (the allocation blocks of flash_bwd.rs and the shape checks of rustytorch's
 * rtx-flash-metal-attention backward.rs):
 *   q, o, dO, dQ : [B, H,    Sq, D]   element type `dtype`
 *   k, v, dK, dV : [B, H_kv, Sk, D]   element type `dtype`
 *   lse          : [B, H,    Sq]      float32, natural-log log-sum-exp of the scaled scores
 *   D (delta)    : [B, H,    Sq]      float32
 * Grouped-query heads: H % H_kv == 0 and query head h uses kv head h / (H / H_kv)
 * (contiguous groups); dK and dV are the sums over the H / H_kv query heads of a group.
 * Causal masking is top-left aligned: query row i may attend key j iff j <= i.
 * Sliding window (`window_size`, the argument autograd_attention.rs passes to both the
 * forward and the backward, and which flash_bwd.rs's backward rejects unless it is 0):
 * window_size = W > 0 keeps W keys per query: row i may attend key j only if j > i - W and,
 * without the causal mask, also j < i + W (same top-left indices as the causal mask).  W = 0
 * means no window; a window of at least max(Sq, Sk) keys cuts nothing.  Negative W is
 * FAB_ERR_INVALID_ARGUMENT.  A row left with no key (possible only with a window and
 * Sq - Sk >= W) gets o = 0 and lse = -inf from fab_fwd, and dq = 0 from fab_bwd; it adds
 * nothing to dk and dv.
 * Supported: dtype FAB_F32 / FAB_F16 / FAB_BF16 (one dtype shared by all element-typed
 * tensors of a call); head dim D in {32, 64, 96, 128}, and also 256 for FAB_F16 / FAB_BF16
 * (kernels are compiled per head dim, as flash_bwd.rs's kernel names carry the head dim).
 *
 * Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 * the call returns without waiting.  Results are valid for later work on the same stream.
 * The calls enqueue kernel launches only (no allocation, copy or memset), so they may be
 * captured into a HIP graph; a replay reads whatever the captured buffers then hold.
 *
 * Errors: every argument is validated before anything is enqueued, so a non-OK status
 * means nothing was launched and no output was written.  fab_last_error() returns a
 * thread-local "argument: reason" message for the last non-OK status of the calling
 * thread.  FAB_ERR_LAUNCH is returned if a launch fails after validation.
 */
#ifndef FAB_H
#define FAB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FAB_F32 = 0, FAB_F16 = 1, FAB_BF16 = 2 } fab_dtype;

typedef enum {
  FAB_OK = 0,
  FAB_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad dims, H % H_kv != 0,
                                   workspace too small, non-finite scale, size limits */
  FAB_ERR_UNSUPPORTED = 2,      /* dtype or head dim not supported                    */
  FAB_ERR_DEVICE = 3,           /* a pointer is not device memory of the current GPU,
                                   or its allocation is smaller than the tensor       */
  FAB_ERR_LAUNCH = 4            /* a kernel launch failed (message from the runtime)  */
} fab_status;

/* Version string of the library. */
const char* fab_version(void);

/* Thread-local message for the last non-OK status returned on this thread ("" if none). */
const char* fab_last_error(void);

/*
 * Bytes of device workspace for the recommended mode of the backward at these sizes (0 if the
 * sizes are invalid); fab_bwd_workspace_bytes_min gives the least fab_bwd accepts (the
 * recompute mode) and fab_bwd_workspace_bytes_ds the size that selects the stored-dS mode (0
 * where that mode cannot run: float32, or a dS buffer past the limits below).
 *
 * The workspace selects how dQ is formed.  With at least fab_bwd_workspace_bytes_ds bytes the
 * dK/dV kernel also stores every dS value it forms and dQ = scale * dS K reads them back
 * ("stored dS": 10 D FLOPs per allowed pair instead of 14 D, for 2 bytes of HBM written and
 * read per pair).  With less (at least fab_bwd_workspace_bytes_min), or for float32, dQ
 * recomputes S and dP ("recompute").  Both give the same result up to float rounding order;
 * each is deterministic.  The recommended mode is stored dS from head dim 96 up, except for
 * problems so small that the two recomputing kernels run in one launch.
 *
 * Layout.  From byte 0, as written by the preprocessing step, float32 pairs
 *   ws[((b * H + h) * Sq_pad + i) * 2 + 0] = lse[b, h, i] * log2(e)
 *   ws[((b * H + h) * Sq_pad + i) * 2 + 1] = D[b, h, i] = sum_d dO[b,h,i,d] * o[b,h,i,d]
 * with Sq_pad = Sq rounded up to a multiple of 64; rows i >= Sq, and rows whose lse is -inf
 * (rows with no allowed key), hold +inf in place of lse * log2(e).  The statistics take
 * fab_bwd_workspace_bytes_min bytes (B * H * Sq_pad * 8, rounded up to 256).  Stored dS
 * follows from the next 4096-byte boundary: per (b, h), Sq rounded up to 128 times Sk rounded
 * up to 256 dtype values, in fragments of 32 keys x 16 query rows in the kernels' own order.
 * Stored dS is taken when that slab is at most 2 GiB, the H / H_kv slabs of a kv-head group
 * stay below 4 GiB and all slabs together at most 32 GiB (for example 2.1 GB at B=2, H=32,
 * S=4096).  fab_bwd overwrites the workspace on every call; its contents on entry do not
 * matter.
 */
size_t fab_bwd_workspace_bytes(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype);
size_t fab_bwd_workspace_bytes_min(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype);
size_t fab_bwd_workspace_bytes_ds(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype);

/*
 * The launches fab_bwd makes for these sizes and a workspace of `workspace_bytes` (-1 if the
 * sizes are invalid or the workspace too small).  Enqueues nothing.
 */
typedef enum {
  FAB_PLAN_RECOMPUTE = 0,             /* dQ kernel (step 1 in its prologue), then dK/dV     */
  FAB_PLAN_RECOMPUTE_ONE_LAUNCH = 1,  /* step 1, then dQ and dK/dV kernels in one launch    */
  FAB_PLAN_STORED_DS = 2,             /* step 1, dK/dV (also stores dS), dQ = scale dS K    */
  FAB_PLAN_F32 = 3                    /* float32: step 1, dK/dV, dQ                         */
} fab_plan;
int fab_bwd_plan(int B, int H, int H_kv, int Sq, int Sk, int D, int dtype, size_t workspace_bytes);

/*
 * Supporting forward (boostr autograd_attention.rs, var_flash_attention: the forward
 * returns the output and the lse that the backward consumes):
 *   o   = softmax(scale * q k^T over the allowed keys) v        [B, H, Sq, D], dtype
 *   lse = natural-log log-sum-exp of the allowed scaled scores  [B, H, Sq],   float32
 * q, k, v, o, lse: device pointers, 16-byte aligned, not overlapping o/lse.  The allowed
 * keys of a row follow `causal` and `window_size` as described at the top of this file.
 */
fab_status fab_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int Sq, int Sk, int D, int dtype,
                   int causal, int window_size, float scale, void* stream);

/*
 * Step 1 of the backward on its own (flash_bwd.rs, "Step 1: Preprocessing"):
 *   D[b, h, i] = sum_d dO[b, h, i, d] * o[b, h, i, d], accumulated in float32,
 * written with the rescaled lse into `workspace` in the layout described at
 * fab_bwd_workspace_bytes.  dO, o: [B, H, Sq, D] dtype; lse: [B, H, Sq] float32.  Device
 * pointers, 16-byte aligned.  fab_bwd runs this step itself; it is exported so that D can be
 * inspected and the step timed, and so that fab_bwd_dkdv / fab_bwd_dq can run on their own.
 */
fab_status fab_bwd_preprocess(const void* dO, const void* o, const float* lse,
                              void* workspace, size_t workspace_bytes,
                              int B, int H, int Sq, int D, int dtype, void* stream);

/*
 * Backward (flash_bwd.rs, flash_attention_bwd_impl; autograd_attention.rs,
 * FlashAttentionBackward::backward):
 *   P  = exp(scale * q k^T - lse) on allowed pairs (causal, window_size), 0 elsewhere
 *   dP = dO v^T,   dS = P * (dP - D) with D = rowsum(dO * o)
 *   dV = sum over the group's query heads of P^T dO
 *   dK = scale * sum over the group's query heads of dS^T q
 *   dQ = scale * dS k
 * Inputs dO, q, o: [B, num_heads, Sq, D]; k, v: [B, num_kv_heads, Sk, D]; lse as produced
 * by fab_fwd.  Outputs dq [B, num_heads, Sq, D], dk and dv [B, num_kv_heads, Sk, D], all in
 * `dtype`; they need no initialisation and every element is written (rows the mask never
 * reaches get 0).  workspace: at least fab_bwd_workspace_bytes_min(...) bytes of device
 * memory; with at least fab_bwd_workspace_bytes(...) the stored-dS mode runs where it applies
 * (see there).  All pointers 16-byte aligned; outputs must not overlap inputs or each other.
 * Deterministic: no atomics, identical inputs and workspace size give bitwise identical
 * outputs.  Launches: stored dS -- step 1, the dK/dV kernel (which also writes dS), then
 * dQ = scale * dS K; recompute (16-bit) -- the dQ kernel (with step 1 folded into its
 * prologue), then the dK/dV kernel, or, where both grids together fit the device at once,
 * step 1 and then both kernels in one launch; float32 -- step 1, dK/dV, dQ.
 */
fab_status fab_bwd(const void* dO, const void* q, const void* k, const void* v,
                   const void* o, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int num_heads, int num_kv_heads, int Sq, int Sk, int D, int dtype,
                   int causal, int window_size, float scale, void* stream);

/*
 * fab_bwd without a workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It computes
 * what fab_bwd computes, with the same kernels, and calls no allocating routine: the per-row
 * statistics that fab_bwd keeps in its workspace go to a static scratch array of the library,
 * 16 MiB per GPU, held from the first call on a device until the process ends.  Limit:
 * B * num_heads * (Sq rounded up to 64) <= 2^21 rows; larger sizes return
 * FAB_ERR_INVALID_ARGUMENT before anything is launched.  Every call on one GPU shares that
 * GPU's scratch: calls that may overlap on one GPU (different streams without ordering, or
 * different threads) race and give undefined results; calls ordered on one stream are safe.
 * The scratch needs no initialisation (each call writes every entry it reads).  Other
 * arguments, outputs and errors as for fab_bwd.
 */
fab_status fab_bwd_noalloc(const void* dO, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, void* dq, void* dk, void* dv,
                           int B, int num_heads, int num_kv_heads, int Sq, int Sk, int D, int dtype,
                           int causal, int window_size, float scale, void* stream);

/*
 * The two kernels of step 2 on their own, for inspection and per-kernel timing; fab_bwd
 * runs them itself after step 1.  `workspace` must hold what fab_bwd_preprocess wrote for
 * the same dO, o and lse.  The workspace size selects the mode as for fab_bwd.  Other
 * arguments as for fab_bwd.
 *   fab_bwd_dkdv writes dk, dv (key-tile outer; each workgroup owns a tile of keys and
 *                sums over every query head of its kv-head group), and in the stored-dS mode
 *                also dS into the workspace.
 *   fab_bwd_dq   writes dq (query-tile outer): in the stored-dS mode from the dS that
 *                fab_bwd_dkdv stored in the same workspace for the same inputs; otherwise it
 *                recomputes S and dP for its query rows.
 */
fab_status fab_bwd_dkdv(const void* dO, const void* q, const void* k, const void* v,
                        void* workspace, size_t workspace_bytes, void* dk, void* dv,
                        int B, int num_heads, int num_kv_heads, int Sq, int Sk, int D,
                        int dtype, int causal, int window_size, float scale, void* stream);
fab_status fab_bwd_dq(const void* dO, const void* q, const void* k, const void* v,
                      const void* workspace, size_t workspace_bytes, void* dq,
                      int B, int num_heads, int num_kv_heads, int Sq, int Sk, int D,
                      int dtype, int causal, int window_size, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FAB_H */
