/*
 * attn.h -- C ABI of libattn: fused multi-head scaled-dot-product attention,
 * forward and backward, for AMD Instinct MI355X (gfx950).
 *
 *   O = softmax(scale * Q K^T + mask) V        (per batch b, head h)
 *
 * computed with an online softmax (running row max and row sum, rescaled per
 * key tile), plus the gradient of any scalar loss L with respect to Q, K, V
 * given dO = dL/dO.
 *
 * Where the operations come from (cited by page title and section):
 *   - Mask-unit (block-local) attention: "hiera-optim 0.1.0" sdist,
 *     hiera_optim/attention/mask_unit.py, MaskUnitAttentionFast.forward --
 *     tokens split into independent windows, a dense softmax attention inside
 *     each window, default scale head_dim^-0.5.
 *   - Causal sliding window: "IHA-CUDA: Interleaved Head Attention Kernels for
 *     Hopper GPUs", section "FLOP Matching" -- a window of W = WSL + 1 keys
 *     including the diagonal.
 *   - Backward split into a row-statistics pre-pass (dPsum, lse), a dK/dV pass
 *     and a dQ pass, with visited tile ranges computed per causal/windowed
 *     mask and fully masked tiles never visited: same page, section
 *     "Repository Structure" (flash_bwd_preprocess, block_info, mask,
 *     softmax).  Here dQ is produced by its own pass over key tiles instead of
 *     an atomic fp32 accumulator, so results are bitwise deterministic.
 *   - Caller-owned outputs, base-pointer alignment checks and device gating
 *     follow the review points of "flashdreams.accelerated API v0 - #486"
 *     (output storage aliasing a cached buffer; base pointer alignment;
 *     rejecting unsupported devices up front instead of failing mid-run).
 *
 * Layouts (contiguous, row-major -- the *_strided entry points below take
 * other row strides; element type `dtype` except lse and the workspace,
 * which are fp32):
 *     Q, O, dO, dQ : [B][H][Nq][d]
 *     K, V, dK, dV : [B][H][Nk][d]
 *     lse          : [B][H][Nq]      natural-log logsumexp of the scaled,
 *                                    masked scores of each query row
 * Element types: bf16 and fp16 (both on the MFMA units, products of 16-bit
 * operands: P and dS are rounded to the input type before their products)
 * and fp32 (vector ALUs).  Accumulation is always fp32.  16-bit outputs are
 * rounded to nearest even.  fp16 inputs follow the hiera-optim test matrix
 * (bf16 / fp16 / fp32; "hiera-optim 0.1.0", Tests).
 *
 * Visibility of key j to query i (absolute indices, top-left aligned):
 *     ATTN_MASK_NONE     every key
 *     ATTN_MASK_CAUSAL   j <= i
 *     ATTN_MASK_SLIDING  i - window < j <= i        (window >= 1)
 *     ATTN_MASK_BLOCK    i / Wq == j / window       (integer division; the
 *                        Nk / window windows of `window` keys each hold
 *                        Wq = Nq / (Nk / window) query rows -- Wq = window when
 *                        Nq == Nk, fewer with pooled queries as in Hiera's
 *                        q_stride > 1 mask units; needs Nk % window == 0 and
 *                        Nq % (Nk / window) == 0)
 * A query row that sees no key gets O = 0, lse = -inf, dQ = 0.
 *
 * Ownership: the caller allocates every buffer, including the backward
 * workspace.  The library allocates no device memory, keeps no per-call
 * state, and is reentrant across streams and host threads.  Outputs are fully
 * overwritten (never accumulated into) and must not overlap any input or each
 * other.  Every base pointer must be 16-byte aligned.
 *
 * Errors: every entry point validates all arguments before touching the
 * device.  A nonzero status means nothing was enqueued and no output was
 * written -- except ATTN_ERR_LAUNCH, the HIP launch status after an enqueue.
 * ATTN_OK means the work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) with no host synchronisation; device faults surface at the
 * caller's next synchronisation.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define ATTN_API __attribute__((visibility("default")))
#else
#define ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype { ATTN_BF16 = 0, ATTN_FP32 = 1, ATTN_FP16 = 2 };

enum attn_mask {
  ATTN_MASK_NONE = 0,
  ATTN_MASK_CAUSAL = 1,
  ATTN_MASK_SLIDING = 2,
  ATTN_MASK_BLOCK = 3
};

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, size < 1, bad mask/window      */
  ATTN_ERR_UNSUPPORTED = 2, /* dtype or head dim d not built (d in 64/96/128) */
  ATTN_ERR_MISALIGNED = 3,  /* a base pointer is not 16-byte aligned          */
  ATTN_ERR_WORKSPACE = 4,   /* workspace null or smaller than required        */
  ATTN_ERR_ALIAS = 5,       /* an output overlaps an input or another output  */
  ATTN_ERR_DEVICE = 6,      /* current device is not gfx950, or HIP query failed */
  ATTN_ERR_LAUNCH = 7       /* a kernel launch reported an error              */
};

/*
 * attn_fwd -- forward pass.
 *   dtype        ATTN_BF16, ATTN_FP16 or ATTN_FP32 (element type of q, k, v,
 *                o and of every other tensor but lse)
 *   B, H         batch and head count (>= 1)
 *   Nq, Nk       query and key sequence lengths (>= 1, <= 2^30; every
 *                (b, h) slice spans at most 2^31 elements, i.e. Nq * d and
 *                Nk * d <= 2^31 for contiguous tensors, and
 *                B * H * ceil(max(Nq, Nk) / 16) < 2^31; ATTN_ERR_INVALID_ARG
 *                otherwise.  Whole tensors may exceed 2^31 elements.)
 *   d            head dimension: 64, 96 or 128
 *   scale        multiplier of Q K^T (e.g. 1/sqrt(d))
 *   mask, window mask mode and its window (ignored for NONE and CAUSAL)
 *   q, k, v      device inputs, layouts above
 *   o            device output [B][H][Nq][d], dtype
 *   lse          device output [B][H][Nq], fp32
 *   stream       hipStream_t to enqueue on (NULL = default stream)
 * Returns an attn_status.
 */
ATTN_API int attn_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
             float scale, int mask, int64_t window,
             const void* q, const void* k, const void* v,
             void* o, float* lse, void* stream);

/*
 * attn_bwd_workspace_size -- bytes of device workspace attn_bwd needs: one
 * fp32 per query row (the row sums D_i = sum_c dO[i][c] * O[i][c], the
 * "dPsum" of the backward pre-pass), rounded up to 256 bytes.  Returns 0 if
 * B, H or Nq is < 1.
 */
ATTN_API size_t attn_bwd_workspace_size(int64_t B, int64_t H, int64_t Nq);

/*
 * attn_bwd_workspace_size_ds -- bytes of workspace with which attn_bwd keeps
 * dS = P * (dP - D) (16-bit) from its dK/dV pass for its dQ pass, so that the
 * dQ pass is the plain product dQ = scale * dS K instead of recomputing S, P
 * and dP (a choice of this library: the pages' backward designs either
 * recompute or accumulate dQ with atomics).  The extra part holds one 32 x 32
 * 16-bit block (2 KB) per key block x query block pair with a visible entry,
 * per (b, h): about 2 bytes per visible (query, key) pair, e.g. 1.35 GB for
 * causal B=1, H=20, N=8192.  It applies to bf16 and fp16, d = 128, and every mask
 * except the block-local one of attn_bwd_fused(); elsewhere, and for any
 * workspace smaller than this, attn_bwd recomputes and the value returned is
 * attn_bwd_workspace_size(B, H, Nq).  Returns 0 for arguments attn_bwd would
 * reject.  A caller short of memory may always pass the smaller size.
 */
ATTN_API size_t attn_bwd_workspace_size_ds(int dtype, int64_t B, int64_t H, int64_t Nq,
                                           int64_t Nk, int64_t d, int mask, int64_t window);

/*
 * attn_bwd -- backward pass: dQ, dK, dV of L given dO = dL/dO.
 *   q, k, v, o, lse  the forward inputs and outputs (o and lse as written by
 *                    attn_fwd for the same arguments)
 *   dout             dO, [B][H][Nq][d], dtype
 *   dq, dk, dv       device outputs, layouts of q, k, v
 *   workspace        device scratch of >= attn_bwd_workspace_size(B, H, Nq)
 *                    bytes, caller-owned; contents on entry are ignored.  With
 *                    >= attn_bwd_workspace_size_ds(...) bytes the dQ pass
 *                    reads dS kept by the dK/dV pass (see there).
 * Other arguments as attn_fwd.  Three kernels run in stream order: the row-sum
 * pre-pass, the dK/dV pass (one workgroup per key tile, looping over visible
 * query tiles) and the dQ pass (one workgroup per query tile, looping over
 * visible key tiles).
 */
ATTN_API int attn_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
             float scale, int mask, int64_t window,
             const void* q, const void* k, const void* v, const void* o,
             const float* lse, const void* dout,
             void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass bits for attn_bwd_passes.
 *   ATTN_PASS_ROWSUM  D_i = sum_c dO[i][c] * O[i][c] into the workspace
 *   ATTN_PASS_DKDV    dK and dV (reads the workspace's D)
 *   ATTN_PASS_DQ      dQ        (reads the workspace's D)
 */
enum attn_pass {
  ATTN_PASS_ROWSUM = 1,
  ATTN_PASS_DKDV = 2,
  ATTN_PASS_DQ = 4,
  ATTN_PASS_ALL = 7
};

/*
 * attn_bwd_fused -- nonzero when attn_bwd runs as ONE fused kernel for these
 * arguments, else 0 (also 0 for arguments attn_bwd would reject).
 *   1  bf16 or fp16 block-local attention whose window divides 64 and whose
 *      query rows per window Wq = Nq / (Nk / window) divide the window (Wq =
 *      window, or pooled queries with an integer q_stride = window / Wq),
 *      where every query row sees keys of its own 64-key tile only
 *      ("hiera-optim 0.1.0" sdist, mask_unit.py: mask-unit windows as
 *      independent dense attentions).  One workgroup holds a whole tile: its
 *      dK/dV waves and its dQ waves run the two backward passes side by
 *      side.  attn_bwd_passes then accepts only ATTN_PASS_ALL.
 *   2  otherwise, bf16 or fp16 with d = 64 or 96, Nk <= 224 and Nq <= 1024,
 *      any mask (the global-attention stages of Hiera-Base at 224x224 --
 *      "hiera-optim 0.1.0", Results and sdist mask_unit.py -- of which the
 *      14x14 grid has 196 tokens): one workgroup holds every key of a
 *      (b, h) and loops over its query rows.  attn_bwd_passes with
 *      ATTN_PASS_ALL runs the fused kernel; a partial pass set runs the
 *      general passes.
 * In both cases the row sums D_i are formed in-kernel as sum_j P_ij dP_ij,
 * the workspace is not used and O is not read.
 */
ATTN_API int attn_bwd_fused(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                            int mask, int64_t window);

/*
 * attn_bwd_passes -- attn_bwd restricted to the passes in the bit set
 * `passes` (1..ATTN_PASS_ALL; anything else is ATTN_ERR_INVALID_ARG),
 * enqueued in the order row sums, dK/dV, dQ.  Where attn_bwd_fused() is 1,
 * any set but ATTN_PASS_ALL is ATTN_ERR_UNSUPPORTED; where it is 2,
 * ATTN_PASS_ALL runs the fused kernel and any other set the general passes
 * (so a caller that enqueues the three bits one call at a time gets the
 * general passes).  attn_bwd is
 * attn_bwd_passes(ATTN_PASS_ALL, ...).  Every argument is validated exactly
 * as in attn_bwd, including the outputs a pass does not write.  The dK/dV
 * and dQ passes read D from the workspace, so they need a row-sum pass with
 * the same o, dout and workspace earlier in stream order; once that pass is
 * done the two are independent of each other and a caller may enqueue them
 * on two streams (with an event from the row-sum pass's stream) -- except
 * with a workspace of attn_bwd_workspace_size_ds() bytes where that exceeds
 * attn_bwd_workspace_size(): then the dQ pass reads the dS blocks the dK/dV
 * pass writes, and must follow it in stream order.  Passing a workspace that
 * holds no row sums (or no dS blocks) gives wrong gradients, not a fault.
 * Use: overlapping the passes, and timing each pass on its own.
 */
ATTN_API int attn_bwd_passes(int passes, int dtype, int64_t B, int64_t H, int64_t Nq,
                             int64_t Nk, int64_t d, float scale, int mask, int64_t window,
                             const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout,
                             void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_check_fwd / attn_check_bwd -- the argument validation of attn_fwd /
 * attn_bwd alone: no device query, no launch.  Same arguments (the stream is
 * not needed).  Returns the status the entry point would return before
 * enqueueing, except that the device check (ATTN_ERR_DEVICE) is not made.
 */
ATTN_API int attn_check_fwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window,
                   const void* q, const void* k, const void* v,
                   const void* o, const float* lse);

ATTN_API int attn_check_bwd(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                   float scale, int mask, int64_t window,
                   const void* q, const void* k, const void* v, const void* o,
                   const float* lse, const void* dout,
                   const void* dq, const void* dk, const void* dv,
                   const void* workspace, size_t workspace_bytes);

/*
 * Strided tensors.  The entry points above take contiguous tensors; the
 * *_strided ones below take, for each [B][H][N][d] tensor, where its rows
 * are: row j of slice (b, h) -- token j, counted window by window for
 * ATTN_MASK_BLOCK -- begins at element
 *     b * batch + h * head + (j / T) * window + (j % T) * token
 * of the tensor's base pointer, and its d elements are contiguous.  T is the
 * tensor's window length: for ATTN_MASK_BLOCK, `window` keys (K, V, dK, dV)
 * or Wq = Nq / (Nk / window) query rows (Q, O, dO, dQ); for the other masks
 * the whole sequence (one window: the `window` stride is not used).
 *
 * This reads Hiera's token order in place: MaskUnitAttentionFast views its
 * qkv projection as (B, T, nw, 3, H, D), token n = t * nw + w, window index
 * fastest ("hiera-optim 0.1.0" sdist, mask_unit.py,
 * MaskUnitAttentionFast.forward), then permutes and copies it into
 * (B * nw, H, T, D).  With batch = N*3*H*D, head = D, window = 3*H*D and
 * token = nw*3*H*D, and K and V at H*D and 2*H*D past Q in the same buffer,
 * the kernels read that projection output directly; O can be written in the
 * same order (its own strides), ready for the output projection.
 *
 * Requirements: strides >= 0 and <= 2^48; the rows of a tensor nest --
 * ordering its dimensions of extent > 1 by stride, the smallest stride is
 * >= d and each next stride is >= the previous stride times its extent (no
 * two rows of one tensor overlap); the last row of a slice ends within 2^31
 * elements of the slice's first (ATTN_ERR_INVALID_ARG otherwise).  Strides
 * of dimensions with extent > 1 are multiples of 16 bytes
 * (ATTN_ERR_MISALIGNED otherwise).  A block layout whose windows do not
 * follow each other at the token stride (window != T * token, more than one
 * window) needs T to be a power of two (ATTN_ERR_UNSUPPORTED otherwise).
 * lse and the workspace stay contiguous.  Inputs may overlap each other
 * (q, k, v as views of one qkv buffer); outputs may not overlap inputs or
 * each other (ATTN_ERR_ALIAS).  Two tensors with the same strides and
 * extents -- interleaved views of one buffer, such as dq, dk, dv in one dqkv
 * buffer -- are checked element-exactly; any other pair by address range.
 */
typedef struct attn_layout {
  int64_t batch, head, window, token; /* element strides */
} attn_layout;

typedef struct attn_layouts {
  attn_layout q, k, v, o;       /* forward and backward */
  attn_layout dout, dq, dk, dv; /* backward only */
} attn_layouts;

/*
 * attn_layouts_contiguous -- the layouts the contiguous entry points use
 * (batch = H*N*d, head = N*d, window = T*d, token = d per tensor) into *out.
 * Returns ATTN_OK, or ATTN_ERR_INVALID_ARG for a null `out` or a geometry
 * attn_fwd would reject.
 */
ATTN_API int attn_layouts_contiguous(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                                     int mask, int64_t window, attn_layouts* out);

/*
 * attn_fwd_strided -- attn_fwd with q, k, v, o at `layouts` (q, k, v, o
 * members; NULL = contiguous).  Validation, results and launch behaviour are
 * those of attn_fwd.
 */
ATTN_API int attn_fwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                              float scale, int mask, int64_t window,
                              const void* q, const void* k, const void* v,
                              void* o, float* lse, const attn_layouts* layouts, void* stream);

/*
 * attn_bwd_strided -- attn_bwd_passes with every tensor at `layouts` (NULL =
 * contiguous).  The workspace sizes are those of the contiguous case.
 */
ATTN_API int attn_bwd_strided(int passes, int dtype, int64_t B, int64_t H, int64_t Nq,
                              int64_t Nk, int64_t d, float scale, int mask, int64_t window,
                              const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout,
                              void* dq, void* dk, void* dv,
                              void* workspace, size_t workspace_bytes,
                              const attn_layouts* layouts, void* stream);

/* attn_check_fwd_strided / attn_check_bwd_strided -- their validation alone,
 * as attn_check_fwd / attn_check_bwd. */
ATTN_API int attn_check_fwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                    int64_t d, float scale, int mask, int64_t window,
                                    const void* q, const void* k, const void* v,
                                    const void* o, const float* lse,
                                    const attn_layouts* layouts);

ATTN_API int attn_check_bwd_strided(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                    int64_t d, float scale, int mask, int64_t window,
                                    const void* q, const void* k, const void* v, const void* o,
                                    const float* lse, const void* dout,
                                    const void* dq, const void* dk, const void* dv,
                                    const void* workspace, size_t workspace_bytes,
                                    const attn_layouts* layouts);

/*
 * IHA premix -- pseudo-token construction of Interleaved Head Attention
 * ("IHA-CUDA: Interleaved Head Attention Kernels for Hopper GPUs", section
 * "Pseudo-Token Mixing"): Q, K and V are each mixed across heads before
 * attention,
 *     Out[h, p] = sum_s W[h, p, s] * X[s]
 * a linear map from H source heads to H x P pseudo-heads at every (batch,
 * position, feature).  Layouts (contiguous):
 *     x, dx     [B][N][H][d]      e.g. a projection output
 *     w         [H][P][H]         W[h][p][s], element type `dtype`
 *     out, dout [B][H][N][P][d]   per head the N * P pseudo-tokens in the
 *                                 order t = n * P + p
 *     dw        [H][P][H]         fp32
 * Attention over each head's pseudo-token sequence (attn_fwd with Nq = Nk =
 * N * P on `out` read as [B][H][N * P][d]) is IHA's joint softmax across the
 * P pseudo-heads; the pages' FLOP matching uses a causal sliding window of
 * W = WSL + 1 = N / (2P) pseudo-tokens.
 * dtype: ATTN_BF16 or ATTN_FP16 (ATTN_ERR_UNSUPPORTED otherwise), fp32
 * accumulation, outputs rounded to nearest even.  d in {64, 96, 128};
 * H <= 32, H * P <= 128, P a power of two (ATTN_ERR_UNSUPPORTED otherwise);
 * H * N * P * d < 2^31 (ATTN_ERR_INVALID_ARG).  Pointers 16-byte aligned;
 * outputs may not overlap inputs or each other.
 */
ATTN_API int attn_premix_fwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                             const void* x, const void* w, void* out, void* stream);

/*
 * attn_premix_bwd_workspace_size -- bytes of fp32 workspace attn_premix_bwd
 * needs: one H*P*H partial dW per workgroup (min(B*N, 1024) of them),
 * rounded up to 256.  0 for unsupported H, P or sizes < 1.
 */
ATTN_API size_t attn_premix_bwd_workspace_size(int64_t B, int64_t N, int64_t H, int64_t P);

/*
 * attn_premix_bwd -- dx = W^T dout (the transposed map) and dw = sum over
 * (b, n, feature) of dout * x^T, for the same arguments as attn_premix_fwd.
 * dw is reduced without atomics: each workgroup writes a partial sum to the
 * workspace (contents on entry ignored) and a second kernel adds them in a
 * fixed order, so results are bitwise deterministic.
 */
ATTN_API int attn_premix_bwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P, int64_t d,
                             const void* x, const void* w, const void* dout, void* dx,
                             float* dw, void* workspace, size_t workspace_bytes, void* stream);

/* attn_check_premix_fwd / attn_check_premix_bwd -- their validation alone. */
ATTN_API int attn_check_premix_fwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P,
                                   int64_t d, const void* x, const void* w, const void* out);
ATTN_API int attn_check_premix_bwd(int dtype, int64_t B, int64_t N, int64_t H, int64_t P,
                                   int64_t d, const void* x, const void* w, const void* dout,
                                   const void* dx, const float* dw, const void* workspace,
                                   size_t workspace_bytes);

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace.  The row sums D go to
 * a scratch array that the library holds in device memory: one copy per GPU,
 * ATTN_NOALLOC_SCRATCH_BYTES bytes, held until the process ends.  Calls whose
 * minimum workspace, attn_bwd_workspace_size(B, H, Nq) = 4 B H Nq bytes
 * rounded up to 256, exceeds that size return ATTN_ERR_WORKSPACE and enqueue
 * nothing (B H Nq <= 4,194,304 rows fit).  The call allocates nothing and
 * records no memset: the row-sum pass writes every D it reads, and the dQ
 * pass recomputes S and dP (no kept dS).  Results equal attn_bwd's with a
 * workspace of attn_bwd_workspace_size(B, H, Nq) bytes.  Every call on one GPU
 * shares that GPU's scratch array, which keeps the last call's contents:
 * calls that overlap on one GPU (two streams, or two threads) race on it and
 * must be ordered by the caller.  Errors as attn_bwd.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
ATTN_API int attn_bwd_noalloc(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                              float scale, int mask, int64_t window,
                              const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout,
                              void* dq, void* dk, void* dv, void* stream);

/* attn_status_string -- static, human-readable name of a status code. */
ATTN_API const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
