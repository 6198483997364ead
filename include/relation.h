/*
 * librelation — exact causal Full / Multi-Head Relation on AMD Instinct MI355X
 * (gfx950). C ABI.
 *
 * The operator is the Self-Exchange Relation of "Ask Self, Ask Others:
 * Relation Is All You Need" (arXiv 2608.20172), Sec. 3.1, applied per head as
 * in Sec. 3.2 (Multi-Head Relation). For one head with p1 = q, p2 = k, I = v
 * (each T x D) and 1-based rows i:
 *
 *   U_ij = scale * q_i . k_j                               (pairwise evidence)
 *   S_i  = sigmoid(U_ii / tau_s)                           (Self)
 *   E_ij = SiLU(U_ij) = U_ij * sigmoid(U_ij),  j < i        (Exchange)
 *   R_ij = S_i if j = i;  E_ij - lambda * ln(i) if j < i;  -inf if j > i
 *   F_i  = softmax(R_i);   Y_i = sum_{j <= i} F_ij v_j      (Flow, transport)
 *
 * Derived per-row quantities (Sec. 4.2; App. A.1.2): the Exchange mass
 * g_i = sum_{j<i} F_ij = sigmoid(A_i - S_i) with
 * A_i = ln sum_{j<i} e^{E_ij} - lambda ln(i), and the row log-normaliser
 * LSE_i = ln Z_i = ln(e^{S_i} + e^{A_i}). Row 1 has no history: A_1 = -inf,
 * g_1 = 0, Y_1 = v_1, LSE_1 = S_1 (App. A.1.8).
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major and contiguous: [B, H, T, D] with D fastest.
 *    Element type is given by `dtype` (REL_F32 = float, REL_BF16 = bfloat16).
 *  - Pointers to tensors are DEVICE pointers (hipMalloc / torch CUDA memory)
 *    on the current HIP device, 16-byte aligned. Scalars are passed by value.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call only enqueues work on that stream and returns; the caller
 *    synchronises. Call order on one stream defines the data flow.
 *  - The library allocates no device memory, keeps no state between calls
 *    (save the static scratch of relation_cache_decode_noalloc), never frees
 *    or retains caller memory, and is safe to call from several host
 *    threads. Outputs must not alias inputs.
 *  - Validation is synchronous, on the host, before anything is enqueued; on
 *    any error nothing is written. Errors reported by the HIP runtime at
 *    launch map to REL_ERR_HIP; faults inside kernels surface at the caller's
 *    next synchronisation, as for any HIP call.
 *  - scale: the pages print U = p1.p2 / d_h; their text drops square roots,
 *    so callers normally pass 1/sqrt(D). Any finite value is accepted.
 *  - tau_s > 0 (the pages fix tau_s = 2); lambda: any finite value (the
 *    pages' learnable layer-wise count correction, Sec. 3.1).
 *  - lambda_dev (relation_fwd, relation_bwd, relation_mhr_fwd,
 *    relation_mhr_bwd): NULL, or a DEVICE float32 scalar, 4-byte aligned,
 *    that the kernels read when they run; `lambda` is then unused (still
 *    checked to be finite: pass 0). A learnable lambda kept on the device
 *    thus needs no host synchronisation per call. Its value is not checked:
 *    a non-finite one gives non-finite outputs.
 */
#ifndef LIBRELATION_RELATION_H
#define LIBRELATION_RELATION_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  REL_OK = 0,
  REL_ERR_NULL = 1,        /* a required pointer is NULL                      */
  REL_ERR_SHAPE = 2,       /* B, H, T < 1, or sizes overflow the index range  *
                            * (one head's T * D or capacity * D must be below *
                            * 2^31 elements; all heads below 2^40)             */
  REL_ERR_UNSUPPORTED = 3, /* dtype / head dimension not built                */
  REL_ERR_PARAM = 4,       /* scale or lambda not finite, tau_s <= 0          */
  REL_ERR_CAPACITY = 5,    /* decode: n_hist < 0 or n_hist + 1 > capacity     */
  REL_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned                */
  REL_ERR_WORKSPACE = 7,   /* workspace NULL or smaller than the queried size */
  REL_ERR_HIP = 8,         /* the HIP runtime reported an error               */
  REL_ERR_SCRATCH = 9      /* more scratch than the static buffer holds       */
} relation_status;

typedef enum { REL_F32 = 0, REL_BF16 = 1 } relation_dtype;

/* Head dimensions built: REL_F32 forward/backward/decode: D in {32, 64};
 * REL_BF16 forward, decode and prefill: D in {48, 64, 80} (the paper's 10M,
 * 30M and 100M head widths); REL_BF16 backward: D in {48, 64, 80}. Other
 * (dtype, D) pairs -> REL_ERR_UNSUPPORTED. */

/*
 * relation_fwd — Multi-Head Relation forward (Sec. 3.1 / 3.2), evaluated
 * exactly by a tiled scan of the historical Exchange entries with running
 * (m, l, z) (Sec. 5.1; App. A.3) and the row completion of App. A.3.5.
 *
 *   q, k, v : in  [B, H, T, D], dtype
 *   y       : out [B, H, T, D], dtype (round to nearest even from fp32)
 *   lse     : out [B, H, T] float32, LSE_i = ln Z_i; NULL to skip. Needed by
 *             relation_bwd.
 *   gate    : out [B, H, T] float32, the Exchange mass g_i; NULL to skip.
 *   workspace, workspace_bytes : optional DEVICE scratch, 256-byte aligned,
 *             of at least relation_fwd_workspace_bytes(...) bytes, owned by
 *             the caller and free again when the stream has passed the call.
 *             With it, a grid too small to fill the GPU splits its long
 *             query blocks over the keys and merges the pieces' (m, l, z)
 *             in a second kernel by App. A.3.2's rule (the same result up to
 *             fp32 rounding order). NULL: one workgroup per query block.
 *             Non-NULL and too small -> REL_ERR_WORKSPACE; misaligned ->
 *             REL_ERR_ALIGN.
 */
relation_status relation_fwd(relation_dtype dtype, int B, int H, int T, int D,
                             const void* q, const void* k, const void* v,
                             void* y, float* lse, float* gate,
                             void* workspace, size_t workspace_bytes,
                             float scale, float tau_s, float lambda,
                             const float* lambda_dev, void* stream);

/* Workspace bytes relation_fwd can use at this shape: 0 when the grid is
 * large enough on its own (and for REL_F32 or an invalid shape). */
size_t relation_fwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D);

/*
 * relation_bwd — gradients of a scalar loss L through relation_fwd, by
 * recomputation (nothing T x T is stored): with G_i = dL/dY_i (App. A.1.7),
 * dL/dF_ij = G_i . v_j, dL/dR_ij = F_ij (G_i . v_j - G_i . Y_i), then through
 * SiLU (j < i), the Self sigmoid (j = i, factor S_i (1 - S_i) / tau_s) and
 * U = scale * q k^T.
 *
 *   q, k, v, y : in [B, H, T, D], dtype (y = relation_fwd's output)
 *   dy         : in [B, H, T, D], dtype (dL/dY)
 *   lse        : in [B, H, T] float32 from relation_fwd
 *   dq, dk, dv : out [B, H, T, D], dtype, overwritten
 *   dlambda    : out, one float32 on the device: dL/dlambda summed over every
 *                batch and head (lambda is one scalar per layer); NULL to skip
 *   workspace  : device scratch of at least relation_bwd_workspace_bytes()
 *                bytes, 256-byte aligned; contents on entry are ignored.
 */
size_t relation_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D);

relation_status relation_bwd(relation_dtype dtype, int B, int H, int T, int D,
                             const void* q, const void* k, const void* v,
                             const void* y, const void* dy, const float* lse,
                             void* dq, void* dk, void* dv, float* dlambda,
                             void* workspace, size_t workspace_bytes,
                             float scale, float tau_s, float lambda,
                             const float* lambda_dev, void* stream);

/*
 * relation_bwd_events — relation_bwd (same operation, App. A.1.7; same
 * arguments, results and errors) that also records two caller-created HIP
 * events on `stream`. ev_main_begin is recorded right before the main
 * backward kernel(s) and ev_main_end right after them. Neither covers the
 * preprocess (row terms, accumulator clear) or the dq finalize. With
 * hipEventElapsedTime, a caller can time the main kernel alone, for example
 * to compare with a profiler's per-kernel durations.
 *   ev_main_begin, ev_main_end : hipEvent_t as void*, owned by the caller;
 *                                either may be NULL (then not recorded).
 * A failed record returns REL_ERR_HIP with the same meaning as a failed
 * launch.
 */
relation_status relation_bwd_events(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* q, const void* k, const void* v,
                                    const void* y, const void* dy, const float* lse,
                                    void* dq, void* dk, void* dv, float* dlambda,
                                    void* workspace, size_t workspace_bytes,
                                    float scale, float tau_s, float lambda,
                                    const float* lambda_dev, void* stream,
                                    void* ev_main_begin, void* ev_main_end);

/*
 * relation_cache_decode — one autoregressive step over the KV-style Relation
 * Cache (named in the paper's first version as its decoding form). The new
 * token of every sequence is at 1-based position i = n_hist + 1; its output
 * is the last row of the forward over the concatenated sequence.
 *
 *   q, k_new, v_new  : in  [B, H, D], dtype (the new token's q, k and v)
 *   k_cache, v_cache : in/out [B, H, capacity, D], dtype. Slots [0, n_hist)
 *                      are read; slot n_hist is overwritten with k_new /
 *                      v_new (an exact copy); every other slot is untouched.
 *   capacity, n_hist : host ints, uniform over the batch; 0 <= n_hist and
 *                      n_hist + 1 <= capacity.
 *   y                : out [B, H, D], dtype
 *   gate             : out [B, H] float32 Exchange mass g; NULL to skip
 *   workspace        : device scratch of at least
 *                      relation_decode_workspace_bytes() bytes (256-byte
 *                      aligned); contents on entry are ignored. Calls that
 *                      run at the same time must not share it.
 */
size_t relation_decode_workspace_bytes(relation_dtype dtype, int B, int H, int D, int capacity);

relation_status relation_cache_decode(relation_dtype dtype, int B, int H, int D,
                                      const void* q, const void* k_new, const void* v_new,
                                      void* k_cache, void* v_cache,
                                      int capacity, int n_hist,
                                      void* y, float* gate,
                                      void* workspace, size_t workspace_bytes,
                                      float scale, float tau_s, float lambda,
                                      void* stream);

/*
 * relation_cache_decode_noalloc — relation_cache_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same step and the same
 * kernels, with the workspace taken from a static device array of the
 * library (8 MiB per GPU, held until the process ends) instead of an
 * argument. It calls no allocator.
 *
 *   Arguments as for relation_cache_decode, without the workspace. The
 *   stream must belong to the current device (else REL_ERR_HIP).
 *   The step uses scratch only when B * H < 256 and n_hist > 0: one fp32
 *   partial of D + 2 values per head and chunk of about 256 history slots,
 *   B * H * ceil(n_hist / 256) * (D + 2) * 4 bytes. A call that needs more
 *   than 8 MiB returns REL_ERR_SCRATCH and does nothing (at D = 64 that is
 *   beyond about 7.8 M slots of history summed over the heads; batches of
 *   256 heads or more need none).
 *   The first call on a device looks up that device's copy of the array.
 *   Every call on one GPU shares it and it keeps the last call's contents
 *   (nothing in it needs to start at zero), so calls that overlap in time
 *   on one GPU (other streams, other threads) race and give wrong results;
 *   calls ordered on one stream are safe.
 */
relation_status relation_cache_decode_noalloc(relation_dtype dtype, int B, int H, int D,
                                              const void* q, const void* k_new,
                                              const void* v_new, void* k_cache, void* v_cache,
                                              int capacity, int n_hist, void* y, float* gate,
                                              float scale, float tau_s, float lambda,
                                              void* stream);

/*
 * relation_cache_decode_ragged — the same step as relation_cache_decode for a
 * batch whose sequences have different history lengths (a ragged Relation
 * Cache). Sequence b's new token is at 1-based position n_hist[b] + 1 and is
 * computed exactly as relation_cache_decode computes it with
 * n_hist = n_hist[b].
 *
 *   n_hist     : in  DEVICE int32 [B], 4-byte aligned. Read on the device; the
 *                library does not change it (the caller advances it).
 *   max_n_hist : host int, an upper bound of n_hist[]: it sizes the launch
 *                (work scales with the actual lengths, the launch with the
 *                bound). 0 <= max_n_hist < capacity, else REL_ERR_CAPACITY.
 *   Other arguments as for relation_cache_decode, with the same workspace
 *   size (relation_decode_workspace_bytes).
 *
 * Device-side values the host cannot check: a sequence with n_hist[b] < 0,
 * n_hist[b] > max_n_hist or n_hist[b] >= capacity gets NaN in y[b] (and in
 * gate[b] when gate is given); its cache rows are not touched.
 */
relation_status relation_cache_decode_ragged(relation_dtype dtype, int B, int H, int D,
                                             const void* q, const void* k_new, const void* v_new,
                                             void* k_cache, void* v_cache, int capacity,
                                             const int* n_hist, int max_n_hist,
                                             void* y, float* gate,
                                             void* workspace, size_t workspace_bytes,
                                             float scale, float tau_s, float lambda,
                                             void* stream);

/*
 * relation_cache_prefill — m new tokens per sequence at once (chunked
 * prefill into the Relation Cache). Sequence b's new tokens sit at 0-based
 * positions n_b .. n_b + m - 1 (1-based i = n_b + t + 1): they are appended
 * to cache slots n_b .. n_b + m - 1 (an exact copy) and each one's row is
 * computed against the cache rows before it and the new tokens up to
 * itself, i.e. rows n_b + 1 .. n_b + m of the forward over the whole
 * sequence (Sec. 3.1; lambda ln i uses the global position).
 *
 *   q, k_new, v_new  : in  [B, H, m, D], bf16 (REL_BF16 and D in
 *                      {48, 64, 80} only; otherwise REL_ERR_UNSUPPORTED)
 *   k_cache, v_cache : in/out [B, H, capacity, D]
 *   n_hist_dev       : NULL: every sequence has n_hist slots of history.
 *                      Otherwise DEVICE int32 [B] per-sequence lengths with
 *                      n_hist their upper bound; a sequence whose length is
 *                      negative, above the bound or leaves no room for m
 *                      tokens gets NaN rows and no append.
 *   n_hist           : 0 <= n_hist and n_hist + m <= capacity, else
 *                      REL_ERR_CAPACITY.
 *   y                : out [B, H, m, D]; lse, gate: out [B, H, m] fp32 or NULL
 *   workspace, workspace_bytes : optional DEVICE scratch as for relation_fwd,
 *                      of relation_prefill_workspace_bytes(...) bytes for the
 *                      same (B, H, D, m, n_hist) and per_sequence =
 *                      (n_hist_dev != NULL): splits the rows' long histories
 *                      over several workgroups. NULL: no split.
 */
relation_status relation_cache_prefill(relation_dtype dtype, int B, int H, int D, int m,
                                       const void* q, const void* k_new, const void* v_new,
                                       void* k_cache, void* v_cache, int capacity,
                                       const int* n_hist_dev, int n_hist,
                                       void* y, float* lse, float* gate,
                                       void* workspace, size_t workspace_bytes,
                                       float scale, float tau_s, float lambda,
                                       void* stream);

/* Workspace bytes relation_cache_prefill can use; 0 when it would not split
 * (or the arguments are invalid). The split assumes per-sequence lengths
 * spread over [0, n_hist] when per_sequence is non-zero. */
size_t relation_prefill_workspace_bytes(relation_dtype dtype, int B, int H, int D, int m,
                                        int n_hist, int per_sequence);

/*
 * relation_mhr_fwd / relation_mhr_bwd — Multi-Head Relation with the two maps
 * that precede the Relation operator in a layer (Sec. 3.1-3.2; App. A.2.2-
 * A.2.3), fused or chained inside the call:
 *
 *   q = RoPE(p1), k = RoPE(p2)   rotary position encoding of the head-wise
 *                                p1, p2 (Sec. 3.1; App. B.3: full head, base
 *                                1e4). Element d pairs with d + D/2 and the
 *                                pair j of the row at 0-based position t
 *                                turns by the angle whose cosine and sine are
 *                                rope_cos[t, j], rope_sin[t, j].
 *   I' = Givens(I)               adjacent information slices mixed pairwise:
 *                                for each pair (a, b) with angle theta[p],
 *                                I'_a = cos I_a + sin I_b,
 *                                I'_b = -sin I_a + cos I_b.
 *                                pairing 0: pairs (1,2), (3,4), ..., (H-1,H);
 *                                pairing 1: (2,3), (4,5), ..., (H,1)
 *                                (1-based heads; the pattern alternates
 *                                between layers). H must be even.
 *   Y = Relation(q, k, I')       exactly as relation_fwd (I' is the only
 *                                information state the head sees, Self term
 *                                included).
 *
 *   p1, p2, I        : in  [B, H, T, D], dtype (unrotated, unmixed)
 *   rope_cos/rope_sin: in  DEVICE float32 [T, D/2], 16-byte aligned; both
 *                      NULL to skip RoPE (one NULL alone: REL_ERR_NULL)
 *   theta            : in  DEVICE float32 [H/2]; NULL to skip the mixing
 *   pairing          : 0 or 1 (REL_ERR_PARAM otherwise; odd H with theta:
 *                      REL_ERR_SHAPE)
 *   y, lse, gate     : as relation_fwd
 *   workspace        : relation_mhr_fwd_workspace_bytes() bytes, 256-byte
 *                      aligned: the rotated keys and mixed values are formed
 *                      there once by a bandwidth-bound pass (every query
 *                      block reads every key tile, so rotating them inside
 *                      the tile loop would repeat the work); REL_BF16 rotates
 *                      its query rows in registers, REL_F32 in the workspace.
 *
 * relation_mhr_bwd: gradients with respect to p1, p2, I, lambda and theta.
 *   dp1, dp2, dI     : out [B, H, T, D], dtype
 *   dlambda          : out DEVICE float32 scalar (NULL to skip)
 *   dtheta           : out DEVICE float32 [H/2] (NULL to skip; ignored
 *                      without theta)
 *   fwd_workspace    : optional: the workspace of the relation_mhr_fwd call
 *                      that produced y and lse, unchanged since (same inputs,
 *                      tables, theta, pairing). The rotated keys and mixed
 *                      values (and, where the forward stored them, the
 *                      rotated queries) are then read from it instead of
 *                      being formed again. NULL: formed here. A workspace
 *                      that does not hold that forward's values gives wrong
 *                      gradients (it cannot be checked).
 *   workspace        : relation_mhr_bwd_workspace_bytes() bytes, 256-byte
 *                      aligned; contents on entry are ignored.
 *   Other arguments as relation_bwd; y and lse are the forward's outputs.
 */
size_t relation_mhr_fwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D);

relation_status relation_mhr_fwd(relation_dtype dtype, int B, int H, int T, int D,
                                 const void* p1, const void* p2, const void* I,
                                 const float* rope_cos, const float* rope_sin,
                                 const float* theta, int pairing,
                                 void* y, float* lse, float* gate,
                                 void* workspace, size_t workspace_bytes,
                                 float scale, float tau_s, float lambda,
                                 const float* lambda_dev, void* stream);

size_t relation_mhr_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D);

relation_status relation_mhr_bwd(relation_dtype dtype, int B, int H, int T, int D,
                                 const void* p1, const void* p2, const void* I,
                                 const float* rope_cos, const float* rope_sin,
                                 const float* theta, int pairing,
                                 const void* y, const void* dy, const float* lse,
                                 void* dp1, void* dp2, void* dI,
                                 float* dlambda, float* dtheta,
                                 const void* fwd_workspace,
                                 void* workspace, size_t workspace_bytes,
                                 float scale, float tau_s, float lambda,
                                 const float* lambda_dev, void* stream);

/*
 * relation_linear_fwd — Linear Relation (Sec. 5.2; App. A.4): historical
 * Others compressed into a D x D state with channel-wise retention, read
 * before the current token is written:
 *   S_t  = sigmoid(scale * p1_t . p2_t / tau_s)       (Self; RoPE leaves it
 *                                                      unchanged)
 *   x^   = x / ||x|| for the rotated p1_t, p2_t (a zero row stays zero)
 *   E_t  = S_t (Diag(alpha_t) C_{t-1})^T p1^_t,  alpha_t = exp(g_t)
 *   Y_t  = I_t + E_t
 *   C_t  = Diag(alpha_t) C_{t-1} + S_t p2^_t I_t^T     (rows: key channel)
 * computed by chunks of 128 tokens (one workgroup per head); exact up to
 * rounding, also under total retention loss (g = -inf gives alpha = 0).
 *
 *   dtype            : REL_BF16 with D = 64 (else REL_ERR_UNSUPPORTED)
 *   p1, p2, I        : in  [B, H, T, D] bf16, 16-byte aligned
 *   g                : in  [B, H, T, D] fp32 log retention (<= 0; the
 *                      upstream retention map of Sec. 5.2 produces it)
 *   rope_cos/rope_sin: in  DEVICE fp32 [T, D/2] as for relation_mhr_fwd
 *                      (row t = 0-based position in this call); both NULL
 *                      to skip RoPE (one NULL alone: REL_ERR_NULL)
 *   state_in         : in  DEVICE fp32 [B, H, D, D] C_0, or NULL for zero
 *   y                : out [B, H, T, D] bf16
 *   state_out        : out DEVICE fp32 [B, H, D, D] the state after the last
 *                      token, or NULL (a later call continues from it)
 *   states           : out DEVICE fp32 [B, H, ceil(T / 128) + 1, D, D]
 *                      (relation_linear_states_bytes() bytes), 16-byte
 *                      aligned, or NULL: the state before every 128-token
 *                      chunk, then the final state. A training step passes
 *                      it to relation_linear_bwd as fwd_states, which then
 *                      skips its own state pass.
 *   scale, tau_s     : finite scale, tau_s > 0 (else REL_ERR_PARAM)
 */
relation_status relation_linear_fwd(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* p1, const void* p2, const void* I,
                                    const float* g, const float* rope_cos,
                                    const float* rope_sin, const float* state_in,
                                    void* y, float* state_out, float* states,
                                    float scale, float tau_s, void* stream);

/*
 * relation_linear_bwd — gradients of relation_linear_fwd with respect to p1,
 * p2, I, g and state_in, given dy and (optionally) the gradient of the final
 * state. Three passes: the state before every 128-token chunk (forward),
 * the gradient of the state after every chunk (backward over the chunks),
 * then every chunk's gradients independently. When B * H is at least 3/4 of
 * the device's CU count, the last two run as one pass (one workgroup per
 * head, chunks from the last, the state gradient kept on chip). The
 * environment variable RELATION_LINEAR_BWD=fused or =chunked forces one form;
 * both give the same gradients up to fp32 rounding of dg. The workspace
 * sizes below cover either form.
 *
 *   p1, p2, I, g, rope_cos/rope_sin, state_in : as relation_linear_fwd
 *   dy               : in  [B, H, T, D] bf16, gradient of y
 *   dstate_out       : in  DEVICE fp32 [B, H, D, D] gradient of state_out,
 *                      or NULL for zero
 *   dp1, dp2, dI     : out [B, H, T, D] bf16
 *   dg               : out [B, H, T, D] fp32, gradient of the log retention
 *   dstate_in        : out DEVICE fp32 [B, H, D, D] gradient of state_in, or
 *                      NULL
 *   fwd_states       : in  DEVICE fp32, 16-byte aligned (the kernels read it
 *                      with 16-byte vector loads), or NULL: the states
 *                      relation_linear_fwd stored for these same inputs
 *                      (its `states` output). Given, the first pass is
 *                      skipped; states of other inputs give wrong gradients,
 *                      with no error.
 *   workspace        : 256-byte aligned. Without fwd_states:
 *                      relation_linear_bwd_workspace_bytes() bytes
 *                      (B * H * (2 ceil(T / 128) + 1) * D * D floats: the
 *                      state before every chunk and the final state, then
 *                      the gradient of the state after every chunk). With
 *                      fwd_states: relation_linear_bwd_reuse_workspace_bytes()
 *                      bytes (B * H * ceil(T / 128) * D * D floats, the state
 *                      gradients only). Smaller: REL_ERR_WORKSPACE.
 * The three size queries return 0 for unsupported (dtype, D) or bad shapes.
 */
size_t relation_linear_states_bytes(relation_dtype dtype, int B, int H, int T, int D);
size_t relation_linear_bwd_workspace_bytes(relation_dtype dtype, int B, int H, int T, int D);
size_t relation_linear_bwd_reuse_workspace_bytes(relation_dtype dtype, int B, int H, int T,
                                                 int D);
relation_status relation_linear_bwd(relation_dtype dtype, int B, int H, int T, int D,
                                    const void* p1, const void* p2, const void* I,
                                    const float* g, const float* rope_cos,
                                    const float* rope_sin, const float* state_in,
                                    const void* dy, const float* dstate_out,
                                    void* dp1, void* dp2, void* dI, float* dg,
                                    float* dstate_in, const float* fwd_states,
                                    void* workspace, size_t workspace_bytes, float scale,
                                    float tau_s, void* stream);

/*
 * relation_linear_step — one decode step of Linear Relation (the recurrent
 * step of Sec. 5.2) for one new token per sequence: the O(D^2) state is the
 * whole decode state (Table 1).
 *   p1, p2, I        : in  [B, H, D] bf16;  g: in [B, H, D] fp32
 *   rope_cos/rope_sin: in  DEVICE fp32 [D/2], the table row of the token's
 *                      position, or both NULL
 *   state            : in/out DEVICE fp32 [B, H, D, D] (C_{t-1} -> C_t)
 *   y                : out [B, H, D] bf16
 * REL_BF16, D = 64 only; 4-byte alignment.
 */
relation_status relation_linear_step(relation_dtype dtype, int B, int H, int D,
                                     const void* p1, const void* p2, const void* I,
                                     const float* g, const float* rope_cos,
                                     const float* rope_sin, float* state, void* y,
                                     float scale, float tau_s, void* stream);

/* Static, NUL-terminated description of a status code (host only). */
const char* relation_status_string(relation_status s);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH (host only). */
int relation_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBRELATION_RELATION_H */
