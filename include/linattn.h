/*
 * linattn.h -- C ABI of the MI355X (gfx950) causal linear-attention library
 * (liblinattn.so). Plain C: pointers, sizes and enums; no C++ or framework types.
 *
 * What is computed. Per batch b and head h, for tokens t = 1..L, with a matrix
 * state S of shape d_k x d_v (row index = key channel):
 *
 *   LA_PLAIN        S_t = S_{t-1} + k_t v_t^T,            o_t = S_t^T q_t
 *                   i.e. O = (Q K^T (.) M) V with M the causal mask including
 *                   the diagonal (tensorplay "Talk Linear Attention", section 2.1,
 *                   parallel form, per-token sum and recurrence).
 *   LA_NORMALIZED   as PLAIN, plus z_t = z_{t-1} + k_t and
 *                   o_t = (S_t^T q_t) / (q_t . z_t). q and k are passed already
 *                   feature-mapped; the library applies no feature map
 *                   (proig-chaa notes "线性注意力", sections 13-14).
 *   LA_DECAY        S_t = gamma_t S_{t-1} + k_t v_t^T with gamma_t = exp(l_t)
 *                   (wln20 "LLM注意力优化：线性注意力", data-dependent decay
 *                   equation; a constant l gives the data-independent decay).
 *   LA_VECTOR_DECAY S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T with one gate per key
 *                   channel, alpha_t = exp(l_t), l_t in R^{d_k}; o_t = S_t^T q_t
 *                   (tensorplay section 5.1: the GLA gate matrix G_t (.) S_{t-1},
 *                   alpha_t broadcast over the value columns; section 5.2 gives
 *                   its chunk form (Q (.) B)(K / B)^T with B the cumulative
 *                   product of the gates).
 *   LA_GATED_DELTA  S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 *                   alpha_t = exp(l_t) (alpha = 1 when log_gate is NULL, i.e. the
 *                   DeltaNet rule), o_t = S_t^T q_t. This is the transpose of the
 *                   pages' S'_t = S'_{t-1} alpha_t (I - beta_t k_t k_t^T) +
 *                   beta_t v_t k_t^T (wln20, Gated DeltaNet section; tensorplay
 *                   section 6.2); outputs are identical.
 *   LA_KDA          Kimi Delta Attention: the gated delta rule with one gate per
 *                   key channel, S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                   + beta_t k_t v_t^T, alpha_t = exp(l_t), l_t in R^{d_k},
 *                   o_t = S_t^T q_t (wln20, Kimi Delta Attention section, read in
 *                   the d_k x d_v orientation: the diagonal gate acts on the key
 *                   channels and the delta-rule factor multiplies from the left).
 *
 * la_chunk_fwd evaluates these in the chunkwise-parallel form (tensorplay
 * section 3.2): per chunk of C tokens an intra-chunk masked product, an
 * inter-chunk term Q S_prev, and a serial state pass from chunk to chunk.
 * la_decode_step applies one token of the recurrence to a stored state
 * (tensorplay section 2.2: constant-size state at inference).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates and frees nothing and keeps no state between calls except the
 *    loaded code objects and a per-process record of the device check.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise the host.
 *  - Arguments are validated before anything is launched; on any error nothing
 *    is launched and no output is touched.
 *  - Layouts are row-major and contiguous:
 *      q, k [B, H, L, d_k];  v, o [B, H, L, d_v];  log_gate, beta [B, H, L];
 *      state [B, H, d_k, d_v];  z [B, H, d_k].
 *    Tensor pointers must be 16-byte aligned.
 *  - dt is the dtype of q, k, v: LA_BF16 or LA_F32. o_dt is the dtype of o:
 *    LA_F32 (any dt) or LA_BF16 (dt = LA_BF16 only; rounded to nearest even from
 *    the fp32 accumulators). Gates, beta, states and normalizers are float32.
 *  - Numerics. fp32 inputs are computed on fp32 tensor-core operands. bf16
 *    inputs are computed on fp16 tensor-core operands with fp32 accumulation:
 *    bf16 values are exact in fp16 for magnitudes in [2^-14, 65504]; smaller
 *    ones keep an absolute error below 2^-25. The state carried from chunk to
 *    chunk stays in fp32 and has no range limit of its own in la_chunk_fwd for
 *    LA_PLAIN, LA_NORMALIZED, LA_DECAY and LA_GATED_DELTA: its fp16 operand
 *    (and the delta rule's pseudo-values) is scaled per chunk by a power of two
 *    chosen from the previous chunk's largest |S|, and the normalizer is
 *    applied in fp32. What remains bounded is per chunk and set by the inputs:
 *    the masked scores q_r . k_s of one chunk must stay below 65504, and the
 *    state may grow at most 256-fold within one chunk (or to at most 65504
 *    from below 256). LA_VECTOR_DECAY and la_chunk_bwd keep an unscaled fp16
 *    state operand: states beyond 65504 are outside their supported range.
 *    Choose o_dt = LA_F32 when the output is compared at a tolerance finer
 *    than bf16's 2^-8 relative spacing.
 *  - No C++ exception crosses this boundary. Thread-safe for distinct streams.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 3

typedef enum la_status {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = 1, /* null required pointer, bad size, misalignment,
                               workspace missing or too small, aliasing */
    LA_ERR_UNSUPPORTED = 2, /* size/variant/dtype combination not built, or the
                               current device is not gfx950 */
    LA_ERR_HIP = 3          /* the HIP runtime reported an error at launch */
} la_status;

typedef enum la_variant {
    LA_PLAIN = 0,
    LA_NORMALIZED = 1,
    LA_DECAY = 2,
    LA_GATED_DELTA = 3,
    LA_VECTOR_DECAY = 4,
    LA_KDA = 5
} la_variant;

typedef enum la_dtype {
    LA_F32 = 0,
    LA_BF16 = 1
} la_dtype;

/*
 * Workspace bytes la_chunk_fwd needs for this problem (written to *bytes).
 * Zero for LA_PLAIN, LA_NORMALIZED, LA_DECAY and LA_VECTOR_DECAY, which run in
 * one fused pass.
 * LA_GATED_DELTA runs a chunk-parallel preparation pass first and stores its
 * per-chunk products there: W and U~ of the chunkwise delta-rule form,
 * B*H*Lp*d_k and B*H*Lp*d_v elements (2 bytes each for bf16 inputs, 4 for
 * fp32), each rounded up to 256 bytes, with Lp = ceil(L/64)*64; for bf16 inputs
 * also the chunk's masked decayed scores, 96 bytes per token (B*H*Lp*96).
 * LA_KDA (bf16 inputs) stores the same three arrays, then q and k with the
 * per-channel gates folded in (2 * B*H*Lp*d_k fp16, each rounded up to 256
 * bytes) and the state's per-channel decay of every chunk (B*H*(Lp/64)*d_k
 * float32, rounded up to 256 bytes).
 * Returns LA_ERR_INVALID_ARG / LA_ERR_UNSUPPORTED like la_chunk_fwd.
 */
la_status la_chunk_fwd_workspace_size(la_variant var, la_dtype dt, int B, int H, int L,
                                      int d_k, int d_v, int C, size_t *bytes);

/*
 * Chunkwise forward over a whole sequence.
 *   q, k, v     inputs (dtype dt), required when L > 0.
 *   log_gate    [B,H,L] float32 log-gates l_t <= 0 (finite): required for
 *               LA_DECAY; optional for LA_GATED_DELTA (NULL = alpha 1); must be
 *               NULL for LA_PLAIN and LA_NORMALIZED. LA_VECTOR_DECAY takes
 *               [B,H,L,d_k] (one gate per key channel), required, entries <= 0:
 *               the chunk form rebases the per-channel decay around the middle
 *               of each 16-token block, and entries below -10 are taken as -10
 *               so that every rebased factor stays below e^80 (a gate of e^-10
 *               already damps the channel's history to 4.5e-5 per token, so
 *               the result moves by at most that fraction of the damped history).
 *               LA_KDA takes [B,H,L,d_k] too, required, with the same -10
 *               floor: its chunk form factors the decay between 16-token blocks
 *               at the block edges (every factor <= 1, fp16 operands) and takes
 *               the 16-token diagonal blocks in fp32 around their middle token.
 *   beta        [B,H,L] float32 in [0,1]: required for LA_GATED_DELTA and LA_KDA,
 *               NULL otherwise.
 *   state_in    [B,H,d_k,d_v] float32 initial state, NULL = zero.
 *   z_in        [B,H,d_k] float32 initial normalizer (LA_NORMALIZED only),
 *               NULL = zero. Must be NULL for the other variants.
 *   o           [B,H,L,d_v] output (dtype o_dt), required when L > 0; must not
 *               overlap any input or other output.
 *   state_out   [B,H,d_k,d_v] float32 final state, NULL = not written. May be
 *               equal to state_in (in-place carry); must not partially overlap it.
 *   z_out       [B,H,d_k] float32 final normalizer (LA_NORMALIZED only), NULL =
 *               not written; must not overlap z_in (every value slice of a head
 *               reads z_in while one of them writes z_out).
 *   B, H, L     batch, heads, tokens: B, H >= 1; L >= 0 (L = 0 only copies
 *               state_in/z_in, or zeros, to state_out/z_out).
 *   d_k         32, 64 or 128.   d_v  32, 64, 96 or 128 (a multiple of 32).
 *   C           chunk length: 64 or 128 (LA_GATED_DELTA, LA_KDA and
 *               LA_VECTOR_DECAY run 128 as two 64-token chunks, which gives the
 *               same result).
 *               L need not be a multiple of C; a ragged last chunk is handled.
 *               Rows of one head are addressed with 32-bit offsets:
 *               ceil(L / C) * C * max(d_k, d_v) >= 2^31 returns
 *               LA_ERR_UNSUPPORTED.
 *               LA_VECTOR_DECAY with LA_F32 inputs supports d_k 32 and 64.
 *               LA_KDA takes LA_BF16 inputs only (LA_F32: LA_ERR_UNSUPPORTED).
 *   workspace   device buffer of at least la_chunk_fwd_workspace_size() bytes
 *               (may be NULL when that size is 0), 256-byte aligned.
 */
la_status la_chunk_fwd(la_variant var, la_dtype dt, la_dtype o_dt, const void *q,
                       const void *k, const void *v, const float *log_gate,
                       const float *beta, const float *state_in, const float *z_in,
                       void *o, float *state_out, float *z_out, int B, int H, int L,
                       int d_k, int d_v, int C, void *workspace, size_t workspace_bytes,
                       void *stream);

/*
 * One recurrent decode step for N sequences x H heads, updating the state in
 * place, then o = S^T q with the updated S (tensorplay section 2.1-2.2):
 *   LA_DECAY        S <- exp(l) S + k v^T (wln20 decay equation)
 *   LA_PLAIN        S <- S + k v^T (log_gate NULL)
 *   LA_GATED_DELTA  r = S^T k;  S <- alpha (S - beta k r^T) + beta k v^T,
 *                   alpha = exp(l), or 1 when log_gate is NULL (DeltaNet)
 *                   (wln20 Gated DeltaNet section, d_k x d_v orientation)
 *   LA_VECTOR_DECAY S <- Diag(exp(l)) S + k v^T, l [N,H,d_k] (tensorplay
 *                   section 5.1)
 *   LA_KDA          r = (Diag(exp(l)) S)^T k;  S <- Diag(exp(l)) S + beta k (v - r)^T,
 *                   l [N,H,d_k] (wln20 Kimi Delta Attention section)
 *   q, k [N,H,d_k], v [N,H,d_v] in dtype dt; o [N,H,d_v] in dtype o_dt (the
 *   step itself is computed in fp32); log_gate [N,H] float32 (required for
 *   LA_DECAY, optional for LA_GATED_DELTA, NULL for LA_PLAIN; [N,H,d_k] and
 *   required for LA_VECTOR_DECAY and LA_KDA); beta [N,H] float32,
 *   required for LA_GATED_DELTA and LA_KDA and NULL otherwise; state [N,H,d_k,d_v] float32,
 *   read and written in place. o must not overlap the state or inputs.
 *   N, H >= 1; d_k, d_v in {32, 64, 128}. LA_NORMALIZED is not supported.
 */
la_status la_decode_step(la_variant var, la_dtype dt, la_dtype o_dt, const void *q,
                         const void *k, const void *v, const float *log_gate,
                         const float *beta, float *state, void *o, int N, int H, int d_k,
                         int d_v, void *stream);

/*
 * Causal depthwise short convolution over the token axis: the token-mixing step
 * applied to the projected q, k and v before the linear-attention recurrence
 * (wln20 "LLM注意力优化：线性注意力", DeltaNet section; kernel size 4 there).
 * For each of q, k, v that is given, per batch b, head h and channel c, with one
 * set of K taps per channel (depthwise):
 *     y_t[c] = sum_{tau=0}^{K-1} w[h][c][tau] * x_{t-tau}[c],   t = 0..L-1,
 * summed in fp32 and rounded to dt (bf16: to nearest even). Inputs before t = 0
 * come from the window state_in, the K-1 inputs preceding this call, oldest
 * first (NULL = zeros). state_out receives the window after the call: the K-1
 * most recent inputs, oldest first, the older ones taken from state_in when
 * L < K-1. A sequence can therefore be convolved in pieces, and L = 1 is the
 * decode step. No activation is applied. One launch covers all given tensors.
 *   dt           dtype of every input, output and window: LA_BF16 or LA_F32.
 *   w_q, w_k, w_v  float32 taps [H, d, K] (d = d_k or d_v); tap tau multiplies
 *                the input tau tokens back. A tensor is convolved when its taps
 *                are given; NULL taps skip it, and then its input, windows and
 *                output must be NULL too. At least one tensor is convolved.
 *   q, k, v      inputs [B,H,L,d_k], [B,H,L,d_k], [B,H,L,d_v] of the convolved
 *                tensors, required when L > 0.
 *   *_state_in   [B,H,K-1,d] or NULL.
 *   q_out, k_out, v_out  outputs, shaped and typed like their inputs; required
 *                for a given tensor when L > 0. They must not overlap any input,
 *                tap array, window or other output (no in-place y = x).
 *   *_state_out  [B,H,K-1,d] or NULL (not written). May equal the same tensor's
 *                state_in (window updated in place); must not otherwise overlap
 *                any other buffer.
 *   B, H >= 1; L >= 0; d_k, d_v multiples of 8, at most 4096 (else
 *   LA_ERR_UNSUPPORTED); K in 1..4 (K > 4: LA_ERR_UNSUPPORTED). Pointers 16-byte
 *   aligned.
 */
la_status la_short_conv(la_dtype dt, const void *q, const void *k, const void *v,
                        const float *w_q, const float *w_k, const float *w_v,
                        const void *q_state_in, const void *k_state_in, const void *v_state_in,
                        void *q_out, void *k_out, void *v_out, void *q_state_out,
                        void *k_state_out, void *v_state_out, int B, int H, int L, int d_k,
                        int d_v, int K, void *stream);

/*
 * la_chunk_fwd of the gated delta rule with the causal depthwise short
 * convolution of q, k and v fused in front (wln20 "LLM注意力优化：线性注意力",
 * DeltaNet section: a kernel-4 short convolution precedes the delta rule). The
 * result is la_chunk_fwd(q', k', v', ...) with x'_t = sum_{tau < K} w[h][c][tau]
 * x_{t - tau} per channel, x_{-j} taken from the incoming window (the inputs
 * before the sequence) or zero, as la_short_conv defines it. The preparation
 * pass reads the raw q, k, v once and convolves them on the way in; the
 * convolved q and k (fp16) go to the workspace for the serial pass, and v' is
 * used where it is formed. The convolved values are rounded to fp16, not bf16.
 *   var, dt      LA_GATED_DELTA and LA_BF16 (others: LA_ERR_UNSUPPORTED).
 *   o_dt, q, k, v, log_gate, beta, state_in, o, state_out, B, H, L, d_k, d_v, C
 *                as for la_chunk_fwd; q, k, v are the raw (unconvolved) inputs.
 *   w_q, w_k, w_v  taps [H, d, K] float32 (d = d_k, d_k, d_v), all required;
 *                tap tau multiplies the input tau tokens back.
 *   K            1..4 (K > 4: LA_ERR_UNSUPPORTED; K < 1: LA_ERR_INVALID_ARG).
 *   *_win_in     [B, H, K-1, d] bf16, the K-1 inputs before the sequence, oldest
 *                first, or NULL (zeros).
 *   *_win_out    [B, H, K-1, d] bf16 or NULL (not written): the K-1 most recent
 *                raw inputs after this call, ready to be the next call's window.
 *                May equal the same tensor's *_win_in (updated in place); must
 *                not otherwise overlap any buffer.
 *   workspace    at least la_chunk_fwd_conv_workspace_size() bytes, 256-byte
 *                aligned: la_chunk_fwd's workspace, then the convolved q and k,
 *                B*H*Lp*d_k fp16 each (Lp = ceil(L/64)*64, each rounded up to 256
 *                bytes), then B*H*3*(2 d_k + d_v) fp16 for the window update.
 * Errors as la_chunk_fwd; nothing is launched on error. Launches: the
 * preparation (convolution included), the serial pass, and when a window is
 * requested one short-convolution launch over the last min(L, K-1) tokens.
 */
la_status la_chunk_fwd_conv_workspace_size(la_variant var, la_dtype dt, int B, int H, int L,
                                           int d_k, int d_v, int C, int K, size_t *bytes);
la_status la_chunk_fwd_conv(la_variant var, la_dtype dt, la_dtype o_dt, const void *q,
                            const void *k, const void *v, const float *w_q, const float *w_k,
                            const float *w_v, int K, const void *q_win_in, const void *k_win_in,
                            const void *v_win_in, void *q_win_out, void *k_win_out,
                            void *v_win_out, const float *log_gate, const float *beta,
                            const float *state_in, void *o, float *state_out, int B, int H, int L,
                            int d_k, int d_v, int C, void *workspace, size_t workspace_bytes,
                            void *stream);

/*
 * Backward pass of la_chunk_fwd (training): gradients of a scalar loss with
 * respect to q, k, v, the log-gates, beta and the initial state, given d_o =
 * dLoss/do and optionally d_state_out = dLoss/d(final state). Reverse-mode of
 * the recurrence above, in its chunk form (tensorplay section 3.2; for the
 * delta rule the WY / UT chunk form of tensorplay section 6.2). The forward
 * states are recomputed from q, k, v, one per chunk, into the workspace, as in
 * the materialized form of tensorplay section 4.1.2 (per-chunk states stored,
 * recomputed for back-propagation instead of kept from the forward). With G
 * the cumulative log-gate, the loss sees the gates only through
 * q_t e^{G_t}, k_t e^{-G_t} (LA_GATED_DELTA: v_t e^{-G_t}) and e^{G_L}, so
 * d_log_gate_t = sum_{u>=t} (q_u . dq_u - k_u . dk_u) + <d_state_out, S_L>
 * (LA_GATED_DELTA: q_u . dq_u - v_u . dv_u).
 *   var          LA_PLAIN, LA_NORMALIZED, LA_DECAY, or LA_GATED_DELTA and
 *                LA_VECTOR_DECAY with dt = LA_BF16 (LA_F32: LA_ERR_UNSUPPORTED).
 *                LA_KDA has no backward (LA_ERR_UNSUPPORTED).
 *                LA_VECTOR_DECAY: the gate-difference identity holds per key
 *                channel, restarted at every chunk end c:
 *                d_log_gate_t[i] = sum_{u>=t in the chunk} (q_u[i] dq_u[i] -
 *                k_u[i] dk_u[i]) + sum_j dS_c[i][j] S_c[i][j], with S_c the state
 *                after the chunk and dS_c its gradient (tensorplay section 5.2,
 *                the per-channel form (Q (.) B)(K / B)^T); gates below -10 are
 *                taken at -10, as in la_chunk_fwd, and the gradient reported for
 *                them is the one at -10. For
 *                LA_NORMALIZED, o = n / den with n the plain output and
 *                den_t = q_t . z_t, so the output gradient splits into the plain
 *                backward of do_t / den_t and a normalizer term with
 *                g_t = -(do_t . o_t) / den_t: dq_t += g_t z_t,
 *                dk_j += sum_{t>=j} g_t q_t + d_z_out, d_z_in = sum_t g_t q_t +
 *                d_z_out (proig-chaa sections 13-14); the forward pass is rerun
 *                for o and den. It computes on fp32 operands (bf16 inputs are
 *                upcast into the workspace): at the first tokens the two terms of
 *                dq cancel to a fraction of their size, below what fp16 operands
 *                resolve at the 2e-2 bound. Shapes: d_k * d_v <= 4096, or
 *                (32, 128) and (128, 32) (else LA_ERR_UNSUPPORTED).
 *   dt           dtype of q, k, v and d_o (LA_BF16 or LA_F32); every gradient
 *                is float32.
 *   q, k, v, log_gate, beta, state_in   as given to la_chunk_fwd (log_gate
 *                [B,H,L,d_k] for LA_VECTOR_DECAY, required when L > 0; beta:
 *                LA_GATED_DELTA only, required when L > 0; log_gate optional
 *                there, NULL = DeltaNet).
 *   d_o          [B,H,L,d_v] in dt, required when L > 0.
 *   d_state_out  [B,H,d_k,d_v] float32 or NULL (zero).
 *   dq, dk       [B,H,L,d_k] float32; dv [B,H,L,d_v] float32; required when L > 0.
 *   d_log_gate   [B,H,L] float32 ([B,H,L,d_k] for LA_VECTOR_DECAY) or NULL (not
 *                computed); only with a log_gate.
 *   d_beta       [B,H,L] float32 or NULL (not computed); LA_GATED_DELTA only.
 *   d_state_in   [B,H,d_k,d_v] float32 or NULL (not written).
 *   z_in, d_z_out  [B,H,d_k] float32 or NULL (zero): the normalizer given to
 *                la_chunk_fwd and the gradient of the final normalizer
 *                (LA_NORMALIZED only).
 *   d_z_in       [B,H,d_k] float32 or NULL (not written; LA_NORMALIZED only).
 *   C            64. d_k, d_v in {32, 64, 128}.
 *   workspace    at least la_chunk_bwd_workspace_size() bytes, 256-byte aligned:
 *                per-chunk states and state gradients (operand precision), the
 *                final state and one float per token; for LA_GATED_DELTA also
 *                W, U~, A_m^T d_o (later U and dU) and T per chunk, in fp16; for
 *                LA_NORMALIZED also the forward's output in fp32, four floats
 *                per token, two d_k vectors per chunk, and for bf16 inputs fp32
 *                copies of q, k, v and d_o (its states are fp32).
 * Outputs and the workspace must not overlap any input or each other.
 */
la_status la_chunk_bwd_workspace_size(la_variant var, la_dtype dt, int B, int H, int L,
                                      int d_k, int d_v, int C, size_t *bytes);
la_status la_chunk_bwd(la_variant var, la_dtype dt, const void *q, const void *k,
                       const void *v, const float *log_gate, const float *beta,
                       const float *state_in, const float *z_in, const void *d_o,
                       const float *d_state_out, const float *d_z_out, float *dq, float *dk,
                       float *dv, float *d_log_gate, float *d_beta, float *d_state_in,
                       float *d_z_in, int B, int H, int L, int d_k, int d_v, int C,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * la_chunk_fwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The same arguments as la_chunk_fwd and the same
 * results. The delta rules' per-chunk products (LA_GATED_DELTA, LA_KDA) go to a static device array of
 * LA_NOALLOC_SCRATCH_BYTES that the library holds on every device it runs on
 * until the process ends; the call itself allocates nothing. When the whole
 * sequence's products do not fit, the sequence is run in pieces of whole
 * chunks, chained through the fp32 state (in state_out when given, else in the
 * scratch), so any L works. LA_ERR_UNSUPPORTED when one chunk of every head
 * does not fit (the workspace of a 64-token sequence plus the carried state
 * above the scratch). Calls on one device share the scratch: calls that may overlap in
 * time on one device (different streams, or host threads) race and must be
 * serialized by the caller. Other variants need no scratch and run as
 * la_chunk_fwd.
 */
#define LA_NOALLOC_SCRATCH_BYTES (64u << 20)
la_status la_chunk_fwd_noalloc(la_variant var, la_dtype dt, la_dtype o_dt, const void *q,
                               const void *k, const void *v, const float *log_gate,
                               const float *beta, const float *state_in, const float *z_in, void *o,
                               float *state_out, float *z_out, int B, int H, int L, int d_k,
                               int d_v, int C, void *stream);

/* Static string naming a status code. */
const char *la_status_str(la_status s);

/* LA_ABI_VERSION of the built library. */
int la_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
