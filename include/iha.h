/*
 * iha.h - C ABI of the MI355X (gfx950) library for the forward pass of
 * Interleaved Head Attention (IHA), for the gradients of the layer (iha_backward) and
 * of its attention step alone (iha_attention_backward, below).
 *
 * What is computed: Algorithm 1 of the "Interleaved Head Attention" page
 * (section 4; arXiv 2602.21371), for one layer and a batch of sequences:
 *   pseudo-head mixing   Q~_{h,j} = sum_m alpha^Q_{m,h,j} X W_Q^(m)   (same for K, V)
 *   pseudo-major stacking of the P pseudo-tokens of every token into P*N rows
 *   per-head attention   softmax(Q-bar_h K-bar_h^T / sqrt(d)) V-bar_h  over those rows
 *   collapse             O_h[t] = sum_{h'} sum_j R_{h,(h'-1)P+j} P_{h',j}[t]
 *   concatenation        X~ = [O_1, ..., O_H]
 * Attention follows the textbook chapter "Attention mechanism"
 * (faketrader.github.io/llm-from-scratch/22-attention.html): scaled dot product
 * (eq. 5.3), softmax restricted to each query's allowed set (eq. 5.11), and an
 * explicit error instead of a NaN for a valid query whose allowed set is empty
 * (section 5.3, "fully masked rows").  Biases are omitted (section 5.1), as in
 * Algorithm 1.
 *
 * Stacked order and masks.  The pseudo-tokens of token t are interleaved
 * (figure 1 of the IHA page): pseudo-token (t, j) has stacked position
 * i = t*P + j (0-based).  The mask modes are defined on i:
 *   IHA_MASK_NONE    every key is visible (Algorithm 1 as printed);
 *   IHA_MASK_CAUSAL  key i' is visible from query i iff i' <= i;
 *   IHA_MASK_WINDOW  key i' is visible iff i - window < i' <= i, with `window`
 *                    counted in stacked positions (the page's sliding window
 *                    of N/(2P); appendix C).  window < 1 leaves every row empty
 *                    and is rejected with IHA_ERR_EMPTY_ROW.
 *
 * Layouts (row-major, contiguous, 0-based):
 *   X        [B][N][D]          dtype IHA_BF16 or IHA_F32
 *   W_Q/K/V  [D][H*d]           same dtype as X; head m's projection W^(m) is
 *                               columns [m*d, (m+1)*d), d = D/H (section 3.1)
 *   alpha_*  [H][H][P] float    alpha[m][h][j]; m = source head summed over,
 *                               h = target head, j = pseudo index
 *   R        [H][H*P]  float    column h'*P + j (0-based form of (h'-1)P + j)
 *   X_out    [B][N][D] float    head h in columns [h*d, (h+1)*d)
 *
 * Precision.  IHA_F32: every step in fp32 (the mixing is folded into the
 * weights).  IHA_BF16: the per-head projections run on the bf16 matrix cores
 * with the exact bf16 inputs and fp32 accumulation, the mixing is applied to
 * those fp32 projections to fp32 accuracy (both operands split into fp16 high
 * and low parts on the matrix cores, fp32 accumulation, about 2^-21 relative;
 * shapes without a matrix-core kernel use fp32 FMAs), and the mixed Q/K/V and
 * the attention probabilities are stored as fp16 for the fp16 matrix cores (fp32
 * accumulation); softmax state, the per-head attention output and X_out are
 * fp32.  Under a causal or window mask the first 32 stacked rows of every
 * (b, h) see the fewest keys and have the largest outputs; their attention is
 * recomputed in fp32 from fp32 copies of their mixed queries, keys and values,
 * so that their absolute error matches the other rows'.
 *
 * Ownership and streams.  The caller owns every buffer; all device pointers
 * must be on the current HIP device.  The library keeps no state between
 * calls and allocates nothing: intermediate tensors live in the caller's
 * workspace.  Work is enqueued on `stream` and the call returns without
 * waiting, unless IHA_FLAG_CHECK is set.  Concurrent calls must not share a
 * workspace.
 *
 * Errors.  Argument problems are detected on the host before anything is
 * enqueued; X_out is then left untouched.  HIP launch failures give
 * IHA_ERR_DEVICE.  With IHA_FLAG_CHECK the call synchronises `stream` and
 * reports device-detected problems, in this order of precedence: an empty
 * allowed set (IHA_ERR_EMPTY_ROW), a non-finite value in X, W_*, alpha_* or R
 * (IHA_ERR_NONFINITE), an fp16 range overflow (IHA_ERR_RANGE, below), and a
 * non-finite value in X_out (IHA_ERR_NONFINITE).
 *
 * fp16 range (IHA_BF16).  The matrix-core operands are fp16, whose largest finite
 * magnitude is 65504.  Valid inputs for this path keep these within it: every
 * per-head projection X W^(m), every mixed value Q~ * log2(e)/sqrt(d), K~ and V~,
 * and every entry of alpha_* and R (the mixing and the collapse split them into
 * fp16 high and low parts).  Inputs of the pages' scale (X ~ N(0,1), W ~ N(0,1/D),
 * alpha ~ N(0,1/H)) stay four orders of magnitude inside it.  With
 * IHA_FLAG_CHECK an input that leaves it returns IHA_ERR_RANGE; without the flag
 * the call returns IHA_OK and the affected outputs of X_out are inf or NaN (the
 * library never rescales silently).  The IHA_F32 path has no such limit.
 */
#ifndef IHA_H
#define IHA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IHA_OK = 0,
  IHA_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, unknown enum */
  IHA_ERR_SHAPE = 2,        /* D not a multiple of H, or a size beyond the supported range */
  IHA_ERR_EMPTY_ROW = 3,    /* some valid query has no visible key */
  IHA_ERR_NONFINITE = 4,    /* IHA_FLAG_CHECK: a non-finite value reached the output */
  IHA_ERR_WORKSPACE = 5,    /* workspace missing or smaller than iha_workspace_bytes() */
  IHA_ERR_UNSUPPORTED = 6,  /* head width d (or H) not compiled for this dtype */
  IHA_ERR_DEVICE = 7,       /* a HIP call failed */
  IHA_ERR_RANGE = 8         /* IHA_FLAG_CHECK: an fp16 operand exceeded 65504 (see "fp16 range") */
} iha_status;

typedef enum { IHA_MASK_NONE = 0, IHA_MASK_CAUSAL = 1, IHA_MASK_WINDOW = 2 } iha_mask_mode;
typedef enum { IHA_F32 = 0, IHA_BF16 = 1 } iha_dtype;

/* Synchronise and report device-detected problems (see "Errors"). */
#define IHA_FLAG_CHECK 1u
/* IHA_BF16 only (else IHA_ERR_UNSUPPORTED): steps 4-5 of Algorithm 1 (unstack, collapse with
 * R, concatenation) run in the attention kernel's epilogue instead of a kernel of their own:
 * X_out is zeroed, then every stacked output row of head h' adds R[h][h'*P + j] times itself
 * into X_out[t][h] for every head h, with fp32 atomic additions.  The result equals the
 * default path's to rounding (the atomics' order varies, so it is not bitwise reproducible).
 * It exists to measure the fused design against the default: each attention workgroup holds
 * one head's outputs while the collapse mixes all heads of a token, so every output element
 * takes H*P atomic additions from different workgroups, and the fused forward measured
 * about 100x slower than the attention plus the separate collapse kernel. */
#define IHA_FLAG_FUSED_COLLAPSE 2u

typedef struct {
  int64_t B;       /* batch size, >= 1 */
  int64_t N;       /* tokens per sequence, >= 1 */
  int64_t D;       /* model width, multiple of H */
  int64_t H;       /* heads, 1..64 */
  int64_t P;       /* pseudo-heads per head, >= 1 */
  int64_t window;  /* IHA_MASK_WINDOW only: window in stacked positions, >= 1 */
  int32_t mask;    /* iha_mask_mode */
  int32_t dtype;   /* iha_dtype of X and W_* */
  uint32_t flags;  /* IHA_FLAG_* */
  uint32_t reserved; /* must be 0 */
} iha_problem;

/* Supported head widths d = D/H: IHA_BF16 takes 64 and 128; IHA_F32 takes
 * 16, 32, 64 and 128.  H is at most 64. */

/* Bytes of workspace iha_forward needs for this problem (written to *bytes).
 * Validates the problem like iha_forward does. */
iha_status iha_workspace_bytes(const iha_problem* prob, size_t* bytes);

/* Which kernel path iha_forward takes for this problem: IHA_PLAN_* bits written
 * to *plan (host-side only, no device work).  IHA_PLAN_MIX_FUSED: the pseudo-head
 * mixing (Algorithm 1, step 2) runs in the epilogue of the projection GEMM, so no
 * fp32 projections of all tokens reach HBM (only those of the first tokens, which
 * the attention launch mixes in fp32 for the first stacked rows) and there is no
 * separate mixing kernel (bf16 with H = 16 and D a multiple of 256, or H = 20 and
 * D a multiple of 320, and P in {1, 2}).  Validates the problem like iha_forward
 * does. */
#define IHA_PLAN_MIX_FUSED 1u
iha_status iha_plan(const iha_problem* prob, uint32_t* plan);

/* The IHA forward pass (Algorithm 1) on `stream`.
 * X, W_Q, W_K, W_V: device, dtype prob->dtype, 16-byte aligned.  alpha_*, R:
 * device float.  X_out: device float [B][N][D], 16-byte aligned.  workspace:
 * device, >= iha_workspace_bytes(), 256-byte aligned.  A misaligned X, W_*, X_out,
 * alpha_* or R returns IHA_ERR_INVALID_ARG, a misaligned workspace
 * IHA_ERR_WORKSPACE, before any launch. */
iha_status iha_forward(const iha_problem* prob, const void* X, const void* W_Q, const void* W_K,
                       const void* W_V, const float* alpha_Q, const float* alpha_K,
                       const float* alpha_V, const float* R, float* X_out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/* iha_forward that also records IHA_TIMED_EVENTS events on `stream` around its
 * steps: [0] start, [1] after the weight preparation (bf16: transpose; fp32:
 * mixing folded into the weights), [2] after the projection GEMMs, [3] after the
 * mixing (fp32 and IHA_PLAN_MIX_FUSED: no separate mixing, recorded right after
 * [2]), [4] after the attention launch (for bf16 inputs under a mask it also
 * computes the first stacked rows in fp32), [5] recorded right after [4] (kept
 * for a stable event count), [6] after the collapse.  Every event record adds a
 * gap of roughly 10 us between the kernels it separates.
 * The events are created by the caller (hipEventCreate) and must not be NULL;
 * a NULL array or entry returns IHA_ERR_INVALID_ARG before any launch. */
#define IHA_TIMED_EVENTS 7
iha_status iha_forward_timed(const iha_problem* prob, const void* X, const void* W_Q,
                             const void* W_K, const void* W_V, const float* alpha_Q,
                             const float* alpha_K, const float* alpha_V, const float* R,
                             float* X_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t* events);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): iha_forward with its workspace in a
 * buffer of IHA_STATIC_WORKSPACE_BYTES that the library holds on each device it runs on
 * (a static device array, created with the library's code object on that device and kept
 * until the process ends).  The caller passes inputs and X_out as for iha_forward; this
 * entry point allocates nothing (no hipMalloc, hipFree or allocating library call; the
 * first call on a device looks the buffer's address up once).  A problem whose
 * iha_workspace_bytes() exceeds IHA_STATIC_WORKSPACE_BYTES returns IHA_ERR_WORKSPACE
 * before any launch.  Every call on a device shares that device's buffer and it keeps the
 * last call's contents (the kernels clear what must start at zero): calls that overlap on
 * one device - from several threads, or on several streams - race and must be serialised
 * by the caller. */
#define IHA_STATIC_WORKSPACE_BYTES (64u << 20)
iha_status iha_forward_static(const iha_problem* prob, const void* X, const void* W_Q,
                              const void* W_K, const void* W_V, const float* alpha_Q,
                              const float* alpha_K, const float* alpha_V, const float* R,
                              float* X_out, hipStream_t stream);

/* The attention step alone (step 3 of Algorithm 1; textbook eq. 5.3 and 5.11),
 * for already stacked, interleaved tensors of stacked length L:
 *   Q, K   fp16 [B][L][H][d]   (row i = stacked position i)
 *   Vt     fp16 [B][H][d][L]   (values, channel-major)
 *   O      float [B][L][H][d]  O[i] = sum_{i' visible} softmax_i'(s) V[i']
 * (all four device pointers 16-byte aligned, else IHA_ERR_INVALID_ARG)
 * with scores s = (q_i . k_i') * score_scale.  The kernel works in base 2, so
 * pass score_scale = log2(e)/sqrt(d) for the textbook's softmax(QK^T/sqrt(d)).
 * mask/window as above on i.  d must be 64 or 128.  IHA_FLAG_CHECK in
 * `flags` synchronises and reports an empty row (IHA_ERR_EMPTY_ROW); that
 * needs a 256-byte device `flag_buf` (otherwise it may be NULL). */
iha_status iha_attention(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask,
                         int64_t window, float score_scale, const void* Q, const void* K,
                         const void* Vt, float* O, uint32_t flags, void* flag_buf,
                         hipStream_t stream);

/* Gradients of that attention step (the backward pass of iha_attention), by the
 * chain rule through the scaled dot product and the row softmax (textbook eq.
 * 5.3 and 5.11): for the upstream gradient dO of O = softmax(s) V with base-2
 * scores s = (q_i . k_i') * score_scale over each row's visible keys,
 *   dV = A^T dO,  dS = A * (dO V^T - rowsum(dO * O)),
 *   dQ = dS K * score_scale * ln 2,  dK = dS^T Q * score_scale * ln 2
 * (A: the probabilities; dS: the gradient of the natural-log scores).
 *   Q, K, V, dO   fp16 [B][L][H][d]   (row i = stacked position i; note that V is
 *                                     row-major here, unlike iha_attention's Vt)
 *   dQ, dK, dV    float [B][L][H][d]
 * All seven device pointers 16-byte aligned, else IHA_ERR_INVALID_ARG.  mask and
 * window as above on i; d must be 64 or 128 (IHA_ERR_UNSUPPORTED), H at most 64
 * and B at most 65535 (IHA_ERR_SHAPE), window >= 1 in window mode
 * (IHA_ERR_EMPTY_ROW).  The forward is recomputed inside (fp16 Q * score_scale,
 * fp16 O, fp32 per-row log-sum-exp) into `workspace`: device, 256-byte aligned,
 * at least iha_attention_backward_workspace() bytes, else IHA_ERR_WORKSPACE.
 * Operands of the matrix-core products are fp16 (the probabilities and dS
 * rounded to fp16), accumulation fp32.  dS = A * (dO_i . V_k - D_i) is finite in fp16
 * while |dO_i . V_k - D_i| stays below 65504 (for example every element of dO and V
 * below 14 in magnitude at d = 128, as |D_i| <= max_k |dO_i . V_k|); beyond that the gradients of the affected rows
 * become infinite, and this entry point has no checking flag (iha_backward's
 * IHA_FLAG_CHECK reports non-finite gradients).  Enqueued on `stream`, no wait. */
iha_status iha_attention_backward_workspace(int64_t B, int64_t L, int64_t H, int64_t d,
                                            size_t* bytes);
iha_status iha_attention_backward(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask,
                                  int64_t window, float score_scale, const void* Q,
                                  const void* K, const void* V, const void* dO, float* dQ,
                                  float* dK, float* dV, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Gradients of the whole layer (reverse mode through Algorithm 1 of the "Interleaved
 * Head Attention" page, section 4: projection, mixing, stacking, attention, collapse),
 * for the loss L = sum(G * X~) with X~ the output of iha_forward on the same inputs:
 *   dR[h][h'*P + j]   = sum_t G[t][h] . P-bar_{h'}[t*P + j]
 *   dP-bar_{h'}[t*P + j] = sum_h R[h][h'*P + j] G[t][h]
 *   dQ-bar, dK-bar, dV-bar: the attention step's chain rule (textbook "Attention
 *                       mechanism", eq. 5.3 and 5.11; as in iha_attention_backward)
 *   dalpha[m][h][j]   = sum_t Y_m[t] . dQ-bar_h[t*P + j]   (and for K, V)
 *   dY_m[t]           = sum_{h, j} alpha[m][h][j] dQ-bar_h[t*P + j]
 *   dW = X^T dY (per projection),  dX = sum over Q, K, V of dY W^T
 * (Y_m: head m of the projection X W; the dot products run over the d channels, the
 * sums over the B*N tokens).  Inputs as for iha_forward with dtype IHA_BF16 only (else
 * IHA_ERR_UNSUPPORTED): X [B][N][D] and W_* [D][D] bf16, alpha_* [H][H][P] and
 * R [H][H*P] float, plus the upstream gradient G float [B][N][D].  Outputs, all float
 * and caller-allocated: dX [B][N][D], dW_* [D][D], dalpha_* [H][H][P], dR [H][H*P].
 * Every pointer device memory, 16-byte aligned, else IHA_ERR_INVALID_ARG.  The limits
 * of iha_forward and iha_attention_backward apply (d = D/H of 64 or 128, P*N stacked
 * rows), and B*N must be at most 2^21 - 64 (IHA_ERR_SHAPE).  workspace: device, 256-byte
 * aligned, at least iha_backward_workspace() bytes, else IHA_ERR_WORKSPACE.
 * Precision: bf16 projections with fp32 accumulation and fp32-accurate mixing, as the forward;
 * the stacked Q~, K~, V~, dP-bar and the attention's probabilities and dS are fp16
 * matrix-core operands; the reductions over tokens run in fp32; dY enters the dW and dX
 * products as bf16 high and low parts (16 significant bits, fp32 accumulation).
 * Stacked values beyond the fp16 range become infinite: IHA_FLAG_CHECK synchronises
 * and reports that (IHA_ERR_RANGE), a non-finite input (IHA_ERR_NONFINITE) or a
 * non-finite gradient.  Without it the call is enqueued on `stream` and returns
 * without waiting. */
iha_status iha_backward_workspace(const iha_problem* prob, size_t* bytes);
iha_status iha_backward(const iha_problem* prob, const void* X, const void* W_Q,
                        const void* W_K, const void* W_V, const float* alpha_Q,
                        const float* alpha_K, const float* alpha_V, const float* R,
                        const float* G, float* dX, float* dW_Q, float* dW_K, float* dW_V,
                        float* dalpha_Q, float* dalpha_K, float* dalpha_V, float* dR,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The inner attention of the Nexus higher-order attention ("Higher-order attention
 * mechanisms" page, section 2, the refined query and key: Attention_q(X) =
 * softmax(Q Q^T / sqrt(d_k)) Q, and the same for K), per head: self-attention whose keys
 * and values are the queries themselves, on the same tiled kernel as iha_attention.
 *   Q   fp16 [B][L][H][d]  (row i = position i), 16-byte aligned
 *   O   float [B][L][H][d] O[i] = sum_{i' visible} softmax_i'(s) Q[i'], 16-byte aligned
 * with base-2 scores s = (q_i . q_i') * score_scale (pass log2(e)/sqrt(d) for the page's
 * softmax(Q Q^T / sqrt(d_k))).  mask/window select the visible positions as for
 * iha_forward (the page's formula has no mask: IHA_MASK_NONE; a causal language model
 * would pass IHA_MASK_CAUSAL).  d must be 64 or 128 (IHA_ERR_UNSUPPORTED); B*H at most
 * 65535 (IHA_ERR_SHAPE).  workspace: device, 256-byte aligned, at least
 * iha_nexus_inner_workspace() bytes (a channel-major copy of Q and the flag word), else
 * IHA_ERR_WORKSPACE.  IHA_FLAG_CHECK synchronises and reports an empty row or a
 * non-finite output.  The products run on fp16 matrix cores with fp32 accumulation (the
 * probabilities rounded to fp16), like iha_attention. */
iha_status iha_nexus_inner_workspace(int64_t B, int64_t L, int64_t H, int64_t d, size_t* bytes);
iha_status iha_nexus_inner(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask, int64_t window,
                           float score_scale, const void* Q, float* O, uint32_t flags, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* iha_status_str(iha_status status);

#ifdef __cplusplus
}
#endif
#endif /* IHA_H */
