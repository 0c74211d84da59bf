/*
 * CPU oracle for the Interleaved Head Attention (IHA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, double-precision
 * implementation used to check the HIP library.  It shares no code, header or
 * table with the HIP path, and the product never links or calls it.  Only the
 * test-suite, the smoke check and the benchmark's CPU-baseline leg load it.
 *
 * Conventions (0-based):
 *   X      [B][N][D]              input sequence
 *   W_*    [D][H*d]               head m's projection is columns [m*d, (m+1)*d)
 *   alpha  [H (m)][H (h)][P (j)]  m = source head that is summed, h = target head
 *   R      [H][H*P]               column h'*P + j
 *   out    [rows][D]              head h in columns [h*d, (h+1)*d)
 * The stacked row of pseudo-token (t, j) has the interleaved position
 * iota = t*P + j; masks are defined on iota.
 */
#ifndef IHA_ORACLE_H
#define IHA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { IHO_OK = 0, IHO_ERR_ARG = 1, IHO_ERR_EMPTY_ROW = 2, IHO_ERR_NONFINITE = 3 };
enum { IHO_MASK_NONE = 0, IHO_MASK_CAUSAL = 1, IHO_MASK_WINDOW = 2 };

/* Single-head attention with strict visibility, row by row.
 * Q [T][dk], K [S][dk], V [S][dv]; query i may read key s iff
 * allowed(qpos[i], kpos[s]) under `mask` (qpos/kpos NULL = identity).
 * O [T][dv] is written; A [T][S] (optional) receives the weights; rowsum [T]
 * (optional) receives the sum of each row's weights.  scale multiplies q.k
 * (pass 1/sqrt(dk)). */
int iho_attention(int64_t T, int64_t S, int64_t dk, int64_t dv, const double* Q, const double* K,
                  const double* V, const int64_t* qpos, const int64_t* kpos, int mask,
                  int64_t window, double scale, double* O, double* A, double* rowsum);

/* Whole IHA forward.  If `tokens` is non-NULL only the listed flat tokens
 * (b*N + t) are produced, in the listed order, into out[ntokens][D]; otherwise
 * all B*N tokens are produced into out[B*N][D].  max_rowsum_dev (optional)
 * receives max |sum_s a_s - 1| over every attention row that was evaluated.
 * nthreads <= 0 uses the OpenMP default. */
int iho_forward(int64_t B, int64_t N, int64_t D, int64_t H, int64_t P, int mask, int64_t window,
                const double* X, const double* WQ, const double* WK, const double* WV,
                const double* aQ, const double* aK, const double* aV, const double* R,
                const int64_t* tokens, int64_t ntokens, double* out, double* max_rowsum_dev,
                int nthreads);

/* Number of OpenMP threads a call with this nthreads argument uses. */
int iho_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
