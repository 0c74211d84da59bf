// Host-side launchers of the IHA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iha {

// Pseudo-head mixing folded into the weights (linearity of Algorithm 1's mixing):
//   Wt[which*PHd + col(h, j, c)][k] = out_scale[which] * sum_m alpha_which[m][h][j] * W_which[k][m*d + c]
// Q/K columns are ordered (j, h, c); V columns (h, c, j).  Wt is [3*P*H*d][D]
// (the contraction index k contiguous).  Also clears the device flag word.
struct FoldArgs {
  const void* W[3];
  const float* alpha[3];
  float out_scale[3];
  void* Wt;
  unsigned* flag;
  int D, H, d, P;
};
hipError_t launch_fold_f32(const FoldArgs& a, hipStream_t s);   // fp32 W -> fp32 Wt (fp32 inputs)

// Projection GEMM C[M][3*PHd] = X[M][D] * Wt^T, written as
//   Q, K : [B][P*N][H][d] (stacked row t*P + j),  Vt : [B][H][d][P*N].
struct GemmArgs {
  const void* A;   // [M][K]
  const void* Bt;  // [Ncol][K]
  void* Q;
  void* K;
  void* Vt;
  int M, Kdim, Ncol, PHd, Ntok, P, H, d;
};
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);

// Layouts of Q and K for the fp16 attention kernel.
constexpr int kQKRowMajor = 0;  // [B][L][H][d]
constexpr int kQKChunked = 1;   // [B][H][d/8][L][8]: 16-byte d-chunks, contiguous over rows

// bf16 inputs under a causal or window mask: the first kPreciseRows stacked rows of every
// (b, h) see the fewest keys and have the largest outputs; they are computed again in fp32.
constexpr int kPreciseRows = 32;
// ... and their outputs, up to stacked row kF32OutRows of every (b, h), stay fp32 (the fp16
// rounding of an output is a quarter of its error; outputs of rows with few keys are large).
constexpr int kF32OutRows = 1024;

// Masked attention over the stacked sequence: O = softmax_2(s) V with base-2 scores
// s = (q . k) * qk_scale.
struct AttnArgs {
  const void* Q;   // [B][L][H][d] or chunked (qk_layout; fp16 kernel only)
  const void* K;   // same layout as Q
  const void* Vt;  // [B][H][d][L]
  float* O;        // [B][L][H][d] fp32, or null with Oh
  half_t* Oh;      // fp16 kernel only: [B][L][H][d] fp16 output instead of O (may be null)
  unsigned* flag;  // may be null
  int B, L, H, d, mask, window;
  float qk_scale;     // multiplies q . k to give base-2 scores
  int64_t o_bstride;  // elements between batches of O (0: L*H*d)
  int qk_layout;      // kQKRowMajor or kQKChunked
  // fp16 kernel, causal or window mask, R > 0: B*H extra workgroups of the same launch
  // compute the first R (<= kPreciseRows) stacked rows of every (b, h) in fp32 into Pe
  // [B][R][H][d] (base-2 scores scaled by escale), from fp32 copies Qe, Ke, Ve [B][R][H][d]
  // or, when Ye is set, from the unmixed fp32 projections Ye [B][T0][3D] of the first
  // T0 = ceil(R / P) tokens (fused row order, H = 16 or 20) mixed here with alpha[3].
  const float* Qe;
  const float* Ke;
  const float* Ve;
  const float* Ye;
  const float* alpha[3];
  float* Pe;       // [B][R2][H][d] fp32: rows < R from the fp32 recomputation, rows R..R2-1
                   // from the tiled kernel (fp32 instead of fp16)
  int R, P, T0;
  int R2;          // R <= R2 <= L
  float escale;
  // fp16 kernel: when set, [B][H][L] base-2 log-sum-exp of every row's visible scores
  // (the row's probabilities are exp2(score - lse)); +inf for a row with no visible key.
  float* lse;
  // fp16 kernel, fused collapse (when set): X~ [B][L/P][H*d] fp32, zeroed beforehand; every
  // output row i = t*P + j of head h adds Rm[hh][h*P + j] * O[i] into X~[t][hh*d ..] for every
  // head hh (fp32 atomics) instead of being stored; rows < R from the fp32 first-row
  // workgroups.  Needs P.
  float* Xf;
  const float* Rm;  // R [H][H*P]
};
hipError_t launch_attn_f16(const AttnArgs& a, hipStream_t s);
// p[0..n) = 0 (n a multiple of 4, p 16-byte aligned); a kernel, so that it may be captured.
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);

// Attention backward over stacked rows (fp16 operands, fp32 gradients).  Inputs Q, K, V, dO
// and outputs dQ, dK, dV are row-major [B][L][H][d]; the rest is workspace the launcher fills:
// Qs = fp16(Q * scale) [B][L][H][d], channel-major QsT, KT, dOT [B][H][d][Lp] (Lp: L rounded
// up to 64, zero padded) and VT [B][H][d][L], the recomputed forward output O (fp16,
// [B][L][H][d]), and per-row lse (base 2) and D = dO . O, [B][H][L] fp32.
struct AttnBwdArgs {
  const half_t* Q;
  const half_t* K;
  const half_t* V;
  const half_t* dO;
  float* dQ;
  float* dK;
  float* dV;
  half_t* Qs;
  half_t* QsT;
  half_t* KT;
  half_t* dOT;
  half_t* VT;
  half_t* O;
  float* lse;
  float* D;
  int B, L, H, d, mask, window, Lp;
  float scale;     // base-2 score scale
  float dq_scale;  // scale * ln 2
  float dk_scale;  // ln 2 (dK is formed from the scaled Q)
};
hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s);

// Q [B][L][H][d] fp16 -> Qt [B][H][d][L] fp16 (channel-major copy; d a multiple of 64).
hipError_t launch_transpose_rows(const half_t* Q, half_t* Qt, int B, int L, int H, int d, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// bf16 projection path: exact bf16 GEMMs (fp32 accumulation) then fp32 mixing.
struct NtArgs {
  const uint16_t* A;  // [I][K] bf16
  const uint16_t* B;  // [J][K] bf16
  float* C;           // [I][ldc] fp32
  int I, J, K;
  int64_t ldc;
  int jbase;          // fused mixing: global token of B's row 0 (the launcher splits tokens)
  // launch_gemm_nt_batched: product z (blockIdx.y) reads A + z*sa, B + z*sb, writes Cz[z].
  int64_t sa, sb;
  float* Cz[3];
  int ks;  // row stride of A and B in elements (0: K); a split-K launch reads K-wide column slices
};
struct ProjArgs {
  const uint16_t* X;      // [B*N][D] bf16
  const uint16_t* W[3];   // [D][D] bf16 (Q, K, V)
  const float* alpha[3];  // [H][H][P]
  uint16_t* Wt;           // [3D][D] bf16 scratch
  float* Yqk;             // [B*N][2D] fp32 scratch
  float* Yvt;             // [D][B*N] fp32 scratch
  half_t* Q;              // [B][P*N][H][d] fp16, multiplied by qscale
  half_t* K;
  half_t* Vt;             // [B][H][d][P*N] fp16
  float* Qe;              // unfused path: fp32 copies of the first R stacked rows (or null)
  float* Ke;
  float* Ve;
  float* Ye;              // fused path: [B][T0][3D] unmixed fp32 projections of the first
                          // T0 tokens (rows as permuted by fused_row), or null
  int B, N, D, H, d, P, R;
  int T0;                 // ceil(R / P): tokens whose pseudo-tokens include a first row
  float qscale;           // factor applied to the fp16 Q (the base-2 score scale)
  unsigned* flag;         // status word, cleared by the first kernel (may be null)
  int ywidth;             // projected matrices per token row of Yqk (0: 2, Q and K)
  half_t* Vrow;           // launch_proj_rowmajor: V~ [B][P*N][H][d] fp16 (row-major)
};
// With P = 4 the fused epilogue writes four stacked outputs per projected value and its
// stores no longer hide behind the products (measured: slower than GEMM + mixing), so the
// fused path stops at P = 2.
inline bool fused_shape(int64_t H, int64_t D, int64_t P) {
  return ((H == 16 && D % 256 == 0) || (H == 20 && D % 320 == 0)) && (P == 1 || P == 2);
}
// True when the projection runs fused with the mixing (H = 16 with D % 256 == 0 or H = 20
// with D % 320 == 0, P in {1,2});
// Q~ and K~ are then written in the chunked layout [B][H][d/8][P*N][8], else row-major.
bool proj_fused(const ProjArgs& pa);
// ev_prep (may be null) is recorded after the weight transpose, ev_gemm after the projection
// GEMMs (with the fused path: after the fused kernel, the mixing included).
hipError_t launch_proj_bf16(const ProjArgs& pa, hipStream_t s, hipEvent_t ev_prep, hipEvent_t ev_gemm);
// Projections and mixing for the backward pass: W transposed into Wt, Y = X [Wt_Q; Wt_K;
// Wt_V]^T into Yqk ([B*N][3D] fp32, kept: the mixing gradient needs it), and the mixed Q~, K~,
// V~ row-major into Q, K, Vrow ([B][P*N][H][d] fp16, Q~ times qscale).  R must be 0.
hipError_t launch_proj_rowmajor(ProjArgs pa, hipStream_t s);
// C[I][ldc] = A[I][K] B[J][K]^T, bf16 operands (K a multiple of 64), fp32 result.
hipError_t launch_gemm_nt_bf16(const NtArgs& g, hipStream_t s);
// `batch` (<= 3) such products of one shape in one launch: product z takes A + z*sa and
// B + z*sb and writes Cz[z] (g.C unused); one product after another where the shape needs the
// launcher's 2 GiB split.
hipError_t launch_gemm_nt_batched(const NtArgs& g, int batch, hipStream_t s);
// The same `batch` products with the contracted dimension g.K split into `splits` equal parts
// (g.K / splits a multiple of 64): part p of product z goes to Cs + (p*batch + z)*I*ldc, then a
// second kernel adds the parts in order into Cz[z].  Cs holds splits*batch*I*ldc floats.
hipError_t launch_gemm_nt_splitk(const NtArgs& g, int batch, int splits, float* Cs, hipStream_t s);
// The gradient of the collapse with respect to the stacked outputs:
//   out[b][t*P + j][h'][c] = sum_h R[h][h'*P + j] * G[b][t][h*d + c]
// G fp32 [B*N][H*d] (16-byte aligned), out fp16 [B][N*P][H][d].
hipError_t launch_expand(const float* G, const float* Rm, half_t* out, int B, int N, int H, int P, int d,
                         hipStream_t s);

// Token reduction of the mixing and collapse gradients:
//   out[a][h*P + j] = sum_t sum_c A[t*lda + a*d + c] * Bm[((t*P + j)*H + h)*d + c]
// over ntok tokens; A fp32, Bm fp32 or fp16 (b_half).  Per-chunk partial sums go to `part`
// (head_reduce_part_bytes() bytes), then a second kernel adds them in a fixed order.
size_t head_reduce_part_bytes(int ntok, int H, int P);
hipError_t launch_head_reduce(const float* A, int64_t lda, const void* Bm, bool b_half, float* out, float* part,
                              int ntok, int H, int P, int d, hipStream_t s);
// dst[r*ldd + c] = hi = bf16(src[r*lds + c]) for r < nr, c < nc (nc a multiple of 4), src
// fp32; dst_lo (may be null) gets bf16(src - hi) at the same offsets.
hipError_t launch_to_bf16(const float* src, int64_t lds, int nr, int nc, uint16_t* dst, uint16_t* dst_lo, int64_t ldd,
                          hipStream_t s);
// dst[c*ldd + r] = bf16(src[r*lds + c]) for c < nc and r < nr_out, zero for r >= nr; src fp32
// (src_bf16 false) or bf16 bits; dst_lo (may be null) as above.  nr <= nr_out <= ldd, nr_out a
// multiple of 64.
hipError_t launch_to_bf16_t(const void* src, bool src_bf16, int64_t lds, int nr, int nc, uint16_t* dst,
                            uint16_t* dst_lo, int64_t ldd, int64_t nr_out, hipStream_t s);
// dst[r*ldd + c] = src[r*lds + c], bf16 bits, for r < nr, c < nc (nc a multiple of 8).
hipError_t launch_copy_bf16(const uint16_t* src, int64_t lds, int nr, int nc, uint16_t* dst, int64_t ldd,
                            hipStream_t s);


// Unstack + collapse + concatenation:
//   out[tok][h*d + c] = sum_{h', j} R[h][h'*P + j] * Pbar[tok*P + j][h'][c]
// Collapse from fp16 stacked outputs Ph [B*N*P][H][d] whose first R stacked rows of every
// sequence come instead from the fp32 rows Pe [B][R][H][d].
hipError_t launch_collapse_h(const half_t* Ph, const float* Pe, int R, const float* Rm, float* out, int B,
                             int N, int H, int P, int d, hipStream_t s);
hipError_t launch_collapse(const float* Pbar, const float* R, float* out, int ntok, int H, int P,
                           int d, hipStream_t s);

// Scans x[0..n) (kind: kValF32, kValBF16 or kValF16 elements): sets `nonfinite_bit` in *flag
// if an element is not finite, and kFlagRange if a finite one exceeds `limit` in magnitude.
constexpr int kValF32 = 0;
constexpr int kValBF16 = 1;
constexpr int kValF16 = 2;
hipError_t launch_check_values(const void* x, int kind, int64_t n, unsigned* flag, unsigned nonfinite_bit,
                               float limit, hipStream_t s);
// *flag = 0 (a one-thread fill kernel).
hipError_t launch_clear_flag(unsigned* flag, hipStream_t s);

}  // namespace iha
