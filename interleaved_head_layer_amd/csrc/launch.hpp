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
hipError_t launch_fold_bf16(const FoldArgs& a, hipStream_t s);  // bf16 W -> fp16 Wt
hipError_t launch_fold_f32(const FoldArgs& a, hipStream_t s);   // fp32 W -> fp32 Wt

// bf16 -> fp16 copy of X (values of N(0,1)-like inputs are exact in fp16).
hipError_t launch_cvt_bf16_f16(const uint16_t* x, void* y, int64_t n, hipStream_t s);

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
hipError_t launch_gemm_f16(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s);

// Masked attention over the stacked sequence: O = softmax_2(s) V with
// s = (q . k) already in base-2 units (the score scale is folded into Q).
struct AttnArgs {
  const void* Q;   // [B][L][H][d]
  const void* K;   // [B][L][H][d]
  const void* Vt;  // [B][H][d][L]
  float* O;        // [B][L][H][d]
  unsigned* flag;  // may be null
  int B, L, H, d, mask, window;
  float qk_scale;  // multiplies q . k (1 when folded into Q)
};
hipError_t launch_attn_f16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s);

// Unstack + collapse + concatenation:
//   out[tok][h*d + c] = sum_{h', j} R[h][h'*P + j] * Pbar[tok*P + j][h'][c]
hipError_t launch_collapse(const float* Pbar, const float* R, float* out, int ntok, int H, int P,
                           int d, hipStream_t s);

// Sets kFlagNonFinite in *flag if any of x[0..n) is not finite.
hipError_t launch_check_finite(const float* x, int64_t n, unsigned* flag, hipStream_t s);
// *flag = 0 (a one-thread fill kernel).
hipError_t launch_clear_flag(unsigned* flag, hipStream_t s);

}  // namespace iha
