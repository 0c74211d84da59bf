// Projection of Algorithm 1 ("Interleaved Head Attention" page, section 4) against the
// folded weights for fp32 inputs: C[M][3*P*H*d] = X[M][D] * Wt^T, M = B*N tokens, written
// straight into the layouts the attention step reads:
//   Q~, K~ : [B][P*N][H][d] (stacked row t*P + j)  -- columns (j, h, c)
//   V~^T   : [B][H][d][P*N] (channel-major)         -- columns (h, c, j)
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// ---------------------------------------------------------------- fp32 GEMM (VALU)
constexpr int FBM = 64, FBN = 64, FBK = 16;

__global__ __launch_bounds__(256) void gemm_qkv_f32_kernel(GemmArgs g) {
  __shared__ float As[FBK][FBM + 4];
  __shared__ float Bs[FBK][FBN + 4];
  const float* __restrict__ A = static_cast<const float*>(g.A);
  const float* __restrict__ Bt = static_cast<const float*>(g.Bt);
  const int M = g.M, K = g.Kdim, Ncol = g.Ncol;
  const int m0 = blockIdx.y * FBM, n0 = blockIdx.x * FBN;
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += FBK) {
    for (int e = tid; e < FBM * FBK; e += 256) {
      const int r = e / FBK, kk = e % FBK;
      const int gm = m0 + r, gn = n0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[static_cast<int64_t>(gm) * K + gk] : 0.f;
      Bs[kk][r] = (gn < Ncol && gk < K) ? Bt[static_cast<int64_t>(gn) * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int PHd = g.PHd, P = g.P, H = g.H, d = g.d, Ntok = g.Ntok;
  const int L = P * Ntok;
  float* Qo = static_cast<float*>(g.Q);
  float* Ko = static_cast<float*>(g.K);
  float* Vt = static_cast<float*>(g.Vt);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + ty * 4 + i, gc = n0 + tx * 4 + j;
      if (gm >= M || gc >= Ncol) continue;
      const int which = gc / PHd;
      if (which < 2) {
        (which == 0 ? Qo : Ko)[static_cast<int64_t>(gm) * PHd + (gc - which * PHd)] = acc[i][j];
      } else {
        const int v = gc - 2 * PHd;
        const int h = v / (d * P), c = (v / P) % d, jj = v % P;
        const int b = gm / Ntok, t = gm % Ntok;
        Vt[(static_cast<int64_t>(b * H + h) * d + c) * L + static_cast<int64_t>(t) * P + jj] = acc[i][j];
      }
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((g.Ncol + FBN - 1) / FBN, (g.M + FBM - 1) / FBM);
  hipLaunchKernelGGL(gemm_qkv_f32_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace iha
