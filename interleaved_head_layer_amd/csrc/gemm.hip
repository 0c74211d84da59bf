// Projection of Algorithm 1 ("Interleaved Head Attention" page, section 4) against
// the folded weights: C[M][3*P*H*d] = X[M][D] * Wt^T, M = B*N tokens.
// Written straight into the layouts the attention step reads:
//   Q~, K~ : [B][P*N][H][d] fp16 (stacked row t*P + j)  -- columns (j, h, c)
//   V~^T   : [B][H][d][P*N] fp16 (channel-major)         -- columns (h, c, j)
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// ---------------------------------------------------------------- fp16 matrix-core GEMM
constexpr int GBM = 128;          // tile rows (tokens)
constexpr int GBN = 128;          // tile columns (folded features)
constexpr int GBK = 64;           // contraction slice per stage
constexpr int GLD = GBK + 8;      // LDS row stride (halves) of the operand tiles
constexpr int GCLD = GBN + 8;     // LDS row stride (halves) of the output tile
constexpr int GThreads = 256;     // 4 waves as 2 x 2, each owning 64 x 64 of C

struct GemmSmem {
  union {
    struct {
      half_t a[GBM * GLD];
      half_t b[GBN * GLD];
    } op;
    half_t c[GBM * GCLD];
  };
};

__device__ __forceinline__ void gemm_load_tile(const half_t* __restrict__ A,
                                               const half_t* __restrict__ Bt, int M, int Ncol,
                                               int K, int m0, int n0, int k0, uint4 (&ra)[4],
                                               uint4 (&rb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = tid / 8 + 32 * p;
    const int ch = tid % 8;
    const int gm = m0 + row;
    const int gn = n0 + row;
    ra[p] = (gm < M) ? *reinterpret_cast<const uint4*>(A + static_cast<int64_t>(gm) * K + k0 + ch * 8)
                     : make_uint4(0, 0, 0, 0);
    rb[p] = (gn < Ncol)
                ? *reinterpret_cast<const uint4*>(Bt + static_cast<int64_t>(gn) * K + k0 + ch * 8)
                : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void gemm_store_tile(GemmSmem& sm, const uint4 (&ra)[4],
                                                const uint4 (&rb)[4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = tid / 8 + 32 * p;
    const int ch = tid % 8;
    *reinterpret_cast<uint4*>(&sm.op.a[row * GLD + ch * 8]) = ra[p];
    *reinterpret_cast<uint4*>(&sm.op.b[row * GLD + ch * 8]) = rb[p];
  }
}

__global__ __launch_bounds__(GThreads, 2) void gemm_qkv_f16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  const half_t* __restrict__ A = static_cast<const half_t*>(g.A);
  const half_t* __restrict__ Bt = static_cast<const half_t*>(g.Bt);
  const int M = g.M, K = g.Kdim, Ncol = g.Ncol;
  const int ntn = (Ncol + GBN - 1) / GBN;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tm = lid / ntn, tn = lid % ntn;
  const int m0 = tm * GBM, n0 = tn * GBN;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[4], rb[4];
  gemm_load_tile(A, Bt, M, Ncol, K, m0, n0, 0, ra, rb);
  gemm_store_tile(sm, ra, rb);
  __syncthreads();

  const int nk = K / GBK;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gemm_load_tile(A, Bt, M, Ncol, K, m0, n0, (kt + 1) * GBK, ra, rb);
#pragma unroll
    for (int s = 0; s < GBK / 16; ++s) {
      half8 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8*>(&sm.op.a[(wm * 64 + i * 32 + l32) * GLD + s * 16 + 8 * hf]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8*>(&sm.op.b[(wn * 64 + j * 32 + l32) * GLD + s * 16 + 8 * hf]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      gemm_store_tile(sm, ra, rb);
      __syncthreads();
    }
  }

  // Epilogue: C tile -> LDS as fp16, then stores shaped for each destination.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const int col = wn * 64 + j * 32 + l32;
        sm.c[row * GCLD + col] = static_cast<half_t>(acc[i][j][r]);
      }
  __syncthreads();

  const int PHd = g.PHd, P = g.P, H = g.H, d = g.d, Ntok = g.Ntok;
  const int L = P * Ntok;
  half_t* Qo = static_cast<half_t*>(g.Q);
  half_t* Ko = static_cast<half_t*>(g.K);
  half_t* Vt = static_cast<half_t*>(g.Vt);

  // Q and K: 8-column chunks (16 bytes), 16 chunks per tile row.
  for (int idx = tid; idx < GBM * (GBN / 8); idx += GThreads) {
    const int row = idx / (GBN / 8);
    const int c8 = idx % (GBN / 8);
    const int gm = m0 + row;
    const int gc = n0 + c8 * 8;
    if (gm >= M || gc >= Ncol) continue;
    const int which = gc / PHd;   // chunks never straddle: PHd is a multiple of 64
    if (which >= 2) continue;
    half_t* dst = (which == 0 ? Qo : Ko) + static_cast<int64_t>(gm) * PHd + (gc - which * PHd);
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&sm.c[row * GCLD + c8 * 8]);
  }
  // V^T: lanes run along tokens for one column; element (t, j) goes to row t*P + j.
  if (n0 + GBN > 2 * PHd) {
    for (int idx = tid; idx < GBM * GBN; idx += GThreads) {
      const int col = idx / GBM;
      const int row = idx % GBM;
      const int gm = m0 + row;
      const int gc = n0 + col;
      if (gm >= M || gc >= Ncol || gc < 2 * PHd) continue;
      const int v = gc - 2 * PHd;
      const int h = v / (d * P);
      const int c = (v / P) % d;
      const int j = v % P;
      const int b = gm / Ntok;
      const int t = gm % Ntok;
      Vt[(static_cast<int64_t>(b * H + h) * d + c) * L + static_cast<int64_t>(t) * P + j] =
          sm.c[row * GCLD + col];
    }
  }
}

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

hipError_t launch_gemm_f16(const GemmArgs& g, hipStream_t s) {
  const int ntm = (g.M + GBM - 1) / GBM;
  const int ntn = (g.Ncol + GBN - 1) / GBN;
  hipLaunchKernelGGL(gemm_qkv_f16_kernel, dim3(ntm * ntn), dim3(GThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  const dim3 grid((g.Ncol + FBN - 1) / FBN, (g.M + FBM - 1) / FBM);
  hipLaunchKernelGGL(gemm_qkv_f32_kernel, grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace iha
