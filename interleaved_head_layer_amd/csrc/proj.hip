// Steps 1-2 of Algorithm 1 ("Interleaved Head Attention" page, section 4) for bf16 inputs:
// the per-head projections X W^(m) as exact bf16 matrix-core GEMMs with fp32 accumulation,
// followed by the pseudo-head mixing Q~_{h,j} = sum_m alpha^Q_{m,h,j} (X W_Q^(m)) in fp32,
// written straight into the stacked layouts the attention step reads.
//
//   wprep   Wt[which*D + n][k] = W_which[k][n]            (bf16, the contraction index k
//                                                          contiguous for the matrix cores)
//   gemm    Y_QK [M][2D]  = X Wt_{Q,K}^T  (token-major)    fp32
//           Y_V^T [D][M]  = Wt_V X^T      (channel-major)  fp32
//   mix_qk  Q~, K~ [B][P*N][H][d] fp16, rows t*P + j
//   mix_v   V~^T  [B][H][d][P*N]  fp16
// The first T0 tokens of every sequence also get fp32 copies (Qe, Ke, Vte) for the
// full-precision first rows.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------- W transpose
// grid: (D/64, D/64, 3); block 256.  64x64 tiles through LDS.
__global__ __launch_bounds__(256) void wprep_kernel(ProjArgs pa) {
  __shared__ uint16_t t[64][65];
  const int which = blockIdx.z;
  const uint16_t* __restrict__ W = pa.W[which];
  const int D = pa.D;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tx = threadIdx.x % 64, ty = threadIdx.x / 64;
  for (int r = ty; r < 64; r += 4) t[r][tx] = W[static_cast<int64_t>(k0 + r) * D + n0 + tx];
  __syncthreads();
  uint16_t* __restrict__ Wt = pa.Wt + static_cast<int64_t>(which) * D * D;
  for (int r = ty; r < 64; r += 4) Wt[static_cast<int64_t>(n0 + r) * D + k0 + tx] = t[tx][r];
}

// ------------------------------------------------------------------- NT GEMM
// C[i][j] = sum_k A[i][k] * B[j][k]; A [I][K], B [J][K] bf16 (k contiguous), C fp32 with
// row stride ldc.  128 x 128 tiles, K slices of 64, 4 waves as 2 x 2 (64 x 64 each).
// Operand slices go global -> LDS directly into a two-stage ring; 128-byte rows with
// 16-byte chunks XOR-swizzled by (row >> 1) & 7 so 16 lanes reading 16 rows hit 16
// bank groups.  Rows past I / J load a clamped valid row; their results are not stored.
constexpr int GT = 128, GK = 64;

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

struct NtSmem {
  uint16_t a[2][GT * GK];
  uint16_t b[2][GT * GK];
};

__device__ __forceinline__ void nt_issue(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                         int I, int J, int K, int i0, int j0, int k0, uint16_t* as,
                                         uint16_t* bs) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // 128 rows x 128 bytes = 16 KB = 4 rounds of 256 x 16 bytes
    const int slot = (p * 4 + w) * 64 + lane;
    const int r = slot / 8, pos = slot % 8;
    const int c = pos ^ gswz(r);
    const uint16_t* sa = A + static_cast<int64_t>(min(i0 + r, I - 1)) * K + k0 + c * 8;
    const uint16_t* sb = B + static_cast<int64_t>(min(j0 + r, J - 1)) * K + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(sa, (__attribute__((address_space(3))) void*)(as + (p * 4 + w) * 512), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(sb, (__attribute__((address_space(3))) void*)(bs + (p * 4 + w) * 512), 16, 0, 0);
  }
}

__global__ __launch_bounds__(256, 2) void gemm_nt_bf16_kernel(NtArgs g) {
  __shared__ __attribute__((aligned(16))) NtSmem sm;
  const uint16_t* __restrict__ A = g.A;
  const uint16_t* __restrict__ B = g.B;
  const int I = g.I, J = g.J, K = g.K;
  const int ntj = (J + GT - 1) / GT;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  // Groups of 8 row tiles sweep the column tiles, so a group's A slices stay in L2.
  const int nti = (I + GT - 1) / GT;
  const int group = lid / (8 * ntj);
  const int first_i = group * 8;
  const int gsize = min(8, nti - first_i);
  const int ti = first_i + (lid % (8 * ntj)) % gsize;
  const int tj = (lid % (8 * ntj)) / gsize;
  const int i0 = ti * GT, j0 = tj * GT;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / GK;
  nt_issue(A, B, I, J, K, i0, j0, 0, sm.a[0], sm.b[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) nt_issue(A, B, I, J, K, i0, j0, (kt + 1) * GK, sm.a[st ^ 1], sm.b[st ^ 1]);
#pragma unroll
    for (int s = 0; s < GK / 16; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + l32;
        af[i] = *reinterpret_cast<const bf16x8*>(&sm.a[st][r * GK + ((s * 2 + hf) ^ gswz(r)) * 8]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + l32;
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sm.b[st][r * GK + ((s * 2 + hf) ^ gswz(r)) * 8]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  // Lane l holds C[8*(r/4) + 4*hf + r%4][l%32] of each 32x32 block.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = j0 + wn * 64 + j * 32 + l32;
      if (col >= J) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = i0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row < I) g.C[static_cast<int64_t>(row) * g.ldc + col] = acc[i][j][r];
      }
    }
}

// ------------------------------------------------------------------- mixing
// One thread owns one (token, channel c): it loads the H source values y_m once and writes
// all H*P outputs  out[h][j] = sum_m alpha[m][h][j] * y_m  (fp32 arithmetic).  The block
// first stages alpha transposed to [h][j][m] in LDS, zero-padded to HMAX source heads, so the
// inner loop is branch-free FMAs on broadcast LDS reads.
template <int HMAX>
__device__ __forceinline__ void stage_alpha(const float* __restrict__ alpha, int H, int P, float* as) {
  for (int e = threadIdx.x; e < H * P * HMAX; e += 256) {
    const int m = e % HMAX, hj = e / HMAX;  // hj = h * P + j
    as[e] = m < H ? alpha[m * H * P + hj] : 0.f;
  }
  __syncthreads();
}

template <int HMAX>
__device__ __forceinline__ float mix_one(const float* as_hj, const float (&ym)[HMAX]) {
  float acc = 0.f;
#pragma unroll
  for (int m = 0; m < HMAX; m += 4) {
    const floatx4 a4 = *reinterpret_cast<const floatx4*>(as_hj + m);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = fmaf(a4[q], ym[m + q], acc);
  }
  return acc;
}

// Q~/K~ (token-major Y, lanes along c): grid (ceil(M*d / 256), 2); stores coalesced along c.
template <int HMAX>
__global__ __launch_bounds__(256) void mix_qk_kernel(ProjArgs pa) {
  extern __shared__ float as[];
  const int which = blockIdx.y;
  const int D = pa.D, d = pa.d, H = pa.H, P = pa.P, N = pa.N;
  stage_alpha<HMAX>(pa.alpha[which], H, P, as);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(pa.B) * N * d) return;
  const int tok = static_cast<int>(e / d), c = static_cast<int>(e % d);
  const float* __restrict__ y = pa.Yqk + static_cast<int64_t>(tok) * 2 * D + which * D + c;
  half_t* __restrict__ out = (which == 0 ? pa.Q : pa.K) + static_cast<int64_t>(tok) * P * D + c;
  float* __restrict__ oute = which == 0 ? pa.Qe : pa.Ke;
  const int b = tok / N, t = tok % N;
  float ym[HMAX];
#pragma unroll
  for (int m = 0; m < HMAX; ++m) ym[m] = y[(m < H ? m : 0) * d];
  for (int h = 0; h < H; ++h)
    for (int j = 0; j < P; ++j) {
      const float acc = mix_one<HMAX>(as + (h * P + j) * HMAX, ym);
      out[static_cast<int64_t>(j) * D + h * d] = static_cast<half_t>(acc);
      const int i = t * P + j;
      if (oute && i < pa.R) oute[(static_cast<int64_t>(b) * pa.R + i) * D + h * d + c] = acc;
    }
}

// V~^T (channel-major Y, lanes along tokens): grid (ceil(M / 256), d); stores coalesced
// along t*P + j.
template <int HMAX>
__global__ __launch_bounds__(256) void mix_v_kernel(ProjArgs pa) {
  extern __shared__ float as[];
  const int c = blockIdx.y;
  const int M = pa.B * pa.N, d = pa.d, H = pa.H, P = pa.P, N = pa.N;
  stage_alpha<HMAX>(pa.alpha[2], H, P, as);
  const int tok = blockIdx.x * 256 + threadIdx.x;
  if (tok >= M) return;
  const int b = tok / N, t = tok % N;
  const int64_t L = static_cast<int64_t>(P) * N;
  float ym[HMAX];
#pragma unroll
  for (int m = 0; m < HMAX; ++m) ym[m] = pa.Yvt[static_cast<int64_t>((m < H ? m : 0) * d + c) * M + tok];
  for (int h = 0; h < H; ++h) {
    half_t* __restrict__ vrow = pa.Vt + (static_cast<int64_t>(b * H + h) * d + c) * L + static_cast<int64_t>(t) * P;
    float* __restrict__ erow = pa.Vte ? pa.Vte + (static_cast<int64_t>(b * H + h) * d + c) * pa.R : nullptr;
    for (int j = 0; j < P; ++j) {
      const float acc = mix_one<HMAX>(as + (h * P + j) * HMAX, ym);
      vrow[j] = static_cast<half_t>(acc);
      const int i = t * P + j;
      if (erow && i < pa.R) erow[i] = acc;
    }
  }
}

template <int HMAX>
void launch_mix(const ProjArgs& pa, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(pa.B) * pa.N;
  const size_t lds = static_cast<size_t>(pa.H) * pa.P * HMAX * sizeof(float);
  hipLaunchKernelGGL((mix_qk_kernel<HMAX>), dim3(static_cast<unsigned>((M * pa.d + 255) / 256), 2), dim3(256), lds, s, pa);
  hipLaunchKernelGGL((mix_v_kernel<HMAX>), dim3(static_cast<unsigned>((M + 255) / 256), pa.d), dim3(256), lds, s, pa);
}

}  // namespace

hipError_t launch_proj_bf16(const ProjArgs& pa, hipStream_t s, hipEvent_t ev_prep) {
  const int D = pa.D, M = pa.B * pa.N;
  hipLaunchKernelGGL(wprep_kernel, dim3(D / 64, D / 64, 3), dim3(256), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_prep && (e = hipEventRecord(ev_prep, s)) != hipSuccess) return e;
  NtArgs g1{};  // Y_QK = X * Wt_QK^T
  g1.A = pa.X;
  g1.B = pa.Wt;
  g1.C = pa.Yqk;
  g1.I = M;
  g1.J = 2 * D;
  g1.K = D;
  g1.ldc = 2 * D;
  const int t1 = ((g1.I + GT - 1) / GT) * ((g1.J + GT - 1) / GT);
  hipLaunchKernelGGL(gemm_nt_bf16_kernel, dim3(t1), dim3(256), 0, s, g1);
  NtArgs g2{};  // Y_V^T = Wt_V * X^T
  g2.A = pa.Wt + static_cast<int64_t>(2) * D * D;
  g2.B = pa.X;
  g2.C = pa.Yvt;
  g2.I = D;
  g2.J = M;
  g2.K = D;
  g2.ldc = M;
  const int t2 = ((g2.I + GT - 1) / GT) * ((g2.J + GT - 1) / GT);
  hipLaunchKernelGGL(gemm_nt_bf16_kernel, dim3(t2), dim3(256), 0, s, g2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pa.H <= 4) launch_mix<4>(pa, s);
  else if (pa.H <= 8) launch_mix<8>(pa, s);
  else if (pa.H <= 16) launch_mix<16>(pa, s);
  else if (pa.H <= 20) launch_mix<20>(pa, s);
  else if (pa.H <= 32) launch_mix<32>(pa, s);
  else launch_mix<64>(pa, s);
  return hipGetLastError();
}

}  // namespace iha
