// Full-precision path for the first stacked rows of every (b, h) under a causal or window
// mask (bf16 inputs).
//
// Why: a stacked row that sees n keys has an output of magnitude about n^-1/2 (it averages
// n value rows with softmax weights), while the fp16 intermediates of the main path carry a
// fixed relative error.  The first rows see only a handful of keys, so their outputs, and
// their absolute errors, are far above the typical output; the output error bound is set
// by them.  These rows (the first 128, one query tile) are recomputed here with fp32
// intermediates throughout: the projection of the first ceil(128/P) tokens runs unfolded
// on the exact bf16 inputs (bf16 matrix cores, fp32 accumulation), the mixing of
// Algorithm 1 is applied in fp32, and attention runs in fp32.  The result overwrites those
// rows of P-bar after the main attention kernel.  Every later row sees more than 128 keys.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int EBM = 128, EBN = 128, EBK = 64;
constexpr int ELD = EBK + 8;

// Y[r][which*D + n] = sum_k X[b][t][k] * W_which[k][n], r = b*T0 + t, t < T0.
// grid: (ceil(D / 128), ceil(B*T0 / 128), 3); block 256 = 4 waves as 2 x 2 of 64 x 64.
__global__ __launch_bounds__(256) void early_proj_kernel(EarlyArgs e) {
  __shared__ __attribute__((aligned(16))) uint16_t As[EBM * ELD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[EBN * ELD];  // [n][k]
  const int which = blockIdx.z;
  const uint16_t* __restrict__ W = e.W[which];
  const int D = e.D, M = e.B * e.T0;
  const int m0 = blockIdx.y * EBM, n0 = blockIdx.x * EBN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;

  floatx16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int k0 = 0; k0 < D; k0 += EBK) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // A: 128 rows x 64 k, 16-byte chunks.
      const int row = tid / 8 + 32 * p, ch = tid % 8;
      const int r = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < M) {
        const int b = r / e.T0, t = r % e.T0;
        v = *reinterpret_cast<const uint4*>(e.X + (static_cast<int64_t>(b) * e.N + t) * D + k0 + ch * 8);
      }
      *reinterpret_cast<uint4*>(&As[row * ELD + ch * 8]) = v;
      // B: 64 k rows x 128 n, read along n, stored transposed as [n][k].
      const int kk = tid / 16 + 16 * p, nc = (tid % 16) * 8;
      uint16_t w8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (n0 + nc + 8 <= D) {
        const uint4 wv = *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(k0 + kk) * D + n0 + nc);
        const uint32_t q[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          w8[2 * s] = static_cast<uint16_t>(q[s] & 0xFFFF);
          w8[2 * s + 1] = static_cast<uint16_t>(q[s] >> 16);
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) Bs[(nc + s) * ELD + kk] = w8[s];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < EBK / 16; ++s) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 32 + l32) * ELD + s * 16 + 8 * hf]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + j * 32 + l32) * ELD + s * 16 + 8 * hf]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const int col = n0 + wn * 64 + j * 32 + l32;
        if (row < M && col < D) e.Y[static_cast<int64_t>(row) * 3 * D + which * D + col] = acc[i][j][r];
      }
}

// Mixing (Algorithm 1) in fp32 for stacked rows i = t*P + j < R:
//   Qe/Ke[b][i][h][c] and Vte[b][h][c][i] = sum_m alpha[m][h][j] * Y[b*T0 + t][which*D + m*d + c]
// grid: (R, B, 3); block 256 over the D = H*d outputs of one row.
__global__ __launch_bounds__(256) void early_mix_kernel(EarlyArgs e) {
  const int i = blockIdx.x, b = blockIdx.y, which = blockIdx.z;
  const int P = e.P, H = e.H, d = e.d, D = e.D, R = e.R;
  const int t = i / P, j = i % P;
  const float* __restrict__ y = e.Y + static_cast<int64_t>(b * e.T0 + t) * 3 * D + which * D;
  const float* __restrict__ alpha = e.alpha[which];
  for (int o = threadIdx.x; o < D; o += 256) {
    const int h = o / d, c = o % d;
    float acc = 0.f;
    for (int m = 0; m < H; ++m) acc = fmaf(alpha[(m * H + h) * P + j], y[m * d + c], acc);
    if (which == 0) e.Qe[(static_cast<int64_t>(b) * R + i) * D + o] = acc;
    else if (which == 1) e.Ke[(static_cast<int64_t>(b) * R + i) * D + o] = acc;
    else e.Vte[(static_cast<int64_t>(b * H + h) * d + c) * R + i] = acc;
  }
}

// Attention of the first R stacked rows in fp32 (causal or window mask; a row i sees keys
// i' <= i, so only keys < R are involved).  Block: 16 query rows of one (b, h); the scores
// of those rows live in LDS, keys and values stream through LDS in chunks of 32.
// grid: (ceil(R / 16), H, B); block 256.
constexpr int ERows = 16, EKeys = 32;

template <int DH>
__global__ __launch_bounds__(256) void early_attn_kernel(EarlyArgs e, float* __restrict__ O,
                                                         int64_t o_bstride, int mask, int window,
                                                         float scale) {
  __shared__ float qs[ERows][DH + 1];
  __shared__ float ks[EKeys][DH + 1];
  __shared__ float vs[DH][EKeys + 1];
  __shared__ float ps[ERows][kPreciseRows + 1];
  __shared__ float inv_l[ERows];
  const int R = e.R, H = e.H, D = e.D;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i0 = blockIdx.x * ERows;
  const int tid = threadIdx.x;
  const float* __restrict__ Qb = e.Qe + static_cast<int64_t>(b) * R * D + h * DH;
  const float* __restrict__ Kb = e.Ke + static_cast<int64_t>(b) * R * D + h * DH;
  const float* __restrict__ Vb = e.Vte + static_cast<int64_t>(b * H + h) * DH * R;

  for (int x = tid; x < ERows * DH; x += 256) {
    const int r = x / DH, c = x % DH;
    qs[r][c] = (i0 + r < R) ? Qb[static_cast<int64_t>(i0 + r) * D + c] : 0.f;
  }
  const int khi = min(R, i0 + ERows);                        // keys <= the last row
  const int klo = mask == kMaskWindow ? max(0, i0 - window + 1) : 0;
  const int kc0 = klo / EKeys * EKeys;

  // Scores s2 = (q . k) * scale for visible pairs, -inf otherwise.
  for (int kc = kc0; kc < khi; kc += EKeys) {
    __syncthreads();
    for (int x = tid; x < EKeys * DH; x += 256) {
      const int kk = x / DH, c = x % DH;
      ks[kk][c] = (kc + kk < R) ? Kb[static_cast<int64_t>(kc + kk) * D + c] : 0.f;
    }
    __syncthreads();
    for (int x = tid; x < ERows * EKeys; x += 256) {
      const int r = x / EKeys, kk = x % EKeys;
      const int i = i0 + r, k = kc + kk;
      float dot = 0.f;
#pragma unroll 8
      for (int c = 0; c < DH; ++c) dot = fmaf(qs[r][c], ks[kk][c], dot);
      const bool vis = k < R && k <= i && (mask != kMaskWindow || k > i - window);
      ps[r][k] = vis ? dot * scale : -__builtin_inff();
    }
  }
  __syncthreads();
  // Row softmax over [kc0, khi): 16 threads per row, max and sum combined with shuffles.
  {
    const int r = tid / 16, sub = tid % 16;
    float mx = -__builtin_inff();
    for (int k = kc0 + sub; k < khi; k += 16) mx = fmaxf(mx, ps[r][k]);
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
    float sum = 0.f;
    for (int k = kc0 + sub; k < khi; k += 16) {
      const float p = (mx == -__builtin_inff()) ? 0.f : fast_exp2(ps[r][k] - mx);
      ps[r][k] = p;
      sum += p;
    }
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
    if (sub == 0) inv_l[r] = sum > 0.f ? 1.f / sum : 0.f;
  }
  // O[i][c] = sum_k p[i][k] v[k][c] / l[i].
  constexpr int PER = ERows * DH / 256;
  float acc[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) acc[q] = 0.f;
  for (int kc = kc0; kc < khi; kc += EKeys) {
    __syncthreads();
    for (int x = tid; x < DH * EKeys; x += 256) {
      const int c = x / EKeys, kk = x % EKeys;
      vs[c][kk] = (kc + kk < R) ? Vb[static_cast<int64_t>(c) * R + kc + kk] : 0.f;
    }
    __syncthreads();
    const int kn = min(EKeys, khi - kc);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int x = tid + 256 * q;
      const int r = x / DH, c = x % DH;
      float a = acc[q];
      for (int kk = 0; kk < kn; ++kk) a = fmaf(ps[r][kc + kk], vs[c][kk], a);
      acc[q] = a;
    }
  }
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int x = tid + 256 * q;
    const int r = x / DH, c = x % DH;
    if (i0 + r < R)
      O[static_cast<int64_t>(b) * o_bstride + static_cast<int64_t>(i0 + r) * D + h * DH + c] =
          acc[q] * inv_l[r];
  }
}

}  // namespace

hipError_t launch_early_qkv(const EarlyArgs& e, hipStream_t s) {
  const int M = e.B * e.T0;
  const dim3 g1((e.D + EBN - 1) / EBN, (M + EBM - 1) / EBM, 3);
  hipLaunchKernelGGL(early_proj_kernel, g1, dim3(256), 0, s, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(early_mix_kernel, dim3(e.R, e.B, 3), dim3(256), 0, s, e);
  return hipGetLastError();
}

}  // namespace iha

namespace iha {
hipError_t launch_early_attn(const EarlyArgs& e, float* O, int64_t o_bstride, int mask, int window,
                             float scale, hipStream_t s) {
  const dim3 grid((e.R + ERows - 1) / ERows, e.H, e.B);
  if (e.d == 64)
    hipLaunchKernelGGL(early_attn_kernel<64>, grid, dim3(256), 0, s, e, O, o_bstride, mask, window, scale);
  else if (e.d == 128)
    hipLaunchKernelGGL(early_attn_kernel<128>, grid, dim3(256), 0, s, e, O, o_bstride, mask, window, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
}  // namespace iha
