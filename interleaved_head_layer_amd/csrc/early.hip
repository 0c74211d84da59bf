// Full-precision attention for the first stacked rows of every (b, h) under a causal or
// window mask (bf16 inputs).
//
// Why: a stacked row that sees n keys has an output of magnitude about n^-1/2 (it averages
// n value rows with softmax weights), while the fp16 intermediates of the main path carry a
// fixed relative error.  The first rows see only a handful of keys, so their outputs, and
// their absolute errors, are far above the typical output; the output error bound is set
// by them.  These rows (the first 128, one query tile) are recomputed here in fp32 from the
// fp32 copies of their projected and mixed queries, keys and values (written by the mixing
// kernels), and overwrite those rows of P-bar after the main attention kernel.  Every later
// row sees more than 128 keys.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

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
