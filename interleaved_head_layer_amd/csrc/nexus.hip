// The inner attention of the Nexus higher-order attention ("Higher-order attention
// mechanisms" page, section 2): Attention_q(X) = softmax(Q Q^T / sqrt(d_k)) Q, per head,
// i.e. self-attention whose keys and values are the queries themselves.  It runs on the
// tiled attention kernel; the only extra step is the values' channel-major copy that
// kernel reads (V^T [B][H][d][L]), made here from the row-major queries.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// Q [B][L][H][d] fp16 -> Qt [B][H][d][L] fp16.  grid: (ceil(L/64), d/64, B*H), block 256.
// A 64-row x 64-channel tile passes through LDS: 16-byte loads of 8 channels of one row, then
// 16-byte stores of 8 rows of one channel (element stores where a chunk crosses L).
__global__ __launch_bounds__(256) void transpose_rows_kernel(const half_t* __restrict__ Q, half_t* __restrict__ Qt,
                                                             int L, int H, int d) {
  __shared__ half_t t[64][64 + 8];  // [row][channel]; the pad staggers the column reads
  const int bh = blockIdx.z, b = bh / H, h = bh % H;
  const int l0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  const half_t* src = Q + (static_cast<int64_t>(b) * L * H + h) * d;  // row l at src + l*H*d
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int x = tid + 256 * q, r = x >> 3, c8 = (x & 7) * 8;
    half8 v;
    if (l0 + r < L) {
      v = *reinterpret_cast<const half8*>(src + static_cast<int64_t>(l0 + r) * H * d + c0 + c8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = static_cast<half_t>(0.f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) t[r][c8 + e] = v[e];
  }
  __syncthreads();
  half_t* dst = Qt + static_cast<int64_t>(bh) * d * L;  // channel c at dst + c*L
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int x = tid + 256 * q, c = x >> 3, r8 = (x & 7) * 8;
    half_t* row = dst + static_cast<int64_t>(c0 + c) * L + l0 + r8;
    if (l0 + r8 + 8 <= L && (L % 8) == 0) {
      half8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = t[r8 + e][c];
      *reinterpret_cast<half8*>(row) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (l0 + r8 + e < L) row[e] = t[r8 + e][c];
    }
  }
}

}  // namespace

hipError_t launch_transpose_rows(const half_t* Q, half_t* Qt, int B, int L, int H, int d, hipStream_t s) {
  if (d % 64 != 0) return hipErrorInvalidValue;
  const dim3 grid((L + 63) / 64, d / 64, B * H);
  hipLaunchKernelGGL(transpose_rows_kernel, grid, dim3(256), 0, s, Q, Qt, L, H, d);
  return hipGetLastError();
}

}  // namespace iha
