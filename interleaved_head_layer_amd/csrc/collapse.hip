// Steps 4-5 of Algorithm 1 ("Interleaved Head Attention" page, section 4): unstack the
// per-head attention outputs, collapse the H*P pseudo-outputs back to H heads through R,
// and concatenate the heads:
//   X~[tok][h*d + c] = sum_{h'} sum_j R[h][h'*P + j] * P_{h',j}[tok][c],
// where P_{h',j}[tok] is stacked row tok*P + j of head h', stored at
// Pbar[(tok*P + j)*H*d + h'*d + c].  Memory-bound: each token reads P*H*d floats and
// writes H*d floats; R (H x HP) sits in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// block: 256 threads = (256 / d) tokens x d channels.  Each thread owns one channel c of
// one token and accumulates all H output heads (HMAX registers, H <= HMAX).
template <int HMAX>
__global__ __launch_bounds__(256) void collapse_kernel(const float* __restrict__ Pbar,
                                                       const float* __restrict__ R,
                                                       float* __restrict__ out, int ntok, int H,
                                                       int P, int d) {
  extern __shared__ float Rs[];  // Rs[(j*H + h')*H + h] = R[h][h'*P + j]
  const int HP = H * P;
  for (int e = threadIdx.x; e < HP * H; e += 256) {
    const int q = e / H, h = e % H;
    const int j = q / H, hp = q % H;
    Rs[e] = R[h * HP + hp * P + j];
  }
  __syncthreads();
  const int per = 256 / d;
  const int tok = blockIdx.x * per + threadIdx.x / d;
  const int c = threadIdx.x % d;
  if (tok >= ntok) return;
  float acc[HMAX];
#pragma unroll
  for (int h = 0; h < HMAX; ++h) acc[h] = 0.f;
  const float* src = Pbar + static_cast<int64_t>(tok) * HP * d + c;
  for (int q = 0; q < HP; ++q) {
    const float pv = src[static_cast<int64_t>(q) * d];
    const float* rq = Rs + q * H;
#pragma unroll
    for (int h = 0; h < HMAX; ++h)
      if (h < H) acc[h] = fmaf(rq[h], pv, acc[h]);
  }
  float* dst = out + static_cast<int64_t>(tok) * H * d + c;
#pragma unroll
  for (int h = 0; h < HMAX; ++h)
    if (h < H) dst[h * d] = acc[h];
}

template <int HMAX>
hipError_t launch_impl(const float* Pbar, const float* R, float* out, int ntok, int H, int P, int d,
                       hipStream_t s) {
  const int per = 256 / d;
  const size_t lds = static_cast<size_t>(H) * H * P * sizeof(float);
  hipLaunchKernelGGL((collapse_kernel<HMAX>), dim3((ntok + per - 1) / per), dim3(256), lds, s,
                     Pbar, R, out, ntok, H, P, d);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_collapse(const float* Pbar, const float* R, float* out, int ntok, int H, int P,
                           int d, hipStream_t s) {
  if (H <= 4) return launch_impl<4>(Pbar, R, out, ntok, H, P, d, s);
  if (H <= 8) return launch_impl<8>(Pbar, R, out, ntok, H, P, d, s);
  if (H <= 16) return launch_impl<16>(Pbar, R, out, ntok, H, P, d, s);
  if (H <= 32) return launch_impl<32>(Pbar, R, out, ntok, H, P, d, s);
  return launch_impl<64>(Pbar, R, out, ntok, H, P, d, s);
}

}  // namespace iha
