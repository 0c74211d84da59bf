// Steps 4-5 of Algorithm 1 ("Interleaved Head Attention" page, section 4): unstack the
// per-head attention outputs, collapse the H*P pseudo-outputs back to H heads through R,
// and concatenate the heads:
//   X~[tok][h*d + c] = sum_{h'} sum_j R[h][h'*P + j] * P_{h',j}[tok][c],
// where P_{h',j}[tok] is stacked row tok*P + j of head h', stored at
// Pbar[(tok*P + j)*H*d + h'*d + c].  Memory-bound: each token reads P*H*d floats and
// writes H*d floats; R (HP x H, zero-padded) sits in LDS.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// block: 256 threads = (256 / (d/4)) tokens x (d/4) channel quads.  Each thread owns four
// consecutive channels of one token (float4 loads and stores) and accumulates all H output
// heads (4 * HMAX registers, H <= HMAX); its H*P loads are issued in unrolled groups.
template <int HMAX>
__global__ __launch_bounds__(256) void collapse_kernel(const float* __restrict__ Pbar,
                                                       const float* __restrict__ R,
                                                       float* __restrict__ out, int ntok, int H,
                                                       int P, int d) {
  extern __shared__ float Rs[];  // Rs[q*HMAX + h] = R[h][h'*P + j], q = j*H + h'; zero for h >= H
  const int HP = H * P;
  for (int e = threadIdx.x; e < HP * HMAX; e += 256) {
    const int q = e / HMAX, h = e % HMAX;
    const int j = q / H, hp = q % H;
    Rs[e] = h < H ? R[h * HP + hp * P + j] : 0.f;
  }
  __syncthreads();
  const int quads = d / 4;
  const int per = 256 / quads;
  const int tok = blockIdx.x * per + threadIdx.x / quads;
  const int c4 = (threadIdx.x % quads) * 4;
  if (tok >= ntok) return;
  floatx4 acc[HMAX];
#pragma unroll
  for (int h = 0; h < HMAX; ++h) acc[h] = floatx4{0.f, 0.f, 0.f, 0.f};
  const float* src = Pbar + static_cast<int64_t>(tok) * HP * d + c4;
  constexpr int G = 8;
  for (int q0 = 0; q0 < HP; q0 += G) {
    floatx4 pv[G];
#pragma unroll
    for (int u = 0; u < G; ++u)
      pv[u] = q0 + u < HP ? *reinterpret_cast<const floatx4*>(src + static_cast<int64_t>(q0 + u) * d)
                          : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (q0 + u >= HP) break;
      const float* rq = Rs + (q0 + u) * HMAX;
#pragma unroll
      for (int h = 0; h < HMAX; h += 4) {
        const floatx4 r4 = *reinterpret_cast<const floatx4*>(rq + h);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[h + e][0] = fmaf(r4[e], pv[u][0], acc[h + e][0]);
          acc[h + e][1] = fmaf(r4[e], pv[u][1], acc[h + e][1]);
          acc[h + e][2] = fmaf(r4[e], pv[u][2], acc[h + e][2]);
          acc[h + e][3] = fmaf(r4[e], pv[u][3], acc[h + e][3]);
        }
      }
    }
  }
  float* dst = out + static_cast<int64_t>(tok) * H * d + c4;
#pragma unroll
  for (int h = 0; h < HMAX; ++h)
    if (h < H) *reinterpret_cast<floatx4*>(dst + h * d) = acc[h];
}

template <int HMAX>
hipError_t launch_impl(const float* Pbar, const float* R, float* out, int ntok, int H, int P, int d,
                       hipStream_t s) {
  const int per = 256 / (d / 4);
  const size_t lds = static_cast<size_t>(H) * P * HMAX * sizeof(float);
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
  if (H <= 20) return launch_impl<20>(Pbar, R, out, ntok, H, P, d, s);
  if (H <= 32) return launch_impl<32>(Pbar, R, out, ntok, H, P, d, s);
  return launch_impl<64>(Pbar, R, out, ntok, H, P, d, s);
}

}  // namespace iha
