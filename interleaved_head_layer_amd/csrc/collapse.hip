// Steps 4-5 of Algorithm 1 ("Interleaved Head Attention" page, section 4): unstack the
// per-head attention outputs, collapse the H*P pseudo-outputs back to H heads through R,
// and concatenate the heads:
//   X~[tok][h*d + c] = sum_{h'} sum_j R[h][h'*P + j] * P_{h',j}[tok][c],
// where P_{h',j}[tok] is stacked row tok*P + j of head h', stored at
// Pbar[(tok*P + j)*H*d + h'*d + c].  Memory-bound: each token reads P*H*d values and
// writes H*d floats; R (HP x H, zero-padded) sits in LDS.  The bf16 forward stores the
// stacked outputs in fp16, except the first stacked rows of every sequence, which come in
// fp32 from a separate buffer (their outputs are the largest; they are recomputed in fp32).
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// Source of the stacked outputs: fp32 Pbar, or fp16 Ph with the first R stacked rows of
// each sequence (N tokens) in fp32 Pe [B][R][H][d].
struct CollapseSrc {
  const float* Pbar;
  const half_t* Ph;
  const float* Pe;
  int R, N;
};

// fp32 stacked outputs.  block: 256 threads = (256 / (d/4)) tokens x (d/4) channel quads.
// Each thread owns four consecutive channels of one token (float4 loads and stores) and
// accumulates all H output heads (4 * HMAX registers, H <= HMAX); its H*P loads are issued
// in unrolled groups.
template <int HMAX>
__global__ __launch_bounds__(256) void collapse_kernel(CollapseSrc src, const float* __restrict__ R,
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
  const int64_t base = static_cast<int64_t>(tok) * HP * d + c4;
  auto fma_row = [&](int q, const floatx4& pv) {
    const float* rq = Rs + q * HMAX;
#pragma unroll
    for (int h = 0; h < HMAX; h += 4) {
      const floatx4 r4 = *reinterpret_cast<const floatx4*>(rq + h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[h + e][0] = fmaf(r4[e], pv[0], acc[h + e][0]);
        acc[h + e][1] = fmaf(r4[e], pv[1], acc[h + e][1]);
        acc[h + e][2] = fmaf(r4[e], pv[2], acc[h + e][2]);
        acc[h + e][3] = fmaf(r4[e], pv[3], acc[h + e][3]);
      }
    }
  };
  constexpr int G = 8;
  for (int q0 = 0; q0 < HP; q0 += G) {
    floatx4 pv[G];
#pragma unroll
    for (int u = 0; u < G; ++u)
      pv[u] = q0 + u < HP ? *reinterpret_cast<const floatx4*>(src.Pbar + base + static_cast<int64_t>(q0 + u) * d)
                          : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (q0 + u >= HP) break;
      fma_row(q0 + u, pv[u]);
    }
  }
  float* dst = out + static_cast<int64_t>(tok) * H * d + c4;
#pragma unroll
  for (int h = 0; h < HMAX; ++h)
    if (h < H) *reinterpret_cast<floatx4*>(dst + h * d) = acc[h];
}

// fp16 stacked outputs: each thread owns four consecutive channels of one token (8-byte
// loads, 16 in flight); the first R stacked rows of each sequence come from the fp32 rows.
template <int HMAX>
__global__ __launch_bounds__(256) void collapse_h_kernel(CollapseSrc src, const float* __restrict__ R,
                                                         float* __restrict__ out, int ntok, int H,
                                                         int P, int d) {
  extern __shared__ float Rs[];
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
  const int64_t base = static_cast<int64_t>(tok) * HP * d + c4;
  auto fma_row = [&](int q, const floatx4& pv) {
    const float* rq = Rs + q * HMAX;
#pragma unroll
    for (int h = 0; h < HMAX; h += 4) {
      const floatx4 r4 = *reinterpret_cast<const floatx4*>(rq + h);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[h + e][0] = fmaf(r4[e], pv[0], acc[h + e][0]);
        acc[h + e][1] = fmaf(r4[e], pv[1], acc[h + e][1]);
        acc[h + e][2] = fmaf(r4[e], pv[2], acc[h + e][2]);
        acc[h + e][3] = fmaf(r4[e], pv[3], acc[h + e][3]);
      }
    }
  };
  const int t = tok % src.N;
  if (__builtin_expect(t * P < src.R, false)) {
    // A token whose first stacked row t*P is below R reads its rows i < R from Pe (fp32).
    const int64_t eb = static_cast<int64_t>(tok / src.N) * src.R;
    constexpr int G = 8;
    for (int q0 = 0; q0 < HP; q0 += G) {
      floatx4 pv[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int q = q0 + u;
        const int i = t * P + q / H;
        if (q >= HP) {
          pv[u] = floatx4{0.f, 0.f, 0.f, 0.f};
        } else if (i < src.R) {
          pv[u] = *reinterpret_cast<const floatx4*>(src.Pe + ((eb + i) * H + q % H) * d + c4);
        } else {
          const half4 v = *reinterpret_cast<const half4*>(src.Ph + base + static_cast<int64_t>(q) * d);
          pv[u] = floatx4{static_cast<float>(v[0]), static_cast<float>(v[1]), static_cast<float>(v[2]),
                          static_cast<float>(v[3])};
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (q0 + u >= HP) break;
        fma_row(q0 + u, pv[u]);
      }
    }
  } else {
    constexpr int G = 16;
    for (int q0 = 0; q0 < HP; q0 += G) {
      half4 pv[G];
#pragma unroll
      for (int u = 0; u < G; ++u)
        if (q0 + u < HP) pv[u] = *reinterpret_cast<const half4*>(src.Ph + base + static_cast<int64_t>(q0 + u) * d);
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (q0 + u >= HP) break;
        fma_row(q0 + u, floatx4{static_cast<float>(pv[u][0]), static_cast<float>(pv[u][1]),
                                static_cast<float>(pv[u][2]), static_cast<float>(pv[u][3])});
      }
    }
  }
  float* dst = out + static_cast<int64_t>(tok) * H * d + c4;
#pragma unroll
  for (int h = 0; h < HMAX; ++h)
    if (h < H) *reinterpret_cast<floatx4*>(dst + h * d) = acc[h];
}

template <int HMAX, bool HALF>
hipError_t launch_impl(const CollapseSrc& src, const float* R, float* out, int ntok, int H, int P, int d,
                       hipStream_t s) {
  const int per = 256 / (d / 4);
  const size_t lds = static_cast<size_t>(H) * P * HMAX * sizeof(float);
  if (HALF)
    hipLaunchKernelGGL((collapse_h_kernel<HMAX>), dim3((ntok + per - 1) / per), dim3(256), lds, s, src, R, out,
                       ntok, H, P, d);
  else
    hipLaunchKernelGGL((collapse_kernel<HMAX>), dim3((ntok + per - 1) / per), dim3(256), lds, s, src, R, out,
                       ntok, H, P, d);
  return hipGetLastError();
}

template <bool HALF>
hipError_t launch_h(const CollapseSrc& src, const float* R, float* out, int ntok, int H, int P, int d,
                    hipStream_t s) {
  if (H <= 4) return launch_impl<4, HALF>(src, R, out, ntok, H, P, d, s);
  if (H <= 8) return launch_impl<8, HALF>(src, R, out, ntok, H, P, d, s);
  if (H <= 16) return launch_impl<16, HALF>(src, R, out, ntok, H, P, d, s);
  if (H <= 20) return launch_impl<20, HALF>(src, R, out, ntok, H, P, d, s);
  if (H <= 32) return launch_impl<32, HALF>(src, R, out, ntok, H, P, d, s);
  return launch_impl<64, HALF>(src, R, out, ntok, H, P, d, s);
}

}  // namespace

hipError_t launch_collapse(const float* Pbar, const float* R, float* out, int ntok, int H, int P,
                           int d, hipStream_t s) {
  const CollapseSrc src{Pbar, nullptr, nullptr, 0, 1};
  return launch_h<false>(src, R, out, ntok, H, P, d, s);
}

hipError_t launch_collapse_h(const half_t* Ph, const float* Pe, int Rrows, const float* R, float* out, int B,
                             int N, int H, int P, int d, hipStream_t s) {
  const CollapseSrc src{nullptr, Ph, Pe, Rrows, N};
  return launch_h<true>(src, R, out, B * N, H, P, d, s);
}

}  // namespace iha
