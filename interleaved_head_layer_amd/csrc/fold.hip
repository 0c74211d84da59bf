// Step 1 of Algorithm 1 ("Interleaved Head Attention" page, section 4) for fp32 inputs:
// pseudo-head mixing.  Since Q~_{h,j} = sum_m alpha_{m,h,j} X W^(m) = X (sum_m alpha_{m,h,j} W^(m)),
// the mixing is applied once to the weights and the projection becomes one plain GEMM
// against the folded weights.  (bf16 inputs take the unfolded path in proj.hip.)
// Also: the device flag word helpers.
//
// Folded weight layout: Wt[col][k], col in [0, 3*P*H*d), k in [0, D) contiguous
// (both GEMM operands then carry the contraction index contiguously).
//   Q, K blocks: col = (j*H + h)*d + c  -> the GEMM writes [tokens][P][H][d], i.e. the
//                                          interleaved stacked rows t*P + j directly.
//   V block:     col = (h*d + c)*P + j  -> for fixed (h, c) the P outputs of a token
//                                          are adjacent, which the GEMM uses to write
//                                          the channel-major V^T [B][H][d][P*N].
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

constexpr int kFoldK = 32;   // rows of W (contraction index k) per block
constexpr int kFoldC = 8;    // head channels c per block
constexpr int kFoldThreads = kFoldK * kFoldC;

template <typename Tin>
__device__ __forceinline__ float load_w(const Tin* p);
template <>
__device__ __forceinline__ float load_w<float>(const float* p) { return *p; }

template <typename Tout>
__device__ __forceinline__ Tout store_cvt(float v);
template <>
__device__ __forceinline__ float store_cvt<float>(float v) { return v; }

// grid: (ceil(D / 32), d / 8, 3 = Q/K/V).  block: 256 threads.
// Dynamic LDS: H * 8 * 32 floats holding W[k0..k0+32)[m*d + c0 .. +8) for every source head m,
// stored as [m][c][k] so that the 32 lanes reading one c see consecutive k.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(kFoldThreads) void fold_kernel(FoldArgs a) {
  extern __shared__ float wsh[];
  const int which = blockIdx.z;
  const Tin* W = static_cast<const Tin*>(a.W[which]);
  const float* alpha = a.alpha[which];
  const int D = a.D, H = a.H, d = a.d, P = a.P;
  const int HD = H * d;
  const int k0 = blockIdx.x * kFoldK;
  const int c0 = blockIdx.y * kFoldC;
  const int tid = threadIdx.x;

  if (which == 0 && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0 && a.flag) *a.flag = 0u;

  // Load: element e -> (m, kk, cc) with cc fastest (8 consecutive channels of one W row).
  for (int e = tid; e < H * kFoldK * kFoldC; e += kFoldThreads) {
    const int m = e / (kFoldK * kFoldC);
    const int kk = (e / kFoldC) % kFoldK;
    const int cc = e % kFoldC;
    const int k = k0 + kk;
    float v = 0.f;
    if (k < D) v = load_w<Tin>(W + static_cast<int64_t>(k) * HD + m * d + c0 + cc);
    wsh[(m * kFoldC + cc) * kFoldK + kk] = v;
  }
  __syncthreads();

  const int kk = tid % kFoldK;
  const int cc = tid / kFoldK;
  const int k = k0 + kk;
  const int c = c0 + cc;
  const int PHd = P * H * d;
  Tout* Wt = static_cast<Tout*>(a.Wt) + static_cast<int64_t>(which) * PHd * D;
  const float scale = a.out_scale[which];
  if (k >= D) return;
  for (int h = 0; h < H; ++h) {
    for (int j = 0; j < P; ++j) {
      float acc = 0.f;
      for (int m = 0; m < H; ++m)
        acc = fmaf(alpha[(m * H + h) * P + j], wsh[(m * kFoldC + cc) * kFoldK + kk], acc);
      const int col = (which < 2) ? (j * H + h) * d + c : (h * d + c) * P + j;
      Wt[static_cast<int64_t>(col) * D + k] = store_cvt<Tout>(acc * scale);
    }
  }
}

__global__ void clear_flag_kernel(unsigned* flag) { *flag = 0u; }

// Sets `nonfinite_bit` for a non-finite element and kFlagRange for a finite one beyond
// `limit` in magnitude (limit = +inf: no range test).
__device__ __forceinline__ float value_of(float v) { return v; }
__device__ __forceinline__ float value_of(bf16_bits v) { return bf16_to_float(v); }
__device__ __forceinline__ float value_of(half_t v) { return static_cast<float>(v); }

template <typename T>
__global__ __launch_bounds__(256) void check_values_kernel(const T* __restrict__ x, int64_t n, unsigned* flag,
                                                           unsigned nonfinite_bit, float limit) {
  unsigned bits = 0u;
  for (int64_t i = blockIdx.x * 256LL + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
    const float v = value_of(x[i]);
    if (!__builtin_isfinite(v))
      bits |= nonfinite_bit;
    else if (__builtin_fabsf(v) > limit)
      bits |= kFlagRange;
  }
  if (bits) atomicOr(flag, bits);
}

template <typename Tin, typename Tout>
hipError_t launch_fold_impl(const FoldArgs& a, hipStream_t s) {
  const dim3 grid((a.D + kFoldK - 1) / kFoldK, a.d / kFoldC, 3);
  const size_t lds = static_cast<size_t>(a.H) * kFoldK * kFoldC * sizeof(float);
  hipLaunchKernelGGL((fold_kernel<Tin, Tout>), grid, dim3(kFoldThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fold_f32(const FoldArgs& a, hipStream_t s) {
  return launch_fold_impl<float, float>(a, s);
}

namespace {
__global__ __launch_bounds__(256) void fill_zero_kernel(floatx4* __restrict__ p, int64_t n4) {
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += static_cast<int64_t>(gridDim.x) * 256)
    p[i] = z;
}
}  // namespace

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 < 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 256 * 8))));
  hipLaunchKernelGGL(fill_zero_kernel, grid, dim3(256), 0, s, reinterpret_cast<floatx4*>(p), n4);
  return hipGetLastError();
}

hipError_t launch_clear_flag(unsigned* flag, hipStream_t s) {
  hipLaunchKernelGGL(clear_flag_kernel, dim3(1), dim3(1), 0, s, flag);
  return hipGetLastError();
}

hipError_t launch_check_values(const void* x, int kind, int64_t n, unsigned* flag, unsigned nonfinite_bit,
                               float limit, hipStream_t s) {
  if (n < 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 256 * 8))));
  switch (kind) {
    case kValF32:
      hipLaunchKernelGGL(check_values_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x), n,
                         flag, nonfinite_bit, limit);
      break;
    case kValBF16:
      hipLaunchKernelGGL(check_values_kernel<bf16_bits>, grid, dim3(256), 0, s,
                         static_cast<const bf16_bits*>(x), n, flag, nonfinite_bit, limit);
      break;
    case kValF16:
      hipLaunchKernelGGL(check_values_kernel<half_t>, grid, dim3(256), 0, s, static_cast<const half_t*>(x), n,
                         flag, nonfinite_bit, limit);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace iha
