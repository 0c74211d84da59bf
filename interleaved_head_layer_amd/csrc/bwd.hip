// Helper kernels of the layer's backward pass (reverse mode through Algorithm 1 of the
// "Interleaved Head Attention" page, section 4): the token reductions that give the mixing
// and collapse gradients, and the bf16 conversions and transposes that feed the weight and
// input gradients to the bf16 matrix-core GEMM.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// Round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ------------------------------------------------------------------- head reduction
// out[a][hj] = sum over tokens t and channels c of A[t][a][c] * B[t][hj][c], where B's row
// for hj = h*P + j is stacked row t*P + j, head h.  A block owns a 16 (a) x 16 (hj) output
// tile and a chunk of tokens; each thread one output.  TS tokens at a time pass through LDS
// (rows padded by 4 floats so the 16 hj rows a wave reads fall in different banks).
constexpr int kRedTile = 16;
constexpr int kRedChunkTarget = 2048;  // chunks x tiles is about this (bounds the partials)

template <typename TB>
__device__ __forceinline__ floatx4 load4(const TB* p);
template <>
__device__ __forceinline__ floatx4 load4<float>(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}
template <>
__device__ __forceinline__ floatx4 load4<half_t>(const half_t* p) {
  typedef half_t half4 __attribute__((ext_vector_type(4)));
  const half4 h = *reinterpret_cast<const half4*>(p);
  return floatx4{static_cast<float>(h[0]), static_cast<float>(h[1]), static_cast<float>(h[2]),
                 static_cast<float>(h[3])};
}

template <typename TB, int DH>
__global__ __launch_bounds__(256) void head_reduce_kernel(const float* __restrict__ A, int64_t lda,
                                                          const TB* __restrict__ Bm, float* __restrict__ part,
                                                          int ntok, int H, int P, int tpc) {
  constexpr int TS = 256 / DH;  // tokens per LDS stage
  constexpr int LD = DH + 4;
  __shared__ float as[TS][kRedTile][LD];
  __shared__ float bs[TS][kRedTile][LD];
  const int HP = H * P;
  const int a0 = blockIdx.y * kRedTile, hj0 = blockIdx.z * kRedTile;
  const int t_begin = blockIdx.x * tpc, t_end = min(ntok, t_begin + tpc);
  const int tid = threadIdx.x, ty = tid / kRedTile, tx = tid % kRedTile;
  float acc = 0.f;
  for (int t0 = t_begin; t0 < t_end; t0 += TS) {
    // TS x 16 rows x DH channels of each operand = 1024 float4 = 4 per thread
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + 256 * q, row = e / (DH / 4), c = (e % (DH / 4)) * 4;
      const int ts = row / kRedTile, r = row % kRedTile, t = t0 + ts;
      floatx4 va{0.f, 0.f, 0.f, 0.f}, vb{0.f, 0.f, 0.f, 0.f};
      if (t < t_end && a0 + r < H) va = load4<float>(A + static_cast<int64_t>(t) * lda + (a0 + r) * DH + c);
      const int hj = hj0 + r;
      if (t < t_end && hj < HP) {
        const int h = hj / P, j = hj % P;
        vb = load4<TB>(Bm + ((static_cast<int64_t>(t) * P + j) * H + h) * DH + c);
      }
      *reinterpret_cast<floatx4*>(&as[ts][r][c]) = va;
      *reinterpret_cast<floatx4*>(&bs[ts][r][c]) = vb;
    }
    __syncthreads();
#pragma unroll
    for (int ts = 0; ts < TS; ++ts)
#pragma unroll 8
      for (int c = 0; c < DH; c += 4) {
        const floatx4 x = *reinterpret_cast<const floatx4*>(&as[ts][ty][c]);
        const floatx4 y = *reinterpret_cast<const floatx4*>(&bs[ts][tx][c]);
        acc += x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
      }
    __syncthreads();
  }
  const int a = a0 + ty, hj = hj0 + tx;
  if (a < H && hj < HP) part[static_cast<int64_t>(blockIdx.x) * H * HP + a * HP + hj] = acc;
}

// out[o] = sum over chunks of part[chunk][o], chunks in order.
__global__ __launch_bounds__(256) void head_reduce_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                              int n, int nchunks) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= n) return;
  float s = 0.f;
  for (int k = 0; k < nchunks; ++k) s += part[static_cast<int64_t>(k) * n + o];
  out[o] = s;
}

struct RedPlan {
  int tiles_y, tiles_z, nchunks, tpc;
};

RedPlan red_plan(int ntok, int H, int P) {
  RedPlan p{};
  p.tiles_y = (H + kRedTile - 1) / kRedTile;
  p.tiles_z = (H * P + kRedTile - 1) / kRedTile;
  const int target = std::max(1, kRedChunkTarget / (p.tiles_y * p.tiles_z));
  const int ntok1 = std::max(ntok, 1);
  p.tpc = std::max(1, (ntok1 + target - 1) / target);
  p.nchunks = (ntok1 + p.tpc - 1) / p.tpc;
  return p;
}

// ------------------------------------------------------------------- bf16 conversions
// Row-major fp32 -> bf16, 4 elements per thread; with dst_lo also the rounding remainder
// bf16(v - hi), so that hi + lo carries 16 significant bits.  grid (ceil(nc/4/64), rows),
// block 64; a block walks rows blockIdx.y, blockIdx.y + gridDim.y, ...
__global__ __launch_bounds__(64) void to_bf16_kernel(const float* __restrict__ src, int64_t lds, int nr, int nc,
                                                     uint16_t* __restrict__ dst, uint16_t* __restrict__ dst_lo,
                                                     int64_t ldd) {
  const int c = (blockIdx.x * 64 + threadIdx.x) * 4;
  if (c >= nc) return;
  for (int r = blockIdx.y; r < nr; r += gridDim.y) {
    const floatx4 v = *reinterpret_cast<const floatx4*>(src + static_cast<int64_t>(r) * lds + c);
    uint16_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = f32_to_bf16(v[e]);
      l[e] = f32_to_bf16(v[e] - bf16_to_float(h[e]));
    }
    const int64_t o = static_cast<int64_t>(r) * ldd + c;
    *reinterpret_cast<uint2*>(dst + o) = make_uint2(h[0] | (static_cast<uint32_t>(h[1]) << 16),
                                                    h[2] | (static_cast<uint32_t>(h[3]) << 16));
    if (dst_lo)
      *reinterpret_cast<uint2*>(dst_lo + o) = make_uint2(l[0] | (static_cast<uint32_t>(l[1]) << 16),
                                                         l[2] | (static_cast<uint32_t>(l[3]) << 16));
  }
}

// Row-major bf16 copy, 8 elements per thread.  grid as for to_bf16_kernel.
__global__ __launch_bounds__(64) void copy_bf16_kernel(const uint16_t* __restrict__ src, int64_t lds, int nr, int nc,
                                                       uint16_t* __restrict__ dst, int64_t ldd) {
  const int c = (blockIdx.x * 64 + threadIdx.x) * 8;
  if (c >= nc) return;
  for (int r = blockIdx.y; r < nr; r += gridDim.y)
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(r) * ldd + c) =
        *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(r) * lds + c);
}

// Transpose to bf16: dst[c][r] = src[r][c] (and the remainder to dst_lo, as above).  A 64 x 64
// tile passes through LDS as floats.  grid (nr_out/64, ceil(nc/64)), block 256: destination
// columns r < nr_out are written, zero for r >= nr.
template <bool SrcBf16>
__global__ __launch_bounds__(256) void to_bf16_t_kernel(const void* __restrict__ src, int64_t lds, int nr, int nc,
                                                        uint16_t* __restrict__ dst, uint16_t* __restrict__ dst_lo,
                                                        int64_t ldd) {
  __shared__ float t[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int r = e / 64, c = e % 64;  // consecutive threads along the source row
    float v = 0.f;
    if (r0 + r < nr && c0 + c < nc) {
      const int64_t off = static_cast<int64_t>(r0 + r) * lds + c0 + c;
      v = SrcBf16 ? bf16_to_float(static_cast<const uint16_t*>(src)[off]) : static_cast<const float*>(src)[off];
    }
    t[r][c] = v;
  }
  __syncthreads();
  for (int e = tid; e < 64 * 32; e += 256) {
    const int c = e / 32, r2 = (e % 32) * 2;  // consecutive threads along the destination row
    if (c0 + c >= nc) continue;
    const float v0 = t[r2][c], v1 = t[r2 + 1][c];
    const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
    const int64_t o = static_cast<int64_t>(c0 + c) * ldd + r0 + r2;
    *reinterpret_cast<uint32_t*>(dst + o) = h0 | (static_cast<uint32_t>(h1) << 16);
    if (dst_lo)
      *reinterpret_cast<uint32_t*>(dst_lo + o) = f32_to_bf16(v0 - bf16_to_float(h0)) |
                                                 (static_cast<uint32_t>(f32_to_bf16(v1 - bf16_to_float(h1))) << 16);
  }
}

}  // namespace

size_t head_reduce_part_bytes(int ntok, int H, int P) {
  const RedPlan p = red_plan(ntok, H, P);
  return static_cast<size_t>(p.nchunks) * H * H * P * sizeof(float);
}

hipError_t launch_head_reduce(const float* A, int64_t lda, const void* Bm, bool b_half, float* out, float* part,
                              int ntok, int H, int P, int d, hipStream_t s) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  const RedPlan p = red_plan(ntok, H, P);
  const dim3 grid(p.nchunks, p.tiles_y, p.tiles_z);
  if (d == 64) {
    if (b_half)
      hipLaunchKernelGGL((head_reduce_kernel<half_t, 64>), grid, dim3(256), 0, s, A, lda,
                         static_cast<const half_t*>(Bm), part, ntok, H, P, p.tpc);
    else
      hipLaunchKernelGGL((head_reduce_kernel<float, 64>), grid, dim3(256), 0, s, A, lda,
                         static_cast<const float*>(Bm), part, ntok, H, P, p.tpc);
  } else {
    if (b_half)
      hipLaunchKernelGGL((head_reduce_kernel<half_t, 128>), grid, dim3(256), 0, s, A, lda,
                         static_cast<const half_t*>(Bm), part, ntok, H, P, p.tpc);
    else
      hipLaunchKernelGGL((head_reduce_kernel<float, 128>), grid, dim3(256), 0, s, A, lda,
                         static_cast<const float*>(Bm), part, ntok, H, P, p.tpc);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = H * H * P;
  hipLaunchKernelGGL(head_reduce_sum_kernel, dim3((n + 255) / 256), dim3(256), 0, s, part, out, n, p.nchunks);
  return hipGetLastError();
}

hipError_t launch_to_bf16(const float* src, int64_t lds, int nr, int nc, uint16_t* dst, uint16_t* dst_lo, int64_t ldd,
                          hipStream_t s) {
  if (nc % 4 != 0) return hipErrorInvalidValue;
  if (nr < 1 || nc < 1) return hipSuccess;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((nc / 4 + 63) / 64, std::min(nr, 65535)), dim3(64), 0, s, src, lds, nr, nc,
                     dst, dst_lo, ldd);
  return hipGetLastError();
}

hipError_t launch_copy_bf16(const uint16_t* src, int64_t lds, int nr, int nc, uint16_t* dst, int64_t ldd,
                            hipStream_t s) {
  if (nc % 8 != 0) return hipErrorInvalidValue;
  if (nr < 1 || nc < 1) return hipSuccess;
  hipLaunchKernelGGL(copy_bf16_kernel, dim3((nc / 8 + 63) / 64, std::min(nr, 65535)), dim3(64), 0, s, src, lds, nr,
                     nc, dst, ldd);
  return hipGetLastError();
}

hipError_t launch_to_bf16_t(const void* src, bool src_bf16, int64_t lds, int nr, int nc, uint16_t* dst,
                            uint16_t* dst_lo, int64_t ldd, int64_t nr_out, hipStream_t s) {
  if (nr_out % 64 != 0 || nr > nr_out || nr_out > ldd || (nc + 63) / 64 > 65535) return hipErrorInvalidValue;
  if (nr_out < 1 || nc < 1) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(nr_out / 64), (nc + 63) / 64);
  if (src_bf16)
    hipLaunchKernelGGL(to_bf16_t_kernel<true>, grid, dim3(256), 0, s, src, lds, nr, nc, dst, dst_lo, ldd);
  else
    hipLaunchKernelGGL(to_bf16_t_kernel<false>, grid, dim3(256), 0, s, src, lds, nr, nc, dst, dst_lo, ldd);
  return hipGetLastError();
}

}  // namespace iha
