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
// out[a][hj] = sum over tokens t and channels c of A[t][a][c] * B[t][hj][c], where B's row for
// hj = h*P + j is stacked row t*P + j, head h: a product whose contracted dimension is (t, c).
// It runs on the matrix cores straight from global memory: a workgroup of 4 waves owns a chunk
// of tokens and a group of up to kRedCB 32-wide hj blocks (grid.y); each wave takes every 4th
// token and accumulates the whole (a, hj) tile.  Per 16-channel step a lane loads 8 channels of
// its A row (a = lane % 32 + 32 rb) and of its B row (hj = lane % 32 + 32 cb), splits them into
// bf16 high and low parts and issues hi*hi + hi*lo + lo*hi (about 2^-16 relative per product,
// fp32 accumulation).  Every operand element is read once.  The waves' tiles are added in LDS
// in wave order and written as the chunk's partial sums.
constexpr int kRedCB = 3;               // hj blocks per workgroup
constexpr int kRedChunkTarget = 2048;   // chunks x hj groups is about this (more chunks keep more loads
                                        // in flight: 512 measured 1.5 % slower, 4096 too; bounds the partials)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf16(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint16_t h = f32_to_bf16(x[e]);
    const uint16_t l = f32_to_bf16(x[e] - __uint_as_float(static_cast<uint32_t>(h) << 16));
    hi[e] = __builtin_bit_cast(__bf16, h);
    lo[e] = __builtin_bit_cast(__bf16, l);
  }
}

template <typename TB>
__device__ __forceinline__ void load8(const TB* p, float (&x)[8]);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const floatx4 u = *reinterpret_cast<const floatx4*>(p), v = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = u[e];
    x[4 + e] = v[e];
  }
}
template <>
__device__ __forceinline__ void load8<half_t>(const half_t* p, float (&x)[8]) {
  const half8 u = *reinterpret_cast<const half8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = static_cast<float>(u[e]);
}

template <typename TB, int DH, int RB>
__global__ __launch_bounds__(256) void head_reduce_kernel(const float* __restrict__ A, int64_t lda,
                                                          const TB* __restrict__ Bm, float* __restrict__ part,
                                                          int ntok, int H, int P, int tpc) {
  constexpr int NS = DH / 16;
  __shared__ float red[RB * 32][kRedCB * 32 + 1];
  const int HP = H * P;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int cb0 = blockIdx.y * kRedCB;
  const int t_begin = blockIdx.x * tpc, t_end = min(ntok, t_begin + tpc);
  floatx16 acc[RB][kRedCB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kRedCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[rb][cb][r] = 0.f;
  // This lane's A rows and B rows (invalid ones read row 0 and are multiplied by zero: their
  // products land in rows / columns that are never written out).
  int arow[RB];
  bool aval[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    aval[rb] = rb * 32 + l32 < H;
    arow[rb] = aval[rb] ? rb * 32 + l32 : 0;
  }
  int64_t boff[kRedCB];
  bool bval[kRedCB];
#pragma unroll
  for (int cb = 0; cb < kRedCB; ++cb) {
    const int hj = (cb0 + cb) * 32 + l32;
    bval[cb] = hj < HP;
    const int hh = bval[cb] ? hj / P : 0, j = bval[cb] ? hj % P : 0;
    boff[cb] = (static_cast<int64_t>(j) * H + hh) * DH;  // + t*P*H*DH
  }
  for (int t = t_begin + w; t < t_end; t += 4) {
    const float* at = A + static_cast<int64_t>(t) * lda;
    const TB* bt = Bm + static_cast<int64_t>(t) * P * H * DH;
#pragma unroll 2
    for (int s = 0; s < NS; ++s) {
      const int c = s * 16 + 8 * hf;
      bf16x8 ah[RB], al[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float x[8];
        load8<float>(at + arow[rb] * DH + c, x);
        if (!aval[rb])
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        split_bf16(x, ah[rb], al[rb]);
      }
#pragma unroll
      for (int cb = 0; cb < kRedCB; ++cb) {
        float x[8];
        load8<TB>(bt + boff[cb] + c, x);
        if (!bval[cb])
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        bf16x8 bh, bl;
        split_bf16(x, bh, bl);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[rb], bh, acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[rb], bl, acc[rb][cb], 0, 0, 0);
          acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[rb], bh, acc[rb][cb], 0, 0, 0);
        }
      }
    }
  }
  // Lane l holds C[8*(r/4) + 4*hf + r%4][l%32] of each 32x32 block: add the waves in order.
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < kRedCB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float& dst = red[rb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)][cb * 32 + l32];
            dst = ww == 0 ? acc[rb][cb][r] : dst + acc[rb][cb][r];
          }
    }
    __syncthreads();
  }
  for (int e = tid; e < RB * 32 * kRedCB * 32; e += 256) {
    const int a = e / (kRedCB * 32), hj = cb0 * 32 + e % (kRedCB * 32);
    if (a < H && hj < HP) part[static_cast<int64_t>(blockIdx.x) * H * HP + a * HP + hj] = red[a][hj - cb0 * 32];
  }
}

// out[o] = sum over chunks of part[chunk][o]: one wave per output, lane k adding chunks k, k+64,
// ... in order, then a fixed shuffle tree (the same order on every call).
__global__ __launch_bounds__(256) void head_reduce_sum_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                              int n, int nchunks) {
  const int o = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (o >= n) return;
  float s = 0.f;
  for (int k = lane; k < nchunks; k += 64) s += part[static_cast<int64_t>(k) * n + o];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) out[o] = s;
}

struct RedPlan {
  int groups, nchunks, tpc;
};

RedPlan red_plan(int ntok, int H, int P) {
  RedPlan p{};
  const int cbs = (H * P + 31) / 32;
  p.groups = (cbs + kRedCB - 1) / kRedCB;
  const int target = std::max(1, kRedChunkTarget / p.groups);
  const int ntok1 = std::max(ntok, 1);
  p.tpc = std::max(4, (ntok1 + target - 1) / target);
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
  if ((d != 64 && d != 128) || H > 64) return hipErrorInvalidValue;
  const RedPlan p = red_plan(ntok, H, P);
  const dim3 grid(p.nchunks, p.groups);
  auto go = [&](auto kern, const auto* b) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, A, lda, b, part, ntok, H, P, p.tpc);
  };
  const half_t* bh = static_cast<const half_t*>(Bm);
  const float* bf = static_cast<const float*>(Bm);
  const bool two = H > 32;
  if (d == 64) {
    if (b_half) two ? go(head_reduce_kernel<half_t, 64, 2>, bh) : go(head_reduce_kernel<half_t, 64, 1>, bh);
    else two ? go(head_reduce_kernel<float, 64, 2>, bf) : go(head_reduce_kernel<float, 64, 1>, bf);
  } else {
    if (b_half) two ? go(head_reduce_kernel<half_t, 128, 2>, bh) : go(head_reduce_kernel<half_t, 128, 1>, bh);
    else two ? go(head_reduce_kernel<float, 128, 2>, bf) : go(head_reduce_kernel<float, 128, 1>, bf);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = H * H * P;
  hipLaunchKernelGGL(head_reduce_sum_kernel, dim3((n + 3) / 4), dim3(256), 0, s, part, out, n, p.nchunks);
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
