// Device-side helpers shared by the IHA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iha {

typedef _Float16 half_t;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_bits;

constexpr int kWave = 64;

// Mask modes on the stacked position (same values as iha_mask_mode).
constexpr int kMaskNone = 0;
constexpr int kMaskCausal = 1;
constexpr int kMaskWindow = 2;

// Bits of the device flag word in the workspace.
constexpr unsigned kFlagEmptyRow = 1u;       // a valid query saw no key
constexpr unsigned kFlagNonFinite = 2u;      // a non-finite value reached the output
constexpr unsigned kFlagRange = 4u;          // an fp16 matrix-core operand left the fp16 range
constexpr unsigned kFlagInputNonFinite = 8u; // a non-finite input value
// Largest finite fp16 magnitude.
constexpr float kF16Max = 65504.f;

__device__ __forceinline__ float bf16_to_float(bf16_bits b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// 32x32x16 fp16 matrix-core product, fp32 accumulate.  Operand layout (wave64):
//   A: lane l supplies A[l % 32][8*(l/32) + 0..7]
//   B: lane l supplies B[8*(l/32) + 0..7][l % 32]
//   D: lane l holds D[8*(r/4) + 4*(l/32) + r%4][l % 32], r = 0..15
__device__ __forceinline__ floatx16 mfma32(half8 a, half8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row of (channel c, source head m) of one weight matrix in the fused layout (H = 16 or 20):
// 8-channel groups of 8H rows; in a group, channel cl's heads m < 16 at rows cl*16 + m and
// (H = 20) its heads 16..19 at rows 128 + cl*4 + (m - 16).
__device__ __forceinline__ int fused_row(int c, int m, int H) {
  return (c >> 3) * (8 * H) + (m < 16 ? (c & 7) * 16 + m : 128 + (c & 7) * 4 + (m - 16));
}

// XCD-aware remap of a flat workgroup id: the hardware deals consecutive
// workgroups round-robin to the 8 XCDs, so consecutive logical ids are given to
// the same XCD (its own L2) instead.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int per = nblocks / kXcd;   // full rounds
  const int full = per * kXcd;
  if (bid >= full) return bid;      // ragged tail keeps its order
  return (bid % kXcd) * per + bid / kXcd;
}

}  // namespace iha
