// Full-precision attention for the first stacked rows of every (b, h) under a causal or
// window mask (bf16 inputs).
//
// Why: a stacked row that sees n keys has an output of magnitude about n^-1/2 (it averages
// n value rows with softmax weights), while the fp16 intermediates of the main path carry a
// fixed relative error.  The first rows see only a handful of keys, so their outputs, and
// their absolute errors, are far above the typical output.  The first kPreciseRows (32)
// stacked rows of every (b, h) are recomputed here in fp32 from fp32 copies of their
// projected and mixed queries, keys and values (written by the mixing step) into a
// separate fp32 buffer that the collapse reads for those rows.  Row 32 and later see at
// least 33 keys, so their fp16 errors are already several times below row 0's.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// Attention of the first R stacked rows in fp32 (causal or window mask; a row i sees keys
// i' <= i, so only keys < R <= 128 are involved).  Block: 32 query rows of one (b, h),
// 512 threads; thread t owns row r = t / 16 and lane g = t % 16 of that row's group.
//   scores:  thread (r, g) computes keys kc0 + g + 16u (u < 8) -> the row's scores sit in
//            the 16 lanes of its group, so max and sum are 16-lane shuffles;
//   P V:     thread (r, g) computes channels g + 16u (u < DH / 16).
// All keys the block needs are staged in LDS at once, then (through the same buffer) all
// values, whose global loads are issued into registers before the score phase.
// grid: (ceil(R / 32), H, B).
constexpr int ERows = 32, EThreads = 512, EGroup = 16;
// LDS rows are padded by 4 floats (float4-aligned, consecutive rows on staggered banks).
template <int DH>
struct EarlySmem {
  static constexpr int QS = (DH > kPreciseRows ? DH : kPreciseRows) + 4;  // Q rows, then P rows
  static constexpr int KS = DH + 4;                                       // K[n][c]
  static constexpr int VS = kPreciseRows + 4;                             // V^T[c][n]
  float qs[ERows][QS];
  float kv[kPreciseRows * KS > DH * VS ? kPreciseRows * KS : DH * VS];    // K, then V^T
};

template <int DH>
__global__ __launch_bounds__(EThreads) void early_attn_kernel(EarlyArgs e, float* __restrict__ O,
                                                              int64_t o_bstride, int mask,
                                                              int window, float scale) {
  using Sm = EarlySmem<DH>;
  __shared__ __attribute__((aligned(16))) Sm sm;
  auto& qs = sm.qs;
  float* kv = sm.kv;
  const int R = e.R, H = e.H, D = e.D;
  const int h = blockIdx.y, b = blockIdx.z;
  const int i0 = blockIdx.x * ERows;
  const int tid = threadIdx.x;
  const int r = tid / EGroup, g = tid % EGroup;
  const float* __restrict__ Qb = e.Qe + static_cast<int64_t>(b) * R * D + h * DH;
  const float* __restrict__ Kb = e.Ke + static_cast<int64_t>(b) * R * D + h * DH;
  const float* __restrict__ Vb = e.Ve + static_cast<int64_t>(b) * R * D + h * DH;

  const int khi = min(R, i0 + ERows);  // keys <= the block's last row
  const int klo = mask == kMaskWindow ? max(0, i0 - window + 1) : 0;
  const int kc0 = klo & ~3;
  const int nk = khi - kc0;             // keys staged (<= 128)
  const int nk4 = (nk + 3) & ~3;        // P V contraction length (zero-padded)
  const int nu = (nk + EGroup - 1) / EGroup;  // score columns per thread in use

  // Stage Q (32 rows) and K (nk rows, zero-filled to a multiple of 16) as float4; every
  // global load of the block (Q, K and the values below) is issued before the first wait.
  constexpr int C4 = DH / 4;
  constexpr int QPT = ERows * C4 / EThreads, KPT = kPreciseRows * C4 / EThreads;
  floatx4 qreg[QPT], kreg[KPT];
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int x = tid + q * EThreads, rr = x / C4, c = (x % C4) * 4;
    qreg[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (i0 + rr < R) qreg[q] = *reinterpret_cast<const floatx4*>(Qb + static_cast<int64_t>(i0 + rr) * D + c);
  }
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int x = tid + q * EThreads, n = x / C4, c = (x % C4) * 4;
    kreg[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (n < nk) kreg[q] = *reinterpret_cast<const floatx4*>(Kb + static_cast<int64_t>(kc0 + n) * D + c);
  }
  // Values V[kc0 + n][c] for n < nk4 into registers as float4 over c (zero past nk); they
  // go to LDS transposed (V^T[c][n]) once the scores are done.
  constexpr int VPT = KPT;
  floatx4 vreg[VPT];
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int x = tid + q * EThreads, n = x / C4, c = (x % C4) * 4;
    vreg[q] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (n < nk) vreg[q] = *reinterpret_cast<const floatx4*>(Vb + static_cast<int64_t>(kc0 + n) * D + c);
  }
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int x = tid + q * EThreads;
    *reinterpret_cast<floatx4*>(&qs[x / C4][(x % C4) * 4]) = qreg[q];
  }
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int x = tid + q * EThreads, n = x / C4;
    if (n < nu * EGroup) *reinterpret_cast<floatx4*>(&kv[n * Sm::KS + (x % C4) * 4]) = kreg[q];
  }
  __syncthreads();

  // Scores of row i0 + r against keys kc0 + g + 16u.
  float s[kPreciseRows / EGroup];
#pragma unroll
  for (int u = 0; u < kPreciseRows / EGroup; ++u) s[u] = 0.f;
#pragma unroll 4
  for (int c = 0; c < DH; c += 4) {
    const floatx4 q4 = *reinterpret_cast<const floatx4*>(&qs[r][c]);
#pragma unroll
    for (int u = 0; u < kPreciseRows / EGroup; ++u) {
      if (u < nu) {
        const floatx4 k4 = *reinterpret_cast<const floatx4*>(&kv[(g + EGroup * u) * Sm::KS + c]);
        s[u] = fmaf(q4[0], k4[0], s[u]);
        s[u] = fmaf(q4[1], k4[1], s[u]);
        s[u] = fmaf(q4[2], k4[2], s[u]);
        s[u] = fmaf(q4[3], k4[3], s[u]);
      }
    }
  }
  const int i = i0 + r;
  float mx = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < kPreciseRows / EGroup; ++u) {
    const int k = kc0 + g + EGroup * u;
    const bool vis = u < nu && k < khi && k <= i && (mask != kMaskWindow || k > i - window);
    s[u] = vis ? s[u] * scale : -__builtin_inff();
    mx = fmaxf(mx, s[u]);
  }
#pragma unroll
  for (int off = EGroup / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, EGroup));
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < kPreciseRows / EGroup; ++u) {
    s[u] = (mx == -__builtin_inff()) ? 0.f : fast_exp2(s[u] - mx);  // exp2(-inf) = 0
    sum += s[u];
  }
#pragma unroll
  for (int off = EGroup / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, EGroup);
  const float inv_l = sum > 0.f ? 1.f / sum : 0.f;
  __syncthreads();  // every thread is done reading Q and K

  // P rows (over the staged key range) into qs, V^T into kv.
#pragma unroll
  for (int u = 0; u < kPreciseRows / EGroup; ++u) qs[r][g + EGroup * u] = s[u];
#pragma unroll
  for (int q = 0; q < VPT; ++q) {
    const int x = tid + q * EThreads;
    const int n = x / C4, c = (x % C4) * 4;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) kv[(c + e4) * Sm::VS + n] = vreg[q][e4];
  }
  __syncthreads();

  // O[i][c] = sum_n p[i][n] v[n][c] / l[i] for channels c = g + 16u.
  constexpr int CU = DH / EGroup;
  float acc[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) acc[u] = 0.f;
#pragma unroll 2
  for (int n = 0; n < nk4; n += 4) {
    const floatx4 p4 = *reinterpret_cast<const floatx4*>(&qs[r][n]);
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const floatx4 v4 = *reinterpret_cast<const floatx4*>(&kv[(g + EGroup * u) * Sm::VS + n]);
      acc[u] = fmaf(p4[0], v4[0], acc[u]);
      acc[u] = fmaf(p4[1], v4[1], acc[u]);
      acc[u] = fmaf(p4[2], v4[2], acc[u]);
      acc[u] = fmaf(p4[3], v4[3], acc[u]);
    }
  }
  if (i < R) {
    float* dst = O + static_cast<int64_t>(b) * o_bstride + static_cast<int64_t>(i) * D + h * DH;
#pragma unroll
    for (int u = 0; u < CU; ++u) dst[g + EGroup * u] = acc[u] * inv_l;
  }
}

}  // namespace
}  // namespace iha

namespace iha {
hipError_t launch_early_attn(const EarlyArgs& e, float* O, int64_t o_bstride, int mask, int window,
                             float scale, hipStream_t s) {
  if (e.R <= 0 || e.R > kPreciseRows) return hipErrorInvalidValue;
  const dim3 grid((e.R + ERows - 1) / ERows, e.H, e.B);
  if (e.d == 64)
    hipLaunchKernelGGL(early_attn_kernel<64>, grid, dim3(EThreads), 0, s, e, O, o_bstride, mask,
                       window, scale);
  else if (e.d == 128)
    hipLaunchKernelGGL(early_attn_kernel<128>, grid, dim3(EThreads), 0, s, e, O, o_bstride, mask,
                       window, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}
}  // namespace iha
