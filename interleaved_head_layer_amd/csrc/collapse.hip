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
  int T0;  // matrix-core kernel: a sequence's first T0 tokens include fp32 rows
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

// fp16 stacked outputs on the matrix cores (H <= 32, d = 64 or 128).  Per token the
// collapse is the product out[h][c] = sum_q Rt[h][q] * Pbar[q][c] over the token's H*P stacked
// values q = j*H + h' (Rt[h][q] = R[h][h'*P + j]); a wave computes one 32-channel block of
// one token with v_mfma_f32_32x32x16_f16: A = Rt (rows h, zero for h >= H), B = the token's
// stacked block, K = q in steps of 16 (zero past H*P).  R is split into fp16 hi + lo parts
// (two products on the exact fp16 stacked values), so the result carries about 2^-22
// relative rounding on top of fp32 accumulation.  The workgroup (d/32 waves) stages each
// token's [H*P][d] fp16 block in LDS (row stride d + 4 halves: the operand reads of rows q
// and q + 8 fall on disjoint banks) and reads B transposed, 8 consecutive q per lane; the
// next token's block is loaded into registers while the current one is multiplied.
// A token whose stacked rows include fp32 rows (stacked rows i < R of a sequence: its first
// T0 = ceil(R / P) tokens) is staged as two fp16 blocks, the high and low parts of each fp32
// value (low part zero for its fp16 rows), and takes a third product Rt_hi * low; these
// tokens come first, one at a time per workgroup.
template <int KS, int NW>
__global__ __launch_bounds__(NW * 64, 2) void collapse_mfma_kernel(CollapseSrc src, const float* __restrict__ R,
                                                               float* __restrict__ out, int ntok, int H, int P,
                                                               int d) {
  constexpr int NT = NW * 64;
  extern __shared__ __attribute__((aligned(16))) uint16_t pl[];  // 2 x [KS*16][d + 4]: value, low part
  const int HP = H * P, ld = d + 4, N = src.N, T0 = src.T0;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  uint16_t* pl2 = pl + KS * 16 * ld;

  // Rows HP .. KS*16-1 stay zero (their A columns are zero too, but LDS must hold no NaN).
  for (int i = HP * ld + tid; i < KS * 16 * ld; i += NT) pl[i] = pl2[i] = 0;
  half8 ah[KS], al[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = ks * 16 + 8 * hf + e;
      const float v = (l32 < H && q < HP) ? R[l32 * HP + (q % H) * P + q / H] : 0.f;
      ah[ks][e] = static_cast<half_t>(v);
      al[ks][e] = static_cast<half_t>(v - static_cast<float>(ah[ks][e]));
    }
  const int c0 = w * 32;
  const int cpr = d / 8;     // 16-byte chunks per stacked row
  const int nch = HP * cpr;  // chunks per token (<= KS * NT)
  auto store_out = [&](int tok, const floatx16& acc) {
    float* dst = out + static_cast<int64_t>(tok) * H * d + c0 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (h < H) dst[static_cast<int64_t>(h) * d] = acc[r];
    }
  };

  // Tokens with fp32 rows: high/low fp16 blocks, three products per k-step.
  const int nearly = (ntok / N) * T0;
  for (int e = blockIdx.x; e < nearly; e += gridDim.x) {
    const int tok = (e / T0) * N + e % T0, t = e % T0;
    const int64_t eb = static_cast<int64_t>(tok / N) * src.R;
    for (int ch = tid; ch < nch; ch += NT) {
      const int q = ch / cpr, c8 = (ch % cpr) * 8;
      const int i = t * P + q / H;
      half8 hi, lo;
      if (i < src.R) {
        const float* p = src.Pe + ((eb + i) * H + q % H) * d + c8;
        const floatx4 a = *reinterpret_cast<const floatx4*>(p), b = *reinterpret_cast<const floatx4*>(p + 4);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float v = k < 4 ? a[k] : b[k - 4];
          hi[k] = static_cast<half_t>(v);
          lo[k] = static_cast<half_t>(v - static_cast<float>(hi[k]));
        }
      } else {
        hi = *reinterpret_cast<const half8*>(src.Ph + (static_cast<int64_t>(tok) * HP + q) * d + c8);
#pragma unroll
        for (int k = 0; k < 8; ++k) lo[k] = static_cast<half_t>(0.f);
      }
      uint2* dh = reinterpret_cast<uint2*>(pl + q * ld + c8);  // 8-byte aligned
      uint2* dl = reinterpret_cast<uint2*>(pl2 + q * ld + c8);
      const uint4 hb = __builtin_bit_cast(uint4, hi), lb = __builtin_bit_cast(uint4, lo);
      dh[0] = make_uint2(hb.x, hb.y);
      dh[1] = make_uint2(hb.z, hb.w);
      dl[0] = make_uint2(lb.x, lb.y);
      dl[1] = make_uint2(lb.z, lb.w);
    }
    __syncthreads();
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8 b, b2;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = (ks * 16 + 8 * hf + k) * ld + c0 + l32;
        b[k] = __builtin_bit_cast(half_t, pl[row]);
        b2[k] = __builtin_bit_cast(half_t, pl2[row]);
      }
      acc = mfma32(ah[ks], b, acc);
      acc = mfma32(al[ks], b, acc);
      acc = mfma32(ah[ks], b2, acc);
    }
    __syncthreads();  // the next token's staging overwrites both blocks
    store_out(tok, acc);
  }

  // The other tokens: tok = blockIdx.x + k * gridDim.x with t >= T0, fp16 blocks only.
  const int ng = gridDim.x;
  auto next_tok = [&](int tok) {
    for (tok += ng; tok < ntok && tok % N < T0; tok += ng) {
    }
    return tok;
  };
  int tok = blockIdx.x;
  if (tok < ntok && tok % N < T0) tok = next_tok(tok);
  uint4 buf[KS];
  auto load = [&](int tk) {
    const uint4* blk = reinterpret_cast<const uint4*>(src.Ph + static_cast<int64_t>(tk) * HP * d);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (k * NT + tid < nch) buf[k] = blk[k * NT + tid];
  };
  if (tok < ntok) load(tok);
  while (tok < ntok) {
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int ch = k * NT + tid;
      if (ch < nch) {
        uint2* dst = reinterpret_cast<uint2*>(pl + (ch / cpr) * ld + (ch % cpr) * 8);  // 8-byte aligned
        dst[0] = make_uint2(buf[k].x, buf[k].y);
        dst[1] = make_uint2(buf[k].z, buf[k].w);
      }
    }
    __syncthreads();
    const int nt = next_tok(tok);
    if (nt < ntok) load(nt);
    floatx16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8 b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = __builtin_bit_cast(half_t, pl[(ks * 16 + 8 * hf + e) * ld + c0 + l32]);
      acc = mfma32(ah[ks], b, acc);
      acc = mfma32(al[ks], b, acc);
    }
    __syncthreads();  // the next token's staging overwrites the block
    store_out(tok, acc);
    tok = nt;
  }
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
  const CollapseSrc src{Pbar, nullptr, nullptr, 0, 1, 0};
  return launch_h<false>(src, R, out, ntok, H, P, d, s);
}

hipError_t launch_collapse_h(const half_t* Ph, const float* Pe, int Rrows, const float* R, float* out, int B,
                             int N, int H, int P, int d, hipStream_t s) {
  const int HP = H * P, KS = (HP + 15) / 16;
  // The matrix-core kernel stages two [KS*16][d + 4] fp16 blocks: at most 64 KB of LDS.
  if (H > 32 || KS > 8 || (d != 64 && d != 128) || 2 * KS * 16 * (d + 4) * 2 > 65536) {
    const CollapseSrc src{nullptr, Ph, Pe, Rrows, N, 0};
    return launch_h<true>(src, R, out, B * N, H, P, d, s);
  }
  const CollapseSrc src{nullptr, Ph, Pe, Rrows, N, (Rrows + P - 1) / P};
  const int ntok = B * N;
  // About 8 tokens per workgroup, but at least 1024 workgroups (or one per token) so that a
  // short batch still spreads over every compute unit.
  const int grid = std::max(1, std::min(std::min(ntok, std::max(ntok / 8, 1024)), 256 * 8));
  const size_t lds = 2 * static_cast<size_t>(KS) * 16 * (d + 4) * sizeof(uint16_t);
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), lds, s, src, R, out, ntok, H, P, d);
  };
  switch (KS * 4 + d / 64) {  // d / 64 in {1, 2}
#define IHA_COLLAPSE_CASE(ks)                                                    \
  case ks * 4 + 1: go(collapse_mfma_kernel<ks, 2>, 128); break;                  \
  case ks * 4 + 2: go(collapse_mfma_kernel<ks, 4>, 256); break;
    IHA_COLLAPSE_CASE(1) IHA_COLLAPSE_CASE(2) IHA_COLLAPSE_CASE(3) IHA_COLLAPSE_CASE(4)
    IHA_COLLAPSE_CASE(5) IHA_COLLAPSE_CASE(6) IHA_COLLAPSE_CASE(7) IHA_COLLAPSE_CASE(8)
#undef IHA_COLLAPSE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace iha
