// Step 3 of Algorithm 1 ("Interleaved Head Attention" page, section 4): per-head
// attention over the P*N stacked rows, softmax(Q-bar K-bar^T / sqrt(d)) V-bar, with the
// visibility rules of the textbook chapter "Attention mechanism" (section 5.3: softmax
// over each query's allowed set, eq. 5.11; causal set j <= i) and the IHA page's
// sliding window (figure 1) on the interleaved stacked position.
//
// Flash-style: the PN x PN score matrix is never formed (the textbook's eq. 5.35 shows
// why); key tiles stream through LDS and each query row keeps a running maximum and
// sum (the shift invariance of softmax, textbook section 5.2, makes the rescaling exact).
// Scores are kept in base 2: s2 = (q . k) * log2(e)/sqrt(d), p = exp2(s2 - max).
//
// A valid query always sees itself (window >= 1 is checked on the host), so its sum is
// at least 1; a row whose sum is zero is reported through the flag word, never divided.
#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

// ------------------------------------------------------------ fp16 matrix-core kernel
//
// Workgroup: 4 waves x 32 query rows = 128 rows of one (b, h); key tiles of 64.
// Per wave and key tile:
//   S^T[64 keys][32 queries] = K_tile * Q^T      two 32x32 blocks, d/16 steps each
//   O^T[d][32 queries]      += V^T_tile * P^T     d/32 blocks, 4 steps each
// With S^T as the product, lane l owns query l%32 and 16 keys of each 32-key block,
// so a row maximum needs one exchange with lane l^32.  Row i of the K operand is
// taken from key sigma(i) so that lane half hf holds keys 16*hf + 0..15 in order;
// those registers are then exactly the B operand (P^T) of the V product, whose A
// operand (V^T) is read as 8 consecutive keys of one channel from LDS.
constexpr int ABM = 128;
constexpr int ABN = 64;
constexpr int AThreads = 256;

__device__ __forceinline__ int sigma_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <int MASK>
__device__ __forceinline__ bool visible(int q, int k, int L, int window) {
  if (k >= L) return false;
  if (MASK == kMaskCausal) return k <= q;
  if (MASK == kMaskWindow) return k <= q && k > q - window;
  return true;
}

template <int DH>
struct AttnSmem {
  static constexpr int KLD = DH + 8;   // K tile row stride (halves)
  static constexpr int VLD = ABN + 8;  // V^T tile row stride (halves)
  half_t k[ABN * KLD];
  half_t v[DH * VLD];
};

template <int DH>
__device__ __forceinline__ void attn_load_tile(const half_t* __restrict__ Kb,
                                               const half_t* __restrict__ Vb, int64_t rs, int L,
                                               int k0, uint4 (&kr)[DH / 32], uint4 (&vr)[DH / 32]) {
  const int tid = threadIdx.x;
  constexpr int KCH = DH / 8;  // 16-byte chunks per K row
#pragma unroll
  for (int p = 0; p < DH / 32; ++p) {
    const int idx = tid + AThreads * p;
    const int row = idx / KCH, ch = idx % KCH;
    const int key = k0 + row;
    kr[p] = key < L ? *reinterpret_cast<const uint4*>(Kb + key * rs + ch * 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int p = 0; p < DH / 32; ++p) {
    const int idx = tid + AThreads * p;
    const int crow = idx / (ABN / 8), ch = idx % (ABN / 8);
    const int key = k0 + ch * 8;
    const half_t* src = Vb + static_cast<int64_t>(crow) * L + key;
    if (key + 8 <= L && (L & 7) == 0) {
      vr[p] = *reinterpret_cast<const uint4*>(src);
    } else {
      uint16_t e[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        e[q] = (key + q < L) ? __builtin_bit_cast(uint16_t, src[q]) : static_cast<uint16_t>(0);
      vr[p] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                         e[6] | (e[7] << 16));
    }
  }
}

template <int DH>
__device__ __forceinline__ void attn_store_tile(AttnSmem<DH>& sm, const uint4 (&kr)[DH / 32],
                                                const uint4 (&vr)[DH / 32]) {
  const int tid = threadIdx.x;
  constexpr int KCH = DH / 8;
#pragma unroll
  for (int p = 0; p < DH / 32; ++p) {
    const int idx = tid + AThreads * p;
    *reinterpret_cast<uint4*>(&sm.k[(idx / KCH) * AttnSmem<DH>::KLD + (idx % KCH) * 8]) = kr[p];
    *reinterpret_cast<uint4*>(&sm.v[(idx / (ABN / 8)) * AttnSmem<DH>::VLD + (idx % (ABN / 8)) * 8]) = vr[p];
  }
}

template <int DH, int MASK>
__global__ __launch_bounds__(AThreads, 2) void attn_fwd_f16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnSmem<DH> sm;
  constexpr int KLD = AttnSmem<DH>::KLD, VLD = AttnSmem<DH>::VLD;
  constexpr int NKS = DH / 16;  // k-steps of the score product
  constexpr int NCB = DH / 32;  // 32-channel blocks of the output
  const int L = a.L, H = a.H, window = a.window;
  const int nqt = (L + ABM - 1) / ABM;

  // Flat id -> (b, h, query tile); consecutive logical ids share (b, h) and run on one
  // XCD.  Causal rows get longer with the tile index, so causal launches them longest first.
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt;
  const int qi = lid % nqt;
  const int qt = (MASK == kMaskCausal) ? (nqt - 1 - qi) : qi;
  const int b = bh / H, h = bh % H;
  const int q0 = qt * ABM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int64_t rs = static_cast<int64_t>(H) * DH;  // stride between stacked rows
  const half_t* __restrict__ Qb = static_cast<const half_t*>(a.Q) + static_cast<int64_t>(b) * L * rs + h * DH;
  const half_t* __restrict__ Kb = static_cast<const half_t*>(a.K) + static_cast<int64_t>(b) * L * rs + h * DH;
  const half_t* __restrict__ Vb = static_cast<const half_t*>(a.Vt) + static_cast<int64_t>(b * H + h) * DH * L;
  float* __restrict__ Ob = a.O + static_cast<int64_t>(b) * L * rs + h * DH;

  const int qrow = q0 + w * 32 + l32;
  half8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    if (qrow < L) {
      qf[s] = *reinterpret_cast<const half8*>(Qb + qrow * rs + s * 16 + 8 * hf);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<half_t>(0.f);
    }
  }

  int klo = 0, khi = L;
  if (MASK != kMaskNone) khi = min(L, q0 + ABM);
  if (MASK == kMaskWindow) klo = max(0, q0 - window + 1);
  const int kt0 = klo / ABN, kt1 = (khi + ABN - 1) / ABN;

  const float scale = a.qk_scale;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  floatx16 o[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[cb][r] = 0.f;

  uint4 kr[DH / 32], vr[DH / 32];
  if (kt0 < kt1) {
    attn_load_tile<DH>(Kb, Vb, rs, L, kt0 * ABN, kr, vr);
    attn_store_tile<DH>(sm, kr, vr);
  }
  __syncthreads();

  const int krow = sigma_row(l32);
  for (int kt = kt0; kt < kt1; ++kt) {
    const int k0 = kt * ABN;
    if (kt + 1 < kt1) attn_load_tile<DH>(Kb, Vb, rs, L, k0 + ABN, kr, vr);

    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const half8 kf = *reinterpret_cast<const half8*>(&sm.k[(kb * 32 + krow) * KLD + ks * 16 + 8 * hf]);
        s[kb] = mfma32(kf, qf[ks], s[kb]);
      }
    }

    // Visibility: only tiles that cross a mask edge or the end of the sequence test keys.
    bool edge = (k0 + ABN > L);
    if (MASK != kMaskNone) edge |= (k0 + ABN - 1 > q0);
    if (MASK == kMaskWindow) edge |= (k0 <= q0 + ABM - 1 - window);
    if (edge) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 16 * hf + r;
          if (!visible<MASK>(qrow, key, L, window)) s[kb][r] = -__builtin_inff();
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    // A row with nothing visible yet keeps m = -inf; its terms use offset 0 so that
    // exp2(-inf - (-inf)) never happens.
    const float m_off = (m_new == -__builtin_inff()) ? 0.f : m_new * scale;
    const float alpha = fast_exp2(m_run * scale - m_off);
    float psum = 0.f;
    half8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kb][r], scale, -m_off));
        psum += p;
        pf[kb][r >> 3][r & 7] = static_cast<half_t>(p);
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const half8 vf = *reinterpret_cast<const half8*>(
              &sm.v[(cb * 32 + l32) * VLD + kb * 32 + 16 * hf + 8 * s2]);
          o[cb] = mfma32(vf, pf[kb][s2], o[cb]);
        }

    __syncthreads();
    if (kt + 1 < kt1) {
      attn_store_tile<DH>(sm, kr, vr);
      __syncthreads();
    }
  }

  const float lt = l_run + __shfl_xor(l_run, 32);
  if (qrow < L) {
    float inv = 0.f;
    if (lt > 0.f) {
      inv = 1.f / lt;
    } else if (a.flag) {
      atomicOr(a.flag, kFlagEmptyRow);
    }
    float* orow = Ob + qrow * rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[cb][4 * q + e] * inv;
        *reinterpret_cast<floatx4*>(orow + cb * 32 + 8 * q + 4 * hf) = v;
      }
  }
}

// ------------------------------------------------------------ fp32 kernel (VALU)
// One thread per query row; the wave walks the union of its rows' key ranges so that
// every lane reads the same key (broadcast loads), and masks per lane.
template <int DH, int MASK>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(AttnArgs a) {
  const int L = a.L, H = a.H, window = a.window;
  const int b = blockIdx.z, h = blockIdx.y;
  const int i = blockIdx.x * 64 + threadIdx.x;
  const int64_t rs = static_cast<int64_t>(H) * DH;
  const float* __restrict__ Qb = static_cast<const float*>(a.Q) + static_cast<int64_t>(b) * L * rs + h * DH;
  const float* __restrict__ Kb = static_cast<const float*>(a.K) + static_cast<int64_t>(b) * L * rs + h * DH;
  const float* __restrict__ Vb = static_cast<const float*>(a.Vt) + static_cast<int64_t>(b * H + h) * DH * L;
  const int ic = min(i, L - 1);
  float q[DH], o[DH];
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    q[c] = Qb[ic * rs + c];
    o[c] = 0.f;
  }
  const int i_first = blockIdx.x * 64;
  const int i_last = min(L - 1, i_first + 63);
  int klo = 0, khi = L;  // union over the wave's rows
  if (MASK != kMaskNone) khi = i_last + 1;
  if (MASK == kMaskWindow) klo = max(0, i_first - window + 1);
  const float scale = a.qk_scale;
  float m = -__builtin_inff(), l = 0.f;
  for (int k = klo; k < khi; ++k) {
    if (!visible<MASK>(i, k, L, window) || i >= L) continue;
    float dot = 0.f;
#pragma unroll
    for (int c = 0; c < DH; ++c) dot = fmaf(q[c], Kb[k * rs + c], dot);
    const float s = dot * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = fast_exp2(m - m_new);
    const float p = fast_exp2(s - m_new);
    l = fmaf(l, alpha, p);
#pragma unroll
    for (int c = 0; c < DH; ++c) o[c] = fmaf(o[c], alpha, p * Vb[static_cast<int64_t>(c) * L + k]);
    m = m_new;
  }
  if (i >= L) return;
  float inv = 0.f;
  if (l > 0.f) {
    inv = 1.f / l;
  } else if (a.flag) {
    atomicOr(a.flag, kFlagEmptyRow);
  }
  float* orow = a.O + static_cast<int64_t>(b) * L * rs + h * DH + i * rs;
#pragma unroll
  for (int c = 0; c < DH; ++c) orow[c] = o[c] * inv;
}

template <int DH, int MASK>
hipError_t launch_f16_impl(const AttnArgs& a, hipStream_t s) {
  const int nqt = (a.L + ABM - 1) / ABM;
  hipLaunchKernelGGL((attn_fwd_f16_kernel<DH, MASK>), dim3(nqt * a.H * a.B), dim3(AThreads), 0, s, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_f16_mask(const AttnArgs& a, hipStream_t s) {
  switch (a.mask) {
    case kMaskNone: return launch_f16_impl<DH, kMaskNone>(a, s);
    case kMaskCausal: return launch_f16_impl<DH, kMaskCausal>(a, s);
    default: return launch_f16_impl<DH, kMaskWindow>(a, s);
  }
}

template <int DH, int MASK>
hipError_t launch_f32_impl(const AttnArgs& a, hipStream_t s) {
  const dim3 grid((a.L + 63) / 64, a.H, a.B);
  hipLaunchKernelGGL((attn_fwd_f32_kernel<DH, MASK>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_f32_mask(const AttnArgs& a, hipStream_t s) {
  switch (a.mask) {
    case kMaskNone: return launch_f32_impl<DH, kMaskNone>(a, s);
    case kMaskCausal: return launch_f32_impl<DH, kMaskCausal>(a, s);
    default: return launch_f32_impl<DH, kMaskWindow>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_f16(const AttnArgs& a, hipStream_t s) {
  switch (a.d) {
    case 64: return launch_f16_mask<64>(a, s);
    case 128: return launch_f16_mask<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_f32(const AttnArgs& a, hipStream_t s) {
  switch (a.d) {
    case 16: return launch_f32_mask<16>(a, s);
    case 32: return launch_f32_mask<32>(a, s);
    case 64: return launch_f32_mask<64>(a, s);
    case 128: return launch_f32_mask<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace iha
