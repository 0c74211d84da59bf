// Step 3 of Algorithm 1 ("Interleaved Head Attention" page, section 4): per-head
// attention over the P*N stacked rows, softmax(Q-bar K-bar^T / sqrt(d)) V-bar, with the
// visibility rules of the textbook chapter "Attention mechanism" (section 5.3: softmax
// over each query's allowed set, eq. 5.11; causal set j <= i) and the IHA page's
// sliding window (figure 1) on the interleaved stacked position.
//
// Flash-style: the PN x PN score matrix is never formed (the textbook's eq. 5.35 shows
// why); key tiles stream through LDS and each query row keeps a running offset and sum
// (the shift invariance of softmax, textbook section 5.2, makes any offset exact).  Scores
// are kept in base 2: s2 = (q . k) * log2(e)/sqrt(d), p = exp2(s2 - m).  The factor is
// applied to Q as it is loaded (a caller that stored Q pre-scaled passes 1, which is exact).
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
constexpr int AWaves = AThreads / 64;

__device__ __forceinline__ int sigma_row(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

template <int MASK>
__device__ __forceinline__ bool visible(int q, int k, int L, int window) {
  if (k >= L) return false;
  if (MASK == kMaskCausal) return k <= q;
  if (MASK == kMaskWindow) return k <= q && k > q - window;
  return true;
}

// K/V^T tile stages in LDS.  Rows are unpadded; 16-byte chunks are XOR-swizzled by row so
// that the matrix-core operand reads of 16 lanes (16 different rows, same logical chunk)
// hit 16 different bank groups.
template <int DH>
struct AttnSmem {
  static constexpr int KLD = DH;   // K tile row (halves)
  static constexpr int VLD = ABN;  // V^T tile row (halves)
  half_t k[2][ABN * KLD];
  half_t v[2][DH * VLD];
};

// K rows: chunk c of row r sits at position c ^ kswz(r).  The score product reads rows
// sigma(l) of 16 lanes = {0-3, 16-19, 4-7, 20-23} (+8): bits 0-2 and bit 4 of r spread them.
template <int DH>
__device__ __forceinline__ int kswz(int r) {
  return DH == 128 ? ((r & 7) | (((r >> 4) & 1) << 3)) : (r & 7);
}
// V^T rows (64 keys = 128 bytes, two rows per 256-byte bank line): chunk c at c ^ ((r >> 1) & 7).
__device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }

// Copy key tile [k0, k0 + 64) into one stage.  DIRECT: buffer loads straight into LDS (no
// registers; needs L % 8 == 0).  Each lane keeps two 32-bit K offsets (the K swizzle takes
// two values over the rounds) and one V offset; the per-round part is a scalar offset.
// Keys past the end read zero (K rows) or a neighbouring channel row (V^T); both are masked
// out by the caller, so every value in LDS is finite.  Otherwise through registers.
template <int DH, bool DIRECT>
struct TileCopy {
  static constexpr int KCH = DH / 8;                  // 16-byte chunks per K row
  static constexpr int ROUNDS = DH * ABN * 2 / (AThreads * 16);
  static constexpr int KRB = AWaves * 64 / KCH;       // K rows per round
  static constexpr int VRB = AWaves * 64 / (ABN / 8); // V^T rows per round
  uint4 kr[DIRECT ? 1 : ROUNDS], vr[DIRECT ? 1 : ROUNDS];
  __amdgpu_buffer_rsrc_t krs, vrs;
  unsigned koff[2], voff;
  int64_t rs, cs;  // K: halves between keys and between 16-byte d-chunks
  int L;

  // kbytes: bytes of K readable from Kb (reads past them return zero).
  __device__ __forceinline__ void init(const half_t* Kb, const half_t* Vb, int64_t rs_, int64_t cs_, int L_,
                                       int64_t kbytes) {
    rs = rs_;
    cs = cs_;
    L = L_;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    if (DIRECT) {
      krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Kb), static_cast<short>(0),
                                              static_cast<int>(kbytes), 0x00020000);
      vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(Vb), static_cast<short>(0),
                                              static_cast<int>(static_cast<int64_t>(DH) * L_ * 2), 0x00020000);
      const int rl = (w * 64 + lane) / KCH, pos = (w * 64 + lane) % KCH;
#pragma unroll
      for (int bit = 0; bit < 2; ++bit) {
        const int sw = (rl & 7) | ((DH == 128 ? bit : 0) << 3);
        koff[bit] = static_cast<unsigned>((rl * rs_ + (pos ^ sw) * cs_) * 2);
      }
      const int cl = (w * 64 + lane) / (ABN / 8), vpos = (w * 64 + lane) % (ABN / 8);
      voff = static_cast<unsigned>((static_cast<int64_t>(cl) * L_ + (vpos ^ vswz(cl)) * 8) * 2);
    }
  }

  __device__ __forceinline__ void issue(const half_t* __restrict__ Kb, const half_t* __restrict__ Vb,
                                        int k0, half_t* kst, half_t* vst) {
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
#pragma unroll
    for (int p = 0; p < ROUNDS; ++p) {
      if (DIRECT) {
        // K row p*KRB + rl: swizzle bit 3 is bit 4 of the row, i.e. (p*KRB >> 4) & 1.
        const int bit = ((p * KRB) >> 4) & 1;
        const unsigned ks_off = static_cast<unsigned>((k0 + p * KRB) * rs * 2);
        const unsigned vs_off = static_cast<unsigned>((static_cast<int64_t>(p) * VRB * L + k0) * 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(kst + (p * AWaves + w) * 512),
                                                 16, koff[bit], ks_off, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(vst + (p * AWaves + w) * 512),
                                                 16, voff, vs_off, 0, 0);
      } else {
        const int slot = (p * AWaves + w) * 64 + lane;
        const int r = slot / KCH, pos = slot % KCH;
        const int key = min(k0 + r, L - 1);
        kr[p] = *reinterpret_cast<const uint4*>(Kb + key * rs + (pos ^ kswz<DH>(r)) * cs);
        const int cr = slot / (ABN / 8), vpos = slot % (ABN / 8);
        const int vkey = k0 + (vpos ^ vswz(cr)) * 8;
        const half_t* vsrc = Vb + static_cast<int64_t>(cr) * L + vkey;
        uint16_t e[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          e[q] = (vkey + q < L) ? __builtin_bit_cast(uint16_t, vsrc[q]) : static_cast<uint16_t>(0);
        vr[p] = make_uint4(e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                           e[6] | (e[7] << 16));
      }
    }
  }
  // Registers -> LDS (register path only).
  __device__ __forceinline__ void commit(half_t* kst, half_t* vst) {
    if (DIRECT) return;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int p = 0; p < ROUNDS; ++p) {
      const int slot = (p * AWaves + w) * 64 + lane;
      *reinterpret_cast<uint4*>(kst + slot * 8) = kr[p];
      *reinterpret_cast<uint4*>(vst + slot * 8) = vr[p];
    }
  }
};

__device__ __forceinline__ void wait_global_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Running softmax state of one lane (one query row, shared with lane l^32).
template <int NCB>
struct RowState {
  float m;          // stale running maximum of the base-2 scores (-inf before any visible key)
  float l;          // this lane's share of the running sum
  floatx16 o[NCB];  // O^T accumulators
};

// Probabilities are computed against the row's current offset m (stale maximum) without a
// per-tile maximum: the lane's tile sum decides.  A sum <= 2^12 bounds every p by 2^12, well
// inside fp16; a larger (or non-finite) sum, or a row with no offset yet, takes the slow
// path that moves m to the row maximum.  Shift invariance of softmax (any subtracted constant
// cancels in the normalisation) makes every such offset exact.  Q is pre-scaled by
// log2(e)/sqrt(d), so scores are base 2; the score product starts from the accumulator -m,
// so its output is already s - m and feeds exp2 directly.
constexpr float kTileSumMax = 4096.f;

typedef float floatx2 __attribute__((ext_vector_type(2)));
template <int DH, int MASK>
__device__ __forceinline__ void attn_tile(bool edge, const half_t* __restrict__ ks, const half_t* __restrict__ vs,
                                          const half8 (&qf)[DH / 16], RowState<DH / 32>& st, floatx16& negm,
                                          int k0, int qrow, int L, int window, int krow, int l32, int hf) {
  constexpr int KLD = AttnSmem<DH>::KLD, VLD = AttnSmem<DH>::VLD;
  constexpr int NKS = DH / 16, NCB = DH / 32;
  // K fragments i = kstep * 2 + kb, read kPre ahead of their product; the first kPre V^T
  // fragments are read after the score product so they arrive during the softmax.
  // Wave priority: the softmax runs at 0; each product phase starts at 1 (score) or 0 (PV)
  // and rises to 3 halfway, so of the two waves sharing a SIMD the one further into its
  // products keeps the matrix core and the other's products wait.  The waves then drift
  // into opposite phases (one's softmax under the other's products) instead of running
  // their products and their softmax at the same time.
  constexpr int NK = 2 * NKS, kPre = 4;
  auto kfrag = [&](int i) {
    const int kr_ = (i & 1) * 32 + krow;
    return *reinterpret_cast<const half8*>(&ks[kr_ * KLD + (((i >> 1) * 2 + hf) ^ kswz<DH>(kr_)) * 8]);
  };
  auto vfrag = [&](int j) {  // j = (kb * 2 + s2) * NCB + cb
    const int cb = j % NCB, ks2 = j / NCB;
    const int vr_ = cb * 32 + l32;
    return *reinterpret_cast<const half8*>(&vs[vr_ * VLD + (((ks2 >> 1) * 4 + 2 * hf + (ks2 & 1)) ^ vswz(vr_)) * 8]);
  };
  half8 kr[NK];
#pragma unroll
  for (int i = 0; i < kPre; ++i) kr[i] = kfrag(i);
  __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(1); __builtin_amdgcn_sched_barrier(0);
  floatx16 s[2];
  constexpr int HK = NK / 2;
#pragma unroll
  for (int i = 0; i < HK; ++i) {
    kr[i + kPre] = kfrag(i + kPre);
    s[i & 1] = mfma32(kr[i], qf[i >> 1], i < 2 ? negm : s[i & 1]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
#pragma unroll
  for (int i = 0; i < HK; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = HK; i < NK; ++i) {
    if (i + kPre < NK) kr[i + kPre] = kfrag(i + kPre);
    s[i & 1] = mfma32(kr[i], qf[i >> 1], s[i & 1]);
  }
  constexpr int NV = 4 * NCB;
  half8 vr[NV];
#pragma unroll
  for (int j = 0; j < kPre; ++j) vr[j] = vfrag(j);
#pragma unroll
  for (int i = HK; i < NK; ++i) {
    if (i + kPre < NK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
  __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
  if (__builtin_expect(edge, false)) {
    // Key k0 + 32 kb + 16 hf + r is visible for r in [lo, lo + n): the same rule as visible(),
    // as one unsigned range test per element.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int base = k0 + kb * 32 + 16 * hf;
      const int last = (MASK == kMaskNone ? L - 1 : min(qrow, L - 1)) - base;
      const int lo = max(MASK == kMaskWindow ? qrow - window + 1 - base : 0, 0);
      const unsigned n = static_cast<unsigned>(max(min(last, 15) + 1 - lo, 0));
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (static_cast<unsigned>(r - lo) >= n) s[kb][r] = -__builtin_inff();
    }
  }
  half8 pf[2][2];
  // Row sums in fp32 from the unrounded probabilities: plain adds overlap the matrix-core
  // products, whereas a packed fp16 dot product stalls them (measured on gfx950).
  auto probs = [&]() __attribute__((always_inline)) {
    float psum0 = 0.f, psum1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const floatx2 e2 = {fast_exp2(s[kb][r]), fast_exp2(s[kb][r + 1])};
        const half2v pr = __builtin_convertvector(e2, half2v);
        pf[kb][r >> 3][r & 7] = pr[0];
        pf[kb][r >> 3][(r & 7) + 1] = pr[1];
        // (the sums start from the first terms rather than from 0 + them: one add fewer each)
        psum0 = kb == 0 && r == 0 ? e2[0] : psum0 + e2[0];
        psum1 = kb == 0 && r == 0 ? e2[1] : psum1 + e2[1];
      }
    return psum0 + psum1;
  };
  // Slow path: a row without an offset yet (its first visible keys), or a tile whose
  // probabilities relative to the offset grew past 2^12 in sum (some p > 2^7 could approach
  // the fp16 range), or a non-finite sum.  The offset then moves to the row maximum and O
  // and l are rescaled; otherwise the tile never computes a maximum at all.
  float tsum = probs();
  const bool unset = st.m == -__builtin_inff();
  if (__builtin_expect(__any(unset || !(tsum <= kTileSumMax)), 0)) {
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(fmaxf(mx, __uint_as_float(sw[0])), __uint_as_float(sw[1]));
    }
    // Each row decides from its own scores: a row without an offset takes its maximum; a row
    // with one moves it only if one of its two lane sums exceeded 2^12 (not merely because
    // another row of the wave needed the slow path), so rows never affect one another's
    // rounding.  (The swap returns this lane's and the other lane's sum in an order that
    // depends on the lane half; their maximum does not care.)
    const auto tw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tsum), __float_as_uint(tsum), false, false);
    const float thi = fmaxf(__uint_as_float(tw[0]), __uint_as_float(tw[1]));
    const bool need = unset ? (mx > -__builtin_inff()) : !(thi <= kTileSumMax);
    const float delta = need ? mx : 0.f;
    const float alpha = !need ? 1.f : unset ? 0.f : fast_exp2(-mx);
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[cb][r] *= alpha;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
    if (need) st.m = unset ? mx : st.m + mx;
    const float nm = st.m == -__builtin_inff() ? 0.f : -st.m;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = nm;
    tsum = probs();
  }
  st.l += tsum;
  __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
  constexpr int HV = NV / 2;
#pragma unroll
  for (int j = 0; j < HV; ++j) {
    vr[j + kPre] = vfrag(j + kPre);
    const int ks2 = j / NCB;
    st.o[j % NCB] = mfma32(vr[j], pf[ks2 >> 1][ks2 & 1], st.o[j % NCB]);
  }
#pragma unroll
  for (int j = 0; j < HV; ++j) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = HV; j < NV; ++j) {
    if (j + kPre < NV) vr[j + kPre] = vfrag(j + kPre);
    const int ks2 = j / NCB;
    st.o[j % NCB] = mfma32(vr[j], pf[ks2 >> 1][ks2 & 1], st.o[j % NCB]);
  }
#pragma unroll
  for (int j = HV; j < NV; ++j) {
    if (j + kPre < NV) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------------ fp32 first rows
// The first R <= kPreciseRows stacked rows of a (b, h) see the fewest keys, so their outputs
// are the largest and the fp16 roundings of the tiled kernel weigh most there (an output that
// averages n value rows is about n^-1/2 in size).  bf16 forwards compute them again in fp32
// on B*H extra workgroups at the end of the fp16 kernel's grid (one per (b, h), 256
// threads).  Their mixed queries, keys and values come as fp32 copies, or are mixed here in
// fp32 from the unmixed projections of the first tokens (Algorithm 1's mixing, one head h).
// Row i sees keys i' <= i (causal) or i - window < i' <= i, so only keys < R take part.
// Thread t owns row r = t / 8 and lane g = t % 8 of the row's group: the scores of keys
// g + 8u, then output channels g + 8u; a row's maximum and sum are 8-lane shuffles.
constexpr int EGroup = 8;
template <int DH, int MASK>
__device__ __forceinline__ void first_rows(const AttnArgs& a, int b, int h, float* smem) {
  constexpr int ER = kPreciseRows;                                 // rows and keys, at most
  constexpr int QS = (DH > ER ? DH : ER) + 4, KS = DH + 4;          // padded LDS rows (floats)
  constexpr int C4 = DH / 4, NU = ER / EGroup, CU = DH / EGroup;
  static_assert(ER * QS + 2 * ER * KS + 3 * 20 * 2 <= sizeof(AttnSmem<DH>) / 4, "LDS");
  float(*qs)[QS] = reinterpret_cast<float(*)[QS]>(smem);          // Q rows, then probabilities
  float(*ks)[KS] = reinterpret_cast<float(*)[KS]>(smem + ER * QS);  // K rows
  float(*vs)[KS] = reinterpret_cast<float(*)[KS]>(smem + ER * QS + ER * KS);  // V rows
  const int R = a.R, H = a.H, D = H * DH, tid = threadIdx.x, r = tid / EGroup, g = tid % EGroup;
  const floatx4 z = {0.f, 0.f, 0.f, 0.f};
  if (a.Ye) {
    // Q~_{h,j}[t][c] = sum_m alpha[m][h][j] Y^(m)[t][c] for rows i = t*P + j < R; Y^(m)[t][c]
    // sits at Ye[b][t][which*D + fused_row(c, m)], four heads m at a time contiguous.  A
    // thread takes (which, t, 4 channels) items and issues all H loads of one at once.
    const int P = a.P, T0 = a.T0, per = T0 * C4;
    float* as = smem + ER * QS + 2 * ER * KS;  // [which][m < 20][j < 2]: alpha[m][h][j], zero padded
    if (tid < 3 * 20 * 2) {
      const int which = tid / 40, m = (tid / 2) % 20, j = tid % 2;
      const float* al = which == 0 ? a.alpha[0] : which == 1 ? a.alpha[1] : a.alpha[2];
      as[tid] = m < H && j < P ? al[(m * H + h) * P + j] : 0.f;
    }
    __syncthreads();
    for (int it = tid; it < 3 * per; it += AThreads) {
      const int which = it / per, t = (it % per) / C4, c = (it % C4) * 4;
      const float* yt = a.Ye + (static_cast<int64_t>(b) * T0 + t) * 3 * D + which * D;
      floatx4 y[5][4];  // [m / 4][e][m % 4]; groups past H repeat the last one (weight zero)
#pragma unroll
      for (int m4 = 0; m4 < 5; ++m4)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          y[m4][e] = *reinterpret_cast<const floatx4*>(yt + fused_row(c + e, 4 * min(m4, H / 4 - 1), H));
      const float* aw = as + which * 40;
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // P <= 2 on this path
        const int n = t * P + j;
        if (j >= P || n >= R) break;
        floatx4 acc = z;
#pragma unroll
        for (int m4 = 0; m4 < 5; ++m4)
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            const float alpha = aw[(4 * m4 + mm) * 2 + j];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(alpha, y[m4][e][mm], acc[e]);
          }
        float* row = which == 0 ? &qs[n][c] : which == 1 ? &ks[n][c] : &vs[n][c];
        *reinterpret_cast<floatx4*>(row) = acc;
      }
    }
  } else {
    const int64_t base = static_cast<int64_t>(b) * R * D + h * DH;
    for (int it = tid; it < ER * C4; it += AThreads) {
      const int n = it / C4, c = (it % C4) * 4;
      const int64_t off = base + static_cast<int64_t>(n) * D + c;
      *reinterpret_cast<floatx4*>(&qs[n][c]) = n < R ? *reinterpret_cast<const floatx4*>(a.Qe + off) : z;
      *reinterpret_cast<floatx4*>(&ks[n][c]) = n < R ? *reinterpret_cast<const floatx4*>(a.Ke + off) : z;
      *reinterpret_cast<floatx4*>(&vs[n][c]) = n < R ? *reinterpret_cast<const floatx4*>(a.Ve + off) : z;
    }
  }
  __syncthreads();
  float sc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) sc[u] = 0.f;
#pragma unroll 4
  for (int c = 0; c < DH; c += 4) {
    const floatx4 q4 = *reinterpret_cast<const floatx4*>(&qs[r][c]);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const floatx4 k4 = *reinterpret_cast<const floatx4*>(&ks[g + EGroup * u][c]);
      sc[u] = fmaf(q4[0], k4[0], sc[u]);
      sc[u] = fmaf(q4[1], k4[1], sc[u]);
      sc[u] = fmaf(q4[2], k4[2], sc[u]);
      sc[u] = fmaf(q4[3], k4[3], sc[u]);
    }
  }
  // Rows and keys >= R were never written: their scores are discarded here and their
  // probabilities are zero.
  float mx = -__builtin_inff();
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int k = g + EGroup * u;
    const bool vis = k < R && k <= r && (MASK != kMaskWindow || k > r - a.window);
    sc[u] = vis ? sc[u] * a.escale : -__builtin_inff();
    mx = fmaxf(mx, sc[u]);
  }
#pragma unroll
  for (int off = EGroup / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, EGroup));
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    sc[u] = mx == -__builtin_inff() ? 0.f : fast_exp2(sc[u] - mx);  // exp2(-inf) = 0
    sum += sc[u];
  }
#pragma unroll
  for (int off = EGroup / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, EGroup);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  __syncthreads();  // every thread is done reading Q
#pragma unroll
  for (int u = 0; u < NU; ++u) qs[r][g + EGroup * u] = sc[u];
  __syncthreads();
  float acc[CU];
#pragma unroll
  for (int u = 0; u < CU; ++u) acc[u] = 0.f;
  for (int n = 0; n < R; ++n) {
    const float p = qs[r][n];
#pragma unroll
    for (int u = 0; u < CU; ++u) acc[u] = fmaf(p, vs[n][g + EGroup * u], acc[u]);
  }
  if (r < R && a.Xf) {  // fused collapse (see the tiled kernel's epilogue)
    const int P = a.P, t = r / P, j = r % P;
    float* xrow = a.Xf + (static_cast<int64_t>(b) * (a.L / P) + t) * D;
    for (int hh = 0; hh < H; ++hh) {
      const float cf = a.Rm[(hh * H + h) * P + j] * inv;
#pragma unroll
      for (int u = 0; u < CU; ++u) atomicAdd(xrow + hh * DH + g + EGroup * u, cf * acc[u]);
    }
  } else if (r < R) {
    float* dst = a.Pe + static_cast<int64_t>(b) * a.R2 * D + static_cast<int64_t>(r) * D + h * DH;
#pragma unroll
    for (int u = 0; u < CU; ++u) dst[g + EGroup * u] = acc[u] * inv;
  }
}

// One step of the main loop: refill the other stage, process key tile kt from stage STAGE
// (a constant, so every fragment address is a per-lane register plus a fixed offset), wait
// for the copy and meet at the barrier.
template <int DH, int MASK, bool DIRECT, int STAGE>
__device__ __forceinline__ void key_tile(AttnSmem<DH>& sm, TileCopy<DH, DIRECT>& cp, const half_t* __restrict__ Kb,
                                         const half_t* __restrict__ Vb, int kt, int kt1, int r0, int L, int window,
                                         const half8 (&qf)[DH / 16], RowState<DH / 32>& st, floatx16& negm, int qrow,
                                         int krow, int l32, int hf) {
  const int k0 = kt * ABN;
  const bool more = kt + 1 < kt1;
  // The other stage was last read before the previous barrier: refill it now.
  if (more) cp.issue(Kb, Vb, k0 + ABN, sm.k[STAGE ^ 1], sm.v[STAGE ^ 1]);
  // A wave skips tiles that hold no visible key for any of its 32 rows; only tiles that
  // cross a mask edge (for its rows) or the end of the sequence test keys.
  bool edge = (k0 + ABN > L), act = true;
  if (MASK != kMaskNone) {
    act = k0 <= r0 + 31;
    edge |= (k0 + ABN - 1 > r0);
  }
  if (MASK == kMaskWindow) {
    act = act && (k0 + ABN - 1 > r0 - window);
    edge |= (k0 <= r0 + 31 - window);
  }
  if (act) attn_tile<DH, MASK>(edge, sm.k[STAGE], sm.v[STAGE], qf, st, negm, k0, qrow, L, window, krow, l32, hf);
  if (more) cp.commit(sm.k[STAGE ^ 1], sm.v[STAGE ^ 1]);
  wait_global_loads();
  __syncthreads();
}

template <int DH, int MASK, bool DIRECT>
__global__ __launch_bounds__(AThreads, 2) void attn_fwd_f16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) AttnSmem<DH> sm;
  constexpr int NKS = DH / 16;  // k-steps of the score product
  constexpr int NCB = DH / 32;  // 32-channel blocks of the output
  const int L = a.L, H = a.H, window = a.window;
  const int nqt = (L + ABM - 1) / ABM;

  // The last B*H workgroups (they fill the slots the tiled workgroups leave idle at the end):
  // fp32 first rows of one (b, h) each.
  const int ne = MASK != kMaskNone && a.R > 0 ? a.B * H : 0;
  const int nmain = static_cast<int>(gridDim.x) - ne;
  if (MASK != kMaskNone && static_cast<int>(blockIdx.x) >= nmain) {
    const int e = blockIdx.x - nmain;
    first_rows<DH, MASK>(a, e / H, e % H, reinterpret_cast<float*>(&sm));
    return;
  }
  // Flat id -> (b, h, query tile); consecutive logical ids share (b, h) and run on one
  // XCD.  Causal rows get longer with the tile index, so causal launches them longest first.
  const int lid = xcd_remap(blockIdx.x, nmain);
  const int bh = lid / nqt;
  const int qi = lid % nqt;
  const int qt = (MASK == kMaskCausal) ? (nqt - 1 - qi) : qi;
  const int b = bh / H, h = bh % H;
  const int q0 = qt * ABM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int64_t rs = static_cast<int64_t>(H) * DH;  // stride between stacked rows of O
  // Q and K: element (row, 16-byte d-chunk cc) of head (b, h) at base + row*qrs + cc*qcs.
  //   row-major [B][L][H][d]:        base = b*L*H*d + h*d,     qrs = H*d, qcs = 8
  //   chunked   [B][H][d/8][L][8]:   base = (b*H + h)*d*L,     qrs = 8,   qcs = 8*L
  const bool chunked = a.qk_layout == kQKChunked;
  const int64_t qbase = chunked ? static_cast<int64_t>(b * H + h) * DH * L : static_cast<int64_t>(b) * L * rs + h * DH;
  const int64_t qrs = chunked ? 8 : rs, qcs = chunked ? static_cast<int64_t>(8) * L : 8;
  const int64_t kbytes = chunked ? static_cast<int64_t>(DH) * L * 2 : (static_cast<int64_t>(L) * rs - h * DH) * 2;
  const half_t* __restrict__ Qb = static_cast<const half_t*>(a.Q) + qbase;
  const half_t* __restrict__ Kb = static_cast<const half_t*>(a.K) + qbase;
  const half_t* __restrict__ Vb = static_cast<const half_t*>(a.Vt) + static_cast<int64_t>(b * H + h) * DH * L;
  const int64_t obase = static_cast<int64_t>(b) * L * rs + h * DH;

  // Q fragments: all loads in flight at once (rows past the end read the last row, whose
  // results are never stored), then the first K/V tile, then the optional scale.
  const int r0 = q0 + w * 32;  // the wave's first row (wave-uniform)
  const int qrow = r0 + l32;
  const int qload = min(qrow, L - 1);
  half8 qf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qf[s] = *reinterpret_cast<const half8*>(Qb + static_cast<int64_t>(qload) * qrs + (2 * s + hf) * qcs);

  int klo = 0, khi = L;
  if (MASK != kMaskNone) khi = min(L, q0 + ABM);
  if (MASK == kMaskWindow) klo = max(0, q0 - window + 1);
  const int kt0 = klo / ABN, kt1 = (khi + ABN - 1) / ABN;

  TileCopy<DH, DIRECT> cp;
  cp.init(Kb, Vb, qrs, qcs, L, kbytes);
  if (kt0 < kt1) {
    cp.issue(Kb, Vb, kt0 * ABN, sm.k[0], sm.v[0]);
    cp.commit(sm.k[0], sm.v[0]);
  }

  // Base-2 score scale folded into Q (skipped when the caller stored Q pre-scaled).
  if (a.qk_scale != 1.f) {
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s][e] = static_cast<half_t>(static_cast<float>(qf[s][e]) * a.qk_scale);
  }
  floatx16 negm;
#pragma unroll
  for (int r = 0; r < 16; ++r) negm[r] = 0.f;
  RowState<NCB> st;
  st.m = -__builtin_inff();
  st.l = 0.f;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.o[cb][r] = 0.f;
  wait_global_loads();
  __syncthreads();

  const int krow = sigma_row(l32);
  // Two key tiles per iteration, one per LDS stage, so that each tile's stage is a constant.
  for (int kt = kt0; kt < kt1; kt += 2) {
    key_tile<DH, MASK, DIRECT, 0>(sm, cp, Kb, Vb, kt, kt1, r0, L, window, qf, st, negm, qrow, krow, l32, hf);
    if (kt + 1 < kt1)
      key_tile<DH, MASK, DIRECT, 1>(sm, cp, Kb, Vb, kt + 1, kt1, r0, L, window, qf, st, negm, qrow, krow, l32, hf);
  }

  const float lt = st.l + __shfl_xor(st.l, 32);
  if (a.lse && hf == 0 && qrow < L)
    a.lse[static_cast<int64_t>(b * H + h) * L + qrow] = lt > 0.f ? st.m + __log2f(lt) : __builtin_inff();
  if (a.Oh && !a.Xf && r0 >= a.R2) {
    // fp16 outputs of a wave whose rows are all past the fp32 ones: the 32 x d block goes
    // through the wave's own stretch of the idle K/V stages (every copy has landed and every
    // wave has passed the last barrier), so that each store writes 16 contiguous bytes per
    // lane and whole rows per instruction instead of 8-byte pieces of 32 rows.
    constexpr int OLD = DH + 8;  // padded LDS row (halves): the 32 rows' writes spread over the banks
    static_assert(AWaves * 32 * OLD * 2 <= sizeof(AttnSmem<DH>), "LDS");
    half_t* ob = reinterpret_cast<half_t*>(&sm) + w * 32 * OLD;
    float inv = lt;
    if (lt > 0.f) {
      inv = 1.f / lt;
    } else if (lt == 0.f) {
      inv = 0.f;
      if (a.flag && qrow < L) atomicOr(a.flag, kFlagEmptyRow);
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        half4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = static_cast<half_t>(st.o[cb][4 * q + e] * inv);
        *reinterpret_cast<half4*>(ob + l32 * OLD + cb * 32 + 8 * q + 4 * hf) = v;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS in order within the wave
    constexpr int CPR = DH / 8;                          // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < 32 * CPR / 64; ++i) {
      const int idx = i * 64 + lane, row = idx / CPR, ch = idx % CPR;
      const half8 v = *reinterpret_cast<const half8*>(ob + row * OLD + ch * 8);
      if (r0 + row < L) *reinterpret_cast<half8*>(a.Oh + obase + static_cast<int64_t>(r0 + row) * rs + ch * 8) = v;
    }
  } else if (qrow < L) {
    // lt > 0 for every valid row; lt == 0 means nothing was visible (reported, output 0);
    // a NaN sum (non-finite input) is passed through to the output.
    float inv = lt;
    if (lt > 0.f) {
      inv = 1.f / lt;
    } else if (lt == 0.f) {
      inv = 0.f;
      if (a.flag) atomicOr(a.flag, kFlagEmptyRow);
    }
    const int64_t orow = obase + static_cast<int64_t>(qrow) * rs;
    if (a.Xf) {
      // Fused collapse: X~[b][t][hh*d + c] += R[hh][h*P + j] * O[t*P + j][c] for every head hh
      // (rows < R come from the fp32 first-row workgroups).
      if (qrow >= a.R) {
        const int P = a.P, t = qrow / P, j = qrow % P;
        float* xrow = a.Xf + (static_cast<int64_t>(b) * (L / P) + t) * rs;
        for (int hh = 0; hh < H; ++hh) {
          const float cf = a.Rm[(hh * H + h) * P + j] * inv;
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                atomicAdd(xrow + hh * DH + cb * 32 + 8 * q + 4 * hf + e, cf * st.o[cb][4 * q + e]);
        }
      }
    } else if (qrow >= a.R && qrow < a.R2) {  // early rows with fp32 outputs: [B][R2][H][d]
      float* dst = a.Pe + (static_cast<int64_t>(b) * a.R2 + qrow) * rs + h * DH;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          floatx4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = st.o[cb][4 * q + e] * inv;
          *reinterpret_cast<floatx4*>(dst + cb * 32 + 8 * q + 4 * hf) = v;
        }
    } else if (a.Oh) {  // fp16 output
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          half4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = static_cast<half_t>(st.o[cb][4 * q + e] * inv);
          *reinterpret_cast<half4*>(a.Oh + orow + cb * 32 + 8 * q + 4 * hf) = v;
        }
    } else {
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          floatx4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = st.o[cb][4 * q + e] * inv;
          *reinterpret_cast<floatx4*>(a.O + orow + cb * 32 + 8 * q + 4 * hf) = v;
        }
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
  float inv = l;  // NaN passes through
  if (l > 0.f) {
    inv = 1.f / l;
  } else if (l == 0.f) {
    inv = 0.f;
    if (a.flag) atomicOr(a.flag, kFlagEmptyRow);
  }
  const int64_t obs = a.o_bstride ? a.o_bstride : static_cast<int64_t>(L) * rs;
  float* orow = a.O + static_cast<int64_t>(b) * obs + h * DH + i * rs;
#pragma unroll
  for (int c = 0; c < DH; ++c) orow[c] = o[c] * inv;
}

template <int DH, int MASK>
hipError_t launch_f16_impl(const AttnArgs& a, hipStream_t s) {
  const int nqt = (a.L + ABM - 1) / ABM;
  if (a.R < 0 || a.R > kPreciseRows || (a.R > 0 && MASK == kMaskNone)) return hipErrorInvalidValue;
  if (a.R2 < a.R || a.R2 > a.L || (a.R2 > a.R && !a.Pe)) return hipErrorInvalidValue;
  const int ne = a.R > 0 ? a.H * a.B : 0;  // first-row workgroups
  const dim3 grid(ne + nqt * a.H * a.B);
  // Buffer loads: 16-byte aligned V^T rows (L % 8 == 0) and 32-bit byte offsets within one
  // batch's K and one head's V^T.
  const bool direct = a.L % 8 == 0 && static_cast<int64_t>(a.L) * a.H * DH * 2 < (int64_t{1} << 31);
  if (direct)
    hipLaunchKernelGGL((attn_fwd_f16_kernel<DH, MASK, true>), grid, dim3(AThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_f16_kernel<DH, MASK, false>), grid, dim3(AThreads), 0, s, a);
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
