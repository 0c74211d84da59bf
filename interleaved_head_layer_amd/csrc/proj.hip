// Steps 1-2 of Algorithm 1 ("Interleaved Head Attention" page, section 4) for bf16 inputs:
// the per-head projections X W^(m) as exact bf16 matrix-core GEMMs with fp32 accumulation,
// followed by the pseudo-head mixing Q~_{h,j} = sum_m alpha^Q_{m,h,j} (X W_Q^(m)) in fp32,
// written straight into the stacked layouts the attention step reads.
//
//   wprep   Wt[which*D + n][k] = W_which[k][n]            (bf16, the contraction index k
//                                                          contiguous for the matrix cores)
//   gemm    Y_QK [M][2D]  = X Wt_{Q,K}^T  (token-major)    fp32
//           Y_V^T [D][M]  = Wt_V X^T      (channel-major)  fp32
//   mix_qk  Q~, K~ [B][P*N][H][d] fp16, rows t*P + j
//   mix_v   V~^T  [B][H][d][P*N]  fp16
// The first T0 tokens of every sequence also get fp32 copies (Qe, Ke, Ve) for the
// full-precision first rows.
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------- W transpose
// grid: (D/64, D/64, 3); block 256.  64x64 tiles through LDS, 16-byte global loads and
// stores (8 bf16 per thread and access).  With `cm`, column n = m*d + c of W (head m,
// channel c) goes to row fused_row(c, m) instead of row n (the fused mixing wants the
// source heads of 8 channels in one wave's rows).
__global__ __launch_bounds__(256) void wprep_kernel(ProjArgs pa, int cm) {
  __shared__ uint16_t t[64][64 + 2];  // [k][n]; the pad staggers the column reads
  const int which = blockIdx.z;
  const uint16_t* __restrict__ W = pa.W[which];
  const int D = pa.D, d = pa.d, H = pa.H;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const int tid = threadIdx.x;
  // The forward's status word starts at zero: this is its first kernel.
  if (pa.flag && (blockIdx.x | blockIdx.y | blockIdx.z | tid) == 0) *pa.flag = 0u;
#pragma unroll
  for (int q = 0; q < 2; ++q) {  // 64 rows of 8 x 16 bytes
    const int x = tid + 256 * q, r = x >> 3, c8 = (x & 7) * 8;
    const uint4 v = *reinterpret_cast<const uint4*>(W + static_cast<int64_t>(k0 + r) * D + n0 + c8);
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[r][c8 + 2 * e] = static_cast<uint16_t>(w4[e] & 0xFFFFu);
      t[r][c8 + 2 * e + 1] = static_cast<uint16_t>(w4[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* __restrict__ Wt = pa.Wt + static_cast<int64_t>(which) * D * D;
#pragma unroll
  for (int q = 0; q < 2; ++q) {  // 64 output rows (n) of 8 x 16 bytes (k)
    const int x = tid + 256 * q, r = x >> 3, k8 = (x & 7) * 8;
    const int n = n0 + r;
    const int row = cm ? fused_row(n % d, n / d, H) : n;
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = static_cast<uint32_t>(t[k8 + 2 * e][r]) | (static_cast<uint32_t>(t[k8 + 2 * e + 1][r]) << 16);
    *reinterpret_cast<uint4*>(Wt + static_cast<int64_t>(row) * D + k0 + k8) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
}

// ------------------------------------------------------------------- NT GEMM
// C[i][j] = sum_k A[i][k] * B[j][k]; A [I][K], B [J][K] bf16 (k contiguous), C fp32 with
// row stride ldc; K a multiple of 64.  TI x 256 tiles (TI = 64 RBW: 256, or 320 for the
// fused mixing with 20 heads and for plain products that need fewer workgroup rounds so),
// 8 waves as 2 x 4 (32 RBW x 64 each: every A fragment read from LDS feeds two matrix-core
// products, every B fragment RBW; small fused grids take 4 waves and 128-column tiles),
// K slices of 64 in a two-stage LDS ring filled by buffer loads straight into LDS, register
// fragments read one k-step ahead of the products that use them.  Rows
// are 128 bytes with 16-byte chunks XOR-swizzled by (row >> 1) & 7, so the 16 lanes that
// read 16 rows of one chunk hit 16 bank groups.  Rows past I / J read zero (buffer range
// check) and their results are not stored.  The operands must each span < 2 GiB (the
// launcher splits larger problems).
constexpr int GTI = 256, GTJ = 256, GK = 64, GWaves = 8, GThreads = GWaves * 64;
constexpr int GRBW = GTI / 64;  // 32-row blocks per wave of the plain GEMM
static_assert(GK == 64, "the main loop walks four k-steps of 16 per slice");

__device__ __forceinline__ int gswz(int r) { return (r >> 1) & 7; }

template <int RBW, int NW = GWaves>
struct NtSmem {
  uint16_t a[2][64 * RBW * GK];
  uint16_t b[2][32 * NW * GK];
};

// Main loop of one (64 RBW) x (32 NW) tile of NW waves (2 x NW/2, each (32 RBW) x 64; NW = 8,
// or 4 for grids too small to give every CU a tile); hands the accumulators to
// epi(acc, i0, j0, wm, wn).
template <int RBW, int NW = GWaves, typename Epi>
__device__ __forceinline__ void gemm_tile(const NtArgs& g, NtSmem<RBW, NW>& sm, Epi&& epi) {
  constexpr int TI = 64 * RBW, TJ = 32 * NW;
  const int I = g.I, J = g.J, K = g.K;
  const int64_t KS = g.ks > 0 ? g.ks : K;  // row stride of A and B
  const int ntj = (J + TJ - 1) / TJ, nti = (I + TI - 1) / TI;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  // Groups of 4 row tiles sweep the column tiles, so a group's A slices stay in L2.
  constexpr int GR = 4;
  const int group = lid / (GR * ntj);
  const int first_i = group * GR;
  const int gsize = min(GR, nti - first_i);
  const int ti = first_i + (lid % (GR * ntj)) % gsize;
  const int tj = (lid % (GR * ntj)) / gsize;
  const int i0 = ti * TI, j0 = tj * TJ;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);

  // Readable bytes end with the last valid row's K values: rows past I / J read zero.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g.A), static_cast<short>(0), static_cast<int>(((I - 1) * KS + K) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(g.B), static_cast<short>(0), static_cast<int>(((J - 1) * KS + K) * 2), 0x00020000);
  // Copy slot (p * NW + wave) * 64 + lane of a stage -> row 8 NW p + 8 * wave + lane / 8,
  // chunk lane % 8; the swizzle depends on the row only through 8 * wave + lane / 8.
  const int rl = 8 * wave + (lane >> 3), pos = lane & 7;
  const unsigned loff = static_cast<unsigned>((rl * KS + (pos ^ gswz(rl)) * 8) * 2);
  auto issue = [&](int k0, int st) {
#pragma unroll
    for (int p = 0; p < TI / (8 * NW); ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(sm.a[st] + (p * NW + wave) * 512), 16, loff,
          static_cast<unsigned>((static_cast<int64_t>(i0 + 8 * NW * p) * KS + k0) * 2), 0, 0);
#pragma unroll
    for (int p = 0; p < TJ / (8 * NW); ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(sm.b[st] + (p * NW + wave) * 512), 16, loff,
          static_cast<unsigned>((static_cast<int64_t>(j0 + 8 * NW * p) * KS + k0) * 2), 0, 0);
  };

  // Per-lane LDS element offsets of the A / B fragments; k-step s reads chunk 2s + hf.
  int ao[RBW], bo[2], asz[RBW], bsz[2];
#pragma unroll
  for (int i = 0; i < RBW; ++i) {
    const int r = wm * 32 * RBW + i * 32 + l32;
    ao[i] = r * GK;
    asz[i] = gswz(r);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wn * 64 + j * 32 + l32;
    bo[j] = r * GK;
    bsz[j] = gswz(r);
  }
  floatx16 acc[RBW][2];
#pragma unroll
  for (int i = 0; i < RBW; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  // Fragments are read one k-step ahead into two register buffers (k-step s of a slice uses
  // buffer s & 1), one LDS read between consecutive products; the products of a slice's last
  // k-step are issued after the slice barrier, next to the first reads of the next slice.
  bf16x8 fa[2][RBW], fb[2][2];
  auto load = [&](int st, int s, int buf) {
#pragma unroll
    for (int i = 0; i < RBW; ++i)
      fa[buf][i] = *reinterpret_cast<const bf16x8*>(&sm.a[st][ao[i] + ((s * 2 + hf) ^ asz[i]) * 8]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      fb[buf][j] = *reinterpret_cast<const bf16x8*>(&sm.b[st][bo[j] + ((s * 2 + hf) ^ bsz[j]) * 8]);
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[buf][i], fb[buf][j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < RBW + 2; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * RBW - (RBW + 2), 0);
  };

  const int nk = K / GK;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) issue((kt + 1) * GK, st ^ 1);  // the other stage was last read before the barrier
    load(st, 0, 0);
    if (kt > 0) mma(1);
    __builtin_amdgcn_sched_barrier(0);
    load(st, 1, 1);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    load(st, 2, 0);
    mma(1);
    __builtin_amdgcn_sched_barrier(0);
    load(st, 3, 1);
    mma(0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
  }
  mma(1);
  epi(acc, i0, j0, wm, wn);
}

// RBW = 4 (256-row tiles) or 5 (320-row tiles: fewer tiles where 256-row tiles would leave
// the chip's last round of workgroups partly empty).
template <int RBW>
__global__ __launch_bounds__(GThreads, 1) void gemm_nt_bf16_kernel(NtArgs g) {
  static_assert(GWaves * 64 * 64 * sizeof(float) <= sizeof(NtSmem<RBW>), "epilogue staging");
  __shared__ __attribute__((aligned(16))) NtSmem<RBW> sm;
  if (gridDim.y > 1 || gridDim.z > 1) {  // batched launch: product blockIdx.y, K part blockIdx.z
    const int z = blockIdx.y, sp = blockIdx.z;
    g.A += z * g.sa + static_cast<int64_t>(sp) * g.K;
    g.B += z * g.sb + static_cast<int64_t>(sp) * g.K;
    // (Cz by selects: a dynamic index would put the argument block in scratch memory.)
    g.C = gridDim.z > 1 ? g.C + (static_cast<int64_t>(sp) * gridDim.y + z) * g.I * g.ldc
                        : z == 0 ? g.Cz[0] : z == 1 ? g.Cz[1] : g.Cz[2];
  }
  gemm_tile<RBW>(g, sm, [&](floatx16 (&acc)[RBW][2], int i0, int j0, int wm, int wn) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
    const int I = g.I, J = g.J;
    // Lane l holds C[8*(r/4) + 4*hf + r%4][l%32] of each 32x32 block.  With 16-byte aligned
    // rows the wave's (32 RBW) x 64 block goes through its own 16 KB of the (now idle) LDS
    // stages in pieces of two 32-row blocks (one for an odd last block) and leaves as 16-byte
    // stores, 256 contiguous bytes per 16 lanes
    // (4-byte stores of 32 columns otherwise).  LDS rows are 64 floats with 16-byte chunk c of
    // row r at c ^ (8 * ((r >> 2) & 1)), so the two lane halves' writes (rows 4 apart) and each
    // 16 lanes' reads of a row hit distinct banks.
    const bool vec = (g.ldc & 3) == 0 && (reinterpret_cast<uintptr_t>(g.C) & 15) == 0;
    if (vec) {
      __syncthreads();  // every wave has read its last fragments from the stages
      float* st = reinterpret_cast<float*>(&sm) + (threadIdx.x >> 6) * 64 * 64;
#pragma unroll
      for (int half = 0; half < (RBW + 1) / 2; ++half) {
        const int nb = 2 * half + 1 < RBW ? 2 : 1;  // 32-row blocks in this piece
#pragma unroll
        for (int ii = 0; ii < nb; ++ii)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = ii * 32 + 8 * (r >> 2) + 4 * hf + (r & 3), col = j * 32 + l32;
              st[row * 64 + (((col >> 2) ^ (((row >> 2) & 1) << 3)) << 2) + (col & 3)] = acc[2 * half + ii][j][r];
            }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS in order within the wave
#pragma unroll
        for (int k = 0; k < 8 * nb; ++k) {
          const int row = 4 * k + (lane >> 4), ch = lane & 15;
          const floatx4 v = *reinterpret_cast<const floatx4*>(st + row * 64 + ((ch ^ (((row >> 2) & 1) << 3)) << 2));
          const int grow = i0 + wm * 32 * RBW + half * 64 + row, gcol = j0 + wn * 64 + 4 * ch;
          if (grow < I) {
            float* dst = g.C + static_cast<int64_t>(grow) * g.ldc + gcol;
            if (gcol + 3 < J) {
              *reinterpret_cast<floatx4*>(dst) = v;
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (gcol + e < J) dst[e] = v[e];
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next half's writes
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < RBW; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = j0 + wn * 64 + j * 32 + l32;
        if (col >= J) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i0 + wm * 32 * RBW + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (row < I) g.C[static_cast<int64_t>(row) * g.ldc + col] = acc[i][j][r];
        }
      }
  });
}

// ------------------------------------------------------------------- fused projection + mixing
// For H = 16 and H = 20 the weight rows of each matrix are permuted (wprep with cm) so that
// a wave's 32*RBW rows are the H source heads of 8 consecutive channels (RBW = H / 4 blocks
// of 32 rows):
//   rows cl*16 + m        (m < 16):  "main" blocks, two channels of 16 source heads each;
//   rows 128 + cl*4 + m-16 (m >= 16, H = 20): one "rest" block, 8 channels x 4 heads.
// A lane's accumulator registers 0..7 (8..15) of a block are rows 8*(e/4) + 4*hf + e%4 of
// its first (second) half: exactly the B operand of a 32x32x16 product whose k-slot
// 8*hf + e stands for that row.  The epilogue mixes in place
//   out[(h, j)][token] = sum_m alpha[m][h][j] * Y[(c, m)][token]
// as alpha^T (A operand, 32 rows (h, j) per block) times the main half of channel c, plus
// (H = 20) alpha^T of heads 16..19, zero outside channel c's four k-slots, times the rest
// half that holds c.  Both operands are split into fp16 hi + lo (three products per pair,
// fp32 accumulation, ~2^-21 relative).  Outputs:
//   V~^T [B][H][d][P*N]           (P consecutive fp16 per lane and head),
//   Q~, K~ [B][H][d/8][P*N][8]    (a wave's 8 channels form one 16-byte chunk per row),
// plus the unmixed fp32 projections of the first tokens (Ye, mixed in fp32 by the
// attention launch); the fp32 projections of the other tokens never reach HBM.
__device__ __forceinline__ void split_f16(const floatx16& y, int cs, half8& bh, half8& bl) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = y[8 * cs + e];
    bh[e] = static_cast<half_t>(x);
    bl[e] = static_cast<half_t>(x - static_cast<float>(bh[e]));
  }
}

// Mixed values of channel cl (0..7 within the wave) for one 32-token column block: lane row
// r is (h, jj) with h*P + jj = mb*32 + 8*(r/4) + 4*hf + r%4, column = the lane's token.
// yh/yl: the fp16 hi/lo B operands of the wave's accumulator block halves of this column
// block ([block][half]); ah/alo: alpha^T of heads 0..15; arh/arl (H = 20): alpha^T of heads
// 16..19 in both element groups.
template <int H, int RBW>
__device__ __forceinline__ floatx16 mix_channel(const half8 (&yh)[RBW][2], const half8 (&yl)[RBW][2], int cl, int hf,
                                                const half8& ah, const half8& alo, const half8& arh,
                                                const half8& arl) {
  floatx16 o;
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.f;
  const half8& bh = yh[cl >> 1][cl & 1];
  const half8& bl = yl[cl >> 1][cl & 1];
  o = mfma32(ah, bh, o);
  o = mfma32(alo, bh, o);
  o = mfma32(ah, bl, o);
  if constexpr (H == 20) {
    // Rest half cl / 4; k-slot 8*hf + e holds channel 4*(cl/4) + 2*(e/4) + hf: keep the
    // element group whose channel is cl.
    const half8& rbh = yh[4][cl >> 2];
    const half8& rbl = yl[4][cl >> 2];
    const int ct = cl & 3;
    const bool g0 = ct == hf, g1 = ct == 2 + hf;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 h4 = __builtin_bit_cast(u32x4, arh), l4 = __builtin_bit_cast(u32x4, arl);
    h4[0] = g0 ? h4[0] : 0u;
    h4[1] = g0 ? h4[1] : 0u;
    h4[2] = g1 ? h4[2] : 0u;
    h4[3] = g1 ? h4[3] : 0u;
    l4[0] = g0 ? l4[0] : 0u;
    l4[1] = g0 ? l4[1] : 0u;
    l4[2] = g1 ? l4[2] : 0u;
    l4[3] = g1 ? l4[3] : 0u;
    const half8 rh = __builtin_bit_cast(half8, h4), rl = __builtin_bit_cast(half8, l4);
    o = mfma32(rh, rbh, o);
    o = mfma32(rl, rbh, o);
    o = mfma32(rh, rbl, o);
  } else {
    (void)arh;
    (void)arl;
  }
  return o;
}

template <int H, int P, int NW>
__global__ __launch_bounds__(NW * 64, 1) void gemm_mix_bf16_kernel(NtArgs g, ProjArgs pa) {
  constexpr int RBW = H / 4, HP = H * P, MB = (HP + 31) / 32;
  __shared__ __attribute__((aligned(16))) NtSmem<RBW, NW> sm;
  gemm_tile<RBW, NW>(g, sm, [&](floatx16 (&acc)[RBW][2], int i0, int j0, int wm, int wn) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
    const int D = pa.D, d = pa.d, N = pa.N, M = pa.B * pa.N;
    const int which = i0 / D;                          // tiles never straddle Q / K / V
    const int c0 = ((i0 % D) + 32 * RBW * wm) / H;     // the wave's 8 channels: c0 .. c0 + 7
    const float* __restrict__ al = pa.alpha[which];
    const int64_t L = static_cast<int64_t>(P) * N;
    // alpha^T operands: lane (row = mb*32 + l32, element e) holds alpha[m][row] for the head m
    // of k-slot 8*hf + e: main m = 8*(e/4) + 4*hf + e%4, rest m = 16 + e%4.  With 20 heads
    // all four kinds go to LDS (free after the main loop) and are read where used, to keep
    // registers for the accumulators; with 16 the main ones stay in registers.
    constexpr bool kLdsAlpha = H == 20;
    half8 ah[kLdsAlpha ? 1 : MB], alo[kLdsAlpha ? 1 : MB];
    half8* at = reinterpret_cast<half8*>(&sm);  // [kind: main hi, main lo, rest hi, rest lo][mb][lane]
    auto alpha_op = [&](int kind, int mb, int row, int e) {
      const int m = kind < 2 ? 8 * (e >> 2) + 4 * ((threadIdx.x & 63) >> 5) + (e & 3) : 16 + (e & 3);
      return row < HP ? al[m * HP + row] : 0.f;
    };
    if constexpr (kLdsAlpha) {
      for (int x = threadIdx.x; x < 2 * MB * 64; x += NW * 64) {  // (rest?, mb, lane)
        const int ln = x & 63, mb = (x >> 6) % MB, kind = 2 * (x / (64 * MB));
        const int row = mb * 32 + (ln & 31), hfx = ln >> 5;
        half8 vh, vl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int m = kind < 2 ? 8 * (e >> 2) + 4 * hfx + (e & 3) : 16 + (e & 3);
          const float a = row < HP ? al[m * HP + row] : 0.f;
          vh[e] = static_cast<half_t>(a);
          vl[e] = static_cast<half_t>(a - static_cast<float>(vh[e]));
        }
        at[((kind + 0) * MB + mb) * 64 + ln] = vh;
        at[((kind + 1) * MB + mb) * 64 + ln] = vl;
      }
      __syncthreads();  // every wave finished its main loop before the LDS was rewritten
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = alpha_op(0, mb, mb * 32 + l32, e);
          ah[mb][e] = static_cast<half_t>(a);
          alo[mb][e] = static_cast<half_t>(a - static_cast<float>(ah[mb][e]));
        }
    }
    // The first tokens' raw fp32 projections (rare column blocks holding a sequence's first
    // T0 tokens) go to Ye[b][t][which*D + row] (row as permuted); the attention launch mixes
    // them in fp32 into the first rows.
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tok = g.jbase + j0 + 64 * wn + 32 * j + l32;
      const int b = tok / N, t = tok % N;
      if (__builtin_expect(__any(tok < M && t < pa.T0), false)) {
        if (tok < M && t < pa.T0) {
          float* ye = pa.Ye + (static_cast<int64_t>(b) * pa.T0 + t) * 3 * D + i0 + 32 * RBW * wm;
#pragma unroll
          for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) ye[32 * i + 8 * (r >> 2) + 4 * hf + (r & 3)] = acc[i][j][r];
        }
      }
    }
    // All accumulators become fp16 hi/lo B operands (the fp32 values are not needed again).
    half8 yh[2][RBW][2], yl[2][RBW][2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < RBW; ++i)
#pragma unroll
        for (int cs = 0; cs < 2; ++cs) split_f16(acc[i][j], cs, yh[j][i][cs], yl[j][i][cs]);
    // mixed channel cl, column block j, output block mb
    auto mixc = [&](int j, int cl, int mb) {
      if constexpr (kLdsAlpha)
        return mix_channel<H, RBW>(yh[j], yl[j], cl, hf, at[(0 * MB + mb) * 64 + lane], at[(1 * MB + mb) * 64 + lane],
                                   at[(2 * MB + mb) * 64 + lane], at[(3 * MB + mb) * 64 + lane]);
      else
        return mix_channel<H, RBW>(yh[j], yl[j], cl, hf, ah[mb], alo[mb], ah[mb], alo[mb]);
    };
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int tok = g.jbase + j0 + 64 * wn + 32 * j + l32;
      const bool ok = tok < M;
      const int b = tok / N, t = tok % N;
      if (which < 2) {
        // Q~ / K~: with 16 heads and one block of 32 output rows (H*P <= 32) a lane gathers its
        // 8 channels of each row, one whole 16-byte chunk per store; otherwise half a chunk at
        // a time, to bound the registers held next to the accumulators.
        half_t* __restrict__ qk = which == 0 ? pa.Q : pa.K;
        const float oscale = which == 0 ? pa.qscale : 1.f;  // Q leaves pre-scaled, one rounding
        half_t* dst = qk + (static_cast<int64_t>(b * H) * (d / 8) + c0 / 8) * L * 8 + static_cast<int64_t>(t) * P * 8;
        if constexpr (MB == 1 && H == 16) {
          half8 stg[16];
#pragma unroll
          for (int cl = 0; cl < 8; ++cl) {
            const floatx16 o = mixc(j, cl, 0);
#pragma unroll
            for (int r = 0; r < 16; ++r) stg[r][cl] = static_cast<half_t>(o[r] * oscale);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hf + (r & 3);
            if (ok && row < HP)
              *reinterpret_cast<half8*>(dst + static_cast<int64_t>(row / P) * (d / 8) * L * 8 + (row % P) * 8) = stg[r];
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              half4 stg[16];
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const floatx16 o = mixc(j, 4 * half + q, mb);
#pragma unroll
                for (int r = 0; r < 16; ++r) stg[r][q] = static_cast<half_t>(o[r] * oscale);
              }
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int row = mb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
                if (ok && row < HP)
                  *reinterpret_cast<half4*>(dst + static_cast<int64_t>(row / P) * (d / 8) * L * 8 + (row % P) * 8 +
                                            4 * half) = stg[r];
              }
            }
        }
      } else {
        // V~^T: P consecutive fp16 per lane and head.
        typedef _Float16 halfp __attribute__((ext_vector_type(P)));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int cl = 0; cl < 8; ++cl) {
            const floatx16 o = mixc(j, cl, mb);
            const int c = c0 + cl;
            half_t* dst = pa.Vt + (static_cast<int64_t>(b * H) * d + c) * L + static_cast<int64_t>(t) * P;
#pragma unroll
            for (int r0 = 0; r0 < 16; r0 += P) {
              const int row = mb * 32 + 8 * (r0 >> 2) + 4 * hf + (r0 & 3);  // jj = 0 of head row / P
              halfp v;
#pragma unroll
              for (int jj = 0; jj < P; ++jj) v[jj] = static_cast<half_t>(o[r0 + jj]);
              if (ok && row < HP) *reinterpret_cast<halfp*>(dst + static_cast<int64_t>(row / P) * d * L) = v;
            }
          }
      }
    }
  });
}

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Launch C = A B^T, splitting A's rows or B's rows into chunks whose bytes fit the 32-bit
// buffer offsets (a chunk is a multiple of the tile height).  One workgroup fills a CU, so
// the launch runs in rounds of (CU count) tiles; 320-row tiles are taken when their rounds
// cover fewer rows per CU than 256-row tiles' (e.g. 2560 x 16384: 512 tiles in 2 rounds of
// 320 rows against 640 tiles in 3 rounds of 256 on 256 CUs).
hipError_t launch_gemm_nt(NtArgs g, hipStream_t s) {
  const int64_t max_rows = ((int64_t{1} << 31) - 1) / (static_cast<int64_t>(g.K) * 2) / GTI * GTI;
  if (max_rows < GTI) return hipErrorInvalidValue;
  if (g.I <= max_rows && g.J <= max_rows) {
    const int64_t cus = device_cus(), ntj = (g.J + GTJ - 1) / GTJ;
    const int64_t t4 = (g.I + 255) / 256 * ntj, t5 = (g.I + 319) / 320 * ntj;
    if ((t5 + cus - 1) / cus * 320 < (t4 + cus - 1) / cus * 256) {
      hipLaunchKernelGGL(gemm_nt_bf16_kernel<5>, dim3(static_cast<unsigned>(t5)), dim3(GThreads), 0, s, g);
      return hipGetLastError();
    }
  }
  const NtArgs full = g;
  for (int64_t i0 = 0; i0 < full.I; i0 += max_rows) {
    for (int64_t j0 = 0; j0 < full.J; j0 += max_rows) {
      NtArgs c = full;
      c.A = full.A + i0 * full.K;
      c.B = full.B + j0 * full.K;
      c.C = full.C + i0 * full.ldc + j0;
      c.I = static_cast<int>(std::min<int64_t>(max_rows, full.I - i0));
      c.J = static_cast<int>(std::min<int64_t>(max_rows, full.J - j0));
      const int tiles = ((c.I + GTI - 1) / GTI) * ((c.J + GTJ - 1) / GTJ);
      hipLaunchKernelGGL(gemm_nt_bf16_kernel<GRBW>, dim3(tiles), dim3(GThreads), 0, s, c);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// ------------------------------------------------------------------- mixing
// A thread loads the H source values y_m of a few (token, channel) pairs once and writes all
// H*P outputs  out[h][j] = sum_m alpha[m][h][j] * y_m  of each (fp32 arithmetic).  The block
// first stages alpha transposed to [h][j][m] in LDS, zero-padded to HMAX source heads, so the
// inner loop is branch-free FMAs on broadcast LDS reads.
template <int HMAX>
__device__ __forceinline__ void stage_alpha(const float* __restrict__ alpha, int H, int P, float* as) {
  for (int e = threadIdx.x; e < H * P * HMAX; e += 256) {
    const int m = e % HMAX, hj = e / HMAX;  // hj = h * P + j
    as[e] = m < H ? alpha[m * H * P + hj] : 0.f;
  }
  __syncthreads();
}

// acc[w] = sum_m alpha[m][h][j] * ym[m][w] for W independent values (channels or tokens).
template <int HMAX, int W>
__device__ __forceinline__ void mix_w(const float* as_hj, const float (&ym)[HMAX][W], float (&acc)[W]) {
#pragma unroll
  for (int w = 0; w < W; ++w) acc[w] = 0.f;
#pragma unroll
  for (int m = 0; m < HMAX; m += 4) {
    const floatx4 a4 = *reinterpret_cast<const floatx4*>(as_hj + m);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < W; ++w) acc[w] = fmaf(a4[q], ym[m + q][w], acc[w]);
  }
}

template <int W>
__device__ __forceinline__ void store_halves(half_t* p, const float (&v)[W], float scale) {
  typedef _Float16 halfw __attribute__((ext_vector_type(W)));
  halfw h;
#pragma unroll
  for (int w = 0; w < W; ++w) h[w] = static_cast<half_t>(v[w] * scale);
  *reinterpret_cast<halfw*>(p) = h;
}
template <>
__device__ __forceinline__ void store_halves<1>(half_t* p, const float (&v)[1], float scale) {
  *p = static_cast<half_t>(v[0] * scale);
}

// Q~/K~ (token-major Y, lanes along c): each thread owns CW consecutive channels of one
// token (vector loads of Y, CW-wide fp16 stores).  grid (ceil(M*d/CW / 256), 2).
template <int HMAX, int CW>
__global__ __launch_bounds__(256) void mix_qk_kernel(ProjArgs pa) {
  extern __shared__ float as[];
  const int which = blockIdx.y;
  const int D = pa.D, d = pa.d, H = pa.H, P = pa.P, N = pa.N;
  stage_alpha<HMAX>(pa.alpha[which], H, P, as);
  const int groups = d / CW;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= static_cast<int64_t>(pa.B) * N * groups) return;
  const int tok = static_cast<int>(e / groups), c = static_cast<int>(e % groups) * CW;
  const int yw = pa.ywidth > 0 ? pa.ywidth : 2;  // projected matrices per token row of Yqk
  const float* __restrict__ y = pa.Yqk + static_cast<int64_t>(tok) * yw * D + which * D + c;
  half_t* __restrict__ out = (which == 0 ? pa.Q : which == 1 ? pa.K : pa.Vrow) + static_cast<int64_t>(tok) * P * D + c;
  float* __restrict__ oute = which == 0 ? pa.Qe : which == 1 ? pa.Ke : nullptr;
  const float oscale = which == 0 ? pa.qscale : 1.f;  // Q leaves pre-scaled, in one rounding
  const int b = tok / N, t = tok % N;
  float ym[HMAX][CW];
#pragma unroll
  for (int m = 0; m < HMAX; ++m) {
    const float* src = y + (m < H ? m : 0) * d;
    if (CW == 4) {
      const floatx4 v = *reinterpret_cast<const floatx4*>(src);
#pragma unroll
      for (int w = 0; w < CW; ++w) ym[m][w] = v[w];
    } else {
#pragma unroll
      for (int w = 0; w < CW; ++w) ym[m][w] = src[w];
    }
  }
  for (int h = 0; h < H; ++h)
    for (int j = 0; j < P; ++j) {
      float acc[CW];
      mix_w<HMAX, CW>(as + (h * P + j) * HMAX, ym, acc);
      store_halves<CW>(out + static_cast<int64_t>(j) * D + h * d, acc, oscale);
      const int i = t * P + j;
      if (oute && i < pa.R) {
#pragma unroll
        for (int w = 0; w < CW; ++w) oute[(static_cast<int64_t>(b) * pa.R + i) * D + h * d + c + w] = acc[w];
      }
    }
}

// V~^T (channel-major Y, lanes along tokens): each thread owns TW consecutive tokens of one
// channel row.  When the TW tokens share a sequence and P is even, the TW*P outputs of a head
// are contiguous and go out as 4-byte pairs.  grid (ceil(M/TW / 256), d).
template <int HMAX, int TW>
__global__ __launch_bounds__(256) void mix_v_kernel(ProjArgs pa) {
  extern __shared__ float as[];
  const int c = blockIdx.y;
  const int M = pa.B * pa.N, d = pa.d, H = pa.H, P = pa.P, N = pa.N;
  stage_alpha<HMAX>(pa.alpha[2], H, P, as);
  const int tok0 = (blockIdx.x * 256 + threadIdx.x) * TW;
  if (tok0 >= M) return;
  const int64_t L = static_cast<int64_t>(P) * N;
  float ym[HMAX][TW];
#pragma unroll
  for (int m = 0; m < HMAX; ++m)
#pragma unroll
    for (int w = 0; w < TW; ++w)
      ym[m][w] = tok0 + w < M ? pa.Yvt[static_cast<int64_t>((m < H ? m : 0) * d + c) * M + tok0 + w] : 0.f;
  const int b0 = tok0 / N, t0 = tok0 % N;
  const bool paired = (P % 2 == 0) && (t0 + TW <= N) && (tok0 + TW <= M);
  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  for (int h = 0; h < H; ++h) {
    if (paired) {
      // Outputs (t, j) and (t, j + 1) are adjacent: 4-byte stores.
      half_t* __restrict__ vrow = pa.Vt + (static_cast<int64_t>(b0 * H + h) * d + c) * L;
      for (int j = 0; j < P; j += 2) {
        float a0[TW], a1[TW];
        mix_w<HMAX, TW>(as + (h * P + j) * HMAX, ym, a0);
        mix_w<HMAX, TW>(as + (h * P + j + 1) * HMAX, ym, a1);
#pragma unroll
        for (int w = 0; w < TW; ++w) {
          const int i = (t0 + w) * P + j;
          const half2v v = {static_cast<half_t>(a0[w]), static_cast<half_t>(a1[w])};
          *reinterpret_cast<half2v*>(vrow + i) = v;
          if (pa.Ve && i < pa.R) {
            float* erow = pa.Ve + static_cast<int64_t>(b0) * pa.R * pa.D + h * d + c;
            erow[static_cast<int64_t>(i) * pa.D] = a0[w];
            if (i + 1 < pa.R) erow[static_cast<int64_t>(i + 1) * pa.D] = a1[w];
          }
        }
      }
      continue;
    }
    for (int j = 0; j < P; ++j) {
      float acc[TW];
      mix_w<HMAX, TW>(as + (h * P + j) * HMAX, ym, acc);
#pragma unroll
      for (int w = 0; w < TW; ++w) {
        const int tok = tok0 + w;
        if (tok >= M) break;
        const int b = tok / N, t = tok % N;
        half_t* __restrict__ vrow = pa.Vt + (static_cast<int64_t>(b * H + h) * d + c) * L;
        vrow[static_cast<int64_t>(t) * P + j] = static_cast<half_t>(acc[w]);
        const int i = t * P + j;
        if (pa.Ve && i < pa.R) pa.Ve[(static_cast<int64_t>(b) * pa.R + i) * pa.D + h * d + c] = acc[w];
      }
    }
  }
}

// ------------------------------------------------------------------- mixing on the matrix cores
// The mixing is a small product per channel c: with rows (h, j) of alpha^T and columns
// tokens,  V~^T_c[(h,j)][t] = sum_m alpha[m][h][j] * Y_V^T[m*d + c][t].  Both operands are
// split into fp16 high and low parts (x = hi + lo, |lo| <= 2^-11 |x|) and three fp16 products
// with fp32 accumulation (hi*hi + lo*hi + hi*lo) give the fp32 result to about 2^-21
// relative, the same as fp32 FMAs; the arithmetic then costs nothing next to the memory
// traffic.
__device__ __forceinline__ half_t hi_f16(float x) { return static_cast<half_t>(x); }
__device__ __forceinline__ half_t lo_f16(float x) {
  return static_cast<half_t>(x - static_cast<float>(static_cast<half_t>(x)));
}

// alpha^T operands: A[(h,j) = mb*32 + l%32][k = ks*16 + 8*(l/32) + e] = alpha[m][h][j],
// zero outside h*P + j < H*P and m < H.
template <int MB, int KS>
__device__ __forceinline__ void alpha_operands(const float* __restrict__ al, int H, int P, half8 (&ah)[MB][KS],
                                               half8 (&alo)[MB][KS]) {
  const int lane = threadIdx.x & 63, HP = H * P;
  float a[MB][KS][8];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = mb * 32 + (lane & 31), m = ks * 16 + 8 * (lane >> 5) + e;
        a[mb][ks][e] = al[(row < HP && m < H) ? m * HP + row : 0];
      }
  __builtin_amdgcn_sched_barrier(0);  // every load above is issued before the first use
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = mb * 32 + (lane & 31), m = ks * 16 + 8 * (lane >> 5) + e;
        const float v = (row < HP && m < H) ? a[mb][ks][e] : 0.f;
        ah[mb][ks][e] = hi_f16(v);
        alo[mb][ks][e] = lo_f16(v);
      }
}

// Q~/K~ from token-major Y on the matrix cores.  For one token the mixing is a product:
// out[(h, j)][c] = sum_m alpha[m][h][j] Y[m][c], alpha^T (rows h*P + j, MB blocks of 32)
// times the token's [H][d] block (KS k-steps of 16 source heads), with the same fp16 hi/lo
// split as above (the vector-unit kernel above spends H*P*H*d fused multiply-adds per token
// on the same result and is bound by them).  A work item is one token and one 64-channel half
// of d; column n of product q is channel 64*half + 2n + q, so a lane loads two consecutive
// channels of each source head at once.  The H*P x 64 fp16 result goes through the wave's own
// LDS block and leaves as 16-byte stores, eight lanes per 128-byte row segment.  A wave walks
// items gw, gw + nw, ... with the next item's loads in flight during the current one's
// products.  Source heads m >= H read head 0 (finite) against zero alpha operands.  d in
// {64, 128}, P in {1, 2, 4}; grid (x, nmat), 256 threads.
typedef float floatx2 __attribute__((ext_vector_type(2)));
template <int MB, int KS, int P>
__global__ __launch_bounds__(256, 2) void mix_qk_mfma_kernel(ProjArgs pa) {
  constexpr int ORW = 64 + 8;  // staged row (halves): 144 bytes, so 32 rows' writes spread over the banks
  __shared__ __attribute__((aligned(16))) half_t ost[4][MB * 32 * ORW];
  const int which = blockIdx.y;
  const int M = pa.B * pa.N, D = pa.D, d = pa.d, H = pa.H, N = pa.N, HP = H * P;
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5, w = threadIdx.x >> 6;
  const int yw = pa.ywidth > 0 ? pa.ywidth : 2;  // projected matrices per token row of Yqk
  half_t* __restrict__ outb = which == 0 ? pa.Q : which == 1 ? pa.K : pa.Vrow;
  float* __restrict__ oute = which == 0 ? pa.Qe : which == 1 ? pa.Ke : nullptr;
  const float oscale = which == 0 ? pa.qscale : 1.f;  // Q leaves pre-scaled, in one rounding
  const int halves = d / 64, nitems = M * halves, nw = gridDim.x * 4;
  int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(w);
  if (item >= nitems) return;
  half_t* os = ost[w];
  // B operand of product q, k-step ks: B[k][n] = Y[m = ks*16 + 8*hf + k%8][64*half + 2n + q].
  int mrow[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = ks * 16 + 8 * hf + e;
      mrow[ks][e] = (m < H ? m : 0) * d;
    }
  auto load = [&](int it, floatx2 (&yv)[KS][8]) {
    const int tk = it / halves, c0 = (it % halves) * 64;
    const float* __restrict__ y = pa.Yqk + static_cast<int64_t>(tk) * yw * D + which * D + c0 + 2 * n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) yv[ks][e] = *reinterpret_cast<const floatx2*>(y + mrow[ks][e]);
  };
  floatx2 yv[KS][8];
  load(item, yv);
  half8 ah[MB][KS], alo[MB][KS];
  alpha_operands<MB, KS>(pa.alpha[which], H, P, ah, alo);
  for (; item < nitems; item += nw) {
    half8 bh[2][KS], bl[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bh[q][ks][e] = hi_f16(yv[ks][e][q]);
          bl[q][ks][e] = lo_f16(yv[ks][e][q]);
        }
    if (item + nw < nitems) load(item + nw, yv);
    const int tok = item / halves, c0 = (item % halves) * 64;
    const int b = tok / N, t = tok % N;
    const bool early = oute != nullptr && t * P < pa.R;  // wave-uniform, rare
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      floatx16 acc[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc[q] = mfma32(ah[mb][ks], bh[q][ks], acc[q]);
          acc[q] = mfma32(alo[mb][ks], bh[q][ks], acc[q]);
          acc[q] = mfma32(ah[mb][ks], bl[q][ks], acc[q]);
        }
      }
      // Lane rows: row = mb*32 + 8*(r/4) + 4*hf + r%4 = h*P + j.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = mb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        const half2v v = {static_cast<half_t>(acc[0][r] * oscale), static_cast<half_t>(acc[1][r] * oscale)};
        *reinterpret_cast<half2v*>(os + row * ORW + 2 * n) = v;
      }
      if (__builtin_expect(early, false)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = mb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
          const int h = row / P, j = row % P, i = t * P + j;
          if (row < HP && i < pa.R) {
            const floatx2 f = {acc[0][r], acc[1][r]};
            *reinterpret_cast<floatx2*>(oute + (static_cast<int64_t>(b) * pa.R + i) * D + h * d + c0 + 2 * n) = f;
          }
        }
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // LDS in order within the wave
    // Row (h, j) of the token: 64 channels at out[(tok*P + j)*D + h*d + c0], 8 chunks of 16 B.
    half_t* __restrict__ out = outb + static_cast<int64_t>(tok) * P * D + c0;
    for (int k = lane; k < HP * 8; k += 64) {
      const int row = k >> 3, ch = k & 7;
      const half8 v = *reinterpret_cast<const half8*>(os + row * ORW + ch * 8);
      *reinterpret_cast<half8*>(out + (row % P) * D + (row / P) * d + ch * 8) = v;
    }
  }
}

// V~^T from Y_V^T.  A work item is one channel c and 32*TQ tokens of one sequence: lane n
// (of 32) loads TQ consecutive tokens TQ*n .. TQ*n + TQ-1, so column n of product block q is
// token TQ*n + q; after the TQ blocks a lane holds, for each of its (h, j) rows, TQ
// consecutive tokens, i.e. TQ*P consecutive fp16 of V~^T[b][h][c][*] (P in {1, 2, 4}).  A
// wave walks items gw, gw + nw, ... (alpha's operands built once, the next item's loads in
// flight during the current one's products); consecutive waves take consecutive token blocks
// of one channel.  TQ = 2 halves the registers of the large cases.  Needs N % (32 TQ) == 0.
template <int P, int MB, int KS, int TQ>
__global__ __launch_bounds__(256, 2) void mix_v_mfma_kernel(ProjArgs pa) {
  typedef float floatq __attribute__((ext_vector_type(TQ)));
  const int M = pa.B * pa.N, d = pa.d, H = pa.H, N = pa.N;
  const int lane = threadIdx.x & 63, n = lane & 31, hf = lane >> 5;
  const int nblk = M / (32 * TQ), nitems = nblk * d, nw = gridDim.x * 4;
  int item = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= nitems) return;
  // B operands, blocks q < TQ: B[k][n] = Y_V^T[m = ks*16 + 8*hf + k%8][token TQ*n + q]; source
  // heads m >= H read head 0 (finite) against zero alpha operands.
  int64_t mrow[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int m = ks * 16 + 8 * hf + e;
      mrow[ks][e] = static_cast<int64_t>(m < H ? m : 0) * d * M;
    }
  auto load = [&](int it, floatq (&y)[KS][8]) {
    const int c = it / nblk, tok0 = (it % nblk) * 32 * TQ;
    const float* __restrict__ src = pa.Yvt + static_cast<int64_t>(c) * M + tok0 + TQ * n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) y[ks][e] = *reinterpret_cast<const floatq*>(src + mrow[ks][e]);
  };
  floatq yall[KS][8];
  load(item, yall);
  half8 ah[MB][KS], alo[MB][KS];
  alpha_operands<MB, KS>(pa.alpha[2], H, P, ah, alo);
  const int64_t L = static_cast<int64_t>(P) * N;
  const int HP = H * P;
  for (; item < nitems; item += nw) {
    half8 bh[TQ][KS], bl[TQ][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bh[q][ks][e] = hi_f16(yall[ks][e][q]);
          bl[q][ks][e] = lo_f16(yall[ks][e][q]);
        }
    if (item + nw < nitems) load(item + nw, yall);
    const int c = item / nblk, tok0 = (item % nblk) * 32 * TQ;
    const int b = tok0 / N, t0 = tok0 % N;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      floatx16 acc[TQ];
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          acc[q] = mfma32(ah[mb][ks], bh[q][ks], acc[q]);
          acc[q] = mfma32(alo[mb][ks], bh[q][ks], acc[q]);
          acc[q] = mfma32(ah[mb][ks], bl[q][ks], acc[q]);
        }
      }
      // Lane rows: row = mb*32 + 8*(r/4) + 4*hf + r%4 = h*P + j.
#pragma unroll
      for (int g = 0; g < 4; ++g) {        // g = r / 4: rows 4*(2g + hf) .. +3
        const int row0 = mb * 32 + 8 * g + 4 * hf;
        if (row0 >= HP) continue;
#pragma unroll
        for (int u = 0; u < 4 / P; ++u) {  // heads among these 4 rows
          const int h = (row0 + u * P) / P;
          if (h >= H) continue;
          // TQ tokens x P pseudo-tokens of head h, stacked positions (t0 + TQ*n + q)*P + j
          typedef _Float16 halfv __attribute__((ext_vector_type(TQ * P)));
          halfv v;
#pragma unroll
          for (int q = 0; q < TQ; ++q)
#pragma unroll
            for (int j = 0; j < P; ++j) v[q * P + j] = static_cast<half_t>(acc[q][4 * g + u * P + j]);
          half_t* dst = pa.Vt + (static_cast<int64_t>(b * H + h) * d + c) * L + static_cast<int64_t>(t0 + TQ * n) * P;
          *reinterpret_cast<halfv*>(dst) = v;
          if (pa.Ve && (t0 + TQ * n) * P < pa.R) {
            float* erow = pa.Ve + static_cast<int64_t>(b) * pa.R * pa.D + h * d + c;
#pragma unroll
            for (int q = 0; q < TQ; ++q)
#pragma unroll
              for (int j = 0; j < P; ++j) {
                const int i = (t0 + TQ * n + q) * P + j;
                if (i < pa.R) erow[static_cast<int64_t>(i) * pa.D] = acc[q][4 * g + u * P + j];
              }
          }
        }
      }
    }
  }
}

template <int P>
bool launch_mix_v_mfma_p(const ProjArgs& pa, hipStream_t s) {
  const int64_t M = static_cast<int64_t>(pa.B) * pa.N;
  const int mb = (pa.H * P + 31) / 32, ks = (pa.H + 15) / 16;
  const dim3 g4(static_cast<unsigned>(std::min<int64_t>((M / 128 * pa.d + 3) / 4, 1024))),
      g2(static_cast<unsigned>(std::min<int64_t>((M / 64 * pa.d + 3) / 4, 1024)));
  // With H <= 16 (one k-step) H*P <= 64; with two k-steps P = 1 needs one row block, P = 2 two.
  if (ks == 1) {
    if (mb == 1) hipLaunchKernelGGL((mix_v_mfma_kernel<P, 1, 1, 4>), g4, dim3(256), 0, s, pa);
    else if constexpr (P >= 2) hipLaunchKernelGGL((mix_v_mfma_kernel<P, 2, 1, 4>), g4, dim3(256), 0, s, pa);
    return true;
  }
  if (mb == 1) hipLaunchKernelGGL((mix_v_mfma_kernel<P, 1, 2, 2>), g2, dim3(256), 0, s, pa);
  else if constexpr (P >= 2) {
    if (mb == 2) hipLaunchKernelGGL((mix_v_mfma_kernel<P, 2, 2, 2>), g2, dim3(256), 0, s, pa);
    else if constexpr (P == 4) {
      if (mb == 3) hipLaunchKernelGGL((mix_v_mfma_kernel<P, 3, 2, 2>), g2, dim3(256), 0, s, pa);
      else hipLaunchKernelGGL((mix_v_mfma_kernel<P, 4, 2, 2>), g2, dim3(256), 0, s, pa);
    }
  }
  return true;
}

bool launch_mix_v_mfma(const ProjArgs& pa, hipStream_t s) {
  if (pa.N % 128 != 0 || pa.H > 32 || pa.H * pa.P > 128) return false;
  switch (pa.P) {
    case 1: return launch_mix_v_mfma_p<1>(pa, s);
    case 2: return launch_mix_v_mfma_p<2>(pa, s);
    case 4: return launch_mix_v_mfma_p<4>(pa, s);
    default: return false;
  }
}

template <int MB, int KS, int P>
void launch_mix_qk_mfma_mk(const ProjArgs& pa, int nmat, hipStream_t s) {
  const int64_t items = static_cast<int64_t>(pa.B) * pa.N * (pa.d / 64);
  const dim3 grid(static_cast<unsigned>(std::min<int64_t>((items + 3) / 4, 1024)), nmat);
  hipLaunchKernelGGL((mix_qk_mfma_kernel<MB, KS, P>), grid, dim3(256), 0, s, pa);
}

template <int KS>
bool launch_mix_qk_mfma_k(const ProjArgs& pa, int nmat, hipStream_t s) {
  const int mb = (pa.H * pa.P + 31) / 32;
  switch (pa.P * 8 + mb) {
    case 1 * 8 + 1: launch_mix_qk_mfma_mk<1, KS, 1>(pa, nmat, s); return true;
    case 2 * 8 + 1: launch_mix_qk_mfma_mk<1, KS, 2>(pa, nmat, s); return true;
    case 2 * 8 + 2: launch_mix_qk_mfma_mk<2, KS, 2>(pa, nmat, s); return true;
    case 4 * 8 + 1: launch_mix_qk_mfma_mk<1, KS, 4>(pa, nmat, s); return true;
    case 4 * 8 + 2: launch_mix_qk_mfma_mk<2, KS, 4>(pa, nmat, s); return true;
    case 4 * 8 + 3: launch_mix_qk_mfma_mk<3, KS, 4>(pa, nmat, s); return true;
    case 4 * 8 + 4: launch_mix_qk_mfma_mk<4, KS, 4>(pa, nmat, s); return true;
    default: return false;
  }
}

// Q~/K~ (and the row-major V~) mixing on the matrix cores when d is 64 or 128, H <= 32,
// H*P <= 128 and P is 1, 2 or 4; false otherwise (the caller then uses the vector-unit kernel).
bool launch_mix_qk_mfma(const ProjArgs& pa, int nmat, hipStream_t s) {
  if ((pa.d != 64 && pa.d != 128) || pa.H > 32 || pa.H * pa.P > 128) return false;
  return pa.H <= 16 ? launch_mix_qk_mfma_k<1>(pa, nmat, s) : launch_mix_qk_mfma_k<2>(pa, nmat, s);
}

template <int HMAX>
void launch_mix(const ProjArgs& pa, hipStream_t s) {
  constexpr int CW = HMAX <= 20 ? 4 : HMAX <= 32 ? 2 : 1;
  constexpr int TW = HMAX <= 32 ? 2 : 1;
  const int64_t M = static_cast<int64_t>(pa.B) * pa.N;
  const size_t lds = static_cast<size_t>(pa.H) * pa.P * HMAX * sizeof(float);
  const int64_t nqk = M * (pa.d / CW);
  if (!launch_mix_qk_mfma(pa, 2, s))
    hipLaunchKernelGGL((mix_qk_kernel<HMAX, CW>), dim3(static_cast<unsigned>((nqk + 255) / 256), 2), dim3(256), lds, s, pa);
  if (launch_mix_v_mfma(pa, s)) return;
  const int64_t nv = (M + TW - 1) / TW;
  hipLaunchKernelGGL((mix_v_kernel<HMAX, TW>), dim3(static_cast<unsigned>((nv + 255) / 256), pa.d), dim3(256), lds, s, pa);
}

template <int HMAX>
void launch_mix_rows(const ProjArgs& pa, int nmat, hipStream_t s) {
  if (launch_mix_qk_mfma(pa, nmat, s)) return;
  constexpr int CW = HMAX <= 20 ? 4 : HMAX <= 32 ? 2 : 1;
  const int64_t M = static_cast<int64_t>(pa.B) * pa.N;
  const size_t lds = static_cast<size_t>(pa.H) * pa.P * HMAX * sizeof(float);
  const int64_t n = M * (pa.d / CW);
  hipLaunchKernelGGL((mix_qk_kernel<HMAX, CW>), dim3(static_cast<unsigned>((n + 255) / 256), nmat), dim3(256), lds, s,
                     pa);
}

}  // namespace

hipError_t launch_gemm_nt_bf16(const NtArgs& g, hipStream_t s) { return launch_gemm_nt(g, s); }

// Cz[z][e] = sum over parts p (in order) of Cs[(p*batch + z)*n + e], n = I * ldc.
__global__ __launch_bounds__(256) void splitk_sum_kernel(NtArgs g, int batch, int splits, int64_t n) {
  const int z = blockIdx.y;
  const floatx4* src = reinterpret_cast<const floatx4*>(g.C);
  floatx4* dst = reinterpret_cast<floatx4*>(g.Cz[z]);
  const int64_t n4 = n / 4;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n4; e += static_cast<int64_t>(gridDim.x) * 256) {
    floatx4 acc = src[static_cast<int64_t>(z) * n4 + e];
    for (int p = 1; p < splits; ++p) acc += src[(static_cast<int64_t>(p) * batch + z) * n4 + e];
    dst[e] = acc;
  }
}

hipError_t launch_gemm_nt_splitk(const NtArgs& g, int batch, int splits, float* Cs, hipStream_t s) {
  if (batch < 1 || batch > 3 || splits < 1 || g.K % (64 * splits) != 0 || (g.I * g.ldc) % 4 != 0)
    return hipErrorInvalidValue;
  if (splits == 1) return launch_gemm_nt_batched(g, batch, s);
  NtArgs c = g;
  c.ks = g.ks > 0 ? g.ks : g.K;
  c.K = g.K / splits;
  c.C = Cs;
  const int64_t max_rows = ((int64_t{1} << 31) - 1) / (static_cast<int64_t>(c.ks) * 2) / GTI * GTI;
  if (max_rows < g.I || max_rows < g.J) return hipErrorInvalidValue;
  const int tiles = ((g.I + GTI - 1) / GTI) * ((g.J + GTJ - 1) / GTJ);
  hipLaunchKernelGGL(gemm_nt_bf16_kernel<GRBW>, dim3(tiles, batch, splits), dim3(GThreads), 0, s, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(g.I) * g.ldc;
  const unsigned blocks = static_cast<unsigned>(std::min<int64_t>((n / 4 + 255) / 256, 1024));
  hipLaunchKernelGGL(splitk_sum_kernel, dim3(blocks, batch), dim3(256), 0, s, c, batch, splits, n);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_batched(const NtArgs& g, int batch, hipStream_t s) {
  if (batch < 1 || batch > 3) return hipErrorInvalidValue;
  const int64_t max_rows = ((int64_t{1} << 31) - 1) / (static_cast<int64_t>(g.K) * 2) / GTI * GTI;
  if (batch == 1 || max_rows < g.I || max_rows < g.J) {
    for (int z = 0; z < batch; ++z) {
      NtArgs c = g;
      c.A = g.A + z * g.sa;
      c.B = g.B + z * g.sb;
      c.C = g.Cz[z];
      const hipError_t e = launch_gemm_nt(c, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  const int tiles = ((g.I + GTI - 1) / GTI) * ((g.J + GTJ - 1) / GTJ);
  hipLaunchKernelGGL(gemm_nt_bf16_kernel<GRBW>, dim3(tiles, batch), dim3(GThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_expand(const float* G, const float* Rm, half_t* out, int B, int N, int H, int P, int d,
                         hipStream_t s) {
  // The mixing kernel with G as the only projected matrix and R as the coefficients: R's
  // [h][h'*P + j] layout is the mixing coefficients' [m][h][j] with m = h.
  ProjArgs pa{};
  pa.alpha[0] = Rm;
  pa.Yqk = const_cast<float*>(G);
  pa.ywidth = 1;
  pa.Q = out;
  pa.qscale = 1.f;
  pa.B = B;
  pa.N = N;
  pa.D = H * d;
  pa.H = H;
  pa.P = P;
  pa.d = d;
  if (H <= 4) launch_mix_rows<4>(pa, 1, s);
  else if (H <= 8) launch_mix_rows<8>(pa, 1, s);
  else if (H <= 16) launch_mix_rows<16>(pa, 1, s);
  else if (H <= 20) launch_mix_rows<20>(pa, 1, s);
  else if (H <= 32) launch_mix_rows<32>(pa, 1, s);
  else launch_mix_rows<64>(pa, 1, s);
  return hipGetLastError();
}

hipError_t launch_proj_rowmajor(ProjArgs pa, hipStream_t s) {
  const int D = pa.D, M = pa.B * pa.N;
  if (!pa.Vrow || pa.R != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wprep_kernel, dim3(D / 64, D / 64, 3), dim3(256), 0, s, pa, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  NtArgs g{};  // Y = X * [Wt_Q; Wt_K; Wt_V]^T, token-major [M][3D]
  g.A = pa.X;
  g.B = pa.Wt;
  g.C = pa.Yqk;
  g.I = M;
  g.J = 3 * D;
  g.K = D;
  g.ldc = 3 * D;
  if ((e = launch_gemm_nt(g, s)) != hipSuccess) return e;
  pa.ywidth = 3;
  if (pa.H <= 4) launch_mix_rows<4>(pa, 3, s);
  else if (pa.H <= 8) launch_mix_rows<8>(pa, 3, s);
  else if (pa.H <= 16) launch_mix_rows<16>(pa, 3, s);
  else if (pa.H <= 20) launch_mix_rows<20>(pa, 3, s);
  else if (pa.H <= 32) launch_mix_rows<32>(pa, 3, s);
  else launch_mix_rows<64>(pa, 3, s);
  return hipGetLastError();
}

bool proj_fused(const ProjArgs& pa) { return fused_shape(pa.H, pa.D, pa.P); }

hipError_t launch_proj_bf16(const ProjArgs& pa, hipStream_t s, hipEvent_t ev_prep, hipEvent_t ev_gemm) {
  const int D = pa.D, M = pa.B * pa.N;
  const bool fused = proj_fused(pa);
  hipLaunchKernelGGL(wprep_kernel, dim3(D / 64, D / 64, 3), dim3(256), 0, s, pa, fused ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_prep && (e = hipEventRecord(ev_prep, s)) != hipSuccess) return e;
  if (fused) {
    NtArgs g{};  // [Q~ K~ V~] = mix(Wt_perm * X^T)
    g.A = pa.Wt;
    g.B = pa.X;
    g.I = 3 * D;
    g.J = M;
    g.K = D;
    const int ti = pa.H == 20 ? 320 : 256;
    // Buffer offsets are 32-bit: the weights must span < 2 GiB, the tokens are split into
    // launches of < 2 GiB of X each (whole 256-token tiles).
    if (static_cast<int64_t>(3) * D * D * 2 >= (int64_t{1} << 31)) return hipErrorInvalidValue;
    const int64_t max_j = ((int64_t{1} << 31) - 1) / (static_cast<int64_t>(D) * 2) / GTJ * GTJ;
    for (int64_t jb = 0; jb < M; jb += max_j) {
      NtArgs c = g;
      c.B = pa.X + jb * D;
      c.J = static_cast<int>(std::min<int64_t>(max_j, M - jb));
      c.jbase = static_cast<int>(jb);
      // 8-wave 256-token tiles; 4-wave 128-token tiles where the former would leave CUs
      // without a tile (one workgroup per CU: twice the tiles at one wave per SIMD).
      const int64_t tiles8 = static_cast<int64_t>(3 * D / ti) * ((c.J + GTJ - 1) / GTJ);
      const bool small = tiles8 < device_cus();
      const int64_t tiles = small ? static_cast<int64_t>(3 * D / ti) * ((c.J + 127) / 128) : tiles8;
      const int key = (pa.H * 8 + pa.P) * 2 + (small ? 1 : 0);
      switch (key) {
        case (16 * 8 + 1) * 2: hipLaunchKernelGGL((gemm_mix_bf16_kernel<16, 1, 8>), dim3(tiles), dim3(512), 0, s, c, pa); break;
        case (16 * 8 + 2) * 2: hipLaunchKernelGGL((gemm_mix_bf16_kernel<16, 2, 8>), dim3(tiles), dim3(512), 0, s, c, pa); break;
        case (20 * 8 + 1) * 2: hipLaunchKernelGGL((gemm_mix_bf16_kernel<20, 1, 8>), dim3(tiles), dim3(512), 0, s, c, pa); break;
        case (20 * 8 + 2) * 2: hipLaunchKernelGGL((gemm_mix_bf16_kernel<20, 2, 8>), dim3(tiles), dim3(512), 0, s, c, pa); break;
        case (16 * 8 + 1) * 2 + 1: hipLaunchKernelGGL((gemm_mix_bf16_kernel<16, 1, 4>), dim3(tiles), dim3(256), 0, s, c, pa); break;
        case (16 * 8 + 2) * 2 + 1: hipLaunchKernelGGL((gemm_mix_bf16_kernel<16, 2, 4>), dim3(tiles), dim3(256), 0, s, c, pa); break;
        case (20 * 8 + 1) * 2 + 1: hipLaunchKernelGGL((gemm_mix_bf16_kernel<20, 1, 4>), dim3(tiles), dim3(256), 0, s, c, pa); break;
        case (20 * 8 + 2) * 2 + 1: hipLaunchKernelGGL((gemm_mix_bf16_kernel<20, 2, 4>), dim3(tiles), dim3(256), 0, s, c, pa); break;
        default: return hipErrorInvalidValue;
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // the mixing (first rows' fp32 copies included) is part of the GEMM
    if (ev_gemm && (e = hipEventRecord(ev_gemm, s)) != hipSuccess) return e;
    return hipSuccess;
  }
  NtArgs g1{};  // Y_QK = X * Wt_QK^T
  g1.A = pa.X;
  g1.B = pa.Wt;
  g1.C = pa.Yqk;
  g1.I = M;
  g1.J = 2 * D;
  g1.K = D;
  g1.ldc = 2 * D;
  if ((e = launch_gemm_nt(g1, s)) != hipSuccess) return e;
  NtArgs g2{};  // Y_V^T = Wt_V * X^T
  g2.A = pa.Wt + static_cast<int64_t>(2) * D * D;
  g2.B = pa.X;
  g2.C = pa.Yvt;
  g2.I = D;
  g2.J = M;
  g2.K = D;
  g2.ldc = M;
  if ((e = launch_gemm_nt(g2, s)) != hipSuccess) return e;
  if (ev_gemm && (e = hipEventRecord(ev_gemm, s)) != hipSuccess) return e;
  if (pa.H <= 4) launch_mix<4>(pa, s);
  else if (pa.H <= 8) launch_mix<8>(pa, s);
  else if (pa.H <= 16) launch_mix<16>(pa, s);
  else if (pa.H <= 20) launch_mix<20>(pa, s);
  else if (pa.H <= 32) launch_mix<32>(pa, s);
  else launch_mix<64>(pa, s);
  return hipGetLastError();
}

}  // namespace iha
