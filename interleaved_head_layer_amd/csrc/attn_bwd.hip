// Gradients of masked softmax attention over stacked rows: the backward pass of the attention
// step of the IHA forward (Algorithm 1 of the "Interleaved Head Attention" page, step 3), by
// the chain rule through the scaled dot product and the row softmax of the textbook chapter
// "Attention mechanism" (eq. 5.3 and 5.11).  With base-2 scores s = (q . k) * scale, the
// probabilities A = exp2(s - lse) of each row over its visible keys, O = A V and the upstream
// gradient dO:
//   dV = A^T dO,   dA = dO V^T,   dS = A * (dA - D)   with D_i = sum_c dO[i][c] O[i][c]
//   dQ = dS K * scale * ln 2,   dK = dS^T Q * scale * ln 2
// (dS is the gradient of the natural-log scores, which are s * ln 2).  The probabilities are
// recomputed from the forward kernel's per-row base-2 log-sum-exp.
//
// Two matrix-core kernels, both with fp16 operands and fp32 accumulation:
//  * dQ: a workgroup holds 128 query rows (32 per wave, with their dO rows, in registers) and
//    walks the key tiles their masks reach, like the forward: S^T = K Q^T and dA^T = V dO^T
//    give one query per lane, dQ^T += K^T dS^T.  It also writes D.
//  * dK, dV: a workgroup holds 128 keys (32 per wave, with their V rows) and walks the query
//    tiles that see them: S = Q K^T and dA = dO V^T give one key per lane, then
//    dV^T += dO^T A and dK^T += Q^T dS.
// The operand that is contracted over in the second product needs the other orientation, so
// a prep kernel writes channel-major copies of Q, K, V and dO once.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace iha {
namespace {

constexpr int BWaves = 4, BThreads = BWaves * 64;
constexpr int QRows = 128;  // queries per dQ workgroup
constexpr int KTile = 64;   // keys per dQ tile
constexpr int KRows = 128;  // keys per dK/dV workgroup
constexpr int QTile = 32;   // queries per dK/dV tile
constexpr int Pad = 8;      // fp16 padding per LDS row (keeps 16-byte rows, spreads banks)

// Rows of a 32-row MFMA A operand are loaded in this order so that lane half hf of the
// product's output holds rows 16*hf .. 16*hf + 15 of the block in its 16 accumulators - the
// layout the next product takes as its contracted (B operand) dimension.
__device__ __forceinline__ int sigma(int i) { return 16 * ((i >> 2) & 1) + 4 * (i >> 3) + (i & 3); }

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int V>
struct Slot {
  static constexpr int value = V;
};

template <int MASK>
__device__ __forceinline__ bool seen(int q, int k, int L, int window) {
  if (q >= L || k >= L) return false;
  if (MASK == kMaskNone) return true;
  return k <= q && (MASK == kMaskCausal || k > q - window);
}

// Channel-major copies [B][H][d][ld] of the row-major [B][L][H][d] inputs (ld = Lp, zero
// padded past L, for Q*scale, K and dO; ld = L for V, which the forward kernel reads), and
// Q*scale rounded to fp16 in row-major form.  One workgroup per (64-row tile, h, b).
template <int DH>
__global__ __launch_bounds__(BThreads) void bwd_prep_kernel(AttnBwdArgs a) {
  // All four tensors' rows are loaded at once (one round trip), staged in LDS, then written
  // channel-major.
  __shared__ __attribute__((aligned(16))) half_t tile[4][64][DH + Pad];
  constexpr int CH = DH / 8, NL = 64 * CH / BThreads;  // 16-byte chunks per thread and tensor
  static_assert(NL * BThreads == 64 * CH, "tile split");
  const int l0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
  const int L = a.L, H = a.H;
  const int64_t rs = static_cast<int64_t>(H) * DH;
  half8 v[4][NL];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const half_t* src = t == 0 ? a.Q : t == 1 ? a.K : t == 2 ? a.V : a.dO;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = threadIdx.x + i * BThreads, r = idx / CH, c8 = idx % CH, l = l0 + r;
      v[t][i] = half8{};
      if (l < L) v[t][i] = *reinterpret_cast<const half8*>(src + (static_cast<int64_t>(b) * L + l) * rs + h * DH + c8 * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int idx = threadIdx.x + i * BThreads, r = idx / CH, c8 = idx % CH, l = l0 + r;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[0][i][e] = static_cast<half_t>(static_cast<float>(v[0][i][e]) * a.scale);
    if (l < L) *reinterpret_cast<half8*>(a.Qs + (static_cast<int64_t>(b) * L + l) * rs + h * DH + c8 * 8) = v[0][i];
#pragma unroll
    for (int t = 0; t < 4; ++t) *reinterpret_cast<half8*>(&tile[t][r][c8 * 8]) = v[t][i];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    half_t* dst = t == 0 ? a.QsT : t == 1 ? a.KT : t == 2 ? a.VT : a.dOT;
    const int ld = t == 2 ? L : a.Lp;
    half_t* base = dst + static_cast<int64_t>(b * H + h) * DH * ld;
    // Eight consecutive lanes write one channel's 64 positions (128 contiguous bytes).
    for (int idx = threadIdx.x; idx < DH * 8; idx += BThreads) {
      const int c = idx / 8, u = idx % 8, l = l0 + 8 * u;
      if (l >= ld) continue;
      half8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = tile[t][8 * u + e][c];
      half_t* p = base + static_cast<int64_t>(c) * ld + l;
      if (t != 2 || ((L & 7) == 0 && l + 8 <= L)) {
        *reinterpret_cast<half8*>(p) = w;
      } else {
        for (int e = 0; e < 8 && l + e < L; ++e) p[e] = w[e];
      }
    }
  }
}

template <int DH, int MASK>
__global__ __launch_bounds__(BThreads) void bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int NKS = DH / 16, NCB = DH / 32, RS = DH + Pad, TS = KTile + Pad;
  // Two stages: the next tile's loads are held in registers during this tile's products.
  __shared__ __attribute__((aligned(16))) half_t ks[2][KTile][RS];  // K rows of the tile
  __shared__ __attribute__((aligned(16))) half_t vs[2][KTile][RS];  // V rows
  __shared__ __attribute__((aligned(16))) half_t kt[2][DH][TS];     // K^T: [channel][key]
  constexpr int NR = KTile * (DH / 8) / BThreads, NT = DH * (KTile / 8) / BThreads;
  static_assert(NR * BThreads == KTile * (DH / 8) && NT * BThreads == DH * (KTile / 8), "tile split");
  const int L = a.L, H = a.H, window = a.window, Lp = a.Lp;
  // Consecutive logical ids share (b, h) and run on one XCD (its L2 keeps their key tiles);
  // causal rows get longer with the tile index, so causal launches them longest first.
  const int nqt = (L + QRows - 1) / QRows;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt, qt = MASK == kMaskCausal ? nqt - 1 - lid % nqt : lid % nqt;
  const int b = bh / H, h = bh % H, q0 = qt * QRows;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int64_t rs = static_cast<int64_t>(H) * DH;
  const int64_t rbase = static_cast<int64_t>(b) * L * rs + h * DH;  // row-major tensors
  const int64_t tbase = static_cast<int64_t>(b * H + h) * DH * Lp;  // channel-major, padded
  const int64_t sbase = static_cast<int64_t>(b * H + h) * L;        // lse, D
  const int r0 = q0 + 32 * w, qrow = r0 + l32, qload = min(qrow, L - 1);

  // This lane's row: Q*scale and dO fragments (B operands), and D = dO . O over the row (the
  // two lane halves hold the two halves of each 16-channel step).
  half8 qf[NKS], gf[NKS];
  float dd = 0.f;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int64_t off = rbase + static_cast<int64_t>(qload) * rs + (2 * s + hf) * 8;
    qf[s] = *reinterpret_cast<const half8*>(a.Qs + off);
    gf[s] = *reinterpret_cast<const half8*>(a.dO + off);
    const half8 of = *reinterpret_cast<const half8*>(a.O + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dd = fmaf(static_cast<float>(gf[s][e]), static_cast<float>(of[e]), dd);
  }
  dd += __shfl_xor(dd, 32);
  const float lse = qrow < L ? a.lse[sbase + qrow] : __builtin_inff();
  if (hf == 0 && qrow < L) a.D[sbase + qrow] = dd;

  floatx16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  int klo = 0, khi = L;
  if (MASK != kMaskNone) khi = min(L, q0 + QRows);
  if (MASK == kMaskWindow) klo = max(0, q0 - window + 1);
  const int kt0 = klo / KTile, kt1 = (khi + KTile - 1) / KTile;
  // Two register sets: tile t+2's loads are issued before tile t's products and stored to LDS
  // after tile t+1's, so each load has two tiles of products to arrive in.
  half8 pk[2][NR], pv[2][NR], pt[2][NT];
  auto load = [&](int k0, auto S) {
    constexpr int z = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int idx = tid + i * BThreads, r = idx / (DH / 8), c8 = idx % (DH / 8), key = k0 + r;
      pk[z][i] = pv[z][i] = half8{};
      if (key < L) {
        const int64_t off = rbase + static_cast<int64_t>(key) * rs + c8 * 8;
        pk[z][i] = *reinterpret_cast<const half8*>(a.K + off);
        pv[z][i] = *reinterpret_cast<const half8*>(a.V + off);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + i * BThreads, c = idx / (KTile / 8), u = idx % (KTile / 8);
      pt[z][i] = *reinterpret_cast<const half8*>(a.KT + tbase + static_cast<int64_t>(c) * Lp + k0 + u * 8);
    }
  };
  auto store = [&](int st, auto S) {
    constexpr int z = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int idx = tid + i * BThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      *reinterpret_cast<half8*>(&ks[st][r][c8 * 8]) = pk[z][i];
      *reinterpret_cast<half8*>(&vs[st][r][c8 * 8]) = pv[z][i];
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + i * BThreads, c = idx / (KTile / 8), u = idx % (KTile / 8);
      *reinterpret_cast<half8*>(&kt[st][c][u * 8]) = pt[z][i];
    }
  };
  if (kt0 < kt1) {
    load(kt0 * KTile, Slot<0>{});
    store(0, Slot<0>{});
  }
  if (kt0 + 1 < kt1) load((kt0 + 1) * KTile, Slot<1>{});
  __syncthreads();
  // Tile kti (parity stg from kt0) is in LDS stage stg; tile kti + 1 is in register set
  // stg ^ 1; set stg is free for tile kti + 2.
  auto step = [&](int kti, auto P) {
    constexpr int stg = decltype(P)::value;
    const int k0 = kti * KTile;
    if (kti + 2 < kt1) load(k0 + 2 * KTile, P);
    // Tiles with no visible key for the wave's rows are skipped; only tiles that cross a mask
    // edge or the end of the sequence test each pair.
    bool act = true, edge = k0 + KTile > L || r0 + 32 > L;
    if (MASK != kMaskNone) {
      act = k0 <= r0 + 31;
      edge |= k0 + KTile - 1 > r0;
    }
    if (MASK == kMaskWindow) {
      act = act && (k0 + KTile - 1 > r0 - window);
      edge |= k0 <= r0 + 31 - window;
    }
    if (act) {
    floatx16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = dp[kb][r] = 0.f;
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        const int kr = kb * 32 + sigma(l32), col = (2 * st + hf) * 8;
        s[kb] = mfma32(*reinterpret_cast<const half8*>(&ks[stg][kr][col]), qf[st], s[kb]);
        dp[kb] = mfma32(*reinterpret_cast<const half8*>(&vs[stg][kr][col]), gf[st], dp[kb]);
      }
    }
    // Lane (l32, hf), accumulator r of block kb: query qrow, key k0 + 32*kb + 16*hf + r.
    half8 dsf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(s[kb][r] - lse);
        if (edge && !seen<MASK>(qrow, k0 + kb * 32 + 16 * hf + r, L, window)) p = 0.f;
        dsf[kb][r >> 3][r & 7] = static_cast<half_t>(p * (dp[kb][r] - dd));
      }
    // Channel blocks innermost: consecutive products go to independent accumulators.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = mfma32(*reinterpret_cast<const half8*>(&kt[stg][cb * 32 + l32][kb * 32 + 16 * hf + 8 * s2]),
                           dsf[kb][s2], acc[cb]);
    }
    // The other stage was last read before the previous barrier.
    if (kti + 1 < kt1) store(stg ^ 1, Slot<stg ^ 1>{});
    __syncthreads();
  };
  for (int kti = kt0; kti < kt1; kti += 2) {
    step(kti, Slot<0>{});
    if (kti + 1 < kt1) step(kti + 1, Slot<1>{});
  }
  // acc[cb] accumulator r: channel cb*32 + 8*(r/4) + 4*hf + r%4 of query qrow.
  if (qrow < L) {
    float* dst = a.dQ + rbase + static_cast<int64_t>(qrow) * rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * a.dq_scale;
        *reinterpret_cast<floatx4*>(dst + cb * 32 + 8 * q4 + 4 * hf) = v;
      }
  }
}

template <int DH, int MASK>
__global__ __launch_bounds__(BThreads) void bwd_dkdv_kernel(AttnBwdArgs a) {
  constexpr int NKS = DH / 16, NCB = DH / 32, RS = DH + Pad, TS = QTile + Pad;
  __shared__ __attribute__((aligned(16))) half_t qs[2][QTile][RS];  // Q*scale rows of the tile
  __shared__ __attribute__((aligned(16))) half_t gs[2][QTile][RS];  // dO rows
  __shared__ __attribute__((aligned(16))) half_t qt[2][DH][TS];     // (Q*scale)^T: [channel][query]
  __shared__ __attribute__((aligned(16))) half_t gt[2][DH][TS];     // dO^T
  __shared__ __attribute__((aligned(16))) float ls[2][QTile], ds[2][QTile];
  constexpr int NR = QTile * (DH / 8) / BThreads, NT = DH * (QTile / 8) / BThreads;
  static_assert(NR * BThreads == QTile * (DH / 8) && NT * BThreads == DH * (QTile / 8), "tile split");
  const int L = a.L, H = a.H, window = a.window, Lp = a.Lp;
  // Key block 0 sees the most queries: ascending ids run the longest first.
  const int nkt = (L + KRows - 1) / KRows;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nkt, kti = lid % nkt;
  const int b = bh / H, h = bh % H, k0 = kti * KRows;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int64_t rs = static_cast<int64_t>(H) * DH;
  const int64_t rbase = static_cast<int64_t>(b) * L * rs + h * DH;
  const int64_t tbase = static_cast<int64_t>(b * H + h) * DH * Lp;
  const int64_t sbase = static_cast<int64_t>(b * H + h) * L;
  const int kw0 = k0 + 32 * w, krow = kw0 + l32, kload = min(krow, L - 1);

  half8 kf[NKS], vf[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int64_t off = rbase + static_cast<int64_t>(kload) * rs + (2 * s + hf) * 8;
    kf[s] = *reinterpret_cast<const half8*>(a.K + off);
    vf[s] = *reinterpret_cast<const half8*>(a.V + off);
  }
  floatx16 dv[NCB], dk[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[cb][r] = dk[cb][r] = 0.f;

  // Queries that see a key of [k0, k0 + KRows): causal q >= k0, window also q < key + window.
  int qlo = 0, qhi = L;
  if (MASK != kMaskNone) qlo = k0;
  if (MASK == kMaskWindow) qhi = min(L, k0 + KRows - 1 + window);
  const int qt0 = qlo / QTile, qt1 = (qhi + QTile - 1) / QTile;
  half8 pq[2][NR], pg[2][NR], pqt[2][NT], pgt[2][NT];  // two register sets, as in the dQ kernel
  float pl[2] = {0.f, 0.f}, pd[2] = {0.f, 0.f};
  auto load = [&](int q0, auto S) {
    constexpr int z = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int idx = tid + i * BThreads, r = idx / (DH / 8), c8 = idx % (DH / 8), q = q0 + r;
      pq[z][i] = pg[z][i] = half8{};
      if (q < L) {
        const int64_t off = rbase + static_cast<int64_t>(q) * rs + c8 * 8;
        pq[z][i] = *reinterpret_cast<const half8*>(a.Qs + off);
        pg[z][i] = *reinterpret_cast<const half8*>(a.dO + off);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + i * BThreads, c = idx / (QTile / 8), u = idx % (QTile / 8);
      const int64_t off = tbase + static_cast<int64_t>(c) * Lp + q0 + u * 8;
      pqt[z][i] = *reinterpret_cast<const half8*>(a.QsT + off);
      pgt[z][i] = *reinterpret_cast<const half8*>(a.dOT + off);
    }
    if (tid < QTile) {
      const int q = q0 + tid;
      pl[z] = q < L ? a.lse[sbase + q] : __builtin_inff();
      pd[z] = q < L ? a.D[sbase + q] : 0.f;
    }
  };
  auto store = [&](int st, auto S) {
    constexpr int z = decltype(S)::value;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int idx = tid + i * BThreads, r = idx / (DH / 8), c8 = idx % (DH / 8);
      *reinterpret_cast<half8*>(&qs[st][r][c8 * 8]) = pq[z][i];
      *reinterpret_cast<half8*>(&gs[st][r][c8 * 8]) = pg[z][i];
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int idx = tid + i * BThreads, c = idx / (QTile / 8), u = idx % (QTile / 8);
      *reinterpret_cast<half8*>(&qt[st][c][u * 8]) = pqt[z][i];
      *reinterpret_cast<half8*>(&gt[st][c][u * 8]) = pgt[z][i];
    }
    if (tid < QTile) {
      ls[st][tid] = pl[z];
      ds[st][tid] = pd[z];
    }
  };
  if (qt0 < qt1) {
    load(qt0 * QTile, Slot<0>{});
    store(0, Slot<0>{});
  }
  if (qt0 + 1 < qt1) load((qt0 + 1) * QTile, Slot<1>{});
  __syncthreads();
  auto step = [&](int qti, auto P) {
    constexpr int stg = decltype(P)::value;
    const int q0 = qti * QTile;
    if (qti + 2 < qt1) load(q0 + 2 * QTile, P);
    // Visible pairs in (query tile) x (the wave's 32 keys): causal needs kw0 <= q0 + 31,
    // window also q0 < kw0 + 31 + window.
    bool act = true, edge = q0 + QTile > L || kw0 + 32 > L;
    if (MASK != kMaskNone) {
      act = kw0 <= q0 + QTile - 1;
      edge |= kw0 + 31 > q0;
    }
    if (MASK == kMaskWindow) {
      act = act && (q0 < kw0 + 31 + window);
      edge |= q0 + QTile - 1 >= kw0 + window;
    }
    if (act) {
    floatx16 s, dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
    for (int st = 0; st < NKS; ++st) {
      const int qr = sigma(l32), col = (2 * st + hf) * 8;
      s = mfma32(*reinterpret_cast<const half8*>(&qs[stg][qr][col]), kf[st], s);
      dp = mfma32(*reinterpret_cast<const half8*>(&gs[stg][qr][col]), vf[st], dp);
    }
    // Lane (l32, hf), accumulator r: key krow, query q0 + 16*hf + r.
    half8 pf[2], sf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = 16 * hf + r;
      float p = fast_exp2(s[r] - ls[stg][qi]);
      if (edge && !seen<MASK>(q0 + qi, krow, L, window)) p = 0.f;
      pf[r >> 3][r & 7] = static_cast<half_t>(p);
      sf[r >> 3][r & 7] = static_cast<half_t>(p * (dp[r] - ds[stg][qi]));
    }
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int c = cb * 32 + l32, col = 16 * hf + 8 * s2;
        dv[cb] = mfma32(*reinterpret_cast<const half8*>(&gt[stg][c][col]), pf[s2], dv[cb]);
        dk[cb] = mfma32(*reinterpret_cast<const half8*>(&qt[stg][c][col]), sf[s2], dk[cb]);
      }
    }
    if (qti + 1 < qt1) store(stg ^ 1, Slot<stg ^ 1>{});
    __syncthreads();
  };
  for (int qti = qt0; qti < qt1; qti += 2) {
    step(qti, Slot<0>{});
    if (qti + 1 < qt1) step(qti + 1, Slot<1>{});
  }
  // dv[cb], dk[cb] accumulator r: channel cb*32 + 8*(r/4) + 4*hf + r%4 of key krow.
  if (krow < L) {
    const int64_t off = rbase + static_cast<int64_t>(krow) * rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        floatx4 v, k;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = dv[cb][4 * q4 + e];
          k[e] = dk[cb][4 * q4 + e] * a.dk_scale;
        }
        *reinterpret_cast<floatx4*>(a.dV + off + cb * 32 + 8 * q4 + 4 * hf) = v;
        *reinterpret_cast<floatx4*>(a.dK + off + cb * 32 + 8 * q4 + 4 * hf) = k;
      }
  }
}

// dV and dK with the query tiles copied straight from global memory into LDS (buffer loads
// that write LDS, no staging registers), as two kernels so that each fits two or more
// workgroups per CU (several waves per SIMD hide one another's latency): one workgroup's
// registers cannot hold both the dV and the dK accumulators (128 per lane at d = 128) next to
// the K and V fragments.  PART 0 computes dV = A^T dO (needs the scores: Q rows and K), PART 1
// dK = dS^T Q (needs the scores and dA = dO V^T: Q and dO rows, K and V); both recompute the
// scores.  LDS rows are unpadded with XOR-swizzled 16-byte chunks:
//   Q*scale and dO rows [32][DH]: chunk c of row r at c ^ rswz(r) (the score products read rows
//     sigma(l) of 16 lanes: the swizzle spreads them over 16 bank groups);
//   (Q*scale)^T and dO^T [DH][32]: 64-byte rows, chunk c of row r at c ^ ((r >> 2) & 3).
template <int DH>
__device__ __forceinline__ int rswz(int r) {
  return DH == 128 ? ((r & 7) | (((r >> 4) & 1) << 3)) : (r & 7);
}
__device__ __forceinline__ int tswz(int r) { return (r >> 2) & 3; }

template <int DH, int PART>
struct SplitSmem {
  half_t q[2][QTile * DH];                // Q*scale rows
  half_t g[2][PART ? QTile * DH : 8];     // dO rows (dK only)
  half_t t[2][DH * QTile];                // dO^T (dV) or (Q*scale)^T (dK)
  float ls[2][QTile], ds[2][QTile];       // 16-byte aligned: the arrays above are multiples of 16 bytes
};

template <int DH, int MASK, int PART>
__device__ __forceinline__ void bwd_split_body(const AttnBwdArgs& a, SplitSmem<DH, PART>& sm) {
  constexpr int NKS = DH / 16, NCB = DH / 32, CH = DH / 8;
  constexpr int RR = QTile * CH / BThreads;  // copy rounds of the row tiles (1 or 2)
  constexpr int TR = DH * 4 / BThreads;      // copy rounds of the transposed tile (1 or 2)
  static_assert(RR * BThreads == QTile * CH && TR * BThreads == DH * 4, "tile split");
  const int L = a.L, H = a.H, window = a.window, Lp = a.Lp;
  const int nkt = (L + KRows - 1) / KRows;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nkt, kti = lid % nkt;
  const int b = bh / H, h = bh % H, k0 = kti * KRows;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rs = static_cast<int64_t>(H) * DH;
  const int64_t rbase = static_cast<int64_t>(b) * L * rs + h * DH;
  const int64_t tbase = static_cast<int64_t>(b * H + h) * DH * Lp;
  const int64_t sbase = static_cast<int64_t>(b * H + h) * L;
  const int kw0 = k0 + 32 * w, krow = kw0 + l32, kload = min(krow, L - 1);

  // Buffer resources: rows of head h (rows >= L read zero) and the padded channel-major copy.
  const int rbytes = static_cast<int>(((static_cast<int64_t>(L) - 1) * rs + DH) * 2);
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(a.Qs + rbase),
                                                                        static_cast<short>(0), rbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(a.dO + rbase),
                                                                        static_cast<short>(0), rbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<half_t*>((PART ? a.QsT : a.dOT) + tbase), static_cast<short>(0), DH * Lp * 2, 0x00020000);
  // Per-lane byte offsets within a tile: LDS chunk P = (round * 4 + w) * 64 + lane holds row
  // P / CH, logical chunk (P % CH) ^ rswz(row) (row tiles), or row P / 4, chunk (P % 4) ^
  // tswz(row) (the transposed tile).
  unsigned roff[RR], toff[TR];
#pragma unroll
  for (int p = 0; p < RR; ++p) {
    const int P = (p * BWaves + w) * 64 + lane, r = P / CH, c = (P % CH) ^ rswz<DH>(r);
    roff[p] = static_cast<unsigned>((r * rs + c * 8) * 2);
  }
#pragma unroll
  for (int p = 0; p < TR; ++p) {
    const int P = (p * BWaves + w) * 64 + lane, r = P / 4, c = (P % 4) ^ tswz(r);
    toff[p] = static_cast<unsigned>((static_cast<int64_t>(r) * Lp + c * 8) * 2);
  }
  auto issue = [&](int q0, int st) {
    const unsigned rso = static_cast<unsigned>(q0 * rs * 2), tso = static_cast<unsigned>(q0 * 2);
#pragma unroll
    for (int p = 0; p < RR; ++p) {
      const int ld = (p * BWaves + w) * 512;  // halves
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (__attribute__((address_space(3))) void*)(sm.q[st] + ld), 16,
                                               roff[p], rso, 0, 0);
      if (PART)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(grs, (__attribute__((address_space(3))) void*)(sm.g[st] + ld), 16,
                                                 roff[p], rso, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < TR; ++p) {
      const int ld = (p * BWaves + w) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(trs, (__attribute__((address_space(3))) void*)(sm.t[st] + ld), 16,
                                               toff[p], tso, 0, 0);
    }
  };

  half8 kf[NKS], vf[PART ? NKS : 1];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int64_t off = rbase + static_cast<int64_t>(kload) * rs + (2 * s + hf) * 8;
    kf[s] = *reinterpret_cast<const half8*>(a.K + off);
    if (PART) vf[s] = *reinterpret_cast<const half8*>(a.V + off);
  }
  floatx16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  int qlo = 0, qhi = L;
  if (MASK != kMaskNone) qlo = k0;
  if (MASK == kMaskWindow) qhi = min(L, k0 + KRows - 1 + window);
  const int qt0 = qlo / QTile, qt1 = (qhi + QTile - 1) / QTile;
  // lse and D of the next tile's queries pass through registers (rows >= L: +inf and 0, so
  // that a masked pair's values stay finite).
  float pl = 0.f, pd = 0.f;
  auto load_ld = [&](int q0) {
    if (tid < QTile) {
      const int q = q0 + tid;
      pl = q < L ? a.lse[sbase + q] : __builtin_inff();
      if (PART) pd = q < L ? a.D[sbase + q] : 0.f;
    }
  };
  if (qt0 < qt1) {
    issue(qt0 * QTile, 0);
    load_ld(qt0 * QTile);
  }
  wait_vmem();
  if (tid < QTile) {
    sm.ls[0][tid] = pl;
    sm.ds[0][tid] = pd;
  }
  __syncthreads();
  const int qr = sigma(l32);
  // One query tile from LDS stage ST (a constant: every fragment address is a per-lane
  // register plus a fixed offset; the loop below takes two tiles per iteration).  The score
  // products' A fragments (Q*scale rows, and dO rows for dK, alternating) and the transposed
  // tile's fragments are read kPre products ahead of use, the first kPre of the latter during
  // the exponentials (dV, at three workgroups per CU, reads two ahead to stay in its registers).
  // Both product phases run at wave priority 2, rising to 3 halfway (the exponentials at 0):
  // the wave further into its products keeps the matrix core.
  constexpr int kPre = PART ? 4 : 2, NA = PART ? 2 * NKS : NKS, NT = 2 * NCB;
  auto tile = [&](int qti, auto stc) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    const int q0 = qti * QTile;
    const bool more = qti + 1 < qt1;
    if (more) {
      issue(q0 + QTile, ST ^ 1);
      load_ld(q0 + QTile);
    }
    bool act = true, edge = q0 + QTile > L || kw0 + 32 > L;
    if (MASK != kMaskNone) {
      act = kw0 <= q0 + QTile - 1;
      edge |= kw0 + 31 > q0;
    }
    if (MASK == kMaskWindow) {
      act = act && (q0 < kw0 + 31 + window);
      edge |= q0 + QTile - 1 >= kw0 + window;
    }
    if (act) {
      auto afrag = [&](int i) {
        const int k = PART ? i >> 1 : i;
        const half_t* base = (PART && (i & 1)) ? sm.g[ST] : sm.q[ST];
        return *reinterpret_cast<const half8*>(base + qr * DH + ((2 * k + hf) ^ rswz<DH>(qr)) * 8);
      };
      auto tfrag = [&](int j) {  // j = cb * 2 + s2
        const int c = (j >> 1) * 32 + l32;
        return *reinterpret_cast<const half8*>(sm.t[ST] + c * QTile + ((2 * hf + (j & 1)) ^ tswz(c)) * 8);
      };
      floatx16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      half8 fa[NA];
#pragma unroll
      for (int i = 0; i < kPre; ++i) fa[i] = afrag(i);
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(2); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NA / 2; ++i) {
        fa[i + kPre] = afrag(i + kPre);
        if (PART && (i & 1)) dp = mfma32(fa[i], vf[i >> 1], dp);
        else s = mfma32(fa[i], kf[PART ? i >> 1 : i], s);
      }
#pragma unroll
      for (int i = 0; i < NA / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = NA / 2; i < NA; ++i) {
        if (i + kPre < NA) fa[i + kPre] = afrag(i + kPre);
        if (PART && (i & 1)) dp = mfma32(fa[i], vf[i >> 1], dp);
        else s = mfma32(fa[i], kf[PART ? i >> 1 : i], s);
      }
      half8 ft[NT];
#pragma unroll
      for (int j = 0; j < kPre; ++j) ft[j] = tfrag(j);
#pragma unroll
      for (int i = NA / 2; i < NA; ++i) {
        if (i + kPre < NA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
      // Lane (l32, hf), accumulator r: key krow, query q0 + 16*hf + r.  PART 0 keeps the
      // probabilities, PART 1 dS = A * (dA - D).  A tile that crosses a mask edge or the
      // sequence end first sets the scores of the queries that do not see the key to -inf (one
      // unsigned range test each), so that the loop below runs without branches; queries past
      // the end have lse = +inf.  The lane's 16 lse (and D) values are four 16-byte LDS reads.
      if (edge) {
        const int base = q0 + 16 * hf;
        const int lo = max(MASK != kMaskNone ? krow - base : 0, 0);
        const int last = (MASK == kMaskWindow ? min(krow + window - 1, L - 1) : L - 1) - base;
        const unsigned n = krow < L ? static_cast<unsigned>(max(min(last, 15) + 1 - lo, 0)) : 0u;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (static_cast<unsigned>(r - lo) >= n) s[r] = -__builtin_inff();
      }
      floatx4 lq[4], dq4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lq[u] = *reinterpret_cast<const floatx4*>(&sm.ls[ST][16 * hf + 4 * u]);
        if (PART) dq4[u] = *reinterpret_cast<const floatx4*>(&sm.ds[ST][16 * hf + 4 * u]);
      }
      half8 pf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = fast_exp2(s[r] - lq[r >> 2][r & 3]);
        if (PART) v *= dp[r] - dq4[r >> 2][r & 3];
        pf[r >> 3][r & 7] = static_cast<half_t>(v);
      }
      // dV^T += dO^T A  or  dK^T += (Q*scale)^T dS.
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(2); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        if (j + kPre < NT) ft[j + kPre] = tfrag(j + kPre);
        acc[j >> 1] = mfma32(ft[j], pf[j & 1], acc[j >> 1]);
      }
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        if (j + kPre < NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = NT / 2; j < NT; ++j) {
        if (j + kPre < NT) ft[j + kPre] = tfrag(j + kPre);
        acc[j >> 1] = mfma32(ft[j], pf[j & 1], acc[j >> 1]);
      }
#pragma unroll
      for (int j = NT / 2; j < NT; ++j) {
        if (j + kPre < NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();
    if (more && tid < QTile) {
      sm.ls[ST ^ 1][tid] = pl;
      sm.ds[ST ^ 1][tid] = pd;
    }
    __syncthreads();
  };
  for (int qti = qt0; qti < qt1; qti += 2) {
    tile(qti, std::integral_constant<int, 0>{});
    if (qti + 1 < qt1) tile(qti + 1, std::integral_constant<int, 1>{});
  }
  if (krow < L) {
    float* dst = (PART ? a.dK : a.dV) + rbase + static_cast<int64_t>(krow) * rs;
    const float sc = PART ? a.dk_scale : 1.f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * sc;
        *reinterpret_cast<floatx4*>(dst + cb * 32 + 8 * q4 + 4 * hf) = v;
      }
  }
}

// dQ with 32-key tiles copied straight from global memory into LDS (K rows, V rows, K^T: 24 KB
// per stage at d = 128), so that two workgroups fit per CU; the same products as bwd_dq_kernel.
constexpr int KT32 = 32;
template <int DH>
struct DqSmem {
  half_t k[2][KT32 * DH];   // K rows, chunk c of row r at c ^ rswz(r)
  half_t v[2][KT32 * DH];   // V rows, likewise
  half_t kt[2][DH * KT32];  // K^T: [channel][key], chunk c of row r at c ^ tswz(r)
};

// (The bodies of the direct-copy kernels are device functions: a kernel whose own lambdas
// issue the LDS-writing buffer loads loses its host-side launch stub with this compiler.)
template <int DH, int MASK>
__device__ __forceinline__ void bwd_dq_direct_body(const AttnBwdArgs& a, DqSmem<DH>& sm) {
  constexpr int NKS = DH / 16, NCB = DH / 32, CH = DH / 8;
  constexpr int RR = KT32 * CH / BThreads, TR = DH * 4 / BThreads;
  static_assert(RR * BThreads == KT32 * CH && TR * BThreads == DH * 4, "tile split");
  const int L = a.L, H = a.H, window = a.window, Lp = a.Lp;
  const int nqt = (L + QRows - 1) / QRows;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = lid / nqt, qt = MASK == kMaskCausal ? nqt - 1 - lid % nqt : lid % nqt;
  const int b = bh / H, h = bh % H, q0 = qt * QRows;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t rs = static_cast<int64_t>(H) * DH;
  const int64_t rbase = static_cast<int64_t>(b) * L * rs + h * DH;
  const int64_t tbase = static_cast<int64_t>(b * H + h) * DH * Lp;
  const int64_t sbase = static_cast<int64_t>(b * H + h) * L;
  const int r0 = q0 + 32 * w, qrow = r0 + l32, qload = min(qrow, L - 1);

  const int rbytes = static_cast<int>(((static_cast<int64_t>(L) - 1) * rs + DH) * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(a.K + rbase),
                                                                        static_cast<short>(0), rbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(a.V + rbase),
                                                                        static_cast<short>(0), rbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(const_cast<half_t*>(a.KT + tbase),
                                                                        static_cast<short>(0), DH * Lp * 2, 0x00020000);
  unsigned roff[RR], toff[TR];
#pragma unroll
  for (int p = 0; p < RR; ++p) {
    const int P = (p * BWaves + w) * 64 + lane, r = P / CH, c = (P % CH) ^ rswz<DH>(r);
    roff[p] = static_cast<unsigned>((r * rs + c * 8) * 2);
  }
#pragma unroll
  for (int p = 0; p < TR; ++p) {
    const int P = (p * BWaves + w) * 64 + lane, r = P / 4, c = (P % 4) ^ tswz(r);
    toff[p] = static_cast<unsigned>((static_cast<int64_t>(r) * Lp + c * 8) * 2);
  }
  auto issue = [&](int k0, int st) {
    const unsigned rso = static_cast<unsigned>(k0 * rs * 2), tso = static_cast<unsigned>(k0 * 2);
#pragma unroll
    for (int p = 0; p < RR; ++p) {
      const int ld = (p * BWaves + w) * 512;  // halves
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(sm.k[st] + ld), 16,
                                               roff[p], rso, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(sm.v[st] + ld), 16,
                                               roff[p], rso, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < TR; ++p) {
      const int ld = (p * BWaves + w) * 512;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(trs, (__attribute__((address_space(3))) void*)(sm.kt[st] + ld), 16,
                                               toff[p], tso, 0, 0);
    }
  };

  int klo = 0, khi = L;
  if (MASK != kMaskNone) khi = min(L, q0 + QRows);
  if (MASK == kMaskWindow) klo = max(0, q0 - window + 1);
  const int kt0 = klo / KT32, kt1 = (khi + KT32 - 1) / KT32;
  if (kt0 < kt1) issue(kt0 * KT32, 0);

  // This lane's row: Q*scale and dO fragments (B operands), and D = dO . O over the row.
  half8 qf[NKS], gf[NKS];
  float dd = 0.f;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int64_t off = rbase + static_cast<int64_t>(qload) * rs + (2 * s + hf) * 8;
    qf[s] = *reinterpret_cast<const half8*>(a.Qs + off);
    gf[s] = *reinterpret_cast<const half8*>(a.dO + off);
    const half8 of = *reinterpret_cast<const half8*>(a.O + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) dd = fmaf(static_cast<float>(gf[s][e]), static_cast<float>(of[e]), dd);
  }
  dd += __shfl_xor(dd, 32);
  const float lse = qrow < L ? a.lse[sbase + qrow] : __builtin_inff();
  if (hf == 0 && qrow < L) a.D[sbase + qrow] = dd;

  floatx16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;
  wait_vmem();
  __syncthreads();
  const int kr = sigma(l32);
  // One key tile from LDS stage ST (a constant; two tiles per iteration below).  The score
  // products' A fragments (K rows and V rows, alternating) and the K^T fragments are read
  // kPre products ahead of use, the first kPre K^T fragments during the exponentials.  Wave
  // priority as in the dK and dV kernels.
  constexpr int kPre = 4, NA = 2 * NKS, NT = 2 * NCB;
  auto tile = [&](int kti, auto stc) __attribute__((always_inline)) {
    constexpr int ST = decltype(stc)::value;
    const int k0 = kti * KT32;
    if (kti + 1 < kt1) issue(k0 + KT32, ST ^ 1);
    bool act = true, edge = k0 + KT32 > L || r0 + 32 > L;
    if (MASK != kMaskNone) {
      act = k0 <= r0 + 31;
      edge |= k0 + KT32 - 1 > r0;
    }
    if (MASK == kMaskWindow) {
      act = act && (k0 + KT32 - 1 > r0 - window);
      edge |= k0 <= r0 + 31 - window;
    }
    if (act) {
      auto afrag = [&](int i) {
        const half_t* base = (i & 1) ? sm.v[ST] : sm.k[ST];
        return *reinterpret_cast<const half8*>(base + kr * DH + ((2 * (i >> 1) + hf) ^ rswz<DH>(kr)) * 8);
      };
      auto tfrag = [&](int j) {  // j = s2 * NCB + cb
        const int c = (j % NCB) * 32 + l32;
        return *reinterpret_cast<const half8*>(sm.kt[ST] + c * KT32 + ((2 * hf + j / NCB) ^ tswz(c)) * 8);
      };
      floatx16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
      half8 fa[NA];
#pragma unroll
      for (int i = 0; i < kPre; ++i) fa[i] = afrag(i);
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(2); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NA / 2; ++i) {
        fa[i + kPre] = afrag(i + kPre);
        if (i & 1) dp = mfma32(fa[i], gf[i >> 1], dp);
        else s = mfma32(fa[i], qf[i >> 1], s);
      }
#pragma unroll
      for (int i = 0; i < NA / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = NA / 2; i < NA; ++i) {
        if (i + kPre < NA) fa[i + kPre] = afrag(i + kPre);
        if (i & 1) dp = mfma32(fa[i], gf[i >> 1], dp);
        else s = mfma32(fa[i], qf[i >> 1], s);
      }
      half8 ft[NT];
#pragma unroll
      for (int j = 0; j < kPre; ++j) ft[j] = tfrag(j);
#pragma unroll
      for (int i = NA / 2; i < NA; ++i) {
        if (i + kPre < NA) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, kPre, 0);
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
      // Lane (l32, hf), accumulator r: query qrow, key k0 + 16*hf + r.  A tile that crosses a
      // mask edge or the sequence end first sets the scores of the keys the row does not see to
      // -inf (one unsigned range test each: keys lo .. lo + n - 1 of the lane's 16 are seen),
      // so that the loop below runs without branches; a row past the end has lse = +inf.
      if (edge) {
        const int base = k0 + 16 * hf;
        const int last = (MASK == kMaskNone ? L - 1 : min(qrow, L - 1)) - base;
        const int lo = max(MASK == kMaskWindow ? qrow - window + 1 - base : 0, 0);
        const unsigned n = static_cast<unsigned>(max(min(last, 15) + 1 - lo, 0));
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (static_cast<unsigned>(r - lo) >= n) s[r] = -__builtin_inff();
      }
      half8 dsf[2];
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dsf[r >> 3][r & 7] = static_cast<half_t>(fast_exp2(s[r] - lse) * (dp[r] - dd));
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(2); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        if (j + kPre < NT) ft[j + kPre] = tfrag(j + kPre);
        acc[j % NCB] = mfma32(ft[j], dsf[j / NCB], acc[j % NCB]);
      }
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        if (j + kPre < NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(3); __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = NT / 2; j < NT; ++j) {
        if (j + kPre < NT) ft[j + kPre] = tfrag(j + kPre);
        acc[j % NCB] = mfma32(ft[j], dsf[j / NCB], acc[j % NCB]);
      }
#pragma unroll
      for (int j = NT / 2; j < NT; ++j) {
        if (j + kPre < NT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0); __builtin_amdgcn_s_setprio(0); __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();
    __syncthreads();
  };
  for (int kti = kt0; kti < kt1; kti += 2) {
    tile(kti, std::integral_constant<int, 0>{});
    if (kti + 1 < kt1) tile(kti + 1, std::integral_constant<int, 1>{});
  }
  if (qrow < L) {
    float* dst = a.dQ + rbase + static_cast<int64_t>(qrow) * rs;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        floatx4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * q4 + e] * a.dq_scale;
        *reinterpret_cast<floatx4*>(dst + cb * 32 + 8 * q4 + 4 * hf) = v;
      }
  }
}

// dQ: about 190 registers at d = 128, two workgroups per CU.
template <int DH, int MASK>
__global__ __launch_bounds__(BThreads, 2) void bwd_dq_direct_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) DqSmem<DH> sm;
  bwd_dq_direct_body<DH, MASK>(a, sm);
}

// dV: about 150-160 registers at d = 128, three workgroups per CU; dK: about 200, two.
template <int DH, int MASK>
__global__ __launch_bounds__(BThreads, 3) void bwd_dv_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) SplitSmem<DH, 0> sm;
  bwd_split_body<DH, MASK, 0>(a, sm);
}
template <int DH, int MASK>
__global__ __launch_bounds__(BThreads, 2) void bwd_dk_kernel(AttnBwdArgs a) {
  __shared__ __attribute__((aligned(16))) SplitSmem<DH, 1> sm;
  bwd_split_body<DH, MASK, 1>(a, sm);
}

template <int DH, int MASK>
hipError_t launch_grads(const AttnBwdArgs& a, hipStream_t s) {
  const int nqt = (a.L + QRows - 1) / QRows, nkt = (a.L + KRows - 1) / KRows;
  // Direct tile copies need 32-bit byte offsets within one (b, h)'s rows and channel-major copy.
  const bool direct = static_cast<int64_t>(a.L) * a.H * DH * 2 < (int64_t{1} << 31) &&
                      static_cast<int64_t>(DH) * a.Lp * 2 < (int64_t{1} << 31);
  // dQ first: it writes D = dO . O, which dK reads.
  if (direct)
    hipLaunchKernelGGL((bwd_dq_direct_kernel<DH, MASK>), dim3(nqt * a.H * a.B), dim3(BThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<DH, MASK>), dim3(nqt * a.H * a.B), dim3(BThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (direct) {
    hipLaunchKernelGGL((bwd_dv_kernel<DH, MASK>), dim3(nkt * a.H * a.B), dim3(BThreads), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dk_kernel<DH, MASK>), dim3(nkt * a.H * a.B), dim3(BThreads), 0, s, a);
  } else
    hipLaunchKernelGGL((bwd_dkdv_kernel<DH, MASK>), dim3(nkt * a.H * a.B), dim3(BThreads), 0, s, a);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_bwd_d(const AttnBwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((bwd_prep_kernel<DH>), dim3(a.Lp / 64, a.H, a.B), dim3(BThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Forward recompute: O (fp16) and the per-row log-sum-exp, from the scaled Q.
  AttnArgs f{};
  f.Q = a.Qs;
  f.K = a.K;
  f.Vt = a.VT;
  f.Oh = a.O;
  f.B = a.B;
  f.L = a.L;
  f.H = a.H;
  f.d = DH;
  f.mask = a.mask;
  f.window = a.window;
  f.qk_scale = 1.f;
  f.qk_layout = kQKRowMajor;
  f.lse = a.lse;
  e = launch_attn_f16(f, s);
  if (e != hipSuccess) return e;
  switch (a.mask) {
    case kMaskNone: return launch_grads<DH, kMaskNone>(a, s);
    case kMaskCausal: return launch_grads<DH, kMaskCausal>(a, s);
    default: return launch_grads<DH, kMaskWindow>(a, s);
  }
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdArgs& a, hipStream_t s) {
  if (a.Lp % 64 != 0 || a.Lp < a.L) return hipErrorInvalidValue;
  switch (a.d) {
    case 64: return launch_bwd_d<64>(a, s);
    case 128: return launch_bwd_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace iha
