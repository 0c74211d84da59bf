// Host side of the C ABI declared in include/iha.h: argument validation, workspace
// layout and the launch sequence of the IHA forward pass (Algorithm 1 of the
// "Interleaved Head Attention" page, section 4).
#include "iha.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxH = 64;
constexpr int64_t kMaxRows = int64_t(1) << 30;   // B*N tokens and P*N stacked rows
constexpr int64_t kMaxElems = int64_t(1) << 40;  // elements of any one tensor

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

struct Layout {
  size_t flag, wt, yqk, yvt, q, k, vt, pbar, pe, qe, ke, vte, ye, total;
  int R;   // precise first stacked rows (0 when unused)
  int R2;  // stacked rows with fp32 attention outputs (R <= R2; 0 when unused)
};

bool d_supported(int32_t dtype, int64_t d) {
  if (dtype == IHA_BF16) return d == 64 || d == 128;
  return d == 16 || d == 32 || d == 64 || d == 128;
}

iha_status validate(const iha_problem* p) {
  if (!p) return IHA_ERR_INVALID_ARG;
  if (p->B < 1 || p->N < 1 || p->D < 1 || p->H < 1 || p->P < 1) return IHA_ERR_INVALID_ARG;
  if (p->mask < IHA_MASK_NONE || p->mask > IHA_MASK_WINDOW) return IHA_ERR_INVALID_ARG;
  if (p->dtype != IHA_F32 && p->dtype != IHA_BF16) return IHA_ERR_INVALID_ARG;
  if ((p->flags & ~(IHA_FLAG_CHECK | IHA_FLAG_FUSED_COLLAPSE)) != 0 || p->reserved != 0) return IHA_ERR_INVALID_ARG;
  if (p->D % p->H != 0) return IHA_ERR_SHAPE;
  if ((p->flags & IHA_FLAG_FUSED_COLLAPSE) && p->dtype != IHA_BF16) return IHA_ERR_UNSUPPORTED;
  if (p->H > kMaxH || p->H * p->H * p->P > 16384) return IHA_ERR_UNSUPPORTED;
  if (!d_supported(p->dtype, p->D / p->H)) return IHA_ERR_UNSUPPORTED;
  if (p->dtype == IHA_BF16) {
    // mixing kernels stage alpha as [H][P][Hmax] floats in 64 KB of LDS
    const int64_t hmax = p->H <= 4 ? 4 : p->H <= 8 ? 8 : p->H <= 16 ? 16 : p->H <= 20 ? 20 : p->H <= 32 ? 32 : 64;
    if (p->H * p->P * hmax > 16384) return IHA_ERR_UNSUPPORTED;
  }
  if (p->B * p->N > kMaxRows || p->P * p->N > kMaxRows || p->P > kMaxRows) return IHA_ERR_SHAPE;
  if (p->B * p->N * p->P * p->D > kMaxElems / 4 || 3 * p->P * p->D * p->D > kMaxElems / 4)
    return IHA_ERR_SHAPE;
  // Every row of a window mask of width < 1 is empty (textbook section 5.3: a legal query
  // with an empty allowed set is an error).
  if (p->mask == IHA_MASK_WINDOW && p->window < 1) return IHA_ERR_EMPTY_ROW;
  return IHA_OK;
}

Layout layout_of(const iha_problem& p) {
  const size_t e = p.dtype == IHA_BF16 ? 2 : 4;
  const size_t d = static_cast<size_t>(p.D / p.H);
  const size_t M = static_cast<size_t>(p.B) * p.N;          // tokens over the batch
  const size_t act = M * p.P * p.H * d;                      // elements of Q~, K~, V~, P-bar
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L.flag = take(kAlign);
  if (p.dtype == IHA_BF16) {
    // transposed weights, fp32 projections (token-major Q|K, channel-major V)
    L.wt = take(3 * static_cast<size_t>(p.D) * p.D * 2);
    if (!iha::fused_shape(p.H, p.D, p.P)) {
      L.yqk = take(M * 2 * p.D * 4);
      L.yvt = take(M * p.D * 4);
    }
  } else {
    L.wt = take(3 * static_cast<size_t>(p.P) * p.D * p.D * 4);  // folded weights
  }
  L.q = take(act * e);
  L.k = take(act * e);
  L.vt = take(act * e);
  L.pbar = take(act * e);  // stacked attention outputs: fp16 (bf16 inputs) or fp32
  // bf16 inputs under a causal or window mask: the first rows' fp32 attention outputs, and
  // fp32 copies of their mixed queries, keys and values (fused path: the unmixed fp32
  // projections of the first tokens instead, mixed by the attention launch).
  if (p.dtype == IHA_BF16 && p.mask != IHA_MASK_NONE) {
    const int64_t R = std::min<int64_t>(iha::kPreciseRows, p.P * p.N);
    L.R = static_cast<int>(R);
    L.R2 = static_cast<int>(std::min<int64_t>(iha::kF32OutRows, p.P * p.N));
    L.pe = take(static_cast<size_t>(p.B) * L.R2 * p.D * 4);
    if (iha::fused_shape(p.H, p.D, p.P)) {
      L.ye = take(static_cast<size_t>(p.B) * ((R + p.P - 1) / p.P) * 3 * p.D * 4);
    } else {
      L.qe = take(static_cast<size_t>(p.B) * R * p.D * 4);
      L.ke = take(static_cast<size_t>(p.B) * R * p.D * 4);
      L.vte = take(static_cast<size_t>(p.B) * R * p.D * 4);
    }
  }
  L.total = off;
  return L;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("IHA_LOG");
    return v && v[0] == '1';
  }();
  return on;
}

#define IHA_HIP(call)                                                              \
  do {                                                                             \
    hipError_t e_ = (call);                                                        \
    if (e_ != hipSuccess) {                                                        \
      if (log_enabled()) std::fprintf(stderr, "[iha] %s: %s\n", #call, hipGetErrorString(e_)); \
      return IHA_ERR_DEVICE;                                                       \
    }                                                                              \
  } while (0)

// Precedence: an empty row, then a non-finite input, then an fp16 range overflow, then a
// non-finite output (which without the two causes before it has no other source).
iha_status read_flag(const unsigned* flag, hipStream_t stream) {
  unsigned host = 0;
  IHA_HIP(hipStreamSynchronize(stream));
  IHA_HIP(hipMemcpy(&host, flag, sizeof(host), hipMemcpyDeviceToHost));
  if (host & iha::kFlagEmptyRow) return IHA_ERR_EMPTY_ROW;
  if (host & iha::kFlagInputNonFinite) return IHA_ERR_NONFINITE;
  if (host & iha::kFlagRange) return IHA_ERR_RANGE;
  if (host & iha::kFlagNonFinite) return IHA_ERR_NONFINITE;
  return IHA_OK;
}

iha_status forward_impl(const iha_problem* prob, const void* X, const void* W_Q, const void* W_K,
                        const void* W_V, const float* alpha_Q, const float* alpha_K,
                        const float* alpha_V, const float* R, float* X_out, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, hipEvent_t* ev) {
  const iha_status v = validate(prob);
  if (v != IHA_OK) return v;
  if (!X || !W_Q || !W_K || !W_V || !alpha_Q || !alpha_K || !alpha_V || !R || !X_out)
    return IHA_ERR_INVALID_ARG;
  // The kernels move X, W and X_out in 16-byte vectors and alpha, R as floats.
  if (!aligned(X, 16) || !aligned(W_Q, 16) || !aligned(W_K, 16) || !aligned(W_V, 16) ||
      !aligned(X_out, 16) || !aligned(alpha_Q, 4) || !aligned(alpha_K, 4) || !aligned(alpha_V, 4) ||
      !aligned(R, 4))
    return IHA_ERR_INVALID_ARG;
  const iha_problem& p = *prob;
  const Layout lay = layout_of(p);
  if (!workspace || workspace_bytes < lay.total ||
      reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return IHA_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  unsigned* flag = reinterpret_cast<unsigned*>(ws + lay.flag);
  const int B = static_cast<int>(p.B), N = static_cast<int>(p.N), D = static_cast<int>(p.D);
  const int H = static_cast<int>(p.H), P = static_cast<int>(p.P), d = D / H;
  const bool bf16 = p.dtype == IHA_BF16;
  if (log_enabled())
    std::fprintf(stderr, "[iha] forward B=%d N=%d D=%d H=%d d=%d P=%d mask=%d window=%lld dtype=%s\n",
                 B, N, D, H, d, P, p.mask, static_cast<long long>(p.window), bf16 ? "bf16" : "f32");

  if (ev) IHA_HIP(hipEventRecord(ev[0], stream));
  int qk_layout = iha::kQKRowMajor;
  if (bf16) {
    // Steps 1-2: exact bf16 projections (fp32 accumulation), fp32 mixing into the stacked
    // fp16 layouts (and fp32 copies of the first rows).
    iha::ProjArgs pa{};
    pa.X = static_cast<const uint16_t*>(X);
    pa.W[0] = static_cast<const uint16_t*>(W_Q);
    pa.W[1] = static_cast<const uint16_t*>(W_K);
    pa.W[2] = static_cast<const uint16_t*>(W_V);
    pa.alpha[0] = alpha_Q;
    pa.alpha[1] = alpha_K;
    pa.alpha[2] = alpha_V;
    pa.Wt = reinterpret_cast<uint16_t*>(ws + lay.wt);
    const bool fused = iha::fused_shape(H, D, P);  // no fp32 projections in HBM
    pa.Yqk = fused ? nullptr : reinterpret_cast<float*>(ws + lay.yqk);
    pa.Yvt = fused ? nullptr : reinterpret_cast<float*>(ws + lay.yvt);
    pa.Q = reinterpret_cast<iha::half_t*>(ws + lay.q);
    pa.K = reinterpret_cast<iha::half_t*>(ws + lay.k);
    pa.Vt = reinterpret_cast<iha::half_t*>(ws + lay.vt);
    if (lay.R > 0 && fused) {
      pa.Ye = reinterpret_cast<float*>(ws + lay.ye);
    } else if (lay.R > 0) {
      pa.Qe = reinterpret_cast<float*>(ws + lay.qe);
      pa.Ke = reinterpret_cast<float*>(ws + lay.ke);
      pa.Ve = reinterpret_cast<float*>(ws + lay.vte);
    }
    pa.B = B;
    pa.N = N;
    pa.D = D;
    pa.H = H;
    pa.d = d;
    pa.P = P;
    pa.R = lay.R;
    pa.T0 = (lay.R + P - 1) / P;
    pa.qscale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
    pa.flag = flag;  // cleared by the weight transpose
    if (iha::proj_fused(pa)) qk_layout = iha::kQKChunked;
    IHA_HIP(iha::launch_proj_bf16(pa, stream, ev ? ev[1] : nullptr, ev ? ev[2] : nullptr));
  } else {
    // Step 1: mixing folded into the weights (fp32); step 2: fp32 projection GEMM.
    iha::FoldArgs fa{};
    fa.W[0] = W_Q;
    fa.W[1] = W_K;
    fa.W[2] = W_V;
    fa.alpha[0] = alpha_Q;
    fa.alpha[1] = alpha_K;
    fa.alpha[2] = alpha_V;
    fa.out_scale[0] = fa.out_scale[1] = fa.out_scale[2] = 1.f;
    fa.Wt = ws + lay.wt;
    fa.flag = flag;
    fa.D = D;
    fa.H = H;
    fa.d = d;
    fa.P = P;
    IHA_HIP(iha::launch_fold_f32(fa, stream));
    if (ev) IHA_HIP(hipEventRecord(ev[1], stream));
    iha::GemmArgs g{};
    g.A = X;
    g.Bt = ws + lay.wt;
    g.Q = ws + lay.q;
    g.K = ws + lay.k;
    g.Vt = ws + lay.vt;
    g.M = B * N;
    g.Kdim = D;
    g.Ncol = 3 * P * H * d;
    g.PHd = P * H * d;
    g.Ntok = N;
    g.P = P;
    g.H = H;
    g.d = d;
    IHA_HIP(iha::launch_gemm_f32(g, stream));
    if (ev) IHA_HIP(hipEventRecord(ev[2], stream));  // no separate mixing step
  }
  if (ev) IHA_HIP(hipEventRecord(ev[3], stream));

  // Step 3: per-head masked attention over the P*N stacked rows.
  iha::AttnArgs at{};
  at.Q = ws + lay.q;
  at.K = ws + lay.k;
  at.Vt = ws + lay.vt;
  at.flag = flag;
  at.B = B;
  at.L = P * N;
  at.H = H;
  at.d = d;
  at.mask = p.mask;
  at.window = p.mask == IHA_MASK_WINDOW
                  ? static_cast<int>(p.window < at.L ? p.window : static_cast<int64_t>(at.L))
                  : 0;
  const float score_scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
  at.qk_scale = score_scale;
  if (bf16) {
    at.qk_scale = 1.f;  // the fp16 Q was stored pre-scaled
    at.qk_layout = qk_layout;
    at.Oh = reinterpret_cast<iha::half_t*>(ws + lay.pbar);  // fp16 stacked outputs
    if (lay.R > 0) {
      // The first stacked rows again, in fp32, by extra workgroups of the same launch (their
      // outputs are the largest).
      if (iha::fused_shape(H, D, P)) {
        at.Ye = reinterpret_cast<const float*>(ws + lay.ye);
        at.alpha[0] = alpha_Q;
        at.alpha[1] = alpha_K;
        at.alpha[2] = alpha_V;
      } else {
        at.Qe = reinterpret_cast<const float*>(ws + lay.qe);
        at.Ke = reinterpret_cast<const float*>(ws + lay.ke);
        at.Ve = reinterpret_cast<const float*>(ws + lay.vte);
      }
      at.Pe = reinterpret_cast<float*>(ws + lay.pe);
      at.R = lay.R;
      at.R2 = lay.R2;
      at.P = P;
      at.T0 = (lay.R + P - 1) / P;
      at.escale = score_scale;
    }
    if (p.flags & IHA_FLAG_FUSED_COLLAPSE) {
      IHA_HIP(iha::launch_fill_zero(X_out, static_cast<int64_t>(B) * N * D, stream));
      at.Xf = X_out;
      at.Rm = R;
      at.P = P;
    }
    IHA_HIP(iha::launch_attn_f16(at, stream));
  } else {
    at.O = reinterpret_cast<float*>(ws + lay.pbar);
    IHA_HIP(iha::launch_attn_f32(at, stream));
  }
  if (ev) IHA_HIP(hipEventRecord(ev[4], stream));
  if (ev) IHA_HIP(hipEventRecord(ev[5], stream));  // (first rows: part of the attention launch)

  // Steps 4-5: unstack, collapse with R, concatenate heads (with the fused collapse the
  // attention launch has done them).
  if (!(p.flags & IHA_FLAG_FUSED_COLLAPSE)) {
    if (bf16)
      IHA_HIP(iha::launch_collapse_h(at.Oh, lay.R2 > 0 ? reinterpret_cast<const float*>(ws + lay.pe) : nullptr,
                                     lay.R2, R, X_out, B, N, H, P, d, stream));
    else
      IHA_HIP(iha::launch_collapse(at.O, R, X_out, B * N, H, P, d, stream));
  }
  if (ev) IHA_HIP(hipEventRecord(ev[6], stream));

  if (p.flags & IHA_FLAG_CHECK) {
    // Inputs: non-finite values; for bf16 inputs also alpha and R beyond the fp16 range (the
    // matrix-core mixing and collapse split them into fp16 high and low parts).  Then the fp16
    // stacked Q~, K~, V~: with finite inputs a non-finite value there means a projection or
    // a mixed value beyond the fp16 range.  Last the output.
    using iha::kFlagInputNonFinite;
    const int xk = bf16 ? iha::kValBF16 : iha::kValF32;
    const float lim = bf16 ? iha::kF16Max : __builtin_inff();
    const int64_t nx = static_cast<int64_t>(B) * N * D, nw = static_cast<int64_t>(D) * D;
    const int64_t na = static_cast<int64_t>(H) * H * P;
    IHA_HIP(iha::launch_check_values(X, xk, nx, flag, kFlagInputNonFinite, __builtin_inff(), stream));
    for (const void* W : {W_Q, W_K, W_V})
      IHA_HIP(iha::launch_check_values(W, xk, nw, flag, kFlagInputNonFinite, __builtin_inff(), stream));
    for (const float* a : {alpha_Q, alpha_K, alpha_V})
      IHA_HIP(iha::launch_check_values(a, iha::kValF32, na, flag, kFlagInputNonFinite, lim, stream));
    IHA_HIP(iha::launch_check_values(R, iha::kValF32, na, flag, kFlagInputNonFinite, lim, stream));
    if (bf16) {
      const int64_t act = static_cast<int64_t>(B) * N * P * D;
      for (size_t off : {lay.q, lay.k, lay.vt})
        IHA_HIP(iha::launch_check_values(ws + off, iha::kValF16, act, flag, iha::kFlagRange, __builtin_inff(),
                                         stream));
    }
    IHA_HIP(iha::launch_check_values(X_out, iha::kValF32, nx, flag, iha::kFlagNonFinite, __builtin_inff(), stream));
    return read_flag(flag, stream);
  }
  return IHA_OK;
}

// Workspace of iha_attention_backward: fp16 Q*scale, channel-major copies (Q*scale, K and dO
// with rows padded to Lp, V with L), the recomputed fp16 forward output, and fp32 lse and D.
struct BwdLayout {
  size_t qs, qst, kt, dot, vt, o, lse, dd, total;
  int64_t Lp;
};

BwdLayout bwd_layout(int64_t B, int64_t L, int64_t H, int64_t d) {
  BwdLayout l{};
  l.Lp = (L + 63) / 64 * 64;
  const size_t E = static_cast<size_t>(B * L * H * d), Et = static_cast<size_t>(B * H * d * l.Lp);
  const size_t S = static_cast<size_t>(B * H * L);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  l.qs = take(E * 2);
  l.qst = take(Et * 2);
  l.kt = take(Et * 2);
  l.dot = take(Et * 2);
  l.vt = take(E * 2);
  l.o = take(E * 2);
  l.lse = take(S * 4);
  l.dd = take(S * 4);
  l.total = off;
  return l;
}

iha_status bwd_validate(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask, int64_t window) {
  if (B < 1 || L < 1 || H < 1 || mask < IHA_MASK_NONE || mask > IHA_MASK_WINDOW) return IHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return IHA_ERR_UNSUPPORTED;
  if (H > kMaxH || B > 65535 || L > kMaxRows || B * (L + 63) * H * d > kMaxElems / 4) return IHA_ERR_SHAPE;
  if (mask == IHA_MASK_WINDOW && window < 1) return IHA_ERR_EMPTY_ROW;
  return IHA_OK;
}

// Workspace of iha_backward (bf16 inputs).  The fp32 projections Y = X [W_Q | W_K | W_V] are
// kept for the mixing gradient and then overwritten with the projection gradients dY.
struct LayerBwdLayout {
  size_t flag, wt, y, qb, kb, vb, dpb, dq, dk, dv, att, part, dycat, dyt, xt, wcat, wsplit, total;
  int64_t Mp;  // tokens rounded up to 64 (the K dimension of the weight-gradient GEMM)
  int splits;  // parts of the weight-gradient GEMM's contracted (token) dimension
  BwdLayout a;
};

// The three weight-gradient products have few 256 x 256 tiles (D/256 squared each): split their
// 2 Mp-long contracted dimension until the launch has about three rounds of workgroups.
int dw_splits(int64_t D, int64_t Mp) {
  const int64_t tiles = ((D + 255) / 256) * ((D + 255) / 256);
  int s = 1;
  while (s < 4 && 3 * tiles * s < 3 * 256 && (2 * Mp) % (64 * 2 * s) == 0) s *= 2;
  return s;
}

LayerBwdLayout layer_bwd_layout(const iha_problem& p) {
  LayerBwdLayout l{};
  const size_t M = static_cast<size_t>(p.B) * p.N, D = static_cast<size_t>(p.D);
  const size_t act = M * p.P * D;  // elements of each stacked tensor
  l.Mp = (static_cast<int64_t>(M) + 63) / 64 * 64;
  l.a = bwd_layout(p.B, p.P * p.N, p.H, p.D / p.H);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  l.flag = take(kAlign);
  l.wt = take(3 * D * D * 2);
  l.y = take(M * 3 * D * 4);
  l.qb = take(act * 2);
  l.kb = take(act * 2);
  l.vb = take(act * 2);
  l.dpb = take(act * 2);
  l.dq = take(act * 4);
  l.dk = take(act * 4);
  l.dv = take(act * 4);
  l.att = take(l.a.total);
  l.part = take(iha::head_reduce_part_bytes(static_cast<int>(M), static_cast<int>(p.H), static_cast<int>(p.P)));
  // bf16 high and low parts of dY (token-major [M][6D]: high 3D then low 3D; channel-major
  // [3D][2Mp]: high Mp then low Mp), X^T twice ([D][2Mp]) and [W_Q | W_K | W_V] twice ([D][6D]).
  l.dycat = take(M * 6 * D * 2);
  l.dyt = take(3 * D * 2 * static_cast<size_t>(l.Mp) * 2);
  l.xt = take(D * 2 * static_cast<size_t>(l.Mp) * 2);
  l.wcat = take(D * 6 * D * 2);
  l.splits = dw_splits(static_cast<int64_t>(D), l.Mp);
  l.wsplit = take(l.splits > 1 ? static_cast<size_t>(l.splits) * 3 * D * D * 4 : 0);
  l.total = off;
  return l;
}

iha_status layer_bwd_validate(const iha_problem* p) {
  const iha_status v = validate(p);
  if (v != IHA_OK) return v;
  if (p->dtype != IHA_BF16) return IHA_ERR_UNSUPPORTED;
  const iha_status a = bwd_validate(p->B, p->P * p->N, p->H, p->D / p->H, p->mask, p->window);
  if (a != IHA_OK) return a;
  // The weight-gradient GEMM reads 256 rows of 2*Mp bf16 values per tile: under 2 GiB.
  if ((p->B * p->N + 63) / 64 * 64 * 2 * 2 * 256 >= (int64_t{1} << 31)) return IHA_ERR_SHAPE;
  return IHA_OK;
}

// Workspace of iha_forward_static: one copy per device, held until the process ends.  In
// host code `scratch` names a host-side stand-in, never the device memory: host code uses
// only the per-device address that hipGetSymbolAddress returns for it.
constexpr size_t kStaticBytes = IHA_STATIC_WORKSPACE_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
iha_status static_workspace(void** ptr) {
  int dev = -1;
  IHA_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return IHA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    IHA_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return IHA_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return IHA_OK;
}

}  // namespace

extern "C" {

iha_status iha_workspace_bytes(const iha_problem* prob, size_t* bytes) {
  if (!bytes) return IHA_ERR_INVALID_ARG;
  const iha_status v = validate(prob);
  if (v != IHA_OK) return v;
  *bytes = layout_of(*prob).total;
  return IHA_OK;
}

iha_status iha_plan(const iha_problem* prob, uint32_t* plan) {
  if (!plan) return IHA_ERR_INVALID_ARG;
  const iha_status v = validate(prob);
  if (v != IHA_OK) return v;
  *plan = prob->dtype == IHA_BF16 && iha::fused_shape(prob->H, prob->D, prob->P) ? IHA_PLAN_MIX_FUSED : 0u;
  return IHA_OK;
}

iha_status iha_forward(const iha_problem* prob, const void* X, const void* W_Q, const void* W_K,
                       const void* W_V, const float* alpha_Q, const float* alpha_K,
                       const float* alpha_V, const float* R, float* X_out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  return forward_impl(prob, X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, X_out, workspace,
                      workspace_bytes, stream, nullptr);
}

iha_status iha_forward_timed(const iha_problem* prob, const void* X, const void* W_Q,
                             const void* W_K, const void* W_V, const float* alpha_Q,
                             const float* alpha_K, const float* alpha_V, const float* R,
                             float* X_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t* events) {
  if (!events) return IHA_ERR_INVALID_ARG;
  for (int i = 0; i < IHA_TIMED_EVENTS; ++i)
    if (!events[i]) return IHA_ERR_INVALID_ARG;
  return forward_impl(prob, X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, X_out, workspace,
                      workspace_bytes, stream, events);
}

iha_status iha_forward_static(const iha_problem* prob, const void* X, const void* W_Q,
                              const void* W_K, const void* W_V, const float* alpha_Q,
                              const float* alpha_K, const float* alpha_V, const float* R,
                              float* X_out, hipStream_t stream) {
  const iha_status v = validate(prob);
  if (v != IHA_OK) return v;
  if (layout_of(*prob).total > kStaticBytes) return IHA_ERR_WORKSPACE;
  void* ws = nullptr;
  const iha_status st = static_workspace(&ws);
  if (st != IHA_OK) return st;
  return forward_impl(prob, X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, X_out, ws, kStaticBytes,
                      stream, nullptr);
}

iha_status iha_attention(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask, int64_t window,
                         float score_scale, const void* Q, const void* K, const void* Vt, float* O,
                         uint32_t flags, void* flag_buf, hipStream_t stream) {
  if (B < 1 || L < 1 || H < 1 || mask < IHA_MASK_NONE || mask > IHA_MASK_WINDOW)
    return IHA_ERR_INVALID_ARG;
  if (!Q || !K || !Vt || !O || !(score_scale > 0.f) || !std::isfinite(score_scale))
    return IHA_ERR_INVALID_ARG;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(Vt, 16) || !aligned(O, 16)) return IHA_ERR_INVALID_ARG;
  if ((flags & ~IHA_FLAG_CHECK) != 0) return IHA_ERR_INVALID_ARG;
  if ((flags & IHA_FLAG_CHECK) && !flag_buf) return IHA_ERR_WORKSPACE;
  if (d != 64 && d != 128) return IHA_ERR_UNSUPPORTED;
  if (L > kMaxRows || B * L * H * d > kMaxElems / 4) return IHA_ERR_SHAPE;
  if (mask == IHA_MASK_WINDOW && window < 1) return IHA_ERR_EMPTY_ROW;
  unsigned* flag = static_cast<unsigned*>(flag_buf);
  if (flag) IHA_HIP(iha::launch_clear_flag(flag, stream));
  iha::AttnArgs at{};
  at.Q = Q;
  at.K = K;
  at.Vt = Vt;
  at.O = O;
  at.flag = flag;
  at.B = static_cast<int>(B);
  at.L = static_cast<int>(L);
  at.H = static_cast<int>(H);
  at.d = static_cast<int>(d);
  at.mask = mask;
  at.window = mask == IHA_MASK_WINDOW ? static_cast<int>(window < L ? window : L) : 0;
  at.qk_scale = score_scale;
  IHA_HIP(iha::launch_attn_f16(at, stream));
  if (flags & IHA_FLAG_CHECK) return read_flag(flag, stream);
  return IHA_OK;
}

iha_status iha_nexus_inner_workspace(int64_t B, int64_t L, int64_t H, int64_t d, size_t* bytes) {
  if (!bytes) return IHA_ERR_INVALID_ARG;
  if (B < 1 || L < 1 || H < 1) return IHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return IHA_ERR_UNSUPPORTED;
  if (L > kMaxRows || B * H > 65535 || B * L * H * d > kMaxElems / 4) return IHA_ERR_SHAPE;
  *bytes = kAlign + align_up(static_cast<size_t>(B * L * H * d) * 2);
  return IHA_OK;
}

iha_status iha_nexus_inner(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask, int64_t window,
                           float score_scale, const void* Q, float* O, uint32_t flags, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  size_t need = 0;
  const iha_status v = iha_nexus_inner_workspace(B, L, H, d, &need);
  if (v != IHA_OK) return v;
  if (mask < IHA_MASK_NONE || mask > IHA_MASK_WINDOW) return IHA_ERR_INVALID_ARG;
  if (!Q || !O || !(score_scale > 0.f) || !std::isfinite(score_scale)) return IHA_ERR_INVALID_ARG;
  if (!aligned(Q, 16) || !aligned(O, 16)) return IHA_ERR_INVALID_ARG;
  if ((flags & ~IHA_FLAG_CHECK) != 0) return IHA_ERR_INVALID_ARG;
  if (mask == IHA_MASK_WINDOW && window < 1) return IHA_ERR_EMPTY_ROW;
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < need) return IHA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  unsigned* flag = reinterpret_cast<unsigned*>(ws);
  auto* Qt = reinterpret_cast<iha::half_t*>(ws + kAlign);
  IHA_HIP(iha::launch_clear_flag(flag, stream));
  IHA_HIP(iha::launch_transpose_rows(static_cast<const iha::half_t*>(Q), Qt, static_cast<int>(B), static_cast<int>(L),
                                     static_cast<int>(H), static_cast<int>(d), stream));
  iha::AttnArgs at{};
  at.Q = Q;
  at.K = Q;
  at.Vt = Qt;
  at.O = O;
  at.flag = flag;
  at.B = static_cast<int>(B);
  at.L = static_cast<int>(L);
  at.H = static_cast<int>(H);
  at.d = static_cast<int>(d);
  at.mask = mask;
  at.window = mask == IHA_MASK_WINDOW ? static_cast<int>(window < L ? window : L) : 0;
  at.qk_scale = score_scale;
  IHA_HIP(iha::launch_attn_f16(at, stream));
  if (flags & IHA_FLAG_CHECK) {
    IHA_HIP(iha::launch_check_values(O, iha::kValF32, B * L * H * d, flag, iha::kFlagNonFinite,
                                     __builtin_inff(), stream));
    return read_flag(flag, stream);
  }
  return IHA_OK;
}

iha_status iha_attention_backward_workspace(int64_t B, int64_t L, int64_t H, int64_t d, size_t* bytes) {
  if (!bytes) return IHA_ERR_INVALID_ARG;
  const iha_status st = bwd_validate(B, L, H, d, IHA_MASK_NONE, 0);
  if (st != IHA_OK) return st;
  *bytes = bwd_layout(B, L, H, d).total;
  return IHA_OK;
}

iha_status iha_attention_backward(int64_t B, int64_t L, int64_t H, int64_t d, int32_t mask, int64_t window,
                                  float score_scale, const void* Q, const void* K, const void* V,
                                  const void* dO, float* dQ, float* dK, float* dV, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  const iha_status st = bwd_validate(B, L, H, d, mask, window);
  if (st != IHA_OK) return st;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV || !(score_scale > 0.f) || !std::isfinite(score_scale))
    return IHA_ERR_INVALID_ARG;
  for (const void* p : {Q, K, V, dO, static_cast<const void*>(dQ), static_cast<const void*>(dK),
                        static_cast<const void*>(dV)})
    if (!aligned(p, 16)) return IHA_ERR_INVALID_ARG;
  const BwdLayout lay = bwd_layout(B, L, H, d);
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < lay.total) return IHA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  iha::AttnBwdArgs a{};
  using iha::half_t;
  a.Q = static_cast<const half_t*>(Q);
  a.K = static_cast<const half_t*>(K);
  a.V = static_cast<const half_t*>(V);
  a.dO = static_cast<const half_t*>(dO);
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.Qs = reinterpret_cast<half_t*>(ws + lay.qs);
  a.QsT = reinterpret_cast<half_t*>(ws + lay.qst);
  a.KT = reinterpret_cast<half_t*>(ws + lay.kt);
  a.dOT = reinterpret_cast<half_t*>(ws + lay.dot);
  a.VT = reinterpret_cast<half_t*>(ws + lay.vt);
  a.O = reinterpret_cast<half_t*>(ws + lay.o);
  a.lse = reinterpret_cast<float*>(ws + lay.lse);
  a.D = reinterpret_cast<float*>(ws + lay.dd);
  a.B = static_cast<int>(B);
  a.L = static_cast<int>(L);
  a.H = static_cast<int>(H);
  a.d = static_cast<int>(d);
  a.mask = mask;
  a.window = mask == IHA_MASK_WINDOW ? static_cast<int>(window < L ? window : L) : 0;
  a.Lp = static_cast<int>(lay.Lp);
  a.scale = score_scale;
  a.dq_scale = score_scale * 0.69314718055994531f;
  a.dk_scale = 0.69314718055994531f;
  IHA_HIP(iha::launch_attn_bwd(a, stream));
  return IHA_OK;
}

iha_status iha_backward_workspace(const iha_problem* prob, size_t* bytes) {
  if (!bytes) return IHA_ERR_INVALID_ARG;
  const iha_status v = layer_bwd_validate(prob);
  if (v != IHA_OK) return v;
  *bytes = layer_bwd_layout(*prob).total;
  return IHA_OK;
}

iha_status iha_backward(const iha_problem* prob, const void* X, const void* W_Q, const void* W_K,
                        const void* W_V, const float* alpha_Q, const float* alpha_K, const float* alpha_V,
                        const float* R, const float* G, float* dX, float* dW_Q, float* dW_K, float* dW_V,
                        float* dalpha_Q, float* dalpha_K, float* dalpha_V, float* dR, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  const iha_status v = layer_bwd_validate(prob);
  if (v != IHA_OK) return v;
  const void* ins[] = {X, W_Q, W_K, W_V, alpha_Q, alpha_K, alpha_V, R, G};
  const void* outs[] = {dX, dW_Q, dW_K, dW_V, dalpha_Q, dalpha_K, dalpha_V, dR};
  for (const void* q : ins)
    if (!q || !aligned(q, 16)) return IHA_ERR_INVALID_ARG;
  for (const void* q : outs)
    if (!q || !aligned(q, 16)) return IHA_ERR_INVALID_ARG;
  const iha_problem& p = *prob;
  const LayerBwdLayout lay = layer_bwd_layout(p);
  if (!workspace || !aligned(workspace, kAlign) || workspace_bytes < lay.total) return IHA_ERR_WORKSPACE;
  using iha::half_t;
  char* ws = static_cast<char*>(workspace);
  unsigned* flag = reinterpret_cast<unsigned*>(ws + lay.flag);
  const int B = static_cast<int>(p.B), N = static_cast<int>(p.N), D = static_cast<int>(p.D);
  const int H = static_cast<int>(p.H), P = static_cast<int>(p.P), d = D / H, M = B * N, L = P * N;
  const int64_t act = static_cast<int64_t>(M) * P * D;
  float* Y = reinterpret_cast<float*>(ws + lay.y);
  auto* Qb = reinterpret_cast<half_t*>(ws + lay.qb);
  auto* Kb = reinterpret_cast<half_t*>(ws + lay.kb);
  auto* Vb = reinterpret_cast<half_t*>(ws + lay.vb);
  auto* dPb = reinterpret_cast<half_t*>(ws + lay.dpb);
  float* dBar[3] = {reinterpret_cast<float*>(ws + lay.dq), reinterpret_cast<float*>(ws + lay.dk),
                    reinterpret_cast<float*>(ws + lay.dv)};
  float* part = reinterpret_cast<float*>(ws + lay.part);
  auto* dYcat = reinterpret_cast<uint16_t*>(ws + lay.dycat);
  auto* dYt = reinterpret_cast<uint16_t*>(ws + lay.dyt);
  auto* Xt = reinterpret_cast<uint16_t*>(ws + lay.xt);
  auto* Wcat = reinterpret_cast<uint16_t*>(ws + lay.wcat);
  const float* alphas[3] = {alpha_Q, alpha_K, alpha_V};
  float* dalphas[3] = {dalpha_Q, dalpha_K, dalpha_V};
  float* dWs[3] = {dW_Q, dW_K, dW_V};
  const uint16_t* Ws[3] = {static_cast<const uint16_t*>(W_Q), static_cast<const uint16_t*>(W_K),
                           static_cast<const uint16_t*>(W_V)};
  if (log_enabled())
    std::fprintf(stderr, "[iha] backward B=%d N=%d D=%d H=%d d=%d P=%d mask=%d window=%lld\n", B, N, D, H, d, P,
                 p.mask, static_cast<long long>(p.window));

  // Forward steps 1-2 again: Y = X W (kept in fp32) and the mixed, stacked Q~, K~, V~ (fp16).
  iha::ProjArgs pa{};
  pa.X = static_cast<const uint16_t*>(X);
  for (int w = 0; w < 3; ++w) {
    pa.W[w] = Ws[w];
    pa.alpha[w] = alphas[w];
  }
  pa.Wt = reinterpret_cast<uint16_t*>(ws + lay.wt);
  pa.Yqk = Y;
  pa.Q = Qb;
  pa.K = Kb;
  pa.Vrow = Vb;
  pa.B = B;
  pa.N = N;
  pa.D = D;
  pa.H = H;
  pa.d = d;
  pa.P = P;
  pa.qscale = 1.f;
  pa.flag = flag;  // cleared by the weight transpose
  IHA_HIP(iha::launch_proj_rowmajor(pa, stream));

  // Collapse (steps 4-5) in reverse: dR = sum over tokens of G (x) P-bar, and the stacked
  // outputs' gradient dP-bar[t*P + j][h'] = sum_h R[h][h'*P + j] G[t][h].
  IHA_HIP(iha::launch_expand(G, R, dPb, B, N, H, P, d, stream));

  // Attention (step 3) in reverse; it recomputes the fp16 forward output P-bar on the way.
  const BwdLayout& al = lay.a;
  char* aws = ws + lay.att;
  iha::AttnBwdArgs a{};
  a.Q = Qb;
  a.K = Kb;
  a.V = Vb;
  a.dO = dPb;
  a.dQ = dBar[0];
  a.dK = dBar[1];
  a.dV = dBar[2];
  a.Qs = reinterpret_cast<half_t*>(aws + al.qs);
  a.QsT = reinterpret_cast<half_t*>(aws + al.qst);
  a.KT = reinterpret_cast<half_t*>(aws + al.kt);
  a.dOT = reinterpret_cast<half_t*>(aws + al.dot);
  a.VT = reinterpret_cast<half_t*>(aws + al.vt);
  a.O = reinterpret_cast<half_t*>(aws + al.o);
  a.lse = reinterpret_cast<float*>(aws + al.lse);
  a.D = reinterpret_cast<float*>(aws + al.dd);
  a.B = B;
  a.L = L;
  a.H = H;
  a.d = d;
  a.mask = p.mask;
  a.window = p.mask == IHA_MASK_WINDOW ? static_cast<int>(p.window < L ? p.window : L) : 0;
  a.Lp = static_cast<int>(al.Lp);
  a.scale = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(d)));
  a.dq_scale = a.scale * 0.69314718055994531f;
  a.dk_scale = 0.69314718055994531f;
  IHA_HIP(iha::launch_attn_bwd(a, stream));
  IHA_HIP(iha::launch_head_reduce(G, D, a.O, true, dR, part, M, H, P, d, stream));

  // Mixing (step 2) in reverse: dalpha[m][h][j] = sum over tokens of Y_m (x) dBar_{h,j}, and
  // dY_m = sum_{h,j} alpha[m][h][j] dBar_{h,j} - a collapse with alpha in place of R.  The dY
  // go where Y was (after the last reduction that reads Y), then to bf16 high and low parts
  // (rounding dY to bf16 alone costs about 2^-9 of the largest gradients): token-major for dX,
  // channel-major for dW.
  const int64_t D3 = 3 * static_cast<int64_t>(D), Mp = lay.Mp;
  for (int w = 0; w < 3; ++w)
    IHA_HIP(iha::launch_head_reduce(Y + static_cast<int64_t>(w) * D, D3, dBar[w], false, dalphas[w], part, M, H, P,
                                    d, stream));
  for (int w = 0; w < 3; ++w) {
    float* dY = Y + static_cast<int64_t>(w) * M * D;
    IHA_HIP(iha::launch_collapse(dBar[w], alphas[w], dY, M, H, P, d, stream));
    IHA_HIP(iha::launch_to_bf16(dY, D, M, D, dYcat + w * D, dYcat + D3 + w * D, 2 * D3, stream));
    uint16_t* t = dYt + static_cast<int64_t>(w) * D * 2 * Mp;
    IHA_HIP(iha::launch_to_bf16_t(dY, false, D, M, D, t, t + Mp, 2 * Mp, Mp, stream));
    for (int half = 0; half < 2; ++half)
      IHA_HIP(iha::launch_copy_bf16(Ws[w], D, D, D, Wcat + half * D3 + w * D, 2 * D3, stream));
  }

  // Projection (step 1) in reverse: dW_m = X^T (dY_m high + low) as one product over 2 Mp
  // tokens, dX = sum_m (dY_m high + low) W_m^T as one product over 6D.
  for (int half = 0; half < 2; ++half)
    IHA_HIP(iha::launch_to_bf16_t(X, true, D, M, D, Xt + half * Mp, nullptr, 2 * Mp, Mp, stream));
  {
    iha::NtArgs g{};  // the three weight gradients in one launch, the token dimension split
    g.A = Xt;
    g.sa = 0;
    g.B = dYt;
    g.sb = static_cast<int64_t>(D) * 2 * Mp;
    for (int w = 0; w < 3; ++w) g.Cz[w] = dWs[w];
    g.I = D;
    g.J = D;
    g.K = static_cast<int>(2 * Mp);
    g.ldc = D;
    IHA_HIP(iha::launch_gemm_nt_splitk(g, 3, lay.splits, reinterpret_cast<float*>(ws + lay.wsplit), stream));
  }
  iha::NtArgs g{};
  g.A = dYcat;
  g.B = Wcat;
  g.C = dX;
  g.I = M;
  g.J = D;
  g.K = static_cast<int>(2 * D3);
  g.ldc = D;
  IHA_HIP(iha::launch_gemm_nt_bf16(g, stream));

  if (p.flags & IHA_FLAG_CHECK) {
    // Non-finite inputs; stacked fp16 tensors beyond the fp16 range; non-finite gradients.
    using iha::kFlagInputNonFinite;
    const float inf = __builtin_inff();
    const int64_t nx = static_cast<int64_t>(M) * D, nw = static_cast<int64_t>(D) * D;
    const int64_t na = static_cast<int64_t>(H) * H * P;
    IHA_HIP(iha::launch_check_values(X, iha::kValBF16, nx, flag, kFlagInputNonFinite, inf, stream));
    IHA_HIP(iha::launch_check_values(G, iha::kValF32, nx, flag, kFlagInputNonFinite, inf, stream));
    for (int w = 0; w < 3; ++w) {
      IHA_HIP(iha::launch_check_values(Ws[w], iha::kValBF16, nw, flag, kFlagInputNonFinite, inf, stream));
      IHA_HIP(iha::launch_check_values(alphas[w], iha::kValF32, na, flag, kFlagInputNonFinite, inf, stream));
    }
    IHA_HIP(iha::launch_check_values(R, iha::kValF32, na, flag, kFlagInputNonFinite, inf, stream));
    for (const half_t* t : {Qb, Kb, Vb, dPb})
      IHA_HIP(iha::launch_check_values(t, iha::kValF16, act, flag, iha::kFlagRange, inf, stream));
    IHA_HIP(iha::launch_check_values(dX, iha::kValF32, nx, flag, iha::kFlagNonFinite, inf, stream));
    for (int w = 0; w < 3; ++w) {
      IHA_HIP(iha::launch_check_values(dWs[w], iha::kValF32, nw, flag, iha::kFlagNonFinite, inf, stream));
      IHA_HIP(iha::launch_check_values(dalphas[w], iha::kValF32, na, flag, iha::kFlagNonFinite, inf, stream));
    }
    IHA_HIP(iha::launch_check_values(dR, iha::kValF32, na, flag, iha::kFlagNonFinite, inf, stream));
    return read_flag(flag, stream);
  }
  return IHA_OK;
}

const char* iha_status_str(iha_status s) {
  switch (s) {
    case IHA_OK: return "IHA_OK";
    case IHA_ERR_INVALID_ARG: return "IHA_ERR_INVALID_ARG: invalid argument";
    case IHA_ERR_SHAPE: return "IHA_ERR_SHAPE: D not a multiple of H, or size out of range";
    case IHA_ERR_EMPTY_ROW: return "IHA_ERR_EMPTY_ROW: a query has no visible key";
    case IHA_ERR_NONFINITE: return "IHA_ERR_NONFINITE: non-finite value in the output";
    case IHA_ERR_WORKSPACE: return "IHA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case IHA_ERR_UNSUPPORTED: return "IHA_ERR_UNSUPPORTED: head width or head count not supported";
    case IHA_ERR_DEVICE: return "IHA_ERR_DEVICE: a HIP call failed";
    case IHA_ERR_RANGE: return "IHA_ERR_RANGE: an intermediate value exceeds the fp16 range";
  }
  return "IHA_ERR_UNKNOWN";
}

}  // extern "C"
