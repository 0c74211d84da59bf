/*
 * CPU oracle for the Interleaved Head Attention (IHA) forward pass, in IEEE double.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg to check the HIP library.  It shares no code
 * with that library and is never part of the product path.
 *
 * It follows the IHA page ("Interleaved Head Attention", section 4,
 * Algorithm 1) step by step, in the page's order:
 *   1. per-head projections X W^(m)                     (section 3.1 notation)
 *   2. pseudo-head mixing  Q~_{h,j} = sum_m alpha^Q_{m,h,j} X W_Q^(m)  (same for K, V)
 *   3. pseudo-major stacking Q-bar_h = [Q~_{h,1}; ...; Q~_{h,P}]  (block rows)
 *   4. per-head attention  softmax(Q-bar K-bar^T / sqrt(d)) V-bar over the PN rows
 *   5. unstack, collapse   O_h[t] = sum_{h'} sum_j R_{h,(h'-1)P+j} P_{h',j}[t]
 *   6. concatenate heads   X~ = [O_1, ..., O_H]
 * Step 4 is done one query row at a time with strict visibility exactly as the
 * textbook chapter on attention states it (section 5.3, Algorithm 5.1):
 * check finiteness, restrict to the allowed set, subtract the row maximum,
 * exponentiate, normalise, and sum the weighted value rows.
 *
 * Readings of the pages taken here (0-based indices throughout):
 *   - The stacked order of Algorithm 1 is block order (row r = j*N + t).  The
 *     figure of the IHA page calls the pseudo-tokens interleaved; masks are
 *     therefore defined on the interleaved position iota(t, j) = t*P + j, and
 *     the block-ordered rows carry that position into the mask.  Without a
 *     mask the order does not matter (permutation equivariance, textbook
 *     section 5.9).
 *   - causal: a key is visible iff iota_k <= iota_q (textbook section 5.3).
 *   - window: iota_q - W_s < iota_k <= iota_q, W_s counted in stacked indices
 *     (N/(2P) in the IHA page's figure 1 and appendix C).
 *   - scale 1/sqrt(d), d = D/H the per-head width.
 *   - alpha[m][h][j]: m is the summed source head, h the target head.
 *   - R column (h'-1)P + j becomes h'*P + j.
 *   - P_{h',j} is the j-th N-row block of P-bar_{h'}.
 *   - An empty allowed set is an error (textbook section 5.3), never a NaN.
 */
#include "iha_oracle.h"

#include <omp.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <limits>
#include <vector>

namespace {

// Allowed set J_i of the textbook (eq. 5.11), on positions.
bool visible(int mask, int64_t window, int64_t qp, int64_t kp) {
  switch (mask) {
    case IHO_MASK_NONE:
      return true;
    case IHO_MASK_CAUSAL:
      return kp <= qp;
    case IHO_MASK_WINDOW:
      return kp <= qp && kp > qp - window;
    default:
      return false;
  }
}

bool all_finite(const double* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

// Algorithm 5.1 (textbook section 5.3) for one valid query row.
int attend_row(const double* q, int64_t S, int64_t dk, int64_t dv, const double* K,
               const double* V, const int64_t* kpos, int64_t qp, int mask, int64_t window,
               double scale, double* o, double* a_row, double* rowsum) {
  std::vector<int64_t> J;
  for (int64_t s = 0; s < S; ++s)
    if (visible(mask, window, qp, kpos ? kpos[s] : s)) J.push_back(s);
  if (J.empty()) return IHO_ERR_EMPTY_ROW;

  // u_s = q k_s^T / sqrt(dk) over the allowed set; c = max u.
  std::vector<double> u(J.size());
  double c = -std::numeric_limits<double>::infinity();
  for (size_t idx = 0; idx < J.size(); ++idx) {
    const double* k = K + J[idx] * dk;
    double dot = 0.0;
    for (int64_t r = 0; r < dk; ++r) dot += q[r] * k[r];
    u[idx] = dot * scale;
    if (!std::isfinite(u[idx])) return IHO_ERR_NONFINITE;
    if (u[idx] > c) c = u[idx];
  }
  // e_s = exp(u_s - c), z = sum e_s (z >= 1 because one term is exp(0)).
  double z = 0.0;
  for (size_t idx = 0; idx < J.size(); ++idx) {
    u[idx] = std::exp(u[idx] - c);
    z += u[idx];
  }
  // a_s = e_s / z;  o <- o + a_s v_s.  Positions outside J take no part.
  for (int64_t r = 0; r < dv; ++r) o[r] = 0.0;
  double sum = 0.0;
  for (size_t idx = 0; idx < J.size(); ++idx) {
    const double a = u[idx] / z;
    sum += a;
    const double* v = V + J[idx] * dv;
    for (int64_t r = 0; r < dv; ++r) o[r] += a * v[r];
    if (a_row) a_row[J[idx]] = a;
  }
  if (rowsum) *rowsum = sum;
  return IHO_OK;
}

}  // namespace

extern "C" int iho_threads(int nthreads) { return nthreads > 0 ? nthreads : omp_get_max_threads(); }

extern "C" int iho_attention(int64_t T, int64_t S, int64_t dk, int64_t dv, const double* Q,
                             const double* K, const double* V, const int64_t* qpos,
                             const int64_t* kpos, int mask, int64_t window, double scale,
                             double* O, double* A, double* rowsum) {
  if (T < 0 || S < 0 || dk < 1 || dv < 1 || !Q || !K || !V || !O) return IHO_ERR_ARG;
  if (mask < IHO_MASK_NONE || mask > IHO_MASK_WINDOW) return IHO_ERR_ARG;
  if (!all_finite(Q, T * dk) || !all_finite(K, S * dk) || !all_finite(V, S * dv))
    return IHO_ERR_NONFINITE;
  if (A)
    for (int64_t i = 0; i < T * S; ++i) A[i] = 0.0;
  std::atomic<int> err{IHO_OK};
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < T; ++i) {
    int e = attend_row(Q + i * dk, S, dk, dv, K, V, kpos, qpos ? qpos[i] : i, mask, window, scale,
                       O + i * dv, A ? A + i * S : nullptr, rowsum ? rowsum + i : nullptr);
    if (e != IHO_OK) err = e;
  }
  return err.load();
}

extern "C" int iho_forward(int64_t B, int64_t N, int64_t D, int64_t H, int64_t P, int mask,
                           int64_t window, const double* X, const double* WQ, const double* WK,
                           const double* WV, const double* aQ, const double* aK,
                           const double* aV, const double* R, const int64_t* tokens,
                           int64_t ntokens, double* out, double* max_rowsum_dev, int nthreads) {
  if (B < 1 || N < 1 || D < 1 || H < 1 || P < 1 || D % H != 0) return IHO_ERR_ARG;
  if (mask < IHO_MASK_NONE || mask > IHO_MASK_WINDOW) return IHO_ERR_ARG;
  if (!X || !WQ || !WK || !WV || !aQ || !aK || !aV || !R || !out) return IHO_ERR_ARG;
  if (mask == IHO_MASK_WINDOW && window < 1) return IHO_ERR_EMPTY_ROW;
  if (!all_finite(X, B * N * D) || !all_finite(WQ, D * D) || !all_finite(WK, D * D) ||
      !all_finite(WV, D * D) || !all_finite(aQ, H * H * P) || !all_finite(aK, H * H * P) ||
      !all_finite(aV, H * H * P) || !all_finite(R, H * H * P))
    return IHO_ERR_NONFINITE;
  if (nthreads > 0) omp_set_num_threads(nthreads);

  const int64_t d = D / H;
  const int64_t PN = P * N;
  const double scale = 1.0 / std::sqrt(static_cast<double>(d));

  // Requested tokens, grouped by sequence: (slot in `out`, t).
  std::vector<std::vector<std::pair<int64_t, int64_t>>> req(B);
  if (tokens) {
    for (int64_t s = 0; s < ntokens; ++s) {
      if (tokens[s] < 0 || tokens[s] >= B * N) return IHO_ERR_ARG;
      req[tokens[s] / N].push_back({s, tokens[s] % N});
    }
  } else {
    for (int64_t b = 0; b < B; ++b)
      for (int64_t t = 0; t < N; ++t) req[b].push_back({b * N + t, t});
  }

  // Position of block-stacked row r = j*N + t is iota = t*P + j.
  std::vector<int64_t> iota(PN);
  for (int64_t j = 0; j < P; ++j)
    for (int64_t t = 0; t < N; ++t) iota[j * N + t] = t * P + j;

  std::atomic<int> err{IHO_OK};
  double maxdev = 0.0;

  for (int64_t b = 0; b < B; ++b) {
    const auto& rq = req[b];
    if (rq.empty()) continue;
    const double* Xb = X + b * N * D;
    const int64_t nq = static_cast<int64_t>(rq.size());

    // Which tokens' queries are needed, and which tokens' keys/values can be read by them.
    std::vector<char> needQ(N, 0), needKV(N, 0);
    for (const auto& st : rq) needQ[st.second] = 1;
    if (!tokens || mask == IHO_MASK_NONE) {
      std::fill(needKV.begin(), needKV.end(), 1);
    } else {
#pragma omp parallel for schedule(static)
      for (int64_t tk = 0; tk < N; ++tk) {
        for (const auto& st : rq) {
          bool hit = false;
          for (int64_t j = 0; j < P && !hit; ++j)
            for (int64_t jk = 0; jk < P && !hit; ++jk)
              hit = visible(mask, window, st.second * P + j, tk * P + jk);
          if (hit) {
            needKV[tk] = 1;
            break;
          }
        }
      }
    }

    // Step 1: per-head projections Y^(m) = X W^(m); all heads at once, Y = X W, [N][H*d].
    std::vector<double> YQ(N * D, 0.0), YK(N * D, 0.0), YV(N * D, 0.0);
    auto project = [&](const double* W, std::vector<double>& Y, const std::vector<char>& need) {
#pragma omp parallel for schedule(dynamic, 8)
      for (int64_t t = 0; t < N; ++t) {
        if (!need[t]) continue;
        double* y = Y.data() + t * D;
        const double* x = Xb + t * D;
        for (int64_t k = 0; k < D; ++k) {
          const double xk = x[k];
          const double* w = W + k * D;
          for (int64_t col = 0; col < D; ++col) y[col] += xk * w[col];
        }
      }
    };
    project(WQ, YQ, needQ);
    project(WK, YK, needKV);
    project(WV, YV, needKV);

    // Step 2: mixing, Qt[h][j][t][c] = sum_m alpha[m][h][j] * Y[t][m*d + c].
    // Step 3: stacking.  With Qt stored as [h][j][t][c], the [PN][d] slice at head h
    // is exactly Q-bar_h with block row r = j*N + t.
    std::vector<double> Qt(H * PN * d, 0.0), Kt(H * PN * d, 0.0), Vt(H * PN * d, 0.0);
    auto mix = [&](const double* alpha, const std::vector<double>& Y, std::vector<double>& M,
                   const std::vector<char>& need) {
#pragma omp parallel for schedule(dynamic, 8)
      for (int64_t t = 0; t < N; ++t) {
        if (!need[t]) continue;
        for (int64_t h = 0; h < H; ++h)
          for (int64_t j = 0; j < P; ++j) {
            double* m_out = M.data() + ((h * P + j) * N + t) * d;
            for (int64_t m = 0; m < H; ++m) {
              const double a = alpha[(m * H + h) * P + j];
              const double* y = Y.data() + t * D + m * d;
              for (int64_t c = 0; c < d; ++c) m_out[c] += a * y[c];
            }
          }
      }
    };
    mix(aQ, YQ, Qt, needQ);
    mix(aK, YK, Kt, needKV);
    mix(aV, YV, Vt, needKV);

    // Step 4: attention per head over the PN stacked rows, for the requested query rows.
    // Pb[h][j][slot][c] = P-bar_h[j*N + t] for the slot's token t.
    std::vector<double> Pb(H * P * nq * d, 0.0);
#pragma omp parallel for schedule(dynamic, 1) reduction(max : maxdev)
    for (int64_t w = 0; w < H * P * nq; ++w) {
      const int64_t h = w / (P * nq);
      const int64_t j = (w / nq) % P;
      const int64_t s = w % nq;
      const int64_t t = rq[s].second;
      const int64_t r = j * N + t;
      const double* Qbar = Qt.data() + h * PN * d;
      const double* Kbar = Kt.data() + h * PN * d;
      const double* Vbar = Vt.data() + h * PN * d;
      double rs = 0.0;
      int e = attend_row(Qbar + r * d, PN, d, d, Kbar, Vbar, iota.data(), iota[r], mask, window,
                         scale, Pb.data() + ((h * P + j) * nq + s) * d, nullptr, &rs);
      if (e != IHO_OK) err = e;
      maxdev = std::max(maxdev, std::fabs(rs - 1.0));
    }
    if (err.load() != IHO_OK) return err.load();

    // Steps 5-6: unstack, collapse with R, concatenate the heads.
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < nq; ++s) {
      double* o = out + rq[s].first * D;
      for (int64_t h = 0; h < H; ++h) {
        double* oh = o + h * d;
        for (int64_t c = 0; c < d; ++c) oh[c] = 0.0;
        for (int64_t hp = 0; hp < H; ++hp)
          for (int64_t j = 0; j < P; ++j) {
            const double rv = R[h * (H * P) + hp * P + j];
            const double* p = Pb.data() + ((hp * P + j) * nq + s) * d;
            for (int64_t c = 0; c < d; ++c) oh[c] += rv * p[c];
          }
      }
    }
  }
  if (max_rowsum_dev) *max_rowsum_dev = maxdev;
  return err.load();
}
