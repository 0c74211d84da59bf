// Drives the CPU oracle (oracle/iha_oracle.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer: small problems in every mask mode, token subsets, P = 1..3,
// window 1, and the error paths (empty allowed set, non-finite input, bad arguments).
// Exits non-zero on a wrong status or a broken invariant; the sanitizers abort on any
// out-of-bounds access, use after free or undefined operation.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "iha_oracle.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++failures;
  }
}

// Deterministic values in [-1, 1) from a 64-bit linear congruential sequence.
struct Lcg {
  uint64_t s;
  double next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return static_cast<double>(s >> 11) / 4503599627370496.0 - 1.0;
  }
};

struct Problem {
  int64_t B, N, D, H, P;
  std::vector<double> X, WQ, WK, WV, aQ, aK, aV, R;
  Problem(int64_t B_, int64_t N_, int64_t D_, int64_t H_, int64_t P_, uint64_t seed)
      : B(B_), N(N_), D(D_), H(H_), P(P_) {
    Lcg g{seed};
    auto fill = [&](std::vector<double>& v, size_t n, double s) {
      v.resize(n);
      for (auto& e : v) e = s * g.next();
    };
    fill(X, B * N * D, 1.0);
    fill(WQ, D * D, 1.0 / std::sqrt(double(D)));
    fill(WK, D * D, 1.0 / std::sqrt(double(D)));
    fill(WV, D * D, 1.0 / std::sqrt(double(D)));
    fill(aQ, H * H * P, 0.5);
    fill(aK, H * H * P, 0.5);
    fill(aV, H * H * P, 0.5);
    fill(R, H * H * P, 0.5);
  }
  int run(int mask, int64_t window, const int64_t* tokens, int64_t nt, std::vector<double>& out,
          double* dev) {
    out.assign((tokens ? nt : B * N) * D, 0.0);
    return iho_forward(B, N, D, H, P, mask, window, X.data(), WQ.data(), WK.data(), WV.data(),
                       aQ.data(), aK.data(), aV.data(), R.data(), tokens, nt, out.data(), dev, 2);
  }
};

}  // namespace

int main() {
  for (int P = 1; P <= 3; ++P)
    for (int mask = IHO_MASK_NONE; mask <= IHO_MASK_WINDOW; ++mask) {
      Problem pr(2, 13, 12, 3, P, 100 + P);
      std::vector<double> full, sub;
      double dev = 1.0;
      const int64_t window = mask == IHO_MASK_WINDOW ? 5 : 0;
      expect(pr.run(mask, window, nullptr, 0, full, &dev) == IHO_OK, "forward status");
      expect(dev < 1e-12, "row sums equal 1");
      for (double v : full) expect(std::isfinite(v), "finite output");
      // A token subset reproduces the same rows exactly.
      const int64_t tok[] = {25, 0, 13, 7};
      expect(pr.run(mask, window, tok, 4, sub, nullptr) == IHO_OK, "subset status");
      for (int s = 0; s < 4; ++s)
        for (int64_t c = 0; c < pr.D; ++c)
          expect(sub[s * pr.D + c] == full[tok[s] * pr.D + c], "subset rows equal full rows");
    }
  {
    Problem pr(1, 9, 8, 2, 2, 7);
    std::vector<double> out;
    expect(pr.run(IHO_MASK_WINDOW, 1, nullptr, 0, out, nullptr) == IHO_OK, "window 1");
    expect(pr.run(IHO_MASK_WINDOW, 0, nullptr, 0, out, nullptr) == IHO_ERR_EMPTY_ROW, "window 0 is empty");
    const int64_t bad_tok[] = {9};
    expect(pr.run(IHO_MASK_NONE, 0, bad_tok, 1, out, nullptr) == IHO_ERR_ARG, "token out of range");
    pr.X[5] = NAN;
    expect(pr.run(IHO_MASK_CAUSAL, 0, nullptr, 0, out, nullptr) == IHO_ERR_NONFINITE, "NaN input");
  }
  {
    // Attention core with explicit positions, weights and row sums.
    const int64_t T = 5, S = 7, dk = 3, dv = 2;
    Lcg g{3};
    std::vector<double> Q(T * dk), K(S * dk), V(S * dv), O(T * dv), A(T * S), rs(T);
    for (auto* v : {&Q, &K, &V})
      for (auto& e : *v) e = g.next();
    const int64_t qpos[] = {0, 2, 4, 6, 8}, kpos[] = {0, 1, 2, 3, 4, 5, 6};
    expect(iho_attention(T, S, dk, dv, Q.data(), K.data(), V.data(), qpos, kpos, IHO_MASK_CAUSAL, 0,
                         1.0 / std::sqrt(3.0), O.data(), A.data(), rs.data()) == IHO_OK,
           "attention status");
    for (int64_t i = 0; i < T; ++i) expect(std::fabs(rs[i] - 1.0) < 1e-14, "attention row sum");
    expect(iho_attention(T, S, dk, dv, Q.data(), K.data(), V.data(), qpos, kpos, IHO_MASK_WINDOW, 0, 1.0,
                         O.data(), nullptr, nullptr) == IHO_ERR_EMPTY_ROW,
           "attention empty row");
    expect(iho_attention(T, S, 0, dv, Q.data(), K.data(), V.data(), nullptr, nullptr, IHO_MASK_NONE, 0, 1.0,
                         O.data(), nullptr, nullptr) == IHO_ERR_ARG,
           "attention bad dk");
  }
  std::printf("oracle driver: %s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
