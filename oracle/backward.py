"""Gradients of the IHA forward in double precision.  TEST INFRASTRUCTURE ONLY.

Reverse-mode differentiation of Algorithm 1 of the "Interleaved Head Attention" page
(section 4), written step by step in plain numpy (float64) for small problems.  The forward
is recomputed here in matrix form - block stacking as Algorithm 1 prints it, masks through
the interleaved position iota(t, j) = t*P + j - and each step's adjoint follows from that
step's definition:

  projection  Y^(m) = X W^(m)                         (IHA page, section 3.1)
  mixing      Q~_{h,j} = sum_m alpha[m, h, j] Y^(m)   (Algorithm 1, the mixing step)
  stacking    Q-bar_h row j*N + t = Q~_{h,j}[t]       (Algorithm 1, the stacking step)
  attention   S = Q-bar K-bar^T / sqrt(d) over each query's allowed keys, A = softmax(S),
              O = A V-bar (textbook "Attention mechanism", eq. 5.3 and 5.11); the softmax
              Jacobian gives dS = A * (dA - rowsum(dA * A))
  collapse    X~[t, h] = sum_{h', j} R[h, h'*P + j] P-bar_{h'}[j*N + t]  (Algorithm 1)

The loss is L = sum(G * X~) for a given upstream gradient G [B, N, D].  Pins: central
finite differences of L (tests/test_oracle_backward.py); the forward part agrees with the
C++ oracle's forward.  attention_grads() is the same attention step on rows that are
already stacked (the form the HIP attention backward takes), pinned the same way.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_WINDOW = 0, 1, 2


def _allowed(L: int, N: int, P: int, mask: int, window: int) -> np.ndarray:
    """[L, L] boolean: query row r may see key row r' (rows in block order r = j*N + t),
    decided on the interleaved positions iota = t*P + j."""
    r = np.arange(L)
    iota = (r % N) * P + r // N
    qi, ki = iota[:, None], iota[None, :]
    if mask == MASK_NONE:
        return np.ones((L, L), dtype=bool)
    if mask == MASK_CAUSAL:
        return ki <= qi
    return (ki <= qi) & (ki > qi - window)


def _allowed_stacked(L: int, mask: int, window: int) -> np.ndarray:
    """[L, L] boolean on stacked positions directly (row i = position i)."""
    i = np.arange(L)
    qi, ki = i[:, None], i[None, :]
    if mask == MASK_NONE:
        return np.ones((L, L), dtype=bool)
    if mask == MASK_CAUSAL:
        return ki <= qi
    return (ki <= qi) & (ki > qi - window)


def attention_grads(Q, K, V, dO, mask: int, window: int) -> Dict[str, np.ndarray]:
    """Masked softmax attention over already stacked rows and its gradients, in float64.

    Q, K, V, dO: [B, L, H, d] with row i = stacked position i (the interleaved order of the
    IHA page's figure 1); the mask is applied to i directly.  Scores S = Q K^T / sqrt(d),
    A = softmax over each query's allowed keys, O = A V (textbook "Attention mechanism",
    eq. 5.3 and 5.11).  For the loss L = sum(dO * O):
      dV = A^T dO,  dA = dO V^T,  dS = A * (dA - rowsum(dA * A)),
      dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
    Returns {"O", "dQ", "dK", "dV", "lse"} (lse = natural log-sum-exp of each row's scores,
    [B, H, L]).  A query with an empty allowed set raises ValueError."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    Q, K, V, dO = f(Q), f(K), f(V), f(dO)
    B, L, H, d = Q.shape
    allowed = _allowed_stacked(L, mask, window)
    if not allowed.any(axis=1).all():
        raise ValueError("a query has an empty allowed set")
    out = {k: np.zeros_like(Q) for k in ("O", "dQ", "dK", "dV")}
    out["lse"] = np.zeros((B, H, L))
    for b in range(B):
        for h in range(H):
            q, k, v, go = Q[b, :, h], K[b, :, h], V[b, :, h], dO[b, :, h]
            S = np.where(allowed, q @ k.T / np.sqrt(d), -np.inf)
            mx = S.max(axis=1, keepdims=True)
            E = np.where(allowed, np.exp(S - mx), 0.0)
            z = E.sum(axis=1, keepdims=True)
            A = E / z
            out["lse"][b, h] = (mx + np.log(z))[:, 0]
            out["O"][b, :, h] = A @ v
            out["dV"][b, :, h] = A.T @ go
            dA = go @ v.T
            dS = A * (dA - (dA * A).sum(axis=1, keepdims=True))
            out["dQ"][b, :, h] = dS @ k / np.sqrt(d)
            out["dK"][b, :, h] = dS.T @ q / np.sqrt(d)
    return out


def forward_and_grads(X, WQ, WK, WV, aQ, aK, aV, R, H: int, P: int, mask: int, window: int,
                      G) -> Dict[str, np.ndarray]:
    """Returns {"out": X~, "X": dL/dX, "WQ": ..., "WK", "WV", "aQ", "aK", "aV", "R"} for
    L = sum(G * X~).  Shapes as in the forward: X [B, N, D], W_* [D, D], alpha_* [H, H, P],
    R [H, H*P], G [B, N, D]."""
    f = lambda a: np.asarray(a, dtype=np.float64)
    X, G = f(X), f(G)
    Ws = [f(WQ), f(WK), f(WV)]
    als = [f(aQ), f(aK), f(aV)]
    R = f(R)
    B, N, D = X.shape
    d = D // H
    L = P * N

    # forward
    Y = [(X @ W).reshape(B, N, H, d) for W in Ws]                    # [b, t, m, c]
    T = [np.einsum("mhj,btmc->bthjc", a, y) for a, y in zip(als, Y)]  # [b, t, h, j, c]
    Bar = [t.transpose(0, 2, 3, 1, 4).reshape(B, H, L, d) for t in T]  # [b, h, j*N + t, c]
    allowed = _allowed(L, N, P, mask, window)
    if not allowed.any(axis=1).all():
        raise ValueError("a query has an empty allowed set")
    A = np.zeros((B, H, L, L))
    Pbar = np.zeros((B, H, L, d))
    for b in range(B):
        for h in range(H):
            S = Bar[0][b, h] @ Bar[1][b, h].T / np.sqrt(d)
            S = np.where(allowed, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            E = np.where(allowed, np.exp(S), 0.0)
            A[b, h] = E / E.sum(axis=1, keepdims=True)
            Pbar[b, h] = A[b, h] @ Bar[2][b, h]
    Rr = R.reshape(H, H, P)                                           # [h, h', j]
    Pu = Pbar.reshape(B, H, P, N, d)                                  # [b, h', j, t, c]
    out = np.einsum("hgj,bgjtc->bthc", Rr, Pu).reshape(B, N, D)

    # backward
    Gr = G.reshape(B, N, H, d)                                        # [b, t, h, c]
    dR = np.einsum("bthc,bgjtc->hgj", Gr, Pu).reshape(H, H * P)
    dPbar = np.einsum("hgj,bthc->bgjtc", Rr, Gr).reshape(B, H, L, d)
    dBar = [np.zeros_like(Bar[0]) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            a = A[b, h]
            dO = dPbar[b, h]
            dBar[2][b, h] = a.T @ dO
            dA = dO @ Bar[2][b, h].T
            dS = a * (dA - (dA * a).sum(axis=1, keepdims=True))
            dBar[0][b, h] = dS @ Bar[1][b, h] / np.sqrt(d)
            dBar[1][b, h] = dS.T @ Bar[0][b, h] / np.sqrt(d)
    grads = {"out": out, "R": dR}
    dX = np.zeros_like(X)
    for w, name in enumerate(["Q", "K", "V"]):
        dT = dBar[w].reshape(B, H, P, N, d).transpose(0, 3, 1, 2, 4)  # [b, t, h, j, c]
        dY = np.einsum("mhj,bthjc->btmc", als[w], dT)                  # [b, t, m, c]
        grads["a" + name] = np.einsum("btmc,bthjc->mhj", Y[w], dT)
        dYf = dY.reshape(B, N, D)
        grads["W" + name] = np.einsum("btk,btn->kn", X, dYf)
        dX += dYf @ Ws[w].T
    grads["X"] = dX
    return grads
