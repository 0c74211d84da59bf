"""Seeded synthetic inputs for the Interleaved Head Attention (IHA) forward pass.

This module only draws random numbers and fixes shapes.  It holds none of the
method's arithmetic, so that both the HIP path and the CPU oracle can take their
inputs from it without sharing any computation.

Shapes follow the notation of "Interleaved Head Attention" (section 3.1 and
Algorithm 1): X is [B, N, D]; W_Q, W_K, W_V are [D, H*d] with head m's
projection W^(m) in columns [m*d, (m+1)*d); the mixing tensors alpha^{Q,K,V}
are [H (source head m, summed)][H (target head h)][P (pseudo index j)]; the
collapse map R is [H][H*P] with column h'*P + j (0-based form of (h'-1)P + j).

Distributions: X ~ N(0, 1), W ~ N(0, 1/D), alpha ~ N(0, 1/H),
R ~ N(0, 1/(H*P)).  With these, the mixed queries and keys have roughly unit
variance and the scaled scores are roughly N(0, 1) (the variance argument of
the textbook chapter on attention, section 5.2).  Draw order is X, W_Q, W_K,
W_V, alpha^Q, alpha^K, alpha^V, R, then any extras, from numpy's PCG64.

For bf16 workloads X and W are rounded to bf16 (round to nearest even) here,
and both sides consume exactly those values; alpha and R stay fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_WINDOW = 2
MASK_NAMES = {"none": MASK_NONE, "causal": MASK_CAUSAL, "window": MASK_WINDOW}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    D: int
    H: int
    P: int
    mask: int
    window: int          # stacked-index window W_s (only used when mask == MASK_WINDOW)
    dtype: str           # "f32" or "bf16": dtype of X and W at the boundary
    seed: int
    identity_mix: bool = False   # alpha[m][h][0] = 1(m == h), other j zero; R = I (P == 1)
    repeated_keys: int = 0       # number of positions that receive one shared copied row of X

    @property
    def d(self) -> int:
        return self.D // self.H

    @property
    def PN(self) -> int:
        return self.P * self.N

    def describe(self) -> str:
        m = {MASK_NONE: "none", MASK_CAUSAL: "causal", MASK_WINDOW: f"window(W_s={self.window})"}[self.mask]
        return (f"{self.name}: B={self.B} N={self.N} D={self.D} H={self.H} d={self.d} P={self.P} "
                f"mask={m} dtype={self.dtype}")


def default_window(N: int, P: int) -> int:
    """Stacked-index sliding window N/(2P) (Figure 1 of the IHA page), floored."""
    return N // (2 * P)


def _wl(name, B, N, D, H, P, mask, dtype, seed, **kw) -> Workload:
    window = default_window(N, P) if mask == MASK_WINDOW else 0
    return Workload(name, B, N, D, H, P, mask, window, dtype, seed, **kw)


# The named workloads.  Seeds are 1000 + their position in this list.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        _wl("tiny_f32_none", 1, 64, 64, 4, 2, MASK_NONE, "f32", 1000),
        _wl("mha_causal_bf16", 2, 1024, 1024, 16, 1, MASK_CAUSAL, "bf16", 1001, identity_mix=True),
        _wl("iha_window_p2_b4_n4096", 4, 4096, 2048, 16, 2, MASK_WINDOW, "bf16", 1002),
        _wl("iha_window_p2_n16384_longctx", 1, 16384, 2048, 16, 2, MASK_WINDOW, "bf16", 1003,
            repeated_keys=64),
        _wl("iha_window_p4_b2_n8192_wide", 2, 8192, 2560, 20, 4, MASK_WINDOW, "bf16", 1004),
        _wl("iha_causal_p4_b2_n8192_wide", 2, 8192, 2560, 20, 4, MASK_CAUSAL, "bf16", 1004),
    ]
}
HEADLINE = ["iha_window_p2_b4_n4096", "iha_window_p2_n16384_longctx",
            "iha_window_p4_b2_n8192_wide", "iha_causal_p4_b2_n8192_wide"]


def custom(B, N, D, H, P, mask, dtype="bf16", seed=7, window: Optional[int] = None, **kw) -> Workload:
    if isinstance(mask, str):
        mask = MASK_NAMES[mask]
    if window is None:
        window = default_window(N, P) if mask == MASK_WINDOW else 0
    return Workload(f"custom_B{B}_N{N}_D{D}_H{H}_P{P}_m{mask}_w{window}_{dtype}", B, N, D, H, P,
                    mask, window, dtype, seed, **kw)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32 holding bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make_inputs(w: Workload) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.  All arrays are float32 and C-contiguous.

    For bf16 workloads X and W_* hold bf16-representable values.  Workloads with
    repeated rows also return ``repeated_pos``: the sorted flat token indices b*N + t
    that received the copied row (int64).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, N, D, H, P = w.B, w.N, w.D, w.H, w.P
    X = rng.standard_normal((B, N, D), dtype=np.float32)
    s = np.float32(1.0 / np.sqrt(D))
    WQ = rng.standard_normal((D, D), dtype=np.float32) * s
    WK = rng.standard_normal((D, D), dtype=np.float32) * s
    WV = rng.standard_normal((D, D), dtype=np.float32) * s
    sa = np.float32(1.0 / np.sqrt(H))
    aQ = rng.standard_normal((H, H, P), dtype=np.float32) * sa
    aK = rng.standard_normal((H, H, P), dtype=np.float32) * sa
    aV = rng.standard_normal((H, H, P), dtype=np.float32) * sa
    R = rng.standard_normal((H, H * P), dtype=np.float32) * np.float32(1.0 / np.sqrt(H * P))
    if w.identity_mix:
        aQ = np.zeros((H, H, P), np.float32)
        aQ[np.arange(H), np.arange(H), 0] = 1.0
        aK = aQ.copy()
        aV = aQ.copy()
        R = np.zeros((H, H * P), np.float32)
        R[np.arange(H), np.arange(H) * P] = 1.0
    pos = None
    if w.repeated_keys:
        row = rng.standard_normal(D, dtype=np.float32)
        pos = rng.choice(B * N, size=w.repeated_keys, replace=False)
        X.reshape(B * N, D)[pos] = row
    if w.dtype == "bf16":
        X, WQ, WK, WV = (round_to_bf16(a) for a in (X, WQ, WK, WV))
    out = dict(X=X, WQ=WQ, WK=WK, WV=WV, aQ=aQ, aK=aK, aV=aV, R=R)
    out = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in out.items()}
    if pos is not None:
        out["repeated_pos"] = np.sort(pos.astype(np.int64))   # flat token indices b*N + t
    return out


def make_params(w: Workload) -> Dict[str, np.ndarray]:
    """Weights, mixing tensors and collapse map of workload ``w`` without X, for inputs too
    large to draw in one array: drawn from PCG64 seeded with (seed, 0) in the order W_Q, W_K,
    W_V, alpha^Q, alpha^K, alpha^V, R, with the distributions of ``make_inputs``."""
    rng = np.random.Generator(np.random.PCG64([w.seed, 0]))
    D, H, P = w.D, w.H, w.P
    s = np.float32(1.0 / np.sqrt(D))
    W = [rng.standard_normal((D, D), dtype=np.float32) * s for _ in range(3)]
    sa = np.float32(1.0 / np.sqrt(H))
    al = [rng.standard_normal((H, H, P), dtype=np.float32) * sa for _ in range(3)]
    R = rng.standard_normal((H, H * P), dtype=np.float32) * np.float32(1.0 / np.sqrt(H * P))
    if w.dtype == "bf16":
        W = [round_to_bf16(a) for a in W]
    out = dict(WQ=W[0], WK=W[1], WV=W[2], aQ=al[0], aK=al[1], aV=al[2], R=R)
    return {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in out.items()}


def make_sequence(w: Workload, b: int) -> np.ndarray:
    """X[b] ([N, D], N(0, 1), bf16-rounded for bf16 workloads) drawn on its own from PCG64
    seeded with (seed, b + 1), so that any one sequence of a large batch can be redrawn."""
    rng = np.random.Generator(np.random.PCG64([w.seed, b + 1]))
    x = rng.standard_normal((w.N, w.D), dtype=np.float32)
    return round_to_bf16(x) if w.dtype == "bf16" else x


def make_stacked_qkv(B: int, PN: int, H: int, d: int, seed: int, scale: float = 1.0):
    """Draw fp16-representable stacked Q-bar, K-bar, V-bar of shape [B, PN, H, d] (interleaved rows).

    Used to exercise the attention step on its own.  Values are float32 holding
    fp16 numbers, N(0, scale^2) before rounding.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = (rng.standard_normal((B, PN, H, d), dtype=np.float32) * np.float32(scale)).astype(np.float16)
    k = (rng.standard_normal((B, PN, H, d), dtype=np.float32) * np.float32(scale)).astype(np.float16)
    v = rng.standard_normal((B, PN, H, d), dtype=np.float32).astype(np.float16)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def make_stacked_grad(B: int, PN: int, H: int, d: int, seed: int) -> np.ndarray:
    """Draw an fp16-representable upstream gradient dO of shape [B, PN, H, d], N(0, 1) before
    rounding (float32 holding fp16 numbers), for the attention backward."""
    rng = np.random.Generator(np.random.PCG64([seed, 99]))
    return rng.standard_normal((B, PN, H, d), dtype=np.float32).astype(np.float16).astype(np.float32)


def make_output_grad(w: Workload) -> np.ndarray:
    """Draw an upstream gradient G of the layer output, [B, N, D] float32, N(0, 1), from PCG64
    seeded with (seed, 98)."""
    rng = np.random.Generator(np.random.PCG64([w.seed, 98]))
    return rng.standard_normal((w.B, w.N, w.D), dtype=np.float32)


def sample_tokens(w: Workload, n: int, seed: int = 0) -> np.ndarray:
    """Flat token indices b*N + t to check at full size: the first and last tokens of each
    sequence (fewest / most visible keys) plus uniformly drawn ones, sorted and unique."""
    rng = np.random.Generator(np.random.PCG64(10_000 + w.seed + seed))
    picks = []
    for b in range(w.B):
        base = b * w.N
        picks += [base + t for t in range(min(4, w.N))]
        picks += [base + w.N - 1 - t for t in range(min(2, w.N))]
    rest = max(0, n - len(picks))
    picks += list(rng.choice(w.B * w.N, size=min(rest, w.B * w.N), replace=False))
    return np.unique(np.array(picks, dtype=np.int64))
