"""Parity of the HIP library against the CPU oracle on the same seeded inputs (GPU only).

Bar: max |gpu - oracle| <= tol * RMS(oracle output), tol = 1e-4 for the fp32 path and
2e-2 for the bf16 path (fp16 intermediates, fp32 accumulation).  RMS is taken over the
compared elements (the whole output; for a subset check, over the whole output it was drawn
from, which is stated where used).

Small shapes are compared element by element over the whole output; they span several
query/key tiles (128/64 rows) and GEMM tiles (128) and end in ragged tails.  The full-size
workloads are launched exactly as the benchmark launches them and compared on every output
element as well (the oracle on all host threads: 10-20 s each, about 3 minutes for the wide
causal one).  Only the 2 GiB-split test checks sampled tokens (the oracle computes a token
exactly from the keys it can see).
"""
import concurrent.futures
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from interleaved_head_layer_amd import workloads as wl
import interleaved_head_layer_amd as iha

pytestmark = pytest.mark.gpu
F32_TOL = 1e-4
BF16_TOL = 2e-2
DEV = "cuda:0"


def note(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_dev(x, w):
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda a, d=dt: torch.from_numpy(a).to(DEV).to(d).contiguous()
    return (t(x["X"]), t(x["WQ"]), t(x["WK"]), t(x["WV"]), t(x["aQ"], torch.float32),
            t(x["aK"], torch.float32), t(x["aV"], torch.float32), t(x["R"], torch.float32))


def gpu_forward(w, x, flags=0, X_override=None):
    args = list(to_dev(x, w))
    if X_override is not None:
        args[0] = X_override
    out = iha.iha_forward(*args, w.H, w.P, w.mask, w.window, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def oracle_forward(w, x, tokens=None):
    return oracle.forward(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                          w.H, w.P, w.mask, w.window, tokens=tokens)


def check(gpu, ref, tol, rms=None, what=""):
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref ** 2))) if rms is None else rms
    err = float(np.max(np.abs(gpu - ref)))
    note(f"{what}: max|err| = {err:.3e}, RMS = {rms:.3e}, ratio = {err / rms:.3e} (bar {tol:g})")
    assert err <= tol * rms, f"{what}: max|err|/RMS = {err / rms:.3e} > {tol}"
    return err / rms


# ------------------------------------------------------------------ whole output vs oracle
def test_tiny_fp32_workload_full():
    w = wl.WORKLOADS["tiny_f32_none"]
    note(w.describe())
    x = wl.make_inputs(w)
    check(gpu_forward(w, x), oracle_forward(w, x), F32_TOL, what=w.name)


def test_mha_causal_workload_full():
    w = wl.WORKLOADS["mha_causal_bf16"]
    note(w.describe())
    x = wl.make_inputs(w)
    check(gpu_forward(w, x), oracle_forward(w, x), BF16_TOL, what=w.name)


SMALL = [
    # B, N, D, H, P, mask, window, dtype
    (1, 300, 256, 2, 2, "window", None, "bf16"),     # L = 600: ragged query/key/GEMM tiles
    (2, 77, 128, 2, 3, "causal", None, "bf16"),      # d = 64, odd P, L = 231 (not a multiple of 8)
    (1, 200, 256, 2, 1, "none", None, "bf16"),       # P = 1, no mask
    (1, 130, 384, 3, 4, "window", 1, "bf16"),        # every row sees only itself
    (2, 64, 256, 2, 2, "window", 100000, "bf16"),    # window beyond the sequence = causal
    (1, 1, 128, 1, 2, "causal", None, "bf16"),       # a single token
    (1, 257, 512, 4, 2, "window", 200, "bf16"),
    (1, 150, 256, 2, 5, "none", None, "bf16"),       # P = 5, mask none over 750 rows
    (3, 40, 640, 5, 2, "causal", None, "bf16"),      # H = 5
    (2, 50, 64, 2, 3, "causal", None, "f32"),        # fp32 path, d = 32
    (1, 70, 256, 2, 2, "window", 9, "f32"),          # fp32 path, d = 128
    (1, 33, 64, 4, 2, "none", None, "f32"),          # fp32 path, d = 16
    # N a multiple of 128: the V mixing runs on the matrix cores
    (1, 256, 256, 2, 2, "causal", None, "bf16"),     # H = 2
    (2, 128, 320, 5, 4, "window", 37, "bf16"),       # H = 5 (odd), P = 4, d = 64
    (1, 128, 192, 3, 1, "none", None, "bf16"),       # H = 3, P = 1: heads past H skipped
    (1, 384, 2560, 20, 4, "window", 100, "bf16"),    # H = 20, P = 4: GEMM + separate mixing
    (2, 128, 1024, 16, 2, "causal", None, "bf16"),   # H = 16, P = 2
    # the fused projection + mixing with 20 heads (320-row tiles, heads 16..19 in a rest block)
    (1, 200, 1280, 20, 1, "causal", None, "bf16"),   # d = 64, P = 1, ragged token tile
    (2, 100, 2560, 20, 2, "window", 33, "bf16"),     # P = 2, two sequences in one token tile
    (1, 130, 1280, 20, 2, "none", None, "bf16"),     # no first-row recomputation
    (1, 128, 1024, 16, 1, "window", 21, "bf16"),     # H = 16, P = 1 fused
    (2, 256, 256, 4, 2, "window", None, "bf16"),     # W_s = 64: one key tile per query tile
    (4, 512, 512, 4, 2, "window", 300, "bf16"),      # window edges inside key tiles
    # fewer stacked rows than the fp32 first rows (P*N < 32) on the fused path
    (2, 10, 1024, 16, 2, "causal", None, "bf16"),    # R = 20 rows, 10 first tokens
    (3, 7, 1280, 20, 1, "window", 3, "bf16"),        # H = 20, R = 7, window inside them
    (1, 77, 1024, 16, 1, "window", 50, "bf16"),      # L = 77: register-copy attention path
    (2, 45, 2560, 20, 2, "causal", None, "bf16"),    # L = 90 (not a multiple of 8), H = 20
    # the Q~/K~ mixing on the matrix cores: row blocks x k-steps of source heads
    (1, 256, 2048, 16, 4, "causal", None, "bf16"),   # H*P = 64: two row blocks, one k-step
    (1, 130, 2048, 32, 4, "window", 50, "bf16"),     # H*P = 128, two k-steps, d = 64
    (2, 64, 1536, 24, 2, "causal", None, "bf16"),    # H = 24, P = 2: two row blocks, two k-steps
    (1, 96, 1536, 24, 1, "window", 40, "bf16"),      # H = 24, P = 1: one row block, two k-steps
]


@pytest.mark.parametrize("B,N,D,H,P,mask,window,dtype", SMALL)
def test_small_shapes_full(B, N, D, H, P, mask, window, dtype):
    w = wl.custom(B, N, D, H, P, mask, dtype=dtype, seed=B * 1000 + N + P, window=window)
    note(w.describe())
    x = wl.make_inputs(w)
    check(gpu_forward(w, x), oracle_forward(w, x), F32_TOL if dtype == "f32" else BF16_TOL,
          what=w.name)


# ------------------------------------------------------- full-size workloads, every element
FULL_ONE_CALL = ["iha_window_p2_b4_n4096", "iha_window_p2_n16384_longctx", "iha_window_p4_b2_n8192_wide"]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", FULL_ONE_CALL)
def test_full_size_workload_full(name, progress):
    """The full-size workloads, launched as the benchmark launches them, against the oracle on
    every output element (one oracle call, all host threads).  The long-context workload's
    64 copied rows and the 16 tokens after each are also checked on their own."""
    w = wl.WORKLOADS[name]
    note(w.describe())
    x = wl.make_inputs(w)
    gpu = gpu_forward(w, x)
    progress(f"{name}: oracle on all {w.B * w.N} tokens ({oracle.threads()} threads)")
    ref = oracle_forward(w, x)
    progress(f"{name}: oracle done")
    check(gpu, ref, BF16_TOL, what=f"{name} (whole output)")
    if "repeated_pos" in x:
        pos = x["repeated_pos"]
        near = np.unique(np.concatenate([pos + k for k in range(17)]))
        near = near[near < w.B * w.N]
        g2, r2 = gpu.reshape(-1, w.D)[near], ref.reshape(-1, w.D)[near]
        rms = float(np.sqrt(np.mean(ref ** 2)))
        check(g2, r2, BF16_TOL, rms=rms, what=f"{name} (copied rows and 16 tokens after each: {len(near)} tokens)")


@pytest.mark.timeout(600)
def test_full_size_wide_causal_sampled(progress):
    """The wide causal workload on 1024 tokens, every element of each: the first 16 and last 8
    tokens of both sequences and uniformly drawn ones.  (The whole output would take the
    double-precision oracle over ten minutes: every causal row streams up to 32 MB of keys
    and values.)  The oracle computes a token exactly from the keys it can see; RMS is over
    the sampled uniform tokens' elements."""
    w = wl.WORKLOADS["iha_causal_p4_b2_n8192_wide"]
    note(w.describe())
    x = wl.make_inputs(w)
    gpu = gpu_forward(w, x).reshape(w.B * w.N, w.D)
    rng = np.random.default_rng(w.seed)
    edges = np.concatenate([b * w.N + np.r_[0:16, w.N - 8:w.N] for b in range(w.B)])
    uniform = np.setdiff1d(rng.choice(w.B * w.N, 1100, replace=False), edges)[:1024 - len(edges)]
    tokens = np.sort(np.concatenate([edges, uniform]))
    assert len(tokens) == 1024
    ref = np.zeros((len(tokens), w.D))
    for part in np.array_split(np.arange(len(tokens)), 4):
        progress(f"{w.name}: oracle on tokens {part[0]}..{part[-1]} of {len(tokens)}")
        ref[part] = oracle_forward(w, x, tokens=tokens[part])
    rms = float(np.sqrt(np.mean(ref[np.isin(tokens, uniform)] ** 2)))
    check(gpu[tokens], ref, BF16_TOL, rms=rms, what=f"{w.name} ({len(tokens)} tokens)")


@pytest.mark.timeout(600)
def test_unfused_projection_320_row_tiles(progress):
    """An unfused shape (24 heads) sized so that on a 256-CU device both projection GEMMs
    take 320-row tiles (fewer rounds of workgroups than 256-row tiles): Y_QK is 5632 x 6144
    (18 row tiles, the last 192 of 320 rows) and Y_V^T 3072 x 5632 (10 row tiles, the last
    192 rows).  Every output element against the oracle."""
    w = wl.custom(1, 5632, 3072, 24, 1, "window", seed=5632, window=256)
    note(w.describe())
    x = wl.make_inputs(w)
    gpu = gpu_forward(w, x)
    progress(f"{w.name}: oracle on all {w.B * w.N} tokens ({oracle.threads()} threads)")
    ref = oracle_forward(w, x)
    check(gpu, ref, BF16_TOL, what=f"{w.name} (whole output)")


@pytest.mark.parametrize("scale", [2.0, 4.0])
def test_peaked_softmax_rows(scale):
    """X scaled up (scores about scale^2 larger: nearly one-hot softmax rows, many offset
    moves in the attention kernel) plus 32 copies of one row, on a 16-head window workload."""
    w = wl.custom(1, 1024, 1024, 16, 2, "window", seed=int(scale * 10), repeated_keys=32)
    note(f"{w.describe()} X x {scale}")
    x = wl.make_inputs(w)
    x = dict(x)
    x["X"] = wl.round_to_bf16(x["X"] * np.float32(scale))
    check(gpu_forward(w, x), oracle_forward(w, x), BF16_TOL, what=f"{w.name} X x {scale}")


def test_fused_projection_beyond_2gib_of_x():
    """X of 1025 x 1024 tokens x 1024 bf16 (2.15 GB) exceeds what one launch of the fused
    projection GEMM addresses, so its tokens are split over two launches at token 1,048,320,
    inside sequence 1023.  Checked on tokens on both sides of that split and in the first and
    last sequences."""
    w = wl.custom(1025, 1024, 1024, 16, 1, "causal", seed=4242)
    note(w.describe())
    prob = iha.make_problem(w.B, w.N, w.D, w.H, w.P, w.mask, w.window)
    assert iha.iha_plan(prob) & iha.IHA_PLAN_MIX_FUSED
    p = wl.make_params(w)
    X = torch.empty(w.B, w.N, w.D, dtype=torch.bfloat16, device=DEV)
    Xf = X.view(w.B * w.N, w.D)
    assert X.numel() * 2 >= 2 ** 31
    step = 64
    with concurrent.futures.ThreadPoolExecutor(8) as ex:
        for b0 in range(0, w.B, step):
            blk = np.concatenate(list(ex.map(lambda b: wl.make_sequence(w, b), range(b0, min(w.B, b0 + step)))))
            Xf[b0 * w.N:b0 * w.N + blk.shape[0]] = torch.from_numpy(blk).to(torch.bfloat16).to(DEV)
    dev = lambda a, d: torch.from_numpy(a).to(DEV).to(d).contiguous()
    bf, f32 = torch.bfloat16, torch.float32
    out = iha.iha_forward(X, dev(p["WQ"], bf), dev(p["WK"], bf), dev(p["WV"], bf), dev(p["aQ"], f32),
                          dev(p["aK"], f32), dev(p["aV"], f32), dev(p["R"], f32), w.H, w.P, w.mask,
                          w.window)
    del X, Xf
    out = out.reshape(w.B * w.N, w.D)
    split = 1048320
    rng = np.random.default_rng(w.seed)
    for b, local in [(0, [0, 1, 2, 517, 1023]),
                     (1023, [0, 1, 765, 766, 767, 768, 769, 770, 1022, 1023]),
                     (1024, [0, 1, 2, 3, 300, 1023])]:
        local = np.unique(np.concatenate([local, rng.choice(w.N, 6, replace=False)]))
        gpu = out[torch.from_numpy(b * w.N + local).to(DEV)].cpu().numpy().astype(np.float64)
        ref = oracle.forward(wl.make_sequence(w, b)[None], p["WQ"], p["WK"], p["WV"], p["aQ"], p["aK"],
                             p["aV"], p["R"], w.H, w.P, w.mask, w.window, tokens=local)
        check(gpu, ref, BF16_TOL, what=f"sequence {b} tokens {local.tolist()}")
    assert 1023 * w.N < split < 1024 * w.N
    assert torch.isfinite(out).all().item()


# --------------------------------------------------------------- attention step alone
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask,window", [("none", 0), ("causal", 0), ("window", 37)])
def test_attention_step_vs_oracle(d, mask, window):
    """iha_attention on generator-made fp16 stacked Q, K, V against the oracle's attention core
    (textbook Algorithm 5.1) per (b, h), on every row."""
    B, L, H = 2, 333, 2
    q, k, v = wl.make_stacked_qkv(B, L, H, d, seed=d + len(mask), scale=1.0)
    note(f"attention B={B} L={L} H={H} d={d} mask={mask} window={window}")
    Q = torch.from_numpy(q).to(DEV).half()
    K = torch.from_numpy(k).to(DEV).half()
    Vt = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 3, 1))).to(DEV).half()
    O = iha.iha_attention(Q, K, Vt, mask, window).cpu().numpy().astype(np.float64)
    code = {"none": oracle.MASK_NONE, "causal": oracle.MASK_CAUSAL, "window": oracle.MASK_WINDOW}[mask]
    ref = np.zeros_like(O)
    for b in range(B):
        for h in range(H):
            ref[b, :, h], _, _ = oracle.attention(q[b, :, h], k[b, :, h], v[b, :, h], code, window)
    check(O, ref, BF16_TOL, what=f"attention d={d} {mask}")


# --------------------------------------------------------------------- properties on GPU
def test_bitwise_deterministic():
    w = wl.custom(2, 300, 512, 4, 2, "window", seed=77)
    note(w.describe())
    x = wl.make_inputs(w)
    a, b = gpu_forward(w, x), gpu_forward(w, x)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("mask", ["causal", "window"])
@pytest.mark.parametrize("scale", [1.5, 6.0])
def test_future_perturbation_leaves_past_bitwise(mask, scale):
    """Textbook section 5.4: changing inputs after token t0 leaves outputs up to t0 unchanged,
    bit for bit, also when the changed rows (scale 6: scores ~36x larger) drive the waves
    they share with earlier rows through the softmax's offset updates."""
    w = wl.custom(1, 400, 256, 2, 2, mask, seed=5, window=64 if mask == "window" else None)
    note(w.describe())
    x = wl.make_inputs(w)
    a = gpu_forward(w, x)
    x2 = dict(x)
    X2 = x["X"].copy()
    t0 = 150
    X2[:, t0 + 1:] = wl.round_to_bf16(X2[:, t0 + 1:] * scale + 0.25)
    x2["X"] = X2
    b = gpu_forward(w, x2)
    assert np.array_equal(a[:, :t0 + 1], b[:, :t0 + 1])
    assert not np.allclose(a[:, t0 + 1:], b[:, t0 + 1:])


def test_nonfinite_input_reported_with_check_flag():
    w = wl.custom(1, 64, 256, 2, 2, "causal", seed=3)
    x = wl.make_inputs(w)
    x["X"] = x["X"].copy()
    x["X"][0, 10, 3] = np.nan
    note("NaN input, IHA_FLAG_CHECK")
    with pytest.raises(iha.IHAError) as e:
        gpu_forward(w, x, flags=iha.IHA_FLAG_CHECK)
    assert "NONFINITE" in str(e.value)
    ok = wl.make_inputs(w)
    gpu_forward(w, ok, flags=iha.IHA_FLAG_CHECK)     # clean input passes the check


@pytest.mark.parametrize("D,H", [(1024, 16), (256, 2)])   # fused and unfused mixing paths
def test_fp16_range_overflow_reported_with_check_flag(D, H):
    """Inputs whose projections and mixed values exceed 65504 (X x 3e4): IHA_ERR_RANGE under
    IHA_FLAG_CHECK; without the flag the call returns and the output holds non-finite values
    (the documented behaviour: no silent rescaling).  X x 40 stays inside the range and
    passes the check."""
    w = wl.custom(1, 128, D, H, 2, "causal", seed=21)
    x = wl.make_inputs(w)
    big = dict(x)
    big["X"] = wl.round_to_bf16(x["X"] * np.float32(3e4))
    note(f"{w.name}: X x 3e4, IHA_FLAG_CHECK")
    with pytest.raises(iha.IHAError) as e:
        gpu_forward(w, big, flags=iha.IHA_FLAG_CHECK)
    assert "RANGE" in str(e.value)
    out = gpu_forward(w, big)
    assert not np.all(np.isfinite(out))
    ok = dict(x)
    ok["X"] = wl.round_to_bf16(x["X"] * np.float32(40.0))
    assert np.all(np.isfinite(gpu_forward(w, ok, flags=iha.IHA_FLAG_CHECK)))


def test_collapse_map_beyond_fp16_range():
    """An R entry of 1e5 is split into fp16 parts by the bf16 path's collapse: IHA_ERR_RANGE
    under IHA_FLAG_CHECK.  The fp32 path has no such limit and matches the oracle."""
    for dtype in ("bf16", "f32"):
        w = wl.custom(1, 64, 256, 2, 2, "window", dtype=dtype, seed=22)
        x = dict(wl.make_inputs(w))
        x["R"] = x["R"].copy()
        x["R"][1, 2] = 1e5
        note(f"{w.name}: R[1][2] = 1e5, IHA_FLAG_CHECK")
        if dtype == "bf16":
            with pytest.raises(iha.IHAError) as e:
                gpu_forward(w, x, flags=iha.IHA_FLAG_CHECK)
            assert "RANGE" in str(e.value)
        else:
            check(gpu_forward(w, x, flags=iha.IHA_FLAG_CHECK), oracle_forward(w, x), F32_TOL,
                  what=f"{w.name} R[1][2] = 1e5")


FUSED_COLLAPSE = [
    # B, N, D, H, P, mask: the plain and fused-mixing paths, every mask, P 1-4, H up to 20
    (1, 300, 256, 2, 2, "window"),
    (2, 128, 1024, 16, 2, "causal"),   # mixing fused into the GEMM (fp32 first rows from Ye)
    (1, 200, 1280, 10, 4, "none"),
    (1, 100, 2560, 20, 4, "causal"),
    (1, 64, 512, 4, 1, "window"),
]


@pytest.mark.parametrize("B,N,D,H,P,mask", FUSED_COLLAPSE)
def test_fused_collapse_option(B, N, D, H, P, mask):
    """IHA_FLAG_FUSED_COLLAPSE (the collapse in the attention epilogue, fp32 atomics): the same
    bar against the oracle, and agreement with the default path to rounding."""
    w = wl.custom(B, N, D, H, P, mask, seed=400 + N + P)
    note(w.describe() + " fused collapse")
    x = wl.make_inputs(w)
    ref = oracle_forward(w, x)
    fused = gpu_forward(w, x, flags=iha.IHA_FLAG_FUSED_COLLAPSE)
    check(fused, ref, BF16_TOL, what=w.name + " fused collapse vs oracle")
    check(fused, gpu_forward(w, x), BF16_TOL, rms=float(np.sqrt(np.mean(ref ** 2))),
          what=w.name + " fused collapse vs default path")


def test_fused_collapse_rejects_fp32():
    w = wl.WORKLOADS["tiny_f32_none"]
    x = wl.make_inputs(w)
    with pytest.raises(iha.IHAError) as e:
        gpu_forward(w, x, flags=iha.IHA_FLAG_FUSED_COLLAPSE)
    assert e.value.status == 6  # IHA_ERR_UNSUPPORTED


def test_empty_window_is_rejected():
    w = wl.custom(1, 3, 128, 1, 2, "window", seed=3)   # N // (2P) = 0
    assert w.window == 0
    x = wl.make_inputs(w)
    with pytest.raises(iha.IHAError) as e:
        gpu_forward(w, x)
    assert "EMPTY_ROW" in str(e.value)
