#!/usr/bin/env python3
"""Throughput of the IHA forward pass on one MI355X.

A step is one whole forward (weight transpose, projection GEMMs + mixing, attention,
first-rows recomputation, collapse) over one batch of synthetic inputs that are resident in
HBM before timing.
Prints one JSON line: pseudo-tokens/s for the whole forward, per-kernel times from HIP
events recorded on the launch stream around every kernel of every timed step, the
roofline position of the dominant kernel and of attention, and the CPU oracle timed on
a bounded sample of the same workload.

Work per unit (algorithmic, the count the pages' convention gives):
  attention  4 * d flops per visible (query, key) pair: QK^T and AV at 2 flops per
             multiply-add (textbook eq. 5.34), masked pairs and softmax not counted
  projection 6 * D^2 flops per token (three D x D projections, eq. 5.34) plus the
             mixing, 6 * D * H * P flops per token (Algorithm 1)
  collapse   bytes: P*H*d*4 read + H*d*4 written per token
  prep       bytes: 3*D^2*2 read + 3*D^2*2 written (bf16 weight transpose)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2.5e15      # dense fp16 / bf16 matrix-core FLOP/s, MI355X
PEAK_MFMA_F32 = 157.3e12
PEAK_HBM = 8.0e12           # bytes/s


def allowed_pairs(L, mask, window):
    """Visible (query, key) pairs per (b, h) over L stacked rows."""
    if mask == 0:
        return L * L
    if mask == 1:
        return L * (L + 1) // 2
    W = min(window, L)
    return W * (W + 1) // 2 + (L - W) * W


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="iha_window_p2_b4_n4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens the CPU oracle computes for the baseline sample")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the forward shards by sequence across GPUs with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import interleaved_head_layer_amd as iha
    from interleaved_head_layer_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = wl.make_inputs(w)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = lambda a, d=dt: torch.from_numpy(a).to(dev).to(d).contiguous()
    X, WQ, WK, WV = t(x["X"]), t(x["WQ"]), t(x["WK"]), t(x["WV"])
    aQ, aK, aV, R = (t(x[k], torch.float32) for k in ("aQ", "aK", "aV", "R"))
    prob = iha.make_problem(w.B, w.N, w.D, w.H, w.P, w.mask, w.window,
                            iha.IHA_BF16 if w.dtype == "bf16" else iha.IHA_F32)
    ws = torch.empty(iha.iha_workspace_bytes(prob), dtype=torch.uint8, device=dev)
    out = torch.empty((w.B, w.N, w.D), dtype=torch.float32, device=dev)

    def step(events=None):
        iha.iha_forward(X, WQ, WK, WV, aQ, aK, aV, R, w.H, w.P, w.mask, w.window,
                        out=out, workspace=ws, events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e in evs:               # create the events before the timed region
        for ev in e:
            ev.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert bool(torch.isfinite(out).all()), "non-finite output"

    ms_step = (t1 - t0) * 1e3 / args.steps
    names = ["prep", "proj_mix", "attention", "first_rows", "collapse"]
    kms = {n: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(args.steps)]))
           for k, n in enumerate(names)}

    B, N, D, H, P, d = w.B, w.N, w.D, w.H, w.P, w.d
    L = P * N
    pairs = allowed_pairs(L, w.mask, w.window)
    attn_flops = 4.0 * d * B * H * pairs
    proj_flops = 6.0 * B * N * D * D + 6.0 * B * N * D * H * P
    collapse_bytes = B * N * (P * H * d * 4 + H * d * 4) + H * H * P * 4
    prep_bytes = 3 * D * D * 2 * 2

    def roof(kind, work, ms):
        if kind == "mfma":
            a = work / (ms * 1e-3) / 1e12
            return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_MFMA_F16 / 1e12,
                    "unit": "TFLOP/s", "frac": round(a / (PEAK_MFMA_F16 / 1e12), 4), "traffic": None}
        a = work / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(a / (PEAK_HBM / 1e9), 4), "traffic": None}

    roofs = {"prep": roof("hbm", prep_bytes, kms["prep"]),
             "proj_mix": roof("mfma", proj_flops, kms["proj_mix"]),
             "attention": roof("mfma", attn_flops, kms["attention"]),
             "collapse": roof("hbm", collapse_bytes, kms["collapse"])}
    dominant = max(kms, key=kms.get)
    value = B * P * N / (ms_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tok = np.sort(np.random.default_rng(0).choice(B * N, args.cpu_tokens, replace=False))
        c0 = time.perf_counter()
        oracle.forward(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                       H, P, w.mask, w.window, tokens=tok)
        cs = time.perf_counter() - c0
        cpu = {"value": round(len(tok) * P / cs, 2), "unit": "pseudo-tokens/s",
               "cores": oracle.threads(), "kind": "oracle",
               "sample": f"{len(tok)} uniformly drawn tokens of {w.name} (all their heads and "
                         f"pseudo-tokens, plus the key/value projections they can see), "
                         f"{cs:.1f} s wall in IEEE double"}

    line = {
        "metric": "IHA fwd pseudo-tokens/s + attention TFLOP/s (% of MI355X bf16 MFMA peak)",
        "value": round(value, 1), "unit": "pseudo-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16-mfma/fp32-acc" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": B, "N": N, "D": D, "H": H, "d": d, "P": P,
                   "mask": ["none", "causal", "window"][w.mask], "window": w.window,
                   "input_dtype": w.dtype, "global_batch": B, "seq_len": N, "parallelism": "none"},
        "roofline": dict(roofs[dominant], kernel=dominant),
        "attention": dict(roofs["attention"], ms=round(kms["attention"], 4),
                          tflops=roofs["attention"]["achieved"]),
        "kernels_ms": {k: round(v, 4) for k, v in kms.items()},
        "kernel_roofline": roofs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
