#!/usr/bin/env python3
"""Throughput of the IHA forward pass on one MI355X.

A step is one whole forward (weight transpose, projection GEMMs, mixing, attention,
first rows, collapse) over one batch of synthetic inputs that are resident in
HBM before timing.
Prints one JSON line: pseudo-tokens/s for the whole forward (K plain forwards back to back),
per-step times from HIP events recorded on the launch stream between the kernels of a second
timed pass of K forwards (every event record adds a gap of about 10 us between kernels, so
the throughput pass records none), the roofline position of the dominant step and of every
step, the same figures (fewer steps) for the other headline workloads, and the CPU oracle
timed on a bounded sample of the main workload.

Work per unit (algorithmic, the count the pages' convention gives):
  attention  4 * d flops per visible (query, key) pair: QK^T and AV at 2 flops per
             multiply-add (textbook eq. 5.34), masked pairs and softmax not counted
  gemm       6 * D^2 flops per token (the three D x D projections, eq. 5.34)
  mix        bytes: 3 * D * 4 read (projected values, fp32) + 3 * P * D * 2 written
             (stacked fp16 Q~, K~, V~) per token.  Where the mixing runs in the GEMM's
             epilogue (IHA_PLAN_MIX_FUSED) the gemm step holds it and the mix step is empty
             (the first rows' fp32 mixing runs in the attention launch)
  collapse   bytes: P*H*d*e read (e = 2: the bf16 forward keeps the stacked outputs in fp16;
             4 for fp32) + H*d*4 written per token
  prep       bytes: 3*D^2*2 read + 3*D^2*2 written (bf16 weight transpose)
"""
import argparse
import ctypes
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


def counter_traffic(workload, step):
    """HBM bytes per step of `step` from the committed rocprofv3 counter summary of
    `workload` (FETCH_SIZE and WRITE_SIZE per dispatch, scaled by the copy reference), or
    None if there is none or the kernel's source changed since the counters were taken."""
    import glob
    import hashlib
    import re
    root = os.path.dirname(os.path.abspath(__file__))
    for path in glob.glob(os.path.join(root, "profiles", "hbm_counters_*.md")):
        m = re.search(r"```json\n(.*?)```", open(path).read(), re.S)
        if not m:
            continue
        info = json.loads(m.group(1))
        if info.get("workload") != workload or step not in info.get("steps", {}):
            continue
        st = info["steps"][step]
        src = os.path.join(root, st["source"])
        if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != st["sha256"]:
            return None
        sc = info["scale"]
        kib = sum((f * sc["FETCH_SIZE"] + w * sc["WRITE_SIZE"]) * n for f, w, n in st["kernels"].values())
        return int(kib * 1024)
    return None


STEPS = ["prep", "gemm", "mix", "attention", "first_rows", "collapse"]


def roof(kind, work, ms):
    if kind == "mfma":
        a = work / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_MFMA_F16 / 1e12,
                "unit": "TFLOP/s", "frac": round(a / (PEAK_MFMA_F16 / 1e12), 4), "traffic": None}
    a = work / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": round(a / (PEAK_HBM / 1e9), 4), "traffic": None}


def run_workload(w, steps, warmup):
    """Time `steps` forwards of workload `w` (after `warmup`); returns inputs and figures."""
    import numpy as np
    import torch
    import interleaved_head_layer_amd as iha
    from interleaved_head_layer_amd import workloads as wl

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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # Second timed pass: the same forwards with HIP events between their kernels.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(iha.TIMED_EVENTS)]
           for _ in range(steps)]
    for e in evs:               # create the events before the timed region
        for ev in e:
            ev.record()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    del X, WQ, WK, WV, aQ, aK, aV, R, ws, out
    torch.cuda.empty_cache()

    fused = bool(iha.iha_plan(prob) & iha.IHA_PLAN_MIX_FUSED)
    ms_step = (t1 - t0) * 1e3 / steps
    ms_step_events = (t3 - t2) * 1e3 / steps
    kms = {n: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(steps)]))
           for k, n in enumerate(STEPS)}
    B, N, D, H, P, d = w.B, w.N, w.D, w.H, w.P, w.d
    L = P * N
    attn_flops = 4.0 * d * B * H * allowed_pairs(L, w.mask, w.window)
    if fused:   # the mixing runs in the GEMM's epilogue: the mix step is empty
        mix = None
    else:
        mix = roof("hbm", B * N * (3 * D * 4 + 3 * P * D * 2), kms["mix"])
    roofs = {"prep": roof("hbm", 3 * D * D * 2 * 2, kms["prep"]),
             "gemm": roof("mfma", 6.0 * B * N * D * D, kms["gemm"]),
             "mix": mix,
             "attention": roof("mfma", attn_flops, kms["attention"]),
             "collapse": roof("hbm", B * N * (P * H * d * (2 if w.dtype == "bf16" else 4) + H * d * 4)
                              + H * H * P * 4, kms["collapse"])}
    roofs = {k: v for k, v in roofs.items() if v is not None}
    return x, {"ms_step": ms_step, "ms_step_events": ms_step_events,
               "value": B * P * N / (ms_step * 1e-3), "kms": kms,
               "roofs": roofs, "mix_fused": fused}


def run_attention_backward(w, steps, warmup):
    """Time iha_attention_backward on the stacked attention of workload `w` (L = P*N rows per
    sequence, its heads, head width, mask and window), inputs resident on the GPU.  Work is
    counted as 2.5x the forward's 4*d*(visible pairs) per head: the gradient products dV, dP,
    dQ and dK plus the recomputed scores, 2*d flops per visible pair each."""
    import torch
    import interleaved_head_layer_amd as iha

    B, H, d, L = w.B, w.H, w.D // w.H, w.P * w.N
    mask = ["none", "causal", "window"][w.mask]
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    q, k, v, go = (torch.randn((B, L, H, d), generator=g, device=dev).half() for _ in range(4))
    nbytes = ctypes.c_size_t(0)
    lib = iha.load_library()
    assert lib.iha_attention_backward_workspace(B, L, H, d, ctypes.byref(nbytes)) == 0
    ws = torch.empty(int(nbytes.value), dtype=torch.uint8, device=dev)
    call = lambda: iha.iha_attention_backward(q, k, v, go, mask, w.window, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    work = 2.5 * 4.0 * d * B * H * allowed_pairs(L, w.mask, w.window)
    return {"shape": {"B": B, "L": L, "H": H, "d": d, "mask": mask, "window": w.window},
            "ms": round(ms, 4), "steps": steps, "work_flop": work,
            "roofline": roof("mfma", work, ms),
            "note": "whole call: prep copies, forward recompute (O, lse), dQ and dK/dV kernels"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # The chip needs ~40 ms of this load to reach its steady clocks: with 5 warm-up forwards
    # the first timed ones run ~10 % slower.
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="iha_window_p2_b4_n4096")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=16384,
                    help="tokens the CPU oracle computes for the baseline sample (at most B*N)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other headline workloads")
    ap.add_argument("--extra-steps", type=int, default=5)
    ap.add_argument("--only-backward", action="store_true",
                    help="time only the attention backward of the workload's attention shape")
    ap.add_argument("--copy-ref", type=int, default=0, metavar="MIB",
                    help="first run a plain device copy of MIB MiB (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: the forward runs on one GPU; --gpus {args.gpus} is not supported "
              "(the forward shards by sequence across GPUs with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    from interleaved_head_layer_amd import workloads as wl

    if args.copy_ref > 0:
        import torch
        src = torch.ones(args.copy_ref << 18, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = wl.WORKLOADS[args.workload]
    if args.only_backward:
        print(json.dumps({"workload": w.name,
                          "attention_backward": run_attention_backward(w, args.steps, args.warmup)}),
              flush=True)
        return
    x, r = run_workload(w, args.steps, args.warmup)
    kms, roofs = r["kms"], r["roofs"]
    dominant = max(roofs, key=lambda k: kms[k])
    for k in roofs:
        roofs[k]["traffic"] = counter_traffic(w.name, k)
    B, N, D, H, P, d = w.B, w.N, w.D, w.H, w.P, w.d

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        tok = np.sort(np.random.default_rng(0).choice(B * N, min(args.cpu_tokens, B * N),
                                                      replace=False))
        c0 = time.perf_counter()
        oracle.forward(x["X"], x["WQ"], x["WK"], x["WV"], x["aQ"], x["aK"], x["aV"], x["R"],
                       H, P, w.mask, w.window, tokens=tok)
        cs = time.perf_counter() - c0
        cpu = {"value": round(len(tok) * P / cs, 2), "unit": "pseudo-tokens/s",
               "cores": oracle.threads(), "kind": "oracle",
               "sample": (f"all {len(tok)} tokens of {w.name} (one whole forward)"
                          if len(tok) == B * N else
                          f"{len(tok)} uniformly drawn tokens of {w.name} (all their heads and "
                          f"pseudo-tokens, plus the key/value projections they can see)")
                         + f", {cs:.1f} s wall in IEEE double"}
    del x

    extra = {}
    bwd = None
    if not args.no_extra:
        bwd = run_attention_backward(w, args.extra_steps, 3)
        for name in wl.HEADLINE + ["mha_causal_bf16"]:   # + the P = 1 MHA configuration
            if name == w.name:
                continue
            _, e = run_workload(wl.WORKLOADS[name], args.extra_steps, 10)
            extra[name] = {"ms_per_step": round(e["ms_step"], 4),
                           "pseudo_tokens_per_s": round(e["value"], 1),
                           "attention": dict(e["roofs"]["attention"],
                                             ms=round(e["kms"]["attention"], 4),
                                             traffic=counter_traffic(name, "attention")),
                           "gemm": dict(e["roofs"]["gemm"], traffic=counter_traffic(name, "gemm")),
                           "mix_fused": e["mix_fused"],
                           "kernels_ms": {k: round(v, 4) for k, v in e["kms"].items()}}

    line = {
        "metric": "IHA fwd pseudo-tokens/s + attention TFLOP/s (% of MI355X bf16 MFMA peak)",
        "value": round(r["value"], 1), "unit": "pseudo-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_step"], 4),
        "ms_per_step_event_pass": round(r["ms_step_events"], 4),
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
        "mix_fused": r["mix_fused"],
        "other_workloads": extra,
        "attention_backward": bwd,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
