#!/usr/bin/env python3
"""Benchmark of the selective state-space scan on one MI355X.

Headline: mssm_selective_scan_fwd on the Mamba-1.4B layer shape (batch 4,
d_inner 4096, seqlen 8192, d_state 16; u, delta, B, C, z in bf16; A, D fp32;
fp32 state; final state written), inputs resident in HBM.  A "step" is one
call of the scan over that batch.  `value` is the effective HBM bandwidth:
algorithmic bytes (every input read once, every output written once) divided
by the time per step.  Also reported: tokens-ch/s (batch*seqlen*d_inner per
second), the roofline of the scan kernel, the fp64 CPU oracle timed on a
bounded sample of the same workload, and the other two entry points (decode
step on the Mamba-2.8B shape, Mamba-2 SSD) as secondary lines inside the
same JSON object.

    python bench.py [--steps K] [--warmup W] [--gpus 1]

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan effective HBM GB/s (% of peak) + B·L·D_inner tokens-ch/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
# Non-packed fp32 VALU issue rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def s6_bytes(batch, dim, L, N, esize, gate=True, skip=True, h0=False, final=True):
    """Algorithmic HBM bytes of one scan: u, delta, (z), y once each; B, C;
    A; (D); (h0); (h_final)."""
    per_tok = (3 + (1 if gate else 0)) * batch * dim * L * esize
    bc = 2 * batch * N * L * esize
    small = dim * N * 4 + (dim * 4 if skip else 0)
    st = batch * dim * N * 4 * ((1 if h0 else 0) + (1 if final else 0))
    return per_tok + bc + small + st


def decode_bytes(batch, dim, N, esize, gate=True, skip=True):
    """State read + write; u, delta, (z), y; B, C; A; (D)."""
    return (2 * batch * dim * N * 4 + (3 + (1 if gate else 0)) * batch * dim * esize
            + 2 * batch * N * esize + dim * N * 4 + (dim * 4 if skip else 0))


def ssd_bytes(batch, L, H, P, N, G, esize, gate=False, skip=True, h0=False, final=False):
    return ((2 + (1 if gate else 0)) * batch * L * H * P * esize + batch * L * H * esize
            + 2 * batch * L * G * N * esize + H * 4 + (H * 4 if skip else 0)
            + batch * H * P * N * 4 * ((1 if h0 else 0) + (1 if final else 0)))


def ssd_flops(batch, L, H, P, N, G, Q):
    """Algorithmic MFMA flops: C B^T once per (b, chunk, group) (causal half),
    Y_diag (causal half), chunk states, Y_off, state pass."""
    nc = (L + Q - 1) // Q
    causal = Q * (Q + 1) / 2
    cb = 2 * batch * nc * G * causal * N
    ydiag = 2 * batch * nc * H * causal * P
    states = 2 * batch * nc * H * Q * N * P
    yoff = 2 * batch * nc * H * Q * N * P
    spass = 2 * batch * nc * H * P * N
    return cb + ydiag + states + yoff + spass


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_launches(fn, steps, warmup, stream):
    """Warm up, then time `steps` calls with HIP events on `stream` (the
    stream the kernels are launched on).  Returns (total ms, per-call ms)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]), per


def bench_s6(args, wl):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    s = wl.shape
    log(f"[bench] generating {wl.name} inputs {s} ({wl.dtype}) ...")
    t0 = time.time()
    inp = synth.s6_inputs(**s, dtype=wl.dtype, seed=wl.seed)
    log(f"[bench] generated in {time.time() - t0:.1f}s; uploading")
    d = {k: to_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    y = torch.empty_like(d["u"])
    hf = torch.empty((s["batch"], s["d_inner"], s["d_state"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"],
                            out=y, h_final=hf, stream=stream)

    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up")
    total_ms, per = time_launches(step, args.steps, args.warmup, stream)
    esize = 2 if wl.dtype == "bf16" else 4
    nbytes = s6_bytes(s["batch"], s["d_inner"], s["seqlen"], s["d_state"], esize)
    ms = total_ms / args.steps
    kern_ms = float(np.mean(per))
    return dict(inp=inp, y=y, hf=hf, ms=ms, per=per, kern_ms=kern_ms, bytes=nbytes)


def parity_sample(inp, y, hf, rows=32, seed=0):
    """fp64 oracle on a few channels of the benchmarked output."""
    import oracle
    from selective_state_space_19_amd import synth
    rng = np.random.default_rng(seed)
    bsz, dim, L = inp["u"].shape
    b = int(rng.integers(0, bsz))
    ds = np.sort(rng.choice(dim, size=min(rows, dim), replace=False))
    sub = {k: synth.widen(inp[k][b:b + 1, ds], inp["dtype"]) for k in ("u", "delta", "z")}
    yo, ho = oracle.s6_scan(sub["u"], sub["delta"], inp["A"][ds], synth.widen(inp["B"][b:b + 1], inp["dtype"]),
                            synth.widen(inp["C"][b:b + 1], inp["dtype"]), inp["D"][ds], sub["z"])
    yg = y[b:b + 1, ds].float().cpu().numpy().astype(np.float64)
    hg = hf[b:b + 1, ds].cpu().numpy().astype(np.float64)
    ey = float(np.max(np.abs(yg - yo)) / np.max(np.abs(yo)))
    eh = float(np.max(np.abs(hg - ho)) / np.max(np.abs(ho)))
    return dict(channels=int(len(ds)), batch_row=b, y_err=ey, h_final_err=eh, tol=2e-2,
                ok=bool(ey <= 2e-2 and eh <= 2e-2))


def cpu_baseline(inp, target_s=12.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the
    benchmarked workload: the first k channels of batch row 0, full length;
    k grows until the run takes about target_s seconds of wall time."""
    import oracle
    from selective_state_space_19_amd import synth
    nth = oracle.default_threads()
    dt = inp["dtype"]
    bsz, dim, L = inp["u"].shape
    N = inp["A"].shape[1]
    B = synth.widen(inp["B"][0:1], dt)
    C = synth.widen(inp["C"][0:1], dt)

    def run(k):
        sub = {key: synth.widen(inp[key][0:1, :k], dt) for key in ("u", "delta", "z")}
        t = time.perf_counter()
        oracle.s6_scan(sub["u"], sub["delta"], inp["A"][:k], B, C, inp["D"][:k], sub["z"], nthreads=nth)
        return time.perf_counter() - t

    k = min(dim, max(nth, 64))
    el = run(k)
    while el < target_s / 4 and k < dim:
        k = min(dim, int(k * max(2.0, min(8.0, target_s / max(el, 1e-3)))))
        el = run(k)
    esize = 2 if dt == "bf16" else 4
    nbytes = s6_bytes(1, k, L, N, esize)
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": nth, "kind": "oracle",
            "sample": f"batch row 0, channels 0..{k - 1} of {dim}, all {L} tokens, d_state {N} "
                      f"({k * L} tokens-ch, fp64 sequential recurrence, {el:.2f} s wall)",
            "tokens_ch_per_s": k * L / el, "seconds": el}


def bench_decode(args):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["decode_mamba2p8b_bf16"]
    s = wl.shape
    bsz, dim, N, steps = s["batch"], s["d_inner"], s["d_state"], s["steps"]
    log(f"[bench] decode: generating {steps} tokens of inputs")
    init = synth.decode_initial(bsz, dim, N, seed=wl.seed)
    toks = [synth.decode_step(init, i, bsz, dim, N, dtype=wl.dtype, seed=wl.seed) for i in range(steps)]
    dev_toks = [{k: to_dev(t[k]) for k in ("u", "delta", "z", "B", "C")} for t in toks]
    A, D = to_dev(init["A"]), to_dev(init["D"])
    # 16 state buffers (16 x 21 MB > 256 MB Infinity Cache): step i uses
    # buffer i % 16, as 16 layers would, so state traffic reaches HBM.
    K = 16
    states = [to_dev(init["state"]) for _ in range(K)]
    ys = [torch.empty((bsz, dim), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    stream = torch.cuda.current_stream()

    def run_all(rotate):
        for i in range(steps):
            t = dev_toks[i]
            mssm.state_update(states[i % K] if rotate else states[0], t["u"], t["delta"], A, t["B"], t["C"], D,
                              t["z"], out=ys[i], stream=stream)

    res = {}
    for label, rot in (("cold_16_buffers", True), ("hot_single_buffer", False)):
        total, per = time_launches(lambda: run_all(rot), 3, 1, stream)
        per_step_ms = total / 3 / steps
        nb = decode_bytes(bsz, dim, N, 2)
        res[label] = dict(us_per_step_wall=per_step_ms * 1e3, GBs=nb / (per_step_ms * 1e-3) / 1e9)
    # kernel-only per-step time via events around single launches (cold set)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        t = dev_toks[i]
        evs[2 * i].record(stream)
        mssm.state_update(states[i % K], t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], out=ys[i], stream=stream)
        evs[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps)]
    nb = decode_bytes(bsz, dim, N, 2)
    res["cold_event_us_per_step"] = float(np.median(per)) * 1e3
    res["cold_event_GBs"] = nb / (np.median(per) * 1e-3) / 1e9
    res["bytes_per_step"] = nb
    res["workload"] = f"{wl.name}: batch {bsz}, d_inner {dim}, d_state {N}, bf16, {steps} tokens"
    return res


def bench_ssd(args):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = wl.shape
    inp = synth.ssd_inputs(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                           dtype=wl.dtype, seed=wl.seed)
    d = {k: to_dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    y = torch.empty_like(d["x"])
    need = mssm.ssd_workspace_size(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"],
                                   s["ngroups"], s["chunk"])
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.ssd_chunk(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=s["chunk"], out=y,
                       workspace=ws, stream=stream)

    total, per = time_launches(step, 20, 3, stream)
    ms = total / 20
    nb = ssd_bytes(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], 2)
    fl = ssd_flops(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], s["chunk"])
    return dict(workload=f"{wl.name}: batch 4, seqlen 4096, 32 heads x 64, d_state 128, chunk 256, bf16",
                us=ms * 1e3, GBs=nb / (ms * 1e-3) / 1e9, hbm_frac=nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                mfma_TFLOPs=fl / (ms * 1e-3) / 1e12,
                mfma_frac=fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                tokens_ch_per_s=s["batch"] * s["seqlen"] * s["nheads"] * s["headdim"] / (ms * 1e-3),
                algorithmic_bytes=nb, algorithmic_flops=fl)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the scan shards by batch/channel with no exchange; see DESIGN.md).", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_19_amd import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    wl = synth.WORKLOADS["s6_mamba1p4b_bf16"]
    r = bench_s6(args, wl)
    s = wl.shape
    tok = s["batch"] * s["seqlen"] * s["d_inner"]
    gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
    kern_gbs = r["bytes"] / (r["kern_ms"] * 1e-3) / 1e9
    elems = tok * s["d_state"]
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Mamba-shaped inputs, see DESIGN.md)",
        "config": {"workload": f"{wl.name}: S6 selective scan, batch {s['batch']}, d_inner {s['d_inner']}, "
                               f"seqlen {s['seqlen']}, d_state {s['d_state']}, bf16 in / fp32 state, "
                               f"z gate, D skip, h_final out",
                   "batch": s["batch"], "d_inner": s["d_inner"], "seqlen": s["seqlen"],
                   "d_state": s["d_state"]},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_ch_per_s": tok / (r["ms"] * 1e-3),
        "roofline": {"bound": "hbm", "achieved": round(kern_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(kern_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "s6_scan_kernel", "algorithmic_bytes_per_launch": r["bytes"],
                     "avg_launch_ms": round(r["kern_ms"], 5)},
        "alu": {"state_updates_per_s": elems / (r["kern_ms"] * 1e-3),
                "valu_lane_instr_per_update": 5,
                "valu_frac_if_exp_full_rate": elems * 5 / (r["kern_ms"] * 1e-3) / VALU_LANE_OPS},
    }
    if not args.no_parity:
        log("[bench] parity sample vs the fp64 oracle")
        out["parity_sample"] = parity_sample(r["inp"], r["y"], r["hf"])
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a sample)")
        out["cpu_baseline"] = cpu_baseline(r["inp"])
    if not args.no_secondary:
        try:
            out["secondary_decode"] = bench_decode(args)
        except Exception as e:  # reported, not hidden
            out["secondary_decode"] = {"error": repr(e)}
        try:
            out["secondary_ssd"] = bench_ssd(args)
        except Exception as e:
            out["secondary_ssd"] = {"error": repr(e)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
