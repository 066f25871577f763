#!/usr/bin/env python3
"""Benchmark of the selective state-space scan on one MI355X.

Headline: mssm_selective_scan_fwd on the Mamba-1.4B layer shape (batch 4,
d_inner 4096, seqlen 8192, d_state 16; u, delta, B, C, z in bf16; A, D fp32;
fp32 state; z gate, D skip, final state written), inputs resident in HBM.
A "step" is one call of the scan over that batch.  `value` is the effective
HBM bandwidth: algorithmic bytes (every input read once, every output
written once) divided by the time per step; also reported: tokens-ch/s
(batch*seqlen*d_inner per second), the roofline of the scan kernel, the
fp64 CPU oracle timed on the same workload, and the other entry points
(decode step at the Mamba-2.8B shape, Mamba-2 SSD) inside the same object.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
                    [--only s6,calib,s6c1,s6fused,s6zoh,s6bwd,decode,decode2,ssd,ssdf32,copy]

Prints exactly one JSON line on stdout; progress goes to stderr.  `--only`
restricts the run (for profiling); `calib` measures the copy / read
ceilings and VALU issue rates on the GPU at hand; `s6c1` times the scan at
the Mamba-130M layer shape (fp32); `ssdf32` the SSD at the Mamba-2 layer
shape with float32 storage (the general chunked kernel); `copy` times a
plain 1 GiB device copy, the reference used to scale the HBM byte counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan effective HBM GB/s (% of peak) + B·L·D_inner tokens-ch/s"
HBM_PEAK_GBS = 8000.0                  # MI355X HBM3E, 8 TB/s
WARM_MS = 100.0                        # wall-clock warm-up before each secondary timing
WARM_MS_HEADLINE = 300.0               # and before the headline timing
# fp32 vector peak: 157.3 TFLOP/s published = 78.6e12 lane-FMA/s (256 CUs x 4 SIMDs
# x 2.4 GHz x 32 fp32 lanes per SIMD per clock; the calibration probes reach
# 0.7-0.8 of it with plain v_fma_f32, no packed math).
FP32_FMA_LANE_PEAK = 157.3e12 / 2
VALU_LANE_SLOTS = 256 * 4 * 16 * 2.4e9           # the 16-lane figure, reported for comparison
# One S6 state element: v_mul (delta*A), v_exp_f32, v_mul (delta*u*B), v_fma (h),
# v_fma (y), counted as 7 flop (mul 1, exp 1, mul 1, fma 2, fma 2).  v_exp_f32
# issues at a quarter of the FMA rate (measured 0.29-0.33 of it) and does not
# overlap the FMAs (measured), so an element takes 4 + 4 = 8 FMA issue slots.
S6_SLOTS_PER_ELEM, S6_FLOP_PER_ELEM = 8, 7
S6_ALU_PEAK_TFLOPS = FP32_FMA_LANE_PEAK / S6_SLOTS_PER_ELEM * S6_FLOP_PER_ELEM / 1e12   # 68.8
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP32_PEAK_TFLOPS = 157.3          # dense fp32 matrix (v_mfma_f32_*_f32), published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def s6_bytes(batch, dim, L, N, esize, gate=True, skip=True, h0=False, final=True):
    """Algorithmic HBM bytes of one scan: u, delta, (z), y once each; B, C; A;
    (D); (h0); (h_final)."""
    per_tok = (3 + (1 if gate else 0)) * batch * dim * L * esize
    bc = 2 * batch * N * L * esize
    small = dim * N * 4 + (dim * 4 if skip else 0)
    st = batch * dim * N * 4 * ((1 if h0 else 0) + (1 if final else 0))
    return per_tok + bc + small + st


def decode_bytes(batch, dim, N, esize, gate=True, skip=True):
    """State read + write; u, delta, (z), y; B, C; A; (D)."""
    return (2 * batch * dim * N * 4 + (3 + (1 if gate else 0)) * batch * dim * esize
            + 2 * batch * N * esize + dim * N * 4 + (dim * 4 if skip else 0))


def decode2_bytes(batch, H, P, N, G, esize, gate=True, skip=True):
    """Mamba-2 decode step: state read + write; x, (z), y; dt; B, C; A, (D)."""
    return (2 * batch * H * P * N * 4 + (2 + (1 if gate else 0)) * batch * H * P * esize + batch * H * esize
            + 2 * batch * G * N * esize + H * 4 + (H * 4 if skip else 0))


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


def profile_fields(profile):
    """The machine-readable block of a kernel's committed rocprofv3 summary
    under profiles/ (traffic per launch, and for some kernels busy shares of
    the VALU or MFMA units), or None when the summary is missing or the
    kernel's sources changed after the counters were taken."""
    try:
        text = open(os.path.join(ROOT, "profiles", profile)).read()
    except OSError:
        return None
    kv = {}
    block = text.partition("## Machine-readable")[2]
    for line in block.splitlines():
        k, sep, v = line.partition(": ")
        if sep:
            kv[k.strip()] = v.strip()
    if "kernel_sources" not in kv or "kernel_source_sha256" not in kv:
        return None
    h = hashlib.sha256()
    for f in kv["kernel_sources"].split():
        try:
            h.update(open(os.path.join(ROOT, "selective_state_space_19_amd", "csrc", f), "rb").read())
        except OSError:
            return None
    return kv if h.hexdigest() == kv["kernel_source_sha256"] else None


def profiled_traffic(profile):
    """HBM bytes per launch of a kernel from its summary under profiles/
    (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter reads for a
    plain 1 GiB copy); None when missing or stale (see profile_fields)."""
    kv = profile_fields(profile)
    return int(kv["traffic_bytes_per_launch"]) if kv and "traffic_bytes_per_launch" in kv else None


def profiled_counters(profile, keys):
    """Counter-derived figures recorded in a kernel's summary (floats), or
    None when missing or stale."""
    kv = profile_fields(profile)
    if not kv:
        return None
    out = {k: float(kv[k]) for k in keys if k in kv}
    return dict(out, source="profiles/" + profile) if out else None


def to_dev(a):
    import torch
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def time_launches(fn, steps, warmup, stream, wall=None, warm_ms=0.0):
    """Warm up (`warmup` calls, then more until `warm_ms` of wall time has
    passed: the GPU's clocks ramp up over tens of milliseconds of load), then
    time `steps` calls with HIP events on `stream` (the stream the kernels are
    launched on), bracketed by device synchronisation.  Returns (total ms,
    per-call ms); if `wall` is a list, the host wall-clock ms of the same
    bracketed region is appended to it."""
    import torch
    t_w = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t_w) * 1e3 < warm_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    if wall is not None:
        wall.append((time.perf_counter() - t0) * 1e3)
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]), per


# --------------------------------------------------------------------------
# S6 scan (headline)
# --------------------------------------------------------------------------
def bench_s6(args):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["s6_mamba1p4b_bf16"]
    s = wl.shape
    log(f"[bench] s6: generating {wl.name} inputs {s} ({wl.dtype})")
    t0 = time.time()
    inp = synth.s6_inputs(**s, dtype=wl.dtype, seed=wl.seed)
    log(f"[bench] s6: generated in {time.time() - t0:.1f}s; uploading")
    d = {k: to_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    y = torch.empty_like(d["u"])
    hf = torch.empty((s["batch"], s["d_inner"], s["d_state"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"],
                            out=y, h_final=hf, stream=stream)

    log(f"[bench] s6: timing {args.steps} steps after {args.warmup} warm-up")
    torch.cuda.synchronize()
    wall = []
    total_ms, per = time_launches(step, args.steps, args.warmup, stream, wall, warm_ms=WARM_MS_HEADLINE)
    nbytes = s6_bytes(s["batch"], s["d_inner"], s["seqlen"], s["d_state"], 2 if wl.dtype == "bf16" else 4)
    return dict(wl=wl, inp=inp, y=y, hf=hf, ms=wall[0] / args.steps, event_ms=total_ms / args.steps, per=per,
                kern_ms=float(np.mean(per)), bytes=nbytes)


def bench_s6fused(args):
    """The scan with its front end fused in, same layer shape as the headline."""
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["s6fused_mamba1p4b_bf16"]
    s = wl.shape
    log(f"[bench] s6 fused: generating {wl.name} inputs")
    inp = synth.s6_fused_inputs(**s, dtype=wl.dtype, seed=wl.seed)
    d = {k: to_dev(inp[k]) for k in ("x", "conv_w", "conv_b", "delta_raw", "delta_bias", "A", "B", "C", "D", "z")}
    y = torch.empty_like(d["x"])
    hf = torch.empty((s["batch"], s["d_inner"], s["d_state"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.selective_scan_fused(d["x"], d["conv_w"], d["delta_raw"], d["A"], d["B"], d["C"], d["D"], d["z"],
                                  conv_b=d["conv_b"], delta_bias=d["delta_bias"], out=y, h_final=hf, stream=stream)

    total, per = time_launches(step, max(5, args.steps // 2), 2, stream, warm_ms=WARM_MS)
    ms = total / max(5, args.steps // 2)
    nb = s6_bytes(s["batch"], s["d_inner"], s["seqlen"], s["d_state"], 2) + s["d_inner"] * (s["d_conv"] + 2) * 4
    tok = s["batch"] * s["d_inner"] * s["seqlen"]
    return {"workload": f"{wl.name}: batch {s['batch']}, d_inner {s['d_inner']}, seqlen {s['seqlen']}, "
                        f"d_state {s['d_state']}, d_conv {s['d_conv']}, bf16",
            "us": ms * 1e3, "GBs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_ch_per_s": tok / (ms * 1e-3), "algorithmic_bytes": nb,
            "traffic_bytes_per_launch": profiled_traffic("s6_scan_fused_mamba1p4b_bf16.md")}


def bench_s6zoh(args):
    """The scan with the zero-order-hold input term, same layer shape as the headline."""
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["s6_mamba1p4b_bf16"]
    s = wl.shape
    log("[bench] s6 zoh: generating inputs")
    inp = synth.s6_inputs(**s, dtype=wl.dtype, seed=wl.seed)
    d = {k: to_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    y = torch.empty_like(d["u"])
    hf = torch.empty((s["batch"], s["d_inner"], s["d_state"]), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"],
                            out=y, h_final=hf, stream=stream, zoh=True)

    steps = max(5, args.steps // 2)
    total, _ = time_launches(step, steps, 2, stream, warm_ms=WARM_MS)
    ms = total / steps
    nb = s6_bytes(s["batch"], s["d_inner"], s["seqlen"], s["d_state"], 2)
    tok = s["batch"] * s["d_inner"] * s["seqlen"]
    return {"workload": f"{wl.name} with the zero-order-hold input term: batch {s['batch']}, d_inner {s['d_inner']}, "
                        f"seqlen {s['seqlen']}, d_state {s['d_state']}, bf16",
            "us": ms * 1e3, "GBs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "tokens_ch_per_s": tok / (ms * 1e-3), "algorithmic_bytes": nb,
            "traffic_bytes_per_launch": profiled_traffic("s6_scan_zoh_mamba1p4b_bf16.md")}


def bench_s6bwd(args):
    """Backward of the scan at the headline layer shape (h0 and final-state
    gradient included)."""
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["s6_mamba1p4b_bf16"]
    s = wl.shape
    log("[bench] s6 backward: generating inputs")
    inp = synth.s6_inputs(**s, dtype=wl.dtype, seed=wl.seed, init_state=True)
    d = {k: to_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    rng = np.random.default_rng(0)
    dout = to_dev(synth.round_to(rng.standard_normal(inp["u"].shape), wl.dtype))
    dhT = to_dev(rng.standard_normal(inp["h0"].shape).astype(np.float32))
    ws = torch.empty(mssm.selective_scan_bwd_workspace_size(s["batch"], s["d_inner"], s["seqlen"], s["d_state"]),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], dout, d["D"], d["z"], d["h0"], dhT,
                                workspace=ws, stream=stream)

    steps = max(3, args.steps // 4)
    total, _ = time_launches(step, steps, 1, stream, warm_ms=WARM_MS)
    ms = total / steps
    # The training pair: the forward that keeps the chunk-start states in the
    # workspace, and the backward that starts from them.
    y = torch.empty_like(d["u"])

    def fwd_save():
        mssm.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], d["h0"], out=y,
                            save_workspace=ws, stream=stream)

    def bwd_saved():
        mssm.selective_scan_bwd(d["u"], d["delta"], d["A"], d["B"], d["C"], dout, d["D"], d["z"], d["h0"], dhT,
                                workspace=ws, saved=True, stream=stream)

    fwd_save()
    total_s, _ = time_launches(bwd_saved, steps, 1, stream, warm_ms=WARM_MS)
    total_f, _ = time_launches(fwd_save, steps, 1, stream, warm_ms=WARM_MS)
    B, D, L, N = s["batch"], s["d_inner"], s["seqlen"], s["d_state"]
    # read u, delta, z, dout (u, delta twice: the states-only forward reads them
    # too); write du, ddelta, dz; dB, dC; the states and partials written and read
    nb = (6 + 3) * B * D * L * 2 + 2 * B * N * L * (2 + 4) + 2 * ws.numel()
    return {"workload": f"{wl.name} backward: batch {B}, d_inner {D}, seqlen {L}, d_state {N}, bf16, "
                        "gate, skip, h0 and final-state gradient",
            "us": ms * 1e3, "us_from_saved_states": total_s / steps * 1e3,
            "us_forward_saving_states": total_f / steps * 1e3,
            "tokens_ch_per_s": B * D * L / (ms * 1e-3), "bytes_moved_estimate": nb,
            "GBs_estimate": nb / (ms * 1e-3) / 1e9, "workspace_bytes": ws.numel(),
            # the plain call: the forward kernel writing the chunk-start states
            # only, the backward kernel from them, the dB / dC block sums
            "traffic_bytes_per_call": {
                "s6_scan_kernel, states only": profiled_traffic("s6_scan_states_mamba1p4b_bf16.md"),
                "s6_scan_bwd_kernel": profiled_traffic("s6_scan_bwd_mamba1p4b_bf16.md"),
                "s6_bwd_reduce_bc_kernel": profiled_traffic("s6_bwd_reduce_bc_mamba1p4b_bf16.md")},
            "traffic_bytes_saved_pair": {
                "s6_scan_kernel saving states": profiled_traffic("s6_scan_fwd_save_mamba1p4b_bf16.md"),
                "s6_scan_bwd_kernel": profiled_traffic("s6_scan_bwd_mamba1p4b_bf16.md")}}


def bench_s6_130m(args):
    """The scan at the Mamba-130M layer shape in fp32 (batch 8, d_inner 1536,
    seqlen 2048, d_state 16).  Two input sets (2 x 405 MB, above the 256 MB
    Infinity Cache) alternate, so every call streams from HBM."""
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["s6_mamba130m_f32"]
    s = wl.shape
    log(f"[bench] s6 130m: generating {wl.name} inputs")
    inp = synth.s6_inputs(**s, dtype=wl.dtype, seed=wl.seed)
    sets = []
    for _ in range(2):
        d = {k: to_dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z")}
        d["y"] = torch.empty_like(d["u"])
        d["hf"] = torch.empty((s["batch"], s["d_inner"], s["d_state"]), dtype=torch.float32, device="cuda")
        sets.append(d)
    stream = torch.cuda.current_stream()
    it = [0]

    def step():
        d = sets[it[0] & 1]
        it[0] += 1
        mssm.selective_scan(d["u"], d["delta"], d["A"], d["B"], d["C"], d["D"], d["z"], out=d["y"], h_final=d["hf"],
                            stream=stream)

    steps = max(10, args.steps)
    total, _ = time_launches(step, steps, 4, stream, warm_ms=WARM_MS)
    ms = total / steps
    nb = s6_bytes(s["batch"], s["d_inner"], s["seqlen"], s["d_state"], 4)
    tok = s["batch"] * s["d_inner"] * s["seqlen"]
    elems = tok * s["d_state"]
    alu = elems * S6_FLOP_PER_ELEM / (ms * 1e-3) / 1e12
    return {"workload": f"{wl.name}: batch {s['batch']}, d_inner {s['d_inner']}, seqlen {s['seqlen']}, "
                        f"d_state {s['d_state']}, fp32, z gate, D skip, h_final out; 2 input sets alternating",
            "us": ms * 1e3, "GBs": nb / (ms * 1e-3) / 1e9, "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "alu_TFLOPs": alu, "alu_frac": alu / S6_ALU_PEAK_TFLOPS,
            "tokens_ch_per_s": tok / (ms * 1e-3), "algorithmic_bytes": nb,
            "workgroups": s["batch"] * ((s["d_inner"] + 63) // 64),
            "traffic_bytes_per_launch": profiled_traffic("s6_scan_mamba130m_f32.md"),
            "counters": profiled_counters("s6_scan_mamba130m_f32.md", ("valu_busy_pct", "valu_instr_per_element"))}


def _calib_lib():
    import ctypes
    path = os.path.join(ROOT, "selective_state_space_19_amd", "libmssm_calib.so")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mssm_calib_copy.argtypes = [vp, vp, i64, i32, vp]
    lib.mssm_calib_read.argtypes = [vp, vp, i64, i32, vp]
    lib.mssm_calib_valu.argtypes = [vp, vp, i32, i32, i32, ctypes.c_float, vp]
    for f in (lib.mssm_calib_copy, lib.mssm_calib_read, lib.mssm_calib_valu):
        f.restype = i32
    return lib


def bench_calib(args):
    """Ceilings measured on this GPU in the same run (libmssm_calib.so):
    a streaming copy and a streaming read of 1 GiB (HBM), a copy of 21 MB
    over 16 rotating buffer pairs (the decode step's state size, cold), and
    the VALU issue rates of v_fma_f32, v_exp_f32 and of the scan's own
    per-element instruction mix."""
    import torch
    lib = _calib_lib()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    res = {}

    def chk(rc):
        if rc != 0:
            raise RuntimeError(f"calibration launch failed: {rc}")

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    blocks = 256 * 16
    total, _ = time_launches(lambda: chk(lib.mssm_calib_copy(a.data_ptr(), b.data_ptr(), n, blocks, sh)), 10, 3,
                             stream, warm_ms=WARM_MS)
    res["copy_1GiB_GBs"] = 2 * n / (total / 10 * 1e-3) / 1e9
    sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    total, _ = time_launches(lambda: chk(lib.mssm_calib_read(a.data_ptr(), sink.data_ptr(), n, blocks, sh)), 10, 3,
                             stream, warm_ms=WARM_MS)
    res["read_1GiB_GBs"] = n / (total / 10 * 1e-3) / 1e9
    del a, b
    m = 64 * 5120 * 16 * 4
    pairs = [(torch.ones(m // 4, dtype=torch.float32, device="cuda"), torch.empty(m // 4, dtype=torch.float32,
                                                                                  device="cuda")) for _ in range(16)]
    it = [0]

    def small():
        src, dst = pairs[it[0] % 16]
        it[0] += 1
        chk(lib.mssm_calib_copy(src.data_ptr(), dst.data_ptr(), m, 256 * 8, sh))

    total, _ = time_launches(small, 64, 16, stream, warm_ms=WARM_MS)
    res["copy_21MB_16_rotating_GBs"] = 2 * m / (total / 64 * 1e-3) / 1e9
    del pairs
    out = torch.empty(256 * 8 * 256, dtype=torch.float32, device="cuda")
    lanes = 256 * 8 * 256
    uni = torch.tensor([0.5, 0.7, -0.3, 0.2, 0.9, 0, 0, 0], dtype=torch.float32, device="cuda")
    secs = {}
    # (mode, iterations, workgroups): 2048 workgroups are 8 waves per SIMD, 512 are 2
    for key, mode, iters, blocks in ((0, 0, 2048, 2048), (1, 1, 1024, 2048), (2, 2, 256, 2048), (3, 3, 512, 2048),
                                     (7, 7, 256, 2048), ("2w2", 2, 256, 512)):
        total, _ = time_launches(lambda: chk(lib.mssm_calib_valu(out.data_ptr(), uni.data_ptr(), blocks, iters, mode,
                                                                 0.5, sh)), 5, 2, stream, warm_ms=WARM_MS)
        secs[key] = (total / 5 * 1e-3, iters, blocks)
    rate = lambda key, per: secs[key][2] * 256 * secs[key][1] * per / secs[key][0]  # noqa: E731
    fma, exp = rate(0, 16), rate(1, 16)
    res["fma_lane_instr_per_s"] = fma
    res["fma_vs_published_fp32_peak"] = fma / FP32_FMA_LANE_PEAK
    res["exp_lane_instr_per_s"] = exp
    res["exp_rate_vs_fma"] = exp / fma
    res["s6_mix_elements_per_s"] = rate(2, 32)
    res["s6_mix_fma_slots_per_element"] = fma / res["s6_mix_elements_per_s"]
    res["s6_mix_scalar_bc_elements_per_s"] = rate(7, 32)
    res["s6_mix_2_waves_per_simd_elements_per_s"] = rate("2w2", 32)
    t3, it3, _ = secs[3]
    res["exp16_fma64_us"] = t3 * 1e6
    res["exp16_fma64_us_if_added"] = lanes * it3 * (16 / exp + 64 / fma) * 1e6
    res["exp16_fma64_us_if_overlapped"] = lanes * it3 * max(16 / exp, 64 / fma) * 1e6
    res["note"] = ("2048 workgroups x 256 threads (8 waves per SIMD) unless marked; the S6 mix is the scan kernel's "
                   "own group layout (16 tokens x 2 states per lane)")
    return res


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


def cpu_baseline(inp, budget_s=30.0):
    """The fp64 oracle, as it stands, on the benchmarked workload: whole batch
    rows, as many as fit in about budget_s seconds of wall time (all of them
    on a host with enough cores)."""
    import oracle
    from selective_state_space_19_amd import synth
    nth = oracle.default_threads()
    dt = inp["dtype"]
    bsz, dim, L = inp["u"].shape
    N = inp["A"].shape[1]
    used, rows = 0.0, 0
    for b in range(bsz):
        sub = {k: synth.widen(inp[k][b:b + 1], dt) for k in ("u", "delta", "z", "B", "C")}
        t = time.perf_counter()
        oracle.s6_scan(sub["u"], sub["delta"], inp["A"], sub["B"], sub["C"], inp["D"], sub["z"], nthreads=nth)
        used += time.perf_counter() - t
        rows += 1
        if used * (rows + 1) / rows > budget_s:
            break
    nbytes = s6_bytes(rows, dim, L, N, 2 if dt == "bf16" else 4)
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.partition(":")[2].strip()
                break
    except OSError:
        pass
    return {"value": nbytes / used / 1e9, "unit": "GB/s", "cores": nth, "kind": "oracle", "cpu_model": model,
            "sample": f"{rows} of {bsz} batch rows of the benchmarked workload ({rows * dim} channels x "
                      f"{L} tokens, d_state {N}), fp64 sequential recurrence, {used:.2f} s wall",
            "tokens_ch_per_s": rows * dim * L / used, "seconds": used,
            "single_thread": cpu_single_thread()}


def cpu_single_thread():
    """The oracle on one thread: the whole tiny workload (1 x 32 x 64,
    N 16, fp32) and one batch row of the Mamba-130M layer shape (1536
    channels x 2048 tokens, N 16, fp32)."""
    import oracle
    from selective_state_space_19_amd import synth
    res = {}
    for name, rows in (("s6_tiny_f32", None), ("s6_mamba130m_f32", 1)):
        wl = synth.WORKLOADS[name]
        shape = dict(wl.shape)
        if rows is not None:
            shape["batch"] = rows
        inp = synth.s6_inputs(**shape, dtype=wl.dtype, seed=wl.seed)
        w = {k: synth.widen(inp[k], "f32") for k in ("u", "delta", "A", "B", "C", "D", "z")}
        reps = 20 if rows is None else 1
        t = time.perf_counter()
        for _ in range(reps):
            oracle.s6_scan(w["u"], w["delta"], w["A"], w["B"], w["C"], w["D"], w["z"], nthreads=1)
        sec = (time.perf_counter() - t) / reps
        tok = shape["batch"] * shape["d_inner"] * shape["seqlen"]
        res[name] = {"sample": "whole workload" if rows is None else f"{rows} of {wl.shape['batch']} batch rows",
                     "seconds": sec, "tokens_ch_per_s": tok / sec,
                     "GBs": s6_bytes(shape["batch"], shape["d_inner"], shape["seqlen"], shape["d_state"], 4,
                                     final=False) / sec / 1e9}
    return res


# --------------------------------------------------------------------------
# Decode (Mamba-2.8B shape, 256 tokens)
# --------------------------------------------------------------------------
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
    dtk = [{k: to_dev(t[k]) for k in ("u", "delta", "z", "B", "C")} for t in toks]
    A, D = to_dev(init["A"]), to_dev(init["D"])
    # 16 state buffers (16 x 21 MB > the 256 MB Infinity Cache): token i uses
    # buffer i % 16, as 16 layers would, so the state traffic reaches HBM.
    K = 16
    states = [to_dev(init["state"]) for _ in range(K)]
    ys = [torch.empty((bsz, dim), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    stream = torch.cuda.current_stream()
    nb = decode_bytes(bsz, dim, N, 2)

    def run_all(rotate):
        for i in range(steps):
            t = dtk[i]
            mssm.state_update(states[i % K] if rotate else states[0], t["u"], t["delta"], A, t["B"], t["C"], D,
                              t["z"], out=ys[i], stream=stream)

    res = {"workload": f"{wl.name}: batch {bsz}, d_inner {dim}, d_state {N}, bf16, {steps} tokens",
           "bytes_per_step": nb, "traffic_bytes_per_launch": profiled_traffic("state_update_mamba2p8b_decode.md")}
    for label, rot in (("cold_16_buffers", True), ("hot_single_buffer", False)):
        total, _ = time_launches(lambda: run_all(rot), 3, 1, stream, warm_ms=WARM_MS)
        us = total / 3 / steps * 1e3
        res[label + "_launches"] = {"us_per_step": us, "GBs": nb / (us * 1e-6) / 1e9}
    # The same 256 tokens captured in one HIP graph (launch overhead removed).
    try:
        for label, rot in (("cold_16_buffers", True), ("hot_single_buffer", False)):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                run_all(rot)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                for i in range(steps):
                    t = dtk[i]
                    mssm.state_update(states[i % K] if rot else states[0], t["u"], t["delta"], A, t["B"], t["C"],
                                      D, t["z"], out=ys[i])
            total, _ = time_launches(g.replay, 5, 2, torch.cuda.current_stream(), warm_ms=WARM_MS)
            us = total / 5 / steps * 1e3
            res[label + "_graph"] = {"us_per_step": us, "GBs": nb / (us * 1e-6) / 1e9,
                                     "hbm_frac": nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    except Exception as e:  # reported, not hidden
        res["graph_error"] = repr(e)
    res["tokens_ch_per_s_cold_graph"] = (bsz * dim / (res["cold_16_buffers_graph"]["us_per_step"] * 1e-6)
                                         if "cold_16_buffers_graph" in res else None)
    return res


# --------------------------------------------------------------------------
# Mamba-2 decode (one SSD token)
# --------------------------------------------------------------------------
def bench_decode2(args):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["decode_mamba2_bf16"]
    s = wl.shape
    bsz, H, P, N, G, steps = s["batch"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], s["steps"]
    log(f"[bench] mamba2 decode: generating {steps} tokens of inputs")
    init = synth.mamba2_decode_initial(bsz, H, P, N, seed=wl.seed)
    toks = [synth.mamba2_decode_step(init, i, bsz, H, P, N, ngroups=G, dtype=wl.dtype, seed=wl.seed)
            for i in range(steps)]
    dtk = [{k: to_dev(t[k]) for k in ("x", "dt", "z", "B", "C")} for t in toks]
    A, D = to_dev(init["A"]), to_dev(init["D"])
    # 8 state buffers (8 x 67 MB > the 256 MB Infinity Cache), token i uses i % 8.
    K = 8
    states = [to_dev(init["state"]) for _ in range(K)]
    ys = [torch.empty((bsz, H, P), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]
    stream = torch.cuda.current_stream()
    nb = decode2_bytes(bsz, H, P, N, G, 2)

    def run_all(rot, strm=None):
        for i in range(steps):
            t = dtk[i]
            mssm.ssd_state_update(states[i % K] if rot else states[0], t["x"], t["dt"], A, t["B"], t["C"], D, t["z"],
                                  out=ys[i], stream=strm)

    res = {"workload": f"{wl.name}: batch {bsz}, {H} heads x {P}, d_state {N}, ngroups {G}, bf16, {steps} tokens",
           "bytes_per_step": nb, "traffic_bytes_per_launch": profiled_traffic("ssd_state_update_mamba2_decode.md")}
    for label, rot in (("cold_8_buffers", True), ("hot_single_buffer", False)):
        total, _ = time_launches(lambda: run_all(rot, stream), 3, 1, stream, warm_ms=WARM_MS)
        us = total / 3 / steps * 1e3
        res[label + "_launches"] = {"us_per_step": us, "GBs": nb / (us * 1e-6) / 1e9}
    try:
        for label, rot in (("cold_8_buffers", True), ("hot_single_buffer", False)):
            g = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                run_all(rot)
            torch.cuda.current_stream().wait_stream(side)
            with torch.cuda.graph(g):
                run_all(rot)
            total, _ = time_launches(g.replay, 5, 2, torch.cuda.current_stream(), warm_ms=WARM_MS)
            us = total / 5 / steps * 1e3
            res[label + "_graph"] = {"us_per_step": us, "GBs": nb / (us * 1e-6) / 1e9,
                                     "hbm_frac": nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}
    except Exception as e:  # reported, not hidden
        res["graph_error"] = repr(e)
    res["tokens_ch_per_s_cold_graph"] = (bsz * H * P / (res["cold_8_buffers_graph"]["us_per_step"] * 1e-6)
                                         if "cold_8_buffers_graph" in res else None)
    return res


# --------------------------------------------------------------------------
# Mamba-2 SSD
# --------------------------------------------------------------------------
def bench_ssd(args):
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = wl.shape
    log("[bench] ssd: generating inputs")
    inp = synth.ssd_inputs(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                           dtype=wl.dtype, seed=wl.seed)
    need = mssm.ssd_workspace_size(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"],
                                   s["ngroups"], s["chunk"])
    # Cold: K input sets (x, dt, B, C, y and the workspace each, about 160 MB)
    # used in turn, so a call's data were last touched K - 1 calls (about
    # 480 MB of traffic) earlier, beyond the 256 MB Infinity Cache.
    K = 4
    sets = []
    for _ in range(K):
        d = {k: to_dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D")}
        d["y"] = torch.empty_like(d["x"])
        d["ws"] = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        sets.append(d)
    stream = torch.cuda.current_stream()
    it = [0]

    def step(chunk=s["chunk"], rotate=True):
        d = sets[it[0] % K] if rotate else sets[0]
        it[0] += 1
        mssm.ssd_chunk(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=chunk, out=d["y"],
                       workspace=d["ws"], stream=stream)

    total, per = time_launches(step, 20, 4, stream, warm_ms=WARM_MS)
    ms = total / 20
    # the dense-block count: every 16 x 16 MFMA block a chunked form would
    # issue, causal blocks in full (the pages' chunked form, not this
    # kernel's triangle skipping); reported beside, labelled
    nc = (s["seqlen"] + s["chunk"] - 1) // s["chunk"]
    Q, Hh, P, N, G = s["chunk"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"]
    dense = 2 * s["batch"] * nc * (G * Q * Q * N + Hh * Q * Q * P + 2 * Hh * Q * N * P + Hh * P * N)
    total_hot, _ = time_launches(lambda: step(rotate=False), 20, 4, stream, warm_ms=WARM_MS)
    # The chunk length is a tile size: the result is the same up to rounding.
    # The same call with 64-token chunks, for comparison (not the workload).
    total64, _ = time_launches(lambda: step(chunk=64), 20, 4, stream, warm_ms=WARM_MS)
    nb = ssd_bytes(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], 2)
    fl = ssd_flops(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], s["chunk"])
    return dict(workload=f"{wl.name}: batch 4, seqlen 4096, 32 heads x 64, d_state 128, ngroups 1, chunk 256, bf16; "
                         f"{K} input sets in turn (cold)",
                us_same_call_chunk64=total64 / 20 * 1e3, us_hot_one_input_set=total_hot / 20 * 1e3,
                us=ms * 1e3, GBs=nb / (ms * 1e-3) / 1e9, hbm_frac=nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                mfma_TFLOPs=fl / (ms * 1e-3) / 1e12, mfma_frac=fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                tokens_ch_per_s=s["batch"] * s["seqlen"] * s["nheads"] * s["headdim"] / (ms * 1e-3),
                us_median=float(np.median(per)) * 1e3, us_min=float(np.min(per)) * 1e3,
                dense_block_flops=dense, mfma_TFLOPs_dense_blocks=dense / (ms * 1e-3) / 1e12,
                mfma_busy=profiled_counters("ssd_main_mamba2_chunk256.md", ("mfma_busy_pct",)),
                algorithmic_bytes=nb, algorithmic_flops=fl, workspace_bytes=need,
                traffic_bytes_per_call={"ssd_prep_kernel": profiled_traffic("ssd_prep_mamba2_chunk256.md"),
                                        "ssd_main_kernel": profiled_traffic("ssd_main_mamba2_chunk256.md")})


def bench_ssd_f32(args):
    """The SSD at the Mamba-2 layer shape with float32 storage, which runs on
    the general chunked kernels (fp32 matrix cores: the chunk scores, then
    the two-role walk; the bf16 MFMA kernels take bf16).  One input
    set (x and y 134 MB each, with dt, B, C about 290 MB: beyond the 256 MB
    Infinity Cache)."""
    import torch
    import selective_state_space_19_amd as mssm
    from selective_state_space_19_amd import synth
    wl = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = wl.shape
    log("[bench] ssd fp32: generating inputs")
    inp = synth.ssd_inputs(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                           dtype="f32", seed=wl.seed)
    d = {k: to_dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D")}
    y = torch.empty_like(d["x"])
    need = mssm.ssd_workspace_size(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                                   s["chunk"])
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step():
        mssm.ssd_chunk(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=s["chunk"], out=y, workspace=ws,
                       stream=stream)

    total, _ = time_launches(step, 10, 2, stream, warm_ms=WARM_MS)
    ms = total / 10
    nb = ssd_bytes(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], 4)
    # the flops of the form these kernels compute: 32-token chunks
    fl = ssd_flops(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"], 32)
    return dict(workload=f"{wl.name} shape with float32 storage: batch 4, seqlen 4096, 32 heads x 64, d_state 128, "
                         f"ngroups 1 (general chunked kernels, fp32 MFMA, 32-token chunks)",
                flops_32_token_chunks=fl, mfma_TFLOPs=fl / (ms * 1e-3) / 1e12,
                mfma_frac_fp32_matrix=fl / (ms * 1e-3) / 1e12 / MFMA_FP32_PEAK_TFLOPS,
                us=ms * 1e3, GBs=nb / (ms * 1e-3) / 1e9, hbm_frac=nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                tokens_ch_per_s=s["batch"] * s["seqlen"] * s["nheads"] * s["headdim"] / (ms * 1e-3),
                algorithmic_bytes=nb,
                traffic_bytes_per_call={"ssd_general_scores_kernel": profiled_traffic("ssd_general_scores_mamba2_f32.md"),
                                        "ssd_general_roles_kernel": profiled_traffic("ssd_general_mamba2_f32.md")},
                mfma_busy=profiled_counters("ssd_general_mamba2_f32.md", ("mfma_busy_pct",)))


def bench_copy(args):
    """A plain 1 GiB device-to-device copy: the reference for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    stream = torch.cuda.current_stream()
    total, _ = time_launches(lambda: b.copy_(a), 5, 2, stream)
    ms = total / 5
    return {"bytes_read": n, "bytes_written": n, "ms": ms, "GBs": 2 * n / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--only", default="s6,calib,s6c1,s6fused,s6zoh,s6bwd,decode,decode2,ssd,ssdf32")
    ap.add_argument("--warm-ms", type=float, default=None,
                    help="wall-clock warm-up before each timing (default: 300 ms headline, 100 ms the others); "
                         "0 for profiling runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the scan shards by batch / channel with no exchange).", file=sys.stderr)
        sys.exit(2)
    parts = set(args.only.split(","))
    if args.warm_ms is not None:
        global WARM_MS, WARM_MS_HEADLINE
        WARM_MS = WARM_MS_HEADLINE = args.warm_ms

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    out = {}
    if "s6" in parts:
        r = bench_s6(args)
        s = r["wl"].shape
        tok = s["batch"] * s["seqlen"] * s["d_inner"]
        elems = tok * s["d_state"]
        gbs = r["bytes"] / (r["ms"] * 1e-3) / 1e9
        kern_s = r["kern_ms"] * 1e-3
        alu_tflops = elems * S6_FLOP_PER_ELEM / kern_s / 1e12
        out.update({
            "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(r["ms"], 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded Mamba-shaped inputs)",
            "config": {"workload": f"{r['wl'].name}: S6 selective scan, batch {s['batch']}, d_inner {s['d_inner']}, "
                                   f"seqlen {s['seqlen']}, d_state {s['d_state']}, bf16 in / fp32 state, z gate, "
                                   f"D skip, h_final out",
                       "batch": s["batch"], "d_inner": s["d_inner"], "seqlen": s["seqlen"], "d_state": s["d_state"]},
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "tokens_ch_per_s": tok / (r["ms"] * 1e-3),
            "event_ms_per_step": round(r["event_ms"], 5),
            "event_us_median": round(float(np.median(r["per"])) * 1e3, 2),
            "event_us_min": round(float(np.min(r["per"])) * 1e3, 2),
            # The scan is bound by VALU issue, not HBM (counters: VALU busy
            # ~92%, HBM ~29%): 8 FMA issue slots per state element at the
            # published fp32 rate (218 us here) outweigh its bytes (135 us at
            # 8 TB/s).  Peak = 78.6e12 FMA slots/s / 8 slots per element x 7 flop.
            "roofline": {"bound": "alu", "achieved": round(alu_tflops, 3), "peak": round(S6_ALU_PEAK_TFLOPS, 3),
                         "unit": "TFLOP/s", "frac": round(alu_tflops / S6_ALU_PEAK_TFLOPS, 4),
                         "traffic": profiled_traffic("s6_scan_mamba1p4b_bf16.md"),
                         "kernel": "s6_scan_kernel", "avg_launch_ms": round(r["kern_ms"], 5),
                         "state_elements_per_launch": elems, "flop_per_element": S6_FLOP_PER_ELEM,
                         "issue_slots_per_element": S6_SLOTS_PER_ELEM,
                         "counters": profiled_counters("s6_scan_mamba1p4b_bf16.md",
                                                       ("valu_busy_pct", "valu_instr_per_element",
                                                        "transcendental_per_element", "issue_slots_per_element"))},
            "roofline_hbm": {"achieved": round(r["bytes"] / kern_s / 1e9, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(r["bytes"] / kern_s / 1e9 / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes_per_launch": r["bytes"]},
        })
        if not args.no_parity:
            log("[bench] s6: parity sample vs the fp64 oracle")
            out["parity_sample"] = parity_sample(r["inp"], r["y"], r["hf"])
        if not args.no_cpu_baseline:
            log("[bench] s6: cpu baseline (the oracle on the same workload)")
            out["cpu_baseline"] = cpu_baseline(r["inp"])
            out["cpu_baseline"]["gpu_over_oracle"] = gbs / out["cpu_baseline"]["value"]
        del r
    if "calib" in parts:
        try:
            out["calibration"] = bench_calib(args)
        except Exception as e:  # reported, not hidden
            out["calibration"] = {"error": repr(e)}
    if "s6c1" in parts:
        try:
            out["secondary_s6_mamba130m_f32"] = bench_s6_130m(args)
        except Exception as e:  # reported, not hidden
            out["secondary_s6_mamba130m_f32"] = {"error": repr(e)}
    if "s6bwd" in parts:
        try:
            out["secondary_s6_backward"] = bench_s6bwd(args)
        except Exception as e:  # reported, not hidden
            out["secondary_s6_backward"] = {"error": repr(e)}
    if "s6zoh" in parts:
        try:
            out["secondary_s6_zoh"] = bench_s6zoh(args)
        except Exception as e:  # reported, not hidden
            out["secondary_s6_zoh"] = {"error": repr(e)}
    if "s6fused" in parts:
        try:
            out["secondary_s6_fused_front_end"] = bench_s6fused(args)
        except Exception as e:  # reported, not hidden
            out["secondary_s6_fused_front_end"] = {"error": repr(e)}
    if "decode" in parts:
        try:
            out["secondary_decode"] = bench_decode(args)
        except Exception as e:  # reported, not hidden
            out["secondary_decode"] = {"error": repr(e)}
    if "decode2" in parts:
        try:
            out["secondary_mamba2_decode"] = bench_decode2(args)
        except Exception as e:
            out["secondary_mamba2_decode"] = {"error": repr(e)}
    if "ssd" in parts:
        try:
            out["secondary_ssd"] = bench_ssd(args)
        except Exception as e:
            out["secondary_ssd"] = {"error": repr(e)}
    if "ssdf32" in parts:
        try:
            out["secondary_ssd_fp32"] = bench_ssd_f32(args)
        except Exception as e:
            out["secondary_ssd_fp32"] = {"error": repr(e)}
    if "copy" in parts:
        out["copy_reference"] = bench_copy(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
