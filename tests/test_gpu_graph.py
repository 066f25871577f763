"""Every entry point inside a captured HIP graph (torch.cuda.graph): a
decode loop, the S6 scan forward variants and backward, the SSD with a
caller's workspace and the no-alloc SSD.  Each graph is replayed several
times with eager work and synchronisations between the replays; the
outputs are filled with NaN before each replay and must come back equal to
the eager calls' bit for bit (dA and dD, summed with atomics, to 1e-6), so
nothing a graph records -- a clear, a fill, a workspace -- holds only on its
first replay."""
import numpy as np
import pytest

import oracle
import selective_state_space_19_amd as mssm
from gpu_util import TOL, dev, host, normwise, say
from selective_state_space_19_amd import synth

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _nan_(ts):
    import torch
    for t in ts:
        t.fill_(float("nan")) if t.dtype.is_floating_point else t.zero_()
    torch.cuda.synchronize()


def _replay_and_check(g, outs, refs, eager_work, name, close=()):
    import torch
    for r in range(REPLAYS):
        _nan_(outs)
        eager_work()                          # the program's own work between replays
        torch.cuda.synchronize()
        say(f"  {name}: replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, refs)):
            if i in close:
                assert normwise(host(o), host(e)) <= 1e-6, (name, r, i)
            else:
                assert torch.equal(o, e), (name, r, i)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_loop_in_a_graph(dt):
    """Eight decode tokens of the S6 layer (batch 3, 130 channels, d_state 16)
    captured as one graph; the state is reset eagerly before each replay."""
    import torch
    b, d, N, K = 3, 130, 16, 8
    init = synth.decode_initial(b, d, N, seed=71, varied=True)
    steps = [synth.decode_step(init, t, b, d, N, dtype=dt, seed=71) for t in range(K)]
    # one allocation per step and array: the entry point wants 16-byte aligned rows
    st = [{k: dev(s[k]) for k in ("u", "delta", "z", "B", "C")} for s in steps]
    A, D = dev(init["A"]), dev(init["D"])
    s0 = dev(init["state"])

    def step(state, t, out=None):
        a = st[t]
        return mssm.state_update(state, a["u"], a["delta"], A, a["B"], a["C"], D, a["z"], out=out)
    say(f"  decode graph {dt}: eager")
    se = s0.clone()
    ye = [step(se, t) for t in range(K)]
    torch.cuda.synchronize()
    sg = s0.clone()
    yg = [torch.empty_like(y) for y in ye]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(K):
            step(sg, t, out=yg[t])
    other = s0.clone()

    def eager_work():
        sg.copy_(s0)
        step(other, 0)
    _replay_and_check(g, yg + [sg], ye + [se], eager_work, f"decode {dt}")
    # and the replayed loop against the oracle (decode steps = one scan)
    seq = lambda k: synth.widen(np.stack([s[k] for s in steps], axis=-1), dt)  # noqa: E731  [b, d|N, K]
    yo, ho = oracle.s6_scan(seq("u"), seq("delta"), init["A"], seq("B"), seq("C"), init["D"], seq("z"),
                            init["state"])
    assert normwise(np.stack([host(y) for y in yg], axis=-1), yo) <= TOL[dt]
    assert normwise(host(sg), ho) <= TOL[dt]


def test_mamba2_decode_loop_in_a_graph():
    """Six Mamba-2 decode tokens (batch 2, 4 heads x 64, d_state 128, 2 groups)."""
    import torch
    b, H, P, N, G, K = 2, 4, 64, 128, 2, 6
    init = synth.mamba2_decode_initial(b, H, P, N, seed=72, varied=True)
    steps = [synth.mamba2_decode_step(init, t, b, H, P, N, ngroups=G, seed=72) for t in range(K)]
    st = [{k: dev(s[k]) for k in ("x", "dt", "z", "B", "C")} for s in steps]
    A, D = dev(init["A"]), dev(init["D"])
    s0 = dev(init["state"])

    def step(state, t, out=None):
        a = st[t]
        return mssm.ssd_state_update(state, a["x"], a["dt"], A, a["B"], a["C"], D, a["z"], out=out)
    say("  mamba2 decode graph: eager")
    se = s0.clone()
    ye = [step(se, t) for t in range(K)]
    torch.cuda.synchronize()
    sg = s0.clone()
    yg = [torch.empty_like(y) for y in ye]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(K):
            step(sg, t, out=yg[t])

    def eager_work():
        sg.copy_(s0)
    _replay_and_check(g, yg + [sg], ye + [se], eager_work, "mamba2 decode")


def test_scan_family_in_a_graph():
    """The Euler, hold-form and front-end scans, the saving forward and both
    backward calls (bf16, batch 2, 100 channels, 300 tokens, d_state 16) in
    one graph."""
    import torch
    b, d, L, N = 2, 100, 300, 16
    inp = synth.s6_inputs(b, d, L, N, dtype="bf16", seed=73, init_state=True, varied=True)
    fin = synth.s6_fused_inputs(b, d, L, N, dtype="bf16", seed=74, init_state=True, conv_history=True, varied=True)
    a = {k: dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")}
    f = {k: dev(fin[k]) for k in ("x", "conv_w", "conv_b", "conv_init", "delta_raw", "delta_bias", "A", "B", "C",
                                  "D", "z", "h0")}
    rng = np.random.default_rng(73)
    dout = dev(synth.round_to(rng.standard_normal((b, d, L)), "bf16"))
    dhT = dev(rng.standard_normal((b, d, N)).astype(np.float32))
    nws = mssm.selective_scan_bwd_workspace_size(b, d, L, N)
    ws_e = torch.empty(nws, dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(nws, dtype=torch.uint8, device="cuda")
    args = [a[k] for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")]
    bargs = [a[k] for k in ("u", "delta", "A", "B", "C")] + [dout]
    bkw = dict(D=a["D"], z=a["z"], h0=a["h0"], dh_final=dhT)
    fargs = [f[k] for k in ("x", "conv_w", "delta_raw", "A", "B", "C", "D", "z", "h0")]
    fkw = dict(conv_b=f["conv_b"], conv_init=f["conv_init"], delta_bias=f["delta_bias"])

    def run(ws, outs=None):
        o = outs or {}
        r = {}
        r["y"], r["hf"] = mssm.selective_scan(*args, return_final_state=True, out=o.get("y"), h_final=o.get("hf"))
        r["yz"], r["hz"] = mssm.selective_scan(*args, return_final_state=True, zoh=True, out=o.get("yz"),
                                               h_final=o.get("hz"))
        r["yf"], r["hff"] = mssm.selective_scan_fused(*fargs, **fkw, return_final_state=True, out=o.get("yf"),
                                                      h_final=o.get("hff"))
        r["ys"], r["hs"] = mssm.selective_scan(*args, return_final_state=True, save_workspace=ws, out=o.get("ys"),
                                               h_final=o.get("hs"))
        g0 = mssm.selective_scan_bwd(*bargs, **bkw)
        g1 = mssm.selective_scan_bwd(*bargs, **bkw, workspace=ws, saved=True)
        for k, v in g0.items():
            r["plain_" + k] = v
        for k, v in g1.items():
            r["saved_" + k] = v
        return r

    say("  scan family graph: eager")
    ref = run(ws_e)
    torch.cuda.synchronize()
    outs = {k: torch.empty_like(ref[k]) for k in ("y", "hf", "yz", "hz", "yf", "hff", "ys", "hs")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        got = run(ws_g, outs)
    keys = sorted(ref)
    close = {i for i, k in enumerate(keys) if k.endswith("_dA") or k.endswith("_dD")}

    def eager_work():
        ws_g.fill_(0xFF)                       # the saved states must be rewritten by the replay
        mssm.selective_scan(*args)
    _replay_and_check(g, [got[k] for k in keys], [ref[k] for k in keys], eager_work, "scan family", close)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_ssd_in_a_graph(dt):
    """The SSD with the caller's workspace (MFMA kernels in bf16, the general
    kernel in fp32), and in bf16 the no-alloc entry point, in one graph."""
    import torch
    b, L, H, P, N, G, Q = 2, 300, 4, 64, 128, 1, 128
    inp = synth.ssd_inputs(b, L, H, P, N, G, dtype=dt, seed=75, gate=True, init_state=True, varied=True)
    a = [dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "h0")]
    need = mssm.ssd_workspace_size(b, L, H, P, N, G, Q)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    say(f"  ssd graph {dt}: eager")
    ye, he = mssm.ssd_chunk(*a, chunk=Q, return_final_state=True, workspace=ws)
    refs = [ye, he]
    if dt == "bf16":
        yn, hn = torch.empty_like(ye), torch.empty_like(he)
        mssm.ssd_chunk_noalloc(*a, chunk=Q, out=yn, h_final=hn)
        refs += [yn.clone(), hn.clone()]
    torch.cuda.synchronize()
    outs = [torch.empty_like(t) for t in refs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mssm.ssd_chunk(*a, chunk=Q, out=outs[0], h_final=outs[1], workspace=ws)
        if dt == "bf16":
            mssm.ssd_chunk_noalloc(*a, chunk=Q, out=outs[2], h_final=outs[3])

    def eager_work():
        ws.fill_(0xFF)
        mssm.ssd_chunk(*a, chunk=Q)            # another call on the same GPU between replays
    _replay_and_check(g, outs, refs, eager_work, f"ssd {dt}")
    if dt == "bf16":
        assert torch.equal(refs[0], refs[2]) and torch.equal(refs[1], refs[3])
