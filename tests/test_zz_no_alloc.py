"""The SSD entry point that allocates nothing (mssm_ssd_chunk_fwd_noalloc,
static per-GPU scratch) against mssm_ssd_chunk_fwd with a caller workspace:
calls in a row, the second smaller (the scratch keeps the first call's
contents), the third on the general kernel; each equal to the workspace
call bit for bit and to the oracle within its dtype's tolerance."""
import numpy as np
import pytest

import oracle
import selective_state_space_19_amd as mssm
from gpu_util import TOL, dev, host, normwise, say
from selective_state_space_19_amd import _lib, synth

pytestmark = pytest.mark.gpu

KEYS = ("x", "dt", "A", "B", "C", "D", "z", "h0")


def _pair(inp, chunk):
    import torch
    args = [dev(inp[k]) for k in KEYS]
    b, L, H, P = inp["x"].shape
    N = inp["B"].shape[-1]
    y_ws, h_ws = mssm.ssd_chunk(*args, chunk=chunk, return_final_state=True)
    y_na = torch.empty_like(args[0])
    h_na = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    mssm.ssd_chunk_noalloc(*args, out=y_na, h_final=h_na, chunk=chunk)
    torch.cuda.synchronize()
    return (y_ws, h_ws), (y_na, h_na)


def test_noalloc_matches_workspace_call_twice():
    import torch
    big = synth.ssd_inputs(4, 4096, 32, 64, 128, 1, dtype="bf16", seed=19004, varied=True)
    small = synth.ssd_inputs(2, 700, 8, 64, 64, 2, dtype="bf16", seed=55, gate=True, init_state=True, varied=True)
    # then the general kernel, whose raw scores also go to the scratch
    general = synth.ssd_inputs(2, 300, 4, 48, 64, 1, dtype="f32", seed=56, gate=True, init_state=True, varied=True)
    for name, inp, chunk in (("Mamba-2 layer, chunk 256", big, 256), ("smaller, gated, h0, chunk 128", small, 128),
                             ("float32, headdim 48 (general kernel)", general, 64)):
        say(f"  noalloc ssd call: {name} x{inp['x'].shape}")
        (y0, h0), (y1, h1) = _pair(inp, chunk)
        assert torch.equal(y0, y1) and torch.equal(h0, h1), name
        yo, ho = oracle.ssd(*(synth.widen(inp[k], "bf16") if inp[k] is not None and inp[k].dtype == np.uint16
                              else inp[k] for k in KEYS))
        ey, eh = normwise(host(y1), yo), normwise(host(h1), ho)
        say(f"  {name}: y err {ey:.3e}  h_final err {eh:.3e}")
        assert ey <= TOL[inp["dtype"]] and eh <= TOL[inp["dtype"]]


def test_noalloc_rejects_sizes_beyond_its_scratch():
    import torch
    b, L, H, P, N = 32, 4096, 32, 64, 128
    assert mssm.ssd_workspace_size(b, L, H, P, N, 1, 256) > _lib.noalloc_scratch_bytes()
    say("  noalloc ssd call: oversize (rejected on the host)")
    x = torch.zeros((b, L, H, P), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((b, L, H), dtype=torch.bfloat16, device="cuda")
    Bm = torch.zeros((b, L, 1, N), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((H,), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(mssm.MssmError) as e:
        mssm.ssd_chunk_noalloc(x, dt, A, Bm, Bm, out=y)
    assert e.value.code == -6 and "static scratch" in e.value.msg
