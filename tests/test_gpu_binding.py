"""The Python binding's argument handling on the GPU: tensors the kernels
write must be contiguous (a silent copy would take the writes), and a call
on a stream other than the current one sees the inputs the current stream
prepared."""
import numpy as np
import pytest

import selective_state_space_19_amd as mssm
from gpu_util import dev, host, normwise, say
from selective_state_space_19_amd import synth

pytestmark = pytest.mark.gpu


def test_strided_outputs_and_state_are_rejected():
    import torch
    say("  binding: strided out / state / h_final")
    inp = synth.s6_inputs(2, 64, 40, 16, dtype="f32", seed=4, init_state=True)
    args = [dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")]
    big = torch.empty((2, 64, 80), device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        mssm.selective_scan(*args, out=big[:, :, ::2])
    hbig = torch.empty((2, 64, 32), device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        mssm.selective_scan(*args, h_final=hbig[:, :, ::2])
    init = synth.decode_initial(2, 64, 16, seed=5)
    tk = synth.decode_step(init, 0, 2, 64, 16, dtype="f32", seed=5)
    st = torch.empty((2, 64, 32), device="cuda")[:, :, :16]
    with pytest.raises(ValueError, match="contiguous"):
        mssm.state_update(st, dev(tk["u"]), dev(tk["delta"]), dev(init["A"]), dev(tk["B"]), dev(tk["C"]))
    st = dev(init["state"])
    yall = torch.zeros((2, 64, 3), device="cuda")
    with pytest.raises(ValueError, match="contiguous"):
        mssm.state_update(st, dev(tk["u"]), dev(tk["delta"]), dev(init["A"]), dev(tk["B"]), dev(tk["C"]),
                          out=yall[:, :, 1])
    # the rejected calls wrote nothing
    assert torch.equal(st, dev(init["state"])) and not bool(yall.any())


def test_side_stream_sees_prepared_inputs():
    """Inputs made non-contiguous on purpose (so the binding copies them on
    the current stream) and a call on a side stream: the result equals the
    plain call's."""
    import torch
    say("  binding: side stream")
    inp = synth.s6_inputs(2, 128, 300, 16, dtype="bf16", seed=6, init_state=True, varied=True)
    args = [dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")]
    y0, h0 = mssm.selective_scan(*args, return_final_state=True)
    # the same values in transposed storage: u, delta, z as [b, L, d] made [b, d, L]
    tr = [a.transpose(1, 2).contiguous().transpose(1, 2) if i in (0, 1, 6) else a for i, a in enumerate(args)]
    assert not tr[0].is_contiguous()
    side = torch.cuda.Stream()
    y1, h1 = mssm.selective_scan(*tr, return_final_state=True, stream=side)
    side.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(h0, h1)
