"""GPU parity of the S6 selective scan (mssm_selective_scan_fwd) against the
fp64 oracle, on the same seeded inputs, through the C ABI."""
import numpy as np
import pytest

import oracle
import selective_state_space_19_amd as mssm
from gpu_util import TOL, dev, host, normwise, say, wide
from selective_state_space_19_amd import synth

pytestmark = pytest.mark.gpu


def _run_gpu(inp, final=True, stream=None):
    say(f"  s6 gpu call: u{inp['u'].shape} {inp['dtype']} z={inp['z'] is not None} "
        f"D={inp['D'] is not None} h0={inp['h0'] is not None}")
    args = [dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")]
    out = mssm.selective_scan(*args, return_final_state=final, stream=stream)
    import torch
    torch.cuda.synchronize()
    return out


def _oracle(inp):
    return oracle.s6_scan(*(wide(inp, k) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")))


def _check(inp, name):
    y, hf = _run_gpu(inp)
    yo, ho = _oracle(inp)
    tol = TOL[inp["dtype"]]
    ey, eh = normwise(host(y), yo), normwise(host(hf), ho)
    say(f"  {name}: y err {ey:.3e}  h_final err {eh:.3e}  (tol {tol})")
    assert np.all(np.isfinite(host(y)))
    assert ey <= tol, f"{name}: y normwise error {ey}"
    assert eh <= tol, f"{name}: h_final normwise error {eh}"


def test_tiny_workload():
    w = synth.WORKLOADS["s6_tiny_f32"]
    _check(synth.s6_inputs(**w.shape, dtype=w.dtype, seed=w.seed), w.name)


CASES = [
    # (batch, d_inner, L, N, dtype, gate, skip, h0)
    (1, 1, 1, 1, "f32", True, True, True),
    (2, 33, 7, 3, "f32", True, False, True),
    (1, 64, 64, 16, "f32", False, True, False),
    (2, 100, 65, 16, "f32", True, True, True),
    (1, 70, 130, 17, "f32", True, True, True),
    (3, 64, 200, 8, "f32", False, False, True),
    (1, 65, 129, 32, "f32", True, True, True),
    (1, 128, 96, 64, "f32", True, True, True),
    (2, 64, 63, 4, "f32", True, True, False),
    (1, 1, 1, 1, "bf16", True, True, True),
    (2, 33, 7, 5, "bf16", True, True, True),
    (2, 100, 200, 16, "bf16", True, True, True),
    (1, 130, 1000, 16, "bf16", True, False, True),
    (1, 64, 257, 64, "bf16", False, True, True),
    (2, 192, 333, 12, "bf16", True, True, False),
    # bf16 lengths that are whole 16-token groups (range-checked group loads)
    (2, 64, 32, 8, "bf16", True, True, True),
    (2, 100, 208, 16, "bf16", True, True, True),
    (1, 130, 1024, 16, "bf16", True, False, True),
    (2, 192, 336, 12, "bf16", True, True, False),
    (1, 64, 272, 64, "bf16", False, True, True),
]


# Every other case draws A[d, n] and D[d] per channel (synth's varied=True),
# so a kernel that reads A or D of the wrong channel fails.
@pytest.mark.parametrize("i,case", list(enumerate(CASES)),
                         ids=lambda c: "b{}_d{}_L{}_N{}_{}_z{}_D{}_h{}".format(*c) if isinstance(c, tuple) else None)
def test_ragged_shapes(i, case):
    b, d, L, N, dt, gate, skip, h0 = case
    varied = i % 2 == 1
    inp = synth.s6_inputs(b, d, L, N, dtype=dt, seed=1000 + b * 7 + d + L + N, gate=gate, skip=skip,
                          init_state=h0, varied=varied)
    _check(inp, "x".join(map(str, case)) + ("_varied" if varied else ""))


def test_mamba130m_workload_full():
    """Mamba-130M layer shape (8 x 1536 x 2048, N 16, fp32): every output."""
    w = synth.WORKLOADS["s6_mamba130m_f32"]
    _check(synth.s6_inputs(**w.shape, dtype=w.dtype, seed=w.seed), w.name)


def test_mamba130m_state_only():
    """Without skip term and gate, y = C h alone; h_final compared on its own."""
    w = synth.WORKLOADS["s6_mamba130m_f32"]
    _check(synth.s6_inputs(**w.shape, dtype=w.dtype, seed=w.seed, gate=False, skip=False), w.name + "_noDz")


def test_mamba130m_varied_params_full():
    """Mamba-130M layer shape with A[d, n] and D[d] drawn per channel
    (synth's varied=True): every output."""
    w = synth.WORKLOADS["s6_mamba130m_f32"]
    _check(synth.s6_inputs(**w.shape, dtype=w.dtype, seed=w.seed, varied=True), w.name + "_varied")


def test_mamba1p4b_workload_full():
    """Mamba-1.4B layer shape (4 x 4096 x 8192, N 16, bf16 in / fp32 state,
    h_final out), in the benchmark's launch configuration: every output and
    every final state against the oracle."""
    w = synth.WORKLOADS["s6_mamba1p4b_bf16"]
    _check(synth.s6_inputs(**w.shape, dtype=w.dtype, seed=w.seed), w.name)


def test_bitwise_deterministic():
    inp = synth.s6_inputs(2, 256, 500, 16, dtype="bf16", seed=77, init_state=True)
    y1, h1 = _run_gpu(inp)
    y2, h2 = _run_gpu(inp)
    import torch
    assert torch.equal(y1, y2) and torch.equal(h1, h2)


@pytest.mark.parametrize("split", [1, 64, 100])
def test_chaining_is_exact(split):
    """scan(L) == scan(first part) then scan(rest, h0 = h_final): the kernel
    walks time strictly in order, so the results are bitwise equal."""
    import torch
    inp = synth.s6_inputs(2, 96, 300, 16, dtype="f32", seed=5, init_state=True)
    y, hf = _run_gpu(inp)
    a = {k: (v[..., :split] if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    b = {k: (np.ascontiguousarray(v[..., split:]) if k in ("u", "delta", "z", "B", "C") else v)
         for k, v in inp.items()}
    a = {k: (np.ascontiguousarray(v) if isinstance(v, np.ndarray) else v) for k, v in a.items()}
    y1, h1 = _run_gpu(a)
    b["h0"] = h1.cpu().numpy()
    y2, h2 = _run_gpu(b)
    assert torch.equal(torch.cat([y1, y2], -1), y)
    assert torch.equal(h2, hf)


def test_nan_poisons_only_its_channel_from_then_on():
    import torch
    inp = synth.s6_inputs(1, 64, 128, 16, dtype="f32", seed=9)
    inp["u"][0, 5, 40] = np.nan
    y, hf = _run_gpu(inp)
    y = host(y)
    assert np.all(np.isnan(y[0, 5, 40:]))
    assert np.all(np.isfinite(y[0, 5, :40]))
    mask = np.ones(64, bool)
    mask[5] = False
    assert np.all(np.isfinite(y[0, mask]))


def test_zero_length_sequence_returns_h0():
    import torch
    inp = synth.s6_inputs(2, 40, 0, 16, dtype="f32", seed=3, init_state=True)
    y, hf = _run_gpu(inp)
    assert y.shape == (2, 40, 0)
    np.testing.assert_array_equal(host(hf), inp["h0"].astype(np.float64))
    inp["h0"] = None
    y, hf = _run_gpu(inp)
    assert np.all(host(hf) == 0.0)


def test_errors_reported():
    import torch
    inp = synth.s6_inputs(1, 64, 64, 16, dtype="f32", seed=3)
    with pytest.raises(mssm.MssmError) as e:
        args = [dev(inp[k]) for k in ("u", "delta", "A", "B", "C", "D", "z", "h0")]
        args[0] = torch.zeros(1 * 64 * 64 + 1, device="cuda")[1:].view(1, 64, 64)   # misaligned
        mssm.selective_scan(*args)
    assert e.value.code == -5
