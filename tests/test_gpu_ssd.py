"""GPU parity of the Mamba-2 SSD (mssm_ssd_chunk_fwd) against the fp64 oracle
(the recurrence run per head channel), through the C ABI."""
import numpy as np
import pytest

import oracle
import selective_state_space_19_amd as mssm
from gpu_util import TOL, dev, host, normwise, say
from selective_state_space_19_amd import synth

pytestmark = pytest.mark.gpu


def _gpu(inp, chunk, final=True):
    s = inp["x"].shape
    say(f"  ssd gpu call: x{s} N{inp['B'].shape[-1]} G{inp['B'].shape[2]} chunk {chunk} "
        f"z={inp['z'] is not None} D={inp['D'] is not None} h0={inp['h0'] is not None}")
    out = mssm.ssd_chunk(*(dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "h0")), chunk=chunk,
                         return_final_state=final)
    import torch
    torch.cuda.synchronize()
    return out


def _oracle(inp):
    return oracle.ssd(*(synth.widen(inp[k], inp["dtype"]) if inp[k] is not None and inp[k].dtype == np.uint16
                        else inp[k] for k in ("x", "dt", "A", "B", "C", "D", "z", "h0")))


def _check(inp, chunk, name, tol=TOL["bf16"]):
    y, hf = _gpu(inp, chunk)
    yo, ho = _oracle(inp)
    ey, eh = normwise(host(y), yo), normwise(host(hf), ho)
    say(f"  {name}: y err {ey:.3e}  h_final err {eh:.3e}  (tol {tol})")
    assert np.all(np.isfinite(host(y)))
    assert ey <= tol and eh <= tol, f"{name}: y {ey} h {eh}"
    return ey, eh


CASES = [
    # (batch, L, H, N, G, chunk, gate, skip, h0)
    (1, 64, 1, 32, 1, 64, False, True, False),
    (1, 100, 2, 64, 1, 64, True, True, True),
    (2, 256, 4, 128, 1, 256, False, True, False),
    (1, 300, 4, 128, 2, 128, True, False, True),
    (2, 513, 2, 256, 1, 256, False, True, True),
    (1, 1, 2, 64, 2, 64, True, True, True),
    (1, 777, 8, 128, 4, 128, True, True, False),
    (2, 1024, 4, 32, 1, 256, False, True, True),
    # gate at chunk 256 (three rounds of row blocks on the output waves, one
    # on the state waves), and the other d_state values at chunk 128 / 256
    (1, 600, 4, 128, 1, 256, True, True, True),
    (1, 300, 2, 64, 1, 256, True, False, False),
    (1, 200, 2, 256, 2, 128, True, True, True),
    (1, 130, 2, 32, 1, 128, False, True, True),
]


# Every other case draws D_h per head (synth's varied=True; A_h is per head always).
@pytest.mark.parametrize("i,case", list(enumerate(CASES)),
                         ids=lambda c: "b{}_L{}_H{}_N{}_G{}_Q{}_z{}_D{}_h{}".format(*c) if isinstance(c, tuple)
                         else None)
def test_ragged_shapes(i, case):
    b, L, H, N, G, Q, gate, skip, h0 = case
    varied = i % 2 == 1
    inp = synth.ssd_inputs(b, L, H, 64, N, G, dtype="bf16", seed=300 + L + H + N, gate=gate, skip=skip,
                           init_state=h0, varied=varied)
    _check(inp, Q, "x".join(map(str, case)) + ("_varied" if varied else ""))


# Sizes the bf16 MFMA kernels do not take run in the general chunked kernel
# (fp32 matrix cores): float32 storage, headdim not a multiple of 32, d_state
# not in {32, 64, 128, 256}.
GENERAL = [
    # (batch, L, H, P, N, G, chunk, dtype, gate, skip, h0)
    (1, 1, 1, 64, 128, 1, 64, "f32", True, True, True),
    (1, 100, 2, 64, 128, 1, 64, "f32", False, True, True),
    (2, 257, 4, 32, 16, 2, 128, "f32", True, True, False),
    (1, 300, 2, 128, 48, 1, 256, "f32", True, False, True),
    (1, 64, 3, 16, 64, 3, 64, "f32", False, True, True),
    (1, 90, 2, 80, 256, 1, 256, "f32", True, True, True),
    (2, 300, 4, 32, 16, 1, 128, "bf16", True, True, True),
    (1, 500, 2, 128, 48, 2, 256, "bf16", False, True, True),
    (1, 200, 2, 16, 80, 1, 64, "bf16", True, True, False),
    (1, 130, 2, 96, 48, 1, 128, "bf16", True, False, True),
    # d_state not a multiple of 16 (padded tiles) or of 4 (element loads of B
    # and C), and odd headdims: both general kernels (d_state above 128: the
    # wide one)
    (1, 70, 2, 7, 1, 1, 64, "f32", True, True, True),
    (2, 129, 3, 33, 37, 3, 128, "f32", False, True, True),
    (1, 100, 2, 40, 100, 2, 256, "bf16", True, False, True),
    (1, 65, 2, 24, 130, 1, 64, "f32", True, True, False),
    (1, 90, 1, 16, 255, 1, 256, "bf16", True, True, True),
]


@pytest.mark.parametrize("i,case", list(enumerate(GENERAL)),
                         ids=lambda c: "b{}_L{}_H{}_P{}_N{}_G{}_Q{}_{}_z{}_D{}_h{}".format(*c) if isinstance(c, tuple)
                         else None)
def test_general_sizes(i, case):
    b, L, H, P, N, G, Q, dt, gate, skip, h0 = case
    inp = synth.ssd_inputs(b, L, H, P, N, G, dtype=dt, seed=900 + L + P + N, gate=gate, skip=skip, init_state=h0,
                           varied=i % 2 == 1)
    _check(inp, Q, "general_" + "x".join(map(str, case)), tol=TOL[dt])


# bf16 at headdims other than 64 that are multiples of 32: the MFMA kernels,
# one workgroup per 32-channel block of a head.
FAST_HEADDIMS = [
    # (batch, L, H, P, N, G, chunk, gate, skip, h0)
    (1, 130, 2, 96, 32, 1, 128, True, False, True),
    (2, 300, 4, 128, 128, 2, 256, True, True, True),
    (1, 513, 3, 32, 64, 1, 64, False, True, True),
    (1, 200, 2, 256, 256, 1, 128, True, True, False),
    (2, 1000, 2, 128, 64, 1, 256, False, True, True),
]


@pytest.mark.parametrize("i,case", list(enumerate(FAST_HEADDIMS)),
                         ids=lambda c: "b{}_L{}_H{}_P{}_N{}_G{}_Q{}_z{}_D{}_h{}".format(*c) if isinstance(c, tuple)
                         else None)
def test_mfma_path_other_headdims(i, case):
    b, L, H, P, N, G, Q, gate, skip, h0 = case
    assert mssm.ssd_workspace_size(b, L, H, P, N, G, Q) > 0        # the MFMA path: its operand tiles
    inp = synth.ssd_inputs(b, L, H, P, N, G, dtype="bf16", seed=950 + L + P + N, gate=gate, skip=skip,
                           init_state=h0, varied=i % 2 == 1)
    _check(inp, Q, "headdim_" + "x".join(map(str, case)))


def test_headdim128_layer_shape():
    """A layer of the same width with 16 heads x 128 (batch 2, seqlen 4096,
    d_state 128, chunk 256, gated, from h0): four 32-channel workgroups per
    head on the MFMA kernels; every output and the final state against the
    oracle."""
    b, L, H, P, N, G, Q = 2, 4096, 16, 128, 128, 1, 256
    assert mssm.ssd_workspace_size(b, L, H, P, N, G, Q) > 0
    inp = synth.ssd_inputs(b, L, H, P, N, G, dtype="bf16", seed=1280, gate=True, init_state=True, varied=True)
    _check(inp, Q, "headdim 128 layer")


def test_mamba2_shape_fp32():
    """The Mamba-2 layer shape (batch 4, seqlen 4096, 32 heads x 64, d_state
    128) with float32 storage: every output within the fp32 tolerance."""
    w = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = w.shape
    inp = synth.ssd_inputs(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                           dtype="f32", seed=w.seed, varied=True)
    _check(inp, s["chunk"], w.name + "_f32", tol=TOL["f32"])


def test_mamba2_workload_full():
    """Mamba-2 layer (batch 4, seqlen 4096, 32 heads x 64, d_state 128,
    ngroups 1, chunk 256), every output against the oracle."""
    w = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = w.shape
    inp = synth.ssd_inputs(s["batch"], s["seqlen"], s["nheads"], s["headdim"], s["d_state"], s["ngroups"],
                           dtype=w.dtype, seed=w.seed)
    _check(inp, s["chunk"], w.name)


def test_mamba2_workload_state_only():
    """Without the skip term y is the SSM alone."""
    w = synth.WORKLOADS["ssd_mamba2_bf16"]
    s = w.shape
    inp = synth.ssd_inputs(2, 1024, 8, 64, 128, 1, dtype=w.dtype, seed=w.seed + 1, skip=False, init_state=True)
    _check(inp, s["chunk"], w.name + "_noD")


@pytest.mark.parametrize("chunk", [64, 256])
def test_strong_decay_blocks(chunk):
    """Token blocks whose decay over 32 tokens exceeds 2^64 (the product of
    its two factors would leave float range) build the diagonal mask element
    by element; the others take the factored form.  Here both kinds mix
    within heads and chunks: dt is scaled by 40 in every other 32-token block
    of head 0 and everywhere in head 2."""
    inp = synth.ssd_inputs(2, 600, 4, 64, 128, 1, dtype="bf16", seed=77, gate=True, init_state=True)
    dt = synth.widen(inp["dt"], "bf16")
    f = np.ones_like(dt)
    f[:, (np.arange(600) // 32) % 2 == 1, 0] = 40.0
    f[:, :, 2] = 40.0
    inp["dt"] = synth.round_to(dt * f, "bf16")
    # decay over each whole 32-token block (log2 units): both kinds occur
    a = synth.widen(inp["dt"], "bf16")[:, :576] * np.abs(inp["A"])[None, None, :] / np.log(2.0)
    span = a.reshape(2, 18, 32, 4)[:, :, 1:, :].sum(axis=2)
    assert (span > 64).any() and (span < 32).any()
    _check(inp, chunk, f"strong_decay_q{chunk}")


def test_chunk_size_invariance():
    """The chunk length only changes rounding (the chunked form is exact)."""
    inp = synth.ssd_inputs(2, 768, 4, 64, 128, 1, dtype="bf16", seed=41, init_state=True)
    outs = [host(_gpu(inp, q)[0]) for q in (64, 128, 256)]
    yo, _ = _oracle(inp)
    for o in outs:
        assert normwise(o, yo) <= TOL["bf16"]
    assert normwise(outs[0], outs[2]) <= TOL["bf16"]


def test_ssd_matches_s6_kernel_on_heads():
    """SSD with one group equals the S6 scan on d_inner = H*P channels with
    A[(h,p), n] = A_h and delta[(h,p), t] = dt[t, h] -- computed here by the
    library's S6 kernel, so the two GPU paths check each other."""
    import torch
    b, L, H, P, N = 1, 512, 4, 64, 64
    inp = synth.ssd_inputs(b, L, H, P, N, 1, dtype="bf16", seed=42, gate=True, init_state=True)
    y, hf = _gpu(inp, 128)
    to = lambda a: dev(np.ascontiguousarray(a))  # noqa: E731
    u = to(np.transpose(inp["x"], (0, 2, 3, 1)).reshape(b, H * P, L))
    dl = to(np.repeat(np.transpose(inp["dt"], (0, 2, 1)), P, axis=1))
    A = to(np.repeat(inp["A"], P)[:, None] * np.ones((1, N), np.float32))
    Bs = to(np.transpose(inp["B"][:, :, 0, :], (0, 2, 1)))
    Cs = to(np.transpose(inp["C"][:, :, 0, :], (0, 2, 1)))
    z = to(np.transpose(inp["z"], (0, 2, 3, 1)).reshape(b, H * P, L))
    ys, hs = mssm.selective_scan(u, dl, A, Bs, Cs, to(np.repeat(inp["D"], P)), z,
                                 to(inp["h0"].reshape(b, H * P, N)), return_final_state=True)
    torch.cuda.synchronize()
    y_as_s6 = np.transpose(host(y), (0, 2, 3, 1)).reshape(b, H * P, L)
    assert normwise(y_as_s6, host(ys)) <= TOL["bf16"]
    assert normwise(host(hf).reshape(b, H * P, N), host(hs)) <= TOL["bf16"]


def test_zero_length_and_errors():
    import torch
    inp = synth.ssd_inputs(1, 0, 2, 64, 64, 1, dtype="bf16", seed=1, init_state=True)
    y, hf = _gpu(inp, 64)
    np.testing.assert_array_equal(host(hf), inp["h0"].astype(np.float64))
    inp = synth.ssd_inputs(1, 64, 2, 64, 64, 1, dtype="bf16", seed=1)
    with pytest.raises(mssm.MssmError) as e:
        mssm.ssd_chunk(*(dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "h0")), chunk=96)
    assert e.value.code == -4
    inp = synth.ssd_inputs(1, 64, 2, 64, 272, 1, dtype="f32", seed=1)
    with pytest.raises(mssm.MssmError) as e:      # d_state above 256
        mssm.ssd_chunk(*(dev(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "z", "h0")), chunk=64)
    assert e.value.code == -4


@pytest.mark.parametrize("chunk", [64, 256])
def test_carried_state_term_isolated(chunk):
    """x = 0 and a large h0: every output is the carried-in state's term
    exp(s_i) C_i H_in (no intra-chunk product, no skip term), which the
    kernel forms from the state rounded to bf16 (an MFMA operand).  Its error
    is measured alone here, against the oracle's fp64 state."""
    inp = synth.ssd_inputs(2, 700, 4, 64, 128, 1, dtype="bf16", seed=91, gate=True, init_state=True, varied=True)
    inp["x"] = np.zeros_like(inp["x"])
    inp["h0"] = (inp["h0"] * 30.0).astype(np.float32)
    ey, eh = _check(inp, chunk, f"carried_state_only_q{chunk}")
    say(f"  carried state alone: y err {ey:.3e} (bf16 state operand), h_final err {eh:.3e}")
