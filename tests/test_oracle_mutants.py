"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU)
and check that the pins catch every one of them.  This shows the pins are
strong enough: a dropped term, a wrong sign or index, a swapped operand or
a wrong update order all fail at least one pin."""
import json
import os

import numpy as np
import pytest

import oracle
from forms import closed_form_s6, normwise_err, ssd_quadratic

SRC = os.path.join(os.path.dirname(oracle.__file__), "mssm_oracle.c")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = {
    "drop_skip_term": ("double o = acc + c->dskip * x;", "double o = acc;"),
    "output_reads_old_state": (
        "h[n] = dA * h[n] + dBu;\n            acc += c->Cm[n * c->s_bn + t * c->s_bt] * h[n];",
        "acc += c->Cm[n * c->s_bn + t * c->s_bt] * h[n];\n            h[n] = dA * h[n] + dBu;"),
    "exp_sign": ("const double dA = exp(d * a);", "const double dA = exp(-d * a);"),
    "B_and_C_swapped": ("(k * x) * c->Bm[", "(k * x) * c->Cm["),
    "gate_sign": ("o *= g / (1.0 + exp(-g));", "o *= g / (1.0 + exp(g));"),
    "initial_state_ignored": ("c->h0 ? c->h0[n * c->s_h] : 0.0", "0.0"),
    "ssd_dt_stride": ("c->s_d = p->H;", "c->s_d = 1;"),
    "step_dropped_from_input": ("expm1(d * a) / a : d) : d;", "expm1(d * a) / a : d) : 1.0;"),
    "zoh_gain_is_euler": ("expm1(d * a) / a : d) : d;", "d : d) : d;"),
    "zoh_gain_sign": ("expm1(d * a) / a", "expm1(-d * a) / a"),
    "zoh_gain_without_minus_one": ("expm1(d * a) / a", "exp(d * a) / a"),
    "ssd_group_map": ("const long g = h / (p->H / p->G);", "const long g = h % p->G;"),
    "final_state_index": ("c->hT[n * c->s_h] = h[n];", "c->hT[n * c->s_h] = h[0];"),
    "ssd_h0_ignores_head_channel": (
        "c->h0 = p->h0 ? p->h0 + ((b * p->H + h) * p->P + q) * p->N : NULL;",
        "c->h0 = p->h0 ? p->h0 + ((b * p->H + h) * p->P) * p->N : NULL;"),
}


def _pins(lib):
    """Return the names of the pins that fail for this library."""
    failed = []
    arr = lambda v: None if v is None else np.asarray(v, np.float64)  # noqa: E731
    for name in ("s6_two_states_three_tokens", "s6_gate_initial_state_varying_step"):
        g = json.load(open(os.path.join(GOLDEN, name + ".json")))
        i = {k: arr(v) for k, v in g["inputs"].items()}
        y, hT = oracle.s6_scan(i["u"], i["delta"], i["A"], i["B"], i["C"], i["D"], i["z"], i["h0"], lib=lib)
        if not (np.allclose(y, g["expected"]["y"], 1e-12, 1e-12) and
                np.allclose(hT, g["expected"]["h_final"], 1e-12, 1e-12)):
            failed.append(name)
    g = json.load(open(os.path.join(GOLDEN, "ssd_two_heads_two_tokens.json")))
    i = {k: arr(v) for k, v in g["inputs"].items()}
    y, hT = oracle.ssd(i["x"], i["dt"], i["A"], i["B"], i["C"], i["D"], i["z"], i["h0"], lib=lib)
    if not (np.allclose(y, g["expected"]["y"], 1e-12, 1e-12) and
            np.allclose(hT, g["expected"]["h_final"], 1e-12, 1e-12)):
        failed.append("golden_ssd")
    rng = np.random.default_rng(0)
    b, d, L, N = 2, 3, 9, 4
    s6 = dict(u=rng.standard_normal((b, d, L)), delta=rng.uniform(0.05, 0.5, (b, d, L)),
              A=-rng.uniform(0.2, 3.0, (d, N)), B=rng.standard_normal((b, N, L)),
              C=rng.standard_normal((b, N, L)), D=rng.standard_normal(d),
              z=rng.standard_normal((b, d, L)), h0=rng.standard_normal((b, d, N)))
    y, hT = oracle.s6_scan(**s6, lib=lib)
    yc, hc = closed_form_s6(**s6)
    if normwise_err(y, yc) > 1e-12 or normwise_err(hT, hc) > 1e-12:
        failed.append("closed_form")
    b, L, H, P, N, G = 2, 11, 4, 3, 5, 2
    sd = dict(x=rng.standard_normal((b, L, H, P)), dt=rng.uniform(0.05, 0.5, (b, L, H)),
              A=-rng.uniform(0.5, 4.0, H), B=rng.standard_normal((b, L, G, N)),
              C=rng.standard_normal((b, L, G, N)), D=rng.standard_normal(H),
              z=rng.standard_normal((b, L, H, P)), h0=rng.standard_normal((b, H, P, N)))
    y, hT = oracle.ssd(**sd, lib=lib)
    yq, hq = ssd_quadratic(**sd)
    if normwise_err(y, yq) > 1e-11 or normwise_err(hT, hq) > 1e-11:
        failed.append("ssd_quadratic")
    # zero-order hold: L held steps equal the exact solution over L*delta
    d, L, N = 2, 13, 3
    a = -rng.uniform(0.1, 3.0, (d, N))
    dl, u0, bn = rng.uniform(0.05, 0.4, d), rng.standard_normal(d), rng.standard_normal(N)
    h0 = rng.standard_normal((1, d, N))
    _, hT = oracle.s6_scan(np.repeat(u0[None, :, None], L, 2), np.repeat(dl[None, :, None], L, 2), a,
                           np.repeat(bn[None, :, None], L, 2), rng.standard_normal((1, N, L)), h0=h0,
                           lib=lib, zoh=True)
    T = L * dl[:, None]
    exact = np.exp(a * T) * h0[0] + np.expm1(a * T) / a * bn[None, :] * u0[:, None]
    if not np.allclose(hT[0], exact, 1e-11, 1e-13):
        failed.append("zoh_exact_solution")
    return failed


def test_unmutated_oracle_passes_every_pin(tmp_path):
    out = str(tmp_path / "lib_ok.so")
    oracle.build(out=out)
    assert _pins(oracle.load(out)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new))
    out = str(tmp_path / f"lib_{name}.so")
    import subprocess
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread", "-o", out,
                    str(mutated), "-lm"], check=True)
    assert _pins(oracle.load(out)), f"mutant {name} passed every pin"
