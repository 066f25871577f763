"""Seeded synthetic inputs with the shapes and distributions of Mamba layers.

This module draws random numbers and rounds them to the storage dtype; it
holds none of the scan's arithmetic.  Both the HIP path and the fp64 oracle
consume exactly the arrays produced here (the oracle widens bf16 exactly).

Distributions ("Mamba Architecture Details" page, "Initialization Strategy"):
the per-channel step dt is log-uniform in [dt_min, dt_max] = [1e-3, 0.1],
floored at 1e-4; the per-token step is delta = softplus(0.5*eps + softplus^-1(dt))
with eps ~ N(0, 1), so that delta > 0 and is centred on dt.  u, z, B, C ~ N(0, 1);
A[d, n] = -(n + 1) (negative, as the page requires); D = 1.  B and C are
per token and shared by all channels of a batch row ([B, N, L]).

``varied=True`` (any generator) instead draws the per-channel / per-head
parameters the way the same page initialises a layer: A[d, n] = -exp(U[0, 1))
for every (channel, state) and D ~ N(0, 1) per channel (Mamba-2: D_h ~ N(0, 1)
per head; A_h is per head already).  These come from their own generator
``PCG64([seed, 2_000_000])``, so every other array is the same as without it.
Parity tests use it so that a kernel that reads A or D of the wrong channel or
head cannot pass.

Mamba-2 SSD workloads ("Mamba - Selective State Space Models" page, "Workflow 3 / Mamba-2"): headdim 64,
d_state 128, ngroups 1; the scalar per-head A_h = -U[1, 16); dt per head.

RNG: numpy PCG64.  The base generator ``PCG64(seed)`` draws the small
per-channel / per-head parameters; batch row ``b`` uses its own child
``PCG64([seed, b])`` (decode step ``s`` uses ``PCG64([seed, 1000 + s])``), so
any batch row can be regenerated alone.  Values are drawn in fp64 and rounded
once: fp32 by IEEE round-to-nearest-even, bf16 by round-to-nearest-even of
that fp32 value.  bf16 arrays are carried as uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

DT_MIN, DT_MAX, DT_FLOOR = 1e-3, 0.1, 1e-4


# --------------------------------------------------------------------------
# dtype helpers
# --------------------------------------------------------------------------
def to_bf16_bits(x) -> np.ndarray:
    """Round to bf16 (RNE of the fp32 value); returns uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint32, copy=True)
    bits += np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    bits >>= np.uint32(16)
    return bits.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype ("f32" -> float32, "bf16" -> uint16 bits)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def widen(a, dtype: str) -> np.ndarray:
    """Exact widening of a stored array to float64 (what the oracle reads)."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _softplus_inv(y):
    return y + np.log(-np.expm1(-y))


def _dt_per_channel(rng, n):
    lo, hi = np.log(DT_MIN), np.log(DT_MAX)
    return np.maximum(np.exp(rng.random(n) * (hi - lo) + lo), DT_FLOOR)


def _delta(rng, dt_inv, shape):
    """softplus(0.5*eps + softplus^-1(dt)); dt_inv broadcasts against shape."""
    return _softplus(0.5 * rng.standard_normal(shape) + dt_inv)


def _varied_params(seed, d_inner, d_state):
    """A[d, n] = -exp(U[0, 1)) per (channel, state) and D[d] ~ N(0, 1) per
    channel ("Mamba Architecture Details", Initialization Strategy), from a
    generator of their own."""
    g = np.random.Generator(np.random.PCG64([seed, 2_000_000]))
    A = (-np.exp(g.random((d_inner, d_state)))).astype(np.float32)
    D = g.standard_normal(d_inner).astype(np.float32)
    return A, D


def _varied_head_skip(seed, nheads):
    """D_h ~ N(0, 1) per head, from a generator of its own."""
    g = np.random.Generator(np.random.PCG64([seed, 2_000_000]))
    return g.standard_normal(nheads).astype(np.float32)


def periodic_window(a, axis: int, start: int, length: int) -> np.ndarray:
    """Tokens start .. start+length-1 of the sequence that repeats `a` along
    `axis` (a holds one period).  Used to build sequences far longer than
    can be generated or checked whole, from one seeded period."""
    if a is None:
        return None
    idx = (start + np.arange(length)) % a.shape[axis]
    return np.take(a, idx, axis=axis)


# --------------------------------------------------------------------------
# S6 selective scan inputs
# --------------------------------------------------------------------------
def s6_inputs(batch, d_inner, seqlen, d_state, dtype="f32", seed=0,
              gate=True, skip=True, init_state=False, varied=False):
    """u, delta, z: [batch, d_inner, seqlen]; B, C: [batch, d_state, seqlen]
    (stored dtype); A: [d_inner, d_state] f32; D: [d_inner] f32 or None;
    h0: [batch, d_inner, d_state] f32 ~ N(0, 0.1) or None."""
    base = np.random.Generator(np.random.PCG64(seed))
    dt_inv = _softplus_inv(_dt_per_channel(base, d_inner))[:, None]
    h0 = None
    if init_state:
        h0 = base.normal(0.0, 0.1, (batch, d_inner, d_state)).astype(np.float32)
    shp = (batch, d_inner, seqlen)
    store = np.uint16 if dtype == "bf16" else np.float32
    u = np.empty(shp, store)
    dl = np.empty(shp, store)
    z = np.empty(shp, store) if gate else None
    Bm = np.empty((batch, d_state, seqlen), store)
    Cm = np.empty((batch, d_state, seqlen), store)
    for b in range(batch):
        rng = np.random.Generator(np.random.PCG64([seed, b]))
        dl[b] = round_to(_delta(rng, dt_inv, (d_inner, seqlen)), dtype)
        u[b] = round_to(rng.standard_normal((d_inner, seqlen)), dtype)
        zb = rng.standard_normal((d_inner, seqlen))
        if gate:
            z[b] = round_to(zb, dtype)
        Bm[b] = round_to(rng.standard_normal((d_state, seqlen)), dtype)
        Cm[b] = round_to(rng.standard_normal((d_state, seqlen)), dtype)
    A = np.broadcast_to(-(np.arange(d_state, dtype=np.float32) + 1.0), (d_inner, d_state)).copy()
    D = np.ones(d_inner, np.float32) if skip else None
    if varied:
        A, Dv = _varied_params(seed, d_inner, d_state)
        D = Dv if skip else None
    return dict(u=u, delta=dl, A=A, B=Bm, C=Cm, D=D, z=z, h0=h0, dtype=dtype)


def s6_fused_inputs(batch, d_inner, seqlen, d_state, d_conv=4, dtype="f32", seed=0, gate=True, skip=True,
                    init_state=False, conv_history=False, varied=False):
    """Inputs of the scan with its front end: x (before the causal conv) and
    the raw step delta_raw (before softplus) [B, D, L] in the stored dtype;
    conv_w [D, d_conv] and conv_b [D] ~ U(-1/sqrt(d_conv), 1/sqrt(d_conv))
    (the default init of a depthwise conv1d); delta_bias[d] =
    softplus^-1(dt[d]) and delta_raw = 0.5 eps, so that
    softplus(delta_raw + delta_bias) has the distribution of s6_inputs'
    delta; conv_init [B, D, d_conv - 1] (stored dtype) if conv_history; the
    rest as s6_inputs."""
    base = np.random.Generator(np.random.PCG64(seed))
    dt_inv = _softplus_inv(_dt_per_channel(base, d_inner))
    bound = 1.0 / np.sqrt(d_conv)
    conv_w = base.uniform(-bound, bound, (d_inner, d_conv)).astype(np.float32)
    conv_b = base.uniform(-bound, bound, d_inner).astype(np.float32)
    h0 = base.normal(0.0, 0.1, (batch, d_inner, d_state)).astype(np.float32) if init_state else None
    store = np.uint16 if dtype == "bf16" else np.float32
    x = np.empty((batch, d_inner, seqlen), store)
    dr = np.empty((batch, d_inner, seqlen), store)
    z = np.empty((batch, d_inner, seqlen), store) if gate else None
    Bm = np.empty((batch, d_state, seqlen), store)
    Cm = np.empty((batch, d_state, seqlen), store)
    ci = np.empty((batch, d_inner, d_conv - 1), store) if conv_history else None
    for b in range(batch):
        rng = np.random.Generator(np.random.PCG64([seed, b]))
        dr[b] = round_to(0.5 * rng.standard_normal((d_inner, seqlen)), dtype)
        x[b] = round_to(rng.standard_normal((d_inner, seqlen)), dtype)
        Bm[b] = round_to(rng.standard_normal((d_state, seqlen)), dtype)
        Cm[b] = round_to(rng.standard_normal((d_state, seqlen)), dtype)
        if gate:
            z[b] = round_to(rng.standard_normal((d_inner, seqlen)), dtype)
        if conv_history:
            ci[b] = round_to(rng.standard_normal((d_inner, d_conv - 1)), dtype)
    A = np.broadcast_to(-(np.arange(d_state, dtype=np.float32) + 1.0), (d_inner, d_state)).copy()
    D = np.ones(d_inner, np.float32) if skip else None
    if varied:
        A, Dv = _varied_params(seed, d_inner, d_state)
        D = Dv if skip else None
    return dict(x=x, conv_w=conv_w, conv_b=conv_b, conv_init=ci, delta_raw=dr,
                delta_bias=dt_inv.astype(np.float32), A=A, B=Bm, C=Cm, D=D, z=z, h0=h0, dtype=dtype)


# --------------------------------------------------------------------------
# Decode (single-token state update) inputs
# --------------------------------------------------------------------------
def decode_initial(batch, d_inner, d_state, seed=0, varied=False):
    """Initial state [batch, d_inner, d_state] f32 ~ N(0, 0.1); A, D; and the
    per-channel softplus^-1(dt) used by every step."""
    base = np.random.Generator(np.random.PCG64(seed))
    state = base.normal(0.0, 0.1, (batch, d_inner, d_state)).astype(np.float32)
    dt_inv = _softplus_inv(_dt_per_channel(base, d_inner))[None, :]
    A = np.broadcast_to(-(np.arange(d_state, dtype=np.float32) + 1.0), (d_inner, d_state)).copy()
    D = np.ones(d_inner, np.float32)
    if varied:
        A, D = _varied_params(seed, d_inner, d_state)
    return dict(state=state, A=A, D=D, dt_inv=dt_inv)


def decode_step(init, step, batch, d_inner, d_state, dtype="bf16", seed=0, gate=True):
    """Per-token inputs of decode step `step`: u, delta, z [batch, d_inner];
    B, C [batch, d_state] (stored dtype)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1000 + step]))
    dl = round_to(_delta(rng, init["dt_inv"], (batch, d_inner)), dtype)
    u = round_to(rng.standard_normal((batch, d_inner)), dtype)
    zb = rng.standard_normal((batch, d_inner))
    z = round_to(zb, dtype) if gate else None
    Bm = round_to(rng.standard_normal((batch, d_state)), dtype)
    Cm = round_to(rng.standard_normal((batch, d_state)), dtype)
    return dict(u=u, delta=dl, z=z, B=Bm, C=Cm, dtype=dtype)


# --------------------------------------------------------------------------
# Mamba-2 SSD inputs
# --------------------------------------------------------------------------
def ssd_inputs(batch, seqlen, nheads, headdim, d_state, ngroups=1, dtype="bf16",
               seed=0, gate=False, skip=True, init_state=False, varied=False):
    """x, z: [batch, seqlen, nheads, headdim]; dt: [batch, seqlen, nheads];
    B, C: [batch, seqlen, ngroups, d_state] (stored dtype); A: [nheads] f32
    = -U[1, 16); D: [nheads] f32 or None; h0: [batch, nheads, headdim,
    d_state] f32 ~ N(0, 0.1) or None."""
    base = np.random.Generator(np.random.PCG64(seed))
    A = (-base.uniform(1.0, 16.0, nheads)).astype(np.float32)
    dt_inv = _softplus_inv(_dt_per_channel(base, nheads))[None, :]
    h0 = None
    if init_state:
        h0 = base.normal(0.0, 0.1, (batch, nheads, headdim, d_state)).astype(np.float32)
    store = np.uint16 if dtype == "bf16" else np.float32
    x = np.empty((batch, seqlen, nheads, headdim), store)
    dt = np.empty((batch, seqlen, nheads), store)
    z = np.empty(x.shape, store) if gate else None
    Bm = np.empty((batch, seqlen, ngroups, d_state), store)
    Cm = np.empty((batch, seqlen, ngroups, d_state), store)
    for b in range(batch):
        rng = np.random.Generator(np.random.PCG64([seed, b]))
        dt[b] = round_to(_delta(rng, dt_inv, (seqlen, nheads)), dtype)
        x[b] = round_to(rng.standard_normal((seqlen, nheads, headdim)), dtype)
        Bm[b] = round_to(rng.standard_normal((seqlen, ngroups, d_state)), dtype)
        Cm[b] = round_to(rng.standard_normal((seqlen, ngroups, d_state)), dtype)
        if gate:
            z[b] = round_to(rng.standard_normal((seqlen, nheads, headdim)), dtype)
    D = np.ones(nheads, np.float32) if skip else None
    if varied and skip:
        D = _varied_head_skip(seed, nheads)
    return dict(x=x, dt=dt, A=A, B=Bm, C=Cm, D=D, z=z, h0=h0, dtype=dtype)


# --------------------------------------------------------------------------
# Mamba-2 decode (single-token SSD state update) inputs
# --------------------------------------------------------------------------
def mamba2_decode_initial(batch, nheads, headdim, d_state, seed=0, varied=False):
    """Initial state [batch, nheads, headdim, d_state] f32 ~ N(0, 0.1); A [nheads]
    = -U[1, 16); D [nheads] = 1; and the per-head softplus^-1(dt) used by every step."""
    base = np.random.Generator(np.random.PCG64(seed))
    A = (-base.uniform(1.0, 16.0, nheads)).astype(np.float32)
    dt_inv = _softplus_inv(_dt_per_channel(base, nheads))[None, :]
    state = base.normal(0.0, 0.1, (batch, nheads, headdim, d_state)).astype(np.float32)
    D = np.ones(nheads, np.float32)
    if varied:
        D = _varied_head_skip(seed, nheads)
    return dict(state=state, A=A, D=D, dt_inv=dt_inv)


def mamba2_decode_step(init, step, batch, nheads, headdim, d_state, ngroups=1, dtype="bf16", seed=0,
                       gate=True):
    """Per-token inputs of Mamba-2 decode step `step`: x, z [batch, nheads, headdim];
    dt [batch, nheads]; B, C [batch, ngroups, d_state] (stored dtype)."""
    rng = np.random.Generator(np.random.PCG64([seed, 1000 + step]))
    dt = round_to(_delta(rng, init["dt_inv"], (batch, nheads)), dtype)
    x = round_to(rng.standard_normal((batch, nheads, headdim)), dtype)
    zb = rng.standard_normal((batch, nheads, headdim))
    z = round_to(zb, dtype) if gate else None
    Bm = round_to(rng.standard_normal((batch, ngroups, d_state)), dtype)
    Cm = round_to(rng.standard_normal((batch, ngroups, d_state)), dtype)
    return dict(x=x, dt=dt, z=z, B=Bm, C=Cm, dtype=dtype)


# --------------------------------------------------------------------------
# The named workloads (Mamba layer shapes from the pages' model table)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "s6" | "decode" | "ssd" | "decode2"
    dtype: str
    seed: int
    shape: dict = field(default_factory=dict)
    note: str = ""


WORKLOADS = {
    # 1 x 32 channels x 64 tokens, d_state 16, fp32: small enough for brute force.
    "s6_tiny_f32": Workload("s6_tiny_f32", "s6", "f32", 19000,
                            dict(batch=1, d_inner=32, seqlen=64, d_state=16),
                            "tiny S6 scan"),
    # Mamba-130M layer: d_model 768, expand 2 -> d_inner 1536.
    "s6_mamba130m_f32": Workload("s6_mamba130m_f32", "s6", "f32", 19001,
                                 dict(batch=8, d_inner=1536, seqlen=2048, d_state=16),
                                 "Mamba-130M layer shape S6 scan"),
    # Mamba-1.4B layer: d_model 2048 -> d_inner 4096; bf16 in, fp32 state, final state out.
    "s6_mamba1p4b_bf16": Workload("s6_mamba1p4b_bf16", "s6", "bf16", 19002,
                                  dict(batch=4, d_inner=4096, seqlen=8192, d_state=16),
                                  "Mamba-1.4B layer shape S6 scan"),
    # Mamba-2.8B layer decode: d_model 2560 -> d_inner 5120; 256 successive tokens.
    "decode_mamba2p8b_bf16": Workload("decode_mamba2p8b_bf16", "decode", "bf16", 19003,
                                      dict(batch=64, d_inner=5120, d_state=16, steps=256),
                                      "Mamba-2.8B decode state update"),
    # Mamba-2 layer: 32 heads x headdim 64 = 2048 = 2 x d_model 1024; chunk 256.
    "ssd_mamba2_bf16": Workload("ssd_mamba2_bf16", "ssd", "bf16", 19004,
                                dict(batch=4, seqlen=4096, nheads=32, headdim=64,
                                     d_state=128, ngroups=1, chunk=256),
                                "Mamba-2 SSD chunked scan"),
    # Mamba-1.4B layer S6 scan with its front end (causal conv d_conv 4 + SiLU, softplus step).
    "s6fused_mamba1p4b_bf16": Workload("s6fused_mamba1p4b_bf16", "s6fused", "bf16", 19006,
                                       dict(batch=4, d_inner=4096, seqlen=8192, d_state=16, d_conv=4),
                                       "Mamba-1.4B layer shape S6 scan with fused conv1d front end"),
    # Mamba-2 layer decode (same layer as above), batch 64, 256 successive tokens.
    "decode_mamba2_bf16": Workload("decode_mamba2_bf16", "decode2", "bf16", 19005,
                                   dict(batch=64, nheads=32, headdim=64, d_state=128, ngroups=1, steps=256),
                                   "Mamba-2 decode state update"),
}
