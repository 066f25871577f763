"""fp64 CPU oracle for the selective state-space scan -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding in ``selective_state_space_19_amd``) never imports it, and
it never imports the product.

The arithmetic lives in ``mssm_oracle.c`` (a plain sequential recurrence in
fp64, one thread per block of independent channels); this module only
converts arrays to contiguous float64 and calls it.  See the C file's header
for what is computed and which passages of the pages it follows:

* S6 selective scan -- "Mamba Architecture Details" page, "Selective State
  Space Mechanism / How S6 Works" (update and output); "State-Space Model
  Optimization Patterns" page, section 7 (A_bar = exp(delta*A)) and section 6
  (skip term D x); gated by silu(z).
* Decode step -- the same update for one token, state updated in place
  ("Hardware-Aware Implementation / Parallel Algorithm", sequential mode).
* Mamba-2 SSD -- Optimization Patterns page, section 2 "State Space Duality":
  the recurrence on (head, head channel) with a scalar A per head.
* S6 backward -- the reverse-mode derivative of the scan ("State-Space
  Model Optimization Patterns" page, section 4: the training pass).
* Mamba-2 decode step -- one token of that recurrence with the state
  [b, H, P, N] updated in place ("Mamba - Selective State Space Models"
  page, "Workflow 3": the Mamba-2 block with headdim and d_state).

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, brute force, invariants and hand-worked values (``tests/golden``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mssm_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True, out: str = LIB_PATH, defines: tuple = ()) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if not force and os.path.exists(out):
        return out
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", "-o", out, _SRC, "-lm"]
    cmd[1:1] = [f"-D{d}" for d in defines]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    d = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.oracle_s6_scan.argtypes = [d] * 10 + [L] * 4 + [ctypes.c_int]
    lib.oracle_s6_scan.restype = ctypes.c_int
    lib.oracle_s6_scan_zoh.argtypes = [d] * 10 + [L] * 4 + [ctypes.c_int]
    lib.oracle_s6_scan_zoh.restype = ctypes.c_int
    lib.oracle_state_update.argtypes = [d] * 9 + [L] * 3 + [ctypes.c_int]
    lib.oracle_state_update.restype = ctypes.c_int
    lib.oracle_ssd.argtypes = [d] * 10 + [L] * 6 + [ctypes.c_int]
    lib.oracle_ssd.restype = ctypes.c_int
    lib.oracle_s6_scan_bwd.argtypes = [d] * 18 + [L] * 4 + [ctypes.c_int]
    lib.oracle_s6_scan_bwd.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the compiled oracle (building it if it is not there yet)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(LIB_PATH))
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def s6_scan(u, delta, A, B, C, D=None, z=None, h0=None, nthreads=None, lib=None, zoh=False):
    """Selective scan.  u, delta, z: [b, d, L]; A: [d, N]; B, C: [b, N, L];
    D: [d]; h0: [b, d, N].  Returns (y [b, d, L], h_final [b, d, N]) in fp64.
    zoh: zero-order-hold input term (exp(delta A) - 1) / A * B instead of the
    Euler delta * B (the Optimization Patterns page, section 7)."""
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z, h0 = _f64(D), _f64(z), _f64(h0)
    bsz, dim, L = u.shape
    N = A.shape[1]
    assert delta.shape == u.shape and A.shape == (dim, N)
    assert B.shape == (bsz, N, L) and C.shape == (bsz, N, L)
    assert D is None or D.shape == (dim,)
    assert z is None or z.shape == u.shape
    assert h0 is None or h0.shape == (bsz, dim, N)
    y = np.empty((bsz, dim, L), np.float64)
    hT = np.empty((bsz, dim, N), np.float64)
    lib = lib or load()
    fn = lib.oracle_s6_scan_zoh if zoh else lib.oracle_s6_scan
    rc = fn(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(z), _ptr(h0), _ptr(y), _ptr(hT), bsz, dim, L, N,
            nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_s6_scan failed")
    return y, hT


def state_update(state, u, delta, A, B, C, D=None, z=None, nthreads=None, lib=None):
    """One decode step.  state: [b, d, N] (not modified; the updated state is
    returned); u, delta, z: [b, d]; A: [d, N]; B, C: [b, N]; D: [d].
    Returns (y [b, d], new_state [b, d, N]) in fp64."""
    st = np.array(state, dtype=np.float64, order="C", copy=True)
    u, delta, A, B, C = map(_f64, (u, delta, A, B, C))
    D, z = _f64(D), _f64(z)
    bsz, dim, N = st.shape
    assert u.shape == (bsz, dim) and delta.shape == (bsz, dim)
    assert A.shape == (dim, N) and B.shape == (bsz, N) and C.shape == (bsz, N)
    y = np.empty((bsz, dim), np.float64)
    lib = lib or load()
    rc = lib.oracle_state_update(_ptr(st), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                 _ptr(D), _ptr(z), _ptr(y), bsz, dim, N,
                                 nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_state_update failed")
    return y, st


def ssd(x, dt, A, B, C, D=None, z=None, h0=None, nthreads=None, lib=None):
    """Mamba-2 SSD as the recurrence on heads.  x, z: [b, L, H, P];
    dt: [b, L, H]; A: [H]; B, C: [b, L, G, N]; D: [H]; h0: [b, H, P, N].
    Returns (y [b, L, H, P], h_final [b, H, P, N]) in fp64."""
    x, dt, A, B, C = map(_f64, (x, dt, A, B, C))
    D, z, h0 = _f64(D), _f64(z), _f64(h0)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (bsz, L, H) and A.shape == (H,)
    assert B.shape == (bsz, L, G, N) and C.shape == B.shape and H % G == 0
    assert D is None or D.shape == (H,)
    assert z is None or z.shape == x.shape
    assert h0 is None or h0.shape == (bsz, H, P, N)
    y = np.empty(x.shape, np.float64)
    hT = np.empty((bsz, H, P, N), np.float64)
    lib = lib or load()
    rc = lib.oracle_ssd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                        _ptr(h0), _ptr(y), _ptr(hT), bsz, L, H, P, N, G,
                        nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_ssd failed")
    return y, hT


def ssd_state_update(state, x, dt, A, B, C, D=None, z=None, nthreads=None, lib=None):
    """One Mamba-2 decode token: the SSD recurrence with seqlen 1 starting
    from `state`.  state: [b, H, P, N]; x, z: [b, H, P]; dt: [b, H];
    A: [H]; B, C: [b, G, N]; D: [H].  Returns (y [b, H, P], new state
    [b, H, P, N]) in fp64; `state` itself is not modified."""
    x, dt, B, C = map(_f64, (x, dt, B, C))
    bsz, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert dt.shape == (bsz, H) and B.shape == (bsz, G, N) and C.shape == B.shape
    assert np.shape(state) == (bsz, H, P, N)
    y, hT = ssd(x[:, None], dt[:, None], A, B[:, None], C[:, None], D,
                None if z is None else _f64(z)[:, None], state, nthreads=nthreads, lib=lib)
    return y[:, 0], hT


def causal_conv_silu(x, conv_w, conv_b=None, conv_init=None):
    """u = silu(causal depthwise conv1d(x)) in fp64 ("Mamba Architecture
    Details" page, "Model Configuration": d_conv; "Mamba Block Structure":
    the convolution and SiLU before the SSM).  x: [b, d, L]; conv_w: [d, K];
    conv_b: [d]; conv_init: [b, d, K-1], the K-1 inputs preceding x (zeros if
    None).  u[b, d, t] = silu(sum_k conv_w[d, k] * xx[b, d, t + k] + conv_b[d])
    with xx = concat(conv_init, x) along t."""
    x, w = _f64(x), _f64(conv_w)
    bsz, dim, L = x.shape
    K = w.shape[1]
    init = np.zeros((bsz, dim, K - 1)) if conv_init is None else _f64(conv_init)
    xx = np.concatenate([init, x], axis=2)
    acc = np.zeros((bsz, dim, L))
    for k in range(K):
        acc += w[None, :, k, None] * xx[:, :, k:k + L]
    if conv_b is not None:
        acc += _f64(conv_b)[None, :, None]
    return acc / (1.0 + np.exp(-acc))


def softplus(v):
    """log(1 + e^v), evaluated without overflow."""
    return np.logaddexp(0.0, _f64(v))


def s6_scan_fused(x, conv_w, conv_b, conv_init, delta_raw, delta_bias, A, B, C, D=None, z=None, h0=None,
                  nthreads=None, lib=None):
    """The S6 scan with its front end: u = causal_conv_silu(x, ...),
    delta = softplus(delta_raw + delta_bias), then s6_scan.  Returns
    (y, h_final) in fp64."""
    u = causal_conv_silu(x, conv_w, conv_b, conv_init)
    dr = _f64(delta_raw)
    if delta_bias is not None:
        dr = dr + _f64(delta_bias)[None, :, None]
    return s6_scan(u, softplus(dr), A, B, C, D, z, h0, nthreads=nthreads, lib=lib)


def s6_scan_bwd(u, delta, A, B, C, D=None, z=None, h0=None, dout=None, dhT=None, nthreads=None, lib=None):
    """Reverse-mode derivative of s6_scan for the loss sum(dout * y) +
    sum(dhT * h_final).  Shapes as s6_scan; dout: [b, d, L]; dhT: [b, d, N]
    (zero if None).  Returns a dict of fp64 arrays du, ddelta [b, d, L],
    dA [d, N], dB, dC [b, N, L], dD [d], dz [b, d, L] (if z), dh0
    [b, d, N] (if h0)."""
    u, delta, A, B, C, dout = map(_f64, (u, delta, A, B, C, dout))
    D, z, h0, dhT = _f64(D), _f64(z), _f64(h0), _f64(dhT)
    bsz, dim, L = u.shape
    N = A.shape[1]
    out = dict(du=np.empty((bsz, dim, L)), ddelta=np.empty((bsz, dim, L)), dA=np.empty((dim, N)),
               dB=np.empty((bsz, N, L)), dC=np.empty((bsz, N, L)), dD=np.empty(dim))
    dz = np.empty((bsz, dim, L)) if z is not None else None
    dh0 = np.empty((bsz, dim, N)) if h0 is not None else None
    lib = lib or load()
    rc = lib.oracle_s6_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                _ptr(dout), _ptr(dhT), _ptr(out["du"]), _ptr(out["ddelta"]), _ptr(out["dA"]),
                                _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(dz), _ptr(dh0),
                                bsz, dim, L, N, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_s6_scan_bwd failed")
    if dz is not None:
        out["dz"] = dz
    if dh0 is not None:
        out["dh0"] = dh0
    return out
