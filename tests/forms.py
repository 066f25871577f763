"""Independent fp64 formulations used to pin the oracle (tests only).

None of these is the oracle: each reaches the recurrence's result by a
different route, so an index, sign or ordering slip in the oracle's loop
shows up as a disagreement.

* ``closed_form_s6``  -- the recurrence unrolled:
      h_t = (prod_{r<=t} dA_r) h0 + sum_{s<=t} (prod_{r=s+1..t} dA_r) dBu_s,
  brute-forced with explicit products (O(L^2) per channel).
* ``blelloch_s6``     -- the work-efficient up-sweep / down-sweep scan of the
  "State-Space Model Optimization Patterns" page, section 11, with the addition replaced by the
  composition of affine maps h -> a h + b:
      (a1, b1) (+) (a2, b2) = (a1 a2, a2 b1 + b2)   ("apply 1, then 2"),
  which is associative; the scan identity of section 1 then gives every h_t.
* ``ssd_quadratic``   -- Optimization Patterns page, section 2 "State Space Duality": for a
  scalar-per-head A the SSM output is a masked attention-like product
      Y = (Lmask o (C B^T)) (dt o X) + D X,
  Lmask[i, j] = exp(A_h sum_{r=j+1..i} dt_r) for i >= j (a semi-separable
  mask, section 10), plus the decayed contribution of the initial state.
* ``ssd_chunked``     -- Optimization Patterns page, section 9 "Chunked Computation": split into
  chunks, local quadratic form plus the chunk's final state, pass states from
  chunk to chunk, combine.  Used to show chunk-size invariance.
"""
from __future__ import annotations

import numpy as np


def silu(g):
    return g / (1.0 + np.exp(-g))


def closed_form_s6(u, delta, A, B, C, D=None, z=None, h0=None):
    u, delta, A, B, C = (np.asarray(a, np.float64) for a in (u, delta, A, B, C))
    bsz, dim, L = u.shape
    N = A.shape[1]
    y = np.zeros((bsz, dim, L))
    hT = np.zeros((bsz, dim, N))
    for b in range(bsz):
        for d in range(dim):
            dA = np.exp(delta[b, d][:, None] * A[d][None, :])          # [L, N]
            dBu = (delta[b, d] * u[b, d])[:, None] * B[b].T              # [L, N]
            init = np.zeros(N) if h0 is None else np.asarray(h0[b, d], np.float64)
            for t in range(L):
                h = np.prod(dA[: t + 1], axis=0) * init
                for s in range(t + 1):
                    h = h + np.prod(dA[s + 1: t + 1], axis=0) * dBu[s]
                o = float(np.dot(C[b, :, t], h))
                if D is not None:
                    o += float(D[d]) * u[b, d, t]
                if z is not None:
                    o *= silu(float(z[b, d, t]))
                y[b, d, t] = o
                if t == L - 1:
                    hT[b, d] = h
            if L == 0:
                hT[b, d] = init
    return y, hT


def _combine(e1, e2):
    """Affine maps as pairs: apply e1, then e2."""
    a1, b1 = e1
    a2, b2 = e2
    return a1 * a2, a2 * b1 + b2


def _blelloch_exclusive(a, b):
    """Exclusive scan over axis 0 (length a power of two), non-commutative op."""
    n = a.shape[0]
    a = a.copy()
    b = b.copy()
    levels = n.bit_length() - 1
    for d in range(levels):                       # up-sweep (reduce)
        step = 1 << (d + 1)
        for k in range(0, n, step):
            lo, hi = k + (1 << d) - 1, k + step - 1
            a[hi], b[hi] = _combine((a[lo], b[lo]), (a[hi], b[hi]))
    a[n - 1], b[n - 1] = 1.0, 0.0                # identity map
    for d in range(levels - 1, -1, -1):           # down-sweep
        step = 1 << (d + 1)
        for k in range(0, n, step):
            lo, hi = k + (1 << d) - 1, k + step - 1
            ta, tb = a[lo].copy(), b[lo].copy()   # total of the left half
            a[lo], b[lo] = a[hi], b[hi]           # left child: parent's prefix
            a[hi], b[hi] = _combine((a[hi], b[hi]), (ta, tb))  # prefix, then left half
    return a, b


def blelloch_s6(u, delta, A, B, C, D=None, z=None, h0=None):
    u, delta, A, B, C = (np.asarray(a, np.float64) for a in (u, delta, A, B, C))
    bsz, dim, L = u.shape
    N = A.shape[1]
    n = 1 << max(0, (L - 1).bit_length()) if L > 0 else 1
    # elements e_t = (dA_t, dBu_t), laid out [t, b, d, N]; padded with identity
    ea = np.ones((n, bsz, dim, N))
    eb = np.zeros((n, bsz, dim, N))
    ea[:L] = np.exp(np.transpose(delta, (2, 0, 1))[..., None] * A[None, None])
    eb[:L] = (np.transpose(delta * u, (2, 0, 1))[..., None] *
              np.transpose(B, (2, 0, 1))[:, :, None, :])
    xa, xb = _blelloch_exclusive(ea, eb)
    ia, ib = _combine((xa, xb), (ea, eb))        # inclusive = exclusive (+) e_t
    init = np.zeros((bsz, dim, N)) if h0 is None else np.asarray(h0, np.float64)
    h = ia[:L] * init[None] + ib[:L]             # [L, b, d, N]
    y = np.einsum("tbdn,bnt->bdt", h, C)
    if D is not None:
        y = y + np.asarray(D, np.float64)[None, :, None] * u
    if z is not None:
        y = y * silu(np.asarray(z, np.float64))
    hT = h[L - 1] if L > 0 else init
    return y, hT


def ssd_quadratic(x, dt, A, B, C, D=None, z=None, h0=None):
    x, dt, A, B, C = (np.asarray(a, np.float64) for a in (x, dt, A, B, C))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hT = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // (H // G)
            s = np.cumsum(dt[b, :, h] * A[h])                         # [L]
            low = np.tril(np.ones((L, L), bool))
            mask = np.exp(np.where(low, s[:, None] - s[None, :], 0.0)) * low
            CB = C[b, :, g, :] @ B[b, :, g, :].T                      # [L, L]
            Xd = dt[b, :, h][:, None] * x[b, :, h, :]                 # [L, P]
            Y = (mask * CB) @ Xd
            w = np.exp(s[-1] - s) * dt[b, :, h]                       # [L]
            Hf = (x[b, :, h, :] * w[:, None]).T @ B[b, :, g, :]       # [P, N]
            if h0 is not None:
                H0 = np.asarray(h0[b, h], np.float64)                 # [P, N]
                Y = Y + np.exp(s)[:, None] * (C[b, :, g, :] @ H0.T)
                Hf = Hf + np.exp(s[-1]) * H0
            if D is not None:
                Y = Y + float(D[h]) * x[b, :, h, :]
            if z is not None:
                Y = Y * silu(np.asarray(z[b, :, h, :], np.float64))
            y[b, :, h, :] = Y
            hT[b, h] = Hf
    return y, hT


def ssd_chunked(x, dt, A, B, C, D=None, z=None, h0=None, chunk=4):
    """Catalogue section 9: per chunk a local quadratic form and the chunk's
    final state; states passed sequentially; the two results combined."""
    x, dt, A, B, C = (np.asarray(a, np.float64) for a in (x, dt, A, B, C))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hT = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // (H // G)
            state = np.zeros((P, N)) if h0 is None else np.asarray(h0[b, h], np.float64).copy()
            for c0 in range(0, L, chunk):
                c1 = min(L, c0 + chunk)
                q = c1 - c0
                s = np.cumsum(dt[b, c0:c1, h] * A[h])                 # local cumsum
                low = np.tril(np.ones((q, q), bool))
                mask = np.exp(np.where(low, s[:, None] - s[None, :], 0.0)) * low
                Cc, Bc = C[b, c0:c1, g, :], B[b, c0:c1, g, :]
                Xd = dt[b, c0:c1, h][:, None] * x[b, c0:c1, h, :]
                Y = (mask * (Cc @ Bc.T)) @ Xd                         # local (diagonal block)
                Y = Y + np.exp(s)[:, None] * (Cc @ state.T)           # carried-in state
                w = np.exp(s[-1] - s) * dt[b, c0:c1, h]
                state = np.exp(s[-1]) * state + (x[b, c0:c1, h, :] * w[:, None]).T @ Bc
                if D is not None:
                    Y = Y + float(D[h]) * x[b, c0:c1, h, :]
                if z is not None:
                    Y = Y * silu(np.asarray(z[b, c0:c1, h, :], np.float64))
                y[b, c0:c1, h, :] = Y
            hT[b, h] = state
    return y, hT


def normwise_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)
