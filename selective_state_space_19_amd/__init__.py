"""MI355X-native selective state-space scan: S6 scan, decode step, Mamba-2 SSD.

Every operation runs in libmssm.so's HIP kernels (gfx950).  This module only
checks tensors and marshals pointers and the current HIP stream through the
C ABI declared in include/mssm.h; PyTorch provides device memory and streams.
There is no CPU fallback: calling on CPU tensors, or without the built
library, raises.
"""
from __future__ import annotations

from ._lib import MSSM_BF16, MSSM_F32, MssmError, check, lib

__all__ = ["selective_scan", "selective_scan_fused", "selective_scan_bwd", "selective_scan_bwd_workspace_size",
           "state_update", "ssd_chunk", "ssd_chunk_noalloc", "ssd_state_update", "ssd_workspace_size", "MssmError",
           "lib"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MSSM_F32
    if t.dtype == torch.bfloat16:
        return MSSM_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _dev(t, name, shape=None, dtype=None, device=None, written=False):
    """Check a tensor argument.  Inputs that are not contiguous are copied;
    a tensor the kernel writes (an output, a workspace, a state updated in
    place) must be contiguous itself, since a copy would take the writes."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if written:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous (the kernel writes it in place)")
        return t
    return t if t.is_contiguous() else t.contiguous()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _stream(stream, device, *tensors):
    """The stream handle to launch on.  Copies and allocations above were
    made on the current stream; when the caller names another stream, it
    first waits for the current one, and every tensor handed to the kernel
    is marked as in use on it, so the caching allocator does not reuse a
    temporary while the kernel may still read or write it."""
    torch = _torch()
    cur = torch.cuda.current_stream(device)
    if stream is None or stream == cur:
        return cur.cuda_stream
    stream.wait_stream(cur)
    for t in tensors:
        if t is not None:
            t.record_stream(stream)
    return stream.cuda_stream


def selective_scan(u, delta, A, B, C, D=None, z=None, h0=None, *, return_final_state=False,
                   out=None, h_final=None, stream=None, zoh=False, save_workspace=None):
    """S6 scan.  u, delta, z: [b, d, L]; B, C: [b, N, L] (float32 or bfloat16,
    all the same); A: [d, N] float32; D: [d] float32; h0: [b, d, N] float32.
    Returns y [b, d, L] (u's dtype), and h_final [b, d, N] float32 if asked.
    zoh: the zero-order-hold input term (exp(delta A) - 1) / A * B instead of
    the Euler delta * B.  save_workspace: a GPU buffer of at least
    selective_scan_bwd_workspace_size(b, d, L, N) bytes that also receives the
    states selective_scan_bwd(..., workspace=it, saved=True) starts from."""
    torch = _torch()
    dev = u.device
    u = _dev(u, "u")
    bsz, dim, L = u.shape
    N = A.shape[-1]
    dt = u.dtype
    code = _dtype_code(u)
    delta = _dev(delta, "delta", u.shape, dt, dev)
    z = _dev(z, "z", u.shape, dt, dev)
    B = _dev(B, "B", (bsz, N, L), dt, dev)
    C = _dev(C, "C", (bsz, N, L), dt, dev)
    A = _dev(A, "A", (dim, N), torch.float32, dev)
    D = _dev(D, "D", (dim,), torch.float32, dev)
    h0 = _dev(h0, "h0", (bsz, dim, N), torch.float32, dev)
    y = _dev(out if out is not None else torch.empty_like(u), "out", u.shape, dt, dev, written=True)
    hf = None
    if return_final_state or h_final is not None:
        hf = h_final if h_final is not None else torch.empty((bsz, dim, N), dtype=torch.float32, device=dev)
        hf = _dev(hf, "h_final", (bsz, dim, N), torch.float32, dev, written=True)
    ins = (u, delta, A, B, C, D, z, h0, y, hf)
    if save_workspace is not None:
        if zoh:
            raise ValueError("save_workspace is for the Euler scan (the backward pass is of that scan)")
        ws = _dev(save_workspace, "save_workspace", device=dev, written=True)
        check(lib().mssm_selective_scan_fwd_save(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                                 _ptr(h0), _ptr(y), _ptr(hf), bsz, dim, L, N, _ptr(ws),
                                                 _nbytes(ws), code, _stream(stream, dev, *ins, ws)))
    else:
        fn = lib().mssm_selective_scan_zoh_fwd if zoh else lib().mssm_selective_scan_fwd
        check(fn(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(hf),
                 bsz, dim, L, N, code, _stream(stream, dev, *ins)))
    return (y, hf) if hf is not None else y


def selective_scan_fused(x, conv_w, delta_raw, A, B, C, D=None, z=None, h0=None, *, conv_b=None, conv_init=None,
                         delta_bias=None, return_final_state=False, out=None, h_final=None, stream=None):
    """S6 scan with its front end: u = silu(causal conv1d(x; conv_w, conv_b,
    history conv_init)), delta = softplus(delta_raw + delta_bias).  x,
    delta_raw, z: [b, d, L]; conv_w: [d, K] float32 (K <= 4); conv_b,
    delta_bias: [d] float32; conv_init: [b, d, K-1] (x's dtype); the rest as
    selective_scan."""
    torch = _torch()
    dev = x.device
    x = _dev(x, "x")
    bsz, dim, L = x.shape
    N = A.shape[-1]
    dt = x.dtype
    code = _dtype_code(x)
    K = conv_w.shape[-1]
    conv_w = _dev(conv_w, "conv_w", (dim, K), torch.float32, dev)
    conv_b = _dev(conv_b, "conv_b", (dim,), torch.float32, dev)
    conv_init = _dev(conv_init, "conv_init", (bsz, dim, K - 1), dt, dev)
    delta_raw = _dev(delta_raw, "delta_raw", x.shape, dt, dev)
    delta_bias = _dev(delta_bias, "delta_bias", (dim,), torch.float32, dev)
    z = _dev(z, "z", x.shape, dt, dev)
    B = _dev(B, "B", (bsz, N, L), dt, dev)
    C = _dev(C, "C", (bsz, N, L), dt, dev)
    A = _dev(A, "A", (dim, N), torch.float32, dev)
    D = _dev(D, "D", (dim,), torch.float32, dev)
    h0 = _dev(h0, "h0", (bsz, dim, N), torch.float32, dev)
    y = _dev(out if out is not None else torch.empty_like(x), "out", x.shape, dt, dev, written=True)
    hf = None
    if return_final_state or h_final is not None:
        hf = h_final if h_final is not None else torch.empty((bsz, dim, N), dtype=torch.float32, device=dev)
        hf = _dev(hf, "h_final", (bsz, dim, N), torch.float32, dev, written=True)
    s = _stream(stream, dev, x, conv_w, conv_b, conv_init, delta_raw, delta_bias, A, B, C, D, z, h0, y, hf)
    check(lib().mssm_selective_scan_fused_fwd(_ptr(x), _ptr(conv_w), _ptr(conv_b), _ptr(conv_init), _ptr(delta_raw),
                                              _ptr(delta_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                              _ptr(h0), _ptr(y), _ptr(hf), bsz, dim, L, N, K, code, s))
    return (y, hf) if hf is not None else y


def selective_scan_bwd_workspace_size(batch, d_inner, seqlen, d_state):
    return int(lib().mssm_selective_scan_bwd_workspace_size(batch, d_inner, seqlen, d_state))


def selective_scan_bwd(u, delta, A, B, C, dout, D=None, z=None, h0=None, dh_final=None, *, workspace=None,
                       saved=False, stream=None):
    """Gradients of the S6 scan for the loss sum(dout * y) + sum(dh_final *
    h_final).  Inputs as selective_scan; dout: [b, d, L] (u's dtype);
    dh_final: [b, d, N] float32.  Returns a dict: du, ddelta (and dz if z)
    [b, d, L] in u's dtype; dA [d, N], dB, dC [b, N, L], dD [d] (if D) and
    dh0 [b, d, N] (if h0) in float32.  saved: `workspace` holds the states
    that selective_scan(..., save_workspace=workspace) kept for these inputs."""
    torch = _torch()
    dev = u.device
    u = _dev(u, "u")
    bsz, dim, L = u.shape
    N = A.shape[-1]
    dt = u.dtype
    code = _dtype_code(u)
    delta = _dev(delta, "delta", u.shape, dt, dev)
    dout = _dev(dout, "dout", u.shape, dt, dev)
    z = _dev(z, "z", u.shape, dt, dev)
    B = _dev(B, "B", (bsz, N, L), dt, dev)
    C = _dev(C, "C", (bsz, N, L), dt, dev)
    A = _dev(A, "A", (dim, N), torch.float32, dev)
    D = _dev(D, "D", (dim,), torch.float32, dev)
    h0 = _dev(h0, "h0", (bsz, dim, N), torch.float32, dev)
    dh_final = _dev(dh_final, "dh_final", (bsz, dim, N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u), "dA": torch.empty((dim, N), **f32),
         "dB": torch.empty((bsz, N, L), **f32), "dC": torch.empty((bsz, N, L), **f32)}
    g["dD"] = torch.empty((dim,), **f32) if D is not None else None
    g["dz"] = torch.empty_like(u) if z is not None else None
    g["dh0"] = torch.empty((bsz, dim, N), **f32) if h0 is not None else None
    need = selective_scan_bwd_workspace_size(bsz, dim, L, N)
    if workspace is None:
        if saved:
            raise ValueError("saved=True needs the workspace the forward call filled")
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    workspace = _dev(workspace, "workspace", device=dev, written=True)
    s = _stream(stream, dev, u, delta, A, B, C, D, z, h0, dout, dh_final, workspace, *g.values())
    fn = lib().mssm_selective_scan_bwd_saved if saved else lib().mssm_selective_scan_bwd
    check(fn(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dout),
             _ptr(dh_final), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
             _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dh0"]), bsz, dim, L, N, _ptr(workspace),
             _nbytes(workspace), code, s))
    return {k: v for k, v in g.items() if v is not None}


def state_update(state, u, delta, A, B, C, D=None, z=None, *, out=None, stream=None):
    """One decode token; `state` [b, d, N] float32 is updated in place.
    u, delta, z: [b, d]; B, C: [b, N]; A: [d, N]; D: [d].  Returns y [b, d]."""
    torch = _torch()
    dev = state.device
    state = _dev(state, "state", dtype=torch.float32, written=True)
    bsz, dim, N = state.shape
    dt = u.dtype
    code = _dtype_code(u)
    u = _dev(u, "u", (bsz, dim), dt, dev)
    delta = _dev(delta, "delta", (bsz, dim), dt, dev)
    z = _dev(z, "z", (bsz, dim), dt, dev)
    B = _dev(B, "B", (bsz, N), dt, dev)
    C = _dev(C, "C", (bsz, N), dt, dev)
    A = _dev(A, "A", (dim, N), torch.float32, dev)
    D = _dev(D, "D", (dim,), torch.float32, dev)
    y = _dev(out if out is not None else torch.empty((bsz, dim), dtype=dt, device=dev), "out", (bsz, dim), dt, dev,
             written=True)
    s = _stream(stream, dev, state, u, delta, A, B, C, D, z, y)
    check(lib().mssm_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                  _ptr(z), _ptr(y), bsz, dim, N, code, s))
    return y


def ssd_state_update(state, x, dt, A, B, C, D=None, z=None, *, out=None, stream=None):
    """One Mamba-2 decode token; `state` [b, H, P, N] float32 is updated in
    place.  x, z: [b, H, P]; dt: [b, H]; B, C: [b, G, N]; A, D: [H] float32.
    Returns y [b, H, P]."""
    torch = _torch()
    dev = state.device
    state = _dev(state, "state", dtype=torch.float32, written=True)
    bsz, H, P, N = state.shape
    G = B.shape[1]
    ty = x.dtype
    code = _dtype_code(x)
    x = _dev(x, "x", (bsz, H, P), ty, dev)
    dt = _dev(dt, "dt", (bsz, H), ty, dev)
    z = _dev(z, "z", (bsz, H, P), ty, dev)
    B = _dev(B, "B", (bsz, G, N), ty, dev)
    C = _dev(C, "C", (bsz, G, N), ty, dev)
    A = _dev(A, "A", (H,), torch.float32, dev)
    D = _dev(D, "D", (H,), torch.float32, dev)
    y = _dev(out if out is not None else torch.empty((bsz, H, P), dtype=ty, device=dev), "out", (bsz, H, P), ty,
             dev, written=True)
    s = _stream(stream, dev, state, x, dt, A, B, C, D, z, y)
    check(lib().mssm_ssd_state_update(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                      _ptr(z), _ptr(y), bsz, H, P, N, G, code, s))
    return y


def ssd_workspace_size(batch, seqlen, nheads, headdim, d_state, ngroups=1, chunk=256):
    return int(lib().mssm_ssd_workspace_size(batch, seqlen, nheads, headdim, d_state, ngroups, chunk))


def ssd_chunk(x, dt, A, B, C, D=None, z=None, h0=None, *, chunk=256, return_final_state=False,
              out=None, h_final=None, workspace=None, stream=None):
    """Mamba-2 SSD.  x, z: [b, L, H, P]; dt: [b, L, H]; B, C: [b, L, G, N]
    (bfloat16); A, D: [H] float32; h0: [b, H, P, N] float32.  Returns y
    [b, L, H, P] bfloat16, and h_final [b, H, P, N] float32 if asked."""
    torch = _torch()
    dev = x.device
    x = _dev(x, "x")
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    ty = x.dtype
    code = _dtype_code(x)
    dt = _dev(dt, "dt", (bsz, L, H), ty, dev)
    B = _dev(B, "B", (bsz, L, G, N), ty, dev)
    C = _dev(C, "C", (bsz, L, G, N), ty, dev)
    z = _dev(z, "z", x.shape, ty, dev)
    A = _dev(A, "A", (H,), torch.float32, dev)
    D = _dev(D, "D", (H,), torch.float32, dev)
    h0 = _dev(h0, "h0", (bsz, H, P, N), torch.float32, dev)
    y = _dev(out if out is not None else torch.empty_like(x), "out", x.shape, ty, dev, written=True)
    hf = None
    if return_final_state or h_final is not None:
        hf = h_final if h_final is not None else torch.empty((bsz, H, P, N), dtype=torch.float32, device=dev)
        hf = _dev(hf, "h_final", (bsz, H, P, N), torch.float32, dev, written=True)
    need = ssd_workspace_size(bsz, L, H, P, N, G, chunk)
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ws = _dev(ws, "workspace", device=dev, written=True)
    s = _stream(stream, dev, x, dt, A, B, C, D, z, h0, y, hf, ws)
    check(lib().mssm_ssd_chunk_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                   _ptr(y), _ptr(hf), bsz, L, H, P, N, G, chunk, _ptr(ws), _nbytes(ws), code, s))
    return (y, hf) if hf is not None else y


def ssd_chunk_noalloc(x, dt, A, B, C, D=None, z=None, h0=None, *, out, h_final=None, chunk=256, stream=None):
    """ssd_chunk for callers that cannot allocate (mssm_ssd_chunk_fwd_noalloc):
    the library's static per-GPU scratch replaces the workspace, and this
    wrapper allocates nothing either -- every tensor, `out` (and `h_final` if
    wanted) included, is the caller's and must already be contiguous.  Calls
    that may overlap on one GPU share the scratch and must not be issued."""
    torch = _torch()
    dev = x.device
    x = _dev(x, "x", written=True)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    ty = x.dtype
    code = _dtype_code(x)
    dt = _dev(dt, "dt", (bsz, L, H), ty, dev, written=True)
    B = _dev(B, "B", (bsz, L, G, N), ty, dev, written=True)
    C = _dev(C, "C", (bsz, L, G, N), ty, dev, written=True)
    z = _dev(z, "z", x.shape, ty, dev, written=True)
    A = _dev(A, "A", (H,), torch.float32, dev, written=True)
    D = _dev(D, "D", (H,), torch.float32, dev, written=True)
    h0 = _dev(h0, "h0", (bsz, H, P, N), torch.float32, dev, written=True)
    y = _dev(out, "out", x.shape, ty, dev, written=True)
    hf = _dev(h_final, "h_final", (bsz, H, P, N), torch.float32, dev, written=True)
    cur = torch.cuda.current_stream(dev)
    s = (stream if stream is not None else cur).cuda_stream
    check(lib().mssm_ssd_chunk_fwd_noalloc(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                           _ptr(y), _ptr(hf), bsz, L, H, P, N, G, chunk, code, s))
    return (y, hf) if hf is not None else y
