"""torch-tensor wrappers of the libssm entry points (marshalling only)."""
from __future__ import annotations

import torch

from ._lib import SSM_BBAR_ZOH, SSM_BF16, SSM_DELTA_SOFTPLUS, SSM_F32, SsmError, load, status_string

_DTYPES = {torch.float32: SSM_F32, torch.bfloat16: SSM_BF16}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"tensor dtype {t.dtype} is not float32 or bfloat16")
    return _DTYPES[t.dtype]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _flags(delta_softplus, bbar):
    if bbar not in ("euler", "zoh"):
        raise ValueError(f"bbar must be 'euler' or 'zoh', not {bbar!r}")
    return (SSM_DELTA_SOFTPLUS if delta_softplus else 0) | (SSM_BBAR_ZOH if bbar == "zoh" else 0)


def _check(name, t, shape, dtype, device, required=True):
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def ssm_status_string(status: int) -> str:
    return status_string(status)


def ssm_scan_fwd_workspace_bytes(batch: int, dim: int, dstate: int, seqlen: int,
                                 dtype: torch.dtype) -> int:
    return int(load().ssm_scan_fwd_workspace_bytes(batch, dim, dstate, seqlen, _DTYPES[dtype]))


def _scan(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, bbar, return_last_state, out,
          workspace, conv):
    lib = load()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    name = "x" if conv is not None else "u"
    _check(name, u, (batch, dim, L), dt, dev)
    _check("delta", delta, (batch, dim, L), dt, dev)
    _check("A", A, (dim, N), torch.float32, dev)
    _check("B", B, (batch, N, L), dt, dev)
    _check("C", C, (batch, N, L), dt, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim, L), dt, dev, required=False)
    _check("delta_bias", delta_bias, (dim,), torch.float32, dev, required=False)
    _check("h0", h0, (batch, dim, N), torch.float32, dev, required=False)
    y = out if out is not None else torch.empty_like(u)
    _check("out", y, (batch, dim, L), dt, dev)
    last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev) if return_last_state else None
    need = int(lib.ssm_scan_fwd_workspace_bytes(batch, dim, N, L, code))
    ws_bytes = 0
    if need > 0:
        if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    flags = _flags(delta_softplus, bbar)
    if conv is None:
        rc = lib.ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(delta_bias), flags, _ptr(h0), _ptr(y), _ptr(last), batch, dim, N,
                              L, code, _ptr(workspace), ws_bytes, stream)
        if rc != 0:
            raise SsmError(rc, "ssm_scan_fwd")
        return (y, last) if return_last_state else y
    w, cb, st_in, want_state = conv
    K = w.shape[1] if w.dim() == 2 else -1
    _check("conv_w", w, (dim, K), torch.float32, dev)
    _check("conv_b", cb, (dim,), torch.float32, dev, required=False)
    _check("conv_state_in", st_in, (batch, dim, K - 1), torch.float32, dev, required=False)
    st_out = (torch.empty((batch, dim, max(K - 1, 0)), dtype=torch.float32, device=dev)
              if want_state else None)
    rc = lib.ssm_conv_scan_fwd(_ptr(u), _ptr(w), _ptr(cb), K, _ptr(st_in),
                               _ptr(st_out) if K > 1 else None, _ptr(delta), _ptr(A), _ptr(B),
                               _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias), flags, _ptr(h0), _ptr(y),
                               _ptr(last), batch, dim, N, L, code, _ptr(workspace), ws_bytes, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_conv_scan_fwd")
    res = (y,)
    if return_last_state:
        res += (last,)
    if want_state:
        res += (st_out,)
    return res[0] if len(res) == 1 else res


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 h0=None, *, bbar="euler", return_last_state=False, out=None, workspace=None):
    """Selective scan over (batch, dim, L) inputs; see include/ssm.h.
    bbar: 'euler' (input term Delta*B*u) or 'zoh' ((exp(Delta*A) - 1)/A*B*u).

    u, delta, z: (batch, dim, L) float32 or bfloat16 (one dtype for all);
    B, C: (batch, N, L) same dtype; A: (dim, N) float32; D, delta_bias: (dim,)
    float32; h0: (batch, dim, N) float32.  Returns y (batch, dim, L) in the
    input dtype, and (y, last_state) when return_last_state is set."""
    return _scan(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, bbar, return_last_state,
                 out, workspace, None)


def ssm_scan_fwd_noalloc(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                         h0=None, *, out, last_state=None, bbar="euler"):
    """ssm_scan_fwd without any allocation: the library's static scratch
    stands in for the workspace, and the caller passes the outputs (out, and
    last_state if wanted).  Nothing here allocates device memory either."""
    lib = load()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    _check("u", u, (batch, dim, L), dt, dev)
    _check("delta", delta, (batch, dim, L), dt, dev)
    _check("A", A, (dim, N), torch.float32, dev)
    _check("B", B, (batch, N, L), dt, dev)
    _check("C", C, (batch, N, L), dt, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim, L), dt, dev, required=False)
    _check("delta_bias", delta_bias, (dim,), torch.float32, dev, required=False)
    _check("h0", h0, (batch, dim, N), torch.float32, dev, required=False)
    _check("out", out, (batch, dim, L), dt, dev)
    _check("last_state", last_state, (batch, dim, N), torch.float32, dev, required=False)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd_noalloc(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                                  _ptr(delta_bias), _flags(delta_softplus, bbar), _ptr(h0), _ptr(out),
                                  _ptr(last_state), batch, dim, N, L, code, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_scan_fwd_noalloc")
    return out


def ssm_conv_scan_fwd(x, conv_w, conv_b, delta, A, B, C, D=None, z=None, delta_bias=None,
                      delta_softplus=True, h0=None, *, conv_state_in=None, return_conv_state=False,
                      bbar="euler", return_last_state=False, out=None, workspace=None):
    """The scan with the causal depthwise conv1d + silu prologue fused in:
    u = silu(conv_b + causal conv of x with conv_w (dim, K), K in 1..4).
    conv_state_in: (batch, dim, K-1) float32, the inputs before t = 0.
    Returns y, then last_state (if return_last_state), then the new conv
    state (if return_conv_state)."""
    return _scan(x, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, bbar, return_last_state,
                 out, workspace, (conv_w, conv_b, conv_state_in, return_conv_state))


def _update(state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, bbar, out, conv):
    lib = load()
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, N = state.shape
    _check("state", state, (batch, dim, N), torch.float32, dev)
    _check("x" if conv is not None else "u", u, (batch, dim), dt, dev)
    _check("delta", delta, (batch, dim), dt, dev)
    _check("A", A, (dim, N), torch.float32, dev)
    _check("B", B, (batch, N), dt, dev)
    _check("C", C, (batch, N), dt, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim), dt, dev, required=False)
    _check("delta_bias", delta_bias, (dim,), torch.float32, dev, required=False)
    y = out if out is not None else torch.empty_like(u)
    _check("out", y, (batch, dim), dt, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    flags = _flags(delta_softplus, bbar)
    if conv is None:
        rc = lib.ssm_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                                  _ptr(D), _ptr(z), _ptr(delta_bias), flags, _ptr(y), batch, dim, N,
                                  code, stream)
        if rc != 0:
            raise SsmError(rc, "ssm_state_update")
        return y
    cs, w, cb = conv
    K = w.shape[1] if w.dim() == 2 else -1
    _check("conv_w", w, (dim, K), torch.float32, dev)
    _check("conv_b", cb, (dim,), torch.float32, dev, required=False)
    _check("conv_state", cs, (batch, dim, K - 1), torch.float32, dev, required=K > 1)
    rc = lib.ssm_conv_state_update(_ptr(cs) if K > 1 else None, _ptr(state), _ptr(u), _ptr(w),
                                   _ptr(cb), K, _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                                   _ptr(z), _ptr(delta_bias), flags, _ptr(y), batch, dim, N, code,
                                   stream)
    if rc != 0:
        raise SsmError(rc, "ssm_conv_state_update")
    return y


def ssm_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=True, *, bbar="euler", out=None):
    """One decode step; `state` (batch, dim, N) float32 is updated in place.
    u, delta, z: (batch, dim); B, C: (batch, N); returns y (batch, dim)."""
    return _update(state, u, delta, A, B, C, D, z, delta_bias, delta_softplus, bbar, out, None)


def ssm_conv_state_update(conv_state, state, x, conv_w, conv_b, delta, A, B, C, D=None, z=None,
                          delta_bias=None, delta_softplus=True, *, bbar="euler", out=None):
    """One decode step with the convolution prologue; conv_state
    (batch, dim, K-1) and state (batch, dim, N) are updated in place."""
    return _update(state, x, delta, A, B, C, D, z, delta_bias, delta_softplus, bbar, out,
                   (conv_state, conv_w, conv_b))


def ssm_scan_bwd_workspace_bytes(batch: int, dim: int, dstate: int, seqlen: int,
                                 dtype: torch.dtype) -> int:
    return int(load().ssm_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, _DTYPES[dtype]))


def _bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, dy, dlast_state, bbar,
         workspace, ckpt):
    lib = load()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    _check("u", u, (batch, dim, L), dt, dev)
    _check("delta", delta, (batch, dim, L), dt, dev)
    _check("A", A, (dim, N), torch.float32, dev)
    _check("B", B, (batch, N, L), dt, dev)
    _check("C", C, (batch, N, L), dt, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim, L), dt, dev, required=False)
    _check("delta_bias", delta_bias, (dim,), torch.float32, dev, required=False)
    _check("h0", h0, (batch, dim, N), torch.float32, dev, required=False)
    _check("dy", dy, (batch, dim, L), dt, dev)
    _check("dlast_state", dlast_state, (batch, dim, N), torch.float32, dev, required=False)
    if ckpt is not None:
        _check("ckpt", ckpt, (batch, (L + 15) // 16, N, dim), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(du=torch.empty_like(u), ddelta=torch.empty_like(u), dA=torch.empty((dim, N), **f32),
             dB=torch.empty_like(B), dC=torch.empty_like(C), dD=torch.empty(dim, **f32),
             dz=torch.empty_like(u) if z is not None else None,
             ddelta_bias=torch.empty(dim, **f32), dh0=torch.empty((batch, dim, N), **f32))
    query = lib.ssm_scan_bwd_ckpt_workspace_bytes if ckpt is not None else lib.ssm_scan_bwd_workspace_bytes
    need = int(query(batch, dim, N, L, code))
    ws_bytes = 0
    if need > 0:
        if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    head = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            _flags(delta_softplus, bbar), _ptr(h0))
    tail = (_ptr(dy), _ptr(dlast_state), _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]),
            _ptr(g["dB"]), _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["ddelta_bias"]),
            _ptr(g["dh0"]), batch, dim, N, L, code, _ptr(workspace), ws_bytes, stream)
    if ckpt is None:
        rc = lib.ssm_scan_bwd(*head, *tail)
        where = "ssm_scan_bwd"
    else:
        rc = lib.ssm_scan_bwd_ckpt(*head, _ptr(ckpt), ckpt.numel() * 4, *tail)
        where = "ssm_scan_bwd_ckpt"
    if rc != 0:
        raise SsmError(rc, where)
    return g


def ssm_scan_bwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 h0=None, *, dy, dlast_state=None, bbar="euler", workspace=None):
    """Gradients through ssm_scan_fwd (input term `bbar`: "euler" or "zoh")
    given dy = dL/dy and optionally dL/dlast_state; the states are
    recomputed, not stored.
    Returns a dict: du, ddelta, dz (None without z) and dB, dC in the input
    dtype; dA, dD, ddelta_bias, dh0 in float32."""
    return _bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, dy, dlast_state, bbar,
                workspace, None)


def ssm_scan_ckpt_bytes(batch: int, dim: int, dstate: int, seqlen: int) -> int:
    return int(load().ssm_scan_ckpt_bytes(batch, dim, dstate, seqlen))


def ssm_scan_bwd_ckpt_workspace_bytes(batch: int, dim: int, dstate: int, seqlen: int,
                                      dtype: torch.dtype) -> int:
    return int(load().ssm_scan_bwd_ckpt_workspace_bytes(batch, dim, dstate, seqlen, _DTYPES[dtype]))


def ssm_scan_fwd_ckpt(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                      h0=None, *, bbar="euler", out=None, ckpt=None, workspace=None):
    """ssm_scan_fwd that also writes the tile checkpoints (the state entering
    every 16-step tile) for ssm_scan_bwd_ckpt.
    Returns (y, last_state, ckpt); ckpt is (batch, ceil(L/16), N, dim) float32."""
    lib = load()
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, L = u.shape
    N = A.shape[1] if A.dim() == 2 else -1
    _check("u", u, (batch, dim, L), dt, dev)
    _check("delta", delta, (batch, dim, L), dt, dev)
    _check("A", A, (dim, N), torch.float32, dev)
    _check("B", B, (batch, N, L), dt, dev)
    _check("C", C, (batch, N, L), dt, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim, L), dt, dev, required=False)
    _check("delta_bias", delta_bias, (dim,), torch.float32, dev, required=False)
    _check("h0", h0, (batch, dim, N), torch.float32, dev, required=False)
    y = out if out is not None else torch.empty_like(u)
    _check("out", y, (batch, dim, L), dt, dev)
    cshape = (batch, (L + 15) // 16, N, dim)
    if ckpt is None:
        ckpt = torch.empty(cshape, dtype=torch.float32, device=dev)
    _check("ckpt", ckpt, cshape, torch.float32, dev)
    last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev)
    need = int(lib.ssm_scan_fwd_workspace_bytes(batch, dim, N, L, code))
    ws_bytes = 0
    if need > 0:
        if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd_ckpt(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                               _ptr(delta_bias), _flags(delta_softplus, bbar), _ptr(h0), _ptr(y),
                               _ptr(last), _ptr(ckpt), ckpt.numel() * 4, batch, dim, N, L, code,
                               _ptr(workspace), ws_bytes, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_scan_fwd_ckpt")
    return y, last, ckpt


def ssm_scan_bwd_ckpt(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                      h0=None, *, ckpt, dy, dlast_state=None, bbar="euler", workspace=None):
    """ssm_scan_bwd from the checkpoints ssm_scan_fwd_ckpt wrote for the same
    inputs: the same gradients, without the forward checkpoint pass."""
    return _bwd(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, dy, dlast_state, bbar,
                workspace, ckpt)


def ssm_ssd_scan_fwd_workspace_bytes(batch: int, dstate: int, seqlen: int, dtype: torch.dtype) -> int:
    return int(load().ssm_ssd_scan_fwd_workspace_bytes(batch, dstate, seqlen, _DTYPES[dtype]))


def ssm_ssd_scan_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, delta_softplus=True, h0=None, *,
                     bbar="euler", return_last_state=False, out=None, workspace=None):
    """The SSD (scalar A per head) scan on the matrix cores; see include/ssm.h.
    x, z: (batch, nheads * 64, L); dt: (batch, nheads, L); A, dt_bias:
    (nheads,) float32; B, C: (batch, N, L); D: (dim,) float32; h0:
    (batch, dim, N) float32.  Returns y, and (y, last_state) when asked."""
    lib = load()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dtp = x.dtype
    code = _code(x)
    batch, dim, L = x.shape
    H = A.shape[0] if A.dim() == 1 else -1
    if H <= 0 or dim % H != 0:
        raise ValueError("x's channel count must be a multiple of the number of heads")
    P = dim // H
    N = B.shape[1] if B.dim() == 3 else -1
    _check("x", x, (batch, dim, L), dtp, dev)
    _check("dt", dt, (batch, H, L), dtp, dev)
    _check("A", A, (H,), torch.float32, dev)
    _check("B", B, (batch, N, L), dtp, dev)
    _check("C", C, (batch, N, L), dtp, dev)
    _check("D", D, (dim,), torch.float32, dev, required=False)
    _check("z", z, (batch, dim, L), dtp, dev, required=False)
    _check("dt_bias", dt_bias, (H,), torch.float32, dev, required=False)
    _check("h0", h0, (batch, dim, N), torch.float32, dev, required=False)
    y = out if out is not None else torch.empty_like(x)
    _check("out", y, (batch, dim, L), dtp, dev)
    last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev) if return_last_state else None
    need = int(lib.ssm_ssd_scan_fwd_workspace_bytes(batch, N, L, code))
    ws_bytes = 0
    if need > 0:
        if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
            raise ValueError(f"workspace must be a contiguous tensor on {dev}")
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_ssd_scan_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                              _ptr(dt_bias), _flags(delta_softplus, bbar), _ptr(h0), _ptr(y),
                              _ptr(last), batch, H, P, N, L, code, _ptr(workspace), ws_bytes, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_ssd_scan_fwd")
    return (y, last) if return_last_state else y
