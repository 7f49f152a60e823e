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


def ssm_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus=True,
                 h0=None, *, bbar="euler", return_last_state=False, out=None, workspace=None):
    """Selective scan over (batch, dim, L) inputs; see include/ssm.h.
    bbar: 'euler' (input term Delta*B*u) or 'zoh' ((exp(Delta*A) - 1)/A*B*u,
    A nonzero).

    u, delta, z: (batch, dim, L) float32 or bfloat16 (one dtype for all);
    B, C: (batch, N, L) same dtype; A: (dim, N) float32; D, delta_bias: (dim,)
    float32; h0: (batch, dim, N) float32.  Returns y (batch, dim, L) in the
    input dtype, and (y, last_state) when return_last_state is set."""
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
    last = torch.empty((batch, dim, N), dtype=torch.float32, device=dev) if return_last_state else None
    need = int(lib.ssm_scan_fwd_workspace_bytes(batch, dim, N, L, code))
    ws_bytes = 0
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
    else:
        workspace = None
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = lib.ssm_scan_fwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                          _ptr(delta_bias), _flags(delta_softplus, bbar), _ptr(h0), _ptr(y),
                          _ptr(last), batch, dim, N, L, code, _ptr(workspace), ws_bytes, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_scan_fwd")
    return (y, last) if return_last_state else y


def ssm_state_update(state, u, delta, A, B, C, D=None, z=None, delta_bias=None,
                     delta_softplus=True, *, bbar="euler", out=None):
    """One decode step; `state` (batch, dim, N) float32 is updated in place.
    u, delta, z: (batch, dim); B, C: (batch, N); returns y (batch, dim)."""
    lib = load()
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("libssm runs on the GPU: tensors must be on a cuda device")
    dt = u.dtype
    code = _code(u)
    batch, dim, N = state.shape
    _check("state", state, (batch, dim, N), torch.float32, dev)
    _check("u", u, (batch, dim), dt, dev)
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
    rc = lib.ssm_state_update(_ptr(state), _ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C),
                              _ptr(D), _ptr(z), _ptr(delta_bias), _flags(delta_softplus, bbar),
                              _ptr(y), batch, dim, N, code, stream)
    if rc != 0:
        raise SsmError(rc, "ssm_state_update")
    return y
