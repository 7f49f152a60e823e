"""ctypes view of libssm.so (include/ssm.h).  Loading fails loudly when the
library has not been built: there is no other implementation to fall back to."""
from __future__ import annotations

import ctypes
import os
import re

from .build import LIB, INCLUDE

SSM_F32, SSM_BF16 = 0, 1
SSM_DELTA_SOFTPLUS, SSM_BBAR_ZOH = 1, 2
_lib = None


class SsmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def header_functions() -> list[str]:
    """Names of the functions include/ssm.h declares."""
    with open(os.path.join(INCLUDE, "ssm.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(ssm_\w+)\s*\(", text)


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise ImportError(f"libssm.so is not built ({LIB}); run "
                          "`python -m selective_state_space_28_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB)
    vp, fp = ctypes.c_void_p, ctypes.c_void_p
    i32, i64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.ssm_scan_fwd_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    lib.ssm_scan_fwd_workspace_bytes.restype = sz
    lib.ssm_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp,
                                 i32, i32, i32, i64, i32, vp, sz, vp]
    lib.ssm_scan_fwd.restype = i32
    lib.ssm_state_update.argtypes = [fp, vp, vp, fp, vp, vp, fp, vp, fp, i32, vp,
                                     i32, i32, i32, i32, vp]
    lib.ssm_state_update.restype = i32
    lib.ssm_conv_scan_fwd.argtypes = [vp, fp, fp, i32, fp, fp, vp, fp, vp, vp, fp, vp, fp, i32,
                                      fp, vp, fp, i32, i32, i32, i64, i32, vp, sz, vp]
    lib.ssm_conv_scan_fwd.restype = i32
    lib.ssm_conv_state_update.argtypes = [fp, fp, vp, fp, fp, i32, vp, fp, vp, vp, fp, vp, fp, i32,
                                          vp, i32, i32, i32, i32, vp]
    lib.ssm_conv_state_update.restype = i32
    lib.ssm_scan_bwd_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    lib.ssm_scan_bwd_workspace_bytes.restype = sz
    lib.ssm_scan_bwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp, vp, vp, fp, vp,
                                 vp, fp, vp, fp, fp, i32, i32, i32, i64, i32, vp, sz, vp]
    lib.ssm_scan_bwd.restype = i32
    lib.ssm_scan_ckpt_bytes.argtypes = [i32, i32, i32, i64]
    lib.ssm_scan_ckpt_bytes.restype = sz
    lib.ssm_scan_fwd_ckpt.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp, fp, sz,
                                      i32, i32, i32, i64, i32, vp, sz, vp]
    lib.ssm_scan_fwd_ckpt.restype = i32
    lib.ssm_scan_bwd_ckpt_workspace_bytes.argtypes = [i32, i32, i32, i64, i32]
    lib.ssm_scan_bwd_ckpt_workspace_bytes.restype = sz
    lib.ssm_scan_bwd_ckpt.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, fp, sz, vp, fp, vp,
                                      vp, fp, vp, vp, fp, vp, fp, fp, i32, i32, i32, i64, i32, vp,
                                      sz, vp]
    lib.ssm_scan_bwd_ckpt.restype = i32
    lib.ssm_ssd_scan_fwd.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp, i32, i32, i32,
                                     i32, i64, i32, vp, sz, vp]
    lib.ssm_ssd_scan_fwd_workspace_bytes.argtypes = [i32, i32, i64, i32]
    lib.ssm_ssd_scan_fwd_workspace_bytes.restype = sz
    lib.ssm_ssd_scan_fwd.restype = i32
    if hasattr(lib, "ssm_scan_fwd_noalloc"):
        lib.ssm_scan_fwd_noalloc.argtypes = [vp, vp, fp, vp, vp, fp, vp, fp, i32, fp, vp, fp,
                                             i32, i32, i32, i64, i32, vp]
        lib.ssm_scan_fwd_noalloc.restype = i32
    lib.ssm_status_string.argtypes = [i32]
    lib.ssm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ssm_status_string(int(status)).decode()
