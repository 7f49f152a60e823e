"""The C ABI without a GPU: libssm.so loads, exports every function that
include/ssm.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os

import pytest

import selective_state_space_28_amd as ssm
from selective_state_space_28_amd._lib import header_functions, load

OK, NULL, SHAPE, DTYPE, ALIGN, WS, HIP, ALIAS, FLAGS, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
P = 0x10000  # a 256-byte aligned fake device address, never dereferenced
R = 0x1000000  # 16 MiB: distinct buffers of a call sit R apart, so none overlaps


def at(k):
    """Fake device address of the k-th distinct buffer of a call."""
    return 0x40000000 + k * R


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == {"ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd", "ssm_state_update",
                          "ssm_conv_scan_fwd", "ssm_conv_state_update", "ssm_scan_bwd_workspace_bytes",
                          "ssm_scan_bwd", "ssm_ssd_scan_fwd", "ssm_ssd_scan_fwd_workspace_bytes",
                          "ssm_scan_fwd_noalloc", "ssm_status_string", "ssm_scan_ckpt_bytes",
                          "ssm_scan_fwd_ckpt", "ssm_scan_bwd_ckpt_workspace_bytes", "ssm_scan_bwd_ckpt"}
    lib = ctypes.CDLL(load()._name)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, WS, HIP, ALIAS, FLAGS, SCRATCH):
        s = ssm.ssm_status_string(code)
        assert s.startswith("SSM_")
    assert "unknown" in ssm.ssm_status_string(42)


def _scan(**kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1, h0=None, y=at(1),
             last=None, batch=1, dim=64, dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                               a["bias"], a["sp"], a["h0"], a["y"], a["last"], a["batch"],
                               a["dim"], a["dstate"], a["L"], a["dtype"], a["ws"], a["wsb"],
                               a["stream"])


def _upd(**kw):
    a = dict(state=at(2), u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1,
             y=at(1), batch=4, dim=64, dstate=16, dtype=1, stream=None)
    a.update(kw)
    return load().ssm_state_update(a["state"], a["u"], a["delta"], a["A"], a["B"], a["C"],
                                   a["D"], a["z"], a["bias"], a["sp"], a["y"], a["batch"],
                                   a["dim"], a["dstate"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(dstate=3), SHAPE), (dict(dstate=32), SHAPE), (dict(dstate=0), SHAPE),
    (dict(batch=-1), SHAPE), (dict(dim=-5), SHAPE), (dict(L=-1), SHAPE),
    (dict(u=None), NULL), (dict(delta=None), NULL), (dict(A=None), NULL), (dict(B=None), NULL),
    (dict(C=None), NULL), (dict(y=None), NULL),
    (dict(u=P + 1), ALIGN), (dict(A=P + 2), ALIGN), (dict(h0=P + 1), ALIGN),
    (dict(dtype=0, u=P + 2), ALIGN), (dict(last=P + 3), ALIGN), (dict(ws=P + 16), ALIGN),
    (dict(y=P), ALIAS), (dict(z=at(1)), ALIAS),
    # overlapping ranges, not only equal pointers: y starting inside u, u
    # starting inside y, last_state inside B, h0 shared with last_state
    (dict(y=P + 0x100), ALIAS), (dict(u=at(1) + 0x1000, delta=at(1) + 0x1000), ALIAS),
    (dict(last=P + 0x40), ALIAS), (dict(h0=at(2), last=at(2)), ALIAS),
    (dict(last=at(1) + 64 * 2048 * 2 - 4), ALIAS), (dict(last=at(1) + 64 * 2048 * 2), WS),
    (dict(sp=4), FLAGS), (dict(sp=-1), FLAGS), (dict(sp=8 | 1), FLAGS),
    # step positions are 32-bit in the kernels: longer sequences are refused
    (dict(L=(1 << 31) - 4096), SHAPE), (dict(L=1 << 40), SHAPE),
])
def test_scan_validation(kw, code):
    assert _scan(**kw) == code


def test_scan_workspace_checked_before_launch(monkeypatch):
    need = load().ssm_scan_fwd_workspace_bytes(1, 64, 16, 2048, 1)
    assert need > 0
    assert _scan(ws=None, wsb=0) == WS
    assert _scan(ws=at(3), wsb=need - 1) == WS
    # the workspace must not overlap a buffer of the call
    assert _scan(ws=at(1) - 256, wsb=need) == ALIAS
    assert _scan(ws=P, wsb=need) == ALIAS


def test_workspace_query_refuses_too_long_sequences():
    q = load().ssm_scan_fwd_workspace_bytes
    longest = (1 << 31) - 4097
    assert q(1, 1, 16, longest, 1) > 0
    assert q(1, 1, 16, longest + 1, 1) == 0
    assert load().ssm_scan_bwd_workspace_bytes(1, 1, 16, longest, 1) > 0
    assert load().ssm_scan_bwd_workspace_bytes(1, 1, 16, longest + 1, 1) == 0


def test_empty_problems_need_no_gpu():
    # batch or dim zero: nothing to do, nothing launched
    assert _scan(batch=0) == OK
    assert _scan(dim=0, u=None, delta=None) == OK
    assert _upd(batch=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), DTYPE), (dict(dstate=6), SHAPE), (dict(batch=-2), SHAPE),
    (dict(state=None), NULL), (dict(u=None), NULL), (dict(B=None), NULL), (dict(y=None), NULL),
    (dict(state=at(2) + 2), ALIGN), (dict(u=P + 1), ALIGN), (dict(bias=P + 1), ALIGN),
    (dict(y=P), ALIAS), (dict(sp=6), FLAGS), (dict(sp=1 << 30), FLAGS),
    (dict(y=at(2) + 4096), ALIAS), (dict(state=P + 256), ALIAS), (dict(state=at(1) - 16), ALIAS),
])
def test_update_validation(kw, code):
    assert _upd(**kw) == code


def test_workspace_query():
    q = load().ssm_scan_fwd_workspace_bytes
    # the 2.8B-shaped layer fills the GPU with channels: no split, so only the
    # B, C records in the input type (batch * L * 2N elements)
    assert q(16, 5120, 16, 2048, 1) == 16 * 2048 * 32 * 2
    assert q(16, 5120, 16, 2048, 0) == 16 * 2048 * 32 * 4
    # the long sequence over few channels is split: records plus carries
    assert q(1, 2048, 16, 65536, 1) > 1 * 65536 * 32 * 4
    assert q(1, 2048, 16, 65536, 7) == 0      # bad dtype
    assert q(1, 2048, 3, 65536, 1) == 0       # bad dstate
    assert q(0, 2048, 16, 65536, 1) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from selective_state_space_28_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB", str(tmp_path / "nope.so"))
    with pytest.raises(ImportError):
        _lib.load()


def test_python_bbar_mode_is_checked():
    import torch
    from selective_state_space_28_amd.ops import _flags
    assert _flags(True, "euler") == 1 and _flags(False, "euler") == 0
    assert _flags(True, "zoh") == 3 and _flags(False, "zoh") == 2
    with pytest.raises(ValueError):
        _flags(True, "bilinear")


def _cscan(**kw):
    a = dict(x=P, w=at(2), cb=None, K=4, sin=None, sout=None, delta=P, A=P, B=P, C=P, D=None,
             z=None, bias=None, fl=1, h0=None, y=at(1), last=None, batch=1, dim=64,
             dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_conv_scan_fwd(a["x"], a["w"], a["cb"], a["K"], a["sin"], a["sout"], a["delta"],
                                    a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["fl"],
                                    a["h0"], a["y"], a["last"], a["batch"], a["dim"], a["dstate"],
                                    a["L"], a["dtype"], a["ws"], a["wsb"], a["stream"])


def _cupd(**kw):
    a = dict(cs=at(3), state=at(4), x=P, w=at(2), cb=None, K=4, delta=P, A=P, B=P, C=P,
             D=None, z=None, bias=None, fl=1, y=at(1), batch=4, dim=64, dstate=16, dtype=1,
             stream=None)
    a.update(kw)
    return load().ssm_conv_state_update(a["cs"], a["state"], a["x"], a["w"], a["cb"], a["K"],
                                        a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                        a["bias"], a["fl"], a["y"], a["batch"], a["dim"],
                                        a["dstate"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), SHAPE), (dict(K=5), SHAPE), (dict(K=-1), SHAPE),
    (dict(w=None), NULL), (dict(x=None), NULL),
    (dict(w=at(2) + 2), ALIGN), (dict(cb=P + 1), ALIGN), (dict(sin=P + 2), ALIGN),
    (dict(sout=P + 3), ALIGN),
    (dict(sin=at(4), sout=at(4)), ALIAS), (dict(sout=at(1)), ALIAS),
    (dict(sin=at(4), sout=at(4) + 64), ALIAS), (dict(sout=at(2) + 16), ALIAS),
    (dict(y=P), ALIAS), (dict(fl=4), FLAGS), (dict(dtype=3), DTYPE), (dict(dstate=5), SHAPE),
])
def test_conv_scan_validation(kw, code):
    assert _cscan(**kw) == code


def test_conv_scan_workspace_checked_before_launch():
    assert _cscan(ws=None, wsb=0) == WS
    assert _cscan(batch=0) == OK
    # the workspace must not overlap the taps, the bias or the carried inputs
    need = load().ssm_scan_fwd_workspace_bytes(1, 64, 16, 2048, 1)
    assert _cscan(ws=at(2), wsb=need) == ALIAS
    assert _cscan(cb=at(3) + 512, ws=at(3), wsb=need) == ALIAS
    assert _cscan(sin=at(3) + 1024, ws=at(3), wsb=need) == ALIAS
    assert _cscan(sout=at(3) + need - 4, ws=at(3), wsb=need) == ALIAS


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), SHAPE), (dict(K=7), SHAPE), (dict(w=None), NULL), (dict(cs=None), NULL),
    (dict(cs=at(3) + 2), ALIGN), (dict(cs=P), ALIAS), (dict(cs=at(1)), ALIAS),
    (dict(cs=at(4) + 512), ALIAS), (dict(cs=at(2) + 4), ALIAS),
    (dict(fl=8), FLAGS), (dict(state=None), NULL),
])
def test_conv_update_validation(kw, code):
    assert _cupd(**kw) == code


def test_conv_update_width_one_needs_no_state():
    # K = 1: no carried inputs; an empty problem returns before any launch
    assert _cupd(cs=None, K=1, batch=0) == OK


def _bwd(**kw):
    a = dict(u=P, delta=at(1), A=at(2), B=at(3), C=at(4), D=None, z=None,
             bias=None, fl=1, h0=None, dy=at(5), dlast=None, du=at(6), dd=at(7),
             dA=at(8), dB=at(9), dC=at(10), dD=None, dz=None, dbias=None, dh0=None,
             batch=1, dim=64, dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_scan_bwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                               a["fl"], a["h0"], a["dy"], a["dlast"], a["du"], a["dd"], a["dA"],
                               a["dB"], a["dC"], a["dD"], a["dz"], a["dbias"], a["dh0"], a["batch"],
                               a["dim"], a["dstate"], a["L"], a["dtype"], a["ws"], a["wsb"],
                               a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(fl=4), FLAGS), (dict(fl=5), FLAGS), (dict(fl=-1), FLAGS), (dict(dtype=7), DTYPE),
    (dict(dstate=12), SHAPE), (dict(L=-3), SHAPE),
    (dict(dy=None), NULL), (dict(du=None), NULL), (dict(dA=None), NULL), (dict(dB=None), NULL),
    (dict(z=at(11)), NULL),
    (dict(du=P + 1), ALIGN), (dict(dA=P + 2), ALIGN), (dict(dlast=P + 1), ALIGN),
    (dict(du=P), ALIAS), (dict(dB=at(3)), ALIAS), (dict(ddelta=None, dd=at(5)), ALIAS),
    (dict(dB=at(3) + 64), ALIAS), (dict(dC=at(9) + 2), ALIAS), (dict(dh0=at(6) + 1024), ALIAS),
    (dict(dD=at(2) + 4), ALIAS),
])
def test_bwd_validation(kw, code):
    assert _bwd(**kw) == code


def test_bwd_workspace_query_and_check():
    lib = load()
    need = lib.ssm_scan_bwd_workspace_bytes(1, 64, 16, 2048, 1)
    fwd = lib.ssm_scan_fwd_workspace_bytes(1, 64, 16, 2048, 1)
    # forward workspace + tile checkpoints + dB/dC partials at least
    assert need >= fwd + 128 * 16 * 64 * 4 + 2 * 16 * 2048 * 4
    assert lib.ssm_scan_bwd_workspace_bytes(0, 64, 16, 2048, 1) == 0
    assert _bwd(ws=None, wsb=0) == WS
    assert _bwd(ws=at(12), wsb=need - 1) == WS
    assert _bwd(ws=at(6) + 256, wsb=need) == ALIAS   # overlaps du
    assert _bwd(batch=0) == OK


# ---- the training pair: forward with tile checkpoints, backward from them ----

CK = 1 * 128 * 16 * 64 * 4   # checkpoints of (batch 1, dim 64, N 16, L 2048)


def test_ckpt_bytes_query():
    lib = load()
    assert lib.ssm_scan_ckpt_bytes(1, 64, 16, 2048) == CK
    assert lib.ssm_scan_ckpt_bytes(3, 70, 4, 2049) == 3 * 129 * 4 * 70 * 4   # a ragged last tile
    assert lib.ssm_scan_ckpt_bytes(1, 64, 16, 16) == 16 * 64 * 4
    assert lib.ssm_scan_ckpt_bytes(1, 64, 16, 0) == 0
    assert lib.ssm_scan_ckpt_bytes(0, 64, 16, 2048) == 0
    assert lib.ssm_scan_ckpt_bytes(1, 64, 12, 2048) == 0      # dstate refused
    assert lib.ssm_scan_ckpt_bytes(1, 64, 16, 1 << 40) == 0   # too long


def _fwdck(**kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1, h0=None, y=at(1),
             last=None, ck=at(3), ckb=CK, batch=1, dim=64, dstate=16, L=2048, dtype=1, ws=None, wsb=0,
             stream=None)
    a.update(kw)
    return load().ssm_scan_fwd_ckpt(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                    a["bias"], a["sp"], a["h0"], a["y"], a["last"], a["ck"], a["ckb"],
                                    a["batch"], a["dim"], a["dstate"], a["L"], a["dtype"], a["ws"],
                                    a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ck=None), NULL), (dict(ckb=CK - 1), WS), (dict(ck=at(3) + 2), ALIGN),
    (dict(ck=at(1) + 256), ALIAS),            # inside y
    (dict(ck=P + 64), ALIAS),                 # inside the inputs
    (dict(last=at(3) + CK - 4), ALIAS),       # last_state at the checkpoints' end
    (dict(dstate=3), SHAPE), (dict(sp=4), FLAGS), (dict(dtype=2), DTYPE), (dict(u=None), NULL),
    (dict(ws=None), WS),                      # every checkpoint check passed: the workspace next
    (dict(ws=at(3) + 4096, wsb=1 << 20), ALIAS),   # workspace inside the checkpoints
    (dict(batch=0), OK), (dict(L=0, ck=None, ckb=0), OK),   # nothing to checkpoint, no HIP call
])
def test_fwd_ckpt_validation(kw, code):
    assert _fwdck(**kw) == code


def _bwdck(**kw):
    a = dict(u=P, delta=at(1), A=at(2), B=at(3), C=at(4), D=None, z=None,
             bias=None, fl=1, h0=None, ck=at(13), ckb=CK, dy=at(5), dlast=None, du=at(6), dd=at(7),
             dA=at(8), dB=at(9), dC=at(10), dD=None, dz=None, dbias=None, dh0=None,
             batch=1, dim=64, dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_scan_bwd_ckpt(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                    a["bias"], a["fl"], a["h0"], a["ck"], a["ckb"], a["dy"], a["dlast"],
                                    a["du"], a["dd"], a["dA"], a["dB"], a["dC"], a["dD"], a["dz"],
                                    a["dbias"], a["dh0"], a["batch"], a["dim"], a["dstate"], a["L"],
                                    a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(ck=None), NULL), (dict(ckb=CK - 4), WS), (dict(ck=at(13) + 1), ALIGN),
    (dict(du=at(13) + 1024), ALIAS),          # a gradient inside the checkpoints
    (dict(dh0=at(13) + CK - 8), ALIAS),
    (dict(dA=at(13)), ALIAS),
    (dict(ck=at(1)), WS),                     # overlapping inputs are allowed: reaches the workspace check
    (dict(fl=4), FLAGS), (dict(dtype=7), DTYPE), (dict(dy=None), NULL),
    (dict(ws=None), WS), (dict(ws=at(13) + 256, wsb=1 << 24), ALIAS),
    (dict(batch=0), OK),
])
def test_bwd_ckpt_validation(kw, code):
    assert _bwdck(**kw) == code


def test_bwd_ckpt_workspace_query():
    """The checkpointed backward's workspace is the plain backward's without
    the checkpoint region."""
    lib = load()
    for shape in ((1, 64, 16, 2048), (2, 70, 4, 1031), (1, 2048, 16, 65536), (3, 5, 1, 17)):
        plain = lib.ssm_scan_bwd_workspace_bytes(*shape, 1)
        ck = lib.ssm_scan_bwd_ckpt_workspace_bytes(*shape, 1)
        cb = lib.ssm_scan_ckpt_bytes(*shape)
        assert ck == plain - (cb + 255) // 256 * 256, shape
    assert lib.ssm_scan_bwd_ckpt_workspace_bytes(0, 64, 16, 2048, 1) == 0
    assert lib.ssm_scan_bwd_ckpt_workspace_bytes(1, 64, 16, 2048, 5) == 0
    need = lib.ssm_scan_bwd_ckpt_workspace_bytes(1, 64, 16, 2048, 1)
    assert _bwdck(ws=at(14), wsb=need - 1) == WS


def _ssd(**kw):
    a = dict(x=P, dt=at(1), A=at(2), B=at(3), C=at(4), D=None, z=None,
             bias=None, fl=1, h0=None, y=at(5), last=None, batch=1, H=4, hd=64, N=128, L=2048,
             dtype=1, ws=at(6), wsb=1 << 24, stream=None)
    a.update(kw)
    return load().ssm_ssd_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                   a["fl"], a["h0"], a["y"], a["last"], a["batch"], a["H"], a["hd"],
                                   a["N"], a["L"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hd=32), SHAPE), (dict(N=8), SHAPE), (dict(N=128, dtype=0), SHAPE), (dict(N=256), SHAPE),
    (dict(H=-1), SHAPE), (dict(L=-1), SHAPE), (dict(dtype=4), DTYPE), (dict(fl=8), FLAGS),
    (dict(x=None), NULL), (dict(dt=None), NULL), (dict(A=None), NULL), (dict(y=None), NULL),
    (dict(x=P + 1), ALIGN), (dict(A=at(2) + 2), ALIGN), (dict(y=P), ALIAS),
    (dict(y=at(1) + 256), ALIAS), (dict(last=at(5) + 0x10000), ALIAS), (dict(ws=at(4) + 4096), ALIAS),
    (dict(ws=at(6) + 16), ALIGN), (dict(ws=None), WS), (dict(wsb=1000), WS),
    # 32-bit byte offsets within a head's rows and a batch row's B, C^T
    (dict(L=1 << 23), SHAPE), (dict(L=1 << 23, N=64, dtype=0), SHAPE),
])
def test_ssd_validation(kw, code):
    assert _ssd(**kw) == code


def test_ssd_workspace_query():
    lib = load()
    # C^T in the input type (rounded to 256 bytes), then 10 float32 16x16 tiles per row and chunk
    assert lib.ssm_ssd_scan_fwd_workspace_bytes(2, 128, 2048, 1) == 2 * 2048 * 128 * 2 + 2 * 32 * 10 * 1024
    assert lib.ssm_ssd_scan_fwd_workspace_bytes(1, 64, 100, 0) == (100 * 64 * 4 + 255) // 256 * 256 + 2 * 10 * 1024
    assert lib.ssm_ssd_scan_fwd_workspace_bytes(0, 64, 100, 0) == 0


def test_ssd_empty_needs_no_gpu():
    assert _ssd(batch=0) == OK
    assert _ssd(H=0, x=None) == OK


def _noalloc(**kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1, h0=None, y=at(1),
             last=None, batch=1, dim=64, dstate=16, L=2048, dtype=1, stream=None)
    a.update(kw)
    return load().ssm_scan_fwd_noalloc(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                       a["bias"], a["sp"], a["h0"], a["y"], a["last"], a["batch"],
                                       a["dim"], a["dstate"], a["L"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), DTYPE), (dict(dstate=3), SHAPE), (dict(u=None), NULL), (dict(y=P + 1), ALIGN),
    (dict(y=P), ALIAS), (dict(sp=4), FLAGS), (dict(batch=0), OK),
    # B, C records alone of batch 1 x 2^20 steps x 32 values of bf16: 64 MiB > 16 MiB
    (dict(L=1 << 20, y=at(8)), SCRATCH),
])
def test_noalloc_validation_without_gpu(kw, code):
    """Everything the allocation-free scan checks, its scratch limit included,
    is checked before its first HIP call."""
    assert _noalloc(**kw) == code


def test_noalloc_limit_matches_the_header():
    import re
    from selective_state_space_28_amd.build import INCLUDE
    with open(os.path.join(INCLUDE, "ssm.h")) as f:
        m = re.search(r"#define SSM_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m is not None
    limit = int(m.group(1)) << int(m.group(2))
    q = load().ssm_scan_fwd_workspace_bytes
    assert q(16, 5120, 16, 2048, 1) <= limit          # the 2.8B-shaped layer fits
    assert q(1, 64, 16, 1 << 20, 1) > limit
