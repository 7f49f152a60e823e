"""The C ABI without a GPU: libssm.so loads, exports every function that
include/ssm.h declares, and rejects bad arguments before any HIP call."""
import ctypes

import pytest

import selective_state_space_28_amd as ssm
from selective_state_space_28_amd._lib import header_functions, load

OK, NULL, SHAPE, DTYPE, ALIGN, WS, HIP, ALIAS, FLAGS = 0, -1, -2, -3, -4, -5, -6, -7, -8
P = 0x10000  # a 256-byte aligned fake device address, never dereferenced


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == {"ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd", "ssm_state_update",
                          "ssm_conv_scan_fwd", "ssm_conv_state_update", "ssm_scan_bwd_workspace_bytes",
                          "ssm_scan_bwd", "ssm_ssd_scan_fwd", "ssm_ssd_scan_fwd_workspace_bytes",
                          "ssm_status_string"}
    lib = ctypes.CDLL(load()._name)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code in (OK, NULL, SHAPE, DTYPE, ALIGN, WS, HIP, ALIAS, FLAGS):
        s = ssm.ssm_status_string(code)
        assert s.startswith("SSM_")
    assert "unknown" in ssm.ssm_status_string(42)


def _scan(**kw):
    a = dict(u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1, h0=None, y=P + 0x100000,
             last=None, batch=1, dim=64, dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_scan_fwd(a["u"], a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                               a["bias"], a["sp"], a["h0"], a["y"], a["last"], a["batch"],
                               a["dim"], a["dstate"], a["L"], a["dtype"], a["ws"], a["wsb"],
                               a["stream"])


def _upd(**kw):
    a = dict(state=P, u=P, delta=P, A=P, B=P, C=P, D=None, z=None, bias=None, sp=1,
             y=P + 0x100000, batch=4, dim=64, dstate=16, dtype=1, stream=None)
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
    (dict(y=P), ALIAS), (dict(z=P + 0x100000), ALIAS),
    (dict(sp=4), FLAGS), (dict(sp=-1), FLAGS), (dict(sp=8 | 1), FLAGS),
])
def test_scan_validation(kw, code):
    assert _scan(**kw) == code


def test_scan_workspace_checked_before_launch(monkeypatch):
    need = load().ssm_scan_fwd_workspace_bytes(1, 64, 16, 2048, 1)
    assert need > 0
    assert _scan(ws=None, wsb=0) == WS
    assert _scan(ws=P, wsb=need - 1) == WS


def test_empty_problems_need_no_gpu():
    # batch or dim zero: nothing to do, nothing launched
    assert _scan(batch=0) == OK
    assert _scan(dim=0, u=None, delta=None) == OK
    assert _upd(batch=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), DTYPE), (dict(dstate=6), SHAPE), (dict(batch=-2), SHAPE),
    (dict(state=None), NULL), (dict(u=None), NULL), (dict(B=None), NULL), (dict(y=None), NULL),
    (dict(state=P + 2), ALIGN), (dict(u=P + 1), ALIGN), (dict(bias=P + 1), ALIGN),
    (dict(y=P), ALIAS), (dict(sp=6), FLAGS), (dict(sp=1 << 30), FLAGS),
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
    a = dict(x=P, w=P + 0x200000, cb=None, K=4, sin=None, sout=None, delta=P, A=P, B=P, C=P, D=None,
             z=None, bias=None, fl=1, h0=None, y=P + 0x100000, last=None, batch=1, dim=64,
             dstate=16, L=2048, dtype=1, ws=None, wsb=0, stream=None)
    a.update(kw)
    return load().ssm_conv_scan_fwd(a["x"], a["w"], a["cb"], a["K"], a["sin"], a["sout"], a["delta"],
                                    a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"], a["fl"],
                                    a["h0"], a["y"], a["last"], a["batch"], a["dim"], a["dstate"],
                                    a["L"], a["dtype"], a["ws"], a["wsb"], a["stream"])


def _cupd(**kw):
    a = dict(cs=P + 0x300000, state=P, x=P, w=P + 0x200000, cb=None, K=4, delta=P, A=P, B=P, C=P,
             D=None, z=None, bias=None, fl=1, y=P + 0x100000, batch=4, dim=64, dstate=16, dtype=1,
             stream=None)
    a.update(kw)
    return load().ssm_conv_state_update(a["cs"], a["state"], a["x"], a["w"], a["cb"], a["K"],
                                        a["delta"], a["A"], a["B"], a["C"], a["D"], a["z"],
                                        a["bias"], a["fl"], a["y"], a["batch"], a["dim"],
                                        a["dstate"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), SHAPE), (dict(K=5), SHAPE), (dict(K=-1), SHAPE),
    (dict(w=None), NULL), (dict(x=None), NULL),
    (dict(w=P + 0x200002), ALIGN), (dict(cb=P + 1), ALIGN), (dict(sin=P + 2), ALIGN),
    (dict(sout=P + 3), ALIGN),
    (dict(sin=P + 0x400000, sout=P + 0x400000), ALIAS), (dict(sout=P + 0x100000), ALIAS),
    (dict(y=P), ALIAS), (dict(fl=4), FLAGS), (dict(dtype=3), DTYPE), (dict(dstate=5), SHAPE),
])
def test_conv_scan_validation(kw, code):
    assert _cscan(**kw) == code


def test_conv_scan_workspace_checked_before_launch():
    assert _cscan(ws=None, wsb=0) == WS
    assert _cscan(batch=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(K=0), SHAPE), (dict(K=7), SHAPE), (dict(w=None), NULL), (dict(cs=None), NULL),
    (dict(cs=P + 0x300002), ALIGN), (dict(cs=P), ALIAS), (dict(cs=P + 0x100000), ALIAS),
    (dict(fl=8), FLAGS), (dict(state=None), NULL),
])
def test_conv_update_validation(kw, code):
    assert _cupd(**kw) == code


def test_conv_update_width_one_needs_no_state():
    # K = 1: no carried inputs; an empty problem returns before any launch
    assert _cupd(cs=None, K=1, batch=0) == OK


def _bwd(**kw):
    a = dict(u=P, delta=P + 0x10000, A=P + 0x20000, B=P + 0x30000, C=P + 0x40000, D=None, z=None,
             bias=None, fl=1, h0=None, dy=P + 0x50000, dlast=None, du=P + 0x60000, dd=P + 0x70000,
             dA=P + 0x80000, dB=P + 0x90000, dC=P + 0xA0000, dD=None, dz=None, dbias=None, dh0=None,
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
    (dict(z=P + 0xB0000), NULL),
    (dict(du=P + 1), ALIGN), (dict(dA=P + 2), ALIGN), (dict(dlast=P + 1), ALIGN),
    (dict(du=P), ALIAS), (dict(dB=P + 0x30000), ALIAS), (dict(ddelta=None, dd=P + 0x50000), ALIAS),
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
    assert _bwd(ws=P, wsb=need - 1) == WS
    assert _bwd(batch=0) == OK


def _ssd(**kw):
    a = dict(x=P, dt=P + 0x10000, A=P + 0x20000, B=P + 0x30000, C=P + 0x40000, D=None, z=None,
             bias=None, fl=1, h0=None, y=P + 0x50000, last=None, batch=1, H=4, hd=64, N=128, L=2048,
             dtype=1, ws=P + 0x1000000, wsb=1 << 24, stream=None)
    a.update(kw)
    return load().ssm_ssd_scan_fwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["z"], a["bias"],
                                   a["fl"], a["h0"], a["y"], a["last"], a["batch"], a["H"], a["hd"],
                                   a["N"], a["L"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(hd=32), SHAPE), (dict(N=8), SHAPE), (dict(N=128, dtype=0), SHAPE), (dict(N=256), SHAPE),
    (dict(H=-1), SHAPE), (dict(L=-1), SHAPE), (dict(dtype=4), DTYPE), (dict(fl=8), FLAGS),
    (dict(x=None), NULL), (dict(dt=None), NULL), (dict(A=None), NULL), (dict(y=None), NULL),
    (dict(x=P + 1), ALIGN), (dict(A=P + 0x20002), ALIGN), (dict(y=P), ALIAS),
    (dict(ws=P + 0x1000010), ALIGN), (dict(ws=None), WS), (dict(wsb=1000), WS),
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
