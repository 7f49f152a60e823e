"""GPU parity of the time-parallel forward scan (scan_wave.hip: each wave one
channel and 4 states, its lanes consecutive chunks of the sequence, the
chunks' affine maps composed across the lanes) against the fp64 oracle.
SSM_SCAN_WAVE=1 selects that kernel wherever it applies (16 states, no
convolution prologue): ragged blocks, ragged channel groups, both storage
types, both input terms, every option, unaligned pointers, non-finite
inputs carried across blocks and a growing state (test_gpu_semantics.py runs
its non-finite and growth cases on this kernel too)."""
import numpy as np
import pytest

import synth
from synth.configs import ScanConfig
from tests.helpers import assert_parity, gpu_scan, oracle_scan, scaled_err, to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import selective_state_space_28_amd as ssm
    ssm.load()
    return torch.device("cuda:0")


@pytest.fixture(autouse=True)
def wave(monkeypatch):
    monkeypatch.setenv("SSM_SCAN_WAVE", "1")


def _case(dtype, b=2, d=7, L=77, seed=21, gate=True, dskip=True):
    cfg = ScanConfig("w", b, d, 16, L, dtype, seed=seed, gate=gate, dskip=dskip, a_jitter=0.1)
    return synth.make_scan_inputs(cfg)


@pytest.mark.parametrize("bbar", ["euler", "zoh"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("L", [1, 9, 511, 512, 513, 1300, 2048])
def test_wave_lengths(dev, dtype, bbar, L):
    inp = _case(dtype, L=L, seed=100 + L)
    h0 = np.random.default_rng(L).standard_normal((2, 7, 16)).astype(np.float32)
    y, last = gpu_scan(inp, dev, h0=h0, bbar=bbar)
    yr, lr = oracle_scan(inp, h0=h0, bbar=bbar)
    print(f"wave {dtype} {bbar} L={L}: y {scaled_err(y, yr):.2e} last {scaled_err(last, lr):.2e}")
    assert_parity(y, yr, dtype)
    assert_parity(last, lr, "f32", "last_state")


@pytest.mark.parametrize("d", [1, 3, 4, 5, 70])
def test_wave_channel_groups(dev, d):
    inp = _case("bf16", b=3, d=d, L=700, seed=40 + d)
    y, last = gpu_scan(inp, dev)
    yr, lr = oracle_scan(inp)
    assert_parity(y, yr, "bf16")
    assert_parity(last, lr, "f32", "last_state")


@pytest.mark.parametrize("opts", [dict(gate=False), dict(dskip=False), dict(gate=False, dskip=False)])
def test_wave_options(dev, opts):
    inp = _case("f32", L=600, seed=7, **opts)
    y, last = gpu_scan(inp, dev)
    yr, lr = oracle_scan(inp)
    assert_parity(y, yr, "f32")
    assert_parity(last, lr, "f32", "last_state")


def test_wave_no_softplus_no_bias(dev):
    inp = _case("f32", L=300, seed=8)
    inp["delta_bias"] = None
    inp["delta"] = np.abs(inp["delta"]).astype(np.float32) * 0.1
    y, last = gpu_scan(inp, dev, softplus=False)
    yr, lr = oracle_scan(inp, softplus=False)
    assert_parity(y, yr, "f32")
    assert_parity(last, lr, "f32", "last_state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wave_unaligned_pointers(dev, dtype):
    """Inputs one element past an aligned start take the element paths."""
    import torch
    import selective_state_space_28_amd as ssm
    inp = _case(dtype, L=1024, seed=9)
    t = {k: to_torch(inp.get(k), dtype, dev) for k in ("u", "delta", "B", "C", "z")}
    A, D, bias = (to_torch(inp[k], "f32", dev) for k in ("A", "D", "delta_bias"))

    def off(x):
        flat = torch.empty(x.numel() + 1, dtype=x.dtype, device=x.device)
        v = flat[1:].view(x.shape)
        v.copy_(x)
        return v
    y = ssm.ssm_scan_fwd(off(t["u"]), off(t["delta"]), A, off(t["B"]), off(t["C"]), D, off(t["z"]), bias)
    torch.cuda.synchronize(dev)
    yr, _ = oracle_scan(inp)
    assert_parity(y.float().cpu().numpy().astype(np.float64), yr, dtype)


@pytest.mark.parametrize("bbar", ["euler", "zoh"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_wave_nonfinite_across_blocks(dev, dtype, bbar):
    """NaN and Inf planted in u, delta and z (the single-block cases are in
    test_gpu_semantics.py) carried across blocks of 512 steps: the outputs
    are non-finite exactly where the oracle's are, and the rest matches."""
    from tests.test_gpu_semantics import _plant, _same_nonfinite
    inp = _case(dtype, b=1, d=6, L=1100, seed=12)
    for key, ch, t, v in (("u", 0, 5, np.nan), ("u", 1, 600, np.inf), ("delta", 2, 513, np.nan),
                          ("z", 3, 1000, -np.inf), ("u", 4, 511, -np.inf), ("delta", 5, 700, np.inf)):
        _plant(inp[key], dtype, (0, ch, t), v)
    y, last = gpu_scan(inp, dev, bbar=bbar)
    yr, lr = oracle_scan(inp, bbar=bbar)
    _, fin = _same_nonfinite(y, yr, f"y ({dtype}, {bbar})")
    assert_parity(y[fin], yr[fin], dtype, "finite part of y")
    _, finl = _same_nonfinite(last, lr, "last_state")
    assert_parity(last[finl], lr[finl], "f32", "finite part of last_state")


def test_wave_growing_state(dev):
    """A > 0: the state grows, and the composed chunk decays are growth factors."""
    inp = _case("f32", b=1, d=5, L=900, seed=13)
    inp["A"] = np.abs(inp["A"]).astype(np.float32) * 0.01
    y, last = gpu_scan(inp, dev)
    yr, lr = oracle_scan(inp)
    assert np.abs(lr).max() > 10 * np.abs(inp["u"]).max()
    assert_parity(y, yr, "f32")
    assert_parity(last, lr, "f32", "last_state")
