"""GPU parity of ssm_scan_bwd against the oracle's fp64 backward (itself
pinned by finite differences of the forward).

Recomputation for backpropagation: "Mamba" paper review, "Optimization".
Each gradient tensor is compared on its own: max|g_gpu - g_ref| <=
tol * max|g_ref| (tol as for the forward: 1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest

import oracle
import synth
from synth.configs import ScanConfig
from tests.helpers import TOL, assert_parity, to_torch, widened

pytestmark = pytest.mark.gpu

GRADS = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "ddelta_bias", "dh0")


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import selective_state_space_28_amd as ssm
    ssm.load()
    return torch.device("cuda:0")


def _case(dtype, b=2, d=70, n=16, L=77, seed=11, gate=True, dskip=True, jitter=0.1):
    cfg = ScanConfig("t", b, d, n, L, dtype, seed=seed, gate=gate, dskip=dskip, a_jitter=jitter)
    inp = synth.make_scan_inputs(cfg)
    rng = np.random.default_rng([seed, 2_000_003])
    dy = rng.standard_normal((b, d, L), dtype=np.float32)
    inp["dy"] = synth.bf16_bits(dy) if dtype == "bf16" else dy
    return inp


def gpu_bwd(inp, dev, h0=None, dlast=None, softplus=True, bbar="euler"):
    import torch
    import selective_state_space_28_amd as ssm
    dt = inp["dtype"]
    t = {k: to_torch(inp.get(k), dt, dev) for k in ("u", "delta", "B", "C", "z", "dy")}
    A, D, bias = (to_torch(inp.get(k), "f32", dev) for k in ("A", "D", "delta_bias"))
    g = ssm.ssm_scan_bwd(t["u"], t["delta"], A, t["B"], t["C"], D, t["z"], bias,
                         delta_softplus=softplus, h0=to_torch(h0, "f32", dev), dy=t["dy"],
                         dlast_state=to_torch(dlast, "f32", dev), bbar=bbar)
    torch.cuda.synchronize(dev)
    return {k: (None if v is None else v.float().cpu().numpy().astype(np.float64)) for k, v in g.items()}


def oracle_bwd(inp, h0=None, dlast=None, softplus=True, nthreads=8, bbar="euler"):
    w = widened(inp)
    dy = synth.widen(inp["dy"], inp["dtype"])
    return oracle.scan_bwd(w["u"], w["delta"], w["A"], w["B"], w["C"], w["D"], w["z"],
                           w["delta_bias"], softplus, h0, dy=dy, dlast=dlast, nthreads=nthreads,
                           bbar=bbar)


def _compare(g, r, dtype, skip=()):
    errs = {}
    for k in GRADS:
        if k in skip or r.get(k) is None:
            continue
        if k == "dD" and g[k] is not None and r[k] is None:
            continue
        # per-token gradients in the storage type, the rest in float32
        tol_kind = dtype if k in ("du", "ddelta", "dz", "dB", "dC") else "f32"
        if dtype == "bf16":
            tol_kind = "bf16"   # every gradient inherits the bf16 rounding of the inputs
        errs[k] = assert_parity(g[k], r[k], tol_kind, k)
    print(" ".join(f"{k} {v:.1e}" for k, v in errs.items()), flush=True)
    return errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_bwd_dstate_variants(dev, dtype, n):
    inp = _case(dtype, n=n, L=93, seed=300 + n)
    g = gpu_bwd(inp, dev)
    r = oracle_bwd(inp)
    _compare(g, r, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 64, 16), (2, 129, 100), (1, 1, 1), (1, 5, 3), (1, 200, 1031)])
def test_bwd_shapes(dev, dtype, shape):
    b, d, L = shape
    inp = _case(dtype, b=b, d=d, L=L, seed=b * 1000 + d + L)
    _compare(gpu_bwd(inp, dev), oracle_bwd(inp), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_h0_dlast_no_gate_no_softplus(dev, dtype):
    inp = _case(dtype, b=2, d=70, L=130, gate=False, dskip=False)
    inp["delta_bias"] = None
    if dtype == "f32":
        inp["delta"] = np.abs(inp["delta"]) * np.float32(0.2)
    else:
        inp["delta"] = synth.bf16_bits(np.abs(synth.bf16_to_f32(inp["delta"])) * np.float32(0.2))
    rng = np.random.default_rng(9)
    h0 = rng.standard_normal((2, 70, 16)).astype(np.float32)
    dlast = rng.standard_normal((2, 70, 16)).astype(np.float32)
    g = gpu_bwd(inp, dev, h0=h0, dlast=dlast, softplus=False)
    r = oracle_bwd(inp, h0=h0, dlast=dlast, softplus=False)
    _compare(g, r, dtype, skip=("dD", "ddelta_bias"))
    # without D and bias their gradients are still the sums the formula gives
    assert_parity(g["dD"], oracle_bwd(dict(inp, D=np.zeros(70, np.float32)), h0=h0, dlast=dlast,
                                      softplus=False)["dD"], "f32", "dD (D = 0)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segs", [2, 3, 7])
def test_bwd_segment_carries(dev, dtype, segs, monkeypatch):
    """Split sequences: checkpoints cross segment starts and the adjoint
    carry composes across segments in reverse."""
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", str(segs))
    inp = _case(dtype, b=2, d=100, L=1037, seed=310 + segs)
    rng = np.random.default_rng(10)
    h0 = (rng.standard_normal((2, 100, 16)) * 0.3).astype(np.float32)
    dlast = rng.standard_normal((2, 100, 16)).astype(np.float32)
    _compare(gpu_bwd(inp, dev, h0=h0, dlast=dlast), oracle_bwd(inp, h0=h0, dlast=dlast), dtype)


def test_bwd_deterministic_bits(dev):
    inp = _case("bf16", b=2, d=200, L=500, seed=320)
    g1 = gpu_bwd(inp, dev)
    g2 = gpu_bwd(inp, dev)
    for k in GRADS:
        if g1[k] is not None:
            assert np.array_equal(g1[k], g2[k]), k


def test_bwd_full_size_c1(dev):
    """The 130M-shaped fp32 workload (batch 8, D 1536, N 16, L 2048), default
    plan, every gradient against the oracle over the whole problem."""
    cfg = synth.SCAN_CONFIGS["c1"]
    print("c1 backward: generating", flush=True)
    inp = _case("f32", b=cfg.batch, d=cfg.dim, n=cfg.dstate, L=cfg.seqlen, seed=cfg.seed, jitter=0.0)
    g = gpu_bwd(inp, dev)
    print("c1 backward: oracle", flush=True)
    r = oracle_bwd(inp, nthreads=16)
    _compare(g, r, "f32")


# ---- the zero-order-hold input term (Bbar = (Abar - 1)/A) ---------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_bwd_zoh_dstate_variants(dev, dtype, n):
    inp = _case(dtype, n=n, L=93, seed=400 + n)
    _compare(gpu_bwd(inp, dev, bbar="zoh"), oracle_bwd(inp, bbar="zoh"), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 129, 100), (1, 200, 1031)])
def test_bwd_zoh_shapes(dev, dtype, shape):
    b, d, L = shape
    inp = _case(dtype, b=b, d=d, L=L, seed=4000 + b * 1000 + d + L)
    _compare(gpu_bwd(inp, dev, bbar="zoh"), oracle_bwd(inp, bbar="zoh"), dtype)


def test_bwd_zoh_zero_and_tiny_A_h0_dlast(dev):
    """A = 0 and |Delta A| below the series threshold take the series forms of
    Bbar and dBbar/dA (Delta and Delta^2/2 at A = 0); h0, dlast, no softplus."""
    inp = _case("f32", b=2, d=70, L=130, seed=410)
    inp["delta_bias"] = None
    inp["delta"] = np.abs(inp["delta"]) * np.float32(0.2)
    inp["A"] = inp["A"].copy()
    inp["A"][0, :] = 0.0
    inp["A"][1, :] = -1e-4
    inp["A"][2, :] = -0.5          # |Delta A| around the series threshold
    rng = np.random.default_rng(11)
    h0 = rng.standard_normal((2, 70, 16)).astype(np.float32)
    dlast = rng.standard_normal((2, 70, 16)).astype(np.float32)
    g = gpu_bwd(inp, dev, h0=h0, dlast=dlast, softplus=False, bbar="zoh")
    r = oracle_bwd(inp, h0=h0, dlast=dlast, softplus=False, bbar="zoh")
    _compare(g, r, "f32")


@pytest.mark.parametrize("segs", [3])
def test_bwd_zoh_segment_carries(dev, segs, monkeypatch):
    monkeypatch.setenv("SSM_SCAN_SEGMENTS", str(segs))
    inp = _case("bf16", b=2, d=100, L=1037, seed=420)
    rng = np.random.default_rng(12)
    h0 = (rng.standard_normal((2, 100, 16)) * 0.3).astype(np.float32)
    dlast = rng.standard_normal((2, 100, 16)).astype(np.float32)
    _compare(gpu_bwd(inp, dev, h0=h0, dlast=dlast, bbar="zoh"),
             oracle_bwd(inp, h0=h0, dlast=dlast, bbar="zoh"), "bf16")
