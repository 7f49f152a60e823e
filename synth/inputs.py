"""Input generators (see the package docstring for the recipe and draw order)."""
from __future__ import annotations

import math

import numpy as np

from .configs import ScanConfig, DecodeConfig, SsdConfig

DT_MIN, DT_MAX = 1e-3, 1e-1


def bf16_bits(x) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest, ties to even.
    (Inputs are finite draws; NaN handling is not needed here.)"""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = b + (((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> the fp32 values they denote (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def widen(arr, dtype: str) -> np.ndarray:
    """Stored tensor -> float64 values it denotes (exact)."""
    if arr is None:
        return None
    if dtype == "bf16":
        return bf16_to_f32(arr).astype(np.float64)
    return np.asarray(arr, dtype=np.float32).astype(np.float64)


def inv_softplus_bias(dt: np.ndarray) -> np.ndarray:
    """bias = ln(e^dt - 1), written as dt + ln(-expm1(-dt)) so small dt keeps
    its digits; softplus(bias) = dt."""
    dt = np.asarray(dt, dtype=np.float64)
    return dt + np.log(-np.expm1(-dt))


def _normal(rng, shape, std, dtype_store):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x) if dtype_store == "bf16" else x


def _params(rng, dim, dstate, a_jitter, dskip):
    A = -np.broadcast_to(np.arange(1, dstate + 1, dtype=np.float64), (dim, dstate)).copy()
    if a_jitter:
        A = A + a_jitter * rng.standard_normal(size=(dim, dstate))
        # kept negative; the clamp cannot bind at these sizes (>= 9 sigma)
        A = np.minimum(A, -1e-4)
    dt = np.exp(rng.uniform(math.log(DT_MIN), math.log(DT_MAX), size=dim))
    bias = inv_softplus_bias(dt).astype(np.float32)
    D = rng.standard_normal(size=dim).astype(np.float32) if dskip else None
    return A.astype(np.float32), bias, D


def make_scan_inputs(cfg: ScanConfig, seed: int | None = None) -> dict:
    """Seeded inputs for one scan workload.  Returns a dict with
    u, delta, B, C, z (float32 arrays or uint16 bf16 bits; z may be None),
    A, delta_bias, D (float32; D may be None), and 'dtype'."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, d, n, L = cfg.batch, cfg.dim, cfg.dstate, cfg.seqlen
    A, bias, D = _params(rng, d, n, cfg.a_jitter, cfg.dskip)
    delta = _normal(rng, (b, d, L), cfg.delta_std, cfg.dtype)
    u = _normal(rng, (b, d, L), 1.0, cfg.dtype)
    B = _normal(rng, (b, n, L), 1.0, cfg.dtype)
    C = _normal(rng, (b, n, L), 1.0, cfg.dtype)
    z = _normal(rng, (b, d, L), 1.0, cfg.dtype) if cfg.gate else None
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=D, z=z, delta_bias=bias, dtype=cfg.dtype)


def make_decode_params(cfg: DecodeConfig, seed: int | None = None) -> dict:
    """Layer parameters and the initial fp32 state of the decode workload."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    A, bias, D = _params(rng, cfg.dim, cfg.dstate, 0.0, cfg.dskip)
    h0 = (rng.standard_normal(size=(cfg.batch, cfg.dim, cfg.dstate), dtype=np.float32)
          * np.float32(cfg.h0_std))
    return dict(A=A, D=D, delta_bias=bias, h0=h0, dtype=cfg.dtype)


def make_decode_step(cfg: DecodeConfig, step: int, seed: int | None = None) -> dict:
    """Token inputs of decode step ``step``: u, delta, z (batch, dim) and
    B, C (batch, N), drawn from default_rng([seed, step])."""
    rng = np.random.default_rng([cfg.seed if seed is None else seed, step])
    b, d, n = cfg.batch, cfg.dim, cfg.dstate
    delta = _normal(rng, (b, d), cfg.delta_std, cfg.dtype)
    u = _normal(rng, (b, d), 1.0, cfg.dtype)
    B = _normal(rng, (b, n), 1.0, cfg.dtype)
    C = _normal(rng, (b, n), 1.0, cfg.dtype)
    z = _normal(rng, (b, d), 1.0, cfg.dtype) if cfg.gate else None
    return dict(u=u, delta=delta, B=B, C=C, z=z, dtype=cfg.dtype)


def impulse_inputs() -> dict:
    """The two-state worked impulse response as scan inputs: Abar = (0.8, 0.4),
    Bbar = (0.5, 1.0), C = (2, -1), x = (1, 0, 0).  Delta = 1 is produced by
    delta_raw = 0 and bias = ln(e - 1) through softplus; A = (ln 0.8, ln 0.4).
    The expected outputs are not computed here (they are the page's values)."""
    L = 3
    u = np.array([[[1.0, 0.0, 0.0]]], dtype=np.float32)
    delta = np.zeros((1, 1, L), dtype=np.float32)
    A = np.array([[math.log(0.8), math.log(0.4)]], dtype=np.float32)
    B = np.array([[[0.5] * L, [1.0] * L]], dtype=np.float32)
    C = np.array([[[2.0] * L, [-1.0] * L]], dtype=np.float32)
    bias = np.array([math.log(math.e - 1.0)], dtype=np.float32)
    return dict(u=u, delta=delta, A=A, B=B, C=C, D=None, z=None, delta_bias=bias, dtype="f32")


def make_conv_params(dim: int, width: int, seed: int, state_batch: int | None = None) -> dict:
    """Convolution prologue parameters, drawn from ``default_rng([seed, 1_000_003])``
    in the order w -> b (-> state): taps w (dim, width) and bias b (dim,)
    uniform in +-1/sqrt(width) (the fan-in of a depthwise filter), and when
    state_batch is given a carried input state (state_batch, dim, width-1)
    ~ N(0, 1).  All float32."""
    rng = np.random.default_rng([seed, 1_000_003])
    bound = 1.0 / math.sqrt(width)
    w = rng.uniform(-bound, bound, size=(dim, width)).astype(np.float32)
    b = rng.uniform(-bound, bound, size=dim).astype(np.float32)
    out = dict(conv_w=w, conv_b=b, conv_state=None)
    if state_batch is not None:
        out["conv_state"] = rng.standard_normal(size=(state_batch, dim, width - 1),
                                                dtype=np.float32)
    return out


def make_ssd_inputs(cfg: SsdConfig, seed: int | None = None) -> dict:
    """Seeded inputs of an SSD workload, drawn in the order
    A_head -> dt (-> dt_bias) -> D -> dt_raw -> x -> B -> C -> z:
    A_head = -U(1, 16) per head; dt_bias = softplus^-1 of a log-uniform step
    in [1e-3, 1e-1]; D, x, B, C, z ~ N(0, 1); dt_raw ~ N(0, delta_std^2).
    x, z: (batch, dim, L); dt_raw: (batch, nheads, L); B, C: (batch, N, L)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    b, H, L = cfg.batch, cfg.nheads, cfg.seqlen
    A = -rng.uniform(1.0, 16.0, size=H).astype(np.float32)
    dtv = np.exp(rng.uniform(math.log(DT_MIN), math.log(DT_MAX), size=H))
    dt_bias = inv_softplus_bias(dtv).astype(np.float32)
    D = rng.standard_normal(size=cfg.dim).astype(np.float32) if cfg.dskip else None
    dt = _normal(rng, (b, H, L), cfg.delta_std, cfg.dtype)
    x = _normal(rng, (b, cfg.dim, L), 1.0, cfg.dtype)
    B = _normal(rng, (b, cfg.dstate, L), 1.0, cfg.dtype)
    C = _normal(rng, (b, cfg.dstate, L), 1.0, cfg.dtype)
    z = _normal(rng, (b, cfg.dim, L), 1.0, cfg.dtype) if cfg.gate else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, dt_bias=dt_bias, dtype=cfg.dtype)
