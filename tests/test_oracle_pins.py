"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself through a retyped formula: each
check is a printed value from the pages (tests/golden/*.json), a closed form,
an identity stated on the pages (convolution = recurrence, scans equal), or an
independent brute-force form from tests/brute.py.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests import brute
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _single_step_abar(A, x, softplus=True):
    """Abar = exp(Delta*A) read off the oracle: one step from h0 = 1 with no
    input (u = 0) and C = 1, so y = last_state = Abar."""
    u = np.zeros((1, 1, 1))
    dr = np.array([[[x]]], dtype=np.float64)
    Am = np.array([[A]], dtype=np.float64)
    B = np.zeros((1, 1, 1))
    C = np.ones((1, 1, 1))
    h0 = np.ones((1, 1, 1))
    y, last = oracle.scan_fwd(u, dr, Am, B, C, h0=h0, delta_softplus=softplus)
    assert y[0, 0, 0] == last[0, 0, 0]
    return y[0, 0, 0]


def _single_step_delta(x):
    """Delta = softplus(x) read off the oracle: A = 0 (Abar = 1), h0 = 0,
    u = B = C = 1, so y = Delta."""
    y, _ = oracle.scan_fwd(np.ones((1, 1, 1)), np.array([[[x]]]), np.zeros((1, 1)),
                           np.ones((1, 1, 1)), np.ones((1, 1, 1)))
    return y[0, 0, 0]


# ---------------------------------------------------------------- worked impulse
def _impulse_setup(through_softplus):
    g = _golden("impulse_response.json")
    L = len(g["x"])
    u = np.array(g["x"], dtype=np.float64).reshape(1, 1, L)
    A = np.log(np.array(g["Abar_diag"])).reshape(1, 2)
    B = np.repeat(np.array(g["Bbar"]).reshape(1, 2, 1), L, axis=2)  # Delta = 1 -> Bbar = B
    C = np.repeat(np.array(g["C"]).reshape(1, 2, 1), L, axis=2)
    if through_softplus:
        dr = np.zeros((1, 1, L))
        bias = np.array([math.log(math.e - 1.0)])   # softplus(ln(e-1)) = 1
        return g, dict(u=u, delta=dr, A=A, B=B, C=C, delta_bias=bias, delta_softplus=True)
    dr = np.ones((1, 1, L))
    return g, dict(u=u, delta=dr, A=A, B=B, C=C, delta_softplus=False)


@pytest.mark.parametrize("through_softplus", [False, True])
def test_worked_impulse_response(through_softplus):
    g, kw = _impulse_setup(through_softplus)
    y, last = oracle.scan_fwd(**kw)
    np.testing.assert_allclose(y[0, 0], g["y"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(last[0, 0], g["h"][-1], rtol=0, atol=1e-12)
    # intermediate states: run the first k steps
    for k in range(1, 4):
        kk = {key: (v[..., :k] if key in ("u", "delta", "B", "C") else v) for key, v in kw.items()}
        _, hk = oracle.scan_fwd(**kk)
        np.testing.assert_allclose(hk[0, 0], g["h"][k - 1], rtol=0, atol=1e-12)


def test_impulse_response_is_the_convolution_kernel():
    g, kw = _impulse_setup(False)
    y, _ = oracle.scan_fwd(**kw)
    yc, K = brute.lti_convolution_y(g["x"], g["Abar_diag"], g["Bbar"], g["C"])
    np.testing.assert_allclose(K, g["kernel"], atol=1e-12)
    np.testing.assert_allclose(y[0, 0], yc, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_lti_recurrence_equals_convolution(seed):
    """Constant Delta, B, C over time: the output equals the convolution of the
    input with (C.Bbar, C.Abar.Bbar, ...)."""
    rng = np.random.default_rng(100 + seed)
    N, L = 3, 40
    A = -rng.uniform(0.1, 2.0, size=N)
    dl = rng.uniform(0.05, 0.8)
    B = rng.standard_normal(N)
    C = rng.standard_normal(N)
    x = rng.standard_normal(L)
    y, _ = oracle.scan_fwd(x.reshape(1, 1, L), np.full((1, 1, L), dl), A.reshape(1, N),
                           np.repeat(B.reshape(1, N, 1), L, axis=2),
                           np.repeat(C.reshape(1, N, 1), L, axis=2), delta_softplus=False)
    yc, _ = brute.lti_convolution_y(x, np.exp(dl * A), dl * B, C)
    np.testing.assert_allclose(y[0, 0], yc, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------- printed values
def test_zoh_values():
    for e in _golden("discretisation_values.json")["zoh_abar"]:
        v = _single_step_abar(e["A"], e["delta"], softplus=False)
        assert abs(v - e["abar"]) <= e["tol"], e


def test_softplus_values():
    for e in _golden("discretisation_values.json")["softplus"]:
        v = _single_step_delta(e["x"])
        assert abs(v - e["value"]) <= e["tol"], e


def test_softplus_then_zoh_values_and_decay_steps():
    g = _golden("discretisation_values.json")
    for e in g["softplus_zoh"]:
        v = _single_step_abar(e["A"], e["x"], softplus=True)
        assert abs(v - e["abar"]) <= e["tol"], e
    for e in g["decay_steps"]:
        a = _single_step_abar(e["A"], e["x"], softplus=True)
        n = -1.0 / math.log(a)
        assert abs(n - e["steps"]) <= e["tol"], e


def test_softplus_zoh_closed_form_is_logistic():
    """With A = -1, exp(-softplus(x)) = 1/(1+e^x) exactly (ln(1+e^x) is the
    softplus; exp of its negative is the logistic of -x).  Checked over a
    wide range, which also covers the overflow-prone and digit-losing ends
    of softplus."""
    for x in np.linspace(-40, 40, 161):
        v = _single_step_abar(-1.0, float(x), softplus=True)
        ref = 1.0 / (1.0 + math.exp(x))
        assert abs(v - ref) <= 1e-15 + 1e-13 * ref, (x, v, ref)


def test_softplus_extremes_finite():
    assert _single_step_delta(1000.0) == 1000.0
    v = _single_step_delta(-1000.0)
    assert v >= 0.0 and v < 1e-300
    assert abs(_single_step_delta(-30.0) - math.exp(-30.0)) < 1e-25


# ------------------------------------------------------------ brute-force sums
def _tiny_case(rng, batch=2, dim=3, N=4, L=12, gate=True, dskip=True, h0=False):
    u = rng.standard_normal((batch, dim, L))
    dr = 0.5 * rng.standard_normal((batch, dim, L))
    A = -rng.uniform(0.2, 3.0, size=(dim, N))
    B = rng.standard_normal((batch, N, L))
    C = rng.standard_normal((batch, N, L))
    bias = rng.uniform(-3.0, -0.5, size=dim)
    D = rng.standard_normal(dim) if dskip else None
    z = rng.standard_normal((batch, dim, L)) if gate else None
    hh = rng.standard_normal((batch, dim, N)) if h0 else None
    return dict(u=u, delta=dr, A=A, B=B, C=C, D=D, z=z, delta_bias=bias, h0=hh)


@pytest.mark.parametrize("gate,dskip,h0", [(False, False, False), (True, True, False),
                                           (True, False, True), (False, True, True)])
def test_oracle_equals_semiseparable_sum(gate, dskip, h0):
    rng = np.random.default_rng(7)
    kw = _tiny_case(rng, gate=gate, dskip=dskip, h0=h0)
    y, _ = oracle.scan_fwd(**kw)
    yb = brute.semiseparable_y(kw["u"], kw["delta"], kw["A"], kw["B"], kw["C"], kw["D"], kw["z"],
                               kw["delta_bias"], True, kw["h0"])
    np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_oracle_equals_semiseparable_sum_on_c0():
    inp = synth.make_scan_inputs(synth.SCAN_CONFIGS["c0"])
    w = {k: synth.widen(inp[k], "f32") for k in ("u", "delta", "B", "C", "z")}
    y, _ = oracle.scan_fwd(w["u"], w["delta"], inp["A"], w["B"], w["C"], inp["D"], w["z"],
                           inp["delta_bias"])
    yb = brute.semiseparable_y(w["u"], w["delta"], inp["A"].astype(np.float64), w["B"], w["C"],
                               inp["D"], w["z"], inp["delta_bias"], True)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-11 * np.abs(yb).max())


def test_no_decay_is_cumulative_sum():
    """A = 0 gives Abar = 1 (no decay, the linear-attention special case):
    y_t = sum_{s<=t} (C_t . B_s) Delta_s u_s."""
    rng = np.random.default_rng(11)
    N, L = 4, 30
    u = rng.standard_normal(L)
    dl = rng.uniform(0.01, 0.5, size=L)
    B = rng.standard_normal((N, L))
    C = rng.standard_normal((N, L))
    y, last = oracle.scan_fwd(u.reshape(1, 1, L), dl.reshape(1, 1, L), np.zeros((1, N)),
                              B.reshape(1, N, L), C.reshape(1, N, L), delta_softplus=False)
    S = np.cumsum(B * (dl * u)[None, :], axis=1)  # (N, L): running sum of inputs
    np.testing.assert_allclose(y[0, 0], np.sum(C * S, axis=0), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(last[0, 0], S[:, -1], rtol=1e-12, atol=1e-12)


def test_zero_delta_ignores_input():
    """Delta = 0: Abar = 1 and the input term vanishes, so the state is held."""
    rng = np.random.default_rng(12)
    kw = _tiny_case(rng, batch=1, dim=2, N=3, L=9, gate=False, dskip=True, h0=True)
    kw["delta"] = np.zeros_like(kw["delta"])
    kw["delta_bias"] = None
    y, last = oracle.scan_fwd(**kw, delta_softplus=False)
    np.testing.assert_array_equal(last, kw["h0"])
    ref = np.einsum("bnl,bdn->bdl", kw["C"], kw["h0"]) + kw["D"][None, :, None] * kw["u"]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-14)


def test_dskip_and_gate_by_definition():
    """D-skip and gate are not stated on the pages (parity unpinned by them);
    pinned by their definitions: with B = 0 the state stays 0 and
    y = D u silu(z); silu(0) = 0; silu(z)/z -> 1 for large z."""
    rng = np.random.default_rng(13)
    kw = _tiny_case(rng, batch=1, dim=3, N=2, L=8)
    kw["B"] = np.zeros_like(kw["B"])
    y, _ = oracle.scan_fwd(**kw)
    z = kw["z"]
    np.testing.assert_allclose(y, kw["D"][None, :, None] * kw["u"] * z / (1 + np.exp(-z)),
                               rtol=1e-14, atol=1e-15)
    kw["z"] = np.zeros_like(z)
    y0, _ = oracle.scan_fwd(**kw)
    assert np.all(y0 == 0.0)
    kw["z"] = np.full_like(z, 60.0)
    y60, _ = oracle.scan_fwd(**kw)
    np.testing.assert_allclose(y60 / 60.0, kw["D"][None, :, None] * kw["u"], rtol=1e-14)


def _oracle_gate(z):
    """silu(z) read off the scan oracle: B = 0 keeps the state at 0, D = 1
    and u = 1, so y = (C.h + D u) silu(z) = silu(z)."""
    z = np.asarray(z, np.float64)
    L = z.size
    y, _ = oracle.scan_fwd(np.ones((1, 1, L)), np.zeros((1, 1, L)), np.full((1, 1), -1.0),
                           np.zeros((1, 1, L)), np.ones((1, 1, L)), D=np.ones(1),
                           z=z.reshape(1, 1, L))
    return y[0, 0]


def _oracle_conv_silu(x):
    """silu(x) read off the convolution oracle: one identity tap, no bias."""
    x = np.asarray(x, np.float64)
    u, _ = oracle.causal_conv1d_silu(x.reshape(1, 1, -1), np.ones((1, 1)))
    return u[0, 0]


def _oracle_decode_gate(z):
    """silu(z) read off the decode oracle, as _oracle_gate."""
    z = np.asarray(z, np.float64)
    n = z.size
    y, _ = oracle.state_update(np.zeros((1, n, 1)), np.ones((1, n)), np.zeros((1, n)),
                               np.full((n, 1), -1.0), np.zeros((1, 1)), np.ones((1, 1)),
                               D=np.ones(n), z=z.reshape(1, n))
    return y[0]


_Z = np.linspace(-30.0, 30.0, 2401)


def _silu_identities_hold(f):
    """The two identities that fix silu(z) = z sigma(z) = z / (1 + e^-z):
    silu(z) - silu(-z) = z (as sigma(z) + sigma(-z) = 1), and
    silu(z) = (z/2)(1 + tanh(z/2)) (as sigma(z) = (1 + tanh(z/2))/2, with
    numpy's tanh on the right; 1 + tanh(z/2) cancels for negative z, so the
    absolute tolerance is a few ulps of z there)."""
    pos, neg = f(_Z), f(-_Z)
    odd = np.allclose(pos - neg, _Z, rtol=0.0, atol=1e-12)
    tanh_form = np.allclose(pos, 0.5 * _Z * (1.0 + np.tanh(0.5 * _Z)), rtol=1e-13, atol=1e-13)
    return odd and tanh_form


@pytest.mark.parametrize("reader", [_oracle_gate, _oracle_conv_silu, _oracle_decode_gate])
def test_silu_identities(reader):
    assert _silu_identities_hold(reader)


@pytest.mark.parametrize("wrong", [
    lambda z: z / (1.0 + np.exp(-z / 2)),        # z sigma(z/2): odd identity holds, tanh form fails
    lambda z: z / (1.0 + np.exp(z)),             # z sigma(-z)
    lambda z: z / (2.0 + np.exp(-z)),            # a wrong constant
    lambda z: np.tanh(z) * z,                    # a different gate
])
def test_silu_identities_reject_wrong_shapes(wrong):
    assert not _silu_identities_hold(wrong)


def test_dskip_enters_linearly_as_D_times_u():
    """The D-skip term adds exactly D u (gated) to the readout: y is affine
    in D with slope u silu(z), and D = 0 leaves the state-space part."""
    rng = np.random.default_rng(14)
    kw = _tiny_case(rng, batch=2, dim=3, N=4, L=11)
    y1, _ = oracle.scan_fwd(**kw)
    kw0 = dict(kw, D=np.zeros_like(kw["D"]))
    y0, _ = oracle.scan_fwd(**kw0)
    kw2 = dict(kw, D=2.0 * kw["D"])
    y2, _ = oracle.scan_fwd(**kw2)
    slope = kw["u"] * _oracle_gate(kw["z"].ravel()).reshape(kw["z"].shape)
    np.testing.assert_allclose(y1 - y0, kw["D"][None, :, None] * slope, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y2 - y1, y1 - y0, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------- scans and the operator
@pytest.mark.parametrize("L", [1, 7, 16, 33])
def test_scans_equal_sequential_and_oracle(L):
    rng = np.random.default_rng(20 + L)
    kw = _tiny_case(rng, batch=1, dim=1, N=3, L=L, gate=False, dskip=False)
    dl = brute.deltas(kw["delta"][0], kw["delta_bias"])  # (1, L)
    elems = brute.affine_elements(kw["u"][0, 0], dl[0], kw["A"][0], kw["B"][0], L)
    seq = brute.sequential_scan(elems)
    for other in (brute.hillis_steele_scan(elems), brute.blelloch_scan(elems),
                  brute.chunked_scan(elems, 4), brute.chunked_scan(elems, 5)):
        for s, o in zip(seq, other):
            np.testing.assert_allclose(o[0], s[0], rtol=1e-13)
            np.testing.assert_allclose(o[1], s[1], rtol=1e-12, atol=1e-14)
    # state after step t is the b-part of e_0 o ... o e_t (zero start)
    hs = np.array([s[1] for s in seq])  # (L, N)
    y_scan = np.sum(kw["C"][0].T * hs, axis=1)
    y, last = oracle.scan_fwd(**kw)
    np.testing.assert_allclose(y[0, 0], y_scan, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(last[0, 0], hs[-1], rtol=1e-12, atol=1e-13)


def test_operator_associative_not_commutative():
    rng = np.random.default_rng(3)
    e = [(rng.uniform(0, 1, 4), rng.standard_normal(4)) for _ in range(3)]
    l = brute.compose(brute.compose(e[0], e[1]), e[2])
    r = brute.compose(e[0], brute.compose(e[1], e[2]))
    np.testing.assert_allclose(l[0], r[0], rtol=1e-15)
    np.testing.assert_allclose(l[1], r[1], rtol=1e-14)
    ab, ba = brute.compose(e[0], e[1]), brute.compose(e[1], e[0])
    assert not np.allclose(ab[1], ba[1])


@pytest.mark.parametrize("split", [1, 17, 40])
def test_segment_split_resumes_exactly(split):
    rng = np.random.default_rng(30)
    kw = _tiny_case(rng, batch=2, dim=3, N=4, L=41, h0=True)
    y, last = oracle.scan_fwd(**kw)
    k1 = {k: (v[..., :split] if k in ("u", "delta", "B", "C", "z") else v) for k, v in kw.items()}
    y1, l1 = oracle.scan_fwd(**k1)
    k2 = {k: (v[..., split:] if k in ("u", "delta", "B", "C", "z") else v) for k, v in kw.items()}
    k2["h0"] = l1
    y2, l2 = oracle.scan_fwd(**k2)
    np.testing.assert_allclose(np.concatenate([y1, y2], axis=-1), y, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l2, last, rtol=1e-13, atol=1e-14)


def test_decode_step_extends_scan():
    """scan over L+1 tokens = scan over L tokens, then one decode step."""
    rng = np.random.default_rng(31)
    kw = _tiny_case(rng, batch=2, dim=3, N=4, L=10, h0=True)
    y, last = oracle.scan_fwd(**kw)
    k1 = {k: (v[..., :-1] if k in ("u", "delta", "B", "C", "z") else v) for k, v in kw.items()}
    _, l1 = oracle.scan_fwd(**k1)
    yd, st = oracle.state_update(l1, kw["u"][..., -1], kw["delta"][..., -1], kw["A"],
                                 kw["B"][..., -1], kw["C"][..., -1], kw["D"], kw["z"][..., -1],
                                 kw["delta_bias"])
    np.testing.assert_allclose(yd, y[..., -1], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, last, rtol=1e-13, atol=1e-14)


def test_decode_steps_equal_scan_from_state():
    """Several decode steps in a row equal one scan started from the same state."""
    rng = np.random.default_rng(32)
    kw = _tiny_case(rng, batch=2, dim=4, N=2, L=6, h0=True)
    y, last = oracle.scan_fwd(**kw)
    st = kw["h0"]
    for t in range(6):
        yd, st = oracle.state_update(st, kw["u"][..., t], kw["delta"][..., t], kw["A"],
                                     kw["B"][..., t], kw["C"][..., t], kw["D"], kw["z"][..., t],
                                     kw["delta_bias"])
        np.testing.assert_allclose(yd, y[..., t], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(st, last, rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- stability
def test_bounded_state_when_A_negative():
    """All A < 0 gives |Abar| < 1 and a bounded state: from a zero start,
    |h_t,n| <= max_s |Delta_s u_s B_s,n| / (1 - max_s Abar_s,n)."""
    inp = synth.make_scan_inputs(synth.SCAN_CONFIGS["c0"])
    w = {k: synth.widen(inp[k], "f32") for k in ("u", "delta", "B", "C")}
    L = w["u"].shape[-1]
    x = w["delta"][0] + inp["delta_bias"].astype(np.float64)[:, None]
    dl = np.logaddexp(0.0, x)  # softplus, numpy's own routine
    for d in range(inp["A"].shape[0]):
        A = inp["A"][d].astype(np.float64)
        amax = np.exp(dl[d][:, None] * A[None, :]).max(axis=0)
        drive = np.abs(dl[d][:, None] * w["u"][0, d][:, None] * w["B"][0].T).max(axis=0)
        bound = drive / (1.0 - amax)
        for t in (1, L // 3, L):
            _, h = oracle.scan_fwd(w["u"][:, d:d + 1, :t], w["delta"][:, d:d + 1, :t],
                                   inp["A"][d:d + 1], w["B"][..., :t], w["C"][..., :t],
                                   delta_bias=inp["delta_bias"][d:d + 1])
            assert np.all(np.abs(h[0, 0]) <= bound * (1 + 1e-12))


def test_positive_A_grows():
    """A > 0 gives Abar > 1: the unforced state grows (the unstable case)."""
    y, last = oracle.scan_fwd(np.zeros((1, 1, 50)), np.full((1, 1, 50), 0.1), np.array([[0.5]]),
                              np.zeros((1, 1, 50)), np.ones((1, 1, 50)), h0=np.ones((1, 1, 1)),
                              delta_softplus=False)
    np.testing.assert_allclose(last[0, 0, 0], math.exp(0.5 * 0.1 * 50), rtol=1e-12)
    assert np.all(np.diff(y[0, 0]) > 0)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(40)
    kw = _tiny_case(rng, batch=3, dim=5, N=4, L=33, h0=True)
    y1, l1 = oracle.scan_fwd(**kw, nthreads=1)
    y4, l4 = oracle.scan_fwd(**kw, nthreads=4)
    np.testing.assert_array_equal(y1, y4)
    np.testing.assert_array_equal(l1, l4)


def test_empty_inputs():
    y, last = oracle.scan_fwd(np.zeros((1, 2, 0)), np.zeros((1, 2, 0)), -np.ones((2, 3)),
                              np.zeros((1, 3, 0)), np.zeros((1, 3, 0)))
    assert y.shape == (1, 2, 0)
    np.testing.assert_array_equal(last, 0.0)


# ------------------------------------------------------- zero-order-hold input
# NN LAB "Mamba" page, "Derivation of the Discrete Transition Matrices": the
# input is held constant over each step, the ODE h' = A h + B x is solved
# over the step, and for diagonal A each state evolves on its own; the
# "Paper: Mamba" course module, "Math & data structures", gives the result
# Abar = exp(Delta A), Bbar = (exp(Delta A) - 1)/A B.  The pins below check
# the oracle's 'zoh' mode against that definition (the ODE), against the
# gated recurrence it reduces to for N = 1, A = -1, B = 1 (the course
# module's Theorem 1), against the A -> 0 limit, and against the unrolled sum.

def test_zoh_is_the_exact_solution_of_the_held_input_ode():
    from scipy.integrate import solve_ivp
    rng = np.random.default_rng(31)
    N, L = 3, 10
    A = -rng.uniform(0.3, 4.0, size=N)
    u = rng.standard_normal(L)
    dl = rng.uniform(0.05, 1.5, size=L)        # large Delta*A: Euler is far off here
    B = rng.standard_normal((N, L))
    C = rng.standard_normal((N, L))
    h0 = rng.standard_normal(N)
    y, last = oracle.scan_fwd(u.reshape(1, 1, L), dl.reshape(1, 1, L), A.reshape(1, N),
                              B.reshape(1, N, L), C.reshape(1, N, L), h0=h0.reshape(1, 1, N),
                              delta_softplus=False, bbar="zoh")
    h = h0.copy()
    for t in range(L):
        f = lambda _, hh, t=t: A * hh + B[:, t] * u[t]
        sol = solve_ivp(f, (0.0, dl[t]), h, method="DOP853", rtol=1e-12, atol=1e-14)
        h = sol.y[:, -1]
        assert abs(y[0, 0, t] - float(C[:, t] @ h)) <= 1e-9 * (1 + abs(y[0, 0, t])), t
    np.testing.assert_allclose(last[0, 0], h, rtol=1e-9, atol=1e-11)
    # and the Euler input term is a different result at these step sizes
    ye, _ = oracle.scan_fwd(u.reshape(1, 1, L), dl.reshape(1, 1, L), A.reshape(1, N),
                            B.reshape(1, N, L), C.reshape(1, N, L), h0=h0.reshape(1, 1, N),
                            delta_softplus=False)
    assert np.max(np.abs(ye - y)) > 1e-2


def test_zoh_single_state_is_the_gated_recurrence():
    """N = 1, A = -1, B = C = 1, Delta = softplus(x): Abar = 1 - sigmoid(x),
    Bbar = sigmoid(x), so h_t = (1 - g_t) h_{t-1} + g_t u_t, g_t = sigmoid(x_t)."""
    rng = np.random.default_rng(32)
    L = 50
    x = 3.0 * rng.standard_normal(L)
    u = rng.standard_normal(L)
    y, last = oracle.scan_fwd(u.reshape(1, 1, L), x.reshape(1, 1, L), -np.ones((1, 1)),
                              np.ones((1, 1, L)), np.ones((1, 1, L)), bbar="zoh")
    h = 0.0
    for t in range(L):
        g = 1.0 / (1.0 + math.exp(-x[t]))
        h = (1.0 - g) * h + g * u[t]
        assert abs(y[0, 0, t] - h) <= 1e-13 * (1 + abs(h)), t
    assert abs(last[0, 0, 0] - h) <= 1e-13 * (1 + abs(h))


def test_zoh_small_A_limit_is_euler():
    """(exp(Delta A) - 1)/A -> Delta as A -> 0, and A = 0 gives Delta itself."""
    rng = np.random.default_rng(33)
    kw = _tiny_case(rng, batch=1, dim=2, N=3, L=20)
    kw["A"] = np.zeros_like(kw["A"])
    ye, le = oracle.scan_fwd(**kw)
    yz, lz = oracle.scan_fwd(**kw, bbar="zoh")
    np.testing.assert_array_equal(yz, ye)
    np.testing.assert_array_equal(lz, le)
    kw["A"] = np.full_like(kw["A"], -1e-9)
    yz, lz = oracle.scan_fwd(**kw, bbar="zoh")
    scale = np.abs(ye).max()
    np.testing.assert_allclose(yz, ye, rtol=0, atol=1e-7 * scale)


@pytest.mark.parametrize("gate,dskip,h0", [(False, False, False), (True, True, True)])
def test_zoh_oracle_equals_semiseparable_sum(gate, dskip, h0):
    rng = np.random.default_rng(34)
    kw = _tiny_case(rng, gate=gate, dskip=dskip, h0=h0)
    y, _ = oracle.scan_fwd(**kw, bbar="zoh")
    yb = brute.semiseparable_y(kw["u"], kw["delta"], kw["A"], kw["B"], kw["C"], kw["D"], kw["z"],
                               kw["delta_bias"], True, kw["h0"], zoh=True)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


def test_zoh_decode_steps_extend_scan():
    rng = np.random.default_rng(35)
    kw = _tiny_case(rng, batch=2, dim=3, N=4, L=14, h0=True)
    yf, lf = oracle.scan_fwd(**kw, bbar="zoh")
    head = {k: (v[..., :9] if k in ("u", "delta", "B", "C", "z") else v) for k, v in kw.items()}
    _, st = oracle.scan_fwd(**head, bbar="zoh")
    for t in range(9, 14):
        yt, st = oracle.state_update(st, kw["u"][..., t], kw["delta"][..., t], kw["A"],
                                     kw["B"][..., t], kw["C"][..., t], kw["D"], kw["z"][..., t],
                                     kw["delta_bias"], bbar="zoh")
        np.testing.assert_allclose(yt, yf[..., t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st, lf, rtol=1e-12, atol=1e-13)


def test_bbar_mode_is_checked():
    with pytest.raises(ValueError):
        oracle.scan_fwd(np.ones((1, 1, 1)), np.ones((1, 1, 1)), -np.ones((1, 1)),
                        np.ones((1, 1, 1)), np.ones((1, 1, 1)), bbar="bilinear")


# ------------------------------------------------------ convolution prologue
# "Mamba" paper review, "Mamba" block description (a convolution and a
# non-linearity before the SSM) and NN LAB "Mamba" page, "Kernel Fusion in
# On-Chip SRAM" (causal 1-D convolution fused with the scan).  Reading:
# depthwise, causal, tap K-1 on the current input, bias, then silu.

def _silu(v):
    return v / (1.0 + np.exp(-v))


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_equals_numpy_convolution(K):
    """Causal conv with taps w[0..K-1] (w[K-1] on the current input) is
    np.convolve with the taps reversed, truncated to the first L outputs."""
    rng = np.random.default_rng(70 + K)
    b, dim, L = 2, 5, 23
    x = rng.standard_normal((b, dim, L))
    w = rng.standard_normal((dim, K))
    cb = rng.standard_normal(dim)
    u, st = oracle.causal_conv1d_silu(x, w, cb)
    for i in range(b):
        for d in range(dim):
            ref = np.convolve(x[i, d], w[d, ::-1])[:L] + cb[d]
            np.testing.assert_allclose(u[i, d], _silu(ref), rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(st, x[:, :, L - (K - 1):] if K > 1 else st)


def test_conv_identity_and_delay_taps():
    rng = np.random.default_rng(75)
    x = rng.standard_normal((1, 3, 12))
    cb = rng.standard_normal(3)
    w = np.zeros((3, 4)); w[:, 3] = 1.0           # current input only
    u, _ = oracle.causal_conv1d_silu(x, w, cb)
    np.testing.assert_allclose(u, _silu(x + cb[None, :, None]), rtol=1e-15)
    w = np.zeros((3, 4)); w[:, 0] = 1.0           # input three steps back
    prev = rng.standard_normal((1, 3, 3))
    u, _ = oracle.causal_conv1d_silu(x, w, None, prev)
    np.testing.assert_allclose(u[..., 3:], _silu(x[..., :-3]), rtol=1e-15)
    np.testing.assert_allclose(u[..., :3], _silu(prev), rtol=1e-15)
    u0, _ = oracle.causal_conv1d_silu(x, w)      # no state: zeros before t = 0
    np.testing.assert_array_equal(u0[..., :3], 0.0)


@pytest.mark.parametrize("split", [1, 2, 7, 19])
def test_conv_state_resumes_exactly(split):
    rng = np.random.default_rng(76)
    x = rng.standard_normal((2, 4, 20))
    w = rng.standard_normal((4, 4))
    cb = rng.standard_normal(4)
    s0 = rng.standard_normal((2, 4, 3))
    u, st = oracle.causal_conv1d_silu(x, w, cb, s0)
    u1, st1 = oracle.causal_conv1d_silu(x[..., :split], w, cb, s0)
    u2, st2 = oracle.causal_conv1d_silu(x[..., split:], w, cb, st1)
    np.testing.assert_array_equal(np.concatenate([u1, u2], -1), u)
    np.testing.assert_array_equal(st2, st)


def test_conv_short_sequence_state_out():
    """L < K-1: the new state keeps the tail of the old one."""
    s0 = np.array([[[1.0, 2.0, 3.0]]])
    x = np.array([[[4.0]]])
    _, st = oracle.causal_conv1d_silu(x, np.ones((1, 4)), None, s0)
    np.testing.assert_array_equal(st, [[[2.0, 3.0, 4.0]]])
    _, st = oracle.causal_conv1d_silu(np.zeros((1, 1, 0)), np.ones((1, 4)), None, s0)
    np.testing.assert_array_equal(st, s0)


def test_conv_decode_steps_equal_the_sequence():
    rng = np.random.default_rng(77)
    x = rng.standard_normal((2, 3, 9))
    w = rng.standard_normal((3, 4))
    cb = rng.standard_normal(3)
    s0 = rng.standard_normal((2, 3, 3))
    u, st = oracle.causal_conv1d_silu(x, w, cb, s0)
    cs = s0
    for t in range(9):
        ut, cs = oracle.conv_step(cs, x[..., t], w, cb)
        np.testing.assert_allclose(ut, u[..., t], rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(cs, st)


def test_conv_scan_is_conv_then_scan():
    """The composed oracle: its y is the scan of the convolution's output,
    and with an identity tap and no bias it is the scan of silu(x)."""
    rng = np.random.default_rng(78)
    kw = _tiny_case(rng, batch=1, dim=2, N=3, L=10)
    x = rng.standard_normal((1, 2, 10))
    w = np.zeros((2, 4)); w[:, 3] = 1.0
    y, last, _ = oracle.conv_scan_fwd(x, w, None, None, kw["delta"], kw["A"], kw["B"], kw["C"],
                                      kw["D"], kw["z"], kw["delta_bias"])
    y2, last2 = oracle.scan_fwd(_silu(x), kw["delta"], kw["A"], kw["B"], kw["C"], kw["D"], kw["z"],
                                kw["delta_bias"])
    np.testing.assert_allclose(y, y2, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(last, last2, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------- backward
# "Mamba" paper review, "Optimization": the backward pass recomputes the
# intermediate states from the inputs.  The oracle's gradients are pinned by
# central finite differences of its own forward pass (fp64): a dropped term,
# a wrong sign or a transposed index in any gradient fails them.

def _loss(kw, dy, dlast, bbar, softplus=True):
    y, last = oracle.scan_fwd(**kw, delta_softplus=softplus, bbar=bbar)
    return float(np.sum(dy * y) + (np.sum(dlast * last) if dlast is not None else 0.0))


def _fd_check(kw, dy, dlast, bbar, softplus=True, rel=2e-7):
    g = oracle.scan_bwd(**kw, delta_softplus=softplus, dy=dy, dlast=dlast, bbar=bbar)
    names = dict(u="du", delta="ddelta", A="dA", B="dB", C="dC", D="dD", z="dz",
                 delta_bias="ddelta_bias", h0="dh0")
    for key, gname in names.items():
        if kw.get(key) is None:
            continue
        x = kw[key]
        fd = np.empty_like(x)
        for i in np.ndindex(x.shape):
            old = x[i]
            eps = 1e-6 * max(1.0, abs(old))
            x[i] = old + eps
            lp = _loss(kw, dy, dlast, bbar, softplus)
            x[i] = old - eps
            lm = _loss(kw, dy, dlast, bbar, softplus)
            x[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        scale = max(np.abs(fd).max(), 1e-300)
        err = np.abs(g[gname] - fd).max() / scale
        assert err <= rel, (gname, bbar, err)
    return g


@pytest.mark.parametrize("bbar", ["euler", "zoh"])
@pytest.mark.parametrize("gate,dskip,h0,dlast", [(True, True, True, True), (False, False, False, False),
                                                 (True, False, False, True)])
def test_backward_equals_finite_differences(bbar, gate, dskip, h0, dlast):
    rng = np.random.default_rng(200)
    kw = _tiny_case(rng, batch=2, dim=3, N=4, L=9, gate=gate, dskip=dskip, h0=h0)
    dy = rng.standard_normal(kw["u"].shape)
    dl = rng.standard_normal((2, 3, 4)) if dlast else None
    _fd_check(kw, dy, dl, bbar)


def test_backward_without_softplus_and_near_zero_A():
    rng = np.random.default_rng(201)
    kw = _tiny_case(rng, batch=1, dim=2, N=3, L=7, h0=True)
    kw["delta"] = np.abs(kw["delta"]) * 0.3
    kw["delta_bias"] = None
    kw["A"][0, 0] = 0.0          # the zero-order-hold coefficient at its A = 0 limit
    kw["A"][1, 1] = -1e-4
    dy = rng.standard_normal(kw["u"].shape)
    for bbar in ("euler", "zoh"):
        _fd_check(kw, dy, None, bbar, softplus=False, rel=1e-6)


def test_backward_threads_do_not_change_results():
    rng = np.random.default_rng(202)
    kw = _tiny_case(rng, batch=3, dim=5, N=4, L=20, h0=True)
    dy = rng.standard_normal(kw["u"].shape)
    g1 = oracle.scan_bwd(**kw, dy=dy, nthreads=1)
    g4 = oracle.scan_bwd(**kw, dy=dy, nthreads=4)
    for k in g1:
        if g1[k] is not None:
            np.testing.assert_allclose(g4[k], g1[k], rtol=1e-13, atol=1e-14)


def test_backward_of_linear_special_case():
    """A = 0, no gate, no D, softplus off: y_t = sum_{s<=t} (C_t . B_s) Delta_s u_s,
    so dC[:, t] = sum_{s<=t} B_s Delta_s u_s dy_t and du_s = Delta_s sum_{t>=s} dy_t (C_t . B_s)."""
    rng = np.random.default_rng(203)
    N, L = 3, 12
    u = rng.standard_normal(L)
    dl = rng.uniform(0.1, 0.9, size=L)
    B = rng.standard_normal((N, L))
    C = rng.standard_normal((N, L))
    dy = rng.standard_normal(L)
    g = oracle.scan_bwd(u.reshape(1, 1, L), dl.reshape(1, 1, L), np.zeros((1, N)),
                        B.reshape(1, N, L), C.reshape(1, N, L), delta_softplus=False,
                        dy=dy.reshape(1, 1, L))
    S = np.cumsum(B * (dl * u)[None, :], axis=1)
    np.testing.assert_allclose(g["dC"][0], S * dy[None, :], rtol=1e-12, atol=1e-13)
    M = np.tril(C.T @ B)          # M[t, s] = C_t . B_s for s <= t
    np.testing.assert_allclose(g["du"][0, 0], dl * (M.T @ dy), rtol=1e-12, atol=1e-13)



# --------------------------------------------------------------------- SSD
# "Mamba" paper review, "Mamba 2": with a scalar-identity A the semiseparable
# matrix is M_ji = A_{j:i} (C_j . B_i), evaluated by chunks (quadratic form
# inside a chunk, the linear recurrence across chunks).  NN LAB "Mamba" page,
# "Bridging Tensor Cores and Recurrence": A = alpha I; intra-chunk dense
# products, inter-chunk state propagation.  Linear attention is the case
# Abar = I.

def _ssd_case(rng, batch=1, H=3, P=4, N=5, L=40):
    x = rng.standard_normal((batch, H * P, L))
    dt = rng.uniform(0.05, 0.6, size=(batch, H, L))
    A = -rng.uniform(0.3, 2.0, size=H)
    B = rng.standard_normal((batch, N, L))
    C = rng.standard_normal((batch, N, L))
    D = rng.standard_normal(H * P)
    h0 = rng.standard_normal((batch, H * P, N))
    return x, dt, A, B, C, D, h0


@pytest.mark.parametrize("chunk", [1, 7, 16, 40, 64])
def test_ssd_equals_chunked_quadratic_form(chunk):
    rng = np.random.default_rng(400 + chunk)
    x, dt, A, B, C, D, h0 = _ssd_case(rng)
    y, _ = oracle.ssd_scan_fwd(x, dt, A, B, C, D, delta_softplus=False, h0=h0)
    yc = brute.ssd_chunked_y(x[0], dt[0], A, B[0], C[0], chunk, D, h0[0])
    np.testing.assert_allclose(y[0], yc, rtol=1e-11, atol=1e-11 * np.abs(yc).max())


def test_ssd_linear_attention_special_case():
    """A = 0: y_t = sum_{s<=t} (C_t . B_s) Delta_s x_s, causal linear attention."""
    rng = np.random.default_rng(410)
    x, dt, A, B, C, _, _ = _ssd_case(rng, H=2, P=3, L=25)
    y, _ = oracle.ssd_scan_fwd(x, dt, np.zeros(2), B, C, delta_softplus=False)
    G = np.tril(C[0].T @ B[0])                       # (L, L) causal C_t . B_s
    for h in range(2):
        for p_ in range(3):
            d = h * 3 + p_
            ref = G @ (dt[0, h] * x[0, d])
            np.testing.assert_allclose(y[0, d], ref, rtol=1e-12, atol=1e-12)


def test_ssd_heads_share_delta_and_decay():
    """Within a head every channel sees the same decay: scaling one
    channel's input scales only its own output (the heads are SISO banks)."""
    rng = np.random.default_rng(411)
    x, dt, A, B, C, _, _ = _ssd_case(rng)
    y, _ = oracle.ssd_scan_fwd(x, dt, A, B, C, delta_softplus=False)
    x2 = x.copy()
    x2[0, 5] *= 3.0
    y2, _ = oracle.ssd_scan_fwd(x2, dt, A, B, C, delta_softplus=False)
    np.testing.assert_allclose(y2[0, 5], 3.0 * y[0, 5], rtol=1e-13)
    np.testing.assert_array_equal(np.delete(y2[0], 5, 0), np.delete(y[0], 5, 0))
