"""Independent formulations used to pin the oracle on tiny inputs.

None of these calls the oracle.  They restate what the pages fix in a
different form from the oracle's sequential loop:

* the unrolled (semiseparable) sum of the recurrence -- "Mamba" paper review,
  section "Mamba 2": y_t = sum_{s<=t} C_t^T A_t ... A_{s+1} B_s x_s;
* the convolution view for a time-invariant system -- "Exercises --
  State-space models (Mamba, S4)": kernel (C Bbar, C Abar Bbar, ...), and the
  statement that convolving with it equals running the recurrence;
* prefix scans over the affine-step operator -- NN LAB "Mamba" page, "The
  Associative Property of Linear Recurrence", and the "Paper: Mamba" course
  module (sequential, Blelloch, Hillis-Steele and chunked scans equal).
  The operator: step t is the map h -> a_t h + b_t; "first i then j" is
  (a_i, b_i) o (a_j, b_j) = (a_j a_i, a_j b_i + b_j), identity (1, 0).
"""
from __future__ import annotations

import math

import numpy as np


def naive_softplus(x: float) -> float:
    """ln(1 + e^x), written directly (fine for the moderate x used here)."""
    return math.log(1.0 + math.exp(x))


def deltas(delta_raw, bias, softplus=True):
    """Per-element Delta for a (dim, L) slab."""
    dim, L = delta_raw.shape
    out = np.empty((dim, L))
    for d in range(dim):
        for t in range(L):
            x = float(delta_raw[d, t]) + (float(bias[d]) if bias is not None else 0.0)
            out[d, t] = naive_softplus(x) if softplus else x
    return out


def semiseparable_y(u, delta_raw, A, B, C, D=None, z=None, bias=None, softplus=True, h0=None,
                    zoh=False):
    """Unrolled-sum form, O(L^2 N) per channel.  Shapes as the oracle's.
    zoh: input coefficient (Abar - 1)/A (zero-order hold, A != 0) instead of
    Delta (Euler)."""
    u = np.asarray(u, np.float64)
    batch, dim, L = u.shape
    N = A.shape[1]
    y = np.zeros((batch, dim, L))
    for b in range(batch):
        dl = deltas(np.asarray(delta_raw[b], np.float64), bias, softplus)  # (dim, L)
        for d in range(dim):
            Ad = np.asarray(A[d], np.float64)
            abar = np.exp(dl[d][:, None] * Ad[None, :])  # (L, N)
            coef = (abar - 1.0) / Ad[None, :] if zoh else np.repeat(dl[d][:, None], N, axis=1)
            for t in range(L):
                acc = 0.0
                for s in range(t + 1):
                    prod = np.ones(N)
                    for r in range(s + 1, t + 1):
                        prod = prod * abar[r]
                    acc += float(np.sum(C[b, :, t] * prod * coef[s] * B[b, :, s] * u[b, d, s]))
                if h0 is not None:
                    prod = np.ones(N)
                    for r in range(0, t + 1):
                        prod = prod * abar[r]
                    acc += float(np.sum(C[b, :, t] * prod * h0[b, d]))
                if D is not None:
                    acc += float(D[d]) * u[b, d, t]
                if z is not None:
                    zz = float(z[b, d, t])
                    acc *= zz / (1.0 + math.exp(-zz))
                y[b, d, t] = acc
    return y


def lti_convolution_y(x, abar, bbar, c):
    """Time-invariant system: y = K * x with K_k = sum_n c_n abar_n^k bbar_n."""
    x = np.asarray(x, np.float64)
    L = len(x)
    k = np.arange(L)[:, None]
    K = np.sum(np.asarray(c)[None, :] * np.power(np.asarray(abar)[None, :], k)
               * np.asarray(bbar)[None, :], axis=1)
    return np.convolve(x, K)[:L], K


def compose(e1, e2):
    """e1 then e2 for affine steps h -> a h + b (elementwise over states)."""
    a1, b1 = e1
    a2, b2 = e2
    return (a2 * a1, a2 * b1 + b2)


def identity_like(e):
    return (np.ones_like(e[0]), np.zeros_like(e[1]))


def sequential_scan(elems):
    out, acc = [], None
    for e in elems:
        acc = e if acc is None else compose(acc, e)
        out.append(acc)
    return out


def hillis_steele_scan(elems):
    """Inclusive log-step scan: at step k, x_i <- x_{i-2^k} o x_i."""
    x = list(elems)
    n, k = len(x), 1
    while k < n:
        x = [x[i] if i < k else compose(x[i - k], x[i]) for i in range(n)]
        k *= 2
    return x


def blelloch_scan(elems):
    """Work-efficient up-sweep / down-sweep, exclusive, then made inclusive."""
    n = len(elems)
    size = 1
    while size < n:
        size *= 2
    ident = identity_like(elems[0])
    t = list(elems) + [ident] * (size - n)
    d = 1
    while d < size:  # up-sweep
        for i in range(2 * d - 1, size, 2 * d):
            t[i] = compose(t[i - d], t[i])
        d *= 2
    t[size - 1] = ident
    d = size // 2
    while d >= 1:  # down-sweep
        for i in range(2 * d - 1, size, 2 * d):
            left = t[i - d]
            t[i - d] = t[i]
            t[i] = compose(t[i], left)
        d //= 2
    return [compose(t[i], elems[i]) for i in range(n)]


def chunked_scan(elems, chunk):
    """Scan each chunk from the identity, scan the chunk totals, then apply
    each chunk's carry-in to its local prefixes."""
    n = len(elems)
    local, totals = [], []
    for c0 in range(0, n, chunk):
        part = sequential_scan(elems[c0:c0 + chunk])
        local.append(part)
        totals.append(part[-1])
    out, carry = [], None
    for ci, part in enumerate(local):
        for p in part:
            out.append(p if carry is None else compose(carry, p))
        carry = totals[ci] if carry is None else compose(carry, totals[ci])
    return out


def affine_elements(u_row, dl_row, A_row, B_b, L):
    """Elements (Abar_t, Bbar_t x_t) of one channel, arrays over states."""
    return [(np.exp(dl_row[t] * A_row), dl_row[t] * B_b[:, t] * u_row[t]) for t in range(L)]


def ssd_chunked_y(x, dt, A_head, B, C, chunk, D=None, h0=None):
    """The SSD evaluation the pages describe, in plain numpy: within each
    chunk the quadratic (masked-attention) form
        Y_diag = (L o (C^T B)) (Delta x),  L[t, s] = exp(sum_{s<k<=t} Delta_k A)
    plus the contribution of the state entering the chunk, and across
    chunks the linear recurrence of the chunk states.  Delta = dt (already
    positive; no softplus or bias here), Euler input term, no gate.
    x: (dim, L) for one batch row, dt: (H, L), B, C: (N, L), h0: (dim, N).
    Independent of the sequential oracle: no per-step recurrence."""
    x = np.asarray(x, np.float64)
    dim, L = x.shape
    H = len(A_head)
    P = dim // H
    N = B.shape[0]
    y = np.zeros((dim, L))
    for h in range(H):
        Xh = x[h * P:(h + 1) * P]                     # (P, L)
        S = np.zeros((N, P)) if h0 is None else np.asarray(h0[h * P:(h + 1) * P], np.float64).T
        for c0 in range(0, L, chunk):
            c1 = min(c0 + chunk, L)
            q = c1 - c0
            dl = np.asarray(dt[h, c0:c1], np.float64)
            la = dl * A_head[h]
            cum = np.cumsum(la)                        # inclusive log-decay from the chunk start
            Lm = np.tril(np.exp(cum[:, None] - cum[None, :]))
            G = C[:, c0:c1].T @ B[:, c0:c1]            # (q, q): C_t . B_s
            Xc = Xh[:, c0:c1] * dl[None, :]            # Delta_s x_s, (P, q)
            Yd = (G * Lm) @ Xc.T                        # (q, P)
            Yo = (np.exp(cum)[:, None] * (C[:, c0:c1].T @ S))   # state entering the chunk
            y[h * P:(h + 1) * P, c0:c1] = (Yd + Yo).T
            w = np.exp(cum[-1] - cum)                   # decay from each step to the chunk end
            S = np.exp(cum[-1]) * S + (B[:, c0:c1] * w[None, :]) @ Xc.T
    if D is not None:
        y += np.asarray(D, np.float64)[:, None] * x
    return y
