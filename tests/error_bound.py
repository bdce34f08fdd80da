"""Per-element error bounds of the GPU layer's outputs (test infrastructure).

The HIP path computes the expert FFN with fp32 accumulation and rounds the
hidden activations H, the expert outputs and y to the storage type (bf16, or
fp32 on the fp32 path).  Applied to the exact intermediates of the same
inputs, each rounding step bounds how far the GPU's value can be from the
exact one, element by element:

  storage rounding   |rnd(v) - v| <= ub |v|: round to nearest with p
                     significand bits has unit roundoff 2^-p, so ub = 2^-8
                     for bf16 (p = 8) and 2^-23 for fp32 (2^-24, doubled)
  fp32 sums          a sum of n products is built from MFMA (or FMA) steps of
                     at most 16 products added to an fp32 accumulator: at most
                     n/16 + 16 roundings, each at most 2^-23 times the partial
                     sum it rounds (2^-23: any rounding direction, also a
                     biased one).  The partial sums of these sums (random
                     signs) are bounded by 4 ||terms||_2, so
                     ACC(n) = 2^-23 (ceil(n/16) + 16) 4 ||terms||_2.
                     The worst case n u sum|terms| grows with n, and for
                     Mixtral-sized sums it exceeds the bf16 rounding it sits
                     beside by a factor of ten; the measured fp32 error is
                     orders of magnitude below ACC.
  first layer        a = W1 u (+ b1):  Ea = ACC(d + 1)
  ReLU               |h' - H| <= Ea + ub (|H| + Ea)
  SwiGLU             h' = rnd(fl(silu'(a') g')), silu' within es of silu and
                     |silu(a') - silu(a)| <= 1.1 |a' - a| (|silu'| < 1.1):
                     D = (1.1 Ea + es (|s| + 1.1 Ea)) (|g| + Eg) + |s| Eg,
                     |h' - H| <= D + (2^-23 + ub) (|H| + D)
  second layer       o = W2 h' (+ b2): P = |W2| Eh (every rounding of H with
                     the worst signs), Eo = P + ACC(f + 1) + ub (|o| + ...)
  combine            y = rnd(sum_j g'_j o'_j), |g' - g| <= 1e-5 g + 1e-7
                     (the gate bar the routing check enforces)

The bound terms are computed in fp32 (their own relative error, at most
about 1e-3, is covered by a 1 % slack).  The tolerance stated for the layer
(max-abs 2e-2, mean relative error 5e-3 as the ratio of L1 norms) is checked
as well; the element bound is what catches a wrong tile, row or column,
which the norms alone can miss.
"""
from __future__ import annotations

import math

import numpy as np

U = 2.0 ** -23              # one fp32 rounding, doubled
ES = 2.0 ** -18             # relative error allowed for the GPU's SiLU (hardware exp2 / rcp)
SILU_SLOPE = 1.1            # max |d silu / da| is 1.0998
GATE_RTOL, GATE_ATOL = 1e-5, 1e-7
SLACK = 1.01                # second-order terms and the fp32 evaluation of the bound


def unit_roundoff(store: str) -> float:
    """Rounding of a stored value: bf16 keeps 8 significand bits (2^-8), fp32 24 (doubled: U)."""
    return 2.0 ** -8 if store == "bf16" else U


def acc_factor(n: int) -> float:
    """ACC(n) / ||terms||_2 for an fp32 sum of n products."""
    return U * (math.ceil(n / 16) + 16) * 4.0


def _f32(a):
    return None if a is None else np.asarray(a, dtype=np.float32)


def expert_bound(u, W1, W2, act: str, b1=None, b2=None, W3=None, store: str = "bf16"):
    """One expert on the rows u (exact input values).

    Returns (o, Eo): the expert output (fp32 evaluation, for magnitudes) and
    the bound on the GPU's stored output, both [rows, d] float64.
    W1, W3 [f, d], W2 [d, f]."""
    ub = unit_roundoff(store)
    u, W1, W2, W3, b1, b2 = (_f32(v) for v in (u, W1, W2, W3, b1, b2))
    d = u.shape[1]
    f = W1.shape[0]
    u2 = u * u
    a = u @ W1.T
    sa = u2 @ (W1 * W1).T
    if b1 is not None:
        a = a + b1[None, :]
        sa = sa + (b1 * b1)[None, :]
    Ea = acc_factor(d + 1) * np.sqrt(sa)
    if act == "relu":
        H = np.maximum(a, 0.0)
        Eh = Ea + ub * (H + Ea)
    elif act == "swiglu":
        g = u @ W3.T
        Eg = acc_factor(d) * np.sqrt(u2 @ (W3 * W3).T)
        with np.errstate(over="ignore"):
            s = a / (1.0 + np.exp(-a))
        H = s * g
        D = (SILU_SLOPE * Ea + ES * (np.abs(s) + SILU_SLOPE * Ea)) * (np.abs(g) + Eg) + np.abs(s) * Eg
        Eh = D + (U + ub) * (np.abs(H) + D) + np.float32(1e-30)
    else:
        raise ValueError(act)
    o = H @ W2.T
    so = (H * H) @ (W2 * W2).T
    if b2 is not None:
        o = o + b2[None, :]
        so = so + (b2 * b2)[None, :]
    P = Eh @ np.abs(W2).T
    pre = P.astype(np.float64) + acc_factor(f + 1) * np.sqrt(so.astype(np.float64))
    Eo = pre + ub * (np.abs(o.astype(np.float64)) + pre)
    return o.astype(np.float64), Eo * SLACK


def _widen(a, dtype):
    """Storage values as fp32 (bf16 patterns are the top 16 bits of fp32)."""
    if a is None:
        return None
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return np.asarray(a, dtype=np.float32)


def layer_bound(cfg: dict, idx: np.ndarray, slot: np.ndarray, gate: np.ndarray, tokens=None):
    """Bound on every element of the GPU's y for the choices (idx, slot, gate).

    Returns (y, Ey) [T, d] float64: y the layer output from the fp32
    evaluation (for magnitudes only), Ey the bound.  A token not in `tokens`
    (when given) gets an infinite bound.  Dropped choices (slot < 0) add
    nothing to either."""
    dt = cfg["dtype"]
    ub = unit_roundoff(dt)
    x = _widen(cfg["x"], dt)
    T, k = idx.shape
    d = x.shape[1]
    want = np.ones(T, dtype=bool)
    if tokens is not None:
        want[:] = False
        want[np.asarray(tokens)] = True
    y = np.zeros((T, d))
    err = np.zeros((T, d))
    mag = np.zeros((T, d))
    g64 = np.asarray(gate, dtype=np.float64)
    for e in np.unique(idx):
        tt, jj = np.nonzero((idx == e) & (slot >= 0) & want[:, None])
        if tt.size == 0:
            continue
        pick = lambda w: None if w is None else _widen(w[e], dt)   # noqa: E731
        o, Eo = expert_bound(x[tt], pick(cfg["W1"]), pick(cfg["W2"]), cfg["act"], b1=pick(cfg["b1"]),
                             b2=pick(cfg["b2"]), W3=pick(cfg["W3"]), store=dt)
        g = g64[tt, jj][:, None]
        dg = GATE_RTOL * g + GATE_ATOL
        # a token meets expert e at most once, so the rows tt are distinct
        y[tt] += g * o
        err[tt] += g * Eo + dg * (np.abs(o) + Eo)
        mag[tt] += (g + dg) * (np.abs(o) + Eo)
    s = err + k * U * mag
    Ey = (s + ub * (np.abs(y) + s)) * SLACK
    Ey[~want] = np.inf
    return y, Ey


def check_elementwise(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, rows=None, what="y"):
    """Every element within its bound; returns the largest |error| / bound."""
    if rows is not None:
        got, ref, bound = got[rows], ref[rows], bound[rows]
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    bad = ~(err <= bound)
    if bad.any():
        i = tuple(int(v) for v in np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the rounding bound, first at "
                             f"{i}: |err| {err[i]:.3e} > bound {bound[i]:.3e}")
    fin = np.isfinite(bound) & (bound > 0)
    return float(np.max(err[fin] / bound[fin])) if fin.any() else 0.0


SILU_GRAD_SLOPE = 0.55      # max |d^2 silu / da^2| is 0.5 (at a = 0)


def expert_backward_bound(u, W1, W2, act: str, dY, b1=None, W3=None, store: str = "bf16", rows_pad=None):
    """Bounds of the GPU's expert-FFN backward for one expert's rows, from the
    same rounding model as the forward: the recomputed A', G', dH' and the
    activation outputs H', dA', dG' are stored (ub), every product sum is an
    fp32 sum (ACC), and the bf16 inputs u, dY and the weights are exact.

      ReLU:   mask' = 1[A' > 0] equals 1[A > 0] wherever |A| > EA; elsewhere
              dA' may be dH' or 0, so the bound there is |dH| + EdH.
      SwiGLU: |silu'(A') - silu'(A)| <= 0.55 |A' - A| (|silu''| <= 0.5) plus
              the hardware exp2 / rcp error es on sigma and a sigma (1 - sigma).

    rows_pad: the contraction length of the weight-gradient sums (rows of the
    expert rounded up to the GPU's K tile); defaults to the row count.
    Returns a dict name -> (exact fp32 evaluation, bound) for du, dW1, dW2,
    dW3 (SwiGLU), db1 and db2, float64 arrays."""
    ub = unit_roundoff(store)
    u, W1, W2, W3, b1, dY = (_f32(v) for v in (u, W1, W2, W3, b1, dY))
    n, d = u.shape
    f = W1.shape[0]
    npad = n if rows_pad is None else rows_pad
    sw = act == "swiglu"
    u2, dY2 = u * u, dY * dY
    aW1, aW2 = np.abs(W1), np.abs(W2)
    a = u @ W1.T
    sa = u2 @ (W1 * W1).T
    if b1 is not None:
        a = a + b1[None, :]
        sa = sa + (b1 * b1)[None, :]
    ea = acc_factor(d + 1) * np.sqrt(sa)
    EA = ea + ub * (np.abs(a) + ea)
    dH = dY @ W2
    edh = acc_factor(d) * np.sqrt(dY2 @ (W2 * W2))
    EdH = edh + ub * (np.abs(dH) + edh)
    out = {}
    if not sw:
        H = np.maximum(a, 0.0)
        EH = EA
        dA = dH * (a > 0)
        sure = np.abs(a) > EA
        EdA = np.where(sure, (a > 0) * EdH + ub * (np.abs(dA) + EdH), (np.abs(dH) + EdH) * (1 + ub))
        dG = EdG = None
    else:
        g = u @ W3.T
        eg = acc_factor(d) * np.sqrt(u2 @ (W3 * W3).T)
        EG = eg + ub * (np.abs(g) + eg)
        with np.errstate(over="ignore"):
            sg = 1.0 / (1.0 + np.exp(-a))
        s = a * sg
        s1 = sg * (1.0 + a * (1.0 - sg))
        ds = SILU_SLOPE * EA + ES * (np.abs(s) + SILU_SLOPE * EA)
        ds1 = SILU_GRAD_SLOPE * EA + ES * (1.0 + np.abs(a) + EA)
        H = s * g
        DH = ds * (np.abs(g) + EG) + np.abs(s) * EG
        EH = DH + (U + ub) * (np.abs(H) + DH)
        dG = dH * s
        DdG = EdH * (np.abs(s) + ds) + np.abs(dH) * ds
        EdG = DdG + (U + ub) * (np.abs(dG) + DdG)
        dA = dH * g * s1
        DdA = (EdH * (np.abs(g) + EG) * (np.abs(s1) + ds1) + np.abs(dH) * EG * (np.abs(s1) + ds1)
               + np.abs(dH) * np.abs(g) * ds1)
        EdA = DdA + (2 * U + ub) * (np.abs(dA) + DdA)

    def fin(v, pre):
        """Bound of a stored result: the propagated and summation error `pre`, then one rounding."""
        v64 = v.astype(np.float64)
        pre = pre.astype(np.float64)
        return v64, (pre + ub * (np.abs(v64) + pre)) * SLACK

    # dX = dA W1 (+ dG W3)
    du = dA @ W1
    pre = EdA @ aW1
    sq = (dA * dA) @ (W1 * W1)
    if sw:
        du = du + dG @ W3
        pre = pre + EdG @ np.abs(W3)
        sq = sq + (dG * dG) @ (W3 * W3)
    out["du"] = fin(du, pre + acc_factor(f * (2 if sw else 1)) * np.sqrt(sq))
    # dW2 = dY^T H', dW1 = dA'^T u, dW3 = dG'^T u (sums over the rows)
    accn = acc_factor(npad)
    out["dW2"] = fin(dY.T @ H, np.abs(dY).T @ EH + accn * np.sqrt(dY2.T @ (H * H)))
    out["dW1"] = fin(dA.T @ u, EdA.T @ np.abs(u) + accn * np.sqrt((dA * dA).T @ u2))
    if sw:
        out["dW3"] = fin(dG.T @ u, EdG.T @ np.abs(u) + accn * np.sqrt((dG * dG).T @ u2))
    out["db2"] = fin(dY.sum(axis=0), accn * np.sqrt(dY2.sum(axis=0)))
    out["db1"] = fin(dA.sum(axis=0), EdA.sum(axis=0) + accn * np.sqrt((dA * dA).sum(axis=0)))
    return out
