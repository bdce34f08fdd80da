"""The per-element error bound of the GPU parity tests, checked on the CPU.

A plain NumPy simulation of the HIP path's arithmetic (fp32 sums, H and the
expert outputs rounded to bf16, the gate product summed in fp32 and rounded
to bf16) must stay inside the bound; the same outputs with one 32 x 32 block
corrupted the way a kernel bug would (a zeroed tile, a neighbouring column
tile, a transposed fragment, rows shifted by one token, a wrong last column)
must fail it.  The norms of the layer's tolerance alone let such blocks pass.
"""
import numpy as np
import pytest

import datagen
from error_bound import check_elementwise, layer_bound
from oracle import moe as O


def _bf16(a32):
    return datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(np.asarray(a32, dtype=np.float32)))


def _simulate(cfg, idx, slot, gate):
    """The kernels' rounding steps in NumPy: fp32 products, bf16 H / outputs / y."""
    dt = cfg["dtype"]
    w = lambda a: None if a is None else O.widen(a, dt).astype(np.float32)   # noqa: E731
    x = w(cfg["x"])
    rnd = _bf16 if dt == "bf16" else (lambda v: np.asarray(v, dtype=np.float32))
    T, k = idx.shape
    acc = np.zeros((T, x.shape[1]), dtype=np.float32)
    for e in np.unique(idx):
        tt, jj = np.nonzero((idx == e) & (slot >= 0))
        if tt.size == 0:
            continue
        u = x[tt]
        a = u @ w(cfg["W1"][e]).T
        if cfg["b1"] is not None:
            a = a + w(cfg["b1"][e])[None, :]
        if cfg["act"] == "relu":
            h = rnd(np.maximum(a, np.float32(0)))
        else:
            g = u @ w(cfg["W3"][e]).T
            h = rnd((a / (np.float32(1) + np.exp(-a))) * g)
        o = h @ w(cfg["W2"][e]).T
        if cfg["b2"] is not None:
            o = o + w(cfg["b2"][e])[None, :]
        o = rnd(o)
        acc[tt] += np.asarray(gate[tt, jj], np.float32)[:, None] * o
    return rnd(acc).astype(np.float64)


CASES = {
    "relu_k1_bias": dict(T=640, d=96, f=160, E=6, k=1, cf=1.0, dtype="bf16", act="relu", ffn_bias=True),
    "swiglu_k2": dict(T=512, d=64, f=136, E=5, k=2, cf=1.25, dtype="bf16", act="swiglu"),
    "f32_relu": dict(T=300, d=32, f=48, E=4, k=1, cf=1.25, dtype="f32", act="relu", ffn_bias=True),
}


def _setup(name):
    p = dict(CASES[name])
    cfg = datagen.random_case(seed=5, logit_scale=3.0, **p)
    ref = O.forward_cfg(cfg)
    idx, slot, gate = ref["expert_idx"], ref["slot"], ref["gate"]
    y_sim = _simulate(cfg, idx, slot, gate)
    _, Ey = layer_bound(cfg, idx, slot, gate)
    return cfg, ref, y_sim, Ey


@pytest.mark.parametrize("name", list(CASES))
def test_simulated_kernel_arithmetic_is_inside_the_bound(name):
    cfg, ref, y_sim, Ey = _setup(name)
    worst = check_elementwise(y_sim, ref["y"], Ey)
    assert 0.0 < worst <= 1.0
    # the bound is not vacuous: a typical element's bound is a small part of its value
    kept = np.abs(ref["y"]) > 0
    assert np.median(Ey[kept] / np.abs(ref["y"][kept])) < (0.25 if cfg["dtype"] == "bf16" else 1e-3)


def _kept_block(ref, Ey, T, d):
    """Token rows r0..r0+31 (all kept) and columns c0..c0+31, not at the edges."""
    kept = np.all(ref["drop_mask"] == 0, axis=1)
    for r0 in range(32, T - 64):
        if kept[r0:r0 + 33].all():
            return r0, 32 if d >= 96 else 0
    raise AssertionError("no block of kept tokens")


def _corrupt(y, r0, c0, how):
    y = y.copy()
    blk = (slice(r0, r0 + 32), slice(c0, c0 + 32))
    if how == "zero":
        y[blk] = 0.0
    elif how == "next_column_tile":
        y[blk] = y[r0:r0 + 32, c0 + 32:c0 + 64] if y.shape[1] >= c0 + 64 else y[r0:r0 + 32, c0 - 32:c0]
    elif how == "transposed":
        y[blk] = y[blk].T.copy()
    elif how == "rows_shifted":
        y[blk] = y[r0 + 1:r0 + 33, c0:c0 + 32]
    elif how == "last_column":
        y[r0:r0 + 32, -1] = y[r0:r0 + 32, -2]
    return y


@pytest.mark.parametrize("name", ["relu_k1_bias", "swiglu_k2"])
@pytest.mark.parametrize("how", ["zero", "next_column_tile", "transposed", "rows_shifted", "last_column"])
def test_corrupted_block_fails_the_bound(name, how):
    cfg, ref, y_sim, Ey = _setup(name)
    r0, c0 = _kept_block(ref, Ey, cfg["T"], cfg["d"])
    bad = _corrupt(y_sim, r0, c0, how)
    with pytest.raises(AssertionError):
        check_elementwise(bad, ref["y"], Ey)


_BIG = {}


def _big():
    """A wider layer with 64 experts, where y is small (about 1e-3), as at full size."""
    if not _BIG:
        big = datagen.random_case(seed=6, T=4096, d=384, f=768, E=64, k=1, cf=1.25, dtype="bf16", act="relu")
        ref = O.forward_cfg(big)
        y = _simulate(big, ref["expert_idx"], ref["slot"], ref["gate"])
        _, Ey = layer_bound(big, ref["expert_idx"], ref["slot"], ref["gate"])
        _BIG.update(cfg=big, ref=ref, y=y, Ey=Ey)
    return _BIG


@pytest.mark.parametrize("how", ["zero", "next_column_tile", "transposed", "rows_shifted"])
def test_norm_tolerance_alone_misses_a_corrupted_block(how):
    """Why the element bound is needed: the corrupted block still meets max-abs 2e-2 and the
    L1 ratio 5e-3, and only the element bound rejects it."""
    b = _big()
    r0, c0 = _kept_block(b["ref"], None, b["cfg"]["T"], b["cfg"]["d"])
    bad = _corrupt(b["y"], r0, c0, how)
    err = np.abs(bad - b["ref"]["y"])
    assert err.max() <= 2e-2 and err.sum() / np.abs(b["ref"]["y"]).sum() <= 5e-3
    check_elementwise(b["y"], b["ref"]["y"], b["Ey"])
    with pytest.raises(AssertionError):
        check_elementwise(bad, b["ref"]["y"], b["Ey"])


def test_dropped_tokens_have_a_zero_bound():
    cfg, ref, y_sim, Ey = _setup("relu_k1_bias")
    gone = np.all(ref["drop_mask"] == 1, axis=1)
    assert gone.any()
    assert (Ey[gone] == 0).all() and (y_sim[gone] == 0).all()


# ---------------------------------------------------------------------------
# the expert backward's bound
# ---------------------------------------------------------------------------

def _simulate_expert_backward(u, W1, W2, act, dY, b1=None, W3=None, store="bf16"):
    """The backward kernels' rounding steps in NumPy: fp32 products, A', G', dH', H', dA', dG'
    and the outputs rounded to the storage type."""
    rnd = _bf16 if store == "bf16" else (lambda v: np.asarray(v, dtype=np.float32))
    f32 = lambda a: None if a is None else np.asarray(a, dtype=np.float32)   # noqa: E731
    u, W1, W2, W3, b1, dY = (f32(v) for v in (u, W1, W2, W3, b1, dY))
    a = rnd(u @ W1.T + (0 if b1 is None else b1[None, :]))
    dH = rnd(dY @ W2)
    out = {}
    if act == "relu":
        H = rnd(np.maximum(a, 0))
        dA = rnd(dH * (a > 0))
        du = rnd(dA @ W1)
    else:
        g = rnd(u @ W3.T)
        sg = 1 / (1 + np.exp(-a))
        s = a * sg
        H = rnd(s * g)
        dA = rnd(dH * g * (sg * (1 + a * (1 - sg))))
        dG = rnd(dH * s)
        du = rnd(dA @ W1 + dG @ W3)
        out["dW3"] = rnd(dG.T @ u)
    out.update(du=du, dW2=rnd(dY.T @ H), dW1=rnd(dA.T @ u), db2=rnd(dY.sum(0)), db1=rnd(dA.sum(0)))
    return {k: v.astype(np.float64) for k, v in out.items()}


def _bwd_case(act, store="bf16", seed=2, n=300, d=64, f=96):
    rng = np.random.default_rng(seed)
    cast = (lambda a: _bf16(a).astype(np.float64)) if store == "bf16" else (lambda a: a.astype(np.float32).astype(np.float64))
    c = dict(u=cast(rng.normal(size=(n, d))), W1=cast(rng.normal(size=(f, d)) * 0.04),
             W2=cast(rng.normal(size=(d, f)) * 0.03), dY=cast(rng.normal(size=(n, d)) * 0.01),
             W3=cast(rng.normal(size=(f, d)) * 0.04) if act == "swiglu" else None,
             b1=cast(rng.normal(size=f) * 0.04) if act == "relu" else None)
    return c


@pytest.mark.parametrize("act,store", [("relu", "bf16"), ("swiglu", "bf16"), ("relu", "f32"), ("swiglu", "f32")])
def test_simulated_backward_is_inside_the_bound(act, store):
    from error_bound import expert_backward_bound
    c = _bwd_case(act, store)
    ref = O.expert_ffn_backward(c["u"], c["W1"], c["W2"], act, c["dY"], b1=c["b1"], W3=c["W3"])
    sim = _simulate_expert_backward(c["u"], c["W1"], c["W2"], act, c["dY"], b1=c["b1"], W3=c["W3"], store=store)
    bnd = expert_backward_bound(c["u"], c["W1"], c["W2"], act, c["dY"], b1=c["b1"], W3=c["W3"], store=store)
    for name, (_, E) in bnd.items():
        w = check_elementwise(sim[name], ref[name], E, what=name)
        assert w <= 1.0


@pytest.mark.parametrize("name,how", [("dW1", "transposed"), ("dW2", "zero"), ("du", "rows_shifted"),
                                      ("dW3", "next_column_tile")])
def test_corrupted_backward_block_fails_the_bound(name, how):
    from error_bound import expert_backward_bound
    c = _bwd_case("swiglu")
    ref = O.expert_ffn_backward(c["u"], c["W1"], c["W2"], "swiglu", c["dY"], W3=c["W3"])
    sim = _simulate_expert_backward(c["u"], c["W1"], c["W2"], "swiglu", c["dY"], W3=c["W3"])
    bnd = expert_backward_bound(c["u"], c["W1"], c["W2"], "swiglu", c["dY"], W3=c["W3"])
    bad = _corrupt(sim[name], 32, 0, how)
    with pytest.raises(AssertionError):
        check_elementwise(bad, ref[name], bnd[name][1], what=name)
