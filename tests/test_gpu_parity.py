"""Parity of the HIP path with the CPU oracle, through the C ABI.

Workloads: the five seeded configurations at full size, plus small ragged
cases (token counts that are not multiples of any tile, expert counts that
are not multiples of 16, widths that leave K and N tails in the GEMMs,
k = 2 and 3, forced drops, the router bias, more than 256 experts, and
capacities that select each row-tile height).
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from oracle import moe as O
from error_bound import check_elementwise, expert_bound
from gpu_util import (AUX_RTOL, Y_TOL, Z_RTOL, check_routing, check_y, device_inputs, host_bits,
                      host_f64, layer_bound, tail_split_parts)

pytestmark = pytest.mark.gpu

FULL = ["tiny", "switch_base", "zipf_skew", "mixtral", "many_expert"]

SMALL = {
    # name: T, d, f, E, k, cf, dtype, act, ffn_bias, router_bias, logit_scale
    "ragged_f32": (333, 24, 40, 5, 1, 1.1, "f32", "relu", True, False, 3.0),
    "ragged_bf16": (1000, 40, 72, 12, 1, 0.9, "bf16", "relu", True, True, 4.0),
    "top2_swiglu": (777, 64, 136, 10, 2, 1.0, "bf16", "swiglu", False, False, 6.0),
    "top3_relu": (517, 32, 96, 7, 3, 0.8, "bf16", "relu", False, False, 5.0),
    "e300_generic": (400, 32, 64, 300, 2, 2.0, "bf16", "relu", False, False, 2.0),
    # 128 < E <= 256: the MFMA router with 128 tokens a block (a ragged last
    # block, a K tail of 8 columns)
    "e200_mfma": (1000, 136, 72, 200, 2, 2.0, "bf16", "relu", False, True, 2.0),
    "f32_swiglu": (150, 16, 24, 6, 2, 1.5, "f32", "swiglu", False, True, 4.0),
    "tiles": (4096, 256, 384, 16, 1, 1.25, "bf16", "relu", True, False, 1.0),
    # experts of at least 512 rows: the 256-row GEMM tiles, with K and N tails
    "big_tiles": (3000, 200, 328, 4, 2, 1.0, "bf16", "relu", True, False, 1.0),
    "big_swiglu": (2048, 136, 200, 2, 1, 1.0, "bf16", "swiglu", False, False, 1.0),
    # at least 256 tiles of 256 x 256 in the second GEMM: the split ring
    # over the whole LDS, with a K tail (f = 264), an N tail (d = 4104) and
    # partly filled row tiles
    "wide_256": (2048, 4104, 264, 8, 2, 1.0, "bf16", "relu", True, False, 1.0),
    # capacity 300 and 170: one 320- or 192-row tile per expert, in the wide
    # column tiles (first GEMM) and the narrow ones (second), with K and N tails
    "tiles_320": (19200, 72, 776, 64, 1, 1.0, "bf16", "relu", True, False, 1.0),
    "tiles_192": (10880, 72, 776, 64, 1, 1.0, "bf16", "relu", True, False, 1.0),
    # capacity 240: row tiles of 128 from the tile map, in the wide column
    # tiles (first GEMM), with K and N tails
    "tiles_128": (12288, 72, 776, 64, 1, 1.25, "bf16", "relu", True, False, 1.0),
    # a last wave of tiles under half the chip, long K: each of those tiles
    # is split along K over several blocks (fused gather and scatter with
    # k = 1, the K tail with d = 1000, ybuf and the combine with k = 2)
    "split_relu": (1200, 1536, 2048, 2, 1, 1.0, "bf16", "relu", True, False, 1.0),
    "split_swiglu": (1100, 1000, 1536, 2, 1, 1.0, "bf16", "swiglu", False, False, 1.0),
    "split_top2": (1000, 1024, 1024, 4, 2, 1.25, "bf16", "relu", False, True, 2.0),
}
SPLIT = ["split_relu", "split_swiglu", "split_top2"]


def _small(name, seed=0):
    T, d, f, E, k, cf, dt, act, fb, rb, sc = SMALL[name]
    return datagen.random_case(seed=seed + 11, T=T, d=d, f=f, E=E, k=k, cf=cf, dtype=dt, act=act,
                               ffn_bias=fb, router_bias=rb, logit_scale=sc)


_CACHE = {}


def _full(name, with_experts=True):
    key = (name, with_experts)
    if key not in _CACHE:
        _CACHE.clear()
        _CACHE[key] = datagen.make(name, seed=0, with_experts=with_experts)
    return _CACHE[key]


def _run_router(cfg):
    t = device_inputs(cfg)
    idx, gate, prob_sum, route_count, zl = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"],
                                                      z_loss=True)
    torch.cuda.synchronize()
    t["z_loss"] = zl
    return t, idx, gate, prob_sum, route_count


def _check_z_loss(z_gpu, z_logits):
    """The router z-loss against the oracle's on the same fp32 logits."""
    ref = O.router_z_loss(z_logits)
    assert abs(float(z_gpu) - ref) <= Z_RTOL * abs(ref), (float(z_gpu), ref)


def _router_checks(cfg, idx, gate, prob_sum, route_count, z_loss=None):
    x64 = O.widen(cfg["x"], cfg["dtype"])
    z = O.router_logits(x64, cfg["W_r"], cfg["b_r"])
    p = O.softmax(z)
    ref_idx = O.top_k(z, cfg["k"])
    ref = dict(z=z, expert_idx=ref_idx, gate=O.gates(z, p, ref_idx))
    gi = idx.cpu().numpy()
    agree = check_routing(gi, gate.cpu().numpy(), ref, cfg["k"])
    E = cfg["E"]
    assert (route_count.cpu().numpy() == O.route_count(gi, E)).all()
    np.testing.assert_allclose(prob_sum.cpu().numpy(), p.sum(axis=0), rtol=2e-6, atol=1e-6)
    if z_loss is not None:
        _check_z_loss(z_loss.cpu()[0], z)
    return z, p, gi, agree


@pytest.mark.parametrize("name", FULL)
def test_router_full(name):
    cfg = _full(name, with_experts=False)
    print(f"router parity: {name} T={cfg['T']} E={cfg['E']} k={cfg['k']}", flush=True)
    t, idx, gate, ps, rc = _run_router(cfg)
    _router_checks(cfg, idx, gate, ps, rc, t["z_loss"])


@pytest.mark.parametrize("name", list(SMALL))
def test_router_small(name):
    cfg = _small(name)
    t, idx, gate, ps, rc = _run_router(cfg)
    _router_checks(cfg, idx, gate, ps, rc, t["z_loss"])


def _dispatch_checks(cfg, t, gi, C):
    idx_t = torch.from_numpy(gi).to(t["x"].device)
    slot, drop, count, xbuf = moe.dispatch(t["x"], idx_t, cfg["E"], C)
    torch.cuda.synchronize()
    rs, rd, rc = O.assign_slots(gi, cfg["E"], C)
    s = slot.cpu().numpy()
    assert (s == rs).all()
    assert (drop.cpu().numpy() == rd).all()
    assert (count.cpu().numpy() == rc).all()
    xb = host_bits(xbuf)
    xh = host_bits(t["x"])
    tt, jj = np.nonzero(s >= 0)
    ee = gi[tt, jj]
    assert (xb[ee, s[tt, jj]] == xh[tt]).all()
    return slot, drop, count, xbuf


@pytest.mark.parametrize("name", FULL)
def test_dispatch_full(name):
    cfg = _full(name, with_experts=False)
    print(f"dispatch parity: {name}", flush=True)
    t, idx, gate, ps, rc = _run_router(cfg)
    z, p, gi, agree = _router_checks(cfg, idx, gate, ps, rc)
    C = O.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    assert moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"]) == C
    _dispatch_checks(cfg, t, gi, C)


@pytest.mark.parametrize("name", list(SMALL))
def test_dispatch_small(name):
    cfg = _small(name)
    t, idx, gate, ps, rc = _run_router(cfg)
    z, p, gi, agree = _router_checks(cfg, idx, gate, ps, rc)
    C = O.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    _dispatch_checks(cfg, t, gi, C)


def _forward_checks(cfg, tokens=None):
    t = device_inputs(cfg)
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], t["x"].dtype,
                           act=cfg["act"], capacity_factor=cfg["cf"], alpha=cfg["alpha"],
                           device=t["x"].device)
    y, aux, idx, gate, drop = plan(t["x"], t["W_r"], t["W1"], t["W2"], W3=t["W3"], b1=t["b1"],
                                   b2=t["b2"], b_r=t["b_r"])
    torch.cuda.synchronize()
    ref = O.forward_cfg(cfg, tokens=tokens)
    gi = idx.cpu().numpy()
    agree = check_routing(gi, gate.cpu().numpy(), ref, cfg["k"])
    # capacity assignment: exact against the oracle's rule on the GPU's own choices
    rs, rd, rc = O.assign_slots(gi, cfg["E"], ref["C"])
    assert (plan.intermediate("slot").cpu().numpy() == rs).all()
    assert (drop.cpu().numpy() == rd).all()
    assert (plan.intermediate("expert_count").cpu().numpy() == rc).all()
    if agree.all():
        assert (rs == ref["slot"]).all() and (rd == ref["drop_mask"]).all()
    # outputs on tokens whose routing and slots agree with the oracle
    same_slots = np.all(rs == ref["slot"], axis=1) & agree
    rows = np.nonzero(same_slots)[0] if tokens is None else np.intersect1d(np.nonzero(same_slots)[0], tokens)
    yg = host_f64(y)
    _, bound = layer_bound(cfg, ref["expert_idx"], ref["slot"], ref["gate"], tokens=tokens)
    err = check_y(yg, ref["y"], rows, cfg["dtype"], bound)
    # the loss: the oracle's definition on the GPU's choices
    aux_ref = O.aux_loss(ref["p"], gi, cfg["E"], cfg["alpha"])
    assert abs(float(aux.cpu()[0]) - aux_ref) <= AUX_RTOL * abs(aux_ref)
    # the router z-loss (independent of the selection)
    _check_z_loss(plan.z_loss.cpu()[0], ref["z"])
    # dropped everywhere -> y == 0
    all_dropped = np.all(rd == 1, axis=1)
    if all_dropped.any():
        assert (yg[all_dropped] == 0).all()
    return err, plan


@pytest.mark.parametrize("name", FULL)
def test_forward_full(name):
    """Full-size workloads, y of every token against the oracle."""
    cfg = _full(name)
    print(f"forward parity: {name} (all tokens)", flush=True)
    err, _ = _forward_checks(cfg)
    print(f"  y max-abs {err[0]:.3e}  mean relative {err[1]:.3e}  largest error/bound {err[2]:.3f}", flush=True)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small(name):
    _forward_checks(_small(name))


@pytest.mark.parametrize("name", ["top2_swiglu"] + SPLIT)
def test_split_api_equals_forward(name):
    """router -> dispatch -> expert_ffn -> combine gives the fused call's outputs bitwise
    (also when the GEMMs split their last wave of tiles)."""
    cfg = _small(name, seed=3)
    t = device_inputs(cfg)
    C = moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    idx, gate, ps, rc, zl = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"], z_loss=True)
    slot, drop, count, xbuf = moe.dispatch(t["x"], idx, cfg["E"], C)
    ybuf = moe.expert_ffn(xbuf, count, t["W1"], t["W2"], W3=t["W3"], act=cfg["act"])
    y, aux = moe.combine(ybuf, idx, slot, gate, ps, rc, cfg["T"], alpha=cfg["alpha"])
    y2, aux2, idx2, gate2, drop2 = moe.forward(t["x"], t["W_r"], t["W1"], t["W2"], W3=t["W3"],
                                               b_r=t["b_r"], k=cfg["k"], capacity_factor=cfg["cf"],
                                               alpha=cfg["alpha"], act=cfg["act"])
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(drop, drop2)
    assert torch.equal(gate.view(torch.int32), gate2.view(torch.int32))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(aux.view(torch.int32), aux2.view(torch.int32))
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], t["x"].dtype,
                           act=cfg["act"], capacity_factor=cfg["cf"], alpha=cfg["alpha"])
    plan(t["x"], t["W_r"], t["W1"], t["W2"], W3=t["W3"], b_r=t["b_r"])
    torch.cuda.synchronize()
    assert torch.equal(zl.view(torch.int32), plan.z_loss.view(torch.int32))


@pytest.mark.parametrize("name", ["switch_base", "top2_swiglu"])
def test_deterministic(name):
    cfg = _full(name) if name in FULL else _small(name)
    t = device_inputs(cfg)
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], t["x"].dtype,
                           act=cfg["act"], capacity_factor=cfg["cf"], alpha=cfg["alpha"])
    outs = []
    for _ in range(2):
        y, aux, idx, gate, drop = plan(t["x"], t["W_r"], t["W1"], t["W2"], W3=t["W3"], b1=t["b1"],
                                       b2=t["b2"], b_r=t["b_r"])
        torch.cuda.synchronize()
        outs.append([host_bits(v).copy() for v in (y, aux, idx, gate, drop)] +
                    [plan.intermediate("slot").cpu().numpy().copy()])
    for a, b in zip(*outs):
        assert (a == b).all()


def _ffn_rows(cfg, per_block=None, seed=7):
    """Expert FFN outputs on the GPU's own dispatch buffer, with their rounding bounds.

    Every kept (expert, row) when `per_block` is None; else `per_block` seeded
    rows of every 32-row block of every expert (the height of one MFMA
    fragment, so every row fragment of every row tile is checked), plus the
    first and last row of each expert.  All columns of a checked row are
    compared, so every column tile and the N tail are covered."""
    t = device_inputs(cfg)
    C = moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    idx, gate, ps, rc, zl = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"], z_loss=True)
    slot, drop, count, xbuf = moe.dispatch(t["x"], idx, cfg["E"], C)
    ybuf = moe.expert_ffn(xbuf, count, t["W1"], t["W2"], W3=t["W3"], b1=t["b1"], b2=t["b2"],
                          act=cfg["act"])
    torch.cuda.synchronize()
    cnt = count.cpu().numpy()
    rng = np.random.default_rng(seed)
    xb = host_f64(xbuf)
    yb = host_f64(ybuf)
    got, ref, bnd = [], [], []
    n = 0
    for e in range(cfg["E"]):
        c = int(cnt[e])
        if c == 0:
            continue
        if per_block is None:
            ms = np.arange(c)
        else:
            pick = [rng.choice(np.arange(b, min(c, b + 32)), size=min(per_block, min(c, b + 32) - b),
                               replace=False) for b in range(0, c, 32)]
            ms = np.unique(np.concatenate(pick + [np.array([0, c - 1])]))
        n += ms.size
        w = lambda a: None if a is None else O.widen(a[e], cfg["dtype"])   # noqa: E731
        ref.append(O.expert_ffn(xb[e, ms], w(cfg["W1"]), w(cfg["W2"]), cfg["act"], b1=w(cfg["b1"]),
                                b2=w(cfg["b2"]), W3=w(cfg["W3"])))
        bnd.append(expert_bound(xb[e, ms], w(cfg["W1"]), w(cfg["W2"]), cfg["act"], b1=w(cfg["b1"]),
                                b2=w(cfg["b2"]), W3=w(cfg["W3"]), store=cfg["dtype"])[1])
        got.append(yb[e, ms])
    return np.concatenate(got), np.concatenate(ref), np.concatenate(bnd), n


@pytest.mark.parametrize("name", ["tiles", "top2_swiglu", "big_tiles", "big_swiglu", "wide_256", "tiles_320",
                                  "tiles_192", "tiles_128", "ragged_f32", "switch_base", "zipf_skew",
                                  "mixtral", "many_expert"] + SPLIT)
def test_expert_ffn_elementwise(name):
    """Each GEMM tile shape against the oracle's expert FFN, every element of the checked rows
    within its rounding bound; the L1 ratio of the layer's tolerance on top."""
    cfg = _full(name) if name in FULL else _small(name)
    got, ref, bnd, n = _ffn_rows(cfg, per_block=None if name not in FULL else 2)
    worst = check_elementwise(got, ref, bnd, what="expert output")
    err = np.abs(got - ref)
    ratio = err.sum() / max(np.abs(ref).sum(), 1e-30)
    print(f"expert FFN parity: {name}, {n} rows, max-abs {err.max():.3e}, L1 ratio {ratio:.3e}, "
          f"largest error/bound {worst:.3f}", flush=True)
    assert ratio <= Y_TOL[cfg["dtype"]][1]


@pytest.mark.parametrize("name", SPLIT)
def test_split_cases_reach_the_split(name):
    """Precondition of the split cases: on the GPU's own expert counts, at least one
    of their two GEMMs splits its last wave (else they would test nothing new)."""
    cfg = _small(name)
    t = device_inputs(cfg)
    C = moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    idx, _, _, _ = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"])
    _, _, count, _ = moe.dispatch(t["x"], idx, cfg["E"], C)
    cnt = count.cpu().numpy()
    d, f, E = cfg["d"], cfg["f"], cfg["E"]
    g1 = tail_split_parts(cnt, C, E, cfg["act"], f, d, gated=cfg["act"] == "swiglu")
    g2 = tail_split_parts(cnt, C, E, cfg["act"], d, f)
    print(f"{name}: counts {cnt.tolist()}, parts per split tile: first GEMM {g1}, second {g2}", flush=True)
    assert max(g1, g2) > 1
