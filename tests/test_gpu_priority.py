"""Priority routing on the GPU (moe_dispatch_priority), through the C ABI.

[CS25-L5], the V-MoE part: the capacity goes to the highest scores first
(ties: lower token index; NaN last), rank-major for k > 1.  Checked bit for
bit against the oracle's assign_slots_priority: slots, drop flags and
expert counts, and every kept row of xbuf against the token's row of x.
Cases cover several list chunks and LDS tiles per expert, rank segments,
equal and non-finite scores, the empty and one-token inputs, and the
largest E; at full size the switch_base routing with the router's first
gate as the score, at its own capacity and at half the even split.
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from oracle import moe as O
from gpu_util import check_routing, check_y, dev, device_inputs, host_bits, host_f64, layer_bound

pytestmark = pytest.mark.gpu


def _check(x_t, idx, pr, E, C):
    """GPU priority dispatch against the oracle; returns the GPU outputs."""
    T = idx.shape[0]
    gi = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    gp = torch.from_numpy(np.ascontiguousarray(pr, dtype=np.float32)).cuda()
    slot, drop, cnt, xbuf = moe.dispatch_priority(x_t, gi, gp, E, C)
    torch.cuda.synchronize()
    rs, rd, rc = O.assign_slots_priority(idx, E, C, pr)
    s = slot.cpu().numpy()
    assert np.array_equal(s, rs), f"{int((s != rs).sum())} slots differ"
    assert np.array_equal(drop.cpu().numpy(), rd)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    if T and C:
        xb = host_bits(xbuf)
        xh = host_bits(x_t)
        tt, jj = np.nonzero(rs >= 0)
        assert np.array_equal(xb[idx[tt, jj], rs[tt, jj]], xh[tt])
    return slot, drop, cnt, xbuf


def _x(T, d, seed=0):
    cfg = datagen.random_case(seed=seed, T=max(T, 1), d=d, f=8, E=2, k=1, cf=1.0, dtype="bf16")
    return dev(cfg["x"][:T], "bf16")


def _idx(rng, T, E, k, skew=0.0):
    z = rng.standard_normal((T, E)) + skew * np.linspace(1, 0, E)[None, :]
    return np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("T,E,k,cf,skew,scores", [
    (1000, 8, 1, 0.5, 0.0, "rand"),          # half the even split
    (1000, 8, 1, 1.25, 2.0, "rand"),         # skewed: one expert overflows
    (3000, 4, 2, 1.0, 0.0, "round"),         # many equal scores, rank segments
    (2000, 6, 3, 0.8, 1.0, "rand"),
    (777, 1024, 8, 1.25, 0.0, "rand"),       # the largest E and k
    (3000, 3, 1, 1.0, 8.0, "rand"),          # most tokens at expert 0: many chunks and tiles
    (500, 5, 2, 1.0, 0.0, "special"),        # NaN, +-inf, +-0 scores
    (300, 7, 2, 1.0, 0.0, "same"),           # one score: the plain token order
    # long segments: the key stream is split over 7 and 8 blocks per entry block
    (12000, 3, 1, 0.8, 8.0, "rand"),
    (20000, 2, 2, 1.0, 0.0, "round"),
])
def test_priority_dispatch_matches_oracle(T, E, k, cf, skew, scores):
    rng = np.random.default_rng(T + E + k)
    idx = _idx(rng, T, E, k, skew)
    pr = rng.random(T).astype(np.float32)
    if scores == "round":
        pr = np.round(pr, 1).astype(np.float32)
    elif scores == "special":
        pr[rng.integers(0, T, 40)] = np.nan
        pr[rng.integers(0, T, 20)] = np.inf
        pr[rng.integers(0, T, 20)] = -np.inf
        pr[rng.integers(0, T, 20)] = 0.0
        pr[rng.integers(0, T, 20)] = -0.0
    elif scores == "same":
        pr[:] = 0.5
    C = O.capacity(T, E, k, cf)
    print(f"priority dispatch: T={T} E={E} k={k} C={C} scores={scores}", flush=True)
    slot, *_ = _check(_x(T, 64), idx, pr, E, C)
    if scores == "same":
        rs, _, _ = O.assign_slots(idx, E, C)
        assert np.array_equal(slot.cpu().numpy(), rs)


@pytest.mark.parametrize("T,C", [(0, 0), (1, 1), (1, 0), (64, 0)])
def test_priority_dispatch_degenerate(T, C):
    rng = np.random.default_rng(5)
    idx = _idx(rng, T, 4, 2)
    pr = rng.random(T).astype(np.float32)
    print(f"priority dispatch degenerate: T={T} C={C}", flush=True)
    _check(_x(T, 32), idx, pr, 4, C)


@pytest.mark.parametrize("cf", [1.25, 0.5])
def test_priority_dispatch_switch_base(cf):
    """Full size: the GPU router's choices, its first gate as the score."""
    cfg = datagen.make("switch_base", seed=0, with_experts=False)
    t = device_inputs(cfg)
    idx, gate, _, _ = moe.router(t["x"], t["W_r"], k=1)
    torch.cuda.synchronize()
    C = O.capacity(cfg["T"], cfg["E"], 1, cf)
    print(f"priority dispatch: switch_base cf={cf} C={C}", flush=True)
    pr = gate[:, 0].contiguous().cpu().numpy()
    _, drop, cnt, _ = _check(t["x"], idx.cpu().numpy(), pr, cfg["E"], C)
    # the kept tokens' scores are never below a dropped token's at the same expert
    gi = idx.cpu().numpy()[:, 0]
    d = drop.cpu().numpy()[:, 0].astype(bool)
    for e in range(cfg["E"]):
        kept, lost = pr[(gi == e) & ~d], pr[(gi == e) & d]
        if kept.size and lost.size:
            assert kept.min() >= lost.max()


def test_priority_layer_end_to_end():
    """router -> priority dispatch (first gate as the score) -> expert FFN ->
    combine at half the even split: every token's y against the oracle's
    experts on the kept choices."""
    cfg = datagen.random_case(seed=61, T=700, d=48, f=64, E=6, k=2, cf=0.5, dtype="bf16", logit_scale=2.0)
    t = device_inputs(cfg)
    idx, gate, ps, rc = moe.router(t["x"], t["W_r"], k=2)
    C = moe.capacity(cfg["T"], cfg["E"], 2, cfg["cf"])
    slot, drop, cnt, xbuf = moe.dispatch_priority(t["x"], idx, gate[:, 0].contiguous(), cfg["E"], C)
    ybuf = moe.expert_ffn(xbuf, cnt, t["W1"], t["W2"], act="relu")
    y, aux = moe.combine(ybuf, idx, slot, gate, ps, rc, cfg["T"], alpha=cfg["alpha"])
    torch.cuda.synchronize()
    x64 = O.widen(cfg["x"], "bf16")
    z = O.router_logits(x64, cfg["W_r"])
    ref_idx = O.top_k(z, 2)
    check_routing(idx.cpu().numpy(), gate.cpu().numpy(), dict(z=z, expert_idx=ref_idx,
                                                              gate=O.gates(z, O.softmax(z), ref_idx)), 2)
    gi = idx.cpu().numpy()
    g = gate.cpu().numpy()
    rs, rd, _ = O.assign_slots_priority(gi, cfg["E"], C, g[:, 0])
    assert np.array_equal(slot.cpu().numpy(), rs) and np.array_equal(drop.cpu().numpy(), rd)
    ref = np.zeros((cfg["T"], cfg["d"]))
    for e in range(cfg["E"]):
        tt, jj = np.nonzero((gi == e) & (rd == 0))
        if tt.size:
            o = O.expert_ffn(x64[tt], O.widen(cfg["W1"][e], "bf16"), O.widen(cfg["W2"][e], "bf16"), "relu")
            ref[tt] += g[tt, jj].astype(np.float64)[:, None] * o
    _, bound = layer_bound(cfg, gi, rs, g)
    check_y(host_f64(y), ref, np.arange(cfg["T"]), "bf16", bound)
