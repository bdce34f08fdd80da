"""The fused layer with an overflow policy (moe_forward_policy), through the C ABI.

Priority routing and re-routing inside one call: the router's choices and
gates against the oracle's (near-tie rule), the capacity slots bit for bit
against the oracle's assign_slots_priority / assign_slots_reroute on the
GPU's own choices and scores, the loss against the oracle's definition on
those choices (re-routing: first choices), and y of every token against the
oracle's experts within the rounding bound.
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from gpu_util import AUX_RTOL, Z_RTOL, check_routing, check_y, device_inputs, host_f64, layer_bound
from oracle import moe as O

pytestmark = pytest.mark.gpu


def _run(cfg, policy, priority=None, stages=2):
    t = device_inputs(cfg)
    k = 1 if policy == "reroute" else cfg["k"]
    out = moe.forward_policy(t["x"], t["W_r"], t["W1"], t["W2"], policy=policy, W3=t["W3"], b1=t["b1"],
                             b2=t["b2"], b_r=t["b_r"], k=k, capacity_factor=cfg["cf"], alpha=cfg["alpha"],
                             act=cfg["act"], priority=priority, stages=stages)
    torch.cuda.synchronize()
    return out


def _router_ref(cfg, kk):
    x64 = O.widen(cfg["x"], cfg["dtype"])
    z = O.router_logits(x64, cfg["W_r"], cfg["b_r"])
    p = O.softmax(z)
    idx = O.top_k(z, kk)
    return z, p, dict(z=z, expert_idx=idx, gate=O.gates(z, p, idx))


def _y_checks(cfg, y, gi, slot, g):
    T = cfg["T"]
    x64 = O.widen(cfg["x"], cfg["dtype"])
    ref = np.zeros((T, cfg["d"]))
    for e in range(cfg["E"]):
        tt, jj = np.nonzero((gi == e) & (slot >= 0))
        if tt.size:
            w = lambda a: None if a is None else O.widen(a[e], cfg["dtype"])   # noqa: E731
            o = O.expert_ffn(x64[tt], w(cfg["W1"]), w(cfg["W2"]), cfg["act"], b1=w(cfg["b1"]), b2=w(cfg["b2"]),
                             W3=w(cfg["W3"]))
            ref[tt] += np.asarray(g, np.float64)[tt, jj][:, None] * o
    _, bound = layer_bound(cfg, gi, slot, g)
    return check_y(host_f64(y), ref, np.arange(T), cfg["dtype"], bound)


CASES = {
    # name: T, d, f, E, k, cf, dtype, act, bias
    "k1_half": (900, 64, 96, 6, 1, 0.5, "bf16", "relu", False),
    "k2_swiglu": (700, 64, 136, 5, 2, 0.6, "bf16", "swiglu", False),
    "f32_bias": (400, 32, 48, 4, 1, 0.7, "f32", "relu", True),
}


def _case(name, seed=41):
    T, d, f, E, k, cf, dt, act, bias = CASES[name]
    return datagen.random_case(seed=seed, T=T, d=d, f=f, E=E, k=k, cf=cf, dtype=dt, act=act, ffn_bias=bias,
                               logit_scale=3.0)


def _check_priority(cfg, priority=None):
    y, aux, zl, idx, gate, drop = _run(cfg, "priority", priority=priority)
    k = cfg["k"]
    z, p, ref = _router_ref(cfg, k)
    gi, g = idx.cpu().numpy(), gate.cpu().numpy()
    agree = check_routing(gi, g, ref, k)
    C = O.capacity(cfg["T"], cfg["E"], k, cfg["cf"])
    score = g[:, 0] if priority is None else priority.cpu().numpy()
    rs, rd, _ = O.assign_slots_priority(gi, cfg["E"], C, score)
    assert np.array_equal(drop.cpu().numpy(), rd)
    assert bool(rd.any()), "the case should drop some choices"
    aux_ref = O.aux_loss(p, gi, cfg["E"], cfg["alpha"])
    assert abs(float(aux.cpu()[0]) - aux_ref) <= AUX_RTOL * abs(aux_ref)
    zr = O.router_z_loss(z)
    assert abs(float(zl.cpu()[0]) - zr) <= Z_RTOL * abs(zr)
    _y_checks(cfg, y, gi, rs, g)
    return agree


@pytest.mark.parametrize("name", list(CASES))
def test_priority_forward(name):
    print(f"priority forward: {name}", flush=True)
    _check_priority(_case(name))


def test_priority_forward_given_scores():
    cfg = _case("k2_swiglu")
    rng = np.random.default_rng(3)
    pr = torch.from_numpy(rng.standard_normal(cfg["T"]).astype(np.float32)).cuda()
    _check_priority(cfg, priority=pr)


def _check_reroute(cfg, stages):
    y, aux, zl, idx, gate, drop = _run(cfg, "reroute", stages=stages)
    z, p, ref = _router_ref(cfg, stages)
    # the preferences are the router's top-`stages`; re-derive them with the
    # GPU's own router to compare the placement bit for bit
    t = device_inputs(cfg)
    pref_t, pg, _, _ = moe.router(t["x"], t["W_r"], k=stages, b_r=t["b_r"])
    torch.cuda.synchronize()
    pref = pref_t.cpu().numpy()
    check_routing(pref, pg.cpu().numpy(), ref, stages)
    C = O.capacity(cfg["T"], cfg["E"], 1, cfg["cf"])
    rex, rsl, rst, _ = O.assign_slots_reroute(pref, cfg["E"], C, stages)
    gi = idx.cpu().numpy()[:, 0]
    assert np.array_equal(gi, rex)
    assert np.array_equal(drop.cpu().numpy()[:, 0], (rex < 0).astype(np.uint8))
    assert bool(np.any((rex >= 0) & (rex != pref[:, 0]))), "some tokens should be re-routed"
    g = gate.cpu().numpy()
    gref = np.where(rex >= 0, p[np.arange(cfg["T"]), np.maximum(rex, 0)], 0.0)
    np.testing.assert_allclose(g[:, 0], gref, rtol=1e-5, atol=1e-7)
    aux_ref = O.aux_loss(p, pref[:, :1], cfg["E"], cfg["alpha"])
    assert abs(float(aux.cpu()[0]) - aux_ref) <= AUX_RTOL * abs(aux_ref)
    _y_checks(cfg, y, rex[:, None], rsl[:, None], g)


@pytest.mark.parametrize("name,stages", [("k1_half", 3), ("f32_bias", 2)])
def test_reroute_forward(name, stages):
    """At capacity factor 1 the popular experts overflow while others keep room, so some
    tokens land on a later choice (below 1 every expert fills in stage 0)."""
    print(f"re-routing forward: {name} stages={stages}", flush=True)
    cfg = _case(name)
    cfg["cf"] = 1.0
    _check_reroute(cfg, stages)


def test_policies_at_switch_base_size():
    cfg = datagen.make("switch_base", seed=0)
    cfg["cf"] = 0.8
    print("priority and re-routing forward: switch_base, capacity factor 0.8 and 1.0", flush=True)
    _check_priority(cfg)
    cfg["cf"] = 1.0
    _check_reroute(cfg, 4)
