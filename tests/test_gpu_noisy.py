"""The noisy top-k router on the GPU (moe_router_noisy), through the C ABI.

Logits H = W_r x (+ b_r) + eps * softplus(W_noise x) with the standard normal
draws eps given as an input ([CMU-L16] section 2.3).  Checked against the
oracle's noisy_router_logits by the same bars as the clean router (indices
bit-exact outside near ties of H, gates, totals, z-loss), plus:
  * the page's zero initialisation: W_r = W_noise = 0 routes every token to
    the expert of its largest draw (its k largest for top-k);
  * the noisy choices feed dispatch, the expert FFN and combine unchanged.
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from oracle import moe as O
from gpu_util import Z_RTOL, check_routing, check_y, dev, device_inputs, host_f64, layer_bound

pytestmark = pytest.mark.gpu

CASES = {
    # name: T, d, E, k, dtype, router_bias.  bf16 with E <= 128 takes the
    # MFMA router on the stacked weight, in halves of 32, 64 or 128 rows
    # (with and without a K tail); E <= 256 the MFMA router in two K passes;
    # fp32 and E > 256 the fp32 FMA router
    "bf16_k1": (1000, 40, 12, 1, "bf16", True),
    "bf16_k2": (777, 64, 10, 2, "bf16", False),
    "e33_k3": (450, 200, 33, 3, "bf16", True),
    "e80_k2": (700, 96, 80, 2, "bf16", False),
    "e128_tail": (333, 72, 128, 1, "bf16", True),
    "e129_k2": (600, 64, 129, 2, "bf16", True),
    "e256_tail": (421, 104, 256, 1, "bf16", False),
    "e200_k3_short": (300, 32, 200, 3, "bf16", True),
    "f32_k3": (517, 32, 7, 3, "f32", False),
    "e300": (400, 32, 300, 2, "bf16", False),
}


def _noise_inputs(cfg, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    E, d, T = cfg["E"], cfg["d"], cfg["T"]
    W_n = (rng.standard_normal((E, d)) * np.sqrt(0.1 / d) * scale).astype(np.float32)
    eps = rng.standard_normal((T, E)).astype(np.float32)
    return W_n, eps


def _run(cfg, W_n, eps):
    t = device_inputs(cfg)
    idx, gate, ps, rc, zl = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"], z_loss=True,
                                       W_noise=dev(W_n, "f32"), noise=dev(eps, "f32"))
    torch.cuda.synchronize()
    return t, idx, gate, ps, rc, zl


def _checks(cfg, W_n, eps, idx, gate, ps, rc, zl):
    x64 = O.widen(cfg["x"], cfg["dtype"])
    H = O.noisy_router_logits(x64, cfg["W_r"], cfg["b_r"], W_n, eps)
    p = O.softmax(H)
    ref_idx = O.top_k(H, cfg["k"])
    gi = idx.cpu().numpy()
    agree = check_routing(gi, gate.cpu().numpy(), dict(z=H, expert_idx=ref_idx, gate=O.gates(H, p, ref_idx)),
                          cfg["k"])
    assert (rc.cpu().numpy() == O.route_count(gi, cfg["E"])).all()
    np.testing.assert_allclose(ps.cpu().numpy(), p.sum(axis=0), rtol=2e-6, atol=1e-6)
    ref_z = O.router_z_loss(H)
    assert abs(float(zl.cpu()[0]) - ref_z) <= Z_RTOL * abs(ref_z)
    return gi, agree


@pytest.mark.parametrize("name", list(CASES))
def test_noisy_router_small(name):
    T, d, E, k, dt, rb = CASES[name]
    cfg = datagen.random_case(seed=31, T=T, d=d, f=8, E=E, k=k, cf=1.25, dtype=dt, router_bias=rb,
                              logit_scale=3.0)
    W_n, eps = _noise_inputs(cfg, 7, scale=3.0)
    print(f"noisy router: {name}", flush=True)
    _checks(cfg, W_n, eps, *_run(cfg, W_n, eps)[1:])


def test_noisy_router_switch_base():
    cfg = datagen.make("switch_base", seed=0, with_experts=False)
    W_n, eps = _noise_inputs(cfg, 11)
    print("noisy router: switch_base", flush=True)
    _checks(cfg, W_n, eps, *_run(cfg, W_n, eps)[1:])


@pytest.mark.parametrize("k", [1, 2])
def test_zero_init_routes_by_the_noise(k):
    cfg = datagen.random_case(seed=41, T=3000, d=32, f=8, E=8, k=k, cf=1.25, dtype="bf16")
    cfg["W_r"] = np.zeros_like(cfg["W_r"])
    W_n, eps = _noise_inputs(cfg, 13)
    W_n = np.zeros_like(W_n)
    print(f"noisy router, zero initialisation, k={k}", flush=True)
    t, idx, gate, ps, rc, zl = _run(cfg, W_n, eps)
    want = np.argsort(-eps, axis=1, kind="stable")[:, :k]
    assert (idx.cpu().numpy() == want).all()
    load = np.bincount(want.reshape(-1), minlength=8) / want.size
    assert np.all(np.abs(load - 1 / 8) < 0.02)


def test_noisy_router_feeds_the_layer():
    """noisy router -> dispatch -> expert_ffn -> combine: y of every token against
    the oracle's experts on the GPU's own choices and gates."""
    cfg = datagen.random_case(seed=51, T=600, d=48, f=72, E=6, k=2, cf=1.0, dtype="bf16",
                              logit_scale=2.0)
    W_n, eps = _noise_inputs(cfg, 17, scale=2.0)
    t, idx, gate, ps, rc, zl = _run(cfg, W_n, eps)
    gi, _ = _checks(cfg, W_n, eps, idx, gate, ps, rc, zl)
    C = moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    slot, drop, count, xbuf = moe.dispatch(t["x"], idx, cfg["E"], C)
    ybuf = moe.expert_ffn(xbuf, count, t["W1"], t["W2"], act=cfg["act"])
    y, aux = moe.combine(ybuf, idx, slot, gate, ps, rc, cfg["T"], alpha=cfg["alpha"])
    torch.cuda.synchronize()
    rs, rd, rc2 = O.assign_slots(gi, cfg["E"], C)
    assert (slot.cpu().numpy() == rs).all() and (drop.cpu().numpy() == rd).all()
    x64 = O.widen(cfg["x"], "bf16")
    g = gate.cpu().numpy().astype(np.float64)
    ref = np.zeros((cfg["T"], cfg["d"]))
    for e in range(cfg["E"]):
        tt, jj = np.nonzero((gi == e) & (rd == 0))
        if tt.size:
            o = O.expert_ffn(x64[tt], O.widen(cfg["W1"][e], "bf16"), O.widen(cfg["W2"][e], "bf16"), cfg["act"])
            ref[tt] += g[tt, jj][:, None] * o
    _, bound = layer_bound(cfg, gi, rs, g)
    check_y(host_f64(y), ref, np.arange(cfg["T"]), "bf16", bound)


@pytest.mark.parametrize("k,dt", [(1, "bf16"), (2, "bf16"), (1, "f32")])
def test_fused_forward_with_noise(k, dt):
    """moe_forward_noisy: the fused layer on the noisy logits; routing, totals
    and z-loss against the oracle's noisy logits, then slots, aux and every
    token's y against the oracle's experts on the GPU's choices and gates."""
    cfg = datagen.random_case(seed=91, T=700, d=64, f=96, E=8, k=k, cf=1.0, dtype=dt, logit_scale=2.0)
    W_n, eps = _noise_inputs(cfg, 19, scale=2.0)
    t = device_inputs(cfg)
    print(f"fused forward with noise: k={k} {dt}", flush=True)
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], k, t["x"].dtype, act=cfg["act"],
                           capacity_factor=cfg["cf"], alpha=cfg["alpha"], device=t["x"].device)
    y, aux, idx, gate, drop = plan(t["x"], t["W_r"], t["W1"], t["W2"], W_noise=dev(W_n, "f32"),
                                   noise=dev(eps, "f32"))
    torch.cuda.synchronize()
    gi, _ = _checks(cfg, W_n, eps, idx, gate, plan.intermediate("prob_sum"), plan.intermediate("route_count"),
                    plan.z_loss)
    C = moe.capacity(cfg["T"], cfg["E"], k, cfg["cf"])
    rs, rd, _ = O.assign_slots(gi, cfg["E"], C)
    assert np.array_equal(drop.cpu().numpy(), rd)
    x64 = O.widen(cfg["x"], dt)
    H = O.noisy_router_logits(x64, cfg["W_r"], cfg["b_r"], W_n, eps)
    ref_aux = O.aux_loss(O.softmax(H), gi, cfg["E"], cfg["alpha"])
    assert abs(float(aux.cpu()[0]) - ref_aux) <= 1e-5 * abs(ref_aux)
    g = gate.cpu().numpy().astype(np.float64)
    ref = np.zeros((cfg["T"], cfg["d"]))
    for e in range(cfg["E"]):
        tt, jj = np.nonzero((gi == e) & (rd == 0))
        if tt.size:
            o = O.expert_ffn(x64[tt], O.widen(cfg["W1"][e], dt), O.widen(cfg["W2"][e], dt), cfg["act"])
            ref[tt] += g[tt, jj][:, None] * o
    _, bound = layer_bound(cfg, gi, rs, g)
    check_y(host_f64(y), ref, np.arange(cfg["T"]), dt, bound)
