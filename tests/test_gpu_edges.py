"""Degenerate and extreme cases of the method on the GPU, through the C ABI.

Each case has a result fixed by the method's definition, checked directly,
on top of the usual parity with the oracle:
  * all logits tied (W_r = 0): every token takes experts 0 .. k-1 (the lower
    index wins ties), so the capacity rule keeps exactly the first C tokens of
    each rank, aux / alpha = 1 (P_i = 1/E for every i), and the router
    z-loss is (ln E)^2;
  * the fp32 router: logits 4.00 and 4.01, which bf16 rounding would tie,
    route to expert 1;
  * one token, one expert, k = E, a capacity of one row, the largest E and
    k the boundary accepts;
  * tokens holding NaN or infinities: indices stay in [0, E) and distinct,
    slots follow the capacity rule, and every finite token's routing and
    output still match the oracle.
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from oracle import moe as O
from gpu_util import check_routing, check_y, device_inputs, host_f64, layer_bound
from test_gpu_parity import _forward_checks

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(seed=101, T=256, d=32, f=64, E=8, k=1, cf=1.25, dtype="bf16", act="relu",
                ffn_bias=False, router_bias=False, logit_scale=2.0)
    base.update(kw)
    return datagen.random_case(**base)


def _run(cfg):
    t = device_inputs(cfg)
    plan = moe.ForwardPlan(cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["k"], t["x"].dtype,
                           act=cfg["act"], capacity_factor=cfg["cf"], alpha=cfg["alpha"],
                           device=t["x"].device)
    y, aux, idx, gate, drop = plan(t["x"], t["W_r"], t["W1"], t["W2"], W3=t["W3"], b1=t["b1"],
                                   b2=t["b2"], b_r=t["b_r"])
    torch.cuda.synchronize()
    return y, aux, idx, gate, drop, plan


@pytest.mark.parametrize("k", [1, 2, 3])
def test_all_ties_take_the_lowest_indices(k):
    cfg = _case(T=300, E=6, k=k, cf=1.0)
    cfg["W_r"] = np.zeros_like(cfg["W_r"])
    T, E = cfg["T"], cfg["E"]
    print(f"all-tie routing: T={T} E={E} k={k}", flush=True)
    y, aux, idx, gate, drop, plan = _run(cfg)
    gi = idx.cpu().numpy()
    assert (gi == np.arange(k)[None, :]).all()
    # k = 1: the full-softmax probability 1/E; k >= 2: renormalised over k
    want = 1.0 / E if k == 1 else 1.0 / k
    np.testing.assert_allclose(gate.cpu().numpy(), want, rtol=1e-6)
    # rank j of every token goes to expert j: the first C tokens keep a slot
    C = O.capacity(T, E, k, cfg["cf"])
    slot = plan.intermediate("slot").cpu().numpy()
    ar = np.arange(T)
    for j in range(k):
        assert (slot[:, j] == np.where(ar < C, ar, -1)).all()
    assert abs(float(aux.cpu()[0]) / cfg["alpha"] - 1.0) <= 1e-5
    # every log-sum-exp is ln E: the z-loss is (ln E)^2
    assert abs(float(plan.z_loss.cpu()[0]) - np.log(E) ** 2) <= 1e-6 * np.log(E) ** 2
    _forward_checks(cfg)


def test_fp32_router_separates_what_bf16_would_tie():
    T, d, E = 64, 8, 2
    cfg = _case(T=T, d=d, f=16, E=E, k=1, cf=2.0)
    x = np.zeros((T, d), dtype=np.float32)
    x[:, 0] = 1.0
    cfg["x"] = datagen.f32_to_bf16_bits(x)
    W_r = np.zeros((E, d), dtype=np.float32)
    W_r[0, 0], W_r[1, 0] = 4.00, 4.01
    cfg["W_r"] = W_r
    print("fp32 router pin: logits 4.00 / 4.01", flush=True)
    _, _, idx, _, _, _ = _run(cfg)
    assert (idx.cpu().numpy() == 1).all()
    _forward_checks(cfg)


@pytest.mark.parametrize("shape", [
    dict(T=1, E=4, k=2, d=16, f=24),                  # one token
    dict(T=200, E=1, k=1),                            # one expert: every token, C = T
    dict(T=300, E=4, k=4, cf=1.0),                    # k = E: every token at every expert
    dict(T=500, E=4, k=1, cf=0.008),                  # capacity of one row per expert
    dict(T=600, E=1024, k=8, d=32, f=32, cf=1.25),    # the largest E and k
    dict(T=70, E=1024, k=1, d=16, f=16, cf=1.0),      # more experts than tokens
], ids=["T1", "E1", "k_eq_E", "C1", "E1024_k8", "E_gt_T"])
def test_degenerate_shapes(shape):
    cfg = _case(**shape)
    print(f"degenerate shape: {shape}", flush=True)
    err, plan = _forward_checks(cfg)
    cnt = plan.intermediate("expert_count").cpu().numpy()
    C = O.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    assert (cnt <= C).all() and cnt.sum() <= cfg["T"] * cfg["k"]


def test_non_finite_tokens():
    cfg = _case(T=256, E=8, k=2, cf=1.25)
    T, E, k = cfg["T"], cfg["E"], cfg["k"]
    x = datagen.bf16_bits_to_f32(cfg["x"]).copy()
    x[3, :] = np.nan
    x[7, 0] = np.inf
    x[11, :] = -np.inf
    x[12, 5] = np.nan
    cfg["x"] = datagen.f32_to_bf16_bits(x)
    print("non-finite tokens 3, 7, 11, 12", flush=True)
    y, aux, idx, gate, drop, plan = _run(cfg)
    gi = idx.cpu().numpy()
    assert gi.min() >= 0 and gi.max() < E
    assert all(len(set(r)) == k for r in gi.tolist())
    C = O.capacity(T, E, k, cfg["cf"])
    rs, rd, rc = O.assign_slots(gi, E, C)
    assert (plan.intermediate("slot").cpu().numpy() == rs).all()
    assert (drop.cpu().numpy() == rd).all()
    assert (plan.intermediate("expert_count").cpu().numpy() == rc).all()
    # finite tokens: routing and gates against the oracle's router on their rows
    x64 = O.widen(cfg["x"], "bf16")
    fin = np.isfinite(x64).all(axis=1)
    z = O.router_logits(x64[fin], cfg["W_r"], cfg["b_r"])
    p = O.softmax(z)
    ref_idx = O.top_k(z, k)
    g = gate.cpu().numpy()
    agree = check_routing(gi[fin], g[fin], dict(z=z, expert_idx=ref_idx, gate=O.gates(z, p, ref_idx)), k)
    # their outputs: the gate-weighted sum of the oracle's experts over the kept choices
    yg = host_f64(y)
    toks = np.nonzero(fin)[0][agree]
    ref = np.zeros((toks.size, cfg["d"]))
    for i, t in enumerate(toks):
        for j in range(k):
            if rd[t, j] == 0:
                e = gi[t, j]
                o = O.expert_ffn(x64[t:t + 1], O.widen(cfg["W1"][e], "bf16"), O.widen(cfg["W2"][e], "bf16"),
                                 cfg["act"])
                ref[i] += float(g[t, j]) * o[0]
    assert np.isfinite(yg[toks]).all()
    _, bound = layer_bound(cfg, gi, rs, g, tokens=toks)
    check_y(yg[toks], ref, np.arange(toks.size), "bf16", bound[toks])
