"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each check cites the passage or identity it follows.  The `check_*`
helpers raise AssertionError; the tests call them on the oracle as it is,
and the planted-mistake tests at the end call them on an oracle with one
plausible mistake patched in, to show that the pins would catch it.
"""
import math

import numpy as np
import pytest
import scipy.special

from conftest import golden
from oracle import moe as O
import datagen


def _route_one(x, W_r, k, b_r=None):
    x64 = np.asarray(x, dtype=np.float64)
    z = O.router_logits(x64, W_r, b_r)
    p = O.softmax(z)
    idx = O.top_k(z, k)
    g = O.gates(z, p, idx)
    return z, p, idx, g


# ---------------------------------------------------------------------------
# softmax: the typical-logit table and a library routine
# ---------------------------------------------------------------------------

def check_softmax_table():
    g = golden("softmax_typical_logits.json")
    for case in g["cases"]:
        p = O.softmax(np.array([case["logits"]]))[0]
        assert np.allclose(np.round(p, g["digits"]), case["probs"], atol=0, rtol=0), p
        assert abs(p.sum() - 1.0) < 1e-15


def test_softmax_table():
    check_softmax_table()


def test_softmax_matches_scipy_and_is_shift_invariant():
    rng = np.random.default_rng(1)
    z = rng.normal(size=(50, 17)) * 30
    assert np.allclose(O.softmax(z), scipy.special.softmax(z, axis=1), rtol=1e-13, atol=1e-300)
    assert np.allclose(O.softmax(z + 1000.0), O.softmax(z), rtol=1e-12)


# ---------------------------------------------------------------------------
# the worked top-2 example
# ---------------------------------------------------------------------------

def _worked_router():
    g = golden("worked_top2.json")
    x = np.array(g["x"])
    l = np.array(g["router_logits"])
    # W_r such that W_r x = l: W_r = l x^T / |x|^2 (the page's x . W_g, transposed)
    W_r = (np.outer(l, x) / np.dot(x, x)).astype(np.float32)
    return g, x, l, W_r


def check_worked_top2():
    g, x, l, W_r = _worked_router()
    z, p, idx, gate = _route_one(x[None, :], W_r, g["k"])
    assert np.allclose(z[0], l, atol=1e-6)
    assert sorted(idx[0].tolist()) == g["kept_experts"]
    assert idx[0].tolist() == [1, 0]          # best first: 1.6 > 1.05
    G = np.zeros(len(l))
    G[idx[0]] = gate[0]
    assert np.round(G, g["digits"]).tolist() == g["G"], G
    # renormalising the full-softmax probabilities of the kept pair gives the same gates
    pk = p[0, idx[0]]
    assert np.allclose(pk / pk.sum(), gate[0], rtol=1e-6)


def test_worked_top2():
    check_worked_top2()


def test_worked_top2_output_is_gate_weighted_sum():
    """y = 0.366 E_0(x) + 0.634 E_1(x) for the worked example, with random experts."""
    g, x, l, W_r = _worked_router()
    rng = np.random.default_rng(3)
    E, d, f = 4, 3, 5
    W1 = rng.normal(size=(E, f, d)).astype(np.float32)
    W2 = rng.normal(size=(E, d, f)).astype(np.float32)
    r = O.forward(x[None, :].astype(np.float32), W_r, W1, W2, k=2, cf=4.0, alpha=0.01,
                  act="relu", dtype="f32")
    e0 = O.expert_ffn(x[None, :], W1[0].astype(np.float64), W2[0].astype(np.float64), "relu")
    e1 = O.expert_ffn(x[None, :], W1[1].astype(np.float64), W2[1].astype(np.float64), "relu")
    G0 = float(r["gate"][0, 1])
    G1 = float(r["gate"][0, 0])
    assert round(G0, 3) == 0.366 and round(G1, 3) == 0.634
    assert np.allclose(r["y"][0], G0 * e0[0] + G1 * e1[0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# ties: the all-zero router
# ---------------------------------------------------------------------------

def check_tie_break():
    g = golden("tie_break.json")
    E, k = g["E"], g["k"]
    rng = np.random.default_rng(5)
    T, d = 200, 12
    x = rng.normal(size=(T, d)).astype(np.float32)
    W_r = np.zeros((E, d), dtype=np.float32)
    r = O.forward(x, W_r, np.zeros((E, 4, d), np.float32), np.zeros((E, d, 4), np.float32),
                  k=k, cf=float(E), alpha=0.01, act="relu", dtype="f32")
    assert (r["expert_idx"] == np.array(g["chosen"])[None, :]).all()
    rc = r["route_count"]
    assert all(rc[e] == 0 for e in g["empty_experts"])
    assert rc[0] == T and rc[1] == T
    # k = 1 with capacity: a closed form -- tokens 0..C-1 keep slot t, the rest drop
    r1 = O.forward(x, W_r, np.zeros((E, 4, d), np.float32), np.zeros((E, d, 4), np.float32),
                   k=1, cf=1.0, alpha=0.01, act="relu", dtype="f32")
    C = r1["C"]
    assert C == 25
    assert (r1["slot"][:C, 0] == np.arange(C)).all()
    assert (r1["slot"][C:, 0] == -1).all() and (r1["drop_mask"][C:, 0] == 1).all()
    assert (r1["drop_mask"][:C, 0] == 0).all()
    assert r1["expert_count"].tolist() == [C] + [0] * (E - 1)


def test_tie_break():
    check_tie_break()


# ---------------------------------------------------------------------------
# fp32 router: the bf16 collapse
# ---------------------------------------------------------------------------

def check_fp32_router():
    g = golden("bf16_collapse.json")
    # the page's scores, with the experts swapped so that a bf16 router
    # (which would tie, and tie-break to expert 0) picks a different expert
    scores = list(reversed(g["logits"]))         # [4.00, 4.01]
    bits = datagen.f32_to_bf16_bits(np.array(scores, np.float32))
    assert (datagen.bf16_bits_to_f32(bits) == g["bf16_value"]).all()   # both collapse to 4.0
    W_r = np.array(scores, dtype=np.float32)[:, None]
    z, p, idx, gate = _route_one(np.ones((1, 1)), W_r, 1)
    assert idx[0, 0] == 1 - g["fp32_argmax"]
    assert z[0, 1] - z[0, 0] > 0.005


def test_fp32_router():
    check_fp32_router()


def test_bf16_spacing():
    g = golden("bf16_collapse.json")
    four = datagen.f32_to_bf16_bits(np.array([4.0], np.float32)).astype(np.uint32)
    nxt = datagen.bf16_bits_to_f32((four + 1).astype(np.uint16))[0]
    assert nxt - 4.0 == g["bf16_spacing_4_to_8"]


def test_router_logits_are_correctly_rounded_fp32():
    """The fp32 logit is the fp64 dot product rounded once (checked with exact fractions)."""
    from fractions import Fraction
    rng = np.random.default_rng(9)
    x = rng.normal(size=(6, 7)).astype(np.float32)
    W = rng.normal(size=(3, 7)).astype(np.float32)
    z = O.router_logits(x.astype(np.float64), W)
    for t in range(6):
        for i in range(3):
            exact = sum(Fraction(float(W[i, j])) * Fraction(float(x[t, j])) for j in range(7))
            below = np.float32(float(exact))
            # the fp32 neighbours of the exact value bracket the result within one ulp
            assert abs(Fraction(float(z[t, i])) - exact) <= abs(
                Fraction(float(np.spacing(np.float32(abs(below)))))) / 2 + Fraction(1, 10**30)


# ---------------------------------------------------------------------------
# auxiliary loss: uniform value 1, Cauchy-Schwarz
# ---------------------------------------------------------------------------

def check_aux_uniform():
    rng = np.random.default_rng(11)
    for k in (1, 2):
        E, T, d = 8, 64, 5
        x = rng.normal(size=(T, d))
        z, p, idx, g = _route_one(x, np.zeros((E, d), np.float32), k)
        # all-zero router: P_i = 1/E exactly, so N sum f_i P_i = sum f_i = 1
        assert abs(O.aux_loss(p, idx, E, 0.01) - 0.01) < 1e-15
    # balanced choices: f_i = 1/E, so N sum f_i P_i = sum P_i = 1 whatever P is
    E = 6
    T = E * 7
    x = np.zeros((T, E))
    x[np.arange(T), np.arange(T) % E] = 1.0
    x += rng.normal(size=x.shape) * 0.01
    W_r = (np.eye(E) * 3.0).astype(np.float32)
    z, p, idx, g = _route_one(x, W_r, 1)
    assert (np.bincount(idx[:, 0], minlength=E) == T // E).all()
    assert abs(O.aux_loss(p, idx, E, 1.0) - 1.0) < 1e-12


def test_aux_uniform():
    check_aux_uniform()


def test_aux_cauchy_schwarz():
    """When P equals f (near one-hot probabilities), N sum f_i^2 >= 1, equality iff uniform."""
    E, T = 5, 100
    x = np.zeros((T, E))
    hot = np.array([0] * 40 + [1] * 30 + [2] * 20 + [3] * 10)
    x[np.arange(T), hot] = 1.0
    W_r = (np.eye(E) * 60.0).astype(np.float32)
    z, p, idx, g = _route_one(x, W_r, 1)
    f = np.bincount(idx[:, 0], minlength=E) / T
    aux = O.aux_loss(p, idx, E, 1.0)
    assert abs(aux - E * np.sum(f * f)) < 1e-12
    assert aux > 1.0


def test_aux_k2_counts_both_ranks():
    """k = 2: f counts both choices over k T, so a balanced pair split gives exactly 1.

    First choices alone are unbalanced here (experts 0 and 3 only), so a loss
    that counted only rank 0 would not give 1.
    """
    E = 4
    pref = [(0, 1), (0, 2), (3, 1), (3, 2)]
    x = np.zeros((len(pref), E))
    for t, (a, b) in enumerate(pref):
        x[t, a] = 2.0
        x[t, b] = 1.0
    W_r = np.eye(E, dtype=np.float32)
    z, p, idx, g = _route_one(x, W_r, 2)
    assert idx.tolist() == [list(q) for q in pref]
    assert (np.bincount(idx.reshape(-1), minlength=E) == 2).all()
    assert abs(O.aux_loss(p, idx, E, 1.0) - 1.0) < 1e-12


# ---------------------------------------------------------------------------
# capacity and slots
# ---------------------------------------------------------------------------

def check_capacity_exercise():
    g = golden("capacity_exercise.json")
    E, k, T, cf = g["E"], g["k"], g["T"], g["cf"]
    C = O.capacity(T, E, k, cf)
    assert C == g["C"]
    t = np.arange(T)
    uni = np.stack([(2 * t) % E, (2 * t + 1) % E], axis=1)
    assert (np.bincount(uni.reshape(-1), minlength=E) == g["uniform_per_expert"]).all()
    slot, drop, cnt = O.assign_slots(uni, E, C)
    assert int(drop.sum()) == g["uniform_dropped"]
    hot = np.where(t[:, None] < 512,
                   np.stack([np.zeros(T, int), 1 + t % 7], axis=1),
                   np.stack([1 + t % 7, 1 + (t + 1) % 7], axis=1))
    n_hot = int((hot == 0).sum())
    assert n_hot == g["hot_expert_assignments"] == round(g["hot_expert_share"] * k * T)
    slot, drop, cnt = O.assign_slots(hot, E, C)
    assert int(drop.sum()) == g["hot_expert_dropped"]
    assert round(100.0 * drop.sum() / (k * T), 1) == g["dropped_fraction_percent"]
    # the dropped ones are the hot expert's latest tokens (token order)
    assert (drop[:C, 0] == 0).all() and (drop[C:512, 0] == 1).all()
    assert cnt[0] == C


def test_capacity_exercise():
    check_capacity_exercise()


def check_rank_major():
    """GShard rule: every first choice is placed before any second choice."""
    idx = np.array([[0, 1], [1, 2]])
    slot, drop, cnt = O.assign_slots(idx, 3, 1)
    # token 1's first choice (expert 1) takes the only slot; token 0's second choice drops
    assert slot[1, 0] == 0 and drop[1, 0] == 0
    assert drop[0, 1] == 1 and slot[0, 1] == -1
    assert cnt.tolist() == [1, 1, 1]


def test_rank_major():
    check_rank_major()


def test_capacity_rounding_covers_even_split():
    """cf = 1: slots cover the ideal even split, so a perfectly even routing never drops."""
    for T, E in [(10, 3), (1000, 7), (16384, 64), (513, 8)]:
        C = O.capacity(T, E, 1, 1.0)
        assert C >= T / E and C - 1 < T / E
        idx = (np.arange(T) % E)[:, None]
        slot, drop, cnt = O.assign_slots(idx, E, C)
        assert drop.sum() == 0
    assert O.capacity(1000, 10, 1, 1.1) == 110
    assert O.capacity(16, 2, 2, 8.0) == 16        # never above T


def test_idle_capacity():
    """No drops and exact C: idle fraction of the slots is 1 - 1/cf ([CMU-L16] section 6.1)."""
    T, E = 1024, 8
    idx = (np.arange(T) % E)[:, None]
    for cf in (2.0, 1.25, 1.0):
        C = O.capacity(T, E, 1, cf)
        slot, drop, cnt = O.assign_slots(idx, E, C)
        assert drop.sum() == 0
        idle = 1.0 - cnt.sum() / (E * C)
        assert abs(idle - (1.0 - 1.0 / cf)) < 1e-12


def test_slot_invariants_random():
    rng = np.random.default_rng(21)
    for k in (1, 2, 3):
        T, E = 300, 7
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
        C = O.capacity(T, E, k, 0.8)
        slot, drop, cnt = O.assign_slots(idx, E, C)
        assert cnt.sum() + drop.sum() == k * T
        assert ((slot >= 0) == (drop == 0)).all()
        for e in range(E):
            s = []
            for j in range(k):
                for t in range(T):
                    if idx[t, j] == e and drop[t, j] == 0:
                        s.append(slot[t, j])
            assert s == list(range(len(s))) and len(s) == cnt[e] <= C


# ---------------------------------------------------------------------------
# experts: the split identity
# ---------------------------------------------------------------------------

def _split_identity(act):
    g = golden("split_identity.json")
    n = g["n_experts"]
    rng = np.random.default_rng(7)
    d, f, T = 6, 4, 5
    W = [rng.normal(size=(f, d)) for _ in range(n)]
    V = [rng.normal(size=(f, d)) for _ in range(n)]
    b = [rng.normal(size=f) for _ in range(n)]
    U = [rng.normal(size=(d, f)) for _ in range(n)]
    c = rng.normal(size=d)
    x = rng.normal(size=(T, d))
    Wd, Vd, bd, Ud = np.vstack(W), np.vstack(V), np.concatenate(b), np.hstack(U)
    if act == "relu":
        dense = (Ud @ np.maximum(Wd @ x.T + bd[:, None], 0.0)).T + c
    else:
        a = Wd @ x.T
        dense = (Ud @ (a * scipy.special.expit(a) * (Vd @ x.T))).T + c
    def expert(i, ci):
        if act == "relu":
            return O.expert_ffn(x, W[i], U[i], "relu", b1=b[i], b2=ci)
        return O.expert_ffn(x, W[i], U[i], "swiglu", b2=ci, W3=V[i])
    split = sum(expert(i, c if i == 0 else np.zeros(d)) for i in range(n))
    assert np.max(np.abs(split - dense)) < 1e-12
    full = sum(expert(i, c) for i in range(n))
    assert np.allclose(full - dense, (n - 1) * c[None, :], atol=1e-12)
    assert np.max(np.abs(full - dense)) > 0.1


def check_split_identity():
    _split_identity("relu")
    _split_identity("swiglu")


def test_split_identity():
    check_split_identity()


def test_silu_values():
    a = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    assert np.allclose(O.silu(a), a * scipy.special.expit(a), rtol=1e-15, atol=1e-300)
    assert O.silu(np.array([1.0]))[0] == pytest.approx(0.7310585786300049, rel=1e-15)


# ---------------------------------------------------------------------------
# sizes the pages print for the Mixtral-shaped workload
# ---------------------------------------------------------------------------

def test_mixtral_sizes():
    g = golden("sizes.json")
    c = datagen.CONFIGS["mixtral"]
    per_expert = 3 * c["d"] * c["f"]
    assert round(per_expert / 1e6, 1) == g["mixtral_expert_params_millions"]
    disp = c["T"] * c["k"] * c["d"] * 2
    assert round(disp / 1e6) == g["mixtral_dispatch_MB"]
    c5 = datagen.CONFIGS["many_expert"]
    assert 2 * c5["E"] * c5["d"] * c5["f"] == 2 ** 31      # ~2.1e9 expert parameters


# ---------------------------------------------------------------------------
# router z-loss ([CMU-L16] section 4.2): mean over tokens of logsumexp^2
# ---------------------------------------------------------------------------

def check_z_loss_zero_router():
    """W_r = 0: every logit is 0, so each token's log-sum-exp is ln E exactly."""
    for E in (1, 2, 8, 64, 256):
        x = np.ones((7, 16))
        z = O.router_logits(x, np.zeros((E, 16), np.float32))
        assert abs(O.router_z_loss(z) - math.log(E) ** 2) <= 1e-12 * max(1.0, math.log(E) ** 2)


def check_z_loss_equal_logits():
    """A row of E equal logits a has log-sum-exp a + ln E: the value is
    mean_t (a_t + ln E)^2, also where exp(a) overflows fp32 and fp64 (a = 800)."""
    E = 8
    a = np.array([0.0, 1.5, -3.0, 80.0, -100.0, 800.0, -800.0])
    z = np.repeat(a[:, None], E, axis=1).astype(np.float32)
    want = float(np.mean((a.astype(np.float32).astype(np.float64) + math.log(E)) ** 2))
    assert abs(O.router_z_loss(z) - want) <= 1e-12 * want


def test_z_loss_zero_router():
    check_z_loss_zero_router()


def test_z_loss_equal_logits():
    check_z_loss_equal_logits()


def test_z_loss_brute_force():
    """Tiny random logits against a pure-Python log-sum-exp, token by token."""
    rng = np.random.default_rng(4)
    z = (rng.standard_normal((9, 5)) * 3).astype(np.float32)
    tot = 0.0
    for row in z.tolist():
        lse = math.log(sum(math.exp(v) for v in row))
        tot += lse * lse
    assert abs(O.router_z_loss(z) - tot / z.shape[0]) <= 1e-12 * tot


# ---------------------------------------------------------------------------
# noisy top-k ([CMU-L16] section 2.3): H = W_r x + eps * softplus(W_noise x)
# ---------------------------------------------------------------------------

def _noisy_case(seed=5, T=40, d=16, E=6):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    W_r = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    W_n = (rng.standard_normal((E, d)) * 0.3).astype(np.float32)
    eps = rng.standard_normal((T, E)).astype(np.float32)
    return x, W_r, W_n, eps


def check_noisy_without_noise():
    """eps = 0: the noisy logits are the clean ones, bit for bit."""
    x, W_r, W_n, eps = _noisy_case()
    H = O.noisy_router_logits(x, W_r, None, W_n, np.zeros_like(eps))
    assert np.array_equal(H, O.router_logits(x, W_r))


def check_noisy_zero_noise_weights():
    """W_noise = 0: softplus(0) = ln 2, so H = z + eps ln 2 (rounded once to fp32)."""
    x, W_r, W_n, eps = _noisy_case()
    H = O.noisy_router_logits(x, W_r, None, np.zeros_like(W_n), eps)
    want = (O.router_logits(x, W_r).astype(np.float64) + eps.astype(np.float64) * math.log(2.0))
    assert np.array_equal(H, want.astype(np.float32))


def check_noisy_zero_init_routes_by_noise():
    """W_r = W_noise = 0 (the page's initialisation): H = eps ln 2, so each
    token goes to the expert of its largest draw (lowest index on ties) --
    the random, even assignment the page describes."""
    x, W_r, W_n, eps = _noisy_case(T=2000, E=8)
    H = O.noisy_router_logits(x, np.zeros_like(W_r), None, np.zeros_like(W_n), eps)
    assert (O.top_k(H, 1)[:, 0] == np.argmax(eps, axis=1)).all()
    load = np.bincount(O.top_k(H, 1)[:, 0], minlength=8) / 2000
    assert np.all(np.abs(load - 1 / 8) < 0.03)


def test_noisy_without_noise():
    check_noisy_without_noise()


def test_noisy_zero_noise_weights():
    check_noisy_zero_noise_weights()


def test_noisy_zero_init_routes_by_noise():
    check_noisy_zero_init_routes_by_noise()


def test_softplus_values():
    """softplus(0) = ln 2, softplus(a) - softplus(-a) = a, and no overflow at +-1000."""
    a = np.array([0.0, 1.0, -3.0, 20.0, 1000.0, -1000.0])
    sp = O.softplus(a)
    assert sp[0] == math.log(2.0)
    assert np.allclose(O.softplus(a) - O.softplus(-a), a, rtol=0, atol=1e-12)
    assert sp[4] == 1000.0 and sp[5] == 0.0 and abs(sp[1] - math.log1p(math.e)) < 1e-15


# ---------------------------------------------------------------------------
# priority routing ([CS25-L5], V-MoE part): capacity goes to the highest
# scores first; ties to the lower token index; rank-major for k > 1
# ---------------------------------------------------------------------------

def _priority_case(seed=9, T=300, E=5, k=2):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((T, E))
    idx = np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int32)
    pr = rng.random(T).astype(np.float32)
    return idx, pr


def check_priority_equal_scores_is_token_order():
    """One score for every token: the visit order is token order, so the
    slots are those of the plain capacity rule."""
    idx, _ = _priority_case()
    C = 50
    got = O.assign_slots_priority(idx, 5, C, np.full(idx.shape[0], 0.25, np.float32))
    ref = O.assign_slots(idx, 5, C)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)


def check_priority_increasing_is_reversed_token_order():
    """Scores increasing with t: the last token goes first, which is the plain
    rule on the reversed token sequence."""
    idx, _ = _priority_case(seed=3)
    T, C = idx.shape[0], 40
    got_s, got_d, got_c = O.assign_slots_priority(idx, 5, C, np.arange(T, dtype=np.float32))
    ref_s, ref_d, ref_c = O.assign_slots(idx[::-1].copy(), 5, C)
    assert np.array_equal(got_s, ref_s[::-1]) and np.array_equal(got_d, ref_d[::-1])
    assert np.array_equal(got_c, ref_c)


def check_priority_keeps_the_highest():
    """k = 1 with half the even split (the page's gamma = 0.5): each expert
    keeps exactly its C highest-scoring tokens (ties: lower index), and its
    slots number them from the highest down; found here per expert by a
    selection over that expert's tokens instead of one sequential fill."""
    rng = np.random.default_rng(17)
    T, E = 400, 4
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    pr = np.round(rng.random(T), 2).astype(np.float32)     # many equal scores
    C = O.capacity(T, E, 1, 0.5)
    slot, drop, cnt = O.assign_slots_priority(idx, E, C, pr)
    for e in range(E):
        toks = [t for t in range(T) if idx[t, 0] == e]
        ranked = sorted(toks, key=lambda t: (-float(pr[t]), t))
        kept = ranked[:C]
        assert cnt[e] == len(kept)
        for r, t in enumerate(ranked):
            if r < C:
                assert slot[t, 0] == r and drop[t, 0] == 0
            else:
                assert slot[t, 0] == -1 and drop[t, 0] == 1


def check_priority_rank_major():
    """k = 2: every token's first choice is placed before any second choice,
    so no expert keeps a second choice while it drops a first choice."""
    idx, pr = _priority_case(seed=21, T=500, E=4)
    slot, drop, _ = O.assign_slots_priority(idx, 4, 200, pr)
    for e in range(4):
        first_dropped = np.any((idx[:, 0] == e) & (drop[:, 0] == 1))
        second_kept = np.any((idx[:, 1] == e) & (drop[:, 1] == 0))
        assert not (first_dropped and second_kept)
        # kept second choices sit after every kept first choice of the expert
        s0 = slot[(idx[:, 0] == e) & (drop[:, 0] == 0), 0]
        s1 = slot[(idx[:, 1] == e) & (drop[:, 1] == 0), 1]
        if s0.size and s1.size:
            assert s1.min() > s0.max()


def test_priority_equal_scores_is_token_order():
    check_priority_equal_scores_is_token_order()


def test_priority_increasing_is_reversed_token_order():
    check_priority_increasing_is_reversed_token_order()


def test_priority_keeps_the_highest():
    check_priority_keeps_the_highest()


def test_priority_rank_major():
    check_priority_rank_major()


def test_priority_worked_example():
    """By hand: one expert, C = 2, scores [NaN, 0.1, 0.5, -inf, 0.5, -0.0, 0.0].
    Order: t2 and t4 (0.5; lower index first), t1, the zeros t5 and t6 (equal:
    -0 = +0), t3 (-inf), t0 (NaN last).  Kept: t2 slot 0, t4 slot 1."""
    pr = np.array([np.nan, 0.1, 0.5, -np.inf, 0.5, -0.0, 0.0], np.float32)
    idx = np.zeros((7, 1), np.int32)
    assert O.priority_order(pr).tolist() == [2, 4, 1, 5, 6, 3, 0]
    slot, drop, cnt = O.assign_slots_priority(idx, 1, 2, pr)
    assert slot[:, 0].tolist() == [-1, -1, 0, -1, 1, -1, -1]
    assert drop[:, 0].tolist() == [1, 1, 0, 1, 0, 1, 1] and cnt.tolist() == [2]


# ---------------------------------------------------------------------------
# backward of the gate side: finite differences of the forward definitions
# (routing held fixed), closed forms, and the page's exercise 2
# ---------------------------------------------------------------------------

def _bwd_case(k, seed=13, T=7, d=5, E=4, drops=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    W = rng.standard_normal((E, d)) * 0.8
    z = x @ W.T
    idx = np.argsort(-z, axis=1, kind="stable")[:, :k]
    out = rng.standard_normal((T, k, 3))
    dy = rng.standard_normal((T, 3))
    drop = np.zeros((T, k), np.uint8)
    if drops:
        drop[1, 0] = 1
        drop[4, k - 1] = 1
    return x, W, idx, out, dy, drop


def _router_loss(x, W, idx, out, dy, drop, k, alpha, zw):
    """The router's loss from the oracle's forward pieces, all in float64:
    <dy, combine(g, drop, out)> + aux + zw * z-loss, with fixed choices."""
    z = x @ W.T
    T = z.shape[0]
    p = O.softmax(z)
    rows = np.arange(T)[:, None]
    g = p[rows, idx] if k == 1 else O.softmax(z[rows, idx])
    y = O.combine(g, drop, out)
    return float(np.sum(dy * y)) + O.aux_loss(p, idx, W.shape[0], alpha) + zw * O.router_z_loss(z)


def check_router_backward_finite_differences(k):
    x, W, idx, out, dy, drop = _bwd_case(k)
    alpha, zw = 0.3, 0.2
    T = x.shape[0]
    rows = np.arange(T)[:, None]
    z = x @ W.T
    p = O.softmax(z)
    g = p[rows, idx] if k == 1 else O.softmax(z[rows, idx])
    dgate, _ = O.combine_backward(dy, g, drop, out)
    dz, dW, db, dx = O.router_backward(x, W, z, idx, dgate, k, alpha, zw)
    h = 1e-6
    for (i, j) in [(0, 0), (1, 3), (2, 1), (3, 4)]:
        Wp, Wm = W.copy(), W.copy()
        Wp[i, j] += h
        Wm[i, j] -= h
        fd = (_router_loss(x, Wp, idx, out, dy, drop, k, alpha, zw) -
              _router_loss(x, Wm, idx, out, dy, drop, k, alpha, zw)) / (2 * h)
        assert abs(fd - dW[i, j]) <= 1e-6 * max(1.0, abs(fd)), (i, j, fd, dW[i, j])
    for (t, j) in [(0, 0), (4, 2), (6, 4)]:
        xp, xm = x.copy(), x.copy()
        xp[t, j] += h
        xm[t, j] -= h
        fd = (_router_loss(xp, W, idx, out, dy, drop, k, alpha, zw) -
              _router_loss(xm, W, idx, out, dy, drop, k, alpha, zw)) / (2 * h)
        assert abs(fd - dx[t, j]) <= 1e-6 * max(1.0, abs(fd)), (t, j, fd, dx[t, j])
    assert np.allclose(db, dz.sum(axis=0), rtol=0, atol=1e-14)


def check_combine_backward_finite_differences():
    x, W, idx, out, dy, drop = _bwd_case(2)
    rng = np.random.default_rng(2)
    g = rng.random((x.shape[0], 2))
    dgate, dout = O.combine_backward(dy, g, drop, out)
    h = 1e-6
    loss = lambda gg, oo: float(np.sum(dy * O.combine(gg, drop, oo)))
    for (t, j) in [(0, 0), (1, 0), (4, 1), (5, 1)]:
        gp, gm = g.copy(), g.copy()
        gp[t, j] += h
        gm[t, j] -= h
        assert abs((loss(gp, out) - loss(gm, out)) / (2 * h) - dgate[t, j]) < 1e-8
        op, om = out.copy(), out.copy()
        op[t, j, 2] += h
        om[t, j, 2] -= h
        assert abs((loss(g, op) - loss(g, om)) / (2 * h) - dout[t, j, 2]) < 1e-8


def test_router_backward_finite_differences_k1():
    check_router_backward_finite_differences(1)


def test_router_backward_finite_differences_k2():
    check_router_backward_finite_differences(2)


def test_combine_backward_finite_differences():
    check_combine_backward_finite_differences()


def test_aux_gradient_vanishes_at_uniform_load():
    """f_i = 1/N: alpha N sum_i f_i P_i = alpha sum_i P_i = alpha, a constant,
    so its gradient is zero whatever the probabilities."""
    rng = np.random.default_rng(4)
    T, E = 12, 4
    z = rng.standard_normal((T, E))
    idx = (np.arange(T) % E)[:, None]
    dz, dW, _, _ = O.router_backward(rng.standard_normal((T, 3)), rng.standard_normal((E, 3)), z, idx,
                                     np.zeros((T, 1)), 1, 0.5, 0.0)
    assert np.abs(dz).max() < 1e-16


def test_z_loss_gradient_at_zero_router():
    """W_r = 0: every logit is 0, lse = ln N and p = 1/N, so d(w z-loss)/dz_ti
    = w (2/T) ln N / N everywhere."""
    T, E, w = 10, 8, 0.001
    idx = np.zeros((T, 1), np.int64)
    dz, _, _, _ = O.router_backward(np.ones((T, 2)), np.zeros((E, 2)), np.zeros((T, E)), idx,
                                    np.zeros((T, 1)), 1, 0.0, w)
    assert np.allclose(dz, w * 2.0 / T * math.log(E) / E, rtol=1e-14, atol=0)


def test_overloaded_expert_is_pushed_down():
    """[CMU-L16] exercise 2: the balance loss's gradient with respect to
    p_i(x_t) is alpha N f_i / T, so the most loaded expert's logit has a
    positive gradient for every token (descent lowers it) and the least
    loaded one a negative one."""
    rng = np.random.default_rng(8)
    T, E = 40, 4
    z = rng.standard_normal((T, E))
    idx = np.where(np.arange(T) < 25, 0, 1 + np.arange(T) % 3)[:, None]     # expert 0 holds 25 of 40
    dz, _, _, _ = O.router_backward(np.zeros((T, 2)), np.zeros((E, 2)), z, idx, np.zeros((T, 1)), 1, 0.1, 0.0)
    f = O.route_count(idx, E)
    assert np.all(dz[:, np.argmax(f)] > 0) and np.all(dz[:, np.argmin(f)] < 0)


# ---------------------------------------------------------------------------
# "No Token Left Behind" re-routing ([CS25-L5]): overflow tries later choices
# ---------------------------------------------------------------------------

def _pref(seed, T, E, R):
    z = np.random.default_rng(seed).standard_normal((T, E))
    return np.argsort(-z, axis=1, kind="stable")[:, :R].astype(np.int32)


def check_reroute_worked_example():
    """By hand: T = 5, E = 2, C = 2, two stages, preferences
    [0,1] [0,1] [0,1] [1,0] [0,1].  Stage 0: t0 -> e0 slot 0, t1 -> e0 slot
    1, t2 finds e0 full, t3 -> e1 slot 0, t4 finds e0 full.  Stage 1: t2 ->
    e1 slot 1; t4 finds e1 full and is dropped."""
    pref = np.array([[0, 1], [0, 1], [0, 1], [1, 0], [0, 1]], np.int32)
    ex, sl, st, cnt = O.assign_slots_reroute(pref, 2, 2, 2)
    assert ex.tolist() == [0, 0, 1, 1, -1] and sl.tolist() == [0, 1, 1, 0, -1]
    assert st.tolist() == [0, 0, 1, 0, -1] and cnt.tolist() == [2, 2]


def check_reroute_places_everyone():
    """E stages and E C >= T: nobody is dropped (a dropped token would have
    found every expert full, so E C tokens would be placed besides it)."""
    T, E = 300, 6
    pref = _pref(5, T, E, E)
    C = O.capacity(T, E, 1, 1.0)
    ex, sl, st, cnt = O.assign_slots_reroute(pref, E, C, E)
    assert np.all(ex >= 0) and cnt.sum() == T


def test_reroute_one_stage_is_the_plain_rule():
    pref = _pref(7, 400, 5, 3)
    C = 60
    ex, sl, st, cnt = O.assign_slots_reroute(pref, 5, C, 1)
    rs, rd, rc = O.assign_slots(pref[:, :1].copy(), 5, C)
    assert np.array_equal(sl, rs[:, 0]) and np.array_equal(ex >= 0, rd[:, 0] == 0)
    assert np.array_equal(cnt, rc)


def test_reroute_no_overflow_stays_in_stage_zero():
    pref = _pref(8, 200, 4, 3)
    ex, sl, st, cnt = O.assign_slots_reroute(pref, 4, 200, 3)
    assert np.all(st == 0) and np.array_equal(ex, pref[:, 0])


def check_reroute_padded_preferences():
    """By hand: an entry outside [0, E) is no choice at that stage.  T = 4,
    E = 2, C = 1, three stages, preferences [-1,0,1] [0,5,1] [-1,-1,-1]
    [0,1,0].  Stage 0: t0 has no choice, t1 -> e0 slot 0, t2 has none, t3
    finds e0 full.  Stage 1: t0 finds e0 full, t2 has none, t3 -> e1 slot
    0.  Stage 2: t0 finds e1 full, t2 has none: both are dropped."""
    pref = np.array([[-1, 0, 1], [0, 5, 1], [-1, -1, -1], [0, 1, 0]], np.int32)
    ex, sl, st, cnt = O.assign_slots_reroute(pref, 2, 1, 3)
    assert ex.tolist() == [-1, 0, -1, 1] and sl.tolist() == [-1, 0, -1, 0]
    assert st.tolist() == [-1, 0, -1, 1] and cnt.tolist() == [1, 1]


def test_reroute_worked_example():
    check_reroute_worked_example()


def test_reroute_padded_preferences():
    check_reroute_padded_preferences()


def test_reroute_places_everyone():
    check_reroute_places_everyone()


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

def _top_k_bf16(z, k):
    bits = datagen.f32_to_bf16_bits(np.asarray(z, np.float32))
    return np.argsort(-datagen.bf16_bits_to_f32(bits), axis=1, kind="stable")[:, :k].astype(np.int32)


def _top_k_high_tie(z, k):
    zz = np.asarray(z, np.float32)[:, ::-1]
    o = np.argsort(-zz, axis=1, kind="stable")[:, :k]
    return (zz.shape[1] - 1 - o).astype(np.int32)


def _gates_raw(z, p, idx):
    return p[np.arange(idx.shape[0])[:, None], idx].astype(np.float32)


def _assign_token_major(idx, E, C):
    T, k = idx.shape
    fill = [0] * E
    slot = np.full((T, k), -1, np.int32)
    drop = np.zeros((T, k), np.uint8)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if fill[e] < C:
                slot[t, j] = fill[e]
                fill[e] += 1
            else:
                drop[t, j] = 1
    return slot, drop, np.array(fill)


def _capacity_floor(T, E, k, cf):
    return int(min(T, math.floor(k * T * cf / E)))


def _softmax_wrong_axis(z):
    e = np.exp(np.asarray(z, np.float64))
    return e / e.sum(axis=0, keepdims=True)   # normalises over tokens, not experts


@pytest.mark.parametrize("name,repl,check", [
    ("top_k", _top_k_bf16, check_fp32_router),
    ("top_k", _top_k_high_tie, check_tie_break),
    ("gates", _gates_raw, check_worked_top2),
    ("assign_slots", _assign_token_major, check_rank_major),
    ("softmax", _softmax_wrong_axis, check_softmax_table),
])
def test_planted_mistake_is_caught(monkeypatch, name, repl, check):
    monkeypatch.setattr(O, name, repl)
    with pytest.raises(Exception):
        check()


def test_planted_capacity_floor_is_caught(monkeypatch):
    monkeypatch.setattr(O, "capacity", _capacity_floor)
    with pytest.raises(AssertionError):
        test_capacity_rounding_covers_even_split()


def test_planted_bias_on_every_expert_is_caught(monkeypatch):
    """An expert FFN that adds its output bias twice breaks the split identity."""
    orig = O.expert_ffn

    def twice(u, W1, W2, act, b1=None, b2=None, W3=None):
        o = orig(u, W1, W2, act, b1, b2, W3)
        return o if b2 is None else o + np.asarray(b2)[None, :]
    monkeypatch.setattr(O, "expert_ffn", twice)
    with pytest.raises(AssertionError):
        check_split_identity()


def test_planted_transposed_weight_is_caught(monkeypatch):
    """Using W1 as [d, f] (x W1 instead of W1 x) breaks the split identity."""
    orig = O.expert_ffn

    def transposed(u, W1, W2, act, b1=None, b2=None, W3=None):
        W1 = np.asarray(W1)
        W1t = W1.T.reshape(W1.shape) if W1.shape[0] != W1.shape[1] else W1.T
        return orig(u, W1t, W2, act, b1, b2, W3)
    monkeypatch.setattr(O, "expert_ffn", transposed)
    with pytest.raises(Exception):
        check_split_identity()


def test_planted_first_rank_only_aux_is_caught(monkeypatch):
    orig = O.aux_loss
    monkeypatch.setattr(O, "aux_loss", lambda p, idx, E, a: orig(p, idx[:, :1], E, a))
    with pytest.raises(AssertionError):
        test_aux_k2_counts_both_ranks()


def _z_loss_max_not_lse(z):
    m = np.max(np.asarray(z, np.float64), axis=-1)
    return float(np.mean(m * m))


def _z_loss_unsquared(z):
    z64 = np.asarray(z, np.float64)
    m = np.max(z64, axis=-1)
    return float(np.mean(m + np.log(np.sum(np.exp(z64 - m[:, None]), axis=-1))))


@pytest.mark.parametrize("repl", [_z_loss_max_not_lse, _z_loss_unsquared])
def test_planted_z_loss_mistake_is_caught(monkeypatch, repl):
    monkeypatch.setattr(O, "router_z_loss", repl)
    failed = 0
    for check in (check_z_loss_zero_router, check_z_loss_equal_logits):
        try:
            check()
        except AssertionError:
            failed += 1
    assert failed >= 1


def _noisy_exp_scale(x64, W_r, b_r, W_noise, eps):
    z = O.router_logits(x64, W_r, b_r).astype(np.float64)
    zn = O.router_logits(x64, W_noise).astype(np.float64)
    return (z + np.asarray(eps, np.float64) * np.exp(zn)).astype(np.float32)   # exp, not softplus


def _noisy_unscaled(x64, W_r, b_r, W_noise, eps):
    z = O.router_logits(x64, W_r, b_r).astype(np.float64)
    return (z + np.asarray(eps, np.float64)).astype(np.float32)               # no learned scale


@pytest.mark.parametrize("repl", [_noisy_exp_scale, _noisy_unscaled])
def test_planted_noisy_mistake_is_caught(monkeypatch, repl):
    monkeypatch.setattr(O, "noisy_router_logits", repl)
    with pytest.raises(AssertionError):
        check_noisy_zero_noise_weights()


def _priority_ascending(priority):
    pr = np.asarray(priority, dtype=np.float64)
    nan = np.isnan(pr)
    return np.lexsort((np.arange(pr.shape[0]), np.where(nan, 0.0, pr), nan))


def _priority_high_tie(priority):
    pr = np.asarray(priority, dtype=np.float64)
    nan = np.isnan(pr)
    return np.lexsort((-np.arange(pr.shape[0]), np.where(nan, 0.0, -pr), nan))


def _priority_token_major(idx, E, C, priority):
    T, k = idx.shape
    fill = [0] * E
    slot = np.full((T, k), -1, np.int32)
    drop = np.zeros((T, k), np.uint8)
    for t in O.priority_order(priority).tolist():
        for j in range(k):
            e = idx[t, j]
            if fill[e] < C:
                slot[t, j] = fill[e]
                fill[e] += 1
            else:
                drop[t, j] = 1
    return slot, drop, np.array(fill)


@pytest.mark.parametrize("name,repl,check", [
    ("priority_order", _priority_ascending, check_priority_keeps_the_highest),
    ("priority_order", _priority_high_tie, check_priority_equal_scores_is_token_order),
    ("assign_slots_priority", _priority_token_major, check_priority_rank_major),
])
def test_planted_priority_mistake_is_caught(monkeypatch, name, repl, check):
    monkeypatch.setattr(O, name, repl)
    with pytest.raises(AssertionError):
        check()


def _router_backward_no_minus_p(x64, W_r, z, idx, dgate, k, alpha, z_weight):
    """The gate path without the -p term of the softmax Jacobian."""
    dz, dW, db, dx = _ORIG_RB(x64, W_r, z, idx, dgate, k, alpha, z_weight)
    T = dz.shape[0]
    p = O.softmax(np.asarray(z, np.float64))
    e = np.asarray(idx)[:, 0]
    g = p[np.arange(T), e]
    dz = dz - (np.asarray(dgate)[:, 0] * g)[:, None] * (-p)
    return dz, dz.T @ x64, dz.sum(0), dz @ W_r


def _router_backward_f_without_k(x64, W_r, z, idx, dgate, k, alpha, z_weight):
    """f counted over kT choices but divided by T only."""
    return _ORIG_RB(x64, W_r, z, idx, dgate, k, alpha * k, z_weight)


def _router_backward_zloss_no_square(x64, W_r, z, idx, dgate, k, alpha, z_weight):
    """The z-loss gradient of (1/T) sum lse instead of (1/T) sum lse^2."""
    dz, _, _, _ = _ORIG_RB(x64, W_r, z, idx, dgate, k, alpha, 0.0)
    p = O.softmax(np.asarray(z, np.float64))
    dz = dz + z_weight * (1.0 / dz.shape[0]) * p
    return dz, dz.T @ x64, dz.sum(0), dz @ W_r


_ORIG_RB = O.router_backward


@pytest.mark.parametrize("repl,check", [
    (_router_backward_no_minus_p, lambda: check_router_backward_finite_differences(1)),
    (_router_backward_f_without_k, lambda: check_router_backward_finite_differences(2)),
    (_router_backward_zloss_no_square, lambda: check_router_backward_finite_differences(2)),
])
def test_planted_router_backward_mistake_is_caught(monkeypatch, repl, check):
    monkeypatch.setattr(O, "router_backward", repl)
    with pytest.raises(AssertionError):
        check()


def test_planted_combine_backward_drop_is_caught(monkeypatch):
    """A combine backward that also sends gradient to dropped choices."""
    def keep_all(dy, gate, drop, out):
        return _ORIG_CB(dy, gate, np.zeros_like(drop), out)
    monkeypatch.setattr(O, "combine_backward", keep_all)
    with pytest.raises(AssertionError):
        check_combine_backward_finite_differences()


_ORIG_CB = O.combine_backward


def _reroute_reverse_later_stages(pref, E, C, stages):
    """Later stages visit the tokens from the last one back."""
    T = pref.shape[0]
    fill = [0] * E
    ex = np.full(T, -1, np.int32)
    sl = np.full(T, -1, np.int32)
    st = np.full(T, -1, np.int32)
    for s in range(stages):
        for t in (range(T) if s == 0 else range(T - 1, -1, -1)):
            if st[t] < 0 and fill[pref[t, s]] < C:
                e = pref[t, s]
                ex[t], sl[t], st[t] = e, fill[e], s
                fill[e] += 1
    return ex, sl, st, np.array(fill)


def _reroute_first_choice_only(pref, E, C, stages):
    """Every stage offers the first choice again (no re-routing)."""
    return _ORIG_RR(np.repeat(pref[:, :1], pref.shape[1], axis=1), E, C, stages)


_ORIG_RR = O.assign_slots_reroute


@pytest.mark.parametrize("repl,check", [
    (_reroute_reverse_later_stages, check_reroute_worked_example),
    (_reroute_first_choice_only, check_reroute_places_everyone),
])
def test_planted_reroute_mistake_is_caught(monkeypatch, repl, check):
    monkeypatch.setattr(O, "assign_slots_reroute", repl)
    with pytest.raises(AssertionError):
        check()


# ---------------------------------------------------------------------------
# the near-tie exemption of the parity rule
# ---------------------------------------------------------------------------

def check_near_tie_table():
    """Hand-worked flags on logits whose gaps are exact binary fractions."""
    g = golden("near_tie.json")
    for case in g["cases"]:
        z = np.array([case["z"]], dtype=np.float32)
        got = bool(O.near_tie_tokens(z, case["k"], g["gap"])[0])
        assert got == case["tie"], case["what"]


def check_near_tie_batch_is_rowwise():
    """A batch gives each row's own flag (no mixing across tokens)."""
    g = golden("near_tie.json")
    for k in (1, 2):
        rows = [c for c in g["cases"] if c["k"] == k and len(c["z"]) == 4]
        z = np.array([c["z"] for c in rows], dtype=np.float32)
        assert O.near_tie_tokens(z, k, g["gap"]).tolist() == [c["tie"] for c in rows]


def test_near_tie_table():
    check_near_tie_table()
    check_near_tie_batch_is_rowwise()


def _near_tie_top2_gap_only(z, k, gap=1e-5):
    """Only the top-1/top-2 gap, whatever k."""
    s = -np.sort(-np.asarray(z, np.float64), axis=1)
    if s.shape[1] < 2:
        return np.zeros(s.shape[0], bool)
    return (s[:, 0] - s[:, 1]) < gap


def _near_tie_one_too_many(z, k, gap=1e-5):
    """Gaps among the k+2 largest instead of the k+1 largest."""
    return _ORIG_NT(z, k + 1, gap)


def _near_tie_index_order(z, k, gap=1e-5):
    """Adjacent gaps in expert-index order instead of sorted order."""
    a = np.asarray(z, np.float64)
    if a.shape[1] < 2:
        return np.zeros(a.shape[0], bool)
    return np.any(np.abs(a[:, 1:] - a[:, :-1]) < gap, axis=1)


def _near_tie_probabilities(z, k, gap=1e-5):
    """Gaps between softmax probabilities instead of fp32 logits."""
    p = O.softmax(np.asarray(z, np.float64))
    return _ORIG_NT(p, k, gap)


_ORIG_NT = O.near_tie_tokens


@pytest.mark.parametrize("repl", [_near_tie_top2_gap_only, _near_tie_one_too_many,
                                  _near_tie_index_order, _near_tie_probabilities])
def test_planted_near_tie_mistake_is_caught(monkeypatch, repl):
    monkeypatch.setattr(O, "near_tie_tokens", repl)
    with pytest.raises(AssertionError):
        check_near_tie_table()


# ---------------------------------------------------------------------------
# expert-side backward: the expert FFN and the dispatch ([CMU-L16] exercise 2,
# section 5: each expert is an ordinary FFN on its routed rows)
# ---------------------------------------------------------------------------

def _expert_case(act, bias, seed=3, rows=5, d=6, f=7):
    rng = np.random.default_rng(seed)
    c = dict(u=rng.normal(size=(rows, d)), W1=rng.normal(size=(f, d)) * 0.5, W2=rng.normal(size=(d, f)) * 0.5,
             W3=rng.normal(size=(f, d)) * 0.5 if act == "swiglu" else None,
             b1=rng.normal(size=f) * 0.3 if bias else None, b2=rng.normal(size=d) * 0.3 if bias else None,
             dout=rng.normal(size=(rows, d)))
    return c


def check_expert_backward_finite_differences(act, bias):
    """Central differences of the oracle's own expert forward (float64, h = 1e-6)
    for every entry of u, W1, W2, W3, b1 and b2."""
    c = _expert_case(act, bias)

    def loss(**over):
        a = dict(c)
        a.update(over)
        o = O.expert_ffn(a["u"], a["W1"], a["W2"], act, b1=a["b1"], b2=a["b2"], W3=a["W3"])
        return float(np.sum(o * c["dout"]))

    # keep every pre-activation away from the ReLU kink, where no derivative exists
    a0 = c["u"] @ c["W1"].T + (0 if c["b1"] is None else c["b1"])
    assert np.min(np.abs(a0)) > 1e-3
    g = O.expert_ffn_backward(c["u"], c["W1"], c["W2"], act, c["dout"], b1=c["b1"], W3=c["W3"])
    want = dict(u="du", W1="dW1", W2="dW2", W3="dW3", b1="db1", b2="db2")
    h = 1e-6
    for name, gname in want.items():
        if c[name] is None:
            continue
        base = c[name]
        num = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            p, m = base.copy(), base.copy()
            p[i] += h
            m[i] -= h
            num[i] = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
        assert np.allclose(g[gname], num, rtol=1e-6, atol=1e-7), (name, np.max(np.abs(g[gname] - num)))


@pytest.mark.parametrize("act,bias", [("relu", True), ("relu", False), ("swiglu", False)])
def test_expert_backward_finite_differences(act, bias):
    check_expert_backward_finite_differences(act, bias)


@pytest.mark.parametrize("act,bias", [("relu", True), ("swiglu", False)])
def test_expert_backward_matches_autograd(act, bias):
    """torch.autograd in float64 on the same FFN (a library's differentiation, independent
    of the hand-derived chain rule), on a wider case."""
    import torch
    c = _expert_case(act, bias, seed=9, rows=40, d=24, f=56)
    t = {k: (None if v is None else torch.tensor(v, dtype=torch.float64, requires_grad=True))
         for k, v in c.items() if k != "dout"}
    a = t["u"] @ t["W1"].T + (t["b1"] if t["b1"] is not None else 0)
    if act == "relu":
        h = torch.relu(a)
    else:
        h = torch.nn.functional.silu(a) * (t["u"] @ t["W3"].T)
    o = h @ t["W2"].T + (t["b2"] if t["b2"] is not None else 0)
    names = [k for k in ("u", "W1", "W2", "W3", "b1", "b2") if t[k] is not None]
    grads = torch.autograd.grad(o, [t[k] for k in names], grad_outputs=torch.tensor(c["dout"]))
    g = O.expert_ffn_backward(c["u"], c["W1"], c["W2"], act, c["dout"], b1=c["b1"], W3=c["W3"])
    for k, ref in zip(names, grads):
        gname = {"u": "du"}.get(k, "d" + k)
        np.testing.assert_allclose(g[gname], ref.numpy(), rtol=1e-12, atol=1e-12)


def _routing_case(seed=4, T=60, E=5, k=2, C=9):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    slot, drop, cnt = O.assign_slots(idx, E, C)
    return rng, idx, slot, drop, cnt


def check_dispatch_adjoint():
    """<dispatch(x), dxbuf> = <x, dispatch_backward(dxbuf)> on the kept rows, with drops."""
    rng, idx, slot, drop, cnt = _routing_case()
    T, k = idx.shape
    E, C, d = 5, 9, 3
    assert drop.any() and (drop == 0).any()
    x = rng.normal(size=(T, d))
    dxbuf = rng.normal(size=(E, C, d))
    xbuf = np.zeros((E, C, d))
    for t in range(T):
        for j in range(k):
            if slot[t, j] >= 0:
                xbuf[idx[t, j], slot[t, j]] = x[t]
    # rows at or beyond an expert's count are never written by the dispatch and never read back
    live = np.arange(C)[None, :] < cnt[:, None]
    lhs = np.sum(xbuf * dxbuf * live[:, :, None])
    rhs = np.sum(x * O.dispatch_backward(dxbuf, idx, slot))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs)), (lhs, rhs)


def check_dispatch_backward_brute():
    """Token by token: dx_t = dx_add_t + the rows of its kept choices."""
    rng, idx, slot, drop, cnt = _routing_case(seed=6, T=40, E=4, k=3, C=20)
    dxbuf = rng.normal(size=(4, 20, 2))
    add = rng.normal(size=(40, 2))
    got = O.dispatch_backward(dxbuf, idx, slot, dx_add=add)
    for t in range(40):
        want = add[t].copy()
        for j in range(3):
            if drop[t, j] == 0:
                want += dxbuf[idx[t, j], slot[t, j]]
        assert np.allclose(got[t], want, rtol=0, atol=1e-15)


def test_dispatch_adjoint():
    check_dispatch_adjoint()


def test_dispatch_backward_brute():
    check_dispatch_backward_brute()


_ORIG_EFB = O.expert_ffn_backward
_ORIG_DB = O.dispatch_backward


def _efb_mask_from_dH(u, W1, W2, act, dout, b1=None, W3=None):
    """ReLU derivative gated by dH > 0 instead of A > 0."""
    g = _ORIG_EFB(u, W1, W2, act, dout, b1=b1, W3=W3)
    a = u @ W1.T + (0 if b1 is None else b1)
    dH = dout @ W2
    dA = dH * (dH > 0)
    g.update(du=dA @ W1, dW1=dA.T @ u, db1=dA.sum(0))
    return g


def _efb_sigmoid_for_silu_grad(u, W1, W2, act, dout, b1=None, W3=None):
    """SwiGLU with sigmoid(a) taken as the derivative of silu(a)."""
    g = _ORIG_EFB(u, W1, W2, act, dout, b1=b1, W3=W3)
    a = u @ W1.T
    gg = u @ W3.T
    dH = dout @ W2
    dA = dH * gg / (1 + np.exp(-a))
    dG = dH * O.silu(a)
    g.update(du=dA @ W1 + dG @ W3, dW1=dA.T @ u)
    return g


def _efb_dW2_from_preactivation(u, W1, W2, act, dout, b1=None, W3=None):
    """dW2 from the pre-activation A instead of the hidden activation H."""
    g = _ORIG_EFB(u, W1, W2, act, dout, b1=b1, W3=W3)
    g["dW2"] = dout.T @ (u @ W1.T + (0 if b1 is None else b1))
    return g


def _efb_no_dG_in_du(u, W1, W2, act, dout, b1=None, W3=None):
    """SwiGLU du without the gate partner's path dG W3."""
    g = _ORIG_EFB(u, W1, W2, act, dout, b1=b1, W3=W3)
    a = u @ W1.T
    dA = (dout @ W2) * (u @ W3.T) * O.silu_grad(a)
    g["du"] = dA @ W1
    return g


def _db_keeps_dropped(dxbuf, idx, slot, dx_add=None):
    """Dropped choices read row 0 of their expert instead of nothing."""
    return _ORIG_DB(dxbuf, idx, np.maximum(slot, 0), dx_add)


@pytest.mark.parametrize("repl,check", [
    (_efb_mask_from_dH, lambda: check_expert_backward_finite_differences("relu", True)),
    (_efb_sigmoid_for_silu_grad, lambda: check_expert_backward_finite_differences("swiglu", False)),
    (_efb_dW2_from_preactivation, lambda: check_expert_backward_finite_differences("relu", False)),
    (_efb_no_dG_in_du, lambda: check_expert_backward_finite_differences("swiglu", False)),
])
def test_planted_expert_backward_mistake_is_caught(monkeypatch, repl, check):
    monkeypatch.setattr(O, "expert_ffn_backward", repl)
    with pytest.raises(AssertionError):
        check()


def test_planted_dispatch_backward_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(O, "dispatch_backward", _db_keeps_dropped)
    with pytest.raises(AssertionError):
        check_dispatch_adjoint()


def check_layer_backward_finite_differences(act):
    """The whole layer with the routing held fixed: L = <dy, y>, y = combine of the gated
    expert outputs.  combine_backward -> experts_backward -> dispatch_backward must give the
    central differences of L with respect to x, W1, W2 (and W3, b1, b2), drops included."""
    rng = np.random.default_rng(12)
    T, d, f, E, k, C = 14, 4, 5, 3, 2, 7
    x = rng.normal(size=(T, d))
    W1, W2 = rng.normal(size=(E, f, d)) * 0.5, rng.normal(size=(E, d, f)) * 0.5
    W3 = rng.normal(size=(E, f, d)) * 0.5 if act == "swiglu" else None
    b1 = rng.normal(size=(E, f)) * 0.3 if act == "relu" else None
    b2 = rng.normal(size=(E, d)) * 0.3 if act == "relu" else None
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    slot, drop, _ = O.assign_slots(idx, E, C)
    assert drop.any()
    gate = rng.uniform(0.2, 0.8, size=(T, k))
    dy = rng.normal(size=(T, d))

    def loss(x_=x, W1_=W1, W2_=W2, W3_=W3, b1_=b1, b2_=b2):
        _, out = O.experts_by_slot(x_, idx, slot, E, C, W1_, W2_, act, b1_, b2_, W3_, dtype="f64")
        return float(np.sum(dy * O.combine(gate, drop, out)))

    _, out = O.experts_by_slot(x, idx, slot, E, C, W1, W2, act, b1, b2, W3, dtype="f64")
    _, dout = O.combine_backward(dy, gate, drop, out)
    dybuf = np.zeros((E, C, d))
    for t in range(T):
        for j in range(k):
            if slot[t, j] >= 0:
                dybuf[idx[t, j], slot[t, j]] = dout[t, j]
    g = O.experts_backward(x, idx, slot, E, C, W1, W2, act, dybuf, b1=b1, W3=W3, dtype="f64")
    g["dx"] = O.dispatch_backward(g["dxbuf"], idx, slot)
    h = 1e-6
    for name, arr, gname in [("x_", x, "dx"), ("W1_", W1, "dW1"), ("W2_", W2, "dW2"), ("W3_", W3, "dW3"),
                             ("b1_", b1, "db1"), ("b2_", b2, "db2")]:
        if arr is None:
            continue
        num = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[i] += h
            m[i] -= h
            num[i] = (loss(**{name: p}) - loss(**{name: m})) / (2 * h)
        assert np.allclose(g[gname], num, rtol=1e-6, atol=1e-7), (gname, np.max(np.abs(g[gname] - num)))


@pytest.mark.parametrize("act", ["relu", "swiglu"])
def test_layer_backward_finite_differences(act):
    check_layer_backward_finite_differences(act)


def test_planted_layer_backward_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(O, "dispatch_backward", _db_keeps_dropped)
    with pytest.raises(AssertionError):
        check_layer_backward_finite_differences("relu")
