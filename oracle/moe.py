"""Vectorised NumPy oracle of the Switch MoE layer forward (test infrastructure).

Page short names used in citations:
  [CS25-L5]  "Lecture05" -- notes on Stanford CS25 lecture 5, "Scaling
             Transformers through Sparsity" (hqhq1025 ai-course-notes)
  [SW-RES]   "训练稳定性、实验结论与局限 / Training Stability, Results &
             Limitations" (nano-ai.tech, switch-results)
  [SW-GLaM]  "从 Switch Transformer 到 GLaM" (blog.euler0525.cn)
  [CMU-L16]  "第 16 讲 · 混合专家（MoE）" -- notes on CMU 10-423 lecture 16
             (semidirectx.com)

Conventions.  T tokens, d model width, f expert hidden width, E experts
(the pages' N or N_e), k experts per token.  Arrays follow the pages'
orientation h = W_r x and FFN(x) = W_2 sigma(W_1 x): W_r is [E, d],
W1 and W3 are [E, f, d], W2 is [E, d, f].  bf16 arrays arrive as uint16
bit patterns and are widened exactly.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# input decoding
# ---------------------------------------------------------------------------

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values as float64 (bf16 patterns are the top 16 bits of fp32;
    "f64" takes float64 inputs as they are, for the finite-difference pins)."""
    if a is None:
        return None
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# O1 router logits
# ---------------------------------------------------------------------------

def router_logits(x64: np.ndarray, W_r: np.ndarray, b_r: np.ndarray | None = None) -> np.ndarray:
    """h(x) = W_r x for every token, as fp32.

    [SW-GLaM] "Dense Scaling 与 MoE 的核心差异", router equation h(x) = W_r x.
    [CS25-L5] "稳定训练" (selective precision) and [SW-RES] section 2.1: the
    router is computed in float32.  The dot products are accumulated in
    float64 and rounded once to fp32, so this is the correctly rounded fp32
    logit.  The optional per-expert bias b_r is the reading taken here for the
    skewed workload (an additive popularity offset inside the fp32 logit).
    """
    z = x64 @ np.asarray(W_r, dtype=np.float64).T
    if b_r is not None:
        z = z + np.asarray(b_r, dtype=np.float64)[None, :]
    return z.astype(np.float32)


def softplus(a: np.ndarray) -> np.ndarray:
    """log(1 + exp(a)) in float64, without overflow for large a."""
    a = np.asarray(a, dtype=np.float64)
    return np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a)))


def noisy_router_logits(x64: np.ndarray, W_r: np.ndarray, b_r: np.ndarray | None,
                        W_noise: np.ndarray, eps: np.ndarray) -> np.ndarray:
    """Noisy top-k logits H = W_r x (+ b_r) + eps * softplus(W_noise x), as fp32.

    [CMU-L16] section 2.3 (noisy top-k of Shazeer et al.): a learned,
    input-dependent noise scale softplus(W_noise x) times standard normal
    draws eps is added to the router logits before the top-k, so a token
    sometimes goes to a lower choice; W_g and W_noise start at zero.  The
    page's formula image is missing; this is the form of the paper it
    cites.  eps [T, E] is an input (the method's random numbers are passed
    in).  The clean logit and the noise logit are the correctly rounded fp32
    values of router_logits; H is formed from them in float64 and rounded
    once to fp32.  H then takes the place of the logits everywhere
    downstream: softmax, selection, gates, the loss statistics and z-loss.
    """
    z = router_logits(x64, W_r, b_r).astype(np.float64)
    zn = router_logits(x64, W_noise).astype(np.float64)
    return (z + np.asarray(eps, dtype=np.float64) * softplus(zn)).astype(np.float32)


# ---------------------------------------------------------------------------
# O2 softmax
# ---------------------------------------------------------------------------

def softmax(z: np.ndarray) -> np.ndarray:
    """p_i = exp(h_i) / sum_j exp(h_j), in float64 along the last axis.

    [SW-GLaM] "Dense Scaling 与 MoE 的核心差异", softmax equation.  The row
    maximum is subtracted first; the quotient is unchanged by it.
    """
    z64 = np.asarray(z, dtype=np.float64)
    m = np.max(z64, axis=-1, keepdims=True)
    e = np.exp(z64 - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# O3 selection
# ---------------------------------------------------------------------------

def top_k(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest fp32 logits per token, best first, int32.

    [SW-GLaM] "Switch Transformer：把 MoE 做简单": i* = argmax_i p_i(x).
    Softmax is strictly increasing in the logit, so ranking the fp32 logits
    ranks the probabilities without ties that exp rounding could create.
    [CMU-L16] section 2.3: top-k keeps the k largest and sets the rest to
    minus infinity.  Ties go to the lower expert index: the same section
    observes that an all-zero router always picks the lowest-indexed experts.
    A stable sort of -z realises exactly that order.
    """
    order = np.argsort(-np.asarray(z, dtype=np.float32), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


# ---------------------------------------------------------------------------
# O4 gates
# ---------------------------------------------------------------------------

def gates(z: np.ndarray, p: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate of each chosen expert, fp32 [T, k].

    k = 1: the full-softmax probability of the chosen expert
    ([SW-GLaM] "Switch Transformer：把 MoE 做简单", y = p_{i*}(x) E_{i*}(x);
    [CS25-L5] "Switch Layer", gate gathered from the probabilities).
    k >= 2: softmax over the kept logits only, the others being minus
    infinity ([CMU-L16] section 2.3 and its worked example,
    softmax([1.05, 1.6]) -> [0.366, 0.634]).
    """
    T, k = idx.shape
    rows = np.arange(T)[:, None]
    if k == 1:
        return p[rows, idx].astype(np.float32)
    zk = np.asarray(z, dtype=np.float64)[rows, idx]
    return softmax(zk).astype(np.float32)


# ---------------------------------------------------------------------------
# O5 auxiliary load-balancing loss
# ---------------------------------------------------------------------------

def route_count(idx: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, rank) choices of each expert, before capacity."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=E).astype(np.int64)


def aux_loss(p: np.ndarray, idx: np.ndarray, E: int, alpha: float) -> float:
    """L_aux = alpha * N * sum_i f_i P_i.

    [SW-GLaM] "负载均衡": f_i = (1/T) sum_x 1[argmax p(x) = i],
    P_i = (1/T) sum_x p_i(x), L_aux = alpha N sum_i f_i P_i.
    For k > 1 f_i counts every (token, rank) choice and divides by k T, so
    that sum_i f_i = 1 and the uniform value N sum f_i P_i = 1 of [CMU-L16]
    section 4.2 holds for every k (that section calls 0.125 the uniform
    load of 8 experts with k = 2).  Choices are counted before capacity,
    since f_i is defined from the router's argmax.  P_i averages the full
    softmax over all T tokens.
    """
    T, k = idx.shape
    f = route_count(idx, E).astype(np.float64) / (k * T)
    P = np.asarray(p, dtype=np.float64).sum(axis=0) / T
    return float(alpha * E * np.sum(f * P))


def router_z_loss(z: np.ndarray) -> float:
    """The router z-loss: the mean over tokens of the squared log-sum-exp
    of that token's router logits, (1/T) sum_t (log sum_i exp z_ti)^2.

    [CMU-L16] section 4.2 (the two regularisers): the z-loss of Zoph et al.
    (2022) penalises large router logits through their logsumexp squared;
    the section's experiment reports this quantity itself (10.2 falling to
    0.2) and the OLMoE weight 0.001 that multiplies it in the training loss,
    so the value here carries no weight.  The page's formula image is
    missing; the definition is the one its text names.  The logits are the
    fp32 ones of router_logits, widened exactly; the log-sum-exp subtracts
    the row maximum first, which leaves it unchanged.
    """
    z64 = np.asarray(z, dtype=np.float64)
    m = np.max(z64, axis=-1)
    lse = m + np.log(np.sum(np.exp(z64 - m[:, None]), axis=-1))
    return float(np.mean(lse * lse))


# ---------------------------------------------------------------------------
# O6 capacity
# ---------------------------------------------------------------------------

def capacity(T: int, E: int, k: int, cf: float) -> int:
    """Expert capacity C = capacity_factor * k * T / E, rounded up, at most T.

    [SW-GLaM] "Expert Capacity 与 Token Dropping": C = (T/N) x capacity factor.
    [CMU-L16] exercise 3 scales it by k (1.25 x 2 x 1024 / 8 = 320); for k = 1
    both agree.  The pages do not say how a fractional C is rounded; [CS25-L5]
    "Capacity Factor" says that with factor 1 the slots just cover the ideal
    even split, so C is rounded up.  The 1e-9 absorbs the binary error of a
    decimal factor (1.1 * 1000 / 10 is 110, not 110.00000000000001).
    A token cannot pick one expert twice, so C never needs to exceed T.
    """
    c = math.ceil(k * T * cf / E - 1e-9)
    return int(min(T, max(0, c)))


# ---------------------------------------------------------------------------
# O7 slots and drops
# ---------------------------------------------------------------------------

def assign_slots(idx: np.ndarray, E: int, C: int):
    """Capacity slots in token order; overflowing choices are dropped.

    [CS25-L5] "Capacity Factor 与 Token Dropping", capacity-aware dispatch:
    tokens are visited in order and appended to their expert's slot list
    while it holds fewer than C entries; otherwise the token skips the
    expert.  For k > 1, [CMU-L16] section 6.1 places every token's first
    choice before any token's second choice (the GShard rule), so the visit
    is rank-major: rank 0 over all tokens, then rank 1, ...

    Returns slot [T, k] int32 (-1 if dropped), drop [T, k] uint8 and
    expert_count [E] int64 (kept entries per expert).
    """
    T, k = idx.shape
    fill = [0] * E
    slot = np.full((T, k), -1, dtype=np.int32)
    drop = np.zeros((T, k), dtype=np.uint8)
    idx_list = np.asarray(idx).tolist()
    for j in range(k):
        for t in range(T):
            e = idx_list[t][j]
            if fill[e] < C:
                slot[t, j] = fill[e]
                fill[e] += 1
            else:
                drop[t, j] = 1
    return slot, drop, np.asarray(fill, dtype=np.int64)


def priority_order(priority: np.ndarray) -> np.ndarray:
    """Token visit order of priority routing: descending priority, equal
    priorities in token order; NaN scores come last (in token order)."""
    pr = np.asarray(priority, dtype=np.float64)
    nan = np.isnan(pr)
    return np.lexsort((np.arange(pr.shape[0]), np.where(nan, 0.0, -pr), nan))


def assign_slots_priority(idx: np.ndarray, E: int, C: int, priority: np.ndarray):
    """Capacity slots under priority routing; overflowing choices are dropped.

    [CS25-L5], the V-MoE part after "什么是视觉 token": with a capacity
    factor below 1 the tokens are first ranked by importance and the
    high-priority ones take the expert slots, so the capacity becomes a
    budget spent on the most important tokens.  This is the capacity rule of
    assign_slots with the token visit order replaced by priority_order
    (descending score, ties to the lower token index), still rank-major for
    k > 1.  The page leaves the score open (a learned hypothesis); the
    default score is the router's gate of the token's first choice, and any
    fp32 score [T] may be given.

    Returns slot [T, k] int32 (-1 if dropped), drop [T, k] uint8 and
    expert_count [E] int64, as assign_slots.
    """
    T, k = idx.shape
    order = priority_order(priority).tolist()
    fill = [0] * E
    slot = np.full((T, k), -1, dtype=np.int32)
    drop = np.zeros((T, k), dtype=np.uint8)
    idx_list = np.asarray(idx).tolist()
    for j in range(k):
        for t in order:
            e = idx_list[t][j]
            if fill[e] < C:
                slot[t, j] = fill[e]
                fill[e] += 1
            else:
                drop[t, j] = 1
    return slot, drop, np.asarray(fill, dtype=np.int64)


def assign_slots_reroute(pref: np.ndarray, E: int, C: int, stages: int):
    """Top-1 capacity slots with multi-stage re-routing of the overflow.

    [CS25-L5] "“No Token Left Behind”为何没有成功": when a token's top-1 expert
    is full, it is sent to its second choice, then its third, until it gets
    a slot (the page reports that this did not improve the model).  Stage s
    visits the tokens still without a slot in token order and offers each
    its choice of rank s, pref[t, s], filling the experts from where the
    earlier stages left them; a token still unplaced after `stages` stages
    is dropped.  Stage 0 alone is assign_slots with k = 1.

    pref [T, R] int: each token's experts in preference order (the router's
    top-R), stages <= R.  The page only speaks of real choices; an entry
    outside [0, E) is read as no choice at that stage (a list shorter than
    R, padded): the token stays unplaced there and is offered its next
    entry at the next stage.  Returns expert [T] (the expert the token
    landed on, -1 if dropped), slot [T] (-1 if dropped), stage [T] (-1 if
    dropped) and expert_count [E].
    """
    T = pref.shape[0]
    fill = [0] * E
    expert = np.full(T, -1, dtype=np.int32)
    slot = np.full(T, -1, dtype=np.int32)
    stage = np.full(T, -1, dtype=np.int32)
    pl = np.asarray(pref).tolist()
    for s in range(stages):
        for t in range(T):
            if stage[t] >= 0:
                continue
            e = pl[t][s]
            if 0 <= e < E and fill[e] < C:
                expert[t], slot[t], stage[t] = e, fill[e], s
                fill[e] += 1
    return expert, slot, stage, np.asarray(fill, dtype=np.int64)


# ---------------------------------------------------------------------------
# O8 experts
# ---------------------------------------------------------------------------

def relu(a):
    return np.maximum(a, 0.0)


def silu(a):
    """Swish with beta = 1: a * sigmoid(a)."""
    return a / (1.0 + np.exp(-a))


def expert_ffn(u: np.ndarray, W1: np.ndarray, W2: np.ndarray, act: str,
               b1: np.ndarray | None = None, b2: np.ndarray | None = None,
               W3: np.ndarray | None = None) -> np.ndarray:
    """One expert applied to the rows of u (float64).

    ReLU expert: y = W_2 sigma(W_1 x + b) + c ([SW-GLaM] "Dense Scaling 与
    MoE 的核心差异", FFN(x) = W_2 sigma(W_1 x); [CMU-L16] section 2.1 adds
    the biases b and c).  SwiGLU expert: (Swish(x W) * (x V)) W_2 ([CMU-L16]
    section 2.3, Mixtral's expert); the page gives no Swish beta, so beta = 1
    (SiLU), and the Mixtral-shaped workload has no biases.
    Here W1 is [f, d] (W), W3 is [f, d] (V), W2 is [d, f].
    """
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    a = u @ W1.T
    if b1 is not None:
        a = a + np.asarray(b1, dtype=np.float64)[None, :]
    if act == "relu":
        h = relu(a)
    elif act == "swiglu":
        g = u @ np.asarray(W3, dtype=np.float64).T
        h = silu(a) * g
    else:
        raise ValueError(act)
    o = h @ W2.T
    if b2 is not None:
        o = o + np.asarray(b2, dtype=np.float64)[None, :]
    return o


def experts_by_slot(x64, idx, slot, E, C, W1, W2, act, b1=None, b2=None, W3=None,
                    dtype="f32", experts=None, tokens=None):
    """Expert outputs of every kept (token, rank), one batch per expert.

    Returns ybuf [E, C, d] float64 (rows at or beyond an expert's count are
    zero) and out [T, k, d] float64 (zero for dropped choices).
    `experts` limits the work to a subset of experts and `tokens` to a
    subset of tokens (everything else stays zero): the same definitions,
    evaluated on a sample of a workload too large to run whole.
    [CS25-L5] "Capacity Factor": run_batched_experts over the slot lists.
    """
    T, k = idx.shape
    d = x64.shape[1]
    ybuf = np.zeros((E, C, d), dtype=np.float64)
    out = np.zeros((T, k, d), dtype=np.float64)
    todo = range(E) if experts is None else experts
    want = np.ones((T, 1), dtype=bool)
    if tokens is not None:
        want = np.zeros((T, 1), dtype=bool)
        want[np.asarray(tokens), 0] = True
    for e in todo:
        tt, jj = np.nonzero((idx == e) & (slot >= 0) & want)
        if tt.size == 0:
            continue
        order = np.argsort(slot[tt, jj], kind="stable")
        tt, jj = tt[order], jj[order]
        o = expert_ffn(x64[tt], widen(W1[e], dtype), widen(W2[e], dtype), act,
                       None if b1 is None else widen(b1[e], dtype),
                       None if b2 is None else widen(b2[e], dtype),
                       None if W3 is None else widen(W3[e], dtype))
        ybuf[e, slot[tt, jj]] = o
        out[tt, jj] = o
    return ybuf, out


# ---------------------------------------------------------------------------
# O9 combine
# ---------------------------------------------------------------------------

def combine(gate: np.ndarray, drop: np.ndarray, out: np.ndarray) -> np.ndarray:
    """y_t = sum over kept choices of gate_{t,j} * E_{t,j}(x_t), float64.

    [CS25-L5] "Switch Layer": the output is the gate times the expert output;
    [CMU-L16] section 2.3: y = G_0 E_0(x) + G_1 E_1(x).  A dropped choice
    contributes nothing: the token continues on the residual connection,
    which the caller adds ([CS25-L5] "Capacity Factor"; [SW-GLaM] "Expert
    Capacity 与 Token Dropping"; [CMU-L16] section 6.1).  Gates are not
    renormalised after a drop ([CMU-L16] section 6.1: the token is left with
    only its other expert).
    """
    keep = (np.asarray(drop) == 0).astype(np.float64)
    w = np.asarray(gate, dtype=np.float64) * keep
    return np.einsum("tj,tjd->td", w, out)


# ---------------------------------------------------------------------------
# O11 backward of the gate side: combine and router
# ---------------------------------------------------------------------------

def combine_backward(dy: np.ndarray, gate: np.ndarray, drop: np.ndarray, out: np.ndarray):
    """Gradients of y = combine(gate, drop, out) given dL/dy, float64.

    y_t = sum over kept j of g_tj E_tj(x_t) is linear in both factors:
    dL/dg_tj = <dy_t, E_tj(x_t)> and dL/dE_tj = g_tj dy_t for kept
    choices; a dropped choice gets zero for both.  Returns (dgate [T, k],
    dout [T, k, d]).
    """
    keep = (np.asarray(drop) == 0).astype(np.float64)
    dy64 = np.asarray(dy, dtype=np.float64)
    dgate = np.einsum("td,tjd->tj", dy64, np.asarray(out, dtype=np.float64)) * keep
    dout = (np.asarray(gate, dtype=np.float64) * keep)[:, :, None] * dy64[:, None, :]
    return dgate, dout


def router_backward(x64: np.ndarray, W_r: np.ndarray, z: np.ndarray, idx: np.ndarray,
                    dgate: np.ndarray, k: int, alpha: float, z_weight: float):
    """Gradient of the router's part of the loss, with the choices held fixed.

    L = sum_tj dgate_tj g_tj + alpha N sum_i f_i P_i + z_weight z_loss, where
    g are the gates (gates(): the full-softmax probability of the choice for
    k = 1, the softmax over the kept logits for k >= 2), f_i the fraction of
    choices of expert i (a constant: the top-k is not differentiated) and
    P_i the mean probability.  [CMU-L16] exercise 2 (the gradient of the
    balance loss with respect to p_i(x) is N f_i / T, times alpha; f carries
    no gradient); the z-loss as router_z_loss, d/dz_ti of (1/T) lse_t^2 being
    (2/T) lse_t p_ti.  Each path goes through the softmax Jacobian to the
    logits z; then dW_r = dz^T x, db_r = sum_t dz_t and the router's part of
    dx is dz W_r.  All in float64 from the fp32 logits z.

    Returns (dz [T, E], dW_r [E, d], db_r [E], dx [T, d]).
    """
    z64 = np.asarray(z, dtype=np.float64)
    T, E = z64.shape
    p = softmax(z64)
    rows = np.arange(T)[:, None]
    dg = np.asarray(dgate, dtype=np.float64)
    dz = np.zeros((T, E))
    if k == 1:
        e = np.asarray(idx)[:, 0]
        g = p[np.arange(T), e]
        onehot = np.zeros((T, E))
        onehot[np.arange(T), e] = 1.0
        dz += (dg[:, 0] * g)[:, None] * (onehot - p)
    else:
        g = softmax(z64[rows, idx])
        s = np.sum(g * dg, axis=1, keepdims=True)
        np.add.at(dz, (np.broadcast_to(rows, idx.shape), idx), g * (dg - s))
    f = route_count(idx, E).astype(np.float64) / (k * T)
    a = alpha * E * f / T
    dz += p * (a[None, :] - (p @ a)[:, None])
    m = np.max(z64, axis=1)
    lse = m + np.log(np.sum(np.exp(z64 - m[:, None]), axis=1))
    dz += z_weight * (2.0 / T) * lse[:, None] * p
    dW = dz.T @ np.asarray(x64, dtype=np.float64)
    db = dz.sum(axis=0)
    dx = dz @ np.asarray(W_r, dtype=np.float64)
    return dz, dW, db, dx


# ---------------------------------------------------------------------------
# O12 backward of the expert side: the expert FFN and the dispatch
# ---------------------------------------------------------------------------

def silu_grad(a):
    """d/da of a sigmoid(a): sigmoid(a) (1 + a (1 - sigmoid(a)))."""
    sg = 1.0 / (1.0 + np.exp(-a))
    return sg * (1.0 + a * (1.0 - sg))


def expert_ffn_backward(u: np.ndarray, W1: np.ndarray, W2: np.ndarray, act: str, dout: np.ndarray,
                        b1: np.ndarray | None = None, W3: np.ndarray | None = None):
    """Gradients of one expert applied to the rows u, given dL/d(output) `dout`.

    The expert is expert_ffn: ReLU y = W_2 relu(W_1 x + b) + c, or SwiGLU
    y = W_2 (silu(W x) * (V x)) ([SW-GLaM] "Dense Scaling 与 MoE 的核心差异";
    [CMU-L16] sections 2.1 and 2.3).  [CMU-L16] exercise 2 and section 5:
    each expert is an ordinary FFN on the rows routed to it, so its backward
    is the chain rule through the two matrix products and the activation,
    with the hidden pre-activations recomputed from u:
      dH = dout W2;  dW2 = dout^T H;  db2 = sum over rows of dout;
      ReLU:   dA = dH * 1[A > 0];  dW1 = dA^T u;  db1 = sum of dA;  du = dA W1
      SwiGLU: dA = dH * G * silu'(A), dG = dH * silu(A);
              dW1 = dA^T u, dW3 = dG^T u;  du = dA W1 + dG W3
    (A = W1 u + b1, G = W3 u; at A = 0 the ReLU derivative is taken as 0).
    All in float64.  Returns a dict with du [rows, d], dW1 [f, d], dW2 [d, f],
    dW3 [f, d] or None, db1 [f] and db2 [d] (zero when the expert has no bias).
    """
    u = np.asarray(u, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    a = u @ W1.T
    if b1 is not None:
        a = a + np.asarray(b1, dtype=np.float64)[None, :]
    dH = dout @ W2
    out = dict(dW3=None, db2=dout.sum(axis=0))
    if act == "relu":
        h = relu(a)
        dA = dH * (a > 0)
        out["du"] = dA @ W1
    elif act == "swiglu":
        W3 = np.asarray(W3, dtype=np.float64)
        g = u @ W3.T
        h = silu(a) * g
        dA = dH * g * silu_grad(a)
        dG = dH * silu(a)
        out["dW3"] = dG.T @ u
        out["du"] = dA @ W1 + dG @ W3
    else:
        raise ValueError(act)
    out["dW2"] = dout.T @ h
    out["dW1"] = dA.T @ u
    out["db1"] = dA.sum(axis=0)
    return out


def experts_backward(x64, idx, slot, E, C, W1, W2, act, dybuf, b1=None, W3=None, dtype="f32"):
    """expert_ffn_backward for every expert over its kept rows in slot order.

    dybuf [E, C, d]: dL/d(expert output) of every kept (expert, slot) row
    (moe_combine_backward's output: gate times dL/dy of the row's token).
    Returns dxbuf [E, C, d] (rows at or beyond an expert's count are zero),
    dW1, dW2, dW3 (or None), db1 [E, f], db2 [E, d], all float64.
    """
    T, k = idx.shape
    d = x64.shape[1]
    f = np.asarray(W1).shape[1]
    dxbuf = np.zeros((E, C, d))
    g = dict(dW1=np.zeros((E, f, d)), dW2=np.zeros((E, d, f)),
             dW3=None if W3 is None else np.zeros((E, f, d)), db1=np.zeros((E, f)), db2=np.zeros((E, d)))
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & (slot >= 0))
        if tt.size == 0:
            continue
        order = np.argsort(slot[tt, jj], kind="stable")
        tt, jj = tt[order], jj[order]
        sl = slot[tt, jj]
        r = expert_ffn_backward(x64[tt], widen(W1[e], dtype), widen(W2[e], dtype), act,
                                np.asarray(dybuf[e, sl], dtype=np.float64),
                                None if b1 is None else widen(b1[e], dtype),
                                None if W3 is None else widen(W3[e], dtype))
        dxbuf[e, sl] = r["du"]
        for name in ("dW1", "dW2", "db1", "db2"):
            g[name][e] = r[name]
        if W3 is not None:
            g["dW3"][e] = r["dW3"]
    g["dxbuf"] = dxbuf
    return g


def dispatch_backward(dxbuf: np.ndarray, idx: np.ndarray, slot: np.ndarray, dx_add=None) -> np.ndarray:
    """The adjoint of the dispatch: dx_t = sum over kept choices (t, j) of
    dxbuf[e_tj, slot_tj] (+ dx_add_t), float64.

    The dispatch copies x_t to row slot_tj of expert e_tj for each kept
    choice ([SW-GLaM] "All-to-All": tokens travel to their experts and the
    results travel back); its transpose gathers those rows back and adds them
    per token.  A dropped choice received no copy and returns nothing (the
    token's residual path carries it, [CS25-L5] "Capacity Factor").
    dx_add is the router's share of dx (router_backward), added here.
    """
    T, k = idx.shape
    d = dxbuf.shape[2]
    dx = np.zeros((T, d)) if dx_add is None else np.array(dx_add, dtype=np.float64)
    for j in range(k):
        keep = slot[:, j] >= 0
        tt = np.nonzero(keep)[0]
        dx[tt] += dxbuf[idx[tt, j], slot[tt, j]]
    return dx


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def route(x, W_r, b_r, k, dtype):
    """Router half of the layer: logits, probabilities, choices and gates."""
    x64 = widen(x, dtype)
    z = router_logits(x64, W_r, b_r)
    p = softmax(z)
    idx = top_k(z, k)
    g = gates(z, p, idx)
    return x64, z, p, idx, g


def forward(x, W_r, W1, W2, *, k, cf, alpha, act, dtype, W3=None, b1=None, b2=None,
            b_r=None, experts=None, tokens=None):
    """The full layer forward; returns a dict of every intermediate.

    Keys: z (fp32 logits), p (float64 probabilities), expert_idx, gate,
    prob_sum (sum_t p), route_count, C, slot, drop_mask, expert_count,
    ybuf [E, C, d], y [T, d] (float64, MoE branch only), aux_loss, z_loss.
    With `tokens` (or `experts`) given, expert outputs, ybuf and y are only
    evaluated for those tokens (experts); the routing is always complete.
    """
    T = x.shape[0]
    E = W_r.shape[0]
    x64, z, p, idx, g = route(x, W_r, b_r, k, dtype)
    C = capacity(T, E, k, cf)
    slot, drop, count = assign_slots(idx, E, C)
    ybuf, out = experts_by_slot(x64, idx, slot, E, C, W1, W2, act, b1, b2, W3,
                                dtype, experts, tokens)
    y = combine(g, drop, out)
    return dict(z=z, p=p, expert_idx=idx, gate=g, prob_sum=p.sum(axis=0),
                route_count=route_count(idx, E), C=C, slot=slot, drop_mask=drop,
                expert_count=count, ybuf=ybuf, y=y,
                aux_loss=aux_loss(p, idx, E, alpha), z_loss=router_z_loss(z))


def forward_cfg(cfg: dict, experts=None, tokens=None) -> dict:
    """forward() on a dict produced by datagen.make / datagen.random_case."""
    return forward(cfg["x"], cfg["W_r"], cfg["W1"], cfg["W2"], k=cfg["k"], cf=cfg["cf"],
                   alpha=cfg["alpha"], act=cfg["act"], dtype=cfg["dtype"], W3=cfg["W3"],
                   b1=cfg["b1"], b2=cfg["b2"], b_r=cfg["b_r"], experts=experts, tokens=tokens)


def near_tie_tokens(z: np.ndarray, k: int, gap: float = 1e-5) -> np.ndarray:
    """Tokens whose k+1 largest fp32 logits have an adjacent gap below `gap`.

    Such a token's choice can flip under any change of summation order, so
    parity treats its selection as not unique (the exemption that the
    layer's parity rule allows).
    """
    E = z.shape[1]
    kk = min(k + 1, E)
    s = -np.sort(-np.asarray(z, dtype=np.float64), axis=1)[:, :kk]
    if kk < 2:
        return np.zeros(z.shape[0], dtype=bool)
    return np.any((s[:, :-1] - s[:, 1:]) < gap, axis=1)
