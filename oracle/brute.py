"""Pure-Python brute force of the Switch MoE layer forward (test infrastructure).

A second, independent statement of the same page definitions as `moe`,
written as explicit per-token, per-element loops over Python floats
(IEEE float64), for tiny inputs only.  It shares no helper with `moe`: the
selection is a linear scan with a strict comparison (not a sort), the slot
lists are Python lists as in the capacity-aware dispatch of the CS25
lecture-5 notes, and every dot product is an explicit loop.  Page short
names are those of `oracle.moe`.
"""
from __future__ import annotations

import math
import struct


def _f32(v: float) -> float:
    """Round a Python float to the nearest fp32 value."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def _bf16(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _val(a, dtype):
    """Nested lists of Python floats from an array of storage values."""
    if a is None:
        return None
    if dtype == "bf16":
        if a.ndim == 1:
            return [_bf16(b) for b in a.tolist()]
        return [_val(r, dtype) for r in a]
    return a.astype(float).tolist()


def forward(x, W_r, W1, W2, *, k, cf, alpha, act, dtype, W3=None, b1=None, b2=None,
            b_r=None):
    T = x.shape[0]
    E = W_r.shape[0]
    d = W_r.shape[1]
    f = W1.shape[1]
    X = _val(x, dtype)
    Wr = W_r.astype(float).tolist()
    br = None if b_r is None else b_r.astype(float).tolist()
    W1v = [_val(W1[e], dtype) for e in range(E)]
    W2v = [_val(W2[e], dtype) for e in range(E)]
    W3v = None if W3 is None else [_val(W3[e], dtype) for e in range(E)]
    b1v = None if b1 is None else [_val(b1[e], dtype) for e in range(E)]
    b2v = None if b2 is None else [_val(b2[e], dtype) for e in range(E)]

    logits, probs, choice, gate = [], [], [], []
    for t in range(T):
        # router h = W_r x in fp32 ([SW-GLaM] router equation; fp32 router)
        z = []
        for i in range(E):
            s = 0.0
            for j in range(d):
                s += Wr[i][j] * X[t][j]
            if br is not None:
                s += br[i]
            z.append(_f32(s))
        # softmax ([SW-GLaM] softmax equation)
        m = max(z)
        ex = [math.exp(v - m) for v in z]
        tot = sum(ex)
        p = [v / tot for v in ex]
        # top-k by repeated strict-max scan: the lowest index wins a tie
        chosen = []
        for _ in range(k):
            best = -1
            for i in range(E):
                if i in chosen:
                    continue
                if best < 0 or z[i] > z[best]:
                    best = i
            chosen.append(best)
        # gate: full-softmax probability for k = 1, softmax of kept logits for k >= 2
        if k == 1:
            g = [_f32(p[chosen[0]])]
        else:
            mk = max(z[i] for i in chosen)
            ek = [math.exp(z[i] - mk) for i in chosen]
            sk = sum(ek)
            g = [_f32(v / sk) for v in ek]
        logits.append(z)
        probs.append(p)
        choice.append(chosen)
        gate.append(g)

    # capacity C = cf * k * T / E rounded up (at most T)
    C = min(T, max(0, math.ceil(k * T * cf / E - 1e-9)))

    # capacity-aware dispatch: rank-major, token order, slot lists per expert
    slots = [[] for _ in range(E)]
    slot = [[-1] * k for _ in range(T)]
    drop = [[0] * k for _ in range(T)]
    for j in range(k):
        for t in range(T):
            e = choice[t][j]
            if len(slots[e]) < C:
                slot[t][j] = len(slots[e])
                slots[e].append((t, j))
            else:
                drop[t][j] = 1

    # experts on their slot lists, then gate-weighted combine
    y = [[0.0] * d for _ in range(T)]
    for e in range(E):
        for (t, j) in slots[e]:
            u = X[t]
            h = []
            for n in range(f):
                a = 0.0
                for q in range(d):
                    a += W1v[e][n][q] * u[q]
                if b1v is not None:
                    a += b1v[e][n]
                if act == "relu":
                    h.append(a if a > 0.0 else 0.0)
                else:
                    b = 0.0
                    for q in range(d):
                        b += W3v[e][n][q] * u[q]
                    h.append(a / (1.0 + math.exp(-a)) * b)
            for c in range(d):
                o = 0.0
                for n in range(f):
                    o += W2v[e][c][n] * h[n]
                if b2v is not None:
                    o += b2v[e][c]
                y[t][c] += gate[t][j] * o

    # auxiliary loss alpha * N * sum f_i P_i ([SW-GLaM] "负载均衡")
    cnt = [0] * E
    for t in range(T):
        for j in range(k):
            cnt[choice[t][j]] += 1
    aux = 0.0
    for i in range(E):
        fi = cnt[i] / (k * T)
        Pi = sum(probs[t][i] for t in range(T)) / T
        aux += fi * Pi
    aux *= alpha * E

    return dict(z=logits, p=probs, expert_idx=choice, gate=gate, C=C, slot=slot,
                drop_mask=drop, expert_count=[len(s) for s in slots], route_count=cnt,
                y=y, aux_loss=aux)
