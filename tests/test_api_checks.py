"""The Python binding rejects tensors that do not match the layouts of the C ABI.

The library receives only pointers and sizes, so a weight of the wrong shape
or an index tensor of the wrong element type would be read past its end or
misread on the device.  Each case here must raise ValueError or TypeError in
the binding, before any library call: the tensors are host tensors, so a
case that got as far as a launch would fail on the device check instead,
with a different message, and the test would notice.
"""
import pytest
import torch

import sparse_mixture_experts_argmax_amd as moe
from sparse_mixture_experts_argmax_amd import api

T, d, f, E, k = 64, 32, 48, 4, 2
bf = torch.bfloat16
f32 = torch.float32
i32 = torch.int32


def _x(dt=bf):
    return torch.zeros((T, d), dtype=dt)


def _w(dt=bf):
    return dict(W1=torch.zeros((E, f, d), dtype=dt), W2=torch.zeros((E, d, f), dtype=dt))


def _idx(kk=k, dt=i32, n=T):
    return torch.zeros((n, kk), dtype=dt)


ROUTER = [
    ("W_r of the wrong width", dict(W_r=torch.zeros((E, d + 8), dtype=f32)), ValueError, "W_r"),
    ("bf16 W_r", dict(W_r=torch.zeros((E, d), dtype=bf)), TypeError, "W_r"),
    ("b_r of the wrong length", dict(b_r=torch.zeros(E + 1, dtype=f32)), ValueError, "b_r"),
    ("noise [E, T]", dict(W_noise=torch.zeros((E, d), dtype=f32), noise=torch.zeros((E, T), dtype=f32)),
     ValueError, "noise"),
    ("W_noise without noise", dict(W_noise=torch.zeros((E, d), dtype=f32)), ValueError, "noise"),
    ("k above E", dict(k=E + 1), ValueError, "k must"),
    ("fp16 tokens", dict(x=torch.zeros((T, d), dtype=torch.float16)), TypeError, "dtype"),
]


@pytest.mark.parametrize("what,over,exc,msg", ROUTER, ids=[c[0] for c in ROUTER])
def test_router_rejects(what, over, exc, msg):
    a = dict(x=_x(), W_r=torch.zeros((E, d), dtype=f32), k=k)
    a.update(over)
    x, W_r = a.pop("x"), a.pop("W_r")
    with pytest.raises(exc, match=msg):
        moe.router(x, W_r, **a)


DISPATCH = [
    ("int64 expert_idx", dict(expert_idx=_idx(dt=torch.int64)), TypeError, "expert_idx"),
    ("expert_idx shorter than T", dict(expert_idx=_idx(n=T - 1)), ValueError, "expert_idx"),
    ("1-D expert_idx", dict(expert_idx=torch.zeros(T, dtype=i32)), ValueError, "expert_idx"),
]


@pytest.mark.parametrize("what,over,exc,msg", DISPATCH, ids=[c[0] for c in DISPATCH])
def test_dispatch_rejects(what, over, exc, msg):
    with pytest.raises(exc, match=msg):
        moe.dispatch(_x(), over["expert_idx"], E, 40)


def test_priority_and_reroute_reject():
    with pytest.raises(ValueError, match="priority"):
        moe.dispatch_priority(_x(), _idx(), torch.zeros(T + 1, dtype=f32), E, 40)
    with pytest.raises(TypeError, match="priority"):
        moe.dispatch_priority(_x(), _idx(), torch.zeros(T, dtype=torch.float64), E, 40)
    with pytest.raises(TypeError, match="pref"):
        moe.dispatch_reroute(_x(), _idx(dt=torch.int64), E, 40, 2)
    with pytest.raises(ValueError, match="stages"):
        moe.dispatch_reroute(_x(), _idx(), E, 40, 3)
    with pytest.raises(ValueError, match="logits"):
        moe.dispatch_reroute(_x(), _idx(), E, 40, 2, logits=torch.zeros((T, E + 1), dtype=f32))


FFN = [
    ("W1 transposed", dict(W1=torch.zeros((E, d, f), dtype=bf)), ValueError, "W1"),
    ("W2 transposed", dict(W2=torch.zeros((E, f, d), dtype=bf)), ValueError, "W2"),
    ("W3 of the wrong width", dict(W3=torch.zeros((E, f + 8, d), dtype=bf), act="swiglu"), ValueError, "W3"),
    ("SwiGLU without W3", dict(act="swiglu"), ValueError, "W3"),
    ("fp32 W2 with bf16 tokens", dict(W2=torch.zeros((E, d, f), dtype=f32)), TypeError, "W2"),
    ("b1 of the wrong length", dict(b1=torch.zeros((E, f + 1), dtype=bf)), ValueError, "b1"),
    ("b2 per expert missing", dict(b2=torch.zeros(d, dtype=bf)), ValueError, "b2"),
    ("int64 expert_count", dict(expert_count=torch.zeros(E, dtype=torch.int64)), TypeError, "expert_count"),
    ("ybuf of another capacity", dict(ybuf=torch.zeros((E, 41, d), dtype=bf)), ValueError, "ybuf"),
]


@pytest.mark.parametrize("what,over,exc,msg", FFN, ids=[c[0] for c in FFN])
def test_expert_ffn_rejects(what, over, exc, msg):
    a = dict(xbuf=torch.zeros((E, 40, d), dtype=bf), expert_count=torch.zeros(E, dtype=i32), **_w())
    a.update(over)
    xbuf, cnt, W1, W2 = a.pop("xbuf"), a.pop("expert_count"), a.pop("W1"), a.pop("W2")
    with pytest.raises(exc, match=msg):
        moe.expert_ffn(xbuf, cnt, W1, W2, **a)


COMBINE = [
    ("slot [T, 1]", dict(slot=_idx(kk=1)), ValueError, "slot"),
    ("fp64 gate", dict(gate=torch.zeros((T, k), dtype=torch.float64)), TypeError, "gate"),
    ("prob_sum of E + 1", dict(prob_sum=torch.zeros(E + 1, dtype=f32)), ValueError, "prob_sum"),
    ("int64 route_count", dict(route_count=torch.zeros(E, dtype=torch.int64)), TypeError, "route_count"),
    ("expert_idx of another T", dict(expert_idx=_idx(n=T + 1)), ValueError, "expert_idx"),
]


@pytest.mark.parametrize("what,over,exc,msg", COMBINE, ids=[c[0] for c in COMBINE])
def test_combine_rejects(what, over, exc, msg):
    a = dict(ybuf=torch.zeros((E, 40, d), dtype=bf), expert_idx=_idx(), slot=_idx(),
             gate=torch.zeros((T, k), dtype=f32), prob_sum=torch.zeros(E, dtype=f32),
             route_count=torch.zeros(E, dtype=i32))
    a.update(over)
    with pytest.raises(exc, match=msg):
        moe.combine(a["ybuf"], a["expert_idx"], a["slot"], a["gate"], a["prob_sum"], a["route_count"], T)


def test_backward_wrappers_reject():
    ybuf = torch.zeros((E, 40, d), dtype=bf)
    with pytest.raises(ValueError, match="dy"):
        moe.combine_backward(torch.zeros((T, d + 8), dtype=bf), ybuf, _idx(), _idx(), torch.zeros((T, k), dtype=f32))
    with pytest.raises(TypeError, match="gate"):
        moe.combine_backward(torch.zeros((T, d), dtype=bf), ybuf, _idx(), _idx(), torch.zeros((T, k), dtype=bf))
    zf = lambda *s: torch.zeros(s, dtype=f32)   # noqa: E731
    with pytest.raises(ValueError, match="logits"):
        moe.router_backward(_x(), zf(E, d), zf(T, E + 1), _idx(), zf(T, k), zf(T, k), torch.zeros(E, dtype=i32))
    with pytest.raises(TypeError, match="route_count"):
        moe.router_backward(_x(), zf(E, d), zf(T, E), _idx(), zf(T, k), zf(T, k), torch.zeros(E, dtype=torch.int64))


PLAN = [
    ("W_r of another E", dict(W_r=torch.zeros((E + 1, d), dtype=f32)), ValueError, "W_r"),
    ("W1 of another dff", dict(W1=torch.zeros((E, f + 8, d), dtype=bf)), ValueError, "W1"),
    ("W2 transposed", dict(W2=torch.zeros((E, f, d), dtype=bf)), ValueError, "W2"),
    ("fp32 W1", dict(W1=torch.zeros((E, f, d), dtype=f32)), TypeError, "W1"),
    ("b_r fp16", dict(b_r=torch.zeros(E, dtype=torch.float16)), TypeError, "b_r"),
    ("noise [T, E + 1]", dict(W_noise=torch.zeros((E, d), dtype=f32), noise=torch.zeros((T, E + 1), dtype=f32)),
     ValueError, "noise"),
]


@pytest.mark.parametrize("what,over,exc,msg", PLAN, ids=[c[0] for c in PLAN])
def test_forward_plan_rejects(what, over, exc, msg):
    plan = moe.ForwardPlan(T, d, f, E, k, bf, act="relu", device="cpu")
    a = dict(W_r=torch.zeros((E, d), dtype=f32), **_w())
    a.update(over)
    W_r, W1, W2 = a.pop("W_r"), a.pop("W1"), a.pop("W2")
    with pytest.raises(exc, match=msg):
        plan(_x(), W_r, W1, W2, **a)


def test_workspace_must_be_bytes():
    with pytest.raises(TypeError, match="workspace"):
        api._ws(torch.zeros(16, dtype=f32), 64, "cpu")


def test_forward_policy_rejects():
    a = dict(W_r=torch.zeros((E, d), dtype=f32), **_w())
    with pytest.raises(ValueError, match="policy"):
        moe.forward_policy(_x(), a["W_r"], a["W1"], a["W2"], policy="bogus")
    with pytest.raises(ValueError, match="top-1"):
        moe.forward_policy(_x(), a["W_r"], a["W1"], a["W2"], policy="reroute", k=2)
    with pytest.raises(ValueError, match="priority"):
        moe.forward_policy(_x(), a["W_r"], a["W1"], a["W2"], policy="priority", k=2,
                           priority=torch.zeros(T + 1, dtype=f32))
