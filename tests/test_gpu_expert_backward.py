"""The expert side of the backward on the GPU (moe_expert_ffn_backward,
moe_dispatch_backward), through the C ABI, against the oracle.

Each expert's gradients (dxbuf rows, dW1, dW2, dW3, db1, db2) are compared
element by element with the oracle's expert_ffn_backward on the GPU's own
inputs (its dispatch rows and dL/d(expert output) rows, exact storage
values), within the rounding bound of tests/error_bound.py; so only the
backward's arithmetic is compared.  Cases: ReLU with and without biases,
SwiGLU, bf16 and fp32, K and N tails, empty and full experts, the 256-row
tiles, and the switch_base and Mixtral-shaped layers at full size fed from
the split forward and moe_combine_backward.  The un-permute is checked
against the oracle's dispatch_backward, with and without the router's dx.
"""
import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from error_bound import U, check_elementwise, expert_backward_bound
from gpu_util import dev, device_inputs, host_bits, host_f64, tail_split_parts
from oracle import moe as O

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1          # a bf16 NaN pattern; fp32 uses its own


def _check_experts(cfg, xbuf, count, dybuf, outs, experts=None):
    """Every output of every (listed) expert against the oracle, within the bound."""
    dxbuf, dW1, dW3, dW2, db1, db2 = outs
    dt = cfg["dtype"]
    xb, dyb = host_f64(xbuf), host_f64(dybuf)
    got = dict(du=host_f64(dxbuf), dW1=host_f64(dW1), dW2=host_f64(dW2),
               dW3=None if dW3 is None else host_f64(dW3), db1=None if db1 is None else host_f64(db1),
               db2=None if db2 is None else host_f64(db2))
    cnt = count.cpu().numpy()
    C = xbuf.shape[1]
    Cp = (C + 63) // 64 * 64
    worst = 0.0
    w = lambda a, e: None if a is None else O.widen(a[e], dt)   # noqa: E731
    for e in (range(cfg["E"]) if experts is None else experts):
        n = int(cnt[e])
        r = O.expert_ffn_backward(xb[e, :n], w(cfg["W1"], e), w(cfg["W2"], e), cfg["act"], dyb[e, :n],
                                  b1=w(cfg["b1"], e), W3=w(cfg["W3"], e))
        b = expert_backward_bound(xb[e, :n], w(cfg["W1"], e), w(cfg["W2"], e), cfg["act"], dyb[e, :n],
                                  b1=w(cfg["b1"], e), W3=w(cfg["W3"], e), store=dt, rows_pad=Cp)
        for name in ("du", "dW1", "dW2", "dW3", "db1", "db2"):
            if got[name] is None or name not in b:
                continue
            g = got[name][e, :n] if name == "du" else got[name][e]
            worst = max(worst, check_elementwise(g, r[name], b[name][1], what=f"{name} of expert {e}"))
    return worst


def _run_backward(cfg, xbuf, count, dybuf, bias_grads):
    t = device_inputs(cfg)
    return moe.expert_ffn_backward(xbuf, count, t["W1"], t["W2"], dybuf, W3=t["W3"], b1=t["b1"], act=cfg["act"],
                                   bias_grads=bias_grads)


SMALL = {
    # name: T, d, f, E, k, cf, dtype, act, bias
    "relu_bias": (900, 64, 96, 6, 1, 1.25, "bf16", "relu", True),
    "relu_tails": (700, 136, 200, 5, 2, 1.0, "bf16", "relu", False),
    "swiglu_tails": (640, 136, 200, 5, 2, 1.25, "bf16", "swiglu", False),
    "big_tiles": (2400, 200, 328, 4, 1, 1.25, "bf16", "relu", True),
    "tiles_320": (19200, 72, 136, 64, 1, 1.0, "bf16", "relu", False),
    "f32_relu_bias": (300, 24, 40, 4, 1, 1.25, "f32", "relu", True),
    "f32_swiglu": (200, 16, 24, 3, 2, 1.5, "f32", "swiglu", False),
    # long K and a last wave of tiles under half the chip: the products over
    # the experts' rows split that wave along K
    "split_swiglu": (1200, 1024, 1536, 4, 2, 1.25, "bf16", "swiglu", False),
    "split_relu": (1200, 1024, 1536, 4, 1, 1.25, "bf16", "relu", True),
}


def _small_inputs(name):
    T, d, f, E, k, cf, dt, act, bias = SMALL[name]
    cfg = datagen.random_case(seed=21, T=T, d=d, f=f, E=E, k=k, cf=cf, dtype=dt, act=act, ffn_bias=bias,
                              logit_scale=3.0)
    C = O.capacity(T, E, k, cf)
    rng = np.random.default_rng(22)
    cnt = rng.integers(0, C + 1, size=E).astype(np.int32)
    cnt[0], cnt[-1] = 0, C                       # an empty and a full expert
    x = O.widen(cfg["x"], dt)
    rows = rng.integers(0, T, size=(E, C))
    xb = x[rows].astype(np.float32)
    dy = (rng.standard_normal((E, C, d)) * 0.01).astype(np.float32)
    if dt == "bf16":
        xb, dy = datagen.f32_to_bf16_bits(xb), datagen.f32_to_bf16_bits(dy)
    return cfg, C, dev(xb, dt), torch.from_numpy(cnt).cuda(), dev(dy, dt)


@pytest.mark.parametrize("name", list(SMALL))
def test_expert_backward_small(name):
    cfg, C, xbuf, count, dybuf = _small_inputs(name)
    print(f"expert backward: {name} E={cfg['E']} C={C} d={cfg['d']} f={cfg['f']} {cfg['dtype']} {cfg['act']}",
          flush=True)
    outs = _run_backward(cfg, xbuf, count, dybuf, bias_grads=cfg["b1"] is not None)
    torch.cuda.synchronize()
    worst = _check_experts(cfg, xbuf, count, dybuf, outs)
    print(f"  largest error / bound {worst:.3f}", flush=True)


def test_expert_backward_leaves_rows_past_the_count():
    """dxbuf rows at or beyond an expert's count are not written."""
    cfg, C, xbuf, count, dybuf = _small_inputs("relu_bias")
    t = device_inputs(cfg)
    dxbuf = torch.full_like(xbuf, 0).view(torch.int16).fill_(SENTINEL).view(xbuf.dtype)
    ws_n = moe.api.L.LIB.moe_expert_ffn_backward_workspace_bytes(cfg["E"], C, cfg["d"], cfg["f"], 1, 0)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    dW1, dW2 = torch.empty_like(t["W1"]), torch.empty_like(t["W2"])
    from sparse_mixture_experts_argmax_amd.api import _ptr, _stream
    L = moe.api.L
    L.check("moe_expert_ffn_backward", L.LIB.moe_expert_ffn_backward(
        _ptr(xbuf), L.MOE_BF16, _ptr(count), cfg["E"], C, cfg["d"], cfg["f"], _ptr(t["W1"]), _ptr(t["b1"]), None,
        _ptr(t["W2"]), L.MOE_ACT_RELU, _ptr(dybuf), _ptr(dxbuf), _ptr(dW1), None, _ptr(dW2), None, None, _ptr(ws),
        ws.numel(), _stream(xbuf.device)))
    torch.cuda.synchronize()
    bits = host_bits(dxbuf)
    cnt = count.cpu().numpy()
    for e in range(cfg["E"]):
        assert (bits[e, cnt[e]:] == np.int16(SENTINEL)).all()


def _layer(cfg, dy_seed=5):
    """The split forward on the GPU, then dL/dy -> combine backward -> expert backward -> router
    backward -> un-permute.  Returns what the checks need."""
    t = device_inputs(cfg)
    C = moe.capacity(cfg["T"], cfg["E"], cfg["k"], cfg["cf"])
    idx, gate, ps, rc, lg = moe.router(t["x"], t["W_r"], k=cfg["k"], b_r=t["b_r"], logits=True)
    slot, drop, cnt, xbuf = moe.dispatch(t["x"], idx, cfg["E"], C)
    ybuf = moe.expert_ffn(xbuf, cnt, t["W1"], t["W2"], W3=t["W3"], b1=t["b1"], b2=t["b2"], act=cfg["act"])
    g = torch.Generator(device="cpu").manual_seed(dy_seed)
    dy = (torch.randn((cfg["T"], cfg["d"]), generator=g) * 0.02).to(t["x"].dtype).cuda()
    dgate, dybuf = moe.combine_backward(dy, ybuf, idx, slot, gate)
    outs = moe.expert_ffn_backward(xbuf, cnt, t["W1"], t["W2"], dybuf, W3=t["W3"], b1=t["b1"], act=cfg["act"],
                                   bias_grads=cfg["b1"] is not None)
    _, _, _, dx_r = moe.router_backward(t["x"], t["W_r"], lg, idx, gate, dgate, rc, alpha=cfg["alpha"])
    dx = moe.dispatch_backward(outs[0], idx, slot, cfg["T"], dx_add=dx_r)
    torch.cuda.synchronize()
    return dict(idx=idx, slot=slot, cnt=cnt, xbuf=xbuf, dybuf=dybuf, outs=outs, dx_r=dx_r, dx=dx)


def _check_unpermute(cfg, L_, experts_checked=None):
    """dx = the router's dx + the kept dxbuf rows: against the oracle's dispatch_backward on
    the GPU's dxbuf, within the fp32 sum's rounding (k + 1 terms)."""
    dxb = host_f64(L_["outs"][0])
    idx, slot = L_["idx"].cpu().numpy(), L_["slot"].cpu().numpy()
    dxr = L_["dx_r"].cpu().numpy().astype(np.float64)
    ref = O.dispatch_backward(dxb, idx, slot, dx_add=dxr)
    mag = O.dispatch_backward(np.abs(dxb), idx, slot, dx_add=np.abs(dxr))
    bound = (cfg["k"] + 1) * U * mag * 1.01
    check_elementwise(L_["dx"].cpu().numpy().astype(np.float64), ref, bound, what="dx")


@pytest.mark.parametrize("name", ["relu_bias", "swiglu_tails", "f32_swiglu"])
def test_layer_backward_small(name):
    T, d, f, E, k, cf, dt, act, bias = SMALL[name]
    cfg = datagen.random_case(seed=23, T=T, d=d, f=f, E=E, k=k, cf=0.7, dtype=dt, act=act, ffn_bias=bias,
                              logit_scale=3.0)
    print(f"layer backward: {name}", flush=True)
    L_ = _layer(cfg)
    assert bool((L_["slot"].cpu().numpy() < 0).any()), "no choice was dropped"
    _check_experts(cfg, L_["xbuf"], L_["cnt"], L_["dybuf"], L_["outs"])
    _check_unpermute(cfg, L_)


@pytest.mark.parametrize("name", ["switch_base", "mixtral"])
def test_layer_backward_full(name):
    cfg = datagen.make(name, seed=0)
    print(f"layer backward at full size: {name}", flush=True)
    L_ = _layer(cfg)
    worst = _check_experts(cfg, L_["xbuf"], L_["cnt"], L_["dybuf"], L_["outs"])
    _check_unpermute(cfg, L_)
    print(f"  largest error / bound {worst:.3f}", flush=True)


def test_dispatch_backward_without_router_share():
    """dx_add = NULL: the kept rows alone; T = 0 writes nothing and succeeds."""
    rng = np.random.default_rng(3)
    T, E, k, C, d = 500, 6, 2, 120, 40
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    slot, drop, _ = O.assign_slots(idx, E, C)
    dxb = datagen.f32_to_bf16_bits(rng.standard_normal((E, C, d)).astype(np.float32))
    gi, gs, gx = torch.from_numpy(idx).cuda(), torch.from_numpy(slot).cuda(), dev(dxb, "bf16")
    dx = moe.dispatch_backward(gx, gi, gs, T)
    torch.cuda.synchronize()
    ref = O.dispatch_backward(O.widen(dxb, "bf16"), idx, slot)
    mag = O.dispatch_backward(np.abs(O.widen(dxb, "bf16")), idx, slot)
    check_elementwise(dx.cpu().numpy().astype(np.float64), ref, k * U * mag * 1.01 + 0.0, what="dx")
    empty = moe.dispatch_backward(gx[:, :0].contiguous(), gi[:0], gs[:0], 0)
    torch.cuda.synchronize()
    assert empty.shape == (0, d)


def test_expert_backward_no_rows():
    """C = 0: nothing to read; every weight and bias gradient is zero."""
    cfg = datagen.random_case(seed=24, T=64, d=32, f=48, E=3, k=1, cf=1.0, dtype="bf16", act="relu", ffn_bias=True)
    t = device_inputs(cfg)
    xbuf = torch.empty((3, 0, 32), dtype=torch.bfloat16, device="cuda")
    count = torch.zeros(3, dtype=torch.int32, device="cuda")
    outs = moe.expert_ffn_backward(xbuf, count, t["W1"], t["W2"], torch.empty_like(xbuf), b1=t["b1"],
                                   bias_grads=True)
    torch.cuda.synchronize()
    for o in (outs[1], outs[3], outs[4], outs[5]):
        assert (o.float() == 0).all()


@pytest.mark.parametrize("name", ["split_swiglu", "split_relu"])
def test_split_cases_reach_the_split(name):
    """Precondition of the split cases: the recomputed pre-activations, dH or dX split
    their last wave of tiles (the products over the experts' rows; act none)."""
    cfg, C, _, count, _ = _small_inputs(name)
    cnt = count.cpu().numpy()
    d, f, E = cfg["d"], cfg["f"], cfg["E"]
    nf = 2 * f if cfg["act"] == "swiglu" else f
    parts = [tail_split_parts(cnt, C, E, "none", f, d), tail_split_parts(cnt, C, E, "none", d, nf)]
    print(f"{name}: counts {cnt.tolist()}, parts per split tile: A/dH {parts[0]}, dX {parts[1]}", flush=True)
    assert max(parts) > 1
