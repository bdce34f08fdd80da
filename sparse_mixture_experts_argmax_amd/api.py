"""Python face of the C ABI: torch tensors in, torch tensors out.

Argument marshalling only -- shapes, dtypes, device pointers and the current
HIP stream are passed to libmoe.so, and every step of the layer runs in its
kernels.  Tensors must live on a ROCm device; bf16 layers take torch.bfloat16
x / expert weights, fp32 layers torch.float32; the router weight, its bias
and the gates are always float32.

Layouts (see include/moe.h): x [T, d]; W_r [E, d]; W1, W3 [E, dff, d];
W2 [E, d, dff]; b1 [E, dff]; b2 [E, d]; b_r [E].
"""
from __future__ import annotations

import torch

from . import _lib as L

_ACT = {"relu": L.MOE_ACT_RELU, "swiglu": L.MOE_ACT_SWIGLU}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.MOE_BF16
    if t.dtype == torch.float32:
        return L.MOE_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr() or None


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _same(dtype, *ts):
    for t in ts:
        if t is not None and t.dtype != dtype:
            raise TypeError(f"expected {dtype}, got {t.dtype}")


def _expect(t, name: str, shape: tuple, dtype=None, optional: bool = False):
    """Checks a tensor argument against its layout before anything reaches the
    library: the C ABI receives only sizes, so a tensor of the wrong shape or
    element type would be read past its end or misread."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {list(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _tokens(x, name: str = "x"):
    """x [T, d] in bfloat16 or float32."""
    if x.dim() != 2:
        raise ValueError(f"{name} must be [T, d], got {list(x.shape)}")
    _dtype_code(x)
    return x.shape


def _routing(expert_idx, T: int, name: str = "expert_idx"):
    """[T, k] int32 routing tensor; returns k."""
    if expert_idx.dim() != 2 or expert_idx.shape[0] != T:
        raise ValueError(f"{name} must be [T={T}, k], got {list(expert_idx.shape)}")
    if expert_idx.dtype != torch.int32:
        raise TypeError(f"{name} must be torch.int32, got {expert_idx.dtype}")
    return expert_idx.shape[1]


def _experts(E: int, d: int, dff: int, dtype, W1, W2, W3=None, b1=None, b2=None):
    """Expert weights in the layout [E, dff, d] / [E, d, dff] of the storage dtype."""
    _expect(W1, "W1", (E, dff, d), dtype)
    _expect(W2, "W2", (E, d, dff), dtype)
    _expect(W3, "W3", (E, dff, d), dtype, optional=True)
    _expect(b1, "b1", (E, dff), dtype, optional=True)
    _expect(b2, "b2", (E, d), dtype, optional=True)


def capacity(T: int, E: int, k: int, capacity_factor: float) -> int:
    """C = ceil(capacity_factor * k * T / E), at most T (host arithmetic in the library)."""
    c = L.LIB.moe_capacity(T, E, k, capacity_factor)
    if c < 0:
        raise ValueError("invalid capacity arguments")
    return int(c)


def workspace_bytes(T, d, dff, E, k, C, dtype, act="relu") -> int:
    code = L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32
    n = L.LIB.moe_workspace_bytes(T, d, dff, E, k, C, code, _ACT[act])
    if n == L.SIZE_MAX:
        raise ValueError("invalid sizes")
    return int(n)


def _workspace(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _ws(workspace, nbytes: int, dev) -> torch.Tensor:
    """The caller's workspace (a uint8 tensor: its numel is its size in bytes) or a new one."""
    if workspace is None:
        return _workspace(nbytes, dev)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D torch.uint8 tensor")
    return workspace


def router(x, W_r, k: int = 1, b_r=None, workspace=None, z_loss: bool = False, W_noise=None,
           noise=None, logits: bool = False):
    """Router: returns (expert_idx [T,k] int32, gate [T,k] fp32, prob_sum [E] fp32, route_count [E] int32),
    and with z_loss=True also the router z-loss [1] fp32 (mean over tokens of the squared
    log-sum-exp of the logits).  With W_noise [E,d] fp32 and noise [T,E] fp32 (standard normal
    draws) the noisy top-k router: the logits become W_r x + noise * softplus(W_noise x).
    With logits=True (plain router) the fp32 logits [T, E] are returned last."""
    T, d = _tokens(x)
    if W_r.dim() != 2:
        raise ValueError(f"W_r must be [E, d], got {list(W_r.shape)}")
    E = W_r.shape[0]
    dev = x.device
    _expect(W_r, "W_r", (E, d), torch.float32)
    _expect(b_r, "b_r", (E,), torch.float32, optional=True)
    if (W_noise is None) != (noise is None):
        raise ValueError("the noisy router needs both W_noise and noise")
    _expect(W_noise, "W_noise", (E, d), torch.float32, optional=True)
    _expect(noise, "noise", (T, E), torch.float32, optional=True)
    if not 1 <= k <= E:
        raise ValueError(f"k must be in [1, E={E}], got {k}")
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    prob_sum = torch.empty(E, dtype=torch.float32, device=dev)
    route_count = torch.empty(E, dtype=torch.int32, device=dev)
    zl = torch.empty(1, dtype=torch.float32, device=dev) if z_loss else None
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None
    if logits and W_noise is not None:
        raise ValueError("logits are returned by the plain router only")
    need = L.LIB.moe_router_workspace_bytes(T, d, E, k)
    if need == L.SIZE_MAX:
        raise ValueError("invalid router sizes")
    ws = _ws(workspace, need, dev)
    if W_noise is None:
        L.check("moe_router", L.LIB.moe_router(
            _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), T, d, E, k, _ptr(idx), _ptr(gate),
            _ptr(prob_sum), _ptr(route_count), _ptr(zl), _ptr(lg), _ptr(ws), ws.numel(), _stream(dev)))
    else:
        L.check("moe_router_noisy", L.LIB.moe_router_noisy(
            _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), _ptr(W_noise), _ptr(noise), T, d, E, k,
            _ptr(idx), _ptr(gate), _ptr(prob_sum), _ptr(route_count), _ptr(zl), _ptr(ws), ws.numel(),
            _stream(dev)))
    out = (idx, gate, prob_sum, route_count)
    if z_loss:
        out += (zl,)
    if logits:
        out += (lg,)
    return out


def router_noalloc(x, W_r, k: int = 1, b_r=None, z_loss: bool = False, logits: bool = False):
    """router() through moe_router_noalloc: the library's static per-GPU scratch instead of a
    workspace (for callers that cannot allocate; the outputs are still the caller's).  Returns
    what router() returns for the same flags."""
    T, d = _tokens(x)
    if W_r.dim() != 2:
        raise ValueError(f"W_r must be [E, d], got {list(W_r.shape)}")
    E = W_r.shape[0]
    dev = x.device
    _expect(W_r, "W_r", (E, d), torch.float32)
    _expect(b_r, "b_r", (E,), torch.float32, optional=True)
    if not 1 <= k <= E:
        raise ValueError(f"k must be in [1, E={E}], got {k}")
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    prob_sum = torch.empty(E, dtype=torch.float32, device=dev)
    route_count = torch.empty(E, dtype=torch.int32, device=dev)
    zl = torch.empty(1, dtype=torch.float32, device=dev) if z_loss else None
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None
    L.check("moe_router_noalloc", L.LIB.moe_router_noalloc(
        _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), T, d, E, k, _ptr(idx), _ptr(gate),
        _ptr(prob_sum), _ptr(route_count), _ptr(zl), _ptr(lg), _stream(dev)))
    out = (idx, gate, prob_sum, route_count)
    if z_loss:
        out += (zl,)
    if logits:
        out += (lg,)
    return out


def dispatch(x, expert_idx, E: int, C: int, workspace=None):
    """Dispatch: returns (slot [T,k] int32, drop_mask [T,k] uint8, expert_count [E] int32, xbuf [E,C,d])."""
    T, d = _tokens(x)
    k = _routing(expert_idx, T)
    dev = x.device
    slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    drop = torch.empty((T, k), dtype=torch.uint8, device=dev)
    count = torch.empty(E, dtype=torch.int32, device=dev)
    xbuf = torch.empty((E, C, d), dtype=x.dtype, device=dev)
    need = L.LIB.moe_dispatch_workspace_bytes(T, E, k)
    if need == L.SIZE_MAX:
        raise ValueError("invalid dispatch sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_dispatch", L.LIB.moe_dispatch(
        _ptr(x), _dtype_code(x), _ptr(expert_idx), T, d, E, k, C, _ptr(slot), _ptr(drop),
        _ptr(count), _ptr(xbuf), _ptr(ws), ws.numel(), _stream(dev)))
    return slot, drop, count, xbuf


def dispatch_priority(x, expert_idx, priority, E: int, C: int, workspace=None):
    """Priority dispatch: as dispatch, with the capacity filled in descending
    priority [T] fp32 (ties: lower token index; NaN last), rank-major.
    Returns (slot, drop_mask, expert_count, xbuf)."""
    T, d = _tokens(x)
    k = _routing(expert_idx, T)
    dev = x.device
    _expect(priority, "priority", (T,), torch.float32)
    slot = torch.empty((T, k), dtype=torch.int32, device=dev)
    drop = torch.empty((T, k), dtype=torch.uint8, device=dev)
    count = torch.empty(E, dtype=torch.int32, device=dev)
    xbuf = torch.empty((E, C, d), dtype=x.dtype, device=dev)
    need = L.LIB.moe_dispatch_priority_workspace_bytes(T, E, k)
    if need == L.SIZE_MAX:
        raise ValueError("invalid dispatch sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_dispatch_priority", L.LIB.moe_dispatch_priority(
        _ptr(x), _dtype_code(x), _ptr(expert_idx), _ptr(priority), T, d, E, k, C, _ptr(slot), _ptr(drop),
        _ptr(count), _ptr(xbuf), _ptr(ws), ws.numel(), _stream(dev)))
    return slot, drop, count, xbuf


def dispatch_reroute(x, pref, E: int, C: int, stages: int, logits=None, workspace=None):
    """Top-1 dispatch with re-routing: stage s offers the unplaced tokens their choice pref[:, s].
    Returns (expert [T], slot [T], drop_mask [T], gate [T] or None, expert_count [E], xbuf)."""
    T, d = _tokens(x)
    R = _routing(pref, T, "pref")
    dev = x.device
    if not 1 <= stages <= R:
        raise ValueError(f"stages must be in [1, R={R}], got {stages}")
    _expect(logits, "logits", (T, E), torch.float32, optional=True)
    expert = torch.empty(T, dtype=torch.int32, device=dev)
    slot = torch.empty(T, dtype=torch.int32, device=dev)
    drop = torch.empty(T, dtype=torch.uint8, device=dev)
    gate = torch.empty(T, dtype=torch.float32, device=dev) if logits is not None else None
    count = torch.empty(E, dtype=torch.int32, device=dev)
    xbuf = torch.empty((E, C, d), dtype=x.dtype, device=dev)
    need = L.LIB.moe_dispatch_reroute_workspace_bytes(T, E)
    if need == L.SIZE_MAX:
        raise ValueError("invalid dispatch sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_dispatch_reroute", L.LIB.moe_dispatch_reroute(
        _ptr(x), _dtype_code(x), _ptr(pref), _ptr(logits), T, d, E, R, stages, C, _ptr(expert), _ptr(slot),
        _ptr(drop), _ptr(gate), _ptr(count), _ptr(xbuf), _ptr(ws), ws.numel(), _stream(dev)))
    return expert, slot, drop, gate, count, xbuf


def combine_backward(dy, ybuf, expert_idx, slot, gate, dybuf=None):
    """Combine backward: returns (dgate [T,k] fp32, dybuf [E,C,d]; kept rows written)."""
    if ybuf.dim() != 3:
        raise ValueError(f"ybuf must be [E, C, d], got {list(ybuf.shape)}")
    E, C, d = ybuf.shape
    T = expert_idx.shape[0]
    k = _routing(expert_idx, T)
    dev = dy.device
    _expect(dy, "dy", (T, d), ybuf.dtype)
    _expect(slot, "slot", (T, k), torch.int32)
    _expect(gate, "gate", (T, k), torch.float32)
    _expect(dybuf, "dybuf", (E, C, d), ybuf.dtype, optional=True)
    dgate = torch.empty((T, k), dtype=torch.float32, device=dev)
    if dybuf is None:
        dybuf = torch.zeros_like(ybuf)
    L.check("moe_combine_backward", L.LIB.moe_combine_backward(
        _ptr(dy), _dtype_code(dy), _ptr(ybuf), _ptr(expert_idx), _ptr(slot), _ptr(gate), T, d, E, k, C,
        _ptr(dgate), _ptr(dybuf), _stream(dev)))
    return dgate, dybuf


def router_backward(x, W_r, logits, expert_idx, gate, dgate, route_count, alpha=1e-2, z_weight=0.0,
                    workspace=None):
    """Router backward: returns (dlogits [T,E], dW_r [E,d], db_r [E], dx [T,d]), all fp32."""
    T, d = _tokens(x)
    if W_r.dim() != 2:
        raise ValueError(f"W_r must be [E, d], got {list(W_r.shape)}")
    E = W_r.shape[0]
    k = _routing(expert_idx, T)
    dev = x.device
    _expect(W_r, "W_r", (E, d), torch.float32)
    _expect(logits, "logits", (T, E), torch.float32)
    _expect(gate, "gate", (T, k), torch.float32)
    _expect(dgate, "dgate", (T, k), torch.float32)
    _expect(route_count, "route_count", (E,), torch.int32)
    dz = torch.empty((T, E), dtype=torch.float32, device=dev)
    dW = torch.empty((E, d), dtype=torch.float32, device=dev)
    db = torch.empty(E, dtype=torch.float32, device=dev)
    dx = torch.empty((T, d), dtype=torch.float32, device=dev)
    need = L.LIB.moe_router_backward_workspace_bytes(T, d, E)
    if need == L.SIZE_MAX:
        raise ValueError("invalid router sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_router_backward", L.LIB.moe_router_backward(
        _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(logits), _ptr(expert_idx), _ptr(gate), _ptr(dgate),
        _ptr(route_count), T, d, E, k, alpha, z_weight, _ptr(dz), _ptr(dW), _ptr(db), _ptr(dx), _ptr(ws),
        ws.numel(), _stream(dev)))
    return dz, dW, db, dx


def expert_ffn(xbuf, expert_count, W1, W2, *, W3=None, b1=None, b2=None, act="relu",
               workspace=None, ybuf=None):
    """Grouped expert FFN: returns ybuf [E, C, d] (rows >= expert_count[e] untouched)."""
    if xbuf.dim() != 3 or W1.dim() != 3:
        raise ValueError("xbuf must be [E, C, d] and W1 [E, dff, d]")
    E, C, d = xbuf.shape
    dff = W1.shape[1]
    dev = xbuf.device
    _dtype_code(xbuf)
    _expect(expert_count, "expert_count", (E,), torch.int32)
    _experts(E, d, dff, xbuf.dtype, W1, W2, W3, b1, b2)
    if act == "swiglu" and W3 is None:
        raise ValueError("the SwiGLU expert needs W3")
    _expect(ybuf, "ybuf", (E, C, d), xbuf.dtype, optional=True)
    if ybuf is None:
        ybuf = torch.empty_like(xbuf)
    need = L.LIB.moe_expert_ffn_workspace_bytes(E, C, dff, _dtype_code(xbuf))
    if need == L.SIZE_MAX:
        raise ValueError("invalid expert sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_expert_ffn", L.LIB.moe_expert_ffn(
        _ptr(xbuf), _dtype_code(xbuf), _ptr(expert_count), E, C, d, dff, _ptr(W1), _ptr(b1),
        _ptr(W3), _ptr(W2), _ptr(b2), _ACT[act], _ptr(ybuf), _ptr(ws), ws.numel(), _stream(dev)))
    return ybuf


def expert_ffn_backward(xbuf, expert_count, W1, W2, dybuf, *, W3=None, b1=None, act="relu", bias_grads=False,
                        workspace=None):
    """Expert FFN backward: returns (dxbuf [E, C, d], dW1, dW3 or None, dW2, db1, db2), the weight
    gradients in the weights' layouts and dtype; db1 [E, dff] and db2 [E, d] only with
    bias_grads=True (ReLU), else None.  dxbuf rows >= expert_count[e] are left unwritten."""
    if xbuf.dim() != 3 or W1.dim() != 3:
        raise ValueError("xbuf must be [E, C, d] and W1 [E, dff, d]")
    E, C, d = xbuf.shape
    dff = W1.shape[1]
    dev = xbuf.device
    _dtype_code(xbuf)
    _expect(expert_count, "expert_count", (E,), torch.int32)
    _experts(E, d, dff, xbuf.dtype, W1, W2, W3, b1)
    _expect(dybuf, "dybuf", (E, C, d), xbuf.dtype)
    if act == "swiglu" and W3 is None:
        raise ValueError("the SwiGLU expert needs W3")
    if act == "swiglu" and bias_grads:
        raise ValueError("the SwiGLU expert has no biases")
    dxbuf = torch.empty_like(xbuf)
    dW1 = torch.empty_like(W1)
    dW2 = torch.empty_like(W2)
    dW3 = torch.empty_like(W3) if W3 is not None else None
    db1 = torch.empty((E, dff), dtype=xbuf.dtype, device=dev) if bias_grads else None
    db2 = torch.empty((E, d), dtype=xbuf.dtype, device=dev) if bias_grads else None
    need = L.LIB.moe_expert_ffn_backward_workspace_bytes(E, C, d, dff, _dtype_code(xbuf), _ACT[act])
    if need == L.SIZE_MAX:
        raise ValueError("invalid expert sizes")
    ws = _ws(workspace, need, dev)
    L.check("moe_expert_ffn_backward", L.LIB.moe_expert_ffn_backward(
        _ptr(xbuf), _dtype_code(xbuf), _ptr(expert_count), E, C, d, dff, _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2),
        _ACT[act], _ptr(dybuf), _ptr(dxbuf), _ptr(dW1), _ptr(dW3), _ptr(dW2), _ptr(db1), _ptr(db2), _ptr(ws),
        ws.numel(), _stream(dev)))
    return dxbuf, dW1, dW3, dW2, db1, db2


def dispatch_backward(dxbuf, expert_idx, slot, T: int, dx_add=None, dx=None):
    """Dispatch backward (un-permute): dx [T, d] fp32 = dx_add + the kept rows of dxbuf per token."""
    if dxbuf.dim() != 3:
        raise ValueError(f"dxbuf must be [E, C, d], got {list(dxbuf.shape)}")
    E, C, d = dxbuf.shape
    k = _routing(expert_idx, T)
    dev = dxbuf.device
    _dtype_code(dxbuf)
    _expect(slot, "slot", (T, k), torch.int32)
    _expect(dx_add, "dx_add", (T, d), torch.float32, optional=True)
    _expect(dx, "dx", (T, d), torch.float32, optional=True)
    if dx is None:
        dx = torch.empty((T, d), dtype=torch.float32, device=dev)
    L.check("moe_dispatch_backward", L.LIB.moe_dispatch_backward(
        _ptr(dxbuf), _dtype_code(dxbuf), _ptr(expert_idx), _ptr(slot), T, d, E, k, C, _ptr(dx_add), _ptr(dx),
        _stream(dev)))
    return dx


def combine(ybuf, expert_idx, slot, gate, prob_sum, route_count, T: int, alpha: float = 1e-2):
    """Combine and aux loss: returns (y [T, d], aux_loss [1] fp32)."""
    if ybuf.dim() != 3:
        raise ValueError(f"ybuf must be [E, C, d], got {list(ybuf.shape)}")
    E, C, d = ybuf.shape
    k = _routing(expert_idx, T)
    dev = ybuf.device
    _dtype_code(ybuf)
    _expect(slot, "slot", (T, k), torch.int32)
    _expect(gate, "gate", (T, k), torch.float32)
    _expect(prob_sum, "prob_sum", (E,), torch.float32)
    _expect(route_count, "route_count", (E,), torch.int32)
    y = torch.empty((T, d), dtype=ybuf.dtype, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    L.check("moe_combine", L.LIB.moe_combine(
        _ptr(ybuf), _dtype_code(ybuf), _ptr(expert_idx), _ptr(slot), _ptr(gate), _ptr(prob_sum),
        _ptr(route_count), T, d, E, k, C, alpha, _ptr(y), _ptr(aux), _stream(dev)))
    return y, aux


class ForwardPlan:
    """The fused layer for fixed sizes, with its outputs and workspace allocated once.

    plan = ForwardPlan(T, d, dff, E, k, dtype, act=..., capacity_factor=..., alpha=...)
    y, aux, idx, gate, drop = plan(x, W_r, W1, W2, W3=..., b1=..., b2=..., b_r=...)
    Each call overwrites the same output tensors; plan.z_loss holds the
    router z-loss of the last call.
    """

    def __init__(self, T, d, dff, E, k, dtype, *, act="relu", capacity_factor=1.25, alpha=1e-2,
                 device="cuda"):
        self.T, self.d, self.dff, self.E, self.k = T, d, dff, E, k
        self.dtype, self.act = dtype, act
        self.capacity_factor, self.alpha = float(capacity_factor), float(alpha)
        self.C = capacity(T, E, k, capacity_factor)
        dev = torch.device(device)
        self.device = dev
        self.y = torch.empty((T, d), dtype=dtype, device=dev)
        self.aux = torch.empty(1, dtype=torch.float32, device=dev)
        self.z_loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.expert_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.gate = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.drop_mask = torch.empty((T, k), dtype=torch.uint8, device=dev)
        self.ws = _workspace(workspace_bytes(T, d, dff, E, k, self.C, dtype, act), dev)
        lay = L.WsLayout()
        L.check("moe_forward_workspace_layout", L.LIB.moe_forward_workspace_layout(
            T, d, dff, E, k, self.C, L.MOE_BF16 if dtype == torch.bfloat16 else L.MOE_F32,
            _ACT[act], lay))
        self.layout = lay

    def __call__(self, x, W_r, W1, W2, *, W3=None, b1=None, b2=None, b_r=None, stream=None, W_noise=None,
                 noise=None):
        """With W_noise [E, d] and noise [T, E] (fp32) the router is the noisy top-k one."""
        if tuple(x.shape) != (self.T, self.d) or x.dtype != self.dtype:
            raise ValueError("x does not match the plan")
        T, d, E = self.T, self.d, self.E
        _expect(W_r, "W_r", (E, d), torch.float32)
        _expect(b_r, "b_r", (E,), torch.float32, optional=True)
        _experts(E, d, self.dff, self.dtype, W1, W2, W3, b1, b2)
        if self.act == "swiglu" and W3 is None:
            raise ValueError("the SwiGLU expert needs W3")
        if (W_noise is None) != (noise is None):
            raise ValueError("the noisy router needs both W_noise and noise")
        _expect(W_noise, "W_noise", (E, d), torch.float32, optional=True)
        _expect(noise, "noise", (T, E), torch.float32, optional=True)
        s = stream.cuda_stream if stream is not None else _stream(self.device)
        if W_noise is not None:
            L.check("moe_forward_noisy", L.LIB.moe_forward_noisy(
                _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), _ptr(W_noise), _ptr(noise), _ptr(W1), _ptr(b1),
                _ptr(W3), _ptr(W2), _ptr(b2), _ACT[self.act], self.T, self.d, self.dff, self.E, self.k,
                self.capacity_factor, self.alpha, _ptr(self.y), _ptr(self.aux), _ptr(self.z_loss),
                _ptr(self.expert_idx), _ptr(self.gate), _ptr(self.drop_mask), _ptr(self.ws), self.ws.numel(), s))
            return self.y, self.aux, self.expert_idx, self.gate, self.drop_mask
        L.check("moe_forward", L.LIB.moe_forward(
            _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2),
            _ptr(b2), _ACT[self.act], self.T, self.d, self.dff, self.E, self.k,
            self.capacity_factor, self.alpha, _ptr(self.y), _ptr(self.aux), _ptr(self.z_loss),
            _ptr(self.expert_idx),
            _ptr(self.gate), _ptr(self.drop_mask), _ptr(self.ws), self.ws.numel(), s))
        return self.y, self.aux, self.expert_idx, self.gate, self.drop_mask

    def intermediate(self, name: str) -> torch.Tensor:
        """A view of an intermediate inside the workspace (valid after a call)."""
        lay, T, k, E, C, d = self.layout, self.T, self.k, self.E, self.C, self.d
        es = 2 if self.dtype == torch.bfloat16 else 4
        spec = {
            "slot": (lay.slot, (T, k), torch.int32, 4),
            "expert_count": (lay.expert_count, (E,), torch.int32, 4),
            "route_count": (lay.route_count, (E,), torch.int32, 4),
            "prob_sum": (lay.prob_sum, (E,), torch.float32, 4),
            "xbuf": (lay.xbuf, (E, C, d), self.dtype, es),
            "ybuf": (lay.ybuf, (E, C, d), self.dtype, es),
            "row_tok": (lay.row_tok, (E, C), torch.int32, 4),
        }[name]
        off, shape, dt, sz = spec
        n = 1
        for s in shape:
            n *= s
        return self.ws[off:off + n * sz].view(dt).view(shape)


def forward_policy(x, W_r, W1, W2, *, policy, W3=None, b1=None, b2=None, b_r=None, k=1, capacity_factor=1.25,
                   alpha=1e-2, act="relu", priority=None, stages=2, workspace=None):
    """The whole layer with an overflow policy: policy="priority" (capacity spent on the highest
    priority [T] fp32 first, default each token's first gate) or "reroute" (k = 1; the router's
    top-`stages` choices offered in stages).  Returns (y, aux_loss, z_loss, expert_idx, gate,
    drop_mask); with "reroute" expert_idx [T, 1] is the landing expert (-1 if dropped)."""
    T, d = _tokens(x)
    if W_r.dim() != 2 or W1.dim() != 3:
        raise ValueError("W_r must be [E, d] and W1 [E, dff, d]")
    E = W_r.shape[0]
    dff = W1.shape[1]
    dev = x.device
    pol = {"priority": L.MOE_POLICY_PRIORITY, "reroute": L.MOE_POLICY_REROUTE}.get(policy)
    if pol is None:
        raise ValueError(f"policy must be 'priority' or 'reroute', got {policy!r}")
    _expect(W_r, "W_r", (E, d), torch.float32)
    _expect(b_r, "b_r", (E,), torch.float32, optional=True)
    _experts(E, d, dff, x.dtype, W1, W2, W3, b1, b2)
    _expect(priority, "priority", (T,), torch.float32, optional=True)
    if pol == L.MOE_POLICY_REROUTE and (k != 1 or priority is not None):
        raise ValueError("re-routing is a top-1 policy (k = 1) and takes no priority")
    kk = k
    need = L.LIB.moe_forward_policy_workspace_bytes(T, d, dff, E, kk, capacity_factor, _dtype_code(x), _ACT[act],
                                                    pol, stages)
    if need == L.SIZE_MAX:
        raise ValueError("invalid sizes or policy arguments")
    ws = _ws(workspace, need, dev)
    y = torch.empty((T, d), dtype=x.dtype, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    zl = torch.empty(1, dtype=torch.float32, device=dev)
    idx = torch.empty((T, kk), dtype=torch.int32, device=dev)
    gate = torch.empty((T, kk), dtype=torch.float32, device=dev)
    drop = torch.empty((T, kk), dtype=torch.uint8, device=dev)
    L.check("moe_forward_policy", L.LIB.moe_forward_policy(
        _ptr(x), _dtype_code(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W3), _ptr(W2), _ptr(b2), _ACT[act],
        T, d, dff, E, kk, capacity_factor, alpha, pol, _ptr(priority), stages, _ptr(y), _ptr(aux), _ptr(zl),
        _ptr(idx), _ptr(gate), _ptr(drop), _ptr(ws), ws.numel(), _stream(dev)))
    return y, aux, zl, idx, gate, drop


def forward(x, W_r, W1, W2, *, W3=None, b1=None, b2=None, b_r=None, k=1, capacity_factor=1.25,
            alpha=1e-2, act="relu"):
    """The whole layer: returns (y, aux_loss, expert_idx, gate, drop_mask)."""
    T, d = _tokens(x)
    if W_r.dim() != 2 or W1.dim() != 3:
        raise ValueError("W_r must be [E, d] and W1 [E, dff, d]")
    E = W_r.shape[0]
    dff = W1.shape[1]
    plan = ForwardPlan(T, d, dff, E, k, x.dtype, act=act, capacity_factor=capacity_factor,
                       alpha=alpha, device=x.device)
    return plan(x, W_r, W1, W2, W3=W3, b1=b1, b2=b2, b_r=b_r)
