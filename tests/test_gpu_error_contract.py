"""The error contract of the C ABI on the GPU: a call whose arguments are
rejected returns its MOE_ERR_* code and writes nothing.

Every output buffer is a real device allocation filled with a sentinel byte
pattern; each case breaks one argument in a way the entry point rejects
before it enqueues anything (a size past a limit, a misaligned pointer, a
missing weight, a workspace one byte short, a capacity above T, a non-finite
scalar), and afterwards every output still holds the sentinel.  The same
rejections are checked without a GPU, with stand-in addresses, in
tests/test_abi_host.py; here the buffers are real, so a write would show.
"""
import pytest
import torch

from sparse_mixture_experts_argmax_amd import _lib as L

pytestmark = pytest.mark.gpu

SENT = 0xA5
T, d, f, E, k, C = 256, 64, 128, 8, 2, 80


def _buf(n):
    return torch.full((n,), SENT, dtype=torch.uint8, device="cuda")


def _untouched(bufs):
    torch.cuda.synchronize()
    for name, b in bufs.items():
        assert bool((b == SENT).all()), f"{name} was written"


@pytest.fixture(scope="module")
def inputs():
    g = torch.Generator(device="cpu").manual_seed(0)
    return dict(x=torch.randn((T, d), generator=g).to(torch.bfloat16).cuda(),
                W_r=torch.randn((E, d), generator=g).cuda(),
                W1=torch.randn((E, f, d), generator=g).to(torch.bfloat16).cuda(),
                W3=torch.randn((E, f, d), generator=g).to(torch.bfloat16).cuda(),
                W2=torch.randn((E, d, f), generator=g).to(torch.bfloat16).cuda(),
                idx=torch.randint(0, E, (T, k), generator=g, dtype=torch.int32).cuda(),
                slot=torch.zeros((T, k), dtype=torch.int32).cuda(),
                gate=torch.rand((T, k), generator=g).cuda(),
                cnt=torch.full((E,), C, dtype=torch.int32).cuda(),
                ps=torch.rand(E, generator=g).cuda(), rc=torch.full((E,), T * k // E, dtype=torch.int32).cuda(),
                xbuf=torch.randn((E, C, d), generator=g).to(torch.bfloat16).cuda())


def _p(t, off=0):
    return t.data_ptr() + off


FORWARD = [
    ("k above E", dict(k=E + 1), L.MOE_ERR_UNSUPPORTED),
    ("E above 1024", dict(E=1025), L.MOE_ERR_UNSUPPORTED),
    ("d not a multiple of 8", dict(d=60), L.MOE_ERR_INVALID_ARGUMENT),
    ("SwiGLU without W3", dict(act=L.MOE_ACT_SWIGLU), L.MOE_ERR_INVALID_ARGUMENT),
    ("misaligned x", dict(x_off=2), L.MOE_ERR_INVALID_ARGUMENT),
    ("capacity factor 0", dict(cf=0.0), L.MOE_ERR_INVALID_ARGUMENT),
    ("alpha not finite", dict(alpha=float("nan")), L.MOE_ERR_INVALID_ARGUMENT),
    ("workspace one byte short", dict(ws_short=1), L.MOE_ERR_WORKSPACE_TOO_SMALL),
    ("T k at 2^31", dict(T=1 << 30), L.MOE_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("what,case,expect", FORWARD, ids=[c[0] for c in FORWARD])
def test_forward_rejects_without_writing(inputs, what, case, expect):
    i = inputs
    a = dict(T=T, d=d, E=E, k=k, act=L.MOE_ACT_RELU, cf=1.25, alpha=0.01, x_off=0, ws_short=0)
    a.update(case)
    need = L.LIB.moe_workspace_bytes(T, d, f, E, k, C, L.MOE_BF16, L.MOE_ACT_RELU)
    out = dict(y=_buf(T * d * 2), aux=_buf(16), zl=_buf(16), idx=_buf(T * k * 4), gate=_buf(T * k * 4),
               drop=_buf(T * k), ws=_buf(need))
    st = L.LIB.moe_forward(_p(i["x"], a["x_off"]), L.MOE_BF16, _p(i["W_r"]), None, _p(i["W1"]), None, None,
                           _p(i["W2"]), None, a["act"], a["T"], a["d"], f, a["E"], a["k"], a["cf"], a["alpha"],
                           _p(out["y"]), _p(out["aux"]), _p(out["zl"]), _p(out["idx"]), _p(out["gate"]),
                           _p(out["drop"]), _p(out["ws"]), need - a["ws_short"], None)
    assert st == expect
    _untouched(out)


ROUTER = [
    ("k above E", dict(k=E + 1), L.MOE_ERR_UNSUPPORTED),
    ("misaligned logits", dict(lg_off=2), L.MOE_ERR_INVALID_ARGUMENT),
    ("workspace one byte short", dict(ws_short=1), L.MOE_ERR_WORKSPACE_TOO_SMALL),
]


@pytest.mark.parametrize("what,case,expect", ROUTER, ids=[c[0] for c in ROUTER])
def test_router_rejects_without_writing(inputs, what, case, expect):
    i = inputs
    a = dict(k=k, lg_off=0, ws_short=0)
    a.update(case)
    need = L.LIB.moe_router_workspace_bytes(T, d, E, k)
    out = dict(idx=_buf(T * 8 * 4), gate=_buf(T * 8 * 4), ps=_buf(E * 4), rc=_buf(E * 4), zl=_buf(16),
               lg=_buf(T * E * 4 + 16), ws=_buf(need))
    st = L.LIB.moe_router(_p(i["x"]), L.MOE_BF16, _p(i["W_r"]), None, T, d, E, a["k"], _p(out["idx"]),
                          _p(out["gate"]), _p(out["ps"]), _p(out["rc"]), _p(out["zl"]), _p(out["lg"], a["lg_off"]),
                          _p(out["ws"]), need - a["ws_short"], None)
    assert st == expect
    _untouched(out)


def test_noalloc_router_rejects_without_writing(inputs):
    """Sizes past the static scratch array: refused, nothing written."""
    i = inputs
    out = dict(idx=_buf(T * 4), gate=_buf(T * 4), ps=_buf(1024 * 4), rc=_buf(1024 * 4))
    st = L.LIB.moe_router_noalloc(_p(i["x"]), L.MOE_BF16, _p(i["W_r"]), None, 1 << 20, d, 1024, 1,
                                  _p(out["idx"]), _p(out["gate"]), _p(out["ps"]), _p(out["rc"]), None, None, None)
    assert st == L.MOE_ERR_WORKSPACE_TOO_SMALL
    _untouched(out)


def test_dispatch_and_combine_reject_without_writing(inputs):
    i = inputs
    need = L.LIB.moe_dispatch_workspace_bytes(T, E, k)
    out = dict(slot=_buf(T * k * 4), drop=_buf(T * k), cnt=_buf(E * 4), xbuf=_buf(E * C * d * 2), ws=_buf(need))
    # a capacity above T
    st = L.LIB.moe_dispatch(_p(i["x"]), L.MOE_BF16, _p(i["idx"]), T, d, E, k, T + 1, _p(out["slot"]),
                            _p(out["drop"]), _p(out["cnt"]), _p(out["xbuf"]), _p(out["ws"]), need, None)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    # a workspace one byte short
    st = L.LIB.moe_dispatch(_p(i["x"]), L.MOE_BF16, _p(i["idx"]), T, d, E, k, C, _p(out["slot"]),
                            _p(out["drop"]), _p(out["cnt"]), _p(out["xbuf"]), _p(out["ws"]), need - 1, None)
    assert st == L.MOE_ERR_WORKSPACE_TOO_SMALL
    _untouched(out)
    cout = dict(y=_buf(T * d * 2), aux=_buf(16))
    st = L.LIB.moe_combine(_p(i["xbuf"]), L.MOE_BF16, _p(i["idx"]), _p(i["slot"]), _p(i["gate"]), _p(i["ps"]),
                           _p(i["rc"]), T, d, E, k, C, float("inf"), _p(cout["y"]), _p(cout["aux"]), None)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    _untouched(cout)


def test_expert_ffn_and_backward_reject_without_writing(inputs):
    i = inputs
    need = L.LIB.moe_expert_ffn_workspace_bytes(E, C, f, L.MOE_BF16)
    out = dict(ybuf=_buf(E * C * d * 2), ws=_buf(need))
    # W3 given to a ReLU expert
    st = L.LIB.moe_expert_ffn(_p(i["xbuf"]), L.MOE_BF16, _p(i["cnt"]), E, C, d, f, _p(i["W1"]), None, _p(i["W3"]),
                              _p(i["W2"]), None, L.MOE_ACT_RELU, _p(out["ybuf"]), _p(out["ws"]), need, None)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    _untouched(out)
    bneed = L.LIB.moe_expert_ffn_backward_workspace_bytes(E, C, d, f, L.MOE_BF16, L.MOE_ACT_SWIGLU)
    bout = dict(dx=_buf(E * C * d * 2), dW1=_buf(E * f * d * 2), dW3=_buf(E * f * d * 2), dW2=_buf(E * d * f * 2),
                ws=_buf(bneed))
    # SwiGLU with W3 but no dW3
    st = L.LIB.moe_expert_ffn_backward(_p(i["xbuf"]), L.MOE_BF16, _p(i["cnt"]), E, C, d, f, _p(i["W1"]), None,
                                       _p(i["W3"]), _p(i["W2"]), L.MOE_ACT_SWIGLU, _p(i["xbuf"]), _p(bout["dx"]),
                                       _p(bout["dW1"]), None, _p(bout["dW2"]), None, None, _p(bout["ws"]), bneed,
                                       None)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    # a workspace one byte short
    st = L.LIB.moe_expert_ffn_backward(_p(i["xbuf"]), L.MOE_BF16, _p(i["cnt"]), E, C, d, f, _p(i["W1"]), None,
                                       _p(i["W3"]), _p(i["W2"]), L.MOE_ACT_SWIGLU, _p(i["xbuf"]), _p(bout["dx"]),
                                       _p(bout["dW1"]), _p(bout["dW3"]), _p(bout["dW2"]), None, None,
                                       _p(bout["ws"]), bneed - 1, None)
    assert st == L.MOE_ERR_WORKSPACE_TOO_SMALL
    _untouched(bout)
    dout = dict(dx=_buf(T * d * 4))
    st = L.LIB.moe_dispatch_backward(_p(i["xbuf"]), L.MOE_BF16, _p(i["idx"]), _p(i["slot"]), T, d, E, k, T + 1,
                                     None, _p(dout["dx"]), None)
    assert st == L.MOE_ERR_INVALID_ARGUMENT
    _untouched(dout)
