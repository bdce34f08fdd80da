"""moe_router_noalloc (the router with the library's static per-GPU scratch
instead of a workspace) against moe_router on the same inputs, through the
C ABI: identical outputs bit for bit, on two calls in a row whose second has
fewer tokens (the scratch keeps the first call's contents), for the MFMA
router (bf16 tokens, E <= 256, the largest workload's router) and the fp32
FMA router (fp32 tokens; E > 256); sizes past the array are refused.
"""
import ctypes

import numpy as np
import pytest
import torch

import datagen
import sparse_mixture_experts_argmax_amd as moe
from sparse_mixture_experts_argmax_amd import _lib as L
from gpu_util import device_inputs, host_bits

pytestmark = pytest.mark.gpu


def _same(a, b):
    for u, v in zip(a, b):
        assert np.array_equal(host_bits(u), host_bits(v))


def _pair(cfg, T):
    t = device_inputs(cfg)
    x = t["x"][:T].contiguous()
    ref = moe.router(x, t["W_r"], k=cfg["k"], b_r=t["b_r"], z_loss=True, logits=True)
    got = moe.router_noalloc(x, t["W_r"], k=cfg["k"], b_r=t["b_r"], z_loss=True, logits=True)
    torch.cuda.synchronize()
    return got, ref


@pytest.mark.parametrize("name,T1,T2", [("many_expert", 32768, 20000), ("zipf_skew", 16384, 1111),
                                        ("mixtral", 8192, 4097)])
def test_noalloc_router_equals_router(name, T1, T2):
    cfg = datagen.make(name, seed=0, with_experts=False)
    print(f"no-alloc router: {name} T={T1} then T={T2}", flush=True)
    for T in (T1, T2):
        got, ref = _pair(cfg, T)
        _same(got, ref)


@pytest.mark.parametrize("dt,E,k", [("f32", 40, 3), ("bf16", 300, 2)])
def test_noalloc_router_other_kernels(dt, E, k):
    cfg = datagen.random_case(seed=31, T=3000, d=64, f=8, E=E, k=k, cf=1.0, dtype=dt, router_bias=True,
                              logit_scale=2.0)
    print(f"no-alloc router: {dt} E={E} k={k}", flush=True)
    for T in (3000, 777):
        got, ref = _pair(cfg, T)
        _same(got, ref)


def test_noalloc_router_refuses_sizes_past_the_array():
    """T = 2^20 tokens of 1024 experts need a larger router workspace than the array."""
    T, d, E = 1 << 20, 64, 1024
    need = L.LIB.moe_router_workspace_bytes(T, d, E, 1)
    assert need > L.LIB.moe_router_noalloc_scratch_bytes()
    x = torch.empty((8, d), dtype=torch.bfloat16, device="cuda")      # never read: refused before launch
    w = torch.empty((8, d), dtype=torch.float32, device="cuda")
    st = L.LIB.moe_router_noalloc(x.data_ptr(), L.MOE_BF16, w.data_ptr(), None, T, d, E, 1, w.data_ptr(),
                                  w.data_ptr(), w.data_ptr(), w.data_ptr(), None, None, None)
    assert st == L.MOE_ERR_WORKSPACE_TOO_SMALL
