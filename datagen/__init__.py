"""Seeded synthetic inputs for the Switch MoE layer forward.

This module only draws inputs: random activations and weights, the
LayerNorm that the activations pass through before the layer, the zipf
popularity bias of the skewed workload and the round-to-nearest-even
storage rounding to bfloat16.  It holds none of the layer's own arithmetic
(router, softmax, selection, capacity, experts, combine, loss), so the CPU
oracle and the HIP path can both consume it without sharing any of that.

Workload shapes follow the pages: a Switch-Base-shaped layer (T5-Base
width, 64 experts, "Switch Transformer" results page, section 3.2 / 3.3),
a Mixtral-shaped top-2 SwiGLU layer (CMU 10-423 lecture 16 notes, section
2.3 and exercise 1), and the reduced truncated-normal initialisation
sigma = sqrt(s / fan_in) with s = 0.1 ("Switch Transformer" results page,
section 2.2).

Random streams: every tensor is drawn from independent PCG64 streams keyed
by (seed, tensor id, chunk), one chunk per expert for weights and per 1024
rows for activations.  This makes generation parallel and lets a run with
fewer tokens see exactly the first rows of the full-size activations.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

# beta of the skewed workload: router bias b_r[i] = beta * log(p_i) with
# p_i proportional to (i+1)^-1.1.  Calibrated once by
# datagen/calibrate_zipf.py (which routes with the oracle) so that 15% of
# the seed-0 tokens overflow at capacity factor 1.0.
ZIPF_S = 1.1
ZIPF_BETA = 0.0327

CONFIGS = {
    # Tiny Switch layer, fp32 throughout, ReLU experts with biases.
    "tiny": dict(T=512, d=64, f=256, E=8, k=1, cf=1.25, dtype="f32",
                 act="relu", ffn_bias=True, router_bias=None, alpha=1e-2),
    # Switch-Base-shaped layer (32 sequences x 512 tokens, 64 experts).
    "switch_base": dict(T=16384, d=768, f=3072, E=64, k=1, cf=1.25, dtype="bf16",
                        act="relu", ffn_bias=False, router_bias=None, alpha=1e-2),
    # Skewed-load stress: zipf-biased router, capacity factor 1.0.
    "zipf_skew": dict(T=16384, d=768, f=3072, E=128, k=1, cf=1.0, dtype="bf16",
                      act="relu", ffn_bias=False, router_bias="zipf", alpha=1e-2),
    # Mixtral-shaped top-2 SwiGLU layer.
    "mixtral": dict(T=8192, d=4096, f=14336, E=8, k=2, cf=1.25, dtype="bf16",
                    act="swiglu", ffn_bias=False, router_bias=None, alpha=1e-2),
    # Many-expert layer: 256 experts, about 2.1e9 expert parameters.
    "many_expert": dict(T=32768, d=1024, f=4096, E=256, k=1, cf=1.25, dtype="bf16",
                        act="relu", ffn_bias=False, router_bias=None, alpha=1e-2),
}

# order of the five workloads as they are numbered elsewhere
CONFIG_ORDER = ["tiny", "switch_base", "zipf_skew", "mixtral", "many_expert"]

_TENSOR_ID = {"x": 1, "W_r": 2, "W1": 3, "W3": 4, "W2": 5, "b1": 6, "b2": 7}
_ROWS_PER_CHUNK = 1024
_S_INIT = 0.1  # reduced initialisation scale


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, name: str, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), _TENSOR_ID[name], int(chunk)])))


def _truncated_normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """N(0, sigma^2) restricted to +-2 sigma by redrawing the tail."""
    z = rng.standard_normal(shape)
    bad = np.abs(z) > 2.0
    while bad.any():
        z[bad] = rng.standard_normal(int(bad.sum()))
        bad = np.abs(z) > 2.0
    return z * sigma


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are always finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to fp32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    return a32 if dtype == "f32" else f32_to_bf16_bits(a32)


def _weights(seed, name, E, rows, cols, fan_in, dtype, pool):
    """One [rows, cols] truncated-normal matrix per expert, stacked to [E, rows, cols]."""
    sigma = math.sqrt(_S_INIT / fan_in)
    out = np.empty((E, rows, cols), dtype=np.float32 if dtype == "f32" else np.uint16)

    def one(e):
        out[e] = _store(_truncated_normal(_rng(seed, name, e), (rows, cols), sigma), dtype)

    list(pool.map(one, range(E)))
    return out


def _activations(seed, T, d, dtype, pool):
    """x ~ N(0,1)[T,d], then LayerNorm over d (eps 1e-5, no affine)."""
    out = np.empty((T, d), dtype=np.float32 if dtype == "f32" else np.uint16)
    nchunk = (T + _ROWS_PER_CHUNK - 1) // _ROWS_PER_CHUNK

    def one(c):
        r0 = c * _ROWS_PER_CHUNK
        r1 = min(T, r0 + _ROWS_PER_CHUNK)
        z = _rng(seed, "x", c).standard_normal((_ROWS_PER_CHUNK, d))[: r1 - r0]
        mu = z.mean(axis=1, keepdims=True)
        var = ((z - mu) ** 2).mean(axis=1, keepdims=True)
        out[r0:r1] = _store((z - mu) / np.sqrt(var + 1e-5), dtype)

    list(pool.map(one, range(nchunk)))
    return out


def zipf_log_popularity(E: int, s: float = ZIPF_S) -> np.ndarray:
    """log p_i for p_i proportional to (i+1)^-s, expert 0 the most popular."""
    w = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    return np.log(w / w.sum())


def make(name: str, seed: int = 0, T: int | None = None, beta: float | None = None,
         with_experts: bool = True) -> dict:
    """Draw the inputs of workload `name`.

    Returns a dict with the config fields and the arrays
      x   [T, d]     fp32 or bf16 bits (uint16)
      W_r [E, d]     fp32                     (h = W_r x)
      b_r [E]        fp32 or None             (skewed workload only)
      W1  [E, f, d]  expert dtype             (first layer, [out, in])
      W3  [E, f, d]  expert dtype or None     (SwiGLU gate partner)
      W2  [E, d, f]  expert dtype             (second layer, [out, in])
      b1  [E, f], b2 [E, d]  or None          (tiny workload only)
    `T` overrides the token count (the first T rows of the full draw).
    `with_experts=False` skips the expert weights (routing-only studies).
    """
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg["seed"] = seed
    if T is not None:
        cfg["T"] = int(T)
    Tn, d, f, E, dt = cfg["T"], cfg["d"], cfg["f"], cfg["E"], cfg["dtype"]
    with ThreadPoolExecutor(_threads()) as pool:
        cfg["x"] = _activations(seed, Tn, d, dt, pool)
        cfg["W_r"] = _weights(seed, "W_r", 1, E, d, d, "f32", pool)[0]
        cfg["b_r"] = None
        if cfg["router_bias"] == "zipf":
            b = ZIPF_BETA if beta is None else beta
            cfg["b_r"] = (b * zipf_log_popularity(E)).astype(np.float32)
        cfg["W1"] = cfg["W3"] = cfg["W2"] = cfg["b1"] = cfg["b2"] = None
        if with_experts:
            cfg["W1"] = _weights(seed, "W1", E, f, d, d, dt, pool)
            if cfg["act"] == "swiglu":
                cfg["W3"] = _weights(seed, "W3", E, f, d, d, dt, pool)
            cfg["W2"] = _weights(seed, "W2", E, d, f, f, dt, pool)
            if cfg["ffn_bias"]:
                cfg["b1"] = _weights(seed, "b1", 1, E, f, d, dt, pool)[0]
                cfg["b2"] = _weights(seed, "b2", 1, E, d, f, dt, pool)[0]
    return cfg


def random_case(seed: int, T: int, d: int, f: int, E: int, k: int, cf: float,
                dtype: str = "f32", act: str = "relu", ffn_bias: bool = False,
                router_bias: bool = False, alpha: float = 1e-2,
                logit_scale: float = 1.0) -> dict:
    """Small free-form case for tests (same init recipe, any shape).

    `logit_scale` multiplies W_r so that routing can be made more or less
    peaked (a large scale forces overflow with small capacity factors).
    """
    cfg = dict(T=T, d=d, f=f, E=E, k=k, cf=cf, dtype=dtype, act=act,
               ffn_bias=ffn_bias, router_bias="rand" if router_bias else None,
               alpha=alpha, name="random", seed=seed)
    with ThreadPoolExecutor(1) as pool:
        cfg["x"] = _activations(seed, T, d, dtype, pool)
        W_r = _weights(seed, "W_r", 1, E, d, d, "f32", pool)[0]
        cfg["W_r"] = (W_r * np.float32(logit_scale)).astype(np.float32)
        cfg["b_r"] = None
        if router_bias:
            cfg["b_r"] = _weights(seed + 7919, "b1", 1, 1, E, 1, "f32", pool)[0, 0] * np.float32(3.0)
        cfg["W1"] = _weights(seed, "W1", E, f, d, d, dtype, pool)
        cfg["W3"] = _weights(seed, "W3", E, f, d, d, dtype, pool) if act == "swiglu" else None
        cfg["W2"] = _weights(seed, "W2", E, d, f, f, dtype, pool)
        cfg["b1"] = cfg["b2"] = None
        if ffn_bias:
            cfg["b1"] = _weights(seed, "b1", 1, E, f, d, dtype, pool)[0]
            cfg["b2"] = _weights(seed, "b2", 1, E, d, f, dtype, pool)[0]
    return cfg
