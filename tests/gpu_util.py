"""Helpers of the GPU parity tests: device copies of the seeded inputs and the
comparison rules.

Comparison rules
  * expert_idx: bit-exact, except tokens whose oracle fp32 logits have an
    adjacent gap below 1e-5 among their k+1 largest ("near ties"); mismatched
    tokens must all be near ties and number fewer than 0.01% of T.
  * slot / drop_mask / expert_count: bit-exact against the oracle's capacity
    assignment re-run on the GPU's own expert_idx (a near-tie flip moves the
    slots of every later token of both experts), and against the oracle's
    directly whenever the indices agree.
  * gates: relative 1e-5 (fp32 softmax over at most 256 terms).
  * y: on tokens whose choices agree; every element within its rounding
    bound (tests/error_bound.py: the bf16 or fp32 rounding steps of the
    kernels applied to the oracle's float64 intermediates), and over the
    rows max-abs 2e-2 and sum|dy| / sum|y_ref| <= 5e-3 (bf16 storage;
    fp32 storage: 1e-5 for both).
  * aux_loss: relative 1e-5 against the oracle's loss on the GPU's choices.
  * z_loss: relative 1e-5 against the oracle's on the same fp32 logits (the
    per-token log-sum-exp is fp32 on the GPU, the sums fp64).
"""
from __future__ import annotations

import numpy as np
import torch

import datagen
from error_bound import check_elementwise, layer_bound  # noqa: F401
from oracle import moe as O

DEV = "cuda:0"

Y_TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-5, 1e-5)}
GATE_RTOL = 1e-5
AUX_RTOL = 1e-5
Z_RTOL = 1e-5
NEAR_TIE_GAP = 1e-5
MAX_TIE_FRACTION = 1e-4


def dev(a, dtype):
    """numpy storage array -> torch tensor on the GPU."""
    if a is None:
        return None
    if dtype == "bf16" and a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host_f64(t: torch.Tensor) -> np.ndarray:
    """fp64 copy; buffers may hold unwritten rows (any bits), which the callers never compare."""
    with np.errstate(invalid="ignore", over="ignore"):
        if t.dtype == torch.bfloat16:
            bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            return datagen.bf16_bits_to_f32(bits).astype(np.float64)
        return t.cpu().numpy().astype(np.float64)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage bits, for bitwise comparisons."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy()
    return t.contiguous().view(torch.int32).cpu().numpy() if t.dtype == torch.float32 else t.cpu().numpy()


def device_inputs(cfg):
    dt = cfg["dtype"]
    return dict(x=dev(cfg["x"], dt), W_r=dev(cfg["W_r"], "f32"), b_r=dev(cfg["b_r"], "f32"),
                W1=dev(cfg["W1"], dt), W3=dev(cfg["W3"], dt), W2=dev(cfg["W2"], dt),
                b1=dev(cfg["b1"], dt), b2=dev(cfg["b2"], dt))


def check_routing(idx_gpu: np.ndarray, gate_gpu: np.ndarray, ref: dict, k: int):
    """Returns the boolean mask of tokens whose choices agree with the oracle."""
    T = idx_gpu.shape[0]
    assert idx_gpu.shape == ref["expert_idx"].shape
    E = ref["z"].shape[1]
    assert idx_gpu.min() >= 0 and idx_gpu.max() < E
    mism = np.any(idx_gpu != ref["expert_idx"], axis=1)
    tie = O.near_tie_tokens(ref["z"], k, NEAR_TIE_GAP)
    assert not np.any(mism & ~tie), f"{int(np.sum(mism & ~tie))} non-tie tokens routed differently"
    assert mism.sum() < max(1.0, MAX_TIE_FRACTION * T) or mism.sum() == 0, \
        f"{int(mism.sum())} near-tie flips out of {T}"
    agree = ~mism
    np.testing.assert_allclose(gate_gpu[agree], ref["gate"][agree], rtol=GATE_RTOL, atol=1e-7)
    return agree


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, rows: np.ndarray, dtype: str, bound: np.ndarray):
    """y on `rows`: each element within `bound` (same shape as y_ref), then the
    layer's norms.  Returns (max-abs error, L1 ratio, largest error / bound)."""
    worst = check_elementwise(y_gpu, y_ref, bound, rows=rows, what="y")
    max_abs, l1 = Y_TOL[dtype]
    a = y_gpu[rows]
    b = y_ref[rows]
    err = np.abs(a - b)
    assert err.max() <= max_abs, f"max-abs {err.max():.3e}"
    denom = np.abs(b).sum()
    ratio = err.sum() / denom if denom > 0 else err.sum()
    assert ratio <= l1, f"mean relative error {ratio:.3e}"
    return float(err.max()), float(ratio), worst


# ---------------------------------------------------------------------------
# Which bf16 grouped-GEMM launches split their last wave of tiles along K.
# A restatement of the library's launch rules (row tile, column tile, the
# split count), used only to check that a test case reaches that path.
# ---------------------------------------------------------------------------

def gemm_row_tile(C: int, act: str) -> int:
    if C >= 512:
        return 256
    if act != "swiglu" and 256 < C <= 320:
        return 320
    if act != "swiglu" and 128 < C <= 192:
        return 192
    return 128


def tail_split_parts(counts, C: int, E: int, act: str, N: int, K: int, gated: bool = False,
                     ncu: int = 256) -> int:
    """Parts per tile of the last wave (1 = no split) of one launch over
    `counts` rows per expert; `act` is the first GEMM's activation (it sets the
    row tile of both), `gated` marks the SwiGLU first GEMM."""
    bm = gemm_row_tile(C, act)
    if C <= bm:
        return 1
    row_tiles = int(sum((int(c) + bm - 1) // bm for c in counts))
    if gated:
        bn = 128
    else:
        mt_est = E * ((C + bm - 1) // bm)
        bn = 256 if mt_est * ((N + 255) // 256) >= 256 else 128
    total = row_tiles * ((N + bn - 1) // bn)
    nk = (K + 63) // 64
    R = total % ncu
    if total == 0 or total >= 32 * ncu or R == 0 or 2 * R > ncu:
        return 1
    ns = min(ncu // R, nk // 8, 2 if total >= 8 * ncu else 8)
    return ns if ns >= 2 else 1
