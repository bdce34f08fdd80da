"""bench.py's stage of each kernel name (CPU only): the profile summaries add
kernel times and counter traffic per stage, so a kernel filed under the wrong
stage would move its bytes into another stage's roofline."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,stage", [
    ("router_mfma_kernel<1, 128, false, 2, 0, 64>", "router"),
    ("router_mfma_kernel<4, 64, false, 1, 0, 64>", "router"),
    ("router_mfma_kernel<16, 32, false, 1, 0, 128>", "router"),
    ("router_generic_kernel<false, false>", "router"),
    ("router_mfma_kernel<4, 64, false, 2, 1, 64>", "noisy_router"),
    ("router_mfma_kernel<16, 32, false, 1, 2, 64>", "noisy_router"),
    ("router_generic_kernel<true, true>", "noisy_router"),
    ("router_split_noisy_kernel", "noisy_router"),
    ("router_bwd_dx_kernel", "gate_backward"),
    ("combine_backward_kernel<true>", "gate_backward"),
    ("slot_rank_kernel", "dispatch"),
    ("slot_index_kernel", "dispatch"),
    ("priority_slot_kernel", "priority_dispatch"),
    ("reroute_place_kernel", "reroute_dispatch"),
    ("gemm_bf16_kernel<Tile<256, 128, 2, 64, 1, 2, 0, 0>, 2, false, false, false, false>", "expert_gemm1"),
    ("gemm_bf16_kernel<Tile<256, 256, 2, 64, 1, 2, 0, 0>, 0, false, false, false, false>", "expert_gemm2"),
    ("gemm_f32_kernel<1, true>", "expert_gemm1"),
    ("combine_kernel<true, 2, 4>", "combine"),
])
def test_kernel_stage(bench, name, stage):
    assert bench.kernel_stage(name) == stage
