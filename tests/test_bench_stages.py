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


def test_mfma_by_stage_from_counter_rows(bench, tmp_path):
    """The MFMA pass summary on two made-up launches of the first GEMM: counted
    flops, duration-weighted MfmaUtil, clock per XCD and the fraction of peak."""
    import csv
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    name = "gemm_bf16_kernel<Tile<256, 128, 2, 64, 1, 2, 3, 2>, 2, false, false, false, false>"
    rows = []
    # launch 1: 1 ms, 2.0 GHz on 8 XCDs, 60 % busy, 1.25 TFLOP; launch 2: 3 ms, 1.5 GHz, 70 %
    for did, dur_ns, ghz, util, flops in [(1, 1_000_000, 2.0, 60.0, 1.25e12), (2, 3_000_000, 1.5, 70.0, 3.75e12)]:
        for cname, val in [("GRBM_GUI_ACTIVE", ghz * dur_ns * 8), ("MfmaUtil", util),
                           ("SQ_INSTS_VALU_MFMA_MOPS_BF16", flops / 512)]:
            rows.append(dict(Dispatch_Id=did, Kernel_Name=name, Counter_Name=cname, Counter_Value=val,
                             Start_Timestamp=10, End_Timestamp=10 + dur_ns))
    with open(tmp_path / "m_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        w.writerows(rows)
    with open(tmp_path / "m_agent_info.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow(dict(Agent_Type="CPU", Num_Xcc=0))
        w.writerow(dict(Agent_Type="GPU", Num_Xcc=8))
    m = bench.mfma_by_stage(str(tmp_path))["expert_gemm1"]
    assert m["launches"] == 2
    assert m["flops_per_launch"] == pytest.approx(2.5e12)
    assert m["avg_us"] == pytest.approx(2000.0)
    assert m["mfma_util_pct"] == pytest.approx((60.0 * 1 + 70.0 * 3) / 4)
    assert m["clock_ghz"] == pytest.approx((2.0 * 1 + 1.5 * 3) / 4)
    assert m["frac_of_peak"] == pytest.approx(5.0e12 / 4e-3 / 2.5e15)
