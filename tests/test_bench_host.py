"""Host logic of bench.py that decides the reported figures (CPU only)."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _entry(kernel, total_ms, launches, M, N, K, flops, nbytes):
    return dict(kernel=kernel, M=M, N=N, K=K, launches=launches, total_ms=total_ms,
                avg_ms=total_ms / launches, flops=flops, bytes=nbytes)


def test_roofline_takes_the_kernel_with_the_largest_summed_time():
    entries = [
        _entry("gemm_f32_dx+k3", 40.0, 2000, 128, 4096, 2048, 1.2174e9, 2.768e7),
        _entry("adamw", 0.2, 20, 1126400, 2, 0, 0.0, 28.0 * 1126400),
        _entry("gemm_f32_fwd+down", 39.0, 2000, 128, 2304, 2048, 1.2164e9, 2.95e7),
    ]
    rl = bench.roofline_of(entries, None)
    assert rl["kernel"] == "gemm_f32_dx+k3" and rl["shape"] == [128, 4096, 2048]
    assert rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s" and rl["peak"] == 157.3
    # 1.2174 GFLOP in 20 us
    assert rl["achieved"] == pytest.approx(1.2174e9 / 20e-6 / 1e12)
    assert rl["frac"] == pytest.approx(rl["achieved"] / 157.3)
    assert rl["avg_us"] == pytest.approx(20.0) and rl["launches"] == 2000


def test_roofline_prices_bf16_products_and_hbm_kernels_against_their_own_peaks():
    bf = bench.roofline_of([_entry("gemm_bf16_fwd", 10.0, 10, 4096, 9728, 2560,
                                   2.0 * 4096 * 9728 * 2560, 1e8)], None)
    assert bf["peak"] == 2516.6 and bf["bound"] == "mfma"
    wq = bench.roofline_of([_entry("gemm_wq_dx", 10.0, 10, 4096, 2560, 9728, 1e12, 1e8)], None)
    assert wq["peak"] == 2516.6
    hb = bench.roofline_of([_entry("k3_v_db", 1.0, 10, 4096, 9728, 32, 0.0, 1.6e8)], None)
    assert hb["bound"] == "hbm" and hb["unit"] == "GB/s" and hb["peak"] == 8000.0
    assert hb["achieved"] == pytest.approx(1.6e8 / 100e-6 / 1e9)


def test_kernel_table_shares_sum_over_the_listed_kernels():
    entries = [_entry("gemm_f32_fwd", 3.0, 3, 64, 64, 64, 5e5, 0.0),
               _entry("reduce", 1.0, 2, 64, 1, 4, 0.0, 4096.0)]
    rows = bench.kernel_table(entries, 4.0)
    assert [r["kernel"] for r in rows] == ["gemm_f32_fwd", "reduce"]
    assert sum(r["share"] for r in rows) == pytest.approx(1.0)
    assert "frac_mfma" in rows[0] and "frac_hbm" in rows[1]


def test_per_label_time_sums_shapes_per_step():
    entries = [_entry("gemm_bf16_fwd", 30.0, 30, 4096, 9728, 2560, 1.0, 0.0),
               _entry("reduce", 5.0, 50, 64, 1, 4, 0.0, 1.0),
               _entry("gemm_bf16_fwd", 10.0, 10, 4096, 2560, 9728, 1.0, 0.0)]
    got = bench.per_label_ms(entries, 10)
    assert list(got) == ["gemm_bf16_fwd", "reduce"]
    assert got["gemm_bf16_fwd"] == pytest.approx(4.0) and got["reduce"] == pytest.approx(0.5)


def test_stored_traffic_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    rec = {"source_sha256": bench.kernel_source_digest(), "copy_factor_fetch": 2.0,
           "copy_factor_write": 1.0,
           "kernels": {"gemm_f32_dx+k3 128x4096x2048": {"fetch_kib": 10.0, "write_kib": 3.0}}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("gemm_f32_dx+k3", [128, 4096, 2048]) == 1024.0 * (10 * 2 + 3)
    assert bench.measured_traffic("gemm_f32_dx+k3", [128, 4096, 1024]) is None
    rec["source_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic("gemm_f32_dx+k3", [128, 4096, 2048]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_trace_summary_groups_dispatches_by_kernel_and_grid(tmp_path):
    hdr = ("Kind,Kernel_Name,Workgroup_Size_X,Workgroup_Size_Y,Workgroup_Size_Z,"
           "Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp\n")
    rows = ["KERNEL_DISPATCH,k_a,256,1,1,2560,1,1,1000,4000\n",
            "KERNEL_DISPATCH,k_a,256,1,1,2560,1,1,5000,6000\n",
            "KERNEL_DISPATCH,k_a,256,1,1,5120,1,1,7000,7500\n",
            "KERNEL_DISPATCH,k_b,64,1,1,64,2,1,0,500\n"]
    (tmp_path / "x_kernel_trace.csv").write_text(hdr + "".join(rows))
    table = bench.summarize_trace(str(tmp_path)).splitlines()
    assert table[2].startswith("| `k_a` | 10x1x1 | 256 | 2 | 0.004 | 2.00 | 1.00 | 3.00 |")
    assert any(l.startswith("| `k_a` | 20x1x1 | 256 | 1 |") for l in table)
    assert any(l.startswith("| `k_b` | 1x2x1 | 64 | 1 | 0.001 | 0.50 |") for l in table)


def test_pmc_summary_averages_each_counter_per_dispatch(tmp_path):
    hdr = "Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
    rows = ["1,k,512,FETCH_SIZE,10\n", "1,k,512,FETCH_SIZE,6\n", "2,k,512,FETCH_SIZE,20\n",
            "3,k,1024,FETCH_SIZE,1\n"]
    (tmp_path / "f_counter_collection.csv").write_text(hdr + "".join(rows))
    table = bench.summarize_pmc(str(tmp_path)).splitlines()
    assert table[0] == "| kernel | grid threads | dispatches | FETCH_SIZE |"
    assert table[2] == "| `k` | 512 | 2 | 18.0 |"
    assert table[3] == "| `k` | 1024 | 1 | 1.0 |"


def test_frozen_flops_of_the_dora_two_slot_step():
    from bwd_adamw_amd import workloads as WL
    # 4 T N K per linear (forward and dX), 36 layers, 2 slots x 2 chunks x 2048 tokens
    assert bench.frozen_flops_per_step(WL.get_config(5)) == 4 * 8192 * 36 * 100925440
