"""Host logic of bench.py that runs without a GPU: the percentile helper and
the oracle CPU baseline (timing, the single-thread run, and its parity check
of a planted output), on small stand-in jobs with CPU tensors."""
from __future__ import annotations

import types

import numpy as np
import pytest
import torch

import bench
import oracle
import workloads
from oracle import compare


def test_percentiles():
    d = [float(i) for i in range(1, 12)]          # 1..11
    assert bench.pct(d, 10) == 2.0 and bench.pct(d, 50) == 6.0 and bench.pct(d, 90) == 10.0
    assert bench.pct([3.0], 10) == 3.0 and bench.pct([3.0], 90) == 3.0
    assert bench.pct(list(reversed(d)), 0) == 1.0 and bench.pct(d, 100) == 11.0


def _job(name, op, dt, M, N, data, y_bits, eps=0.0):
    w = types.SimpleNamespace(name=name, op=op, dt=dt, M=M, N=N, eps=eps, elem_bytes=workloads.ELEM_BYTES[dt])
    if dt == "f32":
        y = torch.from_numpy(np.ascontiguousarray(y_bits).view(np.float32))
    else:
        y = torch.from_numpy(np.ascontiguousarray(y_bits).view(np.int16)).view(
            torch.float16 if dt == "f16" else torch.bfloat16)
    bytes_ = 2 * M * N * w.elem_bytes
    return types.SimpleNamespace(w=w, data=data, y=[y], bytes=bytes_)


def _jobs(plant=False, row=16):
    rng = np.random.default_rng(5)
    x1 = workloads.encode(rng.standard_normal((64, 781)), "f32")
    y1 = compare.round_to(oracle.softmax(x1, "f32"), "f32")
    x2 = workloads.encode(rng.standard_normal((32, 512)), "bf16")
    w2 = workloads.encode(1.0 + 0.3 * rng.standard_normal(512), "bf16")
    y2 = compare.round_to(oracle.rmsnorm(x2, "bf16", 1e-6, weight=w2), "bf16")
    if plant:                                       # a wrong element on a checked row
        y2 = y2.copy()
        y2[row, 7] ^= np.uint16(0x0040)
    return [_job("small_softmax", "softmax", "f32", 64, 781, {"x": x1}, y1),
            _job("small_rmsnorm", "rmsnorm", "bf16", 32, 512, {"x": x2, "weight": w2}, y2, eps=1e-6)]


def test_cpu_baseline_fields():
    n = oracle.num_threads()
    r = bench.cpu_baseline(_jobs(), np)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s" and r["value"] > 0
    assert r["cores"] == n and oracle.num_threads() == n          # thread count restored
    assert r["gpu_parity_on_sample"] is True
    st = r["single_thread"]
    assert st["workload"] == "small_softmax" and st["seconds"] > 0 and st["GBps"] > 0
    assert "cpu_model" in r


def test_cpu_baseline_sees_planted_error():
    assert bench.cpu_baseline(_jobs(plant=True), np)["gpu_parity_on_sample"] is False
    # every row is checked, not a sample of them
    for row in (1, 5, 31):
        r = bench.cpu_baseline(_jobs(plant=True, row=row), np)
        assert r["gpu_parity_on_sample"] is False and r["gpu_parity_rows_checked"] == 64 + 32


def test_kernels_summary_groups_and_scales(tmp_path):
    """rocprof_summary's per-kernel mode on synthetic counter files: the
    calibration copy fixes the scale factors, a group's bytes are the sum of
    its kernels', and the ratio is to the algorithmic bytes given."""
    import csv
    from row_wise_reductions_amd import rocprof_summary as rs

    def counters(d, counter, rows):
        d.mkdir(parents=True)
        with open(d / "x_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for name, v in rows:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})

    kib = 1 << 20          # 1 GiB in KiB
    counters(tmp_path / "cf", "FETCH_SIZE", [(rs.CALIB_KERNEL, kib / 2)])      # fetch counts half: factor 2
    counters(tmp_path / "cw", "WRITE_SIZE", [(rs.CALIB_KERNEL, kib)])          # factor 1
    counters(tmp_path / "f", "FETCH_SIZE", [("ntk::alpha<1>", 100.0), ("ntk::alpha<1>", 300.0), ("ntk::beta<2>", 50.0)])
    counters(tmp_path / "w", "WRITE_SIZE", [("ntk::alpha<1>", 10.0), ("ntk::beta<2>", 400.0)])
    (tmp_path / "t").mkdir()
    with open(tmp_path / "t" / "x_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs"])
        w.writeheader()
        w.writerow({"Name": "ntk::alpha<1>", "Calls": 2, "AverageNs": 1000})
        w.writerow({"Name": "ntk::beta<2>", "Calls": 1, "AverageNs": 3000})
    cmds = tmp_path / "cmds.txt"
    cmds.write_text("cmd one\ncmd two\n")
    md = tmp_path / "out.md"
    args = types.SimpleNamespace(fetch=str(tmp_path / "f"), write=str(tmp_path / "w"), calib_fetch=str(tmp_path / "cf"),
                                 calib_write=str(tmp_path / "cw"), trace=str(tmp_path / "t"),
                                 groups="both=alpha+beta;first=alpha", bytes=2048 * 1024, title="T",
                                 cmds=str(cmds), md=str(md))
    rs.kernels(args)
    text = md.read_text()
    # alpha: fetch mean 200 KiB x 2 + write 10 KiB = 410 KiB; beta: 50 x 2 + 400 = 500 KiB
    assert "| both | 931840 | 0.444 | 4.00 |" in text
    assert "| first | 419840 | 0.200 | 1.00 |" in text
    assert "    cmd one" in text


def test_requests_summary_counts_lines(tmp_path):
    """rocprof_summary's L2 request mode on synthetic counter files: reads
    count as 128-byte lines, writes at 64 or 32 bytes, per call summed over
    the workload's kernels, beside its algorithmic bytes."""
    import csv
    from row_wise_reductions_amd import rocprof_summary as rs

    def counters(d, rows):
        d.mkdir(parents=True)
        with open(d / "x_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for name, vals in rows:
                for c, v in vals.items():
                    w.writerow({"Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})

    zero = {c: 0 for c in rs.REQ_COUNTERS}
    lines = (1 << 30) // 128
    cal = dict(zero, TCC_EA0_RDREQ_sum=lines, TCC_EA0_RDREQ_DRAM_sum=lines, TCC_EA0_WRREQ_sum=2 * lines,
               TCC_EA0_WRREQ_64B_sum=2 * lines, TCC_MISS_sum=3 * lines)
    counters(tmp_path / "c", [(rs.CALIB_KERNEL, cal)])
    w = workloads.BY_NAME["layernorm_f16_4096"]
    k = rs.kernels_of(w)
    assert len(k) == 1
    alg = w.algorithmic_bytes()
    rd = dict(zero, TCC_EA0_RDREQ_sum=1000, TCC_EA0_RDREQ_32B_sum=0, TCC_EA0_WRREQ_sum=3000,
              TCC_EA0_WRREQ_64B_sum=2000, TCC_HIT_sum=1, TCC_MISS_sum=3)
    counters(tmp_path / "r", [("void " + k[0] + "(ntk::RowArgs)", rd)])
    cmds = tmp_path / "cmds.txt"
    cmds.write_text("cmd one\n")
    md = tmp_path / "out.md"
    rs.requests(types.SimpleNamespace(runs=str(tmp_path / "r"), calib=str(tmp_path / "c"), cmds=str(cmds), md=str(md)))
    text = md.read_text()
    assert "(x 128 B = 1.0000 GiB)" in text and "write requests 16777216 (1.0000 GiB)" in text
    assert f"| calibration copy 1 GiB | {lines} | 0 | {lines} | {2 * lines} |" in text
    # 1000 x 128 read + 2000 x 64 + 1000 x 32 written = 288000 bytes
    assert f"| layernorm_f16_4096 | 1000 | 0 | 0 | 3000 | 2000 | 0 | 0.250 | 128000 | 160000 | {alg} | " in text
    assert "    cmd one" in text


def test_waves_summary_pairs_kernel_and_copy(tmp_path):
    """rocprof_summary's wave mode on a synthetic counter file: each
    workload's kernel beside the one-chunk copy at its size (told apart from
    other copies by grid), cycles per wave and the shares of them."""
    import csv
    from row_wise_reductions_amd import rocprof_summary as rs
    w = workloads.BY_NAME["softmax_f32_1024x781"]
    k = rs.kernels_of(w)[0]
    grid = -(-(w.M * w.N * 4 // 16) // 256) * 256
    d = tmp_path / "run"
    d.mkdir()
    with open(d / "x_counter_collection.csv", "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, g, vals in (("void " + k + "(ntk::RowArgs)", 262144, (4096, 409600, 40960, 8192, 327680)),
                              ("void ntcal_copy_kernel<1, 1>(x)", grid, (3124, 312400, 3124, 0, 306152)),
                              ("void ntcal_copy_kernel<1, 1>(x)", 2 * grid, (1, 1, 1, 1, 1))):
            for c, v in zip(rs.WAVE_COUNTERS, vals):
                wr.writerow({"Kernel_Name": name, "Grid_Size": g, "Counter_Name": c, "Counter_Value": v})
    cmds = tmp_path / "cmds.txt"
    cmds.write_text("cmd\n")
    md = tmp_path / "w.md"
    rs.waves(types.SimpleNamespace(run=str(d), cmds=str(cmds), md=str(md)))
    text = md.read_text()
    assert f"| softmax_f32_1024x781 | `{k}` | 4096 | 100 | 0.100 | 0.020 | 0.800 |" in text
    assert "| | copy of its bytes | 3124 | 100 | 0.010 | 0.000 | 0.980 |" in text


def test_override_helper_restores():
    """bench.py's tuning settings (nt.override) are restored on exit,
    nested or not, and a bad setting changes nothing."""
    import row_wise_reductions_amd as nt
    plan = lambda: nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 64, 262144, nt.NT_F32, True)["cooperative"]  # noqa: E731
    assert plan() == 2                        # the cooperative kernel, two rows per workgroup
    with nt.override(NT_COOP="0", NT_NORM_SPLIT_ROWS="5"):
        assert plan() == 0
        with nt.override(NT_COOP="rows1"):
            assert plan() == 1
        assert plan() == 0
    assert plan() == 2
    with pytest.raises(nt.NtError):
        nt.set_override("NT_NO_SUCH_SETTING", "1")
    with pytest.raises(nt.NtError):
        nt.set_override("NT_COOP_SPIN", "-3")
    assert plan() == 2
