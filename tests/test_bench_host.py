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


def _jobs(plant=False):
    rng = np.random.default_rng(5)
    x1 = workloads.encode(rng.standard_normal((64, 781)), "f32")
    y1 = compare.round_to(oracle.softmax(x1, "f32"), "f32")
    x2 = workloads.encode(rng.standard_normal((32, 512)), "bf16")
    w2 = workloads.encode(1.0 + 0.3 * rng.standard_normal(512), "bf16")
    y2 = compare.round_to(oracle.rmsnorm(x2, "bf16", 1e-6, weight=w2), "bf16")
    if plant:                                       # a wrong element on a checked row
        y2 = y2.copy()
        y2[16, 7] ^= np.uint16(0x0040)
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
