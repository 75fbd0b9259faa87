"""Host side of the C ABI, checked without a GPU: the library loads, exports
every function include/nt.h declares, validates arguments before touching
the device, and plans launches as documented.  The pointers passed here are
never dereferenced: every call is expected to fail validation first."""
import os
import subprocess
import re

import pytest

import row_wise_reductions_amd as nt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nt.h")
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
F32, F16, BF16 = nt.NT_F32, nt.NT_F16, nt.NT_BF16


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nt_[a-z_]+)\s*\(", text)))


def test_header_matches_exports():
    names = declared_functions()
    assert set(names) == set(nt.EXPORTED), names
    L = nt.lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported by libnt.so"


def test_exports_are_c_symbols():
    out = os.popen(f"nm -D --defined-only {nt.LIB_PATH}").read()
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), f"{n} is not an extern \"C\" text symbol"


def test_status_strings():
    for code in range(10):
        s = nt.nt_status_string(code)
        assert s and s != "unknown status"
    assert nt.nt_status_string(99) == "unknown status"


@pytest.mark.parametrize("call,code", [
    (lambda: nt.nt_softmax_rows(4, 8, 7, FAKE, FAKE, None, 0, None), 3),
    (lambda: nt.nt_softmax_rows(-1, 8, F32, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_rows(4, 0, F32, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_rows(4, 1 << 31, F32, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_rows(1 << 40, 1 << 30, F32, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_rows(4, 8, F32, None, FAKE, None, 0, None), 1),
    (lambda: nt.nt_softmax_rows(4, 8, F32, FAKE, None, None, 0, None), 1),
    (lambda: nt.nt_softmax_rows(4, 8, F32, FAKE + 2, FAKE, None, 0, None), 5),
    (lambda: nt.nt_softmax_rows(4, 8, F16, FAKE, FAKE + 1, None, 0, None), 5),
    (lambda: nt.nt_softmax_rows(4, 1 << 20, F32, FAKE, FAKE, None, 1 << 20, None), 1),
    (lambda: nt.nt_softmax_rows(4, 1 << 20, F32, FAKE, FAKE, FAKE + 4, 1 << 20, None), 5),
    (lambda: nt.nt_softmax_rows(4, 1 << 20, F32, FAKE, FAKE, FAKE, 8, None), 6),
    (lambda: nt.nt_layernorm_rows(4, 8, F32, float("nan"), FAKE, None, None, FAKE, None, None, None), 4),
    (lambda: nt.nt_layernorm_rows(4, 8, F32, float("inf"), FAKE, None, None, FAKE, None, None, None), 4),
    (lambda: nt.nt_layernorm_rows(4, 8, F32, -1e-5, FAKE, None, None, FAKE, None, None, None), 4),
    (lambda: nt.nt_layernorm_rows(4, 8, F16, 1e-5, FAKE, FAKE + 1, None, FAKE, None, None, None), 5),
    (lambda: nt.nt_layernorm_rows(4, 8, F16, 1e-5, FAKE, None, FAKE + 1, FAKE, None, None, None), 5),
    (lambda: nt.nt_layernorm_rows(4, 8, F16, 1e-5, FAKE, None, None, FAKE, FAKE + 2, None, None), 5),
    (lambda: nt.nt_layernorm_rows(4, 8, F16, 1e-5, FAKE, None, None, FAKE, None, FAKE + 2, None), 5),
    (lambda: nt.nt_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 1, FAKE, None), 5),
    (lambda: nt.nt_rmsnorm_rows(4, 8, 3, 1e-6, FAKE, None, FAKE, None), 3),
    (lambda: nt.nt_rmsnorm_rows(4, 8, BF16, 1e-6, None, None, FAKE, None), 1),
    (lambda: nt.nt_rmsnorm_rows(4, 1 << 31, BF16, 1e-6, FAKE, None, FAKE, None), 2),
    # causal softmax: scale finite and > 0, queries >= 1, offset >= 0
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, 0.0, 4, 0, FAKE, FAKE, None, 0, None), 9),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, -1.0, 4, 0, FAKE, FAKE, None, 0, None), 9),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, float("inf"), 4, 0, FAKE, FAKE, None, 0, None), 9),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, float("nan"), 4, 0, FAKE, FAKE, None, 0, None), 9),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, 1.0, 0, 0, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, 1.0, 4, -1, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_causal_rows(4, 8, 4, 1.0, 4, 0, FAKE, FAKE, None, 0, None), 3),
    (lambda: nt.nt_softmax_causal_rows(4, 0, F32, 1.0, 4, 0, FAKE, FAKE, None, 0, None), 2),
    (lambda: nt.nt_softmax_causal_rows(4, 8, F32, 1.0, 4, 0, None, FAKE, None, 0, None), 1),
    (lambda: nt.nt_softmax_causal_rows(4, 8, BF16, 1.0, 4, 0, FAKE, FAKE + 1, None, 0, None), 5),
    (lambda: nt.nt_softmax_causal_rows(4, 1 << 20, F32, 1.0, 4, 0, FAKE, FAKE, None, 1 << 20, None), 1),
    (lambda: nt.nt_softmax_causal_rows(4, 1 << 20, F32, 1.0, 4, 0, FAKE, FAKE, FAKE, 8, None), 6),
    # fused add + norm: residual and h required, in x's 16-byte phase, h != y
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, None, None, FAKE + 512, FAKE + 768, None), 1),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, None, None, FAKE + 768, None), 1),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, None, FAKE + 256, None, FAKE + 512, FAKE + 768, None), 1),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 257, None, FAKE + 512, FAKE + 768, None), 5),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 258, None, FAKE + 512, FAKE + 768, None), 5),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, None, FAKE + 514, FAKE + 768, None), 5),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, FAKE + 1, FAKE + 512, FAKE + 768, None), 5),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, None, FAKE + 512, FAKE + 512, None), 8),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, -1.0, FAKE, FAKE + 256, None, FAKE + 512, FAKE + 768, None), 4),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, 5, 1e-6, FAKE, FAKE + 256, None, FAKE + 512, FAKE + 768, None), 3),
    (lambda: nt.nt_add_rmsnorm_rows(-2, 8, BF16, 1e-6, FAKE, FAKE + 256, None, FAKE + 512, FAKE + 768, None), 2),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, None, None, None, FAKE + 512, FAKE + 768,
                                      None, None, None), 1),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, FAKE + 260, None, None, FAKE + 512, FAKE + 768,
                                      None, None, None), 5),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, FAKE + 256, FAKE + 2, None, FAKE + 512, FAKE + 768,
                                      None, None, None), 5),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, FAKE + 256, None, None, FAKE + 512, FAKE + 768,
                                      FAKE + 2, None, None), 5),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, FAKE + 256, None, None, FAKE + 512, FAKE + 512,
                                      None, None, None), 8),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, float("nan"), FAKE, FAKE + 256, None, None, FAKE + 512, FAKE + 768,
                                      None, None, None), 4),
    # norms with a workspace: the plain checks, then the workspace's size and alignment
    (lambda: nt.nt_layernorm_rows_ws(4, 1 << 20, F32, -1.0, FAKE, None, None, FAKE, None, None, FAKE, 1 << 20,
                                     None), 4),
    (lambda: nt.nt_layernorm_rows_ws(4, 1 << 20, F32, 1e-5, FAKE, None, None, FAKE, None, None, FAKE, 64, None), 6),
    (lambda: nt.nt_layernorm_rows_ws(4, 1 << 20, F32, 1e-5, FAKE, None, None, FAKE, None, None, FAKE + 4, 1 << 20,
                                     None), 5),
    (lambda: nt.nt_layernorm_rows_ws(4, 1 << 20, F16, 1e-5, FAKE, FAKE + 1, None, FAKE, None, None, FAKE, 1 << 20,
                                     None), 5),
    (lambda: nt.nt_rmsnorm_rows_ws(4, 1 << 20, BF16, 1e-6, FAKE, None, FAKE, FAKE, 0, None), 6),
    (lambda: nt.nt_rmsnorm_rows_ws(4, 1 << 20, BF16, 1e-6, FAKE, None, FAKE, FAKE + 2, 1 << 20, None), 5),
    (lambda: nt.nt_rmsnorm_rows_ws(4, 1 << 20, BF16, 1e-6, None, None, FAKE, FAKE, 1 << 20, None), 1),
    (lambda: nt.nt_rmsnorm_rows_ws(4, 1 << 20, 7, 1e-6, FAKE, None, FAKE, FAKE, 1 << 20, None), 3),
    # overlaps: y partly over x, a workspace over x or y, h or y partly over an input
    (lambda: nt.nt_softmax_rows(4, 8, F32, FAKE, FAKE + 16, None, 0, None), 8),
    (lambda: nt.nt_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE + 62, None, FAKE, None), 8),
    (lambda: nt.nt_layernorm_rows(4, 8, F32, 1e-5, FAKE, None, None, FAKE + 124, None, None, None), 8),
    (lambda: nt.nt_softmax_rows(4, 1 << 20, F32, FAKE, FAKE + (1 << 25), FAKE + 64, 1 << 20, None), 8),
    (lambda: nt.nt_softmax_rows(4, 1 << 20, F32, FAKE, FAKE + (1 << 25), FAKE + (1 << 25) + 64, 1 << 20, None), 8),
    (lambda: nt.nt_rmsnorm_rows_ws(4, 1 << 20, BF16, 1e-6, FAKE, None, FAKE, FAKE + 8, 1 << 20, None), 8),
    (lambda: nt.nt_layernorm_rows_ws(4, 1 << 20, F32, 1e-5, FAKE, None, None, FAKE + (1 << 25), None, None,
                                     FAKE + (1 << 25) - 8, 1 << 20, None), 8),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, None, FAKE + 272, FAKE + 512, None), 8),
    (lambda: nt.nt_add_rmsnorm_rows(4, 8, BF16, 1e-6, FAKE, FAKE + 256, None, FAKE + 512, FAKE + 40, None), 8),
    (lambda: nt.nt_add_layernorm_rows(4, 8, F32, 1e-5, FAKE, FAKE + 256, None, None, FAKE + 512, FAKE + 544,
                                      None, None, None), 8),
])
def test_validation_before_launch(call, code):
    # every case here must fail validation; on a machine with a GPU a library
    # bug could turn a fake pointer into a launch, so these run only without one
    if _gpu_present():
        pytest.skip("fake-pointer validation runs only on a host without a GPU")
    assert code != 0
    assert call() == code


def _gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_empty_is_noop():
    assert nt.nt_softmax_rows(0, 8, F32, None, None, None, 0, None) == 0
    assert nt.nt_layernorm_rows(0, 8, F32, 1e-5, None, None, None, None, None, None, None) == 0
    assert nt.nt_rmsnorm_rows(0, 8, F32, 1e-6, None, None, None, None) == 0
    assert nt.nt_add_rmsnorm_rows(0, 8, F32, 1e-6, None, None, None, None, None, None) == 0
    assert nt.nt_softmax_causal_rows(0, 8, F32, 1.0, 4, 0, None, None, None, 0, None) == 0
    assert nt.nt_add_layernorm_rows(0, 8, F32, 1e-5, None, None, None, None, None, None, None, None, None) == 0
    # a bad eps is still an error for an empty call
    assert nt.nt_rmsnorm_rows(0, 8, F32, -1.0, None, None, None, None) == 4
    assert nt.nt_layernorm_rows_ws(0, 1 << 20, F32, 1e-5, None, None, None, None, None, None, None, 0, None) == 0
    assert nt.nt_rmsnorm_rows_ws(0, 1 << 20, F32, 1e-6, None, None, None, None, 0, None) == 0


def test_workspace_bytes():
    assert nt.nt_softmax_workspace_bytes(1024, 781, F32) == 0          # single pass
    assert nt.nt_softmax_workspace_bytes(131072, 4096, BF16) == 0
    # 1 MiB fp32 rows: 16 chunks of 64 KiB (+1 for a misaligned head) per
    # row, a 16-byte record (two tagged 64-bit words) per chunk, then 16
    # bytes for the tag word of a call captured into a graph
    assert nt.nt_softmax_workspace_bytes(64, 262144, F32) == 64 * 17 * 16 + 16
    assert nt.nt_softmax_workspace_bytes(-1, 8, F32) == 0
    assert nt.nt_softmax_workspace_bytes(4, 8, 9) == 0


def test_plans_of_the_workloads():
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 1024, 781, F32, True)     # 3124-byte rows: misaligned
    assert (p["split"], p["waves_per_row"], p["chunks_per_lane"], p["aligned"]) == (0, 4, 1, 0)
    assert p["rows_per_block"] == 1 and p["grid"] == 1024
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, 4096, F16, True)
    assert (p["split"], p["aligned"]) == (0, 1) and 64 * p["waves_per_row"] * p["chunks_per_lane"] >= 512
    p = nt.nt_plan_launch(nt.NT_OP_RMSNORM, 16384, 8192, BF16, True)
    assert p["split"] == 0 and 64 * p["waves_per_row"] * p["chunks_per_lane"] >= 1024
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 131072, 4096, BF16, True)
    assert p["split"] == 0
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 64, 262144, F32, True)
    # 1024 (row, chunk) pairs of fp32: two rows per cooperative workgroup
    assert p["split"] == 1 and p["row_chunks"] == 16 and p["grid"] == 32 * 16 and p["rows_per_block"] == 2
    assert (p["waves_per_row"], p["chunks_per_lane"]) == (8, 8)
    assert p["workspace_bytes"] == 64 * 16 * 16 + 16 and p["cooperative"] == 2


def test_narrow_row_rule():
    """Rows of at most 256 chunks: 4 waves x 1 chunk at up to 1024 rows;
    beyond, misaligned rows of 65-256 chunks take 2 x 2 (up to 128 chunks,
    and 16-bit softmax up to 256) or 4 x 1, and everything else the menu's
    one-wave shapes.  The causal entry plans as the softmax; the fused add +
    norm entries keep their menus."""
    def shape(op, M, N, dt):
        e = 4 if dt == F32 else 2
        p = nt.nt_plan_launch(op, M, N, dt, (N * e) % 16 == 0)
        return p["waves_per_row"], p["chunks_per_lane"]
    S, L, R = nt.NT_OP_SOFTMAX, nt.NT_OP_LAYERNORM, nt.NT_OP_RMSNORM
    for op in (S, L, R):
        for dt in (F32, F16, BF16):
            for N in (8, 300, 781, 1024, 2048 if dt != F32 else 1000):
                assert shape(op, 1024, N, dt) == (4, 1), (op, dt, N)
    # misaligned, 2048 rows and more
    for M in (2048, 16384):
        assert shape(S, M, 781, F32) == (4, 1)          # 196 chunks
        assert shape(S, M, 301, F32) == (2, 2)          # 77 chunks
        assert shape(S, M, 509, F32) == (2, 2)          # 128 chunks
        assert shape(S, M, 1030, BF16) == (2, 2)        # 130 chunks
        assert shape(S, M, 601, BF16) == (2, 2)
        assert shape(R, M, 781, F32) == (4, 1) and shape(R, M, 301, F32) == (2, 2)
        assert shape(R, M, 901, BF16) == (2, 2) and shape(R, M, 1500, BF16) == (4, 1)
        assert shape(L, M, 781, F32) == (4, 1) and shape(L, M, 509, F32) == (2, 2)
        assert shape(L, M, 901, F16) == (1, 2) and shape(L, M, 1500, F16) == (4, 1)
        assert shape(S, M, 201, F32) == (1, 1)          # 52 chunks: the menu
    # aligned rows beyond 1024 rows keep the menu
    assert shape(S, 4096, 1000, F32) == (1, 4) and shape(S, 4096, 2048, BF16) == (1, 4)
    assert shape(S, 1025, 520, F32) == (1, 4)
    # the fused add + norm entries keep their menus
    p = nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 1024, 781, F32, False)
    assert (p["waves_per_row"], p["chunks_per_lane"]) == (1, 4)
    for M, N, dt in ((1024, 781, F32), (4096, 781, F32), (4096, 1030, BF16), (4096, 1000, F32)):
        a = nt.nt_plan_launch(nt.NT_OP_SOFTMAX_CAUSAL, M, N, dt, (N * (4 if dt == F32 else 2)) % 16 == 0)
        b = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, dt, (N * (4 if dt == F32 else 2)) % 16 == 0)
        assert a == b


def test_persistent_grid_rule(ntenv):
    """The persistent norm kernel's grid: k workgroups per compute unit (256
    on a host without a GPU, as on MI355X), k = max(2, ceil(16 KiB / row
    bytes)) for LayerNorm and max(1, floor(32 KiB / row bytes)) for RMSNorm,
    never more than there are rows; NT_PERSIST_GRID sets it."""
    L, R, AL = nt.NT_OP_LAYERNORM, nt.NT_OP_RMSNORM, nt.NT_OP_ADD_LAYERNORM

    def grid(op, M, N, dt):
        p = nt.nt_plan_launch(op, M, N, dt, True)
        assert p["persistent"] == 1, (op, M, N, dt, p)
        return p["grid"]
    assert grid(L, 4096, 4096, F16) == 2 * 256          # 8 KiB rows
    assert grid(L, 4096, 4096, BF16) == 2 * 256
    assert grid(L, 4096, 3584, F16) == 3 * 256          # 7 KiB
    assert grid(L, 4096, 2048, F16) == 4 * 256          # 4 KiB
    assert grid(L, 4096, 1032, F16) == 8 * 256          # 2064 B: ceil(7.9)
    assert grid(L, 4096, 2048, F32) == 2 * 256          # 8 KiB
    assert grid(L, 16384, 8192, F16) == 2 * 256         # 16 KiB: at least 2
    assert grid(L, 16384, 16384, F16) == 2 * 256        # 32 KiB
    assert grid(AL, 4096, 8192, F16) == 2 * 256
    assert grid(R, 16384, 8192, BF16) == 2 * 256        # 16 KiB
    assert grid(R, 16384, 16384, BF16) == 256           # 32 KiB
    assert grid(R, 4096, 10240, F32) == 256             # 40 KiB
    assert grid(L, 100, 4096, F16) == 100               # fewer rows than workgroups
    ntenv.setenv("NT_PERSIST_GRID", "300")
    assert grid(L, 4096, 4096, F16) == 300 and grid(R, 16384, 8192, BF16) == 300
    assert grid(L, 100, 4096, F16) == 100


def test_cooperative_split_limits():
    # one kernel up to 128 chunks per row (16384 elements each: 8 waves with
    # 32 values per lane), two kernels (16 KiB chunks) beyond
    for dt in (F32, F16, BF16):
        p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 2, 128 * 16384, dt, True)
        assert (p["split"], p["row_chunks"], p["cooperative"]) == (1, 128, 1)
        assert p["waves_per_row"] * p["chunks_per_lane"] * 16 // (4 if dt == F32 else 2) == 256
        p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 2, 128 * 16384 + 8, dt, True)
        assert (p["split"], p["cooperative"], p["waves_per_row"], p["chunks_per_lane"]) == (1, 0, 4, 4)
        assert p["row_chunks"] == -(-(128 * 16384 + 8) * (4 if dt == F32 else 2) // 16 // 1024)
    # never on the single pass
    assert nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 2, 4096, F32, True)["cooperative"] == 0


def test_cooperative_split_can_be_switched_off(ntenv):
    ntenv.setenv("NT_COOP", "0")
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 64, 262144, F32, True)
    assert (p["split"], p["cooperative"]) == (1, 0)


def test_plan_capacity_covers_row():
    for dt, e in ((F32, 4), (F16, 2), (BF16, 2)):
        for N in (1, 7, 64, 255, 256, 781, 1024, 4097, 8192, 30000, 32768 * 4 // e):
            for al in (True, False):
                p = nt.nt_plan_launch(nt.NT_OP_RMSNORM, 8, N, dt, al)
                vec = 16 // e
                need = N // vec if (al and (N * e) % 16 == 0) else (N + 2 * vec - 2) // vec
                if p["split"] == 0:
                    assert 64 * p["waves_per_row"] * p["chunks_per_lane"] >= need, (dt, N, al, p)


def test_wide_rows_take_the_streaming_paths():
    # LayerNorm holds at most 16 values per lane, 32 at 8 waves: 32 KiB of
    # 16-bit row, 64 KiB of fp32 row in one pass
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 1, 16384, BF16, True)["split"] == 0
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, 8200, BF16, True)      # 1025 whole chunks
    assert (p["split"], p["waves_per_row"], p["chunks_per_lane"], p["persistent"]) == (0, 5, 4, 1)
    # 16-bit: 7 x 2 to 896 chunks, 8 x 2 to 1024, then 5 x 4 to 1216 chunks, 6 x 4 to 1408,
    # 8 x 4 to 1472, 7 x 4 to 1792, 8 x 4
    for N, shape in ((4104, (7, 2)), (7168, (7, 2)), (7176, (8, 2)), (8192, (8, 2)), (9728, (5, 4)),
                     (9736, (6, 4)), (11264, (6, 4)), (11272, (8, 4)), (11776, (8, 4)), (11784, (7, 4)),
                     (14336, (7, 4)), (14344, (8, 4)), (16384, (8, 4))):
        p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, N, F16, True)
        assert (p["split"], p["waves_per_row"], p["chunks_per_lane"], p["persistent"]) == (0, *shape, 1), (N, p)
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 1, 16385, BF16, True)
    assert p["split"] == 2 and p["grid"] == 1 and p["threads_per_block"] == 512
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, 8200, F32, True)       # fp32 12 x 4: one row per workgroup
    assert (p["split"], p["waves_per_row"], p["chunks_per_lane"], p["persistent"]) == (0, 12, 4, 0)
    assert p["threads_per_block"] == 768
    for N, shape in ((2048, (2, 4)), (2052, (4, 4)), (2560, (4, 4)), (2564, (8, 2))):   # fp32 4 x 4 to 640 chunks
        p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, N, F32, True)
        assert (p["waves_per_row"], p["chunks_per_lane"], p["persistent"]) == (*shape, 1), (N, p)
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, 12296, F32, True)      # past 12 x 4: 8 x 8
    assert (p["split"], p["waves_per_row"], p["chunks_per_lane"], p["persistent"]) == (0, 8, 8, 0)
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 1, 16384, F32, True)["split"] == 0
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 1, 16385, F32, True)["split"] == 2
    assert nt.nt_plan_launch(nt.NT_OP_ADD_LAYERNORM, 1, 16384, F16, True)["split"] == 0
    assert nt.nt_plan_launch(nt.NT_OP_ADD_LAYERNORM, 1, 16385, F16, True)["split"] == 2
    # RMSNorm fp32 up to 128 KiB single pass, then looped
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM, 7, 32768, F32, True)["split"] == 0
    p = nt.nt_plan_launch(nt.NT_OP_RMSNORM, 7, 32769, F32, True)
    assert p["split"] == 2 and p["grid"] == 7
    # softmax takes the split path instead
    assert nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 1, 32769, F32, True)["split"] == 1
    assert nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 1, 1 << 24, BF16, True)["split"] == 1


def test_grid_fits_dispatch_packet():
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 1 << 34, 8, F32, True)
    assert p["grid"] * p["threads_per_block"] <= 1 << 31
    with pytest.raises(nt.NtError):   # split path cannot stride: too many (row, chunk) pairs
        nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 1 << 24, 1 << 20, F32, True)


def test_env_overrides(ntenv):
    ntenv.setenv("NT_FORCE_SHAPE", "4,4")
    p = nt.nt_plan_launch(nt.NT_OP_RMSNORM, 16, 8192, BF16, True)
    assert (p["waves_per_row"], p["chunks_per_lane"]) == (4, 4)
    ntenv.setenv("NT_FORCE_SHAPE", "1,1")          # too small for the row: ignored
    p = nt.nt_plan_launch(nt.NT_OP_RMSNORM, 16, 8192, BF16, True)
    assert 64 * p["waves_per_row"] * p["chunks_per_lane"] >= 1024
    ntenv.delenv("NT_FORCE_SHAPE")
    ntenv.setenv("NT_FORCE_PATH", "split")
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 16, 4096, F32, True)
    assert p["split"] == 1 and p["row_chunks"] == 1
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM, 16, 4096, F32, True)["split"] == 0


def _kernel_symbols():
    out = subprocess.run(["nm", "-C", nt.LIB_PATH], capture_output=True, text=True, check=True).stdout
    return set(re.findall(r"ntk::(row_resident|row_norm_persistent)<([^>]*)>", out))


def test_forced_shapes_have_kernels(ntenv):
    """A forced single-pass shape is taken only where its kernel is built (else
    the plan ignores it): for every W, K up to 16 and each op and type, the
    kernel the plan would launch is in the library."""
    syms = _kernel_symbols()
    assert len(syms) > 100
    ops = {nt.NT_OP_SOFTMAX: 0, nt.NT_OP_LAYERNORM: 1, nt.NT_OP_RMSNORM: 2}
    taken = 0
    for op, kop in ops.items():
        for dt in (F32, F16, BF16):
            for W in range(1, 17):
                for K in range(1, 17):
                    ntenv.setenv("NT_FORCE_SHAPE", f"{W},{K}")
                    N = 64 * W * K * (4 if dt == F32 else 8)      # exactly W x K chunks per row
                    for aligned in (True, False):
                        p = nt.nt_plan_launch(op, 4096, N - (0 if aligned else 1), dt, aligned)
                        if p["split"] != 0 or (p["waves_per_row"], p["chunks_per_lane"]) != (W, K):
                            continue
                        taken += 1
                        if p["persistent"]:
                            name = ("row_norm_persistent", f"{kop}, {dt}, {W}, {K}, false")
                        else:
                            pr = "true" if op != nt.NT_OP_SOFTMAX else "false"
                            name = ("row_resident", f"{kop}, {dt}, {W}, {K}, {str(aligned).lower()}, {pr}, false")
                        assert name in syms, (op, dt, W, K, aligned, p)
    assert taken > 50
    ntenv.setenv("NT_FORCE_SHAPE", "2,4")   # 16-bit LayerNorm at 2 x 4 (32 values per lane) has no kernel
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, 4096, F16, True)
    assert (p["waves_per_row"], p["chunks_per_lane"]) != (2, 4)


def test_persistent_rule():
    """Persistent workgroups: every LayerNorm; fused add + LayerNorm with 16
    values or more per lane; 16-bit RMSNorm from 1024 chunks per row; fp32
    RMSNorm only on part-filled 8 x 8 shapes (2049..3072 chunks); never the
    fused add + RMSNorm; only on aligned rows with the parameters present."""
    cases = [  # (op, dt, N) -> persistent
        (nt.NT_OP_LAYERNORM, F16, 2048, 1), (nt.NT_OP_LAYERNORM, F16, 4096, 1), (nt.NT_OP_LAYERNORM, F32, 2048, 1),
        (nt.NT_OP_LAYERNORM, F32, 8192, 1), (nt.NT_OP_ADD_LAYERNORM, F16, 4096, 0),
        (nt.NT_OP_ADD_LAYERNORM, F16, 5120, 1), (nt.NT_OP_ADD_LAYERNORM, F16, 8192, 1),
        (nt.NT_OP_ADD_LAYERNORM, F32, 2048, 0), (nt.NT_OP_ADD_LAYERNORM, F32, 4096, 0),
        (nt.NT_OP_ADD_LAYERNORM, F32, 5120, 1), (nt.NT_OP_RMSNORM, BF16, 4096, 0), (nt.NT_OP_RMSNORM, BF16, 8192, 1),
        (nt.NT_OP_RMSNORM, F16, 16384, 1), (nt.NT_OP_RMSNORM, F32, 4096, 0), (nt.NT_OP_RMSNORM, F32, 8320, 1),
        (nt.NT_OP_RMSNORM, F32, 12288, 1), (nt.NT_OP_RMSNORM, F32, 12800, 0), (nt.NT_OP_RMSNORM, F32, 16384, 0),
        (nt.NT_OP_ADD_RMSNORM, BF16, 8192, 0), (nt.NT_OP_ADD_RMSNORM, F32, 4096, 0),
        (nt.NT_OP_ADD_RMSNORM, F32, 10240, 0)]
    for op, dt, N, want in cases:
        p = nt.nt_plan_launch(op, 4096, N, dt, True)
        assert p["split"] == 0 and p["persistent"] == want, (op, dt, N, p)
        assert nt.nt_plan_launch(op, 4096, N, dt, False)["persistent"] == 0
    # the shapes the sweeps chose for the plain norms
    assert [(nt.nt_plan_launch(nt.NT_OP_RMSNORM, 4096, n, dt, True)["waves_per_row"],
             nt.nt_plan_launch(nt.NT_OP_RMSNORM, 4096, n, dt, True)["chunks_per_lane"])
            for n, dt in ((2048, BF16), (4096, BF16), (2048, F32), (4096, F32))] == [(4, 1), (8, 1), (8, 1), (8, 2)]
    assert [(nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, n, dt, True)["waves_per_row"],
             nt.nt_plan_launch(nt.NT_OP_LAYERNORM, 4096, n, dt, True)["chunks_per_lane"])
            for n, dt in ((2048, F16), (4096, F16), (2048, F32))] == [(2, 2), (4, 2), (2, 4)]


def test_fused_add_norm_plans():
    # the fused kernels hold the residual too: RMSNorm at most 32 values per
    # lane in one pass, wider rows take the looped kernel
    p = nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 16384, 8192, BF16, True)
    assert (p["split"], p["persistent"], p["waves_per_row"], p["chunks_per_lane"]) == (0, 0, 8, 2)
    p = nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 8192, 16384, BF16, True)
    assert (p["split"], p["persistent"], p["waves_per_row"], p["chunks_per_lane"]) == (0, 0, 16, 2)
    p = nt.nt_plan_launch(nt.NT_OP_ADD_LAYERNORM, 4096, 4096, F16, True)
    assert (p["split"], p["persistent"], p["waves_per_row"], p["chunks_per_lane"]) == (0, 0, 8, 1)
    p = nt.nt_plan_launch(nt.NT_OP_ADD_LAYERNORM, 4096, 8192, F16, True)
    assert (p["split"], p["persistent"]) == (0, 1)
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM, 4, 8192 * 4, BF16, True)["split"] == 0      # 64 per lane
    assert nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 4, 8192 * 4, BF16, True)["split"] == 2  # looped
    assert nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 4, 8192 * 2, BF16, True)["split"] == 0
    for dt in (F32, F16, BF16):
        for N in (1, 7, 781, 4096, 8192, 30000, 100000):
            for al in (True, False):
                p = nt.nt_plan_launch(nt.NT_OP_ADD_RMSNORM, 8, N, dt, al)
                if p["split"] == 0:
                    assert p["chunks_per_lane"] * (4 if dt == F32 else 8) <= 32, (dt, N, al, p)


def test_causal_softmax_plans():
    # as the softmax, except full 16-bit rows of 512 chunks: the softmax
    # keeps 8 waves x 1 chunk there, causal rows (loads stop at the
    # diagonal) take 4 waves x 2 chunks like part-filled rows
    for (M, N, dt) in ((64, 262144, F32), (3, 781, F32), (2, 1 << 22, F16), (8, 4096, F32), (8, 16384, BF16),
                       (8, 3000, BF16)):
        a = nt.nt_plan_launch(nt.NT_OP_SOFTMAX_CAUSAL, M, N, dt, True)
        b = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, M, N, dt, True)
        assert a == b, (M, N, dt)
    a = nt.nt_plan_launch(nt.NT_OP_SOFTMAX_CAUSAL, 131072, 4096, BF16, True)
    b = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 131072, 4096, BF16, True)
    assert (a["waves_per_row"], a["chunks_per_lane"]) == (4, 2) and (b["waves_per_row"], b["chunks_per_lane"]) == (8, 1)
    # part-filled 16-bit rows of 257..511 chunks: 4 waves x 2 chunks
    p = nt.nt_plan_launch(nt.NT_OP_SOFTMAX, 8, 3000, BF16, True)
    assert (p["waves_per_row"], p["chunks_per_lane"]) == (4, 2)


def test_norm_workspace_bytes():
    LN, RMS = nt.NT_OP_LAYERNORM, nt.NT_OP_RMSNORM
    # rows that fit one pass, or enough rows to fill the GPU: no workspace
    assert nt.nt_norm_workspace_bytes(LN, 4, 8192, BF16) == 0
    assert nt.nt_norm_workspace_bytes(RMS, 4, 30000, F32) == 0
    # (a 32768-wide fp32 row fits when aligned, not with a misaligned head)
    assert nt.nt_norm_workspace_bytes(RMS, 4, 32768, F32) > 0
    assert nt.nt_norm_workspace_bytes(LN, 4096, 1 << 20, BF16) == 0
    # 64 fp32 rows of 1 MiB: 32 KiB chunks (8 waves x 4 chunks) -> 32 per row,
    # 33 for a misaligned head; 32 bytes per chunk (four tagged words) and 8 per row
    assert nt.nt_norm_workspace_bytes(LN, 64, 262144, F32) == 64 * 33 * 32 + 64 * 8 + 16
    # 16 bf16 rows of 2 MiB: 8 KiB chunks fill the grid -> 256 per row (+1)
    assert nt.nt_norm_workspace_bytes(RMS, 16, 1 << 20, BF16) == 16 * 257 * 32 + 16 * 8 + 16
    # other ops and invalid arguments
    for bad in ((nt.NT_OP_SOFTMAX, 4, 1 << 20, F32), (LN, -1, 1 << 20, F32), (LN, 4, 0, F32), (RMS, 4, 1 << 20, 5)):
        assert nt.nt_norm_workspace_bytes(*bad) == 0
    # no rows: nothing to split (a regression: the grid check divided by M)
    for op in (LN, RMS):
        for dt in (F32, F16, BF16):
            assert nt.nt_norm_workspace_bytes(op, 0, 1 << 20, dt) == 0
            ws_op = nt.NT_OP_LAYERNORM_WS if op == LN else nt.NT_OP_RMSNORM_WS
            assert nt.nt_plan_launch(ws_op, 0, 1 << 20, dt, True) == nt.nt_plan_launch(op, 0, 1 << 20, dt, True)


def _split_norm_plan(base, dt, M, nch, coop=True):
    """The split norm's expected plan: ((W, K), one_pass), or None for the
    looped plan.  One pass with 8 waves x 4 chunks per lane (fp32 also 8 x 8:
    RMSNorm first, LayerNorm second) at any row count when the row has at most 16 such chunks,
    the call at least 2048 workgroups, and the op is not 16-bit LayerNorm;
    else two kernels below
    256 (LayerNorm) or 2048 (RMSNorm) rows, with the largest chunk of 8x4,
    8x1, 4x1 giving at least 2048 workgroups (else 4x1)."""
    shapes = ((8, 4), (8, 1), (4, 1))
    P = lambda s: -(-nch // (64 * s[0] * s[1]))  # noqa: E731
    ln = base == nt.NT_OP_LAYERNORM
    if coop and not (ln and dt != F32):
        # fp32: 8 x 8 (64 KiB chunks) too, RMSNorm first, LayerNorm second
        for one in ([(8, 8), (8, 4)] if (not ln and dt == F32) else [(8, 4), (8, 8)] if dt == F32 else [(8, 4)]):
            if P(one) <= 16 and M * P(one) >= 2048:
                return one, True
    if M >= (256 if ln else 2048):
        return None
    return next((s for s in shapes if M * P(s) >= 2048), shapes[-1]), False


def test_split_norm_plans():
    for op, base in ((nt.NT_OP_LAYERNORM_WS, nt.NT_OP_LAYERNORM), (nt.NT_OP_RMSNORM_WS, nt.NT_OP_RMSNORM)):
        for dt, e in ((F32, 4), (F16, 2), (BF16, 2)):
            for M, N in ((1, 40000), (3, 100003), (64, 262144), (16, 1 << 20), (1000, 65536), (255, 20000),
                         (4096, 65536), (300, 262144), (5000, 40003)):
                for al in (True, False):
                    p = nt.nt_plan_launch(op, M, N, dt, al)
                    plain = nt.nt_plan_launch(base, M, N, dt, al)
                    aligned = al and (N * e) % 16 == 0
                    nch = N * e // 16 if aligned else (N + 2 * (16 // e) - 2) // (16 // e)
                    want = _split_norm_plan(base, dt, M, nch) if plain["split"] == 2 else None
                    if want is None:          # one pass, or the looped plan: the workspace changes nothing
                        assert p == plain, (op, dt, M, N, al)
                        continue
                    assert p["split"] == 3, (op, dt, M, N, al, p)
                    assert ((p["waves_per_row"], p["chunks_per_lane"]), bool(p["cooperative"])) == want, \
                        (op, dt, M, N, al, p)
                    per = 64 * p["waves_per_row"] * p["chunks_per_lane"]
                    assert p["row_chunks"] == -(-nch // per) and p["grid"] == M * p["row_chunks"]
                    assert p["workspace_bytes"] == M * p["row_chunks"] * 32 + M * 8 + 16
                    assert p["workspace_bytes"] <= nt.nt_norm_workspace_bytes(base, M, N, dt)
        # many rows of many chunks: looped
        assert nt.nt_plan_launch(op, 4096, 1 << 20, BF16, True)["split"] == 2
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, 256, 1 << 20, BF16, True)["split"] == 2
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 2047, 1 << 20, BF16, True)["split"] == 3


def test_split_norm_rows_switch(ntenv):
    ntenv.setenv("NT_NORM_SPLIT_ROWS", "0")
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 64, 262144, F32, True)["split"] == 2
    assert nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, 64, 262144, F32) == 0
    ntenv.setenv("NT_NORM_SPLIT_ROWS", "100000")
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 4096, 262144, F32, True)["split"] == 3


def test_split_norm_cooperative_switch(ntenv):
    # 128 bf16 rows of 512 KiB: 16 chunks of 32 KiB per row in one pass
    p = nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 128, 262144, BF16, True)
    assert (p["split"], p["cooperative"], p["row_chunks"], p["grid"]) == (3, 1, 16, 2048)
    # not for 16-bit LayerNorm: two kernels (same chunks) at few rows, the looped kernel at many
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, 128, 262144, BF16, True)
    assert (p["split"], p["cooperative"], p["row_chunks"]) == (3, 0, 16)
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, 4096, 131072, F16, True)["split"] == 2
    # one pass at any row count where it applies; fp32 LayerNorm included
    p = nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, 65536, 65536, F32, True)
    assert (p["split"], p["cooperative"], p["row_chunks"]) == (3, 1, 8)
    ntenv.setenv("NT_COOP", "0")
    p2 = nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 128, 262144, BF16, True)
    assert (p2["split"], p2["cooperative"], p2["row_chunks"]) == (3, 0, 16)
    p3 = nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 64, 65536, F32, True)      # 2048 workgroups need 8 KiB chunks
    assert (p3["split"], p3["cooperative"], p3["row_chunks"]) == (3, 0, 32)
    assert nt.nt_plan_launch(nt.NT_OP_LAYERNORM_WS, 65536, 65536, F32, True)["split"] == 2
    # the documented size covers both forms and both alignments (9 chunks
    # of 32 KiB with a misaligned head)
    need = nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, 256, 65536, F32)
    assert need == 256 * 9 * 32 + 256 * 8 + 16
    ntenv.delenv("NT_COOP")
    assert nt.nt_norm_workspace_bytes(nt.NT_OP_RMSNORM, 256, 65536, F32) == need
    assert nt.nt_plan_launch(nt.NT_OP_RMSNORM_WS, 256, 65536, F32, True)["row_chunks"] == 8


def test_planner_survives_extreme_arguments():
    """The host-only calls (plans, workspace sizes) over every op, type and
    extreme sizes, in a child process so that a crash (a division by zero, an
    overflow trap) fails this test instead of the test run: each returns a
    plan, an error status or a size, never a signal."""
    import subprocess
    import sys
    code = r'''
import row_wise_reductions_amd as nt
Ms = (0, 1, 2, 255, 256, 2047, 2048, 4096, 1 << 20, (1 << 31) - 1, 1 << 31, 1 << 40)
Ns = (1, 7, 781, 8192, 16385, 32769, 1 << 20, (1 << 31) - 1, 1 << 31)
n = 0
for op in range(8):
    for M in Ms:
        for N in Ns:
            for dt in (0, 1, 2, 3):
                for al in (True, False):
                    try:
                        nt.nt_plan_launch(op, M, N, dt, al)
                    except nt.NtError:
                        pass
                    n += 1
                if op < 3:
                    nt.nt_softmax_workspace_bytes(M, N, dt)
                    nt.nt_norm_workspace_bytes(op, M, N, dt)
print("ok", n)
'''
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0 and r.stdout.startswith("ok"), (r.returncode, r.stdout[-500:], r.stderr[-2000:])


def test_torch_wrappers_reject_host_tensors():
    """The torch conveniences pass raw addresses to the library: a tensor
    in host memory is refused before any call."""
    import torch
    x = torch.zeros(4, 8)
    for call in (lambda: nt.softmax(x), lambda: nt.softmax_causal(x), lambda: nt.layer_norm(x),
                 lambda: nt.rms_norm(x), lambda: nt.add_layer_norm(x, x), lambda: nt.add_rms_norm(x, x)):
        with pytest.raises(ValueError, match="GPU tensor"):
            call()
    with pytest.raises(TypeError):
        nt.dtype_code(torch.zeros(2, dtype=torch.float64))
