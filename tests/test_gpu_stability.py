"""Barrier discipline of the reductions: each kernel family, run many times
with fresh random inputs and with the same input, must be bitwise stable.  A
missing barrier between a wave writing its partial result to LDS and another
wave reading it, or a reused LDS slot, shows up as an output that changes
from one run to the next.  Families: one wave per row (no LDS), a row over 8
waves (LDS combine), the persistent norm kernel (parity slots across rows),
the looped norm kernel, the cooperative split softmax and the one-pass split
norm (records exchanged between workgroups)."""
from __future__ import annotations

import sys

import pytest

from conftest import gpu_available

pytestmark = pytest.mark.gpu

if not gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

import row_wise_reductions_amd as nt  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


CASES = [
    ("softmax", torch.float32, 1024, 781),          # one wave per row, 4 rows per workgroup
    ("softmax", torch.bfloat16, 64, 4096),          # 8 waves per row, LDS combine
    ("layernorm", torch.float16, 300, 8192),        # persistent, parity slots
    ("rmsnorm", torch.bfloat16, 300, 16384),        # persistent
    ("layernorm", torch.float32, 37, 100003),       # split norm in two kernels (the wrapper gives a workspace)
    ("rmsnorm_plain", torch.float16, 37, 100003),   # looped kernel (plain entry point, no workspace)
    ("softmax", torch.float32, 8, 262144),          # cooperative split softmax
    ("rmsnorm", torch.float32, 256, 65536),         # one-pass split norm
]


def run(op, x, w, b):
    if op == "softmax":
        return (nt.softmax(x),)
    if op == "rmsnorm_plain":
        M, N = x.shape
        y = torch.empty_like(x)
        code = {torch.float32: nt.NT_F32, torch.float16: nt.NT_F16, torch.bfloat16: nt.NT_BF16}[x.dtype]
        assert nt.nt_rmsnorm_rows(M, N, code, 1e-6, x.data_ptr(), w.data_ptr(), y.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream) == 0
        return (y,)
    if op == "layernorm":
        return nt.layer_norm(x, w, b, eps=1e-5)
    return (nt.rms_norm(x, w, eps=1e-6),)


@pytest.mark.parametrize("op,dtype,M,N", CASES)
def test_bitwise_stable_over_many_runs(op, dtype, M, N):
    gen = torch.Generator(device="cuda").manual_seed(M * 7919 + N)
    w = (torch.randn(N, device="cuda", generator=gen) * 0.3 + 1).to(dtype)
    b = (torch.randn(N, device="cuda", generator=gen) * 0.3).to(dtype)
    say(f"case stability {op} {dtype} {M}x{N}")
    # fresh inputs: two runs of each agree
    for trial in range(40):
        x = (torch.randn(M, N, device="cuda", generator=gen) * (1 + trial % 5)).to(dtype)
        a, c = run(op, x, w, b), run(op, x, w, b)
        for u, v in zip(a, c):
            assert torch.equal(u.view(torch.int8), v.view(torch.int8)), f"trial {trial}"
    # one input, many runs back to back: every run equals the first
    x = torch.randn(M, N, device="cuda", generator=gen).to(dtype)
    ref = run(op, x, w, b)
    outs = [run(op, x, w, b) for _ in range(200)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        for u, v in zip(ref, o):
            assert torch.equal(u.view(torch.int8), v.view(torch.int8)), f"repeat {i}"
