"""Comparator (ulp / rounding) and seeded input generator checks (CPU only)."""
import numpy as np
import pytest

from oracle import compare
import workloads


def test_round_to_f32_matches_numpy_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-40, 38, 20000),
                        [0.0, -0.0, 1e-46, 1.5e-45, 3.4e38, 3.5e38, 1e300]])
    got = compare.round_to(v, "f32")
    with np.errstate(over="ignore"):
        want = v.astype(np.float32).view(np.uint32)
    assert np.array_equal(got, want)


def test_round_to_f16_matches_numpy_cast():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
                        [0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -24 * 1.5]])
    got = compare.round_to(v, "f16")
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_round_to_bf16_is_nearest_even():
    rng = np.random.default_rng(3)
    v = rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)
    bits = compare.round_to(v, "bf16")
    val = compare.bits_to_f64(bits, "bf16")
    # neighbours one unit away on either side
    up = compare.bits_to_f64(bits + 1, "bf16")
    dn = compare.bits_to_f64(bits - 1, "bf16")
    d = np.abs(val - v)
    assert np.all(d <= np.abs(up - v)) and np.all(d <= np.abs(dn - v))


def test_round_to_bf16_hand_patterns():
    cases = {1.0: 0x3F80, 1.0078125: 0x3F81,
             1.00390625: 0x3F80,     # halfway 0x3F80/0x3F81 -> even
             1.01171875: 0x3F82,     # halfway 0x3F81/0x3F82 -> even
             -2.0: 0xC000, 0.0: 0x0000, 3.5e38: 0x7F80}
    for v, b in cases.items():
        assert int(compare.round_to(np.array([v]), "bf16")[0]) == b, v
    # the double-rounding trap: just above a bf16 midpoint, below an f32 one
    v = 1.00390625 + 2.0 ** -40
    assert int(compare.round_to(np.array([v]), "bf16")[0]) == 0x3F81


def test_ordinal_distances():
    o = lambda b, dt: int(compare.ordinal(np.array([b]), dt)[0])
    assert o(0x3F81, "bf16") - o(0x3F80, "bf16") == 1
    assert o(0x8000, "bf16") == o(0x0000, "bf16") == 0
    assert o(0x3F80, "bf16") - o(0x3F7F, "bf16") == 1          # across a binade
    assert o(0xBF80, "bf16") - o(0xBF81, "bf16") == 1          # negative side
    assert o(0x0001, "f16") - o(0x8001, "f16") == 2            # +-min subnormal
    assert o(0x3C01, "f16") - o(0x3C00, "f16") == 1
    assert o(0x3F800001, "f32") - o(0x3F800000, "f32") == 1


def test_ulp_distance_and_nan():
    ref = np.array([1.0, np.nan, 0.5])
    gpu = compare.round_to(np.array([1.0078125, np.nan, 0.5]), "bf16")
    d = compare.ulp_distance(gpu, ref, "bf16")
    assert list(d) == [1, 0, 0]


def test_max_rel_err_zero_rules():
    assert compare.max_rel_err([0.0, 1.0], [0.0, 1.0]) == 0.0
    assert compare.max_rel_err([1e-30, 1.0], [0.0, 1.0]) == float("inf")
    assert compare.max_rel_err([1.00001], [1.0]) == pytest.approx(1e-5)


def test_bf16_encoder_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(4)
    f = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    ours = workloads.to_bf16_bits(f)
    theirs = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_generators_deterministic_and_blockwise():
    a = workloads.normal_rows(7, 100, 33, "bf16", block_rows=7)
    b = workloads.normal_rows(7, 100, 33, "bf16", block_rows=100)
    c = workloads.normal_rows(7, 100, 33, "bf16", block_rows=13)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    sub = workloads.normal_rows(7, 100, 33, "bf16", block_rows=9, rows=[0, 5, 64, 99])
    assert np.array_equal(sub, a[[0, 5, 64, 99]])


@pytest.mark.parametrize("name", [w.name for w in workloads.WORKLOADS])
def test_workload_row_subset_matches_prefix(name):
    w = workloads.BY_NAME[name]
    M = min(w.M, 64)
    full = w.make(M=M)
    rows = [0, 1, M // 2, M - 1]
    sub = w.make(rows=rows, M=M)
    assert np.array_equal(sub["x"], full["x"][rows])


def test_workload_structure():
    c = workloads.BY_NAME["causal_softmax_bf16"]
    rows = [0, 1, 4095, 4096, 8191]
    x = c.make(rows=rows, M=8192)["x"]
    for i, r in enumerate(rows):
        q = r % 4096
        assert np.all(x[i, q + 1:] == 0xFF80) and not np.any(x[i, :q + 1] == 0xFF80)
    v = workloads.BY_NAME["vocab_softmax_f32"].make(rows=[0, 63])
    for i in range(2):
        assert np.sum(v["x"][i] == 30.0) == 8
        assert len(set(v["spikes"][i])) == 8
    ln = workloads.BY_NAME["layernorm_f16_4096"].make(M=8)
    assert ln["x"].dtype == np.uint16 and ln["gamma"].shape == (4096,)


def test_algorithmic_bytes():
    b = {w.name: w.algorithmic_bytes() for w in workloads.WORKLOADS}
    assert b["softmax_f32_1024x781"] == 2 * 1024 * 781 * 4
    assert b["layernorm_f16_4096"] == 2 * 4096 * 4096 * 2 + 2 * 4096 * 2 + 2 * 4096 * 4
    assert b["rmsnorm_bf16_16384x8192"] == 2 * 16384 * 8192 * 2 + 8192 * 2
    assert b["causal_softmax_bf16"] == 2 * 131072 * 4096 * 2
    assert b["vocab_softmax_f32"] == 2 * 64 * 262144 * 4


def test_f32_errors_reading_below_the_normal_range():
    """The fp32 bar: relative 1e-5; below 2^-126 also one 2^-149 quantum
    from the correctly rounded value (where the relative bar is finer than
    the format)."""
    q = 2.0 ** -149

    def bits(v):
        return np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32)

    ref = np.array([1.0, 2.0 ** -140, 3.25 * q, 0.4 * q, 0.0, 2.0 ** -126, 2.0 ** -127])
    near_top = 2.0 ** -127 * (1 + 8e-6)         # relative 8e-6 near the top: 2^22 * 8e-6 = 33 quanta
    good = bits([1.0 + 5e-6, 2.0 ** -140 + q, 3.0 * q, 0.0, 0.0, 2.0 ** -126 - q, near_top])
    rel, quanta = compare.f32_errors(good, ref)
    assert rel <= 1e-5 and quanta <= 1.0, (rel, quanta)
    # relative 2e-5 near the top of the subnormal range is beyond both
    assert compare.f32_errors(bits([1.0, 2.0 ** -140, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127 * (1 + 2e-5)]),
                              ref)[1] > 1.0
    # a flushed subnormal (2^-140 is 512 quanta) fails
    assert compare.f32_errors(bits([1.0, 0.0, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127]), ref)[1] == 512.0
    # two quanta off at 2^-140 (relative 2^-8) fails; non-zero where the reference is exactly 0 fails
    assert compare.f32_errors(bits([1.0, 2.0 ** -140 + 2 * q, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127]),
                              ref)[1] == 2.0
    assert compare.f32_errors(bits([1.0, 2.0 ** -140, 3 * q, 0.0, q, 2.0 ** -126, 2.0 ** -127]), ref)[0] == float("inf")
    # the normal range keeps the relative bar
    assert compare.f32_errors(bits([1.0 + 3e-5, 2.0 ** -140, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127]), ref)[0] > 1e-5
    # NaN where the reference is finite fails either part
    assert compare.f32_errors(bits([np.nan, 2.0 ** -140, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127]),
                              ref)[0] == float("inf")
    assert not compare.f32_errors(bits([1.0, np.nan, 3 * q, 0.0, 0.0, 2.0 ** -126, 2.0 ** -127]), ref)[1] <= 1.0


def test_ulp_of_and_attention_bar():
    """ulp_of: the spacing at the correctly rounded value (binade edges,
    subnormals); the attention bar |y - ref| <= ulp + 2^-12 * A."""
    assert list(compare.ulp_of(np.array([1.0, 1.9, 2.0, 0.75, 2.0 ** -130]), "bf16")) == \
        [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -133]
    assert list(compare.ulp_of(np.array([1.0, 1000.0, 2.0 ** -20]), "f16")) == [2.0 ** -10, 2.0 ** -1, 2.0 ** -24]
    ref = np.array([1.0, 0.001, -0.5])
    A = np.array([1.0, 0.8, 0.5])
    bits = compare.round_to(ref, "bf16")
    assert compare.attention_errors(bits, ref, A, "bf16") <= 0.5
    # an output that cancels: 0.001 +- 2^-12 * 0.8 is inside, twice that is not
    near = compare.round_to(np.array([1.0, 0.001 + 1.5e-4, -0.5]), "bf16")
    far = compare.round_to(np.array([1.0, 0.001 + 5e-4, -0.5]), "bf16")
    assert compare.attention_errors(near, ref, A, "bf16") <= 1.0 < compare.attention_errors(far, ref, A, "bf16")
    nan = bits.copy()
    nan[0] = 0x7FC0
    assert compare.attention_errors(nan, ref, A, "bf16") == float("inf")
