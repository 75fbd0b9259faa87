"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with the fact it checks.  They are
run against the real oracle (``test_oracle_pins.py``) and against
deliberately broken builds of it (``test_oracle_mutants.py``), which must
each fail at least one pin.

Expected values never come from the oracle itself: they are closed forms
(written through a different formula than the oracle's), invariants, the
independent pure-Python definition in ``oracle/brute.py``, exhaustive decoder
checks against numpy's binary16 codec, or PyTorch's float64 CPU routines
(an independent library implementation of the same definitions).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32_EPS5 = float(np.float32(1e-5))   # eps as the C ABI receives it (a float)
F32_EPS6 = float(np.float32(1e-6))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-300)))


def _f32(rows):
    return np.ascontiguousarray(np.asarray(rows, dtype=np.float32))


def _rng_rows(seed, M, N, dt, scale=1.0, loc=0.0):
    rng = np.random.default_rng(seed)
    v = (rng.standard_normal((M, N)) * scale + loc).astype(np.float32)
    if dt == "f32":
        return v
    if dt == "f16":
        return v.astype(np.float16).view(np.uint16)
    u = v.view(np.uint32)
    return ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _decode_py(bits_row, dt):
    if dt == "f32":
        return [float(v) for v in bits_row]
    return [brute.decode16(int(b), dt) for b in bits_row]


# ----------------------------------------------------------------------------
# decoders
# ----------------------------------------------------------------------------

def pin_decode_f16_exhaustive(lib):
    """Every binary16 bit pattern decodes to numpy's binary16 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.empty(65536, dtype=np.float64)
    assert lib.or_decode(65536, oracle.F16, bits.ctypes.data, got.ctypes.data) == 0
    ref = bits.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"{(~same).sum()} fp16 patterns decode wrongly"


def pin_decode_bf16_exhaustive(lib):
    """Every bfloat16 pattern decodes to the binary32 with the same top half."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = np.empty(65536, dtype=np.float64)
    assert lib.or_decode(65536, oracle.BF16, bits.ctypes.data, got.ctypes.data) == 0
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f"{(~same).sum()} bf16 patterns decode wrongly"


# ----------------------------------------------------------------------------
# softmax
# ----------------------------------------------------------------------------

def pin_softmax_two_logistic(lib):
    """softmax([0, 1]) is the logistic function: [1/(1+e), 1/(1+e^-1)]."""
    y = oracle.softmax(_f32([[0.0, 1.0]]), "f32", lib=lib)[0]
    want = [1.0 / (1.0 + math.e), 1.0 / (1.0 + math.exp(-1.0))]
    assert _rel(y, want) < 1e-15, (y, want)


def pin_softmax_three_closed_form(lib):
    """softmax([0, 1, 2]) = [1, e, e^2] / (1 + e + e^2) (geometric series)."""
    y = oracle.softmax(_f32([[0.0, 1.0, 2.0]]), "f32", lib=lib)[0]
    den = (math.e ** 3 - 1.0) / (math.e - 1.0)
    want = [1.0 / den, math.e / den, math.e ** 2 / den]
    assert _rel(y, want) < 1e-15, (y, want)


def pin_softmax_large_logits(lib):
    """Huge logits must not overflow: softmax([1000, 999]) = logistic(+-1)."""
    y = oracle.softmax(_f32([[1000.0, 999.0]]), "f32", lib=lib)[0]
    want = [1.0 / (1.0 + math.exp(-1.0)), 1.0 / (1.0 + math.e)]
    assert _rel(y, want) < 1e-15, (y, want)


def pin_softmax_uniform(lib):
    """A constant row of length N gives 1/N everywhere."""
    for N in (1, 2, 781, 4096):
        y = oracle.softmax(np.full((1, N), 0.375, dtype=np.float32), "f32", lib=lib)
        assert _rel(y, np.full((1, N), 1.0 / N)) < 1e-14, N


def pin_softmax_sums_to_one(lib):
    """Every row of a softmax sums to 1."""
    for dt in ("f32", "f16", "bf16"):
        x = _rng_rows(11, 64, 781, dt, scale=3.0)
        y = oracle.softmax(x, dt, lib=lib)
        assert np.max(np.abs(y.sum(axis=1) - 1.0)) < 1e-13, dt


def pin_softmax_ratio_is_exp_difference(lib):
    """y_i / y_j = exp(x_i - x_j): checks the base of the exponential."""
    x = _rng_rows(12, 4, 50, "f32")
    y = oracle.softmax(x, "f32", lib=lib)
    xd = x.astype(np.float64)
    want = np.exp(xd[:, 1:] - xd[:, :1])
    assert _rel(y[:, 1:] / y[:, :1], want) < 1e-13


def pin_softmax_shift_invariance(lib):
    """softmax(x + c) = softmax(x) for inputs where x + c is exact."""
    rng = np.random.default_rng(13)
    cases = [("f32", 2.0 ** -10, 8192, (16.0, -64.0)),
             ("f16", 2.0 ** -6, 512, (16.0,)),
             ("bf16", 2.0 ** -3, 128, (16.0,))]
    for dt, q, kmax, shifts in cases:
        k = rng.integers(-kmax + 1, kmax, size=(8, 300))
        base = (k * q).astype(np.float64)
        for c in shifts:
            a = _encode(base, dt)
            b = _encode(base + c, dt)
            assert np.array_equal(oracle.decode(b, dt), oracle.decode(a, dt) + c)
            ya = oracle.softmax(a, dt, lib=lib)
            yb = oracle.softmax(b, dt, lib=lib)
            assert _rel(ya, yb) < 1e-14, (dt, c)


def _encode(v64, dt):
    f = np.asarray(v64, dtype=np.float32)
    if dt == "f32":
        return np.ascontiguousarray(f)
    if dt == "f16":
        return f.astype(np.float16).view(np.uint16)
    u = f.view(np.uint32)
    return ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def pin_softmax_padding_neutral(lib):
    """A row padded with -inf to the next power of two keeps its softmax on
    the real entries and gets exactly 0 on the padding."""
    with open(os.path.join(GOLDEN, "masked_fill_identities.json")) as f:
        ident = json.load(f)
    assert ident["max_identity"] == "-inf" and ident["exp_of_neg_inf"] == 0.0
    x = _rng_rows(14, 3, 781, "f32")
    pad = np.full((3, 1024), -np.inf, dtype=np.float32)
    pad[:, :781] = x
    y = oracle.softmax(x, "f32", lib=lib)
    yp = oracle.softmax(pad, "f32", lib=lib)
    assert np.array_equal(yp[:, :781], y)
    assert np.all(yp[:, 781:] == 0.0)


def pin_softmax_causal_rows(lib):
    """Causally masked rows: row q has exactly q+1 non-zeros, row 0 is one-hot."""
    N = 64
    x = _rng_rows(15, N, N, "bf16", scale=3.0)
    k = np.arange(N)[None, :]
    q = np.arange(N)[:, None]
    x[k > q] = 0xFF80
    y = oracle.softmax(x, "bf16", lib=lib)
    assert np.array_equal((y != 0).sum(axis=1), np.arange(N) + 1)
    assert y[0, 0] == 1.0 and np.all(y[0, 1:] == 0.0)
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) < 1e-14


def pin_softmax_special_rows(lib):
    """N=1 gives 1; an all -inf row gives NaN (literal -inf - -inf)."""
    assert oracle.softmax(_f32([[-3.5]]), "f32", lib=lib)[0, 0] == 1.0
    y = oracle.softmax(np.full((1, 5), -np.inf, dtype=np.float32), "f32", lib=lib)
    assert np.all(np.isnan(y))


def pin_softmax_brute(lib):
    """oracle.c agrees with the pure-Python fsum definition on tiny rows."""
    for dt in ("f32", "f16", "bf16"):
        for N in list(range(1, 65)) + [127, 255, 257, 781, 1500]:
            x = _rng_rows(1000 + N, 2, N, dt, scale=2.0)
            y = oracle.softmax(x, dt, lib=lib)
            for r in range(2):
                want = brute.softmax_row(_decode_py(x[r], dt))
                assert _rel(y[r], want) < 1e-13, (dt, N)


def pin_softmax_torch(lib):
    """oracle.c agrees with torch.softmax in float64 on the CPU."""
    import torch
    for dt in ("f32", "f16", "bf16"):
        x = _rng_rows(16, 16, 1500, dt, scale=3.0)
        y = oracle.softmax(x, dt, lib=lib)
        xt = torch.from_numpy(oracle.decode(x, dt))
        assert _rel(y, torch.softmax(xt, dim=-1).numpy()) < 1e-13, dt


def pin_softmax_online_matches_plain(lib):
    """The online (running max, rescaled denominator) form equals the plain
    softmax for every block size, including leading fully masked blocks."""
    x = _rng_rows(17, 6, 1000, "f32", scale=2.0)
    x[1, :300] = -np.inf           # leading masked blocks
    x[2, 500:] = -np.inf           # trailing masked blocks
    x[3, ::7] = 30.0               # spikes
    x[4, 999] = 40.0               # late maximum forces a rescale
    y = oracle.softmax(x, "f32", lib=lib)
    for block in (1, 2, 7, 64, 128, 999, 1000, 4096):
        yo = oracle.softmax_online(x, "f32", block, lib=lib)
        assert _rel(yo, y) < 1e-13, block


# ----------------------------------------------------------------------------
# LayerNorm
# ----------------------------------------------------------------------------

def pin_layernorm_hand_case(lib):
    """[1, 2, 3, 4]: mean 5/2, biased variance 5/4, y = [-3, -1, 1, 3]/sqrt(5)."""
    x = _f32([[1.0, 2.0, 3.0, 4.0]])
    y, mu, rs = oracle.layernorm(x, "f32", 0.0, lib=lib)
    s5 = math.sqrt(5.0)
    assert mu[0] == 2.5
    assert _rel(rs, [2.0 / s5]) < 1e-15
    assert _rel(y[0], [-3 / s5, -1 / s5, 1 / s5, 3 / s5]) < 1e-15
    _, _, rs_e = oracle.layernorm(x, "f32", 1e-5, lib=lib)
    assert _rel(rs_e, [1.0 / math.sqrt(1.25 + F32_EPS5)]) < 1e-15


def pin_layernorm_biased_variance(lib):
    """[0, 2] has biased variance 1 (not 2): y = [-1, 1] with eps = 0."""
    y, mu, rs = oracle.layernorm(_f32([[0.0, 2.0]]), "f32", 0.0, lib=lib)
    assert mu[0] == 1.0 and rs[0] == 1.0 and list(y[0]) == [-1.0, 1.0]


def pin_layernorm_unit_moments(lib):
    """gamma=1, beta=0: mean(y) = 0 and mean(y^2) = var / (var + eps)."""
    x = _rng_rows(21, 32, 4096, "f16", loc=3.0)
    y, mu, rs = oracle.layernorm(x, "f16", 1e-5, lib=lib)
    xd = oracle.decode(x, "f16")
    var = ((xd - xd.mean(axis=1, keepdims=True)) ** 2).mean(axis=1)
    assert np.max(np.abs(y.mean(axis=1))) < 1e-12
    assert _rel((y ** 2).mean(axis=1), var / (var + F32_EPS5)) < 1e-12


def pin_layernorm_affine_invariance(lib):
    """With eps = 0, y is unchanged by x -> a*x + c (a > 0); mean -> a*mean + c
    and rstd -> rstd / a."""
    rng = np.random.default_rng(22)
    x = (rng.integers(-4000, 4000, size=(8, 300)) * 2.0 ** -10).astype(np.float32)
    y, mu, rs = oracle.layernorm(x, "f32", 0.0, lib=lib)
    x2 = (x.astype(np.float64) * 4.0 + 8.0).astype(np.float32)     # exact
    assert np.array_equal(x2.astype(np.float64), x.astype(np.float64) * 4.0 + 8.0)
    y2, mu2, rs2 = oracle.layernorm(x2, "f32", 0.0, lib=lib)
    assert _rel(y2, y) < 1e-12
    assert _rel(mu2, mu * 4.0 + 8.0) < 1e-12
    assert _rel(rs2, rs / 4.0) < 1e-12


def pin_layernorm_long_periodic_row(lib):
    """A long row that repeats (0, 1, 1) in bf16 (3 * 2^22 elements) has mean
    exactly 2/3 and biased variance exactly 2/9, so rstd = 1/sqrt(2/9 + eps)
    and y = (x - 2/3) * rstd.  A plain running sum of its squared deviations
    drifts by about 1e-10 relative (its few distinct terms round the same
    way again and again); the oracle's sums must stay within a few
    roundings."""
    reps = 1 << 22
    x = np.tile(np.array([0x0000, 0x3F80, 0x3F80], dtype=np.uint16), reps).reshape(1, 3 * reps)
    y, mu, rs = oracle.layernorm(x, "bf16", 1e-5, lib=lib)
    want = 1.0 / math.sqrt(2.0 / 9.0 + F32_EPS5)
    assert _rel(mu, [2.0 / 3.0]) < 1e-15
    assert _rel(rs, [want]) < 1e-13
    assert _rel(y[0, :3], [-2.0 / 3.0 * want, 1.0 / 3.0 * want, 1.0 / 3.0 * want]) < 1e-13


def pin_rmsnorm_long_periodic_row(lib):
    """RMSNorm of a long row repeating (a, a, b) with a = fp32(0.1), b =
    fp32(0.3) (3 * 2^22 elements): the mean square is exactly (2a^2 + b^2)/3
    (computed here in rationals), so y = x / sqrt(that + eps).  The squares
    carry bits below the last place of the running sum, and a plain running
    sum drifts by about 5e-11 relative; the oracle's stays within a few
    roundings."""
    from fractions import Fraction
    reps = 1 << 22
    a, b = np.float32(0.1), np.float32(0.3)
    x = np.tile(np.array([a, a, b], dtype=np.float32), reps).reshape(1, 3 * reps)
    y = oracle.rmsnorm(x, "f32", 1e-6, lib=lib)
    ms = float((2 * Fraction(float(a)) ** 2 + Fraction(float(b)) ** 2) / 3)
    inv = 1.0 / math.sqrt(ms + float(np.float32(1e-6)))
    assert _rel(y[0, :3], [float(a) * inv, float(a) * inv, float(b) * inv]) < 1e-14


def pin_layernorm_constant_row(lib):
    """A constant row has variance 0: rstd = 1/sqrt(eps) and y = beta."""
    beta = np.array([0.5, -0.25, 2.0], dtype=np.float32)
    gamma = np.array([3.0, 4.0, 5.0], dtype=np.float32)
    y, mu, rs = oracle.layernorm(np.full((1, 3), 7.0, np.float32), "f32", 1e-5,
                                 gamma=gamma, beta=beta, lib=lib)
    assert mu[0] == 7.0
    assert _rel(rs, [1.0 / math.sqrt(F32_EPS5)]) < 1e-15
    assert np.array_equal(y[0], beta.astype(np.float64))


def pin_layernorm_single_element(lib):
    """N = 1: y = beta, mean = x, rstd = 1/sqrt(eps)."""
    y, mu, rs = oracle.layernorm(_f32([[2.5]]), "f32", 1e-5,
                                 gamma=np.array([3.0], np.float32),
                                 beta=np.array([-1.5], np.float32), lib=lib)
    assert y[0, 0] == -1.5 and mu[0] == 2.5
    assert _rel(rs, [1.0 / math.sqrt(F32_EPS5)]) < 1e-15


def pin_layernorm_affine_columns(lib):
    """gamma and beta act per column j: a ramp gamma_j = j+1 and beta_j = -j
    turn column j of the plain result into (j+1)*y_j - j."""
    x = _rng_rows(23, 4, 40, "f32")
    N = 40
    g = np.arange(1, N + 1, dtype=np.float32)
    b = -np.arange(N, dtype=np.float32)
    y0, _, _ = oracle.layernorm(x, "f32", 1e-5, lib=lib)
    y1, _, _ = oracle.layernorm(x, "f32", 1e-5, gamma=g, beta=b, lib=lib)
    assert np.max(np.abs(y1 - (y0 * g + b))) < 1e-12


def pin_layernorm_brute(lib):
    for dt in ("f32", "f16", "bf16"):
        for N in list(range(1, 65)) + [127, 255, 257, 781, 1500]:
            x = _rng_rows(2000 + N, 2, N, dt, loc=2.0)
            g = _rng_rows(3000 + N, 1, N, dt, scale=0.3, loc=1.0)[0]
            b = _rng_rows(4000 + N, 1, N, dt, scale=0.3)[0]
            y, mu, rs = oracle.layernorm(x, dt, 1e-5, gamma=g, beta=b, lib=lib)
            gd, bd = _decode_py(g, dt), _decode_py(b, dt)
            for r in range(2):
                yw, muw, rsw = brute.layernorm_row(_decode_py(x[r], dt), F32_EPS5, gd, bd)
                scale = np.abs(np.asarray(yw)) + 1.0
                assert np.max(np.abs(y[r] - yw) / scale) < 1e-13, (dt, N)
                assert abs(mu[r] - muw) <= 1e-13 * max(1.0, abs(muw)), (dt, N)
                assert _rel([rs[r]], [rsw]) < 1e-13, (dt, N)


def pin_layernorm_torch(lib):
    """oracle.c agrees with torch.nn.functional.layer_norm in float64."""
    import torch
    for dt in ("f32", "f16", "bf16"):
        x = _rng_rows(24, 16, 1500, dt, loc=-4.0)
        g = _rng_rows(25, 1, 1500, dt, scale=0.3, loc=1.0)[0]
        b = _rng_rows(26, 1, 1500, dt, scale=0.3)[0]
        y, mu, rs = oracle.layernorm(x, dt, 1e-5, gamma=g, beta=b, lib=lib)
        xt = torch.from_numpy(oracle.decode(x, dt))
        ref = torch.nn.functional.layer_norm(
            xt, (1500,), torch.from_numpy(oracle.decode(g, dt)),
            torch.from_numpy(oracle.decode(b, dt)), eps=F32_EPS5).numpy()
        assert np.max(np.abs(y - ref) / (np.abs(ref) + 1.0)) < 1e-12, dt
        assert _rel(mu, xt.mean(dim=1).numpy()) < 1e-12, dt


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

def pin_rmsnorm_hand_cases(lib):
    """[3, 4]: mean square 12.5, y = [3, 4] / sqrt(12.5 + eps);
    [1, 1, 1, 1] with eps: every output is 1/sqrt(1 + eps)."""
    y = oracle.rmsnorm(_f32([[3.0, 4.0]]), "f32", 0.0, lib=lib)[0]
    assert _rel(y, [3.0 / math.sqrt(12.5), 4.0 / math.sqrt(12.5)]) < 1e-15
    y = oracle.rmsnorm(_f32([[3.0, 4.0]]), "f32", 1e-6, lib=lib)[0]
    d = math.sqrt(12.5 + F32_EPS6)
    assert _rel(y, [3.0 / d, 4.0 / d]) < 1e-15
    y = oracle.rmsnorm(np.ones((1, 4), np.float32), "f32", 1e-6, lib=lib)[0]
    assert _rel(y, [1.0 / math.sqrt(1.0 + F32_EPS6)] * 4) < 1e-15


def pin_rmsnorm_unit_mean_square(lib):
    """Unit weight: mean(y^2) = ms / (ms + eps)."""
    x = _rng_rows(31, 32, 8192, "bf16")
    y = oracle.rmsnorm(x, "bf16", 1e-6, lib=lib)
    xd = oracle.decode(x, "bf16")
    ms = (xd ** 2).mean(axis=1)
    assert _rel((y ** 2).mean(axis=1), ms / (ms + F32_EPS6)) < 1e-12


def pin_rmsnorm_scale_invariance(lib):
    """With eps = 0, y is unchanged by x -> a*x (a > 0)."""
    x = _rng_rows(32, 8, 300, "f32")
    y = oracle.rmsnorm(x, "f32", 0.0, lib=lib)
    y2 = oracle.rmsnorm((x * np.float32(8.0)).astype(np.float32), "f32", 0.0, lib=lib)
    assert _rel(y2, y) < 1e-13


def pin_rmsnorm_weight_columns(lib):
    """The weight acts per column: w_j = j+1 scales column j by j+1."""
    x = _rng_rows(33, 4, 40, "f32")
    w = np.arange(1, 41, dtype=np.float32)
    y0 = oracle.rmsnorm(x, "f32", 1e-6, lib=lib)
    y1 = oracle.rmsnorm(x, "f32", 1e-6, weight=w, lib=lib)
    assert _rel(y1, y0 * w) < 1e-14


def pin_rmsnorm_brute(lib):
    for dt in ("f32", "f16", "bf16"):
        for N in list(range(1, 65)) + [127, 255, 257, 781, 1500]:
            x = _rng_rows(5000 + N, 2, N, dt)
            w = _rng_rows(6000 + N, 1, N, dt, scale=0.3, loc=1.0)[0]
            y = oracle.rmsnorm(x, dt, 1e-6, weight=w, lib=lib)
            wd = _decode_py(w, dt)
            for r in range(2):
                want = brute.rmsnorm_row(_decode_py(x[r], dt), F32_EPS6, wd)
                assert _rel(y[r], want) < 1e-13, (dt, N)


def pin_rmsnorm_torch(lib):
    """oracle.c agrees with torch.nn.functional.rms_norm in float64."""
    import torch
    for dt in ("f32", "f16", "bf16"):
        x = _rng_rows(34, 16, 1500, dt)
        w = _rng_rows(35, 1, 1500, dt, scale=0.3, loc=1.0)[0]
        y = oracle.rmsnorm(x, dt, 1e-6, weight=w, lib=lib)
        ref = torch.nn.functional.rms_norm(
            torch.from_numpy(oracle.decode(x, dt)), (1500,),
            torch.from_numpy(oracle.decode(w, dt)), eps=F32_EPS6).numpy()
        assert _rel(y, ref) < 1e-13, dt


# ----------------------------------------------------------------------------
# residual add (fused add + norm): h = x + r stored in the input type
# ----------------------------------------------------------------------------

def _wide_pairs(seed, n, dt):
    """Random stored values of `dt` spread over many binades (subnormals,
    exact cancellations and large exponent gaps included), as raw storage."""
    rng = np.random.default_rng(seed)
    if dt == "f32":
        mag = rng.standard_normal(n) * np.exp2(rng.integers(-140, 100, n).astype(np.float64))
        x = mag.astype(np.float32)
        r = (rng.standard_normal(n) * np.exp2(rng.integers(-140, 100, n).astype(np.float64))).astype(np.float32)
        r[: n // 8] = -x[: n // 8]                       # exact cancellation
        return np.nan_to_num(x, posinf=1.0, neginf=-1.0), np.nan_to_num(r, posinf=1.0, neginf=-1.0)
    # every 16-bit pattern except inf/NaN, paired at random
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp_all_ones = (bits & (0x7C00 if dt == "f16" else 0x7F80)) == (0x7C00 if dt == "f16" else 0x7F80)
    finite = bits[~exp_all_ones]
    x = rng.choice(finite, n)
    r = rng.choice(finite, n)
    r[: n // 8] = x[: n // 8] ^ np.uint16(0x8000)        # exact cancellation
    return x, r


def pin_add_matches_ieee_libraries(lib):
    """The stored h (oracle sum rounded once) equals the IEEE sum computed by
    independent libraries: numpy float32 and float16 addition, torch
    bfloat16 addition on the CPU (each rounds a float32 sum once, which for
    these types equals rounding the exact sum)."""
    import torch
    from oracle import compare
    for dt in ("f32", "f16", "bf16"):
        x, r = _wide_pairs(71, 400000, dt)
        got = compare.round_to(oracle.add(x, r, dt, lib=lib), dt)
        if dt == "f32":
            want = (x + r).view(np.uint32)
        elif dt == "f16":
            with np.errstate(over="ignore"):       # sums beyond 65504 round to inf on both sides
                want = (x.view(np.float16) + r.view(np.float16)).view(np.uint16)
        else:
            tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
            tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
            want = (tx + tr).view(torch.int16).numpy().view(np.uint16)
        same = (got == want) | ((compare.ordinal(got, dt) == 0) & (compare.ordinal(want, dt) == 0))
        assert same.all(), (dt, int((~same).sum()))


def pin_add_norm_is_norm_of_stored_sum(lib):
    """The fused definitions are the norms of the stored sum: h equals the
    numpy / torch IEEE sum, and y (and LayerNorm's mean) equal the
    pure-Python norms of that h."""
    for dt in ("f32", "f16", "bf16"):
        for N in (1, 7, 64, 781):
            x = _rng_rows(7000 + N, 3, N, dt, scale=2.0)
            r = _rng_rows(7100 + N, 3, N, dt, scale=0.5, loc=-1.0)
            w = _rng_rows(7200 + N, 1, N, dt, scale=0.3, loc=1.0)[0]
            b = _rng_rows(7300 + N, 1, N, dt, scale=0.3)[0]
            h, y = oracle.add_rmsnorm(x, r, dt, 1e-6, weight=w, lib=lib)
            h2, y2, mean, rstd = oracle.add_layernorm(x, r, dt, 1e-5, gamma=w, beta=b, lib=lib)
            if dt == "f32":
                want = (x + r)
            elif dt == "f16":
                want = (x.view(np.float16) + r.view(np.float16)).view(np.uint16)
            else:
                import torch
                tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
                tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
                want = (tx + tr).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(np.asarray(h).view(np.uint8), np.asarray(want).view(np.uint8)), (dt, N)
            assert np.array_equal(np.asarray(h2).view(np.uint8), np.asarray(want).view(np.uint8)), (dt, N)
            wd, bd = _decode_py(w, dt), _decode_py(b, dt)
            for i in range(3):
                hd = _decode_py(np.asarray(want)[i], dt)
                assert _rel(y[i], brute.rmsnorm_row(hd, F32_EPS6, wd)) < 1e-13, (dt, N)
                yl, ml, rl = brute.layernorm_row(hd, F32_EPS5, wd, bd)
                assert _rel(y2[i], yl) < 1e-12 and _rel([mean[i]], [ml]) < 1e-12, (dt, N)


# ----------------------------------------------------------------------------
# causal scaled softmax (attention scores with the future keys masked)
# ----------------------------------------------------------------------------

_NAN_BITS = {"f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def _causal_cases():
    # (M, N, queries, offset): square causal, wrap over heads, bottom-right
    # alignment (offset = N - queries), offsets past the row
    return [(8, 8, 8, 0), (12, 5, 5, 0), (7, 33, 7, 26), (6, 40, 3, 1), (5, 17, 5, 100), (9, 1, 4, 0)]


def pin_softmax_causal_matches_torch_masked(lib):
    """Causal scaled softmax = torch.softmax (float64) of scale*x with the
    masked keys set to -inf."""
    import torch
    for dt in ("f32", "f16", "bf16"):
        for (M, N, Q, off) in _causal_cases():
            for scale in (1.0, 0.125, 3.0):
                x = _rng_rows(900 + M + N + off, M, N, dt, scale=3.0)
                y = oracle.softmax_causal(x, dt, scale, Q, off, lib=lib)
                xd = torch.from_numpy(oracle.decode(x, dt)) * float(np.float32(scale))
                k = torch.arange(N)[None, :]
                q = (torch.arange(M) % Q)[:, None]
                ref = torch.softmax(xd.masked_fill(k > q + off, float("-inf")), dim=1).numpy()
                assert _rel(y, ref) < 1e-13 or np.abs(y - ref).max() < 1e-15, (dt, M, N, Q, off, scale)
                assert np.all(y[np.broadcast_to((k > q + off).numpy(), y.shape)] == 0.0)


def pin_softmax_causal_never_reads_masked(lib):
    """NaN planted in every masked input changes nothing: masked keys are not
    read, their outputs are exactly 0."""
    for dt in ("f32", "f16", "bf16"):
        M, N, Q, off = 10, 24, 10, 3
        x = _rng_rows(950, M, N, dt, scale=2.0)
        clean = oracle.softmax_causal(x, dt, 0.5, Q, off, lib=lib)
        k = np.arange(N)[None, :]
        masked = k > (np.arange(M) % Q)[:, None] + off
        x2 = x.copy()
        x2[masked] = np.float32(np.nan) if dt == "f32" else _NAN_BITS[dt]
        dirty = oracle.softmax_causal(x2, dt, 0.5, Q, off, lib=lib)
        assert np.array_equal(clean, dirty), dt
        assert np.all(dirty[masked] == 0.0) and np.all(np.isfinite(dirty))


def pin_softmax_causal_closed_forms(lib):
    """Query 0 sees only key 0: [1, 0, ...]; a constant row gives 1/(q+1)
    over the visible keys; two visible keys a, b give the logistic of
    scale*(b - a)."""
    x = np.full((4, 6), 2.5, dtype=np.float32)
    y = oracle.softmax_causal(x, "f32", 0.7, 4, lib=lib)
    for q in range(4):
        assert np.all(y[q, : q + 1] == y[q, 0]) and abs(y[q, 0] - 1.0 / (q + 1)) < 1e-15
        assert np.all(y[q, q + 1:] == 0.0)
    x = np.array([[0.0, 0.0, 9.0], [1.0, 3.0, -5.0]], dtype=np.float32)
    y = oracle.softmax_causal(x, "f32", 0.5, 2, lib=lib)
    assert y[0, 0] == 1.0 and y[0, 1] == 0.0 and y[0, 2] == 0.0
    want = 1.0 / (1.0 + math.exp(-0.5 * 2.0))
    assert abs(y[1, 1] - want) < 1e-15 and abs(y[1, 0] - (1.0 - want)) < 1e-15 and y[1, 2] == 0.0


def pin_softmax_causal_brute(lib):
    """Pure-Python softmax of the scaled visible prefix (tiny rows)."""
    for dt in ("f32", "f16", "bf16"):
        for N in (1, 2, 3, 7, 16, 33):
            M, Q, off = 6, 4, 1
            x = _rng_rows(960 + N, M, N, dt, scale=2.0)
            sc = float(np.float32(0.3))
            y = oracle.softmax_causal(x, dt, 0.3, Q, off, lib=lib)
            for r in range(M):
                vis = min(N, r % Q + off + 1)
                want = brute.softmax_row([sc * v for v in _decode_py(x[r], dt)[:vis]])
                assert _rel(y[r, :vis], want) < 1e-13, (dt, N, r)
                assert np.all(y[r, vis:] == 0.0)




# ----------------------------------------------------------------------------
# attention forward: softmax(scale Q K^T) V ("How Flash Attention Uses Triton")
# ----------------------------------------------------------------------------

def _qkv(seed, BH, Lq, Lk, D, dt, qk_scale=1.0):
    q = _rng_rows(seed, BH * Lq, D, dt, qk_scale).reshape(BH, Lq, D)
    k = _rng_rows(seed + 1, BH * Lk, D, dt, qk_scale).reshape(BH, Lk, D)
    v = _rng_rows(seed + 2, BH * Lk, D, dt).reshape(BH, Lk, D)
    return q, k, v


def _dec(a, dt):
    """Stored values -> float64 through numpy (f32, f16) or the bf16 shift."""
    if dt == "f32":
        return np.asarray(a, dtype=np.float64)
    if dt == "f16":
        return np.asarray(a).view(np.float16).astype(np.float64)
    return (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_attention_single_visible_key(lib):
    """One visible key gives that key's value row exactly: causal query 0
    with offset 0, and every query of a head with one key."""
    for dt in ("f32", "bf16"):
        q, k, v = _qkv(11, 2, 6, 9, 16, dt)
        o = oracle.attention(q, k, v, dt, 0.3, causal=True, offset=0, lib=lib)
        assert np.array_equal(o[:, 0, :], _dec(v[:, 0, :], dt))
        q1, k1, v1 = _qkv(12, 3, 4, 1, 8, dt)
        o1 = oracle.attention(q1, k1, v1, dt, 1.0, lib=lib)
        assert np.array_equal(o1, np.broadcast_to(_dec(v1, dt), (3, 4, 8)))


def pin_attention_equal_scores_give_mean(lib):
    """q = 0 makes every score 0: the output is the plain mean of the visible
    value rows (all of them, or rows 0..i + offset when causal)."""
    BH, Lq, Lk, D = 2, 7, 11, 8
    _, k, v = _qkv(13, BH, Lq, Lk, D, "f32")
    q = np.zeros((BH, Lq, D), dtype=np.float32)
    vd = v.astype(np.float64)
    o = oracle.attention(q, k, v, "f32", 2.0, lib=lib)
    assert _rel(o, np.broadcast_to(vd.mean(axis=1, keepdims=True), o.shape)) < 1e-13
    off = 2
    oc = oracle.attention(q, k, v, "f32", 2.0, causal=True, offset=off, lib=lib)
    for i in range(Lq):
        want = vd[:, :min(Lk, i + off + 1), :].mean(axis=1)
        assert np.max(np.abs(oc[:, i, :] - want)) <= 1e-14 * np.max(np.abs(vd)), i


def pin_attention_two_keys_logistic(lib):
    """Two keys: o = v0 / (1 + e^-(s0 - s1)) + v1 / (1 + e^(s0 - s1)), the
    logistic form, with s_j = scale * q . k_j (values exact in fp32; the
    key count differs from the head dimension, so a transposed K shows)."""
    q = np.array([[[1.0, 2.0, 0.0, -1.0, 0.5]]], dtype=np.float32)
    k = np.array([[[0.5, 0.0, 1.0, 0.0, 2.0], [0.0, 1.0, 0.0, 2.0, -1.0]]], dtype=np.float32)
    v = np.array([[[1.0, -2.0, 3.0, 0.25, 8.0], [-4.0, 0.5, 1.0, 2.0, -1.0]]], dtype=np.float32)
    scale = 0.75
    s0 = scale * (0.5 + 1.0)          # q . k0 = 0.5 + 1
    s1 = scale * (2.0 - 2.0 - 0.5)    # q . k1 = 2 - 2 - 0.5
    a0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    want = a0 * v[0, 0].astype(np.float64) + (1.0 - a0) * v[0, 1].astype(np.float64)
    o = oracle.attention(q, k, v, "f32", scale, lib=lib)
    assert np.max(np.abs(o[0, 0] - want)) < 1e-15 * 8, (o[0, 0], want)


def pin_attention_large_scores(lib):
    """Scores near 700-800 (exp would overflow without the max shift): one
    key dominates by 100 in the exponent, so o equals its value row to
    e^-100."""
    D, Lk = 4, 5
    q = np.array([[[10.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    k = np.zeros((1, Lk, D), dtype=np.float32)
    k[0, :, 0] = [70.0, 80.0, 60.0, 70.0, 65.0]      # scores 700, 800, 600, ...
    v = _rng_rows(14, Lk, D, "f32").reshape(1, Lk, D)
    o = oracle.attention(q, k, v, "f32", 1.0, lib=lib)
    assert np.all(np.isfinite(o)) and np.max(np.abs(o[0, 0] - v[0, 1])) < 1e-40


def pin_attention_value_affine(lib):
    """The weights of a row sum to one: o(V + c) = o(V) + c and
    o(a V) = a o(V) (values chosen so V + c and a V are exact in fp32)."""
    q, k, v = _qkv(15, 2, 6, 10, 8, "f32")
    v = (np.round(v * 64) / 64).astype(np.float32)
    o = oracle.attention(q, k, v, "f32", 0.4, causal=True, offset=3, lib=lib)
    o2 = oracle.attention(q, k, (v + np.float32(3.0)).astype(np.float32), "f32", 0.4, causal=True, offset=3, lib=lib)
    o3 = oracle.attention(q, k, (v * np.float32(-2.0)).astype(np.float32), "f32", 0.4, causal=True, offset=3, lib=lib)
    assert np.max(np.abs(o2 - (o + 3.0))) < 1e-14
    assert np.max(np.abs(o3 - (-2.0 * o))) < 1e-14


def pin_attention_key_permutation(lib):
    """Without a mask, permuting the keys together with their value rows
    leaves every output unchanged (up to the order of the sums)."""
    q, k, v = _qkv(16, 2, 5, 13, 8, "f32")
    perm = np.random.default_rng(17).permutation(13)
    o = oracle.attention(q, k, v, "f32", 0.5, lib=lib)
    op = oracle.attention(q, np.ascontiguousarray(k[:, perm]), np.ascontiguousarray(v[:, perm]), "f32", 0.5,
                          lib=lib)
    assert np.max(np.abs(o - op)) < 1e-14


def pin_attention_torch(lib):
    """PyTorch float64 CPU (matmul, masked_fill with -inf, softmax, matmul)
    on the exactly decoded inputs: several shapes, scales, causal offsets and
    storage types."""
    import torch
    for seed, (BH, Lq, Lk, D, causal, off, scale, dt) in enumerate(
            [(2, 9, 9, 16, True, 0, 0.25, "bf16"), (3, 5, 17, 8, True, 12, 0.35, "f16"),
             (1, 33, 20, 32, False, 0, 1.0 / math.sqrt(32), "f32"), (2, 16, 40, 64, True, 24, 0.125, "bf16")]):
        q, k, v = _qkv(100 + seed, BH, Lq, Lk, D, dt)
        qd, kd, vd = (torch.from_numpy(_dec(a, dt)) for a in (q, k, v))
        s = float(np.float32(scale)) * (qd @ kd.transpose(1, 2))     # scale arrives as a C float
        if causal:
            mask = torch.arange(Lk)[None, :] > (torch.arange(Lq)[:, None] + off)
            s = s.masked_fill(mask, float("-inf"))
        want = (torch.softmax(s, dim=-1) @ vd).numpy()
        o = oracle.attention(q, k, v, dt, scale, causal=causal, offset=off, lib=lib)
        assert np.max(np.abs(o - want)) <= 1e-13 * np.max(np.abs(_dec(v, dt))), (seed, np.max(np.abs(o - want)))


def pin_attention_brute(lib):
    """The pure-Python definition (math.fsum sums, its own 16-bit decoding)
    on tiny heads, causal and not."""
    for dt, (BH, Lq, Lk, D, causal, off) in (("bf16", (2, 4, 6, 5, True, 1)), ("f16", (1, 3, 7, 4, False, 0)),
                                             ("f32", (2, 5, 5, 3, True, 0))):
        q, k, v = _qkv(200 + Lk, BH, Lq, Lk, D, dt)
        o = oracle.attention(q, k, v, dt, 0.6, causal=causal, offset=off, lib=lib)
        for b in range(BH):
            K = [_decode_py(k[b, j], dt) for j in range(Lk)]
            V = [_decode_py(v[b, j], dt) for j in range(Lk)]
            for i in range(Lq):
                vis = min(Lk, i + off + 1) if causal else Lk
                want = brute.attention_row(_decode_py(q[b, i], dt), K, V, float(np.float32(0.6)), vis)
                assert np.max(np.abs(o[b, i] - np.array(want))) < 1e-14, (dt, b, i)


def pin_attention_online_matches_plain(lib):
    """The page's tiled loop (running max, alpha rescale of the accumulator
    and the denominator) equals the plain definition for every block size,
    causal rows included (blocks cut through the diagonal)."""
    q, k, v = _qkv(18, 2, 11, 23, 8, "bf16")
    for causal, off in ((False, 0), (True, 0), (True, 7)):
        o = oracle.attention(q, k, v, "bf16", 0.7, causal=causal, offset=off, lib=lib)
        for block in (1, 2, 5, 16, 23, 40):
            ob = oracle.attention_online(q, k, v, "bf16", 0.7, block, causal=causal, offset=off, lib=lib)
            assert np.max(np.abs(ob - o)) < 1e-13, (causal, off, block)


def pin_attention_abs_scale(lib):
    """The size of the summed terms, sum_j w_j |v_j| / sum_j w_j, is the
    output of the same weights on |V|: it equals o(|V|), bounds |o(V)|, and
    equals o(V) where V is non-negative."""
    q, k, v = _qkv(21, 2, 9, 14, 8, "f32")
    o, oa = oracle.attention(q, k, v, "f32", 0.5, causal=True, offset=2, lib=lib, with_abs=True)
    o_abs = oracle.attention(q, k, np.abs(v), "f32", 0.5, causal=True, offset=2, lib=lib)
    assert np.max(np.abs(oa - o_abs)) < 1e-15 and np.all(np.abs(o) <= oa * (1 + 1e-15))
    _, oa2 = oracle.attention(q, k, np.abs(v), "f32", 0.5, causal=True, offset=2, lib=lib, with_abs=True)
    assert np.max(np.abs(oa2 - o_abs)) < 1e-15


def pin_attention_rows_subset(lib):
    """Computing a subset of rows gives those rows of the full result."""
    q, k, v = _qkv(19, 3, 8, 12, 8, "f16")
    o = oracle.attention(q, k, v, "f16", 0.5, causal=True, offset=4, lib=lib).reshape(24, 8)
    rows = [23, 0, 7, 8, 15, 16]
    o_r, oa_r = oracle.attention(q, k, v, "f16", 0.5, causal=True, offset=4, rows=rows, lib=lib, with_abs=True)
    _, oa = oracle.attention(q, k, v, "f16", 0.5, causal=True, offset=4, lib=lib, with_abs=True)
    assert np.array_equal(o_r, o[rows]) and np.array_equal(oa_r, oa.reshape(24, 8)[rows])


ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
