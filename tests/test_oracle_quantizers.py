"""Pins of the oracle quantizers (Zhou notes sec. 2.2 Eq. (1) worked
example; E2M1 value table; brute-force nearest-code and block-exponent
searches; no clipping; Eq. (9) group error bound)."""
import json
import os

import numpy as np
import pytest

from oracle import quantizers as Q
from oracle.rounding import round_f16


def _worked_group(case, g):
    z = np.full(g, case["fill"], dtype=np.float32)
    for k, v in case["values"].items():
        z[int(k)] = v
    return z[None, :]


def test_int4_worked_example(golden_dir):
    with open(os.path.join(golden_dir, "int4_worked_example.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        z = _worked_group(case, fx["group_size"])
        q, s = Q.quantize_int4(z)
        assert s[0, 0] == case["expect_scale_f16"], case["name"]
        for k, c in case["expect_codes"].items():
            assert q[0, int(k)] == c, (case["name"], k)
        others = [i for i in range(fx["group_size"]) if str(i) not in case["values"]]
        assert np.all(q[0, others] == case["expect_fill_code"])
        deq = Q.decode_int4(q, s)
        for k, v in case.get("expect_dequant", {}).items():
            assert deq[0, int(k)] == v


def _near_half_integer(y, tol=2.0**-18):
    frac = np.abs(y - np.floor(y) - 0.5)
    return frac < tol * np.maximum(1.0, np.abs(y))


@pytest.mark.parametrize("scale", [1e-3, 1.0, 37.0])
def test_int4_codes_are_the_nearest_code(scale):
    rng = np.random.default_rng(7)
    z = (rng.standard_normal((64, 64 * 8)) * scale).astype(np.float32)
    z[3, 5] = 40 * scale      # an outlier in one group
    z[9, 64:128] = 0.0        # an all-zero group
    q, s = Q.quantize_int4(z)
    assert q.min() >= -7 and q.max() <= 7
    srep = np.repeat(s, 64, axis=1)
    cand = np.arange(-7, 8, dtype=np.float64)
    err = np.abs(z.astype(np.float64)[..., None] - srep[..., None] * cand)  # [r, K, 15]
    best = cand[np.argmin(err, axis=-1)]
    # exact ties of |z - s q| are broken towards the even code
    emin = err.min(axis=-1, keepdims=True)
    tie = (err == emin).sum(-1) > 1
    with np.errstate(divide="ignore", invalid="ignore"):     # rows with s = 0 are masked below
        even_best = np.where(tie, 2 * np.round(z / srep / 2), best)
    mism = (q != even_best) & (srep > 0)
    # the only allowed differences: within a hair of a .5 tie, where the
    # reciprocal-multiply reading may fall on the other side
    exact_ratio = z.astype(np.float64) / np.where(srep > 0, srep, 1)
    assert np.all(_near_half_integer(exact_ratio[mism]))
    assert mism.sum() <= 2
    assert np.all(q[9, 64:128] == 0) and s[9, 1] == 0.0


def test_int4_scale_is_fp16_of_amax_over_7():
    rng = np.random.default_rng(3)
    z = rng.uniform(-5, 5, (8, 256)).astype(np.float32)
    _, s = Q.quantize_int4(z)
    amax = np.abs(z.reshape(8, 4, 64)).max(-1).astype(np.float64)
    # amax / 7 in exact arithmetic, rounded once to fp16, differs from the
    # two-step fp32 -> fp16 rounding only if amax/7 is within 2**-24 of a
    # binary16 midpoint, which does not happen for these draws
    assert np.all(s == np.float16(amax / 7).astype(np.float64))


def test_int4_tiny_scale_clamps():
    # a group whose scale falls in the fp16 subnormal range: the rounded
    # scale can be much smaller than amax/7, codes must saturate at +-7
    z = np.zeros((1, 64), dtype=np.float32)
    z[0, 0] = 5e-7
    z[0, 1] = -4.9e-7
    q, s = Q.quantize_int4(z)
    assert 0 < s[0, 0] < 5e-7 / 7 * 1.5
    assert q[0, 0] == 7 and q[0, 1] == -7


def test_int4_scale_saturates_at_fp16_max():
    """A group whose amax / 7 lies past the fp16 range keeps a finite
    scale: 65504, the largest binary16 value, with codes clipped at +-7.
    Both sides of the overflow threshold (amax / 7 = 65520, the midpoint
    between 65504 and 2^16, which rounds to infinity under ties-to-even)
    give that same scale, so the saturated scale is continuous with the
    unsaturated one."""
    z = np.zeros((4, 64), dtype=np.float32)
    z[0, 0] = 7 * 65519.0            # s32 = 65519 rounds down to 65504: finite without saturation
    z[1, 0] = 7 * 65520.0            # s32 = 65520 rounds to +inf in fp16: saturated
    z[2, :8] = [1e30, -1e30, 65504 * 6.6, 65504 * 7.4, 65504 * 3.2, -65504 * 2.5, 65504 * 0.5, 65504 * 0.49]
    z[3, 0] = 3.4e38                 # near the fp32 maximum
    q, s = Q.quantize_int4(z)
    assert np.all(s[:, 0] == 65504.0)
    with np.errstate(over="ignore"):
        assert np.float16(7 * 65519.0 / 7) == np.float16(65504.0) and np.isinf(np.float16(np.float32(65520.0)))
    assert q[0, 0] == 7 and q[1, 0] == 7 and q[3, 0] == 7
    # closed form under the saturated scale: clip(rint(z / 65504), -7, 7),
    # ties to even (-2.5 -> -2, 0.5 -> 0)
    assert list(q[2, :8]) == [7, -7, 7, 7, 3, -2, 0, 0]
    deq = Q.decode_int4(q, s)
    assert np.all(np.isfinite(deq))
    # below the clipping point the Eq. (9) element bound |z - s q| <= s / 2 still holds
    inside = np.abs(z.astype(np.float64)) <= 7.5 * 65504
    assert np.all(np.abs(z.astype(np.float64) - deq)[inside] <= 65504 / 2)


def test_int4_eq9_group_bound():
    rng = np.random.default_rng(11)
    z = (rng.standard_t(3, (32, 64 * 16)) * 0.05).astype(np.float32)
    q, s = Q.quantize_int4(z)
    err = (z.astype(np.float64) - Q.decode_int4(q, s)).reshape(32, 16, 64)
    amax = np.abs(z.astype(np.float64)).reshape(32, 16, 64).max(-1)
    lhs = np.sqrt((err**2).sum(-1))
    # Eq. (9) with the 1/2 factor, q_max = 7, fp16 scale rounding slack
    rhs = np.sqrt(64) / (2 * 7) * amax * (1 + 2.0**-10)
    assert np.all(lhs <= rhs)


def test_e2m1_table_and_ties():
    assert list(Q.E2M1_VALUES) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    cases = {0.25: 0, 0.2499: 0, 0.2501: 1, 0.75: 2, 1.25: 2, 1.75: 4,
             2.5: 4, 3.5: 6, 5.0: 6, 5.01: 7, 6.0: 7, 0.5: 1, 3.0: 5}
    for a, c in cases.items():
        assert Q.e2m1_nearest_code(np.array(a)) == c, a


def test_e2m1_nearest_matches_threshold_form():
    # independent formulation: count of crossed midpoints, with the tie
    # direction of each midpoint fixed by the even-mantissa rule
    a = np.concatenate([np.linspace(0, 7, 70001), np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])])
    c = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
         + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    assert np.all(Q.e2m1_nearest_code(a) == c)


def test_mxfp4_block_exponent_brute_force():
    rng = np.random.default_rng(5)
    amax = np.concatenate([
        np.exp(rng.uniform(-80, 80, 3000)),
        6.0 * np.ldexp(1.0, np.arange(-20, 20)),        # exactly 6 * 2**e
        np.nextafter(6.0 * np.ldexp(1.0, np.arange(-20, 20)), np.inf),
        [0.0, 1e-45, 3e38]]).astype(np.float32)
    e = Q.mxfp4_block_exponent(amax)
    for a, ei in zip(amax.astype(np.float64), e):
        # smallest integer e with a <= 6 * 2**e, clamped to [-127, 127]
        want = -127
        while want < 127 and a > 6.0 * 2.0**want:
            want += 1
        assert ei == want, (a, ei, want)


def test_mxfp4_no_clipping_and_tight_scale():
    rng = np.random.default_rng(9)
    z = (rng.standard_t(3, (16, 32 * 32)) * 3.0).astype(np.float32)
    z[2, :32] = 0.0
    codes, b, e = Q.quantize_mxfp4(z)
    amax = np.abs(z.astype(np.float64)).reshape(16, 32, 32).max(-1)
    scaled_max = amax * np.ldexp(1.0, -e)
    assert np.all(scaled_max <= 6.0)
    nz = amax > 0
    assert np.all(scaled_max[nz] > 3.0)
    assert b[2, 0] == 0 and np.all(codes[2, :32] == 0)
    # every element decodes within half of the local E2M1 spacing
    deq = Q.decode_mxfp4(codes, b)
    err = np.abs(z.astype(np.float64) - deq)
    half_step = np.repeat(np.ldexp(1.0, e), 32, axis=1) * 1.0   # max spacing 2 -> half 1
    assert np.all(err <= half_step)


def test_mxfp4_sign_bit_is_copied():
    z = np.zeros((1, 32), dtype=np.float32)
    z[0, 0] = 6.0
    z[0, 1] = -0.1      # rounds to zero magnitude, keeps the sign bit
    z[0, 2] = -0.0
    z[0, 3] = -3.0
    codes, b, e = Q.quantize_mxfp4(z)
    assert e[0, 0] == 0 and b[0, 0] == 127
    assert codes[0, 0] == 7 and codes[0, 1] == 8 and codes[0, 2] == 8 and codes[0, 3] == 8 | 5


def test_pack_layout():
    nib = np.array([[1, 2, 15, 0]], dtype=np.uint8)
    p = Q.pack_nibbles(nib)
    assert list(p[0]) == [0x21, 0x0F]
    assert np.all(Q.unpack_nibbles(p) == nib)
    assert list(Q.int4_nibbles(np.array([-7, -1, 0, 7]))) == [9, 15, 0, 7]
    assert list(Q.nibble_to_int4(np.array([9, 15, 0, 7]))) == [-7, -1, 0, 7]


def test_quantize_roundtrip_both_formats():
    rng = np.random.default_rng(2)
    z = rng.standard_normal((4, 256)).astype(np.float32)
    for fmt in ("int4", "mxfp4"):
        d = Q.quantize(z, fmt)
        assert np.all(Q.dequantize_packed(d["packed"], d["scales"], fmt) == d["deq"])


def test_int4_exact_ties_round_to_even():
    # scale 1 (amax 7): z * rcp is exactly the half-integer, ties go to even
    z = np.zeros((1, 64), dtype=np.float32)
    z[0, :8] = [7.0, 2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -6.5]
    q, s = Q.quantize_int4(z)
    assert s[0, 0] == 1.0
    assert list(q[0, :8]) == [7, 2, -2, 0, 0, 2, 4, -6]


# ---------------------------------------------------------------- 8-bit (W8A8)
# Zhou notes sec. 8: per-token activations and per-channel weights at 8 bits.

@pytest.mark.parametrize("scale", [1e-3, 1.0, 37.0])
def test_w8_codes_are_the_nearest_code(scale):
    rng = np.random.default_rng(17)
    z = (rng.standard_normal((24, 384)) * scale).astype(np.float32)
    z[3, 5] = 40 * scale      # an outlier in one row
    z[9] = 0.0                # an all-zero row
    q, s = Q.quantize_w8(z)
    assert q.dtype == np.int8 and q.min() >= -127 and q.max() <= 127
    cand = np.arange(-127, 128, dtype=np.float64)
    err = np.abs(z.astype(np.float64)[..., None] - s.astype(np.float64)[:, None, None] * cand)
    best = cand[np.argmin(err, axis=-1)]
    mism = (q != best) & (s[:, None] > 0)
    ratio = z.astype(np.float64) / np.where(s > 0, s, 1)[:, None]
    assert np.all(_near_half_integer(ratio[mism]))
    assert mism.sum() <= 2
    assert np.all(q[9] == 0) and s[9] == 0.0
    # the row maximum lands on the end of the range: nothing is clipped
    amax_pos = np.argmax(np.abs(z), axis=1)
    live = s > 0
    assert np.all(np.abs(q[live, amax_pos[live]]) == 127)


def test_w8_scale_and_closed_forms():
    # amax = 127 * 2^k: the scale is 2^k exactly and integer multiples of it
    # decode without error; ties of the half-integers go to the even code
    z = np.zeros((3, 128), np.float32)
    z[0, :6] = [127.0, -3.0, 2.5, -2.5, 0.5, 126.5]
    z[1, :3] = [127.0 * 2 ** -10, 5 * 2 ** -10, -64 * 2 ** -10]
    z[2, 0] = 1.0                                   # s = fp32(1/127), not exact
    q, s = Q.quantize_w8(z)
    assert s[0] == 1.0 and s[1] == 2.0 ** -10
    assert list(q[0, :6]) == [127, -3, 2, -2, 0, 126]
    assert list(q[1, :3]) == [127, 5, -64]
    assert s[2] == np.float32(1.0) / np.float32(127.0) and q[2, 0] == 127
    d = Q.decode_w8(q[:2], s[:2])
    assert np.array_equal(d[1], z[1].astype(np.float64))
    # a row of fp32 subnormals: s underflows so far that 1/s is infinite;
    # non-zero elements saturate, zeros stay zero
    t = np.zeros((1, 64), np.float32)
    t[0, :3] = [3e-39, -1e-45, 0.0]
    qt, st = Q.quantize_w8(t)
    with np.errstate(over="ignore"):
        assert 0 < st[0] < 2.0 ** -128 and np.isinf(np.float32(1.0) / st[0])
    assert list(qt[0, :4]) == [127, -127, 0, 0]


def test_w8_row_error_bound_and_roundtrip():
    rng = np.random.default_rng(5)
    z = (rng.standard_t(3, (16, 512))).astype(np.float32)
    d = Q.quantize(z, "w8a8")
    assert d["packed"].shape == (16, 512) and d["packed"].dtype == np.uint8
    assert np.array_equal(Q.dequantize_packed(d["packed"], d["scales"], "w8a8"), d["deq"])
    # |z - q s| <= s / 2 (times the fp32 reciprocal's relative error) per element
    bound = d["scales"].astype(np.float64)[:, None] * (0.5 + 1e-6)
    assert np.all(np.abs(z - d["deq"]) <= bound)


def test_mxfp4_ocp_exponent_brute_force_and_relation():
    """OCP rule: e = floor(log2(amax)) - 2, i.e. the largest integer e with
    4 * 2**e <= amax (brute force), clamped to [-127, 127]; it equals the
    default (no clipping) exponent when amax <= 6 * 2**e and is one below
    it otherwise."""
    rng = np.random.default_rng(21)
    amax = np.concatenate([
        np.exp(rng.uniform(-80, 80, 2000)),
        4.0 * np.ldexp(1.0, np.arange(-20, 20)),                    # exact powers of two times 4
        6.0 * np.ldexp(1.0, np.arange(-20, 20)),
        np.nextafter(6.0 * np.ldexp(1.0, np.arange(-20, 20)), np.inf),
        np.nextafter(8.0 * np.ldexp(1.0, np.arange(-20, 20)), 0),
        [0.0, 1e-45, 3e38]]).astype(np.float32)
    e = Q.mxfp4_ocp_block_exponent(amax)
    ec = Q.mxfp4_block_exponent(amax)
    for a, ei, eci in zip(amax.astype(np.float64), e, ec):
        if a == 0:
            assert ei == -127
            continue
        want = 127
        while want > -127 and 4.0 * 2.0**want > a:
            want -= 1
        assert ei == want, (a, ei, want)
        if -126 < ei < 126:
            assert eci == (ei if a <= 6.0 * 2.0**ei else ei + 1), (a, ei, eci)


def test_mxfp4_ocp_saturates_and_keeps_the_grid():
    rng = np.random.default_rng(22)
    z = (rng.standard_t(3, (16, 32 * 16)) * 2.0).astype(np.float32)
    z[0, :32] = 0.0
    z[1, :32] = np.float32(7.0)                # amax 7: e = 0, every element saturates to 6
    z[1, 5] = -7.9
    z[2, :32] = np.linspace(-5.9, 5.9, 32)     # amax 5.9: e = 0, nothing saturates
    codes, b, e = Q.quantize_mxfp4(z, "ocp")
    assert b[0, 0] == 0 and np.all(codes[0, :32] == 0)
    assert e[1, 0] == 0 and np.all(codes[1, :32] & 7 == 7) and codes[1, 5] == 15
    amax = np.abs(z.astype(np.float64)).reshape(16, 16, 32).max(-1)
    scaled_max = amax * np.ldexp(1.0, -e)
    nz = amax > 0
    assert np.all((scaled_max[nz] >= 4.0) & (scaled_max[nz] < 8.0))
    # below the saturation point every element is the nearest E2M1 value;
    # above it, 6
    deq = Q.decode_mxfp4(codes, b)
    s = np.repeat(np.ldexp(1.0, e), 32, axis=1)
    x = np.abs(z.astype(np.float64)) / s
    d = np.abs(deq) / s
    inside = x <= 6.0
    cand = Q.E2M1_VALUES
    nearest = np.min(np.abs(x[inside][:, None] - cand[None, :]), axis=1)
    assert np.all(np.abs(x[inside] - d[inside]) == nearest)
    assert np.all(d[~inside] == 6.0)
    # the default rule never clips: same data, no element saturated
    c2, b2, e2 = Q.quantize_mxfp4(z)
    assert np.all(amax * np.ldexp(1.0, -e2) <= 6.0)
