"""Group-wise 4-bit quantizers of the oracle (test infrastructure only).

Both quantizers group along the reduction dimension K, for activations and
weights alike (Zhou notes, sec. 8: "activations and weights are both group
quantized"; grouping along K is the only reading under which a group's
integer partial product exists).

INT4 (Zhou notes, sec. 2.2, Eq. (1); sec. 8 for group size 64 and a 16-bit
scale).  Per group of 64 values z (fp32):
    amax = max |z|
    s32  = fp32(amax / 7)                      (IEEE fp32 division)
    s16  = fp16(s32)                           (the stored 16-bit scale)
    if s16 overflowed to +inf (s32 >= 65520): s16 = 65504, the largest
           finite fp16 value, and the clamp below saturates the codes
    if s16 == 0: every code is 0
    else: rcp = fp32(1 / s16); q = clamp(rint(fp32(z * rcp)), -7, 7)
Codes run -7..7 (the notes: symmetric coding, the extra negative code is
not used).  Eq. (1) assumes a scale the 16-bit format can hold; for a group
whose amax / 7 lies beyond the fp16 range the reading taken is a saturated
scale: s16 = 65504 and every |z| / s16 above 7.5 takes code +-7 (clipping,
the only way a finite group stays finite under a 16-bit scale).  The scale is rounded to fp16 before quantizing, so decoding is
exactly q * s16.  Dividing by the scale is done as one correctly rounded
reciprocal per group and a multiply per element; this is the reading taken
where Eq. (1) writes Z / s.

MXFP4 (AutoRound doc, export section: E2M1 codes, group size 32, symmetric,
dynamic activation quantization; msModelSlim doc: "per_block mxfp4 minmax").
The pages give no rule for the power-of-two block scale.  Reading taken:
the smallest power of two that makes the block maximum representable, so
nothing is clipped (Eq. (1) and Eq. (9) of the Zhou notes both assume no
clipping):
    e    = smallest integer with amax <= 6 * 2**e, clamped to [-127, 127];
           amax == 0 gives e = -127
    byte = e + 127                             (E8M0)
    code = nearest E2M1 magnitude to |z| * 2**-e, ties to the even
           mantissa; bit 3 is the sign bit of z (fp32 sign, -0 included)
E2M1 magnitudes by code 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6.

MXFP4 with the OCP rule ("mxfp4_ocp"; the msModelSlim doc names MXFP4
blocks without a scale rule, and the OCP Microscaling Formats v1.0
specification fixes one): the shared exponent is
    e    = floor(log2(amax)) - 2           (2 = the exponent of E2M1's
                                            largest normal value, 6 = 1.5 x 2^2)
           clamped to [-127, 127]; amax == 0 gives e = -127
and the elements are the nearest E2M1 values of z * 2**-e saturated at +-6
(magnitudes from 6 up to below 8 can occur and take code 7).  It equals the
default rule's e whenever amax <= 6 * 2**e and is one smaller otherwise,
trading the largest values' clipping for a finer step.

Packing: two codes per byte (Zhou notes, Eq. (12) counts mn/2 bytes);
element 2j goes to the low nibble of byte j, K contiguous, row-major.

W8A8 (Zhou notes, sec. 8: the 8-bit setting quantizes activations per
token, dynamically, and weights per channel, with rank 16).  One scale per
row over all K values (a token row of x^, an out-feature row of R^T):
    amax = max |z| over the row
    s    = fp32(amax / 127)                    (fp32 scale, stored as is)
    if s == 0: every code is 0
    else: rcp = fp32(1 / s); q = clamp(rint(fp32(z * rcp)), -127, 127)
Readings: the symmetric range -127..127 (as INT4 leaves out -8, the 8-bit
code leaves out -128), an fp32 scale (the pages fix 16-bit scales only for
the 4-bit groups), and the same reciprocal-then-multiply division as INT4.
For a row whose scale is an fp32 subnormal below 2^-128, 1/s overflows to
infinity: non-zero elements then take +-127 and zeros stay 0.
Codes are stored one signed byte per element, K contiguous, row-major.

Pins (tests/test_oracle_quantizers.py): the worked example of Zhou notes
sec. 2.2 (range 7 gives step 1; range 1 gives step 1/7), the saturated
scale on both sides of the fp16 overflow threshold, the OCP exponent by
brute-force search and its relation to the default rule, brute-force argmin
over the 15 INT4 codes, the 255 8-bit codes and the 8 E2M1 magnitudes,
brute-force search for e, the no-clipping property and the Eq. (9) per-group
error bound (per row for 8-bit).
"""

import numpy as np

from .rounding import round_f16

INT4_GROUP = 64
MXFP4_GROUP = 32
F16_MAX = 65504.0            # largest finite IEEE binary16 value
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _groups(z, g):
    z = np.asarray(z, dtype=np.float32)
    rows, k = z.shape
    if k % g:
        raise ValueError(f"K={k} is not a multiple of the group size {g}")
    return z.reshape(rows, k // g, g)


def quantize_int4(z):
    """INT4 RTN with per-64 fp16 scales.

    z: [rows, K] fp32 values (already smoothed activations or residual^T).
    Returns (codes int8 [rows, K] in -7..7, scales float64 [rows, K/64]
    holding the fp16 values).
    """
    zg = _groups(z, INT4_GROUP)
    amax = np.max(np.abs(zg), axis=2)                       # fp32, exact
    s32 = (amax / np.float32(7.0)).astype(np.float32)       # fp32 division
    s16 = round_f16(s32)                                    # stored scale
    s16 = np.where(np.isposinf(s16), F16_MAX, s16)          # saturated, not infinite
    s16_32 = s16.astype(np.float32)                         # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        rcp = (np.float32(1.0) / s16_32).astype(np.float32)
        y = (zg * rcp[:, :, None]).astype(np.float32)       # fp32 product
        q = np.clip(np.rint(y), -7, 7)
    q = np.where((s16 == 0)[:, :, None], 0.0, q)
    return q.astype(np.int8).reshape(z.shape), s16


def quantize_w8(z):
    """8-bit RTN with one fp32 scale per row.

    z: [rows, K] fp32.  Returns (codes int8 [rows, K] in -127..127, scales
    float32 [rows]).
    """
    z = np.asarray(z, dtype=np.float32)
    amax = np.max(np.abs(z), axis=1)                        # fp32, exact
    s = (amax / np.float32(127.0)).astype(np.float32)       # fp32 division
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        rcp = (np.float32(1.0) / s).astype(np.float32)
        y = (z * rcp[:, None]).astype(np.float32)           # fp32 product
        q = np.clip(np.rint(y), -127, 127)
    # a zero element is code 0 (also when s is subnormal and 1/s overflows)
    q = np.where((s == 0)[:, None] | (z == 0), 0.0, q)
    return q.astype(np.int8), s


def decode_w8(codes, scales):
    """q * s for every element.  codes [rows, K] int, scales [rows] fp32."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, None]


def mxfp4_block_exponent(amax):
    """Smallest e with amax <= 6 * 2**e, clamped to [-127, 127].

    amax: fp32 array.  Uses amax = f * 2**E (0.5 <= f < 1):
    6 * 2**e >= f * 2**E  <=>  e - E >= log2(f / 6), and f / 6 lies in
    [1/12, 1/6), so e = E - 3 when f <= 3/4 and e = E - 2 otherwise.
    """
    amax = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(amax)
    e = np.where(f <= 0.75, E - 3, E - 2)
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def e2m1_nearest_code(a):
    """Nearest E2M1 magnitude code (0..7) to a >= 0, ties to even mantissa.

    Plain definition: distance to each of the 8 magnitudes; among the
    minimum-distance codes take the one whose mantissa bit (bit 0) is 0.
    """
    a = np.asarray(a, dtype=np.float64)
    d = np.abs(a[..., None] - E2M1_VALUES)                  # [..., 8]
    dmin = d.min(axis=-1, keepdims=True)
    best = d == dmin
    # prefer an even code among ties; there are at most two candidates
    even = best & ((np.arange(8) & 1) == 0)
    choose = np.where(even.any(axis=-1, keepdims=True), even, best)
    return np.argmax(choose, axis=-1).astype(np.int64)


def mxfp4_ocp_block_exponent(amax):
    """OCP shared exponent floor(log2(amax)) - 2, clamped to [-127, 127].

    amax: fp32 array.  With amax = f * 2**E (0.5 <= f < 1), floor(log2(amax))
    is E - 1, so e = E - 3; amax == 0 gives -127.
    """
    amax = np.asarray(amax, dtype=np.float64)
    _, E = np.frexp(amax)
    e = np.where(amax == 0, -127, E - 3)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_mxfp4(z, rule="ceil"):
    """MXFP4 (E2M1 codes, E8M0 scale per 32 elements).

    z: [rows, K] fp32; rule 'ceil' (the default: no clipping) or 'ocp' (the
    OCP floor rule with saturation).  Returns (codes uint8 [rows, K] in 0..15
    with bit 3 the sign, scale bytes uint8 [rows, K/32], exponents int64
    [rows, K/32]).
    """
    zg = _groups(z, MXFP4_GROUP)
    amax = np.max(np.abs(zg), axis=2)
    e = mxfp4_block_exponent(amax) if rule == "ceil" else mxfp4_ocp_block_exponent(amax)
    scaled = np.abs(zg.astype(np.float64)) * np.ldexp(1.0, -e)[:, :, None]
    scaled = np.minimum(scaled, 6.0)                        # saturation (only the ocp rule reaches it)
    mag = e2m1_nearest_code(scaled)
    sign = np.signbit(zg).astype(np.int64)
    codes = (sign << 3) | mag
    return codes.astype(np.uint8).reshape(z.shape), (e + 127).astype(np.uint8), e


def decode_int4(codes, scales):
    """q * s16 for every element.  codes [rows, K] int, scales [rows, K/64]."""
    codes = np.asarray(codes, dtype=np.float64)
    rows, k = codes.shape
    s = np.repeat(np.asarray(scales, dtype=np.float64), INT4_GROUP, axis=1)
    return codes * s


def decode_mxfp4(codes, scale_bytes):
    """E2M1 value * 2**(byte-127).  codes [rows, K] 0..15, bytes [rows, K/32]."""
    codes = np.asarray(codes, dtype=np.int64)
    mag = E2M1_VALUES[codes & 7]
    sign = np.where(codes & 8, -1.0, 1.0)
    e = np.asarray(scale_bytes, dtype=np.int64) - 127
    s = np.repeat(np.ldexp(1.0, e), MXFP4_GROUP, axis=1)
    return sign * mag * s


def int4_nibbles(codes):
    """Two's complement nibble of each INT4 code (0..15)."""
    return (np.asarray(codes, dtype=np.int64) & 0xF).astype(np.uint8)


def nibble_to_int4(n):
    n = np.asarray(n, dtype=np.int64) & 0xF
    return np.where(n >= 8, n - 16, n).astype(np.int8)


def pack_nibbles(nib):
    """[rows, K] values 0..15 -> [rows, K/2] bytes; element 2j in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    if nib.shape[1] % 2:
        raise ValueError("K must be even")
    lo = nib[:, 0::2]
    hi = nib[:, 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out


def quantize(z, fmt):
    """Quantize [rows, K] fp32 values in the named format.

    Returns a dict with 'packed' (u8 [rows, K/2] for the 4-bit formats; for
    w8a8 the int8 codes viewed as u8 [rows, K]), 'scales' (fp16 values as
    float64 for int4, E8M0 bytes for mxfp4, fp32 per row for w8a8) and 'deq'
    (fp64 decoded values).
    """
    if fmt == "w8a8":
        q, s = quantize_w8(z)
        return {"packed": q.view(np.uint8), "scales": s, "codes": q, "deq": decode_w8(q, s)}
    if fmt == "int4":
        q, s = quantize_int4(z)
        return {"packed": pack_nibbles(int4_nibbles(q)), "scales": s,
                "codes": q, "deq": decode_int4(q, s)}
    if fmt in ("mxfp4", "mxfp4_ocp"):
        c, b, _ = quantize_mxfp4(z, "ceil" if fmt == "mxfp4" else "ocp")
        return {"packed": pack_nibbles(c), "scales": b, "codes": c,
                "deq": decode_mxfp4(c, b)}
    raise ValueError(f"unknown format {fmt!r}")


def dequantize_packed(packed, scales, fmt):
    """fp64 decoded matrix from packed codes and scales."""
    if fmt == "w8a8":
        return decode_w8(np.asarray(packed, dtype=np.uint8).view(np.int8), scales)
    nib = unpack_nibbles(packed)
    if fmt == "int4":
        return decode_int4(nibble_to_int4(nib), scales)
    if fmt in ("mxfp4", "mxfp4_ocp"):
        return decode_mxfp4(nib, scales)
    raise ValueError(f"unknown format {fmt!r}")
