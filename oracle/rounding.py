"""Rounding points of the oracle (test infrastructure only).

The pages fix which quantities live in which precision (bf16 factors, fp16
group scales, fp32 residual); they never spell out the rounding mode, so the
oracle takes IEEE round-to-nearest-even everywhere (Zhou notes, sec. 2.2
leaves "round" unspecified; the plain reading is the IEEE default).

Pins (tests/test_oracle_rounding.py): hand-computed bf16/fp16 values, ties
checked against the definition "nearest representable value, even on ties"
by brute force over the representable neighbours.
"""

import numpy as np

BF16_MAX = float.fromhex("0x1.fep127")


def to_f32(x):
    """Round fp64 values to fp32 (IEEE RNE).  Returns a float32 array."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x):
    """Round each value (fp64 or fp32) to the nearest bfloat16 value, RNE.

    bfloat16 keeps 8 significant bits with fp32's exponent range.  The
    rounding is done directly from the exact input (no detour through fp32),
    so an fp64 input is rounded once.  Returns float64 values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])  # x = m * 2**e with 0.5 <= |m| < 1
    # spacing of bf16 values around x: 2**(e-8); subnormals share 2**-133
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x[fin] / quantum) * quantum
    r = np.where(np.abs(r) > BF16_MAX, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def round_f16(x32):
    """Round fp32 values to IEEE binary16 (RNE, with subnormals).

    Returns float64 values of the fp16 results.
    """
    x32 = np.asarray(x32, dtype=np.float32)
    with np.errstate(over="ignore"):                 # out-of-range values become +-inf
        return x32.astype(np.float16).astype(np.float64)


def bf16_bits(v):
    """uint16 bit patterns of bf16-representable values (no rounding)."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    bits = v32.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value is not representable in bfloat16")
    return (bits >> 16).astype(np.uint16)


def bf16_from_bits(b):
    """float64 values of uint16 bfloat16 bit patterns."""
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
