"""Helpers shared by the GPU tests: run the library on a seeded workload and
produce the oracle's view of the same inputs."""
import numpy as np

from oracle import quantizers as Q
from oracle.rounding import bf16_bits as _bf16_bits

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from oracle import forward as F
from oracle import prepare as P


def rel_fro(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


def bf16_to_f64(bits):
    return (np.asarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


class GpuRun:
    """Prepare a layer with the library, run the device path, read back."""

    def __init__(self, d, fmt, rank, alpha, lora=None, use_bias=True, x=None, **prep_kw):
        import torch
        self.torch = torch
        s = d["spec"]
        self.x = d["X"] if x is None else x
        self.M, self.K = self.x.shape
        self.N = d["W"].shape[1]
        self.fmt = fmt
        amax = B.calib_absmax(S.bf16_bits_of(d["X_cal"]))
        self.prep = B.prepare(d["W"], amax, alpha, rank, fmt, lora=lora, **prep_kw)
        self.rank = self.prep["rank"]
        self.bias = d["bias"] if use_bias else None
        bias_bits = S.bf16_bits_of(self.bias) if use_bias else None
        self.layer = B.DeviceLayer(self.prep, bias_bits)
        self.X = torch.from_numpy(S.bf16_bits_of(self.x).view(np.int16)).cuda()
        self.Y = torch.empty((self.M, self.N), dtype=torch.int16, device="cuda")
        self.ws = self.layer.workspace(self.M)

    def forward(self):
        B.linear_forward(self.layer, self.X, self.Y, self.ws)
        self.torch.cuda.synchronize()
        return self

    def y(self, rows=None):
        y = self.Y.cpu().numpy() if rows is None else self.Y[rows].cpu().numpy()
        return bf16_to_f64(y)

    def activations(self):
        ws_host = self.ws.cpu().numpy()
        return B.unpack_activations(ws_host, self.M, self.K, self.rank, self.fmt)


def oracle_layer(d, fmt, rank, alpha, lora=None, **prep_kw):
    return P.prepare(d["W"], P.calib_amax(d["X_cal"]), alpha, rank, fmt, lora=lora, **prep_kw)


def oracle_scales_bits(xs, fmt):
    return np.float16(xs).view(np.uint16) if fmt == "int4" else xs


def oracle_canonical(po):
    """The oracle's prepared layer as the canonical host buffers the library's
    kernel-layout conversion takes (the oracle's own lambda, factors, codes
    and scales: the device then computes from exactly the oracle's operands)."""
    fmt = po["fmt"]
    K = po["inv_lambda"].shape[0]
    N = po["wq_packed"].shape[0]
    if fmt == "int4":
        ws = np.float16(po["ws"]).view(np.uint16)
    elif fmt == "w8a8":
        ws = np.asarray(po["ws"], np.float32)
    else:
        ws = np.asarray(po["ws"], np.uint8)
    rank = po["l1p"].shape[1]
    return {"K": K, "N": N, "rank": rank, "fmt": B.fmt_code(fmt),
            "smooth_inv": np.asarray(po["inv_lambda"], np.float32),
            "wq": np.ascontiguousarray(po["wq_packed"], np.uint8), "ws": ws,
            "l1": _bf16_bits(po["l1p"]).reshape(K, rank), "l2": _bf16_bits(po["l2p"]).reshape(rank, N)}


# Element-wise bound of a device output against the exact (fp64) output of
# the same operands.  The device forms every main-path partial product
# exactly and sums them in fp32 (per MFMA step, per 64-group, or in int32
# with the per-row scales applied after), so the accumulated rounding error
# is at most (K/32 + 16) u32 times the sum of |products| (u32 = 2^-24;
# generous for each format's summation order).  The low-rank branch carries
# x^ and Z as bf16 hi + lo pairs (each within 2^-16 of the value) with fp32
# accumulation: at most 2^-15 times the nested absolute product
# (|x^| |L1'|) |L2'|.  Bias and the last additions add a few u32 of |y|;
# the single bf16 store adds at most half an ulp, 2^-8 |y|.
def elementwise_bound(x, po, bias=None):
    fmt = po["fmt"]
    K = po["inv_lambda"].shape[0]
    xs = F.smooth_activations(x, po["inv_lambda"]).astype(np.float64)
    a_q = F.quantize_activations(x, po["inv_lambda"], fmt)["deq"]
    b_q = Q.dequantize_packed(po["wq_packed"], po["ws"], fmt)
    a_main = np.abs(a_q) @ np.abs(b_q).T
    a_lr = (np.abs(xs) @ np.abs(np.asarray(po["l1p"], np.float64))) @ np.abs(np.asarray(po["l2p"], np.float64))
    y = a_q @ b_q.T + (xs.astype(np.float64) @ np.asarray(po["l1p"], np.float64)) @ np.asarray(po["l2p"], np.float64)
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    e = (K / 32 + 16) * 2.0**-24 * a_main + 2.0**-15 * a_lr + 4 * 2.0**-24 * np.abs(y)
    return 2.0**-8 * (np.abs(y) + e) + e


def assert_elementwise(y_dev, y_ref, bound, what):
    """Every element within its bound; the report names the worst element."""
    d = np.abs(np.asarray(y_dev, np.float64) - y_ref)
    bad = d > bound
    if bad.any():
        i = np.unravel_index(np.argmax(d / np.maximum(bound, 1e-300)), d.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {d.size} elements outside the bound; worst at {i}: "
                             f"dev {y_dev[i]!r} ref {y_ref[i]!r} |d| {d[i]:.3e} bound {bound[i]:.3e}")


def run_on_oracle_layer(po, x, bias=None):
    """Device forward (K-A + K-B through the C ABI) of the oracle's own
    prepared layer on x; returns Y as fp64 and the run's workspace tensor."""
    import torch
    canon = oracle_canonical(po)
    layer = B.DeviceLayer(canon, None if bias is None else S.bf16_bits_of(bias))
    M = x.shape[0]
    X = torch.from_numpy(S.bf16_bits_of(x).view(np.int16)).cuda()
    Y = torch.empty((M, canon["N"]), dtype=torch.int16, device="cuda")
    ws = layer.workspace(M)
    B.linear_forward(layer, X, Y, ws)
    torch.cuda.synchronize()
    return bf16_to_f64(Y.cpu().numpy())


def check_elementwise_on_oracle_layer(po, x, bias, what):
    """Kernel-isolated parity: the device computes from the oracle's
    operands, and every element of Y lies within elementwise_bound of the
    oracle's fp64 forward."""
    y_dev = run_on_oracle_layer(po, x, bias)
    assert np.all(np.isfinite(y_dev)), f"{what}: non-finite output"
    ref = F.forward(x, po, bias)["y"]
    assert_elementwise(y_dev, ref, elementwise_bound(x, po, bias), what)
    return y_dev
