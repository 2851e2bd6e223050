"""Helpers shared by the GPU tests: run the library on a seeded workload and
produce the oracle's view of the same inputs."""
import numpy as np

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
