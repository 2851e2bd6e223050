"""Seeded synthetic inputs shaped like the FLUX layers the method is timed on.

This module only draws random numbers and rounds them to bfloat16; it holds
none of the method's arithmetic.  Both the GPU path and the CPU oracle read
their inputs from here.

Every layer is drawn from numpy's PCG64 with SeedSequence(20261203 + index),
with independent child streams for X, the calibration draw, W, the outlier
positions, the bias and the LoRA factors.  Values are drawn in fp64 and
rounded to bfloat16 (fp64 -> fp32 -> bf16, each step round-to-nearest-even;
this recipe only defines the inputs).

Workloads (M tokens, K in-features, N out-features):
  tiny         256 x 512 -> 512, X ~ N(0,1) with 8 outlier channels x30,
               W ~ N(0, 1/512), alpha 0.5, rank 16, INT4
  flux_qkv     4096 x 3072 -> 9216 = [Wq | Wk | Wv], X ~ N(0,1) with 31
               (1 % of K) outlier channels x50, W ~ N(0, 1/3072), rank 32
               shared down factor, INT4
  flux_mlp_up  4096 x 3072 -> 12288, X ~ Student-t(3), W ~ N(0, 1/3072),
               rank 32, MXFP4
  flux_mlp_down 4096 x 12288 -> 3072, X ~ N(0,1), W ~ N(0, 1/12288) with 4
               outlier input rows x20, alpha in {0.3, 0.5, 0.7}, rank 32, INT4
  flux_lora    8192 x 3072 -> 12288, X as flux_qkv, W as flux_mlp_up, rank 32
               plus a rank-16 LoRA (A ~ N(0, 1/3072), B ~ N(0, 0.01/16),
               strength 1), MXFP4 and INT4
  flux_qkv_w8a8 the flux_qkv shapes and distributions (own seed), rank 16,
               8-bit per-token activations and per-channel weights
A bias ~ N(0, 0.1^2) is drawn for every layer.  The calibration draw has
min(M, 1024) rows from the same distribution and the same outlier channels.

Activations too large to draw on the host (the largest shapes the device
path accepts, gigabytes of X) come from device_normal_bf16: torch's seeded
Philox generator on the device, N(0, 1) in fp32, rounded to bfloat16 by
torch (RNE); tests copy the rows they check back to the host, so both sides
see the same values.
"""

from dataclasses import dataclass, field, replace

import numpy as np

SEED_BASE = 20261203


@dataclass(frozen=True)
class LayerSpec:
    name: str
    index: int
    M: int
    K: int
    N: int
    rank: int
    fmt: str
    alpha: float = 0.5
    x_dist: str = "normal"          # 'normal' | 'student_t3'
    x_outlier_channels: int = 0
    x_outlier_scale: float = 1.0
    w_outlier_rows: int = 0
    w_outlier_scale: float = 1.0
    lora_rank: int = 0
    lora_b_var: float = 0.0
    qkv_splits: tuple = field(default_factory=tuple)

    @property
    def total_rank(self):
        return self.rank + self.lora_rank


SPECS = {
    "tiny": LayerSpec("tiny", 0, 256, 512, 512, 16, "int4",
                      x_outlier_channels=8, x_outlier_scale=30.0),
    "flux_qkv": LayerSpec("flux_qkv", 1, 4096, 3072, 9216, 32, "int4",
                          x_outlier_channels=31, x_outlier_scale=50.0,
                          qkv_splits=(3072, 3072, 3072)),
    "flux_mlp_up": LayerSpec("flux_mlp_up", 2, 4096, 3072, 12288, 32, "mxfp4",
                             x_dist="student_t3"),
    "flux_mlp_down": LayerSpec("flux_mlp_down", 3, 4096, 12288, 3072, 32, "int4",
                               w_outlier_rows=4, w_outlier_scale=20.0),
    "flux_lora": LayerSpec("flux_lora", 4, 8192, 3072, 12288, 32, "mxfp4",
                           x_outlier_channels=31, x_outlier_scale=50.0,
                           lora_rank=16, lora_b_var=0.01 / 16),
    "flux_qkv_w8a8": LayerSpec("flux_qkv_w8a8", 5, 4096, 3072, 9216, 16, "w8a8",
                               x_outlier_channels=31, x_outlier_scale=50.0,
                               qkv_splits=(3072, 3072, 3072)),
}


def spec(name, **overrides):
    """A named workload, optionally with fields replaced (e.g. fmt, M, alpha)."""
    return replace(SPECS[name], **overrides)


def to_bf16_values(x):
    """fp64 -> fp32 -> bf16 (RNE at each step); returns float32 values."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = x32.view(np.uint32).astype(np.uint64)
    # round the low 16 bits to nearest, ties to even
    lsb = (b >> 16) & 1
    b = (b + 0x7FFF + lsb) >> 16
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_of(v32):
    """uint16 patterns of float32 values that are already bf16 values."""
    return (np.asarray(v32, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _draw_x(rng, shape, s, channels):
    if s.x_dist == "student_t3":
        x = rng.standard_t(3.0, size=shape)
    else:
        x = rng.standard_normal(size=shape)
    if len(channels):
        x[:, channels] *= s.x_outlier_scale
    return x


def make_layer(s, with_x=True, m_override=None):
    """Draw one workload.  Returns a dict of float32 arrays holding bf16 values
    (X, X_cal, W, bias, lora_A, lora_B) plus the outlier positions."""
    ss = np.random.SeedSequence(SEED_BASE + s.index)
    c_x, c_cal, c_w, c_out, c_bias, c_lora = ss.spawn(6)
    r_out = np.random.default_rng(c_out)
    channels = np.sort(r_out.choice(s.K, size=s.x_outlier_channels, replace=False)) \
        if s.x_outlier_channels else np.zeros(0, dtype=np.int64)
    wrows = np.sort(r_out.choice(s.K, size=s.w_outlier_rows, replace=False)) \
        if s.w_outlier_rows else np.zeros(0, dtype=np.int64)
    out = {"spec": s, "outlier_channels": channels, "outlier_rows": wrows}
    M = s.M if m_override is None else m_override
    if with_x:
        out["X"] = to_bf16_values(_draw_x(np.random.default_rng(c_x), (M, s.K), s, channels))
    mc = min(s.M, 1024)
    out["X_cal"] = to_bf16_values(_draw_x(np.random.default_rng(c_cal), (mc, s.K), s, channels))
    w = np.random.default_rng(c_w).standard_normal(size=(s.K, s.N)) / np.sqrt(s.K)
    if len(wrows):
        w[wrows, :] *= s.w_outlier_scale
    out["W"] = to_bf16_values(w)
    out["bias"] = to_bf16_values(np.random.default_rng(c_bias).normal(0.0, 0.1, size=s.N))
    if s.lora_rank:
        rl = np.random.default_rng(c_lora)
        out["lora_A"] = to_bf16_values(rl.standard_normal((s.K, s.lora_rank)) / np.sqrt(s.K))
        out["lora_B"] = to_bf16_values(rl.standard_normal((s.lora_rank, s.N)) * np.sqrt(s.lora_b_var))
    return out


def random_bf16(seed, shape, scale=1.0):
    """Plain N(0, scale^2) bf16 values, for kernel-level tests."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 1000 + seed))
    return to_bf16_values(rng.standard_normal(size=shape) * scale)


def random_f32(seed, shape, lo, hi):
    """Uniform fp32 values in [lo, hi), for kernel-level tests."""
    rng = np.random.default_rng(np.random.SeedSequence(SEED_BASE + 2000 + seed))
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def device_normal_bf16(seed, M, K, device="cuda", chunk_rows=1 << 16):
    """[M, K] N(0, 1) bf16 values drawn on the device (torch's seeded
    generator, fp32 rounded to bf16), returned as an int16 tensor of bf16 bit
    patterns.  Drawn in row chunks so that the fp32 draw stays small."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(SEED_BASE + 3000 + seed)
    out = torch.empty((M, K), dtype=torch.int16, device=device)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        v = torch.randn((r1 - r0, K), generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = v.to(torch.bfloat16).view(torch.int16)
        del v
    return out
