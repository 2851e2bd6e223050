"""Inference forward of one SVDQuant layer (test infrastructure only).

Zhou notes sec. 4.2, Eq. (7):  Y^ = (X~ L1) L2 + Q(X~) Q(R),  X~ = X D^-1,
plus the bias, kept on the residual path (msModelSlim doc, "forward
equivalence": residual_out = x R^T + b).  The fused dataflow of Algorithm 2
(Zhou notes sec. 6.1) changes where the work happens, not what is computed,
so the oracle computes each term separately:

O7  x~ = fp32(x * inv_lambda) for every element (bf16 times fp32 is exact in
    fp64, so one cast gives the correctly rounded fp32 product).
O8/O9 group quantization of x~ (oracle.quantizers).
O10 Y_main = A_q B_q^T with A_q, B_q the decoded fp64 matrices.
O11 Z = X diag(inv_lambda) L1' and Y = Y_main + Z L2' + bias, all fp64.

Pins (tests/test_oracle_forward.py): Eq. (8) error identity, the
no-quantization identity of the msModelSlim doc (the two paths sum to x W),
an int64 brute-force per-group GEMM on the tiny layer, and lower error than
plain W4A4 RTN on outlier inputs.
"""

import numpy as np

from .quantizers import quantize, dequantize_packed


def smooth_activations(x, inv_lambda):
    """O7: fp32(x * inv_lambda)."""
    x = np.asarray(x, dtype=np.float64)
    return (x * np.asarray(inv_lambda, dtype=np.float64)[None, :]).astype(np.float32)


def quantize_activations(x, inv_lambda, fmt):
    """O7 + O8/O9: packed codes [M, K/2] and scales of the smoothed input."""
    return quantize(smooth_activations(x, inv_lambda), fmt)


def lowrank_down(x, inv_lambda, l1p):
    """Z = X diag(inv_lambda) L1' in fp64 (the 'lora_down' half)."""
    x = np.asarray(x, dtype=np.float64)
    return (x * np.asarray(inv_lambda, dtype=np.float64)[None, :]) @ np.asarray(l1p, dtype=np.float64)


def forward(x, layer, bias=None):
    """Full forward.  x: [M, K] bf16 values; layer: dict from oracle.prepare.

    Returns a dict with y (fp64 [M, N]) and the intermediates the parity
    tests compare (xq packed codes, xs scales, z).
    """
    fmt = layer["fmt"]
    xa = quantize_activations(x, layer["inv_lambda"], fmt)
    a_q = xa["deq"]
    b_q = dequantize_packed(layer["wq_packed"], layer["ws"], fmt)
    y_main = a_q @ b_q.T
    z = lowrank_down(x, layer["inv_lambda"], layer["l1p"])
    y = y_main + z @ np.asarray(layer["l2p"], dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[None, :]
    return {"y": y, "y_main": y_main, "z": z, "xq": xa["packed"],
            "xs": xa["scales"], "xq_codes": xa["codes"]}


def forward_rows(x_rows, layer, bias=None):
    """Forward of a subset of rows (rows are independent: same result as the
    corresponding rows of forward())."""
    return forward(x_rows, layer, bias)


def plain_w4a4(x, w, fmt):
    """Plain RTN W4A4 without smoothing or low-rank branch: Q(X) Q(W)."""
    xa = quantize(np.asarray(x, dtype=np.float64).astype(np.float32), fmt)["deq"]
    wq = quantize(np.asarray(w, dtype=np.float64).T.astype(np.float32), fmt)["deq"]
    return xa @ wq.T
