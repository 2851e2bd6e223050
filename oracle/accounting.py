"""Closed-form cost accounting (test infrastructure only).

Zhou notes sec. 6.1, Eq. (11):  rho_MAC = (bmr + brn) / (bmn) = r/m + r/n.
Zhou notes sec. 6.2, Eq. (12):  rho_bytes = (mn/2 + 2r(m + n)) / (2mn)
                                          = 1/4 + r/m + r/n.
Algorithmic byte and op counts of the two fused kernels follow from the
tensors each one must read or write once (Algorithm 2 of the notes).

Pins: the values the notes print for a 4096 x 4096 weight with r = 32
(1.5625 %, 26.5625 %, about 3.76x).
"""


def rho_mac(m, n, r):
    return (m * r + r * n) / (m * n)


def rho_bytes(m, n, r):
    return (m * n / 2 + 2 * r * (m + n)) / (2 * m * n)


def group_and_scale_bytes(fmt):
    return (64, 2) if fmt == "int4" else (32, 1)


def main_ops(M, N, K):
    """2MNK: the 4-bit main contraction."""
    return 2 * M * N * K


def lowrank_ops(M, N, K, r):
    return 2 * M * r * (K + N)


def ka_bytes(M, K, r, fmt):
    """Fused smooth + quantize + lora_down: read X, inv_lambda, L1'; write
    packed codes, scales and Z (fp32)."""
    g, sb = group_and_scale_bytes(fmt)
    return 2 * M * K + M * K // 2 + M * (K // g) * sb + 4 * M * r + 2 * K * r + 4 * K


def kb_bytes(M, N, K, r, fmt):
    """W4A4 GEMM + lora_up + bias: read activation codes/scales, weight
    codes/scales, Z, L2', bias; write Y (bf16)."""
    g, sb = group_and_scale_bytes(fmt)
    return (M * K // 2 + M * (K // g) * sb + N * K // 2 + N * (K // g) * sb
            + 4 * M * r + 2 * r * N + 2 * N + 2 * M * N)
