"""Eq. (11)/(12) closed forms and the ratios the Zhou notes print."""
import json
import os

from oracle import accounting as A


def test_eq11_eq12_printed_values(golden_dir):
    with open(os.path.join(golden_dir, "accounting.json")) as f:
        fx = json.load(f)
    e = fx["eq11"]
    assert abs(100 * A.rho_mac(e["m"], e["n"], e["r"]) - e["rho_mac_percent"]) < 1e-12
    e = fx["eq12"]
    rb = A.rho_bytes(e["m"], e["n"], e["r"])
    assert abs(100 * rb - e["rho_bytes_percent"]) < 1e-12
    assert round(1 / rb, 2) == e["compression_approx"]


def test_table4_ratios(golden_dir):
    with open(os.path.join(golden_dir, "accounting.json")) as f:
        fx = json.load(f)
    t, r = fx["table4_ms"], fx["table4_ratios"]
    assert round(100 * (t["svdquant_unfused"] / t["naive_int4"] - 1), 1) == r["unfused_over_naive_percent"]
    assert round(100 * (t["svdquant_fused"] / t["naive_int4"] - 1), 1) == r["fused_over_naive_percent"]
    assert round(t["bf16"] / t["svdquant_fused"], 2) == r["fused_vs_bf16"]
    assert round(t["int8"] / t["svdquant_fused"], 2) == r["fused_vs_int8"]
    m = fx["model_size_gib"]
    assert round(m["bf16"] / m["svdquant"], 2) == m["ratio"]
    a = fx["amdahl"]
    assert round(1 / ((1 - a["f"]) + a["f"] / a["s"]), 2) == a["speedup"]


def test_kernel_byte_counts_flux_mlp_up():
    # X 25.2 MB read, codes 6.3 MB, scales 0.39 MB, Z 0.52 MB for 4096x3072, r 32, mxfp4
    b = A.ka_bytes(4096, 3072, 32, "mxfp4")
    assert abs(b / 1e6 - 32.6) < 0.1
    b = A.kb_bytes(4096, 12288, 3072, 32, "mxfp4")
    assert abs(b / 1e6 - 128.7) < 0.1
    assert A.main_ops(4096, 12288, 3072) == 2 * 4096 * 12288 * 3072


def test_bench_accounting_matches_oracle():
    # bench.py keeps its own copy of the algorithmic byte counts (the oracle
    # serves only its CPU-baseline leg); for the 4-bit formats both agree
    import bench
    for M, N, K, r in [(4096, 9216, 3072, 32), (4096, 12288, 3072, 32), (8192, 12288, 3072, 48), (256, 512, 512, 16)]:
        assert bench.main_ops(M, N, K) == A.main_ops(M, N, K)
        for fmt in ("int4", "mxfp4"):
            assert bench.ka_bytes(M, K, r, fmt) == A.ka_bytes(M, K, r, fmt)
            assert bench.kb_bytes(M, N, K, r, fmt) == A.kb_bytes(M, N, K, r, fmt)
    # 8-bit: one byte per code and one fp32 scale per row
    assert bench.kb_bytes(16, 32, 128, 16, "w8a8") == 16 * 128 + 64 + 32 * 128 + 128 + 4 * 16 * 16 + 2 * 16 * 32 + 64 + 2 * 16 * 32
