"""CPU tests of the C-ABI library's host half: symbol exports, argument
checks, the RTN packers (bit-exact against the oracle), the offline prepare
(against the oracle's own prepare), LoRA attach and the kernel layouts.
No device compute is called here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import rank_gemm_svdq_amd as B
from rank_gemm_svdq_amd import synthetic as S
from oracle import prepare as P
from oracle import quantizers as Q
from oracle.rounding import bf16_from_bits

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "svdq.h")) as f:
        hdr = f.read()
    names = set(re.findall(r"\b(svdq_[a-z_0-9]+)\s*\(", hdr))
    assert len(names) >= 15
    lib = B.lib()
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert B.abi_version() == B.ABI_VERSION == 8
    assert B.status_str(0) == "ok"


def _oracle_scales(ws, fmt):
    return np.float16(ws).view(np.uint16) if fmt == "int4" else ws


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8", "mxfp4_ocp"])
def test_packer_bit_exact_against_oracle(fmt):
    rng = np.random.default_rng(3)
    x = (rng.standard_t(3, (64, 1024)) * 0.7).astype(np.float32)
    x[0, :64] = 0.0                                  # all-zero group
    x[1, :64] = 0.0
    x[1, 0] = 5e-7                                   # fp16-subnormal INT4 scale
    x[2, :64] = np.array([7.0, 2.5, -2.5, 0.5, -0.5, 1.5, 3.5, -6.5] + [0.0] * 56, np.float32)  # exact ties
    x[3, :32] = np.linspace(-6, 6, 32).astype(np.float32)                                     # E2M1 grid
    x[4, :32] = -0.0
    x[5, :32] = 1e-39                                # MXFP4 scale clamped at 2^-127
    x[6] *= 1e4
    x[7, :] = 0.0                                    # all-zero row (8-bit: one scale per row)
    x[8, :] = 0.0
    x[8, :8] = [127.0, -3.0, 2.5, -2.5, 0.5, 126.5, -0.5, 1.5]   # 8-bit exact ties at scale 1
    x[9, :64] *= 1e30                                # INT4 scale past the fp16 range: saturated at 65504
    x[9, 64] = 7 * 65520.0                           # exactly at the fp16 overflow threshold
    x[9, 128] = 7 * 65519.0                          # just below it
    x[10, :32] = 7.0                                 # OCP rule: e = 0, every element saturates to 6
    x[10, 32:64] = np.linspace(-6.0, 6.0, 32)        # amax exactly 6: e = 0 under both rules
    x[10, 64:96] = np.float32(7.99)                  # just below 8
    codes, scales = B.pack_host(x, fmt)
    q = Q.quantize(x, fmt)
    assert np.array_equal(codes, q["packed"])
    assert np.array_equal(scales, _oracle_scales(q["scales"], fmt))


def test_calib_absmax_matches_and_rejects_nan():
    x = S.random_bf16(1, (33, 256), 3.0)
    got = B.calib_absmax(S.bf16_bits_of(x))
    assert np.array_equal(got, P.calib_amax(x))
    bits = S.bf16_bits_of(x).copy()
    bits[3, 7] = 0x7FC0
    with pytest.raises(B.SvdqError) as e:
        B.calib_absmax(bits)
    assert e.value.status == 6


def _compare_prepare(W, amax, alpha, rank, fmt, lora=None, **kw):
    pc = B.prepare(W, amax, alpha, rank, fmt, lora=lora, want_residual=True, **kw)
    po = P.prepare(W, amax, alpha, rank, fmt, lora=lora, **kw)
    assert np.array_equal(pc["lambda"], po["lam32"])
    assert np.array_equal(pc["smooth_inv"], po["inv_lambda"])
    l1, l2 = bf16_from_bits(pc["l1"]), bf16_from_bits(pc["l2"])
    if rank:
        ref = po["l1p"] @ po["l2p"]
        assert np.linalg.norm(l1 @ l2 - ref) <= 1e-4 * np.linalg.norm(ref)
        assert np.allclose(pc["sigma"], po["sigma"][:rank], rtol=1e-10, atol=0)
    assert np.linalg.norm(pc["residual"] - po["r32"]) <= 1e-4 * np.linalg.norm(po["r32"])
    # codes and scales: bit-exact except where the two SVDs land a residual
    # element on the other side of a rounding boundary (never observed here)
    mism = np.mean(pc["wq"] != po["wq_packed"])
    assert mism <= 1e-5
    assert np.mean(pc["ws"] != _oracle_scales(po["ws"], fmt)) <= 1e-5
    return pc, po


@pytest.mark.parametrize("fmt", ["int4", "mxfp4", "w8a8"])
def test_prepare_matches_oracle_tiny(fmt):
    s = S.spec("tiny")
    d = S.make_layer(s)
    pc, po = _compare_prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, fmt)
    assert np.array_equal(pc["wq"], po["wq_packed"])


@pytest.mark.parametrize("name,shape,alpha", [
    ("flux_qkv", {"K": 768, "N": 1152}, 0.5),
    ("flux_mlp_down", {"K": 1536, "N": 384}, 0.3),     # K > N: Gram on the N side
    ("flux_mlp_down", {"K": 1536, "N": 384}, 0.7),
    ("flux_mlp_up", {"K": 768, "N": 1536}, 0.5),
])
def test_prepare_matches_oracle_medium(name, shape, alpha):
    s = S.spec(name, **shape)
    d = S.make_layer(s, with_x=False)
    _compare_prepare(d["W"], P.calib_amax(d["X_cal"]), alpha, s.rank, s.fmt)


def test_prepare_full_rank_and_rank_zero():
    rng = np.random.default_rng(4)
    W = S.to_bf16_values(rng.standard_normal((128, 64)))
    amax = np.abs(rng.standard_normal(128)).astype(np.float32) + 0.1
    pc = B.prepare(W, amax, 0.5, 64, "int4", want_residual=True)
    wt = pc["lambda"][:, None].astype(np.float64) * W
    # factors in bf16 leave a residual of bf16-rounding size only
    assert np.linalg.norm(pc["residual"]) < 1e-2 * np.linalg.norm(wt)
    p0 = B.prepare(W, amax, 0.5, 0, "int4", want_residual=True)
    assert np.array_equal(p0["residual"], wt.astype(np.float32))


def test_prepare_lora_matches_oracle():
    s = S.spec("flux_lora", M=256, K=512, N=768)
    d = S.make_layer(s, with_x=False)
    lora = {"A": d["lora_A"], "B": d["lora_B"], "strength": 0.75}
    pc, po = _compare_prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, s.fmt, lora=lora)
    assert pc["l1"].shape == (512, 48) and pc["l2"].shape == (48, 768)
    # the adapter columns are exactly bf16(D A) and bf16(s B)
    assert np.array_equal(bf16_from_bits(pc["l1"])[:, 32:], po["l1p"][:, 32:])
    assert np.array_equal(bf16_from_bits(pc["l2"])[32:], po["l2p"][32:])


@pytest.mark.parametrize("fmt,rank,early", [("int4", 16, False), ("mxfp4", 48, False), ("mxfp4", 48, True),
                                             ("w8a8", 16, False)])
def test_residual_iterations_match_oracle(fmt, rank, early):
    # AutoRound doc, "Residual iteration": same error sequence, same kept
    # iteration and the same codes as the oracle's loop
    rng = np.random.default_rng(0)
    W = rng.standard_normal((128, 64)).astype(np.float32)
    amax = (np.abs(rng.standard_normal(128)) + 0.1).astype(np.float32)
    pc, po = _compare_prepare(W, amax, 0.5, rank, fmt, residual_iters=10, early_stop=early)
    n = len(po["iter_errors"])
    np.testing.assert_allclose(pc["iter_errors"][:n], po["iter_errors"], rtol=1e-9)
    assert np.isnan(pc["iter_errors"][n:]).all()
    assert pc["best_iter"] == po["best_iter"]
    assert (n < 10) == early


def test_residual_iterations_one_is_default_and_beta_explicit():
    s = S.spec("tiny")
    d = S.make_layer(s, with_x=False)
    amax = P.calib_amax(d["X_cal"])
    a = B.prepare(d["W"], amax, 0.4, 16, "int4")
    b = B.prepare(d["W"], amax, 0.4, 16, "int4", residual_iters=1, beta=0.6)
    for k in ("lambda", "l1", "l2", "wq", "ws", "iter_errors"):
        assert np.array_equal(a[k], b[k]), k
    assert a["best_iter"] == 0
    c = B.prepare(d["W"], amax, 0.4, 16, "int4", beta=0.0)
    po = P.prepare(d["W"], amax, 0.4, 16, "int4", beta=0.0)
    assert np.array_equal(c["lambda"], po["lam32"])
    assert not np.array_equal(c["lambda"], a["lambda"])


def test_error_codes_host():
    lib = B.lib()
    W = np.zeros((128, 64), np.float32)
    amax = np.ones(128, np.float32)
    # bad shapes / formats / alpha / numerics
    with pytest.raises(B.SvdqError) as e:
        B.prepare(np.zeros((100, 64), np.float32), np.ones(100, np.float32), 0.5, 16, "int4")
    assert e.value.status == 2
    with pytest.raises(B.SvdqError) as e:
        B.prepare(W, amax, 1.5, 16, "int4")
    assert e.value.status == 1
    with pytest.raises(B.SvdqError) as e:
        B.prepare(W, amax, 0.5, 24, "int4")
    assert e.value.status == 2
    with pytest.raises(B.SvdqError) as e:
        B.prepare(W, amax, 0.5, 16, "int4", residual_iters=65)
    assert e.value.status == 1
    with pytest.raises(B.SvdqError) as e:
        B.prepare(W, amax, 0.5, 16, "int4", beta=1.5)
    assert e.value.status == 1
    Wn = W.copy()
    Wn[3, 3] = np.nan
    with pytest.raises(B.SvdqError) as e:
        B.prepare(Wn, amax, 0.5, 16, "int4")
    assert e.value.status == 6
    Wr = np.random.default_rng(0).standard_normal((128, 64)).astype(np.float32)
    with pytest.raises(B.SvdqError) as e:
        B.prepare(Wr, amax, 0.5, 16, "int4", max_iters=-1)     # forced solver failure
    assert e.value.status == 6
    assert lib.svdq_layer_sizes(128, 64, 16, 7, C.byref(B.binding.Sizes())) == 4
    assert lib.svdq_layer_sizes(128, 60, 16, 0, C.byref(B.binding.Sizes())) == 2
    assert lib.svdq_layer_sizes(128, 64, 16, 0, None) == 1
    assert B.workspace_bytes(0, 128, 16, 0) == 0
    assert lib.svdq_prepare(None, None, 128, 64, 0.5, 16, 0, None, None) == 1


def test_error_codes_device_entry_points_validate_before_hip():
    """Invalid arguments are rejected on the host before any HIP call (the
    device pointers below are never dereferenced)."""
    lib = B.lib()
    L = B.binding.Layer(256, 256, 32, 1, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None)
    ws = B.workspace_bytes(64, 256, 32, 1)
    assert lib.svdq_linear_forward(None, 0x1000, 64, 0x2000, 0x3000, ws, None) == 1
    assert lib.svdq_linear_forward(C.byref(L), None, 64, 0x2000, 0x3000, ws, None) == 1
    assert lib.svdq_linear_forward(C.byref(L), 0x1008, 64, 0x2000, 0x3000, ws, None) == 3
    assert lib.svdq_linear_forward(C.byref(L), 0x1000, 64, 0x2000, 0x3000, ws - 1, None) == 5
    assert lib.svdq_linear_forward(C.byref(L), 0x1000, 0, 0x2000, 0x3000, ws, None) == 2
    uf = lib.svdq_linear_forward_unfused
    assert uf(None, 0x1000, 64, 0x2000, 0x3000, ws, None) == 1
    assert uf(C.byref(L), 0x1000, 64, 0x2008, 0x3000, ws, None) == 3
    assert uf(C.byref(L), 0x1000, 64, 0x2000, 0x3000, ws - 1, None) == 5
    bad = B.binding.Layer(256, 256, 40, 1, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None)
    assert lib.svdq_quantize_lora_down(C.byref(bad), 0x1000, 64, 0x3000, ws, None) == 2
    badf = B.binding.Layer(256, 256, 32, 4, 0x1000, 0x2000, 0x3000, 0x4000, 0x5000, None)
    assert lib.svdq_gemm_lora_up(C.byref(badf), 0x3000, ws, 64, 0x2000, None) == 4
    mis = B.binding.Layer(256, 256, 32, 1, 0x1004, 0x2000, 0x3000, 0x4000, 0x5000, None)
    assert lib.svdq_gemm_lora_up(C.byref(mis), 0x3000, ws, 64, 0x2000, None) == 3
    # the matrix-unit rate probe: kind, blocks, iterations, sink, alignment
    pr = lib.svdq_mfma_rate_probe
    assert pr(2, 0, 256, 100, 0x1000, None, None) == 1
    assert pr(-1, 0, 256, 100, 0x1000, None, None) == 1
    assert pr(0, 0, 0, 100, 0x1000, None, None) == 1
    assert pr(0, 0, 65536, 100, 0x1000, None, None) == 1
    assert pr(1, 0, 256, 0, 0x1000, None, None) == 1
    assert pr(1, 0, 256, (1 << 20) + 1, 0x1000, None, None) == 1
    assert pr(0, 0, 256, 100, None, None, None) == 1
    assert pr(0, 0, 256, 100, 0x1002, None, None) == 3
    assert pr(0, 1, 256, 100, 0x1000, 0x2004, None) == 3


def _code_off(row, t, b, steps):
    """Codes layout as documented in svdq.h: 1 KB units of 16 rows x one
    step ordered [row / 16][step]; slot 4 (row % 16) + q holds chunk
    q ^ swz(row) of the row-step, swz = row bit 1 + 2 x row bit 3."""
    r = row % 32
    swz = ((r >> 1) & 1) | ((r >> 2) & 2)
    return ((row // 16) * steps + t) * 1024 + (4 * (row % 16) + ((b // 16) ^ swz)) * 16 + b % 16


def _rec_off(row, q, j, ks4):
    """Scale records as documented in svdq.h: dword d = j // 4 of row r at
    unit dword 64 ((r % 64) // 16) + 16 d + r % 16."""
    r = row % 64
    return ((row // 64) * ks4 + q) * 1024 + (64 * (r // 16) + 16 * (j // 4) + r % 16) * 4 + j % 4


def _wrec_row(row):
    """MXFP4 weight records: row 32 p + 8 j + 4 h + i of a 64-row block stored
    as row 16 (2 p + h) + 4 j + i."""
    r = row % 64
    p, j, h, i = r // 32, (r // 8) % 4, (r // 4) % 2, r % 4
    return row - r + 16 * (2 * p + h) + 4 * j + i


def test_workspace_layout_regions():
    for M, K, r, f in [(1, 128, 0, 0), (4096, 3072, 32, 1), (8192, 3072, 48, 0), (17, 512, 16, 1),
                       (17, 512, 16, 2), (4096, 3072, 16, 2)]:
        w = B.workspace_layout(M, K, r, f)
        ks4 = (K // 128 + 3) // 4
        assert w["xq_off"] % 256 == 0 and w["xs_off"] % 256 == 0 and w["z_off"] % 256 == 0
        if f == 2:
            assert w["xq_bytes"] == (M + 15) // 16 * 16 * K
            assert w["xs_bytes"] == (M + 15) // 16 * 16 * 4
        elif f == 0:
            # FP6 codes: main parts (16 bytes per slice) then tails (8 bytes per slice)
            assert w["xq_bytes"] == (M + 15) // 16 * 16 * K // 2 + (M + 31) // 32 * 32 * K // 4
            assert w["xs_bytes"] == (M + 127) // 128 * (K // 128) * 512
        else:
            assert w["xq_bytes"] == (M + 15) // 16 * 16 * K // 2
            assert w["xs_bytes"] == (M + 63) // 64 * 64 * ks4 * 16
        assert w["xs_off"] >= w["xq_off"] + w["xq_bytes"] and w["z_off"] >= w["xs_off"] + w["xs_bytes"]
        assert w["total"] >= w["z_off"] + w["z_bytes"]
        if r:
            assert w["zsplit"] == 1
            assert w["z_bytes"] == w["zsplit"] * M * ((r + 31) // 32 * 32) * 4


E2M3_OF_INT4 = {0: 0x00, 1: 0x08, 2: 0x10, 3: 0x14, 4: 0x18, 5: 0x1A, 6: 0x1C, 7: 0x1E}


def _e2m3(q):
    """FP6 E2M3 code of an integer -7..7, from the format's definition
    (sign bit 5, exponent bits 3-4 with bias 1, mantissa bits 0-2)."""
    return (0x20 if q < 0 else 0) | E2M3_OF_INT4[abs(q)]


def test_e2m3_table_is_the_format():
    def value(c):
        e, m = (c >> 3) & 3, c & 7
        v = m / 8 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8)
        return -v if c & 0x20 else v
    for q in range(-7, 8):
        assert value(_e2m3(q)) == q


def _i4_main_off(row, t, s, steps):
    return ((row // 16) * steps + t) * 1024 + (4 * (row % 16) + (s ^ ((row >> 2) & 3))) * 16


def _i4_tail_off(row, t, s, steps):
    return ((row // 32) * steps + t) * 1024 + 256 * s + 8 * (row % 32)


def _slice_codes(main16, tail8):
    """32 six-bit codes of a slice: dwords 0-3 from the main part, 4-5 from
    the tail, element j at bits 6 j of the 192-bit string."""
    bits = int.from_bytes(bytes(main16) + bytes(tail8), "little")
    return [(bits >> (6 * j)) & 63 for j in range(32)]


def test_int4_kernel_layout_positions():
    """INT4 weights as documented in svdq.h: FP6 E2M3 codes of slice
    s = 2 G + h of each step, dwords 0-3 in 16-row main units with slot
    4 (row % 16) + (s ^ row bits 2-3), dwords 4-5 in 32-row tail units after
    all main parts; scales in 512-byte units of 128 rows x one step."""
    K, N = 640, 144
    steps = K // 128
    rng = np.random.default_rng(0)
    q = rng.integers(-7, 8, (N, K))
    sc = rng.integers(1, 30000, (N, K // 64)).astype(np.uint16)
    prep = {"K": K, "N": N, "rank": 0, "fmt": 0, "smooth_inv": np.ones(K, np.float32),
            "wq": Q.pack_nibbles(Q.int4_nibbles(q)), "ws": sc}
    sizes = B.layer_sizes(K, N, 0, "int4")
    main_bytes = (N + 15) // 16 * steps * 1024
    assert sizes["wq_bytes"] == main_bytes + (N + 31) // 32 * steps * 1024
    kl = B.kernel_layout(prep)
    wk = kl["wq_k"].reshape(-1)
    for n in list(range(0, N, 5)) + [N - 1]:
        for t in range(steps):
            for s_ in range(4):
                a = _i4_main_off(n, t, s_, steps)
                b = main_bytes + _i4_tail_off(n, t, s_, steps)
                codes = _slice_codes(wk[a:a + 16], wk[b:b + 8])
                want = [_e2m3(int(v)) for v in q[n, 128 * t + 32 * s_: 128 * t + 32 * s_ + 32]]
                assert codes == want, (n, t, s_)
    # rows 144..159 of the last tail unit are padding: zero codes
    for t in range(steps):
        for s_ in range(4):
            for n in range(N, (N + 31) // 32 * 32):
                b = main_bytes + _i4_tail_off(n, t, s_, steps)
                assert not wk[b:b + 8].any()
    ws = kl["ws_k"].view(np.uint16).reshape(-1)
    assert ws.size * 2 == sizes["ws_bytes"] == (N + 127) // 128 * steps * 512
    seen = np.zeros(ws.size, bool)
    for n in range(N):
        for t in range(steps):
            for G in range(2):
                i = ((n // 128) * steps + t) * 256 + 128 * G + n % 128
                assert ws[i] == sc[n, 2 * t + G]
                seen[i] = True
    assert np.all(ws[~seen] == 0)


def test_lowrank_factor_layout_positions():
    """Down factor: [step][s][16-column tile < rank/16][lane][i] holding
    L1'[128 step + 32 (lane / 16) + 8 s + i][16 tile + lane % 16]; up factor:
    L2'^T [N][rank rounded up to 32], zero past the rank."""
    K, N = 256, 48
    rng = np.random.default_rng(5)
    for rank in (16, 48, 64):
        l1 = rng.integers(1, 0x7F00, (K, rank)).astype(np.uint16)
        l2 = rng.integers(1, 0x7F00, (rank, N)).astype(np.uint16)
        prep = {"K": K, "N": N, "rank": rank, "fmt": 1, "smooth_inv": np.ones(K, np.float32),
                "wq": np.zeros((N, K // 2), np.uint8), "ws": np.full((N, K // 32), 127, np.uint8),
                "l1": l1, "l2": l2}
        assert B.layer_sizes(K, N, rank, 1)["l1k_bytes"] == K * rank * 2
        kl = B.kernel_layout(prep)
        l1k, nt = kl["l1k"][:K * rank].reshape(K // 128, 4, rank // 16, 64, 8), rank // 16
        for t in range(K // 128):
            for s4 in range(4):
                for tile in range(nt):
                    for lane in range(0, 64, 5):
                        for i in range(8):
                            k = 128 * t + 32 * (lane // 16) + 8 * s4 + i
                            assert l1k[t, s4, tile, lane, i] == l1[k, 16 * tile + lane % 16]
        rp = (rank + 31) // 32 * 32
        l2k = kl["l2k"][:N * rp].reshape(N, rp)
        assert np.array_equal(l2k[:, :rank], l2.T) and np.all(l2k[:, rank:] == 0)


def test_mxfp4_code_layout_positions():
    K, N = 384, 48
    steps = K // 128
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    prep = {"K": K, "N": N, "rank": 0, "fmt": 1, "smooth_inv": np.ones(K, np.float32),
            "wq": codes, "ws": np.full((N, K // 32), 127, np.uint8)}
    wk = B.kernel_layout(prep)["wq_k"].reshape(-1)
    assert wk.size == N * K // 2
    for n in range(N):
        for t in range(steps):
            for b in range(64):
                assert wk[_code_off(n, t, b, steps)] == codes[n, 64 * t + b]


def test_w8a8_code_and_scale_layout_positions():
    # 8-bit codes: byte b of 64-byte step t is element 64 t + b; scales as they are
    K, N = 384, 48
    steps = K // 64
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (N, K)).astype(np.uint8)
    sc = rng.standard_normal(N).astype(np.float32)
    prep = {"K": K, "N": N, "rank": 0, "fmt": 2, "smooth_inv": np.ones(K, np.float32), "wq": codes, "ws": sc}
    kl = B.kernel_layout(prep)
    wk = kl["wq_k"].reshape(-1)
    assert wk.size == N * K
    for n in range(N):
        for t in range(steps):
            for b in range(64):
                assert wk[_code_off(n, t, b, steps)] == codes[n, 64 * t + b]
    assert np.array_equal(kl["ws_k"].view(np.float32), sc)
    s = B.layer_sizes(K, N, 16, 2)
    assert s["wq_canon_bytes"] == N * K and s["ws_canon_bytes"] == N * 4


def test_mxfp4_scale_layout_positions():
    K, N = 1024, 80
    rng = np.random.default_rng(1)
    sc = rng.integers(100, 150, (N, K // 32)).astype(np.uint8)
    prep = {"K": K, "N": N, "rank": 0, "fmt": 1, "smooth_inv": np.ones(K, np.float32),
            "wq": np.zeros((N, K // 2), np.uint8), "ws": sc}
    kl = B.kernel_layout(prep)
    ks4 = (K // 128 + 3) // 4
    row = kl["ws_k"].reshape(-1)
    assert row.size == (N + 63) // 64 * 64 * ks4 * 16
    seen = np.zeros(row.size, bool)
    for n in range(N):
        for b in range(K // 32):
            t, g = divmod(b, 4)
            i = _rec_off(_wrec_row(n), t // 4, 4 * g + t % 4, ks4)
            assert row[i] == sc[n, b]
            seen[i] = True
    assert np.all(row[~seen] == 127)


def test_smooth_candidates_match_oracle():
    from oracle import search as SR
    for g in (2, 4, 20, 33):
        assert B.smooth_candidates(g) == SR.candidates(g)       # same doubles, same order
    assert B.lib().svdq_smooth_candidates(1, None, None) == 0
    assert B.lib().svdq_smooth_candidates(1001, None, None) == 0


def test_smooth_search_validates_before_hip():
    import ctypes as C
    lib = B.lib()
    W = np.ones((512, 256), np.float32)
    res = B.SearchResult(0, -1, 0.0, 0.0, None)
    opts = B.SearchOpts(4, 1, 0, 0)
    fake = C.c_void_p(1 << 20)            # never dereferenced: every case fails validation first
    ws_ok = B.search_workspace_bytes(128, 512, 256, 16, "int4")
    assert ws_ok > 0 and B.search_workspace_bytes(0, 512, 256, 16, "int4") == 0

    def call(w=W.ctypes.data_as(C.c_void_p), K=512, N=256, rank=16, fmt=0, x=fake, M=128, o=opts, ws=fake,
             wsb=ws_ok, r=res):
        return lib.svdq_smooth_search(w, K, N, rank, fmt, x, M, C.byref(o) if o is not None else None, ws, wsb,
                                      None, C.byref(r) if r is not None else None, None)
    assert call(w=None) == 1
    assert call(r=None) == 1
    assert call(o=B.SearchOpts(1, 1, 0, 0)) == 1
    assert call(fmt=7) == 4
    assert call(K=500) == 2
    assert call(rank=24) == 2
    assert call(M=0) == 2
    assert call(x=C.c_void_p((1 << 20) + 2)) == 3
    assert call(ws=C.c_void_p((1 << 20) + 16)) == 3
    assert call(wsb=ws_ok - 1) == 5
    Wn = W.copy()
    Wn[1, 1] = np.inf
    assert call(w=Wn.ctypes.data_as(C.c_void_p)) == 6


def test_reservoir_select_matches_oracle():
    from oracle import search as SR
    for n, k, seed in [(5, 8, 1), (1000, 128, 7), (300, 17, 2 ** 63 + 5), (129, 128, 0), (0, 3, 1), (3, 0, 1)]:
        assert B.reservoir_select(n, k, seed) == SR.reservoir_select(n, k, seed)
    assert B.lib().svdq_reservoir_select(10, 3, 1, None) == -1


def test_binding_rejects_unusable_tensors_before_the_library(monkeypatch):
    """The device entry points take bare pointers; the binding checks dtype,
    shape, contiguity and device first and raises without calling into the
    library (which is replaced here by a function that fails the test)."""
    import types
    import torch
    from rank_gemm_svdq_amd import binding as BD

    def no_call():
        raise AssertionError("the library was called")

    monkeypatch.setattr(BD, "lib", no_call)
    monkeypatch.setattr(BD, "status_str", lambda s: "error")
    lay = types.SimpleNamespace(K=256, N=128, rank=16, fmt=0, struct=None, wq=torch.empty(1, dtype=torch.uint8))
    X = torch.zeros((8, 256), dtype=torch.int16)
    Y = torch.zeros((8, 128), dtype=torch.int16)
    ws = torch.zeros(4096, dtype=torch.uint8)
    cases = [
        (dict(X=X.float()), "dtype"),
        (dict(X=torch.zeros((8, 255), dtype=torch.int16)), "shape"),
        (dict(X=torch.zeros((256, 8), dtype=torch.int16).T), "contiguous"),
        (dict(Y=torch.zeros((8, 127), dtype=torch.int16)), "shape"),
        (dict(Y=torch.zeros((9, 128), dtype=torch.bfloat16)), "shape"),
        (dict(ws=ws.view(torch.int8)), "dtype"),
        (dict(), "GPU memory"),                       # everything right, but host tensors
    ]
    for over, msg in cases:
        a = dict(X=X, Y=Y, ws=ws)
        a.update(over)
        for call in (lambda: BD.linear_forward(lay, a["X"], a["Y"], a["ws"]),
                     lambda: BD.linear_forward_unfused(lay, a["X"], a["Y"], a["ws"])):
            with pytest.raises(BD.SvdqError, match=msg):
                call()
    with pytest.raises(BD.SvdqError, match="dtype"):
        BD.quantize_lora_down(lay, X.float(), ws)
    with pytest.raises(BD.SvdqError, match="shape"):
        BD.gemm_lora_up(lay, ws, 8, torch.zeros((8, 64), dtype=torch.int16))
    with pytest.raises(BD.SvdqError, match="GPU memory"):
        BD.gemm_lora_up(lay, ws, 8, Y)


def test_noalloc_forward_rejects_oversize_before_any_device_call():
    """svdq_linear_forward_noalloc validates the layer and the workspace
    size against its fixed maximum before it touches the device, so the
    rejections below return on a machine without a GPU (the pointers are
    never dereferenced)."""
    lib = B.lib()
    L = B.binding.Layer(3072, 12288, 32, B.MXFP4, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, None)
    M = 40000
    assert B.workspace_bytes(M, 3072, 32, "mxfp4") > B.NOALLOC_MAX_WORKSPACE
    assert lib.svdq_linear_forward_noalloc(C.byref(L), C.c_void_p(0x2000), M, C.c_void_p(0x3000), None) == 5
    assert lib.svdq_linear_forward_noalloc(C.byref(L), None, 16, C.c_void_p(0x3000), None) == 1
    assert lib.svdq_linear_forward_noalloc(C.byref(L), C.c_void_p(0x2008), 16, C.c_void_p(0x3000), None) == 3
    L.rank = 20
    assert lib.svdq_linear_forward_noalloc(C.byref(L), C.c_void_p(0x2000), 16, C.c_void_p(0x3000), None) == 2
