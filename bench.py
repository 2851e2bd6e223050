"""Benchmark of the SVDQuant W4A4 + low-rank linear layer on one MI355X.

One step = one svdq_linear_forward (K-A: smooth + quantize + lora_down, then
K-B: 4-bit GEMM + lora_up + bias) over a resident synthetic FLUX-shaped
layer.  Prints ONE JSON line with the throughput (2MNK / step time), the
roofline of the dominant kernel (K-B) measured with HIP events on the launch
stream, the low-rank overhead over the same kernels at rank 0, a parity
check against the oracle on sampled rows, and the oracle timed on the host
cores as a baseline.

  python bench.py [--steps K] [--warmup W] [--config flux_mlp_up] [--gpus 1]

Profiles: run the same command under rocprofv3 (kernel trace + stats, then
one --pmc pass each for FETCH_SIZE and WRITE_SIZE with --calib-copy, which
adds a device copy of known size to scale the counters), then
  python bench.py --summarize-profiles DIR
writes the text summaries and the per-launch HBM traffic under profiles/.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"mxfp4": 10.1e15, "mxfp4_ocp": 10.1e15, "int4": 5.0e15, "w8a8": 5.0e15}   # dense MFMA peaks: FP4 / int8
PEAK_NAME = {"mxfp4": "fp4 MFMA", "mxfp4_ocp": "fp4 MFMA", "int4": "int8 MFMA", "w8a8": "int8 MFMA"}
DTYPE = {"mxfp4": "fp4", "mxfp4_ocp": "fp4", "int4": "int4", "w8a8": "int8"}   # operand type of the main contraction


# Algorithmic work of one layer (what the kernels must at least move or
# compute, independent of how they tile it).
def main_ops(M, N, K):
    """2MNK: the quantized main contraction."""
    return 2 * M * N * K


def metric_name(name, fmt, M, K, N):
    """The headline metric; the FLUX MLP up projection in MXFP4 is the
    benchmark line, other workloads name their own shape."""
    kind = "W8A8" if fmt == "w8a8" else "W4A4"
    where = "FLUX MLP" if name == "flux_mlp_up" and fmt == "mxfp4" else f"{name} {fmt}"
    return f"{kind}+low-rank linear TOPS and % of MFMA peak ({where} {M}\u00d7{K}\u2192{N})"


def code_and_scale_bytes(rows, K, fmt):
    """Codes plus scales of `rows` quantized rows of K elements."""
    if fmt == "w8a8":
        return rows * K + 4 * rows
    g, sb = (64, 2) if fmt == "int4" else (32, 1)
    return rows * K // 2 + rows * (K // g) * sb


def ka_bytes(M, K, r, fmt):
    """K-A: read X (bf16), 1/lambda, L1'; write codes, scales and Z (bf16 hi + lo)."""
    return 2 * M * K + 4 * K + 2 * K * r + code_and_scale_bytes(M, K, fmt) + 4 * M * r


def kb_bytes(M, N, K, r, fmt):
    """K-B: read activation and weight codes/scales, Z, L2', bias; write Y (bf16)."""
    return (code_and_scale_bytes(M, K, fmt) + code_and_scale_bytes(N, K, fmt)
            + 4 * M * r + 2 * r * N + 2 * N + 2 * M * N)
HBM_PEAK = 8.0e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kb_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the kernel source's code: comments and blank lines are left
    out, so a comment edit keeps counter measurements of the same code."""
    p = os.path.join(ROOT, "rank_gemm_svdq_amd", "csrc", "device_kernels.hip")
    lines = []
    with open(p, encoding="utf-8") as fh:
        for line in fh:
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def measured_traffic(config):
    """HBM bytes per K-B launch from the committed rocprofv3 counter runs, if
    they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(config)
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def kb_kernel_names(fmt, K, rank):
    """Demangled and mangled names of the K-B instantiation a layer launches."""
    ntr = ((rank + 31) // 32 * 32) // 32
    if fmt in ("mxfp4", "mxfp4_ocp"):
        odd = (K // 128) % 2
        return (f"kb_mx_kernel<{ntr}, {'true' if odd else 'false'}, 8, false>",
                f"kb_mx_kernelILi{ntr}ELb{odd}ELi8ELb0E")
    if fmt == "w8a8":
        return (f"kb_mx_kernel<{ntr}, false, 8, true>", f"kb_mx_kernelILi{ntr}ELb0ELi8ELb1E")
    return (f"kb_i4_kernel<{ntr}>", f"kb_i4_kernelILi{ntr}E")


def kb_uses_tail(fmt, M, N, cus):
    """The library's split (kb_mx_main_cols): with 256 x 256 tiles whose last
    round would fill at most a quarter of the compute units, the last columns
    run as a second launch of 128 x 128 tiles."""
    if fmt not in ("mxfp4", "mxfp4_ocp", "w8a8"):
        return False
    tm, tn = (M + 255) // 256, (N + 255) // 256
    tiles = tm * tn
    tail = tiles % cus
    return tiles > cus and tail != 0 and 4 * tail <= cus and (tiles // cus) * cus // tm < tn


def kb_label(fmt, M, N, K, rank, torch):
    main = kb_kernel_names(fmt, K, rank)[0]
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    if kb_uses_tail(fmt, M, N, cus):
        return f"{main} + {kb_tail_names(fmt, K, rank)[0]} (last columns, 128 x 128 tiles)"
    return main


def kb_tail_names(fmt, K, rank):
    """Names of the 128 x 128-tile K-B kernel that takes the last columns
    when 256 x 256 tiles would leave a mostly idle last round (MXFP4 and
    W8A8), or None."""
    if fmt not in ("mxfp4", "mxfp4_ocp", "w8a8"):
        return None
    ntr = ((rank + 31) // 32 * 32) // 32
    w8 = fmt == "w8a8"
    odd = 0 if w8 else (K // 128) % 2
    return (f"kb_mx_tail_kernel<{ntr}, {'true' if odd else 'false'}, {'true' if w8 else 'false'}>",
            f"kb_mx_tail_kernelILi{ntr}ELb{odd}ELb{int(w8)}E")


def oracle_sample(F, X, po, bias, seconds):
    """(rows, passes, seconds) of oracle forward work that takes about
    `seconds`: the first n token rows, n grown until it does, or whole-layer
    passes repeated when the whole layer takes less."""
    M = X.shape[0]
    n = 16
    while True:
        t0 = time.perf_counter()
        F.forward(X[:n], po, bias)
        t = time.perf_counter() - t0
        if t >= 0.5 * seconds:
            return n, 1, t
        if n >= M:
            break
        n = min(M, int(n * min(8.0, max(2.0, seconds / max(t, 1e-3)))))
    passes = max(1, int(round(seconds / max(t, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(passes):
        F.forward(X, po, bias)
    return M, passes, time.perf_counter() - t0


CALIB_BYTES = 256 << 20


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="flux_mlp_up")
    ap.add_argument("--fmt", default=None, help="override the workload's format (int4 | mxfp4 | mxfp4_ocp | w8a8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sustained-peak", action="store_true",
                    help="skip the matrix-unit rate probe (profiling runs leave it out)")
    ap.add_argument("--no-rotate", action="store_true",
                    help="skip the cache-rotated run (distinct buffer sets cycled per step)")
    ap.add_argument("--rotate-sets", type=int, default=0,
                    help="buffer sets of the rotated run (0: enough to exceed 512 MB, at least 3)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--skip-oracle", action="store_true",
                    help="timing only: no oracle parity check and no CPU baseline (profiling runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one device-to-device copy of 256 MiB (counter calibration)")
    ap.add_argument("--print-profile-commands", metavar="DIR", default=None,
                    help="print the rocprofv3 commands whose output --summarize-profiles reads")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="summarise rocprofv3 output under DIR into profiles/ (no GPU needed)")
    ap.add_argument("--smooth-search", type=int, metavar="G", default=0,
                    help="time the smooth-factor grid search (2G-1 candidates) of the workload's layer on "
                         "its calibration rows and print that JSON line instead")
    ap.add_argument("--residual-iters", type=int, metavar="T", default=0,
                    help="time the host preparation of the workload's layer with T residual iterations "
                         "and print that JSON line instead")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the vendor library's plain GEMMs (through torch) on the workload's shape "
                         "beside this library's forward and print that JSON line instead")
    args = ap.parse_args()
    if args.residual_iters:
        return bench_residual(args)
    if args.print_profile_commands:
        cfg = args.config + (f" --fmt {args.fmt}" if args.fmt else "")
        for k, c in profile_commands(args.print_profile_commands, cfg).items():
            print(f"{k}\t{c}")
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.config, args.fmt)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer shards over tokens with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import rank_gemm_svdq_amd as B
    from rank_gemm_svdq_amd import synthetic as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if B.device_check(0) != 0:
        raise SystemExit("device is not gfx950")

    over = {"fmt": args.fmt} if args.fmt else {}
    s = S.spec(args.config, **over)
    if args.smooth_search:
        return bench_search(args, s)
    if args.vendor_gemm:
        return bench_vendor(args, s)
    M, K, N, fmt = s.M, s.K, s.N, s.fmt
    log(f"workload {s.name}: M={M} K={K} N={N} rank={s.rank}+{s.lora_rank} fmt={fmt}")
    d = S.make_layer(s)
    lora = None
    if s.lora_rank:
        lora = {"A": d["lora_A"], "B": d["lora_B"], "strength": 1.0}
    t0 = time.time()
    amax = B.calib_absmax(S.bf16_bits_of(d["X_cal"]))
    prep = B.prepare(d["W"], amax, s.alpha, s.rank, fmt, lora=lora)
    prep0 = B.prepare(d["W"], amax, s.alpha, 0, fmt)
    log(f"host prepare {time.time() - t0:.1f} s")
    bias_bits = S.bf16_bits_of(d["bias"])
    layer = B.DeviceLayer(prep, bias_bits)
    layer0 = B.DeviceLayer(prep0, bias_bits)
    X = torch.from_numpy(S.bf16_bits_of(d["X"]).view(np.int16)).cuda()
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = layer.workspace(M)
    ws0 = layer0.workspace(M)
    stream = torch.cuda.current_stream()

    def per_kernel(lay, wsb, steps):
        """Per-kernel durations: an event before, between and after the two
        launches of every step (these events are not in the headline)."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
               torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1, e2 in ev:
            e0.record(stream)
            B.quantize_lora_down(lay, X, wsb)
            e1.record(stream)
            B.gemm_lora_up(lay, wsb, M, Y)
            e2.record(stream)
        torch.cuda.synchronize()
        return (np.array([a.elapsed_time(b) for a, b, _ in ev]), np.array([b.elapsed_time(c) for _, b, c in ev]))

    def chunk(lay, wsb, steps, fwd=None):
        """Back-to-back forward calls between one pair of events."""
        fwd = fwd or B.linear_forward
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        for _ in range(steps):
            fwd(lay, X, Y, wsb)
        end.record(stream)
        return start, end

    for _ in range(args.warmup):
        B.linear_forward(layer0, X, Y, ws0)
        B.linear_forward(layer, X, Y, ws)
        B.linear_forward_unfused(layer, X, Y, ws)
    torch.cuda.synchronize()
    # rank-0 (plain W4A4) chunks interleaved with the layer's, so both see the
    # same clocks; then the timed region proper: exactly `steps` forwards
    log("timing rank-0 (plain W4A4) and the layer, interleaved")
    trip = []
    for _ in range(5):
        trip.append((chunk(layer0, ws0, 10), chunk(layer, ws, 10),
                     chunk(layer, ws, 10, B.linear_forward_unfused)))
    torch.cuda.synchronize()
    ms0_chunks = np.array([a[0].elapsed_time(a[1]) / 10 for a, _, _ in trip])
    msr_chunks = np.array([b[0].elapsed_time(b[1]) / 10 for _, b, _ in trip])
    msu_chunks = np.array([c[0].elapsed_time(c[1]) / 10 for _, _, c in trip])
    log("timing the layer")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start, end = chunk(layer, ws, args.steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = start.elapsed_time(end) / args.steps
    ka, kb = per_kernel(layer, ws, max(50, args.steps))
    ka0, kb0 = per_kernel(layer0, ws0, max(10, args.steps // 2))
    # spread of single steps (events between consecutive forwards; not the
    # headline, which times the K steps as one region)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(max(50, args.steps) + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for e in ev[1:]:
        B.linear_forward(layer, X, Y, ws)
        e.record(stream)
    torch.cuda.synchronize()
    step_ms = np.array([a.elapsed_time(b) for a, b in zip(ev[:-1], ev[1:])])
    rotated = None
    if not args.no_rotate:
        rotated = rotated_run(args, torch, B, prep, bias_bits, X, M, N, stream)

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    r = prep["rank"]
    t_step = ms * 1e-3
    ops = main_ops(M, N, K)
    tops = ops / t_step
    t_kb = float(np.median(kb)) * 1e-3
    t_ka = float(np.median(ka)) * 1e-3
    kb_achieved = ops / t_kb
    ka_b = ka_bytes(M, K, r, fmt)
    kb_b = kb_bytes(M, N, K, r, fmt)
    traffic = measured_traffic(s.name if not args.fmt else f"{s.name}_{fmt}")
    t_step0 = float(np.median(ms0_chunks)) * 1e-3
    t_stepr = float(np.median(msr_chunks)) * 1e-3
    t_stepu = float(np.median(msu_chunks)) * 1e-3

    sustained = None if args.no_sustained_peak else sustained_peak(torch, B, fmt, stream, kb_achieved)

    cpu, parity = None, None
    if not args.no_cpu_baseline and not args.skip_oracle:
        # The CPU-baseline leg: the fp64 oracle prepares the same layer and
        # runs its forward on a bounded sample of rows on the host cores; the
        # device output of those rows is compared with it on the way.
        from threadpoolctl import threadpool_info
        from oracle import forward as F
        from oracle import prepare as P
        log("cpu baseline: oracle prepare (fp64, LAPACK SVD)")
        t0 = time.time()
        po = P.prepare(d["W"], P.calib_amax(d["X_cal"]), s.alpha, s.rank, fmt, lora=lora)
        t_oracle_prepare = time.time() - t0
        rng = np.random.default_rng(0)
        rows = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 62, replace=False)]))
        B.linear_forward(layer, X, Y, ws)
        torch.cuda.synchronize()
        y = Y[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16)
        y = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        of = F.forward(d["X"][rows], po, d["bias"])
        rel = float(np.linalg.norm(y - of["y"]) / np.linalg.norm(of["y"]))
        xq, xs, _ = B.unpack_activations(ws.cpu().numpy(), M, K, prep["rank"], fmt)
        mism = int(np.sum(xq[rows] != of["xq"]))
        log(f"parity on {len(rows)} rows: rel_fro={rel:.3e} code mismatches={mism}")
        parity = {"rows": int(len(rows)), "rel_fro": rel, "tolerance": 5e-3, "code_mismatches": mism}
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        # bounded sample: the first n token rows of the same layer, n grown
        # until the oracle forward takes about cpu_seconds
        nrows, passes, t_cpu = oracle_sample(F, d["X"], po, d["bias"], args.cpu_seconds)
        what = (f"{passes} passes over all {M} token rows" if nrows == M
                else f"the first {nrows} of {M} token rows")
        cpu = {"value": 2.0 * nrows * passes * N * K / t_cpu / 1e12, "unit": "TOPS", "cores": threads,
               "kind": "oracle",
               "sample": f"oracle forward (fp64: smoothing, quantisation, decoded GEMM, low-rank branch, bias), "
                         f"{what} of the same layer, {t_cpu:.1f} s on {threads} BLAS threads; oracle prepare "
                         f"(LAPACK SVD) took {t_oracle_prepare:.1f} s and is not in the rate",
               "host_cpus": os.cpu_count()}

    out = {
        "metric": metric_name(s.name, fmt, M, K, N),
        "value": tops / 1e12, "unit": "TOPS", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": DTYPE[fmt], "data": "synthetic (seeded FLUX-shaped layer, random weights)",
        "config": {"workload": s.name, "M": M, "K": K, "N": N, "rank": r, "format": fmt,
                   "alpha": s.alpha, "bias": True},
        "pct_of_peak": 100.0 * tops / PEAK[fmt], "peak_name": PEAK_NAME[fmt],
        "roofline": {"bound": "mfma", "achieved": kb_achieved / 1e12, "peak": PEAK[fmt] / 1e12, "unit": "TFLOP/s",
                     "frac": kb_achieved / PEAK[fmt],
                     "traffic": traffic, "kernel": kb_label(fmt, M, N, K, r, torch) + " (quantized GEMM + lora_up + bias)",
                     "algorithmic_ops_per_launch": ops, "algorithmic_bytes_per_launch": kb_b},
        "sustained_peak": sustained,
        "ka": {"us": t_ka * 1e6, "algorithmic_bytes": ka_b, "GB_per_s": ka_b / t_ka / 1e9,
               "frac_of_hbm": ka_b / t_ka / HBM_PEAK},
        "kb_us": t_kb * 1e6,
        "step_us": {"n": int(len(step_ms)), "median": float(np.median(step_ms)) * 1e3,
                    "min": float(step_ms.min()) * 1e3, "max": float(step_ms.max()) * 1e3,
                    "p10": float(np.percentile(step_ms, 10)) * 1e3, "p90": float(np.percentile(step_ms, 90)) * 1e3,
                    "TOPS_at_median": ops / (float(np.median(step_ms)) * 1e-3) / 1e12},
        "kernel_us_spread": {"ka": [float(ka.min()) * 1e3, float(np.median(ka)) * 1e3, float(ka.max()) * 1e3],
                             "kb": [float(kb.min()) * 1e3, float(np.median(kb)) * 1e3, float(kb.max()) * 1e3],
                             "order": "min, median, max"},
        "cache_state": working_set_note(X, M, N, prep, layer),
        "rotated": rotated,
        "lowrank_overhead": t_stepr / t_step0 - 1.0, "rank0_layer_us": t_step0 * 1e6,
        "layer_us_interleaved": t_stepr * 1e6,
        "unfused": {"layer_us": t_stepu * 1e6, "lowrank_overhead": t_stepu / t_step0 - 1.0,
                    "kernels": "quantize; down projection (second pass over X); quantized GEMM + bias; Y += Z L2'"},
        "rank0_ka_us": float(np.median(ka0)) * 1e3, "rank0_kb_us": float(np.median(kb0)) * 1e3,
        "parity": parity,
        "cpu_baseline": cpu,
        "wall_s_timed": wall,
    }
    print(json.dumps(out))


def sustained_peak(torch, B, fmt, stream, kb_achieved):
    """What the matrix units sustain on this device, beside the datasheet
    peak: every compute unit issuing MFMAs of K-B's arithmetic (FP4 for
    MXFP4, int8 for INT4 and W8A8) back to back on changing operands, with
    no memory traffic (svdq_mfma_rate_probe). Random operand bytes toggle
    the most and bound what real data gets; zero operands the least."""
    kind = 0 if fmt in ("mxfp4", "mxfp4_ocp") else 1
    blocks = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    iters = 2000
    per_iter = 32 if kind == 0 else 16
    ops = blocks * 8 * per_iter * iters * 65536
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    marks = torch.zeros(blocks * 16, dtype=torch.int64, device="cuda")
    res = {}
    for name, zero in (("random_operands", 0), ("zero_operands", 1)):
        B.mfma_rate_probe(kind, zero, blocks, iters, sink, marks, stream)
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            B.mfma_rate_probe(kind, zero, blocks, iters, sink, marks, stream)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        m = marks.view(-1, 2).cpu().numpy().astype(np.float64)
        clock = float(np.median(m[:, 0] / (m[:, 1] / 100e6))) / 1e9
        res[name] = {"rate": ops / float(np.median(times)) / 1e12, "clock_GHz": clock}
    rnd = res["random_operands"]["rate"]
    return {"mfma": "scaled 16x16x128 FP4" if kind == 0 else "32x32x32 int8", "unit": "TFLOP/s",
            "random_operands": res["random_operands"], "zero_operands": res["zero_operands"],
            "kb_frac_of_random_operands": kb_achieved / 1e12 / rnd,
            "how": f"{blocks} blocks of two waves per SIMD, {per_iter} MFMAs per wave and iteration, {iters} "
                   "iterations, operands changing every MFMA, no memory traffic; median of 3 launches"}

def working_set_note(X, M, N, prep, layer):
    """How much of one step's data the 256 MB last-level cache can hold
    across back-to-back steps (the warm headline's residency)."""
    import rank_gemm_svdq_amd as B
    per = X.numel() * 2 + M * N * 2 + B.workspace_bytes(M, prep["K"], prep["rank"], prep["fmt"])
    per += sum(t.numel() * t.element_size() for t in (layer.wq, layer.ws, layer.l1k, layer.l2k, layer.smooth_inv)
               if t is not None)
    mb = per / 1e6
    if per <= (256 << 20):
        return (f"warm: the layer's X, weights, workspace and Y ({mb:.0f} MB) fit in the 256 MB last-level cache "
                f"across back-to-back steps; see 'rotated' for a cold-cache run")
    return (f"partly warm: the layer's X, weights, workspace and Y ({mb:.0f} MB) exceed the 256 MB last-level "
            f"cache; see 'rotated' for a cold-cache run")


def rotated_run(args, torch, B, prep, bias_bits, X, M, N, stream):
    """The same forward with the last-level cache defeated: several complete
    sets of X, layer buffers, workspace and Y (distinct device memory, same
    values), the sets cycled step by step, so every step reads operands the
    previous steps have pushed out of the 256 MB cache.  Returns the step
    time as one timed region and per-kernel medians."""
    per_set = X.numel() * 2 + M * N * 2 + B.workspace_bytes(M, prep["K"], prep["rank"], prep["fmt"])
    lay0 = B.DeviceLayer(prep, bias_bits)
    per_set += sum(t.numel() * t.element_size() for t in (lay0.wq, lay0.ws, lay0.l1k, lay0.l2k, lay0.smooth_inv)
                   if t is not None)
    n = args.rotate_sets or max(3, -(-(512 << 20) // per_set))
    sets = []
    for i in range(n):
        lay = lay0 if i == 0 else B.DeviceLayer(prep, bias_bits)
        sets.append((lay, X.clone(), torch.empty((M, N), dtype=torch.int16, device="cuda"), lay.workspace(M)))
    for _ in range(max(2, args.warmup // n)):
        for lay, x, y, w in sets:
            B.linear_forward(lay, x, y, w)
    steps = max(args.steps, 2 * n)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        lay, x, y, w = sets[i % n]
        B.linear_forward(lay, x, y, w)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b, c) in enumerate(ev):
        lay, x, y, w = sets[i % n]
        a.record(stream)
        B.quantize_lora_down(lay, x, w)
        b.record(stream)
        B.gemm_lora_up(lay, w, M, y)
        c.record(stream)
    torch.cuda.synchronize()
    ka = np.array([a.elapsed_time(b) for a, b, _ in ev])
    kb = np.array([b.elapsed_time(c) for _, b, c in ev])
    ops = main_ops(M, N, prep["K"])
    out = {"sets": n, "bytes_per_set": int(per_set), "steps": steps, "ms_per_step": ms,
           "TOPS": ops / (ms * 1e-3) / 1e12, "ka_us_median": float(np.median(ka)) * 1e3,
           "kb_us_median": float(np.median(kb)) * 1e3,
           "ka_GB_per_s": ka_bytes(M, prep["K"], prep["rank"], {0: "int4", 1: "mxfp4", 2: "w8a8", 3: "mxfp4_ocp"}[prep["fmt"]])
           / (float(np.median(ka)) * 1e-3) / 1e9}
    del sets
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------ profile summaries

PROFILE_STEPS = {
    "stats": "--kernel-trace --stats --output-format csv -d {dir}/stats -o run -- "
             "python -u bench.py --config {config} --steps 20 --warmup 5 --skip-oracle --no-sustained-peak",
    "fetch": "--pmc FETCH_SIZE --output-format csv -d {dir}/fetch -o run -- "
             "python -u bench.py --config {config} --steps 3 --warmup 1 --skip-oracle --no-sustained-peak --calib-copy",
    "write": "--pmc WRITE_SIZE --output-format csv -d {dir}/write -o run -- "
             "python -u bench.py --config {config} --steps 3 --warmup 1 --skip-oracle --no-sustained-peak --calib-copy",
    "mfma": "--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_WAVES --output-format csv "
            "-d {dir}/mfma -o run -- python -u bench.py --config {config} --steps 3 --warmup 1 --skip-oracle --no-sustained-peak",
    "waves": "--pmc SQ_WAVES SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_BUSY_CYCLES SQ_INSTS_VMEM_RD "
             "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE --output-format csv "
             "-d {dir}/waves -o run -- python -u bench.py --config {config} --steps 3 --warmup 1 --skip-oracle --no-sustained-peak",
    "l2": "--pmc TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum GRBM_GUI_ACTIVE --output-format csv "
          "-d {dir}/l2 -o run -- python -u bench.py --config {config} --steps 3 --warmup 1 --skip-oracle --no-sustained-peak",
}


def bench_residual(args):
    """Host preparation with residual iteration: seconds per iteration and
    the weight reconstruction error of every iteration (no GPU needed)."""
    import rank_gemm_svdq_amd as B
    from rank_gemm_svdq_amd import synthetic as S

    over = {"fmt": args.fmt} if args.fmt else {}
    s = S.spec(args.config, **over)
    d = S.make_layer(s, with_x=False)
    amax = B.calib_absmax(S.bf16_bits_of(d["X_cal"]))
    T = args.residual_iters
    t0 = time.perf_counter()
    p1 = B.prepare(d["W"], amax, s.alpha, s.rank, s.fmt)
    t1 = time.perf_counter() - t0
    t0 = time.perf_counter()
    p = B.prepare(d["W"], amax, s.alpha, s.rank, s.fmt, residual_iters=T)
    tt = time.perf_counter() - t0
    e = p["iter_errors"]
    assert e[0] == p1["iter_errors"][0]
    out = {
        "metric": "residual_iteration_seconds", "value": (tt - t1) / max(T - 1, 1), "unit": "s/iteration",
        "n_gpus": 0, "higher_is_better": False, "data": "synthetic",
        "config": {"workload": s.name, "K": s.K, "N": s.N, "rank": s.rank, "fmt": s.fmt, "residual_iters": T},
        "prepare_one_iteration_s": t1, "prepare_total_s": tt, "iter_errors": [float(v) for v in e],
        "best_iter": p["best_iter"], "error_reduction": float(1.0 - min(e) / e[0]),
        "host_threads": int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count(),
    }
    print(json.dumps(out), flush=True)


def bench_search(args, s):
    """The smooth-factor grid search of one layer: host preparation of every
    candidate plus its scoring forward on the calibration rows."""
    import torch
    import rank_gemm_svdq_amd as B
    from rank_gemm_svdq_amd import synthetic as S

    d = S.make_layer(s, with_x=False)
    xc = torch.from_numpy(S.bf16_bits_of(d["X_cal"]).view(np.int16)).cuda()
    mc = xc.shape[0]
    g = args.smooth_search
    n = len(B.smooth_candidates(g))
    log(f"smooth search {s.name}: {n} candidates, calibration rows {mc}, K={s.K} N={s.N} rank={s.rank} {s.fmt}")
    t0 = time.perf_counter()
    amax = B.calib_absmax(S.bf16_bits_of(d["X_cal"]))
    B.prepare(d["W"], amax, s.alpha, s.rank, s.fmt)
    t_prep = time.perf_counter() - t0
    log(f"one host preparation {t_prep:.2f} s")
    # scoring forward alone on the calibration rows
    prep = B.prepare(d["W"], amax, s.alpha, s.rank, s.fmt)
    lay = B.DeviceLayer(prep)
    Y = torch.empty((mc, s.N), dtype=torch.int16, device="cuda")
    ws = lay.workspace(mc)
    for _ in range(3):
        B.linear_forward(lay, xc, Y, ws)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        B.linear_forward(lay, xc, Y, ws)
    e1.record()
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / 10
    del lay, ws, Y
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r = B.smooth_search(d["W"], xc, s.rank, s.fmt, grids=g)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"search {wall:.1f} s; winner alpha={r['alpha']} beta={r['beta']} score={r['errors'][r['best']]:.4e}")
    out = {
        "metric": "smooth_search_seconds", "value": wall, "unit": "s", "n_gpus": 1,
        "higher_is_better": False, "dtype": "u4" if s.fmt == "int4" else "fp4", "data": "synthetic",
        "config": {"workload": s.name, "M_cal": int(mc), "K": s.K, "N": s.N, "rank": s.rank, "fmt": s.fmt,
                   "grids": g, "candidates": n},
        "per_candidate_s": wall / n, "host_prepare_s": t_prep, "scoring_forward_ms": fwd_ms,
        "host_threads": int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count(),
        "best": {"alpha": r["alpha"], "beta": r["beta"], "score": float(r["errors"][r["best"]])},
        "scores": [float(e) for e in r["errors"]],
    }
    print(json.dumps(out), flush=True)


def bench_vendor(args, s):
    """Context, not a baseline of this method: the vendor GEMMs reachable
    from torch (hipBLASLt) on the layer's M x K x N with random operands --
    bf16, int8, FP8 E4M3 with one scale per tensor, MXFP4 with E8M0 scales
    per 32 -- next to this library's whole forward (K-A + K-B, low-rank
    branch and bias included) on the layer itself."""
    import torch
    import torch.nn.functional as TF
    import rank_gemm_svdq_amd as B
    from rank_gemm_svdq_amd import synthetic as S

    M, K, N = s.M, s.K, s.N
    ops = main_ops(M, N, K)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / args.steps
        return {"us": us, "TOPS": ops / us / 1e6}

    res = {}
    d = S.make_layer(s)
    lora = {"A": d["lora_A"], "B": d["lora_B"], "strength": 1.0} if s.lora_rank else None
    amax = B.calib_absmax(S.bf16_bits_of(d["X_cal"]))
    prep = B.prepare(d["W"], amax, s.alpha, s.rank, s.fmt, lora=lora)
    lay = B.DeviceLayer(prep, S.bf16_bits_of(d["bias"]))
    X = torch.from_numpy(S.bf16_bits_of(d["X"]).view(np.int16)).cuda()
    Y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = lay.workspace(M)

    def ours(tag):
        res[f"svdq_linear_forward_{tag}"] = timed(lambda: B.linear_forward(lay, X, Y, ws))
        # K-B alone (quantized GEMM + low-rank up projection + bias) on the
        # codes K-A left in the workspace
        B.quantize_lora_down(lay, X, ws)
        res[f"svdq_gemm_lora_up_{tag}"] = timed(lambda: B.gemm_lora_up(lay, ws, M, Y))

    # this library first and last, the vendor GEMMs between (clock drift shows)
    ours("first")
    # K-B once more with uniformly random code bytes in place of both
    # operands' codes (scales kept): the vendor GEMMs below run on random
    # operands too, and random codes keep the matrix units busiest
    wl = B.workspace_layout(M, K, s.rank, s.fmt)
    gr = torch.Generator(device="cuda")
    gr.manual_seed(1)
    wsv = ws.view(torch.uint8) if ws.dtype != torch.uint8 else ws
    xq = wsv[wl["xq_off"]:wl["xq_off"] + wl["xq_bytes"]]
    xq.copy_(torch.randint(0, 256, xq.shape, device="cuda", dtype=torch.uint8, generator=gr))
    wq = lay.wq.view(torch.uint8) if lay.wq.dtype != torch.uint8 else lay.wq
    wq_saved = wq.clone()
    wq.copy_(torch.randint(0, 256, wq.shape, device="cuda", dtype=torch.uint8, generator=gr))
    res["svdq_gemm_lora_up_random_codes"] = timed(lambda: B.gemm_lora_up(lay, ws, M, Y))
    wq.copy_(wq_saved)
    del wq_saved
    g = torch.Generator(device="cuda")
    g.manual_seed(0)
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(N, K, device="cuda", dtype=torch.bfloat16, generator=g)
    res["bf16_matmul"] = timed(lambda: a @ b.t())
    ai = torch.randint(-127, 128, (M, K), device="cuda", dtype=torch.int8, generator=g)
    bi = torch.randint(-127, 128, (N, K), device="cuda", dtype=torch.int8, generator=g)
    res["int8_int_mm"] = timed(lambda: torch._int_mm(ai, bi.t()))
    a8, b8 = a.to(torch.float8_e4m3fn), b.to(torch.float8_e4m3fn)
    one = torch.ones((), device="cuda")
    res["fp8_e4m3_scaled_mm"] = timed(lambda: torch._scaled_mm(a8, b8.t(), one, one, out_dtype=torch.bfloat16))
    af = torch.randint(0, 256, (M, K // 2), device="cuda", dtype=torch.uint8, generator=g).view(torch.float4_e2m1fn_x2)
    bf = torch.randint(0, 256, (N, K // 2), device="cuda", dtype=torch.uint8, generator=g).view(torch.float4_e2m1fn_x2)
    sa = torch.randint(120, 128, (M, K // 32), device="cuda", dtype=torch.uint8, generator=g).view(torch.float8_e8m0fnu)
    sb = torch.randint(120, 128, (N, K // 32), device="cuda", dtype=torch.uint8, generator=g).view(torch.float8_e8m0fnu)
    bw, nsw = TF.ScalingType.BlockWise1x32, TF.SwizzleType.NO_SWIZZLE
    res["mxfp4_scaled_mm"] = timed(lambda: TF.scaled_mm(af, bf.t(), sa, bw, sb, bw, swizzle_a=nsw, swizzle_b=nsw,
                                                        output_dtype=torch.bfloat16))
    del a, b, ai, bi, a8, b8, af, bf, sa, sb

    ours("last")
    out = {
        "metric": "vendor_gemm_context", "unit": "us", "n_gpus": 1, "data": "synthetic",
        "config": {"workload": s.name, "M": M, "K": K, "N": N, "rank": s.rank, "format": s.fmt},
        "ops_per_call": ops, "steps": args.steps, "warmup": args.warmup, "results": res,
    }
    print(json.dumps(out), flush=True)


def profile_commands(d, config):
    return {k: "rocprofv3 " + v.format(dir=d, config=config) for k, v in PROFILE_STEPS.items()}


def _write(path, text):
    with open(path, "w") as fh:
        fh.write(text)


def _csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for f in sorted(files):
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def _matches(name, names):
    return any(n in name for n in names)


def summarize_profiles(d, config, fmt_override=None):
    """Text summaries of a stats run and the FETCH_SIZE / WRITE_SIZE runs
    under d (made by the commands of profile_commands) -> profiles/."""
    sys.path.insert(0, ROOT)
    from rank_gemm_svdq_amd import synthetic as S
    s = S.spec(config, **({"fmt": fmt_override} if fmt_override else {}))
    M, K, N, fmt = s.M, s.K, s.N, s.fmt
    r = s.rank + s.lora_rank
    rp = (r + 31) // 32 * 32 if r else 0
    kb_names = kb_kernel_names(fmt, K, r)
    ka_names = ("ka_kernel",)
    short = {"mxfp4": "kb_mx", "mxfp4_ocp": "kb_mx", "int4": "kb_int4", "w8a8": "kb_w8a8"}[fmt]
    key = s.name if not fmt_override else f"{s.name}_{fmt}"
    cmds = profile_commands(os.path.normpath(d), config + (f" --fmt {fmt_override}" if fmt_override else ""))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)

    # kernel stats
    rows = _csv(_find(os.path.join(d, "stats"), "kernel_stats.csv"))
    col = lambda row, *c: next((row[k] for k in row if any(x.lower() == k.lower() for x in c)), None)
    lines = [f"# Kernel time, {key} (M={M} K={K} N={N} rank={r} {fmt})", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + cmds["stats"], "",
             "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    kb_avg = tail_avg = None
    tail_names = kb_tail_names(fmt, K, r)
    for row in rows:
        name = col(row, "Name", "KernelName")
        calls = int(float(col(row, "Calls")))
        avg = float(col(row, "AverageNs")) / 1e3
        mn, mx = float(col(row, "MinNs")) / 1e3, float(col(row, "MaxNs")) / 1e3
        pct = float(col(row, "Percentage"))
        short_name = name.split("(")[0].replace("void ", "")
        lines.append(f"| {short_name} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.1f} |")
        if _matches(name, kb_names):
            kb_avg = avg
        if tail_names and _matches(name, tail_names):
            tail_avg = avg
    bench_json = os.path.join(d, "stats.json")
    if os.path.exists(bench_json):
        with open(bench_json) as fh:
            b = json.loads(fh.read().strip().splitlines()[-1])
        lines += ["", f"bench.py under the profiler: K-B median {b['kb_us']:.2f} us (HIP events on the launch "
                      f"stream), K-A median {b['ka']['us']:.2f} us, layer {b['value']:.0f} TOPS."]
    if kb_avg is not None and tail_avg is not None:
        ops = main_ops(M, N, K)
        tot = kb_avg + tail_avg
        lines += [f"K-B is two launches here: {kb_names[0]} (256 x 256 tiles, the full rounds) {kb_avg:.2f} us + "
                  f"{tail_names[0]} (128 x 128 tiles, the last columns) {tail_avg:.2f} us = {tot:.2f} us -> "
                  f"{ops / (tot * 1e-6) / 1e12:.0f} TOP/s of 2MNK = {ops:.4g} ops per layer."]
    elif kb_avg is not None:
        ops = main_ops(M, N, K)
        lines += [f"{kb_names[0]}: average {kb_avg:.2f} us -> {ops / (kb_avg * 1e-6) / 1e12:.0f} TOP/s of "
                  f"2MNK = {ops:.4g} ops per launch."]
    kb_layer_avg = None if kb_avg is None else kb_avg + (tail_avg or 0.0)
    _write(os.path.join(ROOT, "profiles", f"{short}_{key}_kernel_stats.md"), "\n".join(lines) + "\n")

    # HBM traffic: FETCH_SIZE / WRITE_SIZE (KiB per dispatch), scaled by a
    # 256 MiB device copy measured in the same run
    out = {}
    for which in ("fetch", "write"):
        cc = _csv(_find(os.path.join(d, which), "counter_collection.csv"))
        cname = "FETCH_SIZE" if which == "fetch" else "WRITE_SIZE"
        per = {}
        for row in cc:
            if row["Counter_Name"] != cname:
                continue
            per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]) * 1024.0)
        copy = [v for n, vs in per.items() if "copyBuffer" in n or "copy" in n.lower() for v in vs]
        big = max(copy) if copy else None           # the 256 MiB calibration copy
        factor = CALIB_BYTES / big if big else None
        kb = [v for n, vs in per.items() if _matches(n, kb_names) for v in vs]
        kt = [v for n, vs in per.items() if tail_names and _matches(n, tail_names) for v in vs]
        ka = [v for n, vs in per.items() if _matches(n, ka_names) for v in vs]
        # per layer: the main launch plus, when there is one, the tail launch
        out[which] = {"copy_counter_bytes": big, "factor": factor,
                      "kb_counter_bytes": (float(np.mean(kb)) + (float(np.mean(kt)) if kt else 0.0)) if kb else None,
                      "ka_counter_bytes": float(np.mean(ka)) if ka else None,
                      "kb_dispatches": len(kb), "kb_tail_dispatches": len(kt), "ka_dispatches": len(ka)}
    f_, w_ = out["fetch"], out["write"]
    kb_alg = kb_bytes(M, N, K, r, fmt)
    ka_alg = ka_bytes(M, K, r, fmt)
    kb_traffic = ka_traffic = None
    if f_["kb_counter_bytes"] and w_["kb_counter_bytes"] and f_["factor"] and w_["factor"]:
        kb_traffic = f_["kb_counter_bytes"] * f_["factor"] + w_["kb_counter_bytes"] * w_["factor"]
    if f_["ka_counter_bytes"] and w_["ka_counter_bytes"] and f_["factor"] and w_["factor"]:
        ka_traffic = f_["ka_counter_bytes"] * f_["factor"] + w_["ka_counter_bytes"] * w_["factor"]
    fmtb = lambda v: "n/a" if v is None else f"{v / 1e6:.2f} MB"
    lines = [f"# HBM traffic per launch, {key} (M={M} K={K} N={N} rank={r} {fmt})", "",
             "Commands (from the repository root, TMPDIR=/tmp):", "", "    " + cmds["fetch"], "    " + cmds["write"], "",
             "Counters are KiB per dispatch; each is scaled by (256 MiB / the same counter on the 256 MiB "
             "device copy of the same run).", "",
             "| | FETCH_SIZE | WRITE_SIZE |", "|---|---|---|",
             f"| calibration copy, counter | {fmtb(f_['copy_counter_bytes'])} | {fmtb(w_['copy_counter_bytes'])} |",
             f"| scale factor | {f_['factor'] or float('nan'):.4f} | {w_['factor'] or float('nan'):.4f} |",
             f"| {kb_names[0]}{' + ' + tail_names[0] if f_['kb_tail_dispatches'] else ''}, counter (mean of "
             f"{f_['kb_dispatches']}{' + ' + str(f_['kb_tail_dispatches']) if f_['kb_tail_dispatches'] else ''}) | "
             f"{fmtb(f_['kb_counter_bytes'])} | {fmtb(w_['kb_counter_bytes'])} |",
             f"| ka_kernel, counter (mean of {f_['ka_dispatches']}) | {fmtb(f_['ka_counter_bytes'])} | "
             f"{fmtb(w_['ka_counter_bytes'])} |", "",
             f"K-B scaled traffic {fmtb(kb_traffic)} against {fmtb(kb_alg)} algorithmic "
             f"({'n/a' if kb_traffic is None else f'{kb_traffic / kb_alg:.2f}x'}).",
             f"K-A scaled traffic {fmtb(ka_traffic)} against {fmtb(ka_alg)} algorithmic "
             f"({'n/a' if ka_traffic is None else f'{ka_traffic / ka_alg:.2f}x'})."]
    _write(os.path.join(ROOT, "profiles", f"{short}_{key}_traffic.md"), "\n".join(lines) + "\n")
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        t = {}
    t[key] = {"kernel": kb_names[0] + (" + " + tail_names[0] if f_["kb_tail_dispatches"] else ""),
              "kernel_source_sha256_16": kernel_source_hash(),
              "bytes_per_launch": kb_traffic, "ka_bytes_per_launch": ka_traffic,
              "kb_algorithmic_bytes": kb_alg, "ka_algorithmic_bytes": ka_alg,
              "fetch": f_, "write": w_, "commands": [cmds["fetch"], cmds["write"]]}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(t, fh, indent=1, sort_keys=True)
    print("\n".join(lines))
    if os.path.isdir(os.path.join(d, "mfma")):
        summarize_mfma(d, key, M, N, K, r, fmt, kb_names, kb_layer_avg, cmds["mfma"], short, tail_names)
    if os.path.isdir(os.path.join(d, "waves")) and os.path.isdir(os.path.join(d, "l2")):
        ka_avg = next((float(col(row, "AverageNs")) / 1e3 for row in rows
                       if _matches(col(row, "Name", "KernelName"), ka_names)), None)
        kernels = {"K-A (ka_kernel)": (ka_names, ka_avg), f"K-B ({kb_names[0]})": (kb_names, kb_avg)}
        if tail_names and tail_avg is not None:
            kernels[f"K-B, last columns ({tail_names[0]})"] = (tail_names, tail_avg)
        summarize_waves(d, key, M, N, K, r, fmt, kernels, (cmds["waves"], cmds["l2"]))


def summarize_mfma(d, key, M, N, K, r, fmt, kb_names, kb_avg, cmd, short, tail_names=None):
    """MFMA utilisation of K-B from counters: SQ_VALU_MFMA_BUSY_CYCLES (summed
    over the SIMDs) per SIMD against SQ_BUSY_CYCLES (summed over the shader
    engines) per engine, i.e. the share of busy cycles in which a SIMD's
    matrix pipe is busy; the engine cycles over the kernel-trace duration
    give the clock the kernel ran at."""
    cc = _csv(_find(os.path.join(d, "mfma"), "counter_collection.csv"))
    agent = [a for a in _csv(_find(os.path.join(d, "mfma"), "agent_info.csv")) if int(a.get("Simd_Count", 0) or 0) > 0]
    simds = int(agent[0]["Simd_Count"])
    engines = int(agent[0]["Num_Shader_Banks"])
    vals, tvals = {}, {}
    for row in cc:
        if _matches(row["Kernel_Name"], kb_names):
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
        elif tail_names and _matches(row["Kernel_Name"], tail_names):
            tvals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    # per layer: the main launch plus the tail launch when there is one
    mean = {k: float(np.mean(v)) + (float(np.mean(tvals[k])) if k in tvals else 0.0) for k, v in vals.items()}
    busy_simd = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simds
    busy_se = mean["SQ_BUSY_CYCLES"] / engines
    ops = main_ops(M, N, K)
    ideal = ops / simds / (PEAK[fmt] / simds / 2.4e9)   # MFMA cycles per SIMD at the dense peak rate
    lines = [f"# MFMA utilisation of K-B, {key} (M={M} K={K} N={N} rank={r} {fmt})", "",
             "Command (from the repository root, TMPDIR=/tmp):", "", "    " + cmd, "",
             f"Agent: {simds} SIMDs, {engines} shader engines. Means over {len(vals.get('SQ_BUSY_CYCLES', []))} "
             f"dispatches of {kb_names[0]}" +
             (f", plus those of {tail_names[0]} (the last columns; {len(tvals.get('SQ_BUSY_CYCLES', []))} "
              "dispatches), summed per layer." if tvals else "."), "",
             "| counter | per dispatch | per SIMD or engine |", "|---|---|---|",
             f"| SQ_VALU_MFMA_BUSY_CYCLES | {mean['SQ_VALU_MFMA_BUSY_CYCLES']:.4g} | {busy_simd:.0f} per SIMD |",
             f"| SQ_BUSY_CYCLES | {mean['SQ_BUSY_CYCLES']:.4g} | {busy_se:.0f} per engine |",
             f"| GRBM_GUI_ACTIVE | {mean['GRBM_GUI_ACTIVE']:.4g} | |",
             f"| SQ_WAVES | {mean['SQ_WAVES']:.4g} | |", "",
             f"MFMA busy / engine busy = {busy_simd / busy_se:.3f} (share of the kernel's busy cycles in which a "
             f"SIMD's matrix pipe works).",
             f"2MNK at the dense {PEAK_NAME[fmt]} rate needs {ideal:.0f} MFMA cycles per SIMD "
             f"(counter: {busy_simd:.0f}, ratio {busy_simd / ideal:.3f})."]
    if kb_avg:
        xcc = int(agent[0].get("Num_Xcc", 0) or 0)
        lines.append(f"Engine busy cycles over the kernel-trace average ({kb_avg:.2f} us): "
                     f"{busy_se / (kb_avg * 1e3):.2f} GHz" +
                     (f"; GRBM_GUI_ACTIVE per XCD ({xcc}) over the same: "
                      f"{mean['GRBM_GUI_ACTIVE'] / xcc / (kb_avg * 1e3):.2f} GHz." if xcc else "."))
    _write(os.path.join(ROOT, "profiles", f"{short}_{key}_mfma.md"), "\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_waves(d, key, M, N, K, r, fmt, kernels, cmds):
    """Residency, waiting and cache behaviour of K-A and K-B from counters.
    SQ_WAVE_CYCLES and SQ_WAIT_* count wave-cycles in the same unit, so their
    ratio is the share of a resident wave's life spent waiting (on anything,
    or on an s_waitcnt); SQ_WAVE_CYCLES over the engines' busy cycles and the
    CU count gives the mean number of resident waves per CU in that unit
    (one wave-cycle is counted per 4 clocks on this agent when the figure
    comes out a quarter of the launch's known waves per CU). TCC_HIT /
    (TCC_HIT + TCC_MISS) is the L2 hit rate of the kernel's requests."""
    agent = [a for a in _csv(_find(os.path.join(d, "waves"), "agent_info.csv")) if int(a.get("Simd_Count", 0) or 0) > 0]
    engines = int(agent[0]["Num_Shader_Banks"])
    cus = int(agent[0].get("Cu_Count", 0) or 0) or 256
    lines = [f"# Residency, waits and L2 hits of K-A and K-B, {key} (M={M} K={K} N={N} rank={r} {fmt})", "",
             "Commands (from the repository root, TMPDIR=/tmp):", "", "    " + cmds[0], "    " + cmds[1], ""]
    for label, (names, avg) in kernels.items():
        vals = {}
        grid = wg = None
        for which in ("waves", "l2"):
            for row in _csv(_find(os.path.join(d, which), "counter_collection.csv")):
                if _matches(row["Kernel_Name"], names):
                    vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    grid, wg = int(row["Grid_Size"]), int(row["Workgroup_Size"])
        if not vals:
            continue
        m = {k: float(np.mean(v)) for k, v in vals.items()}
        busy_se = m["SQ_BUSY_CYCLES"] / engines
        waves_per_cu = m["SQ_WAVE_CYCLES"] / busy_se / cus
        hit = m["TCC_HIT_sum"] / max(1.0, m["TCC_HIT_sum"] + m["TCC_MISS_sum"])
        lines += [f"## {label}", "",
                  f"Launch: {grid // wg} workgroups of {wg // 64} waves ({grid // 64} waves, "
                  f"{grid // 64 / cus:.2f} per CU). Means over {len(vals['SQ_WAVES'])} dispatches.", "",
                  "| counter | per dispatch |", "|---|---|"]
        lines += [f"| {k} | {v:.4g} |" for k, v in sorted(m.items())]
        lines += ["",
                  f"- waiting (any) / wave-cycles: {m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.3f}",
                  f"- waiting on s_waitcnt / wave-cycles: {m['SQ_WAIT_INST_ANY'] / m['SQ_WAVE_CYCLES']:.3f}",
                  f"- wave-cycles per CU per engine-busy cycle: {waves_per_cu:.2f}",
                  f"- LDS bank-conflict cycles / LDS-active cycles: "
                  f"{m['SQ_LDS_BANK_CONFLICT'] / max(1.0, m['SQ_LDS_IDX_ACTIVE']):.3f}",
                  f"- L2 hit rate: {hit:.3f}; L2-to-memory read requests: {m['TCC_EA0_RDREQ_sum']:.4g}"]
        if avg:
            lines.append(f"- engine-busy clock over the kernel-trace average ({avg:.2f} us): "
                         f"{busy_se / (avg * 1e3):.2f} GHz")
        lines.append("")
    _write(os.path.join(ROOT, "profiles", f"ka_kb_{key}_waves.md"), "\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
