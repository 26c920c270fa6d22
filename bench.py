"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = one pass of the hot path over one batch of tokens:
  1x128 activation quantization of X bf16 [4096][7168] (0.1% outlier
  channels x100) -> block-scaled FP8 GEMM with W [7168][7168] (quantized
  128x128 once, before timing, as weights are) -> BF16 C [4096][7168].
The metric is the step's FP8 GEMM throughput in TFLOP/s (2*M*N*K algorithmic
flops per step over the measured step time, quantization included).

Printed as one JSON line, with:
  * roofline: the dominant kernel (the GEMM), its algorithmic flops over its
    average duration measured with HIP events on its stream inside the timed
    region, against the dense FP8 MFMA peak; traffic = HBM bytes per launch
    from committed rocprofv3 FETCH_SIZE / WRITE_SIZE counters, scaled by the
    copy-kernel calibration, or null if the kernel source changed since;
  * parts: each kernel on its own workload with the caches flushed before
    every launch (act quantizer GB/s vs HBM, beside a plain device copy of
    the same byte count, each also back to back over rotating buffers that
    exceed the caches; dense / decode / grouped GEMM TFLOP/s vs MFMA and
    GB/s vs HBM), the power-of-two-scale variants (quantizer, dense and
    grouped GEMM on the block-scaled MFMA) on the same workloads, and the
    backward pass of the same linear layer (the 128x1 transposed quantizer
    on dY and X, the weight transpose, Dgrad on the transposed weights,
    Wgrad over the 4096 tokens);
  * cpu_baseline: the CPU oracle timed on this host on a bounded sample of
    the same step (first 512 tokens, ~11 s of CPU work).

Usage: python bench.py [--gpus 1] [--steps 500] [--warmup 300]
       [--no-parts] [--no-cpu-baseline] [--copy-calib]
The default warmup (~70 ms of steps) lets the GPU reach its sustained clock
before timing; with a few warmup steps the timed region starts while the
clock is still ramping up after input generation, and reads ~20% slow.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_dense_gemm.json")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_token_amd", "csrc", "gemm.hip")

M, N, K = 4096, 7168, 7168
CPU_SAMPLE_ROWS = 512  # ~11 s of oracle work on 16 host threads


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def dense_gemm_bytes(m, n, k, out_bytes=2):
    return m * k + n * k + m * n * out_bytes + 4 * m * (k // 128) + 4 * (n // 128) * (k // 128)


def quant_bytes(m, k):
    return 2 * m * k + m * k + 4 * m * ((k + 127) // 128)


def traffic_from_counters():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when it is missing or was taken on a different gemm.hip."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("gemm_source_sha256") != source_hash(GEMM_SOURCE):
        return None
    return c.get("hbm_bytes_per_launch")


class Timer:
    """HIP events around launches on the current (torch) stream."""

    def __init__(self, torch, n):
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        self.i = 0

    def start(self):
        self.ev[self.i][0].record()

    def stop(self):
        self.ev[self.i][1].record()
        self.i += 1

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.ev[: self.i]) / max(self.i, 1)

    def median_ms(self):
        v = sorted(a.elapsed_time(b) for a, b in self.ev[: self.i])
        return v[len(v) // 2] if v else 0.0


def to_dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def measure_parts(torch, F, I, X, Wb, qa, sa, qw, sw, C, iters=20):
    """Each kernel on its own workload.  Before every launch a 512 MB buffer
    is read (twice the 256 MB Infinity Cache), so operands come from HBM; a
    read leaves no dirty lines whose write-back would land in the timed
    launch."""
    import numpy as np
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    parts = {}

    spread_us = {}  # p10 / p90 of the last measurement, in µs

    def set_spread(v_ms):
        v = sorted(v_ms)
        spread_us["p10_us"] = v[int(0.1 * (len(v) - 1))] * 1e3
        spread_us["p90_us"] = v[int(0.9 * (len(v) - 1) + 0.5)] * 1e3

    def spread():
        return dict(spread_us)

    def timed(fn, n):
        t = Timer(torch, n)
        for _ in range(n):
            flush.sum()
            t.start()
            fn()
            t.stop()
        torch.cuda.synchronize()
        set_spread([a.elapsed_time(b) for a, b in t.ev[: t.i]])
        return t.median_ms()

    # activation quantizer, 4096 x 7168
    ms = timed(lambda: F.fp8_quant_act_1x128(X, qa, sa), iters)
    b = quant_bytes(M, K)
    parts["act_quant_4096x7168"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS,
        "bytes": b}

    # context: a plain device copy moving the quantizer's byte count
    # (44.5 MB read + 44.5 MB written), timed the same way
    src = torch.empty(quant_bytes(M, K) // 2, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src), iters)
    parts["copy_reference_same_bytes"] = {
        "us": ms * 1e3, **spread(), "GB/s": 2 * src.numel() / ms / 1e6,
        "frac_hbm": 2 * src.numel() / ms / 1e6 / PEAK_HBM_GBS}
    del src, dst

    # The same quantizer and copy back to back, as a model's layers call
    # them: one event pair around 6 x 8 launches that rotate over six
    # input/output sets (534 MB, twice the Infinity Cache), so every launch
    # still reads its input from HBM, while the launch latency that a
    # single timed launch includes overlaps the previous kernel.
    def back_to_back(fns, rounds=8, reps=5):
        per_rep = []
        for _ in range(reps):
            flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(rounds):
                for fn in fns:
                    fn()
            b.record()
            torch.cuda.synchronize()
            per_rep.append(a.elapsed_time(b) / (rounds * len(fns)))
        set_spread(per_rep)
        return min(per_rep)

    sets = [(X.clone(), torch.empty_like(qa), torch.empty_like(sa)) for _ in range(6)]
    ms = back_to_back([lambda s=s: F.fp8_quant_act_1x128(s[0], s[1], s[2]) for s in sets])
    b = quant_bytes(M, K)
    parts["act_quant_4096x7168_back_to_back"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS,
        "launches": "6 sets x 8 rounds, best of 5"}
    del sets
    pairs = [(torch.empty(b // 2, dtype=torch.uint8, device="cuda"),
              torch.empty(b // 2, dtype=torch.uint8, device="cuda")) for _ in range(6)]
    ms = back_to_back([lambda p=p: p[1].copy_(p[0]) for p in pairs])
    parts["copy_reference_same_bytes_back_to_back"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    del pairs

    # dense GEMM alone, 4096 x 7168 x 7168
    ms = timed(lambda: F.fp8_block_gemm(qa, sa, qw, sw, out_dtype="bf16", c=C), iters)
    fl = 2 * M * N * K
    parts["dense_gemm_4096x7168x7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS}

    # power-of-two scales: quantizer and dense GEMM on the same workload
    pa, psa = F.fp8_quant_act_1x128_pow2(X)
    pw, psw = F.fp8_quant_weight_128x128_pow2(Wb)
    ms = timed(lambda: F.fp8_quant_act_1x128_pow2(X, pa, psa), iters)
    b = quant_bytes(M, K)
    parts["pow2_act_quant_4096x7168"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    ms = timed(lambda: F.fp8_block_gemm_pow2(pa, psa, pw, psw, out_dtype="bf16", c=C), iters)
    parts["pow2_dense_gemm_4096x7168x7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS}
    del pa, psa, pw, psw

    # backward of the same layer: dY [4096][7168] (same distribution as X
    # without outliers); Dgrad = forward GEMM with the transposed weights,
    # Wgrad = dY^T X from 128x1 tiles
    dy = to_dev_bf16(torch, I.activations(np.random.default_rng(7), M, N, 0.0, 1.0)[0])
    ms = timed(lambda: F.fp8_quant_act_128x1_t(dy), iters)
    b = quant_bytes(M, N)
    parts["bwd_quant_128x1_t_4096x7168"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    qdy, sdy = F.fp8_quant_act_1x128(dy)
    qwt, swt = F.fp8_transpose_weight_128x128(qw, sw)
    # the weight transpose Dgrad reads, once per weight update
    ms = timed(lambda: F.fp8_transpose_weight_128x128(qw, sw, qwt, swt), iters)
    b = 2 * N * K + 2 * 4 * (N // 128) * (K // 128)
    parts["bwd_transpose_weight_7168x7168"] = {
        "us": ms * 1e3, **spread(), "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    ms = timed(lambda: F.fp8_block_gemm(qdy, sdy, qwt, swt, out_dtype="bf16", c=dx), iters)
    parts["bwd_dgrad_4096x7168x7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS}
    qdy_t, sdy_t = F.fp8_quant_act_128x1_t(dy)
    qx_t, sx_t = F.fp8_quant_act_128x1_t(X)
    dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    ms = timed(lambda: F.fp8_block_gemm_wgrad(qdy_t, sdy_t, qx_t, sx_t, out_dtype="f32", dw=dw),
               iters)
    parts["bwd_wgrad_7168x7168_over_4096"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS}
    del dy, qdy, sdy, qwt, swt, dx, qdy_t, sdy_t, qx_t, sx_t, dw

    # decode GEMM, 256 x 2048 x 7168 (split-K with workspace)
    gd = I.config_decode(seed=0)
    xa = to_dev_bf16(torch, gd.a_bf16)
    xw = to_dev_bf16(torch, gd.w_bf16)
    da, dsa = F.fp8_quant_act_1x128(xa)
    dw, dsw = F.fp8_quant_weight_128x128(xw)
    nbytes = F.fp8_gemm_workspace_bytes(256, 2048, 7168, "bf16")
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda") if nbytes else None
    dc = torch.empty((256, 2048), dtype=torch.bfloat16, device="cuda")
    ms = timed(lambda: F.fp8_block_gemm(da, dsa, dw, dsw, out_dtype="bf16", c=dc, workspace=ws),
               iters)
    fl = 2 * 256 * 2048 * 7168
    b = dense_gemm_bytes(256, 2048, 7168)
    parts["decode_gemm_256x2048x7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS,
        "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS,
        "split_k_workspace_bytes": nbytes}
    # back to back, as a decode step calls one layer after another: 40
    # operand sets (16.5 MB of operands each, 700 MB in all) in rotation
    sets = [(da.clone(), dsa.clone(), dw.clone(), dsw.clone(), torch.empty_like(dc))
            for _ in range(40)]
    ms = back_to_back([lambda s=s: F.fp8_block_gemm(s[0], s[1], s[2], s[3], out_dtype="bf16",
                                                    c=s[4], workspace=ws) for s in sets],
                      rounds=2)
    parts["decode_gemm_256x2048x7168_back_to_back"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS,
        "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS,
        "launches": "40 sets x 2 rounds, best of 5"}
    del sets
    del xa, xw, da, dsa, dw, dsw, ws, dc

    # grouped MoE GEMM, 32 experts / 8192 tokens, N=4096, K=7168
    log("bench: generating the grouped workload ...")
    gi = I.config_grouped(seed=0)
    ga = to_dev_bf16(torch, gi.a_bf16)
    gq, gsa = F.fp8_quant_act_1x128(ga)
    del ga
    gwb = to_dev_bf16(torch, gi.w_bf16.reshape(gi.E * gi.N, gi.K))
    gw, gsw = F.fp8_quant_weight_128x128(gwb)
    del gwb
    gw = gw.view(gi.E, gi.N, gi.K)
    gsw = gsw.view(gi.E, gi.N // 128, gi.K // 128)
    off = torch.from_numpy(gi.offsets).cuda()
    gc = torch.empty((gi.T, gi.N), dtype=torch.bfloat16, device="cuda")
    ms = timed(lambda: F.fp8_block_grouped_gemm(gq, gsa, gw, gsw, off, out_dtype="bf16", c=gc),
               iters)
    fl = 2 * int(gi.counts.sum()) * gi.N * gi.K
    b = (gi.T * gi.K + gi.E * gi.N * gi.K + gi.T * gi.N * 2 + 4 * gi.T * (gi.K // 128)
         + 4 * gi.E * (gi.N // 128) * (gi.K // 128))
    parts["grouped_gemm_e32_t8192_n4096_k7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS,
        "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS,
        "counts": [int(c) for c in gi.counts]}
    del gq, gsa, gw, gsw

    # the same grouped workload with power-of-two scales
    ga = to_dev_bf16(torch, gi.a_bf16)
    gq, gsa = F.fp8_quant_act_1x128_pow2(ga)
    del ga
    gwb = to_dev_bf16(torch, gi.w_bf16.reshape(gi.E * gi.N, gi.K))
    gw, gsw = F.fp8_quant_weight_128x128_pow2(gwb)
    del gwb
    gw = gw.view(gi.E, gi.N, gi.K)
    gsw = gsw.view(gi.E, gi.N // 128, gi.K // 128)
    ms = timed(lambda: F.fp8_block_grouped_gemm_pow2(gq, gsa, gw, gsw, off, out_dtype="bf16",
                                                     c=gc), iters)
    parts["pow2_grouped_gemm_e32_t8192_n4096_k7168"] = {
        "us": ms * 1e3, **spread(), "TFLOP/s": fl / ms / 1e9, "frac_mfma": fl / ms / 1e9 / PEAK_FP8_TFLOPS,
        "GB/s": b / ms / 1e6, "frac_hbm": b / ms / 1e6 / PEAK_HBM_GBS}
    del gq, gsa, gw, gsw, gc, flush
    torch.cuda.empty_cache()
    return parts


def copy_calibration(torch, nbytes=1 << 30, iters=5):
    """A plain device copy of known size, for scaling rocprofv3 counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_each_way": nbytes, "iters": iters}


def cpu_baseline(I, X_bits, w_bits):
    """The oracle on the first CPU_SAMPLE_ROWS tokens of the same step."""
    import numpy as np
    import oracle
    x = np.ascontiguousarray(X_bits[:CPU_SAMPLE_ROWS])
    qw, sw = oracle.quant_weight_128x128(w_bits)      # offline weights, not timed
    t0 = time.perf_counter()
    qa, sa = oracle.quant_act_1x128(x)
    oracle.block_gemm(qa, sa, qw, sw)
    dt = time.perf_counter() - t0
    flops = 2 * CPU_SAMPLE_ROWS * N * K
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
            "kind": "oracle", "seconds": dt,
            "sample": f"first {CPU_SAMPLE_ROWS} of {M} tokens: 1x128 quantization of "
                      f"{CPU_SAMPLE_ROWS}x{K} + binary64 block-scaled GEMM "
                      f"{CPU_SAMPLE_ROWS}x{N}x{K}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the hot path is data-parallel and this "
              "build runs it on a single MI355X (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import fp8_fine_grained_token_amd as F
    from fp8_fine_grained_token_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    F.lib()

    log("bench: generating inputs ...")
    X_bits, _ = I.config_quant(seed=0)                       # 4096 x 7168, outliers
    w_bits = I.config_dense(seed=0).w_bf16                   # 7168 x 7168, N(0, 0.02)
    X = to_dev_bf16(torch, X_bits)
    Wb = to_dev_bf16(torch, w_bits)
    qw, sw = F.fp8_quant_weight_128x128(Wb)                  # offline: once, untimed
    qa = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sa = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    gemm_t = Timer(torch, args.steps)

    # Only the GEMM (the roofline kernel) is bracketed by events inside the
    # timed steps: every event record is a command between two kernels.  The
    # quantizer's own time is measured in `parts`.
    def step(timed):
        F.fp8_quant_act_1x128(X, qa, sa)
        if timed:
            gemm_t.start()
        F.fp8_block_gemm(qa, sa, qw, sw, out_dtype="bf16", c=C)
        if timed:
            gemm_t.stop()

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) / args.steps * 1e3
    flops = 2 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = gemm_t.mean_ms()
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(0)
    result = {
        "metric": "FP8 block-scaled GEMM TFLOP/s + % FP8 MFMA peak; act-quant GB/s % HBM",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": "prefill linear: 1x128 act-quant of 4096x7168 bf16 (0.1% outlier "
                               "channels x100) + fp8_block_gemm M=4096 N=7168 K=7168 bf16 out",
                   "M": M, "N": N, "K": K, "weights": "128x128-quantized once before timing",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "dense_gemm_two_kind_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic_from_counters(),
                     "gemm_us": round(gemm_ms * 1e3, 2)},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "memory_bytes": props.total_memory},
        "inputs_sha256": {"X_bf16_4096x7168": hashlib.sha256(X_bits.tobytes()).hexdigest()[:16],
                          "W_bf16_7168x7168": hashlib.sha256(w_bits.tobytes()).hexdigest()[:16]},
    }
    if args.copy_calib:
        result["copy_calibration"] = copy_calibration(torch)
    if not args.no_parts:
        log("bench: per-kernel parts ...")
        result["parts"] = measure_parts(torch, F, I, X, Wb, qa, sa, qw, sw, C)
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline ...")
        result["cpu_baseline"] = cpu_baseline(I, X_bits, w_bits)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
