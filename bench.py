"""Benchmark of the fine-grained FP8 hot path on one MI355X.

One step = one pass of the hot path over one batch of tokens:
  1x128 activation quantization of X bf16 [4096][7168] (0.1% outlier
  channels x100) -> block-scaled FP8 GEMM with W [7168][7168] (quantized
  128x128 once, before timing, as weights are) -> BF16 C [4096][7168].
The metric is the step's FP8 GEMM throughput in TFLOP/s (2*M*N*K algorithmic
flops per step over the measured step time, quantization included).

Order of the run: inputs; the CPU oracle baseline (host only); the
per-kernel parts (each kernel on its own workload); a fixed untimed pre-roll
of steps (PREROLL_S seconds, so the timed region starts at the clock the GPU
sustains on this work); the W warm-up steps; the K timed steps.

Printed as one JSON line, with:
  * roofline: the dominant kernel (the GEMM), its algorithmic flops over its
    average duration measured with HIP events on its stream inside the timed
    region, against the dense FP8 MFMA peak; the shader clock over the
    timed steps, from each compute unit's shader-clock and 100 MHz real-time
    counters read on the GPU just before and just after them (the SMU's
    reported GFX clock, sampled through amdsmi, beside it), and the fraction
    against the peak at that clock; the same kernel's flushed per-part
    fraction;
    traffic = HBM bytes per launch from committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE counters, scaled by the copy-kernel calibration, or null if
    the kernel source changed since;
  * parts: each kernel on its own workload, 5 untimed launches then at least
    50 timed ones, with a 512 MB read before every timed launch so operands
    come from HBM (median, p10, p90); the act quantizer and a plain device
    copy also back to back over rotating buffers that exceed the caches;
    the tiny GEMM as launch latency; dense / decode / grouped GEMMs (TFLOP/s
    vs MFMA, GB/s vs HBM); the power-of-two-scale variants; the fused
    quantize-and-multiply GEMM; the backward pass of the same linear layer;
  * cpu_baseline: the CPU oracle timed on this host: the step on a bounded
    sample (first 512 tokens), and per workload (quantizer GB/s single- and
    multi-threaded, tiny GEMM in full, dense on a sample, decode in full,
    grouped on a per-expert stratified eighth of the rows).

Usage: python bench.py [--gpus 1] [--steps 500] [--warmup 300]
       [--no-parts] [--no-cpu-baseline] [--copy-calib] [--part NAME]
       [--preroll SECONDS]
--part NAME runs only that part (for kernel traces of one kernel) and prints
its JSON.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA
MAX_SCLK_MHZ = 2400.0      # the clock that peak is quoted at
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_dense_gemm.json")
GEMM_SOURCE = os.path.join(ROOT, "fp8_fine_grained_token_amd", "csrc", "gemm.hip")

M, N, K = 4096, 7168, 7168
CPU_SAMPLE_ROWS = 512   # ~11 s of oracle work on 16 host threads
PART_WARMUP = 5
PART_ITERS = 50
PREROLL_S = 0.4         # untimed steps before the warm-up steps


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_hash(path):
    """sha256 of a C/C++/HIP source with its comments removed and its blank
    space collapsed: it changes when the code changes, not when only its
    comments do."""
    import re
    with open(path, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def dense_gemm_bytes(m, n, k, out_bytes=2):
    return m * k + n * k + m * n * out_bytes + 4 * m * (k // 128) + 4 * (n // 128) * (k // 128)


def quant_bytes(m, k):
    return 2 * m * k + m * k + 4 * m * ((k + 127) // 128)


def traffic_from_counters():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when it is missing or was taken on different gemm.hip code."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("gemm_code_sha256") != code_hash(GEMM_SOURCE):
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

    def times_ms(self):
        return [a.elapsed_time(b) for a, b in self.ev[: self.i]]

    def mean_ms(self):
        v = self.times_ms()
        return sum(v) / max(len(v), 1)


class ClockSampler:
    """Shader (GFX) clock of GPU 0 sampled every few ms from the SMU through
    amdsmi while running; reports mean / min / max in MHz."""

    def __init__(self):
        self.samples, self.error, self.max_mhz = [], None, None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            info = amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX)
            self.max_mhz = info.get("max_clk")
        except Exception as e:  # noqa: BLE001 - reported in the JSON
            self._amdsmi = None
            self.error = f"{type(e).__name__}: {e}"

    def _run(self):
        while not self._stop.is_set():
            try:
                info = self._amdsmi.amdsmi_get_clock_info(self._h, self._amdsmi.AmdSmiClkType.GFX)
                self.samples.append(float(info["clk"]))
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(0.002)

    def start(self):
        if self._amdsmi is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        if not self.samples:
            return {"mhz_mean": None, "error": self.error or "no samples"}
        s = self.samples
        return {"mhz_mean": round(sum(s) / len(s), 1), "mhz_min": min(s), "mhz_max": max(s),
                "samples": len(s), "max_sclk_mhz": self.max_mhz, "source": "amdsmi GFX clock"}


class GpuClockProbe:
    """Mean shader clock of each compute unit between two probe launches on
    the current stream, from its shader-clock counter (s_memtime) against the
    100 MHz real-time counter (s_memrealtime), both read on the GPU by
    _build/libfp8probe.so (the benchmark's probe, not the library).  The
    units' shader-clock counters are not aligned with each other, so the two
    launches are matched unit by unit; the result gives each XCD's median
    over its units and the mean over all units."""

    WORKGROUPS = 4096  # 16 per compute unit, so every unit is seen in both launches

    def __init__(self, torch):
        import ctypes
        from fp8_fine_grained_token_amd import build as hip_build
        self.torch = torch
        self.error = None
        self.bufs = [torch.zeros(3 * self.WORKGROUPS, dtype=torch.int64, device="cuda")
                     for _ in range(2)]
        try:
            self.lib = ctypes.CDLL(hip_build.PROBE_LIB_PATH)
            self.lib.fp8probe_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
            self.lib.fp8probe_clock.restype = ctypes.c_int
        except OSError as e:
            self.lib, self.error = None, f"OSError: {e}"

    def mark(self, i):
        if self.lib is None:
            return
        stream = self.torch.cuda.current_stream().cuda_stream
        rc = self.lib.fp8probe_clock(self.bufs[i].data_ptr(), self.WORKGROUPS, stream)
        if rc != 0:
            self.error = f"probe launch status {rc}"

    def result(self):
        """Call after a synchronization that follows mark(1)."""
        if self.lib is None or self.error:
            return {"mhz_mean": None, "error": self.error}
        import numpy as np
        per = []
        for i in range(2):
            v = self.bufs[i].cpu().numpy().reshape(-1, 3)
            d = {}
            for unit, t, r in v:   # each unit's earliest workgroup in the launch
                u = int(unit)
                if u not in d or int(r) < d[u][1]:
                    d[u] = (int(t), int(r))
            per.append(d)
        mhz = {}
        for u in sorted(set(per[0]) & set(per[1])):
            dt = per[1][u][0] - per[0][u][0]
            dr = per[1][u][1] - per[0][u][1]
            if dr > 0 and dt > 0:
                mhz[u] = dt / dr * 100.0
        if not mhz:
            return {"mhz_mean": None, "error": "no compute unit seen in both probe launches"}
        vals = np.array(list(mhz.values()))
        xcds = sorted({u >> 8 for u in mhz})
        per_xcd = [round(float(np.median([m for u, m in mhz.items() if u >> 8 == x])), 1)
                   for x in xcds]
        return {"mhz_mean": round(float(vals.mean()), 1),
                "mhz_p10": round(float(np.percentile(vals, 10)), 1),
                "mhz_p90": round(float(np.percentile(vals, 90)), 1),
                "per_xcd_median_mhz": per_xcd, "compute_units_matched": int(vals.size),
                "source": "s_memtime over s_memrealtime (100 MHz) per compute unit, read by "
                          "probe launches just before and just after the timed steps"}


_GROUPED = []


def grouped_workload(I):
    """The grouped workload's inputs, generated once per run."""
    if not _GROUPED:
        log("bench: generating the grouped workload ...")
        _GROUPED.append(I.config_grouped(seed=0))
    return _GROUPED[0]


def to_dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class Parts:
    """Per-kernel timings.  Before every timed launch a 512 MB buffer is read
    (twice the 256 MB Infinity Cache), so operands come from HBM; a read
    leaves no dirty lines whose write-back would land in the timed launch."""

    def __init__(self, torch, iters=PART_ITERS):
        self.torch = torch
        self.iters = iters
        self.flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        self.out = {}

    @staticmethod
    def _spread(v_ms):
        v = sorted(v_ms)
        return {"p10_us": v[int(0.1 * (len(v) - 1))] * 1e3,
                "p90_us": v[int(0.9 * (len(v) - 1) + 0.5)] * 1e3}

    def timed(self, fn, n=None):
        """Median ms of n flushed launches after PART_WARMUP untimed ones."""
        torch = self.torch
        n = n or self.iters
        for _ in range(PART_WARMUP):
            fn()
        t = Timer(torch, n)
        for _ in range(n):
            self.flush.sum()
            t.start()
            fn()
            t.stop()
        torch.cuda.synchronize()
        v = sorted(t.times_ms())
        return v[len(v) // 2], self._spread(v)

    def back_to_back(self, fns, rounds=8, reps=10):
        """Best per-launch ms over reps of (rounds x len(fns)) launches
        bracketed by one event pair; fns rotate over buffers that exceed the
        caches, so every launch still reads HBM."""
        torch = self.torch
        for fn in fns[:PART_WARMUP]:
            fn()
        per_rep = []
        for _ in range(reps):
            self.flush.sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(rounds):
                for fn in fns:
                    fn()
            b.record()
            torch.cuda.synchronize()
            per_rep.append(a.elapsed_time(b) / (rounds * len(fns)))
        return min(per_rep), self._spread(per_rep)

    def add_bytes(self, name, ms, spread, nbytes, **extra):
        self.out[name] = {"us": ms * 1e3, **spread, "GB/s": nbytes / ms / 1e6,
                          "frac_hbm": nbytes / ms / 1e6 / PEAK_HBM_GBS, "bytes": nbytes, **extra}

    def add_flops(self, name, ms, spread, flops, nbytes=None, **extra):
        d = {"us": ms * 1e3, **spread, "TFLOP/s": flops / ms / 1e9,
             "frac_mfma": flops / ms / 1e9 / PEAK_FP8_TFLOPS}
        if nbytes is not None:
            d.update({"GB/s": nbytes / ms / 1e6, "frac_hbm": nbytes / ms / 1e6 / PEAK_HBM_GBS})
        self.out[name] = {**d, **extra}


def measure_parts(torch, F, I, X, Wb, qa, sa, qw, sw, C, only=None):
    import numpy as np
    P = Parts(torch)
    want = (lambda name: True) if only is None else (lambda name: name == only)

    b = quant_bytes(M, K)
    if want("act_quant_4096x7168"):
        P.add_bytes("act_quant_4096x7168", *P.timed(lambda: F.fp8_quant_act_1x128(X, qa, sa)), b)
    if want("copy_reference_same_bytes"):
        # a plain device copy moving the quantizer's byte count
        src = torch.empty(b // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        P.add_bytes("copy_reference_same_bytes", *P.timed(lambda: dst.copy_(src)), 2 * src.numel())
        del src, dst
    if want("act_quant_4096x7168_back_to_back"):
        # back to back as a model's layers call it: six input/output sets
        # (534 MB, twice the Infinity Cache) in rotation
        sets = [(X.clone(), torch.empty_like(qa), torch.empty_like(sa)) for _ in range(6)]
        ms, sp = P.back_to_back([lambda s=s: F.fp8_quant_act_1x128(s[0], s[1], s[2])
                                 for s in sets])
        P.add_bytes("act_quant_4096x7168_back_to_back", ms, sp, b,
                    launches="6 sets x 8 rounds, best of 10")
        del sets
    if want("copy_reference_same_bytes_back_to_back"):
        pairs = [(torch.empty(b // 2, dtype=torch.uint8, device="cuda"),
                  torch.empty(b // 2, dtype=torch.uint8, device="cuda")) for _ in range(6)]
        ms, sp = P.back_to_back([lambda p=p: p[1].copy_(p[0]) for p in pairs])
        P.add_bytes("copy_reference_same_bytes_back_to_back", ms, sp, b)
        del pairs

    fl = 2 * M * N * K
    if want("dense_gemm_4096x7168x7168"):
        P.add_flops("dense_gemm_4096x7168x7168",
                    *P.timed(lambda: F.fp8_block_gemm(qa, sa, qw, sw, out_dtype="bf16", c=C)), fl,
                    dense_gemm_bytes(M, N, K))

    if want("tiny_gemm_128x256x512_f32"):
        g = I.config_tiny(seed=0)
        ta, tsa = F.fp8_quant_act_1x128(to_dev_bf16(torch, g.a_bf16))
        tw, tsw = F.fp8_quant_weight_128x128(to_dev_bf16(torch, g.w_bf16))
        tc = torch.empty((128, 256), dtype=torch.float32, device="cuda")
        ms, sp = P.timed(lambda: F.fp8_block_gemm(ta, tsa, tw, tsw, out_dtype="f32", c=tc))
        tfl = 2 * 128 * 256 * 512
        P.add_flops("tiny_gemm_128x256x512_f32", ms, sp, tfl,
                    note="launch-latency bound: one launch after a cache flush")
        del ta, tsa, tw, tsw, tc

    if want("pow2_act_quant_4096x7168") or want("pow2_dense_gemm_4096x7168x7168"):
        pa, psa = F.fp8_quant_act_1x128_pow2(X)
        pw, psw = F.fp8_quant_weight_128x128_pow2(Wb)
        if want("pow2_act_quant_4096x7168"):
            P.add_bytes("pow2_act_quant_4096x7168",
                        *P.timed(lambda: F.fp8_quant_act_1x128_pow2(X, pa, psa)), b)
        if want("pow2_dense_gemm_4096x7168x7168"):
            P.add_flops("pow2_dense_gemm_4096x7168x7168",
                        *P.timed(lambda: F.fp8_block_gemm_pow2(pa, psa, pw, psw, out_dtype="bf16",
                                                               c=C)), fl)
        del pa, psa, pw, psw

    if want("fused_quant_gemm_4096x7168x7168"):
        # bf16 activations quantized inside the GEMM (no E4M3 round trip);
        # without a workspace the entry point runs the fused kernel
        P.add_flops("fused_quant_gemm_4096x7168x7168",
                    *P.timed(lambda: F.fp8_block_gemm_fused_quant(X, qw, sw, out_dtype="bf16",
                                                                  c=C)), fl)
    if want("fused_quant_entry_staged_4096x7168x7168"):
        # the same call with the workspace it asks for: at this width it
        # takes the staged plan (the quantizer, then the block GEMM)
        few = torch.empty(F.fp8_fused_quant_workspace_bytes(M, N, K, "bf16"), dtype=torch.uint8,
                          device="cuda")
        P.add_flops("fused_quant_entry_staged_4096x7168x7168",
                    *P.timed(lambda: F.fp8_block_gemm_fused_quant(X, qw, sw, out_dtype="bf16",
                                                                  c=C, workspace=few)), fl)
        del few
    if want("fused_quant_crossover_m4096_k7168"):
        # The fused GEMM against the two-call path (quantizer, then GEMM),
        # each timed from a flushed cache, over the output width N: every
        # 256-column tile re-quantizes its activation rows in the fused
        # kernel, so it wins only for small N.
        import numpy as np
        rows = []
        for n in (256, 512, 1024, 2048, 4096, 7168):
            wq, ws = F.fp8_quant_weight_128x128(
                to_dev_bf16(torch, I.weights(np.random.default_rng(n), (n, K))))
            cn = torch.empty((M, n), dtype=torch.bfloat16, device="cuda")
            # each path in its best configuration: with the split-K
            # workspace it asks for (small N)
            nf = F.fp8_fused_quant_kernel_workspace_bytes(M, n, K, "bf16")
            fws = torch.empty(nf, dtype=torch.uint8, device="cuda") if nf else None
            ms_f, _ = P.timed(lambda: F.fp8_block_gemm_fused_quant(X, wq, ws, out_dtype="bf16",
                                                                   c=cn, workspace=fws))
            # the entry point with its own workspace size: the faster plan
            ne = F.fp8_fused_quant_workspace_bytes(M, n, K, "bf16")
            ews = torch.empty(ne, dtype=torch.uint8, device="cuda") if ne else None
            ms_e, _ = P.timed(lambda: F.fp8_block_gemm_fused_quant(X, wq, ws, out_dtype="bf16",
                                                                   c=cn, workspace=ews))
            nb = F.fp8_gemm_workspace_bytes(M, n, K, "bf16")
            gws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None

            def two_call():
                F.fp8_quant_act_1x128(X, qa, sa)
                F.fp8_block_gemm(qa, sa, wq, ws, out_dtype="bf16", c=cn, workspace=gws)
            ms_t, _ = P.timed(two_call)
            rows.append({"N": n, "fused_us": round(ms_f * 1e3, 2),
                         "two_call_us": round(ms_t * 1e3, 2),
                         "entry_us": round(ms_e * 1e3, 2),
                         "entry_plan": "fused" if ne == nf else "staged",
                         "fused_split_k_workspace_bytes": nf,
                         "entry_workspace_bytes": ne,
                         "two_call_split_k_workspace_bytes": nb,
                         "fused_faster": ms_f < ms_t})
            del wq, ws, cn, gws, fws, ews
        P.out["fused_quant_crossover_m4096_k7168"] = {
            "rows": rows, "note": "M=4096, K=7168, bf16 out; each launch (or pair) after a "
                                  "512 MB cache flush; median of 50; fused = the fused "
                                  "kernel with its split-K workspace, entry = "
                                  "fp8_block_gemm_fused_quant with its own workspace "
                                  "size (its faster plan), two_call = quantizer then "
                                  "block GEMM with its split-K workspace"}

    # backward of the same layer: dY [4096][7168] (same distribution as X
    # without outliers); Dgrad = forward GEMM with the transposed weights,
    # Wgrad = dY^T X from 128x1 tiles
    bwd = [n for n in ("bwd_quant_128x1_t_4096x7168", "bwd_transpose_weight_7168x7168",
                       "bwd_dgrad_4096x7168x7168", "bwd_dgrad_transposed_reads_4096x7168x7168",
                       "bwd_wgrad_7168x7168_over_4096", "pow2_bwd_quant_128x1_t_4096x7168",
                       "pow2_bwd_wgrad_7168x7168_over_4096",
                       "pow2_bwd_dgrad_transposed_reads_4096x7168x7168") if want(n)]
    if bwd:
        dy = to_dev_bf16(torch, I.activations(np.random.default_rng(7), M, N, 0.0, 1.0)[0])
        if want("bwd_quant_128x1_t_4096x7168"):
            P.add_bytes("bwd_quant_128x1_t_4096x7168",
                        *P.timed(lambda: F.fp8_quant_act_128x1_t(dy)), quant_bytes(M, N))
        qdy, sdy = F.fp8_quant_act_1x128(dy)
        qwt, swt = F.fp8_transpose_weight_128x128(qw, sw)
        if want("bwd_transpose_weight_7168x7168"):
            P.add_bytes("bwd_transpose_weight_7168x7168",
                        *P.timed(lambda: F.fp8_transpose_weight_128x128(qw, sw, qwt, swt)),
                        2 * N * K + 2 * 4 * (N // 128) * (K // 128))
        if want("bwd_dgrad_4096x7168x7168"):
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            P.add_flops("bwd_dgrad_4096x7168x7168",
                        *P.timed(lambda: F.fp8_block_gemm(qdy, sdy, qwt, swt, out_dtype="bf16",
                                                          c=dx)), fl)
            del dx
        if want("bwd_dgrad_transposed_reads_4096x7168x7168"):
            # Dgrad on the forward weights, read transposed inside the GEMM
            # (no weight transpose)
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            P.add_flops("bwd_dgrad_transposed_reads_4096x7168x7168",
                        *P.timed(lambda: F.fp8_block_gemm_dgrad(qdy, sdy, qw, sw,
                                                                out_dtype="bf16", dx=dx)), fl)
            del dx
        if want("bwd_wgrad_7168x7168_over_4096"):
            qdy_t, sdy_t = F.fp8_quant_act_128x1_t(dy)
            qx_t, sx_t = F.fp8_quant_act_128x1_t(X)
            dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
            P.add_flops("bwd_wgrad_7168x7168_over_4096",
                        *P.timed(lambda: F.fp8_block_gemm_wgrad(qdy_t, sdy_t, qx_t, sx_t,
                                                                out_dtype="f32", dw=dw)), fl)
            del qdy_t, sdy_t, qx_t, sx_t, dw
        if want("pow2_bwd_quant_128x1_t_4096x7168"):
            P.add_bytes("pow2_bwd_quant_128x1_t_4096x7168",
                        *P.timed(lambda: F.fp8_quant_act_128x1_t_pow2(dy)), quant_bytes(M, N))
        if want("pow2_bwd_wgrad_7168x7168_over_4096"):
            # power-of-two scales: the block-scaled MFMA takes each row's
            # scale, so the tiles are 256 rows tall
            qdy_t, sdy_t = F.fp8_quant_act_128x1_t_pow2(dy)
            qx_t, sx_t = F.fp8_quant_act_128x1_t_pow2(X)
            dw = torch.empty((N, K), dtype=torch.float32, device="cuda")
            P.add_flops("pow2_bwd_wgrad_7168x7168_over_4096",
                        *P.timed(lambda: F.fp8_block_gemm_wgrad_pow2(qdy_t, sdy_t, qx_t, sx_t,
                                                                     out_dtype="f32", dw=dw)), fl)
            del qdy_t, sdy_t, qx_t, sx_t, dw
        if want("pow2_bwd_dgrad_transposed_reads_4096x7168x7168"):
            # Dgrad on pow2-quantized dY and forward weights
            pdy, psdy = F.fp8_quant_act_1x128_pow2(dy)
            pw, psw = F.fp8_quant_weight_128x128_pow2(Wb)
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            P.add_flops("pow2_bwd_dgrad_transposed_reads_4096x7168x7168",
                        *P.timed(lambda: F.fp8_block_gemm_dgrad_pow2(pdy, psdy, pw, psw,
                                                                     out_dtype="bf16", dx=dx)),
                        fl)
            del pdy, psdy, pw, psw, dx
        del dy, qdy, sdy, qwt, swt

    # decode GEMM, 256 x 2048 x 7168 (split-K with workspace)
    dec = [n for n in ("decode_gemm_256x2048x7168", "decode_gemm_256x2048x7168_back_to_back")
           if want(n)]
    if dec:
        gd = I.config_decode(seed=0)
        da, dsa = F.fp8_quant_act_1x128(to_dev_bf16(torch, gd.a_bf16))
        dw, dsw = F.fp8_quant_weight_128x128(to_dev_bf16(torch, gd.w_bf16))
        nbytes = F.fp8_gemm_workspace_bytes(256, 2048, 7168, "bf16")
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda") if nbytes else None
        dc = torch.empty((256, 2048), dtype=torch.bfloat16, device="cuda")
        dfl = 2 * 256 * 2048 * 7168
        db = dense_gemm_bytes(256, 2048, 7168)
        if want("decode_gemm_256x2048x7168"):
            P.add_flops("decode_gemm_256x2048x7168",
                        *P.timed(lambda: F.fp8_block_gemm(da, dsa, dw, dsw, out_dtype="bf16",
                                                          c=dc, workspace=ws)), dfl, db,
                        split_k_workspace_bytes=nbytes)
        if want("decode_gemm_256x2048x7168_back_to_back"):
            # back to back, as a decode step calls one layer after another:
            # 40 operand sets (16.5 MB each, 700 MB in all) in rotation
            sets = [(da.clone(), dsa.clone(), dw.clone(), dsw.clone(), torch.empty_like(dc))
                    for _ in range(40)]
            ms, sp = P.back_to_back([lambda s=s: F.fp8_block_gemm(s[0], s[1], s[2], s[3],
                                                                  out_dtype="bf16", c=s[4],
                                                                  workspace=ws)
                                     for s in sets], rounds=2)
            P.add_flops("decode_gemm_256x2048x7168_back_to_back", ms, sp, dfl, db,
                        launches="40 sets x 2 rounds, best of 10")
            del sets
        del da, dsa, dw, dsw, ws, dc

    # grouped MoE GEMM, 32 experts / 8192 tokens, N=4096, K=7168
    grp = [n for n in ("grouped_gemm_e32_t8192_n4096_k7168",
                       "pow2_grouped_gemm_e32_t8192_n4096_k7168") if want(n)]
    if grp:
        gi = grouped_workload(I)
        off = torch.from_numpy(gi.offsets).cuda()
        gc = torch.empty((gi.T, gi.N), dtype=torch.bfloat16, device="cuda")
        gfl = 2 * int(gi.counts.sum()) * gi.N * gi.K
        gb = (gi.T * gi.K + gi.E * gi.N * gi.K + gi.T * gi.N * 2 + 4 * gi.T * (gi.K // 128)
              + 4 * gi.E * (gi.N // 128) * (gi.K // 128))
        for name, qa_fn, qw_fn, gemm in (
                ("grouped_gemm_e32_t8192_n4096_k7168", F.fp8_quant_act_1x128,
                 F.fp8_quant_weight_128x128, F.fp8_block_grouped_gemm),
                ("pow2_grouped_gemm_e32_t8192_n4096_k7168", F.fp8_quant_act_1x128_pow2,
                 F.fp8_quant_weight_128x128_pow2, F.fp8_block_grouped_gemm_pow2)):
            if not want(name):
                continue
            ga = to_dev_bf16(torch, gi.a_bf16)
            gq, gsa = qa_fn(ga)
            del ga
            gwb = to_dev_bf16(torch, gi.w_bf16.reshape(gi.E * gi.N, gi.K))
            gw, gsw = qw_fn(gwb)
            del gwb
            gw = gw.view(gi.E, gi.N, gi.K)
            gsw = gsw.view(gi.E, gi.N // 128, gi.K // 128)
            extra = {"counts": [int(c) for c in gi.counts]} if not name.startswith("pow2") else {}
            P.add_flops(name, *P.timed(lambda: gemm(gq, gsa, gw, gsw, off, out_dtype="bf16",
                                                    c=gc)), gfl, gb, **extra)
            del gq, gsa, gw, gsw
        del gc, off
    del P.flush
    torch.cuda.empty_cache()
    return P.out


def copy_calibration(torch, nbytes=1 << 30, iters=5):
    """A plain device copy of known size, for scaling rocprofv3 counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(iters):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_each_way": nbytes, "iters": iters}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(I, X_bits, w_bits):
    """The oracle as it stands, on this host's cores: the step on its first
    CPU_SAMPLE_ROWS tokens (the headline figure), and each workload."""
    import numpy as np
    import oracle
    cores = oracle.max_threads()    # OMP_NUM_THREADS, else the host's cores

    def clock(fn):
        t0 = time.perf_counter()
        r = fn()
        return time.perf_counter() - t0, r

    x = np.ascontiguousarray(X_bits[:CPU_SAMPLE_ROWS])
    qw, sw = oracle.quant_weight_128x128(w_bits)      # offline weights, not timed

    def step():
        qa, sa = oracle.quant_act_1x128(x)
        return oracle.block_gemm(qa, sa, qw, sw)
    dt, _ = clock(step)
    flops = 2 * CPU_SAMPLE_ROWS * N * K
    out = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.max_threads(),
           "kind": "oracle", "seconds": dt, "cpu_model": cpu_model(),
           "sample": f"first {CPU_SAMPLE_ROWS} of {M} tokens: 1x128 quantization of "
                     f"{CPU_SAMPLE_ROWS}x{K} + binary64 block-scaled GEMM "
                     f"{CPU_SAMPLE_ROWS}x{N}x{K}"}
    per = {}
    # quantizer, 4096 x 7168 in full: multi- and single-threaded
    b = quant_bytes(M, K)
    dt, _ = clock(lambda: oracle.quant_act_1x128(X_bits))
    per["act_quant_4096x7168"] = {"GB/s": b / dt / 1e9, "seconds": dt, "threads": cores}
    oracle.set_threads(1)
    dt, _ = clock(lambda: oracle.quant_act_1x128(X_bits))
    per["act_quant_4096x7168_single_thread"] = {"GB/s": b / dt / 1e9, "seconds": dt,
                                                "threads": 1}
    oracle.set_threads(cores)
    # tiny GEMM in full
    g = I.config_tiny(seed=0)
    tqa, tsa = oracle.quant_act_1x128(g.a_bf16)
    tqw, tsw = oracle.quant_weight_128x128(g.w_bf16)
    dt, _ = clock(lambda: oracle.block_gemm(tqa, tsa, tqw, tsw))
    per["tiny_gemm_128x256x512"] = {"GFLOP/s": 2 * 128 * 256 * 512 / dt / 1e9, "us": dt * 1e6}
    # dense: the headline sample above (GEMM part)
    per["dense_gemm_4096x7168x7168"] = {"GFLOP/s": flops / out["seconds"] / 1e9,
                                        "sample": f"first {CPU_SAMPLE_ROWS} rows, with their "
                                                  "quantization"}
    # decode in full
    gd = I.config_decode(seed=0)
    dqa, dsa = oracle.quant_act_1x128(gd.a_bf16)
    dqw, dsw = oracle.quant_weight_128x128(gd.w_bf16)
    dt, _ = clock(lambda: oracle.block_gemm(dqa, dsa, dqw, dsw))
    per["decode_gemm_256x2048x7168"] = {"GFLOP/s": 2 * 256 * 2048 * 7168 / dt / 1e9,
                                        "seconds": dt}
    # grouped: every 8th routed row of each expert (stratified eighth)
    gi = grouped_workload(I)
    gqa, gsa = oracle.quant_act_1x128(gi.a_bf16)
    gqw, gsw = oracle.quant_weight_128x128(gi.w_bf16.reshape(gi.E * gi.N, gi.K))
    gqw = gqw.reshape(gi.E, gi.N, gi.K)
    gsw = gsw.reshape(gi.E, gi.N // 128, gi.K // 128)
    rows = np.concatenate([np.arange(gi.offsets[e], gi.offsets[e + 1])[::8]
                           for e in range(gi.E)]).astype(np.int64)
    dt, _ = clock(lambda: oracle.grouped_gemm(gqa, gsa, gqw, gsw, gi.offsets, rows))
    per["grouped_gemm_e32_t8192_n4096_k7168"] = {
        "GFLOP/s": 2 * rows.size * gi.N * gi.K / dt / 1e9, "seconds": dt,
        "sample": f"{rows.size} rows: every 8th routed row of each expert"}
    out["per_workload"] = per
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-parts", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--part", default=None, help="run only this part and print it")
    ap.add_argument("--preroll", type=float, default=PREROLL_S,
                    help="seconds of untimed steps before the warm-up (default %(default)s)")
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
    F.fp8_quant_act_1x128(X, qa, sa)
    torch.cuda.synchronize()

    if args.part:
        parts = measure_parts(torch, F, I, X, Wb, qa, sa, qw, sw, C, only=args.part)
        if not parts:
            print(f"bench.py: no part named {args.part}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps({"parts": parts}), flush=True)
        return

    result_tail = {}
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline ...")
        result_tail["cpu_baseline"] = cpu_baseline(I, X_bits, w_bits)
    if not args.no_parts:
        log("bench: per-kernel parts ...")
        result_tail["parts"] = measure_parts(torch, F, I, X, Wb, qa, sa, qw, sw, C)

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

    # Fixed untimed pre-roll: the step itself for PREROLL_S seconds, so the
    # timed region starts at the clock the GPU sustains on this work rather
    # than on the ramp (20 timed steps are only ~5 ms).  The clock is
    # sampled over the pre-roll's last part and the timed region.
    log("bench: pre-roll and timed steps ...")
    clk = ClockSampler()
    t_pre = time.perf_counter()
    sampling = False
    n_pre = 0
    while time.perf_counter() - t_pre < args.preroll:
        for _ in range(10):
            step(False)
        n_pre += 10
        torch.cuda.synchronize()
        if not sampling and time.perf_counter() - t_pre > 0.5 * args.preroll:
            clk.start()
            sampling = True
    if not sampling:
        clk.start()
    probe = GpuClockProbe(torch)
    for _ in range(args.warmup):
        step(False)
    probe.mark(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    probe.mark(1)
    torch.cuda.synchronize()
    clock = clk.stop()
    sclk = probe.result()
    sclk["amdsmi_gfx_clock"] = clock

    ms_per_step = (t1 - t0) / args.steps * 1e3
    flops = 2 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = gemm_t.mean_ms()
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    props = torch.cuda.get_device_properties(0)
    roof = {"bound": "mfma", "kernel": "dense_gemm_two_kind_kernel",
            "achieved": round(achieved, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic_from_counters(),
            "gemm_us": round(gemm_ms * 1e3, 2), "sclk_timed_region": sclk}
    if sclk.get("mhz_mean"):
        # the same fraction against the FP8 peak at the clock the GPU ran at
        roof["frac_at_running_clock"] = round(
            achieved / (PEAK_FP8_TFLOPS * sclk["mhz_mean"] / MAX_SCLK_MHZ), 4)
    dense_part = result_tail.get("parts", {}).get("dense_gemm_4096x7168x7168")
    if dense_part:
        roof["frac_flushed_part"] = round(dense_part["frac_mfma"], 4)
    result = {
        "metric": "FP8 block-scaled GEMM TFLOP/s + % FP8 MFMA peak; act-quant GB/s % HBM",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": "prefill linear: 1x128 act-quant of 4096x7168 bf16 (0.1% outlier "
                               "channels x100) + fp8_block_gemm M=4096 N=7168 K=7168 bf16 out",
                   "M": M, "N": N, "K": K, "weights": "128x128-quantized once before timing",
                   "parallelism": "single GPU",
                   "preroll": f"CPU baseline, per-kernel parts, then {n_pre} untimed steps "
                              f"({args.preroll} s) before the warm-up steps"},
        "roofline": roof,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count,
                   "memory_bytes": props.total_memory},
        "inputs_sha256": {"X_bf16_4096x7168": hashlib.sha256(X_bits.tobytes()).hexdigest()[:16],
                          "W_bf16_7168x7168": hashlib.sha256(w_bits.tobytes()).hexdigest()[:16]},
    }
    if args.copy_calib:
        result["copy_calibration"] = copy_calibration(torch)
    result.update(result_tail)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
