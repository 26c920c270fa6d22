"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Quantizers: E4M3 bytes and fp32 scale bits must be identical.  GEMMs: the
relative Frobenius error against the oracle's binary64 reference must be
within 1e-3 (FP32 out) / 8e-3 (BF16 out), and within the level FP32
accumulation actually gives.  Inputs come from the seeded generator; every
oracle input is the generator's or the oracle's own output.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import (check_gemm, dev, dev_bf16, gemm_error_bound, grouped_error_bound, host,
                       log, tile_rows, torch)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def quant_act_gpu(bits):
    q, s = B.fp8_quant_act_1x128(dev_bf16(bits))
    return host(q), host(s)


def assert_quant_equal(qg, sg, qo, so, what):
    nbad = int((qg != qo).sum())
    sbad = int((sg.view(np.uint32) != so.view(np.uint32)).sum())
    log(f"  {what}: byte mismatches={nbad} scale mismatches={sbad}")
    if nbad:
        idx = np.argwhere(qg != qo)[:5]
        log("  first mismatches (row, col, gpu, oracle):",
            [(int(i), int(j), int(qg[i, j]), int(qo[i, j])) for i, j in idx])
    assert nbad == 0 and sbad == 0


# ---- activation quantizer ---------------------------------------------------

@pytest.mark.parametrize("M,K", [(1, 128), (3, 300), (17, 7168), (64, 1000), (5, 1001),
                                 (33, 8), (2, 130), (5, 384), (7, 896)])
def test_quant_act_shapes(M, K):
    # (5, 384), (7, 896): 15 and 49 groups, so the last wave of the K % 128
    # == 0 kernel (8 groups per wave) is partly out of range
    x, _ = I.activations(np.random.default_rng(M * 7 + K), M, K, 0.01, 50.0)
    qo, so = oracle.quant_act_1x128(x)
    qg, sg = quant_act_gpu(x)
    assert_quant_equal(qg, sg, qo, so, f"act {M}x{K}")


def test_quant_act_workload_4096x7168():
    x, _ = I.config_quant(seed=0)
    log("  oracle quantizing 4096x7168 ...")
    qo, so = oracle.quant_act_1x128(x)
    qg, sg = quant_act_gpu(x)
    assert_quant_equal(qg, sg, qo, so, "act 4096x7168")


def test_quant_act_special_groups():
    K = 512
    x = np.zeros((6, K), np.uint16)
    x[1, :] = 0x8000                                   # all -0.0
    x[2, 5] = 0x0001                                   # smallest subnormal amax
    x[2, 130] = 0x8001
    x[3, :128] = I.f32_to_bf16_bits(np.linspace(-1, 1, 128, dtype=np.float32))
    x[4, :] = 0x7F7F                                   # largest finite everywhere
    x[5, 256:384] = I.f32_to_bf16_bits(np.float32(448.0 * 2.0 ** -130) * np.ones(128, np.float32))
    qo, so = oracle.quant_act_1x128(x)
    qg, sg = quant_act_gpu(x)
    assert_quant_equal(qg, sg, qo, so, "special groups")


def test_quant_act_misaligned_pointer():
    # a row-offset view whose base is only 2-byte aligned takes the general path
    M, K = 9, 257
    x, _ = I.activations(np.random.default_rng(3), M + 1, K)
    t = torch()
    big = dev_bf16(x)
    view = big.view(-1)[K:].view(M, K)
    q, s = B.fp8_quant_act_1x128(view)
    qo, so = oracle.quant_act_1x128(np.ascontiguousarray(x[1:]))
    assert_quant_equal(host(q), host(s), qo, so, "misaligned")
    del t


def test_quant_act_output_8_byte_aligned():
    # E4M3 output at an 8-byte (not 16-byte) offset: the K % 128 == 0 kernel
    # stores 8 bytes per lane, so it still serves this layout
    M, K = 12, 640
    x, _ = I.activations(np.random.default_rng(5), M, K, 0.01, 50.0)
    t = torch()
    qbuf = t.full((M * K + 16,), 0x5A, dtype=t.uint8, device="cuda")
    q = qbuf[8:8 + M * K].view(M, K)
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    B.fp8_quant_act_1x128(dev_bf16(x), q, s)
    qo, so = oracle.quant_act_1x128(x)
    assert_quant_equal(host(q), host(s), qo, so, "act, 8-byte aligned output")
    hb = host(qbuf)
    assert np.all(hb[:8] == 0x5A) and np.all(hb[8 + M * K:] == 0x5A), "bytes outside q written"


# ---- weight quantizer ---------------------------------------------------------

@pytest.mark.parametrize("N,K", [(256, 512), (200, 130), (128, 7168), (2048, 7168), (3, 5)])
def test_quant_weight_shapes(N, K):
    w = I.weights(np.random.default_rng(N + K), (N, K))
    qo, so = oracle.quant_weight_128x128(w)
    q, s = B.fp8_quant_weight_128x128(dev_bf16(w))
    assert_quant_equal(host(q), host(s), qo, so, f"weight {N}x{K}")


# ---- dense GEMM -----------------------------------------------------------------

def quantize(g):
    qa, sa = oracle.quant_act_1x128(g.a_bf16)
    qw, sw = oracle.quant_weight_128x128(g.w_bf16)
    return qa, sa, qw, sw


def run_gemm(qa, sa, qw, sw, out, workspace=None):
    return B.fp8_block_gemm(dev(qa), dev(sa), dev(qw), dev(sw), out_dtype=out,
                            workspace=workspace)


def test_gemm_tiny_fp32_out():
    g = I.config_tiny(seed=0)
    qa, sa, qw, sw = quantize(g)
    R = oracle.block_gemm(qa, sa, qw, sw)
    check_gemm(run_gemm(qa, sa, qw, sw, "f32"), R, "f32", "tiny 128x256x512 f32",
               gemm_error_bound(qa, sa, qw, sw))


@pytest.mark.parametrize("M", [1, 15, 17, 129, 255, 300])
@pytest.mark.parametrize("N,K", [(128, 128), (384, 640)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_ragged(M, N, K, out):
    g = I.gemm_inputs(M, N, K, seed=M * 1000 + N + K, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    R = oracle.block_gemm(qa, sa, qw, sw)
    check_gemm(run_gemm(qa, sa, qw, sw, out), R, out, f"{M}x{N}x{K} {out}",
               gemm_error_bound(qa, sa, qw, sw))


def test_gemm_decode_workload_with_and_without_workspace():
    g = I.config_decode(seed=0)
    qa, sa, qw, sw = quantize(g)
    log("  oracle GEMM 256x2048x7168 ...")
    R = oracle.block_gemm(qa, sa, qw, sw)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(256, 2048, 7168, "bf16")
    assert nbytes > 0
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    c1 = run_gemm(qa, sa, qw, sw, "bf16", workspace=ws)
    c2 = run_gemm(qa, sa, qw, sw, "bf16")
    splits = nbytes // (256 * 2048 * 4)
    b = gemm_error_bound(qa, sa, qw, sw, splits=splits)
    check_gemm(c1, R, "bf16", "decode split-K", b)
    check_gemm(c2, R, "bf16", "decode no workspace", gemm_error_bound(qa, sa, qw, sw))
    c3 = run_gemm(qa, sa, qw, sw, "f32", workspace=ws)
    check_gemm(c3, R, "f32", "decode split-K f32", b)


@pytest.mark.parametrize("M,N,K,splits", [(128, 128, 8192, 16), (100, 256, 2688, 4)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_split_k_many_and_uneven_splits(M, N, K, splits, out):
    """Split-K with more than eight splits (the reduction gathers partials
    eight at a time) and with a last split shorter than the others (21 K
    blocks over 4 splits of 6); the workspace size shows the split count."""
    g = I.gemm_inputs(M, N, K, seed=M + N + K, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    R = oracle.block_gemm(qa, sa, qw, sw)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, out)
    assert nbytes == splits * M * N * 4, f"{M}x{N}x{K}: workspace {nbytes} B"
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    c1 = run_gemm(qa, sa, qw, sw, out, workspace=ws)
    c2 = run_gemm(qa, sa, qw, sw, out, workspace=ws)
    check_gemm(c1, R, out, f"split-K x{splits} {M}x{N}x{K} {out}",
               gemm_error_bound(qa, sa, qw, sw, splits=splits))
    assert t.equal(c1, c2), "split-K result changed between identical calls"


def test_gemm_split_k_workspace_garbage_and_repeats():
    # The workspace needs no initialization: full of garbage (random bytes,
    # then all ones) before every call, it must still give the oracle's
    # result, bit for bit the same on every call (the partials are summed in
    # a fixed order).
    t = torch()
    M, N, K = 200, 512, 7168
    g = I.gemm_inputs(M, N, K, seed=77, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    R = oracle.block_gemm(qa, sa, qw, sw)
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, "f32")
    assert nbytes > 0
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    gen = t.Generator(device="cuda")
    gen.manual_seed(5)
    outs = []
    for r in range(6):
        if r % 2 == 0:
            ws.random_(0, 256, generator=gen)
        else:
            ws.fill_(0xFF)
        outs.append(run_gemm(qa, sa, qw, sw, "f32", workspace=ws))
    for _ in range(3):  # and back to back on the same workspace
        outs.append(run_gemm(qa, sa, qw, sw, "f32", workspace=ws))
    check_gemm(outs[0], R, "f32", "split-K, garbage workspace",
               gemm_error_bound(qa, sa, qw, sw, splits=nbytes // (M * N * 4)))
    for o in outs[1:]:
        assert t.equal(o, outs[0]), "split-K result changed between calls"


def test_gemm_dense_workload_rows_of_every_tile():
    # 4096 x 7168 x 7168 runs 256-row tiles: three rows of every M tile
    # (and the first and last row), every column, each output within its
    # bound.  The columns cover both tile widths of the two-kind plan.
    g = I.config_dense(seed=0)
    qa, sa, qw, sw = quantize(g)
    c = run_gemm(qa, sa, qw, sw, "bf16")
    rows = tile_rows(4096, 256, per_tile=3)
    log(f"  oracle GEMM on {rows.size} rows of 4096x7168x7168 ...")
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "bf16", "dense workload rows",
               gemm_error_bound(qa, sa, qw, sw, rows))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_big_tiles_ragged_edges(out):
    # Enough 256x256 tiles to take the large-tile path, with a partial last
    # M tile (4000 = 15*256 + 160) and a partial last N tile (7040 = 27*256 +
    # 128): compared on rows from every M tile, including the last ones.
    M, N, K = 4000, 7040, 384
    g = I.gemm_inputs(M, N, K, seed=77, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    c = run_gemm(qa, sa, qw, sw, out)
    rows = np.unique(np.concatenate([np.arange(0, M, 97), [255, 256, 3839, 3840, 3999]]))
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, out, f"big tiles ragged {out}",
               gemm_error_bound(qa, sa, qw, sw, rows))


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gemm_192_wide_tiles_all_columns(out):
    # 4096 x 6144 is planned as 32 x 16 tiles of 256 x 192 (two full rounds):
    # tiles start at column offsets 0 or 64 inside a 128-column weight-scale
    # block, so every way a wave's 48 columns can straddle two blocks occurs.
    # Rows from every M tile, all columns.
    M, N, K = 4096, 6144, 512
    g = I.gemm_inputs(M, N, K, seed=78, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    c = run_gemm(qa, sa, qw, sw, out)
    rows = np.unique(np.concatenate([np.arange(0, M, 127), [255, 256, 4095]]))
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, out, f"192-wide tiles {out}",
               gemm_error_bound(qa, sa, qw, sw, rows))


@pytest.mark.parametrize("shape", [(4096, 4096, 128), (4096, 4096, 256), (4096, 7168, 128)])
def test_gemm_big_tiles_one_or_two_k_blocks(shape):
    # The two-stage pipeline with one or two K blocks: the copies of blocks
    # past the end come from empty buffers.  4096 x 4096 runs 256 tiles of
    # 256 x 256, 4096 x 7168 the two tile widths.
    M, N, K = shape
    g = I.gemm_inputs(M, N, K, seed=80 + K)
    qa, sa, qw, sw = quantize(g)
    c = run_gemm(qa, sa, qw, sw, "f32")
    rows = np.array([0, 17, 255, 256, 1000, 2047, 2048, 4095])
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "f32", f"big tiles {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows))


def test_gemm_two_tile_widths_metamorphic_and_deterministic():
    # 4096 x 7168 runs 256 tiles of 256 x 256 and 256 of 256 x 192: two runs
    # are bitwise identical, and scaling the activation scales by 2^3 scales
    # the FP32 result by exactly 2^3.
    M, N, K = 4096, 7168, 256
    g = I.gemm_inputs(M, N, K, seed=79)
    qa, sa, qw, sw = quantize(g)
    c0 = host(run_gemm(qa, sa, qw, sw, "f32"))
    c1 = host(run_gemm(qa, sa, qw, sw, "f32"))
    c2 = host(run_gemm(qa, sa * np.float32(8.0), qw, sw, "f32"))
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
    assert np.array_equal(c2, c0 * np.float32(8.0))
    rows = np.array([0, 255, 256, 2047, 4095])
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(torch().from_numpy(c0[rows]), R, "f32", "two tile widths",
               gemm_error_bound(qa, sa, qw, sw, rows))


def test_gemm_power_of_two_metamorphic_and_deterministic():
    # Scaling the activation scales by 2^j scales an FP32 result by exactly
    # 2^j; two runs of the same call are bitwise identical.
    g = I.gemm_inputs(200, 256, 1024, seed=9)
    qa, sa, qw, sw = quantize(g)
    c0 = host(run_gemm(qa, sa, qw, sw, "f32"))
    c1 = host(run_gemm(qa, sa, qw, sw, "f32"))
    c2 = host(run_gemm(qa, sa * np.float32(8.0), qw, sw, "f32"))
    assert np.array_equal(c0.view(np.uint32), c1.view(np.uint32))
    assert np.array_equal(c2, c0 * np.float32(8.0))


def test_gemm_zero_scales_give_zero():
    g = I.gemm_inputs(64, 128, 256, seed=10)
    qa, sa, qw, sw = quantize(g)
    c = host(run_gemm(qa, np.zeros_like(sa), qw, sw, "f32"))
    assert np.all(c == 0)


# ---- grouped GEMM -----------------------------------------------------------------

def quantize_grouped(gi):
    qa, sa = oracle.quant_act_1x128(gi.a_bf16)
    E, N, K = gi.w_bf16.shape
    qw, sw = oracle.quant_weight_128x128(gi.w_bf16.reshape(E * N, K))
    return qa, sa, qw.reshape(E, N, K), sw.reshape(E, N // 128, K // 128)


def run_grouped(qa, sa, qw, sw, off, out, c=None):
    return B.fp8_block_grouped_gemm(dev(qa), dev(sa), dev(qw), dev(sw), dev(off.astype(np.int32)),
                                    out_dtype=out, c=c)


@pytest.mark.parametrize("counts,T", [
    ([20, 0, 33, 1, 10], 70),        # empty expert and 6 unrouted rows at the end
    ([0, 0, 300], 300),              # one expert holds every token
    ([129, 127, 1, 0, 256], 513),
    ([0, 0, 0], 16),                 # nothing routed: C untouched
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_edge_cases(counts, T, out):
    E = len(counts)
    gi = I.grouped_inputs(E, T, 256, 384, seed=sum(counts) + E, counts=counts)
    qa, sa, qw, sw = quantize_grouped(gi)
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    t = torch()
    dt = t.float32 if out == "f32" else t.bfloat16
    c = t.full((T, 256), 7.0, dtype=dt, device="cuda")
    run_grouped(qa, sa, qw, sw, gi.offsets, out, c=c)
    ch = host(c)
    routed = int(gi.offsets[-1])
    assert np.all(ch[routed:] == 7.0), "unrouted rows were written"
    if routed:
        check_gemm(c[:routed], R[:routed], out, f"grouped {counts} {out}",
                   grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(routed)))


def _counts_150(case):
    if case == "zipf":
        return None                                   # zipf routing of all 2000 tokens
    if case == "last_expert":
        return [0] * 149 + [700]                      # only the last chunk's last expert
    c = [0] * 150                                     # experts either side of 64 and 128
    c[63], c[64], c[127], c[128], c[149] = 200, 129, 1, 256, 3
    return c


@pytest.mark.parametrize("case", ["zipf", "last_expert", "chunk_boundaries"])
def test_grouped_more_than_64_experts(case):
    # The tile lookup scans the offsets 64 experts per wave step, carrying
    # the prefix maximum and the tile count from one chunk to the next; 150
    # experts make three chunks.  Every routed row is checked.
    E, N, K = 150, 256, 256
    counts = _counts_150(case)
    T = 2000 if counts is None else sum(counts)
    gi = I.grouped_inputs(E, T, N, K, seed=150 + len(case), counts=counts)
    qa, sa, qw, sw = quantize_grouped(gi)
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    c = run_grouped(qa, sa, qw, sw, gi.offsets, "f32")
    routed = int(gi.offsets[-1])
    assert routed > 0 and found[:routed].all()
    check_gemm(c[:routed], R[:routed], "f32", f"grouped {E} experts ({case})",
               grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(routed)))


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_expert_tails(pow2):
    # Experts whose last 128-row M tile holds 1, 63, 64, 65, 127 or 128 rows
    # (one to three M tiles each), two N tiles and 10 K blocks (a scale
    # chunk boundary and a partial chunk); every routed row against the
    # oracle, FP32 out.
    counts = [64, 65, 127, 128, 192, 193, 1, 0, 63, 320]
    E, T, N, K = len(counts), sum(counts) + 5, 512, 1280
    gi = I.grouped_inputs(E, T, N, K, seed=640 + int(pow2), counts=counts)
    if pow2:
        qa, sa = oracle.quant_act_1x128_pow2(gi.a_bf16)
        qw, sw = oracle.quant_weight_128x128_pow2(gi.w_bf16.reshape(E * N, K))
        gemm = B.fp8_block_grouped_gemm_pow2
    else:
        qa, sa = oracle.quant_act_1x128(gi.a_bf16)
        qw, sw = oracle.quant_weight_128x128(gi.w_bf16.reshape(E * N, K))
        gemm = B.fp8_block_grouped_gemm
    qw, sw = qw.reshape(E, N, K), sw.reshape(E, N // 128, K // 128)
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    t = torch()
    c = t.full((T, N), 7.0, dtype=t.float32, device="cuda")
    gemm(dev(qa), dev(sa), dev(qw), dev(sw), dev(gi.offsets.astype(np.int32)),
         out_dtype="f32", c=c)
    ch = host(c)
    routed = int(gi.offsets[-1])
    assert found[:routed].all()
    assert np.all(ch[routed:] == 7.0), "unrouted rows were written"
    check_gemm(c[:routed], R[:routed], "f32", f"grouped expert tails pow2={pow2}",
               grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(routed)))


def test_grouped_garbage_offsets_are_memory_safe():
    # Offsets beyond T and decreasing ranges are clamped/empty: no fault, and
    # rows outside [clamped off[0], clamped off[E]) stay untouched.
    E, T = 4, 100
    gi = I.grouped_inputs(E, T, 128, 256, seed=5, counts=[25, 25, 25, 25])
    qa, sa, qw, sw = quantize_grouped(gi)
    off = np.array([10, 60, 40, 90, 5000], dtype=np.int32)  # decreasing then past T
    t = torch()
    c = t.full((T, 128), 7.0, dtype=t.float32, device="cuda")
    run_grouped(qa, sa, qw, sw, off, "f32", c=c)
    t.cuda.synchronize()
    ch = host(c)
    assert np.all(ch[:10] == 7.0)
    # Clamped and made non-overlapping: expert 0 keeps [10, 60), expert 1 is
    # empty, expert 2 starts where expert 0 ended: [60, 90), expert 3 gets
    # [90, 100).
    eff = np.array([10, 60, 60, 90, 100], np.int32)
    R, _ = oracle.grouped_gemm(qa, sa, qw, sw, eff)
    b = grouped_error_bound(qa, sa, qw, sw, eff, np.arange(T))
    check_gemm(c[10:60], R[10:60], "f32", "garbage offsets expert 0", b[10:60])
    check_gemm(c[60:90], R[60:90], "f32", "garbage offsets expert 2", b[60:90])
    check_gemm(c[90:100], R[90:100], "f32", "garbage offsets expert 3", b[90:100])


def expert_tile_rows(off, tile=128, per_tile=1, salt=0):
    """Rows of every expert's every `tile`-row M tile (the grouped kernel's
    tiles start at each expert's first row), plus each expert's first and
    last row."""
    rows = []
    for e in range(len(off) - 1):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            rows += list(lo + tile_rows(hi - lo, tile, per_tile, salt + e))
    return np.unique(np.array(rows, dtype=np.int64))


def test_grouped_workload_rows_of_every_tile():
    # 32 experts over 8192 tokens: one row inside every 128-row M tile of
    # every expert (plus its first and last row), all 4096 columns, each
    # output within its bound.
    gi = I.config_grouped(seed=0)
    log("  quantizing grouped workload with the oracle ...")
    qa, sa, qw, sw = quantize_grouped(gi)
    c = run_grouped(qa, sa, qw, sw, gi.offsets, "bf16")
    off = gi.offsets
    rows = expert_tile_rows(off)
    log(f"  oracle grouped GEMM on {rows.size} rows ...")
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, off, rows)
    assert found.all()
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "bf16", "grouped workload rows",
               grouped_error_bound(qa, sa, qw, sw, off, rows))


def quantize_grouped_pow2(gi):
    qa, sa = oracle.quant_act_1x128_pow2(gi.a_bf16)
    E, N, K = gi.w_bf16.shape
    qw, sw = oracle.quant_weight_128x128_pow2(gi.w_bf16.reshape(E * N, K))
    return qa, sa, qw.reshape(E, N, K), sw.reshape(E, N // 128, K // 128)


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_full_depth_fp32_every_row(pow2):
    # FP32 output at the workload's depth and width (K = 7168: 56 K blocks,
    # seven activation-scale chunks; N = 4096: 16 N tiles with their own
    # weight-scale blocks), every routed row: expert 0 spans eight 128-row M
    # tiles, expert 1 a ragged 300 (three tiles, the last 44 rows), expert 2
    # is empty, expert 3 has 77 rows.
    counts = [1024, 300, 0, 77]
    E, N, K = 4, 4096, 7168
    T = sum(counts) + 5                                   # 5 unrouted rows
    gi = I.grouped_inputs(E, T, N, K, seed=1401, counts=counts)
    qa, sa, qw, sw = quantize_grouped_pow2(gi) if pow2 else quantize_grouped(gi)
    routed = int(gi.offsets[-1])
    log(f"  oracle grouped GEMM on all {routed} rows at K={K}, N={N} ...")
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    t = torch()
    c = t.full((T, N), 7.0, dtype=t.float32, device="cuda")
    fn = B.fp8_block_grouped_gemm_pow2 if pow2 else B.fp8_block_grouped_gemm
    fn(dev(qa), dev(sa), dev(qw), dev(sw), dev(gi.offsets.astype(np.int32)), out_dtype="f32", c=c)
    ch = host(c)
    assert np.all(ch[routed:] == 7.0), "unrouted rows were written"
    assert found[:routed].all()
    check_gemm(c[:routed], R[:routed], "f32", f"grouped full depth every row (pow2={pow2})",
               grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(routed)))


@pytest.mark.parametrize("pow2", [False, True])
def test_grouped_scale_chunks_not_a_multiple(pow2):
    # K = 2304: G = 18 K blocks, so the last activation-scale chunk (8 blocks
    # each) holds only two, fetched dword by dword; N = 512 (two N tiles);
    # every routed row, FP32 output.
    counts = [0, 1, 129, 300]
    E, N, K = 4, 512, 2304
    T = sum(counts)
    gi = I.grouped_inputs(E, T, N, K, seed=2304, counts=counts)
    qa, sa, qw, sw = quantize_grouped_pow2(gi) if pow2 else quantize_grouped(gi)
    R, found = oracle.grouped_gemm(qa, sa, qw, sw, gi.offsets)
    fn = B.fp8_block_grouped_gemm_pow2 if pow2 else B.fp8_block_grouped_gemm
    c = fn(dev(qa), dev(sa), dev(qw), dev(sw), dev(gi.offsets.astype(np.int32)), out_dtype="f32")
    check_gemm(c, R, "f32", f"grouped G=18 (pow2={pow2})",
               grouped_error_bound(qa, sa, qw, sw, gi.offsets, np.arange(T)))


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 1280), (300, 384, 1280), (4096, 7168, 640)])
def test_gemm_scale_chunks_not_a_multiple(M, N, K):
    # G = 10 or 5 K blocks: the last activation-scale chunk is partial (its
    # scales fetched dword by dword so that nothing past the last row's
    # scales is read).  Big tiles (4096 x 4096), the two tile widths (4096 x
    # 7168) and small tiles (300 x 384), rows of every tile incl. the last.
    g = I.gemm_inputs(M, N, K, seed=M + N + K, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa, qw, sw = quantize(g)
    c = run_gemm(qa, sa, qw, sw, "f32")
    rows = tile_rows(M, 128, per_tile=2)
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    check_gemm(c[torch().from_numpy(rows).cuda()], R, "f32", f"G={K // 128} {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows))


@pytest.mark.parametrize("M,N,K", [
    (256, 256, 32768),   # 256 K blocks: 32 scale chunks; 128 x 64 tiles with split-K
    (4096, 7168, 16384), # both 256-row tile widths over 128 K blocks
])
def test_gemm_long_k(M, N, K):
    # Long inner dimensions: many scale chunks and double-buffer turns, and
    # the FP32 promotion over up to 256 blocks, on rows of every M tile
    g = I.gemm_inputs(M, N, K, seed=K + 5, outlier_frac=0.001, outlier_mult=100.0)
    qa, sa, qw, sw = quantize(g)
    t = torch()
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, "f32")
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    c = run_gemm(qa, sa, qw, sw, "f32", workspace=ws)
    rows = np.arange(M, step=17) if M <= 256 else tile_rows(M, 256, per_tile=1)
    log(f"  {M}x{N}x{K} (workspace {nbytes} B): oracle on {rows.size} rows")
    R = oracle.block_gemm(qa, sa, qw, sw, rows)
    splits = max(1, nbytes // (M * N * 4))
    check_gemm(c[t.from_numpy(rows).cuda()], R, "f32", f"long K {M}x{N}x{K}",
               gemm_error_bound(qa, sa, qw, sw, rows, splits=splits))


def test_quant_then_gemm_chain_matches_oracle_chain():
    # The GPU quantizer's output fed to the GPU GEMM equals the oracle chain.
    g = I.gemm_inputs(96, 256, 768, seed=12, outlier_frac=0.01, outlier_mult=50.0)
    qa_d, sa_d = B.fp8_quant_act_1x128(dev_bf16(g.a_bf16))
    qw_d, sw_d = B.fp8_quant_weight_128x128(dev_bf16(g.w_bf16))
    c = B.fp8_block_gemm(qa_d, sa_d, qw_d, sw_d, out_dtype="f32")
    qa, sa, qw, sw = quantize(g)
    R = oracle.block_gemm(qa, sa, qw, sw)
    check_gemm(c, R, "f32", "quant->gemm chain", gemm_error_bound(qa, sa, qw, sw))
