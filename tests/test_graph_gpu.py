"""The hot path inside a captured HIP graph.

Quantization and the GEMMs allocate nothing, and none of them issues a
memset, so a serving loop can capture them once and replay them: the
split-K path takes its partials from the caller's workspace and reduces
them with a kernel (the no-allocation GEMM from the library's static
scratch array instead).  Each test captures 1x128 activation quantization
followed by a GEMM (plain, split-K, grouped, no-allocation, Dgrad on the
forward weights), or the GEMM with the quantization fused in (also as the
quantizer and block GEMM that its entry point runs for a small M when given
its workspace), into one graph (torch.cuda.CUDAGraph over the library's
launches on the capture stream) and replays it several times.  Between
replays the program's own eager work changes the bf16 input in place and
synchronizes, and every replay must equal, bit for bit, the eager chain on
the same input: the same kernels run on the same bytes, in a fixed
summation order.
"""
import numpy as np
import pytest

from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import dev_bf16, log, torch

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def activations(seed, M, K):
    return dev_bf16(I.activations(np.random.default_rng(seed), M, K, 0.01, 50.0)[0])


def replay_and_check(capture, eager, x, fresh_inputs, what):
    """capture(): the launches to record (static buffers); eager(): the same
    chain into new buffers, returning the outputs to compare."""
    t = torch()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        capture()  # warm-up outside the graph (first-launch work)
    t.cuda.current_stream().wait_stream(s)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        outs = capture()
    for r in range(REPLAYS):
        x.copy_(fresh_inputs[r])  # eager work between replays
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        ref = eager()
        for o, e in zip(outs, ref):
            assert t.equal(o, e), f"{what}: replay {r} differs from the eager chain"
    log(f"  {what}: {REPLAYS} replays equal the eager chain")
    del g


def test_graph_quant_and_split_k_gemm():
    # 64 x 2048 x 7168: the small-M plan splits K through the workspace and
    # reduces the partials with a second kernel
    t = torch()
    M, N, K = 64, 2048, 7168
    x = activations(1, M, K)
    fresh = [activations(10 + r, M, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(2), (N, K))))
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, "bf16")
    assert nbytes > 0
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda")
    q = t.empty((M, K), dtype=t.uint8, device="cuda")
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    c = t.empty((M, N), dtype=t.bfloat16, device="cuda")

    def capture():
        B.fp8_quant_act_1x128(x, q, s)
        B.fp8_block_gemm(q, s, qw, sw, out_dtype="bf16", c=c, workspace=ws)
        return q, s, c

    def eager():
        q2, s2 = B.fp8_quant_act_1x128(x)
        ws2 = t.empty_like(ws)
        return q2, s2, B.fp8_block_gemm(q2, s2, qw, sw, out_dtype="bf16", workspace=ws2)

    replay_and_check(capture, eager, x, fresh, "quant + split-K GEMM 64x2048x7168")


def test_graph_quant_and_gemm_without_workspace():
    # 512 x 1024 x 1024 with FP32 output and no workspace: one launch of the
    # dense kernel over the whole K
    t = torch()
    M, N, K = 512, 1024, 1024
    x = activations(3, M, K)
    fresh = [activations(20 + r, M, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(4), (N, K))))
    q = t.empty((M, K), dtype=t.uint8, device="cuda")
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    c = t.empty((M, N), dtype=t.float32, device="cuda")

    def capture():
        B.fp8_quant_act_1x128(x, q, s)
        B.fp8_block_gemm(q, s, qw, sw, out_dtype="f32", c=c)
        return q, s, c

    def eager():
        q2, s2 = B.fp8_quant_act_1x128(x)
        return q2, s2, B.fp8_block_gemm(q2, s2, qw, sw, out_dtype="f32")

    replay_and_check(capture, eager, x, fresh, "quant + GEMM 512x1024x1024 f32")


def test_graph_quant_and_grouped_gemm():
    # 6 experts over 700 tokens, one expert empty
    t = torch()
    counts = [200, 0, 130, 1, 300, 69]
    gi = I.grouped_inputs(len(counts), 700, 256, 512, seed=5, counts=counts)
    E, N, K = gi.w_bf16.shape
    x = dev_bf16(gi.a_bf16)
    fresh = [activations(30 + r, 700, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(gi.w_bf16.reshape(E * N, K)))
    qw = qw.view(E, N, K)
    sw = sw.view(E, N // 128, K // 128)
    off = t.from_numpy(gi.offsets.astype(np.int32)).cuda()
    q = t.empty((700, K), dtype=t.uint8, device="cuda")
    s = t.empty((700, K // 128), dtype=t.float32, device="cuda")
    c = t.zeros((700, N), dtype=t.bfloat16, device="cuda")

    def capture():
        B.fp8_quant_act_1x128(x, q, s)
        B.fp8_block_grouped_gemm(q, s, qw, sw, off, out_dtype="bf16", c=c)
        return q, s, c

    def eager():
        q2, s2 = B.fp8_quant_act_1x128(x)
        c2 = t.zeros_like(c)
        B.fp8_block_grouped_gemm(q2, s2, qw, sw, off, out_dtype="bf16", c=c2)
        return q2, s2, c2

    replay_and_check(capture, eager, x, fresh, "quant + grouped GEMM, 6 experts")


def test_graph_quant_and_noalloc_split_k_gemm():
    # the no-allocation GEMM is meant for capture: 64 x 2048 x 7168 splits K
    # through the library's static scratch array; every replay equals the
    # eager chain through the workspace GEMM (same plan, same order)
    t = torch()
    M, N, K = 64, 2048, 7168
    x = activations(5, M, K)
    fresh = [activations(40 + r, M, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(6), (N, K))))
    assert B.fp8_gemm_workspace_bytes(M, N, K, "bf16") > 0
    q = t.empty((M, K), dtype=t.uint8, device="cuda")
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    c = t.empty((M, N), dtype=t.bfloat16, device="cuda")

    def capture():
        B.fp8_quant_act_1x128(x, q, s)
        B.fp8_block_gemm_noalloc(q, s, qw, sw, out_dtype="bf16", c=c)
        return q, s, c

    def eager():
        q2, s2 = B.fp8_quant_act_1x128(x)
        ws = t.empty(B.fp8_gemm_workspace_bytes(M, N, K, "bf16"), dtype=t.uint8, device="cuda")
        return q2, s2, B.fp8_block_gemm(q2, s2, qw, sw, out_dtype="bf16", workspace=ws)

    replay_and_check(capture, eager, x, fresh, "quant + no-allocation split-K GEMM 64x2048x7168")


def test_graph_fused_quant_gemm():
    # the quantization fused into the GEMM, with its quantized outputs
    t = torch()
    M, N, K = 96, 512, 1280
    x = activations(7, M, K)
    fresh = [activations(50 + r, M, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(8), (N, K))))
    q = t.empty((M, K), dtype=t.uint8, device="cuda")
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    c = t.empty((M, N), dtype=t.float32, device="cuda")

    def capture():
        B.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32", c=c, q_out=q, sa_out=s)
        return q, s, c

    def eager():
        c2, q2, s2 = B.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32",
                                                   return_quantized=True)
        return q2, s2, c2

    replay_and_check(capture, eager, x, fresh, "fused quantization + GEMM 96x512x1280 f32")


def test_graph_fused_entry_staged_plan():
    # the same entry point with the workspace it asks for: at 96 tokens it
    # takes the staged plan, i.e. the quantizer and the split-K block GEMM
    # (partials in the same workspace); with and without quantized outputs
    t = torch()
    M, N, K = 96, 512, 1280
    x = activations(9, M, K)
    fresh = [activations(60 + r, M, K) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(10), (N, K))))
    nb = B.fp8_fused_quant_workspace_bytes(M, N, K, "f32")
    assert nb > M * K + M * (K // 128) * 4 and B.fp8_gemm_workspace_bytes(M, N, K, "f32") > 0
    ws = t.empty(nb, dtype=t.uint8, device="cuda")
    q = t.empty((M, K), dtype=t.uint8, device="cuda")
    s = t.empty((M, K // 128), dtype=t.float32, device="cuda")
    c = t.empty((M, N), dtype=t.float32, device="cuda")
    c0 = t.empty((M, N), dtype=t.float32, device="cuda")

    def capture():
        B.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32", c=c, q_out=q, sa_out=s,
                                     workspace=ws)
        B.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32", c=c0, workspace=ws)
        return q, s, c, c0

    def eager():
        qa, sa = B.fp8_quant_act_1x128(x)
        gws = t.empty(B.fp8_gemm_workspace_bytes(M, N, K, "f32"), dtype=t.uint8, device="cuda")
        c2 = B.fp8_block_gemm(qa, sa, qw, sw, out_dtype="f32", workspace=gws)
        return qa, sa, c2, c2

    replay_and_check(capture, eager, x, fresh, "fused entry, staged plan 96x512x1280 f32")


def test_graph_dgrad_transposed_split_k():
    # Dgrad on the forward weights (read transposed), small M: split-K
    # through the workspace
    t = torch()
    M, N, Kx = 64, 1024, 2048  # dY [M][N], W [N][Kx], dX [M][Kx]
    dy = activations(9, M, N)
    fresh = [activations(60 + r, M, N) for r in range(REPLAYS)]
    qw, sw = B.fp8_quant_weight_128x128(dev_bf16(I.weights(np.random.default_rng(10), (N, Kx))))
    q = t.empty((M, N), dtype=t.uint8, device="cuda")
    s = t.empty((M, N // 128), dtype=t.float32, device="cuda")
    dx = t.empty((M, Kx), dtype=t.float32, device="cuda")
    nbytes = B.fp8_gemm_workspace_bytes(M, Kx, N, "f32")
    ws = t.empty(max(nbytes, 256), dtype=t.uint8, device="cuda") if nbytes else None

    def capture():
        B.fp8_quant_act_1x128(dy, q, s)
        B.fp8_block_gemm_dgrad(q, s, qw, sw, out_dtype="f32", dx=dx, workspace=ws)
        return q, s, dx

    def eager():
        q2, s2 = B.fp8_quant_act_1x128(dy)
        ws2 = t.empty_like(ws) if ws is not None else None
        return q2, s2, B.fp8_block_gemm_dgrad(q2, s2, qw, sw, out_dtype="f32", workspace=ws2)

    replay_and_check(capture, eager, dy, fresh, "quant + Dgrad (W read transposed) 64x2048 over 1024")
