"""fp8_block_gemm_noalloc against fp8_block_gemm (GPU, through the C ABI).

The no-allocation variant keeps its split-K partial sums in the library's
static device scratch array instead of a caller workspace.  With the same
split plan it must give bitwise the same C as fp8_block_gemm with a
workspace of fp8_gemm_workspace_bytes().  Two calls in a row, the second on
a smaller input (the array keeps the first call's partials: nothing of them
may leak into the second), then the first shape again; a shape without
split-K; and the smaller call checked against the oracle within its
per-output bound.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B
from fp8_fine_grained_token_amd import inputs as I

from .gpu_util import check_gemm, dev, gemm_error_bound, log, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    yield
    t.cuda.synchronize()


def operands(M, N, K, seed):
    g = I.gemm_inputs(M, N, K, seed=seed, outlier_frac=0.01, outlier_mult=20.0)
    qa, sa = oracle.quant_act_1x128(g.a_bf16)
    qw, sw = oracle.quant_weight_128x128(g.w_bf16)
    return qa, sa, qw, sw


def with_workspace(d, out):
    t = torch()
    M, K = d[0].shape
    N = d[2].shape[0]
    nbytes = B.fp8_gemm_workspace_bytes(M, N, K, out)
    ws = t.empty(nbytes, dtype=t.uint8, device="cuda") if nbytes else None
    return B.fp8_block_gemm(*d, out_dtype=out, workspace=ws), nbytes


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_noalloc_equals_workspace_gemm_on_two_calls_second_smaller(out):
    t = torch()
    big = (256, 2048, 7168)     # the decode shape: 4 splits, 8 MiB of partials
    small = (96, 512, 2688)     # fewer, smaller partials in the same array
    ops_big = operands(*big, seed=11)
    ops_small = operands(*small, seed=12)
    d_big = [dev(x) for x in ops_big]
    d_small = [dev(x) for x in ops_small]
    ref_big, nb_big = with_workspace(d_big, out)
    ref_small, nb_small = with_workspace(d_small, out)
    assert nb_big > nb_small > 0, (nb_big, nb_small)
    log(f"  {out}: split-K partials {nb_big} B then {nb_small} B")
    c1 = B.fp8_block_gemm_noalloc(*d_big, out_dtype=out)
    c2 = B.fp8_block_gemm_noalloc(*d_small, out_dtype=out)
    c3 = B.fp8_block_gemm_noalloc(*d_big, out_dtype=out)
    t.cuda.synchronize()
    assert t.equal(c1, ref_big), "first call differs from fp8_block_gemm"
    assert t.equal(c2, ref_small), "second (smaller) call differs from fp8_block_gemm"
    assert t.equal(c3, ref_big), "third call differs from fp8_block_gemm"
    qa, sa, qw, sw = ops_small
    R = oracle.block_gemm(qa, sa, qw, sw)
    check_gemm(c2, R, out, "noalloc small", gemm_error_bound(qa, sa, qw, sw,
                                                              splits=nb_small // (96 * 512 * 4)))


def test_noalloc_without_split_k_and_on_a_side_stream():
    # 4096 x 1024 x 512 fills the GPU without splitting K (no scratch used);
    # the decode shape on a non-default stream uses the scratch array
    t = torch()
    d = [dev(x) for x in operands(4096, 1024, 512, seed=13)]
    ref, nbytes = with_workspace(d, "bf16")
    assert nbytes == 0
    assert t.equal(B.fp8_block_gemm_noalloc(*d, out_dtype="bf16"), ref)
    d2 = [dev(x) for x in operands(256, 2048, 7168, seed=14)]
    ref2, _ = with_workspace(d2, "f32")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        c = B.fp8_block_gemm_noalloc(*d2, out_dtype="f32", stream=s)
    s.synchronize()
    assert t.equal(c, ref2)
