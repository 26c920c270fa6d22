"""GEMM cases run once with the released library and once with the
race-check build (FP8BLK_LIB = _build/libfp8blk_poison.so, where every
LDS-DMA copy first poisons the bytes it will write); see
tests/test_poison_lds_gpu.py.  Each case covers one tile kind and pipeline
of the kernels; inputs are seeded, so both runs see the same bytes.

Run as a script (python tests/poison_cases.py OUT.npz) it computes every case
with whatever library FP8BLK_LIB names and saves the outputs.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run_cases():
    import torch
    import fp8_fine_grained_token_amd as F
    from fp8_fine_grained_token_amd import inputs as I

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).cuda()

    def act(seed, m, k):
        return bf(I.activations(np.random.default_rng(seed), m, k, 0.01, 50.0)[0])

    def wts(seed, n, k):
        return bf(I.weights(np.random.default_rng(seed), (n, k)))

    def ws_for(m, n, k):
        nb = F.fp8_gemm_workspace_bytes(m, n, k, "f32")
        return torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None

    out = {}

    def keep(name, t):
        torch.cuda.synchronize()
        out[name] = t.contiguous().view(torch.uint8).cpu().numpy().copy()

    # dense: two tile widths (4096 x 7168), one 256 x 256 round, small
    # tiles unsplit (G = 10: a partial scale chunk) and split-K
    for name, (m, n, k), split in [("dense_two_kind", (4096, 7168, 512), False),
                                   ("dense_big", (4096, 4096, 1024), False),
                                   ("dense_small", (200, 384, 1280), False),
                                   ("dense_split_k", (64, 1024, 7168), True)]:
        qa, sa = F.fp8_quant_act_1x128(act(1, m, k))
        qw, sw = F.fp8_quant_weight_128x128(wts(2, n, k))
        c = F.fp8_block_gemm(qa, sa, qw, sw, out_dtype="f32",
                             workspace=ws_for(m, n, k) if split else None)
        keep(name, c)
        if name == "dense_two_kind":
            pa, psa = F.fp8_quant_act_1x128_pow2(act(1, m, k))
            pw, psw = F.fp8_quant_weight_128x128_pow2(wts(2, n, k))
            keep("pow2_dense_two_kind", F.fp8_block_gemm_pow2(pa, psa, pw, psw, out_dtype="f32"))
    # no-allocation split-K
    qa, sa = F.fp8_quant_act_1x128(act(3, 64, 7168))
    qw, sw = F.fp8_quant_weight_128x128(wts(4, 2048, 7168))
    keep("noalloc_split_k", F.fp8_block_gemm_noalloc(qa, sa, qw, sw, out_dtype="f32"))
    # grouped: ragged experts, an empty one, G = 18 (partial scale chunk)
    counts = [300, 0, 129, 1, 257, 70]
    gi = I.grouped_inputs(len(counts), sum(counts), 512, 2304, seed=5, counts=counts)
    E, N, K = gi.w_bf16.shape
    off = torch.from_numpy(gi.offsets.astype(np.int32)).cuda()
    for pow2 in (False, True):
        qf = F.fp8_quant_act_1x128_pow2 if pow2 else F.fp8_quant_act_1x128
        wf = F.fp8_quant_weight_128x128_pow2 if pow2 else F.fp8_quant_weight_128x128
        gf = F.fp8_block_grouped_gemm_pow2 if pow2 else F.fp8_block_grouped_gemm
        ga, gsa = qf(bf(gi.a_bf16))
        gw, gsw = wf(bf(gi.w_bf16.reshape(E * N, K)))
        c = torch.zeros((gi.T, N), dtype=torch.float32, device="cuda")
        gf(ga, gsa, gw.view(E, N, K), gsw.view(E, N // 128, K // 128), off, out_dtype="f32", c=c)
        keep("grouped_pow2" if pow2 else "grouped", c)
    # fused quantization (with its quantized outputs)
    x = act(6, 300, 1280)
    qw, sw = F.fp8_quant_weight_128x128(wts(7, 512, 1280))
    c, q, s = F.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32", return_quantized=True)
    keep("fused", c)
    keep("fused_q", q)
    keep("fused_s", s)
    # ... and with its split-K workspace (4 splits of 1024 x 256 x 2304)
    x = act(12, 1024, 2304)
    qw, sw = F.fp8_quant_weight_128x128(wts(13, 256, 2304))
    nf = F.fp8_fused_quant_kernel_workspace_bytes(1024, 256, 2304, "f32")
    assert nf > 0
    fws = torch.empty(nf, dtype=torch.uint8, device="cuda")
    c, q, s = F.fp8_block_gemm_fused_quant(x, qw, sw, out_dtype="f32", return_quantized=True,
                                           workspace=fws)
    keep("fused_split_k", c)
    keep("fused_split_k_q", q)
    # Dgrad on the forward weights: two tile widths, and split-K for small M
    for name, (m, n, kx), split in [("dgrad_two_kind", (4096, 512, 7168), False),
                                    ("dgrad_split_k", (64, 1024, 2048), True)]:
        qd, sd = F.fp8_quant_act_1x128(act(8, m, n))
        qw, sw = F.fp8_quant_weight_128x128(wts(9, n, kx))
        keep(name, F.fp8_block_gemm_dgrad(qd, sd, qw, sw, out_dtype="f32",
                                          workspace=ws_for(m, kx, n) if split else None))
    # pow2 Dgrad reading W transposed, two widths
    qd, sd = F.fp8_quant_act_1x128_pow2(act(14, 4096, 384))
    qw, sw = F.fp8_quant_weight_128x128_pow2(wts(15, 384, 7168))
    keep("dgrad_pow2_two_kind", F.fp8_block_gemm_dgrad_pow2(qd, sd, qw, sw, out_dtype="f32"))
    # Wgrad: the two-width plan of dW 7168 x 7168 (over 256 tokens) and a
    # single-width one
    for name, (n, k, t) in [("wgrad_two_kind", (7168, 7168, 256)), ("wgrad_small", (512, 384, 384))]:
        qy, sy = F.fp8_quant_act_128x1_t(act(10, t, n))
        qx, sx = F.fp8_quant_act_128x1_t(act(11, t, k))
        keep(name, F.fp8_block_gemm_wgrad(qy, sy, qx, sx, out_dtype="f32"))
    # pow2 Wgrad (two-stage 256-row tiles): both widths with ragged last
    # tiles (dW 4100 x 6016 over 640 tokens: 5 K blocks, a partial scale
    # chunk), and one width
    for name, (n, k, t) in [("wgrad_pow2_two_kind", (4100, 6016, 640)),
                            ("wgrad_pow2_small", (520, 896, 256))]:
        qy, sy = F.fp8_quant_act_128x1_t_pow2(act(12, t, n))
        qx, sx = F.fp8_quant_act_128x1_t_pow2(act(13, t, k))
        keep(name + "_q", qy)
        keep(name, F.fp8_block_gemm_wgrad_pow2(qy, sy, qx, sx, out_dtype="f32"))
    return out


if __name__ == "__main__":
    res = run_cases()
    np.savez(sys.argv[1], **res)
    print("cases done:", ", ".join(sorted(res)), flush=True)
