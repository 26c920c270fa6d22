"""Exhaustive GPU quantizer sweep against the oracle.

Every positive finite bf16 amax (32639 values) is paired with every bf16 x of
magnitude <= amax, both signs: about 1.07e9 (x, amax) pairs packed as groups
of 128 (the amax element, alternately +amax and -amax, then 127 values of x),
so the whole input space of one 1x128 group's quantization is covered.  The
GPU bytes and scale bits must equal the oracle's.  This proves the GPU's
quotient (reciprocal plus one FMA correction for amax >= 2^-60, IEEE divide
below), its clamp and the hardware E4M3 conversion on every input they can
see.
"""
import numpy as np
import pytest

import oracle
from fp8_fine_grained_token_amd import binding as B

from .gpu_util import dev_bf16, host, log, torch

pytestmark = pytest.mark.gpu

AMAX_HI = 0x7F80          # exclusive: +inf bits
N_CHUNKS = 8


def sweep_rows(a0: int, a1: int) -> np.ndarray:
    """Groups for amax bit patterns [a0, a1): row = [+-amax, 127 x values]."""
    amax = np.arange(a0, a1, dtype=np.int64)
    nvals = 2 * (amax + 1)                     # magnitudes 0..amax, both signs
    nrows = (nvals + 126) // 127
    total = int(nrows.sum())
    rows = np.zeros((total, 128), dtype=np.uint16)
    row_amax = np.repeat(amax, nrows)
    first_row = np.concatenate([[0], np.cumsum(nrows)[:-1]])
    # alternate the sign of the amax element by row
    sign_bit = ((np.arange(total) & 1).astype(np.uint16) << np.uint16(15))
    rows[:, 0] = row_amax.astype(np.uint16) | sign_bit
    # value stream per amax: magnitudes 0..amax then the same with the sign bit
    val_amax = np.repeat(amax, nvals)
    start = np.repeat(np.concatenate([[0], np.cumsum(nvals)[:-1]]), nvals)
    pos = np.arange(int(nvals.sum()), dtype=np.int64) - start
    mag = pos % (val_amax + 1)
    neg = pos > val_amax
    vals = (mag.astype(np.uint16)) | (neg.astype(np.uint16) << np.uint16(15))
    r = np.repeat(first_row, nvals) + pos // 127
    c = 1 + pos % 127
    rows[r, c] = vals
    return rows


def chunk_bounds():
    # split the amax range so each chunk holds about the same number of pairs
    a = np.arange(1, AMAX_HI, dtype=np.float64)
    cum = np.cumsum(2 * (a + 1))
    cuts = [1] + [int(1 + np.searchsorted(cum, cum[-1] * i / N_CHUNKS)) for i in
                  range(1, N_CHUNKS)] + [AMAX_HI]
    return list(zip(cuts[:-1], cuts[1:]))


@pytest.mark.parametrize("chunk", range(N_CHUNKS))
def test_exhaustive_bf16_sweep(chunk):
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    a0, a1 = chunk_bounds()[chunk]
    x = sweep_rows(a0, a1)
    log(f"  sweep chunk {chunk}: amax bits [{a0:#x}, {a1:#x}), {x.shape[0]} groups")
    qo, so = oracle.quant_act_1x128(x)
    q, s = B.fp8_quant_act_1x128(dev_bf16(x))
    qg, sg = host(q), host(s)
    bad = np.argwhere(qg != qo)
    sbad = int((sg.view(np.uint32) != so.view(np.uint32)).sum())
    if bad.size:
        i, j = bad[0]
        log(f"  first mismatch: group {i} amax bits {x[i, 0]:#06x} x bits {x[i, j]:#06x} "
            f"gpu {qg[i, j]:#04x} oracle {qo[i, j]:#04x}; total {bad.shape[0]}")
    assert bad.shape[0] == 0 and sbad == 0


def test_sweep_packing_covers_every_pair():
    # CPU-side check of the packing on a small amax range (no GPU needed, but
    # kept beside the sweep it describes).
    x = sweep_rows(1, 40)
    pairs = set()
    for row in x:
        a = int(row[0]) & 0x7FFF
        for v in row[1:]:
            pairs.add((a, int(v)))
    for a in range(1, 40):
        for m in range(a + 1):
            assert (a, m) in pairs and (a, m | 0x8000) in pairs
