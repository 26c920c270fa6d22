"""Host logic of the benchmark's shader-clock probe (no GPU).

The probe launches record (compute unit, shader-clock count, real-time
count) per workgroup.  The counters of different compute units are not
aligned with each other, so the clock must come from matching the two
launches unit by unit; these records give units arbitrary counter offsets
and one XCD a lower clock, and check that the per-unit matching recovers
the clocks exactly.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import bench  # noqa: E402


def _probe_with(records):
    p = bench.GpuClockProbe.__new__(bench.GpuClockProbe)
    p.torch, p.error, p.lib = torch, None, object()
    p.bufs = [torch.tensor(np.asarray(r, dtype=np.int64).reshape(-1)) for r in records]
    return p


def _units():
    return [(x << 8) | (se << 5) | (sh << 4) | cu
            for x in range(8) for se in range(4) for sh in range(2) for cu in range(4)]


def _launch(rng, units, offset, mhz, r0, n=4096):
    rows = []
    for i in range(n):
        u = units[i % len(units)] if i < len(units) else units[rng.integers(len(units))]
        r = r0 + int(rng.integers(0, 100))          # workgroups start within 1 us
        rows.append((u, offset[u] + int(mhz[u] * 1e6 * r / 100e6), r))
    return rows


def test_clock_matched_per_compute_unit():
    rng = np.random.default_rng(1)
    units = _units()
    offset = {u: int(rng.integers(0, 1 << 40)) for u in units}   # unaligned counters
    mhz = {u: (1800.0 if u >> 8 == 3 else 2100.0) for u in units}
    before = _launch(rng, units, offset, mhz, 10 ** 9)
    after = _launch(rng, units, offset, mhz, 10 ** 9 + 500_000)   # 5 ms later
    res = _probe_with([before, after]).result()
    assert res["compute_units_matched"] == 256
    med = res["per_xcd_median_mhz"]
    assert len(med) == 8
    assert med[3] == pytest.approx(1800.0, rel=1e-3)
    assert all(m == pytest.approx(2100.0, rel=1e-3) for i, m in enumerate(med) if i != 3)
    assert res["mhz_mean"] == pytest.approx((7 * 2100.0 + 1800.0) / 8, rel=1e-3)  # one XCD in 8


def test_clock_ignores_units_seen_once():
    rng = np.random.default_rng(2)
    units = _units()
    offset = {u: int(rng.integers(0, 1 << 40)) for u in units}
    mhz = {u: 2000.0 for u in units}
    before = _launch(rng, units[:200], offset, mhz, 10 ** 9, n=1000)
    after = _launch(rng, units[100:], offset, mhz, 10 ** 9 + 100_000, n=1000)
    res = _probe_with([before, after]).result()
    assert res["compute_units_matched"] == 100
    assert res["mhz_p10"] == pytest.approx(2000.0, rel=1e-3)
    assert res["mhz_p90"] == pytest.approx(2000.0, rel=1e-3)


def test_clock_reports_missing_probe():
    p = _probe_with([[(0, 1, 1)], [(0, 2, 2)]])
    p.lib, p.error = None, "OSError: not built"
    assert p.result() == {"mhz_mean": None, "error": "OSError: not built"}
