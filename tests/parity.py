"""Helpers of the GPU parity tests (no test functions here).

Tolerance: every element must satisfy |gpu - oracle| <= 1e-2 * max|oracle row|
+ 1e-3, where the row is that row of the tensor being compared (v, the delta
alone, or y).  Integers (segments) compare bit-exactly.
"""
from __future__ import annotations

import sys

import numpy as np

REL, ABS = 1e-2, 1e-3

# every comparison's strict relative figure, max |gpu - oracle| / max |oracle
# row| over its rows: reported at the end of the session (tests/conftest.py),
# not part of the bar
STRICT: list = []


def note(msg: str):
    """Name the GPU case about to run (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def check_rows(gpu, ref, what: str, rel=REL, abs_=ABS):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    tol = rel * np.abs(ref).max(axis=1, keepdims=True) + abs_
    err = np.abs(gpu - ref)
    bad = np.argwhere(~(err <= tol))
    if bad.size:
        r, c = bad[0]
        raise AssertionError(f"{what}: {len(bad)} elements out of tolerance; first at row {r} col {c}: "
                             f"gpu={gpu[r, c]!r} oracle={ref[r, c]!r} tol={tol[r, 0]!r}")
    # strict relative figure (reported, not part of the bar)
    scale = np.maximum(np.abs(ref).max(axis=1, keepdims=True), 1e-300)
    strict = float((err / scale).max())
    STRICT.append((what, strict, int(ref.shape[0])))
    return strict


def bf16_host(t):
    """GPU bf16 tensor -> float64 numpy array."""
    from workloads import bf16_to_f32
    from workloads.device import to_bits
    return bf16_to_f32(to_bits(t)).astype(np.float64)
