"""Algorithmic HBM bytes and FLOPs of one delta step, for roofline reporting.

What the method itself must move ("m07 -- Multi-Adapter (LoRA) Serving",
"6. Deep Dive A", "The cost is bandwidth, not compute": the base weights are
read once per step and each distinct adapter once): every distinct adapter
present in the batch read once at its own rank, every activation tensor read
once, and y read once and written once.  The rank-r intermediate stays on chip
and is not counted.  Split by kernel: the shrink moves A and x, the expand
moves B and y.
"""
from __future__ import annotations

import numpy as np


def step_traffic(ids, num_slots, modules, ranks, fmt=None) -> dict:
    """ids: int [rows] (negative = base only, >= num_slots = skipped);
    modules: [(name, table column, d_in, d_out, x tensor name)];
    ranks: int [num_slots, columns]; fmt: int [num_slots, columns], 1 where
    the factors are int8 with one fp32 scale per row (one byte per value
    plus the scales), else bf16 (two bytes per value)."""
    ids = np.asarray(ids)
    valid = (ids >= 0) & (ids < num_slots)
    slots, counts = np.unique(ids[valid], return_counts=True)
    a_bytes = b_bytes = y_bytes = flops = 0
    x_rows = {}
    for name, col, d_in, d_out, x_name in modules:
        r = np.asarray(ranks)[slots, col].astype(np.int64)
        on = r > 0
        q8 = (np.asarray(fmt)[slots, col] == 1) if fmt is not None else np.zeros(r.shape, bool)
        w = np.where(q8, 1, 2)
        a_bytes += int((w * r * d_in)[on].sum() + 4 * r[on & q8].sum())
        b_bytes += int((w * r * d_out)[on].sum() + 4 * d_out * int((on & q8).sum()))
        rows = int(counts[on].sum())
        y_bytes += 4 * rows * d_out
        flops += int((counts[on] * 2 * r[on] * (d_in + d_out)).sum())
        x_rows[x_name] = (max(rows, x_rows.get(x_name, (0, 0))[0]), d_in)
    x_bytes = sum(2 * n * d for n, d in x_rows.values())
    return {"adapters": a_bytes + b_bytes, "x": x_bytes, "y": y_bytes,
            "total": a_bytes + b_bytes + x_bytes + y_bytes,
            "shrink_bytes": a_bytes + x_bytes, "expand_bytes": b_bytes + y_bytes, "flops": flops}
