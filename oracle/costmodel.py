"""The pages' analytic size, FLOP and byte accounting -- TEST INFRASTRUCTURE ONLY.

Pinned in ``tests/test_costmodel.py`` against every figure the pages print for
this path (``tests/golden/pages_figures.json``).

Sources:
* "m07 -- Multi-Adapter (LoRA) Serving", "2. Scale Numbers": a LoRA on a
  weight of shape (d_out, d_in) has r * (d_in + d_out) parameters; the 70B
  model has 80 layers, hidden size 8192, GQA kv-dim 1024 and FFN 28672; in a
  decode step the base weights are read once while every distinct adapter in
  the batch is read once; extra bytes are quoted as a share of the base read
  (140 GB of bf16 weights, from the page's introduction).
* same page, "6. Deep Dive A": base FLOPs per token per projection
  2 * d_in * d_out, LoRA FLOPs 2 * r * (d_in + d_out).
* "12. Adapter Serving and Multi-Tenant Customization", "What an adapter adds
  to a forward pass": that page sizes all four attention projections as
  [d, d] (its own convention, used only where its figures are checked).
"""
from __future__ import annotations

BF16_BYTES = 2

# 70B shapes ("2. Scale Numbers"): (d_in, d_out) of W for each projection.
LAYERS_70B = 80
D_MODEL = 8192
KV_DIM = 1024
FFN_DIM = 28672
BASE_BYTES_70B = 140e9  # "140 GB of base weights"

SHAPES_70B = {
    "q": (D_MODEL, D_MODEL),
    "k": (D_MODEL, KV_DIM),
    "v": (D_MODEL, KV_DIM),
    "o": (D_MODEL, D_MODEL),
    "gate": (D_MODEL, FFN_DIM),
    "up": (D_MODEL, FFN_DIM),
    "down": (FFN_DIM, D_MODEL),
}
ATTENTION = ("q", "k", "v", "o")
ALL_MODULES = ("q", "k", "v", "o", "gate", "up", "down")


def lora_params(rank: int, d_in: int, d_out: int) -> int:
    """Parameters of one adapted projection: A (r, d_in) plus B (d_out, r)."""
    return rank * (d_in + d_out)


def adapter_params_per_layer(rank: int, modules=ATTENTION, shapes=SHAPES_70B) -> int:
    return sum(lora_params(rank, *shapes[m]) for m in modules)


def adapter_bytes(rank: int, modules=ATTENTION, layers=LAYERS_70B, shapes=SHAPES_70B) -> int:
    """bf16 bytes of one adapter over the whole model."""
    return BF16_BYTES * layers * adapter_params_per_layer(rank, modules, shapes)


def extra_decode_bytes_fraction(rank: int, modules, distinct_adapters: int,
                                base_bytes: float = BASE_BYTES_70B) -> float:
    """Extra bytes read per decode step as a fraction of the base weight read.

    The base weights are read once per step; each distinct adapter in the
    batch is read once.
    """
    return distinct_adapters * adapter_bytes(rank, modules) / base_bytes


def base_flops_per_token(d_in: int, d_out: int) -> int:
    return 2 * d_in * d_out


def lora_flops_per_token(rank: int, d_in: int, d_out: int) -> int:
    """Shrink (2 r d_in) plus expand (2 r d_out)."""
    return 2 * rank * (d_in + d_out)


# The d x d convention of "12. Adapter Serving ...", "What an adapter adds".
SHAPES_DXD = {m: (D_MODEL, D_MODEL) for m in ATTENTION}


def pair_bytes(rank: int, d: int = D_MODEL) -> int:
    """Bytes of one A, B pair for a d x d projection in bf16."""
    return 2 * d * rank * BF16_BYTES


# ---------------------------------------------------------------------------
# Algorithmic bytes and FLOPs of one delta pass over a concrete batch: what
# the method itself must move.  Each distinct adapter present is read once at
# its own rank (the byte model above), each distinct input tensor is read
# once, and y is read once and written once.  v never leaves the chip.

def algorithmic_bytes(ids, modules, rank_of, x_groups) -> dict:
    """ids: row -> slot (negative = base only); modules: list of
    (name, d_in, d_out, x_name); rank_of(slot, name) -> rank; x_groups: set of
    input tensor names.  Returns a dict with adapters / x / y / total bytes
    and flops, counting only rows whose slot has rank > 0 for that module.
    """
    import numpy as np
    ids = np.asarray(ids)
    valid_rows = ids >= 0
    distinct = sorted(set(int(a) for a in ids[valid_rows]))
    adapters = 0
    y_bytes = 0
    flops = 0
    x_rows = {}
    for name, d_in, d_out, x_name in modules:
        rows_m = 0
        for a in distinct:
            r = rank_of(a, name)
            if r <= 0:
                continue
            adapters += BF16_BYTES * lora_params(r, d_in, d_out)
            cnt = int(np.count_nonzero(ids == a))
            rows_m += cnt
            flops += cnt * lora_flops_per_token(r, d_in, d_out)
        y_bytes += 2 * BF16_BYTES * rows_m * d_out
        prev = x_rows.get(x_name, (0, d_in))[0]
        x_rows[x_name] = (max(prev, rows_m), d_in)
    x_bytes = sum(BF16_BYTES * r * d for (r, d) in x_rows.values())
    return {"adapters": adapters, "x": x_bytes, "y": y_bytes,
            "total": adapters + x_bytes + y_bytes, "flops": flops}
