"""Pins of the oracle's multi-adapter composition ("m07 -- Multi-Adapter
(LoRA) Serving", "9. Bottlenecks and Evolution", item 5: two adapters on one
request).

Closed form: two adapters stacked on a row equal one adapter of rank r1 + r2
whose A is A1 over A2 and whose B is [s1 B1 | s2 B2] (with power-of-two
scales, s B is exact in bf16), computed by the single-adapter oracle.
"""
import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32
from workloads import build_workload_for_tests as bw


def stacked_and_concat(seed, rows, d_in, d_out, r1, r2, n1, n2):
    rng = np.random.default_rng(seed)
    slots = n1 + n2
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:n1, 0] = r1
    ranks[n1:, 0] = r2
    scales = np.zeros((slots, 7), np.float32)
    scales[:, 0] = 2.0 ** rng.integers(-2, 3, size=slots)
    ra = np.stack([rng.integers(0, n1, size=rows), n1 + rng.integers(0, n2, size=rows)], 1).astype(np.int32)
    w = bw(seed, rows, slots, d_in, d_out, None, ra[:, 0], ranks=ranks, scales=scales, x_std=1.0)
    # one concatenated adapter per (a1, a2) pair that occurs
    pairs = sorted({(int(a), int(b)) for a, b in ra})
    idx = {p: k for k, p in enumerate(pairs)}
    cranks = np.zeros((len(pairs), 7), np.int32)
    cranks[:, 0] = r1 + r2

    def fill(wc):
        for (a1, a2), k in idx.items():
            A, B = wc.A(k, 0), wc.B(k, 0)
            A[:r1] = w.A(a1, 0)
            A[r1:] = w.A(a2, 0)
            B[:, :r1] = bf16_bits(scales[a1, 0] * bf16_to_f32(w.B(a1, 0)))
            B[:, r1:] = bf16_bits(scales[a2, 0] * bf16_to_f32(w.B(a2, 0)))
    cid = np.array([idx[(int(a), int(b))] for a, b in ra], np.int32)
    wc = bw(seed, rows, len(pairs), d_in, d_out, None, cid, ranks=cranks, ab_fill=fill, x_std=1.0,
            max_rank=r1 + r2)
    assert np.array_equal(wc.x["x"], w.x["x"]) and np.array_equal(wc.y0["q"], w.y0["q"])
    return w, ra, wc


@pytest.mark.parametrize("r1,r2", [(8, 16), (5, 3), (16, 40)])
def test_two_stacked_adapters_equal_their_concatenation(r1, r2):
    w, ra, wc = stacked_and_concat(40 + r1, 24, 96, 40, r1, r2, 3, 4)
    s = oracle.lora_layer_stacked(w, ra)["q"]
    c = oracle.lora_layer(wc)["q"]
    scale = np.abs(c.delta).max()
    assert scale > 0
    assert np.abs(s.delta - c.delta).max() <= 1e-12 * scale
    assert np.abs(s.y - c.y).max() <= 1e-12 * np.abs(c.y).max()


def test_padding_entries_add_nothing_and_order_does_not_matter():
    w, ra, _ = stacked_and_concat(7, 20, 64, 24, 8, 8, 3, 3)
    single = oracle.lora_layer(w)["q"]                     # column 0 alone
    padded = oracle.lora_layer_stacked(w, np.stack([ra[:, 0], -np.ones(20, np.int32)], 1))["q"]
    assert np.array_equal(padded.delta, single.delta) and np.array_equal(padded.y, single.y)
    ab = oracle.lora_layer_stacked(w, ra)["q"]
    ba = oracle.lora_layer_stacked(w, ra[:, ::-1].copy())["q"]
    assert np.array_equal(ab.delta, ba.delta)


def test_same_adapter_twice_doubles_the_delta():
    w, ra, _ = stacked_and_concat(9, 16, 64, 24, 8, 8, 2, 2)
    single = oracle.lora_layer(w)["q"]
    twice = oracle.lora_layer_stacked(w, np.stack([ra[:, 0], ra[:, 0]], 1))["q"]
    assert np.array_equal(twice.delta, 2 * single.delta)
