"""Pins of the oracle's base projection and fused result, y = W.x + delta
("m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": y = Wx + (BA)x(alpha/r))."""
from fractions import Fraction

import numpy as np

import oracle
from workloads import bf16_bits, bf16_to_f32
from workloads import build_workload_for_tests as bw
from workloads.gen import add_base_weights


def small(seed=3, rows=6, d_in=24, d_out=16, rank=4, slots=3):
    ids = np.random.default_rng(seed).integers(-1, slots, size=rows)
    return add_base_weights(bw(seed, rows, slots, d_in, d_out, rank, ids, x_std=1.0))


def test_one_hot_base_weights_gather_x_exactly():
    # W[n, k_n] = 1: (W.x)[b, n] = x[b, k_n]; a transposed W or a wrong index fails
    w = small(rows=5, d_in=40, d_out=24)
    ks = np.random.default_rng(1).integers(0, 40, size=24)
    W = np.zeros((24, 40), np.uint16)
    W[np.arange(24), ks] = 0x3F80
    got = oracle.base_projection(W, w.x["x"])
    want = bf16_to_f32(w.x["x"]).astype(np.float64)[:, ks]
    assert np.array_equal(got, want)


def test_base_projection_exact_rational():
    w = small(rows=3, d_in=16, d_out=8)
    W = w.W["q"]
    got = oracle.base_projection(W, w.x["x"])
    Wf = bf16_to_f32(W)
    xf = bf16_to_f32(w.x["x"])
    for b in range(3):
        for n in range(8):
            exact = sum(Fraction(float(Wf[n, k])) * Fraction(float(xf[b, k])) for k in range(16))
            assert abs(got[b, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_zero_base_gives_the_delta_and_rows_select():
    w = small()
    w.W["q"][:] = 0
    r = oracle.linear_layer(w)["q"]
    assert np.array_equal(r.y, r.delta)
    add_base_weights(w)
    full = oracle.linear_layer(w)["q"]
    rows = np.array([4, 0, 2])
    part = oracle.linear_layer(w, rows=rows)["q"]
    assert np.array_equal(part.y, full.y[rows])
    # the base term is there: y differs from the delta alone
    assert np.abs(full.y - full.delta).max() > 0.1


def test_base_weights_have_unit_output_scale():
    w = small(rows=64, d_in=2048, d_out=64)
    base = oracle.base_projection(w.W["q"], w.x["x"])
    assert 0.8 < base.std() < 1.2
    assert bf16_bits(np.float32(1.0)) == 0x3F80
