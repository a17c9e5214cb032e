"""Pins of the oracle's base projection and fused result, y = W.x + delta
("m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A": y = Wx + (BA)x(alpha/r))."""
from fractions import Fraction

import numpy as np

import oracle
from workloads import bf16_bits, bf16_to_f32
from workloads import build_workload_for_tests as bw
from workloads.gen import Q4Weight, add_base_weights


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


# ---- 4-bit base weights ("12. Adapter Serving and Multi-Tenant Customization",
# "Interactions with other engine mechanisms", Quantization: INT4 base, BF16
# adapter, dequantise and accumulate wide).  W[n][k] = s[n][k // group] * q[n][k].

def _pack(q, pad=0):
    """signed 4-bit values [d_out, d_in] -> bytes [d_out, d_in/2 + pad], the even k in the low nibble"""
    nib = (np.asarray(q) & 0xF).astype(np.uint8)
    packed = nib[:, 0::2] | (nib[:, 1::2] << 4)
    return np.concatenate([packed, np.full((q.shape[0], pad), 0xA5, np.uint8)], axis=1) if pad else packed


def _q4(q, scales, group, pad=0, scale_pad=0):
    d_out, d_in = q.shape
    sc = np.asarray(scales, np.float32)
    if scale_pad:
        sc = np.concatenate([sc, np.full((d_out, scale_pad), 1e30, np.float32)], axis=1)
    return Q4Weight(_pack(q, pad), np.ascontiguousarray(sc), group, d_in, d_out)


def _x(rows, d_in, seed):
    return bf16_bits(np.random.default_rng(seed).normal(0, 1, (rows, d_in)).astype(np.float32))


def test_q4_matches_its_bf16_twin_exactly(d_in=64, d_out=12, group=16, rows=5):
    # power-of-two group scales: s*q is exact in bf16, so the bf16 path over
    # the twin weight gives the same doubles in the same order (padding in
    # the rows of q and of the scales is never read)
    rng = np.random.default_rng(7)
    q = rng.integers(-8, 8, size=(d_out, d_in))
    sc = np.exp2(rng.integers(-6, 2, size=(d_out, d_in // group))).astype(np.float32)
    W = bf16_bits((np.repeat(sc, group, axis=1) * q).astype(np.float32))
    assert np.array_equal(bf16_to_f32(W), np.repeat(sc, group, axis=1) * q)  # the twin is exact
    x = _x(rows, d_in, 1)
    got = oracle.base_projection(_q4(q, sc, group, pad=16, scale_pad=3), x)
    assert np.array_equal(got, oracle.base_projection(W, x))


def test_q4_exact_rational(d_in=32, d_out=6, group=8, rows=3):
    rng = np.random.default_rng(11)
    q = rng.integers(-8, 8, size=(d_out, d_in))
    sc = rng.uniform(0.01, 0.5, size=(d_out, d_in // group)).astype(np.float32)
    x = _x(rows, d_in, 2)
    got = oracle.base_projection(_q4(q, sc, group), x)
    xf = bf16_to_f32(x)
    for b in range(rows):
        for n in range(d_out):
            exact = sum(Fraction(float(sc[n, k // group])) * int(q[n, k]) * Fraction(float(xf[b, k]))
                        for k in range(d_in))
            assert abs(got[b, n] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_q4_one_hot_gathers_scaled_x(d_in=48, d_out=20, group=16):
    # q[n][k_n] = 1 at even and odd k: (W.x)[b, n] = s[n][k_n // group] * x[b, k_n] exactly
    rng = np.random.default_rng(3)
    ks = rng.integers(0, d_in, size=d_out)
    ks[:2] = [0, d_in - 1]
    q = np.zeros((d_out, d_in), np.int64)
    q[np.arange(d_out), ks] = 1
    sc = np.exp2(rng.integers(-3, 3, size=(d_out, d_in // group))).astype(np.float32)
    x = _x(4, d_in, 3)
    got = oracle.base_projection(_q4(q, sc, group), x)
    want = bf16_to_f32(x).astype(np.float64)[:, ks] * sc[np.arange(d_out), ks // group]
    assert np.array_equal(got, want)


def test_q4_codes_decode_in_order():
    # the sixteen codes 0x0 .. 0xF are 0 .. 7, -8 .. -1; x one-hot reads each back
    d_in, group = 32, 32
    codes = np.tile(np.arange(16), 2)
    q = np.where(codes >= 8, codes - 16, codes)[None, :]
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    W = Q4Weight(packed, np.full((1, 1), 0.5, np.float32), group, d_in, 1)
    x = bf16_bits(np.eye(d_in, dtype=np.float32))
    got = oracle.base_projection(W, x)[:, 0]
    assert np.array_equal(got, 0.5 * q[0].astype(np.float64))


def test_q4_quantiser_bounds():
    # the generator's quantiser: |w - s*q| <= s/2 off the clamp, each group's
    # largest magnitude maps to +-7, and the packing round-trips
    from workloads.gen import quantize_q4
    w = small(rows=2, d_in=256, d_out=16)
    qw = quantize_q4(w.W["q"], 128)
    lo = (qw.q & 0xF).astype(np.int64)
    hi = (qw.q >> 4).astype(np.int64)
    q = np.empty((16, 256), np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    q = np.where(q >= 8, q - 16, q)
    wf = bf16_to_f32(w.W["q"]).astype(np.float64)
    s = np.repeat(qw.scales.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(wf - s * q) <= s / 2 + 1e-12)
    assert np.all(np.abs(q).reshape(16, 2, 128).max(axis=2) == 7)
