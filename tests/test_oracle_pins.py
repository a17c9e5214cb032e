"""Pins of the CPU oracle against things other than itself.

* exact rational brute force (fractions) on tiny shapes: every product of two
  bf16 values and every sum is exact, so the fp64 oracle must agree to ~1e-12;
* numpy's BLAS in float64 on a medium shape (a library routine);
* closed forms: a one-hot gather (delta[b, n_i] = x[b, k_i]) and identity
  adapters (delta = x), which catch a wrong row-to-adapter index, a
  transposed operand or a dropped term exactly;
* the merged-weight identity (W + s B A) x - W x = s B (A x) from the LoRA
  forward on "m07 -- Multi-Adapter (LoRA) Serving", "6. Deep Dive A";
* zero cases: B = 0, A = 0, rank 0, base-only id -1, out-of-range ids and
  ranks leave y == y0 exactly;
* linearity in x and in the scale, and row-permutation equivariance;
* segments against Python's stable ``sorted``.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32, build_workload_for_tests as bw


def exact_row(x_row, A, B, scale, y0_row):
    """Exact rational v, delta, y for one row (A [r, d_in], B [d_out, r])."""
    xf = [Fraction(float(t)) for t in bf16_to_f32(x_row)]
    Af = [[Fraction(float(t)) for t in bf16_to_f32(row)] for row in A]
    Bf = [[Fraction(float(t)) for t in bf16_to_f32(row)] for row in B]
    v = [sum(a * b for a, b in zip(Arow, xf)) for Arow in Af]
    s = Fraction(float(np.float32(scale)))
    d = [s * sum(bj * vj for bj, vj in zip(Brow, v)) for Brow in Bf]
    y = [Fraction(float(t)) + dd for t, dd in zip(bf16_to_f32(y0_row), d)]
    return v, d, y


def run_oracle(w, col=0, rows=None):
    A, B, R, S = w.host_table(col)
    spec = w._spec_col(col)
    return oracle.lora_module(w.x[spec.x_name], w.y0[spec.name], w.ids, A, B, R, S, w.max_rank, rows=rows)


def rel_err(got, exact):
    exact = np.array([float(e) for e in exact])
    scale = max(np.abs(exact).max(), 1e-300)
    return np.abs(np.asarray(got, dtype=np.float64) - exact).max() / scale


@pytest.mark.parametrize("d_in,d_out,rank,rows,slots", [
    (1, 1, 1, 3, 2), (3, 5, 2, 4, 3), (8, 16, 8, 6, 3), (24, 8, 3, 5, 4), (40, 24, 5, 7, 2)])
def test_exact_rational(d_in, d_out, rank, rows, slots):
    seed = d_in * 1000 + d_out
    ids = np.random.default_rng(seed).integers(0, slots, size=rows)
    scales = np.full((slots, 7), 0.75, np.float32)
    w = bw(seed, rows, slots, d_in, d_out, rank, ids, scales=scales)
    res = run_oracle(w)
    for b in range(rows):
        a = int(w.ids[b])
        v, d, y = exact_row(w.x["x"][b], w.A(a, 0), w.B(a, 0), w.scales[a, 0], w.y0["q"][b])
        assert rel_err(res.v[b, :rank], v) < 1e-12
        assert np.all(res.v[b, rank:] == 0)
        assert rel_err(res.delta[b], d) < 1e-12
        assert rel_err(res.y[b], y) < 1e-12


def test_against_blas_medium():
    # d_in not a multiple of anything in particular; several ranks.
    rows, slots, d_in, d_out = 9, 3, 1000, 392
    ids = np.array([2, 0, 1, 1, 2, 0, 0, 2, 1])
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = [5, 16, 9]
    w = bw(11, rows, slots, d_in, d_out, None, ids, ranks=ranks, x_std=1.0)
    res = run_oracle(w)
    x = bf16_to_f32(w.x["x"]).astype(np.float64)
    for b in range(rows):
        a = int(ids[b])
        A = bf16_to_f32(w.A(a, 0)).astype(np.float64)
        B = bf16_to_f32(w.B(a, 0)).astype(np.float64)
        v = A @ x[b]
        d = B @ v
        r = ranks[a, 0]
        assert np.abs(res.v[b, :r] - v).max() <= 1e-12 * np.abs(v).max()
        assert np.abs(res.delta[b] - d).max() <= 1e-12 * np.abs(d).max()


def test_merged_weight_identity():
    """(W + s B A) x - W x equals the oracle's delta (the merged form)."""
    rows, slots, d_in, d_out = 6, 3, 64, 48
    ids = np.array([1, 2, 0, 1, 1, 2])
    scales = np.array([[1.0] * 7, [2.0] * 7, [0.5] * 7], np.float32)
    w = bw(5, rows, slots, d_in, d_out, 8, ids, scales=scales, x_std=1.0)
    res = run_oracle(w)
    rng = np.random.default_rng(0)
    W = rng.standard_normal((d_out, d_in)) * 0.02
    x = bf16_to_f32(w.x["x"]).astype(np.float64)
    for b in range(rows):
        a = int(ids[b])
        A = bf16_to_f32(w.A(a, 0)).astype(np.float64)
        B = bf16_to_f32(w.B(a, 0)).astype(np.float64)
        merged = (W + float(scales[a, 0]) * (B @ A)) @ x[b] - W @ x[b]
        assert np.abs(res.delta[b] - merged).max() <= 1e-9 * np.abs(merged).max()


def test_one_hot_gather_closed_form():
    """A_i = e_{k_i}^T in row 0, B_i = e_{n_i} in column 0: delta[b, n_i] = x[b, k_i]."""
    rows, slots, d_in, d_out, rank = 12, 6, 32, 40, 4
    ks = [3, 0, 31, 17, 8, 22]
    ns = [39, 5, 0, 12, 27, 33]

    def fill(w):
        for a in range(slots):
            A, B = w.A(a, 0), w.B(a, 0)
            A[:] = 0
            B[:] = 0
            A[0, ks[a]] = 0x3F80  # 1.0
            B[ns[a], 0] = 0x3F80
    ids = np.random.default_rng(3).integers(0, slots, size=rows)
    w = bw(7, rows, slots, d_in, d_out, rank, ids, ab_fill=fill, x_std=1.0)
    res = run_oracle(w)
    x = bf16_to_f32(w.x["x"]).astype(np.float64)
    for b in range(rows):
        a = ids[b]
        want = np.zeros(d_out)
        want[ns[a]] = x[b, ks[a]]
        assert np.array_equal(res.delta[b], want)


def test_identity_adapter():
    """rank = d, A = B = I: delta = x exactly."""
    d = 16

    def fill(w):
        for a in range(w.num_slots):
            A, B = w.A(a, 0), w.B(a, 0)
            A[:] = 0
            B[:] = 0
            A[np.arange(d), np.arange(d)] = 0x3F80
            B[np.arange(d), np.arange(d)] = 0x3F80
    w = bw(9, 5, 2, d, d, d, np.array([0, 1, 1, 0, 1]), ab_fill=fill, x_std=1.0)
    res = run_oracle(w)
    assert np.array_equal(res.delta, bf16_to_f32(w.x["x"]).astype(np.float64))


def test_zero_cases_leave_y_exactly():
    rows, slots, d_in, d_out = 8, 4, 24, 16
    ids = np.array([0, 1, 2, 3, -1, 0, 7, 2])  # -1 base only, 7 out of range
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = [8, 0, 8, 99]                 # slot 1 untargeted, slot 3 rank > max_rank

    def fill(w):
        w.B(0, 0)[:] = 0       # slot 0: B = 0
        w.A(2, 0)[:] = 0       # slot 2: A = 0
    w = bw(13, rows, slots, d_in, d_out, None, ids, ranks=ranks, ab_fill_after=fill, max_rank=64)
    res = run_oracle(w)
    y0 = bf16_to_f32(w.y0["q"]).astype(np.float64)
    assert np.array_equal(res.y, y0)
    assert np.all(res.delta == 0)
    assert res.num_bad_rank == 1          # row 3 uses slot 3
    seg = oracle.build_segments(ids, slots)
    assert seg.num_bad_ids == 1           # row 6


def test_linearity_and_scale():
    rows, slots, d_in, d_out = 6, 3, 48, 40
    ids = np.array([0, 1, 2, 2, 1, 0])
    w = bw(17, rows, slots, d_in, d_out, 8, ids, x_std=1.0)
    r1 = run_oracle(w)
    # doubling x (exact in bf16) doubles v and delta exactly
    w.x["x"] = bf16_bits(2 * bf16_to_f32(w.x["x"]))
    r2 = run_oracle(w)
    assert np.array_equal(r2.v, 2 * r1.v)
    assert np.array_equal(r2.delta, 2 * r1.delta)
    # scale 2 doubles delta exactly, leaves v
    w.scales[:] = 2.0
    r3 = run_oracle(w)
    assert np.array_equal(r3.v, r2.v)
    assert np.array_equal(r3.delta, 2 * r2.delta)


def test_row_permutation_equivariance():
    rows, slots, d_in, d_out = 10, 4, 32, 24
    ids = np.random.default_rng(1).integers(-1, slots, size=rows)
    w = bw(19, rows, slots, d_in, d_out, 8, ids, x_std=1.0)
    r1 = run_oracle(w)
    p = np.random.default_rng(2).permutation(rows)
    w.x["x"] = w.x["x"][p].copy()
    w.y0["q"] = w.y0["q"][p].copy()
    w.ids = w.ids[p].copy()
    r2 = run_oracle(w)
    assert np.array_equal(r2.y, r1.y[p])
    assert np.array_equal(r2.v, r1.v[p])


def test_selected_rows_match_full():
    w = bw(23, 12, 3, 40, 24, 8, np.arange(12) % 3, x_std=1.0)
    full = run_oracle(w)
    sel = np.array([11, 0, 5])
    part = run_oracle(w, rows=sel)
    assert np.array_equal(part.y, full.y[sel])


@pytest.mark.parametrize("n,slots,seed", [(0, 3, 0), (1, 1, 1), (16, 4, 2), (257, 9, 3), (1000, 64, 4),
                                           (300, 1, 5), (64, 512, 6)])
def test_segments_vs_stable_sort(n, slots, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-2, slots + 2, size=n).astype(np.int32)
    seg = oracle.build_segments(ids, slots)
    valid = [b for b in range(n) if 0 <= ids[b] < slots]
    want = sorted(valid, key=lambda b: ids[b])   # Python's sort is stable
    assert seg.perm.tolist() == want
    assert seg.num_bad_ids == int(np.count_nonzero(ids >= slots))
    # offsets strictly increase, adapters ascend, counts = histogram
    offs = seg.seg_offsets
    assert offs[0] == 0 and offs[-1] == len(valid)
    assert np.all(np.diff(offs) > 0)
    assert np.all(np.diff(seg.seg_adapter) > 0)
    for s in range(seg.num_segments):
        rows_s = seg.perm[offs[s]:offs[s + 1]]
        assert np.all(ids[rows_s] == seg.seg_adapter[s])
        assert np.all(np.diff(rows_s) > 0)
        assert len(rows_s) == np.count_nonzero(ids == seg.seg_adapter[s])


# ---------------------------------------------------------- int8 factors
# int8 adapters with one fp32 scale per row ("9. Bottlenecks and Evolution"
# on "m07 -- Multi-Adapter (LoRA) Serving", item 3).  With power-of-two
# scales every dequantised value is exactly a bf16 value, so the int8 path
# must give bit for bit what the (pinned) bf16 path gives on the same values.

def int8_bf16_twins(seed, rows, slots, d_in, d_out, rank, ids):
    from workloads import gen
    w8 = bw(seed, rows, slots, d_in, d_out, rank, ids, x_std=1.0, fmt=gen.FMT_INT8_ROWS)
    wb = bw(seed, rows, slots, d_in, d_out, rank, ids, x_std=1.0)
    rng = np.random.default_rng(seed)
    for a in range(slots):
        sa, qa = w8.A_q8(a, 0)
        sb, qb = w8.B_q8(a, 0)
        sa[:] = 2.0 ** rng.integers(-9, -3, size=sa.shape)
        sb[:] = 2.0 ** rng.integers(-9, -3, size=sb.shape)
        wb.A(a, 0)[:] = bf16_bits(sa[:, None] * qa.astype(np.float32))
        wb.B(a, 0)[:] = bf16_bits(sb[:, None] * qb.astype(np.float32))
    return w8, wb


@pytest.mark.parametrize("d_in,d_out,rank,rows,slots", [(24, 10, 5, 6, 3), (40, 24, 3, 5, 2), (16, 8, 16, 4, 2)])
def test_int8_matches_bf16_twin_exactly(d_in, d_out, rank, rows, slots):
    ids = np.random.default_rng(d_in + rank).integers(-1, slots, size=rows)
    w8, wb = int8_bf16_twins(d_in * 7 + rank, rows, slots, d_in, d_out, rank, ids)
    r8, rb = oracle.lora_layer(w8)["q"], oracle.lora_layer(wb)["q"]
    assert np.array_equal(r8.v, rb.v)
    assert np.array_equal(r8.delta, rb.delta)
    assert np.array_equal(r8.y, rb.y)
    assert np.abs(rb.delta).max() > 0


def test_int8_exact_rational():
    from workloads import gen
    rows, slots, d_in, d_out, rank = 5, 2, 12, 6, 3
    ids = np.array([0, 1, 1, 0, 1])
    w = bw(77, rows, slots, d_in, d_out, rank, ids, x_std=1.0, fmt=gen.FMT_INT8_ROWS,
           scales=np.full((slots, 7), 0.625, np.float32))
    res = oracle.lora_layer(w)["q"]
    for b in range(rows):
        a = int(ids[b])
        sa, qa = w.A_q8(a, 0)
        sb, qb = w.B_q8(a, 0)
        xf = [Fraction(float(t)) for t in bf16_to_f32(w.x["x"][b])]
        v = [sum(Fraction(float(sa[j])) * int(qa[j, k]) * xf[k] for k in range(d_in)) for j in range(rank)]
        d = [Fraction(0.625) * sum(Fraction(float(sb[n])) * int(qb[n, j]) * v[j] for j in range(rank))
             for n in range(d_out)]
        assert rel_err(res.v[b, :rank], v) < 1e-12
        assert rel_err(res.delta[b], d) < 1e-12


def test_int8_padding_columns_unused():
    # the bytes of A past d_in and of B past the rank in each row are never
    # read, and the rows sit lda8 / ldb8 bytes apart
    from workloads import gen
    ids = np.array([0, 1, 0, 1])
    d_in, d_out, rank = 40, 16, 5
    w = bw(5, 4, 2, d_in, d_out, rank, ids, x_std=1.0, fmt=gen.FMT_INT8_ROWS)
    before = oracle.lora_layer(w)["q"]
    raw = w.pool.view(np.uint8)
    for a in range(2):
        o = 2 * int(w.a_off[a, 0]) + 4 * 8
        full = raw[o:o + rank * gen.lda8(d_in)].reshape(rank, gen.lda8(d_in))
        assert gen.lda8(d_in) == 48 and np.array_equal(full[:, :d_in].view(np.int8), w.A_q8(a, 0)[1])
        full[:, d_in:] = 0x7F
        o = 2 * int(w.b_off[a, 0]) + 4 * d_out
        full = raw[o:o + d_out * gen.ldb8(rank)].reshape(d_out, gen.ldb8(rank))
        full[:, rank:] = 0x7F
    after = oracle.lora_layer(w)["q"]
    assert np.array_equal(before.delta, after.delta)
    assert np.abs(before.delta).max() > 0


def test_int8_quantiser_round_trip():
    # the generator's per-row quantiser: |v - s q| <= s / 2, and the largest
    # magnitude of each row maps to +-127
    from workloads import gen
    v = np.random.default_rng(3).standard_normal((9, 33)).astype(np.float32) * 0.02
    s, q = gen.quantize_rows(v)
    assert np.all(np.abs(v - s[:, None] * q.astype(np.float32)) <= s[:, None] * (0.5 + 1e-6))
    assert np.all(np.abs(q).max(axis=1) == 127)
