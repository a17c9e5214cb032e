"""GPU parity of the fused base projection + delta (lora_linear_layer):
y = bf16(W.x + delta) against the oracle's y = W.x + delta in fp64."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import bf16_to_f32, gen
from workloads import build_workload_for_tests as bw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import adapter_gemv_amd as lg  # noqa: E402
from workloads.device import DeviceWorkload  # noqa: E402


@pytest.fixture(autouse=True)
def _name_case(request):
    note(request.node.nodeid)


class FusedRun:
    """A workload on the device with its base weights; run() fills y."""

    def __init__(self, w, bound_segments=False):
        self.w = w
        self.dw = DeviceWorkload(w, bound_segments=bound_segments)

    def run(self, phases=False):
        w, dw = self.w, self.dw
        for y in dw.y.values():
            y.fill_(float("nan"))  # every element must be written
        dw.build_segments()
        args = (dw.lin_ios, w.num_rows, dw.ids, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)
        if phases:
            lg.linear_shrink(*args)
            lg.linear_expand(*args)
        else:
            lg.linear_layer(*args)
        torch.cuda.synchronize()
        return {m.name: bf16_host(dw.y[m.name]) for m in w.modules}


def check_fused(w, rows=None, bound_segments=False):
    ref = oracle.linear_layer(w, rows=rows)
    got = FusedRun(w, bound_segments).run()
    for m in w.modules:
        g = got[m.name] if rows is None else got[m.name][rows]
        assert np.isfinite(g).all(), m.name
        check_rows(g, ref[m.name].y, f"{w.name}/{m.name} fused y")


SHAPES = [
    # rows, slots, d_in, d_out, ranks, id mode
    (1, 1, 1032, 72, 8, "distinct"),
    (37, 37, 2056, 1000, (16, 0, 64, 5, 33), "distinct"),
    (128, 128, 4096, 1024, 64, "distinct"),
    (129, 40, 1024, 4104, (8, 16, 24), "random"),
    (200, 9, 3080, 520, (64, 1, 40), "random"),
    # short input ranges: fewer rounds of 64 inputs than a pass of the main
    # loop (72: one whole round and a ragged one; 264: five, the last ragged)
    (5, 5, 72, 136, 8, "distinct"),
    (33, 10, 264, 264, (16, 64), "random"),
    # long input ranges (128 or more rounds of 64 inputs; 8200: a ragged last
    # round), one and three row tiles
    (64, 64, 8200, 520, (16, 64, 8), "distinct"),
    (130, 20, 12288, 264, (8, 32, 64), "random"),
    (257, 30, 8192, 136, (64, 0, 16), "random"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"r{s[0]}_{s[2]}x{s[3]}" for s in SHAPES])
def test_fused_shapes(shape):
    rows, slots, d_in, d_out, rank, mode = shape
    rng = np.random.default_rng(rows + d_out)
    ids = {"distinct": rng.permutation(rows) % slots, "random": rng.integers(-1, slots + 2, size=rows)}[mode]
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    scales = np.zeros((slots, 7), np.float32)
    scales[:, 0] = rng.uniform(0.5, 2.0, size=slots)
    w = gen.add_base_weights(bw(400 + rows, rows, slots, d_in, d_out, None, ids, ranks=ranks, scales=scales,
                                x_std=1.0, max_rank=64))
    check_fused(w)


@pytest.mark.parametrize("seed", range(3))
def test_fused_mixed_formats_projections_and_long_segments(seed):
    rng = np.random.default_rng(410 + seed)
    names = ["q", "k", "o"] if seed != 1 else ["gate", "down"]
    shapes = {n: (8 * int(rng.integers(64, 400)), 8 * int(rng.integers(16, 400))) for n in names}
    slots = 20
    lens = rng.integers(1, 3, size=slots)
    lens[:3] = rng.integers(8, 90, size=3)  # long segments take the matrix-core shrink
    ids = np.concatenate([np.repeat(np.arange(slots), lens), -np.ones(5, int)])
    ids = rng.permutation(ids).astype(np.int32)
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    for n in names:
        ranks[:, gen.MODULE_INDEX[n]] = rng.choice([0, 8, 16, 32, 64], size=slots)
    fmt = np.where(rng.random((slots, gen.N_MOD)) < 0.5, gen.FMT_INT8_ROWS, gen.FMT_BF16).astype(np.int32)
    scales = rng.uniform(0.25, 2.0, size=(slots, gen.N_MOD)).astype(np.float32)
    w = gen.build_workload(f"fused{seed}", 410 + seed, ids.size, slots, shapes, ids, ranks, x_std=1.0,
                           scales=scales, fmt=fmt)
    note(f"fused seed {seed}: {ids.size} rows, {[(m.name, m.d_in, m.d_out) for m in w.modules]}")
    check_fused(gen.add_base_weights(w))


def test_fused_one_hot_bit_exact():
    """W[n, k_n] = 1 and adapter a with A = e_{ka} (row 0), B = e_{na}
    (column 0): y[b, n] = bf16(x[b, k_n] + [n == n_a] x[b, k_a]), exactly."""
    rows, slots, d_in, d_out, rank = 150, 30, 2048, 1032, 16
    rng = np.random.default_rng(7)
    kw = rng.integers(0, d_in, size=d_out)
    ka = rng.choice(d_in, slots, replace=False)
    na = rng.choice(d_out, slots, replace=False)

    def fill(w):
        for a in range(slots):
            A, B = w.A(a, 0), w.B(a, 0)
            A[:] = 0
            B[:] = 0
            A[0, ka[a]] = 0x3F80
            B[na[a], 0] = 0x3F80
    ids = rng.integers(-1, slots, size=rows)
    w = bw(8, rows, slots, d_in, d_out, rank, ids, ab_fill=fill, x_std=1.0)
    w.W = {"q": np.zeros((d_out, d_in), np.uint16)}
    w.W["q"][np.arange(d_out), kw] = 0x3F80
    x = bf16_to_f32(w.x["x"])
    want = x[:, kw].copy()
    r = np.arange(rows)
    on = ids >= 0
    want[r[on], na[ids[on]]] += x[r[on], ka[ids[on]]]
    want = bf16_to_f32(gen.bf16_bits(want)).astype(np.float64)  # one rounding of the fp32 sum
    got = FusedRun(w).run()["q"]
    assert np.array_equal(got, want)


def test_fused_full_layer_sampled_rows():
    w = gen.make_workload("fused_layer_r64")
    rows = np.random.default_rng(1).choice(w.num_rows, 12, replace=False).astype(np.int32)
    note(f"fused full layer: rows {list(rows)}")
    check_fused(w, rows=rows, bound_segments=True)  # as the bench runs it


def test_phases_equal_the_whole_call():
    ids = np.random.default_rng(3).integers(-1, 20, size=90)
    w = gen.add_base_weights(bw(430, 90, 20, 2048, 1040, 32, ids, x_std=1.0))
    run = FusedRun(w)
    whole = run.run()["q"]
    split = run.run(phases=True)["q"]
    assert np.array_equal(whole, split)


@pytest.mark.parametrize("max_rank", [5, 13, 30])
def test_fused_max_rank_not_a_multiple_of_eight(max_rank):
    # the v planes hold max_rank values of a rounded-up row: lanes past the rank must read zeros
    rng = np.random.default_rng(max_rank)
    rows, slots = 70, 12
    ids = rng.integers(-1, slots, size=rows)
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = rng.integers(1, max_rank + 1, size=slots)
    ranks[0, 0] = max_rank
    fmt = np.where(rng.random((slots, 7)) < 0.5, gen.FMT_INT8_ROWS, gen.FMT_BF16).astype(np.int32)
    w = gen.add_base_weights(bw(440 + max_rank, rows, slots, 1024, 528, None, ids, ranks=ranks, x_std=1.0,
                                max_rank=max_rank, fmt=fmt))
    check_fused(w)


def test_fused_repeated_calls_same_bits():
    # calls after the first on the same workspace give the same bits, whole or
    # in two parts, and a second fused part after one shrink part too
    rng = np.random.default_rng(441)
    rows, slots = 140, 24
    ids = rng.integers(-1, slots, size=rows)
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = rng.choice([0, 8, 32, 64], size=slots)
    w = gen.add_base_weights(bw(441, rows, slots, 8200, 520, None, ids, ranks=ranks, x_std=1.0, max_rank=64))
    run = FusedRun(w)
    first = run.run()["q"]
    assert np.isfinite(first).all()
    for _ in range(2):
        assert np.array_equal(run.run()["q"], first)
    assert np.array_equal(run.run(phases=True)["q"], first)
    dw = run.dw
    args = (dw.lin_ios, w.num_rows, dw.ids, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)
    dw.y["q"].fill_(float("nan"))
    lg.linear_expand(*args)  # the v planes of the shrink above
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(dw.y["q"]), first)


def test_fused_long_one_hot_bit_exact():
    """The one-hot case over 9000 inputs (141 rounds, a ragged last one):
    every sum has one nonzero term, so y is exact."""
    rows, slots, d_in, d_out, rank = 130, 20, 9000, 520, 16
    rng = np.random.default_rng(17)
    kw = rng.integers(0, d_in, size=d_out)
    ka = rng.choice(d_in, slots, replace=False)
    na = rng.choice(d_out, slots, replace=False)

    def fill(w):
        for a in range(slots):
            A, B = w.A(a, 0), w.B(a, 0)
            A[:] = 0
            B[:] = 0
            A[0, ka[a]] = 0x3F80
            B[na[a], 0] = 0x3F80
    ids = rng.integers(-1, slots, size=rows)
    w = bw(18, rows, slots, d_in, d_out, rank, ids, ab_fill=fill, x_std=1.0)
    w.W = {"q": np.zeros((d_out, d_in), np.uint16)}
    w.W["q"][np.arange(d_out), kw] = 0x3F80
    x = bf16_to_f32(w.x["x"])
    want = x[:, kw].copy()
    r = np.arange(rows)
    on = ids >= 0
    want[r[on], na[ids[on]]] += x[r[on], ka[ids[on]]]
    want = bf16_to_f32(gen.bf16_bits(want)).astype(np.float64)
    assert np.array_equal(FusedRun(w).run()["q"], want)
