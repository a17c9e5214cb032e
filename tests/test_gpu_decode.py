"""GPU parity of the segment builder, shrink, expand and layer calls against the
CPU oracle, through the C ABI, on small and ragged shapes and special cases."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import bf16_bits, bf16_to_f32, gen
from workloads import build_workload_for_tests as bw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only hosts
    pytest.skip("no GPU", allow_module_level=True)

import adapter_gemv_amd as lg  # noqa: E402  (raises if the HIP library is missing)
from workloads.device import DeviceWorkload, to_bits  # noqa: E402


@pytest.fixture(autouse=True)
def _name_case(request):
    note(request.node.nodeid)


# ------------------------------------------------------------------ segments

@pytest.mark.parametrize("n,slots,lo,hi", [
    (0, 3, 0, 3), (1, 1, 0, 1), (16, 4, 0, 4), (63, 8, -1, 9), (64, 64, 0, 64), (65, 7, -2, 7),
    (128, 128, 0, 128), (256, 512, -1, 520), (257, 40, -1, 41), (300, 9000, -1, 9001), (513, 2, 0, 2),
    (1000, 5000, -1, 5000), (1024, 3, 0, 3), (1025, 9, -1, 10), (2000, 10000, 0, 10000),
    (5000, 512, -3, 515), (34816, 32, 0, 32), (40000, 5000, -1, 5001)])
def test_segments_bit_exact(n, slots, lo, hi):
    ids = np.random.default_rng(n * 7 + slots).integers(lo, hi, size=n).astype(np.int32)
    ref = oracle.build_segments(ids, slots)
    seg = lg.Segments(n)
    ws = torch.empty(lg.workspace_bytes(n, slots, 1, 0), dtype=torch.uint8, device="cuda")
    lg.build_segments(torch.from_numpy(ids).cuda(), slots, seg, ws)
    perm, offs, adap, status = seg.host()
    assert np.array_equal(perm, ref.perm)
    assert np.array_equal(offs, ref.seg_offsets)
    assert np.array_equal(adap, ref.seg_adapter)
    assert status == ref.num_bad_ids
    lens = np.diff(ref.seg_offsets.astype(np.int64))
    long = lens[lens >= 8] if n >= 8 else lens[:0]  # the build's SGMV tiles: 128 rows (shrink), 64 (expand)
    assert seg.tile_counts.cpu().tolist() == [int(((long + 127) // 128).sum()), int(((long + 63) // 64).sum())]


def test_segments_sorted_runs():
    # ids already grouped (prefill layout) and all-equal ids
    for ids in (np.repeat(np.arange(32, dtype=np.int32), 300), np.full(3000, 5, np.int32)):
        ref = oracle.build_segments(ids, 40)
        seg = lg.Segments(ids.size)
        ws = torch.empty(lg.workspace_bytes(ids.size, 40, 1, 0), dtype=torch.uint8, device="cuda")
        lg.build_segments(torch.from_numpy(ids).cuda(), 40, seg, ws)
        perm, offs, adap, _ = seg.host()
        assert np.array_equal(perm, ref.perm) and np.array_equal(offs, ref.seg_offsets)


# ------------------------------------------------------------------ helpers

def oracle_all(w):
    return oracle.lora_layer(w)


def run_split(dw):
    """lora_build_segments, then lora_shrink + lora_expand per projection.
    Returns the GPU v per module."""
    w = dw.w
    dw.build_segments()
    vs = {}
    ldv = (w.max_rank + 3) // 4 * 4  # the ABI wants a multiple of 4
    for m in w.modules:
        v = torch.full((w.num_rows, ldv), float("nan"), dtype=torch.float32, device="cuda")
        lg.shrink(dw.x[m.x_name], dw.table, w.num_slots, 7, m.index, dw.seg, w.max_rank, v, dw.ws)
        lg.expand(v, dw.table, w.num_slots, 7, m.index, dw.seg, w.max_rank, dw.y[m.name], dw.ws)
        vs[m.name] = v[:, :w.max_rank]
    return vs


def run_layer(dw):
    dw.build_segments()
    dw.apply_layer()


def run_phases(dw):
    w = dw.w
    dw.build_segments()
    lg.layer_shrink(dw.ios, w.num_rows, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)
    lg.layer_expand(dw.ios, w.num_rows, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)


def run_decode(dw):
    """lora_decode_layer: the segments and every projection, in one launch
    where the batch fits it, else in the three launches."""
    dw.decode_layer()


RUNNERS = {"split": run_split, "layer": run_layer, "phases": run_phases, "decode": run_decode}


def check_workload(w, ref, runner="layer", check_v=True, rows=None):
    """Delta alone (y0 = 0) and y against the oracle; v too on the split path."""
    dw = DeviceWorkload(w)
    dw.reset_y(zero=True)
    vs = RUNNERS[runner](dw)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    valid = (w.ids >= 0) & (w.ids < w.num_slots)
    for m in w.modules:
        r = ref[m.name]
        check_rows(bf16_host(dw.y[m.name])[sel], r.delta, f"{w.name}/{m.name} delta")
        if check_v and vs:
            vg = vs[m.name].cpu().numpy().astype(np.float64)[sel]
            vv = valid if rows is None else valid[rows]
            check_rows(vg[vv], r.v[vv], f"{w.name}/{m.name} v")
    dw.reset_y()
    RUNNERS[runner](dw)
    torch.cuda.synchronize()
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name])[sel], ref[m.name].y, f"{w.name}/{m.name} y")
    return dw


# ------------------------------------------------------------------ parity

@pytest.mark.parametrize("runner", sorted(RUNNERS))
def test_tiny_decode(runner):
    w = gen.tiny()
    check_workload(w, oracle_all(w), runner)


def test_tiny_unit_variance_x():
    w = gen.tiny(x_std=1.0)
    check_workload(w, oracle_all(w), "split")


SHAPES = [
    # rows, slots, d_in, d_out, rank(s), id mode
    (1, 1, 8, 8, 8, "distinct"),
    (63, 63, 1032, 1000, 16, "distinct"),
    (64, 4, 2056, 520, 64, "random"),
    (65, 65, 3064, 4104, 32, "distinct"),
    (40, 1, 1024, 2048, 8, "equal"),
    (33, 9, 2048 + 24, 1024 + 8, (1, 3, 5, 12, 24, 40, 63, 64, 7), "random"),
    (200, 20, 512, 3000, (8, 16, 32, 64), "random"),
    (17, 3, 4096, 1536, (64, 0, 16), "random"),
]


@pytest.mark.parametrize("runner", ["split", "layer"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"r{s[0]}_s{s[1]}_{s[2]}x{s[3]}" for s in SHAPES])
def test_random_shapes(shape, runner):
    rows, slots, d_in, d_out, rank, mode = shape
    rng = np.random.default_rng(rows * 131 + d_in)
    ids = {"distinct": rng.permutation(rows) % slots, "equal": np.zeros(rows, int),
           "random": rng.integers(0, slots, size=rows)}[mode]
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    w = bw(rows + d_in, rows, slots, d_in, d_out, None, ids, ranks=ranks, x_std=1.0)
    check_workload(w, oracle_all(w), runner)


def test_multi_row_segments_and_base_rows():
    # segment sizes 1..40 (crossing the 16-row LDS group), base-only rows mixed in
    sizes = np.arange(1, 41)
    ids = np.repeat(np.arange(40), sizes)
    ids = np.concatenate([ids, -np.ones(30, int)])
    ids = np.random.default_rng(0).permutation(ids)
    w = bw(77, ids.size, 40, 2048, 1024, 32, ids, x_std=1.0)
    for runner in ("split", "layer"):
        check_workload(w, oracle_all(w), runner)


def test_scale_applied():
    scales = np.tile(np.array([[2.0], [0.75], [1.0], [0.5]], np.float32), (1, 7))
    w = bw(31, 24, 4, 1024, 1024, 16, np.arange(24) % 4, scales=scales, x_std=1.0)
    check_workload(w, oracle_all(w), "split")


# ------------------------------------------------------------------ exact cases

def test_one_hot_gather_bit_exact():
    """A_i = e_{k_i}^T in row 0, B_i = e_{n_i} in column 0: delta[b, n_i] = x[b, k_i]
    exactly, zero elsewhere; any wrong gather shows bit-exactly."""
    rows, slots, d_in, d_out, rank = 96, 48, 2048, 1024, 16
    rng = np.random.default_rng(5)
    ks = rng.choice(d_in, slots, replace=False)
    ns = rng.choice(d_out, slots, replace=False)

    def fill(w):
        for a in range(slots):
            A, B = w.A(a, 0), w.B(a, 0)
            A[:] = 0
            B[:] = 0
            A[0, ks[a]] = 0x3F80
            B[ns[a], 0] = 0x3F80
    ids = rng.integers(0, slots, size=rows)
    w = bw(6, rows, slots, d_in, d_out, rank, ids, ab_fill=fill, x_std=1.0)
    for runner in ("split", "layer"):
        dw = DeviceWorkload(w)
        dw.reset_y(zero=True)
        RUNNERS[runner](dw)
        y = bf16_host(dw.y["q"])
        x = bf16_to_f32(w.x["x"]).astype(np.float64)
        want = np.zeros((rows, d_out))
        want[np.arange(rows), ns[ids]] = x[np.arange(rows), ks[ids]]
        assert np.array_equal(y, want), runner


def test_zero_cases_bit_exact_and_status():
    rows, slots, d_in, d_out = 64, 6, 1024, 1024
    ids = np.arange(rows) % 8 - 1          # -1 .. 6: -1 base only, 6 out of range
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = [16, 0, 16, 99, 16, 16]  # slot 1 untargeted, slot 3 rank > max_rank

    def fill(w):
        w.B(0, 0)[:] = 0
        w.A(2, 0)[:] = 0
    w = bw(8, rows, slots, d_in, d_out, None, ids, ranks=ranks, ab_fill_after=fill, max_rank=64, x_std=1.0)
    dw = DeviceWorkload(w)
    y_before = bf16_host(dw.y["q"])
    run_layer(dw)
    _, _, _, status = dw.seg.host()
    y_after = bf16_host(dw.y["q"])
    untouched = np.isin(ids, [-1, 0, 1, 2, 3, 6])
    assert np.array_equal(y_after[untouched], y_before[untouched])
    # the rows whose id is >= num_slots, and the rank-99 entry once (its one segment, one projection)
    assert status == oracle.build_segments(ids, slots).num_bad_ids + 1
    ref = oracle_all(w)
    check_rows(y_after, ref["q"].y, "zero cases y")


def test_deterministic_reruns():
    ids = np.random.default_rng(1).integers(0, 40, 256)
    w = bw(12, 256, 40, 4096, 2048, 64, ids, x_std=1.0)
    dw = DeviceWorkload(w)
    outs = []
    for _ in range(3):
        dw.reset_y()
        run_layer(dw)
        outs.append(bf16_host(dw.y["q"]))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_graph_replay_follows_device_data():
    """Capture segments + layer in a HIP graph; change the row ids and the table
    in device memory; every replay must match an eager run on the new data."""
    rows, slots = 48, 12
    w = bw(21, rows, slots, 1024, 2048, 16, np.arange(rows) % slots, x_std=1.0)
    dw = DeviceWorkload(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dw.reset_y()
        run_layer(dw)  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dw.build_segments()
        dw.apply_layer()
    rng = np.random.default_rng(3)
    for rep in range(4):
        ids = rng.integers(-1, slots, size=rows).astype(np.int32)
        perm_slots = rng.permutation(slots)
        table = dw.pack(dw.pool.data_ptr())[perm_slots]      # slot a now holds adapter perm_slots[a]
        dw.ids.copy_(torch.from_numpy(ids).cuda())
        dw.upload_table(table)
        dw.reset_y()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bf16_host(dw.y["q"])
        dw.reset_y()
        run_layer(dw)
        torch.cuda.synchronize()
        eager = bf16_host(dw.y["q"])
        assert np.array_equal(got, eager), rep
        # and the oracle on the permuted table
        w2 = bw(21, rows, slots, 1024, 2048, 16, ids, x_std=1.0)
        A, B, R, S = w2.host_table(0)
        ref = oracle.lora_module(w2.x["x"], w2.y0["q"], ids, A[perm_slots], B[perm_slots], R[perm_slots],
                                 S[perm_slots], 16)
        check_rows(got, ref.y, f"graph replay {rep}")


# ------------------------------------------------------------------ long segments (matrix-core path)

LONG = [
    # segment lengths, ranks per slot, d_in, d_out
    ([16, 17, 31, 64, 65, 128, 129, 300], (16, 64, 24, 40, 8, 32, 48, 56), 2056, 1000),
    ([16, 40, 200], (4, 12, 1), 1024, 520),
    ([19, 5, 77, 1, 130], (7, 64, 63, 33, 9), 3080, 2048),
]


@pytest.mark.parametrize("runner", ["split", "layer", "phases"])
@pytest.mark.parametrize("case", range(len(LONG)))
def test_long_segments(case, runner):
    lens, ranks_, d_in, d_out = LONG[case]
    ids = np.repeat(np.arange(len(lens)), lens)
    ids = np.random.default_rng(case).permutation(ids)   # rows of a segment need not be adjacent
    ranks = np.zeros((len(lens), 7), np.int32)
    ranks[:, 0] = ranks_
    w = bw(100 + case, ids.size, len(lens), d_in, d_out, None, ids, ranks=ranks, x_std=1.0)
    check_workload(w, oracle_all(w), runner)


def test_long_segments_with_short_and_base_rows():
    # a prefill-like batch: a few long sequences, many single decode rows, base-only rows
    lens = [600, 1, 1, 2, 250, 1, 3, 15, 16, 1000]
    ids = np.concatenate([np.repeat(np.arange(len(lens)), lens), -np.ones(50, int)])
    ranks = np.zeros((len(lens), 7), np.int32)
    ranks[:, 0] = [16, 16, 64, 8, 32, 16, 16, 64, 64, 16]
    w = bw(200, ids.size, len(lens), 4096, 2048, None, ids, ranks=ranks, x_std=1.0)
    for runner in ("split", "layer"):
        check_workload(w, oracle_all(w), runner)


@pytest.mark.parametrize("runner", sorted(RUNNERS))
def test_prefill_folded_partials_mixed_chunks(runner):
    # A prefill-sized batch over projections of 3, 1 and 4 k-chunks (d_in
    # 4104, 2048, 8192 at the 2048-input chunks of a prefill call): the layer
    # calls sum each row's partials into its first chunk between the shrink
    # and the expand, and the one-chunk projection is left as it is.  Ranks
    # differ per projection and slot (some 0), with long, short and base rows.
    lens = [900, 1, 3, 640, 1, 7, 12, 520, 2, 1]
    ids = np.concatenate([np.repeat(np.arange(len(lens)), lens), -np.ones(30, int)])
    ids = np.random.default_rng(11).permutation(ids).astype(np.int32)
    shapes = {"q": (4104, 1032), "k": (2048, 520), "o": (8192, 1024)}
    rng = np.random.default_rng(12)
    ranks = np.zeros((len(lens), gen.N_MOD), np.int32)
    for n in shapes:
        ranks[:, gen.MODULE_INDEX[n]] = rng.choice([0, 8, 16, 40, 64], size=len(lens), p=[0.1, 0.2, 0.2, 0.2, 0.3])
    w = gen.build_workload("fold_mixed", 400, ids.size, len(lens), shapes, ids, ranks,
                           x_of={n: "x_" + n for n in shapes}, x_std=1.0)
    assert w.num_rows >= 2048
    note(f"folded partials runner={runner} rows={w.num_rows}")
    check_workload(w, oracle_all(w), runner)


def test_prefill_phases_expand_twice():
    # A prefill-sized batch (at least 2048 rows, ragged k-chunks): the layer
    # expand only reads the shrink's k-chunk partials, so a second expand
    # after the same shrink gives the same bits.
    lens = [700, 1, 2, 300, 1, 5, 9, 1100, 1]
    ids = np.concatenate([np.repeat(np.arange(len(lens)), lens), -np.ones(40, int)])
    ids = np.random.default_rng(5).permutation(ids)
    ranks = np.zeros((len(lens), 7), np.int32)
    ranks[:, 0] = [64, 16, 8, 32, 64, 13, 40, 16, 64]
    w = bw(300, ids.size, len(lens), 4104, 1032, None, ids, ranks=ranks, x_std=1.0)
    assert w.num_rows >= 2048
    ref = oracle_all(w)
    dw = DeviceWorkload(w)
    dw.build_segments()
    lg.layer_shrink(dw.ios, w.num_rows, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)
    outs = []
    for _ in range(2):
        dw.reset_y(zero=True)
        lg.layer_expand(dw.ios, w.num_rows, dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws)
        torch.cuda.synchronize()
        outs.append(to_bits(dw.y["q"]))
    assert np.array_equal(outs[0], outs[1])
    check_rows(bf16_host(dw.y["q"]), ref["q"].delta, "prefill phases delta")


@pytest.mark.parametrize("d_out", [2 * 2048 + 8, 3 * 512 + 8, 5 * 512 + 24])
@pytest.mark.parametrize("fmt", ["bf16", "int8", "mixed"])
def test_entry_lane_width_in_rank64_launch(fmt, d_out):
    # One row per adapter, entries of many ranks in one launch of rank class
    # 64: each expand item runs at the lane width of its own entry's rank
    # (1, 2, 4 or 8 lanes per output row, fewer load passes at width 1), over
    # whole and ragged n-tiles.  17 segments take 512-output tiles (the
    # smallest), narrower than a low-rank entry's sub-tile, so most of such an
    # item's load passes fall past its tile and read zero.
    ranks_ = np.array([1, 3, 8, 9, 13, 16, 17, 24, 32, 33, 40, 57, 64, 8, 16, 32, 64], np.int32)
    slots = ranks_.size
    ids = np.random.default_rng(11).permutation(slots).astype(np.int32)
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = ranks_
    if fmt == "bf16":
        code = gen.FMT_BF16
    elif fmt == "int8":
        code = gen.FMT_INT8_ROWS
    else:
        code = np.where(np.arange(slots)[:, None] % 2 == 0, gen.FMT_INT8_ROWS, gen.FMT_BF16) * np.ones((1, 7), int)
        code = code.astype(np.int32)
    w = bw(400, slots, slots, 2056, d_out, None, ids, ranks=ranks, x_std=1.0, max_rank=64, fmt=code)
    assert w.max_rank == 64
    for runner in ("layer", "split"):
        check_workload(w, oracle_all(w), runner)
