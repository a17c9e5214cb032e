"""lora_decode_layer (segments and the layer delta: one launch for a decode
batch up to rank 32 whose repeated reads of A stay small, three launches
otherwise) against the oracle through the C ABI: the delta alone and y, every
row, and the segments and status word bit for bit, on the tiny and q_proj
workloads at full size, ragged shapes, repeated ids (multi-row segments on
the one-launch path), both factor formats, bad ids and entries, the
caller's segment bound on both paths, repeated calls, HIP graph replays and
the three-launch paths."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import build_workload_for_tests as bw
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only hosts
    pytest.skip("no GPU", allow_module_level=True)

import adapter_gemv_amd as lg  # noqa: E402
from workloads.device import DeviceWorkload, to_bits  # noqa: E402


@pytest.fixture(autouse=True)
def _name_case(request):
    note(request.node.nodeid)


def run(dw, zero=False):
    dw.reset_y(zero=zero)
    dw.decode_layer()
    torch.cuda.synchronize()


def check_segments(dw, w, extra_status=0, bound=None):
    perm, offs, adap, status = dw.seg.host()
    ref = oracle.build_segments(w.ids, w.num_slots)
    nseg = len(ref.seg_adapter) if bound is None else min(bound, len(ref.seg_adapter))
    assert np.array_equal(adap, ref.seg_adapter[:nseg])
    assert np.array_equal(offs, ref.seg_offsets[:nseg + 1])
    assert np.array_equal(perm, ref.perm[:offs[-1]])
    dropped = int(ref.seg_offsets[-1] - ref.seg_offsets[nseg])
    assert status == ref.num_bad_ids + dropped + extra_status
    lens = np.diff(ref.seg_offsets[:nseg + 1].astype(np.int64))
    long = lens[lens >= 8] if w.num_rows >= 8 else lens[:0]
    assert dw.seg.tile_counts.cpu().tolist() == [int(((long + 127) // 128).sum()), int(((long + 63) // 64).sum())]


def check(w, launches=None, extra_status=0, ref=None, bound_segments=False):
    ref = oracle.lora_layer(w) if ref is None else ref
    dw = DeviceWorkload(w, bound_segments=bound_segments)
    if launches is not None:
        assert dw.decode_launches() == launches
    run(dw, zero=True)
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].delta, f"{w.name}/{m.name} delta")
    run(dw)
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].y, f"{w.name}/{m.name} y")
    check_segments(dw, w, extra_status)
    return dw


def test_tiny_one_launch():
    check(gen.tiny(x_std=1.0), launches=1)


def test_q_proj_full_size_one_launch():
    # 128 rows, 128 distinct rank-16 adapters, 8192 -> 8192: every row; the
    # host's exact distinct count (128) is the bound, as the benchmark runs it
    check(gen.q_proj(), launches=1, bound_segments=True)


SHAPES = [
    # rows, slots, d_in, d_out, rank(s), id mode
    (1, 1, 8, 8, 8, "distinct"),
    (5, 300, 1032, 1000, 16, "distinct"),
    (64, 4, 2056, 520, 32, "random"),
    (65, 65, 3064, 4104, 16, "distinct"),
    (40, 1, 1024, 2048, 8, "equal"),                          # one 40-row segment (blocks of 4 rows)
    (18, 1, 512, 520, 16, "equal"),                           # 18 rows: four blocks of 4 rows and one of 2
    (33, 9, 2048 + 24, 1024 + 8, (1, 3, 5, 12, 24, 28, 31, 7, 2), "random"),
    (200, 20, 512, 3000, (8, 16, 32), "random"),
    (256, 256, 4096, 2048, 16, "distinct"),
    (256, 7, 1024, 1040, (16, 0, 12), "random"),              # an untargeted slot
    (97, 8192, 2048, 1024, 8, "random_wide"),                 # ids over the largest slot table
    # rank 8 and below: one lane per B row, tiles of 4096 columns (two steps
    # of the y update), full and ragged, one- and multi-row segments
    (24, 24, 1024, 4096 + 72, 8, "distinct"),
    (3, 3, 512, 8192, (8, 4, 1), "distinct"),
    (48, 6, 1024, 3000 + 8, 8, "random"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"r{s[0]}_s{s[1]}_{s[2]}x{s[3]}_{s[5]}" for s in SHAPES])
def test_shapes_one_launch(shape):
    rows, slots, d_in, d_out, rank, mode = shape
    rng = np.random.default_rng(rows * 7 + d_in)
    ids = {"distinct": rng.permutation(rows) % slots, "equal": np.zeros(rows, int),
           "random": rng.integers(-1, slots + 1, size=rows),    # base-only and out-of-range ids too
           "random_wide": rng.integers(0, slots, size=rows)}[mode]
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    w = bw(rows + d_in + 5, rows, slots, d_in, d_out, None, ids, ranks=ranks, x_std=1.0)
    check(w, launches=1)


@pytest.mark.parametrize("fmt,max_rank,d_out", [("int8", 32, 2 * 1024 + 8), ("mixed", 32, 2 * 1024 + 8),
                                                 ("int8", 8, 4096 + 8)])
def test_int8_factors(fmt, max_rank, d_out):
    slots, rows = 24, 96
    ids = np.random.default_rng(4).integers(0, slots, size=rows)
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.array([8, 16, 3, 24, 32, 13]), slots).clip(max=max_rank)
    code = gen.FMT_INT8_ROWS if fmt == "int8" else \
        (np.where(np.arange(slots)[:, None] % 2 == 0, gen.FMT_INT8_ROWS, gen.FMT_BF16) * np.ones((1, 7), int)
         ).astype(np.int32)
    w = bw(41, rows, slots, 2056, d_out, None, ids, ranks=ranks, x_std=1.0, max_rank=max_rank, fmt=code)
    check(w, launches=1)


def test_four_projections_zipf_full_size():
    # the Zipf(1.1) batch: 256 rows over 512 paged adapters of ranks 8..64,
    # q/k/v/o, with its exact distinct count as the bound: three launches
    w = gen.zipf_paged()
    check(w, launches=3, bound_segments=True)


def test_layer_of_small_projections_with_shared_inputs():
    # q, k, v share x; all seven projections at rank 16 with small shapes
    w = gen.build_workload("small_layer", 9, 48, 48, {"q": (1024, 1024), "k": (1024, 256), "v": (1024, 256),
                                                        "o": (1024, 1024), "gate": (1024, 2824),
                                                        "up": (1024, 2824), "down": (2824, 1024)},
                           np.random.default_rng(2).permutation(48), np.full((48, 7), 16, np.int32),
                           x_of=gen.X_OF_70B, x_std=1.0, ab_std=0.02, y_std=1.0)
    check(w, launches=1)


@pytest.mark.parametrize("max_rank", [32, 64], ids=["one_launch", "three_launches"])
def test_bad_entries_counted_once(max_rank):
    rows, slots = 64, 6
    ids = np.arange(rows) % 8 - 1          # -1 .. 6: -1 base only, 6 out of range
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = [16, 0, 16, max_rank + 8, 16, 16]  # slot 1 untargeted, slot 3 rank > max_rank
    w = bw(8, rows, slots, 1024, 1024, None, ids, ranks=ranks, max_rank=max_rank, x_std=1.0)
    dw = DeviceWorkload(w)
    assert dw.decode_launches() == (1 if max_rank <= 32 else 3)
    y0 = bf16_host(dw.y["q"])
    run(dw)
    y = bf16_host(dw.y["q"])
    untouched = np.isin(ids, [-1, 1, 3, 6])
    assert np.array_equal(y[untouched], y0[untouched])
    check_rows(y, oracle.lora_layer(w)["q"].y, "bad entries y")
    check_segments(dw, w, extra_status=1)   # the too-high rank of slot 3, once


@pytest.mark.parametrize("max_rank", [16, 64], ids=["one_launch", "three_launches"])
def test_segment_bound_drops_the_highest_slots(max_rank):
    rows, slots = 40, 16
    ids = np.random.default_rng(8).integers(-1, slots + 2, size=rows)  # base-only and bad ids as well
    w = bw(9, rows, slots, 1024, 512, 16, ids, x_std=1.0, max_rank=max_rank)
    distinct = np.unique(ids[(ids >= 0) & (ids < slots)])
    bound = len(distinct) - 3
    kept = distinct[:bound]
    dw = DeviceWorkload(w)
    dw.seg.max_segments = bound
    assert dw.decode_launches() == (1 if max_rank <= 32 else 3)
    run(dw)
    ref = oracle.lora_layer(w)
    y = bf16_host(dw.y["q"])
    keep = np.isin(ids, kept)
    assert keep.sum() > 0 and (~keep & (ids >= 0) & (ids < slots)).sum() > 0
    check_rows(y[keep], ref["q"].y[keep], "bound: kept rows")
    assert np.array_equal(to_bits(dw.y["q"])[~keep], w.y0["q"][~keep])
    check_segments(dw, w, bound=bound)


def test_repeated_calls_on_one_workspace():
    # new ids, ranks and batch sizes on the same workspace, each against the oracle
    ws = torch.zeros(lg.workspace_bytes(256, 64, 32, 3 * 4096), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(17)
    for rep in range(6):
        rows = int(rng.integers(1, 257))
        ids = rng.integers(-1, 64, size=rows)
        rank = int(rng.choice([8, 16, 32]))
        shapes = {"q": (4096, 1024), "k": (4096, 512), "o": (1024, 4096)}
        ranks = np.zeros((64, 7), np.int32)
        ranks[:, [0, 1, 3]] = rank
        w = gen.build_workload(f"rep{rep}", 50 + rep, rows, 64, shapes, ids, ranks,
                               x_of={"q": "x", "k": "x", "o": "xo"}, x_std=1.0, ab_std=0.02, y_std=1.0)
        dw = DeviceWorkload(w)
        assert dw.decode_launches() == 1
        lg.decode_layer(dw.ios, rows, dw.ids, dw.table, 64, dw.seg, w.max_rank, ws)
        torch.cuda.synchronize()
        ref = oracle.lora_layer(w)
        for m in w.modules:
            check_rows(bf16_host(dw.y[m.name]), ref[m.name].y, f"rep {rep} {m.name}")
        check_segments(dw, w)


def test_deterministic_reruns():
    ids = np.random.default_rng(1).integers(0, 40, 200)
    w = bw(12, 200, 40, 4096, 2048, 32, ids, x_std=1.0)
    dw = DeviceWorkload(w)
    assert dw.decode_launches() == 1
    outs = []
    for _ in range(4):
        run(dw)
        outs.append(to_bits(dw.y["q"]))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_graph_replay_follows_device_data():
    rows, slots = 48, 12
    w = bw(21, rows, slots, 1024, 2048, 16, np.arange(rows) % slots, x_std=1.0)
    dw = DeviceWorkload(w)
    assert dw.decode_launches() == 1
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dw.reset_y()
        dw.decode_layer()  # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dw.decode_layer()
    rng = np.random.default_rng(3)
    for rep in range(4):
        ids = rng.integers(-1, slots, size=rows).astype(np.int32)
        perm_slots = rng.permutation(slots)
        dw.ids.copy_(torch.from_numpy(ids).cuda())
        dw.upload_table(dw.pack(dw.pool.data_ptr())[perm_slots])
        dw.reset_y()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = bf16_host(dw.y["q"])
        run(dw)
        assert np.array_equal(got, bf16_host(dw.y["q"])), rep
        w2 = bw(21, rows, slots, 1024, 2048, 16, ids, x_std=1.0)
        A, B, R, S = w2.host_table(0)
        ref = oracle.lora_module(w2.x["x"], w2.y0["q"], ids, A[perm_slots], B[perm_slots], R[perm_slots],
                                 S[perm_slots], 16)
        check_rows(got, ref.y, f"graph replay {rep}")


def test_three_launch_paths():
    # more rows than one block holds; rank 64; and too many repeated reads
    # of A (256 rows with their own rank-32 adapters, 16384 -> 4096: two
    # blocks of 2 tiles per row, each reading its 1 MiB of A: 537 MB)
    ids = np.random.default_rng(2).integers(0, 300, size=300)
    check(bw(70, 300, 300, 1024, 1024, 16, ids, x_std=1.0), launches=3)
    check(bw(71, 16, 16, 2048, 8192, 64, np.arange(16), x_std=1.0), launches=3)
    check(bw(72, 256, 256, 16384, 4096, 32, np.arange(256), x_std=1.0), launches=3)
