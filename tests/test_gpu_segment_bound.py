"""GPU checks of the host bound on the segments of a build (max_segments in
lora_segments_t): a bound at or above the batch's distinct adapters changes
only how the work is cut (results against the oracle as without one); a
bound below it keeps the segments of the lowest slots, counts the rows of the
others into the status word and leaves those rows without a delta."""
import copy

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


def expected_tiles(offs, n):
    """The build's SGMV tile counts: segments of at least 8 rows (batches of
    at least 8 rows) in tiles of 128 rows (shrink) and 64 rows (expand)."""
    lens = np.diff(np.asarray(offs, np.int64))
    long = lens[lens >= 8] if n >= 8 else lens[:0]
    return [int(((long + 127) // 128).sum()), int(((long + 63) // 64).sum())]


def expected_clamp(ids, slots, bound):
    """The oracle's grouping cut to the first `bound` segments: (perm, offsets,
    adapters, status)."""
    ref = oracle.build_segments(ids, slots)
    k = ref.num_segments if bound <= 0 else min(bound, ref.num_segments)
    end = int(ref.seg_offsets[k])
    dropped = int(ref.seg_offsets[-1]) - end
    return ref.perm[:end], ref.seg_offsets[:k + 1], ref.seg_adapter[:k], ref.num_bad_ids + dropped


# one-block builder (<= 1024 rows) and the chunked one; bounds below, at and above the distinct count
@pytest.mark.parametrize("n,slots,lo,hi", [(40, 16, -1, 18), (256, 512, -1, 40), (1024, 64, 0, 64),
                                           (3000, 300, -2, 301), (20000, 40, 0, 40), (7, 3, 0, 3),
                                           (600, 9, -1, 9)])
@pytest.mark.parametrize("frac", [0.0, 0.25, 0.5, 1.0, 2.0])
def test_builder_keeps_the_lowest_slots(n, slots, lo, hi, frac):
    ids = np.random.default_rng(n + slots).integers(lo, hi, size=n).astype(np.int32)
    distinct = lg.segment_bound(ids, slots)
    bound = 0 if frac == 0 else max(1, int(distinct * frac))
    note(f"builder n={n} slots={slots} distinct={distinct} bound={bound}")
    seg = lg.Segments(n, max_segments=bound)
    ws = torch.empty(lg.workspace_bytes(n, slots, 1, 0), dtype=torch.uint8, device="cuda")
    lg.build_segments(torch.from_numpy(ids).cuda(), slots, seg, ws)
    perm, offs, adap, status = seg.host()
    want = expected_clamp(ids, slots, bound)
    assert np.array_equal(perm, want[0])
    assert np.array_equal(offs, want[1])
    assert np.array_equal(adap, want[2])
    assert status == want[3]
    assert seg.tile_counts.cpu().tolist() == expected_tiles(want[1], n)


def run_layer(w, bound):
    dw = DeviceWorkload(w)
    dw.seg.max_segments = bound
    dw.reset_y()
    dw.step()
    torch.cuda.synchronize()
    return dw


def without_dropped(w, keep_slots):
    """The workload with the rows of slots outside keep_slots made base-only."""
    w2 = copy.copy(w)
    ids = np.asarray(w.ids).copy()
    valid = (ids >= 0) & (ids < w.num_slots)
    ids[valid & ~np.isin(ids, keep_slots)] = -1
    w2.ids = ids
    return w2


CASES = [  # rows, slots, d_in, d_out, rank, id sampler
    (128, 128, 4096, 4104, 64, "distinct"),
    (256, 512, 2048, 1032, (8, 16, 64), "zipf"),
    (300, 40, 1024, 2056, (16, 32), "random"),
    (64, 4, 3080, 520, 64, "random"),
]


def ids_for(mode, rows, slots, rng):
    if mode == "distinct":
        return rng.permutation(rows) % slots
    if mode == "zipf":
        return gen.zipf_ids(int(rng.integers(1 << 30)), rows, slots)
    return rng.integers(-1, slots + 1, size=rows)


def workload(case, seed):
    rows, slots, d_in, d_out, rank, mode = case
    rng = np.random.default_rng(seed)
    ids = ids_for(mode, rows, slots, rng).astype(np.int32)
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    return bw(seed, rows, slots, d_in, d_out, None, ids, ranks=ranks, x_std=1.0, max_rank=int(np.max(rank)))


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}_s{c[1]}_{c[5]}" for c in CASES])
def test_exact_bound_matches_the_oracle(case):
    w = workload(case, 900 + case[0])
    bound = lg.segment_bound(w.ids, w.num_slots)
    note(f"exact bound {bound}")
    ref = oracle.lora_layer(w)
    dw = run_layer(w, bound)
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].y, f"{w.name}/{m.name} y, bound {bound}")
    *_, status = dw.seg.host()
    assert status == int(((w.ids >= w.num_slots)).sum())


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}_s{c[1]}_{c[5]}" for c in CASES])
def test_small_bound_drops_the_highest_slots(case):
    w = workload(case, 950 + case[0])
    distinct = lg.segment_bound(w.ids, w.num_slots)
    bound = max(1, distinct // 3)
    ids = np.asarray(w.ids)
    valid = (ids >= 0) & (ids < w.num_slots)
    keep = np.unique(ids[valid])[:bound]
    note(f"bound {bound} of {distinct}: keep slots up to {keep[-1]}")
    ref = oracle.lora_layer(without_dropped(w, keep))
    dw = run_layer(w, bound)
    for m in w.modules:
        got = bf16_host(dw.y[m.name])
        check_rows(got, ref[m.name].y, f"{w.name}/{m.name} y, bound {bound}")
        dropped = valid & ~np.isin(ids, keep)
        assert np.array_equal(got[dropped], bf16_to_f32(w.y0[m.name])[dropped])  # untouched
    *_, status = dw.seg.host()
    assert status == int((ids >= w.num_slots).sum()) + int((valid & ~np.isin(ids, keep)).sum())


@pytest.mark.parametrize("bound", ["exact", "third"])
def test_fused_layer_with_a_bound(bound):
    rng = np.random.default_rng(5)
    rows, slots = 200, 30
    ids = rng.integers(-1, slots, size=rows).astype(np.int32)
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    ranks[:, 0] = rng.choice([8, 16, 64], size=slots)
    w = gen.add_base_weights(bw(960, rows, slots, 2048, 1040, None, ids, ranks=ranks, x_std=1.0, max_rank=64))
    distinct = lg.segment_bound(ids, slots)
    k = distinct if bound == "exact" else distinct // 3
    keep = np.unique(ids[ids >= 0])[:k]
    ref = oracle.linear_layer(without_dropped(w, keep))  # dropped rows: y = W.x
    dw = DeviceWorkload(w)
    dw.seg.max_segments = k
    for y in dw.y.values():
        y.fill_(float("nan"))
    dw.build_segments()
    lg.linear_layer(dw.lin_ios, rows, dw.ids, dw.table, slots, dw.seg, w.max_rank, dw.ws)
    torch.cuda.synchronize()
    got = bf16_host(dw.y["q"])
    assert np.isfinite(got).all()
    check_rows(got, ref["q"].y, f"fused y, bound {k} of {distinct}")


def test_stacked_passes_share_the_bound():
    # column 0: 3 domain adapters; column 1: one style adapter per row.  A
    # bound of 3 fits column 0 and drops most of column 1.
    rng = np.random.default_rng(8)
    rows, n_dom, n_sty = 96, 3, 96
    ranks = np.zeros((n_dom + n_sty, gen.N_MOD), np.int32)
    ranks[:n_dom, 0] = 64
    ranks[n_dom:, 0] = 16
    ra = np.stack([rng.integers(0, n_dom, size=rows), n_dom + rng.permutation(rows)], 1).astype(np.int32)
    w = bw(970, rows, n_dom + n_sty, 2048, 1032, None, ra[:, 0], ranks=ranks, x_std=1.0)
    for bound, keep1 in ((lg.segment_bound(ra, w.num_slots), rows), (3, 3)):
        ra_ref = ra.copy()
        kept = np.sort(ra[:, 1])[:keep1]
        ra_ref[~np.isin(ra[:, 1], kept), 1] = -1
        ref = oracle.lora_layer_stacked(w, ra_ref)
        dw = DeviceWorkload(w)
        dw.seg.max_segments = bound
        dw.reset_y()
        lg.apply_layer_stacked(dw.ios, rows, torch.from_numpy(ra).cuda(), dw.table, w.num_slots, dw.seg,
                               w.max_rank, dw.ws)
        torch.cuda.synchronize()
        check_rows(bf16_host(dw.y["q"]), ref["q"].y, f"stacked y, bound {bound}")
        *_, status = dw.seg.host()
        assert status == rows - keep1
