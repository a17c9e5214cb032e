"""GPU parity of several adapters per row (lora_apply_layer_stacked) against
the oracle's composition: one pass per column of the rows' adapter lists
("m07 -- Multi-Adapter (LoRA) Serving", "9. Bottlenecks and Evolution",
item 5)."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import gen
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


def run_stacked(dw, ra, pass_max_rank=None):
    w = dw.w
    lg.apply_layer_stacked(dw.ios, w.num_rows, torch.from_numpy(np.ascontiguousarray(ra, np.int32)).cuda(),
                           dw.table, w.num_slots, dw.seg, w.max_rank, dw.ws, pass_max_rank=pass_max_rank)
    torch.cuda.synchronize()


def check_stacked(w, ra, pass_max_rank=None, bound_segments=False):
    ref = oracle.lora_layer_stacked(w, ra, pass_max_rank=pass_max_rank)
    dw = DeviceWorkload(w, bound_segments=bound_segments)
    dw.reset_y(zero=True)
    run_stacked(dw, ra, pass_max_rank)
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].delta, f"{w.name}/{m.name} stacked delta")
    dw.reset_y()
    run_stacked(dw, ra, pass_max_rank)
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].y, f"{w.name}/{m.name} stacked y")
    return dw


def test_depth_one_is_the_layer_call_bit_for_bit():
    ids = np.random.default_rng(1).integers(-1, 30, size=100)
    w = bw(61, 100, 30, 2048, 1032, 32, ids, x_std=1.0)
    a, b = DeviceWorkload(w), DeviceWorkload(w)
    a.build_segments()
    a.apply_layer()
    run_stacked(b, ids[:, None])
    assert np.array_equal(bf16_host(a.y["q"]), bf16_host(b.y["q"]))


@pytest.mark.parametrize("pass_max_rank", [None, (64, 24)])
def test_two_adapters_per_decode_row(pass_max_rank):
    # a domain adapter (few, shared) and a style adapter (one per row, some rows without)
    rng = np.random.default_rng(2)
    rows, n_dom, n_sty = 96, 3, 96
    ranks = np.zeros((n_dom + n_sty, 7), np.int32)
    ranks[:n_dom, 0] = 64
    ranks[n_dom:, 0] = rng.choice([8, 16, 24], size=n_sty)
    scales = np.ones((n_dom + n_sty, 7), np.float32)
    scales[:, 0] = rng.uniform(0.5, 2.0, size=n_dom + n_sty)
    ra = np.stack([rng.integers(0, n_dom, size=rows), n_dom + rng.permutation(rows)], 1).astype(np.int32)
    ra[rng.random(rows) < 0.2, 1] = -1
    w = bw(62, rows, n_dom + n_sty, 4096, 2056, None, ra[:, 0], ranks=ranks, scales=scales, x_std=1.0)
    check_stacked(w, ra, pass_max_rank)


def test_entries_above_their_pass_rank_are_skipped_and_counted():
    # style ranks 8..24 under a pass rank of 16: the 24s are device-data errors
    rng = np.random.default_rng(5)
    rows, n_dom, n_sty = 64, 2, 64
    ranks = np.zeros((n_dom + n_sty, 7), np.int32)
    ranks[:n_dom, 0] = 32
    ranks[n_dom:, 0] = rng.choice([8, 16, 24], size=n_sty)
    ra = np.stack([rng.integers(0, n_dom, size=rows), n_dom + rng.permutation(rows)], 1).astype(np.int32)
    w = bw(65, rows, n_dom + n_sty, 2048, 1024, None, ra[:, 0], ranks=ranks, x_std=1.0)
    dw = check_stacked(w, ra, (32, 16))
    *_, status = dw.seg.host()
    assert status > 0
    with pytest.raises(lg.LoraError, match="LORA_ERR_RANK"):
        run_stacked(dw, ra, (65, 16))
    with pytest.raises(lg.LoraError, match="LORA_ERR_RANK"):
        run_stacked(dw, ra, (32, 0))


@pytest.mark.parametrize("seed", range(3))
def test_three_deep_mixed_formats_and_projections(seed):
    """Columns: long shared segments (matrix-core items), short ones, and a
    sparse third adapter; int8 and bf16 entries; several projections."""
    rng = np.random.default_rng(70 + seed)
    names = ["q", "k", "v", "o"] if seed != 1 else ["gate", "down"]
    shapes = {n: (8 * int(rng.integers(64, 400)), 8 * int(rng.integers(64, 400))) for n in names}
    slots = 40
    rows = int(rng.integers(150, 400))
    col0 = rng.integers(0, 3, size=rows)                   # three long segments
    col1 = 3 + rng.integers(0, 30, size=rows)               # short segments
    col2 = np.where(rng.random(rows) < 0.3, 33 + rng.integers(0, 7, size=rows), -1)
    ra = np.stack([col0, col1, col2], 1).astype(np.int32)
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    for n in names:
        ranks[:, gen.MODULE_INDEX[n]] = rng.choice([4, 8, 16, 32, 64], size=slots)
    fmt = np.where(rng.random((slots, gen.N_MOD)) < 0.5, gen.FMT_INT8_ROWS, gen.FMT_BF16).astype(np.int32)
    scales = rng.uniform(0.25, 2.0, size=(slots, gen.N_MOD)).astype(np.float32)
    w = gen.build_workload(f"stacked{seed}", 70 + seed, rows, slots, shapes, ra[:, 0], ranks, x_std=1.0,
                           scales=scales, fmt=fmt)
    note(f"stacked seed {seed}: {rows} rows, {[(m.name, m.d_in, m.d_out) for m in w.modules]}")
    check_stacked(w, ra)


def test_status_sums_the_passes():
    # pass 0: 2 ids past the table, pass 1: 3; no other errors
    rows, slots = 40, 10
    ra = np.stack([np.arange(rows) % slots, (np.arange(rows) * 3) % slots], 1).astype(np.int32)
    ra[[1, 7], 0] = slots + 2
    ra[[2, 3, 30], 1] = slots
    w = bw(63, rows, slots, 1024, 1024, 16, ra[:, 0], x_std=1.0)
    dw = check_stacked(w, ra)
    *_, status = dw.seg.host()
    assert status == 5


def test_zero_rows_resets_the_segments():
    w = bw(64, 8, 4, 256, 256, 8, np.arange(8) % 4, x_std=1.0)
    dw = DeviceWorkload(w)
    lg.apply_layer_stacked(dw.ios, 0, torch.zeros((0, 2), dtype=torch.int32, device="cuda"), dw.table,
                           w.num_slots, dw.seg, w.max_rank, dw.ws)
    torch.cuda.synchronize()
    _, offs, _, status = dw.seg.host()
    assert status == 0


def test_stacked_layer_full_size():
    # the bench's workload: 70B layer, 128 rows, a shared domain adapter (r64) and a style adapter (r16) per row
    w = gen.make_workload("stacked_layer")
    check_stacked(w, w.stack, (64, 16), bound_segments=True)  # as the bench runs it
