"""GPU parity on the seeded workloads at their full sizes.

Rows are compared element by element with the oracle: every row where the
oracle finishes in seconds (decode workloads), and for prefill every row of
two whole segments (the longest and the one of median length) plus the
first, middle and last row of every other segment, of both projections.  v
is compared through lora_shrink on the full 70B layer and on prefill's two
whole segments.
"""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import adapter_gemv_amd as lg  # noqa: E402,F401
from workloads.device import DeviceWorkload  # noqa: E402


def whole_segments(w):
    """Prefill: the rows of the longest sequence and of the one of median length."""
    starts = np.concatenate([[0], np.cumsum(w.seq_lens)[:-1]])
    order = np.argsort(w.seq_lens, kind="stable")
    pick = [order[-1], order[len(order) // 2]]
    return np.concatenate([np.arange(starts[i], starts[i] + w.seq_lens[i]) for i in pick]).astype(np.int32)


def sample_rows(w):
    if w.seq_lens is None:
        return None
    starts = np.concatenate([[0], np.cumsum(w.seq_lens)[:-1]])
    rows = np.concatenate([starts, starts + w.seq_lens // 2, starts + w.seq_lens - 1, whole_segments(w)])
    return np.unique(rows).astype(np.int32)


def make(name):
    if name != "zipf_formed":
        return gen.make_workload(name)
    # the rows the batch former picks from the Zipf queue: the oracle's choice,
    # which the library's former must match exactly
    import oracle.batch_former as bf
    q = gen.zipf_queue()
    sel = bf.form_batch(list(q), **gen.ZIPF_FORMER)
    assert list(lg.form_batch(q, **gen.ZIPF_FORMER)) == sel
    return gen.zipf_paged(ids=q[sel], name=name)


@pytest.mark.parametrize("name", ["tiny", "q_proj_r16", "full_layer_r64", "full_layer_r64_int8", "zipf_paged",
                                  "zipf_formed", "prefill_r16", "prefill_r64"])
def test_workload_full_size(name):
    note(f"workload {name}: generate")
    w = make(name)
    rows = sample_rows(w)
    ref = oracle.lora_layer(w, rows=rows)
    note(f"workload {name}: {w.num_rows} rows, {w.num_slots} slots, modules {[m.name for m in w.modules]}")
    dw = DeviceWorkload(w, bound_segments=True)  # as the bench runs it
    # delta alone
    dw.reset_y(zero=True)
    dw.step()
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name])[sel], ref[m.name].delta, f"{name}/{m.name} delta")
    # onto the base output
    dw.reset_y()
    dw.step()
    torch.cuda.synchronize()
    for m in w.modules:
        check_rows(bf16_host(dw.y[m.name])[sel], ref[m.name].y, f"{name}/{m.name} y")
    _, offs, adap, status = dw.seg.host()
    seg_ref = oracle.build_segments(w.ids, w.num_slots)
    assert np.array_equal(offs, seg_ref.seg_offsets) and np.array_equal(adap, seg_ref.seg_adapter)
    assert status == 0


@pytest.mark.parametrize("name", ["full_layer_r64", "prefill_r64"])
def test_v_through_lora_shrink_full_size(name):
    # v = A . x of every row of a segment, written by lora_shrink (the sum of
    # its k-chunk partials), against the oracle's v; all seven 70B projections
    # for the decode layer, both projections on prefill's two whole segments
    w = gen.make_workload(name)
    rows = None if w.seq_lens is None else whole_segments(w)
    note(f"v through lora_shrink: {name}, {w.num_rows if rows is None else rows.size} rows")
    ref = oracle.lora_layer(w, rows=rows)
    dw = DeviceWorkload(w, bound_segments=True)
    dw.build_segments()
    ldv = (w.max_rank + 3) // 4 * 4
    sel = slice(None) if rows is None else rows
    valid = (w.ids >= 0) & (w.ids < w.num_slots)
    vv = valid if rows is None else valid[rows]
    for m in w.modules:
        v = torch.full((w.num_rows, ldv), float("nan"), dtype=torch.float32, device="cuda")
        lg.shrink(dw.x[m.x_name], dw.table, w.num_slots, 7, m.index, dw.seg, w.max_rank, v, dw.ws)
        torch.cuda.synchronize()
        vg = v[:, :w.max_rank].cpu().numpy().astype(np.float64)[sel]
        check_rows(vg[vv], ref[m.name].v[vv], f"{name}/{m.name} v (lora_shrink)")
