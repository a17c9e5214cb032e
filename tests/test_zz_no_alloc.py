"""lora_apply_layer_noalloc: the layer delta with the library's static device
scratch in place of a caller's workspace, through the C ABI.  Two calls in a
row on one device, the second with a smaller batch, each compared bit for bit
with lora_apply_layer on the same inputs (the same kernels, so the same
bits) and element by element with the oracle."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, check_rows, note
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only hosts
    pytest.skip("no GPU", allow_module_level=True)

import adapter_gemv_amd as lg  # noqa: E402
from workloads.device import DeviceWorkload, to_bits  # noqa: E402


def _check(w):
    dw = DeviceWorkload(w)
    dw.build_segments()
    dw.apply_layer()  # caller's workspace
    want = {k: to_bits(v) for k, v in dw.y.items()}
    dw.reset_y()
    lg.apply_layer_noalloc(dw.ios, w.num_rows, dw.table, w.num_slots, dw.seg, w.max_rank)
    torch.cuda.synchronize()
    ref = oracle.lora_layer(w)
    for m in w.modules:
        got = to_bits(dw.y[m.name])
        assert np.array_equal(got, want[m.name]), f"{w.name} {m.name}: differs from lora_apply_layer"
        check_rows(bf16_host(dw.y[m.name]), ref[m.name].y, f"{w.name} {m.name} y")
    assert int(dw.seg.status.item()) == 0


def test_noalloc_two_calls_second_smaller():
    # 1: every projection of the 70B layer at rank 64 (16 rows, 16 adapters);
    # 2: one projection, 12 rows, Zipf-skewed ids over 8 adapters, mixed ranks
    note("noalloc full_layer r64 rows=16")
    _check(gen.full_layer(rows=16))
    note("noalloc small q rows=12")
    ids = np.array([3, 3, 0, 7, -1, 3, 5, 5, 1, 3, 2, 6], np.int32)
    ranks = np.zeros((8, 7), np.int32)
    ranks[:, 0] = [8, 16, 5, 12, 0, 24, 8, 16]
    from workloads import build_workload_for_tests as bw
    _check(bw(21, 12, 8, 1024, 520, 0, ids, ranks=ranks, x_std=1.0, max_rank=32))


def test_noalloc_refuses_more_than_its_scratch():
    w = gen.tiny()
    dw = DeviceWorkload(w)
    need_rows = lg.STATIC_SCRATCH_BYTES // (64 * 4 * (1 + 7)) + 1  # one 1024-k chunk, rank 64
    x = torch.zeros(need_rows, 1024, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(need_rows, 8, dtype=torch.bfloat16, device="cuda")
    seg = lg.Segments(need_rows)
    assert lg.workspace_bytes(need_rows, 4, 64, 1024) > lg.STATIC_SCRATCH_BYTES
    with pytest.raises(lg.LoraError, match="LORA_ERR_SCRATCH"):
        lg.apply_layer_noalloc({"q": lg.ModuleIO(x, y)}, need_rows, dw.table, 4, seg, 64)
