"""GPU parity of int8 adapters (one fp32 scale per row of A and of B) against the
CPU oracle, through the C ABI: single-row and multi-row decode segments, long
(matrix-core) segments, tables that mix int8 and bf16 entries, and exact
one-hot gathers that check the block layout bit for bit."""
import numpy as np
import pytest

import oracle
from tests.parity import bf16_host, note
from workloads import bf16_to_f32, gen
from workloads import build_workload_for_tests as bw

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU-only hosts
    pytest.skip("no GPU", allow_module_level=True)

from tests.test_gpu_decode import RUNNERS, check_workload  # noqa: E402
from workloads.device import DeviceWorkload  # noqa: E402

Q8 = gen.FMT_INT8_ROWS


@pytest.fixture(autouse=True)
def _name_case(request):
    note(request.node.nodeid)


DECODE = [
    # rows, slots, d_in, d_out, rank(s)
    (64, 64, 4096, 1024, 16),
    (40, 40, 2056, 3000, 64),
    (33, 33, 1032, 1000, (1, 3, 7, 8, 13, 24, 33, 57, 64)),
    (8, 8, 8192, 1024, 32),
]


@pytest.mark.parametrize("runner", sorted(RUNNERS))
@pytest.mark.parametrize("case", range(len(DECODE)))
def test_int8_single_row_decode(case, runner):
    rows, slots, d_in, d_out, rank = DECODE[case]
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    ids = np.random.default_rng(case).permutation(rows) % slots
    w = bw(300 + case, rows, slots, d_in, d_out, None, ids, ranks=ranks, x_std=1.0, fmt=Q8)
    check_workload(w, oracle.lora_layer(w), runner)


def test_int8_multi_row_segments():
    # segment sizes 1..40: multi-row decode items up to the long threshold, then SGMV tiles
    sizes = np.arange(1, 41)
    ids = np.concatenate([np.repeat(np.arange(40), sizes), -np.ones(20, int)])
    ids = np.random.default_rng(4).permutation(ids)
    ranks = np.zeros((40, 7), np.int32)
    ranks[:, 0] = np.resize([8, 16, 32, 64, 5, 40], 40)
    w = bw(311, ids.size, 40, 2048, 1032, None, ids, ranks=ranks, x_std=1.0, fmt=Q8)
    for runner in ("split", "layer"):
        check_workload(w, oracle.lora_layer(w), runner)


LONG = [
    ([16, 17, 64, 65, 129, 300], (16, 64, 24, 40, 8, 56), 2056, 1000),
    ([19, 5, 77, 1, 130], (7, 64, 63, 33, 9), 3080, 2048 + 8),
]


@pytest.mark.parametrize("runner", sorted(RUNNERS))
@pytest.mark.parametrize("case", range(len(LONG)))
def test_int8_long_segments(case, runner):
    lens, ranks_, d_in, d_out = LONG[case]
    ids = np.random.default_rng(10 + case).permutation(np.repeat(np.arange(len(lens)), lens))
    ranks = np.zeros((len(lens), 7), np.int32)
    ranks[:, 0] = ranks_
    w = bw(320 + case, ids.size, len(lens), d_in, d_out, None, ids, ranks=ranks, x_std=1.0, fmt=Q8)
    check_workload(w, oracle.lora_layer(w), runner)


@pytest.mark.parametrize("seed", range(4))
def test_int8_mixed_table_layer(seed):
    """Several projections, every (slot, projection) entry int8 or bf16 at
    random, short and long segments and base-only rows in one batch."""
    rng = np.random.default_rng(330 + seed)
    names = ["q", "k", "v", "o"] if seed % 2 == 0 else ["gate", "down"]
    shapes = {n: (8 * int(rng.integers(64, 520)), 8 * int(rng.integers(64, 520))) for n in names}
    slots = 24
    lens = rng.integers(1, 4, size=slots)
    lens[rng.choice(slots, 3, replace=False)] = rng.integers(8, 200, size=3)
    ids = np.concatenate([np.repeat(np.arange(slots), lens), -np.ones(7, int)])
    ids = rng.permutation(ids).astype(np.int32)
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    for n in names:
        ranks[:, gen.MODULE_INDEX[n]] = rng.choice([0, 4, 8, 16, 24, 32, 48, 64], size=slots)
    fmt = (rng.random((slots, gen.N_MOD)) < 0.5).astype(np.int32) * Q8
    scales = rng.uniform(0.25, 2.0, size=(slots, gen.N_MOD)).astype(np.float32)
    w = gen.build_workload(f"int8mix{seed}", 330 + seed, ids.size, slots, shapes, ids, ranks, x_std=1.0,
                           scales=scales, fmt=fmt)
    note(f"int8 mixed seed {seed}: {ids.size} rows, {[(m.name, m.d_in, m.d_out) for m in w.modules]}")
    check_workload(w, oracle.lora_layer(w), ("split", "layer", "phases")[seed % 3])


@pytest.mark.parametrize("seg_len", [1, 3, 40])
def test_int8_one_hot_gather_bit_exact(seg_len):
    """A_q8 row 0 = e_{k_i} (scale 2^e), B_q8 column 0 = e_{n_i} (scale 2^f):
    delta[b, n_i] = scale_i 2^(e+f) x[b, k_i] exactly and zero elsewhere, so a
    wrong scale offset, value offset or row stride shows bit for bit.  The
    segment length picks the path: single-row decode, multi-row decode, or
    matrix cores."""
    slots, d_in, d_out, rank = 6, 2048 + 8, 1032, 24
    rng = np.random.default_rng(seg_len)
    ks = rng.choice(d_in, slots, replace=False)
    ns = rng.choice(d_out, slots, replace=False)
    ea = rng.integers(-3, 3, size=slots)
    eb = rng.integers(-3, 3, size=slots)
    scales = np.tile(np.array([1.0, 0.5, 2.0, 0.25, 1.0, 4.0], np.float32)[:, None], (1, 7))

    def fill(w):
        for a in range(slots):
            sa, qa = w.A_q8(a, 0)
            sb, qb = w.B_q8(a, 0)
            qa[:] = 0
            qb[:] = 0
            sa[:] = rng.uniform(0.5, 3.0, size=sa.shape)   # rows other than 0 meet zeros
            sb[:] = rng.uniform(0.5, 3.0, size=sb.shape)
            sa[0] = 2.0 ** ea[a]
            sb[ns[a]] = 2.0 ** eb[a]
            qa[0, ks[a]] = 1
            qb[ns[a], 0] = 1
    ids = rng.permutation(np.repeat(np.arange(slots), seg_len))
    rows = ids.size
    w = bw(340 + seg_len, rows, slots, d_in, d_out, rank, ids, ab_fill=fill, x_std=1.0, fmt=Q8, scales=scales)
    x = bf16_to_f32(w.x["x"]).astype(np.float64)
    want = np.zeros((rows, d_out))
    r = np.arange(rows)
    want[r, ns[ids]] = x[r, ks[ids]] * scales[ids, 0] * 2.0 ** (ea[ids] + eb[ids])
    for runner in ("split", "layer"):
        dw = DeviceWorkload(w)
        dw.reset_y(zero=True)
        RUNNERS[runner](dw)
        torch.cuda.synchronize()
        got = bf16_host(dw.y["q"])
        assert np.array_equal(got, want), runner


def test_int8_paged_table():
    # fixed-size pages sized for either format, adapters placed out of order
    w = gen.make_workload("zipf_paged")
    rng = np.random.default_rng(9)
    fmt = np.where(rng.random((w.num_slots, gen.N_MOD)) < 0.5, Q8, gen.FMT_BF16).astype(np.int32)
    w2 = gen.build_workload("zipf_paged_int8", w.seed, w.num_rows, w.num_slots,
                            {m.name: (m.d_in, m.d_out) for m in w.modules}, w.ids, w.ranks,
                            x_of={m.name: m.x_name for m in w.modules}, x_std=1.0,
                            paged_capacity_rank=int(w.ranks.max()),
                            placement=rng.permutation(w.num_slots), fmt=fmt)
    check_workload(w2, oracle.lora_layer(w2), "layer")


@pytest.mark.parametrize("fmt", ["int8", "bf16"])
def test_int8_items_flag_with_either_format(fmt):
    # LORA_MASK_INT8_ITEMS only sizes the shrink's items (twice the k): with
    # or without it, and on bf16 entries too, the delta is within tolerance;
    # the split call with the flag on both parts equals the whole call
    from tests.parity import check_rows
    rows, slots, d_in, d_out = 96, 96, 8192, 1032
    ids = np.random.default_rng(9).permutation(rows)
    w = bw(330, rows, slots, d_in, d_out, 64, ids, x_std=1.0, fmt=Q8 if fmt == "int8" else gen.FMT_BF16)
    ref = oracle.lora_layer(w)["q"]
    dw = DeviceWorkload(w)
    import adapter_gemv_amd as lg
    outs = {}
    for flag in (False, True):
        mask = lg.module_mask(dw.ios, int8_items=flag)
        dw.reset_y(zero=True)
        dw.build_segments()
        lg.apply_layer(dw.ios, rows, dw.table, slots, dw.seg, w.max_rank, dw.ws, module_mask=mask)
        torch.cuda.synchronize()
        outs[flag] = bf16_host(dw.y["q"])
        check_rows(outs[flag], ref.delta, f"{fmt} delta, int8 items {flag}")
    mask = lg.module_mask(dw.ios, int8_items=True)
    dw.reset_y(zero=True)
    dw.build_segments()
    lg.layer_shrink(dw.ios, rows, dw.table, slots, dw.seg, w.max_rank, dw.ws, module_mask=mask)
    lg.layer_expand(dw.ios, rows, dw.table, slots, dw.seg, w.max_rank, dw.ws, module_mask=mask)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_host(dw.y["q"]), outs[True])
