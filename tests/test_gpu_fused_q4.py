"""GPU parity of the fused base projection + delta with 4-bit base weights
(lora_linear_layer_q4): y = bf16(W.x + delta), W[n][k] = s[n][k // 128] *
q[n][k], against the oracle's fp64 y.  "12. Adapter Serving and Multi-Tenant
Customization", "Interactions with other engine mechanisms", Quantization:
an INT4 base with BF16 adapters in one batch with base-only rows."""
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


def run(w, dw=None, phases=False, bound_segments=False):
    dw = dw or DeviceWorkload(w, bound_segments=bound_segments)
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
    return {m.name: bf16_host(dw.y[m.name]) for m in w.modules}, dw


def check_q4(w, rows=None, bound_segments=False):
    ref = oracle.linear_layer(w, rows=rows)
    got, _ = run(w, bound_segments=bound_segments)
    for m in w.modules:
        g = got[m.name] if rows is None else got[m.name][rows]
        assert np.isfinite(g).all(), m.name
        check_rows(g, ref[m.name].y, f"{w.name}/{m.name} q4 fused y")


SHAPES = [
    # rows, slots, d_in, d_out, ranks, id mode
    (1, 1, 1024, 72, 8, "distinct"),
    (37, 37, 2048, 1000, (16, 0, 64, 5, 33), "distinct"),
    (128, 128, 4096, 1024, 64, "distinct"),
    (129, 40, 1024, 4104, (8, 16, 24), "random"),    # base-only and out-of-range ids in the batch
    (200, 9, 3072, 520, (64, 1, 40), "random"),
    (16, 4, 128, 8, 8, "random"),                    # one group, one column tile
    (96, 30, 8320, 264, (8, 64, 0, 32), "random"),   # 65 groups of inputs
    (140, 140, 12288, 136, 64, "distinct"),          # 96 groups, two row tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"r{s[0]}_{s[2]}x{s[3]}" for s in SHAPES])
def test_q4_shapes(shape):
    rows, slots, d_in, d_out, rank, mode = shape
    rng = np.random.default_rng(rows + d_out + 1)
    ids = {"distinct": rng.permutation(rows) % slots, "random": rng.integers(-1, slots + 2, size=rows)}[mode]
    ranks = np.zeros((slots, 7), np.int32)
    ranks[:, 0] = np.resize(np.asarray(rank), slots)
    scales = np.zeros((slots, 7), np.float32)
    scales[:, 0] = rng.uniform(0.5, 2.0, size=slots)
    w = gen.add_base_weights_q4(bw(500 + rows, rows, slots, d_in, d_out, None, ids, ranks=ranks, scales=scales,
                                   x_std=1.0, max_rank=64))
    check_q4(w)


@pytest.mark.parametrize("seed", range(2))
def test_q4_mixed_formats_projections_and_long_segments(seed):
    rng = np.random.default_rng(510 + seed)
    names = ["q", "k", "o"] if seed == 0 else ["gate", "down"]
    shapes = {n: (128 * int(rng.integers(2, 24)), 8 * int(rng.integers(16, 400))) for n in names}
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
    w = gen.build_workload(f"q4fused{seed}", 510 + seed, ids.size, slots, shapes, ids, ranks, x_std=1.0,
                           scales=scales, fmt=fmt)
    note(f"q4 fused seed {seed}: {ids.size} rows, {[(m.name, m.d_in, m.d_out) for m in w.modules]}")
    check_q4(gen.add_base_weights_q4(w))


def test_q4_one_hot_bit_exact():
    """q[n, k_n] = 1 with power-of-two group scales s_n and adapter a with
    A = e_{ka}, B = e_{na}: y[b, n] = bf16(s_n x[b, k_n] + [n == n_a] x[b, k_a]),
    exactly (every product and sum is exact before the one rounding)."""
    rows, slots, d_in, d_out, rank = 150, 30, 2048, 1032, 16
    rng = np.random.default_rng(17)
    kw = rng.integers(0, d_in, size=d_out)
    sw = np.exp2(rng.integers(-2, 3, size=d_out)).astype(np.float32)
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
    q = np.zeros((d_out, d_in), np.int64)
    q[np.arange(d_out), kw] = 1
    nib = q.astype(np.uint8)
    scales = np.exp2(rng.integers(-4, 4, size=(d_out, d_in // 128))).astype(np.float32)  # unused groups: any value
    scales[np.arange(d_out), kw // 128] = sw
    w.W = {"q": gen.Q4Weight((nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8), scales, 128, d_in, d_out)}
    x = bf16_to_f32(w.x["x"])
    want = x[:, kw] * sw
    r = np.arange(rows)
    on = ids >= 0
    want[r[on], na[ids[on]]] += x[r[on], ka[ids[on]]]
    want = bf16_to_f32(gen.bf16_bits(want)).astype(np.float64)
    got, _ = run(w)
    assert np.array_equal(got["q"], want)


def test_q4_padded_rows_of_weights_and_scales():
    # ldwq and lds past the row: the kernel reads d_in / 2 bytes and d_in / 128 scales of each row
    rows, slots, d_in, d_out = 64, 16, 1024, 520
    ids = np.random.default_rng(5).integers(-1, slots, size=rows)
    w = gen.add_base_weights_q4(bw(520, rows, slots, d_in, d_out, 32, ids, x_std=1.0))
    ref = oracle.linear_layer(w)["q"].y
    dw = DeviceWorkload(w)
    W = w.W["q"]
    qpad = torch.full((d_out, d_in // 2 + 48), 0x77, dtype=torch.uint8, device="cuda")
    qpad[:, :d_in // 2] = torch.from_numpy(W.q).cuda()
    spad = torch.full((d_out, d_in // 128 + 5), 1e30, dtype=torch.float32, device="cuda")
    spad[:, :d_in // 128] = torch.from_numpy(W.scales).cuda()
    dw.lin_ios["q"] = lg.LinearQ4IO(dw.x["x"], qpad, spad, dw.y["q"], d_in=d_in, d_out=d_out)
    got, _ = run(w, dw=dw)
    check_rows(got["q"], ref, "q4 padded rows")


def test_q4_phases_equal_the_whole_call():
    ids = np.random.default_rng(13).integers(-1, 20, size=90)
    w = gen.add_base_weights_q4(bw(530, 90, 20, 2048, 1040, 32, ids, x_std=1.0))
    whole, dw = run(w)
    split, _ = run(w, dw=dw, phases=True)
    assert np.array_equal(whole["q"], split["q"])


def test_q4_full_layer_sampled_rows():
    # the 70B layer at rank 64 with 4-bit base weights; 8 of its 128 rows base-only
    w = gen.make_workload("fused_layer_q4_r64")
    rows = np.random.default_rng(2).choice(w.num_rows, 6, replace=False).astype(np.int32)
    rows[0] = 0  # a base-only row (ids[::16] = -1)
    note(f"q4 fused full layer: rows {list(rows)}")
    check_q4(w, rows=rows, bound_segments=True)


def test_q4_repeated_calls_same_bits():
    # later calls on the same workspace give the same bits
    ids = np.random.default_rng(14).integers(-1, 20, size=100)
    w = gen.add_base_weights_q4(bw(531, 100, 20, 8320, 264, 32, ids, x_std=1.0))
    first, dw = run(w)
    assert np.isfinite(first["q"]).all()
    again, _ = run(w, dw=dw)
    assert np.array_equal(again["q"], first["q"])
    phases, _ = run(w, dw=dw, phases=True)
    assert np.array_equal(phases["q"], first["q"])
