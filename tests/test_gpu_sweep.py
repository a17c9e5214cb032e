"""Randomised GPU parity sweep over small multi-projection batches.

Each seeded case draws its projections (1 to 3 of q/k/v/o/gate/up/down)
with dimensions that are multiples of 8 but not of 512.  Slots carry ranks
in [0, 64] (ranks that are not multiples of 8 included) and random scales.
A skewed id draw gives short segments (decode path) and long ones
(matrix-core path) in one batch; base-only rows (id -1) and ids past the
table are mixed in.  The launch-shape choices the host makes from these
sizes (k-chunks, n-tiles, which segments go to the matrix cores) are all
exercised; every case is compared with the oracle on the delta alone, on y,
and on v through the single-projection calls.  The mixed-format cases make
about half the (slot, projection) entries int8 with row scales.
"""
import numpy as np
import pytest

import oracle
from tests.parity import note
from workloads import gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from tests.test_gpu_decode import check_workload  # noqa: E402
from workloads.device import DeviceWorkload  # noqa: E402

RANK_CHOICES = np.array([0, 1, 3, 8, 13, 16, 24, 32, 40, 57, 64])


def random_case(seed: int, big: bool = False, int8: bool = False):
    rng = np.random.default_rng(7000 + seed)
    names = list(rng.choice(gen.MODULE_NAMES, size=int(rng.integers(1, 4)), replace=False))
    dmax = 160 if big else 400
    shapes = {n: (8 * int(rng.integers(1, dmax)), 8 * int(rng.integers(1, dmax))) for n in names}
    rows = int(rng.integers(2048, 2600)) if big else int(rng.integers(1, 300))
    slots = int(rng.integers(1, 40 if big else 200))
    # skewed popularity: a few slots get long runs of rows
    p = 1.0 / np.arange(1, slots + 1) ** 1.3
    p = p[rng.permutation(slots)]
    ids = rng.choice(slots, size=rows, p=p / p.sum()).astype(np.int32)
    ids[rng.random(rows) < 0.05] = -1
    bad = rng.random(rows) < 0.02
    ids[bad] = slots + rng.integers(0, 5, size=int(bad.sum()))
    cap = int(rng.choice([8, 16, 32, 64]))  # the launch's rank class varies by case
    ranks = np.zeros((slots, gen.N_MOD), np.int32)
    for n in names:
        ranks[:, gen.MODULE_INDEX[n]] = rng.choice(RANK_CHOICES[RANK_CHOICES <= cap], size=slots)
    scales = rng.uniform(0.25, 2.0, size=(slots, gen.N_MOD)).astype(np.float32)
    max_rank = max(1, int(ranks.max()))
    if rng.random() < 0.3:
        max_rank = min(64, max_rank + int(rng.integers(1, 16)))  # a launch class above the largest entry
    fmt = None
    if int8:  # about half the entries int8 with row scales
        fmt = np.where(rng.random((slots, gen.N_MOD)) < 0.5, gen.FMT_INT8_ROWS, gen.FMT_BF16).astype(np.int32)
    w = gen.build_workload(f"sweep{seed}", 7000 + seed, rows, slots, shapes, ids, ranks, x_std=1.0, scales=scales,
                           max_rank=max_rank, fmt=fmt)
    return w


@pytest.mark.parametrize("seed", range(14))
def test_random_layer_case(seed):
    w = random_case(seed)
    runner = ("split", "layer", "phases")[seed % 3]
    note(f"sweep seed {seed}: {w.num_rows} rows, {w.num_slots} slots, "
         f"{[(m.name, m.d_in, m.d_out) for m in w.modules]}, max_rank {w.max_rank}, runner {runner}")
    check_workload(w, oracle.lora_layer(w), runner)


@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("seed", range(14))
def test_random_decode_layer_case(seed, int8):
    # the same batches through lora_decode_layer: one launch where the batch
    # fits it (at most 256 rows, launch rank class at most 32), the three
    # launches otherwise; both kinds occur among the seeds
    w = random_case(seed if not int8 else 300 + seed, int8=int8)
    dw = DeviceWorkload(w)
    launches = dw.decode_launches()
    note(f"sweep decode seed {seed} int8 {int8}: {w.num_rows} rows, {w.num_slots} slots, "
         f"{[(m.name, m.d_in, m.d_out) for m in w.modules]}, max_rank {w.max_rank}, launches {launches}")
    assert launches in (1, 3)
    check_workload(w, oracle.lora_layer(w), "decode")


@pytest.mark.parametrize("seed", range(2))
def test_random_prefill_sized_case(seed):
    # at least 2048 rows: the prefill-sized chunking, with short and long segments
    w = random_case(100 + seed, big=True)
    runner = ("split", "layer")[seed % 2]
    note(f"sweep big seed {seed}: {w.num_rows} rows, {w.num_slots} slots, "
         f"{[(m.name, m.d_in, m.d_out) for m in w.modules]}, max_rank {w.max_rank}, runner {runner}")
    check_workload(w, oracle.lora_layer(w), runner)


@pytest.mark.parametrize("seed", range(6))
def test_random_mixed_format_case(seed):
    w = random_case(200 + seed, big=seed == 5, int8=True)
    runner = ("split", "layer", "phases")[seed % 3]
    note(f"sweep int8 seed {seed}: {w.num_rows} rows, {w.num_slots} slots, "
         f"{[(m.name, m.d_in, m.d_out) for m in w.modules]}, max_rank {w.max_rank}, runner {runner}")
    check_workload(w, oracle.lora_layer(w), runner)
