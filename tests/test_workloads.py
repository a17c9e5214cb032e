"""The seeded input generators: determinism, bf16 rounding, and the recipes
of the five workloads (shapes, id distributions, paging)."""
import numpy as np
import torch

from workloads import bf16_bits, bf16_to_f32, gen, normal_bf16


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38], np.float32)]).astype(np.float32)
    ours = bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # ties go to even
    assert bf16_bits(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert bf16_bits(np.array([1.01171875], np.float32))[0] == 0x3F82


def test_draws_are_deterministic_and_thread_independent():
    a = normal_bf16(7, (1, 2), 3 * (1 << 22) + 5, 0.02)
    b = normal_bf16(7, (1, 2), 3 * (1 << 22) + 5, 0.02)
    assert np.array_equal(a, b)
    c = normal_bf16(7, (1, 3), 1000, 0.02)
    assert not np.array_equal(a[:1000], c)
    f = bf16_to_f32(a).astype(np.float64)
    assert abs(f.std() - 0.02) < 1e-3 and abs(f.mean()) < 1e-3


def test_tiny_recipe():
    w = gen.tiny()
    assert w.num_rows == 16 and w.num_slots == 4 and w.max_rank == 8
    assert w.x["x"].shape == (16, 256) and w.y0["q"].shape == (16, 256)
    assert w.ids.min() >= 0 and w.ids.max() < 4
    assert w.A(0, 0).shape == (8, 256) and w.B(3, 0).shape == (256, 8)
    w2 = gen.tiny()
    assert np.array_equal(w.pool, w2.pool) and np.array_equal(w.ids, w2.ids)


def test_zipf_ids():
    ids = gen.zipf_ids(4, 200000, 512, 1.1)
    counts = np.bincount(ids, minlength=512)
    k = np.arange(1, 513.0)
    p = k ** -1.1
    p /= p.sum()
    top = np.sort(counts)[::-1][:5] / ids.size
    assert np.allclose(top, p[:5], atol=0.005)


def test_zipf_paged_recipe():
    w = gen.zipf_paged()
    assert w.num_rows == 256 and w.num_slots == 512
    assert set(np.unique(w.ranks[:, :4])) <= {8, 16, 32, 64}
    assert np.all(w.ranks[:, 4:] == 0)
    # each adapter sits in its own fixed-size page
    page = w.pool.size // 512
    pages = w.a_off[:, 0] // page
    assert len(np.unique(pages)) == 512


def test_prefill_lengths():
    lens = gen._rng(5, gen._R_LEN).integers(128, 2049, size=32)
    assert lens.min() >= 128 and lens.max() <= 2048
