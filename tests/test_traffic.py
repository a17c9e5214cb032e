"""The roofline byte accounting of the package agrees with the oracle's cost
model (written separately from the pages' byte model) on every workload."""
import pytest

from adapter_gemv_amd.traffic import step_traffic
from oracle import costmodel
from workloads import gen


@pytest.mark.parametrize("name", ["tiny", "q_proj_r16", "zipf_paged"])
def test_traffic_matches_costmodel(name):
    w = gen.make_workload(name)
    mods = [(m.name, m.index, m.d_in, m.d_out, m.x_name) for m in w.modules]
    t = step_traffic(w.ids, w.num_slots, mods, w.ranks)
    ref = costmodel.algorithmic_bytes(w.ids, [(m.name, m.d_in, m.d_out, m.x_name) for m in w.modules],
                                      lambda a, n: int(w.ranks[a, w.module(n).index]), None)
    for k in ("adapters", "x", "y", "total", "flops"):
        assert t[k] == ref[k], k
    assert t["shrink_bytes"] + t["expand_bytes"] == t["total"]


def test_full_layer_bytes():
    # 128 rows, 128 distinct rank-64 adapters, 7 projections: 2,707 MB
    w_ids = list(range(128))
    import numpy as np
    ranks = np.full((128, 7), 64)
    mods = [(n, i, *costmodel.SHAPES_70B[n], x) for i, (n, x) in enumerate(
        [("q", "a"), ("k", "a"), ("v", "a"), ("o", "b"), ("gate", "c"), ("up", "c"), ("down", "d")])]
    t = step_traffic(w_ids, 128, mods, ranks)
    assert abs(t["total"] / 1e6 - 2707.5) < 1.0
