"""The pages' printed figures, reproduced from the cost model's formulas.

Each figure comes from tests/golden/pages_figures.json with its page and
section.  A wrong shape, a dropped projection or a wrong factor of two in
``oracle.costmodel`` moves at least one of these outside its printed rounding.
"""
import json
import os

import pytest

from oracle import costmodel as cm

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")))
FIG = {f["id"]: f for f in GOLD["figures"]}

ATT, ALL = cm.ATTENTION, cm.ALL_MODULES
GIB = 2 ** 30
KV_BUDGET_GIB = 172.5


def computed():
    att8 = cm.adapter_bytes(8, ATT)
    att16 = cm.adapter_bytes(16, ATT)
    all64 = cm.adapter_bytes(64, ALL)
    return {
        "flops_ratio_pct": 100 * cm.lora_flops_per_token(16, 8192, 8192) / cm.base_flops_per_token(8192, 8192),
        "base_flops_8192": cm.base_flops_per_token(8192, 8192),
        "lora_flops_r16_8192": cm.lora_flops_per_token(16, 8192, 8192),
        "lora_flops_share_pct_p2": 100 * cm.lora_flops_per_token(16, 8192, 8192) / cm.base_flops_per_token(8192, 8192),
        "pair_bytes_r16": cm.pair_bytes(16),
        "attn_adapter_r16_dxd_bytes": cm.adapter_bytes(16, ATT, shapes=cm.SHAPES_DXD),
        "attn_r8_bytes_MB": att8 / 1e6,
        "all_r64_bytes_GB": all64 / 1e9,
        "all_r64_bytes_GB_intro": all64 / 1e9,
        "attn_r8_share_pct": 100 * att8 / cm.BASE_BYTES_70B,
        "all_r64_share_pct": 100 * all64 / cm.BASE_BYTES_70B,
        "extra_attn_r8_b128_pct": 100 * cm.extra_decode_bytes_fraction(8, ATT, 128),
        "extra_all_r64_b128_pct": 100 * cm.extra_decode_bytes_fraction(64, ALL, 128),
        "extra_all_r64_b64_pct": 100 * cm.extra_decode_bytes_fraction(64, ALL, 64),
        "extra_all_r64_cap32_pct": 100 * cm.extra_decode_bytes_fraction(64, ALL, 32),
        "cost_spread": all64 / att8,
        "mlp_factor": cm.adapter_params_per_layer(1, ALL) / cm.adapter_params_per_layer(1, ATT),
        "ffn_over_hidden": cm.FFN_DIM / cm.D_MODEL,
        "kv_share_100_attn_r8_pct": 100 * 100 * att8 / GIB / KV_BUDGET_GIB,
        "kv_share_100_attn_r16_pct": 100 * 100 * att16 / GIB / KV_BUDGET_GIB,
        "kv_share_100_all_r64_pct": 100 * 100 * all64 / GIB / KV_BUDGET_GIB,
    }


@pytest.mark.parametrize("fid", sorted(FIG))
def test_printed_figure(fid):
    got = computed()[fid]
    f = FIG[fid]
    assert abs(got - f["printed"]) <= f["tol"] + 1e-12, (fid, got, f["printed"], f["cite"])


def test_every_golden_figure_is_checked():
    assert set(FIG) == set(computed())


def test_parameter_count_per_module():
    # r * (d_in + d_out): exact values for the 70B shapes.
    assert cm.lora_params(16, 8192, 8192) == 262144
    assert cm.lora_params(8, 8192, 1024) == 73728
    assert cm.adapter_params_per_layer(1, ATT) == 51200
    assert cm.adapter_params_per_layer(1, ("gate", "up", "down")) == 110592
    # one A,B pair of rank 16 on 8192 x 8192 is 512 KiB of bf16
    assert 2 * cm.lora_params(16, 8192, 8192) == 512 * 1024


def test_envelope():
    env = GOLD["envelope"]
    mods = {"attention": ATT, "all": ALL}
    for m, r, b in env["inside"]:
        assert cm.extra_decode_bytes_fraction(r, mods[m], b) < 0.10, (m, r, b)
    for m, r, b in env["outside"]:
        assert cm.extra_decode_bytes_fraction(r, mods[m], b) > 0.10, (m, r, b)


def test_algorithmic_bytes_full_layer():
    # 128 rows, 128 distinct rank-64 adapters on all seven projections:
    # adapters 2 * 64 * 161792 * 128 bytes, x once per input tensor, y read+write.
    mods = [(n, *cm.SHAPES_70B[n], x) for n, x in
            [("q", "qkv"), ("k", "qkv"), ("v", "qkv"), ("o", "o"), ("gate", "gu"), ("up", "gu"), ("down", "d")]]
    r = cm.algorithmic_bytes(list(range(128)), mods, lambda a, n: 64, {"qkv", "o", "gu", "d"})
    assert r["adapters"] == 2 * 64 * 161792 * 128
    assert r["x"] == 2 * 128 * (8192 * 3 + 28672)
    assert r["y"] == 4 * 128 * (8192 * 2 + 1024 * 2 + 28672 * 2 + 8192)
    assert abs(r["total"] / 1e6 - 2707) < 1
    # shared adapter: one read however many rows use it
    r1 = cm.algorithmic_bytes([5] * 64, mods[:1], lambda a, n: 16, {"qkv"})
    assert r1["adapters"] == 2 * 16 * 16384
