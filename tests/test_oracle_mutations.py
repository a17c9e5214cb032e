"""The oracle's pins are sensitive: each plausible mistake planted in a copy of
the oracle's C source (on the CPU, in a temporary library) fails at least one
pin from ``test_oracle_pins``.  The real oracle is untouched.
"""
import ctypes
import subprocess

import pytest

import oracle
import tests.test_fused_oracle as fused
import tests.test_oracle_pins as pins

SRC = open(oracle._SRC).read()

MUTATIONS = {
    "drop_last_k": ("for (int32_t k = 0; k < d_in; ++k)", "for (int32_t k = 0; k < d_in - 1; ++k)"),
    "wrong_sign": ("s += bf16_value(a[k]) * bf16_value(x[k]);", "s -= bf16_value(a[k]) * bf16_value(x[k]);"),
    "A_transposed": ("s += bf16_value(a[k]) * bf16_value(x[k]);",
                     "s += bf16_value(A[(int64_t)k * rank + j]) * bf16_value(x[k]); (void)a;"),
    "B_transposed": ("s += bf16_value(b[j]) * v[j];", "s += bf16_value(B[(int64_t)j * d_out + n]) * v[j]; (void)b;"),
    "B_compact_rows": ("const uint16_t *b = B + (int64_t)n * ldb;", "const uint16_t *b = B + (int64_t)n * rank; (void)ldb;"),
    "drop_last_rank_term": ("for (int32_t j = 0; j < rank; ++j)\n            s += bf16_value(b[j])",
                            "for (int32_t j = 0; j < rank - 1; ++j)\n            s += bf16_value(b[j])"),
    "no_scale": ("delta[n] = scale * s;", "delta[n] = s; (void)scale;"),
    "wrong_row_adapter": ("int32_t a = (b >= 0 && b < num_rows) ? ids[b] : -1;",
                          "int32_t a = (b >= 0 && b < num_rows) ? ids[(b + 1) % num_rows] : -1;"),
    "no_base_output": ("bf16_value(y0[(int64_t)b * ldy + n]) + dr[n];", "dr[n]; (void)y0;"),
    "unstable_segments": ("for (int32_t b = 0; b < num_rows; ++b)\n            if (ids[b] == a)",
                          "for (int32_t b = num_rows - 1; b >= 0; --b)\n            if (ids[b] == a)"),
    "keeps_bad_ids": ("if (ids[b] >= num_slots)\n            ++bad;", "if (ids[b] >= num_slots)\n            bad += 0;"),
    "q8_no_A_scale": ("s += ((double)sa[j] * (double)a[k]) * bf16_value(x[k]);",
                      "s += ((double)a[k]) * bf16_value(x[k]); (void)sa;"),
    "q8_B_scale_by_column": ("s += ((double)sb[n] * (double)b[j]) * v[j];",
                             "s += ((double)sb[j] * (double)b[j]) * v[j];"),
    "q8_B_rows_by_rank": ("const int8_t *b = qb + (int64_t)n * ldb8;",
                          "const int8_t *b = qb + (int64_t)n * rank; (void)ldb8;"),
    "q8_A_rows_by_d_in": ("const int8_t *a = qa + (int64_t)j * lda8;",
                          "const int8_t *a = qa + (int64_t)j * d_in; (void)lda8;"),
    "q8_A_values_after_rank_scales": ("(const int8_t *)(sa + round_up(rank, 4))", "(const int8_t *)(sa + rank)"),
    "q8_B_values_after_d_out_scales": ("(const int8_t *)(sb + round_up(d_out, 4))", "(const int8_t *)(sb + d_out)"),
    "base_W_transposed": ("s += bf16_value(w[k]) * bf16_value(xr[k]);",
                          "s += bf16_value(W[(int64_t)k * d_out + n]) * bf16_value(xr[k]); (void)w;"),
    "base_drop_last_k": ("for (int32_t k = 0; k < d_in; ++k)\n                s += bf16_value(w[k])",
                         "for (int32_t k = 0; k < d_in - 1; ++k)\n                s += bf16_value(w[k])"),
    "q4_nibbles_swapped": ("uint32_t nib = (k % 2 == 0) ? (row[k / 2] & 0xFu) : (row[k / 2] >> 4);",
                           "uint32_t nib = (k % 2 == 1) ? (row[k / 2] & 0xFu) : (row[k / 2] >> 4);"),
    "q4_unsigned": ("return nib >= 8 ? (int32_t)nib - 16 : (int32_t)nib;", "return (int32_t)nib;"),
    "q4_offset_binary": ("return nib >= 8 ? (int32_t)nib - 16 : (int32_t)nib;", "return (int32_t)nib - 8;"),
    "q4_group_by_modulo": ("s += ((double)sc[k / group]", "s += ((double)sc[k % group]"),
    "q4_no_scale": ("s += ((double)sc[k / group] * (double)q4_value(q, k)) * bf16_value(xr[k]);",
                    "s += ((double)q4_value(q, k)) * bf16_value(xr[k]); (void)sc;"),
    "q4_rows_by_d_in": ("const uint8_t *q = Wq + (int64_t)n * ldwq;",
                        "const uint8_t *q = Wq + (int64_t)n * (d_in / 2); (void)ldwq;"),
    "q4_scale_rows_by_groups": ("const float *sc = Ws + (int64_t)n * lds;",
                                "const float *sc = Ws + (int64_t)n * (d_in / group); (void)lds;"),
}

CHECKS = [
    (pins.test_exact_rational, dict(d_in=8, d_out=16, rank=8, rows=6, slots=3)),
    (pins.test_exact_rational, dict(d_in=24, d_out=8, rank=3, rows=5, slots=4)),
    (pins.test_against_blas_medium, {}),
    (pins.test_one_hot_gather_closed_form, {}),
    (pins.test_identity_adapter, {}),
    (pins.test_merged_weight_identity, {}),
    (pins.test_zero_cases_leave_y_exactly, {}),
    (pins.test_segments_vs_stable_sort, dict(n=257, slots=9, seed=3)),
    (pins.test_int8_matches_bf16_twin_exactly, dict(d_in=24, d_out=10, rank=5, rows=6, slots=3)),
    (pins.test_int8_exact_rational, {}),
    (fused.test_one_hot_base_weights_gather_x_exactly, {}),
    (fused.test_base_projection_exact_rational, {}),
    (fused.test_q4_matches_its_bf16_twin_exactly, {}),
    (fused.test_q4_exact_rational, {}),
    (fused.test_q4_one_hot_gathers_scaled_x, {}),
    (fused.test_q4_codes_decode_in_order, {}),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTATIONS[name]
    assert SRC.count(old) >= 1, name
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new, 1))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-o", str(so), str(src)], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle._configure(ctypes.CDLL(str(so))))
    caught = []
    for fn, kw in CHECKS:
        try:
            fn(**kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
