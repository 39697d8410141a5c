"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is a one-spot textual change to oracle/maxsim_oracle.c (a dropped term, a
wrong sign, a wrong index or bound, a transposed operand, a wrong initial value, a
wrong rounding step). The mutated source is compiled with gcc into a temporary
library on the CPU and the whole pin suite is run against it.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("max_becomes_sum", "if (s > m) { /* strict: the first maximum is kept */\n        m = s;",
     "{\n        m = (m == -INFINITY ? 0.0 : m) + s;"),
    ("max_init_zero", "double m = -INFINITY;", "double m = 0.0;"),
    ("drop_last_doc_token", "for (int64_t j = 0; j < len; j++) {\n      double s = 0.0;\n      for (int k",
     "for (int64_t j = 0; j < len - 1; j++) {\n      double s = 0.0;\n      for (int k"),
    ("drop_last_dim", "for (int k = 0; k < c->d; k++)\n        s += c->q",
     "for (int k = 0; k < c->d - 1; k++)\n        s += c->q"),
    ("drop_last_query_token", "for (int i = 0; i < c->q_len; i++) {\n    double m = -INFINITY;",
     "for (int i = 0; i < c->q_len - 1; i++) {\n    double m = -INFINITY;"),
    ("sign_flip", "s += c->q[(int64_t)i * c->d + k] *", "s -= c->q[(int64_t)i * c->d + k] *"),
    ("query_transposed", "c->q[(int64_t)i * c->d + k]", "c->q[(int64_t)k * c->q_len + i]"),
    ("doc_index_swapped", "decode(c->D, c->dtype, (first + j) * c->d + k)",
     "decode(c->D, c->dtype, (first + k) * c->d + j)"),
    ("ignore_doc_lens", "len = c->doc_lens[b];", "len = c->nd;"),
    ("csr_wrong_start", "first = c->offsets[b];\n    len", "first = c->offsets[b] + 1;\n    len"),
    ("bf16_wrong_shift", "(uint32_t)h << 16", "(uint32_t)h << 15"),
    ("fp16_subnormal_exponent", "ldexp((double)man, -24)", "ldexp((double)man, -25)"),
    ("fp16_normal_exponent", "ldexp((double)(1024 + man), exp - 25)",
     "ldexp((double)(1024 + man), exp - 24)"),
    ("fp16_hidden_bit", "(double)(1024 + man)", "(double)(man)"),
    ("i8_scale_in_double", "volatile float v = (float)dot * scale;",
     "volatile float v = (float)((double)dot * (double)c->qs[i] * (double)c->ds[first + j]);"),
    ("i8_drop_doc_scale", "volatile float scale = c->qs[i] * c->ds[first + j];",
     "volatile float scale = c->qs[i];"),
    ("i8_ties_to_highest", "if (v > m) { /* strict", "if (v >= m) { /* strict"),
    ("i8_max_before_scale", "if (v > m) { /* strict",
     "if ((float)dot * c->qs[i] > m) { /* strict"),
    ("i8_doc_scale_index", "c->ds[first + j]; /* one", "c->ds[j]; /* one"),
    ("pq_table_transposed", "s += c->T[((int64_t)i * c->M + m) * c->K + code];",
     "s += c->T[((int64_t)i * c->K + code) * c->M + m];"),
    ("pq_subvector_interleaved", "decode(Q, dtype, (int64_t)i * d + (int64_t)m * dsub + t)",
     "decode(Q, dtype, (int64_t)i * d + (int64_t)t * M + m)"),
    ("pq_centroid_index", "(double)C[((int64_t)m * K + k) * dsub + t]",
     "(double)C[((int64_t)k * M + m) * dsub + t]"),
    ("pq_code_index", "c->codes[(first + j) * c->M + m]", "c->codes[(first + m) * c->M + j]"),
    ("pq_max_init_zero", "double mx = -INFINITY;", "double mx = 0.0;"),
    ("argmax_ties_to_highest", "if (s > m) { /* strict: the first", "if (s >= m) { /* strict: the first"),
    ("argmax_off_by_one", "m = s;\n        arg = (int32_t)j;", "m = s;\n        arg = (int32_t)j + 1;"),
    ("bwd_drop_grad", "const double g = (double)grad[b];", "const double g = 1.0;"),
    ("bwd_dD_sign", "dD[(first + j) * d + k] += g", "dD[(first + j) * d + k] -= g"),
    ("bwd_dD_wrong_row", "dD[(first + j) * d + k] += g", "dD[(first + (j + 1) % len) * d + k] += g"),
    ("bwd_dQ_wrong_row", "g * decode(D, dtype, (first + j) * d + k)",
     "g * decode(D, dtype, (first + (len - 1 - j)) * d + k)"),
    ("bwd_dQ_transposed", "dQ[(int64_t)i * d + k] += g", "dQ[(int64_t)k * q_len + i] += g"),
    ("bwd_skip_first_query", "for (int i = 0; i < q_len; i++) {\n      const int64_t j",
     "for (int i = 1; i < q_len; i++) {\n      const int64_t j"),
    ("bwd_tok_arg_transposed", "const int64_t j = tok_arg[b * q_len + i];",
     "const int64_t j = tok_arg[(int64_t)i * n_docs + b];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    so = oracle.compile_oracle(str(path), str(tmp_path / f"lib_{name}.so"))
    orc = oracle.Oracle(so)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except ValueError:
            caught.append(pin.__name__ + "(rejected)")
        if caught:
            break
    assert caught, f"mutant {name} passed every pin"


def test_mutant_sites_are_distinct():
    src = open(oracle.SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, name
    assert len({m[0] for m in MUTANTS}) == len(MUTANTS)
    assert os.path.exists(oracle.SRC)
