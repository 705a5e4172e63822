"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins
catch every one of them: a pin set that a dropped term, a wrong sign or index or a
transposed operand slips through would not be pinning anything."""
import os

import pytest

import oracle_pins as P

ORACLE_SRC = os.path.join(P.GOLDEN, "..", "..", "oracle", "pa_oracle.c")

# (name, text in pa_oracle.c, replacement)
MUTANTS = [
    ("gqa_modulo_map", "int g = h / group;", "int g = h % p->kv_heads;"),
    ("scale_divides", "return p->scale * dot;", "return dot / p->scale;"),
    ("no_max_shift", "double w = exp(s[t] - m);", "double w = exp(s[t]);"),
    ("slot_from_division", "long long slot = t % p->page_size;", "long long slot = t / p->page_size % p->page_size;"),
    ("page_major_heads", "((phys * p->page_size + slot) * p->kv_heads + g)",
     "((phys * p->kv_heads + g) * p->page_size + slot)"),
    ("ignore_block_table", "long long phys = p->block_tables[(size_t)b * p->max_pages + lp];",
     "long long phys = (long long)b * p->max_pages + lp;"),
    ("last_token_dropped", "for (long long t = 0; t < L; ++t) {\n        double w",
     "for (long long t = 0; t + 1 < L; ++t) {\n        double w"),
    ("half_bias", "expo - 25", "expo - 24"),
    ("half_subnormal", "ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    ("half_sign_lost", "return sign ? -mag : mag;", "return mag;"),
    ("merge_sign", "double beta = exp(m_p - M);", "double beta = exp(M - m_p);"),
    ("merge_unscaled_sum", "Lsum += beta * l_p;", "Lsum += l_p;"),
    ("query_row_transposed", "((size_t)b * p->query_heads + h) * p->head_dim",
     "((size_t)h * p->batch + b) * p->head_dim"),
    ("values_from_keys", "const uint16_t *vrow = p->v + kv_offset(p, b, t, g);\n        for (int d = 0; d < p->head_dim; ++d) o[d]",
     "const uint16_t *vrow = p->k + kv_offset(p, b, t, g);\n        for (int d = 0; d < p->head_dim; ++d) o[d]"),
    ("not_normalised", "for (int d = 0; d < p->head_dim; ++d) o[d] /= z;", ""),
    ("append_slot_from_division", "long long slot = pos % page_size;",
     "long long slot = pos / page_size % page_size;"),
    ("append_head_major", "((phys * page_size + slot) * kv_heads + g) * (long long)head_dim",
     "((phys * kv_heads + g) * page_size + slot) * (long long)head_dim"),
    ("append_values_from_keys", "v[dst + d] = new_v[src + d];", "v[dst + d] = new_k[src + d];"),
    ("append_source_transposed", "size_t src = ((size_t)b * kv_heads + g)",
     "size_t src = ((size_t)g * batch + b)"),
    ("append_first_sequence_dropped", "for (int b = 0; b < batch; ++b) {\n        long long pos",
     "for (int b = 1; b < batch; ++b) {\n        long long pos"),
    ("zero_page_not_counted", "z += w;\n        if (!in_pool(p, b, t)) continue;",
     "if (!in_pool(p, b, t)) continue;\n        z += w;"),
    ("zero_page_scores_minus_inf", "if (!in_pool(p, b, t)) return 0.0;",
     "if (!in_pool(p, b, t)) return -INFINITY;"),
    ("bad_entries_one_past_context", "for (long long lp = 0; lp < pages; ++lp) {\n            int32_t phys = block_tables",
     "for (long long lp = 0; lp <= pages && lp < max_pages; ++lp) {\n            int32_t phys = block_tables"),
    ("bad_entries_negative_kept", "if (phys >= 0 && phys < num_pages) continue;",
     "if (phys < num_pages) continue;"),
    ("dot_skips_last_dim", "for (int d = 0; d < p->head_dim; ++d)\n        dot +=",
     "for (int d = 0; d + 1 < p->head_dim; ++d)\n        dot +="),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    from oracle import build
    src = open(ORACLE_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} no longer exists in pa_oracle.c"
    mut_src = tmp_path / f"{name}.c"
    mut_src.write_text(src.replace(old, new))
    lib = str(tmp_path / f"lib_{name}.so")
    build.build(src=str(mut_src), out=lib)
    ot = P.OracleUnderTest(lib)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(ot)
        except (AssertionError, ValueError) as e:   # ValueError: the oracle's own error return
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
