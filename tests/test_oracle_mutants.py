"""Planted mistakes in the oracle are caught by the pins (CPU only).

Each mutant is a copy of oracle/decode_oracle.c with one plausible mistake
substituted in (a dropped term, a wrong sign or index, a misread layout, an
off-by-one in a mask).  The copy is compiled into a temporary library and the
whole pin set of oracle_pins.py runs against it; at least one pin must fail.
"""
import os

import pytest

import oracle_pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "decode_oracle.c")

# (name, exact text in the source, replacement)
MUTANTS = [
    ("kv_head_modulo", "int g = h / (p->H / p->KVH);", "int g = h % p->KVH;"),
    ("causal_off_by_one", "int lim = n - seq_tokens(p, b) + t + 1;",
     "int lim = n - seq_tokens(p, b) + t;"),
    ("causal_top_left", "int lim = n - seq_tokens(p, b) + t + 1;", "int lim = t + 1;"),
    ("scale_dropped", "s[j - lo] = p->scale * dot;", "s[j - lo] = dot;"),
    ("scale_squared", "s[j - lo] = p->scale * dot;", "s[j - lo] = p->scale * p->scale * dot;"),
    ("valid_length_ignored",
     "uint32_t nv = p->valid_length ? p->valid_length[b] : (uint32_t)p->S;",
     "uint32_t nv = (uint32_t)p->S;"),
    ("valid_length_not_capped", "return nv < (uint32_t)p->S ? (int)nv : p->S;",
     "return (int)nv;"),
    ("valid_length_capped_signed", "return nv < (uint32_t)p->S ? (int)nv : p->S;",
     "return (int)nv < p->S ? (int)nv : p->S;"),
    # ragged KV layout (per-sequence row offsets into one cache)
    ("kv_offsets_ignored", "row = (size_t)p->kv_offsets[b] + (size_t)j;",
     "row = (size_t)b * p->S + (size_t)j;"),
    ("kv_offsets_off_by_one", "row = (size_t)p->kv_offsets[b] + (size_t)j;",
     "row = (size_t)p->kv_offsets[b] + (size_t)j + 1;"),
    ("kv_offsets_of_next_sequence", "row = (size_t)p->kv_offsets[b] + (size_t)j;",
     "row = (size_t)p->kv_offsets[(b + 1) % p->B] + (size_t)j;"),
    ("sink_scaled", "(double)p->sink[h] : -INFINITY;", "p->scale * (double)p->sink[h] : -INFINITY;"),
    ("sink_not_in_denominator", "if (sigma != -INFINITY) l += exp(sigma - m);",
     "if (sigma != -INFINITY) l += 0.0;"),
    ("merge_sink_per_partition", "L += w;",
     "L += w + ((sigma != -INFINITY) ? exp(sigma - M) : 0.0);"),
    ("page_index_swapped",
     "row = (size_t)phys * p->page_size + (size_t)(j % p->page_size);",
     "row = (size_t)phys * p->page_size + (size_t)(j / p->page_size);"),
    ("page_table_row_stride", "p->page_table[(size_t)b * p->max_pages",
     "p->page_table[(size_t)b * (p->max_pages - 1)"),
    ("mla_value_tail",
     "if (p->v == NULL) return p->k_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);",
     "if (p->v == NULL) return p->k_scale * elem(p->k, kv_index(p, b, j, g, d + (p->D - p->Dv), p->D), "
     "p->kv_dtype);"),
    # 8-bit e4m3 keys / values with per-tensor scales
    ("e4m3_bias_8", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3_subnormal_as_normal", "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp(1.0 + (double)m / 8.0, -7);"),
    ("e4m3_mantissa_4bit", "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 16.0, e - 7);"),
    ("e4m3_top_code_inf", "if (e == 15 && m == 7) return NAN;", "if (e == 15) return INFINITY;"),
    ("e4m3_sign_dropped", "return sign ? -mag : mag;", "return mag;"),
    ("k_scale_dropped", "return p->k_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);\n}",
     "return elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);\n}"),
    ("mla_value_slice_uses_v_scale",
     "if (p->v == NULL) return p->k_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);",
     "if (p->v == NULL) return p->v_scale * elem(p->k, kv_index(p, b, j, g, d, p->D), p->kv_dtype);"),
    ("v_scale_is_k_scale", "return p->v_scale * elem(p->v,", "return p->k_scale * elem(p->v,"),
    ("v_scale_dropped", "return p->v_scale * elem(p->v,", "return elem(p->v,"),
    ("cache_layout_head_major", "return (row * p->KVH + (size_t)g) * (size_t)width + (size_t)d;",
     "return ((size_t)g * ((size_t)p->B * p->S + 1) + row) * (size_t)width + (size_t)d;"),
    ("q_layout_head_token_swapped",
     "size_t qbase = ((first_token(p, b) + (size_t)t) * p->H + h) * (size_t)p->D;",
     "size_t qbase = (((size_t)b * p->H + h) * p->T + t) * (size_t)p->D;"),
    # ragged q (tokens per sequence from q_offsets)
    ("ragged_causal_uses_most_tokens",
     "return p->q_offsets ? (int)(p->q_offsets[b + 1] - p->q_offsets[b]) : p->T;", "return p->T;"),
    ("ragged_boundary_token_misplaced", "(int64_t)p->q_offsets[s + 1] <= token) ++s;",
     "(int64_t)p->q_offsets[s + 1] < token) ++s;"),
    # sparse top-k lists
    ("sparse_list_row_stride", "row = (size_t)p->indices[(size_t)b * p->indices_stride + (size_t)j];",
     "row = (size_t)p->indices[(size_t)b * p->topk_lengths[0] + (size_t)j];"),
    ("sparse_list_ignores_batch", "row = (size_t)p->indices[(size_t)b * p->indices_stride + (size_t)j];",
     "row = (size_t)p->indices[(size_t)j];"),
    ("sparse_position_as_row", "row = (size_t)p->indices[(size_t)b * p->indices_stride + (size_t)j];",
     "row = (size_t)b * p->indices_stride + (size_t)j;"),
    ("sparse_count_off_by_one", "if (p->indices) return p->topk_lengths[b];",
     "if (p->indices) return p->topk_lengths[b] - (p->topk_lengths[b] > 0);"),
    ("sparse_count_is_stride", "if (p->indices) return p->topk_lengths[b];",
     "if (p->indices) return p->indices_stride;"),
    ("max_not_subtracted_in_lse", "double w = exp(s[j] - m);", "double w = exp(s[j]);"),
    ("empty_row_lse_zero", "lse[i] = (l > 0.0) ? m + log(l) : -INFINITY;",
     "lse[i] = (l > 0.0) ? m + log(l) : 0.0;"),
    ("merge_drops_expsum", "double w = part_l[i] * exp(part_m[i] - M);",
     "double w = exp(part_m[i] - M);"),
    ("merge_sign", "double w = part_l[i] * exp(part_m[i] - M);",
     "double w = part_l[i] * exp(M - part_m[i]);"),
    ("merge_sink_twice", "double L = (sigma != -INFINITY) ? exp(sigma - M) : 0.0;",
     "double L = (sigma != -INFINITY) ? 2.0 * exp(sigma - M) : 0.0;"),
    ("partition_skips_first_key", "int lo = lo64 < n ? (int)lo64 : n;",
     "int lo = lo64 + 1 < n ? (int)lo64 + 1 : n;"),
    ("normalise_missing", "for (int d = 0; d < p->Dv; ++d) out[d] /= l;", "(void)0;"),
    ("last_key_dropped", "attend(&p, b, t, h, 0, visible_keys(&p, b, t), 1,",
     "attend(&p, b, t, h, 0, visible_keys(&p, b, t) - (visible_keys(&p, b, t) > 1), 1,"),
]


def test_mutant_substitutions_apply():
    src = open(SRC).read()
    for name, old, _ in MUTANTS:
        assert src.count(old) >= 1, f"mutant {name}: text not found in decode_oracle.c"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src
    mutated = src.replace(old, new)
    path = tmp_path / f"oracle_{name}.c"
    path.write_text(mutated)
    lib_path = O.build(force=True, src=str(path), out=str(tmp_path / f"lib_{name}.so"),
                       extra_flags=("-Wno-unused-variable", "-Wno-unused-but-set-variable",
                                    "-Wno-unused-function"))
    lib = O.load_library(lib_path)
    caught = oracle_pins.failing_pins(lib)
    assert caught, f"planted mistake {name!r} passed every pin"
