"""Planted mistakes in the oracle (CPU only): each mutated build of gqa_oracle.c
must fail at least one pin, which shows the pins can see that kind of mistake."""

import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, original text, mutated text): plausible slips in each part of the definition.
MUTANTS = [
    ("dropped_scale", "s[j] = scale * dot;", "s[j] = dot;"),
    ("softmax_sign", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("tiled_head_map", "return h / (H / G);", "return h % G;"),
    ("causal_excludes_diagonal", "long n = causal ? (long)i + 1 : (long)T;", "long n = causal ? (long)i : (long)T;"),
    ("decode_drops_current_token", "long L = seq_lens[b];", "long L = seq_lens[b] - 1;"),
    ("transposed_k", "dot += q[d] * K[j * (long)D + d];", "dot += q[d] * K[d * n + j];"),
    ("transposed_v", "acc += s[j] * V[j * (long)D + d];", "acc += s[j] * V[d * n + j];"),
    ("unnormalised_by_count", "out[d] = acc / denom;", "out[d] = acc / (double)n;"),
    ("batch_group_swap", "((long)b * G + g) * T_cap * D", "((long)g * B + b) * T_cap * D"),
    ("fp8_bias", "e - 7);", "e - 8);"),
    ("fp8_subnormal", "(double)m / 8.0, -6);", "(double)m / 8.0, -7);"),
    ("fp8_ties_to_odd", "(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    ("fp8_quotient_inverted", "codes[i] = gqa_oracle_e4m3fn_encode(x[i] / scale);",
     "codes[i] = gqa_oracle_e4m3fn_encode(x[i] * scale);"),
    ("fp8_sign_dropped", "return (uint8_t)(best | (neg << 7));", "return (uint8_t)best;"),
    ("chunk_offset_off_by_one", "long p = L - Tq + i;", "long p = L - Tq + i + 1;"),
    ("int4_zero_point_7", "int gqa_oracle_int4_value(int u) { return (u & 15) - 8; }",
     "int gqa_oracle_int4_value(int u) { return (u & 15) - 7; }"),
    ("int4_nibble_order", "int u = (i & 1) ? (byte >> 4) : (byte & 15);", "int u = (i & 1) ? (byte & 15) : (byte >> 4);"),
    ("int4_ties_to_odd", "(f == 0.5 && fmod(r, 2.0) != 0.0)", "(f == 0.5 && fmod(r, 2.0) == 0.0)"),
    # The decode's own coding of the softmax (decode_row).
    ("decode_dropped_scale", "w[t] = qk * scale;", "w[t] = qk;"),
    ("decode_softmax_sign", "const double p = exp(w[t] - lse);", "const double p = exp(lse - w[t]);"),
    ("decode_lse_without_log", "const double lse = top + log(z);", "const double lse = top + z;"),
    ("decode_lse_without_max", "const double lse = top + log(z);", "const double lse = log(z);"),
    ("decode_transposed_v", "const double *vt = V + t * (long)D;", "const double *vt = V + t;"),
    ("decode_skips_last_row", "for (t = 0; t < n; ++t) {\n        const double p", "for (t = 0; t + 1 < n; ++t) {\n        const double p"),
    ("chunk_not_causal_masks", "long n = causal ? (p + 1 < L ? p + 1 : L) : L;", "long n = p + 1 < L ? p + 1 : L;"),
]


@pytest.mark.parametrize("name,orig,mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, mut):
    src = open(oracle.SOURCE).read()
    assert orig in src, f"mutation site for {name} not found"
    mutated = src.replace(orig, mut)
    path = tmp_path / f"{name}.c"
    path.write_text(mutated)
    lib = oracle.compile_c(str(path), str(tmp_path / f"lib{name}.so"))
    orc = oracle.from_library(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
