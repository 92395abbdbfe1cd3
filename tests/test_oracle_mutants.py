"""CPU: the pins are strong enough to catch plausible oracle mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index or bound, a
transposed operand, an exclusive-for-inclusive sum, a wrong rounding rule) in
a copy of the oracle's C source, builds that copy in a temporary directory
with gcc, and requires at least one pin of ``tests/pins.py`` to fail on it.
Mistakes are chosen so that the broken copy still never reads or writes out
of bounds. Nothing here touches a GPU.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
import pins

SRC = obuild.SRC

# (name, original text, planted mistake, which occurrence to replace)
MUTANTS = [
    ("sort_not_stable", "for (int64_t a = 0; a < total; ++a) {\n            if (top_experts[a] == e)",
     "for (int64_t a = total - 1; a >= 0; --a) {\n            if (top_experts[a] == e)", 0),
    ("bins_exclusive", "run += count;\n        bins[e] = (int32_t)run;",
     "bins[e] = (int32_t)run;\n        run += count;", 0),
    ("padded_round_down", "((count + pad_multiple - 1) / pad_multiple)", "(count / pad_multiple)", 0),
    ("capacity_off_by_one", "handed_out >= capacity", "handed_out > capacity", 0),
    ("binned_segment_base", "segment_base = (int64_t)e * capacity;", "segment_base = (int64_t)e;", 0),
    ("padded_start_inclusive", "segment_base = e == 0 ? 0 : padded_bins[e - 1];",
     "segment_base = padded_bins[e];", 0),
    ("walk_counter_off_by_one", "int64_t handed_out = 0;", "int64_t handed_out = e > 0;", 0),
    ("walk_row_transposed", "else row_of[i] = segment_base + handed_out;",
     "else row_of[i] = segment_base + (handed_out ^ 1);", 0),
    ("gather_token_div_2", "int64_t token = indices[i] / K;", "int64_t token = indices[i] / 2;", 0),
    ("scatter_weight_dropped", "double w = weights ? (double)weights[a] : 1.0;", "double w = 1.0;", 0),
    ("scatter_weight_of_k0", "double w = weights ? (double)weights[a] : 1.0;",
     "double w = weights ? (double)weights[t * K] : 1.0;", 0),
    ("scatter_sign", "sum += term;", "sum -= term;", 0),
    ("scatter_skips_last_k", "for (int32_t k = 0; k < K; ++k) {\n                int64_t a = t * K + k;",
     "for (int32_t k = 0; k + 1 < K; ++k) {\n                int64_t a = t * K + k;", 0),
    ("wgrad_grad_row_shift", "pego_load(grad, dtype, t * H + h)", "pego_load(grad, dtype, ((t + 1) % T) * H + h)", 0),
    ("wgrad_drops_h0", "for (int64_t h = 0; h < H; ++h) {\n                double p =",
     "for (int64_t h = 1; h < H; ++h) {\n                double p =", 0),
    ("wgrad_slot_k_reversed", "int64_t i = pos_of[t * K + k];", "int64_t i = pos_of[t * K + (K - 1 - k)];", 0),
    ("dy_weight_dropped", "double w = (double)weights[a];", "double w = 1.0;", 0),
    ("dy_token_shift", "int64_t t = a / K;", "int64_t t = (a / K + 1) % T;", 0),
    ("bf16_ties_away", "double r = nearbyint(m);", "double r = floor(m + 0.5);", 0),
    ("f16_subnormal_scale", "uint16_t fr = (uint16_t)ldexp(r, 24);", "uint16_t fr = (uint16_t)ldexp(r, 23);", 0),
    ("f16_decode_exponent", "ex - 25); /* (1 + fr/1024)", "ex - 24); /* (1 + fr/1024)", 0),
    ("bf16_decode_shift", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;", 0),
    ("compact_pad_zero", "route_experts[t * topk + j] = -1;", "route_experts[t * topk + j] = 0;", 0),
    ("compact_probs_transposed", "pego_load(probs, probs_dtype, t * E + e)",
     "pego_load(probs, probs_dtype, (int64_t)e * T + t)", 0),
    ("compact_backward_slot", "grad_probs[t * E + e] = grad_probs_out[t * topk + j];",
     "grad_probs[t * E + e] = grad_probs_out[t * topk + (topk - 1 - j)];", 0),
    ("router_ties_to_higher_id", "if (best < 0 || score_above(l[e], l[best])) best = e;",
     "if (best < 0 || !score_above(l[best], l[e])) best = e;", 0),
    ("router_nan_ranks_high", "if (isnan(a)) return 0;", "if (isnan(a)) return 1;", 0),
    ("router_no_max_shift", "denom += exp(l[e] - m);", "denom += exp(l[e]);", 0),
    ("router_denominator_skips_last", "for (int32_t e = 0; e < E; ++e) denom", "for (int32_t e = 0; e + 1 < E; ++e) denom", 0),
    ("router_sigmoid_sign", "1.0 / (1.0 + exp(-l[", "1.0 / (1.0 + exp(l[", 0),
    ("router_normalize_ignored", "(float)(normalize ? p[k] / sel : p[k])", "(float)p[k]", 0),
    ("router_selected_sum_first_only", "for (int32_t k = 0; k < K; ++k) sel += p[k];",
     "for (int32_t k = 0; k < 1; ++k) sel += p[k];", 0),
    ("windows_limit_inclusive", "next_row < row_limit[e] ?", "next_row <= row_limit[e] ?", 0),
    ("windows_base_ignored", "int64_t next_row = row_base[e];", "int64_t next_row = row_base[0];", 0),
    ("validate_no_duplicates", "if (seen[a]) flags |= FLAG_INDICES;", "(void)seen[a];", 0),
    ("validate_expected_off", "if (bins[e] <= i) ++expect;", "if (bins[e] < i) ++expect;", 0),
]


def _replace_nth(text, old, new, nth):
    start = -1
    for _ in range(nth + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"mutation anchor not found: {old!r}"
    return text[:start] + new + text[start + len(old):]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new, nth):
    src = tmp_path / "peg_oracle.c"
    src.write_text(_replace_nth(source, old, new, nth))
    (tmp_path / "peg_oracle.h").write_text(open(os.path.join(os.path.dirname(SRC), "peg_oracle.h")).read())
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *obuild.CFLAGS, str(src), "-o", str(lib), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle.load_library(str(lib))
    failed = []
    try:
        for pin in pins.ALL_PINS:
            try:
                pin(oracle)
            except (AssertionError, ValueError) as exc:  # ValueError: oracle refused its own output
                failed.append((pin.__name__, type(exc).__name__))
                break
    finally:
        oracle._lib = saved
    assert failed, f"mutant {name} passed every pin"
