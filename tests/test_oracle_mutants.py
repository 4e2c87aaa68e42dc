"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks
that the pin battery catches every one of them. The real oracle source is
never modified; each mutant is compiled into a temporary directory."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

# (name, original text, mutated text)
MUTANTS = [
    ("gate_up_swapped", "g += x[h] * bf16_value(w13[i * H + h]);\n            u += x[h] * bf16_value(w13[(I + i) * H + h]);",
     "g += x[h] * bf16_value(w13[(I + i) * H + h]);\n            u += x[h] * bf16_value(w13[i * H + h]);"),
    ("silu_sign", "act[i] = g / (1.0 + exp(-g)) * u;", "act[i] = g / (1.0 + exp(g)) * u;"),
    ("silu_on_up", "act[i] = g / (1.0 + exp(-g)) * u;", "act[i] = u / (1.0 + exp(-u)) * g;"),
    ("bias_dropped", "if (bias) s += (double)bias[e];", ""),
    ("tie_to_higher_index", "return a < b;", "return a > b;"),
    ("ascending_topk", "if (row[a] != row[b]) return row[a] > row[b];", "if (row[a] != row[b]) return row[a] < row[b];"),
    ("renorm_ignored", "weights[t * k + j] = norm_topk_prob ? p[order[j]] / sel : p[order[j]];",
     "weights[t * k + j] = p[order[j]];"),
    ("renorm_always", "weights[t * k + j] = norm_topk_prob ? p[order[j]] / sel : p[order[j]];",
     "weights[t * k + j] = p[order[j]] / sel;"),
    ("softmax_negated", "p[e] = exp(row[e] - mx);", "p[e] = exp(mx - row[e]);"),
    ("down_term_dropped", "for (int64_t i = 0; i < I; ++i) s += act[i] * bf16_value(w2[h * I + i]);",
     "for (int64_t i = 1; i < I; ++i) s += act[i] * bf16_value(w2[h * I + i]);"),
    ("router_transposed", "bf16_value(wr[e * H + h])", "bf16_value(wr[h * E + e])"),
    ("combine_wrong_slot", "out[h] += w[j] * y[j * H + h];", "out[h] += w[0] * y[j * H + h];"),
    ("combine_dropped_slot", "for (int64_t j = 0; j < k; ++j)\n        for (int64_t h = 0; h < H; ++h) out[h]",
     "for (int64_t j = 1; j < k; ++j)\n        for (int64_t h = 0; h < H; ++h) out[h]"),
    ("router_token_zero", "oracle_router_logits(x + t * H, wr, bias, 1, H, E, logits);",
     "oracle_router_logits(x, wr, bias, 1, H, E, logits);"),
    ("align_unstable", "for (int64_t i = 0; i < n; ++i)\n            if (ids[i] == e) sorted_ids[fill++] = (int32_t)i;",
     "for (int64_t i = n - 1; i >= 0; --i)\n            if (ids[i] == e) sorted_ids[fill++] = (int32_t)i;"),
    ("align_no_padding", "int64_t padded = (counts[e] + block_m - 1) / block_m * block_m;",
     "int64_t padded = counts[e];"),
    ("norm_eps_dropped", "const double inv = 1.0 / sqrt(ss / (double)H + eps);",
     "const double inv = 1.0 / sqrt(ss / (double)H);"),
    ("norm_sum_not_mean", "const double inv = 1.0 / sqrt(ss / (double)H + eps);",
     "const double inv = 1.0 / sqrt(ss + eps);"),
    ("norm_cast_after_weight", "const double n = round_bf16(bf16_value(rr[h]) * inv);",
     "const double n = bf16_value(rr[h]) * inv;"),
    ("norm_residual_not_added", "float sum = (float)bf16_value(rr[h]) + (float)bf16_value(xr[h]);",
     "float sum = (float)bf16_value(xr[h]);"),
    ("align_sentinel_zero", "for (int64_t r = 0; r < cap; ++r) sorted_ids[r] = (int32_t)n;",
     "for (int64_t r = 0; r < cap; ++r) sorted_ids[r] = 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.OracleLib(oracle.compile_source(str(path), str(tmp_path / f"lib{name}.so")))
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            return  # caught
    pytest.fail(f"no pin catches mutant {name}")
