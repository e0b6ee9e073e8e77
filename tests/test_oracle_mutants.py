"""The oracle pins have teeth: each planted mistake in a copy of the oracle's
C source (built on the CPU into a temporary library) must make the pin suite
fail.  Only the oracle is mutated; nothing here touches a GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "mean_over_H_minus_1": ("ss / (double)H", "ss / (double)(H - 1)"),
    "eps_outside_root": ("sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H) + eps"),
    "rmsnorm_divides_by_rstd": ("bf16_bits_to_double(xr[j]) * r *", "bf16_bits_to_double(xr[j]) / r *"),
    "matmul_drops_last_term": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "matmul_transposed_weight": ("bf16_bits_to_double(wr[k])", "bf16_bits_to_double(wt[(k % N) * ldw + n % K])"),
    "attention_no_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "attention_wrong_group": ("h / group, scale", "h % Hkv, scale"),
    "attention_sees_one_future_key": ("int64_t nvis = (int64_t)q_pos[t] + 1;", "int64_t nvis = (int64_t)q_pos[t] + 2;"),
    "rounding_ties_away": ("nearbyint(ldexp(x, -q))", "round(ldexp(x, -q))"),
    "argmax_ties_highest": ("x[i] > bv", "x[i] >= bv"),
    "rope_wrong_sign": ("double_to_bf16(a * c - b * s)", "double_to_bf16(a * c + b * s)"),
    "rope_adjacent_pairs": ("bf16_bits_to_double(xr[i + half]);", "bf16_bits_to_double(xr[(i + 1) % D]);"),
    "rope_wrong_frequency": ("pow(theta, -2.0 * (double)i / (double)D)", "pow(theta, -1.0 * (double)i / (double)D)"),
    "silu_wrong_sign": ("gv / (1.0 + exp(-gv))", "gv / (1.0 + exp(gv))"),
    "add_subtracts": ("bf16_bits_to_double(a[i]) + bf16_bits_to_double(b[i])",
                      "bf16_bits_to_double(a[i]) - bf16_bits_to_double(b[i])"),
    "addmm_subtracts_bias": ("c[m * ldc + n] += bf16_bits_to_double(bias[n]);", "c[m * ldc + n] -= bf16_bits_to_double(bias[n]);"),
    "addmm_bias_by_row": ("c[m * ldc + n] += bf16_bits_to_double(bias[n]);", "c[m * ldc + n] += bf16_bits_to_double(bias[m % N]);"),
    "mean_over_H_plus_1": ("out[r] = s / (double)H;", "out[r] = s / (double)(H + 1);"),
    "log_softmax_drops_max": ("const double lse = m + log(s);", "const double lse = log(s);"),
    "log_softmax_drops_first_term": ("for (int64_t i = 0; i < V; ++i) s += exp", "for (int64_t i = 1; i < V; ++i) s += exp"),
    "log_softmax_wrong_sign": ("(double)xr[i] - lse;", "lse - (double)xr[i];"),
    "philox_nine_rounds": ("for (int r = 0; r < 10; ++r) {", "for (int r = 0; r < 9; ++r) {"),
    "gumbel_wrong_sign": ("return -log(-log(u));", "return log(-log(u));"),
    "sample_multiplies_by_temperature": ("(double)x[i] / (double)temperature", "(double)x[i] * (double)temperature"),
    "top2_second_may_be_the_top": ("if (i != best && (!have_second", "if ((!have_second"),
    "lm_head_drops_last_term": ("for (int64_t j = 0; j < H; ++j) s += y[j] * bf16_bits_to_double(wr[j]);",
                                "for (int64_t j = 0; j + 1 < H; ++j) s += y[j] * bf16_bits_to_double(wr[j]);"),
    "lm_head_next_vocab_row": ("const uint16_t* wr = wt + v * ldw;", "const uint16_t* wr = wt + ((v + 1) % V) * ldw;"),
    "toy_no_final_norm": ("or_rmsnorm(h + (T - 1) * H, H, final_norm, xn, H, NULL, 1, H, c->eps);",
                          "memcpy(xn, h + (T - 1) * H, (size_t)H * 2);"),
    "toy_value_from_key_slot": ("memcpy(vv + t * Hkv * D, qkv + t * QKV + (Hq + Hkv) * D",
                                "memcpy(vv + t * Hkv * D, qkv + t * QKV + Hq * D"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    n = src.count(old)
    assert n >= 1, f"mutation anchor not found: {old}"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mutant), "-lm"], check=True)
    env = dict(os.environ, BI_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_toy_pins.py"),
                        "-k", "not thread_count"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
