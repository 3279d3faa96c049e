"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of ``oracle/dsa_oracle.c`` with one planted mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong tie rule
...), compiled with gcc into a temporary library.  Every mutant must fail at
least one pin of ``oracle_pins.py``.  Runs on the CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.lib_path()), "dsa_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("relu_dropped", "s += wd[h] * (logit > 0.0 ? logit : 0.0);", "s += wd[h] * logit;"),
    ("relu_wrong_side", "s += wd[h] * (logit > 0.0 ? logit : 0.0);",
     "s += wd[h] * (logit < 0.0 ? logit : 0.0);"),
    ("weight_inside_relu", "s += wd[h] * (logit > 0.0 ? logit : 0.0);",
     "s += (wd[h] * logit > 0.0 ? wd[h] * logit : 0.0);"),
    ("weights_of_row0", "wd[h] = (double)w[(size_t)i * H + h];", "wd[h] = (double)w[h];"),
    ("q_transposed", "load_elem(q, ((size_t)i * H + h) * D + d, dtype)",
     "load_elem(q, ((size_t)i * D + d) * H + h, dtype)"),
    ("slot_shifted", "int slot = t % page_size;", "int slot = (t + 1) % page_size;"),
    ("physical_position", "int page = block_table[(size_t)b * bt_stride + t / page_size];\n            int slot = t % page_size;",
     "int page = t / page_size;\n            int slot = t % page_size;"),
    ("k_scale_ignored", "(load_elem(k_cache, base + d, dtype) * elem_scale(k_scale, tok, D, d, dtype))",
     "load_elem(k_cache, base + d, dtype)"),
    ("q_scale_per_row", "elem_scale(q_scale, (size_t)i * H + h, D, d, dtype)",
     "elem_scale(q_scale, (size_t)i * H, D, d, dtype)"),
    ("mx_block_misplaced", "[r * (size_t)(D / 32) + d / 32]", "[r * (size_t)(D / 32) + (d / 32 + 1) % (D / 32)]"),
    ("mx_block_of_16", "[r * (size_t)(D / 32) + d / 32]", "[r * (size_t)(D / 32) + (d / 16) % (D / 32)]"),
    ("mx_scale_rows_not_strided", "[r * (size_t)(D / 32) + d / 32]", "[r + d / 32]"),
    ("e8m0_bias_126", "ldexp(1.0, (int)code - 127)", "ldexp(1.0, (int)code - 126)"),
    ("e8m0_no_nan", "return code == 255 ? NAN : ldexp", "return code == 256 ? NAN : ldexp"),
    ("causal_off_by_one", "vis[q_offsets[b] + j] = ctx_lens[b] - n + j + 1;",
     "vis[q_offsets[b] + j] = ctx_lens[b] - n + j;"),
    ("causal_all_rows_see_all", "vis[q_offsets[b] + j] = ctx_lens[b] - n + j + 1;",
     "vis[q_offsets[b] + j] = ctx_lens[b];"),
    ("ties_to_higher_position", "return (x->t > y->t) - (x->t < y->t);",
     "return (x->t < y->t) - (x->t > y->t);"),
    ("ascending_scores", "if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;",
     "if (x->s < y->s) return -1;\n    if (x->s > y->s) return 1;"),
    ("not_rearranged", "qsort(out, (size_t)keep, sizeof(int32_t), ascending_i32);", ""),
    ("pad_with_zero", "out[r] = -1;", "out[r] = 0;"),
    ("e4m3_bias_8", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3_subnormal_implicit_one", "v = ldexp((double)m / 8.0, -6);", "v = ldexp(1.0 + (double)m / 8.0, -6);"),
    ("e4m3_no_nan", "if (e == 15 && m == 7)\n        return NAN;", ""),
    ("bf16_low_half", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits;"),
    ("sfa_scale_dropped", "z[r] = scale * dot;", "z[r] = dot;"),
    ("sfa_value_from_tail", "o[e] += p * latent_elem(kv_cache, prow, e, Dqk, Dv, dtype);",
     "o[e] += p * latent_elem(kv_cache, prow, (Dqk - Dv) + e, Dqk, Dv, dtype);"),
    ("kv8_tile_of_64", "dsa_oracle_decode_e8m0(r[Dv + d / 128])", "dsa_oracle_decode_e8m0(r[Dv + (d / 64) % (Dv / 128)])"),
    ("kv8_scale_ignored", "return dsa_oracle_decode_e4m3(r[d]) * dsa_oracle_decode_e8m0(r[Dv + d / 128]);",
     "return dsa_oracle_decode_e4m3(r[d]);"),
    ("kv8_rope_without_scale_gap", "memcpy(&bits, r + Dv + 16 + 2 * (d - Dv), sizeof bits);",
     "memcpy(&bits, r + Dv + 2 * (d - Dv), sizeof bits);"),
    ("sfa_key_without_rope", "for (int d = 0; d < Dqk; ++d)\n                    dot += qd[d]",
     "for (int d = 0; d < Dv; ++d)\n                    dot += qd[d]"),
    ("sfa_not_normalised", "o[e] /= l;", "o[e] /= 1.0;"),
    ("sfa_lse_without_max", "lse[(size_t)i * H + h] = m + log(l);", "lse[(size_t)i * H + h] = log(l);"),
    ("sfa_padding_read", "if (t < 0)\n                    continue;\n                double p",
     "if (t < 0)\n                    t = 0;\n                double p"),
    ("encode_ties_away", "return nearbyint(a / q) * q;", "return round(a / q) * q;"),
    ("encode_truncates", "return nearbyint(a / q) * q;", "return floor(a / q) * q;"),
    ("e4m3_no_saturation", "if (r > 448.0)\n        r = 448.0;", "if (r > 480.0)\n        r = 480.0;"),
    ("e4m3_subnormal_step", "r / ldexp(1.0, -9)", "r / ldexp(1.0, -8)"),
    ("bf16_six_bits", "round_to_grid(fabs((double)x), 7, -126)", "round_to_grid(fabs((double)x), 6, -126)"),
    ("append_at_front", "int p = L - n + j;", "int p = j;"),
    ("append_physical_page", "int page = block_table[(size_t)b * bt_stride + p / page_size];\n            size_t row",
     "int page = p / page_size;\n            size_t row"),
    ("fp8_scale_over_240", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax > 0.0f ? amax / 240.0f : 1.0f"),
    ("fp8_zero_key_scale_0", "amax > 0.0f ? amax / 448.0f : 1.0f", "amax / 448.0f"),
    ("fp8_quotient_in_fp64", "float v = x[d] / s;", "double v = (double)x[d] / s;"),
    ("mx_exponent_minus_7", "e = ex - 1 - 8;", "e = ex - 1 - 7;"),
    ("latent_tile_of_64", "for (int d = 128 * t; d < 128 * t + 128; ++d)\n                        amax",
     "for (int d = 128 * t; d < 128 * t + 64; ++d)\n                        amax"),
    ("latent_exponent_for_256", "while (amax > ldexp(448.0, e))\n        ++e;\n    while (amax <= ldexp(448.0, e - 1))",
     "while (amax > ldexp(256.0, e))\n        ++e;\n    while (amax <= ldexp(256.0, e - 1))"),
    ("latent_exponent_strict", "while (amax > ldexp(448.0, e))\n        ++e;\n    while (amax <= ldexp(448.0, e - 1))",
     "while (amax >= ldexp(448.0, e))\n        ++e;\n    while (amax < ldexp(448.0, e - 1))"),
    ("latent_no_clamp", "return e < -126 ? -126 : (e > 127 ? 127 : e);", "return e;"),
    ("latent_zero_tile_byte_0", "if (amax == 0.0)\n        return 0;\n    int e = ilogb",
     "if (amax == 0.0)\n        return -127;\n    int e = ilogb"),
    ("latent_scale_bytes_reversed", "r[Dv + t] = (uint8_t)(e + 127);", "r[Dv + 15 - t] = (uint8_t)(e + 127);"),
    ("latent_rope_truncated", "uint16_t h = dsa_oracle_encode_bf16(x[d]);\n                    memcpy(r + Dv + 16",
     "uint32_t u_; memcpy(&u_, &x[d], 4); uint16_t h = (uint16_t)(u_ >> 16);\n                    memcpy(r + Dv + 16"),
    ("latent_rope_without_gap", "memcpy(r + Dv + 16 + 2 * (size_t)(d - Dv), &h, sizeof h);",
     "memcpy(r + Dv + 2 * (size_t)(d - Dv), &h, sizeof h);"),
    ("latent_at_front", "int p = L - n + j;\n            int page = block_table[(size_t)b * bt_stride + p / page_size];\n            unsigned char",
     "int p = j;\n            int page = block_table[(size_t)b * bt_stride + p / page_size];\n            unsigned char"),
    ("latent_bf16_truncated", "uint16_t h = dsa_oracle_encode_bf16(x[d]);\n                    memcpy(r + 2 * (size_t)d",
     "uint32_t u_; memcpy(&u_, &x[d], 4); uint16_t h = (uint16_t)(u_ >> 16);\n                    memcpy(r + 2 * (size_t)d"),
    ("mx_zero_block_byte_0", "int e = 0;\n                    if (amax > 0.0f)", "int e = -127;\n                    if (amax > 0.0f)"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutant {name}: pattern not found in the oracle source"
    path_c = tmp_path / f"{name}.c"
    path_c.write_text(src.replace(old, new, 1))
    (tmp_path / "dsa_oracle.h").write_text(open(SRC.replace(".c", ".h")).read())
    path_so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", str(path_c), "-o",
                    str(path_so), "-lm"], check=True)
    return str(path_so)


RUNNER = r"""
import sys
sys.path[:0] = [sys.argv[1], sys.argv[2]]
import oracle, oracle_pins
oracle.load_library(sys.argv[3])
caught = []
for check in oracle_pins.ALL_CHECKS:
    try:
        check()
    except Exception as e:
        caught.append(check.__name__)
        break
print("caught by:", caught)
sys.exit(0 if caught else 3)
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(oracle_mod, tmp_path, name, old, new):
    so = _build_mutant(tmp_path, name, old, new)
    tests_dir = os.path.dirname(os.path.abspath(__file__))
    root = os.path.dirname(tests_dir)
    r = subprocess.run([sys.executable, "-c", RUNNER, root, tests_dir, so], capture_output=True,
                       text=True, timeout=300, env={**os.environ, "OMP_NUM_THREADS": "2"})
    assert r.returncode == 0, f"no pin caught the planted mistake {name}: {r.stdout}{r.stderr[-2000:]}"
