"""Each plausible mistake planted in a copy of oracle.c fails some pin.

The mutants are built on the CPU from a temporary copy of the source; the
real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
import pins

MUTANTS = {
    "f16_subnormal_scale": ("ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    "f16_exponent_bias": ("e - 25", "e - 24"),
    "q8_unsigned": ("int8_t q = (int8_t)blk[2 + i];", "int q = blk[2 + i];"),
    "q4_offset": ("(double)(n - 8)", "(double)(n - 7)"),
    "q4_nibble_order": ("(i < 16) ? (byte & 0x0f) : (byte >> 4)", "(i < 16) ? (byte >> 4) : (byte & 0x0f)"),
    "q4_byte_index": ("blk[2 + (i & 15)]", "blk[2 + (i >> 1)]"),
    "q8_block_stride": ("row + 34 * (i / 32)", "row + 32 * (i / 32)"),
    "scale_dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "softcap_outer_factor": ("softcap * tanh(s[t] / softcap)", "tanh(s[t] / softcap)"),
    "lse_log2": ("lse[r] = mx + log(z);", "lse[r] = mx + log2(z);"),
    "no_normalise": ("for (d = 0; d < head_dim; ++d) acc[d] /= z;", ""),
    "head_map_modulo": ("q_to_kv[h] : h / (n_q_heads / n_kv_heads)", "q_to_kv[h] : h % n_kv_heads"),
    "pos_head_stride_swap": ("kb + j * w->k_pos_stride", "kb + j * w->k_head_stride"),
    "v_read_as_k_type": ("dequant_row(w->v_type", "dequant_row(w->k_type"),
    "combine_weight_sign": ("exp(lse_parts[t][r] - mx)", "exp(mx - lse_parts[t][r])"),
    "combine_no_normalise": ("for (d = 0; d < head_dim; ++d) o_out[r * head_dim + d] /= z;", ""),
    "seq_stride_ignored": ("(int64_t)b * w->k_seq_stride", "(int64_t)0 * w->k_seq_stride"),
    "dot_index_shift": ("qd[d] * kv[d]", "qd[d] * kv[(d + 1) % head_dim]"),
    "combine_lse_drops_max": ("lse_out[r] = mx + log(z);", "lse_out[r] = log(z);"),
    # write path
    "f16enc_truncate": ("m = rint(ldexp(v, 10 - e));", "m = floor(ldexp(v, 10 - e));"),
    "f16enc_subnormal_shift": ("rint(ldexp(v, 24))", "rint(ldexp(v, 23))"),
    "f16enc_overflow_guard": ("if (v >= 65520.0)", "if (v >= 131072.0)"),
    "f16enc_no_carry": ("if (m == 2048.0) {", "if (m > 2048.0) {"),
    "f16enc_bias": ("((e + 15) << 10)", "((e + 14) << 10)"),
    "q8enc_divisor": ("d = amax / 127.0f;", "d = amax / 128.0f;"),
    "q8enc_round_even": ("roundf(v)", "rintf(v)"),
    "q8enc_codes_from_f16_scale": ("blk[2 + i] = (uint8_t)(int8_t)roundf(v);",
                                   "blk[2 + i] = (uint8_t)(int8_t)roundf((float)(x[i] / orc_f16_to_f64(orc_f32_to_f16(d))));"),
    "q4enc_offset": ("const float w = v + 8.5f;", "const float w = v + 8.0f;"),
    "q4enc_scale_sign": ("d = m / -8.0f;", "d = m / 8.0f;"),
    "q4enc_last_largest": ("if (fabsf(x[i]) > amax) {", "if (fabsf(x[i]) >= amax) {"),
    "q4enc_no_clamp": ("if (c > 15) c = 15;", ""),
    "q4enc_nibble_order": ("(uint8_t)(n[i] | (n[i + 16] << 4))", "(uint8_t)(n[2 * i] | (n[2 * i + 1] << 4))"),
    "q4enc_zero_block_sign": ("float amax = 0.0f, m = 0.0f, d, id;", "float amax = 0.0f, m = -0.0f, d, id;"),
    "route_window_edge": ("if (pos < window_cap) {", "if (pos <= window_cap) {"),
    "route_tail_row": ("*row = pos - window_cap;", "*row = pos;"),
    "route_tail_edge": ("if (pos - window_cap < tail_cap) {", "if (pos - window_cap <= tail_cap) {"),
    # causal mask
    "mask_strict": ("return !q_pos || t <= q_pos[b];", "return !q_pos || t < q_pos[b];"),
    "mask_first_seq": ("return !q_pos || t <= q_pos[b];", "return !q_pos || t <= q_pos[0];"),
    "mask_ignored_in_values": ("if (!key_seen(q_pos, b, t)) continue;\n                p = exp",
                               "p = exp"),
    # TBQ3 tier
    "tbq3_decode_signs_swapped": ("acc += hadamard(i, j) * tbq3_s2[j] * y[j];", "acc += hadamard(i, j) * tbq3_s1[j] * y[j];"),
    "tbq3_decode_no_sqrt": ("out[i] = tbq3_s1[i] * acc / sqrt(128.0);", "out[i] = tbq3_s1[i] * acc;"),
    "tbq3_qs_shift": ("const int m = (blk[4 + i / 4] >> (2 * (i % 4))) & 3;", "const int m = (blk[4 + i / 4] >> (i % 4)) & 3;"),
    "tbq3_sign_bit_order": ("const int neg = (blk[36 + i / 8] >> (i % 8)) & 1;",
                            "const int neg = (blk[36 + i / 8] >> (7 - i % 8)) & 1;"),
    "tbq3_level_mean": ("nc[j] = (std_normal_pdf(t[j]) - std_normal_pdf(t[j + 1])) / mass;",
                        "nc[j] = (std_normal_pdf(t[j]) - std_normal_pdf(t[j + 1])) / (2.0 * mass);"),
    "tbq3_threshold": ("for (j = 1; j < 4; ++j) t[j] = 0.5 * (c[j - 1] + c[j]);", "for (j = 1; j < 4; ++j) t[j] = c[j - 1];"),
    "tbq3_seed": ("orc_splitmix64(42, 4, w);", "orc_splitmix64(43, 4, w);"),
    "splitmix_shift": ("z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;", "z = (z ^ (z >> 31)) * 0xbf58476d1ce4e5b9ull;"),
    "tbq3_enc_threshold": ("if (a > 0.5 * (tbq3_lv[j - 1] + tbq3_lv[j])) m = j;", "if (a > tbq3_lv[j - 1]) m = j;"),
    "tbq3_enc_norm_squared": ("    n = sqrt(n);\n", "\n"),
    "tbq3_enc_rotation_order": ("acc += hadamard(i, j) * tbq3_s1[j] * (double)x[j];",
                                "acc += hadamard(i, j) * tbq3_s2[j] * (double)x[j];"),
    "tbq3_block_stride": ("tbq3_block_values(row + 52 * (i / 128), out + i);", "tbq3_block_values(row + 48 * (i / 128), out + i);"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = os.path.join(mutant_dir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(mutant_dir, f"lib{name}.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", so, path, "-lm"])
    mut = oracle.Oracle(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"mutant {name} passed every pin"
