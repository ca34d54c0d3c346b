"""Mutation gate for the oracle (CPU only).

Each mutant plants one plausible slip in a copy of the oracle's C source
(never in the library), builds it with gcc into a temporary directory, and
runs the pins.  A mutant that passes every pin would mean the pins cannot see
that kind of mistake, so each one must fail at least one pin.
"""
import os

import pytest

import oracle
import oracle_pins

# (name, text in q4_oracle.c, replacement)
MUTANTS = [
    ("nibble_order_reversed", "4 * (kk % 8)", "4 * (7 - kk % 8)"),
    ("zero_point_7", "(double)(q - 8) * s", "(double)(q - 7) * s"),
    ("group_of_64", "scales[r * (k / 32) + kk / 32]", "scales[r * (k / 32) + kk / 64]"),
    ("row_stride_halved", "words[r * (k / 8) + kk / 8]", "words[r * (k / 16) + kk / 8]"),
    ("half_exponent_bias", "(double)(1024 + m), e - 25", "(double)(1024 + m), e - 24"),
    ("half_subnormal_scale", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("rne_ties_up", "(fmod(f, 2.0) == 0.0) ? f : f + 1.0", "f + 1.0"),
    ("half_encode_no_overflow", "if (E > 15)", "if (E > 16)"),
    ("silu_sign", "g / (1.0 + exp(-g))", "g / (1.0 + exp(g))"),
    ("silu_on_up", "return q4o_silu(g) * u;", "return q4o_silu(u) * g;"),
    ("argmax_last_tie", "if (v[i] > v[best])", "if (v[i] >= v[best])"),
    ("abs_sum_signed", "asum += fabs(term);", "asum += term;"),
    ("last_k_dropped", "for (int64_t kk = 0; kk < k; ++kk) {", "for (int64_t kk = 0; kk < k - 1; ++kk) {"),
    ("gemm_row_stride", "X + i * k, n, k", "X + i * 32, n, k"),
    ("layout_lanes_transposed", "int64_t lane = s * L + c;", "int64_t lane = c * (64 / L) + s;"),
    ("layout_scale_offset", "(u * CG + j) * 2;", "(j * 2 + u) * 2;"),
    ("layout_pad_scale", "place(dst, r, g, L, CG, TR, TB, NULL, 0);",
     "place(dst, r, g, L, CG, TR, TB, NULL, 0x3c00);"),
    ("layout_tie_smaller_L", "cover < bestCover", "cover <= bestCover"),
    ("layout_gate_up_swapped", "rw = (r % 2 ? w1 : w0)", "rw = (r % 2 ? w0 : w1)"),
    ("layout_tile_rows", "int64_t TR = 2 * (64 / L);", "int64_t TR = 64 / L;"),
    ("norm_sum_not_mean", "sqrt(ss / (double)k + eps)", "sqrt(ss + eps)"),
    ("norm_eps_dropped", "sqrt(ss / (double)k + eps)", "sqrt(ss / (double)k)"),
    ("norm_residual_dropped", "            v += q4o_half_to_double(r[i]);   /* exact: two f16 */",
     "            v += 0.0;"),
    ("norm_gamma_dropped", "q4o_half_to_double(hb) * q4o_half_to_double(gamma[i]) / rms",
     "q4o_half_to_double(hb) / rms"),
    ("rope_adjacent_pair", "q4o_rope_pair(y[h * d + i], y[h * d + i + d / 2], i, d, pos, base, &oi, &oj);",
     "q4o_rope_pair(y[h * d + i], y[h * d + i + 1], i, d, pos, base, &oi, &oj);"),
    ("rope_frequency", "pow(base, -2.0 * (double)i / (double)d)", "pow(base, -1.0 * (double)i / (double)d)"),
    ("rope_sign", "*oi = yi * c - yj * s;", "*oi = yi * c + yj * s;"),
    ("rope_rotates_v", "for (int64_t h = 0; h < nq + nkv; ++h)", "for (int64_t h = 0; h < nq + 2 * nkv; ++h)"),
    ("rope_layout_adjacent", "int64_t src = (pr / (d / 2)) * d + pr % (d / 2) + u * (d / 2);",
     "int64_t src = (pr / (d / 2)) * d + 2 * (pr % (d / 2)) + u;"),
    ("attn_group_modulo", "const int64_t g = h / (nq / nkv);", "const int64_t g = h % nkv;"),
    ("attn_keys_from_v", "q4o_half_to_double(q[h * d + i]) * kv_at(src, 0, g, t, i);",
     "q4o_half_to_double(q[h * d + i]) * kv_at(src, 1, g, t, i);"),
    ("attn_slot", "[(((page * 2 + kv) * src->nkv + g) * 16 + t % 16) * d + i]",
     "[(((page * 2 + kv) * src->nkv + g) * 16 + t / 16) * d + i]"),
    ("attn_slot_major", "[(((page * 2 + kv) * src->nkv + g) * 16 + t % 16) * d + i]",
     "[(((page * 2 + kv) * 16 + t % 16) * src->nkv + g) * d + i]"),
    ("attn_no_scale", "sc[t] = scale * dot;", "sc[t] = dot;"),
    ("attn_unnormalised", "out[h * d + i] = o / den;", "out[h * d + i] = o;"),
    ("attn_softmax_base2", "sc[t] = exp(sc[t] - mx);", "sc[t] = exp2(sc[t] - mx);"),
    ("attn_scaled_twice", "sc[t] = scale * dot;", "sc[t] = scale * dot / sqrt((double)d);"),
    ("attn_magnitude_unnormalised", "a[h * d + i] = m / den;", "a[h * d + i] = m;"),
    ("kv8_max_skips_last", "for (int64_t i = 0; i < d; ++i) {\n        float a = (float)fabs",
     "for (int64_t i = 0; i < d - 1; ++i) {\n        float a = (float)fabs"),
    ("int3_group_of_64", "scales[r * G + col / 32]", "scales[r * G + col / 64]"),
    ("int3_last_k_dropped", "for (int64_t col = 0; col < k; ++col) {", "for (int64_t col = 0; col < k - 1; ++col) {"),
    ("int3_zero_point_3", "((double)(q - 4) * s)", "((double)(q - 3) * s)"),
    ("int3_bits_msb_first", "q |= stream_bit(words3, r, k, 3 * kk + t) << t;",
     "q |= stream_bit(words3, r, k, 3 * kk + t) << (2 - t);"),
    ("int3_row_stride", "words3[r * (3 * k / 32) + b / 32]", "words3[r * (k / 8) + b / 32]"),
    ("int3_no_word_carry", "uint32_t word = words3[r * (3 * k / 32) + b / 32];\n    return (int)((word >> (b % 32)) & 1u);",
     "uint32_t word = words3[r * (3 * k / 32) + b / 32];\n    return (int)((word >> (b % 32)) & 1u) & (b % 32 < 30 || b % 3 == 0 ? 1 : 0);"),
    ("int3_high_half_reversed", "word |= (uint32_t)codes[10 * i + 5 + m] << (16 + 3 * m);",
     "word |= (uint32_t)codes[10 * i + 5 + m] << (16 + 3 * (4 - m));"),
    ("int3_extra_bit_14", "word |= (uint32_t)((codes[30] >> i) & 1) << 15;",
     "word |= (uint32_t)((codes[30] >> i) & 1) << 14;"),
    ("int3_pad_code_0", "codes[i] = real ? code3_at(rw, src, 32 * g + i, k) : 4;",
     "codes[i] = real ? code3_at(rw, src, 32 * g + i, k) : 0;"),
    ("int3_gemm_row_stride", "X + r * k, n, k, Y + r * n", "X + r * 32, n, k, Y + r * n"),
    ("int3_gate_up_swapped", "const uint32_t *rw = w1 ? (r % 2 ? w1 : w0) : w0;",
     "const uint32_t *rw = w1 ? (r % 2 ? w0 : w1) : w0;"),
    ("int3_ffn_up_rows_as_gate", "q4o_gemv3(uw3 + r * (3 * k / 32), us + r * (k / 32), x, 1, k, &uv, &auv);",
     "q4o_gemv3(gw3 + r * (3 * k / 32), gs + r * (k / 32), x, 1, k, &uv, &auv);"),
    ("kv8_scale_128", "float s = m / 127.0f;", "float s = m / 128.0f;"),
    ("kv8_truncate", "q[i] = (int8_t)rintf(t);", "q[i] = (int8_t)t;"),
    ("kv8_append_slot", "q4o_kv_quant_row(row, d, (int8_t *)(blk + (pos % 16) * d), &s);",
     "q4o_kv_quant_row(row, d, (int8_t *)(blk + (pos / 16) * d), &s);"),
    ("kv8_scale_of_slot0", "memcpy(&s, blk + 16 * d + 4 * (t % 16), 4);", "memcpy(&s, blk + 16 * d, 4);"),
    ("kv8_block_size", "(kv * src->nkv + g) * (16 * d + 64);", "(kv * src->nkv + g) * (16 * d);"),
    ("kv8_code_slot", "(double)(int8_t)blk[(t % 16) * d + i]", "(double)(int8_t)blk[(t % 16) + i * 16]"),
    ("norm_unrounded_residual", "const double hv = q4o_half_to_double(q4o_double_to_half(v));",
     "const double hv = v;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(out=str(tmp_path / "libmutant.so"), source=str(path))
    orc = oracle.load(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc, quick=True)
        except AssertionError:
            failed.append(pin.__name__)
        except Exception as e:  # a crash inside a pin also counts as caught
            failed.append(f"{pin.__name__}:{type(e).__name__}")
    assert failed, f"mutant {name} passed every pin"
