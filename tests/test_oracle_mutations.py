"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case copies oracle/oracle.c, plants one plausible mistake by text
substitution (a dropped term, a wrong sign or index, a swapped operand),
compiles the copy with gcc into a temporary directory and runs the pins of
tests/test_oracle_pins.py against it.  At least one pin must fail.  The real
oracle is untouched; the mutants only ever run on the CPU.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "kv_formula_drops_factor_2": ("(uint64_t)2 *", "(uint64_t)1 *", [pins.check_kv_sizes]),
    "f16_exponent_bias_off_by_one": ("e - 25", "e - 24", [pins.check_f16_widen]),
    "bf16_shift_wrong": ("(uint32_t)b << 16", "(uint32_t)b << 15", [pins.check_bf16_widen]),
    "e4m3_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)", [pins.check_e4m3_decode]),
    "e4m3_normal_bias": ("e - 10);", "e - 11);", [pins.check_e4m3_decode]),
    "e4m3_ties_always_down": ("(lo % 2 == 0) ? lo : hi", "lo", [pins.check_e4m3_encode]),
    "e4m3_overflow_to_nan": ("if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
                             "if (a >= 449.0) return 0x7F;", [pins.check_e4m3_encode]),
    "gqa_interleaved_heads": ("const int32_t h = g * G + hh;", "const int32_t h = hh * H_kv + g;",
                              [pins.check_gqa_equals_repeated_mha, pins.check_attention_textbook]),
    "drop_newest_token": ("j < n;", "j < n - 1;",
                          [pins.check_attention_textbook, pins.check_cached_decode_equals_recompute]),
    "logits_read_values": ("widen(K, kv_dtype, kbase + i)", "widen(V, kv_dtype, kbase + i)",
                           [pins.check_attention_textbook]),
    "keys_reversed": ("const int64_t kbase = ((tok_off[b] + j)",
                      "const int64_t kbase = ((tok_off[b] + (n - 1 - j))",
                      [pins.check_attention_textbook, pins.check_attention_closed_forms]),
    "softmax_sign": ("exp(z[j] - m)", "exp(m - z[j])", [pins.check_attention_textbook]),
    "scale_dropped": ("z[j] = s * dot;", "z[j] = dot;", [pins.check_attention_textbook]),
    "no_normalisation": ("o[i] /= l;", "o[i] /= 1.0;",
                         [pins.check_attention_textbook, pins.check_attention_closed_forms]),
    "fp8_key_scale_dropped": ("* (widen(K, kv_dtype, kbase + i) * ks)", "* widen(K, kv_dtype, kbase + i)",
                              [pins.check_fp8_attention_on_dequantised_values]),
    "prefill_queries_at_the_start": ("const int64_t p = n - q_len + (t - q_start[s]);",
                                     "const int64_t p = (t - q_start[s]);",
                                     [pins.check_prefill_vs_library_attention, pins.check_prefill_single_token_is_decode]),
    "prefill_mask_always_causal": ("const int64_t last = causal ? p : n - 1;", "const int64_t last = p;",
                                   [pins.check_prefill_vs_library_attention]),
    "prefill_interleaved_heads": ("const int32_t g = h / G;", "const int32_t g = h % H_kv;",
                                  [pins.check_prefill_vs_library_attention]),
    "prefill_scale_dropped": ("z[j] = sc * dot;", "z[j] = dot;", [pins.check_prefill_vs_library_attention]),
    "fp8_value_scale_dropped": ("(widen(V, kv_dtype, vbase + i) * vs)", "widen(V, kv_dtype, vbase + i)",
                                [pins.check_fp8_attention_on_dequantised_values]),
}


MUTANTS["f64_storage_narrowed"] = ("case OR_F64: return ((const double*)base)[i];",
                                   "case OR_F64: return (float)((const double*)base)[i];",
                                   [pins.check_f64_storage_path])

# The INT8 model is Python: its mutants are loaded as a fresh module.
I8_SRC = os.path.join(os.path.dirname(oracle.__file__), "int8_minmax.py")
I8_MUTANTS = {
    "int8_scale_256": ("np.rint(t * F32(255))", "np.rint(t * F32(256))", [pins.check_int8_formula]),
    "int8_truncates": ("np.rint(t * F32(255))", "np.floor(t * F32(255))", [pins.check_int8_formula]),
    "int8_ties_down": ("np.rint(t * F32(255))", "np.ceil(t * F32(255) - F32(0.5))", [pins.check_int8_formula]),
    "int8_offset_from_max": ("d = x - lo", "d = hi - x", [pins.check_int8_formula, pins.check_int8_round_trip]),
    "int8_value_over_256": ("(lo * (255.0 - c) + hi * c) / 255.0", "(lo * (256.0 - c) + hi * c) / 256.0",
                            [pins.check_int8_round_trip]),
    "int8_value_reversed": ("(lo * (255.0 - c) + hi * c) / 255.0", "(hi * (255.0 - c) + lo * c) / 255.0",
                            [pins.check_int8_round_trip]),
    "int8_no_restart_at_row0": ("if 0 not in rows:", "if True:", [pins.check_int8_fill_invariants]),
    "int8_range_not_widened": ("lo, hi = np.minimum(old_lo, lo), np.maximum(old_hi, hi)", "lo, hi = lo, hi",
                               [pins.check_int8_fill_invariants]),
    "int8_no_reencode": ("codes[h, rest] = encode(value_f32(codes[h, rest], old_lo[h], old_hi[h]), lo[h], hi[h])",
                         "pass", [pins.check_int8_fill_invariants, pins.check_int8_token_fill_vs_one_shot]),
    "int8_reencode_reads_new_range": ("value_f32(codes[h, rest], old_lo[h], old_hi[h])",
                                      "value_f32(codes[h, rest], lo[h], hi[h])",
                                      [pins.check_int8_fill_invariants, pins.check_int8_token_fill_vs_one_shot]),
    "one_shot_range_over_sequence": ("k_min = tile.min(axis=(0, 2))[None, :, None]",
                                     "k_min = x.min(axis=(0, 2))[None, :, None]", [pins.check_int8_one_shot]),
    "one_shot_heads_share_a_range": ("k_max = tile.max(axis=(0, 2))[None, :, None]", "k_max = tile.max()",
                                     [pins.check_int8_one_shot]),
    "one_shot_scale_256": ("* 255.0)\n", "* 256.0)\n", [pins.check_int8_one_shot]),
    "one_shot_truncates": ("q = np.rint(", "q = np.floor(", [pins.check_int8_one_shot]),
    "one_shot_value_reversed": ("(k_min * (255.0 - q) + k_max * q)", "(k_max * (255.0 - q) + k_min * q)",
                                [pins.check_int8_one_shot]),
    "int8_heads_share_a_range": ("lo, hi = new.min(axis=(1, 2)), new.max(axis=(1, 2))",
                                 "lo, hi = np.full(self.H_kv, new.min()), np.full(self.H_kv, new.max())",
                                 [pins.check_int8_fill_invariants]),
}


@pytest.mark.parametrize("name", sorted(I8_MUTANTS))
def test_planted_int8_mistake_is_caught(name):
    import importlib.util
    find, repl, checks = I8_MUTANTS[name]
    with open(I8_SRC) as f:
        src = f.read()
    assert find in src, f"mutation site vanished: {find!r}"
    spec = importlib.util.spec_from_loader(f"int8_mutant_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src.replace(find, repl), f"<{name}>", "exec"), mod.__dict__)
    caught = []
    for check in checks:
        try:
            check(mod)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path, monkeypatch):
    find, repl, checks = MUTANTS[name]
    with open(SRC) as f:
        src = f.read()
    assert find in src, f"mutation site vanished: {find!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(find, repl))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(mutant), "-o", str(so), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.bind(str(so)))
    caught = []
    for check in checks:
        try:
            check()
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
