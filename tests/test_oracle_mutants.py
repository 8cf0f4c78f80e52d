"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins
catch every one.  The real oracle is never modified: each mutant is a patched copy of
pa_oracle.c compiled into a temporary library that replaces the loaded one only for the
duration of one test."""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pa_oracle.c")

# (name, text in pa_oracle.c, replacement)
MUTANTS = [
    ("alibi_sign", "sj += slope * (double)(j - pos);", "sj += slope * (double)(pos - j);"),
    ("alibi_dropped", "if (has_alibi) sj += slope", "if (0) sj += slope"),
    ("scale_dropped", "double sj = (double)L->scale * dot;", "double sj = dot;"),
    ("window_off_by_one", "pos - W + 1 > 0) ? pos - W + 1 : 0;", "pos - W > 0) ? pos - W : 0;"),
    ("slot_offset", "int64_t offset = s % L->block_size;", "int64_t offset = (s + 1) % L->block_size;"),
    ("table_index", "table_row[j / L->block_size]", "table_row[j % L->block_size]"),
    ("kv_head_in_unpage", "cache_index(L, block, offset, g, d);\n            if (L->kv_cache_dtype", "cache_index(L, block, offset, 0, d);\n            if (L->kv_cache_dtype"),
    ("gqa_map_decode", "for (int64_t h = g * G; h < (g + 1) * G; ++h) {\n                for (int64_t d = 0; d < D; ++d) q[d] = elt_to_double(query, i * q_stride + h * D + d",
     "for (int64_t h = g * G; h < (g + 1) * G; ++h) {\n                for (int64_t d = 0; d < D; ++d) q[d] = elt_to_double(query, i * q_stride + ((h % Hkv) * G + h / Hkv) * D + d"),
    ("prefill_local_position", "attend_row(L, q, K, V, c + t, h", "attend_row(L, q, K, V, t + (c > 0 ? c - 1 : 0), h"),
    ("decode_position", "attend_row(L, q, K, V, n - 1, h", "attend_row(L, q, K, V, n > 1 ? n - 2 : 0, h"),
    ("softmax_denominator", "out[d] /= denom;", "out[d] /= (denom + 1e-3);"),
    ("bf16_promotion", "<< 16;\n        float f;", "<< 15;\n        float f;"),
    ("value_plane", "const char *vc = kc + plane * cache_elt_bytes(L);", "const char *vc = kc;"),
    ("copy_direction", "memmove(c + pl * plane + dst * bb, c + pl * plane + src * bb", "memmove(c + pl * plane + src * bb, c + pl * plane + dst * bb"),
    ("copy_key_plane_only", "for (int pl = 0; pl < 2; ++pl) memmove(", "for (int pl = 0; pl < 1; ++pl) memmove("),
    ("softcap_divisor", "sj = cap * tanh(sj / cap);", "sj = cap * tanh(sj);"),
    ("softcap_after_alibi", "if (cap > 0.0) sj = cap * tanh(sj / cap);\n        if (has_alibi) sj += slope * (double)(j - pos);",
     "if (has_alibi) sj += slope * (double)(j - pos);\n        if (cap > 0.0) sj = cap * tanh(sj / cap);"),
    ("softcap_dropped", "if (cap > 0.0) sj = cap", "if (0) sj = cap"),
    ("sink_in_max_only", "double denom = L->sinks ? exp(sink - m) : 0.0;", "double denom = 0.0;"),
    ("sink_wrong_head", "sink = (double)L->sinks[h];", "sink = (double)L->sinks[0];"),
    ("f16_exponent_bias", "e - 25);            /* (1 + f/1024)", "e - 24);            /* (1 + f/1024)"),
    ("f16_subnormal", "ldexp((double)f, -24);", "ldexp((double)f, -25);"),
    ("e4m3_exponent_bias", "ldexp((double)(8 + f), e - 10);", "ldexp((double)(8 + f), e - 9);"),
    ("e4m3_subnormal", "v = ldexp((double)f, -9);", "v = ldexp((double)f, -10);"),
    ("e4m3_ties_odd", "(err == best_err && (c & 1) == 0)", "(err == best_err && (c & 1) == 1)"),
    ("e4m3_no_saturation", "if (a >= 448.0) return sign | 0x7E;", "if (a >= 464.0) return sign | 0x7F;"),
    ("fp8_value_scale", "e4m3_to_double(((const uint8_t *)vc)[idx]) * (double)L->v_scale;",
     "e4m3_to_double(((const uint8_t *)vc)[idx]) * (double)L->k_scale;"),
    ("fp8_quantize_unscaled", "(float)elt_to_double(key, src, L->dtype) / L->k_scale;", "(float)elt_to_double(key, src, L->dtype);"),
    ("multi_position", "attend_row(L, q, K, V, n - Q + t, h,", "attend_row(L, q, K, V, n - 1, h,"),
    ("multi_query_row", "elt_to_double(query, (i * Q + t) * q_stride + h * D + d", "elt_to_double(query, (i * Q) * q_stride + h * D + d"),
    ("swap_plane_stride", "(char *)dst_cache + (pl * dst_blocks + dst) * bb", "(char *)dst_cache + (pl * src_blocks + dst) * bb"),
]


def _build_mutant(name, old, new, workdir):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant {name}: anchor text must occur exactly once"
    path = os.path.join(workdir, f"mut_{name}.c")
    with open(path, "w") as f:
        f.write(text.replace(old, new))
    lib = os.path.join(workdir, f"libmut_{name}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", path, "-o", lib, "-lm"], check=True)
    return lib


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(oracle_lib, name, old, new):
    import ctypes
    with tempfile.TemporaryDirectory() as d:
        lib_path = _build_mutant(name, old, new, d)
        saved_lib, saved_path = oracle._lib, oracle._LIB
        try:
            oracle._lib = None
            oracle._LIB = lib_path
            oracle._load()
            caught = []
            for pin in pins.PINS:
                try:
                    pin()
                except (AssertionError, RuntimeError) as e:
                    caught.append(pin.__name__)
            assert caught, f"no pin caught mutant {name}"
        finally:
            oracle._lib, oracle._LIB = saved_lib, saved_path
