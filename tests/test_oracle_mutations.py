"""Planted mistakes in the oracle (built on the CPU only) must each fail a pin.

Each mutation is a plausible slip in oracle.c: a dropped term, a wrong sign,
a wrong index, a transposed layout, an off-by-one in the causal bound.  The
mutated source is compiled into a temporary library; the pins from
oracle_pins.py run against it and at least one must fail.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTATIONS = {
    "gqa_modulo_mapping": ("h / g, Hkv, D, bs, num_blocks, scale, scores);\n    }\n  }\n  free(scores);\n  return rc;\n}\n\n/* q and",
                           "h % Hkv, Hkv, D, bs, num_blocks, scale, scores);\n    }\n  }\n  free(scores);\n  return rc;\n}\n\n/* q and"),
    "wrong_offset_in_block": ("int64_t base = cache_index(phys, kh, t % bs, 0, Hkv, bs, D);",
                              "int64_t base = cache_index(phys, kh, (t + 1) % bs, 0, Hkv, bs, D);"),
    "floor_loop_bound": ("  for (int d = 0; d < D; ++d) out[d] = 0.0;\n  if (n_keys <= 0) return ORC_OK;\n  if ((n_keys",
                         "  for (int d = 0; d < D; ++d) out[d] = 0.0;\n  n_keys = (n_keys / bs) * bs;\n  if (n_keys <= 0) return ORC_OK;\n  if ((n_keys"),
    "scale_dropped": ("    scores[t] = scale * dot;", "    scores[t] = dot;"),
    "normalisation_dropped": ("  for (int d = 0; d < D; ++d) out[d] /= l;\n  return ORC_OK;\n}",
                              "  return ORC_OK;\n}"),
    "causal_off_by_one": ("pos + 1,\n", "pos,\n"),
    "nhd_layout_transposed": ("return (((blk * Hkv + h) * (int64_t)bs + off) * D) + d;",
                              "return (((blk * bs + off) * (int64_t)Hkv + h) * D) + d;"),
    "softmax_sign": ("    double e = exp(scores[t] - m);\n    l += e;\n    int64_t base",
                     "    double e = exp(m - scores[t]);\n    l += e;\n    int64_t base"),
    "v_read_from_k": ("out[d] += e * (elem(v_cache, base + d, dtype) * v_scale);\n  }\n  for (int d = 0; d < D; ++d) out[d] /= l;",
                      "out[d] += e * (elem(k_cache, base + d, dtype) * v_scale);\n  }\n  for (int d = 0; d < D; ++d) out[d] /= l;"),
    "kv_write_swapped": ("memcpy((char *)k_cache + dst * eb, (const char *)key + src * eb",
                         "memcpy((char *)k_cache + dst * eb, (const char *)value + src * eb"),
    "prefill_position_from_zero": ("int pos = seq_lens[b] - n_b + i;", "int pos = i;"),
    "fp8_exponent_bias_8": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8_subnormal_scale": ("ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    "fp8_ties_to_odd": ("(dd == best_d && (c & 1) == 0)", "(dd == best_d && (c & 1) == 1)"),
    "fp8_search_misses_largest_code": ("for (int c = 0; c < 127; ++c) {\n    double dd", "for (int c = 0; c < 126; ++c) {\n    double dd"),
    "fp8_k_scaled_by_v_scale": ("(elem(k_cache, base + d, dtype) * k_scale)", "(elem(k_cache, base + d, dtype) * v_scale)"),
    "fp8_write_multiplies_scale": ("fp8_code(kx / k_scale)", "fp8_code(kx * k_scale)"),
    "merge_weights_crossed": ("double wd = exp(dst->top - both), ws = exp(src->top - both);",
                              "double wd = exp(src->top - both), ws = exp(dst->top - both);"),
    "block_summary_not_relative_to_top": ("    double w = exp(scores[o] - s->top);", "    double w = exp(scores[o]);"),
    "merge_keeps_old_top": ("  dst->top = both;\n}", "}"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor for %s must match exactly once" % name
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", str(lib), str(mutated), "-lm"],
                   check=True)
    prev = oracle.use_library(str(lib))
    failed = []
    try:
        for pin in ALL_PINS:
            try:
                pin(oracle)
            except (AssertionError, oracle.OracleError) as e:
                failed.append(pin.__name__)
                break
    finally:
        oracle.restore_library(prev)
    assert failed, "mutation %s passed every pin" % name
