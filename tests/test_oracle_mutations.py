"""The oracle's pins are strong enough: plant a plausible mistake in a copy of
the oracle source (on the CPU), rebuild it, and check that at least one pin
fails for every mistake.  The pins run here are the ones in
test_oracle_fp8.py, test_oracle_attention.py, test_oracle_dynamic.py and
test_oracle_prefill.py."""
import os
import subprocess
import sys

import pytest

import oracle
from conftest import ROOT
import test_oracle_attention as ta
import test_oracle_dynamic as tdy
import test_oracle_prefill as tpf
import test_oracle_fp8 as tf

SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

# (name, text in the oracle source, replacement)
MUTATIONS = [
    ("drop the softmax scale", "s[t] = (double)sm_scale * dot;", "s[t] = dot;"),
    ("wrong GQA head mapping", "kv = h / G;", "kv = h % Hkv;"),
    ("off-by-one token in K", "dot += qd[d] * orc_load(k_pool, 0, block, kv, t % ORC_BS,",
     "dot += qd[d] * orc_load(k_pool, 0, block, kv, (t + 1) % ORC_BS,"),
    ("drop the V scale", "vs = fp8 ? (double)v_scale : 1.0;", "vs = 1.0;"),
    ("drop the K scale", "double ks = fp8 ? (double)k_scale : 1.0,", "double ks = 1.0,"),
    ("V tile transposed", "(int64_t)((t / 4) * 16 + d % 16) * x", "(int64_t)((d % 16) * 4 + t / 4) * x"),
    ("K tile token-major", "return (int64_t)(d / x) * (ORC_BS * x) + (int64_t)t * x + d % x;",
     "return (int64_t)t * 128 + d;"),
    ("ties to odd", "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    ("overflow to NaN", "return (uint8_t)(0x7E | sign);", "return (uint8_t)(0x7F | sign);"),
    ("FNUZ exponent bias", "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("subnormal scale", "v = ldexp((double)m / 8.0, -6);", "v = ldexp((double)m / 8.0, -7);"),
    ("reciprocal multiply", "return (float)(x / (double)scale);",
     "return (float)((float)x * (1.0f / scale));"),
    ("fp16 subnormals", "v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    ("denominator squared", "den += w;", "den += w * w;"),
    ("slot offset dropped", "return (int64_t)table_row[pos / ORC_BS] * ORC_BS + pos % ORC_BS;",
     "return (int64_t)table_row[pos / ORC_BS] * ORC_BS;"),
    ("stale table entry read", "int64_t block = row[t / ORC_BS];\n      double w",
     "int64_t block = row[t / ORC_BS + (t >= 16 ? 1 : 0)];\n      double w"),
    # per-block dynamic scales
    ("no requantization when a scale grows", "if (!fresh && s > s_old) {", "if (0) {"),
    ("fresh block keeps its stale scale", "float s_old = fresh ? 0.0f : *stored;",
     "float s_old = *stored;"),
    ("requantization ratio inverted", "float r = oracle_quotient((double)s_old, s);",
     "float r = oracle_quotient((double)s, s_old);"),
    ("block scale ignores the head", "(double)k_bscales[block * Hkv + kv]",
     "(double)k_bscales[block * Hkv]"),
    ("V read with the K block scale", "(double)v_bscales[block * Hkv + kv]",
     "(double)k_bscales[block * Hkv + kv]"),
    ("scale floor dropped", "if (s < floor_scale)\n          s = floor_scale;", ""),
    ("MaxAbs not divided by 448", "oracle_quotient(amax[(b * Hkv + h) * 2 + is_v], 448.0f)",
     "(float)amax[(b * Hkv + h) * 2 + is_v]"),
    ("non-finite inputs measured", "return isfinite(x) ? fabs(x) : 0.0;", "return fabs(x);"),
    ("K MaxAbs taken from V", "if (xk > ak[0])\n          ak[0] = xk;",
     "if (xv > ak[0])\n          ak[0] = xv;"),
    ("new scale not stored", "        *stored = s;\n", ""),
    # chunked prefill
    ("prefill row does not see itself", "int64_t cnt = pos + 1;", "int64_t cnt = pos;"),
    ("prefill position off by one", "int64_t pos = (int64_t)L - n + (r - query_start[b]);",
     "int64_t pos = (int64_t)L - n + (r - query_start[b]) - 1;"),
    ("prefill GQA mapping", "kvh = h / G;", "kvh = h % Hkv;"),
    ("prefill drops the V scale", "double vfac = fp8 ? (double)v_scale : 1.0;", "double vfac = 1.0;"),
    ("prefill normaliser squared", "wsum += w;", "wsum += w * w;"),
    # chunked prefill over per-block scales
    ("prefill block scale ignores the head", "(double)k_bscales[block * Hkv + kvh]",
     "(double)k_bscales[block * Hkv]"),
    ("prefill V read with the K block scale", "(double)v_bscales[blk * Hkv + kvh]",
     "(double)k_bscales[blk * Hkv + kvh]"),
]


def _pins(orc):
    """Run the pins; return the names of those that fail."""
    failed = []
    checks = [
        ("decode table", lambda: tf.test_decode_table_matches_library_view_cast(orc)),
        ("encode fp16", lambda: tf.test_encode_matches_library_on_all_fp16_values(orc)),
        ("encode ties", lambda: tf.test_encode_matches_library_on_midpoints_and_neighbours(orc)),
        ("saturate", lambda: tf.test_encode_hand_cases(orc, 1000.0, 0x7E)),
        ("quotient", lambda: tf.test_quotient_is_correctly_rounded_fp32_division(orc)),
        ("layout golden", lambda: ta.test_layout_offsets_golden(orc)),
        ("slot figure", lambda: ta.test_slot_follows_block_table_figure(orc)),
        ("write offsets fp8", lambda: ta.test_write_places_bytes_at_documented_offsets(orc, True)),
        ("sdpa fp16 G4", lambda: ta.test_decode_matches_library_sdpa(orc, False, 8, 2)),
        ("sdpa fp8 G2", lambda: ta.test_decode_matches_library_sdpa(orc, True, 6, 3)),
        ("single token fp8", lambda: ta.test_decode_single_token_returns_its_value_row(orc, True)),
        ("zero query", lambda: ta.test_decode_zero_query_is_mean_of_values(orc)),
        ("dyn one call", lambda: tdy.test_one_call_fill_matches_library_cast(orc)),
        ("dyn growth 2x", lambda: tdy.test_growth_by_a_power_of_two_requantizes_old_rows_exactly(orc)),
        ("dyn fresh", lambda: tdy.test_offset_zero_starts_a_fresh_block(orc)),
        ("dyn floor", lambda: tdy.test_zero_rows_get_the_floor_scale_and_non_finite_values_are_not_measured(orc)),
        ("dyn sdpa", lambda: tdy.test_decode_with_block_scales_matches_library_sdpa(orc, 8, 2)),
        ("prefill sdpa fp8", lambda: tpf.test_prefill_matches_library_sdpa_with_causal_mask(orc, True, 8, 2)),
        ("prefill causality", lambda: tpf.test_future_tokens_do_not_leak(orc)),
        ("prefill dyn sdpa", lambda: tdy.test_prefill_with_block_scales_matches_library_sdpa(orc, 8, 2)),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_oracle_passes_every_pin(orc):
    assert _pins(orc) == []


_RUNNER = """
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle, test_oracle_mutations as m
oracle._swap_library({lib!r})
print('FAILED:' + ','.join(m._pins(oracle)), flush=True)
"""


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(orc, tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                    str(mutant), "-o", str(lib), "-lm"], check=True)
    # a separate process: a mutant may also crash (an out-of-bounds read),
    # which counts as caught
    code = _RUNNER.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=str(lib))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, env=dict(os.environ, OMP_NUM_THREADS="4"))
    if r.returncode != 0:
        return   # crashed or raised: caught
    line = [x for x in r.stdout.splitlines() if x.startswith("FAILED:")][-1]
    failed = [x for x in line[len("FAILED:"):].split(",") if x]
    assert failed, f"no pin caught the planted mistake '{name}'"
