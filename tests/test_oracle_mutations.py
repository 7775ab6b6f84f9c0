"""The oracle's pins catch planted mistakes.

Each case copies oracle/oracle.c to a temporary directory, plants one
plausible mistake (an off-by-one in the causal mask, a dropped scale, log
base 2, a transposed or wrong operand, a wrong index in the paged layout, a
wrong sign in an online rescale, ...), builds that copy and runs the pin
suites (the tests/test_oracle_*.py files in PIN_SUITES) against it in a
subprocess.  The mutation passes only
if at least one pin fails.  A control run of the unmodified copy must pass.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_decode.py",
              "tests/test_oracle_tiling.py", "tests/test_oracle_bwd.py", "tests/test_oracle_fp8.py",
              "tests/test_oracle_ext.py", "tests/test_oracle_blocks.py", "tests/test_oracle_prefill.py"]

# (name, text in oracle.c, replacement); the text must occur in the source
MUTATIONS = [
    ("prefill_causal_offset_sign",
     "int64_t last = i + ctx - x->Nq;",
     "int64_t last = i - ctx + x->Nq;"),
    ("prefill_causal_excludes_own_token",
     "n = last + 1 < ctx ? last + 1 : ctx;",
     "n = last < ctx ? last : ctx;"),
    ("prefill_query_rows_collapsed",
     "int64_t qbase = item * dx->D;",
     "int64_t qbase = sh * dx->D;"),
    ("prefill_kv_head_mapping",
     "int kvh = h / (dx->H / dx->Hkv);",
     "int kvh = h % dx->Hkv;"),
    ("mask_blocks_last_row_dropped",
     "for (int i = qb * 128; i < qb * 128 + 128 && i < Nq; ++i)",
     "for (int i = qb * 128; i < qb * 128 + 127 && i < Nq; ++i)"),
    ("mask_blocks_halves_swapped",
     "if (any) words[kb / 32] |= 1u << (kb % 32);",
     "if (any) words[nkw + kb / 32] |= 1u << (kb % 32);"),
    ("mask_blocks_row_stride_nk",
     "(int64_t)i * mask_ld + j] != 0)",
     "(int64_t)i * Nk + j] != 0)"),
    ("mask_blocks_key_range_off_by_one",
     "for (int j = kb * 64; j < kb * 64 + 64 && j < Nk; ++j) {",
     "for (int j = kb * 64; j < kb * 64 + 64 && j <= Nk; ++j) {"),
    ("causal_mask_excludes_diagonal",
     "int64_t n = x->causal ? (i + 1 < x->N ? i + 1 : x->N) : x->N;",
     "int64_t n = x->causal ? (i < x->N ? i : x->N) : x->N;"),
    ("scale_dropped",
     "s[j] = x->scale * dot;",
     "s[j] = dot;"),
    ("scores_use_q_twice",
     "or_load(x->k, x->dtype, kvbase + j * x->d + c)",
     "or_load(x->q, x->dtype, base + j * x->d + c)"),
    ("max_not_subtracted_in_lse",
     "    return m + log(l);\n}",
     "    return log(l);\n}"),
    ("lse_log2",
     "    return m + log(l);\n}",
     "    return m + log2(l);\n}"),
    ("output_not_normalised",
     "o[c] = acc / l;",
     "o[c] = acc;"),
    ("value_columns_reversed",
     "return or_load(dv->v, dv->dtype, dv->base + j * dv->d + c);",
     "return or_load(dv->v, dv->dtype, dv->base + j * dv->d + (dv->d - 1 - c));"),
    ("fp16_exponent_bias",
     "mag = ldexp((double)(1024 + f), e - 25);",
     "mag = ldexp((double)(1024 + f), e - 24);"),
    ("tiled_fa1_merge_sign",
     "double w1 = *l1 * exp(*m1 - m), w2 = l2 * exp(m2 - m);",
     "double w1 = *l1 * exp(m - *m1), w2 = l2 * exp(m2 - m);"),
    ("tiled_fa2_rescale_sign",
     "double alpha = exp(m - mnew);",
     "double alpha = exp(mnew - m);"),
    ("dense_kv_head_mapping",
     "int64_t kvbase = (b * x->Hkv + h / (x->H / x->Hkv)) * (int64_t)x->N * x->d;",
     "int64_t kvbase = (b * x->Hkv + h % x->Hkv) * (int64_t)x->N * x->d;"),
    ("decode_kv_head_mapping",
     "int kvh = h / (x->H / x->Hkv);",
     "int kvh = h % x->Hkv;"),
    ("decode_k_layout_chunk_swapped",
     "+ e / x->x) * x->BS + off) * x->x) + e % x->x;",
     "+ e % x->x) * x->BS + off) * x->x) + e / x->x;"),
    ("decode_v_token_off_by_one",
     "or_v_index(x, blk, pv->kvh, e, (int)(t % x->BS))",
     "or_v_index(x, blk, pv->kvh, e, (int)((t + 1) % x->BS))"),
    ("merge_ignores_partition_sums",
     "double w = x->part_l[item * x->P + p] * exp(x->part_m[item * x->P + p] - m_all);",
     "double w = exp(x->part_m[item * x->P + p] - m_all);"),
    ("bwd_dq_without_D",
     "acc += s[j] * (dp[j] - D) * or_load(x->k, x->dtype, kb + j * d + c);",
     "acc += s[j] * dp[j] * or_load(x->k, x->dtype, kb + j * d + c);"),
    ("bwd_dk_without_D",
     "double ds = p * (dp - x->D[st + i]);",
     "double ds = p * dp;"),
    ("bwd_dS_sign",
     "double ds = p * (dp - x->D[st + i]);",
     "double ds = p * (x->D[st + i] - dp);"),
    ("bwd_D_unweighted",
     "D += s[j] * dp[j];",
     "D += dp[j];"),
    ("bwd_dq_scale_dropped",
     "dq[c] = x->scale * acc;",
     "dq[c] = acc;"),
    ("bwd_dk_scale_dropped",
     "for (int c = 0; c < d; ++c) dk[c] *= x->scale;",
     ""),
    ("bwd_dv_reads_q",
     "dv[c] += p * or_load(x->dout, x->dtype, qb + i * d + c);",
     "dv[c] += p * or_load(x->q, x->dtype, qb + i * d + c);"),
    ("bwd_dP_uses_keys",
     "dp[j] = or_dot(x->dout, qb + i * d, x->v, kb + j * d, x->dtype, x->d);",
     "dp[j] = or_dot(x->dout, qb + i * d, x->k, kb + j * d, x->dtype, x->d);"),
    ("bwd_causal_skips_diagonal",
     "for (int64_t i = x->causal ? j : 0; i < N; ++i) {",
     "for (int64_t i = x->causal ? j + 1 : 0; i < N; ++i) {"),
    ("e4m3_exponent_bias_8",
     "return (uint8_t)(s | (uint8_t)((E + 7) << 3) | (uint8_t)m);",
     "return (uint8_t)(s | (uint8_t)((E + 8) << 3) | (uint8_t)m);"),
    ("e4m3_subnormal_step",
     "double m = nearbyint(ldexp(a, 9));",
     "double m = nearbyint(ldexp(a, 10));"),
    ("e4m3_mantissa_truncated",
     "double m = nearbyint((ldexp(a, -E) - 1.0) * 8.0);",
     "double m = floor((ldexp(a, -E) - 1.0) * 8.0);"),
    ("e4m3_decode_bias",
     "else v = ldexp(1.0 + m / 8.0, ef - 7);",
     "else v = ldexp(1.0 + m / 8.0, ef - 8);"),
    ("fp8_block_exponent_offset",
     "e = (ex - 1) - 7;",
     "e = (ex - 1) - 8;"),
    ("fp8_tile_layout_swapped",
     "return ((bh * T + i / 64) * d + c) * 64 + (i % 64);",
     "return ((bh * T + i / 64) * 64 + (i % 64)) * d + c;"),
    ("ext_causal_offset_sign",
     "if (x->causal && j > i + off) return 0;",
     "if (x->causal && j > i - off) return 0;"),
    ("ext_window_left_off_by_one",
     "if (x->wl >= 0 && j < i + off - x->wl) return 0;",
     "if (x->wl >= 0 && j <= i + off - x->wl) return 0;"),
    ("ext_window_right_ignored",
     "if (x->wr >= 0 && j > i + off + x->wr) return 0;",
     ""),
    ("ext_mask_transposed",
     "x->mask[b * x->msb + h * x->msh + i * x->Nk + j]",
     "x->mask[b * x->msb + h * x->msh + j * x->Nq + i]"),
    ("ext_mask_head_stride_dropped",
     "x->mask[b * x->msb + h * x->msh + i * x->Nk + j]",
     "x->mask[b * x->msb + i * x->Nk + j]"),
    ("bwd_group_mapping",
     "for (int64_t h = g * group; h < (g + 1) * group; ++h) {",
     "for (int64_t h = g; h < x->H; h += x->Hkv) {"),
]


def run_pins(workdir, source_text):
    os.makedirs(workdir, exist_ok=True)
    src = os.path.join(workdir, "oracle.c")
    with open(src, "w") as f:
        f.write(source_text)
    env = dict(os.environ, ORACLE_TEST_SOURCE=src, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + PIN_SUITES
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    """Run the pin suites on the unmodified copy and on every mutated copy,
    several subprocesses at a time; results by case name."""
    text = open(SRC).read()
    cases = {"control": text}
    for name, old, new in MUTATIONS:
        cases[name] = text.replace(old, new, 1) if text.count(old) >= 1 else None
    base = tmp_path_factory.mktemp("oracle_mutations")
    workers = max(1, min(8, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))
    results = {n: None for n in cases}  # None: the mutation site was not found
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        futs = {n: pool.submit(run_pins, str(base / n), t) for n, t in cases.items() if t is not None}
        results.update({n: f.result() for n, f in futs.items()})
    return results


def test_control_copy_passes(pin_runs):
    res = pin_runs["control"]
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(pin_runs, name, old, new):
    res = pin_runs[name]
    assert res is not None, "mutation site not found: " + name
    assert res.returncode != 0, "no pin failed for mutation %s:\n%s" % (name, res.stdout[-2000:])
