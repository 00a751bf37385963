"""The oracle's pins catch plausible mistakes (CPU only).

Each case copies oracle.c, plants one slip in the copy, builds it with gcc
into a temporary library, and runs tests/test_oracle_pins.py against that
library (through the oracle's KVD_ORACLE_LIB override) in a subprocess.  The
pin suite must fail for every planted slip.  The committed oracle is never
modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrence to replace: 0-based index)
MUTANTS = [
    ("meta_max_is_min", "if (x > hi) hi = x;", "if (x < hi) hi = x;", 0),
    ("meta_ignores_valid_count", "for (int s = 0; s < nv; ++s)", "for (int s = 0; s < bs; ++s)", 0),
    ("score_min_not_max", "acc += (a > e) ? a : e;", "acc += (a < e) ? a : e;", 0),
    ("score_kmax_only", "acc += (a > e) ? a : e;", "acc += e;", 0),
    ("score_wrong_head_map", "const int j = h / G;", "const int j = h % Hkv;", 0),
    ("group_min_not_max", "if (s > best) best = s;", "if (s < best || best == -INFINITY) best = s;", 0),
    ("topk_ties_to_higher_index", "(s[m] == s[n] && m < n)", "(s[m] == s[n] && m > n)", 0),
    ("topk_keeps_one_too_many", "if (rank < keff) out[w++]", "if (rank <= keff && w < K) out[w++]", 0),
    ("attn_drops_scale", "const double z = scale * dot;", "const double z = dot;", 0),
    ("attn_token_off_by_one", "if (t >= L) break;", "if (t > L) break;", 0),
    ("attn_value_is_key", "const double* v = pool_row(v_pool", "const double* v = pool_row(k_pool", 0),
    ("attn_wrong_kv_head", "const int j = h / G;", "const int j = h % Hkv;", 2),
    ("attn_unnormalised", "for (int c = 0; c < D; ++c) o[c] /= l;", "", 0),
    ("split_chunks_overlap", "i64 p0 = (i64)s * chunk, p1 = p0 + chunk;",
     "i64 p0 = (i64)s * chunk, p1 = p0 + chunk + 1;", 0),
    ("combine_drops_l", "const double w = part_l[r * S + s] * exp(ms - M);",
     "const double w = exp(ms - M);", 0),
    ("mean_divides_by_block_size", "out[c] = sum / nv;", "out[c] = sum / bs;", 0),
    ("mean_counts_every_slot", "for (int s = 0; s < nv; ++s) sum +=", "for (int s = 0; s < bs; ++s) sum +=", 0),
    ("mean_score_wrong_head_map", "const int j = h / G;", "const int j = h % Hkv;", 1),
    ("mean_score_uses_the_first_page", "const i64 p = block_table[(i64)b * maxN + n];\n        const double* km",
     "const i64 p = block_table[(i64)b * maxN];\n        const double* km", 0),
    ("forced_local_off_by_one", "(n + 1) * bs > L - local", "(n + 1) * bs >= L - local", 0),
    ("forced_sink_inclusive", "n * bs < sink", "n * bs <= sink", 0),
    ("forced_not_counted_against_k", "const i64 free_slots = keff - n_forced;",
     "const i64 free_slots = keff;", 0),
    ("forced_blocks_compete_for_rank", "if (is_forced(m, L, bs, sink, local)) continue;", "", 0),
    ("fp8_decode_bias_8", "ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 11)", 0),
    ("fp8_subnormal_step", "ldexp((double)m, -9)", "ldexp((double)m, -10)", 0),
    ("fp8_round_half_away", "double r = nearbyint(a / step) * step;", "double r = round(a / step) * step;", 0),
    ("fp8_no_saturation", "if (r > 448.0) r = 448.0;", "", 0),
    ("fp8_scale_240", "amax / 448.0f", "amax / 240.0f", 0),
    ("fp8_amax_over_every_slot", "for (int s = 0; s < nv; ++s) {\n        const double* row = pool_row(pool",
     "for (int s = 0; s < bs; ++s) {\n        const double* row = pool_row(pool", 0),
    ("fp8_tail_slots_encoded", "if (s >= nv) {\n          memset", "if (s >= bs) {\n          memset", 0),
    ("int4_scale_8", "amax / 7.0f", "amax / 8.0f", 0),
    ("int4_round_half_away", "double r = nearbyint((double)y);", "double r = round((double)y);", 0),
    ("int4_nibbles_swapped", "out[c / 2] |= (uint8_t)((n & 15) << (4 * (c & 1)));",
     "out[c / 2] |= (uint8_t)((n & 15) << (4 * (1 - (c & 1))));", 0),
    ("int4_amax_over_every_slot", "for (int s = 0; s < nv; ++s) {\n        const double* row = pool_row(pool",
     "for (int s = 0; s < bs; ++s) {\n        const double* row = pool_row(pool", 1),
    ("int4_tail_slots_encoded", "if (s >= nv) continue;", "if (s >= bs) continue;", 0),
    ("cache_evicts_highest_mass", "if (mass[ck] < mass[cb] || (mass[ck] == mass[cb] && ck < cb)) best = k;",
     "if (mass[ck] > mass[cb] || (mass[ck] == mass[cb] && ck < cb)) best = k;", 0),
    ("cache_ties_to_higher_slot", "(mass[ck] == mass[cb] && ck < cb)", "(mass[ck] == mass[cb] && ck > cb)", 0),
    ("cache_free_slots_not_first", "for (int c = 0; c < C; ++c) if (sb[c] < 0) cand[nc++] = c;\n      const int n_free = nc;",
     "const int n_free = 0;", 0),
    ("cache_stale_reverse_map", "if (sb[s] >= 0) bsl[sb[s]] = -1;", "", 0),
    ("cache_hits_refetched", "if (s >= 0) { out_slots[pos] = s; in_use[s] = 1; }", "", 0),
    ("cache_misses_in_mass_order", "if (cand[k] < cand[lo]) lo = k;", "if (0) lo = k;", 0),
    ("block_lse_reads_past_the_end", "for (int s = 0; s < bs && n * bs + s < L; ++s) {", "for (int s = 0; s < bs; ++s) {", 0),
    ("slot_mass_sums_heads", "if (w > best) best = w;", "best += w;", 0),
    ("combine_lse_drops_max", "if (lse) lse[r] = M + log(wsum);", "if (lse) lse[r] = log(wsum);", 0),
    ("tier_cooldown_strict", "(i64)step - stamp[p] >= cooldown", "(i64)step - stamp[p] > cooldown", 0),
    ("tier_hit_only_first_head", "for (int j = 0; j < Hkv && !hit; ++j)", "for (int j = 0; j < 1 && !hit; ++j)", 0),
    ("tier_recent_off_by_one", "n * bs + bs - 1 >= L - recent", "n * bs + bs - 1 > L - recent", 0),
    ("tier_decay_swapped", "fmaf(decay, heat[p], 1.0f - decay) : decay * heat[p]",
     "fmaf(1.0f - decay, heat[p], decay) : (1.0f - decay) * heat[p]", 0),
    ("tier_cold_below_inclusive", "!is_recent && h < cold_below", "!is_recent && h <= cold_below", 0),
    ("tier_hot_above_inclusive", "(h > hot_above &&", "(h >= hot_above &&", 0),
    ("tier_stamp_not_set", "stamp[p] = step;\n", "", 0),
    ("tier_recent_not_promoted", "} else if (is_recent || (h > hot_above", "} else if ((h > hot_above", 0),
    ("tier_recent_demoted", "if (!is_recent && h < cold_below)", "if (h < cold_below)", 0),
    ("tier_lists_not_cleared", "for (int n = 0; n < maxN; ++n) { dem[n] = -1; pro[n] = -1; }", "", 0),
    ("tier_miss_keeps_heat", ": decay * heat[p];", ": heat[p];", 0),
]


def _replace_nth(text, old, new, n):
    start = -1
    for _ in range(n + 1):
        start = text.find(old, start + 1)
        if start < 0:
            raise AssertionError(f"pattern not found ({n}): {old!r}")
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,nth", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, nth):
    with open(SRC) as f:
        text = f.read()
    mutated = _replace_nth(text, old, new, nth)
    assert mutated != text
    src = tmp_path / "oracle_mut.c"
    lib = tmp_path / "liboracle_mut.so"
    src.write_text(mutated)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-o", str(lib), str(src), "-lm"], check=True)
    env = dict(os.environ, KVD_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
