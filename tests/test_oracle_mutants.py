"""Plant plausible slips in a copy of oracle.c and check that the pins catch every one.

Each mutant is compiled with gcc into a temporary library and the whole pin
suite (test_oracle_pins.py) runs against it in a child process; a mutant
passes only if at least one pin fails (or the child crashes).
"""
import json
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

MUTANTS = {
    "pool_divides_by_ks_minus_1": ("orc_bf16_from_double(s / ks)", "orc_bf16_from_double(s / (ks - 1))"),
    "pool_window_off_by_one": ("j * bs + (int64_t)m * kst + r;", "j * bs + (int64_t)m * kst + r + 1;"),
    "pool_stride_uses_window": ("j * bs + (int64_t)m * kst + r;", "j * bs + (int64_t)m * ks / 2 * 3 + r;"),
    "pool_pools_partial_block": ("const int64_t nfull = kv_len / bs;", "const int64_t nfull = (kv_len + bs - 1) / bs;"),
    "round_truncates": ("r = rint(a / quantum) * quantum;", "r = floor(a / quantum) * quantum;"),
    "round_wrong_quantum": ("double quantum = ldexp(1.0, e - 7);", "double quantum = ldexp(1.0, e - 8);"),
    "score_min_over_kernels": ("if (dot > best) best = dot;", "if (best == -INFINITY || dot < best) best = dot;"),
    "score_sum_over_kernels": ("if (dot > best) best = dot;", "best = (best == -INFINITY ? 0.0 : best) + dot;"),
    "score_max_over_heads": ("        sum += best;", "        if (hh == 0 || best > sum) sum = best;"),
    "score_strided_heads": ("const int h = g * G + hh;", "const int h = g + hh * Hkv;"),
    "score_own_block_candidate": ("int64_t c = pos[i] / bs;", "int64_t c = pos[i] / bs + 1;"),
    "score_transposed_kernel_index": ("nblk_cap + j) * kpb + m) * D];", "nblk_cap + j) * kpb + (kpb - 1 - m)) * D + (m % 2)];"),
    "select_higher_index_wins_ties": ("return (a->j < b->j) ? -1 : (a->j > b->j);", "return (a->j > b->j) ? -1 : (a->j < b->j);"),
    "select_lowest_scores": ("  if (a->s > b->s) return -1;\n  if (a->s < b->s) return 1;",
                             "  if (a->s < b->s) return -1;\n  if (a->s > b->s) return 1;"),
    "select_in_fp64": ("cs[j].s = (float)R[(int64_t)r * nblk_cap + j];", "cs[j].s = R[(int64_t)r * nblk_cap + j]; cs[j].d = R[(int64_t)r * nblk_cap + j];"),
    "keys_drop_diagonal_token": ("for (int64_t t = own * bs; t <= p; ++t) keys[n++] = t;",
                                 "for (int64_t t = own * bs; t < p; ++t) keys[n++] = t;"),
    "keys_threshold_inclusive": ("    if (dense_threshold > 0 && n_ctx < dense_threshold) {\n      for (int64_t t = 0; t <= p; ++t)",
                                 "    if (dense_threshold > 0 && n_ctx <= dense_threshold) {\n      for (int64_t t = 0; t <= p; ++t)"),
    "tree_drops_prefix_tail": ("for (int64_t t = own * bs; t < P; ++t) keys[n++] = t;", ";"),
    "tree_slot_shift": ("keys[n++] = P + j;\n", "keys[n++] = P + j - (j > 0);\n"),
    "lse_over_block_maxima": ("for (int64_t t = 0; t < c * kpb; ++t) l += exp(s[t] - mx);",
                              "for (int64_t t = 0; t < c * kpb; t += kpb) l += exp(s[t] - mx);"),
    "lse_unscaled": ("s[j * kpb + m] = scale * dot;", "s[j * kpb + m] = dot;"),
    "lse_max_over_heads": ("Rr[j] += exp(best - lse);", "Rr[j] = fmax(Rr[j], exp(best - lse));"),
    "lse_mean_not_max_over_kernels": ("if (s[j * kpb + m] > best) best = s[j * kpb + m];",
                                      "best = (best == -INFINITY ? 0.0 : best) + s[j * kpb + m] / kpb;"),
    "window_start_off_by_one": ("for (int64_t t = p - window + 1 < 0 ? 0 : p - window + 1;",
                                "for (int64_t t = p - window < 0 ? 0 : p - window;"),
    "window_excludes_own_key": ("t <= p && t < kv_len; ++t)\n      keys[n++] = t;",
                                "t < p && t < kv_len; ++t)\n      keys[n++] = t;"),
    "attn_no_scale": ("s[t] = scale * dot;", "s[t] = dot;"),
    "attn_wrong_group_map": ("const int g = h / G;", "const int g = h % Hkv;"),
    "attn_exp_sign": ("const double p = exp(s[t] - mx);", "const double p = exp(mx - s[t]);"),
    "attn_lse_drops_max": ("lse[r] = mx + log(l);", "lse[r] = log(l);"),
    "attn_v_uses_k": ("const uint16_t* vv = &v[", "const uint16_t* vv = &k["),
}


def _mutate(src: str, old: str, new: str, name: str) -> str:
    if name == "select_in_fp64":          # rank on the fp64 score instead of its fp32 rounding
        src = src.replace("typedef struct { float s; int64_t j; } cand_t;",
                          "typedef struct { double s; int64_t j; double d; } cand_t;")
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    return src.replace(old, new, 1)


def _run(name, tmp):
    old, new = MUTANTS[name]
    src = _mutate(open(SRC).read(), old, new, name)
    c_path = os.path.join(tmp, f"{name}.c")
    so_path = os.path.join(tmp, f"{name}.so")
    open(c_path, "w").write(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so_path,
                    c_path, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), so_path],
                       capture_output=True, text=True, timeout=600, env=env)
    if p.returncode != 0:
        return name, ["crashed"]
    return name, json.loads(p.stdout.strip().splitlines()[-1])


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
            results = dict(ex.map(lambda n: _run(n, tmp), sorted(MUTANTS)))
    survivors = [n for n, f in results.items() if not f]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


@pytest.mark.parametrize("name", ["unmutated"])
def test_runner_passes_on_the_real_oracle(name, orc):
    p = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), orc.build(force=False)],
                       capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, p.stderr[-2000:]
    assert json.loads(p.stdout.strip().splitlines()[-1]) == []
