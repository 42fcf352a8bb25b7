"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/moe_oracle.c into a temporary directory, plants one plausible mistake (a
reversed tie-break, a dropped renormalisation, a transposed operand, a wrong rounding mode, ...),
builds it with gcc, and runs the pin tests that should catch it against that build, in a child
process. The case passes when those pins fail. Nothing here touches the GPU.
"""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "check_last_expert_out_of_range": ("if (id < 0 || id >= E) {\n                counts[0]++;",
                                       "if (id < 0 || id > E) {\n                counts[0]++;",
                                       "test_oracle_check.py"),
    "check_repeats_counted_per_pair": ("counts[1]++;\n                    break;",
                                       "counts[1]++;", "test_oracle_check.py"),
    "check_drops_token_offset": ("if (topk_idx[t * k + jj] == id) {", "if (topk_idx[jj] == id) {",
                                 "test_oracle_check.py"),
    "tie_to_higher_id": ("(l[a] == l[b] && a < b)", "(l[a] == l[b] && a > b)",
                         "test_oracle_route.py"),
    "no_renormalisation": ("(float)(p[idx[j]] / kept)", "(float)(p[idx[j]])",
                           "test_oracle_route.py"),
    "softmax_sign": ("p[e] = exp((double)l[e] - mx);", "p[e] = exp(mx - (double)l[e]);",
                     "test_oracle_route.py"),
    "round_robin_ranks": ("it->rank = it->expert / epr;", "it->rank = it->expert % N;",
                          "test_oracle_dispatch.py"),
    "slot_before_token": (
        "if (a->token != b->token) return a->token < b->token ? -1 : 1;\n"
        "    if (a->slot != b->slot) return a->slot < b->slot ? -1 : 1;",
        "if (a->slot != b->slot) return a->slot < b->slot ? -1 : 1;\n"
        "    if (a->token != b->token) return a->token < b->token ? -1 : 1;",
        "test_oracle_dispatch.py"),
    "fnuz_fp8_max": ("amax / 448.0f", "amax / 240.0f", "test_oracle_dispatch.py"),
    "fp8_amax_takes_nan": ("if (a > amax)\n                    amax = a;",
                           "if (!(a <= amax))\n                    amax = a;",
                           "test_oracle_dispatch.py"),
    "fp8_nan_quotient_sign_unset": ("float scaled = copysignf(xv / s[b], xv);",
                                    "float scaled = xv / s[b];", "test_oracle_dispatch.py"),
    "e4m3_subnormal_edge": ("if (ex < -6) ", "if (ex < -7) ", "test_oracle_formats.py"),
    "ties_away_from_zero": ("return nearbyint(a / quantum) * quantum;",
                            "return round(a / quantum) * quantum;", "test_oracle_formats.py"),
    "bf16_min_exponent": ("round_to_format(a, 8, -126)", "round_to_format(a, 8, -125)",
                          "test_oracle_formats.py"),
    "combine_weights_transposed": ("acc += (double)topk_w[t * k + j]",
                                   "acc += (double)topk_w[j * T + t]", "test_oracle_combine.py"),
    "combine_slot0_row_only": ("int64_t row = token_row[t * k + j];\n                acc",
                               "int64_t row = token_row[t * k];\n                acc",
                               "test_oracle_combine.py"),
    "rank_offset_off_by_one": ("rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r];",
                               "rank_offsets[r + 1] = rank_offsets[r] + rank_counts[r] + (r > 0);",
                               "test_oracle_dispatch.py"),
    "ep_source_major_regions": (
        "const int64_t row = ((int64_t)items[n].rank * S + source) * cap + pos;",
        "const int64_t row = ((int64_t)source * N + items[n].rank) * cap + pos;",
        "test_oracle_ep.py"),
    "ep_recv_region_start": ("for (int q = 0; q < l; q++)\n                start += c[q];",
                             "for (int q = 0; q + 1 < l; q++)\n                start += c[q];",
                             "test_oracle_ep.py"),
    "ep_return_skips_row_zero": ("if (grouped_src[g] >= 0)\n            memcpy(",
                                 "if (grouped_src[g] > 0)\n            memcpy(",
                                 "test_oracle_ep.py"),
    "ep_reduce_sums_every_slot": ("if (topk_idx[tt * k + j] / L != rank)\n",
                                  "if (topk_idx[tt * k + j] / L != rank && 0)\n",
                                  "test_oracle_ep_reduce.py"),
    "ep_partial_rows_source_major": (
        "part_row[t * N + r] = on_rank ? (int32_t)(((int64_t)r * S + source) * pcap + p) : -1;",
        "part_row[t * N + r] = on_rank ? (int32_t)(((int64_t)source * N + r) * pcap + p) : -1;",
        "test_oracle_ep_reduce.py"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    before, after, target = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"{name}.so"
    c_path.write_text(src.replace(before, after))
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-shared", "-fPIC",
                           str(c_path), "-o", str(so_path), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(so_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", target)],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "FAILED" in r.stdout, \
        f"mutant {name} survived {target}:\n{r.stdout[-2000:]}"
