"""Plant plausible mistakes in a copy of the oracle and check that the pins
in test_oracle_pins.py catch every one (CPU only; the real oracle source is
never modified).  Each mutant is a textual edit of oracle/oracle.c built to
a temporary library that the pin suite then loads via MOE_ORACLE_LIB."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "bias_sign": ("if (bg) s = s + bg[e];", "if (bg) s = s - bg[e];"),
    "unfused_router": (
        "s = fmaf(elem_f(x, c->dtype, t * d + i), wg[(int64_t)e * d + i], s);",
        "s = s + elem_f(x, c->dtype, t * d + i) * wg[(int64_t)e * d + i];"),
    "router_transposed": ("wg[(int64_t)e * d + i]", "wg[(int64_t)i * c->E + e]"),
    "tie_to_higher_index": ("score[e] > score[best]", "score[e] >= score[best]"),
    "softmax_sign": ("w[j] = exp((double)score[idx[j]] - m);",
                     "w[j] = exp(m - (double)score[idx[j]]);"),
    "softmax_not_normalised": ("w[j] = w[j] / z;", "w[j] = w[j] / (double)k;"),
    "gelu_constant": ("erf(a * M_SQRT1_2)", "erf(a * M_SQRT2)"),
    "silu_sign": ("return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    "up_rows_reused": ("ub + (h + n) * d + i", "ub + n * d + i"),
    "gate_up_swapped": ("hid[n] = silu(g) * u;", "hid[n] = silu(u) * g;"),
    "down_transposed": ("db + o * h + n", "db + n * d + o"),
    "dropped_up_bias": ("if (W->b_up) a += elem(W->b_up, dt, eo * h + n);", ""),
    "dropped_down_bias": (
        "if (c->act == ORACLE_GELU && W->b_down) s += elem(W->b_down, dt, eo * d + o);", ""),
    "combine_unweighted": ("yo[i] += wr[j] * ye[i];", "yo[i] += ye[i];"),
    "shared_dropped": ("for (int64_t i = 0; i < d; ++i) yo[i] += ye[i];\n      }",
                       "}"),
    "perm_src_modulo": ("if (idx[f] != e) continue;\n      perm_src[p] = (int32_t)(f / c->k);",
                        "if (idx[f] != e) continue;\n      perm_src[p] = (int32_t)(f % c->k);"),
    "kept_perm_src_modulo": (
        "if (idx[f] != e || !keep[f]) continue;\n      perm_src[p] = (int32_t)(f / c->k);",
        "if (idx[f] != e || !keep[f]) continue;\n      perm_src[p] = (int32_t)(f % c->k);"),
    "count_from_one": ("counts[e] = 0;", "counts[e] = (e == 0);"),
    "sample_variance": ("var /= n;", "var /= (n - 1);"),
    "lb_missing_E": ("lb *= E;", ""),
    "swiglu_params_2dh": ("(c->act == ORACLE_GELU ? 2 : 3)", "2"),
    "bf16_low_half": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "capacity_off_by_one": ("keep[f] = (capacity == 0 || taken[e] < capacity) ? 1 : 0;",
                            "keep[f] = (capacity == 0 || taken[e] <= capacity) ? 1 : 0;"),
    "capacity_ignored_in_forward": ("if (keep && !keep[t * c->k + j]) continue;", ""),
    "grouping_ignores_drops": ("if (idx[f] != e || !keep[f]) continue;",
                               "if (idx[f] != e) continue;"),
    "bias_selects_uses_biased_scores": ("kept_softmax(raw, idx, c->k, w);",
                                        "kept_softmax(score, idx, c->k, w);"),
    "raw_scores_include_bias": ("    raw[e] = s;\n    if (bg) s = s + bg[e];",
                                "    if (bg) s = s + bg[e];\n    raw[e] = s;"),
    "softmax_all_renormalised": (
        "for (int e = 0; e < E; ++e) z += exp((double)score[e] - m);",
        "for (int j = 0; j < k; ++j) z += exp((double)score[idx[j]] - m);"),
    "softmax_all_off_by_one_sum": (
        "for (int e = 0; e < E; ++e) z += exp((double)score[e] - m);",
        "for (int e = 1; e < E; ++e) z += exp((double)score[e] - m);"),
    "gate_mode_ignored": ("if (c->gate == ORACLE_GATE_BIAS_SELECTS)", "if (0)"),
    "noisy_h_unfused": ("hs[e] = fmaf(noise[t * E + e], sc[e], cs[e]);",
                        "hs[e] = cs[e] + noise[t * E + e] * sc[e];"),
    "noise_transposed": ("hs[e] = fmaf(noise[t * E + e], sc[e], cs[e]);",
                         "hs[e] = fmaf(noise[e * c->T + t], sc[e], cs[e]);"),
    "softplus_missing_log": ("v > 0.0 ? v + log1p(exp(-v)) : log1p(exp(v));",
                             "v > 0.0 ? v + log1p(exp(-v)) : exp(v);"),
    "noisy_threshold_not_excluding": ("order[tk[e] ? k : k - 1]", "order[k - 1]"),
    "smooth_load_uses_noisy_score": ("const double diff = (double)cs[e] - thr;",
                                     "const double diff = (double)hs[e] - thr;"),
    "reroute_always_first_candidate": ("if (o < nc) offer[f] = cand[o];",
                                       "if (o < nc) offer[f] = cand[0];"),
    "reroute_ties_to_higher_index": ("return ea < eb ? -1 : (ea > eb);",
                                     "return ea > eb ? -1 : (ea < eb);"),
    "reroute_candidates_ascending": ("if (sa > sb) return -1;\n  if (sa < sb) return 1;",
                                     "if (sa < sb) return -1;\n  if (sa > sb) return 1;"),
    "reroute_room_off_by_one": ("if (e >= 0 && taken[e] < capacity) {",
                                "if (e >= 0 && taken[e] <= capacity) {"),
    "reroute_forward_ignores_assignment": (
        "const int e = assign ? assign[t * c->k + j] : ix[j];", "const int e = ix[j];"),
    "assign_grouping_perm_src_modulo": (
        "if (assign[f] != e) continue;\n      perm_src[p] = (int32_t)(f / c->k);",
        "if (assign[f] != e) continue;\n      perm_src[p] = (int32_t)(f % c->k);"),
    "smooth_load_cdf_sign": ("return 0.5 * erfc(-z * M_SQRT1_2);",
                             "return 0.5 * erfc(z * M_SQRT1_2);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    sys.path.insert(0, ROOT)
    import oracle
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(lib), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"planted mistake '{name}' passed every pin:\n{r.stdout[-2000:]}"
