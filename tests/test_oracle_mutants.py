"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle.c (a dropped term, a wrong
sign, a wrong index, a transposed operand), builds it on the CPU, swaps it in
for the real oracle and checks that at least one pin in test_oracle.py fails.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j - k0] = tau * dot;", "s[j - k0] = dot;"),
    "exp_sign": ("double p = exp(s[j - k0] - m);", "double p = exp(s[j - k0] + m);"),
    "lse_sign": ("return m + log(l);", "return m - log(l);"),
    "no_normalise": ("for (int64_t d = 0; d < D; ++d) o[d] /= l;", ""),
    "merge_weights_swapped": ("double wa = exp(la[r] - L), wb = exp(lb[r] - L);",
                              "double wb = exp(la[r] - L), wa = exp(lb[r] - L);"),
    "merge_plain_sum": ("double L = M + log(exp(la[r] - M) + exp(lb[r] - M));",
                        "double L = M;"),
    "causal_strict": ("if (causal > 0) return j <= i;", "if (causal > 0) return j < i;"),
    "stripe_transposed": ("return (i % blk) * n + i / blk;", "return (i / blk) * n + i % blk;"),
    "ring_wrong_direction": ("int64_t moved = ((w - r) % n + n) % n;",
                             "int64_t moved = ((w + r) % n + n) % n;"),
    "ring_stationary_swapped": ("if (sched == 0) { *qblk = moved; *kblk = w; }",
                                "if (sched == 1) { *qblk = moved; *kblk = w; }"),
    "shard_off_by_one": ("return (k * S) / n;", "return (k * S + n - 1) / n;"),
    "bwd_delta_sign": ("double dS = P * (dp[j] - delta);", "double dS = P * (dp[j] + delta);"),
    "bwd_dk_no_scale": ("gk[d] += tau * dS * ld(q, dt, (qb + i) * D + d);",
                        "gk[d] += dS * ld(q, dt, (qb + i) * D + d);"),
    "bwd_dv_uses_ds": ("gv[d] += P * ld(dout, dt_do, (qb + i) * D + d);",
                       "gv[d] += dS * ld(dout, dt_do, (qb + i) * D + d);"),
    "proj_transposed_weight": ("ld(w_t, dt, nn * E + e)", "ld(w_t, dt, e * HD + nn)"),
    "model_no_stats_term": ("double lv_elems = 2.0 * S_Q * d / n + S_Q / n;",
                            "double lv_elems = 2.0 * S_Q * d / n;"),
    "model_one_contraction": ("double f = 2.0 * (2.0 * q_block * kv_block * d);",
                              "double f = 2.0 * q_block * kv_block * d;"),
    "model_ring_sends_q": ("double ring_elems = 2.0 * S_KV * d / n;",
                           "double ring_elems = 2.0 * S_Q * d / n;"),
    "model_tie_to_ring": ("return out[3] <= out[4] ? 0 : 1;", "return out[3] < out[4] ? 0 : 1;"),
    "grad_head_index_swapped": ("int64_t h = n / D, d = n % D;", "int64_t d = n / D, h = n % D;"),
    "grad_y_drops_v": ("acc += g_at(gk, dt, H, S, D, b, s, n) * ld(wk_t, dt, n * E + e) +\n"
                       "               g_at(gv, dt, H, S, D, b, s, n) * ld(wv_t, dt, n * E + e);",
                       "acc += g_at(gk, dt, H, S, D, b, s, n) * ld(wk_t, dt, n * E + e);"),
    "grad_w_y_row_off_by_batch": ("acc += g_at(g, dt, H, S, D, b, s, n) * ld(y, dt, (b * S + s) * E + e);",
                                  "acc += g_at(g, dt, H, S, D, b, s, n) * ld(y, dt, s * E + e);"),
}


def all_pins(orc):
    """Every pin in test_oracle.py, each as a zero-argument callable."""
    calls = []
    for causal in (False, True):
        for shape in [(2, 2, 3, 7, 4), (1, 2, 4, 9, 3)]:
            calls.append(lambda s=shape, c=causal: pins.test_forward_brute_force(orc, s, c))
        calls.append(lambda c=causal: pins.test_forward_vs_torch_sdpa(orc, 64, c))
        calls.append(lambda c=causal: pins.test_backward_vs_torch_autograd(orc, c))
    for sched in (0, 1):
        calls.append(lambda s=sched: pins.test_rounds_are_perfect_matchings(orc, 5, s))
        calls.append(lambda s=sched: pins.test_ring_forward_equals_unblocked(orc, 3, s))
        calls.append(lambda s=sched: pins.test_ring_forward_causal_equals_unblocked(orc, 4, s))
    calls += [
        lambda: pins.test_zero_query_gives_mean_of_values(orc),
        lambda: pins.test_causal_first_row(orc),
        lambda: pins.test_merge_identity_and_empty(orc),
        lambda: pins.test_merge_commutative_associative(orc),
        lambda: pins.test_random_noncontiguous_partitions(orc),
        pins.test_schedule_directions,
        lambda: pins.test_shard_bounds(orc),
        lambda: pins.test_backward_finite_differences(orc),
        lambda: pins.test_backward_identities(orc),
        lambda: pins.test_projection_vs_numpy(orc),
        lambda: pins.test_schedule_model_comm_volume_video_mme(orc),
        lambda: pins.test_schedule_model_speedup_closed_form(orc),
        lambda: pins.test_schedule_model_choices(orc),
        lambda: pins.test_recompute_grads_vs_numpy(orc),
        lambda: pins.test_striped_causal_is_causal_on_positions(orc),
        lambda: pins.test_recompute_grads_are_adjoints(orc),
    ]
    return calls


def test_real_oracle_passes_every_pin(orc):
    for call in all_pins(orc):
        call()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(orc, name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not unique"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(text.replace(old, new))
    lib_path = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                           "-o", str(lib_path), str(src), "-lm"])
    real = oracle._load()
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB", str(lib_path))
    mutant = oracle._load()
    assert mutant is not real
    failures = 0
    for call in all_pins(oracle):
        try:
            call()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutant {name}"
