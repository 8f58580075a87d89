"""The oracle's pins catch planted mistakes.

Each case copies oracle/gdn_oracle.c, plants one plausible mistake (a dropped
term, a wrong sign, a wrong index, a transposed operand, a swapped input), builds
the copy on the CPU and runs the pin tests against it.  At least one pin must
fail for every mutant; the real oracle passes all of them (the other test
files).  Nothing here touches a GPU.
"""
import os
import shutil
import subprocess

import pytest

import oracle
from tests import test_oracle_conv as tc
from tests import test_oracle_gdn as tg
from tests import test_oracle_primitives as tp
from tests import test_oracle_tree as tt

# (name, text in gdn_oracle.c, replacement, occurrence to replace (1-based, 0 = all))
MUTANTS = [
    ("exp_drops_ln2_lo", "r = fmaf(-n, ORC_LN2_LO, r);", "r = r;", 1),
    ("exp_wrong_coeff", "case 5: return 1.0f / 120.0f;", "case 5: return 1.0f / 100.0f;", 1),
    ("exp_wrong_threshold", "if (x <= -104.0f) return 0.0f;", "if (x <= -80.0f) return 0.0f;", 1),
    ("bf16_round_half_up", "u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;", 1),
    ("silu_sign", "float e = oracle_exp32(-p);", "float e = oracle_exp32(p);", 1),
    ("conv_taps_reversed", "acc = fmaf(w[(size_t)c * W + j], col[t + j], acc);",
     "acc = fmaf(w[(size_t)c * W + (W - 1 - j)], col[t + j], acc);", 1),
    ("conv64_taps_reversed", "acc += w[(size_t)c * W + j] * col[t + j];",
     "acc += w[(size_t)c * W + (W - 1 - j)] * col[t + j];", 1),
    ("conv_hist_off_by_one", "hist_out[((size_t)b * (W - 1) + j) * C + c] = col[T + j];",
     "hist_out[((size_t)b * (W - 1) + j) * C + c] = col[T + j - 1];", 1),
    ("gate_beta_sign", "*beta = 1.0 / (1.0 + exp(-braw));", "*beta = 1.0 / (1.0 + exp(braw));", 1),
    ("gate_softplus_drops_max", "fmax(a, 0.0) + log1p(exp(-fabs(a)))", "log1p(exp(-fabs(a)))", 1),
    ("gate_A_sign", "*g = -orc_softplus(alpha + dt_bias[h]) * exp(A_log[h]);",
     "*g = orc_softplus(alpha + dt_bias[h]) * exp(A_log[h]) * 0.01;", 1),
    ("gate_ignores_dt_bias", "orc_softplus(alpha + dt_bias[h])", "orc_softplus(alpha)", 1),
    ("no_l2_norm", "double r = 1.0 / sqrt(s + eps);", "double r = 1.0;", 1),
    ("rec_drops_decay", "for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= gam;",
     "for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= 1.0;", 1),
    ("rec_delta_sign", "double u = beta * (v[i] - sk);", "double u = beta * (v[i] + sk);", 1),
    ("rec_drops_beta", "double u = beta * (v[i] - sk);", "double u = (v[i] - sk);", 1),
    ("rec_transposed_state", "for (int j = 0; j < dk; ++j) sk += Si[j] * kn[j];",
     "for (int j = 0; j < dk; ++j) sk += S[(size_t)j * dk + i] * kn[j];", 1),
    ("rec_output_uses_k", "for (int j = 0; j < dk; ++j) sq += Si[j] * qn[j];",
     "for (int j = 0; j < dk; ++j) sq += Si[j] * kn[j];", 1),
    ("rec_head_map_modulo", "const int hk = h / grp;", "const int hk = h % Hk;", 1),
    ("rec_q_from_k_slab", "orc_l2norm(row + (size_t)hk * dk, qn, dk, eps);",
     "orc_l2norm(row + (size_t)Hk * dk + (size_t)hk * dk, qn, dk, eps);", 1),
    ("rec_capture_shifted", "if (H && t < K - 1)\n                    memcpy(H + (((size_t)b * (K - 1) + t) * Hv",
     "if (H && t < K - 1)\n                    memcpy(H + (((size_t)b * (K - 1) + (t > 0 ? t - 1 : 0)) * Hv", 1),
    ("wy_T_sign", "for (int s = 0; s < t; ++s) acc -= A[(size_t)t * L + s] * Tm[(size_t)s * L + col];",
     "for (int s = 0; s < t; ++s) acc += A[(size_t)t * L + s] * Tm[(size_t)s * L + col];", 1),
    ("wy_W_drops_decay", "acc += Tm[(size_t)t * L + s] * bet[s] * exp(G[s]) * Kn",
     "acc += Tm[(size_t)t * L + s] * bet[s] * Kn", 1),
    ("wy_A_drops_beta", "A[(size_t)t * L + s] = s < t ? bet[t] * exp(G[t] - G[s]) * kk",
     "A[(size_t)t * L + s] = s < t ? exp(G[t] - G[s]) * kk", 1),
    ("wy_M_drops_diag", "M[(size_t)t * L + s] = s <= t ?", "M[(size_t)t * L + s] = s < t ?", 1),
    ("wy_output_drops_decay", "double acc = exp(G[t]) * r;", "double acc = r;", 1),
    ("wy_G_not_cumulative", "G[t] = gg[t] + (t > 0 ? G[t - 1] : 0.0);", "G[t] = gg[t];", 1),
    ("wy_final_state_drops_decay", "acc += exp(G[L - 1] - G[s]) * U", "acc += U", 1),
    ("rollback_off_by_one", "+ (a - 1)) * state_bytes", "+ (a > 1 ? a - 2 : 0)) * state_bytes", 1),
    ("rollback_conv_window_row", "+ a) * row_bytes,", "+ (a > 0 ? a - 1 : 0)) * row_bytes,", 1),
    ("tree_follows_index_not_parent", "const int p = orc_parent(parent, b, N, t);", "const int p = t - 1;", 1),
    ("tree_parent_may_be_itself", "return (p >= 0 && p < i) ? p : -1;", "return (p >= 0 && p <= i) ? p : -1;", 1),
    ("tree_window_history_reversed", "for (int h = W - 2; m < W; --h, ++m) col[W - 1 - m]",
     "for (int h = 0; m < W; ++h, ++m) col[W - 1 - m]", 1),
    ("tree_rollback_rows_reversed", "memcpy(rows + (size_t)(W - 2 - m) * rb, (const unsigned char *)x",
     "memcpy(rows + (size_t)m * rb, (const unsigned char *)x", 1),
    ("tree_rollback_keeps_parent_state", "memcpy(dst, (const unsigned char *)H + ((size_t)b * N + n) * state_bytes",
     "memcpy(dst, (const unsigned char *)H + ((size_t)b * N + (n > 0 ? n - 1 : 0)) * state_bytes", 1),
]


def _pin_suite(o):
    """Every pin, with fixed parameters; yields (name, callable)."""
    yield "exp_constants", lambda: tp.test_exp32_constants_are_the_stated_roundings(o)
    yield "exp_ulp", lambda: tp.test_exp32_within_one_ulp_of_libm(o)
    yield "exp_subnormal", lambda: tp.test_exp32_subnormal_range(o)
    yield "exp_special", lambda: tp.test_exp32_special_values(o)
    yield "bf16", lambda: tp.test_bf16_rne_matches_torch(o)
    yield "silu", lambda: tp.test_silu32_against_double_definition(o)
    yield "silu_special", lambda: tp.test_silu32_special_values(o)
    yield "conv_corr", lambda: tc.test_conv_f64_is_correlation_then_silu(o, 4, 4)
    yield "conv_onehot", lambda: tc.test_conv_one_hot_taps(o, 4)
    yield "conv_f32_bf16", lambda: tc.test_conv_f32_close_to_f64(o, True)
    yield "conv_f32_f32", lambda: tc.test_conv_f32_close_to_f64(o, False)
    yield "conv_copies", lambda: tc.test_conv_history_and_window_are_copies(o, 3)
    yield "conv_rollback", lambda: tc.test_conv_rollback_equals_rerun(o, 3)
    yield "gates_lib", lambda: tg.test_gates_against_library_routines(o)
    yield "gates_closed", lambda: tg.test_gate_closed_values(o)
    yield "brute_force", lambda: tg.test_brute_force_matrix_product_d4(o, 2, 4, 3)
    yield "delta_identity", lambda: tg.test_delta_identities_every_step(o)
    yield "zero_gates_act", lambda: tg.test_zero_beta_zero_decay_leaves_state(o, "activated")
    yield "zero_gates_raw", lambda: tg.test_zero_beta_zero_decay_leaves_state(o, "raw")
    yield "one_token", lambda: tg.test_one_token_from_zero_state(o)
    yield "k1_decode", lambda: tg.test_k1_equals_decode_and_first_intermediate(o)
    yield "rollback", lambda: tg.test_rollback_equals_rerun(o, 4)
    yield "wy_ragged", lambda: tg.test_chunked_wy_equals_sequential(o, 16, 5, True)
    yield "wy_prefill", lambda: tg.test_chunked_wy_equals_sequential(o, 130, 64, False)
    yield "wy_strong", lambda: tg.test_chunked_wy_strong_decay_no_ratio_overflow(o)
    yield "head_map", lambda: tg.test_head_map_value_head_reads_key_head_h_div_group(o)
    yield "slab_order", lambda: tg.test_slab_order_q_then_k_then_v(o)
    yield "tree_chain", lambda: tt.test_chain_tree_equals_chain_verify(o, 5)
    yield "tree_paths", lambda: tt.test_every_node_equals_chain_over_its_root_path(o, "forest", 12, 4)
    yield "tree_roots", lambda: tt.test_out_of_range_parents_are_roots(o)
    yield "tree_conv_chain", lambda: tt.test_chain_tree_conv_equals_conv_step_bitwise(o, 3, 4)
    yield "tree_conv_paths", lambda: tt.test_tree_conv_node_equals_conv_step_over_its_path(o, "forest")
    yield "tree_rollback", lambda: tt.test_tree_rollback_equals_path_rerun(o, 4)
    yield "tree_rollback_bytes", lambda: tt.test_tree_rollback_bf16_bytes(o)


def _plant(src: str, old: str, new: str, occ: int) -> str:
    n = src.count(old)
    assert n >= 1, "mutation target not found: %r" % old
    if occ == 0:
        return src.replace(old, new)
    idx = -1
    for _ in range(occ):
        idx = src.index(old, idx + 1)
    return src[:idx] + new + src[idx + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, occ):
    src = open(oracle.SRC).read()
    mutated = _plant(src, old, new, occ)
    assert mutated != src
    csrc = tmp_path / "gdn_oracle_mutant.c"
    csrc.write_text(mutated)
    so = str(tmp_path / "libmutant.so")
    oracle.build(force=True, src=str(csrc), out=so)
    o = oracle.Oracle(so)
    caught = []
    for pin, fn in _pin_suite(o):
        try:
            fn()
        except Exception:  # an assertion (or a shape error) means the pin noticed
            caught.append(pin)
    assert caught, "no pin caught mutant %s" % name


def test_unmutated_copy_passes_every_pin(tmp_path):
    csrc = tmp_path / "gdn_oracle_copy.c"
    shutil.copy(oracle.SRC, csrc)
    so = str(tmp_path / "libcopy.so")
    oracle.build(force=True, src=str(csrc), out=so)
    o = oracle.Oracle(so)
    for pin, fn in _pin_suite(o):
        fn()
