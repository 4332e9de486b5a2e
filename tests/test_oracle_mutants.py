"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins catch
every one of them; this is what makes the pins a check on the oracle and not a restatement."""
import os

import pytest

import oracle
import pins

# (name, text in ssm_oracle.c, replacement, occurrence to replace (0 = first))
MUTANTS = [
    ("bbar_without_delta", "h[n] = abar * h[n] + dt * load_elem(B, dtype, i_tn + n) * xt;",
     "h[n] = abar * h[n] + load_elem(B, dtype, i_tn + n) * xt;"),
    ("exp_sign_flipped", "double abar = exp(dt * (double)A[d * N + n]);",
     "double abar = exp(-dt * (double)A[d * N + n]);"),
    ("readout_before_update",
     "      h[n] = abar * h[n] + dt * load_elem(B, dtype, i_tn + n) * xt;\n"
     "      acc += load_elem(C, dtype, i_tn + n) * h[n];",
     "      acc += load_elem(C, dtype, i_tn + n) * h[n];\n"
     "      h[n] = abar * h[n] + dt * load_elem(B, dtype, i_tn + n) * xt;"),
    ("readout_uses_B", "acc += load_elem(C, dtype, i_tn + n) * h[n];",
     "acc += load_elem(B, dtype, i_tn + n) * h[n];"),
    ("skip_dropped", "double yt = acc + (Dskip ? (double)Dskip[d] * xt : 0.0);\n    if (z) yt *= silu(load_elem(z, dtype, i_td));",
     "double yt = acc;\n    if (z) yt *= silu(load_elem(z, dtype, i_td));"),
    ("skip_after_gate", "double yt = acc + (Dskip ? (double)Dskip[d] * xt : 0.0);\n    if (z) yt *= silu(load_elem(z, dtype, i_td));",
     "double yt = acc;\n    if (z) yt *= silu(load_elem(z, dtype, i_td));\n    yt += (Dskip ? (double)Dskip[d] * xt : 0.0);"),
    ("bias_after_softplus",
     "    double v = load_elem(delta, dtype, i_td) + (delta_bias ? (double)delta_bias[d] : 0.0);\n"
     "    double dt = delta_softplus ? softplus(v) : v;",
     "    double v = load_elem(delta, dtype, i_td);\n"
     "    double dt = (delta_softplus ? softplus(v) : v) + (delta_bias ? (double)delta_bias[d] : 0.0);"),
    ("softplus_missing_log", "if (v > 0.0) return v + log1p(exp(-v));\n  return log1p(exp(v));",
     "if (v > 0.0) return v + exp(-v);\n  return exp(v);"),
    ("softplus_drops_linear_part", "if (v > 0.0) return v + log1p(exp(-v));", "if (v > 0.0) return log1p(exp(-v));"),
    ("silu_is_sigmoid", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("B_C_ignore_batch", "const int64_t i_tn = (b * L + t) * N;", "const int64_t i_tn = t * N;"),
    ("A_transposed", "double abar = exp(dt * (double)A[d * N + n]);", "double abar = exp(dt * (double)A[n * Dm + d]);"),
    ("decode_bbar_without_delta", "h[n] = abar * h[n] + dt * load_elem(B, dtype, b * dstate + n) * xt;",
     "h[n] = abar * h[n] + load_elem(B, dtype, b * dstate + n) * xt;"),
    ("initial_state_ignored", "h[n] = h0 ? h0[ch * dstate + n] : 0.0;", "h[n] = 0.0;"),
    ("selection_wrong_row", "sel_d[k], h, y_out + k * seqlen, 1);", "sel_d[k], h, y_out + k * seqlen, 0);"),
    ("conv_taps_reversed", "acc += (double)w[d * K + k] * v;", "acc += (double)w[d * K + (K - 1 - k)] * v;"),
    ("conv_window_off_by_one", "const int64_t s = t - (K - 1) + k;", "const int64_t s = t - K + k;"),
    ("conv_bias_dropped", "double acc = bias ? (double)bias[d] : 0.0;\n        for (int64_t k = 0; k < K; ++k) {",
     "double acc = 0.0;\n        for (int64_t k = 0; k < K; ++k) {"),
    ("conv_init_state_ignored", "v = init ? load_elem(init, dtype, (b * dim + d) * (K - 1) + (K - 1) + s) : 0.0;\n"
     "          acc +=", "v = 0.0;\n          acc +="),
    ("conv_final_state_first_inputs", "const int64_t s = seqlen - (K - 1) + j;", "const int64_t s = j;"),
    ("conv_update_newest_first", "acc += (double)w[d * K + k] * st[k];", "acc += (double)w[d * K + k] * st[K - 2 - k];"),
    ("conv_update_no_shift", "for (int64_t k = 0; k + 1 < K - 1; ++k) st[k] = st[k + 1];", ""),
    ("bwd_adjoint_not_decayed", "          g[n] *= abar; /* carried to step t-1 */", ""),
    ("bwd_dA_without_dt", "dA[d * N + n] += g[n] * dt * abar * hp[n];", "dA[d * N + n] += g[n] * abar * hp[n];"),
    ("bwd_ddt_uses_new_state", "ddt += g[n] * (Bn * xt + an * abar * hp[n]);", "ddt += g[n] * (Bn * xt + an * abar * h[n]);"),
    ("bwd_dz_without_silu_slope", "dz[i_td] = dy[i_td] * y0 * (sg + zt * sg * (1.0 - sg));", "dz[i_td] = dy[i_td] * y0 * sg;"),
    ("bwd_dx_without_skip", "double dxt = Dskip ? dy0 * (double)Dskip[d] : 0.0, ddt = 0.0;", "double dxt = 0.0, ddt = 0.0;"),
    ("bwd_no_softplus_slope", "const double dd = delta_softplus ? ddt * sigmoid(v) : ddt;", "const double dd = ddt;"),
    ("bwd_dB_without_dt", "dB[i_tn + n] += g[n] * dt * xt;", "dB[i_tn + n] += g[n] * xt;"),
    ("bwd_dC_uses_old_state", "dC[i_tn + n] += dy0 * h[n];", "dC[i_tn + n] += dy0 * hp[n];"),
    ("zoh_missing_division", "return expm1(dt * a) / a * bv * xt;", "return expm1(dt * a) * bv * xt;"),
    ("zoh_plain_exp", "return expm1(dt * a) / a * bv * xt;", "return exp(dt * a) / a * bv * xt;"),
    ("zoh_keeps_delta", "return expm1(dt * a) / a * bv * xt;", "return dt * expm1(dt * a) / a * bv * xt;"),
    ("bwd_zoh_dB_uses_dt", "dB[i_tn + n] += g[n] * phi * xt;", "dB[i_tn + n] += g[n] * dt * xt;"),
    ("bwd_zoh_dx_uses_dt", "dxt += g[n] * phi * Bn;", "dxt += g[n] * dt * Bn;"),
    ("bwd_zoh_ddt_delta_b_form", "ddt += g[n] * abar * (Bn * xt + an * hp[n]);",
     "ddt += g[n] * (Bn * xt + an * abar * hp[n]);"),
    ("bwd_zoh_dA_without_input_term", "dA[d * N + n] += g[n] * (dt * abar * hp[n] + Bn * xt * zoh_dphi_da(dt, an));",
     "dA[d * N + n] += g[n] * dt * abar * hp[n];"),
    ("bwd_zoh_dphi_sign", "return (zz * em + (zz - em)) / (a * a);", "return (zz * em - (zz - em)) / (a * a);"),
    ("bwd_zoh_forward_delta_b", "bbar_x(zoh, dt, (double)A[d * N + n], load_elem(B, dtype, i_tn + n), xt);",
     "bbar_x(0, dt, (double)A[d * N + n], load_elem(B, dtype, i_tn + n), xt);"),
    ("ssd_group_ignored", "const int64_t b = bh / H, h = bh % H, g = h / hpg;", "const int64_t b = bh / H, h = bh % H, g = 0;"),
    ("ssd_no_dt_on_input", "S[p * N + n] = a * S[p * N + n] + d * xv * load_elem(B, dtype, ibc + n);",
     "S[p * N + n] = a * S[p * N + n] + xv * load_elem(B, dtype, ibc + n);"),
    ("ssd_readout_uses_B", "acc += load_elem(C, dtype, ibc + n) * S[p * N + n];", "acc += load_elem(B, dtype, ibc + n) * S[p * N + n];"),
    ("ssd_initial_state_ignored", "      for (int64_t i = 0; i < P * N; ++i) S[i] = h0[bh * P * N + i];",
     "      for (int64_t i = 0; i < P * N; ++i) S[i] = 0.0 * h0[bh * P * N + i];"),
    ("conv_silu_skipped", "out[(b * seqlen + t) * dim + d] = apply_silu ? silu(acc) : acc;",
     "out[(b * seqlen + t) * dim + d] = acc;"),
]


def _run_pins(o):
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError as e:
            failed.append((pin.__name__, str(e)[:80]))
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    src = open(oracle.SOURCE).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = src.replace(old, new, 1)
    path = os.path.join(tmp_path, "mutant.c")
    open(path, "w").write(mutated)
    lib = oracle.build(out_path=os.path.join(tmp_path, f"lib_{name}.so"), src=path)
    failed = _run_pins(oracle.Oracle(lib))
    assert failed, f"no pin caught the planted mistake {name}"


def test_unmutated_copy_passes(tmp_path):
    lib = oracle.build(out_path=os.path.join(tmp_path, "lib_clean.so"))
    assert _run_pins(oracle.Oracle(lib)) == []
