"""Plant one mistake at a time in a copy of the oracle; some pin must fail.

This is how the pins are shown to be sharp enough: a dropped term, a wrong
sign, a wrong index or a transposed operand in the oracle each trips at
least one of them. Mutants are built from the oracle's C source in a
temporary directory with gcc; the real oracle is never modified.
"""
import os
import tempfile

import pytest

import oracle
import pins

SRC = open(oracle.SRC).read()

# (name, text to replace, replacement); each is applied to every occurrence.
MUTANTS = [
    ("update_sign", "h[n] = dA * h[n] + dBx;", "h[n] = dA * h[n] - dBx;"),
    ("step_update_sign", "*hn = dA * *hn + dBx;", "*hn = dA * *hn - dBx;"),
    ("exp_sign", "double dA = exp(dt * A[d * N + n]);", "double dA = exp(-dt * A[d * N + n]);"),
    ("drop_delta_in_B", "double dBx = dt * Bt[IDX3(b, t, n, L, N)] * u;",
     "double dBx = Bt[IDX3(b, t, n, L, N)] * u;"),
    ("zoh_like_B", "double dBx = dt * Bt[IDX3(b, t, n, L, N)] * u;",
     "double dBx = (dA - 1.0) / A[d * N + n] * Bt[IDX3(b, t, n, L, N)] * u;"),
    ("readout_before_update",
     "                h[n] = dA * h[n] + dBx;\n                acc += Ct[IDX3(b, t, n, L, N)] * h[n];",
     "                acc += Ct[IDX3(b, t, n, L, N)] * h[n];\n                h[n] = dA * h[n] + dBx;"),
    ("readout_uses_B", "acc += Ct[IDX3(b, t, n, L, N)] * h[n];", "acc += Bt[IDX3(b, t, n, L, N)] * h[n];"),
    ("drop_skip", "if (Dskip) acc += Dskip[d] * u;", "if (0) acc += Dskip[d] * u;"),
    ("skip_outside_gate",
     "            if (Dskip) acc += Dskip[d] * u;\n            if (z) {\n                double g = z[IDX3(b, t, d, L, D)];\n                acc *= g / (1.0 + exp(-g));\n            }",
     "            if (z) {\n                double g = z[IDX3(b, t, d, L, D)];\n                acc *= g / (1.0 + exp(-g));\n            }\n            if (Dskip) acc += Dskip[d] * u;"),
    ("gate_sigmoid_only", "acc *= g / (1.0 + exp(-g));", "acc *= 1.0 / (1.0 + exp(-g));"),
    ("gate_sign", "acc *= g / (1.0 + exp(-g));", "acc *= g / (1.0 + exp(g));"),
    ("ignore_state_in", "h[n] = state_in ? state_in[IDX3(b, d, n, D, N)] : 0.0;", "h[n] = 0.0;"),
    ("A_transposed", "exp(dt * A[d * N + n])", "exp(dt * A[(n * D + d) % (D * N)])"),
    ("B_indexed_by_channel", "Bt[IDX3(b, t, n, L, N)] * u", "Bt[IDX3(b, t, d % N, L, N)] * u"),
    ("delta_previous_token", "double dt = delta[IDX3(b, t, d, L, D)];",
     "double dt = delta[IDX3(b, (t > 0 ? t - 1 : 0), d, L, D)];"),
    ("x_neighbour_channel", "double u = x[IDX3(b, t, d, L, D)];", "double u = x[IDX3(b, t, (d + 1) % D, L, D)];"),
    ("C_previous_token", "acc += Ct[IDX3(b, t, n, L, N)] * h[n];",
     "acc += Ct[IDX3(b, (t > 0 ? t - 1 : 0), n, L, N)] * h[n];"),
    ("last_state_component_dropped", "for (int64_t n = 0; n < N; ++n) state_out[IDX3(b, d, n, D, N)] = h[n];",
     "for (int64_t n = 0; n + 1 < N; ++n) state_out[IDX3(b, d, n, D, N)] = h[n];"),
    ("batch_row_mixup", "int64_t b = r / D, d = r % D;\n        double h[4096];",
     "int64_t b = 0, d = r % D;\n        double h[4096];"),
    ("softplus_drops_bias", "double u = raw[r * D + d] + (bias ? bias[d] : 0.0);", "double u = raw[r * D + d];"),
    ("softplus_bias_by_row", "(bias ? bias[d] : 0.0)", "(bias ? bias[r % D] : 0.0)"),
    ("softplus_log_not_log1p", "log1p(exp(-fabs(u)))", "log(1.0 + exp(-fabs(u)))"),
    ("softplus_relu_only", "(u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u)))", "(u > 0.0 ? u : 0.0)"),
    ("softplus_tail_sign", "log1p(exp(-fabs(u)))", "log1p(exp(fabs(u)))"),
    ("trap_beta_without_alpha", "double beta = (1.0 - lm) * dt * alpha;", "double beta = (1.0 - lm) * dt;"),
    ("trap_beta_weight_lam", "double beta = (1.0 - lm) * dt * alpha;", "double beta = lm * dt * alpha;"),
    ("trap_gamma_weight_one_minus_lam", "double gamma = lm * dt;", "double gamma = (1.0 - lm) * dt;"),
    ("trap_prev_input_never_advances", "                vprev[n] = v;\n", ""),
    ("trap_prev_input_advanced_early",
     "                h[n] = alpha * h[n] + beta * vprev[n] + gamma * v;\n                vprev[n] = v;\n",
     "                vprev[n] = v;\n                h[n] = alpha * h[n] + beta * vprev[n] + gamma * v;\n"),
    ("trap_earlier_input_ignored", "vprev[n] = (x_prev && B_prev) ? B_prev[b * N + n] * x_prev[b * D + d] : 0.0;",
     "vprev[n] = 0.0;"),
    ("trap_earlier_B_batch_row_0", "B_prev[b * N + n] * x_prev[b * D + d]", "B_prev[n] * x_prev[b * D + d]"),
    ("trap_lam_previous_token", "double lm = lam[IDX3(b, t, d, L, D)];",
     "double lm = lam[IDX3(b, t > 0 ? t - 1 : 0, d, L, D)];"),
    ("bwd_state_grad_not_decayed", "                    G[n] *= a;\n", ""),
    ("bwd_delta_misses_input_term", "gd += G[n] * (A[d * N + n] * a * hp + Bt[bn] * u);", "gd += G[n] * (A[d * N + n] * a * hp);"),
    ("bwd_dA_without_delta", "dA[d * N + n] += G[n] * dt * a * hp;", "dA[d * N + n] += G[n] * a * hp;"),
    ("bwd_dC_uses_previous_state", "dCt[bn] += ds * H[(t + 1) * N + n];", "dCt[bn] += ds * H[t * N + n];"),
    ("bwd_gate_derivative_sigmoid_only", "dgate = sg * (1.0 + zz * (1.0 - sg));", "dgate = sg;"),
    ("bwd_skip_grad_missing", "double gx = Dskip ? ds * Dskip[d] : 0.0;", "double gx = 0.0;"),
    ("bwd_readout_grad_after_decay", "                    G[n] += Ct[bn] * ds;\n", ""),
    ("bwdtrap_input_grad_misses_next_update", "double dv = lm * dt * G[n] + Gb[n];", "double dv = lm * dt * G[n];"),
    ("bwdtrap_next_weight_not_decayed", "Gb[n] = (1.0 - lm) * dt * alpha * G[n];", "Gb[n] = (1.0 - lm) * dt * G[n];"),
    ("bwdtrap_dlam_sign", "gl += G[n] * dt * (v - alpha * vp);", "gl += G[n] * dt * (v + alpha * vp);"),
    ("bwdtrap_ddelta_misses_prev_term", "+ (1.0 - lm) * alpha * vp + lm * v);", "+ lm * v);"),
    ("bwdtrap_decay_arg_without_prev", "double p = H[t * N + n] + (1.0 - lm) * dt * vp;", "double p = H[t * N + n];"),
    ("bwdtrap_dx_prev_from_x", "gp += Gb[n] * B_prev[b * N + n];", "gp += Gb[n] * x_prev[b * D + d];"),
    ("softplus_grad_sigmoid_sign", "g[r * D + d] / (1.0 + exp(-u))", "g[r * D + d] / (1.0 + exp(u))"),
    ("softplus_grad_bias_sum_missing", "            if (gbias) gbias[d] += v;\n", ""),
    ("ssd_group_modulo", "g = h / (H / G);", "g = h % G;"),
    ("ssd_input_without_delta", "+ dt * xt[p] * Bg[n];", "+ xt[p] * Bg[n];"),
    ("ssd_decay_of_group", "double a = exp(dt * A[h]);", "double a = exp(dt * A[g]);"),
    ("ssd_readout_uses_B", "acc += Cg[n] * S[p * N + n];", "acc += Bg[n] * S[p * N + n];"),
    ("ssd_state_transposed", "state_out[r * P * N + i] = S[i];", "state_out[r * P * N + i] = S[(i % P) * N + i / P];"),
    ("ssd_skip_of_head_zero", "if (Dskip) acc += Dskip[h] * xt[p];", "if (Dskip) acc += Dskip[0] * xt[p];"),
    ("trap_step_prev_uses_current_B", "B_prev[b * N + n] * x_prev[r]", "Bt[b * N + n] * x_prev[r]"),
    ("trap_step_beta_without_alpha", "            double beta = (1.0 - lm) * dt * alpha;\n            double gamma = lm * dt;\n            double vp",
     "            double beta = (1.0 - lm) * dt;\n            double gamma = lm * dt;\n            double vp"),
    ("conv_taps_reversed", "u += w[d * 4 + j] * v;", "u += w[d * 4 + 3 - j] * v;"),
    ("conv_three_taps", "for (int64_t j = 0; j < 4; ++j) {\n                    int64_t s", "for (int64_t j = 0; j < 3; ++j) {\n                    int64_t s"),
    ("conv_state_newest_first", "state[IDX3(b, d, s + 3, D, 3)]", "state[IDX3(b, d, -s - 1, D, 3)]"),
    ("conv_state_ignored", "else v = state ? state[IDX3(b, d, s + 3, D, 3)] : 0.0;", "else v = 0.0;"),
    ("conv_drops_bias", "double u = cb ? cb[d] : 0.0;", "double u = 0.0;"),
    ("conv_silu_sign", "out[IDX3(b, t, d, L, D)] = u / (1.0 + exp(-u));", "out[IDX3(b, t, d, L, D)] = u / (1.0 + exp(u));"),
    ("conv_without_silu", "out[IDX3(b, t, d, L, D)] = u / (1.0 + exp(-u));", "out[IDX3(b, t, d, L, D)] = u;"),
    ("convbwd_silu_grad_sigmoid_only", "du[t] = gout[IDX3(b, t, d, L, D)] * sg * (1.0 + u * (1.0 - sg));",
     "du[t] = gout[IDX3(b, t, d, L, D)] * sg;"),
    ("convbwd_taps_not_flipped", "if (t < L) g += w[d * 4 + j] * du[t];", "if (t < L) g += w[d * 4 + 3 - j] * du[t];"),
    ("convbwd_bias_grad_missing", "                if (gb) gb[d] += du[t];\n", ""),
    ("convbwd_state_grad_drops_a_tap", "for (int64_t j = 0; j <= k; ++j)", "for (int64_t j = 0; j < k; ++j)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    assert old in SRC, "mutation site not found: " + name
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"), force=True)
    o = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, FloatingPointError, ValueError) as e:  # a pin tripped
            failed.append(pin.__name__)
            break
    assert failed, "no pin caught mutant " + name
