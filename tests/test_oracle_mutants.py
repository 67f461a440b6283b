"""Mutation check of the oracle's pins: each plausible mistake, planted in a private copy
of the oracle source and built on the CPU, must make at least one pin fail."""
import os
import shutil
import subprocess
import tempfile

import pytest

from oracle import oracle as O
from tests.oracle_pins import PINS

# (name, original text, planted mistake); the original must occur exactly once.
MUTANTS = [
    ("quant_round_half_away", "float v = rintf(p * s);", "float v = roundf(p * s);"),
    ("ternary_round_half_away", "float v = rintf(w[i] / s);", "float v = roundf(w[i] / s);"),
    ("quant_floor_dropped", "float me = mx > 1e-5f ? mx : 1e-5f;", "float me = mx;"),
    ("rms_sum_not_mean", "double r = 1.0 / sqrt(ss / (double)k + eps);",
     "double r = 1.0 / sqrt(ss + eps);"),
    ("acc_wrong_sign", "else if (wr[c] < 0) s -= xr[c];", "else if (wr[c] < 0) s += xr[c];"),
    ("acc_transposed", "const int8_t *xr = qx + row * k, *wr = qw + col * k;",
     "const int8_t *xr = qx + row * k, *wr = qw + (col % m) * k;"),
    ("rescale_drops_weight_scale",
     "y[row * n + col] = (double)acc[row * n + col] * (double)w->scale * a[row] +",
     "y[row * n + col] = (double)acc[row * n + col] * a[row] +"),
    ("recurrence_drops_1_minus_f", "h = f[i] * h + (1.0 - f[i]) * c[i];",
     "h = f[i] * h + c[i];"),
    ("recurrence_ignores_h0", "double h = h0 ? h0[b * D + d] : 0.0;", "double h = 0.0;"),
    ("mlgru_i_f_swapped",
     "double sg = sigmoid_d(r[D + d] + (f_bias ? (double)f_bias[d] : 0.0));",
     "double sg = sigmoid_d(r[d] + (f_bias ? (double)f_bias[d] : 0.0));"),
    ("mlgru_bias_sign",
     "sigmoid_d(r[D + d] + (f_bias ? (double)f_bias[d] : 0.0))",
     "sigmoid_d(r[D + d] - (f_bias ? (double)f_bias[d] : 0.0))"),
    ("gnorm_sum_not_mean", "double r = 1.0 / sqrt(ss / (double)D + eps);",
     "double r = 1.0 / sqrt(ss + eps);"),
    ("gnorm_sigmoid_not_swish",
     "hr[d] * r * (gnorm_w ? (double)gnorm_w[d] : 1.0) * silu_d(g[d]);",
     "hr[d] * r * (gnorm_w ? (double)gnorm_w[d] : 1.0) * sigmoid_d(g[d]);"),
    ("gnorm_gain_dropped",
     "hr[d] * r * (gnorm_w ? (double)gnorm_w[d] : 1.0) * silu_d(g[d]);",
     "hr[d] * r * silu_d(g[d]);"),
    ("glu_silu_on_up", "yg[i] = silu_d(yg[i]) * yu[i];", "yg[i] = yg[i] * silu_d(yu[i]);"),
    ("block_no_attn_residual", "tmp[i] = (double)x[i] + yo[i];", "tmp[i] = yo[i];"),
    ("block_no_mlp_residual", "tmp[i] = (double)y1[i] + glu[i];", "tmp[i] = glu[i];"),
    ("pack_bit_position", "word |= (uint32_t)(v + 1) << (8 * b + 2 * a);",
     "word |= (uint32_t)(v + 1) << (2 * b + 8 * a);"),
    ("quant_gain_dropped", "float p = gamma ? xr[c] * gamma[c] : xr[c];\n            float ap",
     "float p = xr[c];\n            float ap"),
    ("ifg_not_rounded_to_bf16",
     "for (int64_t i = 0; i < M * 3 * D; ++i) ifg[i] = orc_round_bf16(ifg[i]);",
     "for (int64_t i = 0; i < M * 3 * D; ++i) ifg[i] = ifg[i];"),
    ("glu_hidden_not_rounded", "to_act(yg, mm, M * F, act_bf16);", "to_act(yg, mm, M * F, 0);"),
    ("gated_output_not_rounded", "to_act(o, o32, M * D, resid_bf16);", "to_act(o, o32, M * D, 0);"),
    ("ternarize_floor_dropped", "float s = mean_abs > 1e-5f ? mean_abs : 1e-5f;",
     "float s = mean_abs;"),
    ("quant_divides_by_max", "float v = rintf(p * s);", "float v = rintf((p * 127.0f) / me);"),
    ("quant_exact_quotient", "float v = rintf(p * s);",
     "float v = (float)rint((double)p * 127.0 / (double)me);"),
    ("hgrn_bound_ignored", "f[row * D + d] = lb + (1.0 - lb) * sg;", "f[row * D + d] = sg;"),
    ("hgrn_bound_as_scale", "f[row * D + d] = lb + (1.0 - lb) * sg;",
     "f[row * D + d] = lb * sg;"),
    ("hgrn_bound_inclusive_cumsum",
     "            lb[l * D + d] = (float)(acc / tot);\n            acc += exp((double)G[l * D + d] - mx);",
     "            acc += exp((double)G[l * D + d] - mx);\n            lb[l * D + d] = (float)(acc / tot);"),
    ("hgrn_bound_unnormalised", "lb[l * D + d] = (float)(acc / tot);", "lb[l * D + d] = (float)acc;"),
    ("trit_contiguous_layout", "return 20 * w + 4 * i + j;", "return 20 * w + 5 * j + i;"),
    ("trit_floor_not_ceil", "packed[r * rb + by] = (uint8_t)((256 * v + 242) / 243);",
     "packed[r * rb + by] = (uint8_t)((256 * v) / 243);"),
    ("trit_pad_code_zero", "int c = 1;                               /* padding: q = 0 */",
     "int c = 0;"),
    ("trit_digits_reversed", "for (int i = 4; i >= 0; --i) { c[i] = v % 3; v /= 3; }",
     "for (int i = 0; i < 5; ++i) { c[i] = v % 3; v /= 3; }"),
    ("bwd_dx_drops_norm_term", "(double)xr[c] * r3 / (double)k * dot;", "0.0 * dot;"),
    ("bwd_dx_r_not_cubed", "const double r1 = r[row], r3 = r1 * r1 * r1;",
     "const double r1 = r[row], r3 = r1;"),
    ("bwd_g_transposed", "acc += dy[row * n + j] * (double)w->q[j * k + c];",
     "acc += dy[row * n + j] * (double)w->q[(c % n) * k + (j % k)];"),
    ("bwd_dw_without_scale_a", "acc += dy[row * n + j] * (double)q[row * k + c] * a[row];",
     "acc += dy[row * n + j] * (double)q[row * k + c];"),
    ("bwd_dgamma_without_r", "acc += g[row * k + c] * (double)x[row * k + c] * r[row];",
     "acc += g[row * k + c] * (double)x[row * k + c];"),
    ("bwd_recurrence_same_step_f", ": f[(b * T + t + 1) * D + d] * G);", ": f[(b * T + t) * D + d] * G);"),
    ("bwd_df_sign", "(hp - c[i]) * G * (1.0 - lb) * sz * (1.0 - sz);",
     "(c[i] - hp) * G * (1.0 - lb) * sz * (1.0 - sz);"),
    ("bwd_df_ignores_bound", "(hp - c[i]) * G * (1.0 - lb) * sz * (1.0 - sz);",
     "(hp - c[i]) * G * sz * (1.0 - sz);"),
    ("bwd_silu_prime_is_sigmoid", "(1.0 - f[i]) * G * si * (1.0 + r[d] * (1.0 - si));",
     "(1.0 - f[i]) * G * si;"),
    ("bwd_gnorm_drops_mean_term",
     "dho[row * D + d] = rho * dho[row * D + d] - hr[d] * rho * rho * rho / (double)D * dot;",
     "dho[row * D + d] = rho * dho[row * D + d];"),
    ("bwd_dh0_without_f", "if (dh0) dh0[b * D + d] = T > 0 ? f[(b * T) * D + d] * G :",
     "if (dh0) dh0[b * D + d] = T > 0 ? G :"),
    ("bwd_dh_last_dropped", "G = dho[i] + (t == T - 1 ? (dh_last ? dh_last[b * D + d] : 0.0)",
     "G = dho[i] + (t == T - 1 ? 0.0"),
    ("bwd_block_no_residual_dx", "memcpy(dx, dy1, sizeof(double) * (size_t)(M * D));",
     "memset(dx, 0, sizeof(double) * (size_t)(M * D));"),
    ("bwd_block_glu_gate_sigmoid", "dg[i] = dm[i] * up[i] * sg * (1.0 + gp[i] * (1.0 - sg));",
     "dg[i] = dm[i] * up[i] * sg;"),
    ("bwd_block_up_without_gate", "du[i] = dm[i] * gp[i] * sg;", "du[i] = dm[i] * sg;"),
    ("bwd_block_o_grad_skips_glu", "if ((rc = orc_bitlinear_backward(o32, M, w7[3], eps, dy1, dout,",
     "if ((rc = orc_bitlinear_backward(o32, M, w7[3], eps, dy, dout,"),
    ("embedding_no_scale", "double v = (double)qe[(int64_t)ids[t] * D + d] * (double)scale;",
     "double v = (double)qe[(int64_t)ids[t] * D + d];"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, bad):
    src = open(O.SRC).read()
    assert src.count(orig) == 1, f"mutation site for {name} not unique"
    tmp = tempfile.mkdtemp(prefix="orc_mutant_")
    try:
        path = os.path.join(tmp, "mutant.c")
        with open(path, "w") as fh:
            fh.write(src.replace(orig, bad))
        lib = os.path.join(tmp, "libmutant.so")
        subprocess.run(["gcc", *O.CFLAGS, path, "-o", lib, "-lm"], check=True)
        mutant = O.Oracle(lib)
        failed = []
        for pin in PINS:
            try:
                pin(mutant)
            except (AssertionError, ValueError):
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"
    finally:
        shutil.rmtree(tmp)
