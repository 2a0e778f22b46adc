"""The oracle pins must catch plausible mistakes.

Each mutant below plants one small error (a dropped term, a wrong sign, a
wrong index, a swapped operand) in a private copy of oracle.c, builds it on
the CPU and runs the oracle pin tests against it in a subprocess; every
mutant must make them fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "oracle.c")).read()

MUTANTS = {
    "bias_first_entry": ("double u_phi = wh_phi[D];", "double u_phi = wh_phi[0];"),
    "norm_without_bias": ("unit_direction(D + 1, w_phi, wh_phi, &n_phi);\n    unit_direction(D + 1, w_r, wh_r, &n_r);\n    const double amp_phi",
                          "unit_direction(D, w_phi, wh_phi, &n_phi); wh_phi[D] = w_phi[D] / n_phi;\n    unit_direction(D + 1, w_r, wh_r, &n_r);\n    const double amp_phi"),
    "radial_map": ("double qt = rt / (1.0 + rt * rt);\n        double dt", "double qt = rt / (1.0 + rt);\n        double dt"),
    "mode_scaling_uses_D": ("const double amp_phi = tanh(a_phi) / sqrt(M);", "const double amp_phi = tanh(a_phi) / sqrt(D);"),
    "rotation_sign": ("*li = rho * (sth * Ct + cth * St);", "*li = rho * (sth * Ct - cth * St);"),
    "retention_form": ("double rho = exp(-nu * Et);", "double rho = exp(-nu) * Et;"),
    "recurrence_sign": ("double nr = lr * zr - li * zi + br;\n                double ni = lr * zi + li * zr + bi;\n                zr = nr; zi = ni;\n                y[o]",
                        "double nr = lr * zr + li * zi + br;\n                double ni = lr * zi + li * zr + bi;\n                zr = nr; zi = ni;\n                y[o]"),
    "initial_state_dropped": ("zr = z0[((long)bb * M + m) * 2 + 0];", "zr = 0.0;"),
    "gamma_sign": ("double gam_i = hi * pr - hr * pi;", "double gam_i = hr * pi - hi * pr;"),
    "carry_not_conjugated": ("double hr = lr * gr + li * gi;\n                    double hi = lr * gi - li * gr;",
                             "double hr = lr * gr - li * gi;\n                    double hi = lr * gi + li * gr;"),
    "cbar_without_nu": ("cb[bt] += -nu_m * E[bt] * gam_r;", "cb[bt] += -E[bt] * gam_r;"),
    "previous_state_index": ("double pr = zh[2 * t], pi = zh[2 * t + 1];", "double pr = zh[2 * (t + 1)], pi = zh[2 * (t + 1) + 1];"),
    "radial_derivative": ("(1.0 - rt * rt) / ((1.0 + rt * rt) * (1.0 + rt * rt));", "(1.0 - rt * rt) / (1.0 + rt * rt);"),
    "direction_projection_dropped": ("dw_phi[j] = (g_phi[j] - wh_phi[j] * dot_phi) / n_phi;", "dw_phi[j] = g_phi[j] / n_phi;"),
    "amplitude_derivative": ("*da_phi = (1.0 - th_phi * th_phi) / sM * sum_dp;", "*da_phi = th_phi / sM * sum_dp;"),
    "retention_gate_swapped": ("k.a = exp(-8.0 * k.ga * sp);", "k.a = exp(-8.0 * k.gx * sp);"),
    "reset_keeps_multiplier": ("if (rs) { k.a = 0.0; k.m = 1.0; }", "if (rs) { k.a = 0.0; }"),
    "softplus_is_exp": ("return log1p(exp(v));", "return exp(v);"),
    "dla_sigmoid_derivative": ("dla[o] = abar * k.a * (-8.0 * sp) * k.ga * (1.0 - k.ga);", "dla[o] = abar * k.a * (-8.0 * sp) * k.ga;"),
    "dalpha_chain": ("galpha += abar * k.a * (-8.0 * k.ga) * dsp;", "galpha += abar * k.a * (-8.0 * k.ga) * sp;"),
    "sqrt_cap_constant": ("#define RGLRU_SQRT_GRAD_UMIN 2.5e-7", "#define RGLRU_SQRT_GRAD_UMIN 1e-6"),
    "dx_without_multiplier": ("dx[o] = g * k.gx * k.m;", "dx[o] = g * k.gx;"),
    "proj_weight_transposed": ("const double *wr = w + ((long)i * Db + o) * Db;\n                double s = bias[i * Db + o];\n                for (int k = 0; k < Db; ++k) s += wr[k] * xb[k];",
                               "const double *wr = w + (long)i * Db * Db + o;\n                double s = bias[i * Db + o];\n                for (int k = 0; k < Db; ++k) s += wr[(long)k * Db] * xb[k];"),
    "proj_bias_dropped": ("double s = bias[i * Db + o];\n                for (int k = 0; k < Db; ++k) s += wr[k] * xb[k];",
                          "double s = 0.0;\n                for (int k = 0; k < Db; ++k) s += wr[k] * xb[k];"),
    "proj_block_offset": ("const double *xb = x + bt * D + (long)i * Db;", "const double *xb = x + bt * D;"),
    "proj_adjoint_not_transposed": ("s += w[((long)i * Db + o) * Db + k] * dl[bt * D + (long)i * Db + o];",
                                    "s += w[((long)i * Db + k) * Db + o] * dl[bt * D + (long)i * Db + o];"),
    "proj_dw_wrong_input": ("s += dl[bt * D + c] * x[bt * D + (long)i * Db + k];", "s += dl[bt * D + c] * x[bt * D + c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found"
    src = SRC.replace(old, new, 1)
    c = tmp_path / "oracle_mut.c"
    c.write_text(src)
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(c), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_samu.py", "tests/test_oracle_rglru.py",
                        "tests/test_oracle_rglru_proj.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins"
