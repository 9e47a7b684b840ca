"""Mutation check of the oracle's pins: each test copies the oracle source,
plants one plausible mistake (a dropped term, a wrong sign, index or operand),
builds the copy on the CPU and requires that at least one pin rejects it.
The real oracle is never modified."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssm_oracle.cpp")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("input_sign", "h[n] = abar * h[n] + bbar * u;", "h[n] = abar * h[n] - bbar * u;"),
    ("decay_sign", "const double abar = std::exp(dt * a_cont);\n      const double bbar",
     "const double abar = std::exp(-dt * a_cont);\n      const double bbar"),
    ("no_decay", "h[n] = abar * h[n] + bbar * u;", "h[n] = h[n] + bbar * u;"),
    ("drop_skip", "acc + dskip * u;", "acc;"),
    ("skip_on_x", "acc + dskip * u;", "acc + dskip * p.x[(b * L + t) * D + d];"),
    ("zoh_no_div", "std::expm1(dt * a_cont) / a_cont;", "std::expm1(dt * a_cont);"),
    ("zoh_sign", "std::expm1(dt * a_cont) / a_cont;", "std::expm1(-dt * a_cont) / a_cont;"),
    ("readout_B", "acc += Ct[n] * h[n];", "acc += Bt[n] * h[n];"),
    ("readout_before_update",
     "h[n] = abar * h[n] + bbar * u;\n      acc += Ct[n] * h[n];",
     "acc += Ct[n] * h[n];\n      h[n] = abar * h[n] + bbar * u;"),
    ("delta_lag", "double v = p.delta[(b * p.seqlen + t) * p.dim + d];",
     "double v = p.delta[(b * p.seqlen + (t > 0 ? t - 1 : 0)) * p.dim + d];"),
    ("A_transposed", "const double a_cont = p.A[d * N + n];\n      const double abar",
     "const double a_cont = p.A[(n * D + d) % (D * N)];\n      const double abar"),
    ("conv_flipped", "const int64_t src = t - (K - 1) + k;", "const int64_t src = t - k;"),
    ("conv_no_bias", "double z = p.conv_b ? p.conv_b[d] : 0.0;", "double z = 0.0;"),
    ("silu_sign", "return z / (1.0 + std::exp(-z));", "return z / (1.0 + std::exp(z));"),
    ("ignore_h0", "h[n] = p.h0 ? p.h0[(b * D + d) * N + n] : 0.0;", "h[n] = 0.0;"),
    ("B_lag", "const double* Bt = p.Bm + (b * L + t) * N;",
     "const double* Bt = p.Bm + (b * L + (t > 0 ? t - 1 : 0)) * N;"),
    ("C_from_batch0", "const double* Ct = p.Cm + (b * L + t) * N;",
     "const double* Ct = p.Cm + t * N;"),
    ("softplus_no_bias", "if (p.delta_bias) v += p.delta_bias[d];", ""),
    ("softplus_naive", "std::log1p(std::exp(-std::fabs(v)))",
     "std::log(1.0 + std::exp(-std::fabs(v)))"),
    ("softplus_sign", "(v > 0.0 ? v : 0.0)", "(v > 0.0 ? 0.0 : v)"),
    ("gate_before_skip",
     "double out = acc + dskip * u;\n    if (p.z) out *= silu(p.z[(b * L + t) * D + d]);",
     "double out = acc;\n    if (p.z) out *= silu(p.z[(b * L + t) * D + d]);\n    out += dskip * u;"),
    ("gate_sigmoid", "if (p.z) out *= silu(p.z[(b * L + t) * D + d]);",
     "if (p.z) out *= 1.0 / (1.0 + std::exp(-p.z[(b * L + t) * D + d]));"),
    ("conv_state_ignored", "if (!p.conv_state_in || t < -S) return 0.0;", "return 0.0;"),
    ("conv_state_reversed", "return p.conv_state_in[(b * p.dim + d) * S + S + t];",
     "return p.conv_state_in[(b * p.dim + d) * S - 1 - t];"),
    ("conv_state_out_shift", "x_at(p, b, L - S + j, d);", "x_at(p, b, L - S + j - 1, d);"),
    ("bwd_no_adjoint_decay", "g[n] = abar * G;", "g[n] = G;"),
    ("bwd_drop_output_term", "const double G = g[n] + Cn * gy;", "const double G = g[n];"),
    ("bwd_dC_prev_state", "p.dC[(b * L + t) * N + n] += gy * h_now;",
     "p.dC[(b * L + t) * N + n] += gy * h_prev;"),
    ("bwd_ddelta_no_decay_term", "ddt += G * (a_cont * abar * h_prev + df_dt * Bn * u);",
     "ddt += G * (df_dt * Bn * u);"),
    ("bwd_dA_no_input_term", "dA[d * N + n] += G * (dt * abar * h_prev + df_da * Bn * u);",
     "dA[d * N + n] += G * (dt * abar * h_prev);"),
    ("bwd_zoh_dfda_sign", "*df_da = (dt * e - std::expm1(dt * a_cont) / a_cont) / a_cont;",
     "*df_da = (std::expm1(dt * a_cont) / a_cont - dt * e) / a_cont;"),
    ("bwd_du_no_factor", "du += G * f * Bn;", "du += G * Bn;"),
    ("bwd_dD_no_input", "dD[d] += gy * u;", "dD[d] += gy;"),
    ("bwd_dh0_undecayed", "for (int64_t n = 0; n < N; ++n) p.dh0[(b * D + d) * N + n] = g[n];",
     "for (int64_t n = 0; n < N; ++n) p.dh0[(b * D + d) * N + n] = g[n] + 1e-3;"),
    # the per-entry magnitudes that set the gradient tolerances
    ("mag_adjoint_no_decay", "gm[n] = abar * Gm;", "gm[n] = Gm;"),
    ("mag_drop_output_term", "const double Gm = gm[n] + std::fabs(Cn * gy);",
     "const double Gm = gm[n];"),
    ("mag_ddelta_signed_A",
     "mddt += Gm * (std::fabs(a_cont) * abar * hpm + std::fabs(df_dt * Bn * u));",
     "mddt += Gm * (a_cont * abar * hpm + std::fabs(df_dt * Bn * u));"),
    ("mag_state_signed_input", "if (mag) Hm[(t + 1) * N + n] = abar * Hm[t * N + n] + std::fabs(inp);",
     "if (mag) Hm[(t + 1) * N + n] = abar * Hm[t * N + n] + inp;"),
    ("mag_dx_no_skip", "double mdu = std::fabs(dskip * gy), mddt = 0.0;",
     "double mdu = 0.0, mddt = 0.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not unique: %s" % name
    mut_src = tmp_path / ("oracle_%s.cpp" % name)
    mut_src.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mut_src), out=str(tmp_path / ("lib_%s.so" % name)))
    orc = oracle.Oracle(lib)
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError as e:
            failures.append(pin.__name__)
    assert failures, "no pin caught mutant %s" % name
