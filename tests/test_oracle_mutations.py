"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin tests against that
build in a child process: every mutant must fail at least one pin.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTANTS = {
    "drop_D": ("if (d->has_D) yv += J->D[h] * u;", ""),
    "tap_reversed": ("c += J->conv_w[h * K + j] * conv_in(J, i, tau, h, win);",
                     "c += J->conv_w[h * K + (K - 1 - j)] * conv_in(J, i, tau, h, win);"),
    "conv_window_off_by_one": ("int64_t tau = t - (K - 1) + j;", "int64_t tau = t - K + j;"),
    "B_C_swapped": ("yv += Ct[n] * st[n];", "yv += Bt[n] * st[n];"),
    "dt_missing_from_input": ("st[n] = decay * st[n] + dtv * Bt[n] * u;",
                              "st[n] = decay * st[n] + Bt[n] * u;"),
    "exp_sign": ("const double decay = exp(dtv * A_at(J, h, n));",
                 "const double decay = exp(-dtv * A_at(J, h, n));"),
    "y_from_previous_state": ("st[n] = decay * st[n] + dtv * Bt[n] * u;\n                    yv += Ct[n] * st[n];",
                              "yv += Ct[n] * st[n];\n                    st[n] = decay * st[n] + dtv * Bt[n] * u;"),
    "state_written_to_id_row": ("J->state_out[((i * H + h) * P + p) * N + n] = st[n];",
                                "J->state_out[((r * H + h) * P + p) * N + n] = st[n];"),
    "group_map_interleaved": ("const int64_t g = J->grp_of_head[h];", "const int64_t g = h % G;"),
    "bwd_dC_from_previous_state": ("dCt[n] += dyt * h_cur;", "dCt[n] += dyt * h_prev;"),
    "bwd_carry_not_decayed": ("g[n] *= decay;                /* now dL/dh_{t-1} */", ""),
    "bwd_ddt_input_term_dropped": ("ddt += g[n] * (h_prev * decay * An + Bt[n] * u);",
                                   "ddt += g[n] * (h_prev * decay * An);"),
    "bwd_ds_to_sequence_row": ("J->d_s[((r * H + h) * P + p) * N + n] += g[n];",
                               "J->d_s[((i * H + h) * P + p) * N + n] += g[n];"),
    "bwd_softplus_chain_dropped": ("if (d->dt_softplus) ddt *= sigmoid(J->dt[(i * L + t) * H + h]);", ""),
    "conv_bwd_tap_reversed": ("d_sx[(s * d_inner + ch) * len + t + j] += g * w[ch * d_conv + j];",
                              "d_sx[(s * d_inner + ch) * len + t + j] += g * w[ch * d_conv + (d_conv - 1 - j)];"),
    "conv_bwd_dw_window_shift": ("d_w[ch * d_conv + j] += g * row[t + j];",
                                 "d_w[ch * d_conv + j] += g * row[t + d_conv - 1 - j];"),
    "conv_bwd_silu_derivative_is_sigmoid": ("g *= sg * (1.0 + z * (1.0 - sg));", "g *= sg;"),
    "fused_bwd_silu_derivative_is_sigmoid": ("du_t[t] *= sg * (1.0 + c * (1.0 - sg));",
                                             "du_t[t] *= sg;"),
    "fused_bwd_tap_reversed": ("if (t >= 0 && t < L) gin += J->conv_w[h * K + j] * du_t[t];",
                               "if (t >= 0 && t < L) gin += J->conv_w[h * K + (K - 1 - j)] * du_t[t];"),
    "fused_bwd_conv_state_to_sequence_row": (
        "else J->d_conv_state[(r * H + h) * (K - 1) + tau + K - 1] += gin;",
        "else J->d_conv_state[(i * H + h) * (K - 1) + tau + K - 1] += gin;"),
    "fused_bwd_dw_window_shift": ("gw += du_t[t] * conv_in(J, i, t - (K - 1) + j, h, win);",
                                  "gw += du_t[t] * conv_in(J, i, t - j, h, win);"),
    "decode_ring_not_shifted": ("for (int64_t j = 0; j + 1 < K - 1; j++) cs[j] = cs[j + 1];", ""),
    "decode_newest_tap_first": ("return c + w[K - 1] * xin;", "return c + w[0] * xin;"),
    "decode_gate_is_sigmoid": ("if (z) acc *= silu(z[(i * H + h) * P + p]);",
                               "if (z) acc *= sigmoid(z[(i * H + h) * P + p]);"),
    "decode_bias_after_softplus": ("double dd = dt[i * H + h] + (dt_bias ? dt_bias[h] : 0.0);\n            if (d->dt_softplus) dd = softplus(dd);",
                                   "double dd = dt[i * H + h];\n            if (d->dt_softplus) dd = softplus(dd);\n            dd += dt_bias ? dt_bias[h] : 0.0;"),
    "decode_y_from_previous_state": ("st[n] = a * st[n] + dd * B[(i * G + g) * N + n] * u;\n                    acc += C[(i * G + g) * N + n] * st[n];",
                                     "acc += C[(i * G + g) * N + n] * st[n];\n                    st[n] = a * st[n] + dd * B[(i * G + g) * N + n] * u;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src, "mutation site moved; update the table"
    c_file = tmp_path / f"{name}.c"
    c_file.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", str(so), str(c_file),
                           "-lm", "-lpthread"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py",
                        "tests/test_oracle_conv_bwd_pins.py", "tests/test_oracle_decode_pins.py",
                        "tests/test_oracle_fused_bwd_pins.py"],
                       cwd=ROOT, env=dict(os.environ, SSM_ORACLE_LIB=str(so)),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
