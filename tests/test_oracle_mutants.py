"""The oracle's pins reject plausible mistakes.

Each case plants one mistake in a copy of the oracle source (on the CPU,
in a temporary directory), builds it, and runs the pin tests against the
mutant; the pins must fail.  The shipped oracle is never modified.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.cpp")

MUTANTS = {
    "update_transposed": ("const T prod = k[i] * delta[j];",
                          "const T prod = k[j] * delta[i];"),
    "decay_on_value_axis": (
        "for (int j = 0; j < D; ++j) S[i * D + j] = a * S[i * D + j];",
        "for (int j = 0; j < D; ++j) S[j * D + i] = a * S[j * D + i];"),
    "delta_sign": ("delta[j] = beta * (v[j] - u);",
                   "delta[j] = beta * (u - v[j]);"),
    "readout_before_update": (
        "const T prod = q[i] * S[i * D + j];",
        "const T prod = q[i] * (S[i * D + j] - k[i] * delta[j]);"),
    "u_from_q": ("const T prod = k[i] * S[i * D + j];\n      u = u + prod;",
                 "const T prod = q[i] * S[i * D + j];\n      u = u + prod;"),
    "taps_reversed": (
        "const T prod = T(w[t * wstride]) * T(bf16_to_f32(xt));",
        "const T prod = T(w[(W - 1 - t) * wstride]) * T(bf16_to_f32(xt));"),
    "shift_wrong_end": ("cs[(W - 2) * cs_stride] = x;", "cs[0] = x;"),
    "gate_activation_swapped": (
        "const T gj = gate_silu ? gv * sigmoid(gv) : sigmoid(gv);",
        "const T gj = gate_silu ? sigmoid(gv) : gv * sigmoid(gv);"),
    "norm_sum_not_mean": ("ss / T(D) + eps", "ss + eps"),
    "null_only_negative": ("if (s <= 0 || s >= S) {", "if (s < 0 || s >= S) {"),
    "channel_offset": ("const int64_t c = p * C + h * D + i;",
                       "const int64_t c = p * C + h + i * H;"),
    "state_head_offset": ("T* Sst = rec_state + (s * H + h) * D * D;",
                          "T* Sst = rec_state + (s * H + (H - 1 - h)) * D * D;"),
    "gate_head_offset": ("norm_on ? gate + n * C + h * D : nullptr",
                         "norm_on ? gate + n * C : nullptr"),
    "g_row_head_swap": ("gg[i] = T(g[(n * H + h) * D + i]);",
                        "gg[i] = T(g[(h * B + n) * D + i]);"),
    "bf16_round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0u * lsb;"),
    # variants and extra inputs
    "l2_eps_outside_sqrt": ("const T r = T(1) / std::sqrt(ss + T(1e-6));",
                            "const T r = T(1) / (std::sqrt(ss) + T(1e-6));"),
    "q_scale_inverted": ("T(1) / std::sqrt(T(D)));", "std::sqrt(T(D)));"),
    "raw_gate_sign": ("return -(a * softplus(z));", "return a * softplus(z);"),
    "bounded_gate_no_rate": (
        "if (bounded) return lower_bound * sigmoid(a * z);",
        "if (bounded) return lower_bound * sigmoid(z);"),
    "softplus_dropped": ("return x > T(20) ? x : std::log1p(std::exp(x));",
                         "return x;"),
    "raw_beta_not_activated": (
        "beta_nh = sigmoid(T(bf16_to_f32(ex->raw_beta[n * H + h])));",
        "beta_nh = T(bf16_to_f32(ex->raw_beta[n * H + h]));"),
    "tap_major_stride": (
        "const int64_t cs_tap = (fl & F_CONV_TAP_MAJOR) ? 3 * C : 1;",
        "const int64_t cs_tap = (fl & F_CONV_TAP_MAJOR) ? C : 1;"),
    "update_flag_ignored": ("const bool update = !(fl & F_NO_CONV_UPDATE);",
                            "const bool update = true;"),
    "conv_bias_channel": (
        "const T bias = conv_bias ? T(conv_bias[c]) : T(0);",
        "const T bias = conv_bias ? T(conv_bias[c % C]) : T(0);"),
}


def _run_mutant(name, tmp):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, name
    msrc = os.path.join(tmp, name + ".cpp")
    mlib = os.path.join(tmp, name + ".so")
    with open(msrc, "w") as f:
        f.write(src.replace(before, after))
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off",
                    "-fopenmp", "-fPIC", "-shared", msrc, "-o", mlib],
                   check=True, capture_output=True)
    env = dict(os.environ, KDA_ORACLE_LIB=mlib, OMP_NUM_THREADS="1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py"),
         os.path.join(ROOT, "tests", "test_oracle_step.py"),
         os.path.join(ROOT, "tests", "test_oracle_variants.py")],
        cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            codes = dict(zip(MUTANTS, ex.map(lambda n: _run_mutant(n, tmp),
                                             MUTANTS)))
    survived = [n for n, rc in codes.items() if rc == 0]
    assert not survived, f"mutants not caught by any pin: {survived}"
    # rc 1 = tests failed (not an import or collection error)
    assert all(rc == 1 for rc in codes.values()), codes
