"""The pins must catch plausible mistakes in the oracle.

Each mutant is a copy of ``oracle/moe_oracle.c`` with one planted mistake (a
dropped term, a wrong sign, index or operand), compiled with gcc on the CPU;
the pin and brute-force suites run against it in a subprocess and must fail.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "router_bias_dropped": ("      if (bias) s += (double)bias[e];\n", "\n"),
    "tie_to_higher_index": ("if (best < 0 || l[e] > l[best]) best = e;",
                            "if (best < 0 || l[e] >= l[best]) best = e;"),
    "softmax_sign": ("p[e] = exp(l[e] - m);", "p[e] = exp(m - l[e]);"),
    "softmax_unnormalised": ("for (int64_t e = 0; e < E; e++) p[e] /= z;", ""),
    "topk_not_renormalised": ("g[j] = (k >= 2 && normalize) ? p[sel[j]]", "g[j] = (0) ? p[sel[j]]"),
    "aux_uses_last_choice": ("f[ids[t * k]] += 1.0;", "f[ids[t * k + k - 1]] += 1.0;"),
    "aux_missing_N": ("loss *= alpha * (double)E;", "loss *= alpha;"),
    "capacity_floor": ("c = (int64_t)ceil(", "c = (int64_t)floor("),
    "slot_off_by_one": ("rank = n;", "rank = n + 1;"),
    "kept_unclamped": ("kept[e] = (int32_t)(n < C ? n : C);", "kept[e] = (int32_t)n;"),
    "w1_transposed": ("s += weight(w1, w_fmt, s1, F, D, f, i) * elem(xr, x_fmt, row * D + i);",
                      "s += weight(w1, w_fmt, s1, D, F, i, f) * elem(xr, x_fmt, row * D + i);"),
    "gelu_tanh_form": ("return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));",
                       "return 0.5 * z * (1.0 + tanh(0.7978845608028654 * (z + 0.044715 * z * z * z)));"),
    "int8_group_index": ("scale[n * (K / OR_GROUP) + i / OR_GROUP]",
                         "scale[n * (K / OR_GROUP) + (i % (K / OR_GROUP))]"),
    "combine_reads_dropped": ("if (slots[t * k + j] >= 0)\n", "\n"),
    "combine_gate_ignored": ("m += gates[t * k + j] * expert_out", "m += expert_out"),
    "residual_dropped": ("(add_skip ? elem(x, x_fmt, t * D + o) : 0.0)", "0.0"),
    "dense_mlp_dropped": (" + dense[t * D + o];", ";"),
    "zloss_not_squared": ("acc += lz * lz;", "acc += lz;"),
    "quant_round_toward_zero": ("nearbyint(r[i] / s)", "trunc(r[i] / s)"),
    # backward
    "bwd_gelu_grad_missing_term": (
        "return 0.5 * (1.0 + erf(z / sqrt(2.0))) + z * inv_sqrt_2pi * exp(-0.5 * z * z);",
        "return 0.5 * (1.0 + erf(z / sqrt(2.0)));"),
    "bwd_renorm_without_correction": ("normalize) ? (dg[j] - sdg) / S : dg[j]",
                                      "normalize) ? dg[j] / S : dg[j]"),
    "bwd_dropped_get_gradient": ("if (ids[q] != e || slots[q] < 0) continue;",
                                 "if (ids[q] != e) continue;"),
    "bwd_aux_gradient_dropped": (
        "dp[e] = g_aux * alpha * (double)E * f[e] / (double)T;", "dp[e] = 0.0;"),
    "bwd_softmax_jacobian_sign": ("p[e] * (dp[e] - pdp)", "p[e] * (dp[e] + pdp)"),
    "bwd_zloss_grad_halved": ("g_z * 2.0 / (double)T", "g_z * 1.0 / (double)T"),
    "bwd_dw2_uses_preactivation": ("const double hf = gelu(a[f]);", "const double hf = a[f];"),
    # router variants
    "topp_never_stops": ("if (variant == OR_ROUTER_TOP_P && cum > top_p) break;", "if (0) break;"),
    "cosine_without_tau": ("dot / (tau * nu * ne)", "dot / (nu * ne)"),
    "noisy_scale_not_softplus": ("sigma[e] = softplus(z);", "sigma[e] = z;"),
    "noisy_gates_not_renormalised": ("if (variant == OR_ROUTER_NOISY) renorm = 1;",
                                     "if (variant == OR_ROUTER_NOISY) renorm = 0;"),
    "load_p_threshold_counts_itself": ("if (j != e) other[no++] = l[j];", "other[no++] = l[j];"),
    "cov2_sample_variance": ("var /= (double)n;", "var /= (double)(n - 1);"),
    "unused_slot_marked_dropped": ("    slots[a] = -1;\n    drop[a] = 0;", "    slots[a] = -1;\n    drop[a] = 1;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique / missing"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(out=lib, src=str(mut), extra=("-w",))
    env = dict(os.environ, MOE_ORACLE_LIB=lib)
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py"),
         os.path.join(ROOT, "tests", "test_oracle_bruteforce.py"),
         os.path.join(ROOT, "tests", "test_oracle_backward.py"),
         os.path.join(ROOT, "tests", "test_oracle_router_variants.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
