"""The pins must catch a plausible mistake anywhere in the oracle.

Each case plants one mistake in a copy of oracle.c (on the CPU only),
builds it, and runs the pin tests against the broken build in a fresh
process: at least one pin has to fail.  The cases run several at a time.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "scale_without_sqrt_n": ("return sqrtf(t[0]) / sqrtf((float)n);", "return sqrtf(t[0]);"),
    "scale_counts_padding": ("return sqrtf(t[0]) / sqrtf((float)n);",
                             "return sqrtf(t[0]) / sqrtf((float)C);"),
    "adjacent_pair_tree": ("for (int64_t j = 0; j < h; ++j) t[j] = t[j] + t[j + h];",
                           "for (int64_t j = 0; j < h; ++j) t[j] = t[2 * j] + t[2 * j + 1];"),
    "sign_strict": ("const int bit = z[j] >= 0.0f;", "const int bit = z[j] > 0.0f;"),
    "error_sign_flipped": ("z[j] = bit ? z[j] - s : z[j] + s;", "z[j] = bit ? z[j] + s : z[j] - s;"),
    "msb_first_bits": ("words[j / 32] |= 1u << (j % 32);",
                       "words[j / 32] |= 0x80000000u >> (j % 32);"),
    "no_error_feedback": ("z[j] = in[base + j] + err[base + j];", "z[j] = in[base + j];"),
    "sum_not_mean": ("a[base + j] = acc / (float)W;", "a[base + j] = acc;"),
    "no_server_error": ("for (int64_t i = 0; i < n; ++i) y[i] = y[i] + err_s[i];", ""),
    "betas_transposed": ("in[i] = (hp->beta1 * m[i]) + (a1 * grads[w][i]);",
                         "in[i] = (a1 * m[i]) + (hp->beta1 * grads[w][i]);"),
    "ghat_without_beta1": ("const float ghat = (mhat[i] - (hp->beta1 * m[i])) / a1;",
                           "const float ghat = (mhat[i] - m[i]) / a1;"),
    "vfresh_linear": ("v_fresh[i] = (hp->beta2 * v_fresh[i]) + (a2 * (ghat * ghat));",
                      "v_fresh[i] = (hp->beta2 * v_fresh[i]) + (a2 * ghat);"),
    "ratio_inverted": ("const float q = (sqrtf(v_frozen[i]) + hp->eta) / (sqrtf(v_fresh[i]) + hp->eta);",
                       "const float q = (sqrtf(v_fresh[i]) + hp->eta) / (sqrtf(v_frozen[i]) + hp->eta);"),
    "no_relative_cap": ("float f = fminf(fminf(rho[l], hp->f_max), kp * f_prev[l]);",
                        "float f = fminf(rho[l], hp->f_max);"),
    "no_relative_floor": ("f = fmaxf(fmaxf(f, hp->f_min), km * f_prev[l]);",
                          "f = fmaxf(f, hp->f_min);"),
    "update_uses_fresh_variance": ("x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));",
                                   "x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_fresh[i]) + hp->eta)));"),
    "trust_ratio_inverted": ("(float)(sqrt(X) / sqrt(U))", "(float)(sqrt(U) / sqrt(X))"),
    "no_clip": ("c[l] = fminf(fmaxf(r, hp->c_min), hp->c_max);", "c[l] = r;"),
    "variance_linear": ("v[i] = (hp->beta2 * v[i]) + (a2 * (gbar * gbar));",
                        "v[i] = (hp->beta2 * v[i]) + (a2 * gbar);"),
    "gradient_sum_not_mean": ("const float gbar = gsum / (float)W;", "const float gbar = gsum;"),
    "freeze_keeps_errors": ("for (int64_t i = 0; i < N; ++i) err_s[i] = 0.0f;", ""),
    "adam_momentum_undamped": ("m[i] = (hp->beta1 * m[i]) + (a1 * gmean);",
                               "m[i] = (hp->beta1 * m[i]) + gmean;"),
    "adam_variance_linear": ("v[i] = (hp->beta2 * v[i]) + (a2 * (gmean * gmean));",
                             "v[i] = (hp->beta2 * v[i]) + (a2 * gmean);"),
    "adam_eta_inside_sqrt": (": m[i] / (sqrtf(v[i]) + hp->eta);",
                             ": m[i] / sqrtf(v[i] + hp->eta);"),
    "adam_worker_input_no_momentum": ("in[i] = (hp->beta1 * m[i]) + (a1 * gw[i]);",
                                      "in[i] = a1 * gw[i];"),
    "adam_update_with_old_momentum": (
        "x[i] = x[i] - (hp->lr * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));",
        "x[i] = x[i] - (hp->lr * (m[i] / (sqrtf(v_frozen[i]) + hp->eta)));"),
    "adam_momentum_not_replaced": ("    m[i] = mhat[i];\n  }\n  free(in);", "  }\n  free(in);"),
    "bias_sqrt_misplaced": ("u[i] = (m[i] / bc1) / (sqrtf(v[i] / bc2) + hp->eta);",
                            "u[i] = (m[i] / bc1) / ((sqrtf(v[i]) / bc2) + hp->eta);"),
    "bias_step_off_by_one": ("pow((double)beta, (double)t)", "pow((double)beta, (double)(t + 1))"),
    "adam_bias_first_moment_only": ("? (m[i] / bc1) / (sqrtf(v[i] / bc2) + hp->eta)",
                                    "? (m[i] / bc1) / (sqrtf(v[i]) + hp->eta)"),
    "weight_decay_sign": ("u[i] = u[i] + (hp->weight_decay * x[i]);",
                          "u[i] = u[i] - (hp->weight_decay * x[i]);"),
    "weight_decay_dropped_in_compression": (
        "((mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)) + (hp->weight_decay * x[i]))",
        "(mhat[i] / (sqrtf(v_frozen[i]) + hp->eta))"),
    "ema_weights_swapped": ("((1.0f - hp->c_avg_decay) * c[l])", "(hp->c_avg_decay * c[l])"),
    "ema_not_bias_corrected": ("(float)(1.0 - pow((double)d, (double)T_w))", "1.0f"),
    "norm_ratio_not_squared": ("Qf += df * df;", "Qf += df;"),
    "norm_ratio_inverted": ("(float)(sqrt(Qz) / sqrt(Qf))", "(float)(sqrt(Qf) / sqrt(Qz))"),
    "sparse_one_block_too_many": ("return rel < nsel ? rel * 64 + j % 64 : -1;",
                                  "return rel <= nsel ? rel * 64 + j % 64 : -1;"),
    "sparse_blocks_not_cyclic": ("const int64_t rel = ((j / 64) - first_block + nb) % nb;",
                                 "const int64_t rel = (j / 64) - first_block;"),
    "sparse_error_not_cleared": ("        err_w[w][i] = 0.0f;\n      } else {",
                                 "        err_w[w][i] = z;\n      } else {"),
    "sparse_no_local_error": ("        err_w[w][i] = z;\n      }", "        err_w[w][i] = 0.0f;\n      }"),
    "sparse_momentum_not_masked": ("      mhat[i] = 0.0f;\n", "      mhat[i] = hp->beta1 * m[i];\n"),
    "sparse_no_clamp": ("const float r = fminf(fmaxf(q, hp->f_min), hp->f_max);", "const float r = q;"),
    "sparse_update_fresh_variance": ("x[i] = x[i] - (step * (r * (mhat[i] / dz)));",
                                     "x[i] = x[i] - (step * (r * (mhat[i] / (sqrtf(v_fresh[i]) + hp->eta))));"),
    "sparse_sum_not_mean": ("      mhat[i] = acc / (float)W;", "      mhat[i] = acc;"),
    "sparse_step_drops_c_avg": ("const float step = hp->lr * c_avg[l];", "const float step = hp->lr;"),
    "c_drops_c_avg": ("c[l] = c_avg[l] * f;", "c[l] = f;"),
    "c_drops_factor": ("c[l] = c_avg[l] * f;", "c[l] = c_avg[l];"),
    "cap_uses_km": ("float f = fminf(fminf(rho[l], hp->f_max), kp * f_prev[l]);",
                    "float f = fminf(fminf(rho[l], hp->f_max), km * f_prev[l]);"),
    "floor_uses_kp": ("f = fmaxf(fmaxf(f, hp->f_min), km * f_prev[l]);",
                      "f = fmaxf(fmaxf(f, hp->f_min), kp * f_prev[l]);"),
    "f_prev_not_updated": ("    f_prev[l] = f;\n", ""),
    "rho_min_not_max": ("r = (i == off || isnan(q) || q > r) ? q : r;",
                        "r = (i == off || isnan(q) || q < r) ? q : r;"),
    "norm_ratio_zero_guard": ("r = (Qz == 0.0 || Qf == 0.0) ? 1.0f :", "r = (Qz == 0.0 || Qf == 0.0) ? 0.0f :"),
    "decompress_sign_inverted": (
        "out[base + j] = sign_bit(bits, C, k, j) ? scales[k] : -scales[k];",
        "out[base + j] = sign_bit(bits, C, k, j) ? -scales[k] : scales[k];"),
    "warmup_c_sum_replaced": ("c_sum[l] = c_sum[l] + c[l];", "c_sum[l] = c[l];"),
    "freeze_f_prev_not_one": ("    f_prev[l] = 1.0f;\n  }\n}", "    f_prev[l] = 0.5f;\n  }\n}"),
    "freeze_c_avg_not_divided": ("c_avg[l] = c_sum[l] / den;", "c_avg[l] = c_sum[l];"),
    "sign_words_not_cleared": ("  for (int64_t q = 0; q < C / 32; ++q) words[q] = 0u;\n", ""),
    "clip_bounds_swapped": ("c[l] = fminf(fmaxf(r, hp->c_min), hp->c_max);",
                            "c[l] = fmaxf(fminf(r, hp->c_min), hp->c_max);"),
    "trust_ratio_on_updated_x": ("X += (double)x[i] * (double)x[i];",
                                 "X += (double)(x[i] - hp->lr * u[i]) * (double)(x[i] - hp->lr * u[i]);"),
    "padding_slots_not_zeroed": ("t[j] = j < n ? z[j] * z[j] : 0.0f;", "t[j] = j < n ? z[j] * z[j] : t[j];"),
    "sparse_values_not_cleared": ("  for (int64_t q = 0; q < K * per; ++q) vals_s[q] = 0.0f;\n", ""),
    "sparse_worker_values_wrong_slot": (
        "if (vals_w && vals_w[w]) vals_w[w][k * per + slot] = z;",
        "if (vals_w && vals_w[w]) vals_w[w][k * per + (slot ^ 1)] = z;"),
    "sparse_momentum_not_replaced": (
        "        x[i] = x[i] - (step * (r * (mhat[i] / dz)));\n      }\n      m[i] = mhat[i];\n",
        "        x[i] = x[i] - (step * (r * (mhat[i] / dz)));\n      }\n"),
    "momentum_not_replaced": (
        "        x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));\n      m[i] = mhat[i];\n",
        "        x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));\n"),
    "update_with_old_momentum": (
        "        x[i] = x[i] - (step * (mhat[i] / (sqrtf(v_frozen[i]) + hp->eta)));\n      m[i] = mhat[i];\n",
        "        x[i] = x[i] - (step * (m[i] / (sqrtf(v_frozen[i]) + hp->eta)));\n      m[i] = mhat[i];\n"),
    "freeze_v_fresh_not_copied": ("  for (int64_t i = 0; i < N; ++i) v_fresh[i] = v[i];\n", ""),
    "rho_drops_later_nan": ("r = (i == off || isnan(q) || q > r) ? q : r;",
                            "r = (i == off || q > r) ? q : r;"),
    "rho_drops_every_nan": ("r = (i == off || isnan(q) || q > r) ? q : r;",
                            "r = (i == off || q > r || isnan(r)) ? q : r;"),
}


def _run_mutation(name, source, workdir):
    """Builds oracle.c with one planted mistake and runs the pins against it
    in a fresh process; returns (pytest exit code, tail of its output)."""
    old, new = MUTATIONS[name]
    assert source.count(old) == 1, f"mutation anchor not unique: {old!r}"
    os.makedirs(workdir, exist_ok=True)
    src = os.path.join(workdir, "oracle.c")
    with open(src, "w") as f:
        f.write(source.replace(old, new))
    lib = os.path.join(workdir, "liboracle_mut.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), "-o", lib, src, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, ONEBIT_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(request, tmp_path_factory):
    """Runs every selected mutation, several at a time (each in its own
    process), the first time a case asks for it."""
    selected = [it.callspec.params["name"] for it in request.session.items
                if it.module is request.module and hasattr(it, "callspec")]
    source = open(SRC).read()
    base = tmp_path_factory.mktemp("mutants")
    workers = max(1, min(6, (os.cpu_count() or 2) - 2))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        futs = {n: pool.submit(_run_mutation, n, source, str(base / n)) for n in selected}
        return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, outcomes):
    rc, out = outcomes[name]
    assert rc == 1, f"no pin failed for mutation {name}:\n{out}"
