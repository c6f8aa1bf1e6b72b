"""The oracle's pins are sharp: each plausible mistake planted in a copy of
the oracle's C source (a dropped term, a wrong sign or index, a transposed
field order) or of its Python compositions (decoder layer, MoE layer, logits
head) makes the pin suite fail. CPU only; the planted copies live in a
temporary directory: C mutants are loaded through QG_ORACLE_LIB, Python
mutants run from a copy of the package tree, both in a subprocess."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qg_oracle.c")

MUTANTS = [
    ("msb_first_fields", "unsigned shift = (unsigned)(W->bits * (k % per_word));",
     "unsigned shift = (unsigned)(W->bits * (per_word - 1 - k % per_word));"),
    ("wrong_code_mask", "return (word >> shift) & ((1u << W->bits) - 1u);",
     "return (word >> shift) & 0xFu;"),
    ("neighbour_group", "size_t gi = (size_t)n * groups_per_row + k / W->group;",
     "size_t gi = (size_t)n * groups_per_row + (k / W->group + 1) % groups_per_row;"),
    ("dropped_bias", "(double)c * og_half_to_double(W->scales[gi]) + og_half_to_double(W->biases[gi])",
     "(double)c * og_half_to_double(W->scales[gi])"),
    ("bias_sign", "(double)c * og_half_to_double(W->scales[gi]) + og_half_to_double(W->biases[gi])",
     "(double)c * og_half_to_double(W->scales[gi]) - og_half_to_double(W->biases[gi])"),
    ("lut_row_zero", "return og_half_to_double(W->lut[(size_t)n * (1u << W->bits) + c]);",
     "return og_half_to_double(W->lut[c]);"),
    ("reversed_k", "acc += weight_at(W, n, k) * xm[k];",
     "acc += weight_at(W, n, W->K - 1 - k) * xm[k];"),
    ("dropped_residual", "j->y[o] = (j->residual ? j->residual[o] : 0.0) + acc;",
     "j->y[o] = acc;"),
    ("half_subnormal_exp", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    ("eps_outside_sqrt", "double denom = sqrt(ss / K + eps);", "double denom = sqrt(ss / K) + eps;"),
    ("sum_not_mean", "double denom = sqrt(ss / K + eps);", "double denom = sqrt(ss + eps);"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("topk_tie_high_index", "    if (va != vb)\n        return va > vb;\n    return ia < ib;",
     "    if (va != vb)\n        return va > vb;\n    return ia > ib;"),
    ("route_bad_norm", "w[i] = exp(logits[ids[i]] - lmax) / den;",
     "w[i] = exp(logits[ids[i]] - lmax) / (den + 1.0);"),
    ("splitmix_counter_from_zero", "uint64_t z = seed + (counter + 1u) * 0x9E3779B97F4A7C15ull;",
     "uint64_t z = seed + counter * 0x9E3779B97F4A7C15ull;"),
    ("splitmix_shift", "z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;",
     "z = (z ^ (z >> 28)) * 0x94D049BB133111EBull;"),
    ("uniform_52_bits", "return (double)(og_splitmix64(seed, counter) >> 11) * 0x1.0p-53;",
     "return (double)(og_splitmix64(seed, counter) >> 12) * 0x1.0p-53;"),
    ("sample_temperature_times", "w[i] = exp((vals[i] - vals[0]) / temperature);",
     "w[i] = exp((vals[i] - vals[0]) * temperature);"),
    ("sample_no_top_p", "if (prefix >= top_p * total)", "if (prefix >= total)"),
    ("sample_target_not_scaled", "const double target = u * prefix;", "const double target = u;"),
    ("attn_head_mapping", "const int g = h / G;", "const int g = h % Hkv;"),
    ("attn_no_scale", "s[t] = scale * acc;", "s[t] = acc;"),
    ("attn_unnormalized", "out[(size_t)h * d + j] = acc / den;", "out[(size_t)h * d + j] = acc;"),
    ("attn_drops_last_position", "        for (int t = 0; t < n; ++t) {\n            s[t] = exp(s[t] - smax);",
     "        for (int t = 0; t < n; ++t) {\n            if (t == n - 1) { s[t] = 0.0; continue; }\n            s[t] = exp(s[t] - smax);"),
    ("dense_read_as_integer", "        return og_half_to_double((uint16_t)c);", "        return (double)c;"),
    ("byte_mask_for_8bit", "return (word >> shift) & ((1u << W->bits) - 1u);",
     "return (word >> shift) & (W->bits == 8 ? 0x7Fu : ((1u << W->bits) - 1u));"),
    ("sample_greedy_last", "        *token = idx[0];\n        return 0;", "        *token = idx[k - 1];\n        return 0;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut_c = tmp_path / f"{name}.c"
    mut_so = tmp_path / f"{name}.so"
    mut_c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(mut_so), str(mut_c), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, QG_ORACLE_LIB=str(mut_so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"


SRC_PY = os.path.join(ROOT, "oracle", "__init__.py")

PY_MUTANTS = [
    ("decoder_ffn_reads_x", 'u = rmsnorm_swiglu(w["gate"], w["up"], h, w["g_ffn"], eps, nthreads)',
     'u = rmsnorm_swiglu(w["gate"], w["up"], x, w["g_ffn"], eps, nthreads)'),
    ("decoder_norm_weights_swapped",
     'qkv = rmsnorm_gemv(w["qkv"], x, w["g_attn"], eps, None, nthreads)\n    a = qkv[:q_dim]\n'
     '    h = gemv(w["o"], a, x, nthreads)\n    u = rmsnorm_swiglu(w["gate"], w["up"], h, w["g_ffn"], eps,',
     'qkv = rmsnorm_gemv(w["qkv"], x, w["g_ffn"], eps, None, nthreads)\n    a = qkv[:q_dim]\n'
     '    h = gemv(w["o"], a, x, nthreads)\n    u = rmsnorm_swiglu(w["gate"], w["up"], h, w["g_attn"], eps,'),
    ("decoder_wrong_q_slice", "a = qkv[:q_dim]", "a = qkv[-q_dim:]"),
    ("decoder_o_no_residual", 'h = gemv(w["o"], a, x, nthreads)', 'h = gemv(w["o"], a, None, nthreads)'),
    ("decoder_down_residual_x", 'return gemv(w["down"], u, h, nthreads)',
     'return gemv(w["down"], u, x, nthreads)'),
    ("rmsnorm_gemv_drops_residual", "y = gemv(W, Xn, residual, nthreads)",
     "y = gemv(W, Xn, None, nthreads)"),
    ("rmsnorm_gemv_no_norm", "Xn = np.stack([rmsnorm(row, g, eps) for row in X])\n    y = gemv",
     "Xn = X\n    y = gemv"),
    ("swiglu_gate_up_swapped", "u = swiglu(Wg, Wu, Xn, nthreads)", "u = swiglu(Wu, Wg, Xn, nthreads)"),
    ("moe_shared_weighted", "y = y + gemv(shared[2], u, None, nthreads)",
     "y = y + wts[0] * gemv(shared[2], u, None, nthreads)"),
    ("moe_weights_reversed", "for e, we in zip(ids, wts):", "for e, we in zip(ids, wts[::-1]):"),
    ("moe_no_norm", "xn = x if g is None else rmsnorm(x, g, eps)\n    ids, wts",
     "xn = x\n    ids, wts"),
    ("logits_no_norm", "xn = x if g is None else rmsnorm(x, g, eps)\n    z = gemv",
     "xn = x\n    z = gemv"),
    ("expert_slice_next_expert", "out[key] = W_all[key][e * N:(e + 1) * N]",
     'out[key] = W_all[key][((e + 1) % W_all["E"]) * N:((e + 1) % W_all["E"] + 1) * N]'),
]


@pytest.mark.parametrize("name,old,new", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_composition_mistake_is_caught(name, old, new, tmp_path):
    src = open(SRC_PY).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    for d in ("oracle", "synth"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    os.makedirs(tmp_path / "tests")
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    (tmp_path / "oracle" / "__init__.py").write_text(src.replace(old, new))
    import oracle
    env = dict(os.environ, QG_ORACLE_LIB=oracle.build(force=False))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        str(tmp_path / "tests" / "test_oracle.py")],
                       env=env, cwd=str(tmp_path), capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
