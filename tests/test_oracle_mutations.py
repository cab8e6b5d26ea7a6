"""Planted mistakes in the oracle must fail its pins.

Each case copies the oracle's C sources and the oracle test files into a
temporary directory, plants one plausible mistake in the copy (a dropped
term, a wrong sign or operand, a missing decay, a swapped index, an
overwrite instead of an accumulation), builds the copy with gcc and runs the
pin tests that cover that part in a child process.  The case passes when
those pins FAIL on the mutant; a control run checks that the unmodified copy
passes them.  Everything runs on the CPU; the repository's own oracle is
never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (case id, oracle source, exact text, replacement, pin test file)
MUTATIONS = [
    # Sparse State Expansion: the shared partition (weight 1, decay every token, own q/k)
    ("sse_shared_no_decay", "sse_oracle.c",
     "ss[(size_t)row * d + x] = (double)lt[row] * ss[(size_t)row * d + x] +",
     "ss[(size_t)row * d + x] = ss[(size_t)row * d + x] +", "test_oracle_sse.py"),
    ("sse_shared_reads_routed_query", "sse_oracle.c",
     "ot[x] += (double)qs[row] * ss[", "ot[x] += (double)qt[row] * ss[", "test_oracle_sse.py"),
    ("sse_shared_writes_routed_key", "sse_oracle.c",
     "(double)ks[row] * (double)vt[x];", "(double)kt[row] * (double)vt[x];",
     "test_oracle_sse.py"),
    ("sse_shared_gated_write", "sse_oracle.c",
     "(double)ks[row] * (double)vt[x];", "e[pick[0]] * (double)ks[row] * (double)vt[x];",
     "test_oracle_sse.py"),
    ("sse_routed_ungated_write", "sse_oracle.c",
     "si[(size_t)row * d + x] +\n                                                          "
     "e[i] * (double)kt[row] * (double)vt[x];",
     "si[(size_t)row * d + x] +\n                                                          "
     "(double)kt[row] * (double)vt[x];", "test_oracle_sse.py"),
    ("sse_routed_ungated_read", "sse_oracle.c",
     "ot[x] += e[i] * (double)qt[row] * si[(size_t)row * d + x];\n                    }\n"
     "                } else {",
     "ot[x] += (double)qt[row] * si[(size_t)row * d + x];\n                    }\n"
     "                } else {", "test_oracle_sse.py"),
    ("sse_gate_unnormalised", "sse_oracle.c",
     "e[i] = exp((double)g[i] - mx) / z;", "e[i] = exp((double)g[i] - mx);",
     "test_oracle_sse.py"),
    # Sparse Delta Memory: addressing
    ("sdm_score_product", "sdm_oracle.c",
     "float s = h1[a] + h2[b];", "float s = h1[a] * h2[b];", "test_oracle_sdm.py"),
    ("sdm_slot_transposed", "sdm_oracle.c",
     "cand[n].id = a * sqrtN + b;", "cand[n].id = b * sqrtN + a;", "test_oracle_sdm.py"),
    ("sdm_tie_highest_index", "sdm_oracle.c",
     "if (a->id < b->id) return -1;\n    if (a->id > b->id) return 1;",
     "if (a->id > b->id) return -1;\n    if (a->id < b->id) return 1;", "test_oracle_sdm.py"),
    # Sparse Delta Memory: recurrence
    ("sdm_no_decay", "sdm_oracle.c",
     "mt[(size_t)n * dv + c] = a * tab[(size_t)iw[n] * dv + c];",
     "mt[(size_t)n * dv + c] = tab[(size_t)iw[n] * dv + c];", "test_oracle_sdm.py"),
    ("sdm_shared_no_beta", "sdm_oracle.c",
     "mt[(size_t)n * dv + c] + be * gw[n] * ((double)vt[c] - vhat[c]);",
     "mt[(size_t)n * dv + c] + gw[n] * ((double)vt[c] - vhat[c]);", "test_oracle_sdm.py"),
    ("sdm_per_slot_residual_sign", "sdm_oracle.c",
     "be * gw[n] * ((double)vt[c] - mt[(size_t)n * dv + c]);",
     "be * gw[n] * ((double)vt[c] + mt[(size_t)n * dv + c]);", "test_oracle_sdm.py"),
    ("sdm_read_unweighted", "sdm_oracle.c",
     "for (int m = 0; m < R; ++m) s += gr[m] * tab[(size_t)ir[m] * dv + c];",
     "for (int m = 0; m < R; ++m) s += tab[(size_t)ir[m] * dv + c];", "test_oracle_sdm.py"),
    # Sparse Delta Memory: backward by undoing writes
    ("bwd_dw_dropped_term", "sdm_oracle.c",
     "residual_mode == 0 ? be * gres - mdr : be * gres;",
     "residual_mode == 0 ? be * gres : be * gres;", "test_oracle_sdm_backward.py"),
    ("bwd_dmt_sign", "sdm_oracle.c",
     "double dmt = residual_mode == 0 ? gn[c] - gw[n] * dr[c]",
     "double dmt = residual_mode == 0 ? gn[c] + gw[n] * dr[c]", "test_oracle_sdm_backward.py"),
    ("bwd_missing_decay", "sdm_oracle.c",
     "gn[c] = a * dmt;", "gn[c] = dmt;", "test_oracle_sdm_backward.py"),
    ("bwd_per_slot_factor", "sdm_oracle.c",
     ": (1.0 - be * gw[n]) * gn[c];", ": gn[c];", "test_oracle_sdm_backward.py"),
    ("bwd_softmax_uncentred", "sdm_oracle.c",
     "double ds = w[m] * (dw[m] - dot);", "double ds = w[m] * dw[m];",
     "test_oracle_sdm_backward.py"),
    ("bwd_half_index_swap", "sdm_oracle.c",
     "d1[ip[m] / sqrtN] += ds;\n            d2[ip[m] % sqrtN] += ds;",
     "d1[ip[m] % sqrtN] += ds;\n            d2[ip[m] / sqrtN] += ds;",
     "test_oracle_sdm_backward.py"),
    ("bwd_read_grad_overwrites", "sdm_oracle.c",
     "G[(size_t)ir[m] * dv + c] += gr[m] * dyt[c];", "G[(size_t)ir[m] * dv + c] = gr[m] * dyt[c];",
     "test_oracle_sdm_backward.py"),
    ("bwd_dalpha_on_decayed_rows", "sdm_oracle.c",
     "da += sv[(size_t)n * dv + c] * dmt;", "da += a * sv[(size_t)n * dv + c] * dmt;",
     "test_oracle_sdm_backward.py"),
    # read epilogue
    ("norm_sum_not_mean", "sdm_oracle.c",
     "double inv = 1.0 / sqrt(ss / d + eps);", "double inv = 1.0 / sqrt(ss + eps);",
     "test_oracle_norm_gate.py"),
    ("gate_silu_sigmoid_swapped", "sdm_oracle.c",
     "f = act == 1 ? x * sg : sg;", "f = act == 1 ? sg : x * sg;", "test_oracle_norm_gate.py"),
    # Gated DeltaNet / KDA / GDN2
    ("gdn_prediction_from_query", "gdn_oracle.c",
     "pred[c] += (double)kt[i] * st[(size_t)i * dv + c];",
     "pred[c] += (double)qt[i] * st[(size_t)i * dv + c];", "test_oracle_gdn.py"),
    ("gdn_no_beta", "gdn_oracle.c",
     "st[(size_t)i * dv + c] += be * (double)kt[i] * ((double)vt[c] - pred[c]);",
     "st[(size_t)i * dv + c] += (double)kt[i] * ((double)vt[c] - pred[c]);",
     "test_oracle_gdn.py"),
    ("kda_decay_channel_reversed", "gdn_oracle.c",
     "double a = kda ? (double)alpha[bth * dk + i] : (double)alpha[bth];",
     "double a = kda ? (double)alpha[bth * dk + (dk - 1 - i)] : (double)alpha[bth];",
     "test_oracle_gdn.py"),
    ("gdn_read_with_key", "gdn_oracle.c",
     "for (int c = 0; c < dv; ++c) ot[c] += (double)qt[i] * st[(size_t)i * dv + c];\n"
     "            }\n            free(pred);",
     "for (int c = 0; c < dv; ++c) ot[c] += (double)kt[i] * st[(size_t)i * dv + c];\n"
     "            }\n            free(pred);", "test_oracle_gdn.py"),
    ("gdn2_erase_ignores_b", "gdn_oracle.c",
     "const double e = (double)bt[i] * (double)kt[i];", "const double e = (double)kt[i];",
     "test_oracle_gdn.py"),
    ("gdn2_write_ignores_w", "gdn_oracle.c",
     "r[c] = (double)wt[c] * (double)vt[c];", "r[c] = (double)vt[c];", "test_oracle_gdn.py"),
]


def _copy_tree(dst):
    os.makedirs(os.path.join(dst, "oracle"))
    for f in ("__init__.py", "build.py", "sdm_oracle.c", "gdn_oracle.c", "sse_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", f), os.path.join(dst, "oracle", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    for f in os.listdir(os.path.join(ROOT, "tests")):
        if f.startswith("test_oracle_") and f != os.path.basename(__file__) or f in (
                "conftest.py", "helpers.py", "__init__.py"):
            shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))


def _build_and_run(root, test_file):
    env = dict(os.environ, OMP_NUM_THREADS="2")
    subprocess.run([sys.executable, os.path.join(root, "oracle", "build.py")], check=True,
                   capture_output=True, env=env)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(root, "tests", test_file)],
                       capture_output=True, text=True, cwd=root, env=env)
    return r


@pytest.fixture(scope="module")
def pristine(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("oracle_copy"))
    _copy_tree(d)
    return d


def test_unmodified_copy_passes_every_pin(pristine, tmp_path):
    root = str(tmp_path / "ok")
    shutil.copytree(pristine, root)
    for f in sorted({m[4] for m in MUTATIONS}):
        r = _build_and_run(root, f)
        assert r.returncode == 0, f"{f} fails on the unmodified oracle:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("case,src,old,new,test_file", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(pristine, tmp_path, case, src, old, new, test_file):
    root = str(tmp_path / case)
    shutil.copytree(pristine, root)
    path = os.path.join(root, "oracle", src)
    text = open(path).read()
    assert text.count(old) == 1, f"{case}: the text to mutate must occur exactly once in {src}"
    open(path, "w").write(text.replace(old, new))
    r = _build_and_run(root, test_file)
    assert r.returncode == 1, f"{case}: the pins in {test_file} did not catch the planted " \
                              f"mistake (exit {r.returncode}):\n{r.stdout[-1500:]}"
