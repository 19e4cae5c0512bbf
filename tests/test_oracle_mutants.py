"""The oracle's pins catch plausible mistakes: each mutant below is oracle.c with one planted
mistake (a dropped term, a wrong index, a swapped order, a missing rounding point), built as a
separate library and run against every oracle pin (tests/test_oracle_*.py) in a child process
through MONO_ORACLE_LIB. Every mutant must fail at least one pin; the unmodified source, built
the same way, must pass them all. A mistake planted here lives only in a temporary copy of the
oracle, on the CPU.

Each replacement must match the source exactly once, so an edit of oracle.c that moves one of
these lines fails this test loudly instead of silently testing nothing.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = ["tests/test_oracle_hc.py", "tests/test_oracle_router.py", "tests/test_oracle_experts.py",
        "tests/test_oracle_formats.py", "tests/test_oracle_head.py", "tests/test_oracle_mxfp8.py"]

# name: [(text in oracle.c, replacement), ...]
MUTANTS = {
    # model tail: RMS over the H values of one stream instead of the 4H of the row
    "head_rms_over_one_stream": [("const double rms = sqrt(ss / (double)n + s->eps_hc);",
                                  "const double rms = sqrt(ss / (double)s->hidden + s->eps_hc);")],
    # model tail: every pre weight takes the first bias
    "head_first_bias_only": [("(double)m + (double)head_base[i]);",
                              "(double)m + (double)head_base[0]);")],
    # model tail: the head scale dropped
    "head_scale_dropped": [("pw[r * NSTREAM + i] = (float)sigmoid(a * (double)m +",
                            "pw[r * NSTREAM + i] = (float)sigmoid(1.0 * (double)m +")],
    # model tail: head rows read transposed (row i takes the stream-i column block of row 0)
    "head_rows_transposed": [("acc += (double)w_head[(int64_t)i * n + t] * v[t];",
                              "acc += (double)w_head[(t % NSTREAM) * n + (t / NSTREAM) + 0 * i] * v[t];")],
    # collapse: gate 3 - i weights stream i
    "collapse_pairing": [("acc += (double)pre[r * NSTREAM + i] *",
                          "acc += (double)pre[r * NSTREAM + (NSTREAM - 1 - i)] *")],
    # Sinkhorn: columns normalised before rows
    "sinkhorn_columns_first": [(
        "      for (int i = 0; i < NSTREAM; ++i) {\n        double sum = 0.0;\n"
        "        for (int j = 0; j < NSTREAM; ++j) sum += M[i][j];\n"
        "        for (int j = 0; j < NSTREAM; ++j) M[i][j] /= sum;\n      }\n"
        "      for (int j = 0; j < NSTREAM; ++j) {\n        double sum = 0.0;\n"
        "        for (int i = 0; i < NSTREAM; ++i) sum += M[i][j];\n"
        "        for (int i = 0; i < NSTREAM; ++i) M[i][j] /= sum;\n      }\n",
        "      for (int j = 0; j < NSTREAM; ++j) {\n        double sum = 0.0;\n"
        "        for (int i = 0; i < NSTREAM; ++i) sum += M[i][j];\n"
        "        for (int i = 0; i < NSTREAM; ++i) M[i][j] /= sum;\n      }\n"
        "      for (int i = 0; i < NSTREAM; ++i) {\n        double sum = 0.0;\n"
        "        for (int j = 0; j < NSTREAM; ++j) sum += M[i][j];\n"
        "        for (int j = 0; j < NSTREAM; ++j) M[i][j] /= sum;\n      }\n")],
    # Sinkhorn: one iteration short
    "sinkhorn_one_short": [("for (int it = 0; it < s->sinkhorn_iters; ++it)",
                            "for (int it = 1; it < s->sinkhorn_iters; ++it)")],
    # block from the unrounded shared output
    "block_shared_unrounded": [(
        "double sh = Is > 0 ? act_get(s->act, shared_out, (int64_t)r * H + c) : 0.0;",
        "double sh = Is > 0 ? (double)y[c] : 0.0;")],
    # RMSNorm: mean of squares over the unrounded collapse sums
    "norm_rms_of_unrounded_x": [("ss += xv * xv;", "ss += acc * acc;")],
    # expand: comb transposed
    "expand_comb_transposed": [("acc += (double)comb[r * 16 + i * NSTREAM + j] *",
                                "acc += (double)comb[r * 16 + j * NSTREAM + i] *")],
    # router weights gathered from the biased scores
    "weights_from_biased": [("float w = (float)((double)sc[c[j].e] / cl);",
                             "float w = (float)((double)c[j].beta / cl);")],
    # gate and up swapped
    "gate_up_swapped": [("float gf = (float)mat_row_dot(&ex->gate, H, i, vg);",
                         "float gf = (float)mat_row_dot(&ex->up, H, i, vu);"),
                        ("float uf = (float)mat_row_dot(&ex->up, H, i, vu);",
                         "float uf = (float)mat_row_dot(&ex->gate, H, i, vg);")],
    # MXFP8: shared exponent from emax 7 instead of 8
    "mxfp8_emax_7": [("X = (e2 - 1) - 8;", "X = (e2 - 1) - 7;")],
    # MXFP8: no clamp at the largest finite E4M3
    "mxfp8_no_saturation": [("if (r > 448.0) r = 448.0;", "")],
    # MXFP8: ties rounded away from zero
    "mxfp8_ties_away": [("double r = nearbyint(t / q) * q;", "double r = round(t / q) * q;")],
    # MXFP8: the down projection sees the unquantised hidden row
    "mxfp8_down_unquantised": [("y[c] = (float)mat_row_dot(&ex->down, inter, c, vd);",
                                "y[c] = (float)mat_row_dot(&ex->down, inter, c, v);")],
    # MXFP8: the up projection sees the unquantised norm row
    "mxfp8_up_unquantised": [("float uf = (float)mat_row_dot(&ex->up, H, i, vu);",
                              "float uf = (float)mat_row_dot(&ex->up, H, i, v);")],
    # MXFP8: the block maximum taken without the magnitude (negative maxima ignored)
    "mxfp8_signed_max": [("if (fabs(x[i]) > amax) amax = fabs(x[i]);",
                          "if (x[i] > amax) amax = x[i];")],
    # RMSNorm mean over 4 H
    "norm_mean_over_4h": [("double den = sqrt(ss / (double)H + s->eps_norm);",
                           "double den = sqrt(ss / (double)(4 * H) + s->eps_norm);")],
    # post gate without its factor 2
    "post_without_2": [("(float)(2.0 * sigmoid(", "(float)(1.0 * sigmoid(")],
    # routed down outputs rounded to bf16 before the weighted sum
    "routed_y_rounded": [("acc[c] += (double)weights[r * k + j] * (double)y[c];",
                          "acc[c] += (double)weights[r * k + j] * or_bf16_to_f64(or_f32_to_bf16(y[c]));")],
    # an upper clamp on the score sum
    "clamp_upper": [("double cl = fmax((double)sumf, ldexp(1.0, -14));",
                     "double cl = fmin(fmax((double)sumf, ldexp(1.0, -14)), 1.0);")],
    # no epsilon in the RMSNorm
    "norm_no_eps": [("double den = sqrt(ss / (double)H + s->eps_norm);",
                     "double den = sqrt(ss / (double)H);")],
    # no epsilon in the mix RMS
    "mix_no_eps": [("double den = sqrt(ss / (double)n + s->eps_hc);",
                    "double den = sqrt(ss / (double)n);")],
    # Q8_0: the neighbouring block's scale
    "q8_scale_misindexed": [("const double d = or_f16_to_f64(sc[b]);",
                             "const double d = or_f16_to_f64(sc[b ^ 1]);")],
    # MXFP4: nibble order swapped in the dot product
    "fp4_nibbles_swapped": [("unsigned code = (c & 1) ? (w[c / 2] >> 4) : (w[c / 2] & 0xFu);",
                             "unsigned code = (c & 1) ? (w[c / 2] & 0xFu) : (w[c / 2] >> 4);")],
    # ties ordered by descending index
    "ties_index_descending": [("return (a->e > b->e) - (a->e < b->e);",
                               "return (a->e < b->e) - (a->e > b->e);")],
    # no square root on softplus
    "score_without_sqrt": [("sc[e] = (float)sqrt((double)sp);", "sc[e] = sp;")],
    # gate not rounded to bf16 before SwiGLU
    "gate_unrounded": [(
        "double g = (s->act == OR_F32) ? (double)gf : or_bf16_to_f64(or_f32_to_bf16(gf));",
        "double g = (double)gf;")],
    # pre gate reads the post mixes (layout)
    "pre_reads_post_mixes": [("sigmoid(a0 * m[i] + (double)hc_base[i])",
                              "sigmoid(a0 * m[4 + i] + (double)hc_base[i])")],
    # pre gate scaled by the post scale
    "pre_uses_post_scale": [("sigmoid(a0 * m[i] + (double)hc_base[i])",
                             "sigmoid(a1 * m[i] + (double)hc_base[i])")],
    # softplus without the |z| (wrong for negative logits)
    "softplus_signed": [("log1p(exp(-fabs(z)))", "log1p(exp(-z))")],
    # routed scale not applied
    "no_routed_scale": [("weights[r * k + j] = (float)((double)w * s->routed_scale);",
                         "weights[r * k + j] = w;")],
    # carry sum of squares over the input state instead of the new state
    "carry_sumsq_of_input": [(
        "double v = act_get(s->act, new_state, (int64_t)r * n + t);\n        ss += v * v;",
        "double v = act_get(s->act, state, (int64_t)r * n + t);\n        ss += v * v;")],
}


def _mutate(text: str, edits) -> str:
    for old, new in edits:
        n = text.count(old)
        assert n == 1, "replacement target found %d times (oracle.c changed?): %r" % (n, old[:60])
        text = text.replace(old, new)
    return text


def _run_pins(lib_path: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, MONO_ORACLE_LIB=lib_path, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", *PINS],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def outcomes():
    src = open(SRC).read()
    sources = {"unmodified": src}
    for name, edits in MUTANTS.items():
        sources[name] = _mutate(src, edits)
    with tempfile.TemporaryDirectory() as tmp:
        libs = {}
        for name, text in sources.items():
            c = os.path.join(tmp, name + ".c")
            with open(c, "w") as fh:
                fh.write(text)
            # the planted copy keeps oracle.h reachable
            with open(os.path.join(tmp, "oracle.h"), "w") as fh:
                fh.write(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
            libs[name] = os.path.join(tmp, name + ".so")
            oracle.build(c, libs[name])
        workers = max(1, min(6, (os.cpu_count() or 2) - 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            futs = {name: ex.submit(_run_pins, path) for name, path in libs.items()}
            return {name: f.result() for name, f in futs.items()}


def test_unmodified_oracle_passes_every_pin(outcomes):
    r = outcomes["unmodified"]
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, outcomes):
    r = outcomes[name]
    assert r.returncode == 1, "mutant %s passed every pin (rc %d):\n%s" % (
        name, r.returncode, r.stdout[-1500:])
    assert "failed" in r.stdout
