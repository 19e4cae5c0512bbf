"""Oracle pins: router logits and the canonical top-k select.

Pins: an exactly rounded reference sum (math.fsum) for the logits, brute-force
sorting for the selection on tiny inputs with random and crafted ties, the
hand-derived tie cases of tests/golden/topk_ties.txt, softplus closed forms,
the weight invariant sum(w) = rho, and the closed form of the all-zero row with
a grouped bias.
"""

import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def shape(E, k, rho=1.0, rows=1, hidden=32):
    return oracle.make_shape(rows, hidden, E, k, 32, 32, "f32", rho)


def test_logits_match_exactly_rounded_sum():
    rng = np.random.default_rng(0)
    s = oracle.make_shape(2, 256, 16, 4, 32, 32, "f32", 1.0)
    norm = rng.standard_normal((2, 256)).astype(np.float32)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    lg = oracle.router_logits(s, norm, W)
    for r in range(2):
        for e in range(16):
            ref = math.fsum(float(W[e, h]) * float(norm[r, h]) for h in range(256))
            assert lg[r, e] == np.float32(ref) or abs(lg[r, e] - ref) <= 1e-7 * abs(ref) + 1e-12


def _scores(logits, bias):
    """Independent f64 recomputation of s and beta from the definition."""
    s = []
    for z in logits:
        z = float(z)
        sp = np.float32(math.log(1.0 + math.exp(z)) if z < 30 else z + math.log1p(math.exp(-z)))
        s.append(np.float32(math.sqrt(float(sp))))
    beta = [np.float32(float(a) + float(b)) for a, b in zip(s, bias)]
    return s, beta


# 30 random small shapes, then the draft routing shapes (128 experts top-3, 256 top-6)
SELECT_CASES = [(seed, None, None) for seed in range(30)] + [
    (100 + i, E, k) for i, (E, k) in enumerate([(128, 3), (128, 3), (128, 3), (256, 6),
                                                (256, 6), (256, 6)])]


@pytest.mark.parametrize("seed,E,k", SELECT_CASES)
def test_select_matches_brute_force_sort(seed, E, k):
    rng = np.random.default_rng(seed)
    if E is None:
        E = int(rng.integers(2, 17))
        k = int(rng.integers(1, E + 1))
    rho = float(rng.choice([1.0, 2.5]))
    s = shape(E, k, rho)
    mode = seed % 3
    if mode == 0:
        logits = rng.standard_normal(E).astype(np.float32)
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    elif mode == 1:   # crafted ties: repeated logits and biases in interleaved groups
        logits = rng.choice([-1.0, 0.0, 0.5], E).astype(np.float32)
        bias = rng.choice([0.0, 0.05], E).astype(np.float32)
    else:             # all equal: order must be ascending index
        logits = np.full(E, 0.25, np.float32)
        bias = np.zeros(E, np.float32)
    idx, w, _ = oracle.select(s, logits[None], bias)
    sc, beta = _scores(logits, bias)
    order = sorted(range(E), key=lambda e: (-float(beta[e]), e))
    assert idx[0].tolist() == order[:k]
    tot = np.float32(math.fsum(float(sc[e]) for e in order[:k]))
    c = max(float(tot), 2.0 ** -14)
    want = [np.float32(float(np.float32(float(sc[e]) / c)) * rho) for e in order[:k]]
    np.testing.assert_allclose(w[0], np.array(want, np.float32), rtol=1e-6)
    assert abs(float(w[0].astype(np.float64).sum()) - rho) <= 1e-6 * rho


def test_golden_tie_cases():
    n = 0
    for line in open(os.path.join(GOLDEN, "topk_ties.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        head, bias, want = [p.split() for p in line.split("|")]
        E, k, rho = int(head[0]), int(head[1]), float(head[2])
        bias = np.array([float(b) for b in bias], np.float32)
        idx, w, _ = oracle.select(shape(E, k, rho), np.zeros((1, E), np.float32), bias)
        assert idx[0].tolist() == [int(x) for x in want], line
        # equal unbiased scores: every weight is rho / k (to f32 rounding of the division)
        np.testing.assert_allclose(w[0], rho / k, rtol=2e-7)
        n += 1
    assert n >= 6


def test_softplus_closed_forms():
    s = shape(3, 3)
    logits = np.array([[0.0, 100.0, -100.0]], np.float32)
    idx, w, beta = oracle.select(s, logits, np.zeros(3, np.float32))
    assert idx[0].tolist() == [1, 0, 2]
    assert beta[0, 0] == np.float32(10.0)                         # sqrt(softplus(100)) = 10
    assert beta[0, 1] == np.float32(math.sqrt(np.float32(math.log(2.0))))   # softplus(0) = ln 2
    assert 0 < beta[0, 2] < 1e-20                                  # sqrt(e^-100)


def test_bias_steers_selection_only():
    rng = np.random.default_rng(3)
    s = shape(12, 4, 2.5)
    logits = rng.standard_normal((1, 12)).astype(np.float32)
    b1 = np.zeros(12, np.float32)
    i1, w1, _ = oracle.select(s, logits, b1)
    b2 = np.zeros(12, np.float32)
    b2[i1[0]] = 0.01          # raises the selected ones: same selection, same weights
    i2, w2, _ = oracle.select(s, logits, b2)
    assert i1.tolist() == i2.tolist() and w1.tolist() == w2.tolist()


def test_zero_row_grouped_bias_closed_form():
    # workload 4: bias constant over groups of 32; the all-zero row ties inside groups, so the
    # selection is the 8 smallest indices of the best group, ascending, each weight rho / 8
    cfg = synth.CONFIGS[4]
    s = oracle.shape_of(cfg, rows=1)
    d = synth.dense_host(cfg, 0)
    idx, w, _ = oracle.select(s, np.zeros((1, cfg.n_experts), np.float32), d["bias"])
    g = int(np.argmax(d["bias"][::32]))
    assert idx[0].tolist() == list(range(32 * g, 32 * g + 8))
    np.testing.assert_allclose(w[0], cfg.routed_scale / 8, rtol=2e-7)


@pytest.mark.parametrize("ci", [2, 3, 4, 6, 7, 8, 9])
def test_weights_sum_to_scale_on_workload_rows(ci):
    cfg = synth.CONFIGS[ci]
    s = oracle.shape_of(cfg)
    d = synth.dense_host(cfg, 0)
    st = synth.state_host(cfg, 0)
    m = oracle.mix(s, st, d["w_mix"])
    pre, _, _ = oracle.split(s, m, d["hc_scale"], d["hc_base"])
    _, norm = oracle.collapse_norm(s, st, pre, d["w_norm"])
    lg = oracle.router_logits(s, norm, d["w_router"])
    idx, w, beta = oracle.select(s, lg, d["bias"])
    assert np.all(np.abs(w.astype(np.float64).sum(1) - cfg.routed_scale)
                  <= 1e-6 * cfg.routed_scale)
    for r in range(cfg.rows):
        assert len(set(idx[r].tolist())) == cfg.top_k
        assert np.all(np.diff(beta[r]) <= 0)
