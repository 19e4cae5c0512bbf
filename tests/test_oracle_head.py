"""Oracle pins: the model tail (head mix without a split, pre-weighted collapse, output norm).

Pins: a zero head mix gives pre = sigmoid(b) (textbook sigmoid in the test); one-hot head rows
over a row of +-1 values give m = +-1 / sqrt(1 + eps_hc) exactly; four equal streams reduce the
collapse to one scaled row; the head with the first four rows of a layer's mix, its first scale
and first four biases reproduces the pre weights, x and norm of the pinned mix -> split ->
collapse chain bit for bit; permuting the streams together with the head's rows and column
blocks permutes pre and leaves x and norm unchanged.
"""

import math

import numpy as np
import pytest

import oracle
import synth


def shape(rows=2, hidden=64, act="bf16"):
    return oracle.make_shape(rows, hidden, 8, 2, 32, 32, act, 1.0)


def bf(x: float) -> int:
    return oracle.f32_to_bf16(float(np.float32(x)))


def bf_rows(a):
    return np.array([[bf(v) for v in row] for row in np.asarray(a, np.float64).reshape(len(a), -1)],
                    np.uint16)


def sig(z: float) -> float:
    return 1.0 / (1.0 + math.exp(-z))


def as64(a, act="bf16"):
    if act == "f32":
        return np.asarray(a, np.float64)
    return np.array([oracle.bf16_to_f64(int(v)) for v in np.asarray(a).ravel()]).reshape(np.shape(a))


def test_zero_head_mix_gives_sigmoid_of_the_biases():
    s = shape()
    rng = np.random.default_rng(1)
    st = bf_rows(rng.standard_normal((2, 4 * 64))).reshape(2, 4, 64)
    b = np.array([-1.5, -0.25, 0.5, 2.0], np.float32)
    pre, _, _ = oracle.head(s, st, np.zeros((4, 256), np.float32), np.array([0.3], np.float32),
                            b, bf_rows(np.ones((1, 64)))[0])
    for r in range(2):
        assert pre[r].tolist() == [float(np.float32(sig(float(v)))) for v in b]


@pytest.mark.parametrize("a", [0.12, 1.0])
def test_one_hot_head_rows_over_a_unit_row(a):
    """Every state value is +-1, so mean(s^2) = 1 and m_i = s[t_i] / sqrt(1 + eps_hc)."""
    s = shape(rows=1)
    rng = np.random.default_rng(2)
    vals = rng.choice([-1.0, 1.0], size=4 * 64)
    st = bf_rows(vals[None]).reshape(1, 4, 64)
    ts = [3, 70, 129, 255]
    W = np.zeros((4, 256), np.float32)
    for i, t in enumerate(ts):
        W[i, t] = 1.0
    b = np.array([0.1, -0.2, 0.3, -0.4], np.float32)
    pre, _, _ = oracle.head(s, st, W, np.array([a], np.float32), b, bf_rows(np.ones((1, 64)))[0])
    den = math.sqrt(1.0 + s.eps_hc)
    want = [float(np.float32(sig(a * float(np.float32(vals[t] / den)) + float(b[i]))))
            for i, t in enumerate(ts)]
    assert pre[0].tolist() == want


def test_equal_streams_collapse_to_one_scaled_row():
    s = shape(rows=1, hidden=128)
    rng = np.random.default_rng(3)
    s0 = bf_rows(rng.standard_normal((1, 128)))[0]
    st = np.stack([s0] * 4)[None]
    W = (rng.standard_normal((4, 512)) * 0.02).astype(np.float32)
    pre, x, _ = oracle.head(s, st, W, np.array([0.12], np.float32),
                            np.array([0.0, 0.5, -0.5, 1.0], np.float32),
                            bf_rows(np.ones((1, 128)))[0])
    tot = math.fsum(float(p) for p in pre[0])
    want = [bf(float(np.float32(tot * oracle.bf16_to_f64(int(v))))) for v in s0]
    assert x[0].tolist() == want


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_head_with_a_layers_pre_rows_matches_the_mix_split_collapse_chain(act):
    cfg = synth.CONFIGS[1].with_(rows=3, act=act) if act == "f32" else \
        synth.CONFIGS[2].with_(rows=3, hidden=512)
    s = oracle.shape_of(cfg)
    d = synth.dense_host(cfg, 0)
    st = synth.state_host(cfg, 0)
    m = oracle.mix(s, st, d["w_mix"])
    pre_c, _, _ = oracle.split(s, m, d["hc_scale"], d["hc_base"])
    x_c, n_c = oracle.collapse_norm(s, st, pre_c, d["w_norm"])
    pre, x, n = oracle.head(s, st, np.ascontiguousarray(d["w_mix"][:4]), d["hc_scale"][:1],
                            d["hc_base"][:4].copy(), d["w_norm"])
    assert np.array_equal(pre, pre_c)
    assert np.array_equal(x, x_c) and np.array_equal(n, n_c)


def test_stream_permutation_permutes_pre_only():
    cfg = synth.CONFIGS[2].with_(rows=2, hidden=256)
    s = oracle.shape_of(cfg)
    st = synth.state_host(cfg, 1)
    h = synth.head_host(cfg)
    H = cfg.hidden
    perm = [2, 0, 3, 1]
    st_p = st[:, perm, :].copy()
    Wb = h["w_head"].reshape(4, 4, H)                  # [row i][stream][h]
    W_p = Wb[perm][:, perm, :].reshape(4, 4 * H).copy()
    b_p = h["head_base"][perm].copy()
    pre, x, n = oracle.head(s, st, h["w_head"], h["head_scale"], h["head_base"], h["w_norm"])
    pre_p, x_p, n_p = oracle.head(s, st_p, W_p, h["head_scale"], b_p, h["w_norm"])
    np.testing.assert_allclose(pre_p, pre[:, perm], rtol=2e-7, atol=0)
    # x is a sum of four products: a permuted f64 order may differ in the last f64 bit only,
    # which can move a bf16 rounding only at an exact tie
    assert np.mean(x_p == x) > 0.999 and np.mean(n_p == n) > 0.999
