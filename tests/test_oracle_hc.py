"""Oracle pins: mHC mix, split/Sinkhorn, collapse + weighted RMSNorm, expand, carry.

Pins (none retypes the oracle's formula): closed forms for degenerate inputs,
Sinkhorn's theorem (a positive matrix has one doubly-stochastic scaling, found
here by a different algorithm), invariances (scale, permutation, linearity),
conservation of the stream sum through the expand, and the carry identity.
"""

import numpy as np
import pytest

import oracle
import synth


def bf(a):
    return (np.asarray(a, np.uint32) << 16).view(np.float32)


def to_bf(x):
    return np.array([oracle.f32_to_bf16(float(v)) for v in np.ravel(x)], np.uint16).reshape(
        np.shape(x))


def small_shape(rows=2, hidden=64, act="f32"):
    return oracle.make_shape(rows, hidden, 8, 2, 32, 32, act, 1.0)


# ------------------------------------------------------------------------------------------ mix

def test_mix_zero_weights_give_zero():
    s = small_shape()
    st = np.random.default_rng(0).standard_normal((2, 4, 64)).astype(np.float32)
    assert np.all(oracle.mix(s, st, np.zeros((24, 256), np.float32)) == 0)


def test_mix_constant_row_closed_form():
    s = small_shape(rows=1)
    c = -1.75
    st = np.full((1, 4, 64), c, np.float32)
    W = np.random.default_rng(1).standard_normal((24, 256)).astype(np.float32)
    got = oracle.mix(s, st, W)[0]
    # s = c * 1, mean(s^2) = c^2: mixes[j] = c * sum(W[j]) / sqrt(c^2 + eps)
    want = np.array([c * sum(map(float, W[j])) / np.sqrt(c * c + 1e-6) for j in range(24)])
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-6)


def test_mix_is_scale_invariant_and_linear_in_w():
    rng = np.random.default_rng(2)
    s = small_shape(rows=1)
    st = rng.standard_normal((1, 4, 64)).astype(np.float32)
    W1 = rng.standard_normal((24, 256)).astype(np.float32)
    W2 = rng.standard_normal((24, 256)).astype(np.float32)
    m = oracle.mix(s, st, W1)
    np.testing.assert_allclose(oracle.mix(s, (st * 8).astype(np.float32), W1), m, rtol=1e-6,
                               atol=1e-6)
    np.testing.assert_allclose(oracle.mix(s, st, W1 + W2),
                               oracle.mix(s, st, W1) + oracle.mix(s, st, W2), rtol=1e-5,
                               atol=1e-5)


def test_mix_permutation_invariance():
    rng = np.random.default_rng(3)
    s = small_shape(rows=1)
    st = rng.standard_normal((1, 4, 64)).astype(np.float32)
    W = rng.standard_normal((24, 256)).astype(np.float32)
    p = rng.permutation(256)
    m1 = oracle.mix(s, st, W)
    m2 = oracle.mix(s, np.ascontiguousarray(st.reshape(1, 256)[:, p]).reshape(1, 4, 64),
                    np.ascontiguousarray(W[:, p]))
    np.testing.assert_allclose(m1, m2, rtol=1e-6, atol=1e-6)


def test_mix_normalise_first_form_in_f64():
    # the same quantity computed as W @ (s / rms(s)) with numpy's BLAS dot
    rng = np.random.default_rng(4)
    s = small_shape(rows=2, hidden=256, act="bf16")
    st = to_bf(rng.standard_normal((2, 4, 256)))
    W = (rng.standard_normal((24, 1024)) * 0.02).astype(np.float32)
    got = oracle.mix(s, st, W)
    for r in range(2):
        v = bf(st[r]).ravel().astype(np.float64)
        rms = np.linalg.norm(v) / np.sqrt(v.size)
        v = v / np.sqrt(rms * rms + 1e-6)
        np.testing.assert_allclose(got[r], W.astype(np.float64) @ v, rtol=1e-6, atol=1e-7)


# -------------------------------------------------------------------------------- split/Sinkhorn

def sinkhorn_by_scaling(A, iters=20000):
    """Doubly-stochastic scaling D1 A D2 found by fixed-point iteration on the scaling vectors
    in the log domain (a different algorithm from the oracle's alternating normalisation)."""
    la = np.log(A)
    u = np.zeros(4)
    v = np.zeros(4)
    for _ in range(iters):
        u = -np.log(np.exp(la + v[None, :]).sum(1))
        v = -np.log(np.exp(la + u[:, None]).sum(0))
    return np.exp(la + u[:, None] + v[None, :])


def test_split_closed_forms_at_zero():
    s = small_shape(rows=1)
    m = np.zeros((1, 24), np.float32)
    pre, post, comb = oracle.split(s, m, np.array([0.12, 0.08, 0.1], np.float32),
                                   np.zeros(24, np.float32))
    assert np.all(pre == 0.5) and np.all(post == 1.0)
    assert np.all(comb == 0.25)      # constant logits: uniform doubly-stochastic matrix


def test_split_sigmoid_values():
    s = small_shape(rows=1)
    rng = np.random.default_rng(5)
    m = rng.standard_normal((1, 24)).astype(np.float32) * 3
    a = np.array([0.12, 0.08, 0.1], np.float32)
    b = rng.uniform(-1, 1, 24).astype(np.float32)
    pre, post, _ = oracle.split(s, m, a, b)
    from scipy.special import expit
    np.testing.assert_allclose(pre[0], expit(a[0].astype(np.float64) * m[0, :4] + b[:4]),
                               rtol=1e-7)
    np.testing.assert_allclose(post[0], 2 * expit(a[1].astype(np.float64) * m[0, 4:8] + b[4:8]),
                               rtol=1e-7)


def test_sinkhorn_matches_unique_scaling():
    s = small_shape(rows=1)
    rng = np.random.default_rng(6)
    a = np.array([0.12, 0.08, 0.1], np.float32)
    worst = 0.0
    for _ in range(40):
        m = (rng.standard_normal((1, 24)) * 3).astype(np.float32)
        b = rng.uniform(-1, 1, 24).astype(np.float32)
        _, _, comb = oracle.split(s, m, a, b)
        L = a[2].astype(np.float64) * m[0, 8:].astype(np.float64) + b[8:]
        ref = sinkhorn_by_scaling(np.exp(L.reshape(4, 4)))
        worst = max(worst, np.abs(comb[0] - ref).max())
    assert worst < 1e-6


def test_sinkhorn_permutation_equivariance():
    s = small_shape(rows=1)
    rng = np.random.default_rng(7)
    a = np.array([0.12, 0.08, 0.1], np.float32)
    m = (rng.standard_normal((1, 24)) * 3).astype(np.float32)
    b = np.zeros(24, np.float32)
    _, _, c1 = oracle.split(s, m, a, b)
    p = [2, 0, 3, 1]
    m2 = m.copy()
    m2[0, 8:] = m[0, 8:].reshape(4, 4)[p].ravel()
    _, _, c2 = oracle.split(s, m2, a, b)
    np.testing.assert_allclose(c2[0], c1[0][p], atol=2e-7)


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_sinkhorn_invariant_on_workload_rows(ci):
    cfg = synth.CONFIGS[ci]
    s = oracle.shape_of(cfg)
    d = synth.dense_host(cfg, 0)
    for sample in range(4):
        st = synth.state_host(cfg, sample)
        m = oracle.mix(s, st, d["w_mix"])
        _, _, comb = oracle.split(s, m, d["hc_scale"], d["hc_base"])
        assert np.abs(comb.sum(2) - 1).max() <= 1e-6
        assert np.abs(comb.sum(1) - 1).max() <= 1e-6


# ---------------------------------------------------------------------------- collapse + norm

def test_collapse_identical_streams():
    s = small_shape(rows=1, act="f32")
    v = np.random.default_rng(8).standard_normal(64).astype(np.float32)
    st = np.stack([v] * 4)[None]
    pre = np.array([[0.25, 0.5, 0.125, 0.0625]], np.float32)   # exact sum 0.9375
    x, _ = oracle.collapse_norm(s, st, pre, np.ones(64, np.float32))
    np.testing.assert_array_equal(x[0], (v.astype(np.float64) * 0.9375).astype(np.float32))


def test_norm_constant_row_closed_form():
    s = small_shape(rows=1, act="bf16")
    st = to_bf(np.full((1, 4, 64), 0.5))
    pre = np.array([[1.0, 0.0, 0.0, 0.0]], np.float32)
    w = to_bf(np.linspace(0.5, 1.5, 64))
    x, norm = oracle.collapse_norm(s, st, pre, w)
    assert np.all(bf(x) == 0.5)
    want = to_bf(0.5 / np.sqrt(0.25 + 1e-6) * bf(w).astype(np.float64))
    np.testing.assert_array_equal(norm[0], want)


def test_norm_has_unit_rms_over_weight():
    s = small_shape(rows=1, act="f32")
    rng = np.random.default_rng(9)
    st = rng.standard_normal((1, 4, 64)).astype(np.float32) * 5
    pre = np.array([[0.3, 0.6, 0.2, 0.9]], np.float32)
    w = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    _, norm = oracle.collapse_norm(s, st, pre, w)
    r = norm[0].astype(np.float64) / w
    assert abs(np.sqrt((r * r).mean()) - 1) < 1e-6


# ------------------------------------------------------------------------------ expand + carry

def test_expand_identity_comb_zero_post_returns_state():
    s = small_shape(rows=2, act="bf16")
    st = to_bf(np.random.default_rng(10).standard_normal((2, 4, 64)))
    block = to_bf(np.random.default_rng(11).standard_normal((2, 64)))
    comb = np.tile(np.eye(4, dtype=np.float32), (2, 1, 1))
    new, _ = oracle.expand(s, st, block, np.zeros((2, 4), np.float32), comb)
    np.testing.assert_array_equal(new, st)


def test_expand_permutation_comb_moves_streams():
    # comb as a permutation matrix (comb[i][perm[i]] = 1): new_i = state_perm[i] (the reading
    # new_i = sum_j comb_ij * state_j); the 4-cycle is not symmetric, so comb^T would fail
    s = small_shape(rows=2, act="bf16")
    st = to_bf(np.random.default_rng(13).standard_normal((2, 4, 64)))
    block = to_bf(np.random.default_rng(14).standard_normal((2, 64)))
    perm = [1, 2, 3, 0]
    comb = np.zeros((2, 4, 4), np.float32)
    for i, j in enumerate(perm):
        comb[:, i, j] = 1.0
    new, _ = oracle.expand(s, st, block, np.zeros((2, 4), np.float32), comb)
    np.testing.assert_array_equal(new, st[:, perm, :])


def test_expand_post_adds_scaled_block():
    # identity comb: new_i = bf16(post_i * block + state_i), exact in f64 before the rounding
    s = small_shape(rows=1, act="bf16")
    st = to_bf(np.random.default_rng(15).standard_normal((1, 4, 64)))
    block = to_bf(np.random.default_rng(16).standard_normal((1, 64)))
    post = np.array([[0.5, 1.0, 1.5, 2.0]], np.float32)
    comb = np.eye(4, dtype=np.float32)[None]
    new, _ = oracle.expand(s, st, block, post, comb)
    exp = post[0][:, None].astype(np.float64) * bf(block[0]).astype(np.float64)[None, :] + bf(st[0]).astype(np.float64)
    np.testing.assert_array_equal(new[0], to_bf(exp))


def test_expand_conserves_stream_sum():
    # comb columns sum to 1 => sum_i new_i = sum_j state_j + (sum_i post_i) * block
    cfg = synth.CONFIGS[1]
    s = oracle.shape_of(cfg)
    d = synth.dense_host(cfg, 0)
    st = synth.state_host(cfg, 3)
    m = oracle.mix(s, st, d["w_mix"])
    _, post, comb = oracle.split(s, m, d["hc_scale"], d["hc_base"])
    block = np.random.default_rng(12).standard_normal((1, cfg.hidden)).astype(np.float32)
    new, _ = oracle.expand(s, st, block, post, comb)
    lhs = new[0].astype(np.float64).sum(0)
    rhs = st[0].astype(np.float64).sum(0) + post[0].astype(np.float64).sum() * block[0]
    np.testing.assert_allclose(lhs, rhs, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("ci", [1, 2])
def test_carry_identity(ci):
    # mixes from the carry equal the mixes computed directly from the new state
    cfg = synth.CONFIGS[ci]
    s = oracle.shape_of(cfg)
    d0, d1 = synth.dense_host(cfg, 0), synth.dense_host(cfg, 1)
    st = synth.state_host(cfg, 1)
    m = oracle.mix(s, st, d0["w_mix"])
    _, post, comb = oracle.split(s, m, d0["hc_scale"], d0["hc_base"])
    block = synth.state_host(cfg, 2)[:, 0, :].copy()
    new, carry = oracle.expand(s, st, block, post, comb, d1["w_mix"])
    direct = oracle.mix(s, new, d1["w_mix"])
    via = oracle.mix(s, None, None, carry)
    np.testing.assert_allclose(via, direct, rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------- hand-derived fixtures (golden)

GOLDEN = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(__import__("os").path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split(":", 1)
                yield k.strip(), v.split()


@pytest.mark.parametrize("iters", [0, 1, 2])
def test_sinkhorn_steps_match_hand_derivation(iters):
    """tests/golden/sinkhorn_steps.txt: 0, 1 and 2 row-then-column normalisations of a fixed
    4x4 matrix, worked out by hand in exact fractions. Pins the step order (columns first
    would give the transpose) and the iteration count."""
    from fractions import Fraction
    want = {int(k): np.array([float(Fraction(f)) for f in v]).reshape(4, 4)
            for k, v in _golden_lines("sinkhorn_steps.txt")}[iters]
    A = np.ones((4, 4))
    A[0, 0] = 2.0
    base = np.zeros(24, np.float32)
    base[8:] = np.log(A).astype(np.float32).ravel()
    s = oracle.make_shape(1, 64, 8, 2, 32, 32, "f32", 1.0, sinkhorn_iters=iters)
    _, _, comb = oracle.split(s, np.zeros((1, 24), np.float32), np.zeros(3, np.float32), base)
    # f32 comb against the exact fractions: the log 2 input carries ~2e-9 relative error
    np.testing.assert_allclose(comb[0], want, rtol=2e-7, atol=0)


def test_collapse_pairs_gate_i_with_stream_i():
    """tests/golden/collapse_pairing.txt: four distinct streams c_i (h + 1) and distinct
    power-of-two gates; x = 2 (h + 1) exactly (any other pairing of gates and streams gives
    another multiple)."""
    g = dict(_golden_lines("collapse_pairing.txt"))
    pre = np.array([[float(v) for v in g["pre"]]], np.float32)
    c = [float(v) for v in g["c"]]
    mult = float(g["x_over_h_plus_1"][0])
    H = 32
    s = oracle.make_shape(1, H, 8, 2, 32, 32, "bf16", 1.0)
    st = to_bf(np.array([[[ci * (h + 1) for h in range(H)] for ci in c]]))
    x, _ = oracle.collapse_norm(s, st, pre, to_bf(np.ones(H)))
    np.testing.assert_array_equal(bf(x[0]), mult * (np.arange(H) + 1.0))


def test_norm_depends_on_x_only_through_its_bf16_value():
    """The RMSNorm reads the stored (bf16-rounded) x: collapsing a row whose sum rounds
    (x = bf16(v + 0.0035 v)) and collapsing the already rounded x with pre = (1, 0, 0, 0)
    give the same x and therefore the same norm, bit for bit. A mean of squares taken over
    the unrounded sums would differ by about 0.3 % and flip many norm outputs."""
    H = 1024
    s = oracle.make_shape(1, H, 8, 2, 32, 32, "bf16", 1.0)
    rng = np.random.default_rng(21)
    v = to_bf(rng.standard_normal(H))
    w = to_bf(rng.uniform(0.5, 1.5, H))
    zero = np.zeros(H, np.uint16)
    st_a = np.stack([v, v, zero, zero])[None]
    x_a, norm_a = oracle.collapse_norm(s, st_a, np.array([[1.0, 0.0035, 0.0, 0.0]], np.float32), w)
    assert np.mean(x_a[0] != v) > 0.3          # the sums really round
    st_b = np.stack([x_a[0], zero, zero, zero])[None]
    x_b, norm_b = oracle.collapse_norm(s, st_b, np.array([[1.0, 0.0, 0.0, 0.0]], np.float32), w)
    np.testing.assert_array_equal(x_b, x_a)
    np.testing.assert_array_equal(norm_b, norm_a)


def test_epsilons_closed_form_on_tiny_rows():
    """A constant row c = 2^-10 (c^2 ~ 0.95e-6, the size of the epsilons): the mix and the
    RMSNorm both divide by sqrt(c^2 + 1e-6), about 0.7 of what they would without epsilon."""
    c = 2.0 ** -10
    s = small_shape(rows=1, act="bf16")
    st = to_bf(np.full((1, 4, 64), c))
    W = np.random.default_rng(22).standard_normal((24, 256)).astype(np.float32)
    got = oracle.mix(s, st, W)[0]
    want = np.array([c * sum(map(float, W[j])) / np.sqrt(c * c + 1e-6) for j in range(24)])
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-9)
    x, norm = oracle.collapse_norm(s, st, np.array([[1.0, 0.0, 0.0, 0.0]], np.float32),
                                   to_bf(np.ones(64)))
    assert np.all(bf(x) == c)
    assert np.all(norm == to_bf(c / np.sqrt(c * c + 1e-6)))   # 0.6987 -> bf16 0x3F33
