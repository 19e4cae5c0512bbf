"""Pins of the oracle's MXFP8 activation mode for MXFP4 experts (the GLM-5 page, "[ROCm][Perf]
[GLM-5] Fused sparse-layer decode via AITER MonoKernel", Details / Numerics: activations entering
the MXFP4 experts are quantised to MXFP8). The conversion is the OCP MX v1.0 one (READING):
shared exponent floor(log2 max|v|) - 8, E4M3 elements rounded to nearest even and clamped to 448.

Pinned against: the OFP8 table of E4M3 values (golden fixture), the structure of the format
(monotone codes, constant spacing per binade), a brute-force nearest-value search over every
finite E4M3 number, the scale rule's closed form, and the identity that the mode equals the plain
oracle run on the round-tripped activations, for the MXFP4 matrices only.
"""

import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_codes.txt")


def _golden():
    out = {}
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        c, v = line.split()
        out[int(c, 16)] = float(v)
    return out


def test_e4m3_decode_matches_ofp8_table():
    for c, v in _golden().items():
        got = oracle.e4m3_to_f64(c)
        if math.isnan(v):
            assert math.isnan(got), hex(c)
        else:
            assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), hex(c)


def test_e4m3_codes_are_monotone_with_binade_spacing():
    vals = [oracle.e4m3_to_f64(c) for c in range(0x7F)]  # 0x00 .. 0x7E, all finite
    assert all(b > a for a, b in zip(vals, vals[1:]))
    for c in range(1, 0x7F):
        e = (c - 1) >> 3  # spacing of the binade of the lower neighbour
        step = 2.0 ** -9 if e <= 1 else 2.0 ** (e - 7 - 3)
        assert vals[c] - vals[c - 1] == step, hex(c)
    for c in range(0x7F):
        assert oracle.e4m3_to_f64(0x80 | c) == -vals[c]


def _finite_e4m3():
    return np.array([oracle.e4m3_to_f64(c) for c in range(0x7F)])


def _brute_force(block):
    """Nearest finite E4M3 value of v / 2^X for every v (ties to the even code, magnitudes
    beyond 448 to 448), X from the block maximum; returns the dequantised values and X."""
    mags = _finite_e4m3()
    amax = max(abs(float(v)) for v in block)
    if amax == 0.0:
        return np.zeros(len(block)), -127
    X = min(127, max(-127, math.frexp(amax)[1] - 1 - 8))
    out = []
    for v in block:
        t = abs(float(v)) / 2.0 ** X
        d = np.abs(mags - t)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(math.copysign(mags[c], float(v)) * 2.0 ** X)
    return np.array(out), X


def _round_trip(v):
    codes, scales = oracle.mxfp8_quant(v)
    deq = np.array([oracle.e4m3_to_f64(int(c)) for c in codes])
    sc = np.repeat([oracle.e8m0_to_f64(int(s)) for s in scales], 32)
    return deq * sc, codes, scales


def _blocks():
    rng = np.random.default_rng(7)
    mags = _finite_e4m3()
    out = [rng.normal(0, 1, 32), rng.normal(0, 1e-3, 32) * rng.uniform(0.1, 10, 32),
           rng.uniform(-3, 3, 32), np.zeros(32)]
    # exact ties: midpoints between neighbouring E4M3 numbers under scale 2^-8 (max 1.0)
    t = np.zeros(32)
    t[0] = 1.0
    for i in range(1, 32):
        c = 8 + 3 * i
        t[i] = (mags[c] + mags[c + 1]) / 2 * 2.0 ** -8 * (1 if i % 2 else -1)
    out.append(t)
    # saturation: the maximum sits between 448 and 512 times the scale
    s = rng.normal(0, 0.3, 32)
    s[5] = 1.95
    s[9] = -1.8
    out.append(s)
    # subnormal elements next to a large one
    u = np.full(32, 3e-5)
    u[0] = 4.0
    u[1::3] = -7e-5
    out.append(u)
    # amax exactly a power of two, negative
    p = rng.uniform(-0.2, 0.2, 32)
    p[11] = -0.25
    out.append(p)
    return out


@pytest.mark.parametrize("bi", range(8))
def test_quantiser_equals_brute_force_nearest(bi):
    block = _blocks()[bi]
    rt, codes, scales = _round_trip(block)
    want, X = _brute_force(block)
    assert int(scales[0]) == X + 127
    np.testing.assert_array_equal(rt, want)


def test_scale_closed_form():
    for amax, code in [(1.0, 119), (3.0, 120), (0.75, 118), (-2.0, 120), (2.0 ** -20, 99)]:
        v = np.zeros(32)
        v[3] = amax
        _, _, scales = _round_trip(v)
        assert int(scales[0]) == code, amax
    # the largest element lands in [256, 448] after scaling
    rng = np.random.default_rng(3)
    for _ in range(50):
        v = rng.normal(0, rng.uniform(1e-4, 1e2), 32)
        rt, codes, scales = _round_trip(v)
        top = np.abs(rt).max() / oracle.e8m0_to_f64(int(scales[0]))
        assert 256.0 <= top <= 448.0


def test_round_trip_error_bound():
    """Relative error at most half an E4M3 ulp (2^-4) for elements that neither saturate nor
    fall into the subnormal range."""
    rng = np.random.default_rng(11)
    v = rng.normal(0, 1, 32 * 64)
    rt, codes, scales = _round_trip(v)
    sc = np.repeat([oracle.e8m0_to_f64(int(s)) for s in scales], 32)
    t = np.abs(v) / sc
    ok = (t >= 2.0 ** -6) & (t <= 448.0)
    assert ok.sum() > 1500
    assert np.all(np.abs(rt - v)[ok] <= 2.0 ** -4 * np.abs(v)[ok])


def _small(fmt_r, fmt_s):
    return synth.CONFIGS[4].with_(rows=1, hidden=256, n_experts=4, top_k=2, inter=64,
                                  shared_inter=64, routed_fmt=fmt_r, shared_fmt=fmt_s,
                                  grouped_bias=False, zero_rows=())


def _bf16_of(values):
    b = np.array([oracle.f32_to_bf16(float(x)) for x in values], np.uint16)
    back = np.array([oracle.bf16_to_f64(int(x)) for x in b])
    return b, back


@pytest.mark.parametrize("fmt", ["mxfp4", "bf16"])
def test_gate_up_see_round_tripped_norm_for_mxfp4_only(fmt):
    cfg = _small(fmt, "bf16")
    s0 = oracle.shape_of(cfg)
    s8 = oracle.shape_of(cfg.with_(act_quant="mxfp8"))
    ex = synth.expert_host(cfg, 0, 1)
    norm = synth.state_host(cfg, 0)[0, 0, :].copy()  # a bf16 row
    h8 = oracle.expert_hidden(s8, cfg.inter, fmt, ex, norm)
    if fmt == "bf16":
        np.testing.assert_array_equal(h8, oracle.expert_hidden(s0, cfg.inter, fmt, ex, norm))
        return
    vals = np.array([oracle.bf16_to_f64(int(x)) for x in norm])
    rt, _, _ = _round_trip(vals)
    b, back = _bf16_of(rt)
    np.testing.assert_array_equal(back, rt)  # the round trip is exact in bf16
    np.testing.assert_array_equal(h8, oracle.expert_hidden(s0, cfg.inter, fmt, ex, b))
    assert not np.array_equal(h8, oracle.expert_hidden(s0, cfg.inter, fmt, ex, norm))


def test_down_sees_round_tripped_hidden_row():
    cfg = _small("mxfp4", "mxfp4")
    s0 = oracle.shape_of(cfg)
    s8 = oracle.shape_of(cfg.with_(act_quant="mxfp8"))
    R, k, I, Is = 1, cfg.top_k, cfg.inter, cfg.shared_inter
    idx = np.array([[1, 3]], np.int32)
    w = np.array([[1.5, 1.0]], np.float32)
    routed = {e: synth.expert_host(cfg, 0, e) for e in (1, 3)}
    shared = synth.expert_host(cfg, 0, None)
    rng = np.random.default_rng(5)
    hr_v = rng.normal(0, 0.05, (R, k, I))
    hs_v = rng.normal(0, 0.05, (R, Is))
    hr, _ = _bf16_of(hr_v.ravel())
    hs, _ = _bf16_of(hs_v.ravel())
    m8 = oracle.moe(s8, None, idx, w, "mxfp4", routed, "mxfp4", shared, hr, hs)
    hr_rt = np.concatenate([_round_trip(np.array([oracle.bf16_to_f64(int(x)) for x in
                                                  hr[j * I:(j + 1) * I]]))[0] for j in range(k)])
    hs_rt = _round_trip(np.array([oracle.bf16_to_f64(int(x)) for x in hs]))[0]
    m0 = oracle.moe(s0, None, idx, w, "mxfp4", routed, "mxfp4", shared, _bf16_of(hr_rt)[0],
                    _bf16_of(hs_rt)[0])
    for t in ("routed", "shared", "block"):
        np.testing.assert_array_equal(m8[t], m0[t])
    plain = oracle.moe(s0, None, idx, w, "mxfp4", routed, "mxfp4", shared, hr, hs)
    assert not np.array_equal(m8["routed"], plain["routed"])


def test_representable_activations_pass_unchanged():
    """A norm row whose blocks are already E4M3 values under the scale the rule picks gives the
    same hidden row with and without the mode."""
    cfg = _small("mxfp4", "bf16")
    rng = np.random.default_rng(9)
    mags = _finite_e4m3()
    vals = []
    for b in range(cfg.hidden // 32):
        X = int(rng.integers(-14, -4))
        blk = rng.choice(mags[:0x7E], 32) * rng.choice([-1.0, 1.0], 32)
        blk[int(rng.integers(32))] = 320.0  # block maximum in [256, 448]
        vals.extend(blk * 2.0 ** X)
    norm, back = _bf16_of(vals)
    np.testing.assert_array_equal(back, vals)
    ex = synth.expert_host(cfg, 0, 2)
    s0 = oracle.shape_of(cfg)
    s8 = oracle.shape_of(cfg.with_(act_quant="mxfp8"))
    np.testing.assert_array_equal(oracle.expert_hidden(s8, cfg.inter, "mxfp4", ex, norm),
                                  oracle.expert_hidden(s0, cfg.inter, "mxfp4", ex, norm))
