"""Oracle pins: SwiGLU experts with fused dequantisation, routed sum, block.

Pins: dequantise-then-dot with an independent numpy decode (numpy's fp16, the
E2M1 bit-field formula, ldexp for E8M0) and BLAS; SwiGLU special cases (zero
gate, identity-like experts); linearity of the routed sum in the routed scale;
a single-expert selection reducing to w * y.
"""

import math

import numpy as np
import pytest

import oracle
import synth


def bf(a):
    return (np.asarray(a, np.uint32) << 16).view(np.float32)


def to_bf(x):
    return np.array([oracle.f32_to_bf16(float(v)) for v in np.ravel(x)], np.uint16).reshape(
        np.shape(x))


def dequant(fmt, v, s):
    """Independent decode of a [rows][k] matrix to f64 (numpy's fp16, the E2M1 bit-field
    formula, ldexp for E8M0)."""
    import support
    return support.dequant(fmt, v, s)


def silu(x):
    return x / (1.0 + np.exp(-x))


@pytest.mark.parametrize("fmt", ["f32", "bf16", "q8_0", "mxfp4"])
def test_expert_hidden_is_dequantise_then_dot(fmt):
    act = "f32" if fmt == "f32" else "bf16"
    base = synth.CONFIGS[3] if fmt == "q8_0" else synth.CONFIGS[4] if fmt == "mxfp4" else \
        synth.CONFIGS[2] if fmt == "bf16" else synth.CONFIGS[1]
    cfg = base.with_(hidden=256, inter=64, shared_inter=64, routed_fmt=fmt, act=act)
    t = synth.expert_host(cfg, 0, 5)
    s = oracle.make_shape(1, 256, 8, 2, 64, 64, act, 1.0)
    rng = np.random.default_rng(0)
    xr = rng.standard_normal(256)
    norm = xr.astype(np.float32) if act == "f32" else to_bf(xr)
    nv = norm.astype(np.float64) if act == "f32" else bf(norm).astype(np.float64)
    h = oracle.expert_hidden(s, 64, fmt, t, norm)
    G = dequant(fmt, t["gate"], t.get("gate_s")) @ nv
    U = dequant(fmt, t["up"], t.get("up_s")) @ nv
    if act == "f32":
        g, u = G.astype(np.float32).astype(np.float64), U.astype(np.float32).astype(np.float64)
        want = (silu(g) * u).astype(np.float32)
        np.testing.assert_allclose(h, want, rtol=1e-6, atol=1e-7)
    else:
        g = bf(to_bf(G.astype(np.float32))).astype(np.float64)
        u = bf(to_bf(U.astype(np.float32))).astype(np.float64)
        want = bf(to_bf((silu(g) * u).astype(np.float32)))
        got = bf(h)
        # f64 BLAS order differs from the oracle's sequential sum: allow one bf16 step
        np.testing.assert_allclose(got, want, rtol=2 ** -8, atol=1e-6)
        assert np.mean(got == want) > 0.98


def tiny_expert(H, I, gate, up, down):
    return {"gate": np.ascontiguousarray(gate, np.float32),
            "up": np.ascontiguousarray(up, np.float32),
            "down": np.ascontiguousarray(down, np.float32)}


def test_swiglu_special_cases():
    H = I = 32
    s = oracle.make_shape(1, H, 2, 1, I, I, "f32", 1.0)
    x = np.linspace(-3, 3, H).astype(np.float32)
    eye = np.eye(I, dtype=np.float32)
    # gate = up = down = identity: h = silu(x) * x, y = h
    ex = tiny_expert(H, I, eye, eye, eye)
    h = oracle.expert_hidden(s, I, "f32", ex, x)
    np.testing.assert_allclose(h, silu(x.astype(np.float64)) * x, rtol=1e-6)
    # zero gate: silu(0) = 0, so h = 0
    hz = oracle.expert_hidden(s, I, "f32", tiny_expert(H, I, 0 * eye, eye, eye), x)
    assert np.all(hz == 0)
    # single selected expert with identity down: routed = w * h, block = routed + shared
    m = oracle.moe(s, x[None], np.array([[1]]), np.array([[0.75]], np.float32), "f32",
                   {1: ex}, "f32", tiny_expert(H, I, 0 * eye, eye, eye))
    np.testing.assert_allclose(m["routed"][0], 0.75 * h, rtol=1e-6)
    assert np.all(m["shared"] == 0)
    np.testing.assert_array_equal(m["block"][0], m["routed"][0])


def test_routed_sum_linear_in_scale_and_selection_order_free():
    cfg = synth.CONFIGS[2].with_(hidden=256, inter=64, shared_inter=64)
    s = oracle.shape_of(cfg)
    rng = np.random.default_rng(1)
    norm = to_bf(rng.standard_normal((1, 256)))
    ex = {e: synth.expert_host(cfg, 0, e) for e in (3, 9)}
    sh = synth.expert_host(cfg, 0, None)
    idx = np.array([[3, 9, 0, 0, 0, 0, 0, 0]][:1])[:, :8]
    s2 = oracle.make_shape(1, 256, 256, 2, 64, 64, "bf16", 1.0)
    w = np.array([[0.6, 0.4]], np.float32)
    a = oracle.moe(s2, norm, np.array([[3, 9]]), w, "bf16", ex, "bf16", sh)
    b = oracle.moe(s2, norm, np.array([[3, 9]]), (w * 2.5).astype(np.float32), "bf16", ex, "bf16",
                   sh)
    np.testing.assert_allclose(b["routed"], 2.5 * a["routed"], rtol=1e-6, atol=1e-7)
    c = oracle.moe(s2, norm, np.array([[9, 3]]), w[:, ::-1].copy(), "bf16", ex, "bf16", sh)
    np.testing.assert_allclose(c["routed"], a["routed"], rtol=1e-6, atol=1e-7)
    # teacher forcing with the produced hidden rows reproduces the same outputs
    f = oracle.moe(s2, None, np.array([[3, 9]]), w, "bf16", ex, "bf16", sh,
                   h_routed=a["h_routed"], h_shared=a["h_shared"])
    for key in ("routed", "shared", "block"):
        np.testing.assert_array_equal(f[key], a[key])


def _golden(name):
    import os
    out = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    return out


@pytest.mark.parametrize("case", ["shared_rounded", "routed_unrounded"])
def test_block_rounding_points_hand_derived(case):
    """tests/golden/block_rounding.txt: block = bf16(routed + bf16(shared)) with routed kept in
    f32, on exact down products (hidden rows given) where each rounding point changes the
    result bit."""
    want = int(_golden("block_rounding.txt")[case], 16)
    H = I = 32
    s = oracle.make_shape(1, H, 1, 1, I, I, "bf16", 1.0)
    hr = np.zeros((1, 1, I))
    hs = np.zeros((1, I))
    dr = np.zeros((H, I))
    ds = np.zeros((H, I))
    if case == "shared_rounded":
        dr[:, 0], hr[0, 0, 0] = 3 * 2.0 ** -10, 1.0
        ds[:, 0], ds[:, 1], hs[0, :2] = 1.0, 2.0 ** -9, 1.0
    else:
        dr[:, 0], dr[:, 1], hr[0, 0, :2] = 2.0 ** -8, 2.0 ** -16, 1.0
        ds[:, 0], hs[0, 0] = 1.0, 1.0
    z = to_bf(np.zeros((I, H)))
    routed = {0: {"gate": z, "up": z, "down": to_bf(dr)}}
    shared = {"gate": z, "up": z, "down": to_bf(ds)}
    m = oracle.moe(s, None, np.array([[0]]), np.array([[1.0]], np.float32), "bf16", routed,
                   "bf16", shared, h_routed=to_bf(hr), h_shared=to_bf(hs))
    assert np.all(m["block"][0] == want), hex(int(m["block"][0, 0]))
