"""Oracle pins: number formats and weight decodes.

Each decode is checked against an independent definition: numpy's IEEE fp16
and f32 conversions, the E2M1 bit-field formula and the OCP MX table
(tests/golden/e2m1_codes.txt), and ldexp for E8M0.
"""

import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_decode_all_finite_codes():
    codes = np.arange(65536, dtype=np.uint32)
    f = (codes << 16).view(np.float32)
    for c in list(range(0, 65536, 97)) + [0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8000]:
        if np.isnan(f[c]):
            continue
        assert oracle.bf16_to_f64(c) == float(f[c])


@pytest.mark.parametrize("value,expected", [
    (1.0, 0x3F80), (-2.0, 0xC000), (3.140625, 0x4049),
    (1.00390625, 0x3F80),      # 1 + 2^-8: exact tie, rounds to even (down)
    (1.01171875, 0x3F82),      # 1 + 3*2^-8: tie, rounds to even (up)
    (1.0039063692092896, 0x3F81),  # just above the tie: rounds up
    (0.0, 0x0000),
])
def test_bf16_round_to_nearest_even(value, expected):
    assert oracle.f32_to_bf16(value) == expected


def test_bf16_rounding_matches_nearest_on_random_values():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(2000).astype(np.float32)
    for v in x[:400]:
        b = oracle.f32_to_bf16(float(v))
        # nearest bf16 by exhaustive comparison with the two neighbours
        lo = (np.uint32(v.view(np.uint32)) >> 16) << 16
        cand = [np.uint32(lo).view(np.float32), np.uint32(lo + 0x10000).view(np.float32)]
        got = np.uint32(b << 16).view(np.float32)
        d = [abs(float(c) - float(v)) for c in cand]
        assert abs(float(got) - float(v)) == min(d)


def test_fp16_decode_matches_numpy():
    codes = np.arange(65536, dtype=np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    for c in range(0, 65536, 7):
        r = ref[c]
        o = oracle.f16_to_f64(c)
        if np.isnan(r):
            assert math.isnan(o)
        else:
            assert o == r, c


def test_e2m1_golden_table():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_codes.txt"))
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 16
    for code, val in rows:
        got = oracle.e2m1_to_f64(int(code))
        assert got == float(val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_e2m1_bitfield_formula():
    for code in range(16):
        s, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert abs(oracle.e2m1_to_f64(code)) == mag


def test_e8m0_all_codes():
    for e in range(255):
        assert oracle.e8m0_to_f64(e) == math.ldexp(1.0, e - 127)
    assert math.isnan(oracle.e8m0_to_f64(255))


def test_q8_0_matrix_element_is_scale_times_int():
    cfg = synth.CONFIGS[3].with_(hidden=256, inter=64, shared_inter=64)
    t = synth.expert_host(cfg, 0, 3)
    v, sc = t["gate"], t["gate_s"]
    rng = np.random.default_rng(2)
    for _ in range(200):
        r, c = int(rng.integers(v.shape[0])), int(rng.integers(v.shape[1]))
        d = float(sc[r, c // 32:c // 32 + 1].view(np.float16)[0])
        assert oracle.mat_elem("q8_0", v, sc, v.shape[1], r, c) == d * float(v[r, c])


def test_mxfp4_matrix_element_nibble_order():
    # low nibble holds the even element, high nibble the odd one; one e8m0 scale per 32
    vals = np.array([[0x2A, 0xF1] * 16], dtype=np.uint8)   # 64 codes in one row
    scales = np.array([[127 - 2, 127 + 1]], dtype=np.uint8)
    k = 64
    expect = []
    for c in range(k):
        byte = int(vals[0, c // 2])
        code = byte & 0xF if c % 2 == 0 else byte >> 4
        expect.append(oracle.e2m1_to_f64(code) * 2.0 ** (int(scales[0, c // 32]) - 127))
    got = [oracle.mat_elem("mxfp4", vals, scales, k, 0, c) for c in range(k)]
    assert got == expect
    # 0x2A: low nibble 0xA = -1.0, high nibble 0x2 = +1.0; 0xF1: low 0x1 = 0.5, high 0xF = -6
    assert got[:4] == [-0.25, 0.25, 0.125, -1.5]
    assert got[32:36] == [-2.0, 2.0, 1.0, -12.0]
