"""The GPU-vs-oracle checker (tests/support.py) on the CPU: outputs that are the oracle's own
pass every rule, stage-wise and end to end; a 1 % error in the hidden rows, the block or the new
state fails, although 1 % of a value below 0.78 is inside the contract's absolute floor of
2^-7 (the bf16 step rule catches it); a near-tie row is recognised."""

import numpy as np
import pytest

import oracle
import support
import synth

CFG = synth.CONFIGS[2].with_(rows=2, hidden=512, n_experts=32, top_k=4, inter=256,
                             shared_inter=256)


def oracle_as_gpu(cfg, sample=0):
    s = oracle.shape_of(cfg)
    d0, d1 = synth.dense_host(cfg, 0), synth.dense_host(cfg, 1)
    st = synth.state_host(cfg, sample)
    sh = synth.expert_host(cfg, 0, None)
    get = lambda e: synth.expert_host(cfg, 0, e)
    out = oracle.layer(s, st, d0, cfg.routed_fmt, get, cfg.shared_fmt, sh, d1["w_mix"])
    return out, (st, d0, get, sh, d1["w_mix"])


def perturb_bf16(a, rel):
    v = support.bf(a).astype(np.float64) * (1.0 + rel)
    return np.array([oracle.f32_to_bf16(float(x)) for x in v.ravel()], np.uint16).reshape(a.shape)


def test_oracle_outputs_pass_both_comparisons():
    out, args = oracle_as_gpu(CFG)
    support.compare_stagewise(CFG, out, *args)
    rep = support.compare_end_to_end(CFG, out, *args)
    assert "skipped" not in rep


@pytest.mark.parametrize("key", ["h_routed", "block", "new_state", "norm"])
def test_one_percent_error_fails(key):
    out, args = oracle_as_gpu(CFG)
    bad = dict(out)
    bad[key] = perturb_bf16(out[key], 0.01)
    # within the contract's floor: |d| <= 2^-7 max(1, |ref|) holds for most elements
    d = np.abs(support.bf(bad[key]).astype(np.float64) - support.bf(out[key]))
    lim = support.BF16_TOL * np.maximum(1.0, np.abs(support.bf(out[key])))
    assert np.mean(d <= lim) > 0.5
    with pytest.raises(AssertionError, match="bf16 step|elements off|exact g"):
        support.compare_stagewise(CFG, bad, *args)


def test_single_step_flips_pass_the_step_rule():
    out, _ = oracle_as_gpu(CFG)
    h = out["h_routed"].copy().ravel()
    h[::997] ^= 1          # one bf16 step in about 0.1 % of the elements
    support.check_bf16("h_routed", h, out["h_routed"].ravel())
    h[::331] ^= 2          # two or three steps in about 0.3 %
    with pytest.raises(AssertionError, match="bf16 step"):
        support.check_bf16("h_routed", h, out["h_routed"].ravel())


def test_near_tie_rows_are_detected():
    beta = np.array([[3.0, 2.0, 1.0, 1.0 - 5e-6, 0.5],
                     [3.0, 2.0, 1.0, 0.5, 0.4],
                     [3.0, 2.0, 2.0 - 1e-6, 0.5, 0.4],
                     [1.0, 1.0, 1.0, 1.0, 1.0]], np.float32)
    assert support.near_tie_rows(beta, 3) == [0, 2, 3]
    z = np.zeros((4, 5), np.float32)
    # identical logits: the exact ties of row 3 break alike on both sides
    assert support.near_tie_rows(beta, 3, z, z) == [0, 2]


def test_hidden_value_from_an_ambiguous_rounding_is_accepted():
    """A hidden value whose gate sum lies on a bf16 rounding midpoint may come out of either
    rounding; any other deviation of more than the contract is refused."""
    import support
    H, I = 64, 32
    x = np.zeros(H)
    x[0] = 1.0
    norm = support._bf16_bits(x)[None]
    # gate row 0 = 1 + 2^-8 (a midpoint between bf16 1 and 1 + 2^-7) as an f32 weight
    Wg = np.zeros((I, H), np.float32)
    Wu = np.zeros((I, H), np.float32)
    Wg[:, 0] = 1.0 + 2.0 ** -8
    Wu[:, 0] = 1.5
    t = {"gate": Wg, "up": Wu}
    silu = lambda g: g / (1.0 + np.exp(-g))
    ref = support._bf16_bits(silu(1.0) * 1.5 * np.ones(I))[None]       # gate rounded down (even)
    alt = support._bf16_bits(silu(1.0 + 2.0 ** -7) * 1.5 * np.ones(I))[None]
    assert not np.array_equal(ref, alt)
    rows = lambda ix: ("f32", t, 0)
    support.check_hidden("h", alt, ref, "bf16", norm, rows)           # the other rounding of g
    bad = support._bf16_bits(support.bf(ref).astype(np.float64) * 1.03)
    with pytest.raises(AssertionError, match="exact g"):
        support.check_hidden("h", bad, ref, "bf16", norm, rows)


def test_norm_flip_reaches_logits_within_budget_only():
    """A one-step flip of a norm value moves every logit by W_r[e][h] times the step; the end to
    end check allows exactly that first-order effect, and a logit error it does not explain
    still fails."""
    out, args = oracle_as_gpu(CFG)
    s = oracle.shape_of(CFG)
    d0 = args[1]
    norm = out["norm"].copy()
    h = int(np.argmax(np.abs(support.bf(norm[0]))))
    norm[0, h] ^= 1
    flipped = dict(out)
    flipped["norm"] = norm
    flipped["logits"] = oracle.router_logits(s, norm, d0["w_router"])
    moved = np.abs(flipped["logits"][0].astype(np.float64) - out["logits"][0])
    lim = support.F32_TOL * np.maximum(np.abs(out["logits"][0]),
                                       np.sqrt((out["logits"][0].astype(np.float64) ** 2).mean()))
    assert (moved > lim).any(), "the flip must move some logit beyond the plain tolerance"
    rep = support.compare_end_to_end(CFG, flipped, *args)
    assert "skipped" not in rep
    bad = dict(flipped)
    lg = flipped["logits"].copy()
    e = int(np.argmax(np.abs(lg[1])))
    lg[1, e] *= np.float32(1.001)   # row 1 has no flipped norm value
    bad["logits"] = lg
    with pytest.raises(AssertionError, match="e2e logits"):
        support.compare_end_to_end(CFG, bad, *args)
