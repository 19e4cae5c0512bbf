"""Repeated fused launches are byte-identical, also when launches on other inputs and weights run
in between (a stale value read across workgroups or from a previous launch would show here).
Workload: V4.1-like shapes at 2 rows (the path of every multi-row workload) and the 1-row case."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_r1": synth.CONFIGS[2].with_(hidden=1024, n_experts=64, top_k=8, inter=512,
                                      shared_inter=512),
    "q8_r2": synth.CONFIGS[3].with_(rows=2, hidden=1024, n_experts=64, top_k=8, inter=512,
                                    shared_inter=512),
    "fp4_mx8_r3": synth.CONFIGS[10].with_(rows=3, zero_rows=(), grouped_bias=False,
                                          shared_fmt="mxfp4", hidden=1024, n_experts=64,
                                          top_k=8, inter=512, shared_inter=512),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_repeatable_across_interleaved_launches(name):
    import torch
    import support
    cfg = CASES[name]
    g = support.Gpu(cfg, layers=(0, 1))
    a, b = g.state(0), g.state(1)
    wn0, wn1 = g.layers[1]["w_mix"], g.layers[0]["w_mix"]
    ref_a = g.fused(a, 0, None, wn0)
    ref_b = g.fused(b, 1, None, wn1)
    keys = ["idx", "weights", "h_routed", "block", "new_state", "carry", "norm"]
    for it in range(12):
        if it % 2 == 0:
            support.assert_same(g.fused(a, 0, None, wn0), ref_a, keys)
        else:
            support.assert_same(g.fused(b, 1, None, wn1), ref_b, keys)
    assert not np.array_equal(ref_a["new_state"], ref_b["new_state"])


@pytest.mark.parametrize("name", ["tiny_f32_r1"] + list(CASES))
def test_fused_in_place_equals_out_of_place(name):
    """state_out == state_in: no workgroup may overwrite its slice of the state before every
    workgroup has read all of it (the tiny case leaves most workgroups without expert work, so
    they reach the expand first)."""
    import torch
    import support
    cfg = synth.CONFIGS[1] if name == "tiny_f32_r1" else CASES[name]
    g = support.Gpu(cfg, layers=(0, 1))
    wn = g.layers[1]["w_mix"]
    keys = ["idx", "weights", "block", "new_state", "carry", "norm"]
    for sample in (0, 1, 2):
        st = g.state(sample)
        ref = g.fused(st, 0, None, wn)
        inplace = st.clone()
        got = g.fused(inplace, 0, None, wn, state_out=inplace)
        support.assert_same(got, ref, keys)
    del g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", list(CASES))
def test_chained_in_place_halves_equal_unfused(name):
    """Three chained layer halves, each taking the previous carry (so it skips its own mix) and
    overwriting its input state in place, give the same bytes as the unfused calls chained the
    same way (covers the carry at several rows and in-place at several rows)."""
    import torch
    import support
    cfg = CASES[name]
    n = 3
    g = support.Gpu(cfg, layers=tuple(range(n + 1)))
    R, H = cfg.rows, cfg.hidden
    keys = ["mixes", "idx", "weights", "block", "new_state", "carry"]
    st = g.state(4).clone()
    st_u = st.clone()
    carry, carry_u = None, None
    for l in range(n):
        wn = g.layers[l + 1]["w_mix"]
        cout = g.buf(R * 25 * 4)
        ref = g.unfused(st_u, l, carry_u, wn)
        got = g.fused(st, l, carry, wn, state_out=st, carry_out=cout)
        support.assert_same(got, ref, keys)
        st_u = g.buf(R * 4 * H * g.ab)
        st_u.copy_(st)
        carry_u = cout.clone()
        carry = cout
    del g
    torch.cuda.empty_cache()
