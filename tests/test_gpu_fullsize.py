"""GPU parity at the full workload sizes, in the launch configuration the benchmark times (one
mono_ffn_layer launch per layer half on the full grid): every stage against the oracle fed the
GPU's inputs to that stage, and the fused launch byte-identical to the four unfused calls.

Workloads: hidden 5120, 256 experts, top-8, inter 2048, shared inter 2048, rho 2.5, with
  * 1 row and bf16 experts,
  * 6 rows and Q8_0 experts,
  * 8 rows, MXFP4 routed + bf16 shared experts, row 7 all zero, bias grouped by 32,
  * a chain of 8 bf16 layer halves at 1 row linked by the next-pre carry;
and the draft routing shapes at the same widths: 128 experts with top-3 and 256 experts with
top-6, each at 1 row (bf16 experts) and 6 rows (Q8_0 experts); and the 8-row MXFP4 workload with
the activations of the MXFP4 experts quantised to MXFP8.
"""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

OUT_KEYS = ["mixes", "pre", "post", "comb", "x", "norm", "logits", "idx", "weights",
            "h_routed", "h_shared", "shared", "routed", "block", "new_state", "carry"]


def _host(cfg, layer):
    shared = synth.expert_host(cfg, layer, None) if cfg.shared_inter > 0 else None
    return synth.dense_host(cfg, layer), shared


@pytest.mark.parametrize("ci", [2, 3, 4, *synth.DRAFT_CONFIGS, 10])
def test_full_size_layer(ci):
    import torch
    import support
    cfg = synth.CONFIGS[ci]
    print("full-size workload", ci, cfg.name, flush=True)
    g = support.Gpu(cfg, layers=(0, 1))
    st = g.state(5)
    wn = g.layers[1]["w_mix"]
    fused = g.fused(st, 0, None, wn)
    unfused = g.unfused(st, 0, None, wn)
    support.assert_same(fused, unfused, [k for k in OUT_KEYS if k in fused and k in unfused])
    d0, shared = _host(cfg, 0)
    d1 = synth.dense_host(cfg, 1)
    support.set_case("full-size workload %d" % ci)
    rep = support.compare_stagewise(cfg, fused, synth.state_host(cfg, 5), d0,
                                    lambda e: synth.expert_host(cfg, 0, e), shared, d1["w_mix"])
    print(ci, rep, flush=True)
    support.set_case("full-size workload %d end-to-end" % ci)
    e2e = support.compare_end_to_end(cfg, fused, synth.state_host(cfg, 5), d0,
                                     lambda e: synth.expert_host(cfg, 0, e), shared, d1["w_mix"])
    print(ci, "end-to-end", {k: v for k, v in e2e.items() if k != "ref"}, flush=True)
    if ci in (4, 10):
        grp = int(np.argmax(d0["bias"][::32]))
        assert fused["idx"][7].tolist() == list(range(32 * grp, 32 * grp + cfg.top_k))
    del g
    torch.cuda.empty_cache()


def test_chain_of_eight_layers_with_carry():
    import torch
    import support
    import moe_decode_layer_amd as mono
    cfg = synth.CONFIGS[5]
    n = cfg.layers
    print("chain of", n, "layer halves", flush=True)
    g = support.Gpu(cfg, layers=tuple(range(n)))
    R, H = cfg.rows, cfg.hidden
    states = [g.state(0)]
    carries = [None]
    outs = []
    for l in range(n):
        wn = g.layers[l + 1]["w_mix"] if l + 1 < n else None
        new = g.buf(R * 4 * H * g.ab)
        carry = g.buf(R * 25 * 4) if wn is not None else None
        outs.append(g.fused(states[l], l, carries[l], wn, state_out=new, carry_out=carry))
        states.append(new)
        carries.append(carry)
    # the unfused calls chained the same way give the same bytes at every layer
    st_u, carry_u = states[0], None
    for l in range(n):
        wn = g.layers[l + 1]["w_mix"] if l + 1 < n else None
        u = g.unfused(st_u, l, carry_u, wn)
        support.assert_same(outs[l], u, [k for k in OUT_KEYS if k in u and k in outs[l]])
        st_u = states[l + 1]
        carry_u = carries[l + 1]
    # free running inside each layer: the oracle runs the whole layer half from the GPU's input
    # state (and carry) of that layer, with no stage forced
    for l in range(n):
        d, shared = _host(cfg, l)
        wn_h = synth.dense_host(cfg, l + 1)["w_mix"] if l + 1 < n else None
        st_h = support.d2h(states[l], g.adt, (R, 4, H))
        carry_h = support.d2h(carries[l], np.float32, (R, 25)) if carries[l] is not None else None
        support.set_case("chain layer %d end-to-end" % l)
        e2e = support.compare_end_to_end(cfg, outs[l], st_h, d,
                                         lambda e: synth.expert_host(cfg, l, e), shared, wn_h,
                                         carry_in=carry_h)
        print("layer", l, "end-to-end", {k: v for k, v in e2e.items() if k != "ref"}, flush=True)
    # teacher forcing: layer l against the oracle fed the GPU's state and carry of layer l
    for l in range(n):
        support.set_case("chain layer %d" % l)
        d, shared = _host(cfg, l)
        wn_h = synth.dense_host(cfg, l + 1)["w_mix"] if l + 1 < n else None
        st_h = support.d2h(states[l], g.adt, (R, 4, H))
        carry_h = support.d2h(carries[l], np.float32, (R, 25)) if carries[l] is not None else None
        rep = support.compare_stagewise(cfg, outs[l], st_h, d,
                                        lambda e: synth.expert_host(cfg, l, e), shared, wn_h,
                                        carry_in=carry_h)
        if carry_h is not None:
            # the carried mixes equal the mixes computed directly from the state
            import oracle
            direct = oracle.mix(oracle.shape_of(cfg), st_h, d["w_mix"])
            support.check_f32("carried mixes", outs[l]["mixes"], direct)
        print("layer", l, rep, flush=True)
    del g
    torch.cuda.empty_cache()
