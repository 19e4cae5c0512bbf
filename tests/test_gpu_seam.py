"""GPU parity of the attention-half mHC seam and the model tail.

A layer is an attention half and an FFN half, each with its own HC weights. The chain under
test runs, per layer: the attention half's pre side from the previous FFN half's carry
(mono_hc_mix_collapse with the attention half's mix, scales, biases and norm weight), a stand-in
attention (a fixed per-position gain on the attention norm, rounded to bf16, computed on the
host, since attention is outside this library), the attention half's post side with the carry
for the FFN half (mono_hc_expand with the FFN half's mix as the next mix), and the FFN half as
one fused launch whose carry feeds the next layer's attention pre side; after the last layer the
model tail (mono_hc_head) collapses the state and applies the output norm without a split. Every
stage is checked against the oracle fed the GPU's inputs to that stage (tests/support.py rules).
"""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

HEAD_CASES = {
    "tiny_f32_r1": synth.CONFIGS[1],
    "bf16_r3_h576": synth.CONFIGS[2].with_(rows=3, hidden=576, n_experts=24, top_k=6,
                                           inter=96, shared_inter=160),
    "full_bf16_r1": synth.CONFIGS[2],
    "full_q8_r6": synth.CONFIGS[3],
    "full_r8_zero_row": synth.CONFIGS[4],
}


def _head_device(cfg):
    from synth import device as sdev
    import moe_decode_layer_amd as mono
    t = sdev.head(cfg)
    return t, mono.make_head(t["w_head"], t["head_scale"], t["head_base"], t["w_norm"])


def _check_head(cfg, st_h, pre_g, x_g, norm_g):
    import oracle
    import support
    s = oracle.shape_of(cfg)
    h = synth.head_host(cfg)
    pre, _, _ = oracle.head(s, st_h, h["w_head"], h["head_scale"], h["head_base"], h["w_norm"])
    rep = {"pre": support.check_f32("head pre", pre_g, pre)}
    x, norm = oracle.collapse_norm(s, st_h, pre_g, h["w_norm"])
    rep["x"] = support.check_bf16("head x", x_g, x, cfg.act)
    rep["norm"] = support.check_bf16("head norm", norm_g, norm, cfg.act)
    return rep


@pytest.mark.parametrize("name", list(HEAD_CASES))
def test_head_matches_oracle(name):
    import torch
    import support
    import moe_decode_layer_amd as mono
    from moe_decode_layer_amd import host
    from synth import device as sdev
    cfg = HEAD_CASES[name]
    print("model tail", name, flush=True)
    R, H, ab = cfg.rows, cfg.hidden, synth.act_bytes(cfg.act)
    shape = host.shape_of(cfg)
    tensors, head = _head_device(cfg)
    st = sdev.state(cfg, 2)
    pre = torch.zeros(R * 4, dtype=torch.float32, device="cuda")
    x = torch.zeros(R * H * ab, dtype=torch.uint8, device="cuda")
    norm = torch.zeros(R * H * ab, dtype=torch.uint8, device="cuda")
    mono.mono_hc_head(shape, st, head, pre, x, norm, support.stream())
    torch.cuda.synchronize()
    adt = synth.act_np(cfg.act)
    got = (pre.cpu().numpy().reshape(R, 4), x.cpu().numpy().view(adt).reshape(R, H),
           norm.cpu().numpy().view(adt).reshape(R, H))
    support.set_case("model tail %s" % name)
    rep = _check_head(cfg, synth.state_host(cfg, 2), *got)
    print(name, rep, flush=True)
    # x and pre are optional outputs: norm alone gives the same bytes
    norm2 = torch.zeros_like(norm)
    mono.mono_hc_head(shape, st, head, None, None, norm2, support.stream())
    torch.cuda.synchronize()
    assert torch.equal(norm2, norm)
    if cfg.zero_rows:
        for r in cfg.zero_rows:
            assert not np.any(got[2][r]), "an all-zero state row collapses to a zero norm row"


def _stand_in_attention(cfg, norm_bits, layer):
    """bf16(norm * gain) per position (f64 product, one rounding): the same function of its
    input on the GPU's side and the oracle's."""
    import oracle
    g = synth.attn_gain_host(cfg, layer).astype(np.float64)
    v = np.vectorize(oracle.bf16_to_f64)(norm_bits).astype(np.float64) * g[None, :]
    return np.vectorize(lambda z: oracle.f32_to_bf16(float(np.float32(z))))(v).astype(np.uint16)


@pytest.mark.parametrize("ci,layers", [(2, 2), (3, 1)])
def test_layer_chain_with_attention_seam_and_tail(ci, layers):
    import torch
    import oracle
    import support
    import moe_decode_layer_amd as mono
    from synth import device as sdev
    cfg = synth.CONFIGS[ci]
    R, H, ab = cfg.rows, cfg.hidden, synth.act_bytes(cfg.act)
    adt = synth.act_np(cfg.act)
    print("layer chain", ci, cfg.name, "layers", layers, flush=True)
    g = support.Gpu(cfg, layers=tuple(range(layers)))
    s = oracle.shape_of(cfg)
    attn_dev = [sdev.dense(cfg, synth.ATTN_LAYER + l) for l in range(layers)]
    attn_host = [synth.dense_host(cfg, synth.ATTN_LAYER + l) for l in range(layers)]
    attn_struct = [mono.make_layer(a["w_mix"], a["hc_scale"], a["hc_base"], a["w_norm"], None,
                                   None, mono.Experts(), mono.Experts()) for a in attn_dev]
    tensors, head = _head_device(cfg)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32, device="cuda")
    raw = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")
    d2h = lambda t, dt, shp: t.cpu().numpy().view(dt).reshape(shp)
    state = g.state(3)
    state_h = synth.state_host(cfg, 3)
    carry, carry_h = None, None
    for l in range(layers):
        # attention half, pre side (carry from the previous FFN half)
        o = dict(mixes=f32(R * 24), pre=f32(R * 4), post=f32(R * 4), comb=f32(R * 16),
                 x=raw(R * H * ab), norm=raw(R * H * ab))
        mono.mono_hc_mix_collapse(g.shape, state, attn_struct[l], carry, o["mixes"], o["pre"],
                                  o["post"], o["comb"], o["x"], o["norm"], g.ws, support.stream())
        torch.cuda.synchronize()
        out = dict(mixes=d2h(o["mixes"], np.float32, (R, 24)), pre=d2h(o["pre"], np.float32, (R, 4)),
                   post=d2h(o["post"], np.float32, (R, 4)),
                   comb=d2h(o["comb"], np.float32, (R, 4, 4)), x=d2h(o["x"], adt, (R, H)),
                   norm=d2h(o["norm"], adt, (R, H)))
        support.set_case("chain %d layer %d attention pre" % (ci, l))
        support.compare_pre_side(cfg, out, state_h, attn_host[l], carry_h)
        # stand-in attention, then the attention half's post side with the FFN half's mix next
        attn_out_h = _stand_in_attention(cfg, out["norm"], l)
        attn_out = torch.from_numpy(attn_out_h.view(np.uint8).ravel().copy()).cuda()
        w_ffn_mix = g.layers[l]["w_mix"]
        mid, mid_carry = raw(R * 4 * H * ab), f32(R * 25)
        mono.mono_hc_expand(g.shape, state, attn_out, o["post"], o["comb"], w_ffn_mix, mid,
                            mid_carry, g.ws, support.stream())
        torch.cuda.synchronize()
        mid_h, mid_carry_h = d2h(mid, adt, (R, 4, H)), d2h(mid_carry, np.float32, (R, 25))
        new_ref, _ = oracle.expand(s, state_h, attn_out_h, out["post"], out["comb"], None)
        support.set_case("chain %d layer %d attention post" % (ci, l))
        support.check_bf16("attention new state", mid_h, new_ref, cfg.act)
        support.check_f32("attention carry", mid_carry_h,
                          support.oracle_carry(cfg, mid_h, synth.dense_host(cfg, l)["w_mix"]))
        # FFN half, fused, from the attention half's carry; its carry feeds the next layer's
        # attention pre side (none after the last layer: the tail mixes the state itself)
        w_next = attn_dev[l + 1]["w_mix"] if l + 1 < layers else None
        w_next_h = attn_host[l + 1]["w_mix"] if l + 1 < layers else None
        new = raw(R * 4 * H * ab)
        carry_out = f32(R * 25) if w_next is not None else None
        fo = g.fused(mid, l, mid_carry, w_next, state_out=new, carry_out=carry_out)
        d_h = synth.dense_host(cfg, l)
        sh_h = synth.expert_host(cfg, l, None) if cfg.shared_inter > 0 else None
        support.set_case("chain %d layer %d FFN half" % (ci, l))
        rep = support.compare_stagewise(cfg, fo, mid_h, d_h, lambda e: synth.expert_host(cfg, l, e),
                                        sh_h, w_next_h, carry_in=mid_carry_h)
        print("layer", l, {k: v for k, v in rep.items()}, flush=True)
        state, state_h = new, fo["new_state"]
        carry, carry_h = carry_out, (fo["carry"] if w_next is not None else None)
    # model tail
    pre, x, norm = f32(R * 4), raw(R * H * ab), raw(R * H * ab)
    mono.mono_hc_head(g.shape, state, head, pre, x, norm, support.stream())
    torch.cuda.synchronize()
    support.set_case("chain %d model tail" % ci)
    _check_head(cfg, state_h, d2h(pre, np.float32, (R, 4)), d2h(x, adt, (R, H)),
                d2h(norm, adt, (R, H)))
    del g
    torch.cuda.empty_cache()
