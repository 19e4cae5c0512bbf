"""Race shaker: under mono_workspace_set_jitter every wave of the fused launch waits a
pseudo-random time at each phase boundary, which reorders the workgroups' publications (mix
partials, router logits, hidden rows, down outputs, carry partials) and the waves' claims
inside a workgroup. The launch's results do not depend on
timing, so every output must stay byte-identical to the launch without delays, over several
seeds, at small and full size, with no bounded wait expiring."""

import pytest

import synth

pytestmark = pytest.mark.gpu

SMALL = dict(hidden=512, n_experts=32, top_k=4, inter=256, shared_inter=256)
CASES = {
    "bf16_r1": synth.CONFIGS[2].with_(**SMALL),
    "q8_r6": synth.CONFIGS[3].with_(**SMALL),
    "fp4_r8_zero_row": synth.CONFIGS[4].with_(hidden=512, n_experts=64, top_k=8, inter=256,
                                              shared_inter=256),
    "bf16_r3_ragged": synth.CONFIGS[2].with_(rows=3, hidden=576, n_experts=24, top_k=6,
                                             inter=96, shared_inter=160),
    "full_bf16_r1": synth.CONFIGS[2],
    "full_q8_r6": synth.CONFIGS[3],
    # MXFP8 activations: the in-place round trips of the staged hidden rows (by the staging
    # wave between workgroup fences in the one-row flow, by the workgroup behind barriers at
    # several rows) and of the norm rows
    "fp4_mx8_r1_fp4_shared": synth.CONFIGS[10].with_(rows=1, zero_rows=(), grouped_bias=False,
                                                     shared_fmt="mxfp4", **SMALL),
    "fp4_mx8_r8_zero_row": synth.CONFIGS[10].with_(hidden=512, n_experts=64, top_k=8, inter=256,
                                                   shared_inter=256),
    "full_fp4_mx8_r8": synth.CONFIGS[10],
}
KEYS = ["mixes", "pre", "post", "comb", "x", "norm", "logits", "idx", "weights", "h_routed",
        "h_shared", "shared", "routed", "block", "new_state", "carry"]
MAX_TICKS = 3000  # 30 us of the 100 MHz counter per wait


@pytest.mark.parametrize("name", list(CASES))
def test_outputs_do_not_depend_on_timing(name):
    import torch
    import support
    import moe_decode_layer_amd as mono
    cfg = CASES[name]
    print("race shaker", name, flush=True)
    g = support.Gpu(cfg, layers=(0, 1))
    st = g.state(1)
    wn = g.layers[1]["w_mix"]
    ref = g.fused(st, 0, None, wn)
    for seed in (1, 2, 3):
        print("  seed", seed, flush=True)
        mono.mono_workspace_set_jitter(g.ws, MAX_TICKS, seed)
        out = g.fused(st, 0, None, wn)   # asserts that no bounded wait expired
        support.assert_same(out, ref, KEYS)
    mono.mono_workspace_set_jitter(g.ws, 0, 0)
    support.assert_same(g.fused(st, 0, None, wn), ref, KEYS)
    # the delays are real: a launch under the shaker takes longer than one without it
    times = {}
    for ticks in (0, MAX_TICKS):
        mono.mono_workspace_set_jitter(g.ws, ticks, 9)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        new, carry = g.buf(cfg.rows * 4 * cfg.hidden * g.ab), g.buf(cfg.rows * 25 * 4)
        ev[0].record()
        for _ in range(5):
            mono.mono_ffn_layer(g.shape, g.structs[0], wn, st, None, new, carry, g.ws,
                                support.stream())
        ev[1].record()
        torch.cuda.synchronize()
        times[ticks] = ev[0].elapsed_time(ev[1]) * 1e3 / 5
    mono.mono_workspace_set_jitter(g.ws, 0, 0)
    print("  launch us without / with the shaker: %.1f / %.1f" % (times[0], times[MAX_TICKS]))
    assert times[MAX_TICKS] > times[0] + 20.0
    del g
    torch.cuda.empty_cache()
