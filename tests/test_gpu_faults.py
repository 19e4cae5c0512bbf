"""Failure handling of the persistent launch, forced from the host: workgroup 0 withholds the
values it publishes for the other workgroups (its mix partial sums, router logits or hidden
rows) and the wait limit is shortened, so every waiting workgroup's bounded wait expires, the
error word is set and the launch ends normally (no hang, no fault). After mono_workspace_init
the workspace works again and gives the same bytes as a fresh one."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

PH_MIX, PH_ROUTER, PH_GATEUP = 1, 2, 3
SMALL = synth.CONFIGS[2].with_(hidden=512, n_experts=32, top_k=4, inter=256, shared_inter=256)
# several rows take the multi-row down phase (expert-row stretches, tagged outputs)
SMALL_R3 = synth.CONFIGS[3].with_(rows=3, hidden=512, n_experts=32, top_k=4, inter=256,
                                  shared_inter=256)


@pytest.mark.parametrize("rows", [1, 3])
@pytest.mark.parametrize("phase", [PH_MIX, PH_ROUTER, PH_GATEUP])
def test_withheld_values_time_out_and_recover(phase, rows):
    import torch
    import support
    import moe_decode_layer_amd as mono
    print("values withheld at point", phase, "rows", rows, flush=True)
    cfg = SMALL if rows == 1 else SMALL_R3
    g = support.Gpu(cfg, layers=(0, 1))
    st = g.state(0)
    wn = g.layers[1]["w_mix"]
    ref = g.fused(st, 0, None, wn)
    grid = mono.mono_grid_size()
    # 2 ms limit (100 MHz counter); workgroup 0 (it has mix, router and gate/up work) withholds
    mono.mono_workspace_set_debug(g.ws, 200000, 0, phase, support.stream())
    new = g.buf(cfg.rows * 4 * cfg.hidden * 2)
    carry = g.buf(cfg.rows * 25 * 4)
    mono.mono_ffn_layer(g.shape, g.structs[0], wn, st, None, new, carry, g.ws, support.stream())
    status, err = mono.mono_workspace_poll(g.ws, support.stream())
    assert status == mono.MONO_E_TIMEOUT
    assert err[0] == 1 and err[1] == phase and 0 <= err[2] < grid
    assert err[3] == grid   # every workgroup waited there and gave up once
    mono.mono_workspace_init(g.ws, g.shape, support.stream())
    again = g.fused(st, 0, None, wn)
    support.assert_same(again, ref, ["mixes", "logits", "idx", "weights", "h_routed", "block",
                                     "new_state", "carry"])
    del g
    torch.cuda.empty_cache()


def test_short_limit_without_a_fault_still_completes():
    import torch
    import support
    import moe_decode_layer_amd as mono
    g = support.Gpu(SMALL, layers=(0, 1))
    st = g.state(1)
    wn = g.layers[1]["w_mix"]
    ref = g.fused(st, 0, None, wn)
    # 20 ms limit is far above any barrier wait of this workload: no expiry
    mono.mono_workspace_set_debug(g.ws, 2000000, -1, 0, support.stream())
    out = g.fused(st, 0, None, wn)
    support.assert_same(out, ref, ["new_state", "carry", "idx"])
    del g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rows", [1, 3])
def test_launch_after_expired_wait_is_correct_without_init(rows):
    """A launch that ended early leaves stale tagged values behind; the next launch takes a new
    epoch from the start counters, so it accepts none of them and computes the same bytes as
    before, while the error word stays set until the next init."""
    import torch
    import support
    import moe_decode_layer_amd as mono
    cfg = SMALL if rows == 1 else SMALL_R3
    g = support.Gpu(cfg, layers=(0, 1))
    st = g.state(2)
    wn = g.layers[1]["w_mix"]
    ref = g.fused(st, 0, None, wn)
    for phase in (PH_MIX, PH_ROUTER, PH_GATEUP):
        print("withheld at point", phase, "rows", rows, flush=True)
        mono.mono_workspace_set_debug(g.ws, 200000, 0, phase, support.stream())
        new = g.buf(cfg.rows * 4 * cfg.hidden * 2)
        carry = g.buf(cfg.rows * 25 * 4)
        mono.mono_ffn_layer(g.shape, g.structs[0], wn, st, None, new, carry, g.ws,
                            support.stream())
        status, _ = mono.mono_workspace_poll(g.ws, support.stream())
        assert status == mono.MONO_E_TIMEOUT
        mono.mono_workspace_set_debug(g.ws, 0, -1, 0, support.stream())
        out = g.fused(st, 0, None, wn, expect_ok=False)
        support.assert_same(out, ref, ["mixes", "logits", "idx", "weights", "h_routed", "block",
                                       "new_state", "carry"])
        status, _ = mono.mono_workspace_poll(g.ws, support.stream())
        assert status == mono.MONO_E_TIMEOUT      # reported until the next init
    mono.mono_workspace_init(g.ws, g.shape, support.stream())
    assert mono.mono_workspace_poll(g.ws, support.stream())[0] == mono.MONO_OK
    del g
    torch.cuda.empty_cache()
