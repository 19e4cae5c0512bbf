"""mono_ffn_layer_static (the fused launch on the library's static device workspace, for callers
that cannot allocate) gives the same bytes as mono_ffn_layer on a workspace of its own, over
calls in a row whose shape changes: a 6-row Q8_0 step, then a smaller 1-row bf16 step (the
static workspace is re-initialised for the new shape), then the 6-row shape again."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

BIG = synth.CONFIGS[3].with_(hidden=1024, n_experts=64, top_k=8, inter=512, shared_inter=512)
SMALL = synth.CONFIGS[2].with_(hidden=512, n_experts=32, top_k=4, inter=256, shared_inter=256)


def _static_equals_workspace_call(cfg, sample):
    import torch
    import support
    import moe_decode_layer_amd as mono
    print("static workspace call:", cfg.name, "rows", cfg.rows, "hidden", cfg.hidden,
          "sample", sample, flush=True)
    g = support.Gpu(cfg, layers=(0, 1))
    st = g.state(sample)
    wn = g.layers[1]["w_mix"]
    ref = g.fused(st, 0, None, wn)
    out = g.buf(cfg.rows * 4 * cfg.hidden * g.ab)
    carry = g.buf(cfg.rows * 25 * 4)
    mono.mono_ffn_layer_static(g.shape, g.structs[0], wn, st, None, out, carry,
                               support.stream())
    torch.cuda.synchronize()
    new = support.d2h(out, g.adt, (cfg.rows, 4, cfg.hidden))
    c = support.d2h(carry, np.float32, (cfg.rows, 25))
    assert np.array_equal(new.view(np.uint8), ref["new_state"].view(np.uint8))
    assert np.array_equal(c.view(np.uint8), ref["carry"].view(np.uint8))
    del g
    torch.cuda.empty_cache()


def test_static_workspace_matches_over_shape_changes():
    _static_equals_workspace_call(BIG, 0)
    _static_equals_workspace_call(SMALL, 1)     # smaller input: re-initialised for the shape
    _static_equals_workspace_call(BIG, 2)
