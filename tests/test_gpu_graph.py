"""The fused launch captured in a HIP graph (torch.cuda.CUDAGraph): three chained layer halves
(each taking the previous carry) recorded once and replayed several times, with other eager
launches on the same workspace and synchronisations between the replays; every replay gives
the bytes of the eager chain. The calls enqueue kernels only (no memset node, no host sync),
and each replay takes new epochs from the start counters in the workspace."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

CASES = {
    "bf16_r1": synth.CONFIGS[2].with_(hidden=1024, n_experts=64, top_k=8, inter=512,
                                      shared_inter=512),
    "q8_r3": synth.CONFIGS[3].with_(rows=3, hidden=1024, n_experts=64, top_k=8, inter=512,
                                    shared_inter=512),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_chain(name):
    import torch
    import support
    import moe_decode_layer_amd as mono
    cfg = CASES[name]
    print("graph capture of a 3-half chain,", name, flush=True)
    n = 3
    g = support.Gpu(cfg, layers=tuple(range(n + 1)))
    R, H = cfg.rows, cfg.hidden
    st0 = g.state(0)
    outs = [g.buf(R * 4 * H * g.ab) for _ in range(n)]
    carries = [g.buf(R * 25 * 4) for _ in range(n)]

    def chain():
        stream = support.stream()
        prev, cin = st0, None
        for l in range(n):
            mono.mono_ffn_layer(g.shape, g.structs[l], g.layers[l + 1]["w_mix"], prev, cin,
                                outs[l], carries[l], g.ws, stream)
            prev, cin = outs[l], carries[l]

    chain()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs] + [c.clone() for c in carries]
    for t in outs + carries:
        t.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    torch.cuda.synchronize()
    other = g.state(1)
    for rep in range(4):
        for t in outs + carries:
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = outs + carries
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), "replay %d differs in output %d" % (rep, i)
        # eager work on the same workspace between replays
        g.fused(other, 0, None, g.layers[1]["w_mix"])
    st, err = mono.mono_workspace_poll(g.ws, support.stream())
    assert st == mono.MONO_OK, err
    del graph, g
    torch.cuda.empty_cache()
