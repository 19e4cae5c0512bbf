"""The device build of the input generator writes the same bytes as the host build, so the
oracle (fed host-generated experts) and the GPU (fed device-generated experts) see one input."""

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ci", [1, 2, 3, 4])
def test_device_fill_equals_host_fill(ci):
    import torch
    import synth.device as sdev
    cfg = synth.CONFIGS[ci].with_(n_experts=4, rows=synth.CONFIGS[ci].rows)
    d = sdev.layer(cfg, 0)
    torch.cuda.synchronize()
    h = synth.dense_host(cfg, 0)
    for name in ("w_mix", "hc_base", "w_norm", "w_router", "bias", "hc_scale"):
        a = h[name]
        got = d[name].cpu().numpy()[: a.nbytes]
        assert np.array_equal(got, a.view(np.uint8).ravel()), name
    for e in (0, 3):
        he = synth.expert_host(cfg, 0, e)
        for name, a in he.items():
            per = a.nbytes
            got = d["routed"][name].cpu().numpy()[e * per:(e + 1) * per]
            assert np.array_equal(got, a.view(np.uint8).ravel()), (name, e)
    hs = synth.expert_host(cfg, 0, None)
    for name, a in hs.items():
        assert np.array_equal(d["shared"][name].cpu().numpy()[: a.nbytes], a.view(np.uint8).ravel())
    st = sdev.state(cfg, 5).cpu().numpy()
    assert np.array_equal(st, synth.state_host(cfg, 5).view(np.uint8).ravel())
