"""Device-resident synthetic workloads (torch tensors filled by libsynth_dev.so).

Test and benchmark infrastructure: allocates one layer half's tensors for a
workload in HBM and fills them in place with the same streams the host build
produces, so an oracle running on host copies of selected experts sees the
same bytes. Holds no step of the method.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import synth

try:
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _fill(t, g: synth.Gen, count: int, byte_off: int = 0, first: int = 0) -> None:
    synth.fill_device(g, t.data_ptr() + byte_off, count, first, _stream())


def _bytes(n: int, device) -> "torch.Tensor":
    return torch.empty(max(int(n), 16), dtype=torch.uint8, device=device)


def dense(cfg: synth.Config, layer: int, device="cuda") -> Dict[str, "torch.Tensor"]:
    """w_mix, hc_scale, hc_base, w_norm, w_router, bias as device tensors (raw storage)."""
    out = {}
    for name, (g, n, dt) in synth.dense_specs(cfg, layer).items():
        if name == "bias" and cfg.grouped_bias:
            continue
        nbytes = n * np.dtype(dt).itemsize
        t = _bytes(nbytes, device)
        _fill(t, g, n)
        out[name] = t
    host = synth.dense_host(cfg, layer) if cfg.grouped_bias else None
    if host is not None:
        out["bias"] = torch.from_numpy(host["bias"]).to(device).view(torch.uint8)
    out["hc_scale"] = torch.tensor(synth.HC_SCALE, dtype=torch.float32, device=device).view(
        torch.uint8)
    return out


def head(cfg: synth.Config, device="cuda") -> Dict[str, "torch.Tensor"]:
    """w_head, head_scale, head_base, w_norm of the model tail as device tensors (raw storage)."""
    out = {}
    for name, (g, n, dt) in synth.head_specs(cfg).items():
        t = _bytes(n * np.dtype(dt).itemsize, device)
        _fill(t, g, n)
        out[name] = t
    out["head_scale"] = torch.tensor([synth.HEAD_SCALE], dtype=torch.float32,
                                     device=device).view(torch.uint8)
    return out


def experts(cfg: synth.Config, layer: int, shared: bool, device="cuda",
            n: Optional[int] = None) -> Dict[str, "torch.Tensor"]:
    """Stacked expert matrices: gate, up, down (+ gate_s, up_s, down_s) as byte tensors.

    Routed: experts 0..E-1 stacked; shared: one expert."""
    count = 1 if shared else (cfg.n_experts if n is None else n)
    mats = synth.expert_matrices(cfg, layer, None if shared else 0)
    out = {}
    for (name, rows, k, gv, vb, gs, sb) in mats:
        out[name] = _bytes(vb * count, device)
        if gs is not None:
            out[name + "_s"] = _bytes(sb * count, device)
    for e in range(count):
        for (name, rows, k, gv, vb, gs, sb) in synth.expert_matrices(cfg, layer,
                                                                     None if shared else e):
            _fill(out[name], gv, synth.scale_gen_count(gv, vb), byte_off=e * vb)
            if gs is not None:
                _fill(out[name + "_s"], gs, synth.scale_gen_count(gs, sb), byte_off=e * sb)
    return out


def state(cfg: synth.Config, sample: int = 0, device="cuda") -> "torch.Tensor":
    """[R][4][H] state bytes of one input sample (zero rows stay zero)."""
    R, H = cfg.rows, cfg.hidden
    ab = synth.act_bytes(cfg.act)
    t = torch.zeros(R * 4 * H * ab, dtype=torch.uint8, device=device)
    for r in range(R):
        if r in cfg.zero_rows:
            continue
        g = synth.Gen(synth.F32_NORMAL if cfg.act == synth.FMT_F32 else synth.BF16_NORMAL,
                      synth.key(cfg.base_seed, synth.TAG_STATE, sample * 16 + r),
                      synth.normal_c(1.0))
        _fill(t, g, 4 * H, byte_off=r * 4 * H * ab)
    return t


def layer(cfg: synth.Config, layer_index: int = 0, device="cuda") -> Dict[str, "torch.Tensor"]:
    out = dense(cfg, layer_index, device)
    out["routed"] = experts(cfg, layer_index, False, device)
    out["shared"] = experts(cfg, layer_index, True, device) if cfg.shared_inter > 0 else None
    return out
