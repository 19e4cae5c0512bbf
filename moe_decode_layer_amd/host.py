"""Host-side marshalling around the C ABI: argument structs from a workload description and
device tensors, and read-back of the intermediates a launch keeps in its workspace.

Argument packing and memory copies only; no step of the layer runs here. `cfg` is any object
with the workload fields (rows, hidden, n_experts, top_k, inter, shared_inter, act,
routed_fmt, shared_fmt, routed_scale, sinkhorn_iters, eps_hc, eps_norm).
"""

from __future__ import annotations

import ctypes
from typing import Dict, Optional

import numpy as np

from . import _binding as B


def shape_of(cfg, rows: Optional[int] = None) -> B.Shape:
    return B.make_shape(cfg.rows if rows is None else rows, cfg.hidden, cfg.n_experts,
                        cfg.top_k, cfg.inter, cfg.shared_inter, cfg.act, cfg.routed_scale,
                        cfg.sinkhorn_iters, cfg.eps_hc, cfg.eps_norm,
                        act_quant=getattr(cfg, "act_quant", "none"))


def experts_struct(fmt: str, t: Optional[Dict]) -> B.Experts:
    """gate, up, down (+ gate_s, up_s, down_s) device tensors of one stacked expert set."""
    if t is None:
        return B.make_experts(fmt, None, None, None)
    return B.make_experts(fmt, t["gate"], t["up"], t["down"], t.get("gate_s"), t.get("up_s"),
                          t.get("down_s"))


def layer_struct(cfg, d: Dict) -> B.Layer:
    """One layer half's weights: d holds w_mix, hc_scale, hc_base, w_norm, w_router, bias and
    the routed and shared expert tensors."""
    return B.make_layer(d["w_mix"], d["hc_scale"], d["hc_base"], d["w_norm"], d["w_router"],
                        d["bias"], experts_struct(cfg.routed_fmt, d["routed"]),
                        experts_struct(cfg.shared_fmt, d["shared"]))


def current_stream() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


_hip = None


def _hip_lib():
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int]
    return _hip


def device_to_host(ptr: int, nbytes: int, dtype, dims) -> np.ndarray:
    """Copies nbytes at device address ptr into a new host array (after the device is idle)."""
    import torch
    buf = np.empty(int(np.prod(dims)), dtype)
    assert buf.nbytes <= nbytes, (buf.nbytes, nbytes)
    torch.cuda.synchronize()
    rc = _hip_lib().hipMemcpy(buf.ctypes.data, ptr, buf.nbytes, 2)  # hipMemcpyDeviceToHost
    if rc != 0:
        raise RuntimeError("hipMemcpy failed with %d" % rc)
    return buf.reshape(dims)


def ws_tensor(shape: B.Shape, ws, which: int, dtype, dims) -> np.ndarray:
    """One intermediate kept in the workspace (MONO_T_*), copied to the host."""
    p, n = B.mono_workspace_tensor(shape, ws, which)
    return device_to_host(p, n, dtype, dims)


def hidden_rows(shape: B.Shape, ws, which: int, act_dtype, dims) -> np.ndarray:
    """Hidden rows (MONO_T_H_ROUTED / MONO_T_H_SHARED) without their tags: each value is stored
    beside the launch tag (bf16 in the low half of a uint32, f32 in the low half of a uint64)."""
    if act_dtype == np.uint16:
        raw = ws_tensor(shape, ws, which, np.uint32, dims)
        return (raw & 0xFFFF).astype(np.uint16)
    raw = ws_tensor(shape, ws, which, np.uint64, dims)
    return (raw & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
