"""ctypes binding of libmonolayer (include/mono.h): argument marshalling only.

Every function has the name of the C entry point it calls, takes device
pointers as Python ints (or objects with ``data_ptr()``, e.g. torch tensors)
and raises MonoError with the library's full list of failed checks on a
negative status. No step of the layer runs here.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmonolayer.so")

MONO_F32, MONO_BF16, MONO_Q8_0, MONO_MXFP4 = 0, 1, 2, 3
FMT = {"f32": MONO_F32, "bf16": MONO_BF16, "q8_0": MONO_Q8_0, "mxfp4": MONO_MXFP4}
MONO_AQ_NONE, MONO_AQ_MXFP8 = 0, 1
AQ = {"none": MONO_AQ_NONE, "mxfp8": MONO_AQ_MXFP8}
MONO_OK, MONO_E_INVAL, MONO_E_UNSUPPORTED, MONO_E_DEVICE, MONO_E_TIMEOUT = 0, -1, -2, -3, -4
(MONO_T_MIXES, MONO_T_PRE, MONO_T_POST, MONO_T_COMB, MONO_T_X, MONO_T_NORM, MONO_T_LOGITS,
 MONO_T_IDX, MONO_T_WEIGHTS, MONO_T_H_ROUTED, MONO_T_H_SHARED, MONO_T_SHARED, MONO_T_ROUTED,
 MONO_T_BLOCK, MONO_T_CARRY, MONO_T_TRACE) = range(16)

EXPORTS = ("mono_workspace_bytes", "mono_workspace_init", "mono_workspace_poll",
           "mono_workspace_set_debug", "mono_workspace_set_trace", "mono_workspace_set_jitter",
           "mono_workspace_tensor", "mono_last_error",
           "mono_grid_size", "mono_hc_mix_collapse", "mono_router_select", "mono_moe_experts",
           "mono_hc_expand", "mono_hc_head", "mono_ffn_layer", "mono_ffn_layer_static")
MONO_STATIC_WS_BYTES = 8 << 20
MONO_JITTER_MAX_TICKS = 10000


class MonoError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("mono status %d: %s" % (status, message))
        self.status = status
        self.message = message


class Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int), ("hidden", ctypes.c_int), ("n_streams", ctypes.c_int),
                ("n_experts", ctypes.c_int), ("top_k", ctypes.c_int), ("inter", ctypes.c_int),
                ("shared_inter", ctypes.c_int), ("act", ctypes.c_int),
                ("routed_scale", ctypes.c_float), ("sinkhorn_iters", ctypes.c_int),
                ("eps_hc", ctypes.c_float), ("eps_norm", ctypes.c_float),
                ("act_quant", ctypes.c_int)]


class Experts(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("gate_s", ctypes.c_void_p),
                ("up_s", ctypes.c_void_p), ("down_s", ctypes.c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("w_mix", ctypes.c_void_p), ("hc_scale", ctypes.c_void_p),
                ("hc_base", ctypes.c_void_p), ("w_norm", ctypes.c_void_p),
                ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("routed", Experts), ("shared", Experts)]


class Head(ctypes.Structure):
    _fields_ = [("w_head", ctypes.c_void_p), ("head_scale", ctypes.c_void_p),
                ("head_base", ctypes.c_void_p), ("w_norm", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libmonolayer.so; raises if it is not built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libmonolayer.so is not built: run __graft_entry__.build() "
                              "(expected at %s)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, SP, I = ctypes.c_void_p, ctypes.POINTER(Shape), ctypes.c_int
        LP = ctypes.POINTER(Layer)
        sig = {
            "mono_workspace_bytes": (ctypes.c_size_t, [SP]),
            "mono_workspace_init": (I, [P, SP, P]),
            "mono_workspace_poll": (I, [P, ctypes.POINTER(ctypes.c_uint32), P]),
            "mono_workspace_set_debug": (I, [P, ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, P]),
            "mono_workspace_set_trace": (I, [P, I, P]),
            "mono_workspace_set_jitter": (I, [P, ctypes.c_uint32, ctypes.c_uint32]),
            "mono_workspace_tensor": (I, [SP, P, I, ctypes.POINTER(ctypes.c_void_p),
                                          ctypes.POINTER(ctypes.c_size_t)]),
            "mono_last_error": (ctypes.c_char_p, []),
            "mono_grid_size": (I, []),
            "mono_hc_mix_collapse": (I, [SP, P, LP, P, P, P, P, P, P, P, P, P]),
            "mono_router_select": (I, [SP, P, LP, P, P, P, P, P]),
            "mono_moe_experts": (I, [SP, P, P, P, LP, P, P, P, P, P]),
            "mono_hc_expand": (I, [SP, P, P, P, P, P, P, P, P, P]),
            "mono_hc_head": (I, [SP, P, ctypes.POINTER(Head), P, P, P, P]),
            "mono_ffn_layer": (I, [SP, LP, P, P, P, P, P, P, P]),
            "mono_ffn_layer_static": (I, [SP, LP, P, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def ptr(x) -> Optional[int]:
    """Device address of a tensor-like (data_ptr()), an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr()


def _ok(status: int) -> None:
    if status != MONO_OK:
        raise MonoError(status, mono_last_error())


def make_shape(rows, hidden, n_experts, top_k, inter, shared_inter, act="bf16",
               routed_scale=1.0, sinkhorn_iters=20, eps_hc=1e-6, eps_norm=1e-6,
               n_streams=4, act_quant="none") -> Shape:
    return Shape(rows, hidden, n_streams, n_experts, top_k, inter, shared_inter,
                 FMT[act] if isinstance(act, str) else act, routed_scale, sinkhorn_iters,
                 eps_hc, eps_norm, AQ[act_quant] if isinstance(act_quant, str) else act_quant)


def make_experts(fmt, gate, up, down, gate_s=None, up_s=None, down_s=None) -> Experts:
    return Experts(FMT[fmt] if isinstance(fmt, str) else fmt, ptr(gate), ptr(up), ptr(down),
                   ptr(gate_s), ptr(up_s), ptr(down_s))


def make_layer(w_mix, hc_scale, hc_base, w_norm, w_router, bias, routed: Experts,
               shared: Experts) -> Layer:
    return Layer(ptr(w_mix), ptr(hc_scale), ptr(hc_base), ptr(w_norm), ptr(w_router), ptr(bias),
                 routed, shared)


def make_head(w_head, head_scale, head_base, w_norm) -> Head:
    return Head(ptr(w_head), ptr(head_scale), ptr(head_base), ptr(w_norm))


def mono_last_error() -> str:
    return lib().mono_last_error().decode()


def mono_grid_size() -> int:
    return int(lib().mono_grid_size())


def mono_workspace_bytes(shape: Shape) -> int:
    n = int(lib().mono_workspace_bytes(ctypes.byref(shape)))
    if n == 0:
        raise MonoError(MONO_E_INVAL, mono_last_error())
    return n


def mono_workspace_init(ws, shape: Shape, stream=None) -> None:
    _ok(lib().mono_workspace_init(ptr(ws), ctypes.byref(shape), stream))


def mono_workspace_set_debug(ws, spin_limit_ticks=0, fault_wg=-1, fault_phase=0,
                             stream=None) -> None:
    _ok(lib().mono_workspace_set_debug(ptr(ws), spin_limit_ticks, fault_wg, fault_phase, stream))


def mono_workspace_set_trace(ws, enable=True, stream=None) -> None:
    _ok(lib().mono_workspace_set_trace(ptr(ws), 1 if enable else 0, stream))


def mono_workspace_set_jitter(ws, max_ticks=0, seed=0) -> None:
    _ok(lib().mono_workspace_set_jitter(ptr(ws), max_ticks, seed))


def mono_workspace_poll(ws, stream=None):
    """Returns (status, [flag, phase, workgroup, count]) without raising on a timeout."""
    err = (ctypes.c_uint32 * 4)()
    st = lib().mono_workspace_poll(ptr(ws), err, stream)
    if st not in (MONO_OK, MONO_E_TIMEOUT):
        raise MonoError(st, mono_last_error())
    return st, list(err)


def mono_workspace_tensor(shape: Shape, ws, which: int):
    p = ctypes.c_void_p()
    n = ctypes.c_size_t()
    _ok(lib().mono_workspace_tensor(ctypes.byref(shape), ptr(ws), which, ctypes.byref(p),
                                    ctypes.byref(n)))
    return int(p.value or 0), int(n.value)


def mono_hc_mix_collapse(shape, state, layer, carry_in, mixes, pre, post, comb, x, norm, ws,
                         stream=None) -> None:
    _ok(lib().mono_hc_mix_collapse(ctypes.byref(shape), ptr(state), ctypes.byref(layer),
                                   ptr(carry_in), ptr(mixes), ptr(pre), ptr(post), ptr(comb),
                                   ptr(x), ptr(norm), ptr(ws), stream))


def mono_router_select(shape, norm, layer, logits, idx, weights, ws, stream=None) -> None:
    _ok(lib().mono_router_select(ctypes.byref(shape), ptr(norm), ctypes.byref(layer), ptr(logits),
                                 ptr(idx), ptr(weights), ptr(ws), stream))


def mono_moe_experts(shape, norm, idx, weights, layer, shared_out, routed_out, block, ws,
                     stream=None) -> None:
    _ok(lib().mono_moe_experts(ctypes.byref(shape), ptr(norm), ptr(idx), ptr(weights),
                               ctypes.byref(layer), ptr(shared_out), ptr(routed_out), ptr(block),
                               ptr(ws), stream))


def mono_hc_expand(shape, state, block, post, comb, w_mix_next, new_state, carry_out, ws,
                   stream=None) -> None:
    _ok(lib().mono_hc_expand(ctypes.byref(shape), ptr(state), ptr(block), ptr(post), ptr(comb),
                             ptr(w_mix_next), ptr(new_state), ptr(carry_out), ptr(ws), stream))


def mono_hc_head(shape, state, head, pre, x, norm, stream=None) -> None:
    _ok(lib().mono_hc_head(ctypes.byref(shape), ptr(state), ctypes.byref(head), ptr(pre), ptr(x),
                           ptr(norm), stream))


def mono_ffn_layer(shape, layer, w_mix_next, state_in, carry_in, state_out, carry_out, ws,
                   stream=None) -> None:
    _ok(lib().mono_ffn_layer(ctypes.byref(shape), ctypes.byref(layer), ptr(w_mix_next),
                             ptr(state_in), ptr(carry_in), ptr(state_out), ptr(carry_out),
                             ptr(ws), stream))


def mono_ffn_layer_static(shape, layer, w_mix_next, state_in, carry_in, state_out, carry_out,
                          stream=None) -> None:
    _ok(lib().mono_ffn_layer_static(ctypes.byref(shape), ctypes.byref(layer), ptr(w_mix_next),
                                    ptr(state_in), ptr(carry_in), ptr(state_out), ptr(carry_out),
                                    stream))
