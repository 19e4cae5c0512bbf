"""CPU oracle for the MoE decode layer half (ctypes wrapper of ``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()``
and by the benchmark's ``cpu_baseline`` leg, never by the GPU library. It
shares no code with the GPU library. Every function takes and returns numpy
arrays in the storage formats of the layer: f32 tensors as float32, bf16
activations as uint16 bit patterns, quantised weights as their raw bytes.

Parity pins (tests/test_oracle_*.py) check it against closed forms, invariants
and brute force; the one step with no pin beyond those (the whole-layer
composition) is called "parity unpinned" in the design doc.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MONO_ORACLE_LIB names another build of oracle.c (the pin tests run against planted mistakes
# this way, see tests/test_oracle_mutants.py)
LIB = os.environ.get("MONO_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16, Q8_0, MXFP4 = 0, 1, 2, 3
FMT = {"f32": F32, "bf16": BF16, "q8_0": Q8_0, "mxfp4": MXFP4}
# activation quantisation of the expert matvecs: none, or MXFP8 for the MXFP4 matrices
AQ = {"none": 0, "mxfp8": 1}
N_MIX = 24


CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared"]


def build(src: Optional[str] = None, out: Optional[str] = None) -> None:
    cmd = ["gcc", *CFLAGS, "-o", out or LIB, src or os.path.join(_HERE, "oracle.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stderr)


class Shape(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int), ("hidden", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("inter", ctypes.c_int), ("shared_inter", ctypes.c_int),
                ("act", ctypes.c_int), ("sinkhorn_iters", ctypes.c_int),
                ("routed_scale", ctypes.c_double), ("eps_hc", ctypes.c_double),
                ("eps_norm", ctypes.c_double), ("act_quant", ctypes.c_int)]


class Mat(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("values", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class Expert(ctypes.Structure):
    _fields_ = [("gate", Mat), ("up", Mat), ("down", Mat)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P, SP = ctypes.c_void_p, ctypes.POINTER(Shape)
        for name, args in {
            "or_mix": [SP, P, P, P, P],
            "or_split": [SP, P, P, P, P, P, P],
            "or_collapse_norm": [SP, P, P, P, P, P],
            "or_head": [SP, P, P, P, P, P, P, P, P],
            "or_router_logits": [SP, P, P, P],
            "or_select": [SP, P, P, P, P, P],
            "or_expert_hidden": [SP, ctypes.c_int, ctypes.POINTER(Expert), P, P],
            "or_moe": [SP, P, P, P, ctypes.POINTER(Expert), ctypes.POINTER(Expert), ctypes.c_int,
                       P, P, P, P, P],
            "or_expand": [SP, P, P, P, P, P, P, P],
        }.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.or_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_f64.restype = ctypes.c_double
        L.or_f32_to_bf16.argtypes = [ctypes.c_float]
        L.or_f32_to_bf16.restype = ctypes.c_uint16
        L.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.or_f16_to_f64.restype = ctypes.c_double
        L.or_e2m1_to_f64.argtypes = [ctypes.c_uint]
        L.or_e2m1_to_f64.restype = ctypes.c_double
        L.or_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        L.or_e8m0_to_f64.restype = ctypes.c_double
        L.or_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        L.or_e4m3_to_f64.restype = ctypes.c_double
        L.or_mxfp8_quant.argtypes = [P, ctypes.c_int, P, P]
        L.or_mxfp8_quant.restype = ctypes.c_int
        L.or_mat_elem.argtypes = [ctypes.POINTER(Mat), ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_int64]
        L.or_mat_elem.restype = ctypes.c_double
        L.or_threads.restype = ctypes.c_int
        L.or_set_threads.argtypes = [ctypes.c_int]
        L.or_set_threads.restype = None
        _lib = L
    return _lib


def threads() -> int:
    return int(lib().or_threads())


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError("oracle %s failed (%d)" % (what, rc))


def make_shape(rows, hidden, n_experts, top_k, inter, shared_inter, act, routed_scale,
               sinkhorn_iters=20, eps_hc=1e-6, eps_norm=1e-6, act_quant="none") -> Shape:
    return Shape(rows, hidden, n_experts, top_k, inter, shared_inter,
                 F32 if act == "f32" else BF16, sinkhorn_iters, routed_scale, eps_hc, eps_norm,
                 AQ[act_quant])


def shape_of(cfg, rows: Optional[int] = None) -> Shape:
    return make_shape(cfg.rows if rows is None else rows, cfg.hidden, cfg.n_experts, cfg.top_k,
                      cfg.inter, cfg.shared_inter, cfg.act, cfg.routed_scale, cfg.sinkhorn_iters,
                      cfg.eps_hc, cfg.eps_norm, getattr(cfg, "act_quant", "none"))


def _act_dtype(s: Shape):
    return np.float32 if s.act == F32 else np.uint16


def mix(s: Shape, state=None, w_mix=None, carry=None) -> np.ndarray:
    out = np.zeros((s.rows, N_MIX), np.float32)
    _check(lib().or_mix(ctypes.byref(s), _p(state), _p(w_mix), _p(carry), _p(out)), "mix")
    return out


def split(s: Shape, mixes, hc_scale, hc_base):
    pre = np.zeros((s.rows, 4), np.float32)
    post = np.zeros((s.rows, 4), np.float32)
    comb = np.zeros((s.rows, 4, 4), np.float32)
    _check(lib().or_split(ctypes.byref(s), _p(mixes), _p(hc_scale), _p(hc_base), _p(pre),
                          _p(post), _p(comb)), "split")
    return pre, post, comb


def collapse_norm(s: Shape, state, pre, w_norm):
    x = np.zeros((s.rows, s.hidden), _act_dtype(s))
    norm = np.zeros((s.rows, s.hidden), _act_dtype(s))
    _check(lib().or_collapse_norm(ctypes.byref(s), _p(state), _p(pre), _p(w_norm), _p(x),
                                  _p(norm)), "collapse_norm")
    return x, norm


def head(s: Shape, state, w_head, head_scale, head_base, w_norm):
    """Model tail: (pre [R][4], x [R][H], norm [R][H]) without a split."""
    pre = np.zeros((s.rows, 4), np.float32)
    x = np.zeros((s.rows, s.hidden), _act_dtype(s))
    norm = np.zeros((s.rows, s.hidden), _act_dtype(s))
    _check(lib().or_head(ctypes.byref(s), _p(state), _p(w_head), _p(head_scale), _p(head_base),
                         _p(w_norm), _p(pre), _p(x), _p(norm)), "head")
    return pre, x, norm


def router_logits(s: Shape, norm, w_router) -> np.ndarray:
    out = np.zeros((s.rows, s.n_experts), np.float32)
    _check(lib().or_router_logits(ctypes.byref(s), _p(norm), _p(w_router), _p(out)), "logits")
    return out


def select(s: Shape, logits, bias):
    idx = np.zeros((s.rows, s.top_k), np.int32)
    w = np.zeros((s.rows, s.top_k), np.float32)
    beta = np.zeros((s.rows, s.n_experts), np.float32)
    _check(lib().or_select(ctypes.byref(s), _p(logits), _p(bias), _p(idx), _p(w), _p(beta)),
           "select")
    return idx, w, beta


def _mat(fmt: int, values, scales) -> Mat:
    return Mat(fmt, _p(values), _p(scales))


def expert_struct(fmt: str, tensors: Optional[Dict[str, np.ndarray]]) -> Expert:
    """tensors: dict with gate, up, down (+ gate_s, up_s, down_s) as produced by synth."""
    if tensors is None:
        return Expert()
    f = FMT[fmt]
    return Expert(_mat(f, tensors["gate"], tensors.get("gate_s")),
                  _mat(f, tensors["up"], tensors.get("up_s")),
                  _mat(f, tensors["down"], tensors.get("down_s")))


def expert_hidden(s: Shape, inter: int, fmt: str, tensors, norm_row) -> np.ndarray:
    h = np.zeros(inter, _act_dtype(s))
    ex = expert_struct(fmt, tensors)
    _check(lib().or_expert_hidden(ctypes.byref(s), inter, ctypes.byref(ex), _p(norm_row), _p(h)),
           "expert_hidden")
    return h


def moe(s: Shape, norm, idx, weights, routed_fmt: str, routed: Dict[int, Dict[str, np.ndarray]],
        shared_fmt: str, shared: Optional[Dict[str, np.ndarray]], h_routed=None, h_shared=None):
    """Routed experts given as {expert: tensors} (only the selected ones are needed).

    When h_routed / h_shared are given, the down projections use them (teacher forcing)."""
    E = s.n_experts
    arr = (Expert * E)()
    for e, t in routed.items():
        arr[e] = expert_struct(routed_fmt, t)
    sh = expert_struct(shared_fmt, shared)
    dt = _act_dtype(s)
    force = h_routed is not None
    if force:
        hr = np.ascontiguousarray(h_routed, dtype=dt).reshape(s.rows, s.top_k, s.inter)
        hs = np.ascontiguousarray(h_shared, dtype=dt).reshape(s.rows, s.shared_inter)
    else:
        hr = np.zeros((s.rows, s.top_k, s.inter), dt)
        hs = np.zeros((s.rows, s.shared_inter), dt)
    shared_out = np.zeros((s.rows, s.hidden), dt)
    routed_out = np.zeros((s.rows, s.hidden), np.float32)
    block = np.zeros((s.rows, s.hidden), dt)
    _check(lib().or_moe(ctypes.byref(s), _p(norm), _p(np.ascontiguousarray(idx, np.int32)),
                        _p(np.ascontiguousarray(weights, np.float32)), arr, ctypes.byref(sh),
                        1 if force else 0, _p(hr), _p(hs), _p(shared_out), _p(routed_out),
                        _p(block)), "moe")
    return {"h_routed": hr, "h_shared": hs, "shared": shared_out, "routed": routed_out,
            "block": block}


def expand(s: Shape, state, block, post, comb, w_mix_next=None):
    new = np.zeros((s.rows, 4, s.hidden), _act_dtype(s))
    carry = np.zeros((s.rows, N_MIX + 1), np.float32) if w_mix_next is not None else None
    _check(lib().or_expand(ctypes.byref(s), _p(state), _p(block), _p(post), _p(comb),
                           _p(w_mix_next), _p(new), _p(carry)), "expand")
    return new, carry


def layer(s: Shape, state, dense, routed_fmt, routed_get, shared_fmt, shared,
          w_mix_next=None, carry_in=None, force=None) -> Dict[str, np.ndarray]:
    """The whole unfused chain for one layer half.

    routed_get(expert) -> tensors (called for each selected expert). `force` may hold
    GPU-produced "idx"/"weights" to run the expert steps on that selection."""
    out = {}
    out["mixes"] = mix(s, state, dense["w_mix"], carry_in)
    out["pre"], out["post"], out["comb"] = split(s, out["mixes"], dense["hc_scale"],
                                                 dense["hc_base"])
    out["x"], out["norm"] = collapse_norm(s, state, out["pre"], dense["w_norm"])
    out["logits"] = router_logits(s, out["norm"], dense["w_router"])
    out["idx"], out["weights"], out["beta_sorted"] = select(s, out["logits"], dense["bias"])
    idx, w = out["idx"], out["weights"]
    if force is not None:
        idx, w = force["idx"], force["weights"]
    experts = {int(e): routed_get(int(e)) for e in np.unique(idx)}
    m = moe(s, out["norm"], idx, w, routed_fmt, experts, shared_fmt, shared)
    out.update(m)
    out["new_state"], out["carry"] = expand(s, state, m["block"], out["post"], out["comb"],
                                            w_mix_next)
    return out


# format helpers (exact)
def bf16_to_f64(b: int) -> float:
    return float(lib().or_bf16_to_f64(b))


def f32_to_bf16(f: float) -> int:
    return int(lib().or_f32_to_bf16(f))


def f16_to_f64(h: int) -> float:
    return float(lib().or_f16_to_f64(h))


def e2m1_to_f64(c: int) -> float:
    return float(lib().or_e2m1_to_f64(c))


def e8m0_to_f64(e: int) -> float:
    return float(lib().or_e8m0_to_f64(e))


def e4m3_to_f64(c: int) -> float:
    return float(lib().or_e4m3_to_f64(c))


def mxfp8_quant(v) -> tuple:
    """MXFP8 quantisation of a vector (length a multiple of 32): (E4M3 codes, e8m0 scales)."""
    x = np.ascontiguousarray(v, dtype=np.float64)
    codes = np.zeros(x.size, np.uint8)
    scales = np.zeros(x.size // 32, np.uint8)
    _check(lib().or_mxfp8_quant(_p(x), x.size, _p(codes), _p(scales)), "mxfp8_quant")
    return codes, scales


def mat_elem(fmt: str, values, scales, k: int, row: int, col: int) -> float:
    m = _mat(FMT[fmt], values, scales)
    return float(lib().or_mat_elem(ctypes.byref(m), k, row, col))
