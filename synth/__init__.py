"""Seeded synthetic inputs for the MoE decode layer half.

Test and benchmark infrastructure shared by the CPU oracle side and the GPU
side. It holds no step of the method: only the workload recipes (shapes,
formats, value distributions, seeds) and the counter-based generator of
``synth_core.h`` in a host build (``libsynth.so``) and a device build
(``libsynth_dev.so``). Every element is a pure function of
(seed, tensor tag, sub-index, flat index), so a host fill and a device fill of
the same tensor hold the same bytes.

Workloads (stand-ins for the pages' decode widths of 1, 6 and 8 rows; no
checkpoint or dataset is used):

1. tiny fp32 layer half, 1 row: hidden 256, 8 routed experts top-2, inter 128,
   one shared expert (inter 128), scale 1.0, everything f32;
2. V4.1-like half, 1 row, bf16 experts: hidden 5120, 256 experts top-8,
   inter 2048, shared inter 2048, f32 mix and router weights, scale 2.5;
3. the same shapes at 6 rows, routed and shared experts Q8_0 (int8 blocks of 32
   with an fp16 scale per block);
4. the same shapes at 8 rows, routed experts MXFP4 (e2m1 codes, e8m0 scale per
   32), shared expert bf16, row 7 all zeros and the router bias constant over
   groups of 32 consecutive experts, so the zero row ties inside groups;
5. eight consecutive layer halves of workload 2, independent weights.

Distributions: states N(0,1); mix, router and f32/bf16 expert weights
N(0, 0.02); router bias U(-0.1, 0.1); hc base U(-1, 1); hc scale fixed
(0.12, 0.08, 0.10); norm weight U(0.5, 1.5); Q8_0 values uniform on
[-127, 127] and scales U(1e-4, 1e-3) rounded to fp16; MXFP4 codes uniform over
all 16 and e8m0 exponents uniform on [-8, -4].
"""

from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Dict, Iterable, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(_HERE, "libsynth.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")

# encodings (synth_core.h)
F32_NORMAL, BF16_NORMAL, F32_UNIFORM, BF16_UNIFORM, F16_UNIFORM, I8_UNIFORM, BYTES, E8M0 = range(8)
_ELEM = {F32_NORMAL: 4, F32_UNIFORM: 4, BF16_NORMAL: 2, BF16_UNIFORM: 2, F16_UNIFORM: 2,
         I8_UNIFORM: 1, BYTES: 1, E8M0: 1}
_NP = {F32_NORMAL: np.float32, F32_UNIFORM: np.float32, BF16_NORMAL: np.uint16,
       BF16_UNIFORM: np.uint16, F16_UNIFORM: np.uint16, I8_UNIFORM: np.int8, BYTES: np.uint8,
       E8M0: np.uint8}

# tensor tags
TAG_STATE, TAG_W_MIX, TAG_HC_BASE, TAG_W_NORM, TAG_W_ROUTER, TAG_BIAS = 1, 2, 3, 4, 5, 6
TAG_GATE, TAG_UP, TAG_DOWN, TAG_GATE_S, TAG_UP_S, TAG_DOWN_S = 7, 8, 9, 10, 11, 12
TAG_W_HEAD, TAG_HEAD_BASE, TAG_W_OUT_NORM, TAG_ATTN_GAIN = 13, 14, 15, 16
SHARED_INDEX = 0x80000000

HC_SCALE = (0.12, 0.08, 0.10)
N_STREAMS = 4
N_MIX = 24
BLOCK = 32
BIAS_GROUP = 32


def build(verbose: bool = False) -> None:
    """Compiles libsynth.so (gcc) and, when hipcc exists, libsynth_dev.so."""
    cmds = [["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
             "-o", HOST_LIB, os.path.join(_HERE, "synth_host.c")]]
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if os.path.exists(hipcc):
        cmds.append([hipcc, "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC",
                     "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                     "-o", DEV_LIB, os.path.join(_HERE, "synth_dev.hip")])
    for c in cmds:
        r = subprocess.run(c, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("synth build failed: %s\n%s" % (" ".join(c), r.stderr))
        if verbose and r.stderr:
            print(r.stderr)


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build()
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_key.restype = ctypes.c_uint64
        lib.synth_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_draw.restype = ctypes.c_uint64
        lib.synth_draw.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint64, ctypes.c_float, ctypes.c_float, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_int]
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError("libsynth_dev.so is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_fill_device.restype = ctypes.c_int
        lib.synth_fill_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_float,
                                          ctypes.c_float, ctypes.c_int32, ctypes.c_int32,
                                          ctypes.c_void_p]
        _dev = lib
    return _dev


def key(seed: int, tag: int, index: int) -> int:
    return int(_host_lib().synth_key(seed & (2**64 - 1), tag, index & 0xFFFFFFFF))


def draw(k: int, n: int) -> int:
    return int(_host_lib().synth_draw(k, n))


@dataclasses.dataclass(frozen=True)
class Gen:
    """One tensor's stream: encoding, key and parameters."""
    kind: int
    key: int
    p0: float = 0.0
    p1: float = 0.0
    i0: int = 0
    i1: int = 0


def normal_c(sigma: float) -> float:
    return float(np.float32(sigma * math.sqrt(3.0) / 65536.0))


def fill_host(g: Gen, count: int, first: int = 0, out: Optional[np.ndarray] = None,
              threads: int = 0) -> np.ndarray:
    if out is None:
        out = np.empty(count, dtype=_NP[g.kind])
    assert out.flags.c_contiguous and out.nbytes == count * _ELEM[g.kind]
    if threads <= 0:
        threads = min(16, os.cpu_count() or 1)
    rc = _host_lib().synth_fill(out.ctypes.data, g.kind, g.key, first, count, g.p0, g.p1, g.i0,
                                g.i1, threads)
    if rc != 0:
        raise RuntimeError("synth_fill failed")
    return out


def fill_device(g: Gen, ptr: int, count: int, first: int = 0, stream: int = 0) -> None:
    rc = _dev_lib().synth_fill_device(ptr, g.kind, g.key, first, count, g.p0, g.p1, g.i0, g.i1,
                                      stream)
    if rc != 0:
        raise RuntimeError("synth_fill_device failed with hip error %d" % rc)


# ---------------------------------------------------------------------------------------------
# workloads

FMT_F32, FMT_BF16, FMT_Q8_0, FMT_MXFP4 = "f32", "bf16", "q8_0", "mxfp4"


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    rows: int
    hidden: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    act: str
    routed_fmt: str
    shared_fmt: str
    routed_scale: float
    sinkhorn_iters: int = 20
    eps_hc: float = 1e-6
    eps_norm: float = 1e-6
    grouped_bias: bool = False
    zero_rows: tuple = ()
    layers: int = 1
    act_quant: str = "none"  # "mxfp8": activations of the MXFP4 experts quantised to MXFP8

    @property
    def base_seed(self) -> int:
        return 1000 * self.index

    def layer_seed(self, layer: int) -> int:
        return self.base_seed + layer

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[int, Config] = {
    1: Config(1, "tiny fp32 layer half, 1 row", 1, 256, 8, 2, 128, 128, FMT_F32, FMT_F32, FMT_F32,
              1.0),
    2: Config(2, "V4.1-like MoE half, 1 row, bf16 experts", 1, 5120, 256, 8, 2048, 2048, FMT_BF16,
              FMT_BF16, FMT_BF16, 2.5),
    3: Config(3, "V4.1-like MoE half, 6 rows, Q8_0 experts", 6, 5120, 256, 8, 2048, 2048, FMT_BF16,
              FMT_Q8_0, FMT_Q8_0, 2.5),
    4: Config(4, "V4.1-like MoE half, 8 rows, MXFP4 routed + bf16 shared, zero row", 8, 5120, 256, 8,
              2048, 2048, FMT_BF16, FMT_MXFP4, FMT_BF16, 2.5, grouped_bias=True, zero_rows=(7,)),
    5: Config(5, "chain of 8 V4.1-like bf16 layer halves, 1 row", 1, 5120, 256, 8, 2048, 2048,
              FMT_BF16, FMT_BF16, FMT_BF16, 2.5, layers=8),
    # draft-stage routing shapes: 128 experts with top-3 (the draft stages) and 256 experts
    # with top-6 (the single-box ds4 router), at the same hidden and expert widths
    6: Config(6, "draft MoE half, 128 experts top-3, 1 row, bf16 experts", 1, 5120, 128, 3, 2048,
              2048, FMT_BF16, FMT_BF16, FMT_BF16, 2.5),
    7: Config(7, "draft MoE half, 128 experts top-3, 6 rows, Q8_0 experts", 6, 5120, 128, 3, 2048,
              2048, FMT_BF16, FMT_Q8_0, FMT_Q8_0, 2.5),
    8: Config(8, "MoE half, 256 experts top-6, 1 row, bf16 experts", 1, 5120, 256, 6, 2048, 2048,
              FMT_BF16, FMT_BF16, FMT_BF16, 2.5),
    9: Config(9, "MoE half, 256 experts top-6, 6 rows, Q8_0 experts", 6, 5120, 256, 6, 2048, 2048,
              FMT_BF16, FMT_Q8_0, FMT_Q8_0, 2.5),
    # workload 4 with the activations of the MXFP4 experts quantised to MXFP8 (E4M3, e8m0 per 32)
    10: Config(10, "V4.1-like MoE half, 8 rows, MXFP4 routed with MXFP8 activations + bf16 shared, "
               "zero row", 8, 5120, 256, 8, 2048, 2048, FMT_BF16, FMT_MXFP4, FMT_BF16, 2.5,
               grouped_bias=True, zero_rows=(7,), act_quant="mxfp8"),
}
DRAFT_CONFIGS = (6, 7, 8, 9)


def _act_normal(act: str) -> int:
    return F32_NORMAL if act == FMT_F32 else BF16_NORMAL


def _act_uniform(act: str) -> int:
    return F32_UNIFORM if act == FMT_F32 else BF16_UNIFORM


def act_np(act: str):
    return np.float32 if act == FMT_F32 else np.uint16


def act_bytes(act: str) -> int:
    return 4 if act == FMT_F32 else 2


def matrix_specs(fmt: str, rows: int, k: int, seed: int, tag_v: int, tag_s: int, index: int):
    """Streams and byte sizes of one [rows][k] expert matrix in `fmt`.

    Returns (values Gen, values bytes, scales Gen or None, scales bytes). Q8_0 and MXFP4 use
    blocks of 32 along k; MXFP4 packs two codes per byte, low nibble first.
    """
    n = rows * k
    if fmt == FMT_F32:
        return Gen(F32_NORMAL, key(seed, tag_v, index), normal_c(0.02)), 4 * n, None, 0
    if fmt == FMT_BF16:
        return Gen(BF16_NORMAL, key(seed, tag_v, index), normal_c(0.02)), 2 * n, None, 0
    nb = n // BLOCK
    if fmt == FMT_Q8_0:
        lo, hi = np.float32(1e-4), np.float32(1e-3)
        return (Gen(I8_UNIFORM, key(seed, tag_v, index)), n,
                Gen(F16_UNIFORM, key(seed, tag_s, index), float(lo), float(np.float32(hi - lo))),
                2 * nb)
    if fmt == FMT_MXFP4:
        return (Gen(BYTES, key(seed, tag_v, index)), n // 2,
                Gen(E8M0, key(seed, tag_s, index), i0=-8, i1=-4), nb)
    raise ValueError(fmt)


def expert_bytes(fmt: str, inter: int, hidden: int) -> int:
    tot = 0
    for rows, k in ((inter, hidden), (inter, hidden), (hidden, inter)):
        _, vb, _, sb = matrix_specs(fmt, rows, k, 0, TAG_GATE, TAG_GATE_S, 0)
        tot += vb + sb
    return tot


def expert_matrices(cfg: Config, layer: int, expert: Optional[int]):
    """[(name, rows, k, values Gen, values bytes, scales Gen, scales bytes)] for gate, up, down.

    expert=None selects the shared expert."""
    seed = cfg.layer_seed(layer)
    if expert is None:
        fmt, inter, idx = cfg.shared_fmt, cfg.shared_inter, SHARED_INDEX
    else:
        fmt, inter, idx = cfg.routed_fmt, cfg.inter, expert
    out = []
    for name, rows, k, tv, ts in (("gate", inter, cfg.hidden, TAG_GATE, TAG_GATE_S),
                                  ("up", inter, cfg.hidden, TAG_UP, TAG_UP_S),
                                  ("down", cfg.hidden, inter, TAG_DOWN, TAG_DOWN_S)):
        gv, vb, gs, sb = matrix_specs(fmt, rows, k, seed, tv, ts, idx)
        out.append((name, rows, k, gv, vb, gs, sb))
    return out


def dense_specs(cfg: Config, layer: int):
    """Streams of the per-layer dense tensors: name -> (Gen or None, count, numpy dtype)."""
    seed = cfg.layer_seed(layer)
    H, E = cfg.hidden, cfg.n_experts
    uni = lambda lo, hi: (float(np.float32(lo)), float(np.float32(np.float32(hi) - np.float32(lo))))
    lo, w = uni(-1.0, 1.0)
    specs = {
        "w_mix": (Gen(F32_NORMAL, key(seed, TAG_W_MIX, 0), normal_c(0.02)), N_MIX * N_STREAMS * H,
                  np.float32),
        "hc_base": (Gen(F32_UNIFORM, key(seed, TAG_HC_BASE, 0), lo, w), N_MIX, np.float32),
        "w_router": (Gen(F32_NORMAL, key(seed, TAG_W_ROUTER, 0), normal_c(0.02)), E * H,
                     np.float32),
    }
    lo, w = uni(0.5, 1.5)
    specs["w_norm"] = (Gen(_act_uniform(cfg.act), key(seed, TAG_W_NORM, 0), lo, w), H,
                       act_np(cfg.act))
    lo, w = uni(-0.1, 0.1)
    nb = (E + BIAS_GROUP - 1) // BIAS_GROUP if cfg.grouped_bias else E
    specs["bias"] = (Gen(F32_UNIFORM, key(seed, TAG_BIAS, 0), lo, w), nb, np.float32)
    return specs


# the attention half of layer l uses the dense HC tensors (w_mix, hc_scale, hc_base, w_norm) of
# layer ATTN_LAYER + l, drawn like a layer half's
ATTN_LAYER = 500
HEAD_SCALE = 0.12


def head_specs(cfg: Config):
    """Streams of the model-tail head: its 4-row mix, 4 biases and the output norm weight."""
    seed = cfg.base_seed
    H = cfg.hidden
    uni = lambda lo, hi: (float(np.float32(lo)), float(np.float32(np.float32(hi) - np.float32(lo))))
    lo, w = uni(-1.0, 1.0)
    specs = {
        "w_head": (Gen(F32_NORMAL, key(seed, TAG_W_HEAD, 0), normal_c(0.02)), N_STREAMS * N_STREAMS * H,
                   np.float32),
        "head_base": (Gen(F32_UNIFORM, key(seed, TAG_HEAD_BASE, 0), lo, w), N_STREAMS, np.float32),
    }
    lo, w = uni(0.5, 1.5)
    specs["w_norm"] = (Gen(_act_uniform(cfg.act), key(seed, TAG_W_OUT_NORM, 0), lo, w), H,
                       act_np(cfg.act))
    return specs


def head_host(cfg: Config) -> Dict[str, np.ndarray]:
    out = {name: fill_host(g, n) for name, (g, n, dt) in head_specs(cfg).items()}
    out["w_head"] = out["w_head"].reshape(N_STREAMS, N_STREAMS * cfg.hidden)
    out["head_scale"] = np.array([HEAD_SCALE], dtype=np.float32)
    return out


def attn_gain_host(cfg: Config, layer: int) -> np.ndarray:
    """Per-position gains [H] of the stand-in attention of layer `layer` (uniform in [-1, 1])."""
    lo, w = float(np.float32(-1.0)), float(np.float32(2.0))
    return fill_host(Gen(F32_UNIFORM, key(cfg.layer_seed(layer), TAG_ATTN_GAIN, 0), lo, w),
                     cfg.hidden)


def dense_host(cfg: Config, layer: int) -> Dict[str, np.ndarray]:
    out = {}
    for name, (g, n, dt) in dense_specs(cfg, layer).items():
        out[name] = fill_host(g, n)
    if cfg.grouped_bias:
        v = out["bias"]
        out["bias"] = np.repeat(v, BIAS_GROUP)[: cfg.n_experts].copy()
    out["hc_scale"] = np.array(HC_SCALE, dtype=np.float32)
    H = cfg.hidden
    out["w_mix"] = out["w_mix"].reshape(N_MIX, N_STREAMS * H)
    out["w_router"] = out["w_router"].reshape(cfg.n_experts, H)
    return out


def expert_host(cfg: Config, layer: int, expert: Optional[int]) -> Dict[str, np.ndarray]:
    """One expert's matrices on the host: gate/up/down values (+ *_s scales), row-major."""
    out = {}
    for name, rows, k, gv, vb, gs, sb in expert_matrices(cfg, layer, expert):
        v = fill_host(gv, vb // _ELEM[gv.kind])
        out[name] = v.reshape(rows, -1)
        if gs is not None:
            out[name + "_s"] = fill_host(gs, sb // _ELEM[gs.kind]).reshape(rows, -1)
    return out


def state_host(cfg: Config, sample: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """[rows][4][H] HC state of input `sample` (act storage: f32 or bf16 bits)."""
    R = cfg.rows if rows is None else rows
    H = cfg.hidden
    out = np.zeros((R, N_STREAMS, H), dtype=act_np(cfg.act))
    for r in range(R):
        if r in cfg.zero_rows:
            continue
        g = Gen(_act_normal(cfg.act), key(cfg.base_seed, TAG_STATE, sample * 16 + r),
                normal_c(1.0))
        fill_host(g, N_STREAMS * H, out=out[r].reshape(-1))
    return out


def scale_gen_count(g: Gen, nbytes: int) -> int:
    return nbytes // _ELEM[g.kind]
