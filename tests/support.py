"""GPU test support: run the library through its C ABI and compare with the oracle.

Comparison rules (written out here and used by every parity test):
  * bf16 tensors (x, norm, hidden rows, shared, block, new state):
        |gpu - ref| <= 2^-7 * max(1, |ref|)              per element
  * f32 tensors (mixes, pre, post, comb, logits, weights, routed, carry):
        |gpu - ref| <= 1e-4 * max(|ref|, rms(ref row))   per element
    (the rms floor keeps near-zero dot products from failing a pure relative test)
  * expert indices: bit-exact where the oracle's gap between the k-th and (k+1)-th biased
    score exceeds 1e-5 (set), and in order where every adjacent gap inside the top-k does too;
    exact ties (the zero row) are identical on both sides and must follow the canonical order.
Each stage is compared with the oracle fed the GPU's own inputs to that stage (teacher
forcing), so one rounding flip upstream does not cascade.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np

import moe_decode_layer_amd as mono
import oracle
import synth

try:
    import torch
    import synth.device as sdev
except ImportError:  # pragma: no cover
    torch = None

BF16_TOL = 2.0 ** -7
F32_TOL = 1e-4
GAP = 1e-5


def bf(a) -> np.ndarray:
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def as_f32(a, act: str) -> np.ndarray:
    return np.asarray(a, np.float32) if act == "f32" else bf(a)


from moe_decode_layer_amd.host import (experts_struct, hidden_rows, layer_struct,  # noqa: E402,F401
                                       shape_of, ws_tensor)


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def d2h(t, dtype, shape) -> np.ndarray:
    a = t.detach().cpu().numpy().view(np.uint8) if t.dtype == torch.uint8 else \
        t.detach().cpu().contiguous().view(torch.uint8).numpy()
    n = int(np.prod(shape)) * np.dtype(dtype).itemsize
    return a[:n].view(dtype).reshape(shape).copy()


class Gpu:
    """One workload's layer(s) resident on the GPU plus a workspace."""

    def __init__(self, cfg: synth.Config, layers=(0,), device="cuda"):
        self.cfg = cfg
        self.dev = device
        self.layers = {l: sdev.layer(cfg, l, device) for l in layers}
        self.structs = {l: layer_struct(cfg, d) for l, d in self.layers.items()}
        self.shape = shape_of(cfg)
        self.ws = torch.zeros(mono.mono_workspace_bytes(self.shape), dtype=torch.uint8,
                              device=device)
        mono.mono_workspace_init(self.ws, self.shape, stream())
        self.ab = synth.act_bytes(cfg.act)
        self.adt = synth.act_np(cfg.act)

    def buf(self, nbytes: int):
        return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=self.dev)

    def state(self, sample: int):
        return sdev.state(self.cfg, sample, self.dev)

    # ---------------------------------------------------------------- unfused: four calls
    def unfused(self, state, layer=0, carry_in=None, w_next=None) -> Dict[str, np.ndarray]:
        c, s, L = self.cfg, self.shape, self.structs[layer]
        R, H, E, K, I, Is = c.rows, c.hidden, c.n_experts, c.top_k, c.inter, c.shared_inter
        ab = self.ab
        b = {n: self.buf(z) for n, z in dict(
            mixes=R * 24 * 4, pre=R * 16, post=R * 16, comb=R * 64, x=R * H * ab,
            norm=R * H * ab, logits=R * E * 4, idx=R * K * 4, weights=R * K * 4,
            shared=R * H * ab, routed=R * H * 4, block=R * H * ab, new=R * 4 * H * ab,
            carry=R * 25 * 4).items()}
        st = stream()
        mono.mono_hc_mix_collapse(s, state, L, carry_in, b["mixes"], b["pre"], b["post"],
                                  b["comb"], b["x"], b["norm"], self.ws, st)
        mono.mono_router_select(s, b["norm"], L, b["logits"], b["idx"], b["weights"], self.ws, st)
        mono.mono_moe_experts(s, b["norm"], b["idx"], b["weights"], L, b["shared"], b["routed"],
                              b["block"], self.ws, st)
        mono.mono_hc_expand(s, state, b["block"], b["post"], b["comb"], w_next, b["new"],
                            b["carry"] if w_next is not None else None, self.ws, st)
        torch.cuda.synchronize()
        adt = self.adt
        out = dict(
            mixes=d2h(b["mixes"], np.float32, (R, 24)), pre=d2h(b["pre"], np.float32, (R, 4)),
            post=d2h(b["post"], np.float32, (R, 4)), comb=d2h(b["comb"], np.float32, (R, 4, 4)),
            x=d2h(b["x"], adt, (R, H)), norm=d2h(b["norm"], adt, (R, H)),
            logits=d2h(b["logits"], np.float32, (R, E)), idx=d2h(b["idx"], np.int32, (R, K)),
            weights=d2h(b["weights"], np.float32, (R, K)), shared=d2h(b["shared"], adt, (R, H)),
            routed=d2h(b["routed"], np.float32, (R, H)), block=d2h(b["block"], adt, (R, H)),
            new_state=d2h(b["new"], adt, (R, 4, H)))
        out["h_routed"] = hidden_rows(s, self.ws, mono.MONO_T_H_ROUTED, adt, (R, K, I))
        out["h_shared"] = (hidden_rows(s, self.ws, mono.MONO_T_H_SHARED, adt, (R, Is)) if Is > 0
                           else np.zeros((R, 0), adt))
        if w_next is not None:
            out["carry"] = d2h(b["carry"], np.float32, (R, 25))
        return out

    # ---------------------------------------------------------------- fused: one launch
    def fused(self, state, layer=0, carry_in=None, w_next=None, state_out=None,
              carry_out=None) -> Dict[str, np.ndarray]:
        c, s, L = self.cfg, self.shape, self.structs[layer]
        R, H, E, K, I, Is = c.rows, c.hidden, c.n_experts, c.top_k, c.inter, c.shared_inter
        new = state_out if state_out is not None else self.buf(R * 4 * H * self.ab)
        carry = carry_out if carry_out is not None else (
            self.buf(R * 25 * 4) if w_next is not None else None)
        mono.mono_ffn_layer(s, L, w_next, state, carry_in, new, carry, self.ws, stream())
        torch.cuda.synchronize()
        st, err = mono.mono_workspace_poll(self.ws, stream())
        assert st == mono.MONO_OK, "device-side wait expired: %s" % err
        adt, ws = self.adt, self.ws
        T = lambda which, dt, dims: ws_tensor(s, ws, which, dt, dims)
        out = dict(
            mixes=T(mono.MONO_T_MIXES, np.float32, (R, 24)),
            pre=T(mono.MONO_T_PRE, np.float32, (R, 4)),
            post=T(mono.MONO_T_POST, np.float32, (R, 4)),
            comb=T(mono.MONO_T_COMB, np.float32, (R, 4, 4)),
            x=T(mono.MONO_T_X, adt, (R, H)), norm=T(mono.MONO_T_NORM, adt, (R, H)),
            logits=T(mono.MONO_T_LOGITS, np.float32, (R, E)),
            idx=T(mono.MONO_T_IDX, np.int32, (R, K)),
            weights=T(mono.MONO_T_WEIGHTS, np.float32, (R, K)),
            h_routed=hidden_rows(s, ws, mono.MONO_T_H_ROUTED, adt, (R, K, I)),
            h_shared=(hidden_rows(s, ws, mono.MONO_T_H_SHARED, adt, (R, Is)) if Is > 0
                      else np.zeros((R, 0), adt)),
            shared=T(mono.MONO_T_SHARED, adt, (R, H)),
            routed=T(mono.MONO_T_ROUTED, np.float32, (R, H)),
            block=T(mono.MONO_T_BLOCK, adt, (R, H)),
            new_state=d2h(new, adt, (R, 4, H)))
        if w_next is not None:
            out["carry"] = d2h(carry, np.float32, (R, 25))
        return out


# ------------------------------------------------------------------------------ comparisons

def check_bf16(name, got, ref, act="bf16"):
    g, r = as_f32(got, act).astype(np.float64), as_f32(ref, act).astype(np.float64)
    if act == "f32":
        return check_f32(name, g, r)
    d = np.abs(g - r)
    lim = BF16_TOL * np.maximum(1.0, np.abs(r))
    bad = d > lim
    assert not bad.any(), "%s: %d/%d elements off, worst |d|=%.3g at ref %.4g" % (
        name, int(bad.sum()), bad.size, float(d.max()), float(r.ravel()[np.argmax(d)]))
    return float(d.max())


def check_f32(name, got, ref):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    r2 = r.reshape(r.shape[0], -1) if r.ndim > 1 else r.reshape(1, -1)
    g2 = g.reshape(r2.shape)
    rms = np.sqrt((r2 * r2).mean(axis=1, keepdims=True))
    lim = F32_TOL * np.maximum(np.abs(r2), rms)
    d = np.abs(g2 - r2)
    bad = d > lim
    assert not bad.any(), "%s: %d/%d elements off, worst rel %.3g" % (
        name, int(bad.sum()), bad.size, float((d / np.maximum(lim, 1e-30)).max() * F32_TOL))
    return float((d / np.maximum(np.maximum(np.abs(r2), rms), 1e-30)).max())


def check_selection(got_idx, got_w, ref_idx, ref_w, beta_sorted, k):
    """Index rule of the module docstring; weights compared aligned by expert index.
    Returns the rows whose selection is decided by a near tie (forced downstream)."""
    near = []
    for r in range(ref_idx.shape[0]):
        b = beta_sorted[r]
        boundary = (b[k - 1] - b[k]) if b.shape[0] > k else np.inf
        inner = np.diff(b[:k]) * -1.0
        if boundary > GAP:
            assert set(got_idx[r].tolist()) == set(ref_idx[r].tolist()), (r, got_idx[r], ref_idx[r])
            if np.all(inner > GAP) or np.all(inner == 0):
                assert got_idx[r].tolist() == ref_idx[r].tolist(), (r, got_idx[r], ref_idx[r])
            gm = dict(zip(got_idx[r].tolist(), got_w[r].tolist()))
            rm = dict(zip(ref_idx[r].tolist(), ref_w[r].tolist()))
            check_f32("weights[%d]" % r, np.array([gm[e] for e in rm]), np.array(list(rm.values())))
        else:
            near.append(r)
    return near


def compare_stagewise(cfg: synth.Config, out: Dict[str, np.ndarray], state_h, dense_h,
                      routed_get, shared_h, w_next_h=None, carry_in=None) -> Dict[str, float]:
    """Each stage of `out` (GPU) against the oracle fed the GPU's inputs to that stage."""
    s = oracle.shape_of(cfg)
    act = cfg.act
    rep = {}
    if carry_in is None:
        ref_mix = oracle.mix(s, state_h, dense_h["w_mix"])
    else:
        ref_mix = oracle.mix(s, None, None, carry_in)
    rep["mixes"] = check_f32("mixes", out["mixes"], ref_mix)
    pre, post, comb = oracle.split(s, out["mixes"], dense_h["hc_scale"], dense_h["hc_base"])
    rep["pre"] = check_f32("pre", out["pre"], pre)
    rep["post"] = check_f32("post", out["post"], post)
    rep["comb"] = check_f32("comb", out["comb"].reshape(cfg.rows, 16), comb.reshape(cfg.rows, 16))
    x, norm = oracle.collapse_norm(s, state_h, out["pre"], dense_h["w_norm"])
    rep["x"] = check_bf16("x", out["x"], x, act)
    rep["norm"] = check_bf16("norm", out["norm"], norm, act)
    lg = oracle.router_logits(s, out["norm"], dense_h["w_router"])
    rep["logits"] = check_f32("logits", out["logits"], lg)
    idx, w, beta = oracle.select(s, out["logits"], dense_h["bias"])
    rep["near_tie_rows"] = check_selection(out["idx"], out["weights"], idx, w, beta, cfg.top_k)
    gidx, gw = out["idx"], out["weights"]
    experts = {int(e): routed_get(int(e)) for e in np.unique(gidx)}
    m = oracle.moe(s, out["norm"], gidx, gw, cfg.routed_fmt, experts, cfg.shared_fmt, shared_h)
    rep["h_routed"] = check_bf16("h_routed", out["h_routed"], m["h_routed"], act)
    if cfg.shared_inter > 0:
        rep["h_shared"] = check_bf16("h_shared", out["h_shared"], m["h_shared"], act)
    f = oracle.moe(s, None, gidx, gw, cfg.routed_fmt, experts, cfg.shared_fmt, shared_h,
                   h_routed=out["h_routed"], h_shared=out["h_shared"] if cfg.shared_inter > 0
                   else np.zeros((cfg.rows, 0), synth.act_np(act)))
    rep["routed"] = check_f32("routed", out["routed"], f["routed"])
    if cfg.shared_inter > 0:
        rep["shared"] = check_bf16("shared", out["shared"], f["shared"], act)
    # block from the GPU's routed and shared (one rounding)
    rb = oracle_block(cfg, out["routed"], out["shared"])
    rep["block"] = check_bf16("block", out["block"], rb, act)
    new, carry = oracle.expand(s, state_h, out["block"], out["post"], out["comb"], w_next_h)
    rep["new_state"] = check_bf16("new_state", out["new_state"], new, act)
    if w_next_h is not None:
        # the carry of the GPU's own new state
        rep["carry"] = check_f32("carry", out["carry"], oracle_carry(cfg, out["new_state"], w_next_h))
    return rep


def oracle_block(cfg, routed, shared):
    """block = bf16(f32(routed + shared)) of the GPU's routed and shared rows, rounded by the
    oracle's bf16 rounding."""
    act = cfg.act
    r = np.asarray(routed, np.float64)
    sh = as_f32(shared, act).astype(np.float64) if cfg.shared_inter > 0 else 0.0
    v = (r + sh).astype(np.float32)
    if act == "f32":
        return v
    return np.array([oracle.f32_to_bf16(float(x)) for x in v.ravel()], np.uint16).reshape(v.shape)


def oracle_carry(cfg, new_state, w_next):
    """Carry of the GPU's new state through the oracle's expand with post = 0, comb = I
    (new = state exactly), so the carry is the oracle's own."""
    s = oracle.shape_of(cfg)
    R, H = cfg.rows, cfg.hidden
    eye = np.tile(np.eye(4, dtype=np.float32), (R, 1, 1))
    zero_post = np.zeros((R, 4), np.float32)
    blk = np.zeros((R, H), synth.act_np(cfg.act))
    new2, carry = oracle.expand(s, np.ascontiguousarray(new_state), blk, zero_post, eye, w_next)
    assert np.array_equal(new2, new_state)
    return carry


def assert_same(a: Dict[str, np.ndarray], b: Dict[str, np.ndarray], keys) -> None:
    for k in keys:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), "fused != unfused: " + k
