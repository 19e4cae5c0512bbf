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
  * secondary rule for bf16 tensors: at most 0.1 % of the elements (at least one) more than
    one bf16 step from the oracle's value (ULP_SHARE), counting elements of at least 2^-6 of
    the tensor's rms (smaller ones are near-cancellations; the contract still bounds them).
  * SwiGLU hidden values: an element outside these rules is accepted only when it equals (within
    one step) the result of another admissible rounding of its gate or up sum (check_hidden).
  * free-running (end-to-end) comparison: the same rules for every bf16 tensor up to the
    hidden rows; the logits, the routing weights and every tensor after the hidden rows also
    get an error budget, the first-order effect of the measured differences of their inputs
    (see compare_end_to_end).
Each stage is compared with the oracle fed the GPU's own inputs to that stage (teacher
forcing), so one rounding flip upstream does not cascade; compare_end_to_end also compares
every output with the oracle run free from the same input when no selection rests on a near
tie. Statistics of every comparison (maximum deviations, bf16 step histograms) collect in
REPORT, written as JSON at the end of a session when MONO_PARITY_REPORT names a file.
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
              carry_out=None, expect_ok=True) -> Dict[str, np.ndarray]:
        c, s, L = self.cfg, self.shape, self.structs[layer]
        R, H, E, K, I, Is = c.rows, c.hidden, c.n_experts, c.top_k, c.inter, c.shared_inter
        new = state_out if state_out is not None else self.buf(R * 4 * H * self.ab)
        carry = carry_out if carry_out is not None else (
            self.buf(R * 25 * 4) if w_next is not None else None)
        mono.mono_ffn_layer(s, L, w_next, state, carry_in, new, carry, self.ws, stream())
        torch.cuda.synchronize()
        st, err = mono.mono_workspace_poll(self.ws, stream())
        assert st == mono.MONO_OK or not expect_ok, "device-side wait expired: %s" % err
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

# Secondary rule beside the contract: a bf16 tensor may have at most this share of its elements
# more than one bf16 step (ulp) away from the oracle (at least one element is always allowed).
# The kernels and the oracle round the same f32 values, which differ only in summation order,
# so a rounding decision flips rarely; a systematic error of a fraction of a percent fails.
ULP_SHARE = 1e-3

# Per-tensor statistics of every comparison made in this process: {case: {tensor: stats}}.
REPORT: Dict[str, Dict[str, Dict]] = {}
_case = ["-"]


def set_case(name: str) -> None:
    """Names the comparisons that follow in REPORT."""
    _case[0] = name


def _record(name: str, stats: Dict) -> None:
    REPORT.setdefault(_case[0], {})[name] = stats


def _ordered(a) -> np.ndarray:
    """bf16 bit patterns as integers in value order (+0 and -0 coincide)."""
    a = np.asarray(a, np.uint16).astype(np.int64)
    return np.where(a & 0x8000, -(a & 0x7FFF), a)


def bf16_ulps(got, ref) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bf16 bit patterns."""
    return np.abs(_ordered(got) - _ordered(ref))


# The step rule counts elements at least this fraction of their tensor's rms: a smaller value is
# a near-cancellation of its sum, whose relative error is not bounded (the contract's absolute
# floor still applies to it).
STEP_FLOOR = 2.0 ** -6


def _significant(r: np.ndarray) -> np.ndarray:
    rms = np.sqrt(np.mean(r * r)) if r.size else 0.0
    return np.abs(r) >= STEP_FLOOR * rms


def check_bf16(name, got, ref, act="bf16", extra=None, steps=True):
    """Contract rule (plus `extra`, an absolute allowance per element for errors carried in from
    an input, used only by the free-running comparison) and, with `steps`, the bf16 step
    rule."""
    if act == "f32":
        return check_f32(name, got, ref)
    g, r = as_f32(got, act).astype(np.float64), as_f32(ref, act).astype(np.float64)
    d = np.abs(g - r)
    lim = BF16_TOL * np.maximum(1.0, np.abs(r))
    if extra is not None:
        lim = lim + np.broadcast_to(extra, lim.shape)
    bad = d > lim
    if bad.any():
        at = np.argwhere(bad)[:4]
        pairs = ", ".join("%s: %.5g vs %.5g" % (tuple(int(i) for i in ix), g[tuple(ix)],
                                                r[tuple(ix)]) for ix in at)
        raise AssertionError("%s: %d/%d elements off, worst |d|=%.3g at ref %.4g; first: %s" % (
            name, int(bad.sum()), bad.size, float(d.max()), float(r.ravel()[np.argmax(d)]),
            pairs))
    u = bf16_ulps(got, ref).ravel()
    n = u.size
    far = int(((u > 1) & _significant(r).ravel()).sum())
    hist = {k: int(v) for k, v in zip(("0", "1", "2", "3-7", "8+"),
                                      np.histogram(u, [0, 1, 2, 3, 8, 1 << 20])[0])}
    _record(name, dict(kind="bf16", n=n, max_abs=float(d.max()) if n else 0.0,
                       max_ulp=int(u.max()) if n else 0, ulp_hist=hist))
    allowed = max(1, int(ULP_SHARE * n))
    assert not steps or far <= allowed, \
        "%s: %d/%d elements more than 1 bf16 step off (allowed %d), hist %s" % (
            name, far, n, allowed, hist)
    return float(d.max()) if n else 0.0


def _bf16_bits(v) -> np.ndarray:
    """Round-to-nearest-even bf16 bit patterns of f64 values (through f32)."""
    u = np.asarray(v, np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _bf16_choices(v: float, slack: float):
    """bf16 values a rounding of any value in [v - slack, v + slack] may give, as the two ends
    and the nearest of v (a sum computed in another order lands anywhere in that window)."""
    return sorted({float(bf(_bf16_bits([t]))[0]) for t in (v - slack, v, v + slack)})


# Distance from a bf16 rounding midpoint, relative to the sum of the magnitudes of a dot
# product's terms, within which the kernels' f32 sum (another summation order than the
# oracle's exact one) may round the other way.
FLIP_REL = 2.0 ** -16


_E4M3 = None


def mx8_round_trip(x) -> np.ndarray:
    """The MXFP8 round trip of an activation row (the oracle's quantiser and E4M3 decode)."""
    global _E4M3
    if _E4M3 is None:
        _E4M3 = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    codes, scales = oracle.mxfp8_quant(x)
    return _E4M3[codes] * np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32)


def check_hidden(name, got, ref, act, norm, rows, aq="none") -> float:
    """SwiGLU hidden values h = bf16(silu(g) u) with g = bf16(W_g . x) and u = bf16(W_u . x): the
    contract and step rules, except that an element outside them is accepted when it is within
    one bf16 step of h computed from some admissible rounding of g and u. Admissible: the exact
    (f64) g and u from the weights, rounded to nearest, or to the other neighbour where the exact
    value lies within FLIP_REL * sum |w x| of a rounding midpoint. rows(index) -> (fmt, expert tensors,
    activation row index) for the leading indices of the element."""
    if act == "f32":
        return check_f32(name, got, ref)
    g, r = as_f32(got, act).astype(np.float64), as_f32(ref, act).astype(np.float64)
    d = np.abs(g - r)
    lim = BF16_TOL * np.maximum(1.0, np.abs(r))
    u = bf16_ulps(got, ref)
    far_mask = (u > 1) & _significant(r)
    suspect = np.argwhere((d > lim) | far_mask)
    justified = 0
    nrm = bf(norm).astype(np.float64)
    for ix in suspect:
        ix = tuple(int(i) for i in ix)
        fmt, t, arow = rows(ix[:-1])
        i = ix[-1]
        x = nrm[arow]
        if aq == "mxfp8" and fmt == "mxfp4":  # the input the MXFP4 matrices see
            x = mx8_round_trip(x)
        wg = support_dequant_row(fmt, t["gate"], t.get("gate_s"), i)
        wu = support_dequant_row(fmt, t["up"], t.get("up_s"), i)
        gv, uv = float(wg @ x), float(wu @ x)
        gs, us = FLIP_REL * float(np.abs(wg) @ np.abs(x)), FLIP_REL * float(np.abs(wu) @ np.abs(x))
        cands = [float(bf(_bf16_bits([gg / (1.0 + np.exp(-gg)) * uu]))[0])
                 for gg in _bf16_choices(gv, gs) for uu in _bf16_choices(uv, us)]
        # within one step of the range the admissible roundings span
        o = _ordered(_bf16_bits(cands))
        mine = int(_ordered(np.array([np.asarray(got)[ix]], np.uint16))[0])
        ok = int(o.min()) - 1 <= mine <= int(o.max()) + 1
        assert ok, "%s%s: %.6g vs oracle %.6g; exact g %.8g, u %.8g allow %s" % (
            name, ix, g[ix], r[ix], gv, uv, ["%.6g" % c for c in cands])
        if len(set(cands)) > 1:
            justified += 1
            far_mask[ix] = False
    n = u.size
    far = int(far_mask.sum())
    hist = {k: int(v) for k, v in zip(("0", "1", "2", "3-7", "8+"),
                                      np.histogram(u.ravel(), [0, 1, 2, 3, 8, 1 << 20])[0])}
    _record(name, dict(kind="bf16 hidden", n=n, max_abs=float(d.max()) if n else 0.0,
                       max_ulp=int(u.max()) if n else 0, ulp_hist=hist,
                       justified_by_input_rounding=justified))
    allowed = max(1, int(ULP_SHARE * n))
    assert far <= allowed, "%s: %d/%d elements more than 1 bf16 step off (allowed %d), hist %s" % (
        name, far, n, allowed, hist)
    return float(d.max()) if n else 0.0


def support_dequant_row(fmt: str, v, sc, i: int) -> np.ndarray:
    """Row i of a [rows][k] weight matrix decoded to f64 (see dequant)."""
    return dequant(fmt, v[i:i + 1], None if sc is None else sc[i:i + 1])[0]


def check_f32(name, got, ref, extra=None):
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    r2 = r.reshape(r.shape[0], -1) if r.ndim > 1 else r.reshape(1, -1)
    g2 = g.reshape(r2.shape)
    rms = np.sqrt((r2 * r2).mean(axis=1, keepdims=True))
    lim = F32_TOL * np.maximum(np.abs(r2), rms)
    if extra is not None:
        lim = lim + np.asarray(extra, np.float64).reshape(r2.shape)
    d = np.abs(g2 - r2)
    bad = d > lim
    assert not bad.any(), "%s: %d/%d elements off, worst rel %.3g" % (
        name, int(bad.sum()), bad.size, float((d / np.maximum(lim, 1e-30)).max() * F32_TOL))
    nz = np.abs(r2) > 0
    pure = float((d[nz] / np.abs(r2[nz])).max()) if nz.any() else 0.0
    floored = float((d / np.maximum(np.maximum(np.abs(r2), rms), 1e-30)).max())
    _record(name, dict(kind="f32", n=int(d.size), max_rel_floored=floored, max_rel=pure,
                       max_abs=float(d.max()) if d.size else 0.0))
    return floored


def near_tie_rows(beta_sorted, k, got_logits=None, ref_logits=None):
    """Rows whose selection a rounding difference could change: the oracle's gap at the k-th
    place or between adjacent places inside the top-k is at most GAP. A gap of exactly 0 counts
    as a tie the two sides break alike only when both computed the same logits for the row
    (the zero row), otherwise as near."""
    rows = []
    for r in range(beta_sorted.shape[0]):
        b = beta_sorted[r].astype(np.float64)
        gaps = -np.diff(b[: k + 1]) if b.shape[0] > k else -np.diff(b[:k])
        same = (got_logits is not None and ref_logits is not None and
                np.array_equal(np.asarray(got_logits[r]).view(np.uint32),
                               np.asarray(ref_logits[r]).view(np.uint32)))
        if np.any((gaps <= GAP) & ((gaps > 0) | (not same))):
            rows.append(r)
    return rows


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


def compare_pre_side(cfg: synth.Config, out: Dict[str, np.ndarray], state_h, dense_h,
                     carry_in=None) -> Dict[str, float]:
    """The HC pre side of `out` (mixes, pre, post, comb, x, norm) against the oracle fed the
    GPU's inputs to each stage: the mix from the state or from the carry, the split from the
    GPU's mixes, the collapse and norm from the GPU's pre weights."""
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
    return rep


def compare_stagewise(cfg: synth.Config, out: Dict[str, np.ndarray], state_h, dense_h,
                      routed_get, shared_h, w_next_h=None, carry_in=None) -> Dict[str, float]:
    """Each stage of `out` (GPU) against the oracle fed the GPU's inputs to that stage."""
    s = oracle.shape_of(cfg)
    act = cfg.act
    rep = compare_pre_side(cfg, out, state_h, dense_h, carry_in)
    lg = oracle.router_logits(s, out["norm"], dense_h["w_router"])
    rep["logits"] = check_f32("logits", out["logits"], lg)
    idx, w, beta = oracle.select(s, out["logits"], dense_h["bias"])
    rep["near_tie_rows"] = check_selection(out["idx"], out["weights"], idx, w, beta, cfg.top_k)
    gidx, gw = out["idx"], out["weights"]
    experts = {int(e): routed_get(int(e)) for e in np.unique(gidx)}
    m = oracle.moe(s, out["norm"], gidx, gw, cfg.routed_fmt, experts, cfg.shared_fmt, shared_h)
    rep["h_routed"] = check_hidden("h_routed", out["h_routed"], m["h_routed"], act, out["norm"],
                                   lambda rj: (cfg.routed_fmt, experts[int(gidx[rj])], rj[0]),
                                   cfg.act_quant)
    if cfg.shared_inter > 0:
        rep["h_shared"] = check_hidden("h_shared", out["h_shared"], m["h_shared"], act,
                                       out["norm"], lambda r_: (cfg.shared_fmt, shared_h, r_[0]),
                                       cfg.act_quant)
    # down projections, routed sum, shared rounding and block: the oracle fed the GPU's hidden
    # rows (one rounding flip in h does not cascade)
    f = oracle.moe(s, None, gidx, gw, cfg.routed_fmt, experts, cfg.shared_fmt, shared_h,
                   h_routed=out["h_routed"], h_shared=out["h_shared"] if cfg.shared_inter > 0
                   else np.zeros((cfg.rows, 0), synth.act_np(act)))
    rep["routed"] = check_f32("routed", out["routed"], f["routed"])
    if cfg.shared_inter > 0:
        rep["shared"] = check_bf16("shared", out["shared"], f["shared"], act)
    rep["block"] = check_bf16("block", out["block"], f["block"], act)
    new, carry = oracle.expand(s, state_h, out["block"], out["post"], out["comb"], w_next_h)
    rep["new_state"] = check_bf16("new_state", out["new_state"], new, act)
    if w_next_h is not None:
        # the carry of the GPU's own new state
        rep["carry"] = check_f32("carry", out["carry"], oracle_carry(cfg, out["new_state"], w_next_h))
    return rep


def dequant(fmt: str, v, sc=None) -> np.ndarray:
    """A [rows][k] weight matrix decoded to f64 with numpy (independent of the oracle's decode):
    bf16 bits, Q8_0 int8 x fp16 scale per 32, MXFP4 e2m1 (low nibble first) x 2^(e - 127)."""
    if fmt == "f32":
        return np.asarray(v, np.float64)
    if fmt == "bf16":
        return bf(v).astype(np.float64)
    if fmt == "q8_0":
        return v.astype(np.float64) * np.repeat(sc.view(np.float16).astype(np.float64), 32, axis=1)
    lo, hi = v & 0xF, v >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(v.shape[0], -1).astype(np.int64)
    e, m = (codes >> 1) & 3, codes & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0, e - 1) * (1 + m / 2))
    return np.where(codes & 8, -mag, mag) * np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127),
                                                       32, axis=1)


def compare_end_to_end(cfg: synth.Config, out: Dict[str, np.ndarray], state_h, dense_h,
                       routed_get, shared_h, w_next_h=None, carry_in=None) -> Dict:
    """Every output of `out` (GPU) against the oracle run free from the same input, with no
    teacher forcing, when no row's selection rests on a near tie; otherwise the result holds
    {"skipped": rows} and nothing is compared (the stage-wise comparison covers those rows).
    The oracle's outputs are returned under "ref" either way.

    Error budget. The bf16 tensors (x, norm, hidden rows) are held to the contract and step
    rules. A legitimate rounding flip (one bf16 step) of a norm value reaches every logit, and
    one of a hidden value every output of the down projection, and cancellation between routed
    and shared can enlarge it again, so each later tensor may differ by its own contract
    tolerance plus the first-order effect of the measured differences of its inputs through the
    absolute values of the weights:
      logits:  |W_r| . |dnorm|        weights: d(rho s_j / sum s) through ds = s'(z) dz
      routed:  sum_j |w_j| (|W_d[e_j]| . |dh_j|)              shared: |W_ds| . |dh_s|
      block:   the allowed differences of routed and shared
      new:     post * (the allowed difference of block)
      carry:   |W_next| . |dnew| and sum 2 |new| |dnew| + dnew^2 for the sum of squares,
    where dh and dnew are the GPU's differences from the oracle (exact: both are bf16)."""
    s = oracle.shape_of(cfg)
    act = cfg.act
    ref = oracle.layer(s, state_h, dense_h, cfg.routed_fmt, routed_get, cfg.shared_fmt,
                       shared_h, w_next_h, carry_in)
    near = near_tie_rows(ref["beta_sorted"], cfg.top_k, out["logits"], ref["logits"])
    if near:
        return {"skipped": near, "ref": ref}
    rep = {"ref": ref}
    R, H, K = cfg.rows, cfg.hidden, cfg.top_k
    for key in ("mixes", "pre", "post"):
        rep[key] = check_f32("e2e " + key, out[key], ref[key])
    rep["comb"] = check_f32("e2e comb", out["comb"].reshape(R, 16), ref["comb"].reshape(R, 16))
    assert np.array_equal(out["idx"], ref["idx"]), (out["idx"], ref["idx"])
    for key in ("x", "norm"):
        rep[key] = check_bf16("e2e " + key, out[key], ref[key], act)
    f64 = lambda a: as_f32(a, act).astype(np.float64)
    # a legitimate one-step flip of a norm value reaches every logit through |W_r|, and the
    # weights through the derivative of s = sqrt(softplus(z)) and the row division
    dnorm = np.abs(f64(out["norm"]) - f64(ref["norm"]))                    # [R][H]
    ext_lg = dnorm @ np.abs(np.asarray(dense_h["w_router"], np.float64)).T  # [R][E]
    rep["logits"] = check_f32("e2e logits", out["logits"], ref["logits"], extra=ext_lg)
    z = np.asarray(ref["logits"], np.float64)
    zr = np.sqrt((z * z).mean(axis=1, keepdims=True))
    dz = F32_TOL * np.maximum(np.abs(z), zr) + ext_lg
    sp = np.logaddexp(0.0, z)
    sc = np.sqrt(sp)
    ds = dz / (1.0 + np.exp(-z)) / (2.0 * np.maximum(sc, 1e-30))          # |ds/dz| dz
    idx = np.asarray(ref["idx"])
    ssel = np.take_along_axis(sc, idx, axis=1)
    dsel = np.take_along_axis(ds, idx, axis=1)
    tot = np.maximum(ssel.sum(axis=1, keepdims=True), 2.0 ** -14)
    ext_w = cfg.routed_scale * (dsel / tot + ssel * dsel.sum(axis=1, keepdims=True) / tot ** 2)
    rep["weights"] = check_f32("e2e weights", out["weights"], ref["weights"], extra=ext_w)
    cache = {}
    getx = lambda e: cache.setdefault(e, routed_get(e))
    rep["h_routed"] = check_hidden("e2e h_routed", out["h_routed"], ref["h_routed"], act,
                                   out["norm"],
                                   lambda rj: (cfg.routed_fmt, getx(int(ref["idx"][rj])), rj[0]),
                                   cfg.act_quant)
    if cfg.shared_inter > 0:
        rep["h_shared"] = check_hidden("e2e h_shared", out["h_shared"], ref["h_shared"], act,
                                       out["norm"], lambda r_: (cfg.shared_fmt, shared_h, r_[0]),
                                       cfg.act_quant)

    def down_input_dev(fmt, got_h, ref_h):
        """|difference| of what the down projections see: the hidden rows, or with MXFP8
        activations for an MXFP4 matrix their round trips (a one-step change of h can move a
        quantisation step or a block scale)."""
        a, b = f64(got_h), f64(ref_h)
        if cfg.act_quant == "mxfp8" and fmt == "mxfp4":
            sh = a.shape
            a = np.stack([mx8_round_trip(v) for v in a.reshape(-1, sh[-1])]).reshape(sh)
            b = np.stack([mx8_round_trip(v) for v in b.reshape(-1, sh[-1])]).reshape(sh)
        return np.abs(a - b)

    dh = down_input_dev(cfg.routed_fmt, out["h_routed"], ref["h_routed"])  # [R][K][I]
    w = np.abs(np.asarray(ref["weights"], np.float64))
    ext_routed = np.zeros((R, H))
    for e in np.unique(ref["idx"]):
        rows, slots = np.nonzero(ref["idx"] == e)
        if not np.any(dh[rows, slots]):
            continue
        t = getx(int(e))
        aw = np.abs(dequant(cfg.routed_fmt, t["down"], t.get("down_s")))   # [H][I]
        for r, j in zip(rows, slots):
            ext_routed[r] += w[r, j] * (aw @ dh[r, j])
    rep["routed"] = check_f32("e2e routed", out["routed"], ref["routed"], extra=ext_routed)
    r64 = np.asarray(ref["routed"], np.float64)
    rms = np.sqrt((r64 * r64).mean(axis=1, keepdims=True))
    d_routed = F32_TOL * np.maximum(np.abs(r64), rms) + ext_routed
    d_shared = 0.0
    if cfg.shared_inter > 0:
        dhs = down_input_dev(cfg.shared_fmt, out["h_shared"], ref["h_shared"])  # [R][Is]
        ext_shared = np.zeros((R, H))
        if np.any(dhs):
            aw = np.abs(dequant(cfg.shared_fmt, shared_h["down"], shared_h.get("down_s")))
            ext_shared = dhs @ aw.T
        rep["shared"] = check_bf16("e2e shared", out["shared"], ref["shared"], act,
                                   extra=ext_shared, steps=False)
        d_shared = BF16_TOL * np.maximum(1.0, np.abs(f64(ref["shared"]))) + ext_shared
    ext_block = d_routed + d_shared
    rep["block"] = check_bf16("e2e block", out["block"], ref["block"], act, extra=ext_block,
                              steps=False)
    d_block = BF16_TOL * np.maximum(1.0, np.abs(f64(ref["block"]))) + ext_block
    ext_new = np.asarray(ref["post"], np.float64)[:, :, None] * d_block[:, None, :]
    rep["new_state"] = check_bf16("e2e new_state", out["new_state"], ref["new_state"], act,
                                  extra=ext_new, steps=False)
    if w_next_h is not None:
        dn = np.abs(f64(out["new_state"]) - f64(ref["new_state"])).reshape(R, -1)
        nv = np.abs(f64(ref["new_state"])).reshape(R, -1)
        ext_carry = np.zeros((R, 25))
        ext_carry[:, :24] = dn @ np.abs(np.asarray(w_next_h, np.float64)).T
        ext_carry[:, 24] = (2 * nv * dn + dn * dn).sum(axis=1)
        rep["carry"] = check_f32("e2e carry", out["carry"], ref["carry"], extra=ext_carry)
    return rep


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


def write_report(path: str) -> None:
    """REPORT as JSON (one object per case, one entry per compared tensor)."""
    import json
    import os
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(REPORT, fh, indent=1, sort_keys=True)
