"""Benchmark of the fused layer-half launch (mono_ffn_layer) on one MI355X.

A step is one pass of the whole hot path over one batch: mHC mix -> split/Sinkhorn ->
collapse + RMSNorm -> router + top-k -> shared and routed SwiGLU experts -> block -> expand ->
carry of the next layer half's mix sums, as ONE persistent launch, with inputs resident in HBM.

Headline workload: the V4.1-like layer half at 1 row with bf16 experts (hidden 5120, 256
experts top-8, inter 2048, shared inter 2048). The 6-row Q8_0 and the 8-row MXFP4 (bf16 shared,
one zero row) workloads are measured in the same run and reported under "rows6" and "rows8",
the 8-row workload with the MXFP4 experts' activations quantised to MXFP8 under "rows8_mxfp8",
and the chain of 8 bf16 layer halves (each taking the previous one's carry) under "chain8". Steps rotate over `--copies` independent weight copies and 64
seeded input states, so routing changes every step and no weight is re-read from the 256 MB
last-level cache; each step's algorithmic bytes count every distinct selected expert once.
The timed steps run twice: with an event pair around every launch (the per-launch durations
behind "launch_us" and the roofline) and back to back between one event pair (steps/s and
ms_per_step: per-launch event records between the kernels are not part of the throughput).

Prints ONE JSON line (rank 0, N = 1 only).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "MoE decode layer steps/s and achieved HBM GB/s (% peak) at 1 and 6 rows"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dense_bytes(cfg, carry: bool) -> int:
    H, E = cfg.hidden, cfg.n_experts
    ab = 4 if cfg.act == "f32" else 2
    b = 24 * 4 * H * 4 * (2 if carry else 1)       # w_mix (+ the next layer's, for the carry)
    b += E * H * 4 + E * 4 + H * ab + 3 * 4 + 24 * 4  # router, bias, norm weight, hc params
    return b


def step_bytes(cfg, idx_rows: np.ndarray, carry: bool) -> int:
    import synth
    per_routed = synth.expert_bytes(cfg.routed_fmt, cfg.inter, cfg.hidden)
    per_shared = synth.expert_bytes(cfg.shared_fmt, cfg.shared_inter, cfg.hidden)
    n_distinct = len(np.unique(idx_rows))
    return n_distinct * per_routed + (per_shared if cfg.shared_inter else 0) + dense_bytes(cfg, carry)


class Workload:
    def __init__(self, cfg, copies: int):
        import torch
        from moe_decode_layer_amd import host
        import moe_decode_layer_amd as mono
        import synth.device as sdev
        self.cfg, self.copies = cfg, copies
        t0 = time.time()
        self.layers = [sdev.layer(cfg, l) for l in range(copies)]
        self.structs = [host.layer_struct(cfg, d) for d in self.layers]
        self.states = [sdev.state(cfg, s) for s in range(64)]
        self.shape = host.shape_of(cfg)
        self.ws = torch.zeros(mono.mono_workspace_bytes(self.shape), dtype=torch.uint8,
                              device="cuda")
        mono.mono_workspace_init(self.ws, self.shape, host.current_stream())
        ab = 4 if cfg.act == "f32" else 2
        self.out = torch.zeros(cfg.rows * 4 * cfg.hidden * ab, dtype=torch.uint8, device="cuda")
        self.carry = torch.zeros(cfg.rows * 25 * 4, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        log("  %s: %d weight copies resident (%.1f GB) in %.1f s" % (
            cfg.name, copies, copies * self.weight_gb(), time.time() - t0))

    def weight_gb(self) -> float:
        import synth
        c = self.cfg
        b = c.n_experts * synth.expert_bytes(c.routed_fmt, c.inter, c.hidden)
        if c.shared_inter:
            b += synth.expert_bytes(c.shared_fmt, c.shared_inter, c.hidden)
        return (b + dense_bytes(c, False)) / 1e9

    def launch(self, i: int):
        import moe_decode_layer_amd as mono
        from moe_decode_layer_amd import host
        l = i % self.copies
        nxt = self.layers[(l + 1) % self.copies]["w_mix"]
        mono.mono_ffn_layer(self.shape, self.structs[l], nxt, self.states[i % 64], None, self.out,
                            self.carry, self.ws, host.current_stream())

    def selection(self, i: int) -> np.ndarray:
        import moe_decode_layer_amd as mono
        from moe_decode_layer_amd import host
        self.launch(i)
        import torch
        torch.cuda.synchronize()
        return host.ws_tensor(self.shape, self.ws, mono.MONO_T_IDX, np.int32,
                                 (self.cfg.rows, self.cfg.top_k))

    def run(self, steps: int, warmup: int):
        import torch
        # algorithmic bytes of every step (selection depends on layer copy and input)
        nbytes = [step_bytes(self.cfg, self.selection(i), True) for i in range(steps)]
        for i in range(warmup):
            self.launch(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            self.launch(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in ev])
        return dict(span_ms=self.back_to_back(steps, self.launch), dur_ms=dur_ms,
                    bytes=np.array(nbytes))

    @staticmethod
    def back_to_back(steps: int, launch) -> float:
        """Milliseconds for `steps` steps enqueued back to back between one pair of events (the
        throughput figure; the per-launch events of the other pass are not in it)."""
        import torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            launch(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)


def seam_timings(cfg, reps: int = 50) -> dict:
    """Mean launch time of the attention half's seam calls and of the model tail at one row,
    each on its own inputs resident in HBM: the attention pre side from the previous FFN half's
    carry (mono_hc_mix_collapse), its post side with the carry for the FFN half
    (mono_hc_expand), and the tail (mono_hc_head: head mix, collapse, output norm)."""
    import torch
    import moe_decode_layer_amd as mono
    from moe_decode_layer_amd import host
    import synth
    import synth.device as sdev
    R, H = cfg.rows, cfg.hidden
    ab = 4 if cfg.act == "f32" else 2
    shape = host.shape_of(cfg)
    ws = torch.zeros(mono.mono_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    mono.mono_workspace_init(ws, shape, host.current_stream())
    attn = sdev.dense(cfg, synth.ATTN_LAYER)
    ffn_mix = sdev.dense(cfg, 0)["w_mix"]
    L = mono.make_layer(attn["w_mix"], attn["hc_scale"], attn["hc_base"], attn["w_norm"], None,
                        None, mono.Experts(), mono.Experts())
    ht = sdev.head(cfg)
    head = mono.make_head(ht["w_head"], ht["head_scale"], ht["head_base"], ht["w_norm"])
    st = sdev.state(cfg, 0)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32, device="cuda")
    raw = lambda n: torch.zeros(n, dtype=torch.uint8, device="cuda")
    carry = torch.rand(R * 25, device="cuda") + 1.0
    mixes, pre, post, comb = f32(R * 24), f32(R * 4), f32(R * 4), f32(R * 16)
    x, norm, blk = raw(R * H * ab), raw(R * H * ab), raw(R * H * ab)
    new, carry2 = raw(R * 4 * H * ab), f32(R * 25)
    s = host.current_stream()
    calls = {
        "attn_pre_from_carry": lambda: mono.mono_hc_mix_collapse(
            shape, st, L, carry, mixes, pre, post, comb, x, norm, ws, s),
        "attn_post_with_carry": lambda: mono.mono_hc_expand(
            shape, st, blk, post, comb, ffn_mix, new, carry2, ws, s),
        "model_tail": lambda: mono.mono_hc_head(shape, st, head, pre, x, norm, s),
    }
    out = {"workload": cfg.name + ": attention-half seam and model tail", "rows": R}
    for name, fn in calls.items():
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        out[name + "_us"] = a.elapsed_time(b) * 1e3 / reps
    return out


class ChainWorkload:
    """The 8-layer-half chain at 1 row: one step is 8 fused launches, layer l taking the carry of
    layer l - 1 (its mix matvec skipped) and producing the next one's, the last with no carry.
    Each layer's weights are distinct and resident (129 GB in all), so every launch streams its
    own experts."""

    def __init__(self, cfg):
        import torch
        from moe_decode_layer_amd import host
        import moe_decode_layer_amd as mono
        import synth.device as sdev
        self.cfg = cfg
        n = cfg.layers
        t0 = time.time()
        self.layers = [sdev.layer(cfg, l) for l in range(n)]
        self.structs = [host.layer_struct(cfg, d) for d in self.layers]
        self.states = [sdev.state(cfg, s) for s in range(64)]
        self.shape = host.shape_of(cfg)
        self.ws = torch.zeros(mono.mono_workspace_bytes(self.shape), dtype=torch.uint8,
                              device="cuda")
        mono.mono_workspace_init(self.ws, self.shape, host.current_stream())
        ab = 4 if cfg.act == "f32" else 2
        nb = cfg.rows * 4 * cfg.hidden * ab
        self.bufs = [torch.zeros(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
        self.carry = [torch.zeros(cfg.rows * 25 * 4, dtype=torch.uint8, device="cuda")
                      for _ in range(2)]
        torch.cuda.synchronize()
        log("  %s: %d layer halves resident in %.1f s" % (cfg.name, n, time.time() - t0))

    def step(self, i: int, on_layer=None):
        import moe_decode_layer_amd as mono
        from moe_decode_layer_amd import host
        n = self.cfg.layers
        st = self.states[i % 64]
        carry_in = None
        for l in range(n):
            nxt = self.layers[l + 1]["w_mix"] if l + 1 < n else None
            out, cout = self.bufs[l % 2], self.carry[l % 2]
            mono.mono_ffn_layer(self.shape, self.structs[l], nxt, st, carry_in, out,
                                cout if nxt is not None else None, self.ws, host.current_stream())
            if on_layer is not None:
                on_layer(l)
            st, carry_in = out, cout

    def step_bytes(self, i: int) -> int:
        """Algorithmic bytes of step i: per layer the distinct selected experts, the shared
        expert, the router, bias and norm weight, W_mix of layer 0 (its own mix) and of every
        next layer (the carry)."""
        import torch
        import moe_decode_layer_amd as mono
        from moe_decode_layer_amd import host
        import synth
        c = self.cfg
        per_routed = synth.expert_bytes(c.routed_fmt, c.inter, c.hidden)
        per_shared = synth.expert_bytes(c.shared_fmt, c.shared_inter, c.hidden)
        ab = 4 if c.act == "f32" else 2
        w_mix = 24 * 4 * c.hidden * 4
        total = [0]

        def on_layer(l):
            torch.cuda.synchronize()
            idx = host.ws_tensor(self.shape, self.ws, mono.MONO_T_IDX, np.int32,
                                    (c.rows, c.top_k))
            b = len(np.unique(idx)) * per_routed + (per_shared if c.shared_inter else 0)
            b += c.n_experts * c.hidden * 4 + c.n_experts * 4 + c.hidden * ab + 3 * 4 + 24 * 4
            b += (w_mix if l == 0 else 0) + (w_mix if l + 1 < c.layers else 0)
            total[0] += b

        self.step(i, on_layer)
        return total[0]

    def run(self, steps: int, warmup: int):
        import torch
        nbytes = [self.step_bytes(i) for i in range(steps)]
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            self.step(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        dur_ms = np.array([a.elapsed_time(b) for a, b in ev])
        return dict(span_ms=Workload.back_to_back(steps, self.step), dur_ms=dur_ms,
                    bytes=np.array(nbytes))


def summarize(res, cfg):
    dur = res["dur_ms"]
    gbs = res["bytes"] / (dur * 1e-3) / 1e9
    avg_ms = float(dur.mean())
    return dict(
        steps_per_s=len(dur) / (res["span_ms"] * 1e-3),
        ms_per_step=res["span_ms"] / len(dur),
        launch_us_median=float(np.median(dur) * 1e3), launch_us_p10=float(np.percentile(dur, 10) * 1e3),
        launch_us_p90=float(np.percentile(dur, 90) * 1e3), launch_us_mean=avg_ms * 1e3,
        bytes_per_step_mean=float(res["bytes"].mean()),
        achieved_gbs=float(res["bytes"].mean() / (avg_ms * 1e-3) / 1e9),
        achieved_gbs_median=float(np.median(gbs)))


def cpu_oracle_rate(cfg, budget_s: float, threads: int, n_inputs: int = 4, cache=None):
    """The oracle, timed on `threads` host cores over whole layer-half steps of a workload.

    Steps cycle over `n_inputs` seeded input states until `budget_s` seconds of oracle compute
    have passed (at least one step); the selected experts' weights are generated on the host
    outside the timed region and kept for later steps (in `cache`)."""
    import oracle
    import synth
    oracle.set_threads(threads)
    s = oracle.shape_of(cfg)
    d0, d1 = synth.dense_host(cfg, 0), synth.dense_host(cfg, 1)
    shared = synth.expert_host(cfg, 0, None)
    states = [synth.state_host(cfg, i) for i in range(n_inputs)]
    cache = {} if cache is None else cache
    done, spent = 0, 0.0
    while spent < budget_s or done == 0:
        st = states[done % n_inputs]
        # routing (timed), then any missing expert weights generated (untimed), then the rest
        t0 = time.perf_counter()
        mixes = oracle.mix(s, st, d0["w_mix"])
        pre, post, comb = oracle.split(s, mixes, d0["hc_scale"], d0["hc_base"])
        x, norm = oracle.collapse_norm(s, st, pre, d0["w_norm"])
        lg = oracle.router_logits(s, norm, d0["w_router"])
        idx, w, _ = oracle.select(s, lg, d0["bias"])
        spent += time.perf_counter() - t0
        for e in np.unique(idx):
            if int(e) not in cache:
                cache[int(e)] = synth.expert_host(cfg, 0, int(e))
        ex = {int(e): cache[int(e)] for e in np.unique(idx)}
        t0 = time.perf_counter()
        m = oracle.moe(s, norm, idx, w, cfg.routed_fmt, ex, cfg.shared_fmt, shared)
        oracle.expand(s, st, m["block"], post, comb, d1["w_mix"])
        spent += time.perf_counter() - t0
        done += 1
    return dict(value=done / spent, unit="steps/s", cores=threads, kind="oracle",
                sample="%d full layer-half steps of the same workload (%s) cycling over %d "
                       "seeded inputs, %.1f s of oracle compute on %d thread(s); expert weights "
                       "generated outside the timed region" % (
                           done, cfg.name, n_inputs, spent, threads))


def cpu_baseline(cfg1, cfg6, budget_s: float):
    """The oracle on all host cores and on one core, for the 1-row and the 6-row workloads.
    The headline value is all cores at 1 row."""
    import oracle
    n_all = oracle.threads()
    c1, c6 = {}, {}
    one_row = cpu_oracle_rate(cfg1, budget_s, n_all, cache=c1)
    one_row["one_core"] = cpu_oracle_rate(cfg1, budget_s, 1, cache=c1)
    if cfg6 is not None:
        six = cpu_oracle_rate(cfg6, budget_s, n_all, n_inputs=2, cache=c6)
        six["one_core"] = cpu_oracle_rate(cfg6, budget_s, 1, n_inputs=2, cache=c6)
        one_row["rows6"] = six
    oracle.set_threads(n_all)
    return one_row


# ---- HBM traffic from rocprofv3 counters -------------------------------------------------

KERNEL_SOURCES = ["mono_kernels.h", "mono_internal.h", "mono_launch.hip", "mono_k_bf16.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_ffn_layer_traffic.md")


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "moe_decode_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the 1-row kernel recorded from FETCH_SIZE/WRITE_SIZE runs, or
    None when the file is absent or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip("` ")] = v.strip().strip("`")
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _counter_rows(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def pmc_summary(fetch_csv: str, write_csv: str):
    """Per-kernel mean FETCH_SIZE and WRITE_SIZE (KiB per dispatch) and dispatch counts from
    two rocprofv3 --pmc counter CSVs."""
    agg = {}
    for path, ctr in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        for r in _counter_rows(path):
            if r.get("Counter_Name") != ctr:
                continue
            name = r["Kernel_Name"]
            key = (name, ctr)
            d = agg.setdefault(key, {})
            # one value per dispatch (summed over dimensions if split)
            d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, ctr), d in agg.items():
        out.setdefault(name, {})[ctr] = (float(np.mean(list(d.values()))), len(d))
    return out


def trace_summary(trace_csv: str):
    """Per-workload statistics of the layer kernel from a rocprofv3 --kernel-trace CSV.

    The run builds its workloads one after another, each with weight fills and a workspace init
    before its launches, so a maximal run of layer-kernel dispatches with no fill or init in
    between is one workload (device copies of read-backs are ignored)."""
    segs, cur = [], None
    for r in _counter_rows(trace_csv):
        name = r["Kernel_Name"]
        if "k_ffn_layer" in name:
            if cur is None or cur["name"] != name:
                cur = dict(name=name, us=[], vgpr=r["VGPR_Count"], agpr=r["Accum_VGPR_Count"],
                           sgpr=r["SGPR_Count"], lds=r["LDS_Block_Size"],
                           scratch=r["Scratch_Size"], grid=r["Grid_Size_X"],
                           wg=r["Workgroup_Size_X"])
                segs.append(cur)
            cur["us"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        elif "synth_fill" in name or "k_ws_init" in name:
            cur = None
    return segs


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--copies", type=int, default=4, help="independent weight copies rotated")
    ap.add_argument("--cpu-budget", type=float, default=5.0,
                    help="seconds of oracle compute per CPU-baseline leg (4 legs)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-rows6", action="store_true", help="skip the 6- and 8-row workloads")
    ap.add_argument("--no-chain", action="store_true", help="skip the 8-layer chain")
    ap.add_argument("--no-seam", action="store_true",
                    help="skip the attention-half seam and model-tail timings")
    ap.add_argument("--no-drafts", action="store_true",
                    help="skip the draft routing shapes (128 experts top-3, 256 experts top-6)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="first run a plain device copy of this size (counter calibration)")
    ap.add_argument("--trace-summary", metavar="KERNEL_TRACE_CSV",
                    help="summarise a rocprofv3 --kernel-trace CSV per workload and exit")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc counter CSVs and exit (no GPU use)")
    args = ap.parse_args()
    if args.trace_summary:
        for sg in trace_summary(args.trace_summary):
            us = np.array(sg["us"])
            # a workload ends with its two timed passes of --steps launches: per-launch events,
            # then back to back
            b2b = us[-args.steps:]
            per = us[-2 * args.steps:-args.steps] if len(us) >= 2 * args.steps else b2b
            print("%s\tdispatches=%d mean=%.1f median=%.1f min=%.1f max=%.1f timed_mean=%.1f "
                  "back_to_back_mean=%.1f vgpr=%s agpr=%s sgpr=%s lds=%s scratch=%s grid=%sx%s" % (
                      sg["name"], len(us), us.mean(), np.median(us), us.min(), us.max(),
                      per.mean(), b2b.mean(), sg["vgpr"], sg["agpr"], sg["sgpr"], sg["lds"],
                      sg["scratch"], int(sg["grid"]) // max(int(sg["wg"]), 1), sg["wg"]))
        return
    if args.pmc_summary:
        for name, d in sorted(pmc_summary(*args.pmc_summary).items()):
            print("%s\t%s" % (name, "\t".join("%s=%.1f KiB x%d" % (c, v, n)
                                              for c, (v, n) in sorted(d.items()))))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (--gpus %d "
              "refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_decode_layer_amd as mono
    import synth
    mono.lib()  # fails loudly when the HIP library is not built
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calib_mib:
        n = args.copy_calib_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 2.0, out=dst)   # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        log("  copy calibration: 5 x elementwise copy of %d MiB" % args.copy_calib_mib)
        del src, dst

    cfg1 = synth.CONFIGS[2]
    log("building workloads")
    w1 = Workload(cfg1, args.copies)
    r1 = summarize(w1.run(args.steps, args.warmup), cfg1)
    log("  1 row:", json.dumps(r1))
    del w1
    torch.cuda.empty_cache()
    extra = {}
    if not args.no_rows6:
        for key, ci in (("rows6", 3), ("rows8", 4), ("rows8_mxfp8", 10)):
            cfgx = synth.CONFIGS[ci]
            wx = Workload(cfgx, args.copies)
            rx = summarize(wx.run(args.steps, args.warmup), cfgx)
            log("  %s:" % key, json.dumps(rx))
            extra[key] = dict(workload=cfgx.name, rows=cfgx.rows, act_quant=cfgx.act_quant,
                              steps_per_s=rx["steps_per_s"],
                              launch_us_median=rx["launch_us_median"],
                              launch_us_mean=rx["launch_us_mean"],
                              achieved_gbs=rx["achieved_gbs"],
                              frac=rx["achieved_gbs"] / PEAK_HBM_GBS,
                              bytes_per_step=rx["bytes_per_step_mean"])
            del wx
            torch.cuda.empty_cache()
    if not args.no_drafts:
        drafts = {}
        for ci in synth.DRAFT_CONFIGS:
            cfgx = synth.CONFIGS[ci]
            wx = Workload(cfgx, args.copies)
            rx = summarize(wx.run(args.steps, args.warmup), cfgx)
            log("  draft %d:" % ci, json.dumps(rx))
            drafts["e%d_k%d_r%d" % (cfgx.n_experts, cfgx.top_k, cfgx.rows)] = dict(
                workload=cfgx.name, steps_per_s=rx["steps_per_s"],
                launch_us_median=rx["launch_us_median"], achieved_gbs=rx["achieved_gbs"],
                frac=rx["achieved_gbs"] / PEAK_HBM_GBS, bytes_per_step=rx["bytes_per_step_mean"])
            del wx
            torch.cuda.empty_cache()
        extra["drafts"] = drafts
    if not args.no_seam:
        extra["seam"] = seam_timings(cfg1)
        log("  seam:", json.dumps(extra["seam"]))
    if not args.no_chain:
        cfg5 = synth.CONFIGS[5]
        wc = ChainWorkload(cfg5)
        rc = summarize(wc.run(max(args.steps // 2, 1), args.warmup), cfg5)
        log("  chain:", json.dumps(rc))
        extra["chain8"] = dict(workload=cfg5.name, layer_halves=cfg5.layers,
                               chain_steps_per_s=rc["steps_per_s"],
                               chain_us_mean=rc["launch_us_mean"],
                               us_per_layer_half=rc["launch_us_mean"] / cfg5.layers,
                               achieved_gbs=rc["achieved_gbs"],
                               frac=rc["achieved_gbs"] / PEAK_HBM_GBS,
                               bytes_per_chain=rc["bytes_per_step_mean"])
        del wc
        torch.cuda.empty_cache()
    cpu = None if args.no_cpu else cpu_baseline(
        cfg1, None if args.no_rows6 else synth.CONFIGS[3], args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": r1["steps_per_s"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r1["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg1.name, "rows": 1, "hidden": cfg1.hidden,
                   "n_experts": cfg1.n_experts, "top_k": cfg1.top_k, "inter": cfg1.inter,
                   "shared_inter": cfg1.shared_inter, "weights": "bf16",
                   "weight_copies_rotated": args.copies, "inputs_rotated": 64,
                   "launch": "mono_ffn_layer, one persistent launch per step"},
        "roofline": {"bound": "hbm", "achieved": r1["achieved_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": r1["achieved_gbs"] / PEAK_HBM_GBS,
                     "traffic": recorded_traffic(),
                     "algorithmic_bytes": r1["bytes_per_step_mean"],
                     "kernel_source_hash": kernel_source_hash()},
        "launch_us": {"median": r1["launch_us_median"], "p10": r1["launch_us_p10"],
                      "p90": r1["launch_us_p90"], "mean": r1["launch_us_mean"]},
        "bytes_per_step": r1["bytes_per_step_mean"],
        **extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
