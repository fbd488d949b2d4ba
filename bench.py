#!/usr/bin/env python3
"""Benchmark of one masked-diffusion denoising step on one MI355X.

A step is the whole hot path on one batch of seeded synthetic input:
K/V scatter + sparse-query attention (pass 1) + column sums (pass 2) +
posterior / KL lock test / unmask selection, through the two C-ABI calls
on one stream (its time is "value").  Two schedules of the same step with
dlm_posterior on a second stream are reported beside it: its logit stream
from the start of the step ("ms_per_step_two_streams") and from the end of
pass 1 (mask_desc.pass1_done, "ms_per_step_posterior_after_pass1"); in both
its selection waits for the column sums through select.score_ready.
Inputs are resident in HBM before timing starts.  Each timed loop (the
whole step, pass 1 alone, both attention passes, the posterior alone)
rotates over enough copies of its inputs that the bytes it touches total at
least twice the 256 MB Infinity Cache.  The lock flags are in/out, so every
call gets its own copy of the entry flags, made before timing: every step
does the same work.

Prints ONE JSON line.  Headline workload: the SureLock sparse-query step
(B=4, 32 heads x 128, N=8192 with 2048 active rows per batch entry;
posterior 8192 x 126464), the largest single-GPU configuration.  The other
three workloads (LLaDA-like bidirectional layer, multi-block group mask,
long-prefix Attn-Sampler) are timed the same way and reported under
"workloads" in the same line.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from typing import Optional

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20


def visible_pairs(a, counted_only=False) -> int:
    """Sum over active rows (only those feeding the column sums when
    counted_only) and q-heads of the number of visible keys."""
    import numpy as np
    n = np.arange(a.kv_len)
    tot = 0
    for b in range(a.B):
        pos = a.active_idx[b]
        if counted_only:
            pos = pos[(pos >= a.cs_lo) & (pos < a.cs_hi)]
        if a.kind == 0:
            tot += len(pos) * a.kv_len * a.Hq
            continue
        if a.kind == 1:
            kb = np.where(n < a.prefix_len, -1, (n - a.prefix_len) // a.block_size)
            qb = (pos - a.prefix_len) // a.block_size
            vis = (kb[None, :] <= qb[:, None])
        else:
            # int64 throughout: a DUMMY slot's key code must stay above every
            # group id and the prefix's below (no narrowing to the int32 ids)
            slot = np.clip((n - a.prefix_len) // a.block_size, 0, a.n_slots - 1)
            grp = a.slot_group[b].astype(np.int64)
            kcode = np.where(a.slot_state[b][slot] == 0, np.int64(np.iinfo(np.int64).max), grp[slot])
            kcode = np.where(n < a.prefix_len, np.int64(np.iinfo(np.int64).min), kcode)
            qc = grp[(pos - a.prefix_len) // a.block_size]
            vis = kcode[None, :] <= qc[:, None]
        tot += int(vis.sum()) * a.Hq
    return tot


# Sources whose change invalidates a stored counter measurement, per kernel
# tag (the summaries under profiles/ record a SHA-256 of these).
COUNTER_SOURCES = {
    "attn_fwd": ("denoising_step_amd/csrc/attn_kernels.hip", "denoising_step_amd/csrc/dlm_internal.h",
                 "denoising_step_amd/build.py"),
    "colsum": ("denoising_step_amd/csrc/attn_kernels.hip", "denoising_step_amd/csrc/dlm_internal.h",
               "denoising_step_amd/build.py"),
    "posterior": ("denoising_step_amd/csrc/posterior_kernels.hip", "denoising_step_amd/csrc/dlm_internal.h",
                  "denoising_step_amd/build.py"),
}
TRAFFIC_SOURCES = COUNTER_SOURCES["attn_fwd"]


def source_digest(tag: str = "attn_fwd") -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in COUNTER_SOURCES[tag]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _summary_fields(path: str) -> dict:
    """The machine-read "- key: value" lines of a profiles/ summary."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return {}
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    return fields


def stored_traffic(workload: str):
    """HBM bytes per pass-1 launch from the committed counter summary
    (profiles/attn_fwd_<workload>_counters.md), or None when there is none
    or the kernel sources changed since the counters were taken."""
    return (stored_counters("attn_fwd", workload) or {}).get("traffic_bytes_per_launch")


def stored_counters(tag: str, workload: str):
    """Per-launch counter figures of kernel `tag` on `workload` from the
    committed summary profiles/<tag>_<workload>_counters.md (numeric
    fields only), or None when there is none or the kernel sources changed
    since the counters were taken."""
    fields = _summary_fields(os.path.join(ROOT, "profiles", f"{tag}_{workload}_counters.md"))
    if not fields or fields.get("source_sha256") != source_digest(tag):
        return None
    out = {}
    for k, v in fields.items():
        try:
            out[k] = int(v)
        except ValueError:
            try:
                out[k] = float(v)
            except ValueError:
                pass
    out["summary"] = f"profiles/{tag}_{workload}_counters.md"
    return out


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(path: str, kernel_re: Optional[str] = None) -> str:
    """Markdown table of a rocprofv3 kernel_trace.csv: per kernel (those
    whose name matches kernel_re, if given), the dispatch count and the
    mean, median, min and max duration in us."""
    import re
    import statistics
    by = {}
    for r in _read_csv(path):
        if kernel_re and not re.search(kernel_re, r["Kernel_Name"]):
            continue
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault(r["Kernel_Name"], []).append(d)
    lines = ["| kernel | calls | mean us | median us | min us | max us | total us |",
             "|---|---|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {statistics.fmean(v):.2f} | {statistics.median(v):.2f} | "
                     f"{min(v):.2f} | {max(v):.2f} | {sum(v):.1f} |")
    return "\n".join(lines)


LOOP_KERNELS = ("kv_scatter_kernel", "attn_fwd_kernel", "attn_combine_kernel", "colsum_kernel",
                "colsum_reduce_kernel", "posterior_stream_kernel", "posterior_finish_kernel", "posterior_fused_kernel",
                "block_buffer_kernel")


def summarize_loop_trace(path: str) -> str:
    """Per-step table of the last run in a kernel trace of `bench.py --loop`
    (the graph replays), plus, per run, the gaps on the GPU around each
    step: from the stand-in model's last kernel to the step's first, and
    from the step's last kernel to the next kernel."""
    import statistics

    def short(n):
        return n.split("(dlm")[0].split("::")[-1].split("<")[0].split("(")[0]

    rows = sorted(_read_csv(path), key=lambda r: int(r["Start_Timestamp"]))
    ks = [(short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    segs, i = [], 0                       # maximal runs of step kernels: one step each
    while i < len(ks):
        if ks[i][0] in LOOP_KERNELS:
            j = i
            while j + 1 < len(ks) and ks[j + 1][0] in LOOP_KERNELS:
                j += 1
            segs.append((i, j))
            i = j + 1
        else:
            i += 1
    # runs: a Block Buffer initialisation (a lone block_buffer segment) starts each
    runs, cur = [], []
    for a, b in segs:
        if a == b and ks[a][0] == "block_buffer_kernel":
            if cur:
                runs.append(cur)
            cur = []
        else:
            cur.append((a, b))
    if cur:
        runs.append(cur)
    cols = [c for c in LOOP_KERNELS if any(k[0] == c for k in ks)]   # kernels the run launched
    out = ["| step | " + " | ".join(c.replace("_kernel", "") for c in cols) + " | sum |",
           "|---" * (len(cols) + 2) + "|"]
    for si, (a, b) in enumerate(runs[-1]):
        d = {c: 0.0 for c in cols}
        for n, t0, t1 in ks[a:b + 1]:
            d[n] += (t1 - t0) / 1e3
        out.append(f"| {si + 1} | " + " | ".join(f"{d[c]:.1f}" for c in cols) + f" | {sum(d.values()):.1f} |")
    out += ["", "| run | steps | kernel time ms | gaps inside steps us | entry gap median us | exit gap median us |",
            "|---|---|---|---|---|---|"]
    for ri, run in enumerate(runs):
        busy = inside = 0.0
        ent, ext = [], []
        for a, b in run:
            busy += sum(t1 - t0 for _, t0, t1 in ks[a:b + 1]) / 1e3
            inside += ((ks[b][2] - ks[a][1]) - sum(t1 - t0 for _, t0, t1 in ks[a:b + 1])) / 1e3
            if a > 0:
                ent.append((ks[a][1] - ks[a - 1][2]) / 1e3)
            if b + 1 < len(ks):
                ext.append((ks[b + 1][1] - ks[b][2]) / 1e3)
        out.append(f"| {ri + 1} | {len(run)} | {busy / 1e3:.3f} | {inside:.1f} | "
                   f"{statistics.median(ent) if ent else float('nan'):.2f} | "
                   f"{statistics.median(ext) if ext else float('nan'):.2f} |")
    return "\n".join(out)


def summarize_pmc(path: str) -> str:
    """Markdown table of a rocprofv3 counter_collection.csv: per kernel and
    counter, the per-dispatch value (summed over the counter's instances)
    as mean, median, min and max over the dispatches."""
    import statistics
    per = {}
    for r in _read_csv(path):
        key = (r["Kernel_Name"], r["Counter_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    by = {}
    for (k, c, _), v in per.items():
        by.setdefault((k, c), []).append(v)
    lines = ["| kernel | counter | dispatches | mean | median | min | max |",
             "|---|---|---|---|---|---|---|"]
    for (k, c), v in sorted(by.items()):
        lines.append(f"| `{k}` | {c} | {len(v)} | {statistics.fmean(v):.6g} | {statistics.median(v):.6g} | "
                     f"{min(v):.6g} | {max(v):.6g} |")
    return "\n".join(lines)


def copy_probe(n_bytes: int = 256 << 20, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) of a profiler run."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n_bytes, "reps": reps}), flush=True)


def hbm_ceilings(gib: int = 2, reps: int = 10) -> dict:
    """Streaming rates of two library kernels on this GPU, for context beside
    the 8 TB/s nameplate: torch's device-to-device copy (read + write bytes
    per second) and torch's read-only full reduction (torch.sum), each over
    GiB-sized buffers that rotate past the MALL, timed with HIP events.
    They are reference points, not ceilings: the posterior stream reads
    faster than torch.sum does."""
    import torch
    n = (gib << 30) // 4
    bufs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    dst = torch.empty_like(bufs[0])
    out = {}
    for name, fn, bytes_per in (("copy_gbs", lambda i: dst.copy_(bufs[i % 2]), 8 * n),
                                ("read_gbs", lambda i: torch.sum(bufs[i % 2]), 4 * n)):
        ms = time_loop(fn, 2, reps, 3)
        out[name] = round(bytes_per / ms / 1e6, 0)
    out["method"] = (f"{gib} GiB fp32 buffers, two rotating; copy = torch copy_ (read + write bytes), "
                     "read = torch.sum (read bytes); HIP events over 10 calls after 3 warm-up; "
                     "library kernels, reference points rather than ceilings")
    del bufs, dst
    torch.cuda.empty_cache()
    return out


def time_loop(fn, n_sets, steps, warmup, per_step=False):
    """ms per call over `steps` timed calls after `warmup` untimed ones,
    bracketed by synchronisations; with per_step, also every call's own
    duration (an event between consecutive calls)."""
    import torch
    for i in range(warmup):
        fn(i % n_sets)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1 if per_step else 2)]
    ev[0].record()
    for i in range(steps):
        fn(i % n_sets)
        if per_step:
            ev[i + 1].record()
    ev[-1].record()
    torch.cuda.synchronize()
    mean = ev[0].elapsed_time(ev[-1]) / steps        # ms per call
    if not per_step:
        return mean
    return mean, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def cpu_baseline(w, budget_heads=None, budget_rows=1024):
    """Time the oracle, as it stands, on a bounded sample of the workload and
    scale to the metric's unit (rows/s of a whole step): attention and
    column sums on a few whole GQA groups of q-heads (the per-head work is
    identical across heads), the posterior on the first rows."""
    import oracle
    from workloads import AttnCase
    a, p = w.attn, w.post
    H = budget_heads or max(1, min(a.Hq, 8))
    # keep whole GQA groups so the sample has the workload's structure
    H = max(a.G, (H // a.G) * a.G)
    sub = AttnCase(**{**a.__dict__, "Hq": H, "Hkv": H // a.G, "q": a.q[:, :H],
                      "k": a.k[:, :H // a.G], "v": a.v[:, :H // a.G],
                      "cache_k": a.cache_k[:, :H // a.G], "cache_v": a.cache_v[:, :H // a.G]})
    t0 = time.perf_counter()
    kv = oracle.effective_kv(sub)
    _, lse = oracle.attention(sub, kv=kv)
    oracle.colsum(sub, lse, kv=kv)
    t_attn_sample = time.perf_counter() - t0
    t_attn = t_attn_sample * (a.Hq / H)
    rows = min(p.R, budget_rows)
    t0 = time.perf_counter()
    oracle.posterior(p.logits[:rows], p.prev[:rows], p.locked[:rows], p.eps)
    t_post_sample = time.perf_counter() - t0
    t_post = t_post_sample * (p.R / rows)
    t_step = t_attn + t_post
    threads = oracle.num_threads()
    return {"value": a.B * a.M / t_step, "unit": "rows/s", "cores": threads,
            "kind": "oracle",
            "sample": f"attention + column sums on {H} of {a.Hq} q-heads (scaled x{a.Hq / H:g}), "
                      f"posterior on {rows} of {p.R} rows (scaled x{p.R / rows:g}); "
                      f"{t_attn_sample + t_post_sample:.1f} s of CPU wall time sampled, "
                      f"estimated step time {t_step:.2f} s",
            "omp_threads": threads, "affinity_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def loop_bench(args):
    """A whole SureLock-style run at the LLaDA-8B layer shape: one 1024-
    position block of which the first 512 are an unmasked prompt (recomputed
    until it locks) and 512 are masked, 32 heads of width 128, vocabulary
    126464, the 16 most confident rows unmasked per step, eps 1e-3.  Each
    step is the hot path (attention over the M_t computed rows, the
    posterior of the unlocked rows, the Block Buffer advance), timed per
    step eagerly and as replays of one captured HIP graph; the stand-in for
    the model (q / k / v rows, logits that settle geometrically per
    position) runs between the timed regions.  Prints one JSON line."""
    import statistics
    import types

    import numpy as np
    import torch

    import workloads as W
    from denoising_step_amd.loop import DeviceLoop

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    B, H, D, n, V = 1, 32, 128, 1024, 126464
    n_prompt, k_step = 512, 16
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    std = 1.0 / math.sqrt(D)

    def randn(shape, scale):
        return torch.randn(shape, generator=gen, device=dev).mul_(scale)

    base = randn((B, n, V), 3.0)
    dec0 = torch.zeros((B, n), dtype=torch.uint8, device=dev)
    dec0[:, :n_prompt] = 1
    tok0 = torch.where(dec0 == 1, base.argmax(-1).to(torch.int32), torch.full_like(dec0, -1, dtype=torch.int32))
    case = types.SimpleNamespace(
        name="llada_surelock_run", B=B, Hq=H, Hkv=H, D=D, prefix_len=0, block_size=n, n_slots=1,
        max_active=1, T=n, V=V, eps=1e-3, mode=W.SEL_TOPK_CONF, k=k_step, tau=0.9,
        cache_k=randn((B, H, n, D), std).to(torch.bfloat16), cache_v=randn((B, H, n, D), std).to(torch.bfloat16),
        q=None, k_new=None, v_new=None, logits=None, decoded0=dec0, tokens0=tok0)

    class Run(DeviceLoop):
        def __init__(self):
            super().__init__(case)
            self.qb = randn((B, H, n, D), std).to(torch.bfloat16)
            self.kb = randn((B, H, n, D), std).to(torch.bfloat16)
            self.vb = randn((B, H, n, D), std).to(torch.bfloat16)
            self.rate = torch.empty((B, n), device=dev).uniform_(0.5, 0.75, generator=gen)
            self.noise_seed = args.seed + 1

        def feed(self, t, stream=None):
            with torch.cuda.stream(stream):
                idx = (self.bb.active_idx - self.P).clamp_(min=0).long()
                for src, dst in ((self.qb, self.q), (self.kb, self.k), (self.vb, self.v)):
                    torch.gather(src, 2, idx[:, None, :, None].expand(B, H, n, D), out=dst)
                if t > 0:
                    self.y.copy_(self.x)
                g = torch.Generator(device=dev)
                g.manual_seed(self.noise_seed * 100003 + t)
                torch.randn(self.x.shape, generator=g, device=dev, out=self.x)
                self.x.mul_((self.rate ** t)[..., None]).add_(base)
                if t == 0:
                    self.y.copy_(self.x)

    run = Run()
    s = torch.cuda.Stream()

    # 1. the row counts of the run (host reads between steps: not timed)
    run.start(s)
    m_t, n_steps = [], 0
    while True:
        st = run.state()
        if int(st["n_open"].sum()) == 0 or n_steps >= n:
            break
        m_t.append(int(st["m_active"].sum()))
        run.feed(n_steps, s)
        run.step(s)
        n_steps += 1
    torch.cuda.synchronize()
    tokens_ref = run.bb.tokens.cpu()

    def timed(replay):
        run.start(s)
        torch.cuda.synchronize()
        g = run.capture(s) if replay else None
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_steps)]
        for t in range(n_steps):
            run.feed(t, s)
            ev[t][0].record(s)
            if replay:
                with torch.cuda.stream(s):
                    g.replay()
            else:
                run.step(s)
            ev[t][1].record(s)
        torch.cuda.synchronize()
        assert torch.equal(run.bb.tokens.cpu(), tokens_ref), "the timed run diverged"
        return [a.elapsed_time(b) * 1e3 for a, b in ev]

    timed(False)                       # warm-up
    eager = timed(False)
    graph = timed(True)
    # a full recompute computes every row at every step: each step at the cost
    # of the run's own steps that compute every row (nothing locked yet), the
    # median of those, not the first alone (one sample)
    n_full = max(1, sum(1 for m in m_t if m == m_t[0]))
    full = n_steps * statistics.median(eager[:n_full])
    full_graph = n_steps * statistics.median(graph[:n_full])
    line = {
        "metric": "hot-path time of a whole SureLock run (per denoising step)",
        "unit": "us", "n_gpus": 1, "steps": n_steps, "data": "synthetic (seeded, drawn on the device)",
        "config": {"workload": case.name, "B": B, "Hq": H, "Hkv": H, "D": D, "positions": n,
                   "prompt_unmasked": n_prompt, "vocab": V, "selection": "top-16 confidence per step",
                   "eps": case.eps},
        "M_t": m_t,
        "step_us_eager": [round(x, 1) for x in eager],
        "step_us_graph": [round(x, 1) for x in graph],
        "total_ms_eager": round(sum(eager) / 1e3, 3),
        "total_ms_graph": round(sum(graph) / 1e3, 3),
        "full_recompute_ms": round(full / 1e3, 3),
        "full_recompute_ms_graph": round(full_graph / 1e3, 3),
        "rows_computed_frac": round(sum(m_t) / (n_steps * n), 4),
        "time_frac_of_full": round(sum(graph) / full_graph, 4),
        "time_frac_of_full_eager": round(sum(eager) / full, 4),
    }
    print(json.dumps(line), flush=True)


def layer_bench(args):
    """The active-row projections and feed-forward of one LLaDA-8B-shaped
    layer (width 4096, 32 heads of 128, SwiGLU width 12288, B=1, 2048
    positions) for a range of active-row counts M_t: each call timed alone
    with HIP events, against the bf16 MFMA peak (2 M N K flops) and the
    weight bytes read (the bound at small M_t), with the weights in the
    packed layout (dlm_pack_weights, what a server keeps resident) and
    row-major.  Two sets of weights rotate so their footprint exceeds the
    256 MB MALL.  Prints one JSON line."""
    import torch

    import denoising_step_amd as dlm

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    d, Hq, Hkv, D, F, n_pos = 4096, 32, 32, 128, 12288, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)

    def w(shape, fan_in):
        return (torch.randn(shape, generator=gen, device=dev) / math.sqrt(fan_in)).to(torch.bfloat16)

    sets = [dict(qkv=w(((Hq + 2 * Hkv) * D, d), d), o=w((d, Hq * D), Hq * D), g=w((F, d), d),
                 u=w((F, d), d), dn=w((d, F), F)) for _ in range(2)]
    packed = [{k: dlm.dlm_pack_weights(t) for k, t in s_.items()} for s_ in sets]
    x = torch.randn((1, n_pos, d), generator=gen, device=dev).to(torch.bfloat16)
    res = []
    m_list = [int(v) for v in args.layer_m.split(",")] if args.layer_m else [1024, 512, 256, 128, 64, 32, 16]
    layouts = [("packed", packed), ("row_major", sets)]
    if args.layer_layout != "both":
        layouts = [lw for lw in layouts if lw[0] == args.layer_layout]
    for M in m_list:
        act = torch.sort(torch.randperm(n_pos, generator=gen, device=dev)[:M])[0].to(torch.int32)[None]
        q = torch.empty((1, Hq, M, D), dtype=torch.bfloat16, device=dev)
        k = torch.empty((1, Hkv, M, D), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        ao = torch.randn((1, Hq, M, D), generator=gen, device=dev).to(torch.bfloat16)
        h = torch.empty((1, M, d), dtype=torch.bfloat16, device=dev)
        row = {"M_t": M}
        for layout, ws_ in layouts:
            L = dlm.LayerDesc(B=1, n_pos=n_pos, d=d, M=M, active_idx=act, Hq=Hq, Hkv=Hkv, D=D, F=F,
                              weights_packed=layout == "packed")
            ws = torch.empty(max(1, dlm.dlm_layer_workspace_bytes(L)), dtype=torch.uint8, device=dev)
            calls = {
                "qkv": (lambda i: dlm.dlm_proj_qkv(L, x, ws_[i]["qkv"], q, k, v, ws),
                        (Hq + 2 * Hkv) * D, d),
                "out": (lambda i: dlm.dlm_proj_out(L, x, ao, ws_[i]["o"], h, ws), d, Hq * D),
                "ffn": (lambda i: dlm.dlm_ffn(L, h, ws_[i]["g"], ws_[i]["u"], ws_[i]["dn"], x, ws),
                        None, None),
            }
            r = {}
            for name, (fn, N, K) in calls.items():
                ms = time_loop(fn, 2, args.steps, args.warmup)
                if name == "ffn":
                    flops = 2.0 * M * (2 * F * d + d * F)
                    wbytes = 3.0 * F * d * 2
                else:
                    flops = 2.0 * M * N * K
                    wbytes = 2.0 * N * K
                r[name] = {"us": round(ms * 1e3, 2), "tflops": round(flops / ms / 1e9, 1),
                           "mfma_frac": round(flops / ms / 1e9 / 2500.0, 3),
                           "weight_gbs": round(wbytes / ms / 1e6, 0),
                           "hbm_frac": round(wbytes / ms / 1e6 / 8000.0, 3)}
            row[layout] = r
            print(f"layer M_t={M} {layout}: " + " ".join(
                f"{n}={r[n]['us']}us/{r[n]['tflops']}TF/{r[n]['weight_gbs'] / 1000:.2f}TB/s" for n in calls),
                file=sys.stderr, flush=True)
        res.append(row)
    line = {"metric": "active-row projections and feed-forward of one layer", "unit": "us",
            "n_gpus": 1, "dtype": "bf16", "data": "synthetic (random weights drawn on the device)",
            "config": {"workload": "layer_llada", "d": d, "Hq": Hq, "Hkv": Hkv, "D": D, "F": F,
                       "positions": n_pos},
            "peak": {"mfma_bf16_tflops": 2500.0, "hbm_gbs": 8000.0}, "rows": res}
    print(json.dumps(line), flush=True)


def r2l_bench(args):
    """The R2LM right-to-left scan at the Bifocal page's serving shape (batch
    8, a 256-token generation block, width 2048, 16 states), the correction
    added to the hidden stream: timed with HIP events; bound by the
    exponentials (one per state update: B L E N of them) on the
    transcendental unit, and reported against HBM bytes too.  Prints one
    JSON line."""
    import torch

    import denoising_step_amd as dlm
    import workloads as W
    from denoising_step_amd.runner import bf16_to_device

    torch.cuda.set_device(0)
    c = W.r2l_bifocal(seed=args.seed)
    dev = torch.device("cuda")
    bf = lambda a: bf16_to_device(a, dev)
    n_sets = 8                      # rotate inputs past the MALL
    sets = [dict(u=bf(c.u), dl=bf(c.delta), Bm=bf(c.Bm), Cm=bf(c.Cm), x=bf(c.x)) for _ in range(n_sets)]
    A = torch.from_numpy(c.A).to(dev)
    D = torch.from_numpy(c.Dv).to(dev)

    def call(i):
        s_ = sets[i]
        dlm.dlm_r2l_scan(c.B, c.L, c.E, c.N, c.gate, s_["u"], s_["dl"], A, s_["Bm"], s_["Cm"], D, x=s_["x"])

    ms = time_loop(call, n_sets, args.steps, args.warmup)
    updates = float(c.B) * c.L * c.E * c.N
    # one state update: at least 4 full-rate fp32 VALU ops (delta*A, delta*u*B, the state FMA,
    # the output FMA) and one quarter-rate exp: 4/16 + 1/4 = 0.5 SIMD clocks per lane;
    # 256 CUs x 4 SIMDs at 2.4 GHz
    peak = 256 * 4 * 2.4e9 / 0.5
    nbytes = float(c.B) * c.L * c.E * 2 * 4 + 2.0 * c.B * c.L * c.N * 2   # u, delta, x read + x write; B, C
    line = {"metric": "R2LM right-to-left scan per denoising step", "unit": "us", "n_gpus": 1,
            "value_us": round(ms * 1e3, 2), "dtype": "bf16 in, fp32 scan",
            "data": "synthetic (seeded)",
            "config": {"workload": c.name, "B": c.B, "L": c.L, "E": c.E, "N": c.N},
            "roofline": {"bound": "alu", "achieved": round(updates / ms / 1e9, 3),
                         "peak": round(peak / 1e12, 3), "unit": "T state updates/s",
                         "frac": round(updates / ms * 1e3 / peak, 3),
                         "hbm_gbs": round(nbytes / ms / 1e6, 0), "hbm_frac": round(nbytes / ms / 1e6 / 8000.0, 3)}}
    print(json.dumps(line), flush=True)


HEADLINE = "surelock_sparse"
EXTRAS = ("llada_bidirectional", "mbd_multiblock", "long_prefix_sampler")
ATTN_TARGET, POST_TARGET = 0.5, 0.7
LOOPS = ("step", "step_two_streams", "step_after_pass1", "pass1", "passes12", "posterior")


def _nbytes(*ts) -> int:
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


def loop_footprints(ds) -> dict:
    """Bytes of device memory one timed call of each loop touches in one
    input set (what rotation must keep out of the 256 MB MALL)."""
    attn_ws = _nbytes(ds.attn_ws)
    pass1 = _nbytes(ds.q, ds.cache_k, ds.cache_v, ds.out, ds.lse)
    post = _nbytes(ds.logits, ds.prev, ds.locked, ds.sel, ds.kl, ds.conf, ds.post_ws)
    step = pass1 + _nbytes(ds.k, ds.v, ds.colsum) + attn_ws + post
    return {"step": step, "step_two_streams": step, "step_after_pass1": step, "pass1": pass1,
            "passes12": pass1 + _nbytes(ds.colsum) + attn_ws, "posterior": post}


def measure_workload(name, args, loops=LOOPS, with_cpu=False, spread=True):
    """Time the loops of one workload; returns the per-workload record."""
    import numpy as np
    import torch

    import workloads as W
    import denoising_step_amd as dlm
    from denoising_step_amd.runner import DeviceStep

    w = W.get(name, seed=args.seed)
    a, p = w.attn, w.post
    print(f"bench: {name}: {w.description}", file=sys.stderr, flush=True)
    first = DeviceStep(w)
    fp = loop_footprints(first)
    # every timed loop cycles >= 2x the MALL with the bytes that loop touches
    need = {k: max(1, math.ceil(2 * MALL_BYTES / fp[k])) for k in loops}
    n_sets = max(need.values())
    sets = [first] + [DeviceStep(w) for _ in range(n_sets - 1)]
    stream = torch.cuda.current_stream()
    # one fresh copy of the entry lock flags per call, made before timing
    # (the flags are in/out; every timed call must see the same entry state)
    n_calls = (args.steps + args.warmup) * (len(loops) + (1 if spread else 0))
    lock_bufs = [sets[i % n_sets].locked0.clone() for i in range(n_calls)]
    calls = [0]

    def fresh_lock():
        calls[0] += 1
        return lock_bufs[(calls[0] - 1) % len(lock_bufs)]

    def step(i):
        sets[i].run(stream, locked=fresh_lock())

    def step_two_streams(i):
        sets[i].run(stream, locked=fresh_lock(), overlap=True)

    def step_after_pass1(i):   # the posterior on a second stream from the end of pass 1
        sets[i].run(stream, locked=fresh_lock(), overlap="pass1")

    def pass1(i):              # no fresh K/V (already in the cache), no column sums
        ds = sets[i]
        dlm.dlm_step_attn(ds.q, None, None, ds.kv, ds.active_idx, ds.md, ds.out, ds.lse, None, stream)

    def passes12(i):           # both attention passes, no fresh K/V
        ds = sets[i]
        dlm.dlm_step_attn(ds.q, None, None, ds.kv, ds.active_idx, ds.md, ds.out, ds.lse, ds.colsum, stream)

    def posterior(i):
        sets[i].run_posterior(stream, locked=fresh_lock())

    fns = {"step": step, "step_two_streams": step_two_streams, "step_after_pass1": step_after_pass1, "pass1": pass1,
           "passes12": passes12, "posterior": posterior}
    ms = {}
    for k in loops:
        ms[k] = time_loop(fns[k], n_sets, args.steps, args.warmup)
        print(f"bench: {name}: {k}: {ms[k] * 1e3:.2f} us/call", file=sys.stderr, flush=True)

    pairs = visible_pairs(a)
    alg_flops = 4.0 * a.D * pairs                       # QK^T and PV, 2 flops per MAC
    cs_flops = 2.0 * a.D * visible_pairs(a, counted_only=True)   # pass 2 recomputes QK^T
    unlocked = int((p.locked == 0).sum())
    post_bytes = 8.0 * unlocked * p.V
    rec = {"config": {"workload": name, "B": a.B, "Hq": a.Hq, "Hkv": a.Hkv, "D": a.D,
                      "kv_len": a.kv_len, "active_rows": a.M, "posterior_rows": p.R, "vocab": p.V,
                      "mask": ["full", "block_causal", "group"][a.kind], "selection": p.mode},
           "rows_per_step": a.B * a.M,
           "timing": {"n_sets": n_sets, "warmup": args.warmup, "steps": args.steps,
                      "loops": {k: {"footprint_mb_per_set": round(fp[k] / 2**20, 1),
                                    "mb_cycled": round(n_sets * fp[k] / 2**20, 1),
                                    "mall_multiple": round(n_sets * fp[k] / MALL_BYTES, 2)}
                                for k in loops}}}
    if "step" in ms:
        rec["ms_per_step"] = ms["step"]
        rec["rows_per_s"] = a.B * a.M / (ms["step"] * 1e-3)
        if spread:
            # single-step spread from its own loop: an event after every step
            # adds a small gap, so ms_per_step comes from the loop without
            _, step_ms = time_loop(step, n_sets, args.steps, 0, per_step=True)
            rec["step_ms_p10_p50_p90"] = [float(x) for x in np.percentile(np.array(step_ms), [10, 50, 90])]
    if "step_two_streams" in ms:
        rec["ms_per_step_two_streams"] = ms["step_two_streams"]
    if "step_after_pass1" in ms:
        rec["ms_per_step_posterior_after_pass1"] = ms["step_after_pass1"]
    if "step" in ms:
        # The step as the library runs it fastest for this shape: serial, or
        # with the posterior's logit stream on a second stream from the end of
        # pass 1 (mask_desc.pass1_done; the calling stream waits for it at the
        # end of every step, so each timed step holds all of its work).
        rec["ms_per_step_serial"] = ms["step"]
        rec["config"]["schedule"] = "serial"
        if ms.get("step_after_pass1", float("inf")) < ms["step"]:
            rec["ms_per_step"] = ms["step_after_pass1"]
            rec["rows_per_s"] = a.B * a.M / (ms["step_after_pass1"] * 1e-3)
            rec["config"]["schedule"] = "posterior on a second stream from the end of pass 1"
    if "pass1" in ms:
        t = alg_flops / (ms["pass1"] * 1e-3) / 1e12
        rec["attention_pass1"] = {
            "bound": "mfma",
            "kernel": "attention pass 1 (sparse-query flash attention; with the key-split merge "
                      "when the launch plan splits keys)",
            "achieved": t, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": t / PEAK_BF16_TFLOPS,
            "target": ATTN_TARGET, "target_met": t / PEAK_BF16_TFLOPS >= ATTN_TARGET,
            "per_launch_flops": alg_flops, "avg_launch_us": ms["pass1"] * 1e3,
            "traffic": stored_traffic(name),
            "counters": stored_counters("attn_fwd", name)}
    if "passes12" in ms:
        t = (alg_flops + cs_flops) / (ms["passes12"] * 1e-3) / 1e12
        rec["attention_passes_1_2"] = {
            "achieved": t, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": t / PEAK_BF16_TFLOPS,
            "target": ATTN_TARGET, "target_met": t / PEAK_BF16_TFLOPS >= ATTN_TARGET,
            "flops": alg_flops + cs_flops, "avg_call_us": ms["passes12"] * 1e3,
            "counters": stored_counters("colsum", name)}
    if "posterior" in ms:
        g = post_bytes / (ms["posterior"] * 1e-3) / 1e9
        rec["posterior_roofline"] = {
            "bound": "hbm", "achieved": g, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": g / PEAK_HBM_GBS,
            "target": POST_TARGET, "target_met": g / PEAK_HBM_GBS >= POST_TARGET,
            "per_launch_bytes": post_bytes, "avg_launch_us": ms["posterior"] * 1e3,
            "counters": stored_counters("posterior", name)}
    # executed bf16 MFMA FLOPs per call (profiler counters) over the live time
    c1 = (rec.get("attention_pass1") or {}).get("counters") or {}
    c2 = (rec.get("attention_passes_1_2") or {}).get("counters") or {}
    f1 = c1.get("executed_mfma_flops_per_launch")
    f2 = c2.get("executed_mfma_flops_per_launch")
    for key, ms_key, flops in (("attention_pass1", "pass1", f1),
                               ("attention_passes_1_2", "passes12", f1 + f2 if f1 and f2 else None)):
        if key in rec and flops:
            t = flops / (ms[ms_key] * 1e-3) / 1e12
            rec[key]["executed_mfma_flops"] = flops
            rec[key]["executed_tflops"] = t
            rec[key]["executed_frac"] = t / PEAK_BF16_TFLOPS
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w)
    del sets, lock_bufs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def dominant_roofline(rec) -> dict:
    """The roofline object of the kernel that takes the largest share of
    the step: attention pass 1 or the posterior stream (their own loops)."""
    p1, po = rec["attention_pass1"], rec["posterior_roofline"]
    if po["avg_launch_us"] > p1["avg_launch_us"]:
        r = {k: po[k] for k in ("bound", "achieved", "peak", "unit", "frac")}
        r.update(kernel="posterior stream (KL, confidence, lock) + selection",
                 per_launch_bytes=po["per_launch_bytes"], avg_launch_us=po["avg_launch_us"],
                 traffic=(po.get("counters") or {}).get("traffic_bytes_per_launch"),
                 counters=po.get("counters"))
    else:
        r = {k: p1[k] for k in ("bound", "achieved", "peak", "unit", "frac", "kernel", "per_launch_flops",
                                "avg_launch_us", "traffic", "counters")}
    r["chosen_as"] = "largest single-kernel share of the step time, from the loops below"
    return r


def _pmc_per_dispatch(path, kernel_re):
    """{(kernel, dispatch): {counter: value summed over instances}} of the
    dispatches whose kernel name matches kernel_re."""
    import re
    per = {}
    for r in _read_csv(path):
        if not re.search(kernel_re, r["Kernel_Name"]):
            continue
        d = per.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def _per_launch(per, counter):
    """Per launch: the median over dispatches of each matching kernel, summed
    over the kernels (a launch of the posterior is its stream and finish)."""
    import statistics
    by = {}
    for (k, _), c in per.items():
        if counter in c:
            by.setdefault(k, []).append(c[counter])
    return sum(statistics.median(v) for v in by.values())


def counter_fields(tag, kernel_re, sq=None, fetch=None, write=None, copy_fetch=None, copy_write=None,
                   copy_bytes=256 << 20) -> str:
    """The machine-read lines of a profiles/<tag>_<workload>_counters.md
    summary from rocprofv3 counter_collection.csv files: executed bf16 MFMA
    FLOPs (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512), MFMA-busy cycles, VALU
    instructions per MFMA, co-issue and dependency-wait shares (one SQ pass);
    HBM bytes from FETCH_SIZE and WRITE_SIZE (KiB), each scaled by what it
    reads for a plain device copy of copy_bytes."""
    lines = [f"- source_sha256: `{source_digest(tag)}`"]
    if sq:
        per = _pmc_per_dispatch(sq, kernel_re)
        lines.append("- kernel: `" + "`, `".join(sorted({k for k, _ in per})) + "`")
        mops = _per_launch(per, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        busy = _per_launch(per, "SQ_VALU_MFMA_BUSY_CYCLES")
        mfma = _per_launch(per, "SQ_INSTS_MFMA")
        valu = _per_launch(per, "SQ_INSTS_VALU")
        lines += [f"- executed_mfma_flops_per_launch: {int(round(mops * 512))}",
                  f"- mfma_busy_cycles_per_launch: {int(round(busy))}",
                  # busy cycles spread over the 1024 SIMDs at the 2.4 GHz nameplate clock
                  f"- mfma_busy_us_at_nameplate: {busy / 1024 / 2.4e3:.2f}",
                  f"- valu_per_mfma: {valu / mfma:.3f}",
                  f"- coexec_frac_of_mfma_busy: "
                  f"{_per_launch(per, 'SQ_VALU_MFMA_COEXEC_CYCLES') / busy:.3f}",
                  f"- wait_frac_of_wave_cycles: "
                  f"{_per_launch(per, 'SQ_WAIT_INST_ANY') / _per_launch(per, 'SQ_WAVE_CYCLES'):.3f}"]
    if fetch and write and copy_fetch and copy_write:
        kib = copy_bytes / 1024
        fs = kib / _per_launch(_pmc_per_dispatch(copy_fetch, "copyBuffer"), "FETCH_SIZE")
        ws = kib / _per_launch(_pmc_per_dispatch(copy_write, "copyBuffer"), "WRITE_SIZE")
        f_kib = _per_launch(_pmc_per_dispatch(fetch, kernel_re), "FETCH_SIZE")
        w_kib = _per_launch(_pmc_per_dispatch(write, kernel_re), "WRITE_SIZE")
        lines += [f"- fetch_scale: {fs:.4f}", f"- write_scale: {ws:.4f}",
                  f"- fetch_kib_per_launch: {f_kib:.0f}", f"- write_kib_per_launch: {w_kib:.0f}",
                  f"- traffic_bytes_per_launch: {int(round((f_kib * fs + w_kib * ws) * 1024))}"]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline workload only (no per-workload extras)")
    ap.add_argument("--only", choices=LOOPS,
                    help="run only this loop on --config (profiler runs) and print its record")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration) and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="CSV [REGEX]",
                    help="summarise a rocprofv3 kernel_trace.csv (per-kernel mean / median; only the "
                         "kernels matching REGEX if given) and exit")
    ap.add_argument("--summarize-loop-trace", metavar="CSV",
                    help="per-step table and step gaps of a kernel trace of --loop, and exit")
    ap.add_argument("--summarize-pmc", metavar="CSV",
                    help="summarise a rocprofv3 counter_collection.csv (per kernel and counter) and exit")
    ap.add_argument("--counter-fields", nargs="+", metavar="ARG",
                    help="TAG KERNEL_RE [sq=CSV] [fetch=CSV write=CSV copy_fetch=CSV copy_write=CSV]: print "
                         "the machine-read lines of a counter summary and exit")
    ap.add_argument("--loop", action="store_true",
                    help="time a whole multi-step SureLock run instead (its own JSON line)")
    ap.add_argument("--layer", action="store_true",
                    help="time a layer's active-row projections and feed-forward instead")
    ap.add_argument("--layer-m", metavar="M,M,...",
                    help="with --layer: only these active-row counts")
    ap.add_argument("--layer-layout", choices=("both", "packed", "row_major"), default="both",
                    help="with --layer: the weight layouts to time")
    ap.add_argument("--r2l", action="store_true",
                    help="time the R2LM right-to-left scan instead")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is a design, not a build", file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace[:2]))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_loop_trace:
        print(summarize_loop_trace(args.summarize_loop_trace))
        return
    if args.counter_fields:
        tag, kre, *kv = args.counter_fields
        print(counter_fields(tag, kre, **dict(x.split("=", 1) for x in kv)))
        return
    if args.copy_probe:
        copy_probe()
        return
    if args.loop:
        loop_bench(args)
        return
    if args.layer:
        layer_bench(args)
        return
    if args.r2l:
        r2l_bench(args)
        return

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.only:
        rec = measure_workload(args.config, args, loops=(args.only,), spread=False)
        print(json.dumps(rec), flush=True)
        return

    head = measure_workload(args.config, args, with_cpu=not args.no_cpu_baseline)
    res = {
        "metric": "active query-rows/s per denoising step",
        "value": head["rows_per_s"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the pages' workloads, no trained weights)",
        "config": head["config"],
        "roofline": dominant_roofline(head),
    }
    ceil = hbm_ceilings()
    res["hbm_reference_rates"] = ceil
    pr = head["posterior_roofline"]
    pr["vs_torch_sum_read"] = round(pr["achieved"] / ceil["read_gbs"], 3) if ceil.get("read_gbs") else None
    for k in ("attention_pass1", "attention_passes_1_2", "posterior_roofline", "step_ms_p10_p50_p90",
              "ms_per_step_serial", "ms_per_step_two_streams", "ms_per_step_posterior_after_pass1", "timing"):
        res[k] = head[k]
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head["cpu_baseline"]
    if not args.no_extras:
        res["workloads"] = {}
        for name in EXTRAS:
            if name == args.config:
                continue
            rec = measure_workload(name, args)
            res["workloads"][name] = {
                "config": rec["config"], "rows_per_s": rec["rows_per_s"], "ms_per_step": rec["ms_per_step"],
                "step_ms_p10_p50_p90": rec["step_ms_p10_p50_p90"],
                "ms_per_step_serial": rec["ms_per_step_serial"],
                "ms_per_step_two_streams": rec["ms_per_step_two_streams"],
                "ms_per_step_posterior_after_pass1": rec["ms_per_step_posterior_after_pass1"],
                "attention_pass1": rec["attention_pass1"], "attention_passes_1_2": rec["attention_passes_1_2"],
                "posterior_roofline": rec["posterior_roofline"], "timing": rec["timing"]}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
