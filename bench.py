#!/usr/bin/env python3
"""Throughput of MLA decode over a paged latent KV cache on one MI355X.

One step = one pass of the whole path over one batch: split schedule
(mla_get_split_metadata), then mla_decode_fwd (attention kernel + LSE merge of
split sequences); the tiny workload (one sequence of four pages) runs the
unsplit single-launch path. Inputs are seeded synthetic data already resident
in HBM. To keep the 256 MB Infinity Cache from serving repeat reads, steps
rotate over several copies of the page pool.

By default the six decode workloads are measured and ONE JSON line is printed.
Its headline (value, ms_per_step, roofline, cpu_baseline) is the largest one,
fp8 (batch 128, 128 heads, q_len 2 causal, 8192 cached tokens, fp8 cache), and
its `configs` array holds every workload:
  step_ms     whole step, replayed from captured HIP graphs: median, min and
              mean over the timed steps (each step bracketed by events)
  kernel_ms   each kernel of the step alone (attention, metadata, combine),
              from HIP events recorded by the kernel dispatches: median, min,
              mean over >= 50 launches
  tflops, kv_gbps, frac_step   the whole step against the binding roofline
  frac_kernel                  the attention kernel alone (mean launch)
  traffic                      HBM bytes per attention launch from the
                               committed rocprofv3 counters (null if the
                               kernel source changed since)
`clocks` holds the graphics clock of each XCD and the memory clock read with
the amdsmi library while the headline workload runs.

--config NAME measures one workload (also varlen, fp8mma, prefill, extend).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + effective KV GB/s, % of roofline, per batch/heads/q_len"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA
DECODE_CONFIGS = ["tiny", "share16", "share16_fp8", "mtp", "ragged", "fp8"]
HEADLINE = "fp8"
# the tiny workload's four pages are one work unit either way: one launch,
# no schedule, no merge
UNSPLIT = {"tiny"}


def algorithmic(w):
    """Bytes and flops the method itself must move / compute for one step."""
    import numpy as np
    B, H = w.batch, w.num_heads
    q_lens = [int(x) for x in w.q_lens]
    L = w.seqlens.astype(np.int64)
    e, f = (2, 0) if w.kv_dtype == "bf16" else (1, 4)
    kv = int(np.sum(L * (576 * e + f)))
    pages = int(np.sum((L + 63) // 64))
    q_bytes = sum(q_lens) * H * 576 * 2
    out_bytes = sum(q_lens) * H * (512 + 1) * 4
    meta = 4 * pages + 4 * B + (4 * (B + 1) if w.varlen else 0)
    vis = 0
    for b in range(B):
        s = q_lens[b]
        for i in range(s):
            vis += max(0, min(int(L[b]), int(L[b]) - s + i + 1))
    flops = 2 * H * (576 + 512) * vis
    return dict(kv_bytes=kv, bytes=kv + q_bytes + out_bytes + meta, flops=flops, exps=H * vis,
                pages=pages, tokens=int(np.sum(L)))


def kernel_source_digest() -> str:
    """SHA-256 of the attention kernel sources with comments and blank space
    removed, so that editing a comment does not count as changing a kernel."""
    import hashlib
    src = ""
    for name in ("mla_device.h", "mla_kernels.hip", "mla_decode_so.hip", "mla_prefill.hip", "mla_prefill_q8.hip"):
        with open(os.path.join(ROOT, "mla_decode_attention_amd", "csrc", name)) as f:
            src += f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    src = "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())
    return hashlib.sha256(src.encode()).hexdigest()


def measured_traffic(config_name: str):
    """HBM bytes per attention-kernel launch from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the kernel
    source has changed since the counters were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "hbm_traffic.json")) as f:
            t = json.load(f)
        sha = kernel_source_digest()
    except OSError:
        return None
    if t.get("kernel_source_sha256") != sha or config_name not in t.get("configs", {}):
        return None
    return int(t["configs"][config_name]["bytes"])


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(w, seconds: float):
    """The oracle as it stands, on whole sequences in batch order (starting
    over after the last) until `seconds` pass."""
    import oracle
    e, f = (2, 0) if w.kv_dtype == "bf16" else (1, 4)
    done, kv, flops = 0, 0, 0
    t0 = time.perf_counter()
    while True:
        b = done % w.batch
        if w.varlen:
            oracle.mla_decode_varlen(w.q_bits, w.cu_q, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                                     w.kv_dtype, w.kv_scale, batch_indices=[b])
        else:
            oracle.mla_decode(w.q_bits, w.cache, w.block_table, w.seqlens, w.softmax_scale,
                              w.kv_dtype, w.kv_scale, batch_indices=[b])
        L = int(w.seqlens[b])
        s = int(w.q_lens[b])
        kv += L * (576 * e + f)
        flops += 2 * w.num_heads * 1088 * sum(max(0, min(L, L - s + i + 1)) for i in range(s))
        done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    tflops = flops / dt / 1e12
    mfma_bound = w.num_heads * int(max(w.q_lens)) > 16
    return {"value": round(tflops, 6) if mfma_bound else round(kv / dt / 1e9, 4),
            "unit": "TFLOP/s" if mfma_bound else "GB/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{done} whole-sequence evaluations in batch order ({done / w.batch:.2f} passes over "
                      f"the {w.batch} sequences), {dt:.1f} s wall, fp64 numpy",
            "tflops": round(tflops, 6), "kv_gbps": round(kv / dt / 1e9, 4), "seconds": round(dt, 2)}


def stats(ms):
    """median / min / mean of a list of times (ms), rounded."""
    if not ms:
        return None
    return {"median": round(statistics.median(ms), 5), "min": round(min(ms), 5),
            "mean": round(sum(ms) / len(ms), 5), "n": len(ms)}


def read_clocks(submit, done, sync, steps):
    """Graphics clock of each XCD and the memory clock (MHz), read in this
    process with the amdsmi library (no child program) while the GPU works
    through `steps` queued steps (`submit()` queues one, `done()` tells whether
    the queue has drained); None if the library or the metrics are not
    available. The firmware's readings lag a load change, so samples from the
    first 0.1 s are dropped; per XCD the median of the rest."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception:
        return None

    def mhz(v):
        vals = v if isinstance(v, (list, tuple)) else [v]
        return [int(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 10000]
    gfx, mem = [], []
    try:
        h = amdsmi.amdsmi_get_processor_handles()[0]
        for _ in range(steps):
            submit()
        t0 = time.time()
        while not done() and time.time() - t0 < 10:
            time.sleep(0.02)
            if time.time() - t0 < 0.1:
                continue
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            g = mhz(m.get("current_gfxclks", []))
            if g:
                gfx.append(g)
            mem += mhz(m.get("current_uclk", []))
        sync()
    except Exception:
        return None
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
    if not gfx:
        return None
    n = min(len(g) for g in gfx)
    return {"sclk_mhz": [int(statistics.median(g[i] for g in gfx)) for i in range(n)],
            "mclk_mhz": [int(statistics.median(mem))] if mem else [], "samples": len(gfx),
            "source": "amdsmi gpu metrics (current_gfxclks, current_uclk), sampled every 20 ms during ~1 s "
                      "of queued graph replays"}


def roofline_for(alg, fp8_mma):
    """(bound, T_roof seconds) of one step's algorithmic work."""
    t_hbm = alg["bytes"] / (PEAK_HBM_GBPS * 1e9)
    peak = PEAK_FP8_TFLOPS if fp8_mma else PEAK_BF16_TFLOPS
    t_mfma = alg["flops"] / (peak * 1e12)
    return ("hbm", t_hbm, peak) if t_hbm >= t_mfma else ("mfma", t_mfma, peak)


class DecodeRun:
    """One decode workload on the device: inputs, plan, step, timings."""

    def __init__(self, name, args, fp8_mma=False):
        import numpy as np
        import torch
        import mla_decode_attention_amd as mla
        from workloads import config, CONFIG_TEXT
        self.mla, self.torch = mla, torch
        self.name = name
        self.fp8_mma = fp8_mma
        self.wname = "fp8" if fp8_mma else name
        t_gen = time.perf_counter()
        self.w = w = config(self.wname, seed=0)
        self.alg = algorithmic(w)
        self.text = CONFIG_TEXT[self.wname] + (
            "; queries and P in E4M3 on fp8 MFMA (mla_decode_fwd_fp8mma)" if fp8_mma else "")
        print(f"[bench] {name}: generated in {time.perf_counter() - t_gen:.1f} s; "
              f"KV {self.alg['kv_bytes'] / 1e6:.1f} MB, {self.alg['flops'] / 1e9:.1f} GFLOP",
              file=sys.stderr, flush=True)
        dev = torch.device("cuda:0")
        self.q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        if w.kv_dtype == "bf16":
            kv0 = torch.from_numpy(w.cache.view(np.int16)).to(dev).view(torch.bfloat16)
            scale0 = None
        else:
            kv0 = torch.from_numpy(w.cache).to(dev)
            scale0 = torch.from_numpy(w.kv_scale).to(dev)
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sl = torch.from_numpy(w.seqlens).to(dev)
        pool_bytes = kv0.numel() * kv0.element_size()
        self.sets = args.sets or max(1, min(8, math.ceil(768e6 / max(pool_bytes, 1))))
        self.kvs = [kv0] + [kv0.clone() for _ in range(self.sets - 1)]
        self.scales = [scale0] + [None if scale0 is None else scale0.clone() for _ in range(self.sets - 1)]
        if w.varlen:
            self.cu_q = torch.from_numpy(w.cu_q).to(dev)
            T = int(w.cu_q[-1])
            self.out = torch.empty((T, w.num_heads, 512), dtype=torch.float32, device=dev)
            self.lse = torch.empty((T, w.num_heads), dtype=torch.float32, device=dev)
        else:
            self.out = torch.empty((w.batch, w.q_len, w.num_heads, 512), dtype=torch.float32, device=dev)
            self.lse = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device=dev)
        self.split = not (name in UNSPLIT and not args.num_units)
        self.units = 0
        self.plan = None
        if self.split:
            self.units = args.num_units or mla.default_num_units(w.batch, w.q_len, w.num_heads, varlen=w.varlen)
            self.plan = mla.get_split_metadata(self.sl, w.q_len, w.num_heads, num_units=self.units,
                                               min_tiles_per_unit=args.min_tiles, varlen=w.varlen)
        self.min_tiles = args.min_tiles
        self.latent = None
        if args.append_tokens:
            g = torch.Generator(device="cpu").manual_seed(1)
            lat32 = torch.randn((w.batch, args.append_tokens, 576), generator=g)
            self.latent = lat32.to(torch.bfloat16).to(dev)
        self.graphs = None

    def step(self, i):
        mla, w = self.mla, self.w
        k = i % self.sets
        if self.latent is not None:
            mla.append_kv(self.latent, self.bt, self.sl, self.kvs[k], self.scales[k])
        if self.split:
            mla.get_split_metadata(self.sl, w.q_len, w.num_heads, num_units=self.units,
                                   min_tiles_per_unit=self.min_tiles, metadata=self.plan.metadata,
                                   workspace=self.plan.workspace, varlen=w.varlen)
        if w.varlen:
            mla.decode_varlen(self.q, self.cu_q, w.q_len, self.kvs[k], self.bt, self.sl, w.softmax_scale,
                              kv_scale=self.scales[k], plan=self.plan, out=self.out, lse=self.lse)
        else:
            mla.decode(self.q, self.kvs[k], self.bt, self.sl, w.softmax_scale, kv_scale=self.scales[k],
                       plan=self.plan, out=self.out, lse=self.lse, fp8_mma=self.fp8_mma)

    def time_kernels(self, reps):
        """Each kernel of the step alone: events recorded by its dispatches."""
        mla, torch = self.mla, self.torch
        torch.cuda.synchronize()
        mla.profile_enable(True)
        for k in (mla.PROFILE_ATTENTION, mla.PROFILE_METADATA, mla.PROFILE_COMBINE):
            mla.profile_read_launches(k, capacity=0)
        for i in range(reps):
            self.step(i)
        torch.cuda.synchronize()
        mla.profile_enable(False)
        return {kind: mla.profile_read_launches(k, capacity=reps + 8)
                for kind, k in (("attention", mla.PROFILE_ATTENTION), ("metadata", mla.PROFILE_METADATA),
                                ("combine", mla.PROFILE_COMBINE))}

    def capture(self, eager):
        torch = self.torch
        if eager:
            return
        self.graphs = []
        for k in range(self.sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(k)
            self.graphs.append(g)

    def run_step(self, i):
        if self.graphs is None:
            self.step(i)
        else:
            self.graphs[i % self.sets].replay()

    def time_steps(self, steps, warmup):
        """K steps back to back, an event between consecutive steps: per-step
        times and the mean over the bracketed region."""
        torch = self.torch
        for i in range(warmup):
            self.run_step(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record()
        for i in range(steps):
            self.run_step(i)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return per, ev[0].elapsed_time(ev[steps]) / steps

    def entry(self, kern, per_step, mean_step, traffic_name):
        """The config's record for the JSON line."""
        w, alg = self.w, self.alg
        bound, t_roof, peak = roofline_for(alg, self.fp8_mma)
        st = stats(per_step)
        attn = stats(kern["attention"])
        step_med_s = st["median"] * 1e-3
        kv_gbps = alg["kv_bytes"] / step_med_s / 1e9
        tflops = alg["flops"] / step_med_s / 1e12
        traffic = measured_traffic(traffic_name)
        return {
            "name": self.name,
            "workload": self.text,
            "batch": w.batch, "heads": w.num_heads,
            "q_len": w.q_len if not w.varlen else "per-sequence, max %d" % w.q_len,
            "kv_dtype": w.kv_dtype, "tokens": alg["tokens"], "pages": alg["pages"],
            "path": "split (metadata + attention + merge)" if self.split else "unsplit (one attention launch)",
            "num_units": self.units if self.split else None,
            "pool_copies": self.sets,
            "algorithmic_bytes": alg["bytes"], "algorithmic_flops": alg["flops"], "kv_bytes": alg["kv_bytes"],
            "bound": bound, "t_roof_us": round(t_roof * 1e6, 2), "peak": peak,
            "step_ms": st, "step_ms_bracketed_mean": round(mean_step, 5),
            "kernel_ms": {"attention": attn, "metadata": stats(kern["metadata"]),
                          "combine": stats(kern["combine"])},
            "tflops": round(tflops, 2), "kv_gbps": round(kv_gbps, 1),
            "frac_step": round(t_roof / step_med_s, 4),
            "frac_kernel": round(t_roof / (attn["mean"] * 1e-3), 4),
            "frac_kernel_median": round(t_roof / (attn["median"] * 1e-3), 4),
            "traffic_bytes": traffic,
            "traffic_ratio": None if traffic is None else round(traffic / alg["bytes"], 3),
        }


def roofline_object(e, kernel_name):
    """The contract's roofline object for the dominant (attention) kernel:
    algorithmic work per launch over its mean dispatch-timed launch."""
    attn_s = e["kernel_ms"]["attention"]["mean"] * 1e-3
    if e["bound"] == "hbm":
        achieved, unit = e["algorithmic_bytes"] / attn_s / 1e9, "GB/s"
        peak = PEAK_HBM_GBPS
    else:
        achieved, unit = e["algorithmic_flops"] / attn_s / 1e12, "TFLOP/s"
        peak = e["peak"]
    return {"bound": e["bound"], "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": e["traffic_bytes"],
            "kernel": kernel_name, "kernel_ms": e["kernel_ms"]["attention"]["mean"],
            "kernel_ms_median": e["kernel_ms"]["attention"]["median"],
            "launches": e["kernel_ms"]["attention"]["n"],
            "frac_step": e["frac_step"],
            "algorithmic_bytes": e["algorithmic_bytes"], "algorithmic_flops": e["algorithmic_flops"],
            "t_roof_us": e["t_roof_us"]}


KERNEL_NAMES = {"tiny": "decode_kernel_pc", "share16": "decode_kernel_pc", "share16_fp8": "decode_kernel_pc8",
                "mtp": "decode_kernel_so<false>",
                "ragged": "decode_kernel_so<false>", "fp8": "decode_kernel_so<true>", "varlen": "decode_kernel_so<false>",
                "fp8mma": "decode_kernel_so8"}


def bench_decode(args):
    import torch
    torch.cuda.set_device(torch.device("cuda:0"))
    names = DECODE_CONFIGS if args.config == "all" else [args.config]
    headline = HEADLINE if args.config == "all" else args.config
    reps = max(args.reps, 50)
    entries, head = [], None
    clocks = None
    for name in names:
        run = DecodeRun(name, args, fp8_mma=(name == "fp8mma"))
        if args.calib_copy_mib:
            a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
            b = torch.empty_like(a)
            b.copy_(a)
            torch.cuda.synchronize()
            del a, b
        for i in range(args.warmup):
            run.step(i)
        kern = run.time_kernels(reps)
        run.capture(args.eager)
        per, mean = run.time_steps(args.steps if name == headline else max(args.steps, 50), args.warmup)
        e = run.entry(kern, per, mean, name)
        entries.append(e)
        print(f"[bench] {name}: step median {e['step_ms']['median'] * 1e3:.1f} us, attention kernel mean "
              f"{e['kernel_ms']['attention']['mean'] * 1e3:.1f} us, frac_step {e['frac_step']:.3f}, "
              f"frac_kernel {e['frac_kernel']:.3f}", file=sys.stderr, flush=True)
        if name == headline:
            head = (run, e, mean)
            if not args.no_clocks:
                i_box = [0]

                def submit():
                    run.run_step(i_box[0])
                    i_box[0] += 1
                n_busy = max(50, int(1.0 / max(e["step_ms"]["median"] * 1e-3, 1e-5)))
                clocks = read_clocks(submit, lambda: torch.cuda.current_stream().query(),
                                     torch.cuda.synchronize, n_busy)
        if name != headline:
            del run
            torch.cuda.empty_cache()

    run, e, mean = head
    alg = run.alg
    step_s = mean * 1e-3
    value = alg["flops"] / step_s / 1e12 if e["bound"] == "mfma" else alg["kv_bytes"] / step_s / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2 if e["bound"] == "mfma" else 1),
        "unit": "TFLOP/s" if e["bound"] == "mfma" else "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(mean, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if run.fp8_mma else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{e['name']}: {e['workload']}", "batch": e["batch"], "heads": e["heads"],
                   "q_len": e["q_len"], "kv_dtype": e["kv_dtype"], "tokens": e["tokens"], "pages": e["pages"],
                   "path": e["path"], "num_units": e["num_units"], "pool_copies": e["pool_copies"], "seed": 0,
                   "append_tokens": args.append_tokens,
                   "step_launch": "direct launches" if args.eager else "HIP graph replay"},
        "tflops": round(alg["flops"] / step_s / 1e12, 2),
        "kv_gbps": round(alg["kv_bytes"] / step_s / 1e9, 1),
        "roofline": roofline_object(e, KERNEL_NAMES.get(e["name"], "decode_kernel")),
        "clocks": clocks,
        "configs": entries,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(run.w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def prefill_algorithmic(w):
    """Flops (QK 192 + PV 128 multiply-adds per visible (row, key) pair per
    head) and bytes (q, k_nope, k_rope, v once; out and lse) of one call."""
    vis = 0
    for N, L in zip(w.q_lens, w.k_lens):
        N, L = int(N), int(L)
        vis += N * (L - N) + N * (N + 1) // 2
    H = w.num_heads
    flops = 2 * H * (192 + 128) * vis
    Tq, Tk = int(w.cu_q[-1]), int(w.cu_k[-1])
    nbytes = Tq * H * 192 * 2 + Tk * (H * 128 * 2 + 64 * 2 + H * 128 * 2) + Tq * H * (128 + 1) * 4
    return dict(flops=flops, bytes=nbytes, visible_pairs=vis)


def prefill_cpu_baseline(w, seconds: float):
    """The prefill oracle on a bounded sample: the first rows of sequence 0,
    as an extend (a query at position p sees keys 0..p), doubling the row
    count until `seconds` pass."""
    import numpy as np
    import oracle
    N0, L0 = int(w.q_lens[0]), int(w.k_lens[0])
    n, flops, dt = 16, 0, 0.0
    t0 = time.perf_counter()
    while True:
        n = min(n, N0)
        p_end = L0 - N0 + n            # keys 0 .. p_end - 1 cover the first n queries
        t1 = time.perf_counter()
        oracle.mla_prefill(w.q_bits[:n], w.k_nope_bits[:p_end], w.k_rope_bits[:p_end], w.v_bits[:p_end],
                           np.array([0, n], np.int32), np.array([0, p_end], np.int32), w.softmax_scale)
        dt_i = time.perf_counter() - t1
        flops = 2 * w.num_heads * 320 * (n * (p_end - n) + n * (n + 1) // 2)
        dt = dt_i
        if n == N0 or time.perf_counter() - t0 >= seconds or dt_i * 4 > seconds:
            break
        n *= 2
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"first {n} of {N0} queries of sequence 0 (an extend over its first {p_end} keys), "
                      f"{dt:.1f} s wall for that call, fp64 numpy", "seconds": round(dt, 2)}


def bench_prefill(args):
    import numpy as np
    import torch
    import mla_decode_attention_amd as mla
    from workloads import prefill_config, PREFILL_TEXT

    quant = args.config.endswith("_q8")
    wname = args.config[:-3] if quant else args.config
    w = prefill_config(wname, seed=0)
    alg = prefill_algorithmic(w)
    print(f"[bench] {args.config}: {alg['flops'] / 1e12:.2f} TFLOP per call", file=sys.stderr, flush=True)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dv = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)
    q, kn, kr, v = dv(w.q_bits), dv(w.k_nope_bits), dv(w.k_rope_bits), dv(w.v_bits)
    cq = torch.from_numpy(w.cu_q).to(dev)
    ck = torch.from_numpy(w.cu_k).to(dev)
    Tq, H = q.shape[0], w.num_heads
    out = torch.empty((Tq, H, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((Tq, H), dtype=torch.float32, device=dev)
    max_q = int(w.q_lens.max())
    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    qkv = mla.prefill_quantize_kv(kn, kr, v, ck) if quant else None

    def step():
        if quant:   # the dynamic quantisation of K and V is part of every call
            mla.prefill_quant(q, kn, kr, v, cq, ck, max_q, w.softmax_scale, out=out, lse=lse, qkv=qkv)
        else:
            mla.prefill(q, kn, kr, v, cq, ck, max_q, w.softmax_scale, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    reps = max(args.reps, 50)
    mla.profile_enable(True)
    mla.profile_read_launches(mla.PROFILE_ATTENTION, capacity=0)
    mla.profile_read_launches(mla.PROFILE_QUANTIZE, capacity=0)
    for _ in range(reps):
        step()
    torch.cuda.synchronize()
    mla.profile_enable(False)
    kern = stats(mla.profile_read_launches(mla.PROFILE_ATTENTION, capacity=reps + 8))
    qkern = stats(mla.profile_read_launches(mla.PROFILE_QUANTIZE, capacity=reps + 8)) if quant else None
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = stats([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    step_ms = ev[0].elapsed_time(ev[args.steps]) / args.steps
    tflops = alg["flops"] / (step_ms * 1e-3) / 1e12
    achieved = alg["flops"] / (kern["mean"] * 1e-3) / 1e12
    # the quantised path contracts INT8 x INT8 (QK) and FP8 x FP8 (PV): both
    # dense peaks are 5.0 POP/s / PFLOP/s on MI355X
    peak = PEAK_FP8_TFLOPS if quant else PEAK_BF16_TFLOPS
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(args.config),
            "kernel": "prefill_q8_kernel" if quant else "prefill_kernel", "kernel_ms": kern["mean"],
            "kernel_ms_median": kern["median"], "launches": kern["n"],
            "frac_step": round(alg["flops"] / (peak * 1e12) / (per["median"] * 1e-3), 4),
            "algorithmic_bytes": alg["bytes"], "algorithmic_flops": alg["flops"],
            "t_roof_us": round(alg["flops"] / (peak * 1e12) * 1e6, 2)}
    if quant:
        Tk = int(w.cu_k[-1])
        slots = Tk // 64 + w.batch
        qbytes = Tk * H * (128 + 128) * 2 + Tk * 64 * 2 + slots * H * (12288 + 8192 + 256 + 4)
        roof["quantizer"] = {"kernel": "quant_kv_kernel", "ms_mean": qkern["mean"], "ms_median": qkern["median"],
                             "launches": qkern["n"], "algorithmic_bytes": qbytes,
                             "GB/s": round(qbytes / (qkern["mean"] * 1e-3) / 1e9, 1)}
    line = {
        "metric": METRIC,
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8" if quant else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {PREFILL_TEXT[wname]}"
                               + ("; INT8 Q.K^T, FP8 P.V, K/V quantised in every call" if quant else ""),
                   "batch": w.batch, "heads": H,
                   "query_tokens": Tq, "key_tokens": int(w.cu_k[-1]), "visible_pairs": alg["visible_pairs"],
                   "seed": 0},
        "step_ms": per,
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--reps", type=int, default=100, help="kernel launches timed per workload (at least 50)")
    ap.add_argument("--config", default="all",
                    choices=["all", "tiny", "share16", "share16_fp8", "mtp", "ragged", "fp8", "varlen", "fp8mma",
                             "prefill", "extend", "prefill_q8", "extend_q8"],
                    help="all = the six decode workloads, headline fp8; fp8mma = the fp8 workload on "
                         "mla_decode_fwd_fp8mma (queries and P in E4M3, fp8 matrix cores; an approximation of "
                         "the default path); prefill / extend = the second workload (mla_prefill_fwd); "
                         "prefill_q8 / extend_q8 = the same on the quantised path (mla_prefill_quantize_kv + "
                         "mla_prefill_quant_fwd)")
    ap.add_argument("--sets", type=int, default=0, help="pool copies to rotate (0 = auto)")
    ap.add_argument("--num-units", type=int, default=0, help="split work units (0 = library default)")
    ap.add_argument("--min-tiles", type=int, default=0,
                    help="minimum tiles per split unit (0 = library default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clocks", action="store_true", help="do not read the clocks (amdsmi library)")
    ap.add_argument("--append-tokens", type=int, default=0,
                    help="also run the cache append (mla_append_kv) of this many new tokens per sequence "
                         "in every step, before the decode (their rows are the last positions of each "
                         "sequence)")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as direct launches (default: replay of a captured HIP graph of the "
                         "step, as a serving loop runs a decode step)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the library "
              "has no multi-GPU path; the per-GPU kernel is the whole computation.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        ap.error("--steps must be >= 1")

    if args.config in ("prefill", "extend", "prefill_q8", "extend_q8"):
        return bench_prefill(args)
    return bench_decode(args)


if __name__ == "__main__":
    main()
