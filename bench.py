#!/usr/bin/env python3
"""Throughput of MLA decode over a paged latent KV cache on one MI355X.

One step = one pass of the whole path over one batch: split schedule
(mla_get_split_metadata), then mla_decode_fwd (attention kernel + LSE merge of
split sequences). Inputs are seeded synthetic data already resident in HBM.
To keep the 256 MB Infinity Cache from serving repeat reads, steps rotate over
several copies of the page pool (each step reads a copy it did not read in the
previous few steps).

Prints ONE JSON line (default workload: batch 64, 16 heads, q_len 1, seqlens
U[1024,4096], bf16 cache) with:
  value      effective KV GB/s of the whole step (KV bytes / step time), the
             step replayed from a captured HIP graph (--eager: direct launches)
  roofline   the attention kernel alone: algorithmic bytes (HBM-bound shapes)
             or flops (MFMA-bound shapes) per launch / its mean launch time,
             timed with HIP events on its own stream, vs the MI355X peak
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA decode TFLOP/s + effective KV GB/s, % of roofline, per batch/heads/q_len"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0        # MI355X dense fp8 MFMA (context for the fp8 cache)


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
    import re
    src = ""
    for name in ("mla_kernels.hip", "mla_prefill.hip"):
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


def cpu_baseline(w, seconds: float):
    """The oracle as it stands, on whole sequences in batch order (starting
    over after the last) until `seconds` pass."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} whole-sequence evaluations in batch order ({done / w.batch:.2f} passes over "
                      f"the {w.batch} sequences), {dt:.1f} s wall, fp64 numpy", "tflops": flops / dt / 1e12,
            "seconds": round(dt, 2)}


def prefill_algorithmic(w):
    """Flops (QK 192 + PV 128 multiply-adds per visible (row, key) pair per
    head) and bytes (q, k_nope, k_rope, v once; out and lse) of one call."""
    import numpy as np
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
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {N0} queries of sequence 0 (an extend over its first {p_end} keys), "
                      f"{dt:.1f} s wall for that call, fp64 numpy", "seconds": round(dt, 2)}


def bench_prefill(args):
    import numpy as np
    import torch
    import mla_decode_attention_amd as mla
    from workloads import prefill_config, PREFILL_TEXT

    w = prefill_config(args.config, seed=0)
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

    def step():
        mla.prefill(q, kn, kr, v, cq, ck, max_q, w.softmax_scale, out=out, lse=lse)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    mla.profile_enable(True)
    mla.profile_read()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    mla.profile_enable(False)
    step_ms = t0.elapsed_time(t1) / args.steps
    k_total, launches = mla.profile_read()
    k_ms = k_total / max(launches, 1)
    tflops = alg["flops"] / (step_ms * 1e-3) / 1e12
    achieved = alg["flops"] / (k_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(args.config),
            "kernel": "prefill_kernel", "kernel_ms": round(k_ms, 5), "launches": launches,
            "algorithmic_bytes": alg["bytes"], "algorithmic_flops": alg["flops"],
            "t_roof_us": round(alg["flops"] / (PEAK_BF16_TFLOPS * 1e12) * 1e6, 2)}
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {PREFILL_TEXT[args.config]}", "batch": w.batch, "heads": H,
                   "query_tokens": Tq, "key_tokens": int(w.cu_k[-1]), "visible_pairs": alg["visible_pairs"],
                   "seed": 0},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = prefill_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="share16",
                    choices=["tiny", "share16", "mtp", "ragged", "fp8", "varlen", "fp8mma", "prefill", "extend"],
                    help="workload; fp8mma = the fp8 workload on mla_decode_fwd_fp8mma (queries and P in "
                         "E4M3, fp8 matrix cores; an approximation of the default path); prefill / extend = "
                         "the second workload (mla_prefill_fwd, un-absorbed MLA, value in TFLOP/s)")
    ap.add_argument("--sets", type=int, default=0, help="pool copies to rotate (0 = auto)")
    ap.add_argument("--num-units", type=int, default=0, help="split work units (0 = library default)")
    ap.add_argument("--min-tiles", type=int, default=0,
                    help="minimum tiles per split unit (0 = library default)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): this build "
              "has no multi-GPU path; the per-GPU kernel is the whole computation.", file=sys.stderr)
        sys.exit(2)

    if args.config in ("prefill", "extend"):
        return bench_prefill(args)

    import numpy as np
    import torch
    import mla_decode_attention_amd as mla
    from workloads import config, CONFIG_TEXT

    fp8_mma = args.config == "fp8mma"
    wname = "fp8" if fp8_mma else args.config
    t_gen = time.perf_counter()
    w = config(wname, seed=0)
    alg = algorithmic(w)
    print(f"[bench] {args.config}: generated in {time.perf_counter() - t_gen:.1f} s; "
          f"KV {alg['kv_bytes'] / 1e6:.1f} MB, {alg['flops'] / 1e9:.1f} GFLOP", file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    if w.kv_dtype == "bf16":
        kv0 = torch.from_numpy(w.cache.view(np.int16)).to(dev).view(torch.bfloat16)
        scale0 = None
    else:
        kv0 = torch.from_numpy(w.cache).to(dev)
        scale0 = torch.from_numpy(w.kv_scale).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seqlens).to(dev)
    pool_bytes = kv0.numel() * kv0.element_size()
    sets = args.sets or max(1, min(8, math.ceil(768e6 / max(pool_bytes, 1))))
    kvs = [kv0] + [kv0.clone() for _ in range(sets - 1)]
    scales = [scale0] + [None if scale0 is None else scale0.clone() for _ in range(sets - 1)]
    if w.varlen:
        cu_q = torch.from_numpy(w.cu_q).to(dev)
        T = int(w.cu_q[-1])
        out = torch.empty((T, w.num_heads, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((T, w.num_heads), dtype=torch.float32, device=dev)
    else:
        out = torch.empty((w.batch, w.q_len, w.num_heads, 512), dtype=torch.float32, device=dev)
        lse = torch.empty((w.batch, w.q_len, w.num_heads), dtype=torch.float32, device=dev)
    units = args.num_units or mla.default_num_units(w.batch, w.q_len, w.num_heads, varlen=w.varlen)
    plan = mla.get_split_metadata(sl, w.q_len, w.num_heads, num_units=units, min_tiles_per_unit=args.min_tiles)

    if args.calib_copy_mib:
        a = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    latent = None
    if args.append_tokens:
        g = torch.Generator(device="cpu").manual_seed(1)
        lat32 = torch.randn((w.batch, args.append_tokens, 576), generator=g)
        latent = lat32.to(torch.bfloat16).to(dev)

    def step(i):
        if latent is not None:
            k = i % sets
            mla.append_kv(latent, bt, sl, kvs[k], scales[k])
        mla.get_split_metadata(sl, w.q_len, w.num_heads, num_units=units, metadata=plan.metadata,
                               workspace=plan.workspace)
        k = i % sets
        if w.varlen:
            mla.decode_varlen(q, cu_q, w.q_len, kvs[k], bt, sl, w.softmax_scale, kv_scale=scales[k], plan=plan,
                              out=out, lse=lse)
        else:
            mla.decode(q, kvs[k], bt, sl, w.softmax_scale, kv_scale=scales[k], plan=plan, out=out, lse=lse,
                       fp8_mma=fp8_mma)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # attention kernel alone: direct launches, each recording HIP events with its own dispatch
    mla.profile_enable(True)
    mla.profile_read()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    mla.profile_enable(False)
    step_ms = t0.elapsed_time(t1) / args.steps
    main_ms_total, launches = mla.profile_read()
    main_ms = main_ms_total / max(launches, 1)

    # whole step: one captured graph per pool copy (split schedule, attention,
    # merge), replayed in turn
    if not args.eager:
        graphs = []
        for k in range(sets):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % sets].replay()
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            graphs[i % sets].replay()
        t1.record()
        torch.cuda.synchronize()
        step_ms = t0.elapsed_time(t1) / args.steps

    step_s = step_ms * 1e-3
    main_s = main_ms * 1e-3
    kv_gbps = alg["kv_bytes"] / step_s / 1e9
    tflops = alg["flops"] / step_s / 1e12
    t_hbm = alg["bytes"] / (PEAK_HBM_GBPS * 1e9)
    peak_mfma = PEAK_FP8_TFLOPS if fp8_mma else PEAK_BF16_TFLOPS   # the contraction dtype's peak
    t_mfma = alg["flops"] / (peak_mfma * 1e12)
    if t_hbm >= t_mfma:
        achieved = alg["bytes"] / main_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None}
    else:
        achieved = alg["flops"] / main_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_mfma,
                "unit": "TFLOP/s", "frac": round(achieved / peak_mfma, 4), "traffic": None}
    roof["traffic"] = measured_traffic(args.config)
    roof.update({"kernel": "decode_kernel", "kernel_ms": round(main_ms, 5), "launches": launches,
                 "algorithmic_bytes": alg["bytes"], "algorithmic_flops": alg["flops"],
                 "t_roof_us": round(max(t_hbm, t_mfma) * 1e6, 2)})

    line = {
        "metric": METRIC,
        "value": round(kv_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8" if fp8_mma else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {CONFIG_TEXT[wname]}" + (
                       "; queries and P in E4M3 on fp8 MFMA (mla_decode_fwd_fp8mma)" if fp8_mma else ""),
                   "batch": w.batch,
                   "heads": w.num_heads, "q_len": w.q_len if not w.varlen else "per-sequence, max %d" % w.q_len,
                   "query_tokens": int(sum(w.q_lens)), "kv_dtype": w.kv_dtype,
                   "tokens": alg["tokens"], "pages": alg["pages"], "num_units": units,
                   "min_tiles_per_unit": args.min_tiles or "library default",
                   "pool_copies": sets, "seed": 0, "append_tokens": args.append_tokens,
                   "step_launch": "direct launches" if args.eager else "HIP graph replay"},
        "tflops": round(tflops, 2),
        "kv_gbps": round(kv_gbps, 1),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
