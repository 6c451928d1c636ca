#!/usr/bin/env python3
"""Benchmark of the hybrid-batch paged-attention step on one MI355X.

A step is one iteration of the whole per-layer path, as a serving loop runs
it: the host batch builder (stall-free: decodes, then chunks, then
admissions), the metadata pack, one launch that copies the packed metadata
from pinned host memory and appends the new K/V to the paged cache, the
hybrid attention, and the commit of the batch.  Every step starts from a
copy of the same scheduler state, so every step runs the same batch; the
host half of later steps overlaps the GPU half of earlier ones.  q / k / v
rows and the paged cache are resident in HBM before the timed region.

The default workload is the largest single-GPU configuration: the
LLaMA2-70B-shaped layer (64 q heads / 8 kv heads / d 128) at token budget
1536 -- 256 running decodes with contexts uniform in 512..8191 plus two
prefill chunks (one prompt mid-prefill, one admitted).  `--workload` picks
another; `--suite` times every workload and the Falcon-180B budget sweep.

Prints ONE JSON line.  `value` is tokens/s of the layer (T tokens per step
over the wall time of K steps, bracketed by device synchronisations).
Beside it: the roofline of the dominant kernel (the attention, timed with HIP
events on its own stream on every 4th timed step), the host costs of the
builder / upload / commit, and the CPU oracle timed on this machine's host
cores as a baseline.
"""
from __future__ import annotations

import os

# BLAS threads of the CPU oracle leg: set before NumPy is first imported,
# to the CPUs this process may run on (an explicit setting is kept).
_AFFINITY = len(os.sched_getaffinity(0))
for _var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_var, str(_AFFINITY))

import argparse  # noqa: E402
import hashlib  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 matrix cores
WORKLOADS = {"tiny": 1, "mistral7b": 2, "yi34b": 3, "llama2-70b": 4, "falcon180b-tp4": 5}
DEFAULT_WORKLOAD = "llama2-70b"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic.json")
# The attention path's device code and the host plan that orders its work:
# a change to either can change what the counters read.
ATTN_SOURCES = [os.path.join(ROOT, "chunked_prefill_decode_amd", "csrc", f)
                for f in ("kernels.hip", "plan.cpp", "common.h")]


def algorithmic_work(inst, batch, window: int = 0):
    """Bytes the attention step must move and flops it must do (per launch).

    KV bytes: every decode reads its ctx+1 keys once per kv head (grouped
    heads share them); every chunk reads its o earlier keys plus its own C
    (the re-read of the earlier chunks); plus reading Q and writing O.
    With a sliding window w only keys some row sees count: from
    max(0, ctx - w + 1) (the first row's window) to ctx + n.
    Flops: 4*Hq*d per (row, visible key) -- QK^T and PV at 2 flops/MAC.
    The append kernel moves 2*T*kvb (read the new rows, write the cache)."""
    Hq, Hkv, d = inst.num_q_heads, inst.num_kv_heads, inst.head_dim
    kvb = 2 * Hkv * d * 2
    v = batch.view()
    cu, ctx = v["cu_seqlens_q"], v["context_lens"]
    kv_bytes, flops = 0, 0
    for s in range(len(ctx)):
        n, c = int(cu[s + 1] - cu[s]), int(ctx[s])
        lo = max(0, c - window + 1) if window else 0
        kv_bytes += (c + n - lo) * kvb
        # the row at position p sees p+1 keys, or min(p+1, w) with a window
        flops += 4 * Hq * d * sum(min(p + 1, window) if window else p + 1 for p in range(c, c + n))
    T = cu[-1]
    qo_bytes = 2 * T * Hq * d * 2
    return dict(attn_bytes=kv_bytes + qo_bytes, attn_flops=flops, append_bytes=2 * T * kvb,
                kv_bytes=kv_bytes, qo_bytes=qo_bytes)


def kernel_source_digest() -> str:
    """sha256[:16] over the attention sources, in order."""
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_key(inst, window: int) -> str:
    return inst.name if not window else f"{inst.name} window={window}"


def load_traffic(workload: str):
    """HBM traffic per attention launch from committed rocprofv3 counter runs,
    only if they were taken on the current kernel source."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    r = rec.get(workload)
    if not r or r.get("kernel_sha") != kernel_source_digest():
        return None
    return r.get("bytes_per_launch")


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return int(max([p.get("num_threads", 1) for p in threadpool_info()] or [1]))


def cpu_baseline(inst, step, seconds: float, window: int = 0):
    """The fp64 oracle on the same workload, on this machine's host cores.

    Sample: the whole batch the oracle's own builder makes for the instance
    (every decode and chunk row), repeated until `seconds` have passed (at
    least once); the GPU's output rows of the same batch are compared with
    the oracle's on that sample.  Also: the tiny workload on one BLAS thread,
    and the oracle's batch builder (Python) against the library's (C++) per
    iteration of the 40-iteration LLaMA2-70B-shaped schedule."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import workloads as W
    from oracle import attention as OA
    from oracle import inputs as OI

    t_in = time.perf_counter()
    seqs, q, kv, rows = OI.step_inputs(inst, step.hist, step.q_gen, step.k_new_gen, step.v_new_gen,
                                       step.free_pages)
    kv = [kv[i] for i in range(len(kv))]           # gathered (float32) before the timed region
    prep_s = time.perf_counter() - t_in
    reps, t0 = 0, time.perf_counter()
    while True:
        want = OA.attend(seqs, q, kv, inst.softmax_scale, window)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    got = step.out.float().cpu().numpy().astype(np.float64)[rows]
    err = np.abs(got - want)
    out = {"value": round(len(rows) * reps / el, 1), "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
           "sample": f"whole {inst.name} batch (T={len(rows)}: {step.D} decodes + {step.S - step.D} chunk(s)) as "
                     f"the oracle builds it, fp64 NumPy attention, {reps} repetition(s) in {el:.1f} s "
                     f"(input gathering {prep_s:.1f} s, not timed); host has {os.cpu_count()} logical CPUs, "
                     f"{_AFFINITY} in affinity, OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS')}",
           "gpu_vs_oracle": {"rows": len(rows), "max_abs": float(err.max()), "mean_abs": float(err.mean()),
                             "decode_rows_max_abs": float(err[:step.D].max()) if step.D else None,
                             "chunk_rows_max_abs": float(err[step.D:].max()) if len(rows) > step.D else None}}

    # the tiny workload on one thread
    from chunked_prefill_decode_amd.runner import GpuStep
    tiny = W.make_config(1)
    ts = GpuStep(tiny, gen_device="cpu")
    tseqs, tq, tkv, trows = OI.step_inputs(tiny, ts.hist, ts.q_gen, ts.k_new_gen, ts.v_new_gen)
    tkv = [tkv[i] for i in range(len(tkv))]
    with threadpool_limits(1):
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 1.0:
            OA.attend(tseqs, tq, tkv, tiny.softmax_scale)
            n += 1
        el1 = time.perf_counter() - t0
    out["single_thread_tiny"] = {"value": round(len(trows) * n / el1, 1), "unit": "tokens/s", "cores": 1,
                                 "sample": f"tiny batch (T={len(trows)}), {n} repetitions in {el1:.2f} s"}
    out["build_batch_us"] = builder_timing()
    return out


def builder_timing(iters: int = 40):
    """Host batch builder per iteration of the 40-iteration LLaMA2-70B-shaped
    schedule (Poisson arrivals, seed 2004): the oracle's Python builder
    against the library's, each with its commit, on mirrored states."""
    import workloads as W
    from chunked_prefill_decode_amd.runner import load_scheduler
    from oracle import inputs as OI
    inst = W.make_config(4)
    arrivals = W.poisson_arrivals(iters, 5000)
    ns, os_ = load_scheduler(inst), OI.load_scheduler(inst)
    cap = len(inst.injected) + len(inst.waiting) + sum(len(a) for a in arrivals) + 1
    from chunked_prefill_decode_amd import native as N
    hb = N.HostBatch(cap, inst.token_budget, inst.max_blocks_per_seq)
    t_n = t_o = c_n = c_o = 0.0
    for it in range(iters):
        for r in arrivals[it]:
            ns.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
            os_.add_request(r.req_id, r.prompt_len, r.max_new_tokens)
        t0 = time.perf_counter()
        N.sa_build_batch(ns.h, hb)
        t1 = time.perf_counter()
        ob = os_.build_batch()
        t2 = time.perf_counter()
        ns.commit(hb)
        t3 = time.perf_counter()
        os_.commit(ob)
        t4 = time.perf_counter()
        t_n += t1 - t0
        t_o += t2 - t1
        c_n += t3 - t2
        c_o += t4 - t3
    k = 1e6 / iters
    return {"iterations": iters, "native_build": round(t_n * k, 2), "oracle_build": round(t_o * k, 2),
            "native_commit": round(c_n * k, 2), "oracle_commit": round(c_o * k, 2)}


def measure(inst, args, window: int = 0, with_cold: bool = True) -> dict:
    """Times K steps of the whole path on one workload; returns the bench
    fields (without the CPU baseline)."""
    import torch
    from chunked_prefill_decode_amd.runner import GpuStep, StepLoop
    step = GpuStep(inst, gen_device="cuda", window=window)
    stream = torch.cuda.current_stream()
    work = algorithmic_work(inst, step.batch, window)
    detail = min(args.steps, 20)                  # untimed steps that time the upload + append launch
    loop = StepLoop(step, args.warmup + args.steps + detail, stream)

    for i in range(args.warmup):
        loop.run(i)
    torch.cuda.synchronize()
    # timed steps: on every SAMPLE-th one the attention launch sits between an
    # event that ends the upload + append and one after it; the other steps
    # record no event (each record sits between kernels on the GPU)
    marks = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        k = args.warmup + i                       # every step whose index is a multiple of SAMPLE (at least one)
        marks.append(loop.run(k, timing=k % StepLoop.SAMPLE == 0 or (i == 0 and args.steps < StepLoop.SAMPLE)))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    attn_all = sorted(a.elapsed_time(b) for _, a, b in marks if a is not None)
    befores = [torch.cuda.Event(enable_timing=True) for _ in range(detail)]
    ups = [loop.run(args.warmup + args.steps + i, before=befores[i])[1] for i in range(detail)]
    torch.cuda.synchronize()
    append_ms = sum(a.elapsed_time(b) for a, b in zip(befores, ups)) / max(1, detail)
    attn_ms = sum(attn_all) / len(attn_all)
    pct = lambda q: attn_all[min(len(attn_all) - 1, int(q * len(attn_all)))] * 1e3

    # cold launches: read a 1 GiB buffer first (fills L2 and the 256 MB
    # Infinity Cache with clean lines of it), outside the events
    cold_us = None
    if with_cold and args.cold_reps > 0:
        scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        sink = torch.empty((), dtype=torch.float32, device="cuda")
        ev_cold = []
        for _ in range(args.cold_reps):
            torch.amax(scratch, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step.attend()
            e1.record(stream)
            ev_cold.append((e0, e1))
        torch.cuda.synchronize()
        cold = sorted(a.elapsed_time(b) * 1e3 for a, b in ev_cold)
        cold_us = {"median": round(cold[len(cold) // 2], 2), "p10": round(cold[len(cold) // 10], 2),
                   "p90": round(cold[min(len(cold) - 1, (9 * len(cold)) // 10)], 2)}
        del scratch, sink

    # host rows of the path, timed on their own
    from chunked_prefill_decode_amd import native as N
    reps = 200
    t = time.perf_counter()
    for _ in range(reps):
        N.sa_build_batch(step.sched.h, step.batch)
    build_us = (time.perf_counter() - t) * 1e6 / reps
    t = time.perf_counter()
    for _ in range(reps):
        N.sa_batch_pack(step.batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages,
                        step.staging.numpy(), step.meta.data_ptr(), window)
    pack_us = (time.perf_counter() - t) * 1e6 / reps
    t = time.perf_counter()
    for _ in range(reps):
        N.sa_batch_upload(step.batch, inst.num_q_heads, inst.num_kv_heads, inst.head_dim, inst.num_pages,
                          step.staging, step.meta, window=window)
        stream.synchronize()
    upload_us = (time.perf_counter() - t) * 1e6 / reps
    clones = [step.sched.clone() for _ in range(reps)]
    batches = [c.build_batch(cap_seqs=step.cap_seqs) for c in clones]
    t = time.perf_counter()
    for c, b in zip(clones, batches):
        c.commit(b)
    commit_us = (time.perf_counter() - t) * 1e6 / reps
    del clones, batches

    gbs = work["attn_bytes"] / (attn_ms * 1e-3) / 1e9
    tfs = work["attn_flops"] / (attn_ms * 1e-3) / 1e12
    t_hbm = work["attn_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = work["attn_flops"] / (MFMA_BF16_PEAK_TFS * 1e12)
    hbm_bound = t_hbm >= t_mfma
    roofline = {
        "kernel": "sa_hybrid_attn (attn_kernel + merge_kernel)",
        "bound": "hbm" if hbm_bound else "mfma",
        "achieved": round(gbs if hbm_bound else tfs, 1),
        "peak": HBM_PEAK_GBS if hbm_bound else MFMA_BF16_PEAK_TFS,
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "frac": round((gbs / HBM_PEAK_GBS) if hbm_bound else (tfs / MFMA_BF16_PEAK_TFS), 4),
        "traffic": load_traffic(traffic_key(inst, window)),
        "algorithmic_bytes": work["attn_bytes"],
        "algorithmic_flops": work["attn_flops"],
        "avg_launch_us": round(attn_ms * 1e3, 2),
        "other_fraction": round((tfs / MFMA_BF16_PEAK_TFS) if hbm_bound else (gbs / HBM_PEAK_GBS), 4),
    }
    return {
        "step": step, "ms_per_step": ms_per_step, "tokens_per_s": step.T / (ms_per_step * 1e-3),
        "roofline": roofline, "work": work,
        "kernels_us": {"upload_append": round(append_ms * 1e3, 2), "hybrid_attn": round(attn_ms * 1e3, 2),
                       "hybrid_attn_median": round(pct(0.5), 2), "hybrid_attn_p10": round(pct(0.1), 2),
                       "hybrid_attn_p90": round(pct(0.9), 2)},
        "hybrid_attn_cold_us": cold_us,
        "cold_frac": (None if cold_us is None else round(
            (work["attn_bytes"] / (cold_us["median"] * 1e-6) / 1e9 / HBM_PEAK_GBS) if hbm_bound else
            (work["attn_flops"] / (cold_us["median"] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFS), 4)),
        "host_us": {"build_batch": round(build_us, 2), "pack": round(pack_us, 2),
                    "upload_pack_and_copy_synchronous": round(upload_us, 2), "commit": round(commit_us, 2)},
        "attn_tflops": round(tfs, 2), "attn_gbs": round(gbs, 1),
        "upload_bytes": int(step.staging.numel()),
    }


def workload_config(inst, step, window: int) -> dict:
    return {"workload": f"{inst.name} layer: Hq={inst.num_q_heads} Hkv={inst.num_kv_heads} "
                        f"d={inst.head_dim}, B={inst.token_budget}, {step.D} decodes + "
                        f"{step.S - step.D} prefill chunk(s), 16-token pages"
                        + (f", sliding window {window}" if window else ""),
            "token_budget": inst.token_budget, "tokens_per_step": step.T, "decodes": step.D,
            "prefill_chunks": step.S - step.D, "seed": inst.seed, "sliding_window": window,
            "parallelism": "single GPU"}


def suite(args) -> dict:
    """Every workload and the Falcon-180B budget sweep, one line each."""
    import torch
    import workloads as W
    runs = [(w, None) for w in ("mistral7b", "yi34b", "llama2-70b", "falcon180b-tp4")]
    runs += [("falcon180b-tp4", B) for B in W.SWEEP_BUDGETS + W.SWEEP_DIAGNOSTIC if B != 2048]
    rows = []
    for name, B in runs:
        inst = W.make_config(WORKLOADS[name], B)
        m = measure(inst, args, 0, with_cold=True)
        r = m["roofline"]
        row = {"workload": inst.name, "T": m["step"].T, "decodes": m["step"].D, "ms_per_step": round(m["ms_per_step"], 4),
               "tokens_per_s": round(m["tokens_per_s"], 1), "attn_us": r["avg_launch_us"],
               "attn_cold_us": m["hybrid_attn_cold_us"]["median"] if m["hybrid_attn_cold_us"] else None,
               "upload_append_us": m["kernels_us"]["upload_append"], "bound": r["bound"], "frac": r["frac"],
               "hbm_frac": round(m["attn_gbs"] / HBM_PEAK_GBS, 4),
               "mfma_frac": round(m["attn_tflops"] / MFMA_BF16_PEAK_TFS, 4),
               "algorithmic_bytes": r["algorithmic_bytes"], "algorithmic_flops": r["algorithmic_flops"],
               "host_us": m["host_us"]}
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del m
        torch.cuda.empty_cache()
    return {"suite": "hybrid_attn per workload", "steps": args.steps, "warmup": args.warmup, "results": rows}


def chunking_study(args) -> dict:
    """One prompt prefilled unchunked and in chunks (the re-read cost of
    chunked prefills), alone and with decodes riding in every iteration.
    Shape: one tensor-parallel-2 share of a Yi-34B layer (28 q heads, 4 kv
    heads, d 128), an 8192-token prompt, 32 decodes of 2000 cached tokens."""
    import torch
    from chunked_prefill_decode_amd.runner import ChunkingStudy
    L, Hq, Hkv, d, D = args.study_len, 28, 4, 128, 32
    study = ChunkingStudy(L, Hq, Hkv, d, decodes=D, dec_ctx=2000, seed=6000)
    stream = torch.cuda.current_stream()
    kvb = 2 * Hkv * d * 2

    def timed(its, reps):
        for it in its:                                   # warm-up
            study.append(it)
            study.attend(it)
        tot_a, tot_p = [], []
        for _ in range(reps):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in its]
            for it, e in zip(its, ev):
                e[0].record(stream)
                study.append(it)
                e[1].record(stream)
                study.attend(it)
                e[2].record(stream)
            torch.cuda.synchronize()
            tot_p.append(sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3)
            tot_a.append(sum(e[1].elapsed_time(e[2]) for e in ev) * 1e3)
        tot_a.sort()
        tot_p.sort()
        return tot_a[len(tot_a) // 2], tot_p[len(tot_p) // 2]

    flops = 4 * Hq * d * (L * (L + 1) // 2)
    rows, base = [], None
    dec_only = study.iteration(0, 0, with_decodes=True, with_chunk=False)
    dec_us, _ = timed([dec_only], args.study_reps)
    for C in [L] + [c for c in (2048, 1024, 512) if c < L]:
        for with_dec in (False, True):
            its = study.schedule(C, with_decodes=with_dec)
            attn_us, app_us = timed(its, args.study_reps)
            reread = sum(it.c0 for it in its) * kvb
            r = {"chunk": C, "iterations": len(its), "decodes_per_iteration": D if with_dec else 0,
                 "attn_us": round(attn_us, 1), "append_us": round(app_us, 1),
                 "prompt_kv_bytes": sum(it.c0 + it.C for it in its) * kvb, "reread_kv_bytes": reread,
                 "prompt_tflops": round(flops / (attn_us * 1e-6) / 1e12, 1)}
            if not with_dec:
                if C == L:
                    base = attn_us
                r["overhead_vs_unchunked"] = round(attn_us / base - 1, 4)
            else:
                alone = next(x["attn_us"] for x in rows if x["chunk"] == C and x["decodes_per_iteration"] == 0)
                r["decode_marginal_us_per_iteration"] = round((attn_us - alone) / len(its), 2)
            rows.append(r)
    return {"study": "chunked prefill overhead", "layer": "Yi-34B TP-2 share: Hq=28 Hkv=4 d=128",
            "prompt_len": L, "decode_ctx": 2000, "decodes_alone_us": round(dec_us, 1),
            "reps": args.study_reps, "results": rows}


def policy_study(args) -> dict:
    """The same request trace under stall-free batching and the two baselines
    (prefill-prioritizing, decode-prioritizing), every iteration's append +
    attention timed on the GPU; simulated time advances by the measured
    kernel time.  Shape: Yi-34B TP-2 layer share (28 q / 4 kv heads, d 128);
    requests with arxiv-summarization-like lengths (prompt median 7059,
    output median 208, lognormal sigma 0.6, total <= 8192), Poisson arrivals."""
    import numpy as np
    from chunked_prefill_decode_amd.runner import PolicyTrace
    rng = np.random.default_rng(2004)
    n, rate_per_us = args.study_requests, args.study_rate / 1e6
    times = np.cumsum(rng.exponential(1.0 / rate_per_us, n))
    arrivals = []
    for i in range(n):
        L = int(np.clip(round(np.exp(rng.normal(np.log(7059), 0.6))), 64, 7800))
        O = int(np.clip(round(np.exp(rng.normal(np.log(208), 0.6))), 1, 8192 - L))
        arrivals.append((float(times[i]), L, O))
    tr = PolicyTrace(28, 4, 128, num_pages=40000, max_tokens=8192)
    tr.run(0, 2048, 0, [(0.0, a[1], 4) for a in arrivals[:4]])   # warm-up: kernels loaded, caches touched
    runs = [("stall-free B=512", 0, 512, 0), ("stall-free B=2048", 0, 2048, 0),
            ("prefill-first", 1, 8192, 8192), ("decode-first", 2, 8192, 8192)]
    out = []
    for name, policy, budget, limit in runs:
        r = tr.run(policy, budget, limit, arrivals)
        r["policy"] = name
        out.append(r)
        print(f"{name}: {r['iterations']} iterations", file=sys.stderr, flush=True)
    return {"study": "batch-building policies on one attention layer", "layer": "Yi-34B TP-2 share: Hq=28 Hkv=4 d=128",
            "requests": n, "arrival_rate_per_s": args.study_rate, "results": out}


def linear_study(args) -> dict:
    """The token-batch linear layers of one decoder layer (QKV, O, MLP) at
    M = the workload's token budget and over a sweep of M, through sa_linear;
    torch.matmul (hipBLASLt) on the same operands is timed beside it as
    context.  Per GEMM: median of HIP-event timings over warm repetitions,
    achieved TFLOP/s and GB/s (bytes: x, w and y once each) against the
    bound with the larger roofline time."""
    import torch
    import workloads as W
    from chunked_prefill_decode_amd import native as N
    model = args.workload if args.workload in W.LINEAR_LAYERS else "mistral7b"
    budget = W.make_config(WORKLOADS[model]).token_budget
    sweep = sorted({256, 257, 512, 513, 1024, 1025, 2048, 2049, budget, budget + 1})
    stream = torch.cuda.current_stream()
    reps = args.study_reps

    def timed(fn):
        for _ in range(3):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        # a spin kernel holds the stream while the host enqueues every
        # repetition, so the events time the GEMMs back to back and not the
        # host's launch latency
        torch.cuda._sleep(20_000_000)
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        return t[len(t) // 2]

    rows = []
    for i, (name, Nn, K) in enumerate(W.LINEAR_LAYERS[model]):
        w = W.linear_weight_bf16(Nn, K, 300 + i, "cuda")
        w_t = w.t().contiguous()                    # [K, N]: a plain 2-D product for torch
        for M in sweep:
            x = W.normal_bf16((M, K), 400 + M, "cuda")
            y = torch.empty(M, Nn, dtype=torch.bfloat16, device="cuda")
            ws = torch.zeros(max(N.sa_linear_workspace_size(M, Nn, K), 256), dtype=torch.uint8, device="cuda")
            us = timed(lambda: N.sa_linear(x, w, y, M, Nn, K, ws))
            ref_us = timed(lambda: torch.matmul(x, w_t))
            flops, nbytes = 2 * M * Nn * K, 2 * (M * K + Nn * K + M * Nn)
            t_hbm, t_mfma = nbytes / (HBM_PEAK_GBS * 1e3), flops / (MFMA_BF16_PEAK_TFS * 1e6)   # us
            bound = "hbm" if t_hbm >= t_mfma else "mfma"
            rows.append({"gemm": name, "M": M, "N": Nn, "K": K, "us": round(us, 2), "tflops": round(flops / us / 1e6, 1),
                         "gbs": round(nbytes / us / 1e3, 1), "bound": bound,
                         "frac": round(max(t_hbm, t_mfma) / us, 4), "torch_matmul_us": round(ref_us, 2)})
            print(f"{model} {name} M={M}: {us:.1f} us ({rows[-1]['frac']:.2f} of {bound} roofline), "
                  f"torch.matmul {ref_us:.1f} us", file=sys.stderr, flush=True)
            del x, y, ws
        del w, w_t
    per_layer = {M: round(sum(r["us"] for r in rows if r["M"] == M), 1) for M in sweep}
    per_layer_ref = {M: round(sum(r["torch_matmul_us"] for r in rows if r["M"] == M), 1) for M in sweep}
    return {"study": "token-batch linear layers of one decoder layer", "model": model, "token_budget": budget,
            "layer_us_by_M": per_layer, "layer_us_torch_matmul_by_M": per_layer_ref, "gemms": rows}


def kernel_rates_study(args) -> dict:
    """The attention kernel on two isolated item kinds, for its roofline
    reading without the mix of a real batch:
    - chunk tiles: S prefill chunks of one 32-row block each over the same
      4096 keys (every sequence's block table names the same 256 pages, so
      the keys stay in L2) -> 2 * S equal chunk items of 128 key tiles, for
      d = 64 (Hq 16 / Hkv 2) and d = 128 (Hq 32 / Hkv 8); S = 256 / 64 fills
      one round of 512 workgroups;
    - decode stream: the LLaMA2-70B-shaped decodes alone (256 decodes,
      contexts U{512..8191}, Hq 64 / Hkv 8 / d 128, shuffled distinct pages:
      ~4.5 GB of K/V from HBM), and the same decodes with each sequence's
      pages consecutive."""
    import numpy as np
    import torch
    from chunked_prefill_decode_amd import native as N
    from chunked_prefill_decode_amd.runner import batch_from_arrays, new_workspace

    dev = "cuda:0"
    reps = args.study_reps

    def timed(batch, Hq, Hkv, d, P, kc, vc):
        nbytes = N.sa_batch_upload_size(batch, Hq, Hkv, d)
        staging = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        meta = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        bd = N.sa_batch_upload(batch, Hq, Hkv, d, P, staging, meta)
        T = batch.num_tokens
        q = torch.empty(T, Hq, d, dtype=torch.bfloat16, device=dev).normal_()
        out = torch.empty(T, Hq, d, dtype=torch.bfloat16, device=dev)
        ws = new_workspace(N.sa_hybrid_attn_workspace_size(bd), dev)
        scale = 1.0 / d ** 0.5
        for _ in range(3):
            N.sa_hybrid_attn(q, kc, vc, bd, scale, out, ws)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            N.sa_hybrid_attn(q, kc, vc, bd, scale, out, ws)
        e1.record()
        torch.cuda.synchronize()
        assert torch.isfinite(out.float()).all()
        return e0.elapsed_time(e1) * 1e3 / reps, int(bd.num_work_items)

    rows = []
    ctx, L, P = 4064, 32, 256
    for d, Hq, Hkv, S in ((64, 16, 2, 256), (128, 32, 8, 64)):
        g = torch.Generator(device=dev).manual_seed(8000 + d)
        kc = torch.empty(P, Hkv, 16, d, dtype=torch.bfloat16, device=dev).normal_(generator=g)
        vc = torch.empty(P, Hkv, d, 16, dtype=torch.bfloat16, device=dev).normal_(generator=g)
        bt = np.tile(np.arange(P, dtype=np.int32), (S, 1))
        slots = np.tile(np.arange(ctx, ctx + L, dtype=np.int32), S)
        batch = batch_from_arrays([L] * S, [ctx] * S, bt, slots, num_decodes=0)
        us, items = timed(batch, Hq, Hkv, d, P, kc, vc)
        flops = 4 * Hq * d * S * sum(ctx + i + 1 for i in range(L))
        rows.append({"case": f"chunk tiles d={d}", "Hq": Hq, "Hkv": Hkv, "chunks": S, "items": items,
                     "key_tiles_per_item": (ctx + L) // 32, "attn_us": round(us, 2),
                     "tiles_per_us_per_item": round((ctx + L) / 32 / us, 3),
                     "tflops": round(flops / us / 1e6, 1), "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFS, 4)})
        del kc, vc

    Hq, Hkv, d, S = 64, 8, 128, 256
    rng = np.random.default_rng(8128)
    dctx = rng.integers(512, 8192, S)
    npg = (dctx + 1 + 15) // 16
    P = int(npg.sum())
    shuffled = rng.permutation(P).astype(np.int32)
    g = torch.Generator(device=dev).manual_seed(8129)
    kc = torch.empty(P, Hkv, 16, d, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    vc = torch.empty(P, Hkv, d, 16, dtype=torch.bfloat16, device=dev).normal_(generator=g)
    byts = int((dctx + 1).sum()) * Hkv * d * 2 * 2 + 2 * S * Hq * d * 2
    # the same walks over the allocator's shuffled pages, then over pages
    # handed out in order (each sequence's pages consecutive)
    for case, perm in (("decode stream d=128", shuffled),
                       ("decode stream d=128, pages in order", np.arange(P, dtype=np.int32))):
        bt = np.full((S, 512), -1, np.int32)
        off = 0
        for s in range(S):
            bt[s, :npg[s]] = perm[off:off + npg[s]]
            off += int(npg[s])
        slots = np.array([bt[s, dctx[s] // 16] * 16 + dctx[s] % 16 for s in range(S)], np.int32)
        batch = batch_from_arrays([1] * S, dctx.tolist(), bt, slots, num_decodes=S)
        us, items = timed(batch, Hq, Hkv, d, P, kc, vc)
        rows.append({"case": case, "Hq": Hq, "Hkv": Hkv, "decodes": S, "items": items,
                     "kv_bytes": byts, "attn_us": round(us, 2), "gbs": round(byts / us / 1e3, 1),
                     "hbm_frac": round(byts / us / 1e3 / HBM_PEAK_GBS, 4)})
    return {"study": "attention kernel rates on isolated item kinds", "reps": reps, "results": rows}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--budget", type=int, default=None, help="override the token budget B")
    ap.add_argument("--window", type=int, default=0, help="sliding-window attention over this many keys (0: none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="attention launches timed after flushing L2 and the Infinity Cache (0: skip)")
    ap.add_argument("--suite", action="store_true", help="time every workload and the budget sweep")
    ap.add_argument("--study", choices=["chunking", "policies", "linear", "kernel-rates"], default=None,
                    help="run a study instead of the benchmark step and print its JSON line")
    ap.add_argument("--study-len", type=int, default=8192)
    ap.add_argument("--study-reps", type=int, default=20)
    ap.add_argument("--study-requests", type=int, default=64)
    ap.add_argument("--study-rate", type=float, default=400.0, help="policies study: arrivals per second")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one elementwise kernel reading and writing 1 GiB each "
                         "(counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the attention step shards by heads with no exchange; see the design notes).", file=sys.stderr)
        return 2

    import torch
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    from chunked_prefill_decode_amd import native  # noqa: F401  (fails loudly if the library is missing)
    if args.study:
        study = {"chunking": chunking_study, "policies": policy_study, "linear": linear_study,
                 "kernel-rates": kernel_rates_study}[args.study]
        print(json.dumps(study(args)), flush=True)
        return 0
    if args.suite:
        print(json.dumps(suite(args)), flush=True)
        return 0
    inst = W.make_config(WORKLOADS[args.workload], args.budget)

    if args.calibrate_copy:
        # an elementwise kernel that reads 1 GiB and writes 1 GiB (fp32 x 1.0):
        # the reference for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    m = measure(inst, args, args.window)
    step = m["step"]
    line = {
        "metric": "hybrid-batch attention tokens/s per layer",
        "value": round(m["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": workload_config(inst, step, args.window),
        "roofline": m["roofline"],
        "kernels_us": m["kernels_us"],
        "hybrid_attn_cold_us": m["hybrid_attn_cold_us"],
        "cold_frac": m["cold_frac"],
        "host_us": m["host_us"],
        "upload_bytes": m["upload_bytes"],
        "attn_tflops": m["attn_tflops"],
        "attn_gbs": m["attn_gbs"],
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inst, step, args.cpu_seconds, args.window)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
