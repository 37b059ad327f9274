#!/usr/bin/env python3
"""Benchmark of the paged GQA decode hot path on one MI355X.

One step = one full decode pass over one batch: the partition kernel
(block-table gather, GQA group Q load, QK^T, online softmax, PV, partial
epilogue) followed by the cross-partition merge kernel, on the caller's stream.
The host-side partition heuristic runs once per workload (it only needs the
table shape, no device data).

Default workload: Llama-3-8B-shaped decode -- 32 sequences, H_q=32, H_kv=8,
D=128, block_size 16, context lengths uniform in [512, 4096], blocks shuffled
across a pool 1.25x the need, bf16 N(0,1) data (seeded, synthetic).  R
independent copies of the KV pool and its tables (same lengths) are rotated
step by step so that the 256 MB Infinity Cache cannot serve repeated reads.

Output: one JSON line (metric, value = KV tokens/s over the timed steps, ...)
with a `roofline` object for the partition kernel (its average duration from
HIP events around the same number of back-to-back launches on the stream the
kernels run on) and a `cpu_baseline` object (the fp64 CPU oracle timed on this
host's cores on a bounded sample of the same workload).

`--workload` selects another of the synthetic workloads for reporting (the
long-context split-KV, large ragged batch, or ragged prefill cases).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV tokens/sec and achieved HBM GB/s (% of peak), paged GQA decode, 1 MI355X"
PEAK_HBM_GBPS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SOURCE = os.path.join(ROOT, "paged_kv_cache_34_amd", "csrc", "decode_kernels.h")
APPEND_SOURCE = os.path.join(ROOT, "paged_kv_cache_34_amd", "csrc", "kvcache.hip")
PREFILL_SOURCE = os.path.join(ROOT, "paged_kv_cache_34_amd", "csrc", "prefill.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def counter_traffic(kernel_tag: str, source: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    if there is none for this kernel and workload or the kernel source changed
    since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel_tag}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"^source_sha256_16:\s*(\w+)", text, re.M)
    m_b = re.search(r"^hbm_bytes_per_launch:\s*([\d.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != source_sha(source):
        return None
    return float(m_b.group(1))


def ensure_library():
    import paged_kv_cache_34_amd as pa
    if not os.path.exists(pa.LIBRARY):
        from paged_kv_cache_34_amd import build
        build.build()
    pa.library()
    return pa


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------
def decode_copies(workload: str, copies: int):
    """`copies` cases with identical lengths and shapes, independent pools and tables."""
    import numpy as np
    import workloads
    base = workloads.NAMED[workload]()
    out = [base]
    for r in range(1, copies):
        rng = np.random.default_rng(10_000 * r + base.seed)
        layout = "fragmented" if workload == "large_ragged_decode" else "shuffled"
        out.append(workloads.build_case(f"{workload}#copy{r}", base.seed, base.seq_lens,
                                        base.num_q_heads, base.num_kv_heads, base.head_dim,
                                        layout=layout, rng=rng,
                                        partition_size=base.partition_size,
                                        max_blocks_per_seq=base.max_blocks_per_seq))
    return out


def to_device(case):
    import numpy as np
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    d = dict(q=bf(case.q), k=bf(case.k_cache), v=bf(case.v_cache),
             bt=torch.from_numpy(case.block_tables).cuda(), sl=torch.from_numpy(case.seq_lens).cuda())
    if case.cu_seqlens is not None:
        d["cu"] = torch.from_numpy(case.cu_seqlens).cuda()
    return d


def to_fp8_cache(pa, case, d):
    """Quantize a device copy of a bf16 case into an FP8 cache with the
    library's own append kernel: every token of every sequence is appended
    (its rows gathered from the bf16 pool through the block table)."""
    import numpy as np
    import torch
    lens = torch.from_numpy(case.seq_lens.astype(np.int64)).cuda()
    S, bs = case.num_seqs, case.block_size
    seq_of = torch.repeat_interleave(torch.arange(S, device="cuda"), lens)
    starts = torch.cumsum(lens, 0) - lens
    tok = torch.arange(int(lens.sum()), device="cuda") - starts[seq_of]
    phys = d["bt"][seq_of, tok // bs].long()
    k_rows = d["k"][phys, :, tok % bs, :].contiguous()
    v_rows = d["v"][phys, :, tok % bs, :].contiguous()
    cu = torch.zeros(S + 1, dtype=torch.int32, device="cuda")
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    shape = tuple(d["k"].shape)
    kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    vc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    vs = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    pa.paged_attn_kv_append_fp8(k_rows, v_rows, d["bt"], d["sl"], cu, int(case.seq_lens.max()),
                                kc, vc, ks, vs)
    torch.cuda.synchronize()
    return dict(q=d["q"], k=kc, v=vc, ks=ks, vs=vs, bt=d["bt"], sl=d["sl"])


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on host cores, bounded sample
# ---------------------------------------------------------------------------
def host_cpu():
    """nproc (CPUs this process may run on), the machine's logical CPU count
    and the CPU model name, as the host reports them."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count()
    return {"nproc": nproc, "logical_cpus": os.cpu_count(), "cpu_model": model}


def cpu_baseline(case, seconds: float, prefill: bool):
    import oracle
    orc = oracle.get()
    host = host_cpu()
    if prefill:
        t0 = time.perf_counter()
        orc.prefill_case(case)
        dt = time.perf_counter() - t0
        import numpy as np
        n = (case.cu_seqlens[1:] - case.cu_seqlens[:-1]).astype(np.float64)
        c = case.seq_lens - n
        flops = 4.0 * case.head_dim * case.num_q_heads * float(np.sum(n * c + n * (n + 1) / 2))
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(),
                "kind": "oracle", **host,
                "sample": f"one full pass of the {case.name} workload ({case.total_q} query rows), "
                          f"{dt:.1f} s wall"}
    P = case.partition_size
    reps, t_total = 0, 0.0
    while t_total < seconds or reps == 0:
        t0 = time.perf_counter()
        if P:
            ml, es, to = orc.partials_case(case, P)
            orc.reduce(ml, es, to, case.seq_lens, P)
        else:
            orc.decode_case(case)
        t_total += time.perf_counter() - t0
        reps += 1
    what = "partials + merge" if P else "single-pass decode"
    return {"value": case.kv_tokens * reps / t_total, "unit": "KV tokens/s",
            "cores": orc.num_threads(), "kind": "oracle", **host,
            "sample": f"the full {case.name} workload ({case.num_seqs} sequences, {case.kv_tokens} KV "
                      f"tokens), oracle {what}, repeated {reps}x in {t_total:.1f} s"}


# ---------------------------------------------------------------------------
# runs
# ---------------------------------------------------------------------------
def run_decode(args, pa, passes=("fused", "dist", "ceiling")):
    """The decode step of args.workload, timed cold over rotated pool copies;
    `passes` adds the fused entry point's step, the step-time distribution and
    warm case, and the read / gather ceilings."""
    import numpy as np
    import torch
    copies = args.copies or (3 if args.workload == "llama3_8b_decode" else 2)
    t0 = time.perf_counter()
    cases = decode_copies(args.workload, copies)
    log(f"generated {copies} copies of {args.workload} in {time.perf_counter() - t0:.1f} s")
    c0 = cases[0]
    if args.partition_size is not None:
        P = args.partition_size
    elif c0.partition_size:
        P = c0.partition_size
    else:
        P = pa.paged_attn_choose_partition_size(c0.num_seqs, c0.num_kv_heads, int(c0.seq_lens.max()),
                                                c0.kv_tokens)
    devs = [to_device(c) for c in cases]
    fp8 = args.kv_dtype == "fp8"
    xp = args.kv_layout == "xpacked"
    tok = args.kv_layout == "tokens"
    if fp8 and (xp or tok):
        raise SystemExit("--kv-layout xpacked / tokens hold bf16 values")
    if tok:  # one-token pages: the same blocks' tokens as slots 16 * block + slot (torch: plumbing)
        import numpy as np
        for c, d in zip(cases, devs):
            nb, hkv, bs, D = d["k"].shape
            d["k"] = d["k"].permute(0, 2, 1, 3).contiguous().view(nb * bs, hkv, D)
            d["v"] = d["v"].permute(0, 2, 1, 3).contiguous().view(nb * bs, hkv, D)
            idx = [int(c.block_tables[s, t // bs]) * bs + t % bs
                   for s, L in enumerate(c.seq_lens) for t in range(int(L))]
            ip = np.zeros(c.num_seqs + 1, np.int32)
            ip[1:] = np.cumsum(c.seq_lens)
            d["indptr"] = torch.from_numpy(ip).cuda()
            d["indices"] = torch.from_numpy(np.asarray(idx, np.int32)).cuda()
    if xp:  # the same cache rearranged on the GPU (torch permute: plumbing, not the method)
        for d in devs:
            nb, hkv, bs, D = d["k"].shape
            d["k"] = d["k"].view(nb, hkv, bs, D // 8, 8).permute(0, 1, 3, 2, 4).contiguous()
            d["v"] = d["v"].permute(0, 1, 3, 2).contiguous()
    if fp8:
        t0 = time.perf_counter()
        devs = [to_fp8_cache(pa, c, d) for c, d in zip(cases, devs)]
        log(f"quantized {copies} pool copies to FP8 on the GPU in {time.perf_counter() - t0:.1f} s")
    npart = pa.paged_attn_num_partitions(c0.max_blocks_per_seq, c0.block_size, P) if P else 1
    ws = pa.DecodeWorkspace(c0.num_seqs, c0.num_q_heads, c0.head_dim, npart, "cuda",
                            num_kv_heads=c0.num_kv_heads) if P else None
    # the merge is a separate kernel unless --merge fused asks for the
    # last-workgroup merge inside the partition kernel
    fused = bool(P) and args.merge == "fused"
    if fused and fp8:
        raise SystemExit("--merge fused is not available with --kv-dtype fp8")

    def decode_call(d, out_or_none):
        kw = dict(max_logits=ws.max_logits, exp_sums=ws.exp_sums, tmp_out=ws.tmp_out,
                  max_num_partitions=npart) if P else dict(out=out_or_none)
        if fp8:
            pa.paged_attn_decode_fp8(d["q"], d["k"], d["v"], d["ks"], d["vs"], d["bt"], d["sl"], scale,
                                     P, stream=stream, **kw)
        elif xp:
            pa.paged_attn_decode_xpacked(d["q"], d["k"], d["v"], d["bt"], d["sl"], scale, P,
                                         stream=stream, **kw)
        elif tok:
            pa.paged_attn_decode_tokens(d["q"], d["k"], d["v"], d["indptr"], d["indices"],
                                        c0.max_blocks_per_seq * c0.block_size, scale, P,
                                        stream=stream, **kw)
        else:
            pa.paged_attn_decode(d["q"], d["k"], d["v"], d["bt"], d["sl"], scale, P, stream=stream, **kw)
    out = torch.empty_like(devs[0]["q"])
    scale = float(c0.scale)
    stream = torch.cuda.current_stream()

    def step(i):
        d = devs[i % copies]
        if fused:
            pa.paged_attn_decode_fused(d["q"], d["k"], d["v"], d["bt"], d["sl"], scale, P, out,
                                       ws.max_logits, ws.exp_sums, ws.tmp_out, ws.counters,
                                       stream=stream)
            return
        decode_call(d, out)
        if P and tok:
            pa.paged_attn_decode_reduce_indptr(ws.max_logits, ws.exp_sums, ws.tmp_out, d["indptr"], P,
                                               out, stream=stream)
        elif P:
            pa.paged_attn_decode_reduce(ws.max_logits, ws.exp_sums, ws.tmp_out, d["sl"], P, out,
                                        stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: whole steps, nothing else on the stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    # timed region 2: the partition kernel alone, the same launches back to back
    # (one event pair around all of them, as a profiler times kernel execution)
    def decode_only(i):
        d = devs[i % copies]
        if fused:
            step(i)
            return
        decode_call(d, out)

    torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        decode_only(i)
    k1.record(stream)
    torch.cuda.synchronize()
    ms_kernel = k0.elapsed_time(k1) / args.steps
    # timed region 3 (bf16 block cache, separate merge timed above): the same
    # steps through the fused entry point, reported beside the main line
    ms_fused = None
    if P and "fused" in passes and not (fused or fp8 or xp or tok):
        def fused_step(i):
            d = devs[i % copies]
            pa.paged_attn_decode_fused(d["q"], d["k"], d["v"], d["bt"], d["sl"], scale, P, out,
                                       ws.max_logits, ws.exp_sums, ws.tmp_out, ws.counters,
                                       stream=stream)
        for i in range(args.warmup):
            fused_step(i)
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for i in range(args.steps):
            fused_step(i)
        f1.record(stream)
        torch.cuda.synchronize()
        ms_fused = f0.elapsed_time(f1) / args.steps
    # timed region 4: the step-time distribution (an event between steps) and
    # the warm case (one pool copy reused, so part of it stays cached)
    def per_step(fn, n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        evs[0].record(stream)
        for i in range(n):
            fn(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        return np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(n)])
    dist = warm = None
    if "dist" in passes:
        dist = per_step(step, max(args.steps, 100))
        warm = per_step(lambda i: step(0), max(args.steps, 100))
    # leave the output of a full step behind (the partials above are not merged)
    step(0)
    torch.cuda.synchronize()

    tokens = c0.kv_tokens
    # algorithmic bytes per KV token: K and V of every kv head -- bf16 values,
    # or E4M3 codes plus one fp32 scale per (position, kv head) each
    bytes_per_token = c0.num_kv_heads * 2 * (c0.head_dim + 4 if fp8 else 2 * c0.head_dim)
    kv_bytes = tokens * bytes_per_token
    step_gbps = kv_bytes / (ms_step * 1e-3) / 1e9
    kern_gbps = kv_bytes / (ms_kernel * 1e-3) / 1e9
    traffic = counter_traffic("decode_fp8" if fp8 else "decode_xpacked" if xp else "decode",
                              DECODE_SOURCE, args.workload)
    ceiling = None if (args.no_read_ceiling or "ceiling" not in passes) else read_ceiling(pa, kv_bytes, copies, cases, devs)
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 kv, bf16 q" if fp8 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload + ("_fp8" if fp8 else "") + ("_xpacked" if xp else "")
                        + ("_tokens" if tok else ""),
            "kv_cache": ("fp8 e4m3 + per-position fp32 scales" if fp8 else "bf16")
                        + (", x-packed K / transposed V" if xp else "")
                        + (", one-token pages (kv_indptr + page indices)" if tok else ""),
            "num_seqs": c0.num_seqs,
            "num_q_heads": c0.num_q_heads,
            "num_kv_heads": c0.num_kv_heads,
            "head_dim": c0.head_dim,
            "block_size": c0.block_size,
            "kv_tokens": tokens,
            "seq_len_min": int(c0.seq_lens.min()),
            "seq_len_max": int(c0.seq_lens.max()),
            "partition_size": P,
            "merge": "fused into the partition kernel" if fused else ("separate kernel" if P else "none (single pass)"),
            "kv_pool_copies_rotated": copies,
        },
        "hbm_gbps": step_gbps,
        "hbm_pct_of_peak": 100.0 * step_gbps / PEAK_HBM_GBPS,
        "accumulate": "fp32",
        "roofline": {
            "bound": "hbm",
            "kernel": ("paged_decode_compact_kernel (fused merge)" if fused else "paged_decode_compact_kernel")
                      + (" <FP8>" if fp8 else "") + (" <x-packed>" if xp else "")
                      + (" <token-granular>" if tok else ""),
            "achieved": kern_gbps,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": kern_gbps / PEAK_HBM_GBPS,
            "traffic": traffic,
            "kernel_ms": ms_kernel,
            "algorithmic_bytes_per_launch": kv_bytes,
        },
    }
    if args.cold_only:
        result["cold_only"] = ("only the warmup, the timed steps and the partition kernel's own timed "
                               "launches ran, every one on a rotated (cold) pool copy")
    if dist is not None:
        result["step_distribution"] = {
            "per_step_events": int(dist.size), "median_ms": float(np.median(dist)),
            "p10_ms": float(np.percentile(dist, 10)), "p90_ms": float(np.percentile(dist, 90)),
            "warm_one_copy_median_ms": float(np.median(warm)),
            "note": "an event between consecutive steps (timed separately from ms_per_step); warm = the "
                    "same pool copy every step, so part of it stays in the 256 MB Infinity Cache"}
    if ms_fused is not None:
        result["fused_merge"] = {
            "entry_point": "paged_attn_decode_fused (stream-K schedule, merge in the last workgroup)",
            "ms_per_step": ms_fused, "value": tokens / (ms_fused * 1e-3), "unit": "KV tokens/s",
            "hbm_gbps": kv_bytes / (ms_fused * 1e-3) / 1e9,
            "frac_of_peak": kv_bytes / (ms_fused * 1e-3) / 1e9 / PEAK_HBM_GBPS}
    if ceiling is not None:
        ceiling["kernel_frac_of_same_bytes_read"] = kern_gbps / ceiling["same_bytes_rotated_gbps"]
        ceiling["kernel_frac_of_large_read"] = kern_gbps / ceiling["large_buffer_gbps"]
        if "gather_tiles_gbps" in ceiling:
            ceiling["kernel_frac_of_tile_gather"] = kern_gbps / ceiling["gather_tiles_gbps"]
            ceiling["step_frac_of_tile_gather"] = step_gbps / ceiling["gather_tiles_gbps"]
        result["read_ceiling"] = ceiling
    return result, cases[0]


def gather_ceiling(pa, cases, devs):
    """Paged-gather ceiling from the library's gather probe: the decode's own
    K/V tiles of the rotated pool copies, read through their block tables,
    best over grids of 1..32 workgroups per CU; per-(kv head, block) tiles in
    the decode's order, whole blocks (all kv heads of a block together), and
    the tiles read through load-to-LDS instructions."""
    import numpy as np
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    c0 = cases[0]
    # an E4M3 cache (one byte per element) is read as bf16 tiles of half the
    # head dim: the same bytes, block by block (its scales are not read)
    fp8 = devs[0]["k"].dtype == torch.uint8
    probe_d = c0.head_dim // 2 if fp8 else c0.head_dim
    if c0.num_seqs > 1024 or probe_d not in (64, 128, 256):
        return {}
    view = (lambda t: t.view(torch.bfloat16)) if fp8 else (lambda t: t)
    pref = np.zeros(c0.num_seqs + 1, np.int32)
    pref[1:] = np.cumsum((c0.seq_lens.astype(np.int64) + 15) // 16)
    prefd = torch.from_numpy(pref).cuda()
    nbytes = int(pref[-1]) * c0.num_kv_heads * 2 * 16 * probe_d * 2
    out = {}
    for whole in (0, 1, 2):
        best = None
        for m in (1, 2, 4, 8, 16, 32):
            partial = torch.empty(m * cus, dtype=torch.int32, device="cuda")
            call = lambda i: pa.paged_attn_gather_probe(view(devs[i % len(devs)]["k"]), view(devs[i % len(devs)]["v"]),
                                                        devs[i % len(devs)]["bt"], prefd, whole, partial,
                                                        stream=stream)
            for i in range(3):
                call(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 30
            e0.record(stream)
            for i in range(reps):
                call(i)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            if best is None or ms < best[0]:
                best = (ms, m * cus)
        key = ("gather_tiles", "gather_blocks", "gather_tiles_to_lds")[whole]
        out[key + "_gbps"] = nbytes / (best[0] * 1e-3) / 1e9
        out[key + "_ms"] = best[0]
        out[key + "_workgroups"] = best[1]
    out["gather_bytes"] = nbytes
    out["gather_probe"] = ("paged_attn_gather_probe over the decode's rotated pool copies: tiles = the K and V "
                           "tile of one (sequence, kv head, block) per wave in the decode's order; blocks = "
                           "consecutive waves read one block's H_kv tiles of K then V; tiles_to_lds = the "
                           "tiles through load-to-LDS instructions into a two-piece LDS ring per wave; best "
                           "of 1..32 workgroups per CU" + ("; E4M3 cache: its code tiles read as bf16 tiles of "
                           "half the head dim (gather_bytes = the codes, without the scales)" if fp8 else ""))
    log(f"gather ceiling: tiles {out['gather_tiles_gbps']:.0f} GB/s ({out['gather_tiles_ms'] * 1e3:.1f} us), "
        f"whole blocks {out['gather_blocks_gbps']:.0f} GB/s ({out['gather_blocks_ms'] * 1e3:.1f} us), "
        f"tiles to LDS {out['gather_tiles_to_lds_gbps']:.0f} GB/s ({out['gather_tiles_to_lds_ms'] * 1e3:.1f} us)")
    return out


def read_ceiling(pa, nbytes: int, copies: int, cases=None, devs=None):
    """Measured HBM read ceiling from the library's read-stream probe: the best
    rate over grids of 16..256 workgroups per CU, on one large buffer (steady
    streaming) and on `copies` rotated buffers of `nbytes` each (the decode's
    own bytes per launch, read cold); plus, given the decode's pool copies,
    the paged-gather ceiling of its own tiles."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()

    def rate(bufs, nwg, reps):
        partial = torch.empty(nwg, dtype=torch.int32, device="cuda")
        for i in range(3):
            pa.paged_attn_read_probe(bufs[i % len(bufs)], partial, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            pa.paged_attn_read_probe(bufs[i % len(bufs)], partial, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        return bufs[0].numel() * bufs[0].element_size() / (ms * 1e-3) / 1e9, ms, nwg

    grids = [m * cus for m in (16, 32, 64, 128, 256)]
    big = [torch.empty(1 << 30, dtype=torch.int32, device="cuda")]       # 4 GiB
    large_gbps, _, large_nwg = max(rate(big, g, 8) for g in grids)
    del big
    n16 = (nbytes + 15) // 16 * 4
    same = [torch.empty(n16, dtype=torch.int32, device="cuda") for _ in range(copies)]
    same_gbps, same_ms, same_nwg = max(rate(same, g, 30) for g in grids)
    del same
    torch.cuda.empty_cache()
    log(f"read ceiling: {large_gbps:.0f} GB/s over 4 GiB ({large_nwg} workgroups), {same_gbps:.0f} GB/s "
        f"over {copies} rotated buffers of {nbytes / 1e6:.1f} MB ({same_ms * 1e3:.1f} us each, "
        f"{same_nwg} workgroups)")
    res = {"probe": "paged_attn_read_probe (16-byte nontemporal loads, XOR-folded), best of "
                    "16..256 workgroups per CU",
           "large_buffer_bytes": 1 << 32, "large_buffer_gbps": large_gbps, "large_buffer_workgroups": large_nwg,
           "same_bytes": nbytes, "same_bytes_rotated_copies": copies,
           "same_bytes_rotated_gbps": same_gbps, "same_bytes_ms": same_ms, "same_bytes_workgroups": same_nwg}
    if cases is not None and devs is not None:
        res.update(gather_ceiling(pa, cases, devs))
    return res


def run_prefill(args, pa):
    import numpy as np
    import torch
    import workloads
    case = workloads.ragged_prefill()
    d = to_device(case)
    out = torch.empty_like(d["q"])
    stream = torch.cuda.current_stream()
    scale = float(case.scale)
    split = args.prefill_form == "split"
    ws = None
    if split:
        ws = pa.PrefillWorkspace(case.num_seqs, case.total_q, case.num_q_heads, case.num_kv_heads,
                                 case.head_dim, case.max_blocks_per_seq, 16, "cuda")
        log(f"split-KV prefill, key chunk {ws.kv_chunk}, workspace {ws.buffer.numel() / 1e6:.1f} MB")

    def step():
        if split:
            pa.paged_attn_prefill_ragged_split(d["q"], d["k"], d["v"], d["bt"], d["sl"], d["cu"],
                                               case.max_q_len, scale, out, workspace=ws.buffer,
                                               stream=stream)
        else:
            pa.paged_attn_prefill_ragged(d["q"], d["k"], d["v"], d["bt"], d["sl"], d["cu"],
                                         case.max_q_len, scale, out, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    n = (case.cu_seqlens[1:] - case.cu_seqlens[:-1]).astype(np.float64)
    c = case.seq_lens - n
    flops = 4.0 * case.head_dim * case.num_q_heads * float(np.sum(n * c + n * (n + 1) / 2))
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "causal TFLOP/s, ragged paged prefill, 1 MI355X",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "ragged_prefill", "num_seqs": case.num_seqs, "total_q": case.total_q,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "kv_tokens": case.kv_tokens,
                   "form": "split-KV" if split else "single pass",
                   "kv_chunk": ws.kv_chunk if split else 0},
        "kv_gbps": case.kv_bytes / (ms * 1e-3) / 1e9,
        # the split form is one API call of two launches (chunks, then merge);
        # its time is taken over both, so the merge counts against the kernel
        "roofline": {"bound": "mfma",
                     "kernel": ("paged_prefill_split_kernel+paged_prefill_merge_kernel" if split
                                else "paged_prefill_kernel"),
                     "achieved": tflops,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": counter_traffic("prefill", PREFILL_SOURCE, "ragged_prefill"),
                     "kernel_ms": ms, "algorithmic_flops_per_launch": flops},
    }
    return result, case


def run_append(args, pa):
    """KV append of the ragged prefill batch's new rows (its 16 sequences'
    U[1, 256] new tokens after U[0, 8192] cached ones): bf16 copy or FP8
    quantize-and-write into the paged cache, HBM-bound."""
    import numpy as np
    import torch
    import workloads
    case = workloads.ragged_prefill()
    d = to_device(case)
    fp8 = args.kv_dtype == "fp8"
    total, hkv, D = case.total_q, case.num_kv_heads, case.head_dim
    g = torch.Generator(device="cuda").manual_seed(case.seed)
    k_new = torch.randn((total, hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((total, hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    shape = tuple(d["k"].shape)
    if fp8:
        kc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        vc = torch.zeros(shape, dtype=torch.uint8, device="cuda")
        ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
        vs = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    maxn = case.max_q_len

    def step():
        if fp8:
            pa.paged_attn_kv_append_fp8(k_new, v_new, d["bt"], d["sl"], d["cu"], maxn, kc, vc, ks, vs,
                                        stream=stream)
        else:
            pa.paged_attn_kv_append(k_new, v_new, d["bt"], d["sl"], d["cu"], maxn, d["k"], d["v"],
                                    stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(args.steps):
        step()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    # algorithmic bytes: the new K and V rows read (bf16) and written (bf16, or
    # E4M3 codes plus one fp32 scale per row)
    rows = total * hkv * 2
    nbytes = rows * D * 2 + rows * (D + 4 if fp8 else 2 * D)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {
        "metric": "KV append bandwidth, paged KV cache write, 1 MI355X",
        "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 -> fp8-e4m3" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": "kv_append" + ("_fp8" if fp8 else ""), "num_seqs": case.num_seqs,
                   "new_tokens": total, "num_kv_heads": hkv, "head_dim": D},
        "roofline": {"bound": "hbm", "kernel": "paged_kv_append_fp8_kernel" if fp8 else "paged_kv_append_kernel",
                     "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                     "traffic": counter_traffic("append_fp8" if fp8 else "append", APPEND_SOURCE, "kv_append"),
                     "kernel_ms": ms, "algorithmic_bytes_per_launch": nbytes},
    }, None


def secondary_lines(args, pa):
    """The other configurations, timed in the same run as the headline line
    (no CPU baseline for them): the long-context split-KV and large ragged
    decode (separate merge and fused entry point) and the ragged prefill."""
    import torch
    out = {}
    t0 = time.perf_counter()
    for wl in ("long_split_decode", "large_ragged_decode"):
        sub = argparse.Namespace(**vars(args))
        sub.workload, sub.steps, sub.warmup, sub.cold_only = wl, args.secondary_steps, 200, False
        sub.kv_dtype, sub.kv_layout, sub.merge, sub.partition_size, sub.copies = "bf16", "tile", "separate", None, None
        r, _ = run_decode(sub, pa, passes=("fused",))
        rf = r["roofline"]
        out[wl] = {"ms_per_step": r["ms_per_step"], "kv_tokens_per_s": r["value"],
                   "hbm_gbps": r["hbm_gbps"], "hbm_pct_of_peak": r["hbm_pct_of_peak"],
                   "partition_kernel_ms": rf["kernel_ms"], "partition_kernel_frac": rf["frac"],
                   "partition_size": r["config"]["partition_size"], "kv_tokens": r["config"]["kv_tokens"],
                   "pool_copies_rotated": r["config"]["kv_pool_copies_rotated"], "steps": sub.steps}
        if "fused_merge" in r:
            out[wl]["fused_ms_per_step"] = r["fused_merge"]["ms_per_step"]
            out[wl]["fused_kv_tokens_per_s"] = r["fused_merge"]["value"]
            out[wl]["fused_frac_of_peak"] = r["fused_merge"]["frac_of_peak"]
        torch.cuda.empty_cache()
    sub = argparse.Namespace(**vars(args))
    # (600 warmup steps, ~0.1 s: the inputs are generated on the host just
    # before, and the GPU's clocks drop while it idles)
    sub.workload, sub.steps, sub.warmup, sub.prefill_form = "ragged_prefill", args.secondary_steps, 600, "split"
    r, _ = run_prefill(sub, pa)
    out["ragged_prefill"] = {"ms_per_step": r["ms_per_step"], "tflops": r["value"],
                             "frac_of_bf16_peak": r["roofline"]["frac"], "kv_chunk": r["config"]["kv_chunk"],
                             "total_q": r["config"]["total_q"], "steps": sub.steps}
    torch.cuda.empty_cache()
    out["note"] = (f"timed in this run after the headline ({args.secondary_steps} steps each, cold rotated "
                   f"pool copies for decode; {time.perf_counter() - t0:.0f} s including input generation)")
    return out


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """A plain device-to-device copy of known size, for scaling HBM counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": nbytes, "bytes_written_per_copy": nbytes,
                                           "copies": reps}}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000,
                    help="untimed steps before the timed ones (the default keeps the GPU busy for "
                         "50 ms or more first, so that its clocks have left their idle state: with 20, "
                         "the ragged prefill measured 6%% slower)")
    ap.add_argument("--workload", default="llama3_8b_decode",
                    choices=["llama3_8b_decode", "long_split_decode", "large_ragged_decode",
                             "ragged_prefill", "tiny_decode", "kv_append"])
    ap.add_argument("--kv-layout", default="tile", choices=["tile", "xpacked", "tokens"],
                    help="decode workloads: row-major [blocks, H_kv, 16, D] tiles, x-packed K "
                         "[blocks, H_kv, D/8, 16, 8] with transposed V [blocks, H_kv, D, 16], or "
                         "one-token pages [slots, H_kv, D] addressed by kv_indptr + page indices")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="decode workloads and kv_append: bf16 cache, or FP8 (E4M3 codes with "
                         "per-position scales) quantized on the GPU by the library's append kernel")
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--copies", type=int, default=None,
                    help="independent KV pool copies rotated across steps (default 3, or 2 for >1 GB pools)")
    ap.add_argument("--merge", default="separate", choices=["fused", "separate"],
                    help="cross-partition merge: a separate kernel (default: the reduce entry point "
                         "of the C ABI) or fused into one launch (stream-K schedule; the default "
                         "decode line also times it, as fused_merge)")
    ap.add_argument("--prefill-form", default="split", choices=["split", "single"],
                    help="ragged_prefill: split-KV entry point (default) or the single-pass one")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the read-stream probe that measures the HBM read ceiling (decode workloads)")
    ap.add_argument("--cold-only", action="store_true",
                    help="only the warmup and the timed cold steps (plus the partition kernel's own timed "
                         "launches): no fused, per-step, warm, ceiling, secondary or CPU passes -- the mode "
                         "whose rocprofv3 traces match the line")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary configurations the default decode line carries")
    ap.add_argument("--secondary-steps", type=int, default=50)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (the reference kernel for HBM counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the decode would shard by sequence or by kv head, one GPU per share). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    pa = ensure_library()
    if args.workload == "ragged_prefill":
        result, case = run_prefill(args, pa)
    elif args.workload == "kv_append":
        result, case = run_append(args, pa)
    else:
        result, case = run_decode(args, pa, passes=() if args.cold_only else ("fused", "dist", "ceiling"))
    if (args.workload == "llama3_8b_decode" and not (args.cold_only or args.no_secondary)
            and args.kv_dtype == "bf16" and args.kv_layout == "tile" and args.merge == "separate"):
        log("timing the secondary configurations")
        result["secondary"] = secondary_lines(args, pa)
    if (not (args.no_cpu_baseline or args.cold_only) and case is not None and args.kv_dtype == "bf16"
            and args.kv_layout == "tile"):
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds, args.workload == "ragged_prefill")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
