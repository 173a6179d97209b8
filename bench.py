"""Benchmark one decode step (paged KV write of the step's tokens + paged
attention decode) on one MI355X and print ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7b-decode-bf16]

A step is the whole hot path over one batch: paged_kv_cache_write of each
sequence's newest token, the decode partition kernel and the split reduce.
Inputs are seeded synthetic tensors already resident in HBM.  `value` is the
algorithmic KV bytes the decode reads per step divided by the step time
(GB/s); `roofline` is the partition kernel's algorithmic bytes over its own
event-timed duration against the 8 TB/s HBM peak; `cpu_baseline` times the
CPU oracle (float64 numpy, one BLAS thread) on a bounded sample of the same
workload.  `block_copy` times whole-block copies on the same pool: a
device-to-device copy (copy-on-write) and swapping blocks out to pinned host
memory and back in.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged-decode attention: KV bytes read GB/s (% of HBM peak); seq-heads/s"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
WORKLOADS = {"tiny-fp32": 1, "7b-decode-bf16": 2, "32k-gqa-bf16": 3,
             "shared-prefix-bf16": 4, "fp8-kv": 5}
DEFAULT_WORKLOAD = "7b-decode-bf16"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.txt")
KERNEL_SOURCES = ("decode_valu.hip", "decode_mfma.hip", "pkv_device.h", "pkv_internal.h")
PREFILL_SOURCES = ("prefill_mfma.hip", "pkv_device.h", "pkv_internal.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="tokens per partition; -1 = the workload's own, 0 = library choice")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill", default="prefill-chunk-gqa-bf16",
                    help="chunked-prefill workload timed beside the decode step ('none': skip)")
    ap.add_argument("--beam-fork", default="beam-fork-gqa-bf16",
                    help="multi-query step over forked tables timed beside the decode step "
                         "('none': skip)")
    ap.add_argument("--no-block-copy", action="store_true",
                    help="skip the block copy / swap measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate CPU time budget for the oracle sample")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a device-to-device copy of this many MiB (5 times), to scale "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes_each_way": n * 4, "launches": 5}), flush=True)


def kv_bytes(w):
    """Algorithmic bytes a decode reads: every distinct (physical block, KV
    head) tile once, valid token rows only, K and V, plus FP8 scales."""
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]
    rows = {}
    for i in range(w.S):
        n = int(w.context_lens[i])
        nb = -(-n // w.block_size)
        for j in range(nb):
            b = int(w.block_tables[i, j])
            rows[b] = max(rows.get(b, 0), min(w.block_size, n - j * w.block_size))
    tokens = sum(rows.values())
    total = tokens * w.H_kv * w.D * elem * 2
    if w.cache_dtype == "fp8":
        total += len(rows) * w.H_kv * 4 * 2
    return total, len(rows)


def kernel_source_hash(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for name in sources:
        p = os.path.join(ROOT, "paged_kv_cache_370_amd", "csrc", name)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, sources=KERNEL_SOURCES):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 PMC summary, if it was taken on the current kernel
    sources; else None."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    src = kernel_source_hash(sources)
    for line in open(COUNTERS_FILE):
        parts = line.split()
        if len(parts) >= 4 and parts[0] == "traffic" and parts[1] == workload and parts[2] == src:
            return float(parts[3])
    return None


def cpu_baseline(w, budget_s, min_s=10.0):
    """The oracle's decode, sequence by sequence on one host thread, repeated
    over the batch until at least min_s seconds of work (or stopped at
    budget_s): a bounded sample of the same workload."""
    import oracle
    from threadpoolctl import threadpool_limits

    kc, vc, ks, vs = w.key_cache, w.value_cache, w.key_scale, w.value_scale
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]
    t_total = 0.0
    done_bytes = 0
    done = 0
    with threadpool_limits(limits=1):
        while t_total < min(min_s, budget_s):
            for i in range(w.S):
                n = int(w.context_lens[i])
                sub_tab = w.block_tables[i:i + 1]
                t0 = time.perf_counter()
                oracle.paged_attention_decode(w.q[i:i + 1], kc, vc, sub_tab,
                                              w.context_lens[i:i + 1], w.scale, w.block_size,
                                              ks, vs)
                t_total += time.perf_counter() - t0
                done_bytes += n * w.H_kv * w.D * elem * 2
                done += 1
                if t_total >= budget_s:
                    break
            if done == 0:
                break
    passes = done / w.S if w.S else 0.0
    return {"value": done_bytes / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"float64 numpy oracle decode, {done} sequence decodes ({passes:.2f} passes "
                      f"over the {w.S} sequences; {done * w.H} seq-heads, "
                      f"{done_bytes / 1e6:.1f} MB of KV) in {t_total:.1f} s on one host thread",
            "seq_heads_per_s": done * w.H / t_total}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return

    import torch
    import paged_kv_cache_370_amd as pkv
    import workloads

    pkv.load()
    cfg = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = workloads.make_config(cfg)
    gen_s = time.perf_counter() - t0
    total_bytes, nblocks = kv_bytes(w)
    ps = w.partition_size if args.partition_size < 0 else args.partition_size

    dev = torch.device("cuda:0")

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q = t(w.q)
    kc, vc = t(w.key_cache), t(w.value_cache)
    ks = t(w.key_scale) if w.key_scale is not None else None
    vs = t(w.value_scale) if w.value_scale is not None else None
    tables, lens = t(w.block_tables), t(w.context_lens)
    writes = [(t(k), t(v), t(s)) for k, v, s in w.writes]
    out = torch.empty_like(q)
    qc, cc = pkv.dtype_code(q), pkv.dtype_code(kc)
    P = pkv.decode_partition_size(w.S, w.H, w.H_kv, w.D, w.block_size, w.max_context_len, qc, cc, ps)
    ws_bytes = pkv.decode_workspace_size(w.S, w.H, w.H_kv, w.D, w.block_size, w.max_context_len,
                                         qc, cc, ps)
    dws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)  # counters start at 0
    wws_bytes = pkv.write_workspace_size(max(len(x[2]) for x in writes), w.H_kv, w.num_blocks, cc)
    wws = torch.empty(max(wws_bytes, 1), dtype=torch.uint8, device=dev) if wws_bytes else None

    # Setup writes (FP8: the bulk write of positions 0..n-2) are not part of a step.
    setup = writes[:-1]
    step_write = writes[-1]
    setup_ms = None
    if setup:
        # The first run loads the write kernels; the timed second run writes
        # the same tokens to the same slots, with the same result (every
        # block it writes is fresh again, so its scales are set again from
        # the same values).
        for k, v, s in setup:
            pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k, v, s in setup:
            pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)
        e1.record()
        torch.cuda.synchronize()
        setup_ms = e0.elapsed_time(e1)

    def step(ev=None):
        k, v, s = step_write
        if ev: ev[0].record()
        pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)
        if ev: ev[1].record()
        pkv.paged_attention_decode_partitions(out, q, kc, vc, tables, lens, w.max_context_len,
                                              w.scale, ks, vs, partition_size=ps, workspace=dws)
        if ev: ev[2].record()
        pkv.paged_attention_decode_reduce(out, lens, w.H_kv, w.block_size, w.max_context_len, cc,
                                          partition_size=ps, workspace=dws)
        if ev: ev[3].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K whole steps back to back, bracketed by two events only
    # (an event between kernels adds a marker packet to the queue).
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_step = ms_total / args.steps
    # Per-kernel times: the same K steps again with an event around each
    # kernel, on the stream the kernels run on.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    ms_step_with_events = float(np.mean([e[0].elapsed_time(e[3]) for e in evs]))
    write_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    part_ms_in_step = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    red_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in evs]))
    # The partition kernel's launch duration for the roofline: K launches
    # back to back between two events (the kernel is idempotent: same
    # inputs, same outputs, its counters return to zero), so the average
    # holds one launch gap instead of two event packets.
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    p0.record()
    for _ in range(args.steps):
        pkv.paged_attention_decode_partitions(out, q, kc, vc, tables, lens, w.max_context_len,
                                              w.scale, ks, vs, partition_size=ps, workspace=dws)
    p1.record()
    torch.cuda.synchronize()
    part_ms = p0.elapsed_time(p1) / args.steps

    value = total_bytes / (ms_step * 1e-3) / 1e9
    achieved = total_bytes / (part_ms * 1e-3) / 1e9
    traffic = recorded_traffic(args.workload)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8e4m3-kv/bf16-q"}[w.cache_dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name, "seqs": w.S, "q_heads": w.H, "kv_heads": w.H_kv,
            "head_size": w.D, "block_size": w.block_size, "max_context": w.max_context_len,
            "mean_context": round(float(np.mean(w.context_lens)), 1),
            "partition_size": P, "kv_bytes_per_step": total_bytes, "kv_blocks_read": nblocks,
            "step": "paged_kv_cache_write + decode partitions + reduce",
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.S * w.H / (ms_step * 1e-3), 1),
        "kernel_ms": {"write": round(write_ms, 5), "decode_partitions": round(part_ms, 5),
                      "decode_partitions_in_step": round(part_ms_in_step, 5),
                      "decode_reduce": round(red_ms, 5),
                      "step_with_events": round(ms_step_with_events, 5)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "decode partition kernel",
            "kernel_sources": kernel_source_hash(),
        },
        "input_generation_s": round(gen_s, 2),
    }
    if setup_ms is not None:
        setup_bytes = sum(x[0].numel() * x[0].element_size() * 2 for x in setup)
        result["setup_write"] = {"ms": round(setup_ms, 3),
                                 "source_bytes": setup_bytes,
                                 "GB_per_s_source_read": round(setup_bytes / setup_ms / 1e6, 1)}
        if w.cache_dtype == "fp8":
            # the source is read twice (amax, then encode), one byte written per element
            codes = sum(x[0].numel() * 2 for x in setup)
            result["setup_write"]["GB_per_s_hbm"] = round((2 * setup_bytes + codes) / setup_ms / 1e6, 1)
    if not args.no_block_copy:
        result["block_copy"] = block_copy_bench(pkv, torch, kc, vc, ks, vs, args.steps)
    if w.shared_blocks > 0:
        result["read_once"] = read_once_bench(pkv, torch, w, out, q, kc, vc, ks, vs, tables, lens,
                                              total_bytes, args.steps)
    if args.prefill != "none":
        result["prefill"] = prefill_bench(pkv, torch, args.prefill, args.steps)
    if args.beam_fork != "none":
        result["beam_fork"] = beam_fork_bench(pkv, torch, args.beam_fork, args.steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_for(w, writes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def block_copy_bench(pkv, torch, kc, vc, ks, vs, reps, copy_pairs=1024, swap_pairs=256):
    """Times paged_kv_block_copy on the workload's pool: copy_pairs random
    blocks into a second device pool (the copy-on-write shape: HBM read and
    write), and swap_pairs blocks out to a pinned host pool and back in
    (PCIe).  Bytes count the K and V tiles (and FP8 scales) moved once."""
    rng = np.random.default_rng(7)
    nb = kc.shape[0]
    dev = kc.device
    block_bytes = 2 * kc[0].numel() * kc.element_size() + (
        2 * ks[0].numel() * 4 if ks is not None else 0)

    def pool(blocks, pinned=False):
        mk = (lambda t: torch.empty((blocks,) + tuple(t.shape[1:]), dtype=t.dtype,
                                    pin_memory=True)) if pinned else (
            lambda t: torch.empty((blocks,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev))
        return (mk(kc), mk(vc), mk(ks) if ks is not None else None,
                mk(vs) if vs is not None else None)

    def timed(src, dst, pairs):
        pkv.paged_kv_block_copy(src[0], src[1], dst[0], dst[1], pairs, src[2], src[3], dst[2],
                                dst[3])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            pkv.paged_kv_block_copy(src[0], src[1], dst[0], dst[1], pairs, src[2], src[3],
                                    dst[2], dst[3])
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        n = pairs.shape[0]
        return {"pairs": n, "us": round(us, 2), "bytes_moved": n * block_bytes,
                "GB_per_s": round(n * block_bytes / (us * 1e-6) / 1e9, 1)}

    src = (kc, vc, ks, vs)
    n = min(copy_pairs, nb)
    pairs = torch.from_numpy(np.stack([rng.choice(nb, n, replace=False), rng.permutation(n)],
                                      axis=1).astype(np.int32)).to(dev)
    out = {"block_bytes": block_bytes,
           "device_copy": timed(src, pool(n), pairs)}
    m = min(swap_pairs, nb)
    host = pool(m, pinned=True)
    out_pairs = torch.from_numpy(np.stack([rng.choice(nb, m, replace=False), rng.permutation(m)],
                                          axis=1).astype(np.int32)).to(dev)
    out["swap_out"] = timed(src, host, out_pairs)
    in_pairs = torch.from_numpy(np.stack([rng.permutation(m), rng.permutation(m)],
                                         axis=1).astype(np.int32)).to(dev)
    out["swap_in"] = timed(host, pool(m), in_pairs)
    out["note"] = ("device_copy moves each byte HBM to HBM (it is read and written: 2x the "
                   "bytes in HBM traffic); swaps cross PCIe once")
    return out


def prefill_flops(lens, M, H, D):
    """Algorithmic flops of causal multi-token attention: token t of a
    sequence of n tokens sees e = n - M + t + 1 positions; per query head
    QK^T and PV take 2 * D * e multiply-adds each (4 * D * e flops)."""
    e = np.concatenate([np.asarray(n) - M + np.arange(M) + 1 for n in lens])
    return int(4 * D * H * e.sum())


def prefill_bench(pkv, torch, name, reps):
    """Times one chunked-prefill step (paged_kv_cache_write of the chunk's
    K/V, then paged_attention_prefill) on a synthetic workload, and the
    attention launch alone back to back, against the bf16 MFMA peak."""
    import workloads
    w = workloads.make_prefill(name)
    dev = torch.device("cuda:0")

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, kc, vc = t(w.q), t(w.key_cache), t(w.value_cache)
    tables, lens = t(w.block_tables), t(w.context_lens)
    key, value, slots = (t(x) for x in w.writes[-1])
    out = torch.empty_like(q)
    M = w.query_tokens
    need = pkv.prefill_workspace_size(w.S, M, w.H, w.H_kv, w.D, w.block_size, w.max_context_len,
                                      1, 1, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    def attn():
        pkv.paged_attention_prefill(out, q, kc, vc, tables, lens, w.max_context_len, w.scale,
                                    workspace=ws)

    def step():
        pkv.paged_kv_cache_write(key, value, kc, vc, slots)
        attn()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    step_ms, attn_ms = timed(step), timed(attn)
    flops = prefill_flops(w.context_lens, M, w.H, w.D)
    kv, _ = kv_bytes(w)   # each sequence's K and V read once
    tflops = flops / (attn_ms * 1e-3) / 1e12
    return {"workload": w.name, "seqs": w.S, "chunk_tokens": M, "q_heads": w.H,
            "kv_heads": w.H_kv, "head_size": w.D, "block_size": w.block_size,
            "context": int(w.max_context_len), "workspace_bytes": need,
            "flops_per_step": flops, "ms_per_step": round(step_ms, 5),
            "tokens_per_s": round(w.S * M / (step_ms * 1e-3), 1),
            "attention_ms": round(attn_ms, 5),
            "kv_bytes": kv,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic(w.name, PREFILL_SOURCES),
                         "kernel": "tiled prefill kernel",
                         "kernel_sources": kernel_source_hash(PREFILL_SOURCES)}}


def read_once_bench(pkv, torch, w, out, q, kc, vc, ks, vs, tables, lens, unique_bytes, reps):
    """Times paged_attention_decode_shared_prefix on the shared-prefix
    workload: the prefix once per KV head for all sequences, each sequence's
    suffix, and the merge (three launches), K calls back to back."""
    prefix = w.shared_blocks * w.block_size
    qc, cc = pkv.dtype_code(q), pkv.dtype_code(kc)
    need = pkv.shared_prefix_workspace_size(w.S, w.H, w.H_kv, w.D, w.block_size,
                                            w.max_context_len, prefix, qc, cc, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=q.device)

    def call():
        pkv.paged_attention_decode_shared_prefix(out, q, kc, vc, tables, lens, w.max_context_len,
                                                 w.scale, prefix, ks, vs, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"prefix_tokens": prefix, "ms_per_call": round(ms, 5),
            "GB_per_s_unique": round(unique_bytes / (ms * 1e-3) / 1e9, 1),
            "note": "decode of the same batch (prefix pass + suffix partitions + reduce); "
                    "compare with kernel_ms decode_partitions + decode_reduce"}


def beam_fork_bench(pkv, torch, name, reps):
    """Times one multi-query step over forked tables (paged_kv_cache_write of
    each beam's query tokens, then paged_attention_prefill) on a synthetic
    beam-search batch.  Bytes count each distinct (block, KV head) tile once:
    the prompt blocks the beams share are read from HBM once."""
    import workloads
    w = workloads.make_beam_fork(name)
    dev = torch.device("cuda:0")

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    q, kc, vc = t(w.q), t(w.key_cache), t(w.value_cache)
    tables, lens = t(w.block_tables), t(w.context_lens)
    key, value, slots = (t(x) for x in w.writes[-1])
    out = torch.empty_like(q)
    M = w.query_tokens
    need = pkv.prefill_workspace_size(w.S, M, w.H, w.H_kv, w.D, w.block_size, w.max_context_len,
                                      1, 1, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)

    def attn():
        pkv.paged_attention_prefill(out, q, kc, vc, tables, lens, w.max_context_len, w.scale,
                                    workspace=ws)

    def step():
        pkv.paged_kv_cache_write(key, value, kc, vc, slots)
        attn()

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    step_ms, attn_ms = timed(step), timed(attn)
    unique, nblocks = kv_bytes(w)
    logical = int(np.sum(w.context_lens)) * w.H_kv * w.D * 2 * 2
    gbs = unique / (attn_ms * 1e-3) / 1e9
    return {"workload": w.name, "beams": w.S, "query_tokens_per_beam": M, "q_heads": w.H,
            "kv_heads": w.H_kv, "head_size": w.D, "block_size": w.block_size,
            "context": int(w.max_context_len), "kv_bytes_unique": unique,
            "kv_bytes_logical": logical, "ms_per_step": round(step_ms, 5),
            "attention_ms": round(attn_ms, 5),
            "beam_tokens_per_s": round(w.S * M / (step_ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "kernel": "decode kernel, multi-token mode (unique bytes)"}}


def cpu_baseline_for(w, writes, budget):
    """The oracle first performs the workload's writes itself (untimed), so it
    decodes the same cache state the GPU step decodes."""
    import oracle
    kc, vc, ks, vs = w.key_cache, w.value_cache, w.key_scale, w.value_scale
    for k, v, s in w.writes:
        if w.cache_dtype == "fp8":
            kc, vc, ks, vs = oracle.paged_kv_cache_write(k, v, kc, vc, s, w.block_size, ks, vs)
        else:
            kc, vc = oracle.paged_kv_cache_write(k, v, kc, vc, s, w.block_size)
    w = workloads_replace(w, key_cache=kc, value_cache=vc, key_scale=ks, value_scale=vs)
    return cpu_baseline(w, budget)


def workloads_replace(w, **kw):
    import workloads
    return workloads.Workload(**{**w.__dict__, **kw})


if __name__ == "__main__":
    main()
