"""Benchmark the paged-decode hot path on one MI355X and print ONE JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 7b-decode-bf16]

A step is the whole hot path over one batch: the write of each sequence's
newest token into its paged slot, then the decode over the whole context.
With bf16 queries and cache it is one call, paged_attention_decode_write (the
write inside the decode's launch, bit for bit the two calls' result; the two
calls are timed beside it as step_two_calls); otherwise paged_kv_cache_write,
then paged_attention_decode.  The decode is one launch when every context
spans at most 4 partitions (the decode kernel merges the partials itself),
else the partition kernel and the split reduce.  Inputs are seeded synthetic
tensors already resident in HBM.  Every GPU figure is a per-iteration HIP-event time with the MALL (256 MB)
and L2s flushed before the iteration by writing a 512 MiB buffer outside the
events; the median (with p10/p90) over K iterations is reported, and
back-to-back warm times beside it.

  value        algorithmic KV bytes the decode reads per step / median step
               time (GB/s) on the headline workload;
  roofline     the decode kernel's algorithmic bytes over its launch time
               (launches back to back, as rocprofv3 reports them), against the
               8 TB/s HBM peak;
  workloads    the 32K-context, shared-prefix and FP8 workloads measured the
               same way, each with its own roofline;
  ceiling_gbs  a streaming read of 1 GiB (and 4 KiB- and 2 KiB-tile gathers) by the
               library's probe kernels: what HBM delivers to a plain read;
  cpu_baseline the CPU oracle (float64 NumPy, untuned) on a bounded sample of
               the headline workload, on every core of this process's CPU share
               (one single-threaded worker per core) and on one thread.
Beside them: block copy / swap, a chunked-prefill step and a multi-query step
over forked tables.
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
             "shared-prefix-bf16": 4, "fp8-kv": 5, "shared-prefix-long-bf16": 6}
DEFAULT_WORKLOAD = "7b-decode-bf16"
DEFAULT_ALSO = "32k-gqa-bf16,shared-prefix-bf16,fp8-kv,shared-prefix-long-bf16"
CPU_SHARE = 16   # host cores one GPU's jobs may use at most
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
    ap.add_argument("--prefill-also", default="prefill-chunk-gqa-fp8",
                    help="comma-separated further chunked-prefill workloads ('none': skip)")
    ap.add_argument("--beam-fork", default="beam-fork-gqa-bf16",
                    help="multi-query step over forked tables timed beside the decode step "
                         "('none': skip)")
    ap.add_argument("--no-block-copy", action="store_true",
                    help="skip the block copy / swap measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of each oracle leg (one thread, all cores)")
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated decode workloads measured beside the headline one "
                         "('none': skip)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="MiB written before each timed iteration to evict the MALL (0: none)")
    ap.add_argument("--flush-mode", default="write+read",
                    choices=["write+read", "write", "read", "none"],
                    help="how the MALL is flushed before each timed iteration")
    ap.add_argument("--no-probe", dest="probe", action="store_false",
                    help="skip the HBM read / gather ceiling probes")
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


# ----------------------------------------------------------- CPU oracle

_CPU_W = None     # the workload the forked oracle workers decode (inherited)


def _oracle_one(i):
    """The oracle's decode of sequence i of _CPU_W (one sequence, every head)."""
    import oracle
    w = _CPU_W
    oracle.paged_attention_decode(w.q[i:i + 1], w.key_cache, w.value_cache,
                                  w.block_tables[i:i + 1], w.context_lens[i:i + 1], w.scale,
                                  w.block_size, w.key_scale, w.value_scale)


def _oracle_worker(args):
    """Decode sequences first, first + step, .. of _CPU_W with one BLAS thread
    until budget_s seconds have passed; returns (sequences, KV bytes, busy s)."""
    first, step, budget_s = args
    from threadpoolctl import threadpool_limits
    w = _CPU_W
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[w.cache_dtype]
    done = nbytes = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < budget_s:
            for i in range(first, w.S, step):
                _oracle_one(i)
                done += 1
                nbytes += int(w.context_lens[i]) * w.H_kv * w.D * elem * 2
                if time.perf_counter() - t0 >= budget_s:
                    break
    return done, nbytes, time.perf_counter() - t0


def cpu_baseline(w, budget_s):
    """The oracle as it stands (float64 NumPy, untuned), on a bounded sample of
    the workload: one host thread, then one single-threaded worker process per
    core of this process's CPU share, each decoding its own sequences until
    budget_s.  Runs before anything touches the GPU (the workers are forked)."""
    import multiprocessing as mp
    global _CPU_W
    _CPU_W = w
    affinity = len(os.sched_getaffinity(0))
    cores = max(1, min(affinity, CPU_SHARE))
    one_n, one_b, one_t = _oracle_worker((0, 1, budget_s))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        parts = pool.map(_oracle_worker, [(k, cores, budget_s) for k in range(cores)])
    wall = time.perf_counter() - t0
    n_all = sum(p[0] for p in parts)
    b_all = sum(p[1] for p in parts)
    return {"value": round(b_all / wall / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"float64 numpy oracle decode of {w.name}: {n_all} sequence decodes "
                      f"({n_all / w.S:.2f} passes over the {w.S} sequences, "
                      f"{b_all / 1e6:.0f} MB of KV) in {wall:.1f} s on {cores} worker processes "
                      f"with one BLAS thread each (os.sched_getaffinity: {affinity} cores; "
                      f"at most {CPU_SHARE} used)",
            "seq_heads_per_s": round(n_all * w.H / wall, 1),
            "single_thread": {"value": round(one_b / one_t / 1e9, 4), "unit": "GB/s",
                              "cores": 1, "sequences": one_n,
                              "seq_heads_per_s": round(one_n * w.H / one_t, 1),
                              "seconds": round(one_t, 1)}}


def oracle_state(w):
    """The workload after its writes, done by the oracle (so the CPU decodes
    the cache state the GPU step decodes)."""
    import oracle
    kc, vc, ks, vs = w.key_cache, w.value_cache, w.key_scale, w.value_scale
    for k, v, s in w.writes:
        if w.cache_dtype == "fp8":
            kc, vc, ks, vs = oracle.paged_kv_cache_write(k, v, kc, vc, s, w.block_size, ks, vs)
        else:
            kc, vc = oracle.paged_kv_cache_write(k, v, kc, vc, s, w.block_size)
    return workloads_replace(w, key_cache=kc, value_cache=vc, key_scale=ks, value_scale=vs)


# ------------------------------------------------------------ GPU timing

def progress(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "p10": round(float(np.percentile(a, 10)), 5),
            "p90": round(float(np.percentile(a, 90)), 5), "mean": round(float(a.mean()), 5),
            "n": int(a.size)}


class Timer:
    """Per-iteration HIP events on torch's current stream (the stream the
    library launches on), with the MALL flushed before each iteration.

    Flush modes: "write+read" (default) writes flush_mib MiB and then reads a
    second buffer of the same size, so the 256 MB MALL and the L2s hold only
    clean lines of that buffer when the events start; "write" only writes
    (the dirty lines it leaves are written back while the timed kernel runs,
    which slows even a plain read); "read" only reads."""

    def __init__(self, torch, flush_mib, mode="write+read"):
        self.torch = torch
        self.mode = mode
        self.flush = self.flush_rd = None
        if flush_mib > 0 and mode != "none":
            if "write" in mode:
                self.flush = torch.empty(flush_mib << 20, dtype=torch.uint8, device="cuda")
            if "read" in mode:
                self.flush_rd = torch.ones((flush_mib << 20) // 4, dtype=torch.float32,
                                           device="cuda")
                self.sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def _flush(self, i):
        if self.flush is not None:
            self.flush.fill_(i & 0xFF)
        if self.flush_rd is not None:
            import paged_kv_cache_370_amd as pkv
            pkv.hbm_read_probe(self.flush_rd, self.sink)

    def flushed(self, fn, iters, before=None):
        """fn timed alone in each of iters iterations; before (untimed) and the
        flush (a 512 MiB write, evicting the 256 MB MALL and the L2s) run
        first, outside the events."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        torch.cuda.synchronize()
        for i in range(iters):
            if before is not None:
                before()
            self._flush(i)
            ev[i][0].record()
            fn()
            ev[i][1].record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def warm(self, fn, iters):
        """Mean ms of iters back-to-back calls between two events (caches
        warm, no flush)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters


def to_device(torch, a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def measure_decode(pkv, torch, timer, w, ps, steps, warmup, traffic_key):
    """One decode workload on the GPU: the step (write of the step's tokens +
    paged_attention_decode) and the decode call alone, and when the call is
    two launches its partition kernel alone, each with flushed per-iteration
    events; roofline of the decode kernel on the workload's algorithmic
    bytes."""
    t = lambda a: to_device(torch, a)
    total_bytes, nblocks = kv_bytes(w)
    q = t(w.q)
    kc, vc = t(w.key_cache), t(w.value_cache)
    ks = t(w.key_scale) if w.key_scale is not None else None
    vs = t(w.value_scale) if w.value_scale is not None else None
    tables, lens = t(w.block_tables), t(w.context_lens)
    writes = [(t(k), t(v), t(s)) for k, v, s in w.writes]
    out = torch.empty_like(q)
    qc, cc = pkv.dtype_code(q), pkv.dtype_code(kc)
    P = pkv.decode_partition_size(w.S, w.H, w.H_kv, w.D, w.block_size, w.max_context_len, qc,
                                  cc, ps)
    NP = -(-w.max_context_len // P)
    # paged_attention_decode is one launch when no context needs a merge, or
    # when the matrix-core kernel merges them itself (bf16 queries, 2 to 4
    # partitions per context, partitions of at most 256 blocks)
    one_launch = NP == 1 or (qc == pkv.PKV_BF16 and NP <= 4 and P // w.block_size <= 256)
    ws_bytes = pkv.decode_workspace_size(w.S, w.H, w.H_kv, w.D, w.block_size,
                                         w.max_context_len, qc, cc, ps)
    dws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")  # counters start at 0
    wws_bytes = pkv.write_workspace_size(max(len(x[2]) for x in writes), w.H_kv, w.num_blocks, cc)
    wws = torch.zeros(wws_bytes, dtype=torch.uint8, device="cuda") if wws_bytes else None

    res = {"workload": w.name, "seqs": w.S, "q_heads": w.H, "kv_heads": w.H_kv,
           "head_size": w.D, "block_size": w.block_size, "cache": w.cache_dtype,
           "max_context": w.max_context_len,
           "mean_context": round(float(np.mean(w.context_lens)), 1), "partition_size": P,
           "partitions": NP, "decode_launches": 1 if one_launch else 2,
           "kv_bytes_per_step": total_bytes, "kv_blocks_read": nblocks}

    # Setup writes (the FP8 bulk write of positions 0..n-2) are not part of a
    # step.  Their first run loads the kernels; the timed second run writes
    # the same tokens to the same slots with the same result.
    setup, step_write = writes[:-1], writes[-1]
    if setup:
        def bulk():
            for k, v, s in setup:
                pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)
        bulk()
        setup_ms = timer.flushed(bulk, 1)[0]
        setup_bytes = sum(x[0].numel() * x[0].element_size() * 2 for x in setup)
        res["setup_write"] = {"ms": round(setup_ms, 3), "source_bytes": setup_bytes,
                              "GB_per_s_source_read": round(setup_bytes / setup_ms / 1e6, 1)}
        if w.cache_dtype == "fp8":
            # the source is read twice (amax, then encode), one byte written per element
            codes = sum(x[0].numel() * 2 for x in setup)
            res["setup_write"]["GB_per_s_hbm"] = round((2 * setup_bytes + codes) / setup_ms / 1e6,
                                                       1)

    def write():
        k, v, s = step_write
        pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)

    def partitions():
        pkv.paged_attention_decode_partitions(out, q, kc, vc, tables, lens, w.max_context_len,
                                              w.scale, ks, vs, partition_size=ps, workspace=dws)

    def reduce():
        pkv.paged_attention_decode_reduce(out, lens, w.H_kv, w.block_size, w.max_context_len, cc,
                                          partition_size=ps, workspace=dws)

    def decode():
        pkv.paged_attention_decode(out, q, kc, vc, tables, lens, w.max_context_len, w.scale, ks,
                                   vs, partition_size=ps, workspace=dws)

    def two_calls():
        write()
        decode()

    # bf16 queries and cache, one new token per sequence at its newest
    # position: the step is paged_attention_decode_write (the write inside
    # the decode's launch; bit for bit the two calls' result)
    k_new, v_new, s_new = step_write
    newest = np.array([w.block_tables[i, (n - 1) // w.block_size] * w.block_size
                       + (n - 1) % w.block_size if n > 0 else -1
                       for i, n in enumerate(w.context_lens)])
    fused = (qc == pkv.PKV_BF16 and cc == pkv.PKV_BF16 and len(w.writes[-1][2]) == w.S
             and np.array_equal(w.writes[-1][2], newest))

    def step_fused():
        pkv.paged_attention_decode_write(out, q, k_new, v_new, kc, vc, s_new, tables, lens,
                                         w.max_context_len, w.scale, partition_size=ps,
                                         workspace=dws)

    step = step_fused if fused else two_calls
    res["step"] = ("paged_attention_decode_write (write fused into the decode launch)" if fused
                   else "paged_kv_cache_write + paged_attention_decode")
    for _ in range(warmup):
        step()
    step_ms = timer.flushed(step, steps)
    decode_ms = timer.flushed(decode, steps, before=write)
    warm = {"step": round(timer.warm(step, steps), 5),
            "decode": round(timer.warm(decode, steps), 5),
            "write": round(timer.warm(write, steps), 5)}
    st, dc = stats(step_ms), stats(decode_ms)
    flushed = {"step": st, "decode": dc}
    if fused:  # the same step as two calls, for comparison
        flushed["step_two_calls"] = stats(timer.flushed(two_calls, steps))
        warm["step_two_calls"] = round(timer.warm(two_calls, steps), 5)
    if one_launch:
        kernel_ms, kernel_flushed = warm["decode"], dc
    else:
        pt = stats(timer.flushed(partitions, steps, before=write))
        warm["decode_partitions"] = round(timer.warm(partitions, steps), 5)
        warm["decode_reduce"] = round(timer.warm(reduce, steps), 5)
        flushed["decode_partitions"] = pt
        kernel_ms, kernel_flushed = warm["decode_partitions"], pt
    res.update({
        "ms_per_step": st["median"],
        "GB_per_s": round(total_bytes / (st["median"] * 1e-3) / 1e9, 2),
        "pct_hbm_peak": round(100.0 * total_bytes / (st["median"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "seq_heads_per_s": round(w.S * w.H / (st["median"] * 1e-3), 1),
        "flushed_ms": flushed,
        "decode_GB_per_s": round(total_bytes / (dc["median"] * 1e-3) / 1e9, 2),
        "decode_pct_hbm_peak": round(100.0 * total_bytes / (dc["median"] * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 2),
        "warm_ms_back_to_back": warm,
    })
    # The kernel's own launch duration: K launches back to back between two
    # events (what rocprofv3 reports per launch); an event pair around a
    # single flushed launch adds its marker packets (a few us) to the kernel.
    # Flushing does not change the kernel's time (the 256 MB MALL cannot hold
    # a ~1 GB working set), so the two differ by the event packets only.
    achieved = total_bytes / (kernel_ms * 1e-3) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                       "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                       "traffic": recorded_traffic(traffic_key),
                       "kernel": ("decode kernel (partials merged in the kernel)"
                                  if one_launch and NP > 1 else
                                  "decode kernel" if one_launch else "decode partition kernel"),
                       "kernel_us": round(kernel_ms * 1e3, 2),
                       "flushed_event_us": {"mean": round(kernel_flushed["mean"] * 1e3, 2),
                                            "median": round(kernel_flushed["median"] * 1e3, 2)},
                       "kernel_sources": kernel_source_hash()}
    if w.shared_blocks > 0:
        res["read_once"] = read_once_bench(pkv, torch, timer, w, out, q, kc, vc, ks, vs, tables,
                                           lens, total_bytes, steps)
    return res


def probe_bench(pkv, torch, timer, iters, gib=1):
    """Practical HBM ceiling on this device: a streaming read of a 1 GiB
    buffer, and gathers of whole tiles in random order over the same buffer:
    4 KiB (one (block, KV head) tile of a bf16 cache at bs 16, D 128) and
    2 KiB (bf16 at bs 8, or FP8 at bs 16), flushed per iteration like the
    decode timings."""
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(11)
    pkv.hbm_read_probe(buf, sink)
    rd = stats(timer.flushed(lambda: pkv.hbm_read_probe(buf, sink), iters))
    res = {"bytes": nbytes, "read_GB_per_s": round(nbytes / (rd["median"] * 1e-3) / 1e9, 1),
           "read_ms": rd}
    for tile, key in ((4096, "gather_4KiB_tiles"), (2048, "gather_2KiB_tiles")):
        ids = rng.permutation(nbytes // tile).astype(np.int32)
        assert ids.min() >= 0 and (int(ids.max()) + 1) * tile <= nbytes   # every tile inside buf
        tiles = torch.from_numpy(ids).cuda()
        pkv.hbm_gather_probe(buf, tiles, tile, sink)
        ga = stats(timer.flushed(lambda: pkv.hbm_gather_probe(buf, tiles, tile, sink), iters))
        res[key + "_GB_per_s"] = round(nbytes / (ga["median"] * 1e-3) / 1e9, 1)
        res[key + "_ms"] = ga
        del tiles
    res["gather_ms"] = res["gather_4KiB_tiles_ms"]
    return res


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib)
        return

    import workloads

    cfg = WORKLOADS[args.workload]
    t0 = time.perf_counter()
    w = workloads.make_config(cfg)
    gen_s = time.perf_counter() - t0
    ps = w.partition_size if args.partition_size < 0 else args.partition_size

    # The CPU oracle runs first, before anything touches the GPU.
    cpu = None
    if not args.no_cpu_baseline:
        progress(f"CPU oracle baseline on {w.name}")
        cpu = cpu_baseline(oracle_state(w), args.cpu_seconds)

    import torch
    import paged_kv_cache_370_amd as pkv
    pkv.load()
    timer = Timer(torch, args.flush_mib, args.flush_mode)
    progress(f"decode {w.name}")
    head = measure_decode(pkv, torch, timer, w, ps, args.steps, args.warmup, args.workload)
    del w

    result = {
        "metric": METRIC,
        "value": head["GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8e4m3-kv/bf16-q"}[head["cache"]],
        "data": "synthetic",
        "config": {k: head[k] for k in ("workload", "seqs", "q_heads", "kv_heads", "head_size",
                                        "block_size", "max_context", "mean_context",
                                        "partition_size", "partitions", "decode_launches",
                                        "kv_bytes_per_step", "kv_blocks_read")},
        "pct_hbm_peak": head["pct_hbm_peak"],
        "seq_heads_per_s": head["seq_heads_per_s"],
        "timing": (f"median of per-iteration HIP events; before each iteration, outside the "
                   f"events, the MALL is flushed ({args.flush_mode}, {args.flush_mib} MiB)"),
        "step": head["step"] + (" (one launch" + (", partials merged in the decode kernel)"
                                                  if head["partitions"] > 1 else ")")
                                if head["decode_launches"] == 1 else
                                " (partition kernel + reduce)"),
        "flushed_ms": head["flushed_ms"],
        "decode_GB_per_s": head["decode_GB_per_s"],
        "decode_pct_hbm_peak": head["decode_pct_hbm_peak"],
        "warm_ms_back_to_back": head["warm_ms_back_to_back"],
        "roofline": head["roofline"],
        "input_generation_s": round(gen_s, 2),
    }
    for k in ("setup_write", "read_once"):
        if k in head:
            result[k] = head[k]
    if args.probe:
        progress("HBM read / gather probes")
        result["ceiling"] = probe_bench(pkv, torch, timer, args.steps)
        result["ceiling_gbs"] = result["ceiling"]["read_GB_per_s"]
    extra = [x for x in args.also.split(",") if x and x != "none" and x != args.workload]
    if extra:
        result["workloads"] = {}
    for name in extra:
        progress(f"decode {name}")
        wx = workloads.make_config(WORKLOADS[name])
        result["workloads"][name] = measure_decode(pkv, torch, timer, wx, wx.partition_size,
                                                   args.steps, args.warmup, name)
        del wx
        torch.cuda.empty_cache()
    if not args.no_block_copy:
        progress("block copy / swap")
        result["block_copy"] = block_copy_bench(pkv, torch, args.steps)
    if args.prefill != "none":
        progress(f"prefill {args.prefill}")
        result["prefill"] = prefill_bench(pkv, torch, args.prefill, args.steps)
        extra = [x for x in args.prefill_also.split(",") if x and x not in ("none", args.prefill)]
        if extra:
            result["prefill_workloads"] = {}
        for name in extra:
            progress(f"prefill {name}")
            result["prefill_workloads"][name] = prefill_bench(pkv, torch, name, args.steps)
            torch.cuda.empty_cache()
    if args.beam_fork != "none":
        progress(f"beams over forked tables {args.beam_fork}")
        result["beam_fork"] = beam_fork_bench(pkv, torch, args.beam_fork, args.steps)
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def block_copy_bench(pkv, torch, reps, pool_blocks=4096, copy_pairs=1024, swap_pairs=256):
    """Times paged_kv_block_copy on a pool of the 7B-class shape (bf16, 32 KV
    heads, bs 16, D 128: 256 KiB per block with K and V): copy_pairs random
    blocks into a second device pool (the copy-on-write shape: HBM read and
    write), and swap_pairs blocks out to a pinned host pool and back in
    (PCIe).  Bytes count the K and V tiles moved once."""
    rng = np.random.default_rng(7)
    dev = torch.device("cuda")
    shape = (pool_blocks, 32, 16, 128)
    kc = torch.randn(shape, device=dev).to(torch.bfloat16)
    vc = torch.randn(shape, device=dev).to(torch.bfloat16)
    block_bytes = 2 * kc[0].numel() * kc.element_size()

    def pool(blocks, pinned=False):
        if pinned:
            mk = lambda: torch.empty((blocks,) + shape[1:], dtype=kc.dtype, pin_memory=True)
        else:
            mk = lambda: torch.empty((blocks,) + shape[1:], dtype=kc.dtype, device=dev)
        return (mk(), mk())

    def timed(src, dst, pairs):
        call = lambda: pkv.paged_kv_block_copy(src[0], src[1], dst[0], dst[1], pairs)
        call()
        us = stats([1e3 * x for x in Timer(torch, 0).flushed(call, reps)])["median"]
        n = pairs.shape[0]
        return {"pairs": n, "us": round(us, 2), "bytes_moved": n * block_bytes,
                "GB_per_s": round(n * block_bytes / (us * 1e-6) / 1e9, 1)}

    src = (kc, vc)
    n = min(copy_pairs, pool_blocks)
    pairs = torch.from_numpy(np.stack([rng.choice(pool_blocks, n, replace=False),
                                       rng.permutation(n)], axis=1).astype(np.int32)).to(dev)
    out = {"block_bytes": block_bytes, "device_copy": timed(src, pool(n), pairs)}
    m = min(swap_pairs, pool_blocks)
    host = pool(m, pinned=True)
    out_pairs = torch.from_numpy(np.stack([rng.choice(pool_blocks, m, replace=False),
                                           rng.permutation(m)], axis=1).astype(np.int32)).to(dev)
    out["swap_out"] = timed(src, host, out_pairs)
    in_pairs = torch.from_numpy(np.stack([rng.permutation(m), rng.permutation(m)],
                                         axis=1).astype(np.int32)).to(dev)
    out["swap_in"] = timed(host, pool(m), in_pairs)
    out["note"] = ("median of per-call events, no flush; device_copy moves each byte HBM to HBM "
                   "(read and written: 2x the bytes in HBM traffic); swaps cross PCIe once")
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
    ks = t(w.key_scale) if w.key_scale is not None else None
    vs = t(w.value_scale) if w.value_scale is not None else None
    tables, lens = t(w.block_tables), t(w.context_lens)
    writes = [tuple(t(x) for x in wr) for wr in w.writes]
    key, value, slots = writes[-1]
    out = torch.empty_like(q)
    M = w.query_tokens
    cc = pkv.dtype_code(kc)
    need = pkv.prefill_workspace_size(w.S, M, w.H, w.H_kv, w.D, w.block_size, w.max_context_len,
                                      1, cc, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    wws_bytes = pkv.write_workspace_size(max(len(x[2]) for x in writes), w.H_kv, w.num_blocks, cc)
    wws = torch.zeros(wws_bytes, dtype=torch.uint8, device=dev) if wws_bytes else None
    # FP8 caches: the positions before the chunk are written once, untimed
    for k, v, s in writes[:-1]:
        pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)

    def attn():
        pkv.paged_attention_prefill(out, q, kc, vc, tables, lens, w.max_context_len, w.scale, ks,
                                    vs, workspace=ws)

    def step():
        pkv.paged_kv_cache_write(key, value, kc, vc, slots, ks, vs, workspace=wws)
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
            "cache": w.cache_dtype,
            "context": int(w.max_context_len), "workspace_bytes": need,
            "flops_per_step": flops, "ms_per_step": round(step_ms, 5),
            "tokens_per_s": round(w.S * M / (step_ms * 1e-3), 1),
            "attention_ms": round(attn_ms, 5),
            "kv_bytes": kv,
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                         "traffic": recorded_traffic(w.name, PREFILL_SOURCES),
                         "kernel": "tiled prefill kernel" + (
                             " (after the FP8 stage to bf16, timed with it)"
                             if w.cache_dtype == "fp8" else ""),
                         "kernel_sources": kernel_source_hash(PREFILL_SOURCES)}}


def read_once_bench(pkv, torch, timer, w, out, q, kc, vc, ks, vs, tables, lens, unique_bytes,
                    reps):
    """Times paged_attention_decode_shared_prefix on the shared-prefix
    workload (the prefix once per KV head for all sequences, each sequence's
    suffix, and the merge), flushed per iteration like the decode."""
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
    st = stats(timer.flushed(call, reps))
    return {"prefix_tokens": prefix, "ms_per_call": st["median"], "flushed_ms": st,
            "GB_per_s_unique": round(unique_bytes / (st["median"] * 1e-3) / 1e9, 1),
            "note": "decode of the same batch through the read-once call; compare with "
                    "flushed_ms.decode"}


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
    ks = t(w.key_scale) if w.key_scale is not None else None
    vs = t(w.value_scale) if w.value_scale is not None else None
    tables, lens = t(w.block_tables), t(w.context_lens)
    writes = [tuple(t(x) for x in wr) for wr in w.writes]
    key, value, slots = writes[-1]
    out = torch.empty_like(q)
    M = w.query_tokens
    cc = pkv.dtype_code(kc)
    need = pkv.prefill_workspace_size(w.S, M, w.H, w.H_kv, w.D, w.block_size, w.max_context_len,
                                      1, cc, 0)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    wws_bytes = pkv.write_workspace_size(max(len(x[2]) for x in writes), w.H_kv, w.num_blocks, cc)
    wws = torch.zeros(wws_bytes, dtype=torch.uint8, device=dev) if wws_bytes else None
    # FP8 caches: the positions before the chunk are written once, untimed
    for k, v, s in writes[:-1]:
        pkv.paged_kv_cache_write(k, v, kc, vc, s, ks, vs, workspace=wws)

    def attn():
        pkv.paged_attention_prefill(out, q, kc, vc, tables, lens, w.max_context_len, w.scale, ks,
                                    vs, workspace=ws)

    def step():
        pkv.paged_kv_cache_write(key, value, kc, vc, slots, ks, vs, workspace=wws)
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


def workloads_replace(w, **kw):
    import workloads
    return workloads.Workload(**{**w.__dict__, **kw})


if __name__ == "__main__":
    main()
