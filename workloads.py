"""Seeded synthetic inputs for paged KV write + PagedAttention decode.

This module only draws random numbers and lays out inputs; it performs none of
the method's arithmetic (no attention, no quantisation, no cache write).  It is
the one module that both the CPU oracle and the GPU path take their inputs
from.  Everything is numpy on the host; callers move arrays to the device.

Array conventions: float32 arrays hold fp32; uint16 arrays hold bfloat16 bit
patterns; uint8 arrays hold FP8 E4M3FN codes.

Layouts:
  q                      [S][H][D]
  key_cache, value_cache [num_blocks][H_kv][block_size][D]
  key_scale, value_scale [num_blocks][H_kv] float32 (FP8 caches only)
  block_tables           [S][max_blocks] int32
  context_lens           [S] int32 (this step's token included)
  writes                 list of (key [T][H_kv][D], value [T][H_kv][D],
                         slot_mapping [T] int32), applied in order before decode

Named workloads (sizes as the decode workloads are specified; each gets its own
seed):
  1 tiny-fp32        2 seqs (37, 80 tokens), 4 MHA heads, D 64, bs 16, pool 16
  2 7b-decode-bf16   64 seqs, U[128,2048] tokens, 32/32 heads, D 128, bs 16
  3 32k-gqa-bf16     8 seqs x 32768 tokens, 64/8 heads, D 128, bs 8
  4 shared-prefix    128 seqs, 512-token shared prefix + U[64,1024], 32/8 heads
  5 fp8-kv           256 seqs, lognormal(median 1024, sigma 1) clipped [16,8192],
                     40/8 heads, D 128, bs 16, e4m3 cache written from bf16
  6 shared-prefix-long  workload 4 with an 8192-token shared prefix: a KV head's
                     prefix (4 MiB of K and V) no longer fits the 4 MiB L2 of
                     the XCD that serves it beside the suffixes
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) samples stored as fp32 or bf16 bits; drawn in chunks."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.float32 if dtype == "f32" else np.uint16)
    chunk = 1 << 24
    for lo in range(0, total, chunk):
        hi = min(total, lo + chunk)
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        out[lo:hi] = x if dtype == "f32" else bf16_bits(x)
    return out.reshape(shape)


def _poison(dtype: str):
    return {"f32": np.float32(np.nan), "bf16": BF16_NAN, "fp8": FP8_NAN}[dtype]


def _np_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


@dataclass
class Workload:
    name: str
    S: int
    H: int
    H_kv: int
    D: int
    block_size: int
    q_dtype: str          # "f32" | "bf16"
    cache_dtype: str      # "f32" | "bf16" | "fp8"
    src_dtype: str        # dtype of the K/V handed to the write
    num_blocks: int
    q: np.ndarray
    key_cache: np.ndarray
    value_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    writes: List[Tuple[np.ndarray, np.ndarray, np.ndarray]] = field(default_factory=list)
    key_scale: Optional[np.ndarray] = None
    value_scale: Optional[np.ndarray] = None
    scale: float = 0.0
    partition_size: int = 0
    shared_blocks: int = 0
    query_tokens: int = 1

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.S else 0


def build_workload(name, S, H, H_kv, D, block_size, q_dtype, cache_dtype, lens,
                   seed, free_frac=0.1, prefix_tokens=0, fill="random",
                   layout_seed=None, partition_size=0, src_dtype=None,
                   max_blocks=None, num_blocks=None, query_tokens=1):
    """Build one seeded workload.

    query_tokens = M > 1 (a prefill chunk): q is [S][M][H][D] and the step
    write supplies the M newest positions n-M .. n-1 of every sequence
    (every n >= M); with M = 1, q is [S][H][D] and the step is position n-1.

    fill="random": the pool already holds N(0,1) K/V for positions < n-1 of
        every sequence; the step write supplies position n-1.
    fill="write":  the pool starts fully poisoned; writes supply positions
        0..n-2 (one bulk call) and then n-1 (the step call).
    fill="write-all": one write supplies positions 0..n-1.

    Token values in the write modes depend only on `seed` and the lengths, not
    on block size or placement; placement comes from `layout_seed`.
    Free blocks, unused table entries' targets and rows past n hold NaN.
    prefix_tokens > 0: the first prefix_tokens//bs blocks are one physical
    copy shared by every sequence (reference-counted sharing); the prefix
    values are then identical across sequences.
    """
    lens = np.asarray(lens, dtype=np.int64)
    assert len(lens) == S
    bs = block_size
    src_dtype = src_dtype or ("bf16" if cache_dtype == "fp8" else cache_dtype)
    rng_layout = np.random.default_rng(seed + 7919 if layout_seed is None else layout_seed)
    rng_val = np.random.default_rng(seed)

    nb = (lens + bs - 1) // bs
    assert prefix_tokens % bs == 0
    pb = prefix_tokens // bs
    if pb:
        assert np.all(lens > prefix_tokens)
    private = nb - pb
    used = pb + int(private.sum())
    if num_blocks is None:
        num_blocks = int(np.ceil(used * (1.0 + free_frac))) if free_frac else used
        num_blocks = max(num_blocks, 1)
    assert num_blocks >= used
    mb = int(max_blocks or max(1, int(nb.max()) if S else 1))

    perm = rng_layout.permutation(num_blocks).astype(np.int32)
    free_ids = perm[used:]
    tables = np.empty((S, mb), dtype=np.int32)
    fill_id = free_ids[0] if len(free_ids) else perm[0]
    tables[:] = fill_id
    cursor = pb
    for i in range(S):
        tables[i, :pb] = perm[:pb]
        k = int(private[i])
        tables[i, pb:pb + k] = perm[cursor:cursor + k]
        cursor += k

    pool_shape = (num_blocks, H_kv, bs, D)
    M = int(query_tokens)
    assert M >= 1 and (M == 1 or np.all(lens >= M))
    q = _normal(rng_val, (S, H, D) if M == 1 else (S, M, H, D), q_dtype)

    if fill == "random":
        kc = _normal(rng_val, pool_shape, cache_dtype)
        vc = _normal(rng_val, pool_shape, cache_dtype)
        poison = _poison(cache_dtype)
        if len(free_ids):
            kc[free_ids] = poison
            vc[free_ids] = poison
        for i in range(S):
            if lens[i] == 0:
                continue
            for pos in range(int(lens[i]) - M, int(nb[i]) * bs):   # the step's rows and after
                kc[tables[i, pos // bs], :, pos % bs, :] = poison
                vc[tables[i, pos // bs], :, pos % bs, :] = poison
        positions = [np.arange(n - M, n) if n > 0 else np.zeros(0, np.int64) for n in lens]
        writes = [_step_write(rng_val, tables, positions, H_kv, D, bs, src_dtype)]
    else:
        kc = np.full(pool_shape, _poison(cache_dtype), dtype=_np_dtype(cache_dtype))
        vc = np.full(pool_shape, _poison(cache_dtype), dtype=_np_dtype(cache_dtype))
        if fill == "write-all":
            groups = [[np.arange(n) for n in lens]]
        else:
            groups = [[np.arange(max(n - M, 0)) for n in lens],
                      [np.arange(n - M, n) if n > 0 else np.zeros(0, np.int64) for n in lens]]
        writes = []
        for g_idx, positions in enumerate(groups):
            if pb and g_idx == 0:
                # The shared prefix is written once, through sequence 0's table.
                positions = [p if i == 0 else p[p >= prefix_tokens] for i, p in enumerate(positions)]
            writes.append(_step_write(rng_val, tables, positions, H_kv, D, bs, src_dtype))

    ks = vs = None
    if cache_dtype == "fp8":
        ks = np.full((num_blocks, H_kv), np.nan, dtype=np.float32)
        vs = np.full((num_blocks, H_kv), np.nan, dtype=np.float32)

    return Workload(name=name, S=S, H=H, H_kv=H_kv, D=D, block_size=bs,
                    q_dtype=q_dtype, cache_dtype=cache_dtype, src_dtype=src_dtype,
                    num_blocks=num_blocks, q=q, key_cache=kc, value_cache=vc,
                    block_tables=tables, context_lens=lens.astype(np.int32),
                    writes=writes, key_scale=ks, value_scale=vs,
                    scale=float(np.float32(1.0 / np.sqrt(D))),
                    partition_size=partition_size, shared_blocks=pb, query_tokens=M)


def _step_write(rng, tables, positions, H_kv, D, bs, src_dtype):
    """New K/V rows for the given token positions and their flat slots."""
    slots = []
    for i, pos in enumerate(positions):
        pos = np.asarray(pos, dtype=np.int64)
        slots.append(tables[i, pos // bs].astype(np.int64) * bs + pos % bs)
    slot_mapping = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)
    T = len(slot_mapping)
    key = _normal(rng, (T, H_kv, D), src_dtype)
    value = _normal(rng, (T, H_kv, D), src_dtype)
    return key, value, slot_mapping


# ---------------------------------------------------------------------------
# Named workloads.  reduced=True keeps heads, head size, block size and dtypes
# but shrinks batch and lengths so the oracle finishes in seconds; the reduced
# cases still span several partitions and end on ragged tails.

def config_lengths(cfg: int, rng: np.random.Generator, reduced: bool):
    if cfg == 1:
        return np.array([37, 80])
    if cfg == 2:
        S = 6 if reduced else 64
        lo, hi = (1, 700) if reduced else (128, 2048)
        return rng.integers(lo, hi + 1, size=S)
    if cfg == 3:
        S = 2 if reduced else 8
        n = 2100 if reduced else 32768
        return np.full(S, n)
    if cfg == 4:
        S = 5 if reduced else 128
        hi = 300 if reduced else 1024
        return 512 + rng.integers(64 if not reduced else 1, hi + 1, size=S)
    if cfg == 5:
        S = 12 if reduced else 256
        z = rng.standard_normal(S)
        n = np.round(np.exp(np.log(1024.0) + z)).astype(np.int64)
        return np.clip(n, 16, 1200 if reduced else 8192)
    if cfg == 6:
        S = 5 if reduced else 128
        hi = 300 if reduced else 1024
        return LONG_PREFIX[reduced] + rng.integers(64 if not reduced else 1, hi + 1, size=S)
    raise ValueError(cfg)


# Shared prefix of workload 6 (full size, reduced).
LONG_PREFIX = {False: 8192, True: 1024}


CONFIG_NAMES = {1: "tiny-fp32", 2: "7b-decode-bf16", 3: "32k-gqa-bf16",
                4: "shared-prefix-bf16", 5: "fp8-kv", 6: "shared-prefix-long-bf16"}


def make_config(cfg: int, reduced: bool = False, seed: Optional[int] = None,
                layout_seed: Optional[int] = None) -> Workload:
    seed = cfg if seed is None else seed
    lens = config_lengths(cfg, np.random.default_rng(1000 + seed), reduced)
    name = CONFIG_NAMES[cfg] + ("-reduced" if reduced else "")
    if cfg == 1:
        return build_workload(name, 2, 4, 4, 64, 16, "f32", "f32", lens, seed,
                              num_blocks=16, fill="write-all", layout_seed=layout_seed)
    if cfg == 2:
        return build_workload(name, len(lens), 32, 32, 128, 16, "bf16", "bf16", lens, seed,
                              layout_seed=layout_seed)
    if cfg == 3:
        return build_workload(name, len(lens), 64, 8, 128, 8, "bf16", "bf16", lens, seed,
                              free_frac=0.0, partition_size=512, layout_seed=layout_seed)
    if cfg == 4:
        return build_workload(name, len(lens), 32, 8, 128, 16, "bf16", "bf16", lens, seed,
                              prefix_tokens=512, layout_seed=layout_seed)
    if cfg == 5:
        return build_workload(name, len(lens), 40, 8, 128, 16, "bf16", "fp8", lens, seed,
                              fill="write", layout_seed=layout_seed)
    if cfg == 6:
        return build_workload(name, len(lens), 32, 8, 128, 16, "bf16", "bf16", lens, seed,
                              prefix_tokens=LONG_PREFIX[reduced], layout_seed=layout_seed)
    raise ValueError(cfg)


PREFILL_CONFIGS = {
    # name: (S, M, H, H_kv, D, bs, cache, context length per sequence)
    "prefill-chunk-gqa-bf16": (4, 512, 32, 8, 128, 16, "bf16", 4096),
    "prefill-chunk-mha-bf16": (4, 512, 32, 32, 128, 16, "bf16", 4096),
    "prefill-chunk-gqa-fp8": (4, 512, 32, 8, 128, 16, "fp8", 4096),
}


def make_prefill(name: str, reduced: bool = False, seed: int = 31) -> Workload:
    """A chunked-prefill step: each sequence's newest M tokens are the chunk
    (written by the step, then attending causally to all positions before
    them).  reduced=True shrinks the context and chunk for the oracle."""
    S, M, H, H_kv, D, bs, cache, n = PREFILL_CONFIGS[name]
    if reduced:
        S, M, n = 2, 40, 300
    lens = np.full(S, n)
    return build_workload(name + ("-reduced" if reduced else ""), S, H, H_kv, D, bs, "bf16",
                          cache, lens, seed, free_frac=0.05,
                          fill="write" if cache == "fp8" else "random", query_tokens=M)


BEAM_CONFIGS = {
    # name: (prompts, beams, prompt length, tokens generated since the fork,
    #        query tokens per beam, H, H_kv, D, bs)
    "beam-fork-gqa-bf16": (16, 4, 2001, 64, 4, 32, 8, 128, 16),
}


def make_beam_fork(name: str = "beam-fork-gqa-bf16", reduced: bool = False,
                   seed: int = 41) -> Workload:
    """Beams forked from shared prompts (beam-search style), several query
    tokens per beam.

    Each of P prompts of L tokens is forked into B beams.  The beams of a
    prompt reference the prompt's whole blocks (one physical copy); the
    prompt's last, partial block was copied per beam when the beam first
    wrote into it (copy-on-write), so its first L % bs rows hold the prompt's
    values in every beam's private copy.  Each beam then holds T tokens of
    its own, and this step's M query tokens (positions n-M .. n-1, written by
    the step) end the sequence: n = L + T + M.  Free blocks and rows past n
    hold NaN.  q is [P*B][M][H][D]."""
    P, B, L, T, M, H, H_kv, D, bs = BEAM_CONFIGS[name]
    if reduced:
        P, L, T = 2, 70, 9
    rng_layout = np.random.default_rng(seed + 7919)
    rng = np.random.default_rng(seed)
    S = P * B
    n = L + T + M
    nb = -(-n // bs)
    shared = L // bs                      # whole prompt blocks
    private = nb - shared                 # the copied partial block and the beam's own
    used = P * shared + S * private
    num_blocks = int(np.ceil(used * 1.05))
    perm = rng_layout.permutation(num_blocks).astype(np.int32)
    tables = np.full((S, nb), perm[-1], dtype=np.int32)
    cur = 0
    for p in range(P):
        ids = perm[cur:cur + shared]
        cur += shared
        for b in range(B):
            tables[p * B + b, :shared] = ids
    for i in range(S):
        tables[i, shared:] = perm[cur:cur + private]
        cur += private
    kc = np.full((num_blocks, H_kv, bs, D), _poison("bf16"), dtype=np.uint16)
    vc = np.full((num_blocks, H_kv, bs, D), _poison("bf16"), dtype=np.uint16)
    q = _normal(rng, (S, M, H, D), "bf16")
    for p in range(P):
        pk = _normal(rng, (L, H_kv, D), "bf16")
        pv = _normal(rng, (L, H_kv, D), "bf16")
        for b in range(B):
            i = p * B + b
            for pos in range(L):
                kc[tables[i, pos // bs], :, pos % bs] = pk[pos]
                vc[tables[i, pos // bs], :, pos % bs] = pv[pos]
    for i in range(S):
        bk = _normal(rng, (T, H_kv, D), "bf16")
        bv = _normal(rng, (T, H_kv, D), "bf16")
        for t in range(T):
            pos = L + t
            kc[tables[i, pos // bs], :, pos % bs] = bk[t]
            vc[tables[i, pos // bs], :, pos % bs] = bv[t]
    writes = [_step_write(rng, tables, [np.arange(n - M, n)] * S, H_kv, D, bs, "bf16")]
    return Workload(name=name + ("-reduced" if reduced else ""), S=S, H=H, H_kv=H_kv, D=D,
                    block_size=bs, q_dtype="bf16", cache_dtype="bf16", src_dtype="bf16",
                    num_blocks=num_blocks, q=q, key_cache=kc, value_cache=vc,
                    block_tables=tables, context_lens=np.full(S, n, dtype=np.int32),
                    writes=writes, scale=float(np.float32(1.0 / np.sqrt(D))),
                    query_tokens=M)


def unshare_blocks(w: Workload) -> Workload:
    """Twin of a workload in which every sequence owns a private copy (same
    bytes) of each block that more than one table references."""
    counts = {}
    nbs = [-(-int(n) // w.block_size) for n in w.context_lens]
    for i in range(w.S):
        for b in w.block_tables[i, :nbs[i]]:
            counts[int(b)] = counts.get(int(b), 0) + 1
    tables = w.block_tables.copy()
    extra_k, extra_v = [], []
    nxt = w.num_blocks
    for i in range(w.S):
        for j in range(nbs[i]):
            b = int(w.block_tables[i, j])
            if counts[b] > 1:
                extra_k.append(w.key_cache[b])
                extra_v.append(w.value_cache[b])
                tables[i, j] = nxt
                nxt += 1
    kc = np.concatenate([w.key_cache, np.stack(extra_k)]) if extra_k else w.key_cache
    vc = np.concatenate([w.value_cache, np.stack(extra_v)]) if extra_v else w.value_cache
    return Workload(**{**w.__dict__, "name": w.name + "-unshared", "num_blocks": nxt,
                       "key_cache": kc, "value_cache": vc, "block_tables": tables,
                       "shared_blocks": 0})


def duplicate_shared_blocks(w: Workload) -> Workload:
    """Twin of a shared-prefix workload: each sequence gets private copies of
    the shared blocks (same bytes), appended to the pool."""
    pb = w.shared_blocks
    assert pb > 0 and w.writes and w.cache_dtype != "fp8"
    shared_ids = w.block_tables[0, :pb].copy()
    extra = w.S * pb
    kc = np.concatenate([w.key_cache, np.repeat(w.key_cache[shared_ids][None], w.S, 0).reshape(
        (extra,) + w.key_cache.shape[1:])])
    vc = np.concatenate([w.value_cache, np.repeat(w.value_cache[shared_ids][None], w.S, 0).reshape(
        (extra,) + w.value_cache.shape[1:])])
    tables = w.block_tables.copy()
    for i in range(w.S):
        tables[i, :pb] = w.num_blocks + i * pb + np.arange(pb)
    return Workload(**{**w.__dict__, "name": w.name + "-duplicated", "num_blocks": w.num_blocks + extra,
                       "key_cache": kc, "value_cache": vc, "block_tables": tables,
                       "shared_blocks": 0})
