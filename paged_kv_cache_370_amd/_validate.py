"""Host-side checks of the caller's contract, run before a call when the
environment sets PAGEDKV_DEBUG=1 (any value but "" or "0").

The library checks sizes, dtypes and pointers itself, but the contents of
block tables, context lengths and slot mappings are the caller's contract and
are not checked on the device (an id outside the pool is an out-of-bounds
access).  Shared blocks with reference counts and copy-on-write are where such
bugs come from (page "vLLM的诞生背景：大模型推理的痛点与PagedAttention的破局",
limitations paragraph), so in debug mode the binding copies those arrays to the
host (a synchronising copy) and raises ContractError naming the first
violation before anything is enqueued:

  * context lengths: 0 <= n <= max_context_len and n <= max_blocks * block_size
    (and n >= M for a chunk of M query tokens);
  * block tables: the entries a sequence uses (the first ceil(n / bs)) name
    blocks of the pool, 0 <= id < num_blocks;
  * slot mappings: every non-negative slot lies in the pool and no slot repeats;
  * shared-prefix calls: every table begins with the same prefix blocks;
  * block copies: ids inside their pools, distinct destinations, and no
    destination that is also a source when both pools are one;
  * workspaces handed in by the caller: the leading counters (the 4 KiB
    work-queue header and the partition arrival counters) are zero.
"""

import os

import numpy as np

SCHED_BYTES = 4096


class ContractError(ValueError):
    """The arguments break the caller's contract of the C ABI."""


def enabled() -> bool:
    return os.environ.get("PAGEDKV_DEBUG", "") not in ("", "0")


def _host(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t
    return t.detach().cpu().numpy()


def _first(mask) -> int:
    return int(np.flatnonzero(mask)[0])


def check_decode(where, context_lens, block_tables, num_blocks, block_size, max_context_len,
                 query_tokens=1):
    """Lengths within the launch's bound and the table, and every used table
    entry inside the pool."""
    lens = _host(context_lens).astype(np.int64).reshape(-1)
    tables = _host(block_tables).astype(np.int64)
    if tables.ndim != 2 or tables.shape[0] != lens.shape[0]:
        raise ContractError(f"{where}: block_tables must be [S][max_blocks] with S = "
                            f"{lens.shape[0]} rows, got shape {tuple(tables.shape)}")
    max_blocks = tables.shape[1]
    bad = lens < 0
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: context_lens[{i}] = {lens[i]} is negative")
    bad = lens > max_context_len
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: context_lens[{i}] = {lens[i]} exceeds max_context_len "
                            f"{max_context_len}")
    bad = lens > max_blocks * block_size
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: context_lens[{i}] = {lens[i]} exceeds max_blocks * "
                            f"block_size = {max_blocks * block_size}")
    if query_tokens > 1:
        bad = lens < query_tokens
        if bad.any():
            i = _first(bad)
            raise ContractError(f"{where}: context_lens[{i}] = {lens[i]} is shorter than the "
                                f"{query_tokens} query tokens it must hold")
    used = np.arange(max_blocks)[None, :] < ((lens + block_size - 1) // block_size)[:, None]
    bad = used & ((tables < 0) | (tables >= num_blocks))
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise ContractError(f"{where}: block_tables[{i}][{j}] = {tables[i, j]} is outside the "
                            f"pool of {num_blocks} blocks")


def check_shared_prefix(where, block_tables, prefix_tokens, block_size):
    tables = _host(block_tables)
    pb = prefix_tokens // block_size
    if pb == 0 or tables.shape[0] == 0:
        return
    bad = np.any(tables[:, :pb] != tables[0:1, :pb], axis=1)
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: the table of sequence {i} does not begin with the "
                            f"{pb} prefix blocks of sequence 0")


def check_slots(where, slot_mapping, num_blocks, block_size):
    slots = _host(slot_mapping).astype(np.int64).reshape(-1)
    live = slots[slots >= 0]
    bad = live >= num_blocks * block_size
    if bad.any():
        s = int(live[_first(bad)])
        raise ContractError(f"{where}: slot {s} is outside the pool of {num_blocks} blocks of "
                            f"{block_size}")
    uniq, counts = np.unique(live, return_counts=True)
    if np.any(counts > 1):
        s = int(uniq[_first(counts > 1)])
        raise ContractError(f"{where}: slot {s} appears {int(counts[counts > 1][0])} times in "
                            f"one call")


def check_newest_slots(where, slot_mapping, context_lens, block_tables, block_size):
    """A write fused into a decode: every written slot is its sequence's
    newest position (context_lens[i] - 1) through its own table."""
    slots = _host(slot_mapping).astype(np.int64).reshape(-1)
    lens = _host(context_lens).astype(np.int64).reshape(-1)
    tables = _host(block_tables).astype(np.int64)
    if slots.shape[0] != lens.shape[0]:
        raise ContractError(f"{where}: slot_mapping holds {slots.shape[0]} slots for "
                            f"{lens.shape[0]} sequences")
    for i in np.nonzero(slots >= 0)[0]:
        n = int(lens[i])
        if n < 1:
            raise ContractError(f"{where}: sequence {i} writes slot {int(slots[i])} but holds "
                                f"no position (context_lens = {n})")
        want = int(tables[i, (n - 1) // block_size]) * block_size + (n - 1) % block_size
        if int(slots[i]) != want:
            raise ContractError(f"{where}: slot_mapping[{i}] = {int(slots[i])} is not the slot "
                                f"{want} of the sequence's newest position {n - 1}")


def check_write_workspace(where, workspace):
    """An FP8 write's workspace holds per-block entries that must be zero at
    the call (every call leaves them zero): a non-zero count or maximum would
    give a block a wrong scale."""
    if workspace is None:
        return
    if isinstance(workspace, np.ndarray):
        data = workspace.reshape(-1).view(np.uint8)
    else:
        import torch
        data = workspace.reshape(-1).view(torch.uint8).cpu().numpy()
    if np.any(data != 0):
        raise ContractError(f"{where}: the FP8 write workspace must be zero at the call (byte "
                            f"{_first(data != 0)} is {int(data[_first(data != 0)])})")


def check_block_pairs(where, block_pairs, src_blocks, dst_blocks, same_pool):
    pairs = _host(block_pairs).astype(np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    bad = (src < 0) | (src >= src_blocks)
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: source block {src[i]} (pair {i}) is outside its pool of "
                            f"{src_blocks} blocks")
    bad = (dst < 0) | (dst >= dst_blocks)
    if bad.any():
        i = _first(bad)
        raise ContractError(f"{where}: destination block {dst[i]} (pair {i}) is outside its "
                            f"pool of {dst_blocks} blocks")
    uniq, counts = np.unique(dst, return_counts=True)
    if np.any(counts > 1):
        raise ContractError(f"{where}: destination block {int(uniq[_first(counts > 1)])} is "
                            f"written by more than one pair")
    if same_pool:
        both = np.intersect1d(src, dst)
        if both.size:
            raise ContractError(f"{where}: block {int(both[0])} is both a source and a "
                                f"destination within one pool")


def check_workspace_header(where, workspace, counter_bytes=SCHED_BYTES):
    """The counters at the front of a decode workspace must start at zero: the
    work-queue counters a persistent launch claims items from (non-zero, the
    launch would skip items) and the partition arrival counters of the fused
    merge (non-zero, a row group would be merged before all its partitions
    arrived, or never)."""
    if workspace is None:
        return
    n = max(int(counter_bytes), SCHED_BYTES)
    if isinstance(workspace, np.ndarray):
        head = workspace.reshape(-1).view(np.uint8)[:n]
    else:
        import torch
        head = workspace.reshape(-1).view(torch.uint8)[:n].cpu().numpy()
    if np.any(head != 0):
        i = _first(head != 0)
        what = "work-queue counters" if i < SCHED_BYTES else "partition arrival counters"
        raise ContractError(f"{where}: byte {i} of the workspace's first {n} bytes ({what}) "
                            f"is not zero: allocate it zero-filled and do not share it between "
                            f"calls that may overlap")
