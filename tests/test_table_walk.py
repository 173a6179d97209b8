"""CPU replay of the decode kernel's block-table indexing (no GPU).

Each wave of a work item loads one slice of the item's table entries: lane l
of wave w reads entry tab_off + first_blk + (w + 4 (l div EPC)) EPC + l mod EPC
of its sequence's row, clamped to the row's last entry, where EPC = 32 / bs
entries cover one 32-token chunk and tab_off = len_off / bs skips the prefix
entries in the suffix launch of the shared-prefix call.  The replay checks,
for the plain decode and both launches of the shared-prefix call at the full
workload sizes, that every read lies inside block_tables ([S][max_blocks])
and that every valid position of an item is served by its own table entry.
"""

import numpy as np
import pytest

import workloads

NW, CHUNK = 4, 32


def _reads(lens, max_blocks, bs, P, tab_off, seqs):
    """Table indices every lane of every item reads, and the entries the
    item's valid positions need."""
    epc = CHUNK // bs
    lanes = np.arange(64)
    waves = np.arange(NW)[:, None]
    slot = (waves + NW * (lanes[None, :] // epc)) * epc + lanes[None, :] % epc   # [NW][64]
    reads, needs, served = [], [], []
    for i in seqs:
        n = int(lens[i])
        nparts = max(1, -(-n // P))
        for part in range(nparts):
            start, end = part * P, min(n, part * P + P)
            first_blk = start // bs
            entry = np.minimum(tab_off + first_blk + slot, max_blocks - 1)
            reads.append(i * max_blocks + entry.reshape(-1))
            # the chunk of position t belongs to wave (t - start) // 32 % NW and
            # uses lane slot ((t - start) // 32 // NW) * epc + (t % 32) // bs
            for t in range(start, end, bs):
                c = (t - start) // CHUNK
                w, k = c % NW, c // NW
                lane = k * epc + (t - start) % CHUNK // bs
                served.append(int(entry[w, lane]))
                needs.append(tab_off + t // bs)
    return np.concatenate(reads), np.array(needs), np.array(served)


def _lengths(cfg):
    """The workload's context lengths (the draw make_config uses) and its
    table width: one entry per block of the longest context."""
    lens = workloads.config_lengths(cfg, np.random.default_rng(1000 + cfg), False)
    bs = {2: 16, 3: 8, 4: 16, 5: 16}[cfg]
    return np.asarray(lens, np.int64), bs, int(-(-int(lens.max()) // bs))


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_plain_decode_reads_stay_in_the_table(cfg):
    lens, bs, max_blocks = _lengths(cfg)
    P = {2: 512, 3: 512, 5: 1024}[cfg]
    reads, needs, served = _reads(lens, max_blocks, bs, P, 0, range(len(lens)))
    assert reads.min() >= 0 and reads.max() < len(lens) * max_blocks
    assert np.array_equal(needs, served)


def test_shared_prefix_items_read_inside_the_table():
    lens, bs, max_blocks = _lengths(4)        # 128 sequences, 512-token prefix, bs 16
    prefix, P = 512, 512
    # prefix items: sequence 0's table, the prefix positions only
    reads, needs, served = _reads([prefix], max_blocks, bs, P, 0, [0])
    assert reads.max() < max_blocks and np.array_equal(needs, served)
    # suffix items: every sequence's positions after the prefix, entries
    # offset by the prefix's blocks
    tab_off = prefix // bs
    reads, needs, served = _reads(lens - prefix, max_blocks, bs, P, tab_off, range(len(lens)))
    assert reads.min() >= 0 and reads.max() < len(lens) * max_blocks
    assert np.array_equal(needs, served)


def test_suffix_items_of_contexts_ending_at_the_prefix():
    """Tables no longer than the prefix: the suffix items are empty,
    and the clamp keeps the reads on the row's last entry."""
    bs, prefix, max_blocks = 16, 64, 4
    reads, needs, served = _reads(np.array([0, 0, 0]), max_blocks, bs, 512, prefix // bs,
                                  range(3))
    assert reads.max() < 3 * max_blocks and needs.size == 0
