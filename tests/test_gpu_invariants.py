"""GPU invariants the pages imply: non-contiguous storage, shared prefix blocks,
block size and partition size as tuning knobs."""

import sys

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import TOL, DeviceWorkload, max_err, oracle_caches, oracle_decode, out_f64, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(w, ps=0):
    dw = DeviceWorkload(w)
    dw.write()
    out = dw.decode(partition_size=ps)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("cache", ["f32", "bf16", "fp8"])
def test_block_permutation_is_bitwise_invariant(cache):
    qd = "f32" if cache == "f32" else "bf16"
    outs = []
    for ls in (1, 2):
        w = workloads.build_workload("perm", 4, 16, 4, 128, 16, qd, cache, [300, 17, 600, 64], 5,
                                     fill="write", layout_seed=ls)
        _say(f"case permutation {cache} layout_seed={ls}")
        outs.append(to_host(_run(w, ps=256)))
    assert np.array_equal(outs[0].view(np.uint8), outs[1].view(np.uint8))


def test_shared_prefix_equals_duplicated_bitwise():
    w = workloads.make_config(4, reduced=True)
    d = workloads.duplicate_shared_blocks(w)
    _say("case shared prefix vs duplicated")
    a = _run(w)
    b = _run(d)
    assert np.array_equal(to_host(a).view(np.uint8), to_host(b).view(np.uint8))
    ref = oracle_decode(d, *oracle_caches(d))
    assert max_err(out_f64(a), ref) <= TOL["bf16"]


@pytest.mark.parametrize("cache", ["f32", "bf16"])
def test_block_size_and_partition_within_tolerance(cache):
    qd = "f32" if cache == "f32" else "bf16"
    lens = [1000, 33, 515]
    ref = None
    for bs in (8, 16, 32):
        w = workloads.build_workload("bs", 3, 8, 2, 64, bs, qd, cache, lens, 9, fill="write",
                                     layout_seed=bs)
        if ref is None:
            ref = oracle_decode(w, *oracle_caches(w))
        for ps in (0, 4 * bs, 512):
            _say(f"case block size {bs} partition {ps} {cache}")
            dw = DeviceWorkload(w)
            dw.write()
            out = dw.decode(partition_size=ps)
            torch.cuda.synchronize()
            assert max_err(out_f64(out), ref) <= TOL[cache]


def test_poison_in_free_blocks_and_tail_rows_is_not_read():
    w = workloads.make_config(2, reduced=True)
    _say("case poison")
    dw = DeviceWorkload(w)
    dw.write()
    out = dw.decode(partition_size=64)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out_f64(out)))
