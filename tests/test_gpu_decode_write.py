"""GPU parity of paged_attention_decode_write (the step's write fused into
the decode launch): bit for bit the output and the caches of
paged_kv_cache_write followed by paged_attention_decode, and within the bf16
bar of the oracle; sequences that write nothing read their newest position
from the cache."""

import sys

import numpy as np
import pytest
import torch

import workloads
import oracle
from gpu_helpers import TOL, max_err, oracle_caches, oracle_decode, out_f64, to_dev, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_370_amd as pkv
    pkv.load()


def _newest_slots(w):
    lens, tables, bs = w.context_lens, w.block_tables, w.block_size
    return np.array([tables[i, (n - 1) // bs] * bs + (n - 1) % bs for i, n in enumerate(lens)],
                    dtype=np.int32)


def _both(w, ps, slots=None, key=None, value=None, prewrite=False):
    """(two-call out, kc, vc), (fused out, kc, vc) on the same inputs."""
    import paged_kv_cache_370_amd as pkv
    k0, v0, s0 = w.writes[-1]
    assert np.array_equal(s0, _newest_slots(w))  # the step write is each sequence's newest position
    key = k0 if key is None else key
    value = v0 if value is None else value
    slots = s0 if slots is None else slots
    res = []
    for fused in (False, True):
        kc, vc = to_dev(w.key_cache), to_dev(w.value_cache)
        for k, v, s in w.writes[:-1]:
            pkv.paged_kv_cache_write(to_dev(k), to_dev(v), kc, vc, to_dev(s))
        if prewrite:  # the newest positions already cached (their own rows)
            pkv.paged_kv_cache_write(to_dev(k0), to_dev(v0), kc, vc, to_dev(s0))
        q, tables, lens = to_dev(w.q), to_dev(w.block_tables), to_dev(w.context_lens)
        dk, dv, ds = to_dev(key), to_dev(value), to_dev(slots)
        out = torch.empty_like(q)
        if fused:
            pkv.paged_attention_decode_write(out, q, dk, dv, kc, vc, ds, tables, lens,
                                             w.max_context_len, w.scale, partition_size=ps)
        else:
            pkv.paged_kv_cache_write(dk, dv, kc, vc, ds)
            pkv.paged_attention_decode(out, q, kc, vc, tables, lens, w.max_context_len, w.scale,
                                       partition_size=ps)
        torch.cuda.synchronize()
        res.append((to_host(out), to_host(kc), to_host(vc)))
    return res


def _assert_same(a, b, what):
    for x, y, name in zip(a, b, ("out", "key cache", "value cache")):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f"{what}: {name} differs"


@pytest.mark.parametrize("seed", range(10))
def test_random_shapes_bitwise_and_oracle(seed):
    rng = np.random.default_rng(2100 + seed)
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    H_kv = int(rng.integers(1, 5))
    G = int(rng.choice([1, 2, 4, 5, 8, 16, 20]))
    S = int(rng.integers(1, 12))
    lens = rng.integers(1, 1400, size=S)
    lens[0] = 1 if seed % 3 == 0 else lens[0]          # the new token is the whole context
    ps = [0, 2 * bs, 128, 256, 512, 64][seed % 6]       # whole, merged in-kernel, reduce kernel
    w = workloads.build_workload(f"dw{seed}", S, H_kv * G, H_kv, D, bs, "bf16", "bf16", lens,
                                 seed)
    _say(f"case decode-write {seed} D={D} bs={bs} H_kv={H_kv} G={G} S={S} ps={ps} "
         f"lens={list(lens)}")
    two, one = _both(w, ps)
    _assert_same(two, one, f"seed {seed}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    got = (one[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = max_err(got, ref)
    _say(f"  bitwise equal; max_err vs oracle {err:.3e}")
    assert err <= TOL["bf16"], err


def test_sequences_that_write_nothing_read_the_cache():
    """Slots outside the pool (negative, or past it) write nothing; those
    sequences attend to the cached row of their newest position, not to the
    new rows passed for them."""
    rng = np.random.default_rng(7)
    lens = rng.integers(2, 900, size=9)
    w = workloads.build_workload("dw-skip", 9, 16, 4, 128, 16, "bf16", "bf16", lens, 7)
    k0, v0, s0 = w.writes[-1]
    slots = s0.copy()
    slots[[1, 4]] = -1
    slots[7] = w.num_blocks * w.block_size + 3
    key = k0.copy()
    value = v0.copy()
    for i in (1, 4, 7):  # rows that must not be used: other bf16 values
        bits = rng.standard_normal(key[i].shape).astype(np.float32).view(np.uint32) >> 16
        key[i] = bits.astype(np.uint16)
        value[i] = key[i][::-1]
    for ps in (0, 256):
        two, one = _both(w, ps, slots=slots, key=key, value=value, prewrite=True)
        _assert_same(two, one, f"ps {ps}")
        # against the oracle: the cache holds the original rows everywhere
        kc, vc, ks, vs = oracle_caches(w)
        ref = oracle_decode(w, kc, vc, ks, vs)
        got = (one[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        err = max_err(got, ref)
        _say(f"case skipped slots ps={ps}: bitwise equal, max_err {err:.3e}")
        assert err <= TOL["bf16"], err


def test_fp32_runs_the_two_launches():
    """fp32 queries and cache (vector-ALU kernel): the write, then the decode."""
    lens = [1, 37, 80, 300]
    w = workloads.build_workload("dw-f32", 4, 8, 2, 64, 16, "f32", "f32", lens, 3)
    for ps in (0, 64):
        two, one = _both(w, ps)
        _assert_same(two, one, f"f32 ps {ps}")
    _say("case fp32: bitwise equal")


def test_fp8_cache_is_refused():
    import paged_kv_cache_370_amd as pkv
    w = workloads.build_workload("dw-fp8", 2, 8, 2, 128, 16, "bf16", "fp8", [20, 40], 5,
                                 fill="write")
    k, v, s = (to_dev(x) for x in w.writes[-1])
    kc, vc = to_dev(w.key_cache), to_dev(w.value_cache)
    q, tables, lens = to_dev(w.q), to_dev(w.block_tables), to_dev(w.context_lens)
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_attention_decode_write(torch.empty_like(q), q, k, v, kc, vc, s, tables, lens,
                                         w.max_context_len, w.scale)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_timed_workloads_bitwise(cfg):
    """The bf16 decode workloads the benchmark times (7B-class, 32K, shared
    prefix), full size, in their launch configuration: the fused step equals
    the two calls bit for bit."""
    w = workloads.make_config(cfg)
    _say(f"case full size {w.name} S={w.S} P={w.partition_size}")
    two, one = _both(w, w.partition_size)
    _assert_same(two, one, w.name)
    _say("  bitwise equal")


@pytest.mark.parametrize("ps", [0, 64])
def test_batch_beyond_the_scan_limit(ps):
    """More sequences than the decode kernel sorts in LDS (512): its plain
    item order, with the fused write, equals the two calls bit for bit."""
    rng = np.random.default_rng(61)
    lens = rng.integers(1, 300, size=600)
    w = workloads.build_workload("dw-wide", 600, 8, 2, 128, 16, "bf16", "bf16", lens, 61)
    _say(f"case 600 sequences ps={ps}")
    two, one = _both(w, ps)
    _assert_same(two, one, f"600 sequences ps {ps}")
    _say("  bitwise equal")
