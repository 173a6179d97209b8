"""GPU parity of the multi-token (chunked prefill) attention against the CPU
oracle: every output element within 2e-2 (bf16 cache) or 6e-2 (FP8 cache) of
the float64 oracle on the stored cache, on small shapes whole and on a long
chunk at sampled tokens.  Also: one query token is the decode path bit for
bit."""

import sys

import numpy as np
import pytest
import torch

import workloads
import oracle
from gpu_helpers import TOL, DeviceWorkload, max_err, oracle_caches, out_f64, to_host

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_370_amd as pkv
    pkv.load()


def _prefill(dw, ps, out=None):
    import paged_kv_cache_370_amd as pkv
    w = dw.w
    out = torch.empty_like(dw.q) if out is None else out
    pkv.paged_attention_prefill(out, dw.q, dw.kc, dw.vc, dw.tables, dw.lens, w.max_context_len,
                                w.scale, dw.ks, dw.vs, partition_size=ps)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    rng = np.random.default_rng(500 + seed)
    cache = ["bf16", "fp8"][seed % 2]
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([8, 16, 32]))
    H_kv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    M = int(rng.choice([2, 3, 7, 16, 40]))
    S = int(rng.integers(1, 5))
    lens = rng.integers(M, M + 600, size=S)
    if seed % 3 == 0:
        lens[0] = M                        # the whole sequence is the chunk
    w = workloads.build_workload(f"prefill{seed}", S, H_kv * G, H_kv, D, bs, "bf16", cache, lens,
                                 seed, fill="write" if cache == "fp8" else "random",
                                 query_tokens=M)
    ps = int(rng.choice([0, 2 * bs, 128, 256]))
    _say(f"case prefill{seed} cache={cache} D={D} bs={bs} H_kv={H_kv} G={G} M={M} "
         f"lens={list(lens)} ps={ps}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         bs, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    out = _prefill(dw, ps)
    err = max_err(out_f64(out), ref)
    _say(f"  max_err={err:.3e}")
    assert err <= TOL[cache], err


@pytest.mark.parametrize("seed", range(12))
def test_tiled_shapes(seed):
    """bf16 caches with at least 64 (token, head) rows per KV head: the tiled
    kernel, over whole contexts and over explicit partitions (split reduce),
    several row tiles with a ragged last one, and chunks that are the whole
    sequence (the causal triangle)."""
    rng = np.random.default_rng(900 + seed)
    D = [128, 64][seed % 2]
    bs = [16, 8, 32][seed % 3]
    H_kv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8]))
    M = int(rng.choice([64, 100, 200])) if G == 1 else int(rng.choice([16, 33, 70, 130]))
    S = int(rng.integers(1, 4))
    lens = rng.integers(M, M + 900, size=S)
    if seed % 4 == 1:
        lens[:] = M                        # prompt processed from scratch
    ps = [0, 0, 64, 256, 4 * bs, 192][seed % 6]
    ps = ps - ps % bs
    w = workloads.build_workload(f"tiled{seed}", S, H_kv * G, H_kv, D, bs, "bf16", "bf16", lens,
                                 seed, query_tokens=M)
    _say(f"case tiled{seed} D={D} bs={bs} H_kv={H_kv} G={G} M={M} lens={list(lens)} ps={ps}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         bs, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    out = _prefill(dw, ps)
    err = max_err(out_f64(out), ref)
    _say(f"  max_err={err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("seed", range(8))
def test_tiled_fp8_shapes(seed):
    """FP8 caches with at least 64 (token, head) rows per KV head: the blocks
    the sequences reach are staged to bf16, then the tiled kernel runs on
    them; whole contexts and explicit partitions, every block size, chunks
    that are the whole sequence, and tables that share blocks."""
    rng = np.random.default_rng(1300 + seed)
    D = [128, 64][seed % 2]
    bs = [16, 8, 32][seed % 3]
    H_kv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4, 8]))
    M = int(rng.choice([64, 100, 200])) if G == 1 else int(rng.choice([16, 33, 70, 130]))
    S = int(rng.integers(1, 4))
    lens = rng.integers(M, M + 900, size=S)
    if seed % 4 == 1:
        lens[:] = M
    ps = [0, 256, 0, 4 * bs, 192, 64][seed % 6]
    ps = ps - ps % bs
    w = workloads.build_workload(f"tiled-fp8-{seed}", S, H_kv * G, H_kv, D, bs, "bf16", "fp8",
                                 lens, seed, fill="write", query_tokens=M)
    if seed % 4 == 3 and S > 1:  # the first blocks of every table name sequence 0's
        shared = min(int(lens.min()) - M, 128) // bs
        w.block_tables[1:, :shared] = w.block_tables[0, :shared]
    _say(f"case tiled-fp8-{seed} D={D} bs={bs} H_kv={H_kv} G={G} M={M} lens={list(lens)} "
         f"ps={ps}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         bs, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    out = _prefill(dw, ps)
    err = max_err(out_f64(out), ref)
    _say(f"  max_err={err:.3e}")
    assert err <= TOL["fp8"], err


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_tiled_short_contexts_beside_split_ones(cache):
    """Sequences within one partition beside ones split over several (the
    grid covers the longest): the short ones are finished by their first
    partition, and their later, empty partitions leave the output alone."""
    lens = np.array([64, 900, 70, 64, 513])
    w = workloads.build_workload(f"tiled-short-{cache}", 5, 16, 2, 128, 16, "bf16", cache, lens,
                                 17, fill="write" if cache == "fp8" else "random",
                                 query_tokens=64)
    _say(f"case tiled short beside split {cache} lens={list(lens)}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         16, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    for ps in (128, 256):
        err = max_err(out_f64(_prefill(dw, ps)), ref)
        _say(f"  ps={ps} max_err={err:.3e}")
        assert err <= TOL[cache], (ps, err)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 3.0])
def test_tiled_scale_edge_cases(scale):
    """Negative, zero and large softmax scales on the tiled kernel (a zero
    scale weighs every visible position equally)."""
    lens = [300, 170]
    w = workloads.build_workload("tiled-scale", 2, 8, 2, 128, 16, "bf16", "bf16", lens, 5,
                                 query_tokens=64)
    w.scale = scale
    _say(f"case tiled scale={scale}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         16, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    for ps in (0, 128):
        err = max_err(out_f64(_prefill(dw, ps)), ref)
        _say(f"  ps={ps} max_err={err:.3e}")
        assert err <= TOL["bf16"], (ps, err)


def test_beam_fork_multi_query():
    """Beams forked from shared prompts, four query tokens each (decode
    kernel's multi-token mode): parity with the oracle, and bitwise the same
    output as with every beam owning private copies of the prompt blocks."""
    w = workloads.make_beam_fork(reduced=True)
    _say(f"case beam fork S={w.S} M={w.query_tokens} lens={list(w.context_lens)}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         w.block_size)
    outs = []
    for x in (w, workloads.unshare_blocks(w)):
        dw = DeviceWorkload(x)
        dw.write()
        outs.append(to_host(_prefill(dw, 0)))
    got = (outs[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # bf16 bits
    err = max_err(got, ref)
    _say(f"  max_err={err:.3e}")
    assert err <= TOL["bf16"], err
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_many_short_chunks_whole_contexts(cache):
    """64 sequences x 8 KV heads of 4-token chunks (512 items): the library
    attends each whole context in one item, without partials."""
    rng = np.random.default_rng(91)
    lens = rng.integers(4, 900, size=64)
    w = workloads.build_workload(f"short-chunks-{cache}", 64, 32, 8, 128, 16, "bf16", cache, lens,
                                 91, fill="write" if cache == "fp8" else "random", query_tokens=4)
    _say(f"case many short chunks {cache}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle.paged_attention_prefill(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         w.block_size, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    for ps in (0, 256):
        err = max_err(out_f64(_prefill(dw, ps)), ref)
        _say(f"  ps={ps} max_err={err:.3e}")
        assert err <= TOL[cache], (ps, err)


def test_one_query_token_is_decode():
    w = workloads.make_config(2, reduced=True)
    _say(f"case prefill M=1 vs decode {w.name}")
    dw = DeviceWorkload(w)
    dw.write()
    import paged_kv_cache_370_amd as pkv
    for ps in (0, 64):
        dec = dw.decode(partition_size=ps).clone()
        q4 = dw.q[:, None]
        out = torch.empty_like(q4)
        pkv.paged_attention_prefill(out, q4, dw.kc, dw.vc, dw.tables, dw.lens, w.max_context_len,
                                    w.scale, partition_size=ps)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out[:, 0]), to_host(dec)), ps


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_long_chunk_sampled_tokens(cache):
    """A 512-token chunk at the end of 3000-3600-token contexts, 32 query heads
    over 8 KV heads, 512-token partitions: every element of sampled tokens."""
    rng = np.random.default_rng(77)
    M = 512
    lens = rng.integers(3000, 3601, size=3)
    w = workloads.build_workload(f"chunk-{cache}", 3, 32, 8, 128, 16, "bf16", cache, lens, 11,
                                 fill="write" if cache == "fp8" else "random", query_tokens=M)
    _say(f"case long chunk {cache} lens={list(lens)} M={M}")
    kc, vc, ks, vs = oracle_caches(w)
    dw = DeviceWorkload(w)
    dw.write()
    out = out_f64(_prefill(dw, 512))
    for t in (0, 1, 100, 255, 256, 400, 510, 511):
        ref = oracle.paged_attention_decode(w.q[:, t], kc, vc, w.block_tables,
                                            w.context_lens - M + t + 1, w.scale, 16, ks, vs)
        err = max_err(out[:, t], ref)
        _say(f"  token {t} max_err={err:.3e}")
        assert err <= TOL[cache], (t, err)


@pytest.mark.parametrize("name", sorted(workloads.PREFILL_CONFIGS))
def test_timed_prefill_workloads_sampled_tokens(name):
    """The chunked-prefill workloads the benchmark times, at full size and in
    its launch configuration (the library's partitions; FP8 staged for the
    tiled kernel): every element of sampled tokens against the oracle."""
    w = workloads.make_prefill(name)
    M = w.query_tokens
    _say(f"case timed prefill {name} S={w.S} M={M} lens={list(w.context_lens)}")
    kc, vc, ks, vs = oracle_caches(w)
    dw = DeviceWorkload(w)
    dw.write()
    out = out_f64(_prefill(dw, 0))
    for t in (0, 137, 384, M - 1):
        ref = oracle.paged_attention_decode(w.q[:, t], kc, vc, w.block_tables,
                                            w.context_lens - M + t + 1, w.scale, w.block_size,
                                            ks, vs)
        err = max_err(out[:, t], ref)
        _say(f"  token {t} max_err={err:.3e}")
        assert err <= TOL[w.cache_dtype], (t, err)
