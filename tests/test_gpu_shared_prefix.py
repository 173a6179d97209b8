"""GPU parity of the shared-prefix decode (the prefix read once per KV head for
all sequences, merged with each sequence's own positions) against the CPU
oracle's decode: within 2e-2 (bf16 cache) or 6e-2 (FP8 cache) of the float64
oracle on the stored cache.  A zero prefix is the plain decode bit for bit."""

import sys

import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import (TOL, DeviceWorkload, max_err, oracle_caches, oracle_decode, out_f64,
                         to_host)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import paged_kv_cache_370_amd as pkv
    pkv.load()


def _shared(dw, prefix, ps=0, lens=None, max_ctx=None):
    import paged_kv_cache_370_amd as pkv
    w = dw.w
    out = torch.empty_like(dw.q)
    pkv.paged_attention_decode_shared_prefix(
        out, dw.q, dw.kc, dw.vc, dw.tables, dw.lens if lens is None else lens,
        w.max_context_len if max_ctx is None else max_ctx, w.scale, prefix, dw.ks, dw.vs,
        partition_size=ps)
    torch.cuda.synchronize()
    return out


def test_shared_prefix_workload_reduced():
    w = workloads.make_config(4, reduced=True)
    prefix = w.shared_blocks * w.block_size
    _say(f"case shared-prefix reduced S={w.S} prefix={prefix} lens={list(w.context_lens)}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    for ps in (0, 64, 256):
        err = max_err(out_f64(_shared(dw, prefix, ps)), ref)
        _say(f"  ps={ps} max_err={err:.3e}")
        assert err <= TOL["bf16"], (ps, err)


def test_long_prefix_workload_reduced():
    """The long-prefix variant of the shared-prefix workload (the prefix
    longer than the suffixes): the read-once call and the plain decode, both
    against the oracle."""
    w = workloads.make_config(6, reduced=True)
    prefix = w.shared_blocks * w.block_size
    assert prefix == workloads.LONG_PREFIX[True]
    _say(f"case shared-prefix-long reduced S={w.S} prefix={prefix} lens={list(w.context_lens)}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    err = max_err(out_f64(dw.decode()), ref)
    _say(f"  plain decode max_err={err:.3e}")
    assert err <= TOL["bf16"], err
    for ps in (0, 256):
        err = max_err(out_f64(_shared(dw, prefix, ps)), ref)
        _say(f"  read-once ps={ps} max_err={err:.3e}")
        assert err <= TOL["bf16"], (ps, err)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes(seed):
    rng = np.random.default_rng(700 + seed)
    cache = ["bf16", "fp8"][seed % 2]
    D = int(rng.choice([64, 128]))
    bs = [16, 8, 32][seed % 3]
    H_kv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 4, 5, 8]))
    S = int(rng.integers(3, 9))
    prefix = bs * int(rng.integers(1, 40))
    lens = prefix + rng.integers(1, 500, size=S)
    w = workloads.build_workload(f"shared{seed}", S, H_kv * G, H_kv, D, bs, "bf16", cache, lens,
                                 seed, prefix_tokens=prefix,
                                 fill="write" if cache == "fp8" else "random")
    # some sequences shorter than the prefix (still on the shared blocks), one empty
    short = w.context_lens.copy()
    if seed % 2 == 0:
        short[0] = max(prefix - 7, 1)
        short[1] = 0
    w.context_lens = short
    ps = [0, 2 * bs, 128, 0][seed % 4]
    _say(f"case shared{seed} cache={cache} D={D} bs={bs} H_kv={H_kv} G={G} prefix={prefix} "
         f"lens={list(short)} ps={ps}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    out = out_f64(_shared(dw, prefix, ps))
    err = max_err(out, ref)
    _say(f"  max_err={err:.3e}")
    assert err <= TOL[cache], err
    assert np.all(out[short == 0] == 0)


@pytest.mark.parametrize("cache,G,S", [("bf16", 20, 6), ("fp8", 40, 3), ("bf16", 1, 520)])
def test_wide_groups_and_long_batches(cache, G, S):
    """Query-head groups wider than 16 (a sequence's heads split across the
    prefix items' 16-row chunks, and the suffix items' row groups), and a
    batch past the 512 sequences the kernel sorts in LDS (its plain item
    order)."""
    rng = np.random.default_rng(1100 + G)
    bs, H_kv = 16, 2 if G < 40 else 1
    prefix = 3 * bs
    lens = prefix + rng.integers(1, 200, size=S)
    w = workloads.build_workload(f"shared-wide-{cache}-G{G}-S{S}", S, H_kv * G, H_kv, 64, bs,
                                 "bf16", cache, lens, 1110 + G, prefix_tokens=prefix,
                                 fill="write" if cache == "fp8" else "random")
    short = w.context_lens.copy()
    short[0] = prefix - 5                    # shorter than the prefix
    w.context_lens = short
    _say(f"case shared wide cache={cache} G={G} S={S} prefix={prefix}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    for ps in (0, 32):
        err = max_err(out_f64(_shared(dw, prefix, ps)), ref)
        _say(f"  ps={ps} max_err={err:.3e}")
        assert err <= TOL[cache], (ps, err)


def test_zero_prefix_is_decode():
    w = workloads.make_config(2, reduced=True)
    dw = DeviceWorkload(w)
    dw.write()
    dec = dw.decode().clone()
    assert np.array_equal(to_host(_shared(dw, 0)), to_host(dec))


@pytest.mark.parametrize("cache", ["bf16", "fp8"])
def test_repeated_calls_on_one_workspace(cache):
    """One workspace serves repeated shared-prefix calls (sequences shorter
    than the prefix and an empty one included): its work-queue counters are
    zero after each call, and every call gives the same bits."""
    import paged_kv_cache_370_amd as pkv
    rng = np.random.default_rng(880)
    S, H_kv, G, bs = 40, 2, 4, 16
    prefix = 20 * bs
    lens = prefix + rng.integers(1, 300, size=S)
    w = workloads.build_workload(f"shared-merged-{cache}", S, H_kv * G, H_kv, 128, bs, "bf16",
                                 cache, lens, 881, prefix_tokens=prefix,
                                 fill="write" if cache == "fp8" else "random")
    short = w.context_lens.copy()
    short[3] = prefix - 5                    # shorter than the prefix
    short[4] = 0
    w.context_lens = short
    _say(f"case shared merged {cache} S={S} prefix={prefix}")
    kc, vc, ks, vs = oracle_caches(w)
    ref = oracle_decode(w, kc, vc, ks, vs)
    dw = DeviceWorkload(w)
    dw.write()
    qc, cc = 1, {"bf16": 1, "fp8": 2}[cache]
    need = pkv.shared_prefix_workspace_size(S, w.H, H_kv, 128, bs, w.max_context_len, prefix,
                                            qc, cc, 0)
    zero = 4096
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for k in range(3):
        out = torch.full_like(dw.q, float("nan"))
        pkv.paged_attention_decode_shared_prefix(out, dw.q, dw.kc, dw.vc, dw.tables, dw.lens,
                                                 w.max_context_len, w.scale, prefix, dw.ks,
                                                 dw.vs, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:zero].count_nonzero()) == 0, k
        err = max_err(out_f64(out), ref)
        _say(f"  call {k} max_err={err:.3e}")
        assert err <= TOL[cache], (k, err)
        assert np.all(out_f64(out)[4] == 0)
        outs.append(to_host(out))
    assert all(np.array_equal(o, outs[0]) for o in outs[1:])
