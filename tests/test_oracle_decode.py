"""Pins for the oracle's PagedAttention decode (CPU only).

Pinned against: brute force (tests/brute_force.py: per-token table walk in
pure Python), torch's scaled_dot_product_attention in float64 (a library
routine), closed forms, the invariants the pages imply (non-contiguous
storage, shared prefix blocks, block size as a tuning knob, grouped heads),
and the blockwise-pseudocode counter-example.  The last tests plant mistakes
in copies of the oracle and check that a pin catches each.
"""

import numpy as np
import pytest
import torch

import workloads
from brute_force import brute_decode
from oracle import paged_attention_decode, paged_attention_decode_one, paged_kv_cache_write
from oracle import attention as oracle_attention


def _apply_writes(w):
    kc, vc, ks, vs = w.key_cache, w.value_cache, w.key_scale, w.value_scale
    for key, value, slots in w.writes:
        if w.cache_dtype == "fp8":
            kc, vc, ks, vs = paged_kv_cache_write(key, value, kc, vc, slots, w.block_size, ks, vs)
        else:
            kc, vc = paged_kv_cache_write(key, value, kc, vc, slots, w.block_size)
    return kc, vc, ks, vs


def _decode(w, kc, vc, ks, vs):
    return paged_attention_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                  w.block_size, ks, vs)


def test_brute_force_config1():
    w = workloads.make_config(1)
    kc, vc, _, _ = _apply_writes(w)
    ours = _decode(w, kc, vc, None, None)
    ref = np.array(brute_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                w.block_size, "f32", "f32"))
    assert np.max(np.abs(ours - ref)) <= 1e-12


def _tiny_random(seed):
    rng = np.random.default_rng(seed)
    S = int(rng.integers(1, 4))
    H_kv = int(rng.integers(1, 3))
    G = int(rng.integers(1, 3))
    D = int(rng.choice([2, 4, 8]))
    bs = int(rng.choice([1, 2, 4, 8, 16]))
    cache = ["f32", "bf16", "fp8"][seed % 3]
    q = "f32" if cache == "f32" else "bf16"
    lens = rng.integers(0 if seed % 5 == 0 else 1, 41, size=S)
    if lens.max() == 0:
        lens[0] = 1
    return workloads.build_workload(f"tiny{seed}", S, H_kv * G, H_kv, D, bs, q, cache, lens,
                                    seed, fill="write", free_frac=0.5)


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_random_tiny(seed):
    w = _tiny_random(seed)
    kc, vc, ks, vs = _apply_writes(w)
    ours = _decode(w, kc, vc, ks, vs)
    ref = np.array(brute_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                w.block_size, w.q_dtype, w.cache_dtype, ks, vs))
    assert np.max(np.abs(ours - ref)) <= 1e-12
    assert np.all(ours[w.context_lens == 0] == 0)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_matches_torch_sdpa_fp64(cfg):
    w = workloads.make_config(cfg, reduced=True)
    kc, vc, ks, vs = _apply_writes(w)
    ours = _decode(w, kc, vc, ks, vs)
    G = w.H // w.H_kv
    qf = oracle_attention.element_values(w.q)
    for i in range(w.S):
        n = int(w.context_lens[i])
        K = oracle_attention.gather_sequence(kc, ks, w.block_tables[i], n, w.block_size)
        V = oracle_attention.gather_sequence(vc, vs, w.block_tables[i], n, w.block_size)
        Kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, 0)
        Vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, 0)
        qt = torch.from_numpy(qf[i][:, None, :])
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=w.scale)
        assert np.max(np.abs(ours[i] - ref[:, 0, :].numpy())) <= 1e-12


def test_decode_one_matches_full():
    w = workloads.make_config(4, reduced=True)
    kc, vc, _, _ = _apply_writes(w)
    full = _decode(w, kc, vc, None, None)
    for i, h in [(0, 0), (2, 13), (4, 31)]:
        one = paged_attention_decode_one(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                         w.block_size, i, h)
        assert np.array_equal(one, full[i, h])


# ---------------------------------------------------------------- closed forms

def _mini(n, D=8, H=2, bs=4, seed=0):
    return workloads.build_workload("mini", 1, H, H, D, bs, "f32", "f32", [n], seed,
                                    fill="write-all")


def test_single_token_returns_its_value():
    w = _mini(1)
    kc, vc, _, _ = _apply_writes(w)
    out = _decode(w, kc, vc, None, None)
    assert np.array_equal(out[0], w.writes[0][1][0].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    w = _mini(23)
    w.q[:] = 0
    kc, vc, _, _ = _apply_writes(w)
    out = _decode(w, kc, vc, None, None)
    mean = w.writes[0][1].astype(np.float64).mean(axis=0)
    assert np.max(np.abs(out[0] - mean)) <= 1e-12


def test_dominant_key_selects_its_value():
    w = _mini(19)
    key, value, slots = w.writes[0]
    key = key.copy()
    key[7] = (w.q[0] * 1e3).astype(np.float32)        # score of token 7 >> the rest
    w.writes[0] = (key, value, slots)
    kc, vc, _, _ = _apply_writes(w)
    out = _decode(w, kc, vc, None, None)
    assert np.max(np.abs(out[0] - value[7])) <= 1e-12


# ------------------------------------------------------------------ invariants

def test_block_permutation_invariant():
    a = workloads.make_config(2, reduced=True, layout_seed=11)
    b = workloads.make_config(2, reduced=True, layout_seed=12)
    assert not np.array_equal(a.block_tables, b.block_tables)
    # same token values, different physical placement
    fa = workloads.build_workload("p", 3, 4, 2, 16, 8, "bf16", "bf16", [50, 7, 33], 5,
                                  fill="write", layout_seed=1)
    fb = workloads.build_workload("p", 3, 4, 2, 16, 8, "bf16", "bf16", [50, 7, 33], 5,
                                  fill="write", layout_seed=2)
    assert not np.array_equal(fa.block_tables, fb.block_tables)
    oa = _decode(fa, *_apply_writes(fa))
    ob = _decode(fb, *_apply_writes(fb))
    assert np.array_equal(oa, ob)


def test_shared_prefix_equals_duplicated():
    w = workloads.make_config(4, reduced=True)
    d = workloads.duplicate_shared_blocks(w)
    assert np.all(w.block_tables[:, :32] == w.block_tables[0, :32])
    assert len(np.unique(d.block_tables[:, :32])) == 32 * d.S
    assert np.array_equal(_decode(w, *_apply_writes(w)), _decode(d, *_apply_writes(d)))


@pytest.mark.parametrize("cache", ["bf16", "f32"])
def test_block_size_invariant(cache):
    q = "f32" if cache == "f32" else "bf16"
    outs = []
    for bs in (8, 16, 32):
        w = workloads.build_workload("bs", 3, 6, 3, 32, bs, q, cache, [100, 17, 64], 9,
                                     fill="write", layout_seed=bs)
        outs.append(_decode(w, *_apply_writes(w)))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_gqa_equals_mha_with_repeated_kv():
    w = workloads.build_workload("g", 2, 8, 2, 16, 8, "bf16", "bf16", [45, 20], 4, fill="write")
    kc, vc, _, _ = _apply_writes(w)
    G = 4
    kr = np.repeat(kc, G, axis=1)
    vr = np.repeat(vc, G, axis=1)
    gqa = _decode(w, kc, vc, None, None)
    mha = paged_attention_decode(w.q, kr, vr, w.block_tables, w.context_lens, w.scale, w.block_size)
    assert np.array_equal(gqa, mha)


def test_poison_outside_context_is_never_read():
    w = workloads.make_config(2, reduced=True)
    kc, vc, _, _ = _apply_writes(w)
    assert np.isnan((kc.astype(np.uint32) << 16).view(np.float32)).any()   # poison present
    out = _decode(w, kc, vc, None, None)
    assert np.all(np.isfinite(out))


def test_blockwise_pseudocode_is_not_the_formula():
    """The article's loop (softmax per block, results added) equals the formula
    only when the context fits in one block."""
    for n, differs in ((16, False), (40, True)):
        w = _mini(n, D=8, H=1, bs=16, seed=3)
        kc, vc, _, _ = _apply_writes(w)
        ref = _decode(w, kc, vc, None, None)
        K = oracle_attention.gather_sequence(kc, None, w.block_tables[0], n, 16)[:, 0]
        V = oracle_attention.gather_sequence(vc, None, w.block_tables[0], n, 16)[:, 0]
        q = w.q[0, 0].astype(np.float64)
        per_block = np.zeros(8)
        for j in range(0, n, 16):
            s = K[j:j + 16] @ q * w.scale
            p = np.exp(s - s.max())
            per_block += (p / p.sum()) @ V[j:j + 16]
        assert (np.max(np.abs(per_block - ref[0, 0])) > 1e-3) == differs


# ------------------------------------------------- planted mistakes are caught

def _mutant_decode(kind):
    def run(q, kc, vc, tables, lens, scale, bs, ks=None, vs=None):
        qf = oracle_attention.element_values(np.asarray(q))
        S, H, D = qf.shape
        H_kv = kc.shape[1]
        G = H // H_kv
        out = np.zeros((S, H, D))
        for i in range(S):
            n = int(lens[i])
            if n == 0:
                continue
            K = oracle_attention.gather_sequence(kc, ks, tables[i], n, bs)
            V = oracle_attention.gather_sequence(vc, vs, tables[i], n, bs)
            for h in range(H):
                g = h % H_kv if kind == "head_map" else h // G
                Kg, Vg = K[:, g, :], V[:, g, :]
                if kind == "transposed_v":
                    Vg = V[:, g, :][::-1]
                s = Kg @ qf[i, h] * (1.0 if kind == "no_scale" else float(np.float32(scale)))
                if kind == "last_row_dropped" and n > 1:
                    s, Vg = s[:-1], Vg[:-1]
                p = np.exp(s - s.max())
                out[i, h] = (p @ Vg) / p.sum()
        return out
    return run


@pytest.mark.parametrize("kind", ["head_map", "no_scale", "last_row_dropped", "transposed_v"])
def test_planted_mistakes_fail_brute_force(kind):
    w = workloads.build_workload("m", 2, 4, 2, 8, 4, "f32", "f32", [13, 6], 21, fill="write")
    kc, vc, ks, vs = _apply_writes(w)
    ref = np.array(brute_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale,
                                w.block_size, "f32", "f32"))
    bad = _mutant_decode(kind)(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.block_size)
    good = _decode(w, kc, vc, None, None)
    assert np.max(np.abs(good - ref)) <= 1e-12
    assert np.max(np.abs(bad - ref)) > 1e-6
