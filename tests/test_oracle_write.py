"""Pins for the oracle's paged KV write (CPU only).

Pinned against: a per-token, per-element re-addressing of the pool written in
this file (round trip), byte-for-byte preservation of every untouched slot,
torch's float8_e4m3fn conversion for FP8 codes of freshly scaled blocks, the
closed form of the block scale, and the E4M3 error bound.
"""

import numpy as np
import pytest
import torch

import workloads
from oracle import paged_kv_cache_write, fp8_decode


def _read_token(cache, table_row, t, bs):
    """Row of token t of one sequence: [H_kv][D], addressed one token at a time."""
    return cache[int(table_row[t // bs]), :, t % bs, :]


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_round_trip_and_untouched_bytes(cfg):
    w = workloads.make_config(cfg, reduced=True)
    kc, vc = w.key_cache, w.value_cache
    for key, value, slots in w.writes:
        nk, nv = paged_kv_cache_write(key, value, kc, vc, slots, w.block_size)
        touched = np.zeros(kc.shape[0] * w.block_size, bool)
        touched[slots[slots >= 0]] = True
        touched = touched.reshape(kc.shape[0], w.block_size)
        for new, old, src in ((nk, kc, key), (nv, vc, value)):
            # untouched rows keep their exact bytes (NaN poison included)
            mask = ~touched[:, None, :, None] & np.ones(old.shape, bool)
            assert np.array_equal(new.view(np.uint8).reshape(old.shape + (-1,))[mask],
                                  old.view(np.uint8).reshape(old.shape + (-1,))[mask])
            for t, s in enumerate(slots):
                row = new[s // w.block_size, :, s % w.block_size, :]
                assert np.array_equal(row.view(np.uint8), src[t].view(np.uint8))
        kc, vc = nk, nv
    # after all writes every position < n reads back the bytes that were written
    if cfg == 1:
        src = np.concatenate([wr[0] for wr in w.writes])
        t0 = 0
        for i, n in enumerate(w.context_lens):
            for t in range(n):
                assert np.array_equal(_read_token(kc, w.block_tables[i], t, w.block_size).view(np.uint32),
                                      src[t0 + t].view(np.uint32))
            t0 += n


def test_negative_slots_skip_and_duplicates_rejected():
    rng = np.random.default_rng(3)
    kc = np.zeros((4, 2, 8, 16), np.float32)
    key = rng.standard_normal((3, 2, 16)).astype(np.float32)
    slots = np.array([5, -1, 17], np.int32)
    nk, nv = paged_kv_cache_write(key, key, kc, kc, slots, 8)
    assert np.array_equal(nk[0, :, 5], key[0]) and np.array_equal(nk[2, :, 1], key[2])
    assert np.count_nonzero(nk) == np.count_nonzero(key[[0, 2]])
    with pytest.raises(AssertionError):
        paged_kv_cache_write(key, key, kc, kc, np.array([5, 5, 1], np.int32), 8)


def _fp8_setup(seed=0, T=40, H=3, D=32, bs=16, nblk=6):
    rng = np.random.default_rng(seed)
    src = workloads.bf16_bits(rng.standard_normal((T, H, D)).astype(np.float32) * 3)
    kc = np.full((nblk, H, bs, D), 0x7F, np.uint8)
    ks = np.full((nblk, H), np.nan, np.float32)
    return rng, src, kc, ks


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_fp8_fresh_blocks_match_torch_and_closed_form_scale():
    rng, src, kc, ks = _fp8_setup()
    # 40 tokens: block 4 gets offsets 0..15, block 1 gets 0..15, block 3 gets 0..7
    slots = np.concatenate([4 * 16 + np.arange(16), 1 * 16 + np.arange(16), 3 * 16 + np.arange(8)]).astype(np.int32)
    nk, nv, nks, nvs = paged_kv_cache_write(src, src, kc, kc.copy(), slots, 16, ks, ks.copy())
    x = torch.from_numpy(_bf16_to_f32(src))
    for blk, rows in ((4, slice(0, 16)), (1, slice(16, 32)), (3, slice(32, 40))):
        amax = x[rows].abs().amax(dim=(0, 2))                       # [H] float32
        scale = torch.clamp(amax / torch.tensor(448.0), min=torch.finfo(torch.float32).tiny)
        assert np.array_equal(nks[blk], scale.numpy())
        ref = (x[rows] / scale[None, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        n = rows.stop - rows.start
        assert np.array_equal(nk[blk, :, :n, :], ref.transpose(1, 0, 2))
        # the largest element of each (block, head) is encoded as +-448
        got = nk[blk, :, :n, :]
        assert np.all(np.max(got & 0x7F, axis=(1, 2)) == 0x7E)
    # untouched block keeps poison, untouched scale stays NaN
    assert np.all(nk[0] == 0x7F) and np.all(np.isnan(nks[0]))


def test_fp8_append_reuses_scale_and_saturates():
    rng, src, kc, ks = _fp8_setup(seed=1, T=20)
    slots_a = (2 * 16 + np.arange(10)).astype(np.int32)
    nk, _, nks, _ = paged_kv_cache_write(src[:10], src[:10], kc, kc, slots_a, 16, ks, ks)
    big = src[10:12].copy()
    big[0, 0, 0] = workloads.bf16_bits(np.array([1e4], np.float32))[0]
    slots_b = (2 * 16 + np.array([10, 11])).astype(np.int32)
    nk2, _, nks2, _ = paged_kv_cache_write(big, big, nk, nk, slots_b, 16, nks, nks)
    assert np.array_equal(nks2, nks, equal_nan=True)   # offset 0 not written: scale kept
    assert nk2[2, 0, 10, 0] == 0x7E                    # 1e4 / scale saturates
    assert np.array_equal(nk2[2, :, :10], nk[2, :, :10])


def test_fp8_error_bound():
    w = workloads.make_config(5, reduced=True)
    kc, vc, ks, vs = w.key_cache, w.value_cache, w.key_scale, w.value_scale
    key, value, slots = w.writes[0]
    kc, vc, ks, vs = paged_kv_cache_write(key, value, kc, vc, slots, w.block_size, ks, vs)
    x = _bf16_to_f32(key).astype(np.float64)
    blk = slots // w.block_size
    off = slots % w.block_size
    deq = fp8_decode(kc[blk, :, off, :]) * ks[blk][:, :, None].astype(np.float64)
    s = ks[blk][:, :, None].astype(np.float64)
    y = np.abs(x) / s
    # half an E4M3 ulp: 2^-4 relative in the normal range, 2^-10 absolute below 2^-6
    bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * (1 + 2.0 ** -20) * s
    assert np.all(np.abs(deq - x) <= bound)


# ------------------------------------------------- planted mistakes are caught

def _mutant_write(old, new):
    """A copy of the oracle's write with one line of its source changed."""
    import importlib.util
    import types
    import oracle.cache_write as cw
    src = open(cw.__file__).read()
    assert old in src, old
    mod = types.ModuleType("mutant_cache_write")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), cw.__file__, "exec"), mod.__dict__)
    return mod.paged_kv_cache_write


def _round_trip_pin(write):
    w = workloads.make_config(2, reduced=True)
    key, value, slots = w.writes[0]
    nk, _ = write(key, value, w.key_cache, w.value_cache, slots, w.block_size)
    for t, s in enumerate(slots):
        if not np.array_equal(nk[s // w.block_size, :, s % w.block_size, :].view(np.uint8),
                              key[t].view(np.uint8)):
            return False
    return True


def _scale_pin(write):
    rng, src, kc, ks = _fp8_setup()
    slots = (4 * 16 + np.arange(16)).astype(np.int32)
    _, _, nks, _ = write(src[:16], src[:16], kc, kc.copy(), slots, 16, ks, ks.copy())
    amax = torch.from_numpy(_bf16_to_f32(src[:16])).abs().amax(dim=(0, 2))
    scale = torch.clamp(amax / torch.tensor(448.0), min=torch.finfo(torch.float32).tiny)
    return np.array_equal(nks[4], scale.numpy())


def _append_pin(write):
    rng, src, kc, ks = _fp8_setup(seed=1, T=20)
    nk, _, nks, _ = write(src[:10], src[:10], kc, kc, (2 * 16 + np.arange(10)).astype(np.int32),
                          16, ks, ks)
    _, _, nks2, _ = write(src[10:12], src[10:12], nk, nk,
                          (2 * 16 + np.array([10, 11])).astype(np.int32), 16, nks, nks)
    return np.array_equal(nks2, nks, equal_nan=True)


@pytest.mark.parametrize("old,new,pin", [
    ("off = s % block_size", "off = (s + 1) % block_size", _round_trip_pin),
    ("np.maximum(amax / np.float32(FP8_MAX), _FLT_MIN)",
     "np.maximum(amax / np.float32(FP8_MAX - 1), _FLT_MIN)", _scale_pin),
    ("fresh[blk[off == 0]] = True", "fresh[blk] = True", _append_pin),
])
def test_planted_mistakes_are_caught(old, new, pin):
    assert pin(paged_kv_cache_write)
    assert not pin(_mutant_write(old, new))
