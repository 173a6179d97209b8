"""Oracle for the paged KV write (test infrastructure).

What it computes (the plain definition):

* The pool is ``cache[num_blocks][num_kv_heads][block_size][head_size]``: each
  physical block holds, per KV head, ``block_size`` token rows of
  ``head_size`` elements.  This follows the Block structure of the dpshk.com
  PagedAttention article ("企业官网建设流程全解析", section 2.1: a block of a
  fixed number of tokens, default 16, holding keys and values of shape
  [block_size, head_size]); the KV-head axis sits outside the token axis so
  each (block, head) tile is contiguous.
* Token ``t`` goes to flat slot ``s = slot_mapping[t]`` (a slot is
  ``physical_block * block_size + offset``); a negative slot means "skip".
  The pages do not name the slot mapping; it is the write-side addressing of
  the block table ("vLLM的诞生背景…" page, section "PagedAttention的破局思路":
  logical blocks map to physical blocks through a block table).
* fp32 and bf16 caches receive the source bits unchanged.
* FP8 (E4M3FN) caches, section 3.2 of the dpshk.com article (FP8 storage of
  blocks).  The pages give no scale rule, so this library reads it as:
  one float32 scale per (physical block, KV head), separately for K and V.
  A call that writes offset 0 of a block sets that block's scales from the
  largest magnitude among the tokens this call writes into the block:
  ``scale = max(fp32(amax / 448), FLT_MIN)``.  Any other call reuses the
  stored scale.  Each element is encoded as ``encode(fp32(x / scale))`` with
  IEEE float32 division, round-to-nearest-even and saturation to +-448.

Slots within one call must be distinct (asserted here).
"""

import numpy as np

from .fp8_e4m3 import fp8_encode, FP8_MAX

_FLT_MIN = np.float32(np.finfo(np.float32).tiny)


def _source_as_f32(x: np.ndarray) -> np.ndarray:
    """fp32 or bf16-bit-pattern source -> float32 (exact)."""
    if x.dtype == np.float32:
        return x
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    raise TypeError(f"unsupported source dtype {x.dtype}")


def paged_kv_cache_write(key, value, key_cache, value_cache, slot_mapping,
                         block_size, key_scale=None, value_scale=None):
    """Return copies of the caches (and scales, for FP8) after the write.

    key, value     : [T][H_kv][D]  float32 or uint16 (bf16 bits)
    key_cache, ... : [num_blocks][H_kv][block_size][D]  same dtype as the
                     source, or uint8 for FP8 (then the source may be fp32 or
                     bf16 and key_scale/value_scale [num_blocks][H_kv] float32
                     are required)
    slot_mapping   : [T] integer; < 0 skips the token
    """
    key = np.asarray(key)
    value = np.asarray(value)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    num_blocks = kc.shape[0]

    keep = np.nonzero(slots >= 0)[0]
    s = slots[keep]
    assert len(np.unique(s)) == len(s), "slots within one call must be distinct"
    assert np.all(s < num_blocks * block_size), "slot outside the pool"
    blk = s // block_size
    off = s % block_size

    if kc.dtype != np.uint8:
        assert kc.dtype == key.dtype and vc.dtype == value.dtype
        # Advanced indices around a slice: the token axis comes first.
        kc[blk, :, off, :] = key[keep]
        vc[blk, :, off, :] = value[keep]
        return kc, vc

    ks = np.array(key_scale, dtype=np.float32, copy=True)
    vs = np.array(value_scale, dtype=np.float32, copy=True)
    for src, cache, scl in ((key, kc, ks), (value, vc, vs)):
        x = _source_as_f32(src[keep])                      # [T'][H_kv][D]
        fresh = np.zeros(num_blocks, dtype=bool)
        fresh[blk[off == 0]] = True
        amax = np.zeros(scl.shape, dtype=np.float32)       # [num_blocks][H_kv]
        np.maximum.at(amax, blk, np.abs(x).max(axis=2))
        new_scale = np.maximum(amax / np.float32(FP8_MAX), _FLT_MIN)
        scl[fresh] = new_scale[fresh]
        per_token = scl[blk]                               # [T'][H_kv]
        cache[blk, :, off, :] = fp8_encode(x / per_token[:, :, None])
    return kc, vc, ks, vs
