"""Oracle for whole-block copies between pools (test infrastructure).

What it computes (the plain definition): for each pair ``(s, d)``, block
``d`` of the destination pool becomes block ``s`` of the source pool, every
KV head's K and V tile and, for FP8 pools, the block's K and V scales.  This
is the copy-on-write of a shared block before a sequence writes into it
(page "vLLM的诞生背景：大模型推理的痛点与PagedAttention的破局", limitations
paragraph) and the swapping of blocks to CPU memory and back (page
"PagedAttention 与连续批处理：LLM Serving 的底层架构拆解", section
"PagedAttention：把显存做成虚拟内存").  Pools have the layout
``[num_blocks][num_kv_heads][block_size][head_size]`` (see ``cache_write``);
copies move bit patterns, so no arithmetic is involved.

Reading: the pages do not say what happens when a pair's destination is
another pair's source.  Every copy reads the source pool as it was before
the call, and destinations must be distinct (asserted), which is the only
case in which the order of the copies cannot matter.
"""

import numpy as np


def paged_kv_block_copy(src_key, src_value, dst_key, dst_value, pairs, src_key_scale=None,
                        src_value_scale=None, dst_key_scale=None, dst_value_scale=None):
    """Returns new (dst_key, dst_value, dst_key_scale, dst_value_scale) arrays;
    the inputs are not modified.  Scales are None for non-FP8 pools."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    dsts = [int(d) for d in pairs[:, 1]]
    assert len(set(dsts)) == len(dsts), "destination blocks must be distinct"
    src = [np.array(a, copy=True) if a is not None else None
           for a in (src_key, src_value, src_key_scale, src_value_scale)]
    out = [np.array(a, copy=True) if a is not None else None
           for a in (dst_key, dst_value, dst_key_scale, dst_value_scale)]
    for s, d in pairs:
        for a_src, a_out in zip(src, out):
            if a_out is not None:
                a_out[d] = a_src[s]
    return tuple(out)
