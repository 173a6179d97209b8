"""CPU oracle for paged KV write and PagedAttention decode.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or run anything in this package.  The library
(``paged_kv_cache_370_amd``) never imports it and must fail loudly rather than
fall back to it.

The oracle is a plain, slow, obviously-correct statement of what the hot path
computes, written from the three web pages on PagedAttention:

* page "企业官网建设流程全解析" (dpshk.com article on PagedAttention), sections
  2.1 (Block / BlockTable), 2.2 (attention formula and blockwise loop),
  2.3 (sharing by reference count), 3.2 (FP8 storage of blocks);
* page "vLLM的诞生背景：大模型推理的痛点与PagedAttention的破局", section
  "PagedAttention的破局思路" (logical blocks mapped to physical blocks through
  a block table);
* page "PagedAttention 与连续批处理：LLM Serving 的底层架构拆解", section
  "PagedAttention：把显存做成虚拟内存" (attention finds each page through the
  page table; pages swapped to CPU memory and back);
* copy-on-write of shared blocks: page "vLLM的诞生背景…", limitations
  paragraph (``block_copy``).

Floating point is evaluated in float64, except where a reading fixes float32
(the FP8 scale and the division before encoding; see ``cache_write``).

Array conventions (shared with the C ABI only by documentation, never by code):

* float32 arrays hold fp32 data;
* uint16 arrays hold bfloat16 bit patterns;
* uint8 arrays hold OCP FP8 E4M3FN codes.

Every function here has an independent pin in ``tests/test_oracle_*.py``
(brute force, a library routine, closed forms, invariants, format constants).
"""

from .fp8_e4m3 import fp8_decode, fp8_encode, FP8_MAX, fp8_finite_values
from .cache_write import paged_kv_cache_write
from .block_copy import paged_kv_block_copy
from .attention import (
    paged_attention_decode,
    paged_attention_decode_one,
    paged_attention_prefill,
    gather_sequence,
    element_values,
)

__all__ = [
    "fp8_decode",
    "fp8_encode",
    "FP8_MAX",
    "fp8_finite_values",
    "paged_kv_cache_write",
    "paged_kv_block_copy",
    "paged_attention_decode",
    "paged_attention_decode_one",
    "paged_attention_prefill",
    "gather_sequence",
    "element_values",
]
