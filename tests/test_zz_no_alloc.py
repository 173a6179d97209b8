"""paged_attention_decode_noalloc (the library's own per-device workspace)
against paged_attention_decode with a caller workspace: bit-identical output
through the C ABI, on two calls in a row, the second with a smaller batch."""

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


@pytest.mark.parametrize("cfg", [3, 5])
def test_noalloc_matches_the_workspace_entry_point(cfg):
    import paged_kv_cache_370_amd as pkv
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    pkv.load()
    big = workloads.make_config(cfg, reduced=True)
    small = workloads.build_workload(f"small-{cfg}", 2, big.H, big.H_kv, big.D, big.block_size,
                                     big.q_dtype, big.cache_dtype, [700, 33], 90 + cfg,
                                     fill="write" if big.cache_dtype == "fp8" else "random")
    for k, w in enumerate((big, small)):
        for ps in (0, 64):
            _say(f"case noalloc cfg{cfg} call {k} {w.name} S={w.S} ps={ps}")
            kc, vc, ks, vs = oracle_caches(w)
            ref = oracle_decode(w, kc, vc, ks, vs)
            dw = DeviceWorkload(w)
            dw.write()
            expect = dw.decode(partition_size=ps).clone()
            got = torch.full_like(dw.q, float("nan"))
            pkv.paged_attention_decode_noalloc(got, dw.q, dw.kc, dw.vc, dw.tables, dw.lens,
                                               w.max_context_len, w.scale, dw.ks, dw.vs,
                                               partition_size=ps)
            torch.cuda.synchronize()
            assert np.array_equal(to_host(got).view(np.uint16), to_host(expect).view(np.uint16))
            err = max_err(out_f64(got), ref)
            _say(f"  bit-identical; max_err vs oracle {err:.3e}")
            assert err <= TOL[w.cache_dtype]


def test_noalloc_rejects_a_batch_beyond_its_workspace():
    import paged_kv_cache_370_amd as pkv
    q = torch.zeros(256, 64, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(8, 8, 8, 128, dtype=torch.bfloat16, device="cuda")
    tables = torch.zeros(256, 4096, dtype=torch.int32, device="cuda")
    lens = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedKVError, match="workspace"):
        pkv.paged_attention_decode_noalloc(torch.empty_like(q), q, kc, kc, tables, lens, 32768,
                                           0.1, partition_size=512)
