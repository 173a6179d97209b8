"""The bf16 split partials (CPU only): what storing each partition's
unnormalised output acc_p as bf16 adds to the error of the merged result.

The kernels keep each partition's running maximum m_p and sum l_p in float32
and its output acc_p = sum_t exp(s_t - m_p) v_t in bf16 (rounded to nearest
even from the float32 accumulator) when the queries are bf16; the merge
    out = sum_p e^{m_p - M} acc_p / sum_p e^{m_p - M} l_p
is a convex combination of the partitions' outputs acc_p / l_p, so a
relative rounding of at most 2^-9 on every acc_p moves each output element
by at most 2^-9 * max_t |V[t][d]| (acc_p / l_p is itself a convex combination
of V rows).  The test takes the partials exactly (float64), rounds acc_p the
way the kernels store it, merges, and checks the change against that bound
and against the 2e-2 bf16 tolerance, on the 32K-context shape (64 partitions
of 512 tokens) and on FP8 data (partitions of 1024 and 4096 tokens).
"""

import numpy as np
import pytest

import workloads
from oracle.fp8_e4m3 import fp8_decode, fp8_encode

U = 2.0 ** -9


def _bf16_store(x64):
    """float64 -> float32 accumulator -> bf16 bits (RNE) -> value."""
    bits = workloads.bf16_bits(x64.astype(np.float32))
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _split_merge(q, K, V, scale, P, round_acc):
    """Softmax attention of q [G][D] over K, V [n][D] through partitions of P
    tokens, each kept as (m_p, l_p, acc_p); acc_p optionally bf16-rounded."""
    s = (q @ K.T) * scale                                   # [G][n]
    n = K.shape[0]
    ms, ls, accs = [], [], []
    for a in range(0, n, P):
        sp = s[:, a:a + P]
        m = sp.max(axis=1, keepdims=True)
        e = np.exp(sp - m)
        acc = e @ V[a:a + P]
        ms.append(m); ls.append(e.sum(axis=1, keepdims=True))
        accs.append(_bf16_store(acc) if round_acc else acc)
    M = np.max(np.concatenate(ms, axis=1), axis=1, keepdims=True)
    wts = [np.exp(m - M) for m in ms]
    L = sum(w * l for w, l in zip(wts, ls))
    return sum(w * acc for w, acc in zip(wts, accs)) / L


def _exact(q, K, V, scale):
    s = (q @ K.T) * scale
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e @ V) / e.sum(axis=1, keepdims=True)


def _bf16_values(rng, shape):
    return (workloads.bf16_bits(rng.standard_normal(shape, dtype=np.float32)).astype(np.uint32)
            << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("n,P,fp8", [(32768, 512, False), (8192, 1024, True), (8192, 4096, True),
                                     (2000, 512, False)])
def test_bf16_partials_stay_within_the_convex_bound(n, P, fp8):
    rng = np.random.default_rng(n + P)
    G, D = 8, 128
    q = _bf16_values(rng, (G, D))
    K = _bf16_values(rng, (n, D))
    V = _bf16_values(rng, (n, D))
    if fp8:                                    # dequantised E4M3 values, one scale per 16 rows
        for X in (K, V):
            for a in range(0, n, 16):
                sc = np.float32(max(np.abs(X[a:a + 16]).max() / 448.0, 1e-38))
                X[a:a + 16] = fp8_decode(fp8_encode((X[a:a + 16] / sc).astype(np.float32))) * sc
    scale = float(np.float32(1.0 / np.sqrt(D)))
    exact = _exact(q, K, V, scale)
    split = _split_merge(q, K, V, scale, P, round_acc=False)
    assert np.max(np.abs(split - exact)) <= 1e-12          # the merge itself is exact
    rounded = _split_merge(q, K, V, scale, P, round_acc=True)
    added = np.abs(rounded - exact)
    bound = U * np.max(np.abs(V), axis=0)[None, :]
    assert np.all(added <= bound * (1 + 1e-6))
    # far inside the bf16 tolerance (and the output's own final bf16 rounding)
    assert added.max() <= 2e-2 / 8
    print(f"n={n} P={P} fp8={fp8}: partitions {-(-n // P)}, added max {added.max():.2e}, "
          f"mean {added.mean():.2e}, bound {bound.max():.2e}")
