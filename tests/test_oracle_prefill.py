"""Pins for the oracle's multi-token (prefill) attention (CPU only).

Pinned against: a causal-masked matrix formulation written here (all query
tokens at once against the sequence's gathered K/V, positions after a
token's own set to -inf before a row softmax), the decode oracle for one
token and for the last token, and causality (poisoning positions after a
token leaves that token's output unchanged)."""

import numpy as np
import pytest

from oracle import paged_attention_decode, paged_attention_prefill, element_values


def _pool(rng, S, M, H_kv, G, D, bs, lens, cache="f32"):
    nbs = [-(-int(n) // bs) for n in lens]
    num_blocks = sum(nbs) + 3
    perm = rng.permutation(num_blocks)
    tables = np.zeros((S, max(nbs)), np.int32)
    k = 0
    for i, nb in enumerate(nbs):
        tables[i, :nb] = perm[k:k + nb]
        k += nb
    kc = rng.standard_normal((num_blocks, H_kv, bs, D)).astype(np.float32)
    vc = rng.standard_normal((num_blocks, H_kv, bs, D)).astype(np.float32)
    q = rng.standard_normal((S, M, H_kv * G, D)).astype(np.float32)
    return q, kc, vc, tables


def _matrix_prefill(q, kc, vc, tables, lens, scale, bs):
    """All M tokens of a sequence at once: Q K^T over the sequence's positions
    (gathered one position at a time), causal mask, row softmax, times V."""
    S, M, H, D = q.shape
    H_kv = kc.shape[1]
    G = H // H_kv
    out = np.zeros(q.shape)
    for i in range(S):
        n = int(lens[i])
        K = np.stack([kc[tables[i][p // bs], :, p % bs, :] for p in range(n)]).astype(np.float64)
        V = np.stack([vc[tables[i][p // bs], :, p % bs, :] for p in range(n)]).astype(np.float64)
        pos = n - M + np.arange(M)
        mask = np.arange(n)[None, :] > pos[:, None]           # [M][n]: future positions
        for h in range(H):
            Sc = q[i, :, h].astype(np.float64) @ K[:, h // G].T * np.float64(np.float32(scale))
            Sc[mask] = -np.inf
            P = np.exp(Sc - Sc.max(axis=1, keepdims=True))
            out[i, :, h] = (P @ V[:, h // G]) / P.sum(axis=1, keepdims=True)
    return out


@pytest.mark.parametrize("seed", range(4))
def test_matches_causal_matrix_formulation(seed):
    rng = np.random.default_rng(seed)
    S, M, H_kv, G, D, bs = 3, int(rng.integers(1, 9)), 2, int(rng.choice([1, 2, 4])), 8, 4
    lens = rng.integers(M, M + 30, size=S)
    q, kc, vc, tables = _pool(rng, S, M, H_kv, G, D, bs, lens)
    a = paged_attention_prefill(q, kc, vc, tables, lens, 0.3, bs)
    b = _matrix_prefill(q, kc, vc, tables, lens, 0.3, bs)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_one_token_is_decode_and_last_token_sees_everything():
    rng = np.random.default_rng(7)
    S, M, H_kv, G, D, bs = 4, 5, 2, 2, 16, 8
    lens = rng.integers(M, 60, size=S)
    q, kc, vc, tables = _pool(rng, S, M, H_kv, G, D, bs, lens)
    out = paged_attention_prefill(q, kc, vc, tables, lens, 0.25, bs)
    last = paged_attention_decode(q[:, -1], kc, vc, tables, lens, 0.25, bs)
    assert np.array_equal(out[:, -1], last)
    one = paged_attention_prefill(q[:, :1], kc, vc, tables, lens, 0.25, bs)
    assert np.array_equal(one[:, 0], paged_attention_decode(q[:, 0], kc, vc, tables, lens, 0.25,
                                                             bs))


def test_future_positions_are_never_read():
    rng = np.random.default_rng(9)
    S, M, H_kv, G, D, bs = 2, 6, 1, 3, 8, 4
    lens = np.array([17, 9])
    q, kc, vc, tables = _pool(rng, S, M, H_kv, G, D, bs, lens)
    ref = paged_attention_prefill(q, kc, vc, tables, lens, 0.5, bs)
    t = 2
    for i in range(S):
        for p in range(int(lens[i]) - M + t + 1, int(lens[i])):   # after token t's position
            kc[tables[i][p // bs], :, p % bs, :] = np.nan
            vc[tables[i][p // bs], :, p % bs, :] = np.nan
    out = paged_attention_prefill(q, kc, vc, tables, lens, 0.5, bs)
    assert np.array_equal(out[:, :t + 1], ref[:, :t + 1])
    assert np.all(np.isnan(out[:, t + 1:]))


def test_beam_fork_sharing_is_invisible():
    """Beams that reference their prompt's blocks give exactly the output of
    the same beams each owning private copies of those blocks."""
    import workloads
    from gpu_helpers import oracle_caches
    w = workloads.make_beam_fork(reduced=True)
    u = workloads.unshare_blocks(w)
    assert u.num_blocks > w.num_blocks
    outs = []
    for x in (w, u):
        kc, vc, _, _ = oracle_caches(x)
        outs.append(paged_attention_prefill(x.q, kc, vc, x.block_tables, x.context_lens, x.scale,
                                            x.block_size))
    assert np.all(np.isfinite(outs[0]))
    assert np.array_equal(outs[0], outs[1])
