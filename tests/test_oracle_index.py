"""Pins of the oracle's indexer: scoring, position top-k, block pool, Reindex.

The pages define the selections (position top-512 and block top-2048 from one
scoring, block score = max, pool = expanded blocks, Reindex = rescoring the
pool) but print no worked example.  The score formula comes with the tiny
Full-layer workload.  Pins: per-head reduction to a plain dot product (numpy),
linearity in the head weights, exact power-of-two equivariance, brute-force
orderings (numpy.lexsort), and the pool containment invariant.
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import oracle
from refdeq import bf16_to_f64, dequant


def _cache(n, seed, scale=1.0):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((n, 128)) * scale).astype(np.float32)
    return x, *oracle.quantize(x, 32, oracle.E8M0)


def _q(H, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(H, 128, generator=g)
    return syn.as_bf16_bits(q).numpy()


def test_score_single_head_is_relu_dot():
    _, c, s = _cache(300, 1)
    q = _q(1, 2)
    k = dequant(c, s, 32, 0)
    want = np.maximum(k @ bf16_to_f64(q)[0], 0.0)
    got = oracle.score(c, s, q, np.ones(1, np.float32))
    np.testing.assert_allclose(got, want.astype(np.float32), rtol=2e-7, atol=0)


def test_score_is_weighted_sum_over_heads():
    _, c, s = _cache(200, 3)
    H = 8
    q = _q(H, 4)
    k = dequant(c, s, 32, 0)
    qf = bf16_to_f64(q)
    per_head = []
    for h in range(H):
        w = np.zeros(H, np.float32)
        w[h] = 1.0
        per_head.append(oracle.score(c, s, q, w).astype(np.float64))
        np.testing.assert_allclose(per_head[-1], np.maximum(k @ qf[h], 0), rtol=2e-7)
    w = np.random.default_rng(5).uniform(0, 1, H).astype(np.float32)
    got = oracle.score(c, s, q, w).astype(np.float64)
    lin = sum(float(w[h]) * per_head[h] for h in range(H))
    np.testing.assert_allclose(got, lin, rtol=1e-6)
    assert (got >= 0).all()
    # negative weights stay linear
    w2 = -w
    np.testing.assert_allclose(oracle.score(c, s, q, w2), -got, rtol=1e-7)


def test_score_power_of_two_equivariance():
    x, c, s = _cache(256, 6)
    q = _q(16, 7)
    w = np.random.default_rng(8).uniform(0, 1, 16).astype(np.float32)
    base = oracle.score(c, s, q, w)
    c4, s4 = oracle.quantize(x * 4, 32, oracle.E8M0)
    assert (c4 == c).all() and (s4.astype(int) == s.astype(int) + 2).all()
    assert (oracle.score(c4, s4, q, w) == 4 * base).all()


def _brute_topk(scores, k, ids=None):
    ids = np.arange(len(scores)) if ids is None else np.asarray(ids)
    ok = ~np.isnan(scores)
    sc, idv = scores[ok], ids[ok]
    order = np.lexsort((idv, -sc.astype(np.float64)))
    pick = np.sort(idv[order[:k]])
    return np.concatenate([pick, -np.ones(k - len(pick), np.int64)])


@pytest.mark.parametrize("trial", range(40))
def test_topk_brute_force_with_ties(trial):
    g = np.random.default_rng(100 + trial)
    n = int(g.integers(0, 64))
    k = int(g.integers(1, 17))
    mode = trial % 4
    if mode == 0:
        s = g.standard_normal(n).astype(np.float32)
    elif mode == 1:
        s = np.full(n, 1.5, np.float32)  # all equal
    elif mode == 2:
        s = g.integers(0, 4, n).astype(np.float32)  # many ties
    else:
        s = g.integers(-2, 3, n).astype(np.float32)
        s[g.random(n) < 0.2] = np.nan  # absent entries
    got = oracle.topk_ids(s, k)
    want = _brute_topk(s, k)
    assert (got == want).all(), (s, k, got, want)
    sel = got[got >= 0]
    assert len(sel) == min(k, int((~np.isnan(s)).sum()))
    rest = np.setdiff1d(np.where(~np.isnan(s))[0], sel)
    if len(sel) and len(rest):
        assert s[sel].min() >= s[rest].max()
        # ties at the threshold take the lowest positions
        thr = s[sel].min()
        tied_out = rest[s[rest] == thr]
        tied_in = sel[s[sel] == thr]
        if len(tied_out):
            assert tied_in.max() < tied_out.min()


@pytest.mark.parametrize("L,nb", [(64, 3), (61, 4), (4096, 64), (1000, 2048), (8, 1), (0, 4)])
def test_block_pool_invariants(L, nb):
    g = np.random.default_rng(L + nb)
    s = g.integers(0, 50, L).astype(np.float32)  # ties on purpose
    pool, pl, bs = oracle.block_pool(s, 8, nb)
    nblk = (L + 7) // 8
    # block scores are maxima (upper bounds of every member)
    for b in range(nblk):
        assert bs[b] == s[8 * b: 8 * b + 8].max()
    # the chosen blocks are exactly the brute-force top-nb by (bscore desc, block asc)
    want_blocks = _brute_topk(bs, nb)
    want_blocks = want_blocks[want_blocks >= 0]
    want_pool = np.concatenate([np.arange(8 * b, min(8 * b + 8, L)) for b in want_blocks]) if len(want_blocks) else np.zeros(0, int)
    assert pl == len(want_pool)
    assert (pool[:pl] == want_pool).all()
    assert (pool[pl:] == -1).all()
    assert (np.diff(pool[:pl]) > 0).all()
    if L % 8 == 0:
        assert pl == 8 * min(nb, L // 8)
    if nb * 8 >= L:
        assert (pool[:pl] == np.arange(L)).all()


def test_top512_is_inside_the_2048_block_pool():
    # with n_blocks >= k every top-k position is in the pool: each block ranked
    # ahead of block(p) holds a distinct position ranked ahead of p.
    x, c, s = _cache(20000, 11)
    q = _q(8, 12)
    w = np.random.default_rng(13).uniform(0, 1, 8).astype(np.float32)
    topk, pool, pl, sc = oracle.index_full(c, s, 20000, q, w, 512, 8, 2048)
    assert pl == 16384
    assert np.isin(topk, pool[:pl]).all()
    # both selections come from the same scores
    assert (topk == oracle.topk_ids(sc, 512)).all()
    p2, pl2, _ = oracle.block_pool(sc, 8, 2048)
    assert pl2 == pl and (p2 == pool).all()
    # and those scores are the per-position scores
    assert (sc == oracle.score(c, s, q, w)).all()


def test_reindex_with_same_query_reproduces_full_topk():
    x, c, s = _cache(9000, 21)
    q = _q(16, 22)
    w = np.random.default_rng(23).uniform(0, 1, 16).astype(np.float32)
    topk, pool, pl, sc = oracle.index_full(c, s, 9000, q, w, 512, 8, 1024)
    t2, ps = oracle.index_pool(c, s, 9000, pool, pl, q, w, 512)
    assert (t2 == topk).all()
    assert (ps == sc[pool[:pl]]).all()
    # a different query picks inside the same pool
    q2 = _q(16, 24)
    t3, _ = oracle.index_pool(c, s, 9000, pool, pl, q2, w, 512)
    assert np.isin(t3, pool[:pl]).all()


def test_reindex_masks_invalid_pool_entries():
    x, c, s = _cache(100, 31)
    q = _q(8, 32)
    w = np.ones(8, np.float32)
    pool = np.array([3, 5, -1, 7, 150, 9, 11], np.int32)
    t, ps = oracle.index_pool(c, s, 100, pool, 7, q, w, 4)
    assert np.isnan(ps[2]) and np.isnan(ps[4])
    valid = np.array([3, 5, 7, 9, 11])
    full = oracle.score(c, s, q, w)
    assert (t == _brute_topk(full[valid], 4, valid)).all()


def test_duplicate_rows_tie_and_prefer_lower_position():
    x, c, s = _cache(64, 41)
    for dst in [5, 17, 40, 63]:
        c[dst] = c[2]
        s[dst] = s[2]
    q = _q(8, 42)
    w = np.ones(8, np.float32)
    sc = oracle.score(c, s, q, w)
    assert sc[5] == sc[2] == sc[17] == sc[40] == sc[63]
    k = int((sc > sc[2]).sum()) + 2
    t = oracle.topk_ids(sc, k)
    assert 2 in t and 5 in t and 17 not in t


def test_boosted_workload_rows_rank_high():
    wl = syn.small("b", 1, B=1, cap=8192, H_idx=8, k=512, n_blocks=64, boost_rows=64, boost_factor=4.0)
    x = syn.idx_values(wl, 0).numpy()
    c, s = oracle.quantize(x, 32, oracle.E8M0)
    q = syn.index_query(wl, 0).numpy()[0]
    w = syn.index_weights(wl, 0).numpy()[0]
    sc = oracle.score(c, s, q, w)
    x0 = syn.normal((8192, 128), wl.seed, "idx", 0).numpy()
    c0, s0 = oracle.quantize(x0, 32, oracle.E8M0)
    sc0 = oracle.score(c0, s0, q, w)
    pos = syn.boost_positions(wl, 0).numpy()
    assert (sc[pos] == 4 * sc0[pos]).all()
    t = oracle.topk_ids(sc, 512)
    assert np.isin(pos, t).sum() >= 48  # most boosted rows rank in the top 6%
