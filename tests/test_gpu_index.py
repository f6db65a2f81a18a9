"""GPU parity of the hierarchical sparse indexer (Full and Reindex modes).

Policy:
  * scores: within 1e-5 relative of the oracle (floor 1e-7 x the largest score);
  * selection exactness: the GPU's top-k and pool equal a numpy brute-force
    selection (lexsort by score desc, index asc) applied to the GPU's own
    scores -- bit for bit, no exceptions;
  * end to end: GPU indices vs the oracle's; any difference must be a
    certified near-tie of the oracle's k-th (block) score.
Edge cases: ragged lengths (not multiples of 8, below k, zero), every head
count, n_blocks = 0 / < k / >= k, masked pool entries, duplicate rows (exact
ties), determinism across runs.
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import (DEV, brute_pool, brute_topk, build_gpu_cache, certify_topk,
                        oracle_cache_seq, say, score_close)

pytestmark = pytest.mark.gpu


def _run_full(wl, cache, lens, layer=0, k=None, n_blocks=None):
    q = syn.index_query(wl, layer, DEV)
    w = syn.index_weights(wl, layer, DEV)
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    topk, pool, pool_len, scores = K.index_full(
        cache["idx_codes"], cache["idx_scales"], lt, q, w, k=k or wl.k,
        n_blocks=wl.n_blocks if n_blocks is None else n_blocks, return_scores=True)
    torch.cuda.synchronize()
    return q, w, topk.cpu().numpy(), pool.cpu().numpy(), pool_len.cpu().numpy(), scores.cpu().numpy()


def _check_full(wl, cache, lens, k, n_blocks, layer=0):
    q, w, topk, pool, pool_len, scores = _run_full(wl, cache, lens, layer, k, n_blocks)
    qn, wn = q.cpu().numpy(), w.cpu().numpy()
    certified = 0
    for b, L in enumerate(lens):
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, qn[b], wn[b],
                                            k, 8, n_blocks)
        gs = scores[b, :L]
        score_close(gs, rs)
        # selection exactness on the GPU's own scores
        assert np.array_equal(topk[b], brute_topk(gs, k)), f"seq {b}: top-k is not the exact top-k of the GPU scores"
        if n_blocks > 0:
            bp, bpl, _ = brute_pool(gs, n_blocks)
            assert pool_len[b] == bpl
            assert np.array_equal(pool[b], bp), f"seq {b}: pool is not exact on the GPU scores"
            assert pool_len[b] == rpl
            # pool blocks vs the oracle's, certified near-ties only
            gblk = np.unique(pool[b][pool[b] >= 0] // 8)
            rblk = np.unique(rp[rp >= 0] // 8)
            _, _, rbs = brute_pool(rs, n_blocks)
            certified += certify_topk(gblk, rblk, rbs, n_blocks)
        certified += certify_topk(topk[b], rt, rs, k)
    return certified


@pytest.mark.parametrize("H", [8, 16, 32, 64])
def test_index_full_tiny_workload_shapes(H):
    wl = syn.small("t", 10 + H, B=2, cap=4096, H_idx=H, k=512, n_blocks=64)
    say(f"index_full tiny H={H}")
    cache = build_gpu_cache(wl, 0)
    n = _check_full(wl, cache, [4096, 4096], 512, 64)
    say(f"  certified near-ties: {n}")


@pytest.mark.parametrize("lens,k,nb", [
    ([3000, 2989, 5, 0], 512, 64),      # ragged, below k, empty
    ([5000, 4093, 777, 8], 100, 2048),  # pool covers everything
    ([6000, 6000, 17, 1], 256, 0),       # no pool
    ([6000, 5999, 600, 64], 16, 4),      # n_blocks < k
])
def test_index_full_ragged(lens, k, nb):
    wl = syn.small("r", 7, B=len(lens), cap=6016, H_idx=32, k=k, n_blocks=nb)
    say(f"index_full ragged lens={lens} k={k} nb={nb}")
    cache = build_gpu_cache(wl, 0)
    _check_full(wl, cache, lens, k, nb)


def test_index_full_several_tiles_mid_size():
    wl = syn.small("m", 3, B=3, cap=40000, H_idx=64, k=512, n_blocks=2048, boost_rows=64, boost_factor=4.0)
    say("index_full 3 x 40000, pool 16384")
    cache = build_gpu_cache(wl, 0)
    _check_full(wl, cache, [40000, 39997, 20001], 512, 2048)


def test_duplicate_rows_tie_exactly_and_prefer_lower_index():
    wl = syn.small("d", 5, B=1, cap=4096, H_idx=64, k=64, n_blocks=16)
    cache = build_gpu_cache(wl, 0)
    # copy one row's bytes to many places on the device
    src = 100
    dst = torch.tensor([7, 300, 301, 1999, 2500, 4095], device=DEV)
    for key in ("idx_codes", "idx_scales"):
        cache[key][0, dst] = cache[key][0, src].clone()
    q, w, topk, pool, pool_len, scores = _run_full(wl, cache, [4096])
    s = scores[0]
    assert len(set(s[[src, 7, 300, 301, 1999, 2500, 4095]].view(np.uint32).tolist())) == 1
    assert np.array_equal(topk[0], brute_topk(s, 64))
    # zero every other row, so the seven copies tie for the top and straddle k = 4
    qbits = q
    ic = cache["idx_codes"].clone()
    isc = cache["idx_scales"].clone()
    ic[0] = 0
    ic[0, dst] = cache["idx_codes"][0, src]
    ic[0, src] = cache["idx_codes"][0, src]
    topk2, pool2, pl2 = K.index_full(ic, isc, torch.tensor([4096], dtype=torch.int32, device=DEV), qbits,
                                     w, k=4, n_blocks=2)
    t2 = topk2.cpu().numpy()[0]
    assert list(t2) == [7, src, 300, 301], t2
    p2 = pool2.cpu().numpy()[0]
    assert list(p2[:16]) == list(range(0, 8)) + list(range(96, 104))


def test_all_scores_equal_take_lowest_indices():
    """Every key equal (all-zero codes score exactly 0): the selection takes
    the lowest indices, and its radix search ends before any histogram pass."""
    wl = syn.small("eq", 29, B=2, cap=65536, H_idx=64, k=512, n_blocks=2048)
    say("index_full / index_pool with every score equal, 2 x 65536")
    cache = build_gpu_cache(wl, 0)
    ic = torch.zeros_like(cache["idx_codes"])
    lens = torch.tensor([65536, 40001], dtype=torch.int32, device=DEV)
    q = syn.index_query(wl, 0, DEV)
    w = syn.index_weights(wl, 0, DEV)
    topk, pool, pool_len, scores = K.index_full(ic, cache["idx_scales"], lens, q, w, k=512, n_blocks=2048,
                                                return_scores=True)
    torch.cuda.synchronize()
    assert (scores[0] == 0).all() and (scores[1, :40001] == 0).all()
    assert (topk.cpu().numpy() == np.arange(512)).all()
    assert (pool.cpu().numpy() == np.arange(2048 * 8)).all()
    assert pool_len.cpu().numpy().tolist() == [2048 * 8, 2048 * 8]
    t2 = K.index_pool(ic, cache["idx_scales"], lens, pool, pool_len, q, w, k=512)
    assert (t2.cpu().numpy() == np.arange(512)).all()
    # a pool of 40 entries and k = 512: every entry is taken, the rest is -1
    pl = torch.tensor([40, 40], dtype=torch.int32, device=DEV)
    t3 = K.index_pool(ic, cache["idx_scales"], lens, pool, pl, q, w, k=512).cpu().numpy()
    assert (t3[:, :40] == np.arange(40)).all() and (t3[:, 40:] == -1).all()


@pytest.mark.parametrize("B,cap,kind", [(2, 262144, "random"), (2, 262144, "ties"), (2, 262144, "crowd"),
                                         (1, 524288, "random"), (1, 524288, "ties")])
def test_full_selection_many_blocks_exact(B, cap, kind):
    """Selections over more than 16K blocks per sequence (32 or 64 keys per
    thread), where the prefilter's survivors are compacted before the search:
    the top-k and the pool are exactly the brute-force ones on the GPU's own
    scores.  "ties": the rows are copies of 48 distinct rows, so scores take at
    most 48 values and tie across the threshold; "crowd": a fifth of the rows
    copy the best-scoring row, so the keys at or above the sampled bound
    outnumber the compaction buffer and the selection falls back to the full
    search; "random": the synthetic cache as it is."""
    wl = syn.small("sel" + kind, 31, B=B, cap=cap, H_idx=64, k=512, n_blocks=2048)
    say(f"index_full selection {B} x {cap}, {kind}")
    cache = build_gpu_cache(wl, 0)
    lens = [cap - 12345 * b for b in range(B)]
    g = torch.Generator(device="cpu").manual_seed(1000 + cap + len(kind))
    if kind == "ties":
        src = torch.randint(0, cap, (48,), generator=g)
        pick = src[torch.randint(0, 48, (cap,), generator=g)].to(DEV)
        for key in ("idx_codes", "idx_scales"):
            cache[key][:] = cache[key][:, pick]
    elif kind == "crowd":
        s0 = _run_full(wl, cache, lens)[5]
        for b in range(B):
            best = int(np.nanargmax(s0[b, :lens[b]]))
            at = torch.randperm(cap, generator=g)[: cap // 5].to(DEV)
            for key in ("idx_codes", "idx_scales"):
                cache[key][b, at] = cache[key][b, best].clone()
    _, _, topk, pool, pool_len, scores = _run_full(wl, cache, lens)
    for b, L in enumerate(lens):
        gs = scores[b, :L]
        assert np.array_equal(topk[b], brute_topk(gs, 512)), f"seq {b}: top-k is not exact on the GPU scores"
        bp, bpl, _ = brute_pool(gs, 2048)
        assert pool_len[b] == bpl
        assert np.array_equal(pool[b], bp), f"seq {b}: pool is not exact on the GPU scores"


def test_determinism_two_runs_bitwise():
    wl = syn.small("det", 9, B=2, cap=20000, H_idx=64, k=512, n_blocks=2048)
    cache = build_gpu_cache(wl, 0)
    lens = [20000, 15000]
    a = _run_full(wl, cache, lens)
    b = _run_full(wl, cache, lens)
    for x, y in zip(a[2:5], b[2:5]):   # top-k, pool, pool_len
        assert np.array_equal(x, y)
    for i, n in enumerate(lens):       # scores: only the visible positions are defined
        assert np.array_equal(a[5][i, :n].view(np.uint32), b[5][i, :n].view(np.uint32))


def test_index_pool_matches_oracle_and_reproduces_full_topk():
    wl = syn.small("p", 21, B=3, cap=30000, H_idx=64, k=512, n_blocks=1024, n_reindex=2)
    say("index_pool 3 x 30000")
    cache = build_gpu_cache(wl, 0)
    lens = [30000, 29999, 9000]
    q0, w0, topk, pool, pool_len, scores = _run_full(wl, cache, lens)
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    pool_t = torch.from_numpy(pool).to(DEV)
    pl_t = torch.from_numpy(pool_len).to(DEV)
    # same query as the Full layer -> same top-k, same scores at pool positions
    t_same, ps_same = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool_t, pl_t, q0, w0,
                                   k=512, return_scores=True)
    t_same = t_same.cpu().numpy()
    ps_same = ps_same.cpu().numpy()
    for b in range(3):
        n = pool_len[b]
        assert np.array_equal(t_same[b], topk[b])
        assert np.array_equal(ps_same[b, :n].view(np.uint32), scores[b, pool[b, :n]].view(np.uint32))
    # a Reindex layer's own query vs the oracle (pool from the oracle's own Full layer)
    q1 = syn.index_query(wl, 1, DEV)
    w1 = syn.index_weights(wl, 1, DEV)
    q0n, w0n, q1n, w1n = (t.cpu().numpy() for t in (q0, w0, q1, w1))
    for b, L in enumerate(lens):
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        _, rpool, rpl, _ = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, q0n[b], w0n[b],
                                            512, 8, 1024)
        rt, rps = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, rpool, rpl, q1n[b], w1n[b], 512)
        pt = torch.zeros(1, 1024 * 8, dtype=torch.int32, device=DEV) - 1
        pt[0, :] = torch.from_numpy(rpool).to(DEV)
        gt, gps = K.index_pool(cache["idx_codes"][b:b + 1], cache["idx_scales"][b:b + 1],
                               lt[b:b + 1], pt, torch.tensor([rpl], dtype=torch.int32, device=DEV),
                               q1[b:b + 1], w1[b:b + 1], k=512, return_scores=True)
        gt = gt.cpu().numpy()[0]
        gps = gps.cpu().numpy()[0, :rpl]
        score_close(gps, rps)
        assert np.array_equal(gt, brute_topk(gps, 512, rpool[:rpl]))
        diff = set(gt.tolist()) ^ set(rt.tolist())
        if diff:
            pos_to_score = {int(p): float(s) for p, s in zip(rpool[:rpl], rps)}
            kth = np.sort(rps)[::-1][511]
            for p in diff:
                if p >= 0:
                    assert abs(pos_to_score[p] - kth) <= 2e-5 * abs(kth) + 1e-7 * np.abs(rps).max()


def test_index_pool_masks_invalid_entries():
    wl = syn.small("pm", 23, B=1, cap=2048, H_idx=16, k=8, n_blocks=0)
    cache = build_gpu_cache(wl, 0)
    q = syn.index_query(wl, 0, DEV)
    w = syn.index_weights(wl, 0, DEV)
    # valid entries ascending (the documented precondition); masked entries anywhere
    pool = torch.tensor([[3, 5, -1, 7, 4000, 9, 11, 2047, -5, 12, 13, 1500]], dtype=torch.int32, device=DEV)
    L = 2000
    t, ps = K.index_pool(cache["idx_codes"], cache["idx_scales"], torch.tensor([L], dtype=torch.int32, device=DEV),
                         pool, torch.tensor([12], dtype=torch.int32, device=DEV), q, w, k=8, return_scores=True)
    ps = ps.cpu().numpy()[0]
    assert np.isnan(ps[[2, 4, 7, 8]]).all()
    ref = oracle_cache_seq(wl, 0, 0, cache, need_main=False)
    rt, rps = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, pool.cpu().numpy()[0], 12,
                                q.cpu().numpy()[0], w.cpu().numpy()[0], 8)
    score_close(ps, rps)
    assert np.array_equal(t.cpu().numpy()[0], rt)


@pytest.mark.parametrize("pool_cap,misalign", [(16384, False), (16384, True), (12347, False), (4096, True)])
def test_index_pool_selection_layouts(pool_cap, misalign):
    """Reindex selection exact on the GPU's own pool scores: pool_cap a
    multiple of 8 or ragged, scores in a caller buffer 4 bytes past a 16-byte
    boundary; pool lengths full, ending inside a group, one group and a single
    entry, and zero; k = 512, 100 and 1; the two-phase call equals the fused
    one."""
    B, cap = 4, 40000
    say(f"index_pool selection pool_cap={pool_cap} misaligned={misalign}")
    wl = syn.small("pl", 31 + pool_cap, B=B, cap=cap, H_idx=64, k=512, n_blocks=0)
    cache = build_gpu_cache(wl, 0)
    lt = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(pool_cap + misalign)
    plen = np.array([pool_cap, pool_cap - 5, 9, 0], np.int32)
    pool = np.full((B, pool_cap), -1, np.int32)
    for b in range(B):
        pool[b, :plen[b]] = np.sort(rng.choice(cap, plen[b], replace=False))
    pool_t = torch.from_numpy(pool).to(DEV)
    pl_t = torch.from_numpy(plen).to(DEV)
    q, w = syn.index_query(wl, 0, DEV), syn.index_weights(wl, 0, DEV)
    pws = torch.empty(K.lib().csa2_index_pool_workspace(B, pool_cap, 512), dtype=torch.uint8, device=DEV)
    if misalign:
        ps = torch.empty(B * pool_cap + 1, dtype=torch.float32, device=DEV)[1:].view(B, pool_cap)
        assert ps.data_ptr() % 16 == 4
    else:
        ps = torch.empty(B, pool_cap, dtype=torch.float32, device=DEV)
    K.index_pool_score(cache["idx_codes"], cache["idx_scales"], lt, pool_t, pl_t, q, w, pws, pool_scores=ps)
    fused = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool_t, pl_t, q, w, k=512)
    psn = ps.cpu().numpy()
    for k in (512, 100, 1):
        tk = K.index_pool_select(pool_t, pl_t, pws, k=k, pool_scores=ps).cpu().numpy()
        for b in range(B):
            n = plen[b]
            assert np.array_equal(tk[b], brute_topk(psn[b, :n], k, pool[b, :n])), (k, b)
        if k == 512:
            assert np.array_equal(tk, fused.cpu().numpy())


# ------------------------------------------------------------ FP4 indexer query
# The query quantised to MX-FP4 (E2M1, E8M0 per 32 dims) by csa2_quantize_fp4;
# the oracle quantises the same float query itself (bytes must agree), and
# its dequantised values -- exactly representable in bf16 -- go into the
# unchanged oracle scorer.
def _fp4_query(q_bits):
    qf = q_bits.view(torch.bfloat16).float()
    B, H, _ = qf.shape
    c, s = K.quantize_fp4(qf.reshape(B * H, 128).contiguous(), 32, K.E8M0)
    return qf, c.view(B, H, 64), s.view(B, H, 4)


def _oracle_fp4_query_bits(qf_b, qc_b, qs_b):
    rc, rs = oracle.quantize(qf_b, 32, oracle.E8M0)
    assert np.array_equal(rc, qc_b) and np.array_equal(rs, qs_b), "FP4 query bytes differ from the oracle's"
    v = oracle.dequantize(rc, rs, 32, oracle.E8M0).astype(np.float32)
    u = v.view(np.uint32)
    assert ((u & 0xFFFF) == 0).all(), "a dequantised FP4 query value is not a bf16 value"
    return (u >> 16).astype(np.uint16)


@pytest.mark.parametrize("H", [8, 16, 64])
def test_index_full_fp4_query_matches_oracle(H):
    wl = syn.small("f4", 61 + H, B=3, cap=20000, H_idx=H, k=512, n_blocks=512)
    say(f"index_full FP4 query, H={H}")
    cache = build_gpu_cache(wl, 0)
    lens = [20000, 19993, 7001]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = syn.index_query(wl, 0, DEV)
    w = syn.index_weights(wl, 0, DEV)
    qf, qc, qs = _fp4_query(q)
    topk, pool, pool_len, scores = K.index_full(cache["idx_codes"], cache["idx_scales"], lt, (qc, qs), w,
                                                k=512, n_blocks=512, return_scores=True)
    torch.cuda.synchronize()
    topk, pool, pool_len, scores = (t.cpu().numpy() for t in (topk, pool, pool_len, scores))
    qfn, qcn, qsn, wn = qf.cpu().numpy(), qc.cpu().numpy(), qs.cpu().numpy(), w.cpu().numpy()
    certified = 0
    for b, L in enumerate(lens):
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        qb = _oracle_fp4_query_bits(qfn[b], qcn[b], qsn[b])
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, qb, wn[b], 512, 8, 512)
        gs = scores[b, :L]
        score_close(gs, rs)
        assert np.array_equal(topk[b], brute_topk(gs, 512))
        bp, bpl, _ = brute_pool(gs, 512)
        assert pool_len[b] == bpl == rpl and np.array_equal(pool[b], bp)
        certified += certify_topk(topk[b], rt, rs, 512)
    say(f"  certified near-ties: {certified}")


def test_index_pool_fp4_query_matches_oracle_and_bf16_selection_rules():
    wl = syn.small("p4", 71, B=2, cap=30000, H_idx=64, k=512, n_blocks=1024, n_reindex=1)
    say("index_pool FP4 query")
    cache = build_gpu_cache(wl, 0)
    lens = [30000, 12345]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q0, w0 = syn.index_query(wl, 0, DEV), syn.index_weights(wl, 0, DEV)
    _, pool, pool_len = K.index_full(cache["idx_codes"], cache["idx_scales"], lt, q0, w0, k=512, n_blocks=1024)
    q1, w1 = syn.index_query(wl, 1, DEV), syn.index_weights(wl, 1, DEV)
    qf, qc, qs = _fp4_query(q1)
    # masked entries: one invalid position per sequence
    pool[0, 5] = -1
    pool[1, 9] = 40000
    t, ps = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool, pool_len, (qc, qs), w1, k=512,
                         return_scores=True)
    torch.cuda.synchronize()
    t, ps, pooln, pln = t.cpu().numpy(), ps.cpu().numpy(), pool.cpu().numpy(), pool_len.cpu().numpy()
    for b, L in enumerate(lens):
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        qb = _oracle_fp4_query_bits(qf.cpu().numpy()[b], qc.cpu().numpy()[b], qs.cpu().numpy()[b])
        n = int(pln[b])
        rt, rps = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, pooln[b], n, qb, w1.cpu().numpy()[b], 512)
        score_close(ps[b, :n], rps)
        assert np.array_equal(t[b], brute_topk(ps[b, :n], 512, pooln[b, :n]))
        pos_scores = {int(p): float(s) for p, s in zip(pooln[b, :n], rps) if not np.isnan(s)}
        diff = set(t[b].tolist()) ^ set(rt.tolist())
        kth = np.sort(rps[~np.isnan(rps)])[::-1][511]
        for p in diff:
            if p >= 0:
                assert abs(pos_scores[p] - kth) <= 2e-5 * abs(kth) + 1e-7 * np.nanmax(np.abs(rps))


# ------------------------------------------------- several queries per cache
@pytest.mark.parametrize("B,Q,H,k,nb", [(8, 5, 64, 512, 64), (3, 4, 16, 100, 2048), (2, 1, 8, 64, 16)])
def test_index_full_mq_equals_one_query_calls(B, Q, H, k, nb):
    # each query row of the multi-query call must be bit-identical to the
    # single-query call on its sequence's cache, and match the oracle
    say(f"index_full_mq B={B} Q={Q} H={H} k={k} n_blocks={nb}")
    cap = 6000
    wl = syn.small("mq", 70 + B + Q, B=B, cap=cap, H_idx=H, k=k, n_blocks=nb)
    cache = build_gpu_cache(wl, 0)
    lens = [cap, cap - 11, 999, 5, 0, 4096, 3001, 64][:B]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q = torch.stack([syn.index_query(wl, i, DEV) for i in range(Q)], 1).contiguous()   # [B][Q][H][128]
    w = torch.stack([syn.index_weights(wl, i, DEV) for i in range(Q)], 1).contiguous()  # [B][Q][H]
    topk, pool, pool_len, scores = K.index_full_mq(cache["idx_codes"], cache["idx_scales"], lt, q, w, k=k,
                                                   n_blocks=nb, return_scores=True)
    torch.cuda.synchronize()
    topk, pool, pool_len, scores = (t.cpu().numpy() for t in (topk, pool, pool_len, scores))
    for i in range(Q):
        t1, p1, pl1, s1 = K.index_full(cache["idx_codes"], cache["idx_scales"], lt, q[:, i].contiguous(),
                                       w[:, i].contiguous(), k=k, n_blocks=nb, return_scores=True)
        torch.cuda.synchronize()
        t1, p1, pl1, s1 = (t.cpu().numpy() for t in (t1, p1, pl1, s1))
        assert np.array_equal(topk[:, i], t1) and np.array_equal(pool_len[:, i], pl1)
        assert np.array_equal(pool[:, i], p1)
        for b, L in enumerate(lens):
            assert np.array_equal(scores[b, i, :L].view(np.uint32), s1[b, :L].view(np.uint32))
    # oracle on a sample of (sequence, query) rows
    qn, wn = q.cpu().numpy(), w.cpu().numpy()
    certified = 0
    for b, i in sorted({(0, 0), (0, Q - 1), (B - 1, Q // 2), (min(1, B - 1), 0)}):
        L = lens[b]
        if L == 0:
            assert np.all(topk[b, i] == -1)
            continue
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, qn[b, i], wn[b, i],
                                            k, 8, nb)
        score_close(scores[b, i, :L], rs)
        assert np.array_equal(topk[b, i], brute_topk(scores[b, i, :L], k))
        certified += certify_topk(topk[b, i], rt, rs, k)
        assert pool_len[b, i] == rpl
    say(f"  certified near-ties: {certified}")



@pytest.mark.parametrize("B,Q,H,k,nb,fp4", [(8, 5, 64, 512, 64, False), (3, 3, 32, 700, 300, False),
                                             (2, 1, 8, 64, 16, False), (8, 5, 64, 512, 64, True),
                                             (3, 2, 16, 100, 40, True)])
def test_index_pool_mq_equals_one_query_calls(B, Q, H, k, nb, fp4):
    # Reindex for several queries per cache: each query row rescores its own
    # pool (the multi-query Full call's) and must be bit-identical to the
    # single-query Reindex call on its sequence's cache, and match the oracle
    say(f"index_pool_mq B={B} Q={Q} H={H} k={k} n_blocks={nb} fp4 query={fp4}")
    cap = 6000
    wl = syn.small("pmq", 90 + B + Q, B=B, cap=cap, H_idx=H, k=k, n_blocks=nb)
    cache = build_gpu_cache(wl, 0)
    lens = [cap, 5999, 1001, 7, 0, 4096, 3000, 65][:B]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    q0 = torch.stack([syn.index_query(wl, i, DEV) for i in range(Q)], 1).contiguous()
    w0 = torch.stack([syn.index_weights(wl, i, DEV) for i in range(Q)], 1).contiguous()
    _, pool, pool_len = K.index_full_mq(cache["idx_codes"], cache["idx_scales"], lt, q0, w0, k=k, n_blocks=nb)
    q1 = torch.stack([syn.index_query(wl, Q + i, DEV) for i in range(Q)], 1).contiguous()
    w1 = torch.stack([syn.index_weights(wl, Q + i, DEV) for i in range(Q)], 1).contiguous()
    qarg, qrow = q1, lambda i: q1[:, i].contiguous()
    if fp4:
        # FP4 queries (E2M1 + E8M0 per 32 dims); the oracle scores their
        # dequantised values, exact in bf16
        qc, qs = K.quantize_fp4(q1.view(torch.bfloat16).float().reshape(-1, 128).contiguous(), 32, K.E8M0)
        qc, qs = qc.view(B, Q, H, 64), qs.view(B, Q, H, 4)
        qarg, qrow = (qc, qs), lambda i: (qc[:, i].contiguous(), qs[:, i].contiguous())
    topk, ps = K.index_pool_mq(cache["idx_codes"], cache["idx_scales"], lt, pool, pool_len, qarg, w1, k=k,
                               return_scores=True)
    torch.cuda.synchronize()
    pln = pool_len.cpu().numpy()
    for i in range(Q):
        t1, s1 = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool[:, i].contiguous(),
                              pool_len[:, i].contiguous(), qrow(i), w1[:, i].contiguous(), k=k,
                              return_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(topk[:, i], t1), f"query {i}: top-k differs from the single-query call"
        for b in range(B):
            n = int(pln[b, i])
            assert torch.equal(ps[b, i, :n].view(torch.int32), s1[b, :n].view(torch.int32))
    # the oracle on a sample of (sequence, query) rows
    topk, ps, pooln = topk.cpu().numpy(), ps.cpu().numpy(), pool.cpu().numpy()
    qn, wn = q1.cpu().numpy(), w1.cpu().numpy()
    for b, i in sorted({(0, 0), (0, Q - 1), (B - 1, Q // 2), (min(1, B - 1), Q - 1)}):
        n = int(pln[b, i])
        if n == 0:
            assert np.all(topk[b, i] == -1)
            continue
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        qb = qn[b, i]
        if fp4:
            qb = _oracle_fp4_query_bits(q1.view(torch.bfloat16).float().cpu().numpy()[b, i],
                                        qc.cpu().numpy()[b, i], qs.cpu().numpy()[b, i])
        _, rps = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], lens[b], pooln[b, i], n, qb, wn[b, i], k)
        score_close(ps[b, i, :n], rps)
        assert np.array_equal(topk[b, i], brute_topk(ps[b, i, :n], k, pooln[b, i, :n]))


@pytest.mark.parametrize("B,Q,H", [(8, 5, 64), (3, 2, 16)])
def test_index_full_mq_fp4_query_equals_one_query_calls(B, Q, H):
    # FP4 queries (E2M1 + E8M0 per 32 dims): each query row of the
    # multi-query call is bit-identical to the single-query FP4 call
    say(f"index_full_mq FP4 query B={B} Q={Q} H={H}")
    cap, k, nb = 5000, 512, 64
    wl = syn.small("mq4", 80 + B + Q, B=B, cap=cap, H_idx=H, k=k, n_blocks=nb)
    cache = build_gpu_cache(wl, 0)
    lens = [cap, 4093, 777, 64, 0, 3000, 5000, 1][:B]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qb = torch.stack([syn.index_query(wl, i, DEV) for i in range(Q)], 1).contiguous()
    qc, qs = K.quantize_fp4(qb.view(torch.bfloat16).float().reshape(-1, 128).contiguous(), 32, K.E8M0)
    qc, qs = qc.view(B, Q, H, 64), qs.view(B, Q, H, 4)
    w = torch.stack([syn.index_weights(wl, i, DEV) for i in range(Q)], 1).contiguous()
    topk, pool, pool_len, scores = K.index_full_mq(cache["idx_codes"], cache["idx_scales"], lt, (qc, qs), w, k=k,
                                                   n_blocks=nb, return_scores=True)
    torch.cuda.synchronize()
    for i in range(Q):
        t1, p1, pl1, s1 = K.index_full(cache["idx_codes"], cache["idx_scales"], lt,
                                       (qc[:, i].contiguous(), qs[:, i].contiguous()), w[:, i].contiguous(), k=k,
                                       n_blocks=nb, return_scores=True)
        torch.cuda.synchronize()
        assert torch.equal(topk[:, i], t1) and torch.equal(pool[:, i], p1) and torch.equal(pool_len[:, i], pl1)
        for b, L in enumerate(lens):
            assert torch.equal(scores[b, i, :L].view(torch.int32), s1[b, :L].view(torch.int32))
    # the oracle on a sample of (sequence, query) rows, scoring the dequantised
    # FP4 query (exact in bf16)
    topk, pool, pool_len, scores = (t.cpu().numpy() for t in (topk, pool, pool_len, scores))
    qfn = qb.view(torch.bfloat16).float().cpu().numpy()
    qcn, qsn, wn = qc.cpu().numpy(), qs.cpu().numpy(), w.cpu().numpy()
    certified = 0
    for b, i in sorted({(0, 0), (0, Q - 1), (B - 1, Q // 2), (min(1, B - 1), Q - 1), (min(2, B - 1), 0)}):
        L = lens[b]
        if L == 0:
            assert np.all(topk[b, i] == -1) and pool_len[b, i] == 0
            continue
        ref = oracle_cache_seq(wl, b, 0, cache, need_main=False)
        qbits = _oracle_fp4_query_bits(qfn[b, i], qcn[b, i], qsn[b, i])
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, qbits, wn[b, i], k, 8,
                                            nb)
        score_close(scores[b, i, :L], rs)
        assert np.array_equal(topk[b, i], brute_topk(scores[b, i, :L], k))
        bp, bpl, _ = brute_pool(scores[b, i, :L], nb)
        assert pool_len[b, i] == bpl == rpl and np.array_equal(pool[b, i], bp)
        certified += certify_topk(topk[b, i], rt, rs, k)
    say(f"  certified near-ties against the oracle: {certified}")


# ------------------------------------------------ the two phases of each call
def test_index_phases_equal_fused_calls():
    # scoring then selection as separate calls gives the fused calls' results
    # bit for bit, with the scores in the workspace or in a caller buffer
    say("index phases: score + select against the fused calls")
    B, cap, k, nb = 3, 20000, 512, 512
    wl = syn.small("ph", 77, B=B, cap=cap, H_idx=64, k=k, n_blocks=nb, n_reindex=1)
    cache = build_gpu_cache(wl, 0)
    lens = [cap, cap - 7, 7001]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ic, isc = cache["idx_codes"], cache["idx_scales"]
    q, w = syn.index_query(wl, 0, DEV), syn.index_weights(wl, 0, DEV)
    t0, p0, pl0, s0 = K.index_full(ic, isc, lt, q, w, k=k, n_blocks=nb, return_scores=True)
    L = K.lib()
    nws = L.csa2_index_full_workspace(B, cap, k, 8, nb)
    ws1 = torch.empty(nws, dtype=torch.uint8, device=DEV)
    K.index_full_score(ic, isc, lt, q, w, ws1)
    t1, p1, pl1 = K.index_full_select(cap, lt, ws1, k=k, n_blocks=nb)
    ws2 = torch.empty(nws, dtype=torch.uint8, device=DEV)
    s2 = torch.empty(B, cap, dtype=torch.float32, device=DEV)
    K.index_full_score(ic, isc, lt, q, w, ws2, scores=s2)
    t2, p2, pl2 = K.index_full_select(cap, lt, ws2, k=k, n_blocks=nb, scores=s2)
    q1, w1 = syn.index_query(wl, 1, DEV), syn.index_weights(wl, 1, DEV)
    tk0, ps0 = K.index_pool(ic, isc, lt, p0, pl0, q1, w1, k=k, return_scores=True)
    pws = torch.empty(L.csa2_index_pool_workspace(B, nb * 8, k), dtype=torch.uint8, device=DEV)
    K.index_pool_score(ic, isc, lt, p0, pl0, q1, w1, pws)
    tk1 = K.index_pool_select(p0, pl0, pws, k=k)
    pws2 = torch.empty_like(pws)
    ps2 = torch.empty(B, nb * 8, dtype=torch.float32, device=DEV)
    K.index_pool_score(ic, isc, lt, p0, pl0, q1, w1, pws2, pool_scores=ps2)
    tk2 = K.index_pool_select(p0, pl0, pws2, k=k, pool_scores=ps2)
    torch.cuda.synchronize()
    for t, p, pl in ((t1, p1, pl1), (t2, p2, pl2)):
        assert torch.equal(t, t0) and torch.equal(p, p0) and torch.equal(pl, pl0)
    for b, Lb in enumerate(lens):
        assert torch.equal(s2[b, :Lb].view(torch.int32), s0[b, :Lb].view(torch.int32))
    assert torch.equal(tk1, tk0) and torch.equal(tk2, tk0)
    n = pl0.cpu().numpy()
    for b in range(B):
        assert torch.equal(ps2[b, : n[b]].view(torch.int32), ps0[b, : n[b]].view(torch.int32))
