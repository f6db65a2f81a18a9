"""GPU parity of the paged cache: every paged call against the contiguous
call on the same data, bit for bit.

The caches of the contiguous tests are copied into a pool of pages in a
seeded random order (page ids beyond each sequence's length are left as
garbage, which the kernels must clamp into the pool).  Index top-k, pool,
pool length and scores must equal the contiguous call's; the returned pool
rows must be exactly the table's translation of the returned positions;
attention over the returned rows must equal attention over the positions
(same rows, same order, so the same bits); appends must land on the rows
the table names.

The paged results also face the oracle directly: the logical cache of each
sequence is gathered from the pool through the table on the host, checked
equal to the oracle's quantisation of the generator's values, and the
oracle's index_full, index_pool and attention on it are compared with the
paged top-k, pool, pool scores, Reindex top-k and attention outputs (scores
within tolerance, selections exact on the GPU's own scores and equal to the
oracle's up to certified near-ties, attention within 1e-2).
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import DEV, attn_close, brute_pool, brute_topk, build_gpu_cache, certify_topk, say, score_close

pytestmark = pytest.mark.gpu

PLANES = (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4))


def _paginate(cache, lens, shift, seed, spare=7):
    """Pool + table holding the same entries as the contiguous cache."""
    B, cap = cache["idx_codes"].shape[:2]
    P = 1 << shift
    mp = (cap + P - 1) // P
    n_pages = B * mp + spare
    g = np.random.default_rng(seed)
    perm = g.permutation(n_pages).astype(np.int32)
    table = perm[: B * mp].reshape(B, mp).copy()
    pool = K.paged_alloc(n_pages, shift, DEV)
    for b in range(B):
        for j in range(mp):
            lo, hi = j * P, min(cap, (j + 1) * P)
            r0 = int(table[b, j]) * P
            for key, _ in PLANES:
                pool[key][r0:r0 + hi - lo] = cache[key][b, lo:hi]
        # pages past the length: garbage ids (clamped by the kernels)
        used = (lens[b] + P - 1) // P
        table[b, used:] = np.where(np.arange(mp - used) % 2 == 0, -5, 1 << 30)[: mp - used]
    return pool, torch.from_numpy(table).to(DEV), table


def _logical(pool, tabn, shift, b, L):
    """Sequence b's first L entries gathered from the pool through the table (host)."""
    rows = _phys(tabn, shift, b, np.arange(L))
    return {key: pool[key].cpu().numpy()[rows] for key, _ in PLANES}


def _oracle_planes(wl, b, L, fmt, logical):
    """The oracle's quantisation of sequence b's first L entries, checked equal
    to the entries the table addresses."""
    xi = syn.idx_values(wl, b, DEV, rows=wl.cap).cpu().numpy()[:L]
    xm = syn.main_values(wl, b, DEV, rows=wl.cap).cpu().numpy()[:L]
    ic, isc = oracle.quantize(xi, 32, oracle.E8M0)
    mc, ms = oracle.quantize(xm, 16, fmt)
    for key, ref in (("idx_codes", ic), ("idx_scales", isc), ("main_codes", mc), ("main_scales", ms)):
        assert np.array_equal(logical[key], ref), f"sequence {b}: paged {key} differ from the oracle's"
    return dict(idx_codes=ic, idx_scales=isc, main_codes=mc, main_scales=ms)


def _phys(table, shift, b, pos):
    pos = np.asarray(pos)
    P = 1 << shift
    out = np.where(pos >= 0, table[b, np.maximum(pos, 0) // P].astype(np.int64) * P + np.maximum(pos, 0) % P, -1)
    return out.astype(np.int32)


@pytest.mark.parametrize("shift,fmt", [(6, 0), (8, 1)])
def test_paged_index_and_attention_equal_contiguous(shift, fmt):
    say(f"paged cache shift={shift} fmt={fmt}")
    B, cap = 3, 4096
    wl = syn.small("pg", 90 + shift, B=B, cap=cap, H_idx=16, k=256, n_blocks=64)
    cache = build_gpu_cache(wl, fmt)
    lens = [cap - 37, 1000, 300]
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    pool, tab, tabn = _paginate(cache, lens, shift, 5 + shift)
    q, w = syn.index_query(wl, 0, DEV), syn.index_weights(wl, 0, DEV)
    t0, p0, pl0, s0 = K.index_full(cache["idx_codes"], cache["idx_scales"], lt, q, w, k=256, n_blocks=64,
                                   return_scores=True)
    t1, tr1, p1, pr1, pl1, s1 = K.index_full_paged(pool, tab, shift, lt, q, w, k=256, n_blocks=64,
                                                   return_scores=True)
    torch.cuda.synchronize()
    t0, p0, pl0, s0 = (x.cpu().numpy() for x in (t0, p0, pl0, s0))
    t1, tr1, p1, pr1, pl1, s1 = (x.cpu().numpy() for x in (t1, tr1, p1, pr1, pl1, s1))
    assert np.array_equal(t0, t1) and np.array_equal(p0, p1) and np.array_equal(pl0, pl1)
    for b, L in enumerate(lens):
        assert np.array_equal(s0[b, :L].view(np.uint32), s1[b, :L].view(np.uint32))
        assert np.array_equal(tr1[b], _phys(tabn, shift, b, t1[b]))
        assert np.array_equal(pr1[b], _phys(tabn, shift, b, p1[b]))
    # Reindex over the pool rows
    q2, w2 = syn.index_query(wl, 1, DEV), syn.index_weights(wl, 1, DEV)
    pool_t, pool_r, pool_l = (torch.from_numpy(x).to(DEV) for x in (p1, pr1, pl1))
    tk0 = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool_t, pool_l, q2, w2, k=256)
    tk1, tkr1 = K.index_pool_rows(pool, pool_t, pool_r, pool_l, q2, w2, k=256)
    torch.cuda.synchronize()
    tk0, tk1, tkr1 = (x.cpu().numpy() for x in (tk0, tk1, tkr1))
    assert np.array_equal(tk0, tk1)
    for b in range(B):
        assert np.array_equal(tkr1[b], _phys(tabn, shift, b, tk1[b]))
    # attention over the rows, with a main-format window taken from the cache
    qa = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(shift)) * 0.5).to(DEV)
    swa_len = torch.tensor([128, 40, 0], dtype=torch.int32, device=DEV)
    win = dict(swa_codes=cache["main_codes"], swa_scales=cache["main_scales"], swa_len=swa_len, swa_stride=cap,
               swa_cap=128)
    o0, l0 = K.sparse_attn_decode(qa, cache["main_codes"], cache["main_scales"], lt, torch.from_numpy(t1).to(DEV),
                                  fmt, return_lse=True, **win)
    o1, l1 = K.sparse_attn_decode_rows(qa, pool, torch.from_numpy(tr1).to(DEV), fmt, return_lse=True, **win)
    _, ps1 = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pool_t, pool_l, q2, w2, k=256,
                          return_scores=True)
    torch.cuda.synchronize()
    assert torch.equal(o0.cpu(), o1.cpu()) and torch.equal(l0.cpu(), l1.cpu())

    # ---- the paged results against the oracle on the logical cache
    qn, wn, q2n, w2n = (x.cpu().numpy() for x in (q, w, q2, w2))
    ps1, o1n, swl = ps1.cpu().numpy(), o1.cpu(), swa_len.cpu().numpy()
    cert = 0
    for b, L in enumerate(lens):
        ref = _oracle_planes(wl, b, L, fmt, _logical(pool, tabn, shift, b, L))
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"], ref["idx_scales"], L, qn[b], wn[b], 256, 8, 64)
        score_close(s1[b, :L], rs)
        assert np.array_equal(t1[b], brute_topk(s1[b, :L], 256))
        bp, bpl, _ = brute_pool(s1[b, :L], 64)
        assert pl1[b] == bpl == rpl and np.array_equal(p1[b], bp)
        cert += certify_topk(t1[b], rt, rs, 256)
        n = int(pl1[b])
        rti, rps = oracle.index_pool(ref["idx_codes"], ref["idx_scales"], L, p1[b], n, q2n[b], w2n[b], 256)
        score_close(ps1[b, :n], rps)
        assert np.array_equal(tk1[b], brute_topk(ps1[b, :n], 256, p1[b, :n]))
        pos_scores = np.full(L, np.nan)
        pos_scores[p1[b, :n]] = rps
        cert += certify_topk(tk1[b], rti, pos_scores, 256)
        sl = int(swl[b])
        ro, _ = oracle.attention(qa[b].cpu().numpy(), ref["main_codes"], ref["main_scales"], L, fmt, t1[b],
                                 ref["main_codes"][:sl], ref["main_scales"][:sl], sl, 1 / np.sqrt(512))
        attn_close(o1n[b:b + 1], ro[None])
    say(f"  paged against the oracle: certified near-ties {cert}")


def test_paged_attention_throughput_kernel_equal_contiguous():
    # 48 sequences with 64 heads take the all-heads kernel
    say("paged attention, throughput kernel")
    B, cap, shift, k = 48, 1024, 7, 512
    wl = syn.small("pga", 95, B=B, cap=cap, H_idx=8, k=k, n_blocks=0)
    cache = build_gpu_cache(wl, 0)
    lens = [cap] * B
    lt = torch.tensor(lens, dtype=torch.int32, device=DEV)
    pool, tab, tabn = _paginate(cache, lens, shift, 11)
    g = np.random.default_rng(3)
    topk = np.stack([g.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)
    topk[0, :7] = -1
    rows = np.stack([_phys(tabn, shift, b, topk[b]) for b in range(B)])
    # the FP8 window rings come from the oracle's ring writer (host), so the
    # attention check below shares its inputs with the oracle
    lat = syn.as_bf16_bits(torch.randn(B, 128, 512, generator=torch.Generator().manual_seed(4)))
    ring = oracle.window_write(lat.numpy().view(np.uint16), np.full(B, 5000, np.int64), 128, rope=True)
    win = dict(swa_codes=torch.from_numpy(ring["data"]).to(DEV), swa_scales=torch.from_numpy(ring["scales"]).to(DEV),
               swa_len=torch.from_numpy(ring["swa_len"]).to(DEV), swa_stride=128, swa_cap=128, swa_fmt=K.SWA_FP8)
    qa = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(9)) * 0.5).to(DEV)
    qp = torch.arange(B, dtype=torch.int64, device=DEV) * 977 + 5128
    o0 = K.sparse_attn_decode(qa, cache["main_codes"], cache["main_scales"], lt, torch.from_numpy(topk).to(DEV), 0,
                              q_pos=qp, **win)
    o1 = K.sparse_attn_decode_rows(qa, pool, torch.from_numpy(rows).to(DEV), 0, q_pos=qp, **win)
    torch.cuda.synchronize()
    assert torch.equal(o0.cpu(), o1.cpu())
    # against the oracle on the logical cache, one sequence of each XCD residue
    o1n, qpn, qan = o1.cpu(), qp.cpu().numpy(), qa.cpu().numpy()
    worst = 0.0
    for b in (0, 9, 18, 27, 36, 45, 6, 15):  # b mod 8 = 0..7
        ref = _oracle_planes(wl, b, cap, 0, _logical(pool, tabn, shift, b, cap))
        ro, _ = oracle.attention(qan[b], ref["main_codes"], ref["main_scales"], cap, 0, topk[b], ring["data"][b],
                                 ring["scales"][b], int(ring["swa_len"][b]), 1 / np.sqrt(512), q_pos=int(qpn[b]),
                                 swa_fmt=1)
        worst = max(worst, attn_close(o1n[b:b + 1], ro[None]))
    say(f"  paged throughput kernel against the oracle: worst rel err {worst:.2e}")


@pytest.mark.parametrize("m", [1, 2])
def test_paged_append_lands_on_table_rows(m):
    say(f"paged append m={m}")
    B, cap, shift = 4, 512, 6
    P = 1 << shift
    wl = syn.Workload("pgw", 97 + m, B=B, cap=1, H_idx=8, k=1, block=8, n_blocks=0, write_tokens=8 * B, write_m=1)
    lat, gate, wproj = syn.write_inputs(wl, DEV)
    cont = {key: torch.zeros(B, cap, wd, dtype=torch.uint8, device=DEV) for key, wd in PLANES}
    mp = cap // P
    n_pages = B * mp + 3
    perm = np.random.default_rng(m).permutation(n_pages).astype(np.int32)
    tabn = perm[: B * mp].reshape(B, mp)
    tab = torch.from_numpy(tabn).to(DEV)
    pool = K.paged_alloc(n_pages, shift, DEV)
    l0 = torch.tensor([0, 63, 64, cap - 3], dtype=torch.int32, device=DEV)   # page edges and a full sequence
    l1 = l0.clone()
    st0 = K.append_state(B, DEV) if m == 2 else None
    st1 = K.append_state(B, DEV) if m == 2 else None
    for step in range(8):
        tok = lat[step * B:(step + 1) * B]
        gt = gate[step * B:(step + 1) * B] if gate is not None else tok
        K.cache_append(tok, gt, m, wproj, 0, cont, l0, state=st0, rope=True)
        K.cache_append_paged(tok, gt, m, wproj, 0, pool, tab, shift, l1, state=st1, rope=True)
    torch.cuda.synchronize()
    assert torch.equal(l0, l1)
    ln = l0.cpu().numpy()
    for b in range(B):
        rows = _phys(tabn, shift, b, np.arange(ln[b]))
        for key, _ in PLANES:
            got = pool[key].cpu().numpy()[rows]
            want = cont[key][b, : ln[b]].cpu().numpy()
            assert np.array_equal(got, want), (b, key)
