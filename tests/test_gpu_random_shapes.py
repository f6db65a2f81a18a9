"""Seeded random shapes through the whole decode path, against the oracle.

Each case draws a batch, a cache capacity, per-sequence lengths (zero and
full among them), indexer heads, k, the pool size (no pool in some cases),
attention heads, a window capacity with per-sequence window lengths, the
main-KV scale format, and an optional query position (RoPE); then checks, per
sequence:

- the Full indexer's scores against the oracle's, its top-k and pool exactly
  against brute force on the GPU's own scores, and its top-k against the
  oracle's up to certified near-ties;
- a Reindex layer over the GPU's pool (its own query): scores against the
  oracle run on the same pool, top-k exactly against brute force on the GPU's
  pool scores;
- attention over the GPU's top-k plus a separate window buffer, against the
  oracle's attention on the oracle's own quantisation of the same rows
  (outputs within 1e-2, log-sum-exp within the test's tolerance);
- the multi-query attention call (Q = 2..5 queries per sequence, each with
  its own positions) bit for bit against the single-query call over B*Q
  sequences holding copies of the caches.

The shapes are small enough for the oracle, and span several tiles, ragged
tails and the degenerate cases (empty sequences, one-entry windows, k larger
than the visible entries)."""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import (DEV, attn_close, brute_pool, brute_topk, build_gpu_cache, certify_topk,
                        oracle_cache_seq, say, score_close)
from test_gpu_attention import _rope_lse_tol

pytestmark = pytest.mark.gpu

SEEDS = list(range(16))


def _case(seed):
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(1, 11))
    cap = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 2000)), int(r.integers(2000, 6000))]))
    lens = r.integers(0, cap + 1, B)
    lens[0] = cap
    if B > 2:
        lens[1] = 0
    H_idx = int(r.choice([8, 16, 32, 64]))
    k = int(r.choice([1, int(r.integers(2, 64)), int(r.integers(64, 700)), int(r.integers(700, 2049))],
                     p=[0.15, 0.3, 0.4, 0.15]))
    n_blocks = int(r.choice([0, int(r.integers(1, 40)), int(r.integers(40, 600))]))
    H_attn = int(r.choice([16, 32, 64]))
    W = int(r.choice([0, 1, int(r.integers(2, 129)), 128], p=[0.15, 0.15, 0.5, 0.2]))
    fmt = int(r.integers(0, 2))
    rope = bool(r.integers(0, 2))
    return dict(B=B, cap=cap, lens=lens.astype(np.int32), H_idx=H_idx, k=k, n_blocks=n_blocks, H_attn=H_attn,
                W=W, fmt=fmt, rope=rope, r=r)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_shapes_against_oracle(seed):
    c = _case(seed)
    B, cap, lens, H_idx, k, nb, H, W, fmt = (c[x] for x in ("B", "cap", "lens", "H_idx", "k", "n_blocks", "H_attn",
                                                             "W", "fmt"))
    r = c["r"]
    say(f"random shapes seed={seed}: B={B} cap={cap} lens={lens.tolist()} H_idx={H_idx} k={k} blocks={nb} "
        f"H={H} W={W} fmt={fmt} rope={c['rope']}")
    wl = syn.small(f"rs{seed}", 500 + seed, B=B, cap=cap, H_idx=H_idx, k=k, n_blocks=nb)
    cache = build_gpu_cache(wl, fmt)
    lt = torch.from_numpy(lens).to(DEV)

    # ---- Full indexer
    q0, w0 = syn.index_query(wl, 0, DEV), syn.index_weights(wl, 0, DEV)
    topk, pool, pool_len, scores = K.index_full(cache["idx_codes"], cache["idx_scales"], lt, q0, w0, k=k,
                                                n_blocks=nb, return_scores=True)
    topk, pool, pool_len, scores = (t.cpu().numpy() for t in (topk, pool, pool_len, scores))
    refs = [oracle_cache_seq(wl, b, fmt, cache) for b in range(B)]
    q0n, w0n = q0.cpu().numpy(), w0.cpu().numpy()
    cert = 0
    for b in range(B):
        L = int(lens[b])
        ref = refs[b]
        rt, rp, rpl, rs = oracle.index_full(ref["idx_codes"][:L], ref["idx_scales"][:L], L, q0n[b], w0n[b], k, 8,
                                            nb)
        score_close(scores[b, :L], rs)
        assert np.array_equal(topk[b], brute_topk(scores[b, :L], k)), f"top-k of sequence {b}"
        cert += certify_topk(topk[b], rt, rs, k)
        if nb > 0:
            bp, bpl, _ = brute_pool(scores[b, :L], nb)
            assert pool_len[b] == bpl and np.array_equal(pool[b], bp), f"pool of sequence {b}"

    # ---- Reindex over the GPU's pool
    if nb > 0:
        q1, w1 = syn.index_query(wl, 1, DEV), syn.index_weights(wl, 1, DEV)
        pt, plt_ = torch.from_numpy(pool).to(DEV), torch.from_numpy(pool_len).to(DEV)
        t1, ps = K.index_pool(cache["idx_codes"], cache["idx_scales"], lt, pt, plt_, q1, w1, k=k,
                              return_scores=True)
        t1, ps = t1.cpu().numpy(), ps.cpu().numpy()
        q1n, w1n = q1.cpu().numpy(), w1.cpu().numpy()
        for b in range(B):
            n = int(pool_len[b])
            _, rps = oracle.index_pool(refs[b]["idx_codes"], refs[b]["idx_scales"], int(lens[b]), pool[b], n,
                                       q1n[b], w1n[b], k)
            score_close(ps[b, :n], rps)
            assert np.array_equal(t1[b], brute_topk(ps[b, :n], k, pool[b, :n])), f"Reindex top-k of sequence {b}"

    # ---- attention over the GPU's top-k and a separate window buffer
    qa = syn.attn_query(wl, 0, DEV)[:, :H].contiguous()
    qpos = None
    if c["rope"]:
        qpos = torch.from_numpy(r.integers(0, 1 << 20, B).astype(np.int64)).to(DEV)
    kw = {}
    wref = [None] * B
    swl = np.zeros(B, np.int32)
    if W > 0:
        wwl = syn.small(f"rsw{seed}", 700 + seed, B=B, cap=W, H_idx=8, k=1, n_blocks=0)
        wc = build_gpu_cache(wwl, fmt)
        swl = r.integers(0, W + 1, B).astype(np.int32)
        swl[0] = W
        kw = dict(swa_codes=wc["main_codes"], swa_scales=wc["main_scales"], swa_len=torch.from_numpy(swl).to(DEV),
                  swa_stride=W, swa_cap=W)
        wref = [oracle_cache_seq(wwl, b, fmt, wc) for b in range(B)]
    out, lse = K.sparse_attn_decode(qa, cache["main_codes"], cache["main_scales"], lt,
                                    torch.from_numpy(topk).to(DEV), fmt, return_lse=True, q_pos=qpos, **kw)
    o, l = out.cpu(), lse.cpu().numpy()
    qan = qa.cpu().numpy()
    sm = 1.0 / np.sqrt(512)
    for b in range(B):
        wr = wref[b]
        ro, rl = oracle.attention(qan[b], refs[b]["main_codes"], refs[b]["main_scales"], int(lens[b]), fmt, topk[b],
                                  wr["main_codes"] if wr else None, wr["main_scales"] if wr else None,
                                  int(swl[b]), sm, q_pos=None if qpos is None else int(qpos[b]))
        visible = np.isfinite(rl)
        if not visible.any():
            assert (o[b].view(torch.bfloat16).float() == 0).all() and np.isneginf(l[b]).all()
            continue
        attn_close(o[b:b + 1], ro[None])
        tol = 1e-4
        if qpos is not None:
            sel = [int(p) for p in topk[b] if 0 <= p < lens[b]]
            rows = [oracle.dequantize(refs[b]["main_codes"][sel], refs[b]["main_scales"][sel], 16, fmt)] if sel else []
            if swl[b] > 0:
                rows.append(oracle.dequantize(wr["main_codes"][:swl[b]], wr["main_scales"][:swl[b]], 16, fmt))
            tol = _rope_lse_tol(qan[b], np.concatenate(rows) if rows else np.zeros((0, 512)), int(qpos[b]))
        np.testing.assert_allclose(l[b][visible], rl[visible], atol=tol, rtol=0)
        assert np.isneginf(l[b][~visible]).all()
    # ---- the same shapes with Q queries per sequence in one call: bit for bit
    # the single-query call over B*Q sequences holding copies of the caches
    Q = int(r.integers(2, 6))
    kq = max(1, min(k, 600))
    tq = np.full((B, Q, kq), -1, np.int32)
    for b in range(B):
        for i in range(Q):
            m = min(kq, int(lens[b]))
            tq[b, i, :m] = r.choice(int(lens[b]), m, replace=False) if m else []
    qq = syn.as_bf16_bits(torch.from_numpy(r.standard_normal((B, Q, H, 512)).astype(np.float32))).to(DEV)
    qpq = torch.from_numpy(r.integers(0, 1 << 20, (B, Q)).astype(np.int64)).to(DEV) if c["rope"] else None
    om, lm = K.sparse_attn_decode_mq(qq, cache["main_codes"], cache["main_scales"], lt, torch.from_numpy(tq).to(DEV),
                                     fmt, return_lse=True, q_pos=qpq, **kw)
    kwr = {}
    if W > 0:
        kwr = dict(swa_codes=kw["swa_codes"].repeat_interleave(Q, 0).contiguous(),
                   swa_scales=kw["swa_scales"].repeat_interleave(Q, 0).contiguous(),
                   swa_len=kw["swa_len"].repeat_interleave(Q), swa_stride=W, swa_cap=W)
    orr, lrr = K.sparse_attn_decode(qq.view(B * Q, H, 512), cache["main_codes"].repeat_interleave(Q, 0).contiguous(),
                                    cache["main_scales"].repeat_interleave(Q, 0).contiguous(), lt.repeat_interleave(Q),
                                    torch.from_numpy(tq.reshape(B * Q, kq)).to(DEV), fmt, return_lse=True,
                                    q_pos=None if qpq is None else qpq.view(-1), **kwr)
    torch.cuda.synchronize()
    assert torch.equal(om.view(B * Q, H, 512), orr), f"multi-query attention (Q={Q}) differs"
    assert torch.equal(lm.view(B * Q, H).view(torch.int32), lrr.view(torch.int32))
    say(f"  ok (certified near-tie index differences: {cert}; multi-query Q={Q})")
