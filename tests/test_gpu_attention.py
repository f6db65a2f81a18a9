"""GPU parity of the sparse attention and of the cache write.

Attention: per (sequence, head) max|o - r| / max|r| <= 1e-2 against the fp64
oracle (output in bf16); the log-sum-exp within 1e-4 absolute.  Edge cases:
masked and out-of-range top-k slots, duplicate slots (attended twice), window
shorter than its capacity, no window, an empty sequence, both scale formats,
16/32/64 heads, k not a multiple of the 64-row chunk.

Cache write: FP4 bytes equal the oracle's except where a certificate holds:
the oracle's pre-quantisation value lies within 1e-5 relative of an E2M1
midpoint of its group's scale, or the group maximum lies within 1e-5 of a
scale boundary (then the whole group may differ).
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import DEV, attn_close, say

pytestmark = pytest.mark.gpu


def _rope_lse_tol(q_bits, rows, qpos, sm_scale=1 / np.sqrt(512)):
    """Log-sum-exp tolerance when the query is rotated by the compressed RoPE.
    The kernels round the rotated query to bf16 (their MFMA operand), the
    oracle keeps it exact: each logit may move by up to 2^-9 of
    sm_scale * sum over the 64 rotated dims of |q_rot[d] * row[d]|; 2^-8 of
    the largest such sum over heads and rows bounds the lse difference, on
    top of the 1e-4 accumulation tolerance."""
    qf = (np.asarray(q_bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qr = np.stack([oracle.rope(qf[h], qpos) for h in range(qf.shape[0])])[:, 448:]
    worst = (np.abs(qr) @ np.abs(np.asarray(rows, np.float64)[:, 448:]).T).max() if len(rows) else 0.0
    return 1e-4 + 2.0 ** -8 * sm_scale * worst


def _make_cache(B, cap, fmt, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(B, cap, 512, generator=g, device=DEV)
    c, s = K.quantize_fp4(x, 16, fmt)
    xc = x.cpu().numpy()
    rc, rs = oracle.quantize(xc, 16, fmt)
    assert np.array_equal(rc, c.cpu().numpy()) and np.array_equal(rs, s.cpu().numpy())
    return c, s, rc, rs


@pytest.mark.parametrize("fmt,H,rope", [(0, 16, False), (1, 16, False), (0, 64, False), (1, 64, False),
                                         (0, 64, True), (1, 32, True)])
def test_attention_parity_with_window(fmt, H, rope):
    say(f"attention parity fmt={fmt} H={H} rope={rope}")
    B, cap, k, W = 3, 3000, 512, 128
    c, s, rc, rs = _make_cache(B, cap, fmt, 1 + fmt + H)
    g = np.random.default_rng(5)
    topk = np.stack([np.sort(g.choice(cap, k, replace=False)) for _ in range(B)]).astype(np.int32)
    topk[0, 10] = -1
    topk[0, 11] = cap + 7           # out of range: masked
    topk[1, 20] = topk[1, 21]       # duplicate: attended twice
    topk[2, 300:] = -1              # short selection
    lens = np.array([cap, cap - 100, cap], np.int32)
    topk[1, 30] = cap - 50          # beyond len[1]: masked
    swa_len = np.array([128, 100, 0], np.int32)
    q = syn.as_bf16_bits(torch.randn(B, H, 512, generator=torch.Generator().manual_seed(9)) * 0.5)
    qd = q.to(DEV)
    qpos = np.array([3000, 400, 1 << 30], np.int64) if rope else None
    out, lse = K.sparse_attn_decode(qd, c, s, torch.from_numpy(lens).to(DEV), torch.from_numpy(topk).to(DEV),
                                    fmt, swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swa_len).to(DEV),
                                    swa_stride=cap, swa_cap=W, swa_row0=cap - W, return_lse=True,
                                    q_pos=None if qpos is None else torch.from_numpy(qpos).to(DEV))
    torch.cuda.synchronize()
    ref = np.zeros((B, H, 512), np.float32)
    rl = np.zeros((B, H), np.float32)
    for b in range(B):
        ref[b], rl[b] = oracle.attention(q[b].numpy(), rc[b], rs[b], lens[b], fmt, topk[b],
                                         rc[b, cap - W:], rs[b, cap - W:], swa_len[b], 1 / np.sqrt(512),
                                         q_pos=None if qpos is None else int(qpos[b]))
    worst = attn_close(out.cpu(), ref)
    for b in range(B):
        tol = 1e-4
        if rope:
            sel = [p for p in topk[b] if 0 <= p < lens[b]] + list(range(cap - W, cap - W + swa_len[b]))
            tol = _rope_lse_tol(q[b].numpy(), oracle.dequantize(rc[b][sel], rs[b][sel], 16, fmt), int(qpos[b]))
        np.testing.assert_allclose(lse.cpu().numpy()[b], rl[b], atol=tol, rtol=0)
    say(f"  worst relative error {worst:.2e}")


@pytest.mark.parametrize("fmt", [0, 1])
def test_attention_query_magnitudes_across_bf16_range(fmt):
    """Query heads from bf16's smallest subnormal to its largest finite value
    (the E4M3 path stages each head in fp16 times 2^-k, k chosen per head):
    heads scaled by 2^e for e from -120 to 100, an all-zero head, a head whose
    only non-zero component is the smallest subnormal, and heads holding one
    or two components near the largest value the path allows.  Rows come from N(0, 1), so every logit is
    finite in fp32 and the oracle's fp64 answer is the reference; the
    log-sum-exp is compared relative to its size."""
    say(f"attention query magnitudes fmt={fmt}")
    B, cap, k, W, H = 2, 1200, 300, 64, 16
    c, s, rc, rs = _make_cache(B, cap, fmt, 41 + fmt)
    g = np.random.default_rng(13)
    topk = np.stack([np.sort(g.choice(cap - W, k, replace=False)) for _ in range(B)]).astype(np.int32)
    lens = np.full(B, cap, np.int32)
    swa_len = np.full(B, W, np.int32)
    qf = torch.randn(B, H, 512, generator=torch.Generator().manual_seed(17)) * 0.5
    exps = [-120, -60, -20, -8, 0, 6, 14, 15, 16, 30, 60, 100]
    for h, e in enumerate(exps):
        qf[:, h] *= 2.0 ** e
    q = syn.as_bf16_bits(qf)
    q[:, 12] = 0                                   # all-zero head
    q[:, 13] = 0
    q[:, 13, 77] = 1                               # smallest bf16 subnormal, alone
    # near bf16's maximum: with E8M0 rows (bf16 operands, fp32 products) only
    # up to 2^124, so that q.k itself stays within fp32; with E4M3 rows (fp16
    # operands scaled per head) bf16's largest values
    big, top = (0x7D80, 0x7D80) if fmt == 0 else (0x7F78, 0x7F7F)
    q[:, 14, 5] = big                              # among N(0, 0.25) components
    q[:, 15, 300] = top
    q[:, 15, 301] = (top | 0x8000) - 0x10000       # and its negative (int16 bits)
    out, lse = K.sparse_attn_decode(q.to(DEV), c, s, torch.from_numpy(lens).to(DEV), torch.from_numpy(topk).to(DEV),
                                    fmt, swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swa_len).to(DEV),
                                    swa_stride=cap, swa_cap=W, swa_row0=cap - W, return_lse=True)
    torch.cuda.synchronize()
    ref = np.zeros((B, H, 512), np.float32)
    rl = np.zeros((B, H), np.float64)
    for b in range(B):
        ref[b], rl[b] = oracle.attention(q[b].numpy(), rc[b], rs[b], lens[b], fmt, topk[b],
                                         rc[b, cap - W:], rs[b, cap - W:], swa_len[b], 1 / np.sqrt(512))
    assert np.isfinite(rl).all()
    worst = attn_close(out.cpu(), ref)
    np.testing.assert_allclose(lse.cpu().numpy().astype(np.float64), rl, rtol=1e-5, atol=1e-4)
    say(f"  worst relative error {worst:.2e}")


def test_attention_odd_sizes_and_empty():
    fmt = 0
    B, cap, k = 2, 700, 77
    c, s, rc, rs = _make_cache(B, cap, fmt, 3)
    g = np.random.default_rng(6)
    topk = g.integers(0, cap, (B, k)).astype(np.int32)
    lens = np.array([cap, 0], np.int32)   # second sequence attends nothing
    q = syn.as_bf16_bits(torch.randn(B, 32, 512, generator=torch.Generator().manual_seed(2)))
    out, lse = K.sparse_attn_decode(q.to(DEV), c, s, torch.from_numpy(lens).to(DEV),
                                    torch.from_numpy(topk).to(DEV), fmt, return_lse=True)
    ref0, l0 = oracle.attention(q[0].numpy(), rc[0], rs[0], cap, fmt, topk[0], None, None, 0, 1 / np.sqrt(512))
    o = out.cpu()
    attn_close(o[:1], ref0[None])
    assert (o[1].view(torch.bfloat16).float() == 0).all()
    lse = lse.cpu().numpy()
    assert np.isneginf(lse[1]).all()
    np.testing.assert_allclose(lse[0], l0, atol=1e-4)


@pytest.mark.parametrize("k,W", [(600, 128), (2048, 128), (1100, 0)])
def test_attention_long_selection(k, W):
    """Selections longer than one 640-row register batch (several batches joined)."""
    say(f"attention long selection k={k} W={W}")
    fmt = 1
    B, cap = 2, 5000
    c, s, rc, rs = _make_cache(B, cap, fmt, 11 + k)
    g = np.random.default_rng(k)
    topk = np.stack([g.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)
    topk[1, k // 2:] = -1
    lens = np.array([cap, cap], np.int32)
    swa_len = np.array([W, W // 2], np.int32)
    q = syn.as_bf16_bits(torch.randn(B, 16, 512, generator=torch.Generator().manual_seed(k)) * 0.7)
    kw = dict(swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swa_len).to(DEV), swa_stride=cap,
              swa_cap=W, swa_row0=cap - W) if W else {}
    out, lse = K.sparse_attn_decode(q.to(DEV), c, s, torch.from_numpy(lens).to(DEV),
                                    torch.from_numpy(topk).to(DEV), fmt, return_lse=True, **kw)
    torch.cuda.synchronize()
    ref = np.zeros((B, 16, 512), np.float32)
    rl = np.zeros((B, 16), np.float32)
    for b in range(B):
        ref[b], rl[b] = oracle.attention(q[b].numpy(), rc[b], rs[b], lens[b], fmt, topk[b],
                                         rc[b, cap - W:] if W else None, rs[b, cap - W:] if W else None,
                                         swa_len[b], 1 / np.sqrt(512))
    worst = attn_close(out.cpu(), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), rl, atol=1e-4, rtol=0)
    say(f"  worst relative error {worst:.2e}")


def test_attention_workspace_reuse_deterministic():
    """Repeated calls on one workspace give identical bits and match the oracle."""
    fmt = 0
    B, cap, k, W, H = 3, 2000, 512, 128, 64
    c, s, rc, rs = _make_cache(B, cap, fmt, 21)
    g = np.random.default_rng(21)
    topk = torch.from_numpy(np.stack([g.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)).to(DEV)
    lens = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    swl = torch.full((B,), W, dtype=torch.int32, device=DEV)
    q = syn.as_bf16_bits(torch.randn(B, H, 512, generator=torch.Generator().manual_seed(21))).to(DEV)
    nbytes = K.lib().csa2_attn_workspace(B, H, k, W)
    # only the leading counter region must be zero; the rest may hold anything
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    ws[:262144].zero_()
    outs = []
    for _ in range(3):
        o = K.sparse_attn_decode(q, c, s, lens, topk, fmt, swa_codes=c, swa_scales=s, swa_len=swl,
                                 swa_stride=cap, swa_cap=W, swa_row0=cap - W, _ws=ws)
        outs.append(o.clone())
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])
    assert int(ws[:262144].count_nonzero()) == 0   # counters left at zero
    ref = np.stack([oracle.attention(q[b].cpu().numpy(), rc[b], rs[b], cap, fmt, topk[b].cpu().numpy(),
                                     rc[b, cap - W:], rs[b, cap - W:], W, 1 / np.sqrt(512))[0] for b in range(B)])
    attn_close(outs[0].cpu(), ref)


@pytest.mark.parametrize("fmt", [0, 1])
def test_attention_decode_batch_shape(fmt):
    """16 sequences x 64 heads x (512 + 128) rows: the one-workgroup-per-CU chunking."""
    say(f"attention at the decode-step shape fmt={fmt}")
    B, cap, k, W, H = 16, 1500, 512, 128, 64
    c, s, rc, rs = _make_cache(B, cap, fmt, 31 + fmt)
    g = np.random.default_rng(31)
    topk = np.stack([g.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)
    topk[3, :40] = -1
    lens = np.full(B, cap, np.int32)
    swa_len = np.full(B, W, np.int32)
    swa_len[5] = 7
    q = syn.as_bf16_bits(torch.randn(B, H, 512, generator=torch.Generator().manual_seed(31)) * 0.6)
    out, lse = K.sparse_attn_decode(q.to(DEV), c, s, torch.from_numpy(lens).to(DEV), torch.from_numpy(topk).to(DEV),
                                    fmt, swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swa_len).to(DEV),
                                    swa_stride=cap, swa_cap=W, swa_row0=cap - W, return_lse=True)
    torch.cuda.synchronize()
    ref = np.zeros((B, H, 512), np.float32)
    rl = np.zeros((B, H), np.float32)
    for b in range(B):
        ref[b], rl[b] = oracle.attention(q[b].numpy(), rc[b], rs[b], lens[b], fmt, topk[b],
                                         rc[b, cap - W:], rs[b, cap - W:], swa_len[b], 1 / np.sqrt(512))
    worst = attn_close(out.cpu(), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), rl, atol=1e-4, rtol=0)
    say(f"  worst relative error {worst:.2e}")


def _big_batch_case(B, cap, k, W, fmt, seed, sample, rope=False):
    """B sequences quantised on the GPU; the oracle re-quantises the sampled
    ones (bytes must agree) and attends with its own bytes."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.randn(B, cap, 512, generator=g, device=DEV)
    c, s = K.quantize_fp4(x, 16, fmt)
    rng = np.random.default_rng(seed)
    topk = np.stack([rng.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)
    lens = np.full(B, cap, np.int32)
    swa_len = np.full(B, W, np.int32)
    # edge cases on the first sequences (all of them sampled)
    topk[0, 10] = -1
    topk[0, 11] = cap + 7                 # out of range: masked
    topk[1, 20] = topk[1, 21]             # duplicate: attended twice
    topk[2, k // 3:] = -1                 # short selection
    lens[3] = cap - 100
    topk[3, 30] = cap - 50                # beyond len: masked
    swa_len[4] = min(W, 7)                # short window
    lens[5], swa_len[5] = 0, 0            # attends nothing
    topk[6, :] = -1                       # window only
    picks = sorted(set(range(8)) | set(rng.choice(B, min(sample, B), replace=False).tolist()))
    q = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(seed)) * 0.6)
    qpos = rng.integers(0, 1 << 31, B, dtype=np.int64) if rope else None
    ref = {}
    tols = {}
    xc = x.cpu().numpy()
    cc, scc = c.cpu().numpy(), s.cpu().numpy()
    for b in picks:
        rc, rs = oracle.quantize(xc[b], 16, fmt)
        assert np.array_equal(rc, cc[b]) and np.array_equal(rs, scc[b])
        tols[b] = 1e-4
        if qpos is not None:
            sel = [p for p in topk[b] if 0 <= p < lens[b]] + list(range(cap - W, cap - W + swa_len[b]))
            tols[b] = _rope_lse_tol(q[b].numpy(), oracle.dequantize(rc[sel], rs[sel], 16, fmt), int(qpos[b]))
        ref[b] = oracle.attention(q[b].numpy(), rc, rs, lens[b], fmt, topk[b], rc[cap - W:] if W else None,
                                  rs[cap - W:] if W else None, swa_len[b], 1 / np.sqrt(512),
                                  q_pos=None if qpos is None else int(qpos[b]))
    args = (q.to(DEV), c, s, torch.from_numpy(lens).to(DEV), torch.from_numpy(topk).to(DEV), fmt)
    kw = dict(swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swa_len).to(DEV), swa_stride=cap, swa_cap=W,
              swa_row0=cap - W) if W else {}
    if qpos is not None:
        kw["q_pos"] = torch.from_numpy(qpos).to(DEV)
    return args, kw, picks, ref, tols


@pytest.mark.parametrize("B,k,W,fmt,rope", [(48, 512, 128, 0, False), (64, 512, 128, 1, False),
                                            (128, 600, 100, 0, False), (256, 77, 0, 1, False),
                                            (256, 512, 128, 0, False), (64, 512, 128, 0, True),
                                            (256, 512, 128, 1, True),
                                            # 3 splits; 2 splits where 3 would overfill the chip
                                            (72, 512, 128, 1, False), (84, 600, 128, 0, True),
                                            # 8-wave split kernel (below 48 sequences, past one round of 10-wave)
                                            (40, 512, 128, 0, True), (28, 300, 128, 1, False)])
def test_attention_large_batch(B, k, W, fmt, rope):
    """Batches that take the all-heads throughput kernel: 4, 3, 2 and 1 splits
    per sequence (ragged chunk ranges, k not a multiple of the 32-row chunk),
    and, below 48 sequences past one round of 10-wave workgroups, the 8-wave
    split kernel;
    both scale formats; masked, duplicate, out-of-range and empty selections,
    short and missing windows.  Repeated calls on one workspace give identical
    bits and leave the completion counters at zero."""
    say(f"attention large batch B={B} k={k} W={W} fmt={fmt} rope={rope}")
    cap = 1200
    args, kw, picks, ref, tols = _big_batch_case(B, cap, k, W, fmt, 100 + B + k, 16, rope)
    H = 64
    nbytes = K.lib().csa2_attn_workspace(B, H, k, W)
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device=DEV)
    ws[:262144].zero_()
    out, lse = K.sparse_attn_decode(*args, return_lse=True, _ws=ws, **kw)
    out2 = K.sparse_attn_decode(*args, _ws=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    assert int(ws[:262144].count_nonzero()) == 0
    o = out.cpu()
    l = lse.cpu().numpy()
    worst = 0.0
    for b in picks:
        r, rl = ref[b]
        if b == 5:
            assert (o[b].view(torch.bfloat16).float() == 0).all() and np.isneginf(l[b]).all()
            continue
        worst = max(worst, attn_close(o[b:b + 1], r[None]))
        np.testing.assert_allclose(l[b], rl, atol=tols[b], rtol=0)
    say(f"  {len(picks)} sequences checked, worst relative error {worst:.2e}")


@pytest.mark.parametrize("B,Q,k,W,fmt,rope", [(3, 5, 512, 128, 0, False), (16, 5, 512, 128, 1, True),
                                              (2, 3, 100, 0, 0, False), (1, 1, 64, 16, 1, False),
                                              (12, 4, 300, 128, 0, True)])
def test_attention_multi_query(B, Q, k, W, fmt, rope):
    """Q queries per sequence in one call (csa2_sparse_attn_decode_mq), each
    with its own index list over its sequence's cache and window: bit for bit
    what csa2_sparse_attn_decode gives over B*Q sequences holding copies of
    the caches (the same kernel shape: 15 and 48+ query rows pick the split
    and the all-heads kernel), and each sampled query row against the oracle."""
    say(f"attention multi-query B={B} Q={Q} k={k} W={W} fmt={fmt} rope={rope}")
    cap = 3000
    g = torch.Generator(device=DEV).manual_seed(900 + B * Q + k)
    x = torch.randn(B, cap, 512, generator=g, device=DEV)
    c, s = K.quantize_fp4(x, 16, fmt)
    rng = np.random.default_rng(900 + B + Q)
    lens = np.full(B, cap, np.int32)
    lens[-1] = cap - 777
    topk = np.stack([np.stack([rng.choice(int(lens[b]), k, replace=False) for _ in range(Q)])
                     for b in range(B)]).astype(np.int32)
    topk[0, 0, 3] = -1
    topk[0, Q - 1, 5] = cap + 9          # out of range: masked
    swl = np.full(B, W, np.int32)
    if B > 1 and W:
        swl[1] = W // 3
    q = syn.as_bf16_bits(torch.randn(B, Q, 64, 512, generator=torch.Generator().manual_seed(B * 7 + Q)))
    qpos = torch.from_numpy(rng.integers(0, 1 << 20, (B, Q)).astype(np.int64)) if rope else None
    lt = torch.from_numpy(lens).to(DEV)
    kw = dict(swa_codes=c, swa_scales=s, swa_len=torch.from_numpy(swl).to(DEV), swa_stride=cap, swa_cap=W,
              swa_row0=cap - W) if W else {}
    out, lse = K.sparse_attn_decode_mq(q.to(DEV), c, s, lt, torch.from_numpy(topk).to(DEV), fmt, return_lse=True,
                                       q_pos=None if qpos is None else qpos.to(DEV), **kw)
    # the same B*Q query rows as separate sequences over copies of the caches
    cr, sr = c.repeat_interleave(Q, 0).contiguous(), s.repeat_interleave(Q, 0).contiguous()
    kwr = dict(swa_codes=cr, swa_scales=sr, swa_len=torch.from_numpy(np.repeat(swl, Q)).to(DEV), swa_stride=cap,
               swa_cap=W, swa_row0=cap - W) if W else {}
    out_r, lse_r = K.sparse_attn_decode(q.view(B * Q, 64, 512).to(DEV), cr, sr, lt.repeat_interleave(Q),
                                        torch.from_numpy(topk.reshape(B * Q, k)).to(DEV), fmt, return_lse=True,
                                        q_pos=None if qpos is None else qpos.view(-1).to(DEV), **kwr)
    torch.cuda.synchronize()
    assert torch.equal(out.view(B * Q, 64, 512), out_r)
    assert torch.equal(lse.view(B * Q, 64).view(torch.int32), lse_r.view(torch.int32))
    o, l = out.cpu(), lse.cpu().numpy()
    cc, scc = c.cpu().numpy(), s.cpu().numpy()
    for b, i in sorted({(0, 0), (0, Q - 1), (B - 1, Q // 2), (min(1, B - 1), Q - 1)}):
        rc, rs = cc[b], scc[b]
        ro, rl = oracle.attention(q[b, i].numpy(), rc, rs, int(lens[b]), fmt, topk[b, i], rc[cap - W:] if W else None,
                                  rs[cap - W:] if W else None, int(swl[b]), 1 / np.sqrt(512),
                                  q_pos=None if qpos is None else int(qpos[b, i]))
        attn_close(o[b, i:i + 1], ro[None])
        tol = 1e-4
        if qpos is not None:
            sel = [int(p) for p in topk[b, i] if 0 <= p < lens[b]] + list(range(cap - W, cap - W + int(swl[b])))
            tol = _rope_lse_tol(q[b, i].numpy(), oracle.dequantize(rc[sel], rs[sel], 16, fmt), int(qpos[b, i]))
        np.testing.assert_allclose(l[b, i], rl, atol=tol, rtol=0)


def test_attention_window_only_separate_buffer():
    fmt = 1
    B, cap, W = 2, 64, 128
    c, s, rc, rs = _make_cache(B, cap, fmt, 4)
    wc, ws_, rwc, rws = _make_cache(B, W, fmt, 5)
    q = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(3)))
    topk = torch.full((B, 1), -1, dtype=torch.int32)
    swa_len = np.array([128, 1], np.int32)
    out = K.sparse_attn_decode(q.to(DEV), c, s, torch.full((B,), cap, dtype=torch.int32, device=DEV),
                               topk.to(DEV), fmt, swa_codes=wc, swa_scales=ws_,
                               swa_len=torch.from_numpy(swa_len).to(DEV), swa_stride=W, swa_cap=W)
    ref = np.stack([oracle.attention(q[b].numpy(), rc[b], rs[b], cap, fmt, topk[b].numpy(), rwc[b], rws[b],
                                     swa_len[b], 1 / np.sqrt(512))[0] for b in range(B)])
    attn_close(out.cpu(), ref)


# ---------------------------------------------------------------- cache write
def _certified_code_mismatch(vals, ref_codes, ref_scales, got_codes, got_scales, group, fmt, rotated=False):
    """Count byte mismatches; assert each is covered by a certificate.  With
    rotated=True, dims 448..511 carry the compressed RoPE: there a value's
    error scales with its pair's norm (which can be far above the value), so
    the 1e-5 slack is taken relative to the larger of the two."""
    n_bad = 0
    rows, dim = vals.shape
    slack = np.abs(vals.astype(np.float64))
    if rotated:
        pr = np.hypot(vals[:, 448::2].astype(np.float64), vals[:, 449::2].astype(np.float64))
        slack[:, 448:] = np.maximum(slack[:, 448:], np.repeat(pr, 2, axis=1))
    deq_s = np.vectorize(lambda b: oracle.scale_value(int(b), fmt))
    for r in np.where((ref_codes != got_codes).any(1) | (ref_scales != got_scales).any(1))[0]:
        for gi in range(dim // group):
            sl = slice(gi * group, (gi + 1) * group)
            cs = slice(gi * group // 2, (gi + 1) * group // 2)
            if ref_scales[r, gi] == got_scales[r, gi] and np.array_equal(ref_codes[r, cs], got_codes[r, cs]):
                continue
            v = vals[r, sl].astype(np.float64)
            amax = np.abs(v).max()
            if ref_scales[r, gi] != got_scales[r, gi]:
                # the group max must sit at a scale boundary: 6*s(b) for the oracle's b or b-1
                b = int(ref_scales[r, gi])
                edges = [6 * oracle.scale_value(bb, fmt) for bb in (b - 1, b) if bb >= 0]
                gs_ = slack[r, sl].max()
                assert min(abs(amax - e) / max(e, gs_) for e in edges if e > 0) <= 1e-5, (r, gi, amax, edges)
                n_bad += 1
                continue
            s = float(deq_s(ref_scales[r, gi]))
            for i in range(group):
                byte = (gi * group + i) // 2
                sh = 4 * (i % 2)
                if ((ref_codes[r, byte] >> sh) & 15) == ((got_codes[r, byte] >> sh) & 15):
                    continue
                mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * s
                a = abs(v[i])
                sl_i = slack[r, gi * group + i]
                assert np.min(np.abs(a - mids) / np.maximum(np.maximum(mids, sl_i), 1e-300)) <= 1e-5, \
                    (r, gi, i, a / s)
                n_bad += 1
    return n_bad


@pytest.mark.parametrize("fmt", [0, 1])
def test_cache_write_nonfinite_gates(fmt):
    """Two-token pooling (m = 2) with infinite and NaN gates, against the
    oracle's softmax exp(g_t - max) / sum: a +inf gate, a NaN gate or two -inf
    gates make the channel NaN (exp(inf - inf)), so the whole entry is NaN
    after RMSNorm and encodes as zero codes and zero scale bytes; a single
    -inf gate gives the other token the whole weight."""
    say(f"cache write non-finite gates fmt={fmt}")
    n = 64
    wl = syn.small("w", 77, B=1, cap=1, H_idx=8, k=1, n_blocks=0, write_tokens=2 * n, write_m=2)
    lat, gate, w = syn.write_inputs(wl, "cpu")
    g = gate.numpy().view(np.uint16).copy()
    pinf, ninf, qnan = 0x7F80, 0xFF80, 0x7FC0
    g[0, 5] = pinf                       # entry 0: +inf beside a finite gate
    g[3, 100] = ninf                     # entry 1: -inf beside a finite gate
    g[4, 7] = g[5, 7] = ninf             # entry 2: two -inf gates
    g[6, 300] = qnan                     # entry 3: NaN gate
    g[8, 0] = g[9, 0] = pinf             # entry 4: two +inf gates
    g[10, 511], g[11, 511] = ninf, pinf  # entry 5: -inf and +inf
    g[12, 20], g[13, 21] = ninf, ninf    # entry 6: one -inf in each of two channels
    g[15, 64:80] = ninf                  # entry 7: a whole 16-channel group from one token
    gate = torch.from_numpy(g.view(np.int16))
    got = K.cache_write(lat.to(DEV), gate.to(DEV), 2, w.to(DEV), fmt)
    torch.cuda.synchronize()
    ref = oracle.cache_write(lat.numpy(), gate.numpy(), 2, w.numpy(), fmt)
    gt = {k_: v.cpu().numpy() for k_, v in got.items()}
    nan_rows = [0, 2, 3, 4, 5]
    assert np.isnan(ref["y"][nan_rows]).all() and not np.isnan(ref["y"][[1, 6, 7]]).any()
    for k_ in ("main_codes", "main_scales", "idx_codes", "idx_scales"):
        assert (gt[k_][nan_rows] == 0).all() and (ref[k_][nan_rows] == 0).all(), k_
    fin = [r for r in range(n) if r not in nan_rows]
    nm = _certified_code_mismatch(ref["y"][fin], ref["main_codes"][fin], ref["main_scales"][fin],
                                  gt["main_codes"][fin], gt["main_scales"][fin], 16, fmt)
    nk = _certified_code_mismatch(ref["k"][fin], ref["idx_codes"][fin], ref["idx_scales"][fin],
                                  gt["idx_codes"][fin], gt["idx_scales"][fin], 32, 0)
    say(f"  certified mismatches: main {nm}, indexer {nk}")
    assert nm + nk <= 2


def _rope_positions(n, seed):
    """Entry positions for the compressed RoPE: 0, small, 400 (pair 16 turns by
    1 rad), and large values up to 2^31 - 1."""
    g = np.random.default_rng(seed)
    p = g.integers(0, 1 << 31, n, dtype=np.int64)
    p[: min(n, 4)] = [0, 1, 400, (1 << 31) - 1][: min(n, 4)]
    return p


@pytest.mark.parametrize("m,fmt,gamma,n,rope", [(1, 0, False, 1024, False), (2, 1, False, 1024, False),
                                                (2, 0, True, 1024, False), (4, 1, True, 1024, False),
                                                (1, 0, False, 37, False), (2, 1, True, 37, False),
                                                (1, 0, False, 1024, True), (2, 1, True, 1024, True),
                                                (1, 1, False, 37, True),
                                                # the general pooling loop (odd m, the largest m)
                                                (3, 0, True, 37, False), (8, 1, False, 300, True),
                                                # 4 and 8 column tiles per workgroup (from 2,033 and 4,081 entries)
                                                (1, 1, False, 2100, True), (2, 0, False, 4100, False),
                                                (2, 1, True, 4100, True)])
def test_cache_write_parity(m, fmt, gamma, n, rope):
    say(f"cache write m={m} fmt={fmt} gamma={gamma} entries={n} rope={rope}")
    wl = syn.small("w", 31 + m, B=1, cap=1, H_idx=8, k=1, n_blocks=0, write_tokens=n * m, write_m=m)
    lat, gate, w = syn.write_inputs(wl, DEV)
    gm = (torch.linspace(0.5, 1.5, 512, device=DEV) if gamma else None)
    pos = _rope_positions(n, 7 + n) if rope else None
    got = K.cache_write(lat, gate, m, w, fmt, gamma=gm, eps=1e-6,
                        rope_pos=None if pos is None else torch.from_numpy(pos).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.cache_write(lat.cpu().numpy(), gate.cpu().numpy(), m, w.cpu().numpy(), fmt,
                             gamma=None if gm is None else gm.cpu().numpy(), eps=1e-6, rope_pos=pos)
    g = {k_: v.cpu().numpy() for k_, v in got.items()}
    nm = _certified_code_mismatch(ref["y"], ref["main_codes"], ref["main_scales"], g["main_codes"],
                                  g["main_scales"], 16, fmt, rotated=rope)
    nk = _certified_code_mismatch(ref["k"], ref["idx_codes"], ref["idx_scales"], g["idx_codes"],
                                  g["idx_scales"], 32, 0)
    say(f"  certified mismatches: main {nm}, indexer {nk}")
    if n < 100:
        assert nm + nk <= 2
        return
    # nearly all bytes are identical
    assert (g["main_codes"] == ref["main_codes"]).mean() > 0.999
    assert (g["idx_codes"] == ref["idx_codes"]).mean() > 0.999



@pytest.mark.parametrize("m,fmt,rope", [(1, 0, False), (1, 1, True), (2, 0, True), (2, 1, False)])
def test_cache_append_streams_like_a_batch_write(m, fmt, rope):
    """Tokens appended one step at a time land where a batch write of the
    same tokens puts them: rows len0.., RoPE at the row index, the first token
    of an m = 2 group held until its partner; a sequence with one free row
    takes one entry, a full one takes nothing; other rows are untouched."""
    say(f"cache append m={m} fmt={fmt} rope={rope}")
    B, cap, steps = 5, 40, 11
    len0 = np.array([0, 3, 10, 39, 40], np.int32)
    g = torch.Generator().manual_seed(50 + m + fmt)
    lat = syn.as_bf16_bits(torch.randn(steps, B, 512, generator=g))
    gate = syn.as_bf16_bits(torch.randn(steps, B, 512, generator=g))
    w = (torch.randn(512, 128, generator=g) / np.sqrt(512)).float()
    cache = {k_: torch.full((B, cap, wd), 0xAB, dtype=torch.uint8, device=DEV)
             for k_, wd in (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4))}
    lengths = torch.from_numpy(len0.copy()).to(DEV)
    state = K.append_state(B, DEV) if m == 2 else None
    wd = w.to(DEV)
    for t in range(steps):
        K.cache_append(lat[t].to(DEV), gate[t].to(DEV), m, wd, fmt, cache, lengths, state=state, rope=rope)
    torch.cuda.synchronize()
    got = {k_: v.cpu().numpy() for k_, v in cache.items()}
    n_entries = steps // m
    want_len = np.minimum(cap, len0 + n_entries)
    want_len[len0 >= cap] = len0[len0 >= cap]
    assert np.array_equal(lengths.cpu().numpy(), want_len)
    if m == 2:
        held = state[:4 * B].view(torch.int32).cpu().numpy()
        assert np.array_equal(held, np.where(len0 + n_entries <= cap, steps % 2, 0))
    for b in range(B):
        ne = int(want_len[b] - len0[b])
        rows = slice(int(len0[b]), int(want_len[b]))
        if ne > 0:
            toks = slice(0, ne * m)
            ref = oracle.cache_write(lat[toks, b].numpy(), gate[toks, b].numpy(), m, w.numpy(), fmt,
                                     rope_pos=np.arange(len0[b], len0[b] + ne, dtype=np.int64) if rope else None)
            nm = _certified_code_mismatch(ref["y"], ref["main_codes"], ref["main_scales"],
                                          got["main_codes"][b, rows], got["main_scales"][b, rows], 16, fmt,
                                          rotated=rope)
            nk = _certified_code_mismatch(ref["k"], ref["idx_codes"], ref["idx_scales"],
                                          got["idx_codes"][b, rows], got["idx_scales"][b, rows], 32, 0)
            assert nm + nk <= 2
        for k_ in got:
            assert (got[k_][b, : int(len0[b])] == 0xAB).all() and (got[k_][b, int(want_len[b]):] == 0xAB).all()
