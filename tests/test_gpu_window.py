"""GPU parity of the FP8 sliding-window ring and of attention over it.

Window write: record bytes equal the oracle's except where a certificate
holds -- the oracle's pre-quantisation value sits within 1e-5 relative of an
E4M3 midpoint, or the group maximum within 1e-5 of a scale boundary (then the
whole 64-dim group may differ), or, on the RoPE dims, the value sits within
1e-5 x its pair's norm of a bf16 midpoint (a rotated component's error scales
with the pair's norm, not with the component, which can be near zero);
swa_len and every untouched slot are exact.

Attention over FP8 window records (both kernels: the latency split kernel
below 48 sequences, the throughput kernel from 48): the window is written by
the oracle; per
(sequence, head) max|o - r| / max|r| <= 1e-2 and the log-sum-exp within
1e-4 (plus the RoPE allowance).  A single window row with no selected entry
must come back bit for bit: the kernel's decode of every finite E4M3 code.
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import DEV, attn_close, say
from test_gpu_attention import _make_cache, _rope_lse_tol

pytestmark = pytest.mark.gpu

_MAGS = np.array([oracle.scale_value(c, oracle.E4M3) for c in range(127)])
_MIDS = 0.5 * (_MAGS[1:] + _MAGS[:-1])


def _latent(B, n, seed):
    x = torch.randn(B, n, 512, generator=torch.Generator().manual_seed(seed))
    return syn.as_bf16_bits(x)


def _bf16_mid_ok(y, got_bits, scale):
    """got_bits is one of y's two bf16 neighbours and y lies within 1e-5 x
    scale of their midpoint (scale: the RoPE pair's norm, which bounds how far
    an angle error moves a rotated component; it can be far above |y|)."""
    u = np.float32(y).view(np.uint32)
    lo = np.uint32(u & 0xFFFF0000)
    hi = np.uint32(lo + 0x10000)
    vl, vh = lo.view(np.float32).astype(np.float64), hi.view(np.float32).astype(np.float64)
    mid = 0.5 * (vl + vh)
    return int(got_bits) in (int(lo >> 16), int(hi >> 16)) and abs(float(y) - mid) <= 1e-5 * scale


def _certify(y, rd, rs, gd, gs):
    """Mismatches of one record (oracle rd/rs vs GPU gd/gs) with their certificates."""
    n_bad = 0
    assert gs[7] == 0
    for gi in range(7):
        sl = slice(64 * gi, 64 * gi + 64)
        if rs[gi] == gs[gi] and np.array_equal(rd[sl], gd[sl]):
            continue
        v = y[sl].astype(np.float64)
        if rs[gi] != gs[gi]:
            amax = np.abs(v).max()
            b = int(rs[gi])
            edges = [448.0 * 2.0 ** (bb - 127) for bb in (b - 1, b)]
            assert min(abs(amax - e) / e for e in edges) <= 1e-5, (gi, amax, b, int(gs[gi]))
            n_bad += 1
            continue
        s = 2.0 ** (int(rs[gi]) - 127)
        for i in np.where(rd[sl] != gd[sl])[0]:
            a = abs(v[i]) / s
            assert np.min(np.abs(a - _MIDS) / _MIDS) <= 1e-5, (gi, i, a)
            n_bad += 1
    gb, rb = gd[448:].view(np.uint16), rd[448:].view(np.uint16)
    for i in np.where(gb != rb)[0]:
        p0 = 448 + (i & ~1)
        pair = float(np.hypot(y[p0], y[p0 + 1]))
        assert _bf16_mid_ok(y[448 + i], gb[i], max(abs(float(y[448 + i])), pair)), (i, y[448 + i], pair)
        n_bad += 1
    return n_bad


@pytest.mark.parametrize("n,W,rope,gamma", [(1, 128, False, False), (5, 128, True, True), (200, 128, True, False),
                                            (40, 37, False, True), (128, 128, True, True)])
def test_window_write_parity(n, W, rope, gamma):
    say(f"window write n={n} W={W} rope={rope} gamma={gamma}")
    B = 3
    x = _latent(B, n, 100 + n + W)
    pos0 = np.array([0, 126, (1 << 31) + 5], np.int64)
    gm = np.linspace(0.5, 1.5, 512).astype(np.float32) if gamma else None
    data0 = np.full((B, W, 576), 0xAA, np.uint8)
    sc0 = np.full((B, W, 8), 0x55, np.uint8)
    ref = oracle.window_write(x.numpy().view(np.uint16), pos0, W, gamma=gm, rope=rope, data=data0.copy(),
                              scales=sc0.copy())
    win = dict(data=torch.from_numpy(data0).to(DEV), scales=torch.from_numpy(sc0).to(DEV),
               swa_len=torch.full((B,), -7, dtype=torch.int32, device=DEV))
    K.window_write(x.to(DEV), torch.from_numpy(pos0).to(DEV), win, eps=1e-6, rope=rope,
                   gamma=None if gm is None else torch.from_numpy(gm).to(DEV))
    torch.cuda.synchronize()
    gd, gs = win["data"].cpu().numpy(), win["scales"].cpu().numpy()
    assert np.array_equal(win["swa_len"].cpu().numpy(), ref["swa_len"])
    n_bad = 0
    for b in range(B):
        for slot in range(W):
            hits = [i for i in range(n) if (pos0[b] + i) % W == slot]
            if not hits:  # untouched: exactly the fill pattern on both sides
                assert np.all(gd[b, slot] == 0xAA) and np.all(gs[b, slot] == 0x55)
                continue
            y = ref["y"][b, max(hits)]
            n_bad += _certify(y, ref["data"][b, slot], ref["scales"][b, slot], gd[b, slot], gs[b, slot])
    say(f"  certified mismatches: {n_bad}")


def test_window_write_skips_negative_positions():
    B, W = 2, 128
    x = _latent(B, 3, 5)
    win = dict(data=torch.full((B, W, 576), 0x11, dtype=torch.uint8, device=DEV),
               scales=torch.full((B, W, 8), 0x22, dtype=torch.uint8, device=DEV),
               swa_len=torch.full((B,), 9, dtype=torch.int32, device=DEV))
    K.window_write(x.to(DEV), torch.tensor([-1, 4], dtype=torch.int64, device=DEV), win)
    torch.cuda.synchronize()
    d, s = win["data"].cpu().numpy(), win["scales"].cpu().numpy()
    assert np.all(d[0] == 0x11) and np.all(s[0] == 0x22)
    assert list(win["swa_len"].cpu().numpy()) == [9, 7]
    assert not np.all(d[1, 4:7] == 0x11) and np.all(d[1, :4] == 0x11) and np.all(d[1, 7:] == 0x11)


@pytest.mark.parametrize("H,fmt", [(16, 0), (64, 1)])
def test_single_window_row_decodes_exactly(H, fmt):
    # no selected entry, one window row per sequence: the output of every head
    # is that row, which bf16 holds exactly (E4M3 x 2^k and bf16 dims)
    say(f"window record decode H={H} fmt={fmt}")
    B, W = 4, 8
    g = np.random.default_rng(77)
    data = np.zeros((B, W, 576), np.uint8)
    sc = np.zeros((B, W, 8), np.uint8)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    for b in range(B):
        d = g.permutation(np.concatenate([codes, codes]))[:448]
        d[:254] = np.roll(codes, b)  # every finite code in every sequence
        data[b, 0, :448] = d
        rope = (g.standard_normal(64) * 2.0 ** g.integers(-3, 4, 64)).astype(np.float32)
        rope = np.where(np.abs(rope) < 2 ** -6, 2 ** -6, rope).astype(np.float32)
        data[b, 0, 448:] = syn.as_bf16_bits(torch.from_numpy(rope)).numpy().view(np.uint8)
        sc[b, 0, :7] = g.integers(124, 131, 7)
    want = oracle.fp8_record_decode(data[:, 0], sc[:, 0])
    want_bits = syn.as_bf16_bits(torch.from_numpy(want.astype(np.float32)))
    assert np.array_equal(want_bits.view(torch.bfloat16).double().numpy(), want)  # exact in bf16
    c, s, _, _ = _make_cache(B, 64, fmt, 8)
    q = syn.as_bf16_bits(torch.randn(B, H, 512, generator=torch.Generator().manual_seed(3)))
    out = K.sparse_attn_decode(q.to(DEV), c, s, torch.full((B,), 64, dtype=torch.int32, device=DEV),
                               torch.zeros(B, 0, dtype=torch.int32, device=DEV), fmt,
                               swa_codes=torch.from_numpy(data).to(DEV), swa_scales=torch.from_numpy(sc).to(DEV),
                               swa_len=torch.ones(B, dtype=torch.int32, device=DEV), swa_stride=W, swa_cap=W,
                               swa_fmt=K.SWA_FP8)
    torch.cuda.synchronize()
    # compared as values: code 0x80 is -0, which a sum of products returns as +0
    o = out.cpu().view(torch.bfloat16).double()
    wv = want_bits.view(torch.bfloat16).double()
    for b in range(B):
        assert torch.equal(o[b], wv[b].expand(H, 512)), b


def _fp8_windows(B, W, seed, rope):
    """Window rings written by the oracle from seeded latents: sequence b holds
    n_b tokens from position pos0_b (some windows partly filled)."""
    g = np.random.default_rng(seed)
    n = 130
    x = _latent(B, n, seed).numpy().view(np.uint16)
    pos0 = g.integers(0, 1 << 20, B).astype(np.int64)
    pos0[: min(B, 2)] = 0  # rings that start at position 0
    data = np.zeros((B, W, 576), np.uint8)
    sc = np.zeros((B, W, 8), np.uint8)
    r = oracle.window_write(x, pos0, W, rope=rope, data=data, scales=sc)
    swa_len = r["swa_len"].copy()
    if B > 1:
        swa_len[1] = min(37, W - 1)
    if B > 2:
        swa_len[2] = 0
    return data, sc, swa_len, pos0 + n


@pytest.mark.parametrize("B,k,fmt,rope,W", [(1, 512, 0, False, 128), (3, 500, 1, True, 128),
                                            (16, 512, 0, True, 128), (64, 512, 1, False, 128),
                                            (64, 500, 0, True, 128), (48, 40, 1, True, 128),
                                            (256, 512, 0, True, 128), (256, 480, 1, False, 128),
                                            (3, 512, 0, True, 37), (64, 500, 1, False, 37),
                                            (40, 500, 0, True, 128)])
def test_attention_fp8_window_parity(B, k, fmt, rope, W):
    say(f"attention over FP8 window B={B} k={k} fmt={fmt} rope={rope} W={W}")
    cap = 1500
    c, s, rc, rs = _make_cache(B, cap, fmt, 40 + B + k)
    g = np.random.default_rng(B + k)
    topk = np.stack([np.sort(g.choice(cap, k, replace=False)) for _ in range(B)]).astype(np.int32)
    topk[0, 5] = -1
    lens = np.full(B, cap, np.int32)
    data, sc, swa_len, qp = _fp8_windows(B, W, 60 + B, rope)
    q = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(B)) * 0.5)
    qpos = qp if rope else None
    out, lse = K.sparse_attn_decode(q.to(DEV), c, s, torch.from_numpy(lens).to(DEV),
                                    torch.from_numpy(topk).to(DEV), fmt, swa_codes=torch.from_numpy(data).to(DEV),
                                    swa_scales=torch.from_numpy(sc).to(DEV),
                                    swa_len=torch.from_numpy(swa_len).to(DEV), swa_stride=W, swa_cap=W,
                                    return_lse=True, swa_fmt=K.SWA_FP8,
                                    q_pos=None if qpos is None else torch.from_numpy(qpos).to(DEV))
    torch.cuda.synchronize()
    picks = sorted(set(range(min(B, 4))) | set(g.choice(B, min(B, 6), replace=False).tolist()))
    o, lo = out.cpu(), lse.cpu().numpy()
    worst = 0.0
    for b in picks:
        ref, rl = oracle.attention(q[b].numpy(), rc[b], rs[b], lens[b], fmt, topk[b], data[b], sc[b], swa_len[b],
                                   1 / np.sqrt(512), q_pos=None if qpos is None else int(qpos[b]), swa_fmt=1)
        worst = max(worst, attn_close(o[b:b + 1], ref[None]))
        tol = 1e-4
        if rope:
            sel = [p for p in topk[b] if 0 <= p < lens[b]]
            rows = np.concatenate([oracle.dequantize(rc[b][sel], rs[b][sel], 16, fmt),
                                   oracle.fp8_record_decode(data[b, :swa_len[b]], sc[b, :swa_len[b]])])
            tol = _rope_lse_tol(q[b].numpy(), rows, int(qpos[b]))
        np.testing.assert_allclose(lo[b], rl, atol=tol, rtol=0)
    say(f"  worst relative error {worst:.2e}")
