"""Pins of the oracle's sparse attention and cache write.

Attention: the selected main-KV rows concatenated with the window rows, each
row both key and value, dequantised first.  Pinned against torch's
scaled_dot_product_attention in float64 on independently dequantised rows,
and against closed forms (identical rows, zero query, one dominant row).

Cache write: per-channel softmax pooling over m tokens, RMSNorm, FP4 of the
latent and of its 512->128 projection.  Pinned against torch softmax /
rms_norm in float64 and closed forms (equal gates give the mean; an identity
projection copies the first 128 channels).
"""
import numpy as np
import pytest
import torch

import csa2_synth as syn
import oracle
from refdeq import bf16_to_f64, dequant


def _main_cache(n, seed, fmt):
    x = np.random.default_rng(seed).standard_normal((n, 512)).astype(np.float32)
    c, s = oracle.quantize(x, 16, fmt)
    return c, s


def _qbits(H, D, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return syn.as_bf16_bits(torch.randn(H, D, generator=g) * scale).numpy()


@pytest.mark.parametrize("fmt", [oracle.E8M0, oracle.E4M3])
def test_attention_matches_sdpa_fp64(fmt):
    n, H = 300, 16
    c, s = _main_cache(n, 1, fmt)
    sc, ss = _main_cache(20, 2, fmt)
    topk = np.random.default_rng(3).choice(n, 40, replace=False).astype(np.int32)
    topk[5] = -1          # masked
    topk[7] = n + 3       # out of range: masked
    topk[9] = topk[10]    # duplicate: attended twice
    q = _qbits(H, 512, 4, 0.2)
    scale = 1.0 / np.sqrt(512)
    out, lse = oracle.attention(q, c, s, n, fmt, topk, sc, ss, 20, scale)
    valid = topk[(topk >= 0) & (topk < n)]
    rows = np.concatenate([dequant(c[valid], s[valid], 16, fmt), dequant(sc, ss, 16, fmt)])
    qf = torch.from_numpy(bf16_to_f64(q))[None]
    R = torch.from_numpy(rows)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(qf, R, R, scale=float(np.float32(scale)))[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-6)
    logits = (bf16_to_f64(q) @ rows.T) * float(np.float32(scale))
    ref_lse = np.log(np.exp(logits - logits.max(1, keepdims=True)).sum(1)) + logits.max(1)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-6)


def test_attention_closed_forms():
    fmt = oracle.E4M3
    c, s = _main_cache(50, 5, fmt)
    row = dequant(c[7:8], s[7:8], 16, fmt)[0]
    q = _qbits(4, 512, 6)
    # every attended row identical -> output is that row
    out, _ = oracle.attention(q, c, s, 50, fmt, np.full(10, 7, np.int32), c[7:8].repeat(3, 0),
                              s[7:8].repeat(3, 0), 3, 0.05)
    np.testing.assert_allclose(out, np.broadcast_to(row, out.shape), rtol=1e-6, atol=1e-7)
    # zero query -> mean of the rows
    q0 = np.zeros((2, 512), np.uint16)
    idx = np.array([1, 4, 9, 30], np.int32)
    out, lse = oracle.attention(q0, c, s, 50, fmt, idx, None, None, 0, 0.05)
    mean = dequant(c[idx], s[idx], 16, fmt).mean(0)
    np.testing.assert_allclose(out[0], mean, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(lse, np.log(4.0), rtol=1e-6)
    # one dominant logit -> that row
    rows = dequant(c[idx], s[idx], 16, fmt)
    qd = syn.as_bf16_bits(torch.from_numpy(rows[2] * 50.0)[None].float()).numpy()
    out, _ = oracle.attention(qd, c, s, 50, fmt, idx, None, None, 0, 1.0)
    np.testing.assert_allclose(out[0], rows[2], rtol=1e-5, atol=1e-5)
    # nothing attended -> zeros and -inf
    out, lse = oracle.attention(q[:1], c, s, 50, fmt, np.full(4, -1, np.int32), None, None, 0, 1.0)
    assert (out == 0).all() and np.isneginf(lse).all()


# ------------------------------------------------------------------ cache write
def _write_inputs(T, seed):
    g = torch.Generator().manual_seed(seed)
    lat = syn.as_bf16_bits(torch.randn(T, 512, generator=g)).numpy()
    gate = syn.as_bf16_bits(torch.randn(T, 512, generator=g)).numpy()
    w = (torch.randn(512, 128, generator=g) / np.sqrt(512)).numpy()
    return lat, gate, w


@pytest.mark.parametrize("fmt", [oracle.E8M0, oracle.E4M3])
def test_cache_write_m1_is_rmsnorm(fmt):
    lat, _, w = _write_inputs(64, 1)
    o = oracle.cache_write(lat, None, 1, w, fmt, eps=1e-6)
    x = torch.from_numpy(bf16_to_f64(lat))
    ref = torch.nn.functional.rms_norm(x, (512,), eps=float(np.float32(1e-6))).numpy()
    assert (o["y"] == ref.astype(np.float32)).mean() > 0.999
    np.testing.assert_allclose(o["y"], ref, rtol=1e-7, atol=0)
    c, s = oracle.quantize(o["y"], 16, fmt)
    assert (c == o["main_codes"]).all() and (s == o["main_scales"]).all()
    kref = o["y"].astype(np.float64) @ w.astype(np.float64)
    np.testing.assert_allclose(o["k"], kref, rtol=1e-6, atol=1e-7)
    ck, sk = oracle.quantize(o["k"], 32, oracle.E8M0)
    assert (ck == o["idx_codes"]).all() and (sk == o["idx_scales"]).all()
    rms = np.sqrt((o["y"].astype(np.float64) ** 2).mean(1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)


def test_cache_write_m2_softmax_pooling():
    lat, gate, w = _write_inputs(128, 2)
    o = oracle.cache_write(lat, gate, 2, w, oracle.E8M0)
    x = torch.from_numpy(bf16_to_f64(lat)).view(64, 2, 512)
    g = torch.from_numpy(bf16_to_f64(gate)).view(64, 2, 512)
    pooled = (x * g.softmax(dim=1)).sum(dim=1)
    ref = torch.nn.functional.rms_norm(pooled, (512,), eps=float(np.float32(1e-6))).numpy()
    np.testing.assert_allclose(o["y"], ref, rtol=2e-7, atol=1e-7)


def test_cache_write_equal_gates_average_and_identity_projection():
    lat, gate, _ = _write_inputs(64, 3)
    gate[:] = gate[0:1, :]  # equal gates across tokens -> plain mean
    w = np.zeros((512, 128), np.float32)
    w[:128, :128] = np.eye(128, dtype=np.float32)
    gamma = np.linspace(0.5, 1.5, 512).astype(np.float32)
    o = oracle.cache_write(lat, gate, 4, w, oracle.E4M3, gamma=gamma)
    x = bf16_to_f64(lat).reshape(16, 4, 512).mean(1)
    r = 1 / np.sqrt((x**2).mean(1, keepdims=True) + np.float32(1e-6))
    np.testing.assert_allclose(o["y"], x * r * gamma, rtol=1e-6, atol=1e-7)
    assert (o["k"] == o["y"][:, :128]).all()
