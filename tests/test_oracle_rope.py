"""Pins of the oracle's compressed RoPE (test infrastructure only).

[ggaaooppeenngg.github.io, "架构解析：KV Cache 压缩的极限在哪里", 3.2 and 7]: entries
are rotated with RoPE of base 160000 after RMSNorm and before FP4; 64 of the
512 dims carry position (128 B of bf16 beside 448 without).  Readings: the
last 64 dims, adjacent pairs, angle pos * 160000^(-2j/64).

Pins: closed-form angles (pair 0 turns by pos; pair 16 by pos / 400, since
160000^(-1/2) = 1/400), identity at position 0, norm preservation,
composition and inverse, the relative-position property of dot products,
untouched dims 0..447; the cache write rotates the main entry only; the
attention's Q RoPE / inverse RoPE against a brute-force softmax with
explicit 2x2 rotation blocks on a tiny case.
"""
import math

import numpy as np
import pytest

import oracle


def _e(i):
    v = np.zeros(512)
    v[i] = 1.0
    return v


def test_pair0_turns_by_the_position():
    for p in (1, 2, 7, 1000):
        r = oracle.rope(_e(448), p)
        assert r[448] == pytest.approx(math.cos(p), abs=1e-12)
        assert r[449] == pytest.approx(math.sin(p), abs=1e-12)
        r = oracle.rope(_e(449), p)
        assert r[448] == pytest.approx(-math.sin(p), abs=1e-12)
        assert r[449] == pytest.approx(math.cos(p), abs=1e-12)


def test_pair16_turns_by_position_over_400():
    # 160000^(-32/64) = 1/400: position 400 turns pair 16 (dims 480, 481) by exactly 1 rad
    r = oracle.rope(_e(480), 400)
    assert r[480] == pytest.approx(math.cos(1.0), abs=1e-12)
    assert r[481] == pytest.approx(math.sin(1.0), abs=1e-12)
    r = oracle.rope(_e(480), 200)
    assert r[480] == pytest.approx(math.cos(0.5), abs=1e-12)


def test_last_pair_frequency():
    p = 123456
    ang = p * 160000.0 ** (-62.0 / 64.0)
    r = oracle.rope(_e(510), p)
    assert r[510] == pytest.approx(math.cos(ang), abs=1e-9)
    assert r[511] == pytest.approx(math.sin(ang), abs=1e-9)


def test_identity_norm_composition_inverse_and_untouched_dims():
    g = np.random.default_rng(3)
    for _ in range(5):
        x = g.standard_normal(512)
        a, b = int(g.integers(0, 1 << 20)), int(g.integers(0, 1 << 20))
        assert np.array_equal(oracle.rope(x, 0), x)
        ra = oracle.rope(x, a)
        assert np.linalg.norm(ra) == pytest.approx(np.linalg.norm(x), rel=1e-13)
        assert np.array_equal(ra[:448], x[:448])
        np.testing.assert_allclose(oracle.rope(ra, b), oracle.rope(x, a + b), atol=1e-9)
        np.testing.assert_allclose(oracle.rope(ra, a, inverse=True), x, atol=1e-9)


def test_relative_position_property():
    g = np.random.default_rng(4)
    u, v = g.standard_normal(512), g.standard_normal(512)
    for a, b in ((5, 3), (100000, 99000), (17, 900)):
        lhs = oracle.rope(u, a) @ oracle.rope(v, b)
        rhs = oracle.rope(u, a - b) @ v if a >= b else u @ oracle.rope(v, b - a)
        assert lhs == pytest.approx(rhs, rel=1e-11, abs=1e-11)


def test_cache_write_rotates_the_main_entry_only():
    g = np.random.default_rng(5)
    T = 6
    lat = (g.standard_normal((T, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    w = (g.standard_normal((512, 128)) / np.sqrt(512)).astype(np.float32)
    pos = np.array([0, 1, 2, 400, 77777, 524287], np.int64)
    plain = oracle.cache_write(lat, None, 1, w, 0)
    rot = oracle.cache_write(lat, None, 1, w, 0, rope_pos=pos)
    for j in range(T):
        want = oracle.rope(plain["y"][j].astype(np.float64), pos[j]).astype(np.float32)
        np.testing.assert_array_equal(rot["y"][j], want)
    np.testing.assert_array_equal(rot["k"], plain["k"])          # the indexer key: no position
    np.testing.assert_array_equal(rot["idx_codes"], plain["idx_codes"])
    # position 0 leaves the entry bytes unchanged
    np.testing.assert_array_equal(rot["main_codes"][0], plain["main_codes"][0])
    c, s = oracle.quantize(rot["y"], 16, 0)
    np.testing.assert_array_equal(c, rot["main_codes"])
    np.testing.assert_array_equal(s, rot["main_scales"])


def _rot_matrix(p, inverse=False):
    """Explicit block-diagonal rotation of dims 448..511 (2x2 blocks)."""
    M = np.eye(512)
    for j in range(32):
        a = p * 160000.0 ** (-2.0 * j / 64.0) * (-1.0 if inverse else 1.0)
        i = 448 + 2 * j
        M[i, i], M[i, i + 1] = math.cos(a), -math.sin(a)
        M[i + 1, i], M[i + 1, i + 1] = math.sin(a), math.cos(a)
    return M


def test_attention_q_rope_and_inverse_rope_brute_force():
    g = np.random.default_rng(6)
    H, n, p = 2, 5, 321
    x = g.standard_normal((n, 512)).astype(np.float32)
    codes, scales = oracle.quantize(x, 16, 0)
    rows = oracle.dequantize(codes, scales, 16, 0).astype(np.float64)
    q = (g.standard_normal((H, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    topk = np.arange(n, dtype=np.int32)
    sc = 1 / np.sqrt(512)
    out, lse = oracle.attention(q, codes, scales, n, 0, topk, None, None, 0, sc, q_pos=p)
    R, Rinv = _rot_matrix(p), _rot_matrix(p, inverse=True)
    for h in range(H):
        lg = sc * rows @ (R @ qf[h])
        w = np.exp(lg - lg.max())
        o = Rinv @ (w @ rows / w.sum())
        np.testing.assert_allclose(out[h], o, rtol=0, atol=1e-6)
        assert lse[h] == pytest.approx(lg.max() + np.log(w.sum()), abs=1e-6)
    # without a position the same call is plain attention
    out0, _ = oracle.attention(q, codes, scales, n, 0, topk, None, None, 0, sc)
    for h in range(H):
        lg = sc * rows @ qf[h]
        w = np.exp(lg - lg.max())
        np.testing.assert_allclose(out0[h], w @ rows / w.sum(), rtol=0, atol=1e-6)
