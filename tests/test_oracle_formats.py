"""Pins of the oracle's formats: byte accounting, decode tables, quantiser.

The pages print the byte figures and the E2M1 / E4M3 layouts; the rounding rule
is a reading (smallest scale that covers the group max, nearest value, ties to
the even code).  These tests fix the oracle against the printed numbers, the
torch float8 decoders (a library routine independent of the oracle) and exact
invariants of the rounding rule.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ byte accounting
def test_byte_accounting_matches_pages():
    g = _gold("byte_accounting.json")
    x = np.zeros((1, 512), np.float32)
    c, s = oracle.quantize(x, 16, oracle.E4M3)
    main = c.nbytes + s.nbytes
    xk = np.zeros((1, 128), np.float32)
    ck, sk = oracle.quantize(xk, 32, oracle.E8M0)
    idx = ck.nbytes + sk.nbytes
    assert main == g["main_kv_bytes_per_entry"] == 288
    assert idx == g["indexer_k_bytes_per_entry"] == 68
    assert main + idx == g["kv_source_record_bytes"]
    per_token = sum((main + idx) / g["compress_ratio_of_source"][str(l)] for l in g["kv_source_layers"])
    assert per_token == g["global_kv_bytes_per_token"] == 890
    # Reindex layers own no indexer K; counting one per Reindex layer is the miscount.
    wrong = per_token + idx * len(g["index_source_layers_extra"])
    assert wrong == g["miscount_if_reindex_layers_owned_k"]
    assert per_token * g["tokens_1m"] == g["global_kv_mib_at_1m_tokens"] * 2**20
    # one 1M-token sequence of the decoder source (m=2 entries as in the write+decode workload)
    assert 524288 * 356 == 186646528 == 178 * 2**20


# ---------------------------------------------------------------- decode tables
def test_e2m1_table():
    g = _gold("e2m1.json")
    got = [oracle.e2m1_value(i) for i in range(16)]
    assert got == g["values"]
    assert [np.signbit(v) for v in got[8:]] == [True] * 8


def test_scale_decode_matches_torch_float8():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    e8 = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    e4 = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for i in range(256):
        v8 = oracle.scale_value(i, oracle.E8M0)
        v4 = oracle.scale_value(i, oracle.E4M3)
        if np.isnan(e8[i]):
            assert np.isnan(v8)
        else:
            assert v8 == e8[i], i
        if np.isnan(e4[i]):
            assert np.isnan(v4)
        else:
            assert v4 == e4[i], i
    assert oracle.scale_value(0x7E, oracle.E4M3) == _gold("e2m1.json")["e4m3_max"]


# ------------------------------------------------------------------ quantiser
MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _scale_codes(fmt):
    return range(0, 255) if fmt == oracle.E8M0 else range(1, 0x7F)


def _sv(b, fmt):
    return oracle.scale_value(b, fmt)


@pytest.mark.parametrize("fmt,group", [(oracle.E8M0, 16), (oracle.E4M3, 16), (oracle.E8M0, 32)])
def test_every_code_and_scale_round_trips(fmt, group):
    rows = []
    expect_codes = []
    expect_scale = []
    for b in _scale_codes(fmt):
        s = _sv(b, fmt)
        for c in range(16):
            x = np.zeros(group, np.float64)
            x[0] = 6.0 * s  # pins the scale to b
            x[1] = (-1 if c & 8 else 1) * MAGS[c & 7] * s
            if np.float32(x[0]) != x[0] or np.float32(x[1]) != x[1]:
                continue  # below fp32 subnormal range: not an fp32 input
            rows.append(x.astype(np.float32))
            code1 = 0 if (c & 7) == 0 else c  # a zero magnitude encodes as +0
            expect_codes.append((7, code1))
            expect_scale.append(b)
    X = np.stack(rows)
    codes, scales = oracle.quantize(X, group, fmt)
    assert (scales[:, 0] == np.array(expect_scale)).all()
    assert ((codes[:, 0] & 15) == 7).all()
    assert ((codes[:, 0] >> 4) == np.array([e[1] for e in expect_codes])).all()
    assert (codes[:, 1:] == 0).all()


@pytest.mark.parametrize("fmt", [oracle.E8M0, oracle.E4M3])
def test_midpoints_go_to_even_code(fmt):
    # (midpoint between codes lo and lo+1, code a tie takes)
    mids = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]
    for b in [100, 127, 140] if fmt == oracle.E8M0 else [0x30, 0x38, 0x41, 0x7E]:
        s = _sv(b, fmt)
        for lo, (t, want) in enumerate(mids):
            m = np.float32(t * s)
            x = np.zeros(16, np.float32)
            x[0] = 6 * s
            x[2] = m
            x[3] = -m
            x[4] = np.nextafter(m, np.float32(np.inf))   # just above -> upper code
            x[5] = np.nextafter(m, np.float32(0))        # just below -> lower code
            c, sc = oracle.quantize(x[None], 16, fmt)
            assert sc[0, 0] == b
            assert (c[0, 1] & 15) == want, (b, t)
            assert (c[0, 1] >> 4) == (want | 8 if want else 0), (b, t)
            assert (c[0, 2] & 15) == lo + 1, (b, t)
            assert (c[0, 2] >> 4) == lo, (b, t)


def test_amax_zero_and_scale_boundary():
    c, s = oracle.quantize(np.zeros((1, 32), np.float32), 32, oracle.E8M0)
    assert s[0, 0] == 0 and (c == 0).all()
    c, s = oracle.quantize(-np.zeros((1, 16), np.float32), 16, oracle.E4M3)
    assert s[0, 0] == 0 and (c == 0).all()
    # amax = f * 2^E: E8M0 code E+125 when f <= 1.5, else E+126
    for E in range(-20, 20):
        for f, off in [(1.0, 125), (1.25, 125), (1.5, 125), (1.5000001, 126), (1.75, 126)]:
            x = np.zeros((1, 32), np.float32)
            x[0, 5] = np.float32(f) * np.float32(2.0**E)
            _, s = oracle.quantize(x, 32, oracle.E8M0)
            assert s[0, 0] == E + off, (E, f)


def test_e4m3_saturation_above_2688():
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 3000.0
    x[0, 1] = 2600.0
    x[0, 2] = 2000.0
    c, s = oracle.quantize(x, 16, oracle.E4M3)
    assert s[0, 0] == 0x7E
    assert (c[0, 0] & 15) == 7 and (c[0, 0] >> 4) == 7
    assert (c[0, 1] & 15) == 6  # 2000/448 = 4.46 -> 4.0


@pytest.mark.parametrize("fmt,group", [(oracle.E8M0, 16), (oracle.E4M3, 16), (oracle.E8M0, 32)])
def test_random_invariants(fmt, group):
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((3000, group)) * np.exp(rng.uniform(-8, 8, (3000, 1)))).astype(np.float32)
    top = _sv(max(_scale_codes(fmt)), fmt)
    X = X[np.abs(X).max(1) <= 6 * top]  # saturation is pinned separately
    codes, scales = oracle.quantize(X, group, fmt)
    deq = oracle.dequantize(codes, scales, group, fmt)
    s = np.array([_sv(int(b), fmt) for b in scales[:, 0]])[:, None]
    ax = np.abs(X.astype(np.float64))
    assert (ax <= 6 * s).all()
    # nearest representable value: error at most half the local gap
    half_gap = np.where(ax < 2 * s, 0.25, np.where(ax < 4 * s, 0.5, 1.0)) * s
    assert (np.abs(ax - np.abs(deq)) <= half_gap).all()
    # the scale is the smallest one that covers the group max
    for i in range(0, X.shape[0], 37):
        b = int(scales[i, 0])
        if b > min(_scale_codes(fmt)):
            assert 6 * _sv(b - 1, fmt) < ax[i].max()
    # signs preserved for non-zero codes; zero codes are +0
    nz = deq != 0
    assert (np.sign(deq[nz]) == np.sign(X[nz])).all()
    nib = np.stack([codes & 15, codes >> 4], -1).reshape(X.shape)
    assert not (nib == 8).any()
    # value idempotence: quantising the dequantised values reproduces them.
    # It holds for E8M0 and for normal E4M3 scales (the largest code is then
    # always 7, so the scale is re-chosen identically); an E4M3 subnormal scale
    # can leave the group max at code 6 and the re-chosen scale shrinks.
    c2, s2 = oracle.quantize(deq.astype(np.float32), group, fmt)
    deq2 = oracle.dequantize(c2, s2, group, fmt)
    keep = np.ones(X.shape[0], bool) if fmt == oracle.E8M0 else scales[:, 0] >= 0x08
    assert keep.sum() > X.shape[0] // 2
    assert (deq2[keep] == deq[keep]).all()


def test_e8m0_power_of_two_equivariance():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((500, 32)).astype(np.float32)
    c0, s0 = oracle.quantize(X, 32, oracle.E8M0)
    for j in [-5, -1, 1, 2, 7]:
        c1, s1 = oracle.quantize(X * np.float32(2.0**j), 32, oracle.E8M0)
        assert (c1 == c0).all()
        assert (s1.astype(int) == s0.astype(int) + j).all()


def test_e4m3_code_idempotence_for_normal_scales():
    rng = np.random.default_rng(4)
    X = (rng.standard_normal((2000, 16)) * 3).astype(np.float32)
    c, s = oracle.quantize(X, 16, oracle.E4M3)
    assert (s >= 0x08).all()  # normal E4M3 scales (>= 2^-6)
    deq = oracle.dequantize(c, s, 16, oracle.E4M3).astype(np.float32)
    c2, s2 = oracle.quantize(deq, 16, oracle.E4M3)
    assert (c2 == c).all() and (s2 == s).all()
