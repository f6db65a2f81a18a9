"""GPU parity of the FP4 quantiser and of the device-side FP4 decode.

The quantiser is integer/exact-compare work: bit-exact against the oracle on
exhaustive code x scale constructions, midpoints, zeros, saturation and wide
random data.  The device decode (gfx950 scaled converts) is probed through
single-row attention: with one attended row the softmax weight is exactly 1,
so the output equals the dequantised row, which is exact in bf16.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_mxfp4_amd as K
import oracle
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _scale_codes(fmt):
    return range(0, 255) if fmt == 0 else range(1, 0x7F)


def _gpu_quant(X, group, fmt):
    x = torch.from_numpy(np.ascontiguousarray(X, np.float32)).to(DEV)
    c, s = K.quantize_fp4(x, group, fmt)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("fmt,group", [(0, 16), (1, 16), (0, 32)])
def test_quantize_exhaustive_codes_and_scales(fmt, group):
    say(f"quantize exhaustive fmt={fmt} group={group}")
    rows = []
    for b in _scale_codes(fmt):
        s = oracle.scale_value(b, fmt)
        for c in range(16):
            x = np.zeros(group, np.float64)
            x[0] = 6.0 * s
            x[1] = (-1 if c & 8 else 1) * MAGS[c & 7] * s
            x[2] = -x[1] * 0.5
            x[3] = 0.75 * s          # tie -> even code 2
            x[4] = 2.5 * s           # tie -> even code 4
            x[5] = -1.25 * s         # tie -> even code 2
            x[6] = 5.0 * s           # tie -> even code 6
            x[7] = 0.25 * s          # tie -> code 0
            with np.errstate(over="ignore"):
                if not np.all(np.isfinite(x.astype(np.float32))):
                    continue
            rows.append(x.astype(np.float32))
    X = np.stack(rows)
    c_ref, s_ref = oracle.quantize(X, group, fmt)
    c_gpu, s_gpu = _gpu_quant(X, group, fmt)
    assert np.array_equal(s_gpu, s_ref)
    assert np.array_equal(c_gpu, c_ref)


@pytest.mark.parametrize("fmt,group", [(0, 16), (1, 16), (0, 32)])
def test_quantize_scale_boundaries(fmt, group):
    """Group maxima at 6 s for every scale code s and at its fp32 neighbours
    (one and two ulps either side): the scale byte changes exactly there.
    The other values sit on E2M1 midpoints of the chosen scale."""
    say(f"quantize scale boundaries fmt={fmt} group={group}")
    rows = []
    for b in _scale_codes(fmt):
        with np.errstate(over="ignore"):
            top = np.float32(6.0 * oracle.scale_value(b, fmt))
        if not np.isfinite(top) or top == 0:
            continue
        cands = [top]
        for d in (1, 2):
            lo = hi = top
            for _ in range(d):
                lo = np.nextafter(lo, np.float32(0))
                hi = np.nextafter(hi, np.float32(np.inf))
            cands += [lo, hi]
        for a in cands:
            if not np.isfinite(a) or a == 0:
                continue
            x = np.zeros(group, np.float32)
            x[0] = a
            x[1] = -a
            x[2:9] = np.float32(a / 6) * np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
            rows.append(x)
    X = np.stack(rows)
    c_ref, s_ref = oracle.quantize(X, group, fmt)
    c_gpu, s_gpu = _gpu_quant(X, group, fmt)
    assert np.array_equal(s_gpu, s_ref)
    assert np.array_equal(c_gpu, c_ref)


@pytest.mark.parametrize("fmt,group", [(0, 16), (1, 16), (0, 32)])
def test_quantize_random_wide_range_and_edges(fmt, group):
    say(f"quantize random fmt={fmt} group={group}")
    g = np.random.default_rng(11 + fmt + group)
    n = 20000
    X = (g.standard_normal((n, 128)) * np.exp(g.uniform(-30, 30, (n, 1)))).astype(np.float32)
    X[0] = 0.0
    X[1] = -0.0
    X[2, :] = np.float32(1e-40)      # subnormal inputs
    X[3, :] = 3000.0                 # E4M3 saturation
    X[4, ::2] = np.float32(2.0 ** -149)
    X[5] = np.nextafter(np.float32(1.5), np.float32(2)) * (2.0 ** np.arange(128) % 7)
    c_ref, s_ref = oracle.quantize(X, group, fmt)
    c_gpu, s_gpu = _gpu_quant(X, group, fmt)
    bad = np.where((c_gpu != c_ref).any(1) | (s_gpu != s_ref).any(1))[0]
    assert len(bad) == 0, f"rows differ: {bad[:10]}"


@pytest.mark.parametrize("fmt,group", [(0, 16), (1, 16), (0, 32)])
def test_quantize_nonfinite_inputs(fmt, group):
    """NaN is ignored by the group maximum and encodes as +0; an infinity
    saturates the scale byte and encodes as the largest magnitude; finite
    values beside an infinity round to zero.  (The E8M0 path encodes on the
    gfx950 scaled convert, which saturates NaN and keeps the sign of zero:
    both are corrected, and these rows pin that.)"""
    say(f"quantize non-finite fmt={fmt} group={group}")
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    g = np.random.default_rng(5 + fmt + group)
    X = (g.standard_normal((12, 64)) * 3).astype(np.float32)
    X[0, 0] = nan                      # one NaN in a finite group
    X[1, :group] = nan                 # a group of NaNs only
    X[2, 3] = inf
    X[3, 5] = -inf
    X[4, :group] = -nan
    X[5, 1], X[5, 2] = inf, nan
    X[6, :group] = -inf
    X[7, ::3] = nan                    # NaNs scattered over every group
    X[8, :] = -np.float32(1e-3)        # small negatives beside a large value: zero codes must be +0
    X[8, 0] = 6.0
    X[9, :] = -0.0
    X[10, ::2] = nan
    X[10, 1::2] = -np.float32(2.0 ** -140)
    c_ref, s_ref = oracle.quantize(X, group, fmt)
    c_gpu, s_gpu = _gpu_quant(X, group, fmt)
    assert np.array_equal(s_gpu, s_ref)
    assert np.array_equal(c_gpu, c_ref)


def test_quantize_rejects_bad_arguments():
    x = torch.zeros(4, 48, device=DEV)
    with pytest.raises(K.Csa2Error):
        K.quantize_fp4(x, 32, 0)  # 48 is not a multiple of 32


@pytest.mark.parametrize("fmt", [0, 1])
def test_device_decode_through_single_row_attention(fmt):
    say(f"device decode probe fmt={fmt}")
    # rows: every code byte in every position, under a spread of scale bytes
    scales = list(range(100, 150)) if fmt == 0 else list(range(0x08, 0x78, 2))
    R = len(scales) * 2
    codes = np.zeros((R, 256), np.uint8)
    sc = np.zeros((R, 32), np.uint8)
    for i, sb in enumerate(scales):
        for half in range(2):
            r = 2 * i + half
            codes[r] = (np.arange(256) + 128 * half) % 256
            sc[r] = sb
    if fmt == 1:
        sc[1, 5] = 0x01  # smallest E4M3 scale (subnormal, 2^-9)
    B = R
    main_c = torch.from_numpy(codes).to(DEV).view(B, 1, 256)
    main_s = torch.from_numpy(sc).to(DEV).view(B, 1, 32)
    topk = torch.zeros(B, 1, dtype=torch.int32, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    q = torch.zeros(B, 16, 512, dtype=torch.int16, device=DEV)
    out = K.sparse_attn_decode(q, main_c.contiguous(), main_s.contiguous(), lens, topk, fmt)
    torch.cuda.synchronize()
    got = out.view(torch.bfloat16).float().cpu().numpy()
    ref = oracle.dequantize(codes, sc, 16, fmt)
    for h in range(16):
        np.testing.assert_array_equal(got[:, h, :], ref.astype(np.float32))


def test_device_decode_smallest_e8m0_scale():
    """E8M0 byte 0 (2^-127): the decoded values are bf16 subnormals."""
    codes = np.arange(256, dtype=np.uint8)[None].repeat(2, 0)
    sc = np.zeros((2, 32), np.uint8)
    sc[1] = 1
    main_c = torch.from_numpy(codes).to(DEV).view(2, 1, 256).contiguous()
    main_s = torch.from_numpy(sc).to(DEV).view(2, 1, 32).contiguous()
    out = K.sparse_attn_decode(torch.zeros(2, 16, 512, dtype=torch.int16, device=DEV), main_c, main_s,
                               torch.ones(2, dtype=torch.int32, device=DEV),
                               torch.zeros(2, 1, dtype=torch.int32, device=DEV), 0)
    got = out.view(torch.bfloat16).float().cpu().numpy()[:, 0, :]
    ref = oracle.dequantize(codes, sc, 16, 0).astype(np.float32)
    np.testing.assert_array_equal(got, ref)
