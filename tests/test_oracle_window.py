"""Pins of the oracle's FP8 sliding-window record and ring
[ggaaooppeenngg.github.io, "DeepSeek-V4.1-Flash 架构解析", sections 4.1 and 7;
weigao.cc, "DeepSeek V4.1 Flash：从架构到推理成本", section 10.1;
jokeuncle.pages.dev, "两张架构图里藏着 890 字节", 顺便算清另外三笔账].

What fixes each pin: the OCP E4M3 code table (bias 7, largest finite 448, the
value the pages multiply by 6 for the FP4 range), the byte counts the pages
print (448 + 128 + 8 = 584 B per token, 576 B of data), torch's own bf16
rounding, brute force over single-token writes, and an exact identity between
window formats on values both represent exactly.
"""
import numpy as np
import pytest
import torch

import oracle


def _rec(vals):
    """one record from a 512-float row"""
    return oracle.fp8_record(np.asarray(vals, np.float32).reshape(1, 512))


def test_e4m3_code_table():
    # OCP E4M3: S.EEEE.MMM, bias 7, exponent 0 subnormal, S.1111.111 NaN
    v = lambda c: oracle.scale_value(c, oracle.E4M3)  # noqa: E731
    assert v(0x00) == 0.0 and v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9
    assert v(0x08) == 2.0 ** -6 and v(0x38) == 1.0 and v(0x3F) == 1.875 and v(0x40) == 2.0
    assert v(0x7E) == 448.0 and np.isnan(v(0x7F)) and v(0xB8) == -1.0 and v(0xFE) == -448.0


def test_every_finite_code_round_trips_at_unit_scale():
    # a group whose max is 448 takes scale 2^0 (byte 127); every finite
    # magnitude then encodes to its own code
    for c in range(0x7F):
        row = np.zeros(512, np.float32)
        row[0] = 448.0
        row[1] = oracle.scale_value(c, oracle.E4M3)
        row[2] = -row[1]
        d, s = _rec(row)
        assert s[0, 0] == 127
        assert d[0, 1] == c and d[0, 2] == (c | 0x80 if c else 0), c
    # and the decode gives the value back
    row = np.zeros(512, np.float32)
    row[:127] = [oracle.scale_value(c, oracle.E4M3) for c in range(127)]
    row[127] = 448.0
    d, s = _rec(row)
    assert np.array_equal(oracle.fp8_record_decode(d, s)[0, :128], row[:128].astype(np.float64))


@pytest.mark.parametrize("x,code", [(1.0625, 0x38), (1.1875, 0x3A), (1.0624, 0x38), (1.0626, 0x39),
                                    (0.9375 * 2.0 ** -6, 0x08), (2.0 ** -10, 0x00),
                                    (1.5 * 2.0 ** -9, 0x02), (2.0 ** -10 * 1.001, 0x01), (440.0, 0x7E),
                                    (432.0, 0x7E), (431.0, 0x7D), (-1.0625, 0x38 | 0x80)])
def test_nearest_with_ties_to_even(x, code):
    row = np.zeros(512, np.float32)
    row[0] = 448.0
    row[1] = x
    d, s = _rec(row)
    assert s[0, 0] == 127 and d[0, 1] == code, (x, hex(d[0, 1]))


@pytest.mark.parametrize("amax,byte", [(448.0, 127), (448.0 * (1 + 2 ** -20), 128), (56.0, 124),
                                       (57.0, 125), (1.0, 119), (0.0, 0), (448.0 * 2.0 ** -120, 7)])
def test_scale_is_smallest_power_of_two_without_clipping(amax, byte):
    row = np.zeros(512, np.float32)
    row[64 + 5] = -amax  # group 1
    d, s = _rec(row)
    assert s[0, 1] == byte
    if amax > 0:
        assert 448.0 * 2.0 ** (byte - 127) >= np.float32(amax) > 448.0 * 2.0 ** (byte - 128)
        assert d[0, 64 + 5] & 0x80
    assert np.all(d[0, :64] == 0) and s[0, 0] == 0 and s[0, 7] == 0


def test_record_byte_counts_match_the_pages():
    d, s = _rec(np.ones(512))
    # 448 B position-free + 128 B RoPE = 576 B data, + 8 B scale = 584 B
    assert d.shape[-1] == 448 + 128 == 576 and d.shape[-1] + s.shape[-1] == 584


def test_rope_dims_are_bf16_nearest_even():
    g = np.random.default_rng(3)
    row = g.standard_normal(512).astype(np.float32) * 3
    # values that sit exactly between two bf16 patterns
    row[448] = np.float32(1.0 + 2 ** -8)  # tie -> 1.0 (even)
    row[449] = np.float32(1.0 + 3 * 2 ** -8)  # tie -> 1 + 2^-6 (even)
    d, s = _rec(row)
    want = torch.from_numpy(row[448:]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = d[0, 448:].view(np.uint16)
    assert np.array_equal(got, want)
    assert oracle.fp8_record_decode(d, s)[0, 448] == 1.0


def test_fp8_error_bound():
    # nearest rounding: |x - deq| <= half a code step (2^(e-3) * scale at x's binade)
    g = np.random.default_rng(5)
    row = g.standard_normal(512).astype(np.float32) * 4
    d, s = _rec(row)
    dq = oracle.fp8_record_decode(d, s)[0]
    for gi in range(7):
        sc = 2.0 ** (int(s[0, gi]) - 127)
        x = row[64 * gi:64 * gi + 64].astype(np.float64) / sc
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(x), 1e-300))), -6)
        assert np.all(np.abs(x - dq[64 * gi:64 * gi + 64] / sc) <= 2.0 ** (e - 3) / 2 + 1e-12)


def _latent(B, n, seed):
    g = np.random.default_rng(seed)
    x = torch.from_numpy(g.standard_normal((B, n, 512)).astype(np.float32)).to(torch.bfloat16)
    return x.view(torch.int16).numpy().view(np.uint16)


def test_ring_holds_the_last_tokens():
    W = 128
    x = _latent(2, 200, 11)
    pos0 = np.array([0, 1000], np.int64)
    r = oracle.window_write(x, pos0, W, rope=True)
    assert list(r["swa_len"]) == [128, 128]
    for b in range(2):
        for slot in range(W):
            # the last token of the 200 whose position is congruent to the slot
            i = max(i for i in range(200) if (pos0[b] + i) % W == slot)
            one = oracle.window_write(x[b:b + 1, i:i + 1], pos0[b:b + 1] + i, W, rope=True)
            assert np.array_equal(r["data"][b, slot], one["data"][0, slot])
            assert np.array_equal(r["scales"][b, slot], one["scales"][0, slot])


def test_partial_window_leaves_other_slots():
    W = 128
    x = _latent(1, 3, 12)
    data = np.full((1, W, 576), 0xAA, np.uint8)
    sc = np.full((1, W, 8), 0x55, np.uint8)
    r = oracle.window_write(x, np.array([5], np.int64), W, data=data, scales=sc)
    assert r["swa_len"][0] == 8
    touched = [5, 6, 7]
    for slot in range(W):
        if slot in touched:
            assert not np.all(data[0, slot] == 0xAA) and sc[0, slot, 7] == 0
        else:
            assert np.all(data[0, slot] == 0xAA) and np.all(sc[0, slot] == 0x55)


def test_window_rows_are_the_normalised_rotated_latent():
    # the record decodes to the cache write's m = 1 entry (same RMSNorm and
    # RoPE at the same position) within FP8 rounding; RoPE dims within bf16
    x = _latent(1, 4, 13)
    gm = np.linspace(0.5, 1.5, 512).astype(np.float32)
    pos = np.array([0, 1, 400, 77777], np.int64)
    r = oracle.window_write(x.reshape(4, 1, 512), pos, 128, gamma=gm, rope=True)
    cw = oracle.cache_write(x[0], x[0], 1, np.zeros((512, 128), np.float32), oracle.E8M0, gamma=gm,
                            eps=1e-6, rope_pos=pos)
    assert np.array_equal(r["y"][:, 0], cw["y"])
    dq = oracle.fp8_record_decode(r["data"][np.arange(4), pos % 128], r["scales"][np.arange(4), pos % 128])
    y = cw["y"].astype(np.float64)
    assert np.all(np.abs(dq[:, 448:] - y[:, 448:]) <= np.abs(y[:, 448:]) * 2.0 ** -8)
    assert np.all(np.abs(dq[:, :448] - y[:, :448]) <= np.abs(y[:, :448]) * 2.0 ** -4 + 2.0 ** -9 * 2.0 ** -6 * 64)


def test_attention_over_fp8_window_equals_main_format_window_on_shared_values():
    # rows drawn from values both formats hold exactly (E2M1 magnitudes at
    # scale 1, which E4M3 represents too; bf16 holds them exactly): the two
    # window formats must give the same attention, to the last bit
    g = np.random.default_rng(21)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    W, n = 37, 64
    rows = mags[g.integers(0, 8, (W, 512))] * np.where(g.random((W, 512)) < 0.5, -1, 1).astype(np.float32)
    rows[:, ::16] = 6.0  # every 16-group and 64-group hits the same max: scale 1 in both formats
    fc, fs = oracle.quantize(rows, 16, oracle.E8M0)
    assert np.array_equal(oracle.dequantize(fc, fs, 16, oracle.E8M0), rows.astype(np.float64))
    d, s = oracle.fp8_record(rows)
    assert np.array_equal(oracle.fp8_record_decode(d, s), rows.astype(np.float64))
    mc, ms = oracle.quantize(g.standard_normal((n, 512)).astype(np.float32), 16, oracle.E8M0)
    q = torch.from_numpy(g.standard_normal((4, 512)).astype(np.float32)).to(torch.bfloat16)
    q = q.view(torch.int16).numpy().view(np.uint16)
    topk = g.permutation(n)[:20].astype(np.int32)
    a, la = oracle.attention(q, mc, ms, n, 0, topk, fc, fs, W, 0.05, q_pos=123)
    b, lb = oracle.attention(q, mc, ms, n, 0, topk, d, s, W, 0.05, q_pos=123, swa_fmt=1)
    assert np.array_equal(a, b) and np.array_equal(la, lb)
    # a wrong window length is seen
    c, _ = oracle.attention(q, mc, ms, n, 0, topk, d, s, W - 1, 0.05, q_pos=123, swa_fmt=1)
    assert not np.array_equal(a, c)
