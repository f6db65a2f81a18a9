"""CPU oracle of the CSA2 decode hot path (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``liboracle_csa2.so`` (built
from ``csa2_oracle.c`` by ``oracle/build.py``) with numpy arrays; it never
imports the HIP package, and the HIP package never imports it.

Every function follows a passage of the pages on DeepSeek V4.1 Flash; the
citation is in the C source next to each definition.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle_csa2.so")

E8M0 = 0
E4M3 = 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b  # noqa: WPS433 (build on first use, CPU only)

        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.oracle_e2m1.restype = ctypes.c_double
    lib.oracle_e2m1.argtypes = [ctypes.c_uint8]
    lib.oracle_scale_value.restype = ctypes.c_double
    lib.oracle_scale_value.argtypes = [ctypes.c_uint8, i32]
    lib.oracle_quantize_group.argtypes = [P, i32, i32, P, P]
    lib.oracle_quantize_rows.argtypes = [P, i64, i32, i32, i32, P, P]
    lib.oracle_dequantize_rows.argtypes = [P, P, i64, i32, i32, i32, P]
    lib.oracle_cache_write.argtypes = [P, P, i64, i32, P, f32, P, i32, P, P, P, P, P, P, P]
    lib.oracle_rope.argtypes = [P, i64, i32]
    lib.oracle_score.argtypes = [P, P, P, i64, P, P, i32, P]
    lib.oracle_topk_ids.restype = i64
    lib.oracle_topk_ids.argtypes = [P, P, i64, i64, P]
    lib.oracle_block_pool.restype = i64
    lib.oracle_block_pool.argtypes = [P, i64, i32, i32, P, P]
    lib.oracle_index_full.restype = i64
    lib.oracle_index_full.argtypes = [P, P, i64, P, P, i32, i32, i32, i32, P, P, P]
    lib.oracle_index_pool.argtypes = [P, P, i64, P, i64, P, P, i32, i32, P, P]
    lib.oracle_attention.argtypes = [P, i32, P, P, i64, i32, P, i32, P, P, i32, i32, f32, P, P, P]
    lib.oracle_fp8_record.argtypes = [P, P, P]
    lib.oracle_fp8_record_decode.argtypes = [P, P, i64, P]
    lib.oracle_window_write.argtypes = [P, i64, i32, P, f32, i32, P, i32, P, P, P, P]
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


# --------------------------------------------------------------------- formats
def e2m1_value(nibble: int) -> float:
    return float(_load().oracle_e2m1(nibble & 15))


def scale_value(byte: int, fmt: int) -> float:
    return float(_load().oracle_scale_value(byte & 255, fmt))


def quantize(x: np.ndarray, group: int, fmt: int):
    """fp32 [..., dim] -> (codes u8 [..., dim/2], scales u8 [..., dim/group])."""
    x = _c(x, np.float32)
    dim = x.shape[-1]
    rows = x.size // dim if dim else 0
    codes = np.zeros(x.shape[:-1] + (dim // 2,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (dim // group,), np.uint8)
    _load().oracle_quantize_rows(_p(x), rows, dim, group, fmt, _p(codes), _p(scales))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, group: int, fmt: int) -> np.ndarray:
    """(codes, scales) -> float64 [..., dim]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    dim = codes.shape[-1] * 2
    rows = codes.size // codes.shape[-1] if codes.shape[-1] else 0
    out = np.zeros(codes.shape[:-1] + (dim,), np.float64)
    _load().oracle_dequantize_rows(_p(codes), _p(scales), rows, dim, group, fmt, _p(out))
    return out


# ----------------------------------------------------------------- cache write
def rope(x, pos, inverse=False):
    """Compressed RoPE of one 512-d vector (fp64 copy returned): dims 448..511
    as 32 adjacent pairs turned by pos * 160000^(-2j/64)."""
    v = np.array(x, dtype=np.float64, copy=True).reshape(512)
    _load().oracle_rope(_p(v), int(pos), 1 if inverse else 0)
    return v


def cache_write(latent_bf16, gate_bf16, m, w_idx, main_fmt, gamma=None, eps=1e-6, rope_pos=None):
    """latent/gate: uint16 bf16 bits [T][512]; w_idx fp32 [512][128];
    rope_pos: int64 [T/m] entry positions for the compressed RoPE, or None.

    Returns dict(main_codes, main_scales, idx_codes, idx_scales, y, k); y is
    the (rotated) main entry before quantisation, k the indexer key.
    """
    latent = _c(latent_bf16, np.uint16)
    T = latent.shape[0]
    gate = None if m == 1 else _c(gate_bf16, np.uint16)
    w = _c(w_idx, np.float32)
    g = None if gamma is None else _c(gamma, np.float32)
    n = T // m
    out = dict(
        main_codes=np.zeros((n, 256), np.uint8),
        main_scales=np.zeros((n, 32), np.uint8),
        idx_codes=np.zeros((n, 64), np.uint8),
        idx_scales=np.zeros((n, 4), np.uint8),
        y=np.zeros((n, 512), np.float32),
        k=np.zeros((n, 128), np.float32),
    )
    rp = None if rope_pos is None else _c(rope_pos, np.int64)
    if rp is not None and rp.shape != (n,):
        raise ValueError("rope_pos must hold one position per entry")
    _load().oracle_cache_write(
        _p(latent), _p(gate), T, m, _p(g), float(eps), _p(w), main_fmt, _p(rp),
        _p(out["main_codes"]), _p(out["main_scales"]), _p(out["idx_codes"]),
        _p(out["idx_scales"]), _p(out["y"]), _p(out["k"]),
    )
    return out


# --------------------------------------------------------------------- indexer
def score(idx_codes, idx_scales, q_bf16, w, pos=None):
    """Scores of positions `pos` (default all rows) of one sequence."""
    ic = _c(idx_codes, np.uint8)
    isc = _c(idx_scales, np.uint8)
    q = _c(q_bf16, np.uint16)
    w = _c(w, np.float32)
    H = q.shape[0]
    if pos is None:
        n = ic.shape[0]
        pp = None
    else:
        pp = _c(pos, np.int32)
        n = pp.shape[0]
    s = np.zeros(n, np.float32)
    _load().oracle_score(_p(ic), _p(isc), _p(pp), n, _p(q), _p(w), H, _p(s))
    return s


def topk_ids(scores, k, ids=None):
    """(score desc, id asc) top-k; ascending ids, -1 padded; NaN = absent."""
    s = _c(scores, np.float32)
    n = s.shape[0]
    idv = None if ids is None else _c(ids, np.int64)
    out = np.zeros(k, np.int64)
    _load().oracle_topk_ids(_p(s), _p(idv), n, k, _p(out))
    return out


def block_pool(scores, block, n_blocks):
    s = _c(scores, np.float32)
    L = s.shape[0]
    nb = (L + block - 1) // block
    bs = np.zeros(max(nb, 1), np.float32)
    pool = np.zeros(max(n_blocks * block, 1), np.int32)
    pl = _load().oracle_block_pool(_p(s), L, block, n_blocks, _p(bs), _p(pool))
    return pool[: n_blocks * block], int(pl), bs[:nb]


def index_full(idx_codes, idx_scales, length, q_bf16, w, k, block, n_blocks):
    """One sequence.  Returns (topk int32 [k], pool int32 [n_blocks*block], pool_len, scores)."""
    ic = _c(idx_codes, np.uint8)
    isc = _c(idx_scales, np.uint8)
    q = _c(q_bf16, np.uint16)
    w = _c(w, np.float32)
    H = q.shape[0]
    topk = np.zeros(k, np.int32)
    pool = np.zeros(max(n_blocks * block, 1), np.int32)
    sc = np.zeros(max(length, 1), np.float32)
    pl = _load().oracle_index_full(_p(ic), _p(isc), length, _p(q), _p(w), H, k, block, n_blocks,
                                   _p(topk), _p(pool), _p(sc))
    return topk, pool[: n_blocks * block], int(pl), sc[:length]


def index_pool(idx_codes, idx_scales, length, pool, pool_len, q_bf16, w, k):
    ic = _c(idx_codes, np.uint8)
    isc = _c(idx_scales, np.uint8)
    pv = _c(pool, np.int32)
    q = _c(q_bf16, np.uint16)
    w = _c(w, np.float32)
    H = q.shape[0]
    topk = np.zeros(k, np.int32)
    ps = np.zeros(max(pool_len, 1), np.float32)
    _load().oracle_index_pool(_p(ic), _p(isc), length, _p(pv), pool_len, _p(q), _p(w), H, k,
                              _p(topk), _p(ps))
    return topk, ps[:pool_len]


# ------------------------------------------------------------------- attention
def attention(q_bf16, main_codes, main_scales, length, main_fmt, topk, swa_codes, swa_scales,
              swa_len, sm_scale, q_pos=None, swa_fmt=0):
    """One sequence: q uint16 [H][512]. Returns (out fp32 [H][512], lse fp32 [H]).
    q_pos: the query's position for Q RoPE and output inverse RoPE, or None.
    swa_fmt 0: window rows in the main format ([W][256] codes, [W][32] scales);
    swa_fmt 1: FP8 window records ([W][576] data, [W][8] scales)."""
    q = _c(q_bf16, np.uint16)
    H = q.shape[0]
    mc = _c(main_codes, np.uint8)
    ms = _c(main_scales, np.uint8)
    t = _c(topk, np.int32)
    if swa_len > 0:
        sc = _c(swa_codes, np.uint8)
        ss = _c(swa_scales, np.uint8)
    else:
        sc = ss = None
    out = np.zeros((H, 512), np.float32)
    lse = np.zeros(H, np.float32)
    qp = None if q_pos is None else np.array([q_pos], np.int64)
    _load().oracle_attention(_p(q), H, _p(mc), _p(ms), length, main_fmt, _p(t), t.shape[0],
                             _p(sc), _p(ss), swa_len, int(swa_fmt), float(sm_scale), _p(qp), _p(out),
                             _p(lse))
    return out, lse


def fp8_record(y):
    """Rows float32 [..][512] -> FP8 window records (data u8 [..][576], scales u8 [..][8])."""
    y = _c(y, np.float32)
    lead = y.shape[:-1]
    y2 = y.reshape(-1, 512)
    data = np.zeros((y2.shape[0], 576), np.uint8)
    sc = np.zeros((y2.shape[0], 8), np.uint8)
    for r in range(y2.shape[0]):
        _load().oracle_fp8_record(_p(y2[r]), _p(data[r]), _p(sc[r]))
    return data.reshape(*lead, 576), sc.reshape(*lead, 8)


def fp8_record_decode(data, scales):
    """FP8 window records -> float64 rows [..][512]."""
    d = _c(data, np.uint8)
    s = _c(scales, np.uint8)
    lead = d.shape[:-1]
    out = np.zeros((int(np.prod(lead, dtype=np.int64)), 512), np.float64)
    _load().oracle_fp8_record_decode(_p(d), _p(s), out.shape[0], _p(out))
    return out.reshape(*lead, 512)


def window_write(latent, pos0, W, gamma=None, eps=1e-6, rope=False, data=None, scales=None):
    """Write tokens into the FP8 window ring.  latent bf16 bits [B][n][512];
    pos0 int64 [B] (position of token 0); W slots.  data/scales (u8 [B][W][576],
    [B][W][8]) are updated in place when given (else start zeroed).
    Returns dict(data, scales, swa_len int32 [B], y float32 [B][n][512])."""
    x = _c(latent, np.uint16)
    B, n = x.shape[0], x.shape[1]
    p0 = _c(pos0, np.int64)
    if data is None:
        data = np.zeros((B, W, 576), np.uint8)
    if scales is None:
        scales = np.zeros((B, W, 8), np.uint8)
    assert data.dtype == np.uint8 and data.flags.c_contiguous and data.shape == (B, W, 576)
    assert scales.dtype == np.uint8 and scales.flags.c_contiguous and scales.shape == (B, W, 8)
    g = None if gamma is None else _c(gamma, np.float32)
    swa_len = np.zeros(B, np.int32)
    y = np.zeros((B, n, 512), np.float32)
    _load().oracle_window_write(_p(x), B, n, _p(g), float(eps), int(bool(rope)), _p(p0), W, _p(data),
                                _p(scales), _p(swa_len), _p(y))
    return dict(data=data, scales=scales, swa_len=swa_len, y=y)
