"""ctypes binding of libcsa2.so: argument marshalling only.

Every function below checks tensor dtypes/shapes/devices, passes raw device
pointers and the current HIP stream to the C ABI (include/csa2.h) and raises
on a non-zero status.  All computation happens in the HIP kernels; there is no
fallback path: if the library is missing, importing a function raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libcsa2.so")

E8M0 = 0
E4M3 = 1
SWA_MAIN = 0  # window rows in the main-KV format
SWA_FP8 = 1  # window rows as FP8 records (576 + 8 B)

_lib = None


class Csa2Error(RuntimeError):
    pass


def lib():
    """Load libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise Csa2Error(
            f"{LIB_PATH} is missing: build it with `python -m compressed_kv_cache_mxfp4_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    L.csa2_status_string.restype = ctypes.c_char_p
    L.csa2_status_string.argtypes = [ctypes.c_int]
    L.csa2_version.restype = ctypes.c_char_p
    L.csa2_quantize_fp4.argtypes = [P, i64, i32, i32, i32, P, P, P]
    L.csa2_cache_write.argtypes = [P, P, i64, i32, P, f32, P, i32, P, P, P, P, P, P]
    L.csa2_append_state_bytes.restype = sz
    L.csa2_append_state_bytes.argtypes = [i32]
    L.csa2_cache_append.argtypes = [P, P, i32, i32, P, f32, P, i32, i32, P, P, P, P, i64, P, P, P]
    L.csa2_index_full_workspace.restype = sz
    L.csa2_index_full_workspace.argtypes = [i32, i64, i32, i32, i32]
    L.csa2_index_full.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.csa2_index_full_score.argtypes = [P, P, i64, P, i32, P, P, i32, i32, P, P, sz, P]
    L.csa2_index_full_select.argtypes = [i64, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.csa2_index_pool_score.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, i32, P, P, sz, P]
    L.csa2_index_pool_select.argtypes = [i32, P, P, i32, i32, P, P, P, sz, P]
    L.csa2_index_pool_workspace.restype = sz
    L.csa2_index_pool_workspace.argtypes = [i32, i32, i32]
    L.csa2_index_pool.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, i32, i32, P, P, P, sz, P]
    L.csa2_index_full_mq_workspace.restype = sz
    L.csa2_index_full_mq_workspace.argtypes = [i32, i32, i64, i32, i32, i32]
    L.csa2_index_full_mq.argtypes = [P, P, i64, P, i32, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.csa2_index_full_mq_fp4q.argtypes = [P, P, i64, P, i32, i32, P, P, P, i32, i32, i32, i32, P, P, P, P, P, sz,
                                          P]
    L.csa2_index_full_fp4q.argtypes = [P, P, i64, P, i32, P, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    L.csa2_index_pool_fp4q.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, P, i32, i32, P, P, P, sz, P]
    L.csa2_attn_workspace.restype = sz
    L.csa2_attn_workspace.argtypes = [i32, i32, i32, i32]
    L.csa2_sparse_attn_decode.argtypes = [P, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32,
                                          P, i32, f32, P, P, P, P, sz, P]
    L.csa2_sparse_attn_decode_noalloc.argtypes = [P, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32,
                                                  P, i32, f32, P, P, P, P]
    L.csa2_sparse_attn_decode_mq.argtypes = [P, i32, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32,
                                             P, i32, f32, P, P, P, P, sz, P]
    L.csa2_index_pool_mq.argtypes = [P, P, i64, P, i32, i32, P, P, i32, P, P, i32, i32, P, P, P, sz, P]
    L.csa2_index_pool_mq_fp4q.argtypes = [P, P, i64, P, i32, i32, P, P, i32, P, P, P, i32, i32, P, P, P, sz, P]
    L.csa2_window_write.argtypes = [P, i32, i32, P, f32, i32, P, i32, P, P, P, P]
    L.csa2_cache_append_paged.argtypes = [P, P, i32, i32, P, f32, P, i32, i32, P, P, P, P, i64, P, i32, i32, P, P, P]
    L.csa2_index_full_paged.argtypes = [P, P, i64, P, i32, i32, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, P,
                                        P, sz, P]
    L.csa2_index_pool_rows.argtypes = [P, P, i64, i32, P, P, P, i32, P, P, i32, i32, P, P, P, P, sz, P]
    L.csa2_sparse_attn_decode_rows.argtypes = [P, i32, P, P, i64, i32, P, i32, i32, P, P, i64, i32, P, i32, f32, P,
                                               P, P, P, sz, P]
    _lib = L
    return L


def _check(rc: int, what: str):
    if rc != 0:
        msg = lib().csa2_status_string(rc).decode()
        raise Csa2Error(f"{what}: {msg} (status {rc})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _req(t: torch.Tensor, name: str, dtype, dev=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


_WS = {}


def workspace(nbytes: int, dev: torch.device, kind: str = "index") -> torch.Tensor:
    """A cached, zero-initialised uint8 device buffer of at least nbytes, one
    per (device, stream, kind).  Calls on one stream are ordered, so they may
    share it.  The attention workspace starts with completion counters that
    must be zero and that every call leaves at zero, so it is never shared
    with the indexer's scratch."""
    key = (dev, torch.cuda.current_stream(dev).cuda_stream, kind)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _WS[key] = buf
    return buf


def _bits16(t: torch.Tensor) -> torch.Tensor:
    """bf16 tensors are passed as their 16-bit patterns."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t


# ------------------------------------------------------------------ quantiser
def quantize_fp4(x: torch.Tensor, group: int, fmt: int, codes=None, scales=None):
    """fp32 [..., dim] -> (codes u8 [..., dim/2], scales u8 [..., dim/group])."""
    _req(x, "x", torch.float32)
    dim = x.shape[-1]
    rows = x.numel() // dim if dim else 0
    dev = x.device
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (dim // 2,), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (dim // group,), dtype=torch.uint8, device=dev)
    _req(codes, "codes", torch.uint8, dev)
    _req(scales, "scales", torch.uint8, dev)
    _check(lib().csa2_quantize_fp4(_ptr(x), rows, dim, group, fmt, _ptr(codes), _ptr(scales),
                                   _stream(dev)), "csa2_quantize_fp4")
    return codes, scales


# ---------------------------------------------------------------- cache write
def cache_write(latent, gate, m: int, w_idx, main_fmt: int, gamma=None, eps: float = 1e-6,
                out=None, rope_pos=None):
    """latent/gate bf16 (or int16 bits) [T][512]; w_idx fp32 [512][128];
    rope_pos int64 [T/m] entry positions for the compressed RoPE (or None).

    Returns dict(main_codes [T/m][256], main_scales [T/m][32], idx_codes [T/m][64],
    idx_scales [T/m][4]); `out` may supply these tensors (e.g. views into a cache).
    """
    latent = _bits16(latent)
    _req(latent, "latent", torch.int16)
    dev = latent.device
    T = latent.shape[0]
    if m > 1:
        gate = _bits16(gate)
        _req(gate, "gate", torch.int16, dev, latent.shape)
    else:
        gate = None
    _req(w_idx, "w_idx", torch.float32, dev, (512, 128))
    if gamma is not None:
        _req(gamma, "gamma", torch.float32, dev, (512,))
    n = T // m
    if out is None:
        out = dict(
            main_codes=torch.empty(n, 256, dtype=torch.uint8, device=dev),
            main_scales=torch.empty(n, 32, dtype=torch.uint8, device=dev),
            idx_codes=torch.empty(n, 64, dtype=torch.uint8, device=dev),
            idx_scales=torch.empty(n, 4, dtype=torch.uint8, device=dev),
        )
    for key, width in (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4)):
        _req(out[key], key, torch.uint8, dev, (n, width))
    if rope_pos is not None:
        _req(rope_pos, "rope_pos", torch.int64, dev, (n,))
    _check(lib().csa2_cache_write(_ptr(latent), _ptr(gate), T, m, _ptr(gamma), float(eps),
                                  _ptr(w_idx), main_fmt, _ptr(rope_pos), _ptr(out["main_codes"]),
                                  _ptr(out["main_scales"]), _ptr(out["idx_codes"]),
                                  _ptr(out["idx_scales"]), _stream(dev)), "csa2_cache_write")
    return out


# -------------------------------------------------------------------- indexer
def append_state(B: int, device) -> torch.Tensor:
    """Zero-filled state for cache_append with m = 2 (held first tokens)."""
    return torch.zeros(max(int(lib().csa2_append_state_bytes(B)), 256), dtype=torch.uint8, device=device)


def cache_append(latent, gate, m: int, w_idx, main_fmt: int, cache: dict, lengths, state=None,
                 gamma=None, eps: float = 1e-6, rope: bool = False):
    """Decode-time append of one token per sequence into the cache planes.

    latent/gate bf16 (or int16 bits) [B][512]; cache: dict of the planes
    main_codes [B][cap][256], main_scales [B][cap][32], idx_codes [B][cap][64],
    idx_scales [B][cap][4]; lengths int32 [B] (advanced in place); state from
    append_state(B) when m == 2.  With rope, each entry is rotated at its row index.
    """
    latent = _bits16(latent)
    _req(latent, "latent", torch.int16)
    dev = latent.device
    B = latent.shape[0]
    _req(latent, "latent", torch.int16, dev, (B, 512))
    if m not in (1, 2):
        raise ValueError("m must be 1 or 2")
    if m == 2:
        gate = _bits16(gate)
        _req(gate, "gate", torch.int16, dev, (B, 512))
        if state is None:
            raise ValueError("m == 2 needs the append state")
        _req(state, "state", torch.uint8, dev)
        if state.numel() < lib().csa2_append_state_bytes(B):
            raise ValueError("append state too small")
    else:
        gate = None
    _req(w_idx, "w_idx", torch.float32, dev, (512, 128))
    if gamma is not None:
        _req(gamma, "gamma", torch.float32, dev, (512,))
    cap = cache["main_codes"].shape[1]
    for key, width in (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4)):
        _req(cache[key], key, torch.uint8, dev, (B, cap, width))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    _check(lib().csa2_cache_append(_ptr(latent), _ptr(gate), B, m, _ptr(gamma), float(eps), _ptr(w_idx),
                                   main_fmt, 1 if rope else 0, _ptr(cache["main_codes"]),
                                   _ptr(cache["main_scales"]), _ptr(cache["idx_codes"]),
                                   _ptr(cache["idx_scales"]), cap, _ptr(lengths),
                                   _ptr(state) if m == 2 else None, _stream(dev)), "csa2_cache_append")


def window_alloc(B: int, W: int = 128, device="cuda"):
    """Zeroed FP8 window ring: data u8 [B][W][576], scales u8 [B][W][8], swa_len int32 [B]."""
    return dict(data=torch.zeros(B, W, 576, dtype=torch.uint8, device=device),
                scales=torch.zeros(B, W, 8, dtype=torch.uint8, device=device),
                swa_len=torch.zeros(B, dtype=torch.int32, device=device))


def window_write(latent, pos0, window: dict, gamma=None, eps: float = 1e-6, rope: bool = False):
    """Write n tokens per sequence into the FP8 window ring (window_alloc's dict,
    updated in place).  latent bf16 (or int16 bits) [B][n][512]; pos0 int64 [B]:
    position of token 0; token at position p goes to slot p mod W."""
    latent = _bits16(latent)
    _req(latent, "latent", torch.int16)
    dev = latent.device
    B, n = latent.shape[0], latent.shape[1]
    _req(latent, "latent", torch.int16, dev, (B, n, 512))
    W = window["data"].shape[1]
    _req(window["data"], "window data", torch.uint8, dev, (B, W, 576))
    _req(window["scales"], "window scales", torch.uint8, dev, (B, W, 8))
    _req(window["swa_len"], "swa_len", torch.int32, dev, (B,))
    _req(pos0, "pos0", torch.int64, dev, (B,))
    if gamma is not None:
        _req(gamma, "gamma", torch.float32, dev, (512,))
    _check(lib().csa2_window_write(_ptr(latent), B, n, _ptr(gamma), float(eps), 1 if rope else 0, _ptr(pos0), W,
                                   _ptr(window["data"]), _ptr(window["scales"]), _ptr(window["swa_len"]),
                                   _stream(dev)), "csa2_window_write")


# ---------------------------------------------------------------- paged cache
def paged_alloc(n_pages: int, page_shift: int, device="cuda"):
    """Zeroed pool of n_pages pages of 2^page_shift entries: the four planes
    main_codes [R][256], main_scales [R][32], idx_codes [R][64], idx_scales [R][4]."""
    R = n_pages << page_shift
    return {k_: torch.zeros(R, wd, dtype=torch.uint8, device=device)
            for k_, wd in (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4))}


def _pool_rows(pool):
    R = pool["main_codes"].shape[0]
    for key, width in (("main_codes", 256), ("main_scales", 32), ("idx_codes", 64), ("idx_scales", 4)):
        _req(pool[key], key, torch.uint8, pool["main_codes"].device, (R, width))
    return R


def cache_append_paged(latent, gate, m: int, w_idx, main_fmt: int, pool: dict, table, page_shift: int, lengths,
                       state=None, gamma=None, eps: float = 1e-6, rope: bool = False):
    """cache_append into a paged pool (paged_alloc's dict); table int32 [B][max_pages]."""
    latent = _bits16(latent)
    dev = latent.device
    B = latent.shape[0]
    _req(latent, "latent", torch.int16, dev, (B, 512))
    if m == 2:
        gate = _bits16(gate)
        _req(gate, "gate", torch.int16, dev, (B, 512))
        if state is None or state.numel() < lib().csa2_append_state_bytes(B):
            raise ValueError("m == 2 needs the append state")
    else:
        gate = None
    R = _pool_rows(pool)
    _req(table, "table", torch.int32, dev, (B, table.shape[1]))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    _check(lib().csa2_cache_append_paged(_ptr(latent), _ptr(gate), B, m, _ptr(gamma), float(eps), _ptr(w_idx),
                                         main_fmt, 1 if rope else 0, _ptr(pool["main_codes"]),
                                         _ptr(pool["main_scales"]), _ptr(pool["idx_codes"]), _ptr(pool["idx_scales"]),
                                         R, _ptr(table), page_shift, table.shape[1], _ptr(lengths),
                                         _ptr(state) if m == 2 else None, _stream(dev)), "csa2_cache_append_paged")


def index_full_paged(pool: dict, table, page_shift: int, lengths, q, w, k: int = 512, n_blocks: int = 2048,
                     return_scores: bool = False, out=None, _ws=None):
    """index_full over a paged pool.  Returns (topk, topk_rows, pool, pool_rows,
    pool_len[, scores]); positions are logical, *_rows are pool rows."""
    q = _bits16(q)
    dev = q.device
    B, H = q.shape[0], q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 128))
    _req(w, "w", torch.float32, dev, (B, H))
    R = _pool_rows(pool)
    _req(table, "table", torch.int32, dev, (B, table.shape[1]))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    cap = table.shape[1] << page_shift
    out = out or {}
    nb8 = max(n_blocks * 8, 1)
    res = {}
    for key, shape in (("topk", (B, k)), ("topk_rows", (B, k)), ("pool", (B, nb8)), ("pool_rows", (B, nb8)),
                       ("pool_len", (B,))):
        res[key] = out.get(key)
        if res[key] is None:
            res[key] = torch.empty(*shape, dtype=torch.int32, device=dev)
    scores = out.get("scores")
    if return_scores and scores is None:
        scores = torch.empty(B, cap, dtype=torch.float32, device=dev)
    ws = _ws if _ws is not None else workspace(lib().csa2_index_full_workspace(B, cap, k, 8, n_blocks), dev)
    _check(lib().csa2_index_full_paged(_ptr(pool["idx_codes"]), _ptr(pool["idx_scales"]), R, _ptr(table), page_shift,
                                       table.shape[1], _ptr(lengths), B, _ptr(q), _ptr(w), H, k, 8, n_blocks,
                                       _ptr(res["topk"]), _ptr(res["topk_rows"]), _ptr(res["pool"]),
                                       _ptr(res["pool_rows"]), _ptr(res["pool_len"]), _ptr(scores), _ptr(ws),
                                       ws.numel(), _stream(dev)), "csa2_index_full_paged")
    r = (res["topk"], res["topk_rows"], res["pool"][:, : n_blocks * 8], res["pool_rows"][:, : n_blocks * 8],
         res["pool_len"])
    return r + (scores,) if return_scores else r


def index_pool_rows(pool: dict, cand, cand_rows, cand_len, q, w, k: int = 512, out=None, _ws=None):
    """Reindex over a paged pool: candidates given by logical positions `cand`
    and pool rows `cand_rows` [B][pool_cap].  Returns (topk, topk_rows)."""
    q = _bits16(q)
    dev = q.device
    B, H = q.shape[0], q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 128))
    _req(w, "w", torch.float32, dev, (B, H))
    R = _pool_rows(pool)
    pool_cap = cand.shape[1]
    _req(cand, "pool", torch.int32, dev, (B, pool_cap))
    _req(cand_rows, "pool_rows", torch.int32, dev, (B, pool_cap))
    _req(cand_len, "pool_len", torch.int32, dev, (B,))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=dev)
    topk_rows = out.get("topk_rows")
    if topk_rows is None:
        topk_rows = torch.empty(B, k, dtype=torch.int32, device=dev)
    wsb = lib().csa2_index_pool_workspace(B, pool_cap, k)
    ws = _ws if _ws is not None else workspace(max(wsb, 256), dev)
    _check(lib().csa2_index_pool_rows(_ptr(pool["idx_codes"]), _ptr(pool["idx_scales"]), R, B, _ptr(cand),
                                      _ptr(cand_rows), _ptr(cand_len), pool_cap, _ptr(q), _ptr(w), H, k, _ptr(topk),
                                      _ptr(topk_rows), None, _ptr(ws), ws.numel(), _stream(dev)),
           "csa2_index_pool_rows")
    return topk, topk_rows


def sparse_attn_decode_rows(q, pool: dict, rows, main_fmt: int, swa_codes=None, swa_scales=None, swa_len=None,
                            swa_stride: int = 0, swa_cap: int = 0, swa_fmt: int = 0, sm_scale: Optional[float] = None,
                            return_lse: bool = False, out=None, _ws=None, q_pos=None):
    """sparse_attn_decode with the selected entries as pool rows [B][k] of a paged pool."""
    q = _bits16(q)
    dev = q.device
    B, H = q.shape[0], q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 512))
    R = _pool_rows(pool)
    k = rows.shape[1]
    _req(rows, "rows", torch.int32, dev, (B, k))
    if swa_cap > 0:
        _req(swa_len, "swa_len", torch.int32, dev, (B,))
        rb, sb = (576, 8) if swa_fmt == SWA_FP8 else (256, 32)
        need = (B - 1) * swa_stride + swa_cap
        if swa_codes.numel() < need * rb or swa_scales.numel() < need * sb:
            raise ValueError("window planes smaller than B rows of swa_stride")
    if q_pos is not None:
        _req(q_pos, "q_pos", torch.int64, dev, (B,))
    if sm_scale is None:
        sm_scale = 1.0 / (512 ** 0.5)
    o = None if out is None else out.get("out")
    if o is None:
        o = torch.empty(B, H, 512, dtype=torch.int16, device=dev)
    lse = torch.empty(B, H, dtype=torch.float32, device=dev) if return_lse else None
    ws = _ws if _ws is not None else workspace(lib().csa2_attn_workspace(B, H, k, swa_cap), dev, "attn")
    _check(lib().csa2_sparse_attn_decode_rows(
        _ptr(q), H, _ptr(pool["main_codes"]), _ptr(pool["main_scales"]), R, main_fmt, _ptr(rows), k, B,
        _ptr(swa_codes) if swa_cap else None, _ptr(swa_scales) if swa_cap else None, swa_stride, swa_cap,
        _ptr(swa_len) if swa_cap else None, int(swa_fmt) if swa_cap else 0, float(sm_scale), _ptr(q_pos), _ptr(o),
        _ptr(lse), _ptr(ws), ws.numel(), _stream(dev)), "csa2_sparse_attn_decode_rows")
    return (o, lse) if return_lse else o


def _index_query(q, dev, B):
    """bf16 queries [B][H][128] -> (H, q bits, None, None); FP4 queries given as
    (codes u8 [B][H][64], E8M0 scales u8 [B][H][4]) -> (H, None, codes, scales)."""
    if isinstance(q, (tuple, list)):
        qc, qs = q
        H = qc.shape[1]
        _req(qc, "q codes", torch.uint8, dev, (B, H, 64))
        _req(qs, "q scales", torch.uint8, dev, (B, H, 4))
        return H, None, qc, qs
    q = _bits16(q)
    H = q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 128))
    return H, q, None, None


def index_full(idx_codes, idx_scales, lengths, q, w, k: int = 512, n_blocks: int = 2048,
               block: int = 8, return_scores: bool = False, out=None, _ws=None):
    """Full-mode indexer over B sequences.

    idx_codes u8 [B][cap][64], idx_scales u8 [B][cap][4], lengths int32 [B],
    q bf16/int16 [B][H][128] -- or an FP4 query (codes u8 [B][H][64], E8M0
    scales u8 [B][H][4]), which selects csa2_index_full_fp4q -- and w fp32 [B][H].
    Returns (topk int32 [B][k], pool int32 [B][n_blocks*block], pool_len int32 [B]
    [, scores fp32 [B][cap]]).
    """
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_codes, "idx_codes", torch.uint8, dev, (B, cap, 64))
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    H, q, qc, qs = _index_query(q, dev, B)
    _req(w, "w", torch.float32, dev, (B, H))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=dev)
    pool = out.get("pool")
    if pool is None:
        pool = torch.empty(B, max(n_blocks * block, 1), dtype=torch.int32, device=dev)
    pool_len = out.get("pool_len")
    if pool_len is None:
        pool_len = torch.empty(B, dtype=torch.int32, device=dev)
    scores = out.get("scores")
    if return_scores and scores is None:
        scores = torch.empty(B, cap, dtype=torch.float32, device=dev)
    wsb = lib().csa2_index_full_workspace(B, cap, k, block, n_blocks)
    ws = _ws if _ws is not None else workspace(wsb, dev)
    if qc is None:
        _check(lib().csa2_index_full(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, _ptr(q),
                                     _ptr(w), H, k, block, n_blocks, _ptr(topk), _ptr(pool),
                                     _ptr(pool_len), _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)),
               "csa2_index_full")
    else:
        _check(lib().csa2_index_full_fp4q(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B,
                                          _ptr(qc), _ptr(qs), _ptr(w), H, k, block, n_blocks, _ptr(topk),
                                          _ptr(pool), _ptr(pool_len), _ptr(scores), _ptr(ws), ws.numel(),
                                          _stream(dev)),
               "csa2_index_full_fp4q")
    pool = pool[:, : n_blocks * block]
    if return_scores:
        return topk, pool, pool_len, scores
    return topk, pool, pool_len


def index_full_score(idx_codes, idx_scales, lengths, q, w, ws, scores=None, block: int = 8):
    """Phase 1 of index_full (csa2_index_full_score): scores (into `scores`
    fp32 [B][cap] when given, else the workspace) and block maxima (into the
    workspace `ws`, csa2_index_full_workspace bytes).  bf16 queries only."""
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_codes, "idx_codes", torch.uint8, dev, (B, cap, 64))
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    q = _bits16(q)
    H = q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 128))
    _req(w, "w", torch.float32, dev, (B, H))
    if scores is not None:
        _req(scores, "scores", torch.float32, dev, (B, cap))
    _check(lib().csa2_index_full_score(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, _ptr(q), _ptr(w),
                                       H, block, _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)),
           "csa2_index_full_score")


def index_full_select(cap: int, lengths, ws, k: int = 512, n_blocks: int = 2048, scores=None, block: int = 8,
                      out=None):
    """Phase 2 of index_full (csa2_index_full_select): the top-k and the pool
    from the scores and block maxima a preceding index_full_score left in
    `ws` (and `scores`, if it was given one).  Returns (topk, pool, pool_len)."""
    dev = lengths.device
    B = lengths.shape[0]
    _req(lengths, "lengths", torch.int32, dev, (B,))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=dev)
    pool = out.get("pool")
    if pool is None:
        pool = torch.empty(B, max(n_blocks * block, 1), dtype=torch.int32, device=dev)
    pool_len = out.get("pool_len")
    if pool_len is None:
        pool_len = torch.empty(B, dtype=torch.int32, device=dev)
    _check(lib().csa2_index_full_select(cap, _ptr(lengths), B, k, block, n_blocks, _ptr(topk), _ptr(pool),
                                        _ptr(pool_len), _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)),
           "csa2_index_full_select")
    return topk, pool[:, : n_blocks * block], pool_len


def index_pool_mq(idx_codes, idx_scales, lengths, pool, pool_len, q, w, k: int = 512,
                  return_scores: bool = False, out=None, _ws=None):
    """Reindex for Q queries per sequence (csa2_index_pool_mq): pool int32
    [B][Q][pool_cap], pool_len [B][Q], q bf16 [B][Q][H][128] -- or FP4 queries
    (codes u8 [B][Q][H][64], E8M0 scales u8 [B][Q][H][4],
    csa2_index_pool_mq_fp4q) -- w fp32 [B][Q][H]; the indexer cache and
    lengths [B] are per sequence.  Returns topk int32 [B][Q][k] (and the pool
    scores fp32 [B][Q][pool_cap])."""
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_codes, "idx_codes", torch.uint8, dev, (B, cap, 64))
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    if isinstance(q, (tuple, list)):
        qc, qs = q
        Q, H = qc.shape[1], qc.shape[2]
        _req(qc, "q codes", torch.uint8, dev, (B, Q, H, 64))
        _req(qs, "q scales", torch.uint8, dev, (B, Q, H, 4))
        q = None
    else:
        q = _bits16(q)
        if q.dim() != 4:
            raise ValueError("q must be [B][Q][H][128]")
        Q, H = q.shape[1], q.shape[2]
        _req(q, "q", torch.int16, dev, (B, Q, H, 128))
    _req(w, "w", torch.float32, dev, (B, Q, H))
    pool_cap = pool.shape[2]
    _req(pool, "pool", torch.int32, dev, (B, Q, pool_cap))
    _req(pool_len, "pool_len", torch.int32, dev, (B, Q))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    ps = out.get("pool_scores")
    if return_scores and ps is None:
        ps = torch.empty(B, Q, pool_cap, dtype=torch.float32, device=dev)
    ws = _ws if _ws is not None else workspace(lib().csa2_index_pool_workspace(B * Q, pool_cap, k), dev, "pool")
    if q is None:
        _check(lib().csa2_index_pool_mq_fp4q(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, Q,
                                             _ptr(pool), _ptr(pool_len), pool_cap, _ptr(qc), _ptr(qs), _ptr(w), H,
                                             k, _ptr(topk), _ptr(ps), _ptr(ws), ws.numel(), _stream(dev)),
               "csa2_index_pool_mq_fp4q")
    else:
        _check(lib().csa2_index_pool_mq(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, Q, _ptr(pool),
                                        _ptr(pool_len), pool_cap, _ptr(q), _ptr(w), H, k, _ptr(topk), _ptr(ps),
                                        _ptr(ws), ws.numel(), _stream(dev)), "csa2_index_pool_mq")
    return (topk, ps) if return_scores else topk


def index_pool_score(idx_codes, idx_scales, lengths, pool, pool_len, q, w, ws, pool_scores=None):
    """Phase 1 of index_pool (csa2_index_pool_score): pool scores (into
    `pool_scores` when given, else `ws`) and group maxima (into `ws`)."""
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    pool_cap = pool.shape[1]
    _req(pool, "pool", torch.int32, dev, (B, pool_cap))
    _req(pool_len, "pool_len", torch.int32, dev, (B,))
    q = _bits16(q)
    H = q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 128))
    _req(w, "w", torch.float32, dev, (B, H))
    if pool_scores is not None:
        _req(pool_scores, "pool_scores", torch.float32, dev, (B, pool_cap))
    _check(lib().csa2_index_pool_score(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, _ptr(pool),
                                       _ptr(pool_len), pool_cap, _ptr(q), _ptr(w), H, _ptr(pool_scores), _ptr(ws),
                                       ws.numel(), _stream(dev)), "csa2_index_pool_score")


def index_pool_select(pool, pool_len, ws, k: int = 512, pool_scores=None, out=None):
    """Phase 2 of index_pool (csa2_index_pool_select): the layer's top-k."""
    dev = pool.device
    B, pool_cap = pool.shape
    _req(pool, "pool", torch.int32, dev, (B, pool_cap))
    _req(pool_len, "pool_len", torch.int32, dev, (B,))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=dev)
    _check(lib().csa2_index_pool_select(B, _ptr(pool), _ptr(pool_len), pool_cap, k, _ptr(topk), _ptr(pool_scores),
                                        _ptr(ws), ws.numel(), _stream(dev)), "csa2_index_pool_select")
    return topk


def index_full_mq(idx_codes, idx_scales, lengths, q, w, k: int = 512, n_blocks: int = 2048,
                  block: int = 8, return_scores: bool = False, out=None, _ws=None):
    """Full-mode indexer for Q queries per sequence sharing the sequence's cache
    (e.g. a verify block).  q bf16/int16 [B][Q][H][128] -- or FP4 queries
    (codes u8 [B][Q][H][64], E8M0 scales u8 [B][Q][H][4]) -- w fp32 [B][Q][H],
    lengths int32 [B].  Returns (topk [B][Q][k], pool [B][Q][n_blocks*block],
    pool_len [B][Q] [, scores fp32 [B][Q][cap]])."""
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_codes, "idx_codes", torch.uint8, dev, (B, cap, 64))
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    if isinstance(q, (tuple, list)):
        qc, qs = q
        Q, H = qc.shape[1], qc.shape[2]
        _req(qc, "q codes", torch.uint8, dev, (B, Q, H, 64))
        _req(qs, "q scales", torch.uint8, dev, (B, Q, H, 4))
        q = None
    else:
        q = _bits16(q)
        Q, H = q.shape[1], q.shape[2]
        _req(q, "q", torch.int16, dev, (B, Q, H, 128))
        qc = qs = None
    _req(w, "w", torch.float32, dev, (B, Q, H))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, Q, k, dtype=torch.int32, device=dev)
    pool = out.get("pool")
    if pool is None:
        pool = torch.empty(B, Q, max(n_blocks * block, 1), dtype=torch.int32, device=dev)
    pool_len = out.get("pool_len")
    if pool_len is None:
        pool_len = torch.empty(B, Q, dtype=torch.int32, device=dev)
    scores = out.get("scores")
    if return_scores and scores is None:
        scores = torch.empty(B, Q, cap, dtype=torch.float32, device=dev)
    wsb = lib().csa2_index_full_mq_workspace(B, Q, cap, k, block, n_blocks)
    ws = _ws if _ws is not None else workspace(wsb, dev)
    if qc is None:
        _check(lib().csa2_index_full_mq(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, Q, _ptr(q),
                                        _ptr(w), H, k, block, n_blocks, _ptr(topk), _ptr(pool), _ptr(pool_len),
                                        _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)), "csa2_index_full_mq")
    else:
        _check(lib().csa2_index_full_mq_fp4q(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B, Q, _ptr(qc),
                                             _ptr(qs), _ptr(w), H, k, block, n_blocks, _ptr(topk), _ptr(pool),
                                             _ptr(pool_len), _ptr(scores), _ptr(ws), ws.numel(), _stream(dev)),
               "csa2_index_full_mq_fp4q")
    pool = pool[:, :, : n_blocks * block]
    if return_scores:
        return topk, pool, pool_len, scores
    return topk, pool, pool_len


def index_pool(idx_codes, idx_scales, lengths, pool, pool_len, q, w, k: int = 512,
               return_scores: bool = False, out=None, _ws=None):
    """Reindex mode: rescore pool [B][pool_cap] with (q, w), top-k per sequence.
    q: bf16 [B][H][128], or an FP4 query (codes, scales) as in index_full."""
    _req(idx_codes, "idx_codes", torch.uint8)
    dev = idx_codes.device
    B, cap = idx_codes.shape[0], idx_codes.shape[1]
    _req(idx_scales, "idx_scales", torch.uint8, dev, (B, cap, 4))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    pool_cap = pool.shape[1]
    _req(pool, "pool", torch.int32, dev, (B, pool_cap))
    _req(pool_len, "pool_len", torch.int32, dev, (B,))
    H, q, qc, qs = _index_query(q, dev, B)
    _req(w, "w", torch.float32, dev, (B, H))
    out = out or {}
    topk = out.get("topk")
    if topk is None:
        topk = torch.empty(B, k, dtype=torch.int32, device=dev)
    ps = out.get("pool_scores")
    if return_scores and ps is None:
        ps = torch.empty(B, pool_cap, dtype=torch.float32, device=dev)
    wsb = lib().csa2_index_pool_workspace(B, pool_cap, k)
    ws = _ws if _ws is not None else workspace(wsb, dev, "pool")
    if qc is None:
        _check(lib().csa2_index_pool(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B,
                                     _ptr(pool), _ptr(pool_len), pool_cap, _ptr(q), _ptr(w), H, k,
                                     _ptr(topk), _ptr(ps), _ptr(ws), ws.numel(), _stream(dev)),
               "csa2_index_pool")
    else:
        _check(lib().csa2_index_pool_fp4q(_ptr(idx_codes), _ptr(idx_scales), cap, _ptr(lengths), B,
                                          _ptr(pool), _ptr(pool_len), pool_cap, _ptr(qc), _ptr(qs), _ptr(w),
                                          H, k, _ptr(topk), _ptr(ps), _ptr(ws), ws.numel(), _stream(dev)),
               "csa2_index_pool_fp4q")
    return (topk, ps) if return_scores else topk


# ------------------------------------------------------------------ attention
def sparse_attn_decode(q, main_codes, main_scales, lengths, topk, main_fmt: int,
                       swa_codes=None, swa_scales=None, swa_len=None, swa_stride: int = 0,
                       swa_cap: int = 0, swa_row0: int = 0, sm_scale: Optional[float] = None,
                       return_lse: bool = False, out=None, _ws=None, q_pos=None, swa_fmt: int = 0):
    """Sparse attention over topk rows ++ window rows.

    q bf16/int16 [B][H][512]; main planes [B][cap][256] / [B][cap][32];
    topk int32 [B][k]; window row r of sequence b is row swa_row0 + b*swa_stride + r
    of the contiguous tensors swa_codes / swa_scales, so the window may be a
    separate buffer or the tail of the main cache (swa_codes=main_codes,
    swa_row0=cap-128, swa_stride=cap); swa_len int32 [B].  swa_fmt 0: window rows
    in the main format (rows of 256 B / 32 B); swa_fmt 1 (SWA_FP8): FP8 window
    records (rows of 576 B / 8 B, as window_write produces).
    q_pos int64 [B]: query positions for Q RoPE and output inverse RoPE (or None).
    Returns out bf16 bits (int16) [B][H][512] (and lse fp32 [B][H]).
    """
    q = _bits16(q)
    _req(q, "q", torch.int16)
    dev = q.device
    B, H = q.shape[0], q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 512))
    cap = main_codes.shape[1]
    _req(main_codes, "main_codes", torch.uint8, dev, (B, cap, 256))
    _req(main_scales, "main_scales", torch.uint8, dev, (B, cap, 32))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    k = topk.shape[1]
    _req(topk, "topk", torch.int32, dev, (B, k))
    if swa_cap > 0:
        if swa_codes.dtype != torch.uint8 or swa_scales.dtype != torch.uint8:
            raise TypeError("window planes must be uint8")
        if swa_codes.device != dev or swa_scales.device != dev:
            raise ValueError("window planes on another device")
        if not (swa_codes.is_contiguous() and swa_scales.is_contiguous()):
            raise ValueError("window planes must be contiguous")
        if swa_fmt not in (SWA_MAIN, SWA_FP8):
            raise ValueError("swa_fmt must be 0 (main format) or 1 (FP8 records)")
        rb, sb = (576, 8) if swa_fmt == SWA_FP8 else (256, 32)
        need = swa_row0 + (B - 1) * swa_stride + swa_cap
        if swa_row0 < 0 or swa_codes.numel() < need * rb or swa_scales.numel() < need * sb:
            raise ValueError("window planes smaller than swa_row0 + B rows of swa_stride")
        _req(swa_len, "swa_len", torch.int32, dev, (B,))
    if sm_scale is None:
        sm_scale = 1.0 / (512 ** 0.5)
    if q_pos is not None:
        _req(q_pos, "q_pos", torch.int64, dev, (B,))
    o = None if out is None else out.get("out")
    if o is None:
        o = torch.empty(B, H, 512, dtype=torch.int16, device=dev)
    lse = None
    if return_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    wsb = lib().csa2_attn_workspace(B, H, k, swa_cap)
    ws = _ws if _ws is not None else workspace(wsb, dev, "attn")
    _check(lib().csa2_sparse_attn_decode(
        _ptr(q), H, _ptr(main_codes), _ptr(main_scales), cap, main_fmt, _ptr(lengths), _ptr(topk), k,
        B, ctypes.c_void_p(swa_codes.data_ptr() + rb * swa_row0) if swa_cap else None,
        ctypes.c_void_p(swa_scales.data_ptr() + sb * swa_row0) if swa_cap else None,
        swa_stride, swa_cap, _ptr(swa_len) if swa_cap else None, int(swa_fmt) if swa_cap else 0,
        float(sm_scale), _ptr(q_pos), _ptr(o),
        _ptr(lse), _ptr(ws), ws.numel(), _stream(dev)), "csa2_sparse_attn_decode")
    return (o, lse) if return_lse else o


def sparse_attn_decode_mq(q, main_codes, main_scales, lengths, topk, main_fmt: int,
                          swa_codes=None, swa_scales=None, swa_len=None, swa_stride: int = 0,
                          swa_cap: int = 0, swa_row0: int = 0, sm_scale: Optional[float] = None,
                          return_lse: bool = False, out=None, _ws=None, q_pos=None, swa_fmt: int = 0):
    """Q queries per sequence in one call (csa2_sparse_attn_decode_mq): q bf16/int16
    [B][Q][H][512], topk int32 [B][Q][k], q_pos int64 [B][Q] or None; the caches,
    lengths [B] and windows (as in sparse_attn_decode) are per sequence.  Returns
    out bf16 bits (int16) [B][Q][H][512] (and lse fp32 [B][Q][H])."""
    q = _bits16(q)
    _req(q, "q", torch.int16)
    dev = q.device
    if q.dim() != 4:
        raise ValueError("q must be [B][Q][H][512]")
    B, Q, H = q.shape[0], q.shape[1], q.shape[2]
    _req(q, "q", torch.int16, dev, (B, Q, H, 512))
    cap = main_codes.shape[1]
    _req(main_codes, "main_codes", torch.uint8, dev, (B, cap, 256))
    _req(main_scales, "main_scales", torch.uint8, dev, (B, cap, 32))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    k = topk.shape[2]
    _req(topk, "topk", torch.int32, dev, (B, Q, k))
    rb, sb = (576, 8) if swa_fmt == SWA_FP8 else (256, 32)
    if swa_cap > 0:
        if swa_codes.dtype != torch.uint8 or swa_scales.dtype != torch.uint8:
            raise TypeError("window planes must be uint8")
        if swa_codes.device != dev or swa_scales.device != dev:
            raise ValueError("window planes on another device")
        if not (swa_codes.is_contiguous() and swa_scales.is_contiguous()):
            raise ValueError("window planes must be contiguous")
        if swa_fmt not in (SWA_MAIN, SWA_FP8):
            raise ValueError("swa_fmt must be 0 (main format) or 1 (FP8 records)")
        need = swa_row0 + (B - 1) * swa_stride + swa_cap
        if swa_row0 < 0 or swa_codes.numel() < need * rb or swa_scales.numel() < need * sb:
            raise ValueError("window planes smaller than swa_row0 + B rows of swa_stride")
        _req(swa_len, "swa_len", torch.int32, dev, (B,))
    if sm_scale is None:
        sm_scale = 1.0 / (512 ** 0.5)
    if q_pos is not None:
        _req(q_pos, "q_pos", torch.int64, dev, (B, Q))
    o = None if out is None else out.get("out")
    if o is None:
        o = torch.empty(B, Q, H, 512, dtype=torch.int16, device=dev)
    lse = torch.empty(B, Q, H, dtype=torch.float32, device=dev) if return_lse else None
    ws = _ws if _ws is not None else workspace(lib().csa2_attn_workspace(B * Q, H, k, swa_cap), dev, "attn")
    _check(lib().csa2_sparse_attn_decode_mq(
        _ptr(q), H, Q, _ptr(main_codes), _ptr(main_scales), cap, main_fmt, _ptr(lengths), _ptr(topk), k, B,
        ctypes.c_void_p(swa_codes.data_ptr() + rb * swa_row0) if swa_cap else None,
        ctypes.c_void_p(swa_scales.data_ptr() + sb * swa_row0) if swa_cap else None,
        swa_stride, swa_cap, _ptr(swa_len) if swa_cap else None, int(swa_fmt) if swa_cap else 0,
        float(sm_scale), _ptr(q_pos), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(dev)),
        "csa2_sparse_attn_decode_mq")
    return (o, lse) if return_lse else o


def sparse_attn_decode_noalloc(q, main_codes, main_scales, lengths, topk, main_fmt: int, out, lse=None,
                               swa_codes=None, swa_scales=None, swa_len=None, swa_stride: int = 0,
                               swa_cap: int = 0, swa_row0: int = 0, sm_scale: Optional[float] = None,
                               q_pos=None, swa_fmt: int = 0):
    """sparse_attn_decode through csa2_sparse_attn_decode_noalloc: the library's
    own per-GPU scratch instead of a workspace, and caller-provided outputs
    (`out` int16 [B][H][512], optional `lse` fp32 [B][H]), so that neither
    this call nor the library allocates.  Arguments as sparse_attn_decode."""
    q = _bits16(q)
    _req(q, "q", torch.int16)
    dev = q.device
    B, H = q.shape[0], q.shape[1]
    _req(q, "q", torch.int16, dev, (B, H, 512))
    cap = main_codes.shape[1]
    _req(main_codes, "main_codes", torch.uint8, dev, (B, cap, 256))
    _req(main_scales, "main_scales", torch.uint8, dev, (B, cap, 32))
    _req(lengths, "lengths", torch.int32, dev, (B,))
    k = topk.shape[1]
    _req(topk, "topk", torch.int32, dev, (B, k))
    _req(out, "out", torch.int16, dev, (B, H, 512))
    if lse is not None:
        _req(lse, "lse", torch.float32, dev, (B, H))
    rb, sb = (576, 8) if swa_fmt == SWA_FP8 else (256, 32)
    if swa_cap > 0:
        if swa_codes.dtype != torch.uint8 or swa_scales.dtype != torch.uint8:
            raise TypeError("window planes must be uint8")
        if swa_codes.device != dev or swa_scales.device != dev:
            raise ValueError("window planes on another device")
        if not (swa_codes.is_contiguous() and swa_scales.is_contiguous()):
            raise ValueError("window planes must be contiguous")
        need = swa_row0 + (B - 1) * swa_stride + swa_cap
        if swa_row0 < 0 or swa_codes.numel() < need * rb or swa_scales.numel() < need * sb:
            raise ValueError("window planes smaller than swa_row0 + B rows of swa_stride")
        _req(swa_len, "swa_len", torch.int32, dev, (B,))
    if sm_scale is None:
        sm_scale = 1.0 / (512 ** 0.5)
    if q_pos is not None:
        _req(q_pos, "q_pos", torch.int64, dev, (B,))
    _check(lib().csa2_sparse_attn_decode_noalloc(
        _ptr(q), H, _ptr(main_codes), _ptr(main_scales), cap, main_fmt, _ptr(lengths), _ptr(topk), k,
        B, ctypes.c_void_p(swa_codes.data_ptr() + rb * swa_row0) if swa_cap else None,
        ctypes.c_void_p(swa_scales.data_ptr() + sb * swa_row0) if swa_cap else None,
        swa_stride, swa_cap, _ptr(swa_len) if swa_cap else None, int(swa_fmt) if swa_cap else 0,
        float(sm_scale), _ptr(q_pos), _ptr(out), _ptr(lse), _stream(dev)), "csa2_sparse_attn_decode_noalloc")
    return out
