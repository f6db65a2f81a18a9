"""Host-only checks of the C-ABI library (no GPU needed).

The library loads, exports every function declared in include/csa2.h, and the
host-side argument validation rejects bad calls with the documented status
before anything is launched (so these calls never touch a device).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")
LIB = os.path.join(ROOT, "compressed_kv_cache_mxfp4_amd", "lib", "libcsa2.so")

CSA2_OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_SCRATCH = range(8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from compressed_kv_cache_mxfp4_amd import build

        build.build()
    L = ctypes.CDLL(LIB)
    L.csa2_status_string.restype = ctypes.c_char_p
    return L


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert {"csa2_cache_write", "csa2_cache_append", "csa2_append_state_bytes", "csa2_index_full",
            "csa2_index_pool", "csa2_sparse_attn_decode", "csa2_window_write", "csa2_index_full_mq", "csa2_index_full_mq_fp4q",
            "csa2_cache_append_paged", "csa2_index_full_paged", "csa2_index_pool_rows",
            "csa2_sparse_attn_decode_rows", "csa2_sparse_attn_decode_mq", "csa2_index_pool_mq", "csa2_index_pool_mq_fp4q",
            "csa2_quantize_fp4"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in csa2.h but not exported"


def test_status_strings(lib):
    for code in range(8):
        assert lib.csa2_status_string(code) != b"unknown status"
    assert lib.csa2_status_string(99) == b"unknown status"


P = ctypes.c_void_p
FAKE = P(0x1000)       # never dereferenced: validation fails first
FAKE_ODD = P(0x1001)


def test_quantize_validation(lib):
    f = lib.csa2_quantize_fp4
    f.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P]
    assert f(FAKE, 4, 48, 32, 0, FAKE, FAKE, None) == ERR_SHAPE       # dim % group
    assert f(FAKE, 4, 64, 8, 0, FAKE, FAKE, None) == ERR_SHAPE        # group
    assert f(FAKE, 4, 64, 32, 7, FAKE, FAKE, None) == ERR_UNSUP       # format
    assert f(None, 4, 64, 32, 0, FAKE, FAKE, None) == ERR_NULL
    assert f(FAKE_ODD, 4, 64, 32, 0, FAKE, FAKE, None) == ERR_ALIGN
    assert f(None, 0, 64, 32, 0, None, None, None) == CSA2_OK         # empty: nothing to do


def test_cache_write_validation(lib):
    f = lib.csa2_cache_write
    f.argtypes = [P, P, ctypes.c_int64, ctypes.c_int32, P, ctypes.c_float, P, ctypes.c_int32, P, P, P, P, P, P]
    assert f(FAKE, FAKE, 7, 2, None, 1e-6, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE  # T % m
    assert f(FAKE, FAKE, 8, 9, None, 1e-6, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE  # m
    assert f(FAKE, None, 8, 2, None, 1e-6, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_NULL  # gate
    assert f(FAKE, None, 8, 1, None, 1e-6, FAKE, 5, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_UNSUP
    assert f(FAKE_ODD, None, 8, 1, None, 1e-6, FAKE, 0, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_ALIGN
    assert f(FAKE, None, 8, 1, None, 1e-6, FAKE, 0, FAKE_ODD, FAKE, FAKE, FAKE, FAKE, None) == ERR_ALIGN  # positions
    assert f(FAKE, None, 8, 1, None, 1e-6, P(0x1004), 0, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_ALIGN  # w_idx


def test_cache_append_validation(lib):
    f = lib.csa2_cache_append
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f.argtypes = [P, P, i32, i32, P, ctypes.c_float, P, i32, i32, P, P, P, P, i64, P, P, P]
    lib.csa2_append_state_bytes.restype = ctypes.c_size_t
    lib.csa2_append_state_bytes.argtypes = [i32]
    assert lib.csa2_append_state_bytes(16) == 256 + 16 * 2048
    assert lib.csa2_append_state_bytes(0) == 0
    base = [FAKE, FAKE, 4, 2, None, 1e-6, FAKE, 0, 1, FAKE, FAKE, FAKE, FAKE, 4096, FAKE, FAKE, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return f(*args)

    assert call(3, 3) == ERR_SHAPE        # m
    assert call(13, 0) == ERR_SHAPE       # cap
    assert call(7, 9) == ERR_UNSUP        # scale format
    assert call(15, None) == ERR_NULL     # state needed for m = 2
    assert call(14, None) == ERR_NULL     # lengths
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(2, 0) == CSA2_OK          # empty batch: nothing to do
    args = list(base)
    args[3], args[1], args[15] = 1, None, None   # m = 1: gate and state not needed
    args[0] = None
    assert f(*args) == ERR_NULL                  # but the latent is


def _index_full(lib):
    f = lib.csa2_index_full
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, ctypes.c_size_t, P]
    lib.csa2_index_full_workspace.restype = ctypes.c_size_t
    lib.csa2_index_full_workspace.argtypes = [i32, i64, i32, i32, i32]
    return f


def test_index_full_validation(lib):
    f = _index_full(lib)
    ok = dict(ic=FAKE, isc=FAKE, cap=4096, len=FAKE, B=2, q=FAKE, w=FAKE, H=64, k=512, block=8, nb=2048,
              topk=FAKE, pool=FAKE, pl=FAKE, sc=None, ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ic"], a["isc"], a["cap"], a["len"], a["B"], a["q"], a["w"], a["H"], a["k"], a["block"],
                 a["nb"], a["topk"], a["pool"], a["pl"], a["sc"], a["ws"], a["wsb"], None)

    assert call(H=48) == ERR_UNSUP
    assert call(block=16) == ERR_UNSUP
    assert call(k=0) == ERR_SHAPE
    assert call(k=4096) == ERR_SHAPE
    assert call(nb=4096) == ERR_SHAPE
    assert call(cap=(1 << 20) + 1) == ERR_SHAPE
    assert call(q=None) == ERR_NULL
    assert call(pool=None) == ERR_NULL
    assert call(pool=None, pl=None, nb=0, ws=None) == ERR_WS
    assert call(ic=FAKE_ODD) == ERR_ALIGN
    need = lib.csa2_index_full_workspace(2, 4096, 512, 8, 2048)
    assert need >= 2 * 4096 * 4
    assert call(wsb=need - 1) == ERR_WS
    assert call(B=0) == CSA2_OK


def test_index_fp4q_validation(lib):
    """The FP4-query indexer calls validate like the bf16 ones, plus their two
    query planes (codes 16-byte aligned, scales any alignment)."""
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    f = lib.csa2_index_full_fp4q
    f.argtypes = [P, P, i64, P, i32, P, P, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    ok = dict(ic=FAKE, isc=FAKE, cap=4096, len=FAKE, B=2, qc=FAKE, qs=FAKE_ODD, w=FAKE, H=64, k=512, block=8,
              nb=2048, topk=FAKE, pool=FAKE, pl=FAKE, sc=None, ws=FAKE, wsb=1 << 40)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["ic"], a["isc"], a["cap"], a["len"], a["B"], a["qc"], a["qs"], a["w"], a["H"], a["k"],
                 a["block"], a["nb"], a["topk"], a["pool"], a["pl"], a["sc"], a["ws"], a["wsb"], None)

    assert call(H=48) == ERR_UNSUP
    assert call(block=16) == ERR_UNSUP
    assert call(k=0) == ERR_SHAPE
    assert call(qc=None) == ERR_NULL
    assert call(qs=None) == ERR_NULL
    assert call(qc=FAKE_ODD) == ERR_ALIGN
    assert call(ws=None) == ERR_WS
    assert call(B=0) == CSA2_OK
    g = lib.csa2_index_pool_fp4q
    g.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, P, i32, i32, P, P, P, sz, P]
    base = [FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 16384, FAKE, FAKE_ODD, FAKE, 64, 512, FAKE, None, FAKE,
            1 << 30, None]

    def callp(i, v):
        args = list(base)
        args[i] = v
        return g(*args)

    assert callp(7, 20000) == ERR_SHAPE   # pool_cap
    assert callp(11, 12) == ERR_UNSUP     # heads
    assert callp(8, None) == ERR_NULL     # q codes
    assert callp(9, None) == ERR_NULL     # q scales
    assert callp(8, FAKE_ODD) == ERR_ALIGN
    assert callp(16, 16) == ERR_WS
    assert callp(4, 0) == CSA2_OK


def test_index_pool_and_attention_validation(lib):
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f = lib.csa2_index_pool
    f.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, i32, i32, P, P, P, ctypes.c_size_t, P]
    assert f(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 20000, FAKE, FAKE, 64, 512, FAKE, None, FAKE, 1 << 30, None) == ERR_SHAPE
    assert f(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 16384, FAKE, FAKE, 12, 512, FAKE, None, FAKE, 1 << 30, None) == ERR_UNSUP
    assert f(FAKE, FAKE, 4096, FAKE, 2, None, FAKE, 16384, FAKE, FAKE, 64, 512, FAKE, None, FAKE, 1 << 30, None) == ERR_NULL
    assert f(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 16384, FAKE, FAKE, 64, 512, FAKE, None, FAKE, 16, None) == ERR_WS
    a = lib.csa2_sparse_attn_decode
    a.argtypes = [P, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32, P, i32, ctypes.c_float, P, P, P,
                  P, ctypes.c_size_t, P]
    base = [FAKE, 64, FAKE, FAKE, 4096, 0, FAKE, FAKE, 512, 16, FAKE, FAKE, 4096, 128, FAKE, 0, 0.04, None,
            FAKE, None, FAKE, 1 << 40, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return a(*args)

    assert call(1, 40) == ERR_UNSUP      # heads (multiple of 16 required)
    assert call(5, 3) == ERR_UNSUP       # scale format
    assert call(13, 129) == ERR_SHAPE    # window > 128
    assert call(12, 100) == ERR_SHAPE    # stride < window
    assert call(8, 5000) == ERR_SHAPE    # k
    assert call(16, float("nan")) == ERR_SHAPE
    assert call(15, 2) == ERR_UNSUP      # window format
    assert call(0, None) == ERR_NULL
    assert call(10, None) == ERR_NULL    # window planes missing
    assert call(21, 8) == ERR_WS
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(17, FAKE_ODD) == ERR_ALIGN  # query positions
    args = list(base)
    args[15], args[11] = 1, P(0x1004)     # FP8 window records: scale rows need 8-byte alignment
    assert a(*args) == ERR_ALIGN


def test_attention_mq_validation(lib):
    # Q queries per sequence: Q in 1..CSA2_MAX_QUERIES_PER_SEQ, the workspace
    # sized for B*Q query rows, and every check of the one-query call
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    a = lib.csa2_sparse_attn_decode_mq
    a.argtypes = [P, i32, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32, P, i32, ctypes.c_float, P, P, P,
                  P, ctypes.c_size_t, P]
    base = [FAKE, 64, 5, FAKE, FAKE, 4096, 0, FAKE, FAKE, 512, 16, FAKE, FAKE, 4096, 128, FAKE, 0, 0.04, None,
            FAKE, None, FAKE, 1 << 40, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return a(*args)

    assert call(2, 0) == ERR_SHAPE        # Q
    assert call(2, 17) == ERR_SHAPE       # Q beyond CSA2_MAX_QUERIES_PER_SEQ
    assert call(1, 40) == ERR_UNSUP
    assert call(14, 129) == ERR_SHAPE     # window > 128
    assert call(9, 5000) == ERR_SHAPE     # k
    assert call(0, None) == ERR_NULL
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(10, 0) == CSA2_OK         # empty batch
    # the workspace must hold B*Q = 80 query rows, not B = 16
    need = lib.csa2_attn_workspace(80, 64, 512, 128)
    assert lib.csa2_attn_workspace(16, 64, 512, 128) < need
    assert call(22, need - 1) == ERR_WS


def test_index_pool_mq_validation(lib):
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f = lib.csa2_index_pool_mq
    f.argtypes = [P, P, i64, P, i32, i32, P, P, i32, P, P, i32, i32, P, P, P, ctypes.c_size_t, P]
    base = [FAKE, FAKE, 4096, FAKE, 2, 5, FAKE, FAKE, 16384, FAKE, FAKE, 64, 512, FAKE, None, FAKE, 1 << 40, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return f(*args)

    assert call(5, 0) == ERR_SHAPE        # Q
    assert call(5, 17) == ERR_SHAPE
    assert call(8, 20000) == ERR_SHAPE    # pool capacity
    assert call(11, 12) == ERR_UNSUP      # indexer heads
    assert call(6, None) == ERR_NULL
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(4, 0) == CSA2_OK          # empty batch
    need = lib.csa2_index_pool_workspace(10, 16384, 512)
    assert call(16, need - 1) == ERR_WS   # the workspace holds B*Q = 10 rows
    g = lib.csa2_index_pool_mq_fp4q
    g.argtypes = [P, P, i64, P, i32, i32, P, P, i32, P, P, P, i32, i32, P, P, P, ctypes.c_size_t, P]
    base4 = base[:9] + [FAKE, FAKE] + base[10:]
    for i, v, want in [(5, 0, ERR_SHAPE), (5, 17, ERR_SHAPE), (9, None, ERR_NULL), (10, None, ERR_NULL),
                       (9, FAKE_ODD, ERR_ALIGN), (12, 12, ERR_UNSUP), (4, 0, CSA2_OK)]:
        args = list(base4)
        args[i] = v
        assert g(*args) == want, (i, v)
    args = list(base4)
    args[17] = need - 1
    assert g(*args) == ERR_WS


def test_attention_noalloc_validation(lib):
    # the no-alloc attention call validates like the workspace call, and
    # refuses a problem larger than its fixed per-GPU scratch before touching
    # any device (all of these fail before the scratch address is taken)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    a = lib.csa2_sparse_attn_decode_noalloc
    a.argtypes = [P, i32, P, P, i64, i32, P, P, i32, i32, P, P, i64, i32, P, i32, ctypes.c_float, P, P, P, P]
    base = [FAKE, 64, FAKE, FAKE, 4096, 0, FAKE, FAKE, 512, 16, FAKE, FAKE, 4096, 128, FAKE, 0, 0.04, None,
            FAKE, None, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return a(*args)

    assert lib.csa2_status_string(ERR_SCRATCH) == b"problem larger than the library's fixed attention scratch"
    assert call(1, 40) == ERR_UNSUP
    assert call(13, 129) == ERR_SHAPE
    assert call(0, None) == ERR_NULL
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(9, 0) == CSA2_OK                     # empty batch: nothing to do
    # 256 sequences x 64 heads x 17 chunks of partials exceed 32 MiB
    args = list(base)
    args[8], args[9] = 2048, 256
    assert a(*args) == ERR_SCRATCH
    assert lib.csa2_attn_workspace(256, 64, 2048, 128) > (32 << 20)


def test_index_phase_validation(lib):
    # the score / select halves of the indexer calls validate like the fused calls
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    fs = lib.csa2_index_full_score
    fs.argtypes = [P, P, i64, P, i32, P, P, i32, i32, P, P, sz, P]
    fsel = lib.csa2_index_full_select
    fsel.argtypes = [i64, P, i32, i32, i32, i32, P, P, P, P, P, sz, P]
    ps = lib.csa2_index_pool_score
    ps.argtypes = [P, P, i64, P, i32, P, P, i32, P, P, i32, P, P, sz, P]
    psel = lib.csa2_index_pool_select
    psel.argtypes = [i32, P, P, i32, i32, P, P, P, sz, P]
    big = 1 << 40
    assert fs(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 12, 8, None, FAKE, big, None) == ERR_UNSUP   # heads
    assert fs(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 64, 4, None, FAKE, big, None) == ERR_UNSUP   # block
    assert fs(FAKE, FAKE, (1 << 20) + 1, FAKE, 2, FAKE, FAKE, 64, 8, None, FAKE, big, None) == ERR_SHAPE
    assert fs(None, FAKE, 4096, FAKE, 2, FAKE, FAKE, 64, 8, None, FAKE, big, None) == ERR_NULL
    assert fs(FAKE_ODD, FAKE, 4096, FAKE, 2, FAKE, FAKE, 64, 8, None, FAKE, big, None) == ERR_ALIGN
    assert fs(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 64, 8, None, FAKE, 64, None) == ERR_WS
    assert fs(FAKE, FAKE, 4096, FAKE, 0, FAKE, FAKE, 64, 8, None, None, 0, None) == CSA2_OK      # empty batch
    assert fsel(4096, FAKE, 2, 0, 8, 2048, FAKE, FAKE, FAKE, None, FAKE, big, None) == ERR_SHAPE  # k
    assert fsel(4096, FAKE, 2, 512, 8, 4096, FAKE, FAKE, FAKE, None, FAKE, big, None) == ERR_SHAPE  # n_blocks
    assert fsel(4096, FAKE, 2, 512, 8, 2048, FAKE, None, FAKE, None, FAKE, big, None) == ERR_NULL  # pool
    assert fsel(4096, FAKE, 2, 512, 8, 2048, FAKE, FAKE, FAKE, None, FAKE, 64, None) == ERR_WS
    assert ps(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 20000, FAKE, FAKE, 64, None, FAKE, big, None) == ERR_SHAPE
    assert ps(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 16384, FAKE, FAKE, 12, None, FAKE, big, None) == ERR_UNSUP
    assert ps(FAKE, FAKE, 4096, FAKE, 2, None, FAKE, 16384, FAKE, FAKE, 64, None, FAKE, big, None) == ERR_NULL
    assert ps(FAKE, FAKE, 4096, FAKE, 2, FAKE, FAKE, 16384, FAKE, FAKE, 64, None, FAKE, 16, None) == ERR_WS
    assert psel(2, FAKE, FAKE, 16384, 4096, FAKE, None, FAKE, big, None) == ERR_SHAPE             # k
    assert psel(2, FAKE, None, 16384, 512, FAKE, None, FAKE, big, None) == ERR_NULL
    assert psel(2, FAKE, FAKE, 16384, 512, FAKE, None, FAKE, 16, None) == ERR_WS


def test_window_write_validation(lib):
    i32 = ctypes.c_int32
    f = lib.csa2_window_write
    f.argtypes = [P, i32, i32, P, ctypes.c_float, i32, P, i32, P, P, P, P]
    base = [FAKE, 4, 1, None, 1e-6, 1, FAKE, 128, FAKE, FAKE, FAKE, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return f(*args)

    assert call(7, 129) == ERR_SHAPE      # more than 128 slots
    assert call(7, 0) == ERR_SHAPE
    assert call(2, -1) == ERR_SHAPE       # tokens
    assert call(4, -1.0) == ERR_SHAPE     # eps
    assert call(1, 0) == CSA2_OK          # nothing to write
    assert call(2, 0) == CSA2_OK
    assert call(6, None) == ERR_NULL      # positions
    assert call(10, None) == ERR_NULL     # swa_len
    assert call(0, FAKE_ODD) == ERR_ALIGN
    assert call(9, P(0x1004)) == ERR_ALIGN  # scale rows: 8-byte aligned
    assert call(6, P(0x1004)) == ERR_ALIGN  # int64 positions


def test_index_full_mq_validation(lib):
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f = lib.csa2_index_full_mq
    f.argtypes = [P, P, i64, P, i32, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, ctypes.c_size_t, P]
    lib.csa2_index_full_mq_workspace.restype = ctypes.c_size_t
    lib.csa2_index_full_mq_workspace.argtypes = [i32, i32, i64, i32, i32, i32]
    lib.csa2_index_full_workspace.restype = ctypes.c_size_t
    lib.csa2_index_full_workspace.argtypes = [i32, i64, i32, i32, i32]
    # the workspace is that of B*Q single-query rows
    assert lib.csa2_index_full_mq_workspace(16, 5, 131072, 512, 8, 2048) == \
        lib.csa2_index_full_workspace(80, 131072, 512, 8, 2048)
    assert lib.csa2_index_full_mq_workspace(16, 17, 131072, 512, 8, 2048) == 0
    base = [FAKE, FAKE, 4096, FAKE, 4, 5, FAKE, FAKE, 64, 512, 8, 64, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None]

    def call(i, v):
        args = list(base)
        args[i] = v
        return f(*args)

    assert call(5, 0) == ERR_SHAPE        # queries per sequence
    assert call(5, 17) == ERR_SHAPE
    assert call(9, 0) == ERR_SHAPE        # k
    assert call(8, 12) == ERR_UNSUP       # heads
    assert call(10, 16) == ERR_UNSUP      # block
    assert call(4, 0) == CSA2_OK          # no sequences
    assert call(6, None) == ERR_NULL
    assert call(6, FAKE_ODD) == ERR_ALIGN
    assert call(17, 64) == ERR_WS


def test_paged_validation(lib):
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    f = lib.csa2_index_full_paged
    f.argtypes = [P, P, i64, P, i32, i32, P, i32, P, P, i32, i32, i32, i32, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    # pool of 64 pages of 2^8 entries, 16 pages per sequence
    base = [FAKE, FAKE, 64 << 8, FAKE, 8, 16, FAKE, 4, FAKE, FAKE, 64, 512, 8, 64, FAKE, FAKE, FAKE, FAKE, FAKE,
            None, FAKE, 1 << 40, None]

    def call(i, v, fn=f, b=base):
        args = list(b)
        args[i] = v
        return fn(*args)

    assert call(4, 5) == ERR_SHAPE            # pages of fewer than 64 entries
    assert call(4, 21) == ERR_SHAPE
    assert call(2, (64 << 8) + 3) == ERR_SHAPE  # pool not whole pages
    assert call(2, 1 << 27) == ERR_SHAPE        # pool beyond 32-bit byte offsets
    assert call(5, 5000) == ERR_SHAPE           # logical capacity above the limit
    assert call(3, None) == ERR_NULL            # block table
    assert call(15, None) == ERR_NULL           # topk rows
    assert call(17, None) == ERR_NULL           # pool rows with a pool
    assert call(3, FAKE_ODD) == ERR_ALIGN
    assert call(21, 64) == ERR_WS
    assert call(7, 0) == CSA2_OK
    a = lib.csa2_cache_append_paged
    a.argtypes = [P, P, i32, i32, P, ctypes.c_float, P, i32, i32, P, P, P, P, i64, P, i32, i32, P, P, P]
    ab = [FAKE, None, 4, 1, None, 1e-6, FAKE, 0, 1, FAKE, FAKE, FAKE, FAKE, 64 << 8, FAKE, 8, 16, FAKE, None, None]
    assert call(15, 3, a, ab) == ERR_SHAPE
    assert call(14, None, a, ab) == ERR_NULL
    assert call(3, 2, a, ab) == ERR_NULL        # m = 2 needs gate and state
    assert call(2, 0, a, ab) == CSA2_OK
    r = lib.csa2_index_pool_rows
    r.argtypes = [P, P, i64, i32, P, P, P, i32, P, P, i32, i32, P, P, P, P, ctypes.c_size_t, P]
    rb = [FAKE, FAKE, 1 << 16, 4, FAKE, FAKE, FAKE, 16384, FAKE, FAKE, 64, 512, FAKE, FAKE, None, FAKE, 1 << 40, None]
    assert call(5, None, r, rb) == ERR_NULL     # pool rows
    assert call(13, None, r, rb) == ERR_NULL    # topk rows
    assert call(7, 20000, r, rb) == ERR_SHAPE
    assert call(2, 0, r, rb) == ERR_SHAPE
    t = lib.csa2_sparse_attn_decode_rows
    t.argtypes = [P, i32, P, P, i64, i32, P, i32, i32, P, P, i64, i32, P, i32, ctypes.c_float, P, P, P, P,
                  ctypes.c_size_t, P]
    tb = [FAKE, 64, FAKE, FAKE, 1 << 16, 0, FAKE, 512, 16, FAKE, FAKE, 128, 128, FAKE, 1, 0.04, None, FAKE, None,
          FAKE, 1 << 40, None]
    assert call(6, None, t, tb) == ERR_NULL     # rows
    assert call(4, 1 << 27, t, tb) == ERR_SHAPE
    assert call(14, 3, t, tb) == ERR_UNSUP
    assert call(10, P(0x1004), t, tb) == ERR_ALIGN  # FP8 window scales
    assert call(20, 16, t, tb) == ERR_WS
