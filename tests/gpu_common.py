"""Helpers shared by the GPU parity tests.

Inputs come from csa2_synth (seeded, shared with the oracle); the GPU caches
are quantised by the HIP quantiser and the oracle's caches by the oracle's
quantiser from the same fp32 values, and the two are asserted bit-identical
before anything else is compared.  Nothing here feeds a HIP result into the
oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import csa2_synth as syn
import compressed_kv_cache_mxfp4_amd as K
import oracle

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def build_gpu_cache(wl: syn.Workload, main_fmt: int, rows: int | None = None, device=DEV):
    """Quantise the workload's synthetic cache on the GPU."""
    cap = rows or wl.cap
    B = wl.B
    c = dict(
        main_codes=torch.empty(B, cap, 256, dtype=torch.uint8, device=device),
        main_scales=torch.empty(B, cap, 32, dtype=torch.uint8, device=device),
        idx_codes=torch.empty(B, cap, 64, dtype=torch.uint8, device=device),
        idx_scales=torch.empty(B, cap, 4, dtype=torch.uint8, device=device),
    )
    for b in range(B):
        xm = syn.main_values(wl, b, device, rows=cap)
        K.quantize_fp4(xm, 16, main_fmt, c["main_codes"][b], c["main_scales"][b])
        xi = syn.idx_values(wl, b, device, rows=cap)
        K.quantize_fp4(xi, 32, K.E8M0, c["idx_codes"][b], c["idx_scales"][b])
        del xm, xi
    return c


def oracle_cache_seq(wl: syn.Workload, b: int, main_fmt: int, gpu_cache, rows: int | None = None,
                     need_main: bool = True):
    """The oracle's own cache of sequence b (from the generator's fp32 values
    on the same device, downloaded), checked bit-identical to the GPU's."""
    cap = rows or wl.cap
    xi = syn.idx_values(wl, b, DEV, rows=cap).cpu().numpy()
    ic, isc = oracle.quantize(xi, 32, oracle.E8M0)
    assert np.array_equal(ic, gpu_cache["idx_codes"][b].cpu().numpy()), "indexer-K codes differ"
    assert np.array_equal(isc, gpu_cache["idx_scales"][b].cpu().numpy()), "indexer-K scales differ"
    out = dict(idx_codes=ic, idx_scales=isc)
    if need_main:
        xm = syn.main_values(wl, b, DEV, rows=cap).cpu().numpy()
        mc, ms = oracle.quantize(xm, 16, main_fmt)
        assert np.array_equal(mc, gpu_cache["main_codes"][b].cpu().numpy()), "main codes differ"
        assert np.array_equal(ms, gpu_cache["main_scales"][b].cpu().numpy()), "main scales differ"
        out.update(main_codes=mc, main_scales=ms)
    return out


def oracle_main_rows(wl: syn.Workload, b: int, main_fmt: int, gpu_cache, rows, cap: int | None = None):
    """The oracle's quantisation of main-KV rows `rows` of sequence b (from the
    generator's fp32 values), checked bit-identical to the same rows of the
    GPU cache.  Quantisation is row by row, so a subset of rows is exactly the
    corresponding subset of the whole cache's bytes."""
    rows = np.asarray(rows, np.int64)
    gi = torch.from_numpy(rows).to(DEV)
    x = syn.main_values(wl, b, DEV, rows=cap or wl.cap)
    xs = x[gi].cpu().numpy()
    del x
    mc, ms = oracle.quantize(xs, 16, main_fmt)
    assert np.array_equal(mc, gpu_cache["main_codes"][b][gi].cpu().numpy()), "main codes differ"
    assert np.array_equal(ms, gpu_cache["main_scales"][b][gi].cpu().numpy()), "main scales differ"
    return mc, ms


def remap_positions(sel, rows):
    """Positions of `sel` as indices into the sorted row list `rows` (-1 stays
    -1; a position not in `rows` is an error)."""
    lut = {int(r): i for i, r in enumerate(rows)}
    return np.array([lut[int(p)] if p >= 0 else -1 for p in sel], np.int32)


# ---------------------------------------------------------------- tolerances
def score_close(gpu, ref):
    """Scores agree within 1e-5 relative, with a floor of 1e-7 x the largest."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    ok = ~np.isnan(r)
    assert np.array_equal(np.isnan(g), np.isnan(r)), "masked entries differ"
    if not ok.any():
        return
    floor = 1e-7 * np.abs(r[ok]).max()
    err = np.abs(g[ok] - r[ok])
    tol = 1e-5 * np.abs(r[ok]) + floor
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} scores off; worst rel {np.max(err / np.maximum(np.abs(r[ok]), floor)):.3g}"


def score_tol(x, ref_max):
    return 1e-5 * abs(float(x)) + 1e-7 * float(ref_max)


def brute_topk(scores, k, ids=None):
    """(score desc, id asc) top-k by numpy.lexsort; ascending ids, -1 padded."""
    s = np.asarray(scores, np.float64)
    ids = np.arange(len(s)) if ids is None else np.asarray(ids, np.int64)
    ok = ~np.isnan(s)
    s, ids = s[ok], ids[ok]
    s = np.where(s == 0, 0.0, s)
    order = np.lexsort((ids, -s))
    pick = np.sort(ids[order[:k]])
    return np.concatenate([pick, -np.ones(k - len(pick), np.int64)])


def brute_pool(scores, n_blocks, block=8):
    s = np.asarray(scores, np.float64)
    L = len(s)
    nb = (L + block - 1) // block
    pad = np.full(nb * block, -np.inf)
    pad[:L] = s
    bs = pad.reshape(nb, block).max(1)
    blocks = brute_topk(bs, n_blocks)
    blocks = blocks[blocks >= 0]
    pos = [np.arange(b * block, min(b * block + block, L)) for b in blocks]
    pool = np.concatenate(pos) if pos else np.zeros(0, np.int64)
    out = -np.ones(n_blocks * block, np.int64)
    out[: len(pool)] = pool
    return out, len(pool), bs


def certify_topk(gpu_sel, ref_sel, ref_scores, k):
    """Every index in the symmetric difference must be a near-tie of the
    oracle's k-th score (within the score tolerance).  Returns the count."""
    g = set(int(x) for x in gpu_sel if x >= 0)
    r = set(int(x) for x in ref_sel if x >= 0)
    diff = g ^ r
    if not diff:
        return 0
    rs = np.asarray(ref_scores, np.float64)
    valid = rs[~np.isnan(rs)]
    kth = np.sort(valid)[::-1][min(k, len(valid)) - 1]
    mx = np.abs(valid).max()
    for p in diff:
        assert abs(rs[p] - kth) <= 2 * score_tol(kth, mx), f"index {p} differs and is not a near-tie"
    return len(diff)


def attn_close(out_gpu_bits, ref, tol=1e-2):
    """Per (sequence, head): max|o - r| / max|r| <= tol.  Returns the worst ratio."""
    o = torch.as_tensor(out_gpu_bits).view(torch.bfloat16).float().cpu().numpy()
    r = np.asarray(ref, np.float64)
    num = np.abs(o - r).max(-1)
    den = np.maximum(np.abs(r).max(-1), 1e-30)
    ratio = num / den
    assert (ratio <= tol).all(), f"attention off: worst {ratio.max():.3g}"
    return float(ratio.max())
