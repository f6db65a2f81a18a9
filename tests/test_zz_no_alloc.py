"""The attention entry point that allocates nothing
(csa2_sparse_attn_decode_noalloc) against the workspace entry point
(csa2_sparse_attn_decode): the same kernels on the same inputs, so outputs and
log-sum-exps must be bit-identical.  Two calls in a row, the second with a
smaller problem (the library's scratch keeps the first call's contents), for
both attention kernels and both main-KV scale formats, then a problem larger
than the scratch, which must be refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import compressed_kv_cache_mxfp4_amd as K
import csa2_synth as syn
from gpu_common import DEV, build_gpu_cache, say

pytestmark = pytest.mark.gpu


def _case(B, cap, k, W, fmt, seed):
    wl = syn.small("na", seed, B=B, cap=cap, H_idx=8, k=k, n_blocks=0)
    cache = build_gpu_cache(wl, fmt)
    g = np.random.default_rng(seed)
    topk = np.stack([g.choice(cap, k, replace=False) for _ in range(B)]).astype(np.int32)
    topk[0, : min(5, k)] = -1
    lens = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    q = syn.as_bf16_bits(torch.randn(B, 64, 512, generator=torch.Generator().manual_seed(seed))).to(DEV)
    win = dict(swa_codes=cache["main_codes"], swa_scales=cache["main_scales"],
               swa_len=torch.tensor([W - (b % 3) for b in range(B)], dtype=torch.int32, device=DEV),
               swa_stride=cap, swa_cap=W, swa_row0=cap - W)
    return cache, lens, torch.from_numpy(topk).to(DEV), q, win


@pytest.mark.parametrize("fmt", [0, 1])
def test_noalloc_attention_equals_workspace_call(fmt):
    # (B, cap, k, W): the all-heads kernel (48 sequences), then the split kernel
    # on a smaller problem; then the split kernel once more, smaller still
    for B, cap, k, W in [(48, 2048, 512, 128), (16, 4096, 512, 128), (3, 1000, 200, 40)]:
        say(f"noalloc attention fmt={fmt} B={B} cap={cap} k={k} W={W}")
        cache, lens, topk, q, win = _case(B, cap, k, W, fmt, 7 + B + fmt)
        ref, ref_lse = K.sparse_attn_decode(q, cache["main_codes"], cache["main_scales"], lens, topk, fmt,
                                            return_lse=True, **win)
        out = torch.full((B, 64, 512), 0x7FC0, dtype=torch.int16, device=DEV)
        lse = torch.full((B, 64), float("nan"), dtype=torch.float32, device=DEV)
        K.sparse_attn_decode_noalloc(q, cache["main_codes"], cache["main_scales"], lens, topk, fmt, out, lse,
                                     **win)
        torch.cuda.synchronize()
        assert torch.equal(out.cpu(), ref.cpu()), "outputs differ from the workspace call"
        assert torch.equal(lse.cpu().view(torch.int32), ref_lse.cpu().view(torch.int32)), "lse differs"
        del cache


def test_noalloc_attention_refuses_a_problem_beyond_its_scratch():
    # 256 sequences x 64 heads x 2048 + 128 rows needs far more than 32 MiB of
    # partials: refused by the host check, nothing launched, outputs untouched
    B, cap, k = 256, 64, 2048
    L = K.lib()
    assert L.csa2_attn_workspace(B, 64, k, 64) > 32 << 20
    q = torch.zeros(B, 64, 512, dtype=torch.int16, device=DEV)
    mc = torch.zeros(B, cap, 256, dtype=torch.uint8, device=DEV)
    ms = torch.zeros(B, cap, 32, dtype=torch.uint8, device=DEV)
    lens = torch.full((B,), cap, dtype=torch.int32, device=DEV)
    topk = torch.zeros(B, k, dtype=torch.int32, device=DEV)
    out = torch.full((B, 64, 512), 5, dtype=torch.int16, device=DEV)
    with pytest.raises(K.Csa2Error, match="scratch"):
        K.sparse_attn_decode_noalloc(q, mc, ms, lens, topk, 0, out, swa_codes=mc, swa_scales=ms,
                                     swa_len=lens, swa_stride=cap, swa_cap=64)
    torch.cuda.synchronize()
    assert bool((out == 5).all())
