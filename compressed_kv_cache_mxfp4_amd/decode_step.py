"""One CSA2 decoder step over a shared FP4 global KV cache.

The layer schedule follows the pages: the first decoder layer is a Full layer
(scores every visible entry, picks its top-512 and builds the candidate pool),
each later index-producing layer is a Reindex layer (rescores only the pool
with its own indexer query), and every index-producing layer is followed by
Reuse layers that attend with the last top-512 [jokeuncle.pages.dev,
"两张架构图里藏着 890 字节", section 二 (schedule); ggaaooppeenngg.github.io,
"DeepSeek-V4.1-Flash 架构解析", section 3.3 (1 full scoring + 4 pool rescorings
+ 15 inheritances per step); syt-nju.github.io, Figure 4 (modes)].  Every
layer's attention reads the same main KV with its own query and window.

This module only sequences C-ABI calls on the current stream; all arithmetic
is in the HIP kernels.  Buffers are allocated once in `DecodeStep.__init__`
so that `run()` allocates nothing.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib as K


class DecodeStep:
    def __init__(self, cache: dict, lengths: torch.Tensor, *, k: int = 512, n_blocks: int = 2048,
                 n_reindex: int = 4, reuse_per_index: int = 3, main_fmt: int = K.E8M0,
                 swa_cap: int = 128, swa: Optional[dict] = None, H_attn: int = 64,
                 sm_scale: Optional[float] = None):
        self.cache = cache
        self.lengths = lengths
        dev = lengths.device
        B, cap = cache["idx_codes"].shape[:2]
        self.B, self.cap = B, cap
        self.k, self.n_blocks = k, n_blocks
        self.n_reindex, self.reuse = n_reindex, reuse_per_index
        self.main_fmt = main_fmt
        self.H_attn = H_attn
        self.sm_scale = sm_scale if sm_scale is not None else 1.0 / (512 ** 0.5)
        # window: by default the last swa_cap entries of each sequence's main
        # cache; or one dict for every layer, or a list with one per attention
        # layer (each layer's own window, e.g. an FP8 ring: fmt=SWA_FP8)
        if swa is None:
            # the tail view is each sequence's last swa_cap entries only when
            # every sequence is full (one host read of the lengths, here and
            # never in run())
            if not bool((lengths == cap).all()):
                raise ValueError("the default window is the last swa_cap entries of a full cache: with lengths "
                                 "below the capacity pass each sequence's window as `swa`")
            swa = dict(codes=cache["main_codes"], scales=cache["main_scales"], row0=cap - swa_cap,
                       stride=cap, length=torch.full((B,), swa_cap, dtype=torch.int32, device=dev))
        self.swa = swa
        self.swa_cap = swa_cap
        n_idx = 1 + n_reindex
        self.topk = [torch.empty(B, k, dtype=torch.int32, device=dev) for _ in range(n_idx)]
        self.pool = torch.empty(B, max(n_blocks * 8, 1), dtype=torch.int32, device=dev)
        self.pool_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.n_attn = n_idx * (1 + reuse_per_index)
        self.out = [torch.empty(B, H_attn, 512, dtype=torch.int16, device=dev) for _ in range(self.n_attn)]
        # workspaces sized once (shared by the calls of a step, which are stream-ordered)
        L = K.lib()
        self.ws_full = torch.empty(max(L.csa2_index_full_workspace(B, cap, k, 8, n_blocks), 256),
                                   dtype=torch.uint8, device=dev)
        self.ws_pool = torch.empty(max(L.csa2_index_pool_workspace(B, max(n_blocks * 8, 1), k), 256),
                                   dtype=torch.uint8, device=dev)
        # zero-filled once: the attention calls keep their completion counters at zero
        self.ws_attn = torch.zeros(max(L.csa2_attn_workspace(B, H_attn, k, swa_cap), 256),
                                   dtype=torch.uint8, device=dev)

    def schedule(self) -> List[Tuple[str, int]]:
        """(mode, index-layer id) for each attention layer, in order."""
        s = []
        for i in range(1 + self.n_reindex):
            s.append(("full" if i == 0 else "reindex", i))
            s.extend(("reuse", i) for _ in range(self.reuse))
        return s

    def run_index(self, idx_qw: Sequence[Tuple[torch.Tensor, torch.Tensor]]):
        c = self.cache
        q, w = idx_qw[0]
        K.index_full(c["idx_codes"], c["idx_scales"], self.lengths, q, w, k=self.k,
                     n_blocks=self.n_blocks,
                     out=dict(topk=self.topk[0], pool=self.pool, pool_len=self.pool_len),
                     _ws=self.ws_full)
        for i in range(1, 1 + self.n_reindex):
            q, w = idx_qw[i]
            K.index_pool(c["idx_codes"], c["idx_scales"], self.lengths, self.pool, self.pool_len, q,
                         w, k=self.k, out=dict(topk=self.topk[i]), _ws=self.ws_pool)

    def run_attention(self, attn_q: Sequence[torch.Tensor]):
        c = self.cache
        for j, (mode, i) in enumerate(self.schedule()):
            s = self.swa[j] if isinstance(self.swa, (list, tuple)) else self.swa
            K.sparse_attn_decode(attn_q[j], c["main_codes"], c["main_scales"], self.lengths,
                                 self.topk[i], self.main_fmt, swa_codes=s["codes"],
                                 swa_scales=s["scales"], swa_len=s["length"],
                                 swa_stride=s["stride"], swa_cap=self.swa_cap, swa_row0=s["row0"],
                                 swa_fmt=s.get("fmt", K.SWA_MAIN), sm_scale=self.sm_scale,
                                 out=dict(out=self.out[j]), _ws=self.ws_attn)

    def run(self, idx_qw, attn_q):
        self.run_index(idx_qw)
        self.run_attention(attn_q)
        return self

    def capture(self, idx_qw, attn_q) -> "torch.cuda.CUDAGraph":
        """Record one step into a HIP graph (torch.cuda.CUDAGraph); `graph.replay()`
        then launches the same kernels on the same buffers with one host call.

        The inputs (queries, weights, cache, lengths) are read at replay time
        from the addresses recorded here, so refill them in place.  The step
        records no memset and allocates nothing (buffers come from __init__),
        and the attention completion counters are left at zero by every call,
        so replays are independent.  The first eager call of each kernel sets
        its launch attributes, so run() once before capturing.
        """
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.run(idx_qw, attn_q)
        return graph
