"""Seeded synthetic inputs for the CSA2 decode workloads.

This module is shared by the HIP path's tests/benchmark and by the CPU oracle's
tests.  It holds none of the method's arithmetic: it only draws random numbers
(with torch generators, on the device the caller asks for) and arranges them
into the shapes and structures of the workloads.  Quantisation, scoring,
selection and attention are done by the consumers.

Workloads (the decode step over a compressed FP4 cache, at the context sizes
the pages discuss: 128K to 1M tokens):

  tiny    B=1,  M=4096,   indexer H=8,  top-512, 64 blocks (512-position pool)
  full128 B=16, M=131072, H=64, top-512, 2048 blocks; 64 rows per query get 4x K
  step128 full128 shapes, 1 Full + 4 Reindex + 15 Reuse layers (20 attention calls)
  write1m cache write of 8192 tokens (m=2) + decode B=4 over M=524288 entries
  stress  B=64, M=262144, full decoder step; 5% of blocks 3x K, exact duplicates

Every tensor is derived from (workload seed, stream name, index) through its
own torch.Generator, so any piece can be regenerated alone and identically.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import torch

MAIN_DIM = 512
IDX_DIM = 128


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    cap: int              # compressed entries per sequence (all visible)
    H_idx: int            # indexer heads
    k: int                # index top-k
    block: int
    n_blocks: int         # candidate blocks (0 = no pool)
    H_attn: int = 64
    swa: int = 128
    n_reindex: int = 0    # Reindex layers after the Full layer
    reuse_per_index: int = 0  # Reuse layers after each index-producing layer
    boost_rows: int = 0   # rows per query whose indexer K is scaled by boost_factor
    boost_factor: float = 1.0
    cluster_frac: float = 0.0   # fraction of blocks scaled by cluster_factor
    cluster_factor: float = 1.0
    write_tokens: int = 0  # cache-write tokens (0 = no write stage)
    write_m: int = 1

    @property
    def n_attn_calls(self) -> int:
        return (1 + self.n_reindex) * (1 + self.reuse_per_index)

    @property
    def pool_cap(self) -> int:
        return self.n_blocks * self.block


WORKLOADS = {
    "tiny": Workload("tiny", 0, B=1, cap=4096, H_idx=8, k=512, block=8, n_blocks=64),
    "full128": Workload("full128", 1, B=16, cap=131072, H_idx=64, k=512, block=8,
                        n_blocks=2048, boost_rows=64, boost_factor=4.0),
    "step128": Workload("step128", 2, B=16, cap=131072, H_idx=64, k=512, block=8,
                        n_blocks=2048, n_reindex=4, reuse_per_index=3, boost_rows=64,
                        boost_factor=4.0),
    "write1m": Workload("write1m", 3, B=4, cap=524288, H_idx=64, k=512, block=8,
                        n_blocks=2048, write_tokens=8192, write_m=2),
    "stress": Workload("stress", 4, B=64, cap=262144, H_idx=64, k=512, block=8,
                       n_blocks=2048, n_reindex=4, reuse_per_index=3, cluster_frac=0.05,
                       cluster_factor=3.0),
    # one encoder source layer at 128K tokens: m = 2 entries, Full scoring with
    # its own top-512 and no candidate pool, then its attention
    "enc128": Workload("enc128", 5, B=16, cap=65536, H_idx=64, k=512, block=8, n_blocks=0),
}


def derive_seed(seed: int, stream: str, index: int = 0) -> int:
    h = hashlib.sha256(f"csa2/{seed}/{stream}/{index}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, stream: str, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(derive_seed(seed, stream, index))
    return g


def normal(shape, seed: int, stream: str, index: int = 0, device="cpu", std: float = 1.0):
    g = _gen(seed, stream, index, device)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return x * std if std != 1.0 else x


def uniform(shape, seed: int, stream: str, index: int = 0, device="cpu"):
    g = _gen(seed, stream, index, device)
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)


def randperm(n: int, seed: int, stream: str, index: int = 0) -> torch.Tensor:
    g = _gen(seed, stream, index, "cpu")
    return torch.randperm(n, generator=g)


def as_bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """Round fp32 to bf16 (nearest-even, torch's conversion) and return the bits as int16."""
    return x.to(torch.bfloat16).view(torch.int16)


# ------------------------------------------------------------------ the cache
def main_values(wl: Workload, b: int, device="cpu", rows: Optional[int] = None):
    """Pre-quantisation main-KV latents of sequence b: fp32 [cap][512], N(0,1)."""
    return normal((rows or wl.cap, MAIN_DIM), wl.seed, "main", b, device)


def boost_positions(wl: Workload, b: int) -> torch.Tensor:
    """Rows of sequence b whose indexer K is scaled (distinct, ascending)."""
    if wl.boost_rows == 0:
        return torch.zeros(0, dtype=torch.int64)
    return torch.sort(randperm(wl.cap, wl.seed, "boost", b)[: wl.boost_rows]).values


def cluster_blocks(wl: Workload, b: int) -> torch.Tensor:
    """Blocks of sequence b that carry clustered high-score positions (ascending)."""
    nb = wl.cap // wl.block
    n = int(round(wl.cluster_frac * nb))
    if n == 0:
        return torch.zeros(0, dtype=torch.int64)
    return torch.sort(randperm(nb, wl.seed, "cluster", b)[:n]).values


def idx_values(wl: Workload, b: int, device="cpu", rows: Optional[int] = None):
    """Pre-quantisation indexer keys of sequence b: fp32 [cap][128], N(0,1),
    with the workload's structure applied:
      boost:   boost_rows random rows scaled by boost_factor;
      cluster: cluster_frac of the blocks scaled by cluster_factor; in every
               16th chosen block (i % 16 == 7) rows 1..7 copy row 0, and in
               every 32nd chosen block (i % 32 == 31) all 8 rows copy the
               previous chosen block, so exact score ties occur.
    """
    n = rows or wl.cap
    x = normal((n, IDX_DIM), wl.seed, "idx", b, device)
    if wl.boost_rows:
        pos = boost_positions(wl, b).to(device)
        pos = pos[pos < n]
        x[pos] *= wl.boost_factor
    if wl.cluster_frac > 0:
        blocks = cluster_blocks(wl, b).tolist()
        blk = wl.block
        xb = x[: (n // blk) * blk].view(-1, blk, IDX_DIM)
        for i, bl in enumerate(blocks):
            if bl >= xb.shape[0]:
                continue
            xb[bl] *= wl.cluster_factor
            if i % 32 == 31 and blocks[i - 1] < xb.shape[0]:
                xb[bl] = xb[blocks[i - 1]]
            elif i % 16 == 7:
                xb[bl, 1:] = xb[bl, 0]
    return x


# ------------------------------------------------------------ query-side data
def index_query(wl: Workload, layer: int, device="cpu"):
    """Indexer query of an index-producing layer: bf16 bits [B][H][128], N(0,1)."""
    q = normal((wl.B, wl.H_idx, IDX_DIM), wl.seed, "idx_q", layer, device)
    return as_bf16_bits(q)


def index_weights(wl: Workload, layer: int, device="cpu"):
    """Per-head weights of an index-producing layer: fp32 [B][H], U(0,1)."""
    return uniform((wl.B, wl.H_idx), wl.seed, "idx_w", layer, device)


def attn_query(wl: Workload, layer: int, device="cpu"):
    """Main query of an attention layer: bf16 bits [B][H_attn][512], N(0,1)."""
    q = normal((wl.B, wl.H_attn, MAIN_DIM), wl.seed, "attn_q", layer, device)
    return as_bf16_bits(q)


# --------------------------------------------------------------- cache write
def write_inputs(wl: Workload, device="cpu", tokens: Optional[int] = None):
    """Cache-write inputs: latent, gate bf16 bits [T][512] N(0,1) and the
    indexer projection fp32 [512][128] N(0, 1/512)."""
    T = tokens or wl.write_tokens
    latent = as_bf16_bits(normal((T, MAIN_DIM), wl.seed, "latent", 0, device))
    gate = as_bf16_bits(normal((T, MAIN_DIM), wl.seed, "gate", 0, device))
    w = normal((MAIN_DIM, IDX_DIM), wl.seed, "wproj", 0, device, std=(1.0 / MAIN_DIM) ** 0.5)
    return latent, gate, w


def small(name: str, seed: int, B: int, cap: int, H_idx: int, k: int, n_blocks: int, **kw):
    """A workload of arbitrary (small) shape for parity tests."""
    return Workload(name, seed, B=B, cap=cap, H_idx=H_idx, k=k, block=8, n_blocks=n_blocks, **kw)
