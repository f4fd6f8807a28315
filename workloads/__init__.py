"""Seeded synthetic workloads for the CSA2 layer step.

This module draws inputs and nothing else: random bf16 latent rows, indexer
rows, indexer queries, head weights, attention queries, sequence lengths and
page tables.  It contains none of the arithmetic the layer computes (no
quantisation, no scoring, no selection, no attention).  Both the fp64 oracle
and the GPU path consume exactly the arrays produced here.

Every array is drawn per (seed, purpose, sequence or layer) from its own
seeded ``torch.Generator``, so any piece can be regenerated on its own, on the
device it was first drawn on, without materialising the rest.  Host draws use
torch's CPU generator; device draws use torch's device generator.  The two
produce different streams, so a case must be drawn and checked on one device.

Shapes follow the five workloads the pages motivate (64K and 1M contexts,
Top-512; "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression",
Method: sparse attention trained at 64K and extended to 1M tokens).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch

D_LATENT = 512          # main-KV latent width (one row = 256 B codes + 16 B scales)
D_INDEX = 128           # indexer-K / indexer-Q width (E4M3 bytes)
KV_ROW_BYTES = 272
IDXK_ROW_BYTES = 128

FULL, REINDEX, REUSE = 0, 1, 2
MODE_NAMES = {FULL: "full", REINDEX: "reindex", REUSE: "reuse"}

# purpose tags for the per-piece generators
_TAG_KV, _TAG_IK, _TAG_QI, _TAG_W, _TAG_Q, _TAG_LEN, _TAG_PERM, _TAG_CTR = 1, 2, 3, 4, 5, 6, 7, 8
CLUSTER_BLOCK = 64      # entries per centre of a clustered indexer-K


def _seed_of(seed: int, tag: int, index: int) -> int:
    """A fixed 63-bit seed for one (seed, purpose, index) piece (splitmix64 mix)."""
    x = (seed * 0x9E3779B97F4A7C15 + tag * 0xBF58476D1CE4E5B9 + index * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    x ^= x >> 30
    x = (x * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
    x ^= x >> 27
    x = (x * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
    x ^= x >> 31
    return x & 0x7FFFFFFFFFFFFFFF


def _gen(seed: int, tag: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(seed, tag, index))
    return g


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """fp32 draws -> bf16 bit patterns (int16 storage; read as uint16)."""
    return x.to(torch.bfloat16).view(torch.int16)


@dataclasses.dataclass
class CaseSpec:
    """One workload: sequence lengths, layer group and value distributions."""
    name: str
    seed: int
    cached: List[int]               # cached entries per sequence before the step
    n_new: int                      # rows appended per sequence at the step (decode: 1; prefill: chunk)
    h_idx: int                      # indexer heads
    h: int                          # attention heads
    k: int = 512
    modes: Sequence[int] = (FULL,)
    integer_indexer: bool = False   # indexer K/Q integers in [-8, 8], w in {1, 2}
    page_size: int = 1024
    shuffle_pages: bool = False
    prefill: bool = False           # queries are the n_new appended rows (causal), else one query per sequence
    extra_pages: int = 0            # unused pages in the pool (exercise page ids beyond the used range)
    pool_k: int = 0                 # > 0: hierarchical indexer, the Full layer's Top-pool_k is the Reindex pool
    clustered: bool = False         # indexer-K rows near a per-64-entry-block centre (block structure to prune on)

    @property
    def num_seqs(self) -> int:
        return len(self.cached)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(D_LATENT)

    def seq_len_after(self, s: int) -> int:
        return self.cached[s] + self.n_new

    @property
    def nq(self) -> int:
        return self.n_new if self.prefill else self.num_seqs

    def q_seq(self) -> np.ndarray:
        if self.prefill:
            return np.zeros(self.n_new, dtype=np.int32)
        return np.arange(self.num_seqs, dtype=np.int32)

    def q_vis(self) -> np.ndarray:
        """Visible entries per query: decode sees everything after the append;
        prefill query i sees the cached context plus new rows 0..i."""
        if self.prefill:
            return (self.cached[0] + 1 + np.arange(self.n_new)).astype(np.int32)
        return np.array([self.seq_len_after(s) for s in range(self.num_seqs)], dtype=np.int32)

    def max_pages(self) -> int:
        return max((self.seq_len_after(s) + self.page_size - 1) // self.page_size for s in range(self.num_seqs))

    def total_pages(self) -> int:
        return sum((self.seq_len_after(s) + self.page_size - 1) // self.page_size
                   for s in range(self.num_seqs)) + self.extra_pages


def page_table(spec: CaseSpec) -> np.ndarray:
    """[num_seqs][max_pages] int32; unused slots are -1.  In-order unless shuffled."""
    npages = spec.total_pages()
    if spec.shuffle_pages:
        perm = torch.randperm(npages, generator=_gen(spec.seed, _TAG_PERM, 0, "cpu")).numpy().astype(np.int32)
    else:
        perm = np.arange(npages, dtype=np.int32)
    mp = spec.max_pages()
    pt = np.full((spec.num_seqs, mp), -1, dtype=np.int32)
    nxt = 0
    for s in range(spec.num_seqs):
        n = (spec.seq_len_after(s) + spec.page_size - 1) // spec.page_size
        pt[s, :n] = perm[nxt:nxt + n]
        nxt += n
    return pt


def slots_for(spec: CaseSpec, pt: np.ndarray, s: int, t0: int, t1: int) -> np.ndarray:
    """Physical slot ids (page * page_size + offset) of entries [t0, t1) of sequence s."""
    t = np.arange(t0, t1, dtype=np.int64)
    return (pt[s, t // spec.page_size].astype(np.int64) * spec.page_size + (t % spec.page_size)).astype(np.int32)


def kv_rows(spec: CaseSpec, s: int, device="cpu") -> torch.Tensor:
    """bf16 bits [seq_len_after(s)][512] of sequence s: N(0,1) latent rows."""
    n = spec.seq_len_after(s)
    x = torch.randn(n, D_LATENT, generator=_gen(spec.seed, _TAG_KV, s, device), device=device)
    return _bf16_bits(x)


def idxk_rows(spec: CaseSpec, s: int, device="cpu") -> torch.Tensor:
    """bf16 bits [seq_len_after(s)][128] of sequence s: integers in [-8, 8] or N(0,1).

    Clustered: entry t lies near the centre of its 64-entry block t // 64
    (one centre per block and dimension): integer centres in [-6, 6], with an
    integer offset in {-1, 0, 1} in the eighth of the (block, dimension)
    pairs drawn to vary; or N(0,1) centres plus N(0, 0.02^2) offsets."""
    n = spec.seq_len_after(s)
    g = _gen(spec.seed, _TAG_IK, s, device)
    if spec.clustered:
        nb = (n + CLUSTER_BLOCK - 1) // CLUSTER_BLOCK
        gc = _gen(spec.seed, _TAG_CTR, s, device)
        if spec.integer_indexer:
            ctr = torch.randint(-6, 7, (nb, D_INDEX), generator=gc, device=device).to(torch.float32)
            vary = (torch.randint(0, 8, (nb, D_INDEX), generator=gc, device=device) == 0).to(torch.float32)
            off = torch.randint(-1, 2, (n, D_INDEX), generator=g, device=device).to(torch.float32)
            off = off * vary.repeat_interleave(CLUSTER_BLOCK, dim=0)[:n]
        else:
            ctr = torch.randn(nb, D_INDEX, generator=gc, device=device)
            off = 0.02 * torch.randn(n, D_INDEX, generator=g, device=device)
        x = ctr.repeat_interleave(CLUSTER_BLOCK, dim=0)[:n] + off
    elif spec.integer_indexer:
        x = torch.randint(-8, 9, (n, D_INDEX), generator=g, device=device).to(torch.float32)
    else:
        x = torch.randn(n, D_INDEX, generator=g, device=device)
    return _bf16_bits(x)


def layer_queries(spec: CaseSpec, layer: int, device="cpu"):
    """Per-layer query inputs.

    Returns (q_idx E4M3 bytes [nq][h_idx][128] uint8, w fp32 [nq][h_idx],
    q bf16 bits [nq][h][512] int16).  The indexer query is drawn as integers in
    [-8, 8] (exact in E4M3) or N(0,1) and stored through torch's float8_e4m3fn
    cast; this is input preparation, not part of the layer.
    """
    nq = spec.nq
    g = _gen(spec.seed, _TAG_QI, layer, device)
    if spec.integer_indexer:
        qi = torch.randint(-8, 9, (nq, spec.h_idx, D_INDEX), generator=g, device=device).to(torch.float32)
    else:
        qi = torch.randn(nq, spec.h_idx, D_INDEX, generator=g, device=device)
    q_idx = qi.to(torch.float8_e4m3fn).view(torch.uint8)
    g = _gen(spec.seed, _TAG_W, layer, device)
    if spec.integer_indexer:
        w = torch.randint(1, 3, (nq, spec.h_idx), generator=g, device=device).to(torch.float32)
    else:
        w = torch.randn(nq, spec.h_idx, generator=g, device=device)
    g = _gen(spec.seed, _TAG_Q, layer, device)
    q = _bf16_bits(torch.randn(nq, spec.h, D_LATENT, generator=g, device=device))
    return q_idx, w, q


def ragged_lengths(seed: int, n: int = 64, lo: int = 4096, ratio: int = 256, cap: int = 1 << 24) -> List[int]:
    """Context lengths log-uniform in [lo, lo*ratio): floor(lo * ratio**u), u ~ U[0,1).
    The whole vector is redrawn from the same stream while its sum exceeds cap."""
    g = _gen(seed, _TAG_LEN, 0, "cpu")
    while True:
        u = torch.rand(n, generator=g, dtype=torch.float64).numpy()
        lens = [int(math.floor(lo * ratio ** float(x))) for x in u]
        if sum(lens) <= cap:
            return lens


# ---------------------------------------------------------------------------
# The five workloads (index = position in the list of configurations).
# ---------------------------------------------------------------------------

def config(i: int, integer_indexer: Optional[bool] = None) -> CaseSpec:
    """Workload i at full size.

    0: one Full decode query, 4,096 cached entries, 4 indexer heads with
       integer values, w in {1, 2}, 16 heads, seed 0.
    1: 32 decode sequences x 64K cached + 1 appended, group Full, Reindex,
       Reuse, Reuse; 8 indexer heads N(0,1); 64 heads; seed 1.
    2: causal prefill, 4,096 appended rows against 65,536 cached, one
       sequence, Full; seed 2.
    3: 8 sequences x 1,048,576 cached entries, Full only, no append; seed 3.
    4: 64 ragged sequences (log-uniform 4K..1M, sum <= 2^24) in 64-entry
       pages with a shuffled table, the group of workload 1; seed 4.
    """
    if i == 0:
        s = CaseSpec("full_decode_4k_int", 0, [4096], 0, 4, 16, modes=(FULL,), integer_indexer=True)
    elif i == 1:
        s = CaseSpec("decode_b32_64k_group", 1, [65536] * 32, 1, 8, 64, modes=(FULL, REINDEX, REUSE, REUSE))
    elif i == 2:
        s = CaseSpec("prefill_4096_vs_64k", 2, [65536], 4096, 8, 64, modes=(FULL,), prefill=True)
    elif i == 3:
        s = CaseSpec("decode_b8_1m_full", 3, [1 << 20] * 8, 0, 8, 64, modes=(FULL,), page_size=4096)
    elif i == 4:
        s = CaseSpec("ragged_paged_decode_group", 4, ragged_lengths(4), 1, 8, 64,
                     modes=(FULL, REINDEX, REUSE, REUSE), page_size=64, shuffle_pages=True)
    else:
        raise ValueError(i)
    if integer_indexer is not None:
        s = dataclasses.replace(s, integer_indexer=integer_indexer,
                                name=s.name + ("_int" if integer_indexer and not s.name.endswith("_int") else ""))
    return s


def small_case(name: str, seed: int, cached: List[int], n_new: int = 1, h_idx: int = 8, h: int = 16,
               k: int = 512, modes=(FULL, REINDEX, REUSE, REUSE), integer_indexer: bool = False,
               page_size: int = 64, shuffle_pages: bool = True, prefill: bool = False,
               extra_pages: int = 3, pool_k: int = 0, clustered: bool = False) -> CaseSpec:
    """A reduced workload for oracle-checked parity: same structure, small sizes."""
    return CaseSpec(name, seed, list(cached), n_new, h_idx, h, k=k, modes=tuple(modes),
                    integer_indexer=integer_indexer, page_size=page_size,
                    shuffle_pages=shuffle_pages, prefill=prefill, extra_pages=extra_pages, pool_k=pool_k,
                    clustered=clustered)
