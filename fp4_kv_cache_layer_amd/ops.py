"""Python binding of the CSA2 C ABI: argument marshalling only.

Every function takes device tensors, passes their pointers and the current
HIP stream to libcsa2.so, and raises if the library reports an error.  The
computation itself runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib as L

FULL, REINDEX, REUSE = L.CSA2_FULL, L.CSA2_REINDEX, L.CSA2_REUSE
KV_ROW_BYTES, IDXK_ROW_BYTES, D_LATENT, D_INDEX = 272, 128, 512, 128


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("CSA2 ops take device tensors")
    if not t.is_contiguous():
        raise ValueError("CSA2 ops take contiguous tensors")
    return t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, dtypes, name: str):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")


def _shape(t: Optional[torch.Tensor], dtypes, shape, name: str) -> None:
    """t (if given) has one of dtypes and exactly this shape (the kernels read
    the sizes the arguments imply, so a shorter or wider tensor would be read
    out of bounds or misread)."""
    if t is None:
        return
    _need(t, dtypes, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


_I32 = (torch.int32,)


_BF16 = (torch.int16, torch.bfloat16, torch.uint16)


class Cache:
    """One Full layer's paged global cache in device memory.

    kv    [num_pages][page_size][272] uint8 (E2M1 codes + E8M0 scales)
    idx_k [num_pages][page_size][128] uint8 (E4M3FN)
    page_table [num_seqs][max_pages] int32, seq_lens [num_seqs] int32.
    bounds (optional, bounds=True): [num_pages * page_size / 64][256] uint8,
    the block-level representation of the indexer-K that block-level pruning
    reads (csa2_idxk_bounds_build; layer steps refresh the blocks they append
    to).
    """

    def __init__(self, num_pages: int, page_size: int, page_table: torch.Tensor,
                 seq_lens: Optional[torch.Tensor] = None, device="cuda", kv=None, idx_k=None, bounds: bool = False):
        self.kv = kv if kv is not None else torch.zeros((num_pages, page_size, KV_ROW_BYTES), dtype=torch.uint8, device=device)
        self.idx_k = idx_k if idx_k is not None else torch.zeros((num_pages, page_size, IDXK_ROW_BYTES), dtype=torch.uint8, device=device)
        self.page_table = page_table.to(device=device, dtype=torch.int32).contiguous()
        ns = self.page_table.shape[0]
        self.seq_lens = (seq_lens if seq_lens is not None else torch.zeros(ns, dtype=torch.int32)).to(device=device, dtype=torch.int32).contiguous()
        self.num_pages, self.page_size = num_pages, page_size
        self.bounds = (torch.zeros((num_pages * page_size // L.PRUNE_BLOCK, L.PRUNE_BOUND_BYTES), dtype=torch.uint8,
                                   device=device) if bounds else None)
        self._view = L.CacheView(_ptr(self.kv), _ptr(self.idx_k), _ptr(self.page_table), _ptr(self.seq_lens),
                                 num_pages, page_size, ns, self.page_table.shape[1],
                                 _ptr(self.bounds) if bounds else None)

    def build_bounds(self, first_block: int = 0, n_blocks: Optional[int] = None, stream=None) -> None:
        """Recomputes the block-level representation of blocks
        first_block .. first_block + n_blocks - 1 (default: all) from idx_k."""
        if n_blocks is None:
            n_blocks = self.num_pages * self.page_size // L.PRUNE_BLOCK - first_block
        L.check("csa2_idxk_bounds_build",
                L.load().csa2_idxk_bounds_build(ctypes.byref(self._view), first_block, n_blocks, _stream(stream)))

    @property
    def view(self) -> L.CacheView:
        return self._view

    @property
    def num_seqs(self) -> int:
        return self.page_table.shape[0]

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


def csa2_workspace_bytes(mode: int, nq: int, max_vis: int, h_idx: int, h: int, k: int) -> int:
    return int(L.load().csa2_workspace_bytes(mode, nq, max_vis, h_idx, h, k))


def workspace_state_bytes(nq: int) -> int:
    """Leading workspace bytes that carry state between calls (three
    per-query counters: round_up(nq * 12, 256)); the rest carries none (see
    csa2_workspace_bytes in include/csa2.h)."""
    return (nq * 12 + 255) // 256 * 256


def workspace_prune_masks(ws: torch.Tensor, nq: int, max_vis: int) -> torch.Tensor:
    """The CSA2_STEP_PRUNE block masks of the last pruned call on ws, a
    [nq][ceil(max_vis / 2048)] int32 view (bit i of word c: block 32c + i of
    the query's visible range was pruned; words past a query's visible range
    are not written).  Layout as csa2_workspace_bytes documents it: state
    head, candidates, their keys, chunk floors, masks, block maximum keys."""
    vstride = (max_vis + 2 + 63) // 64 * 64
    fstride = (max_vis + 2047) // 2048
    off = workspace_state_bytes(nq) + 2 * nq * vstride * 4 + nq * fstride * 4
    return ws[off: off + nq * fstride * 4].view(torch.int32).view(nq, fstride)


def pruned_block_fraction(masks: torch.Tensor, q_vis) -> float:
    """Share of the visible 64-entry blocks a mask view marks, over all queries."""
    import numpy as np
    m = masks.cpu().numpy().view(np.uint8).reshape(masks.shape[0], -1)
    pruned = total = 0
    for i, v in enumerate(q_vis):
        nb = (int(v) + 63) // 64
        pruned += int(np.unpackbits(m[i], bitorder="little")[:nb].sum())
        total += nb
    return pruned / max(total, 1)


def csa2_workspace_init(ws: torch.Tensor, stream=None) -> None:
    L.check("csa2_workspace_init", L.load().csa2_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def workspace(mode: int, nq: int, max_vis: int, h_idx: int, h: int, k: int, device="cuda", stream=None) -> torch.Tensor:
    """A zero-initialised workspace sized for the given call shape."""
    n = csa2_workspace_bytes(mode, nq, max_vis, h_idx, h, k)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)
    csa2_workspace_init(ws, stream)
    return ws


def csa2_append_quant_fp4(cache: Cache, slots: torch.Tensor, kv_rows: torch.Tensor, idxk_rows: torch.Tensor,
                          stream=None) -> None:
    _need(slots, (torch.int32,), "slots")
    _need(kv_rows, _BF16, "kv_rows")
    _need(idxk_rows, _BF16, "idxk_rows")
    n = slots.numel()
    if kv_rows.numel() != n * D_LATENT or idxk_rows.numel() != n * D_INDEX:
        raise ValueError("append: row tensors do not match the slot count")
    L.check("csa2_append_quant_fp4", L.load().csa2_append_quant_fp4(
        ctypes.byref(cache.view), _ptr(slots), _ptr(kv_rows), _ptr(idxk_rows), n, _stream(stream)))


def csa2_index_topk(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, q_seq: torch.Tensor, q_vis: torch.Tensor,
                    k: int, max_vis: int, ws: torch.Tensor, out_idx: Optional[torch.Tensor] = None,
                    out_cnt: Optional[torch.Tensor] = None, stream=None,
                    dense: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Indexer scores + Top-K.  dense=True calls csa2_prefill_index_topk (every
    query in sequence q_seq[0]: one FP8 matrix product with a causal mask)."""
    nq, h_idx = q_idx.shape[0], q_idx.shape[1]
    _shape(q_idx, (torch.uint8,), (nq, h_idx, D_INDEX), "q_idx")
    _shape(w, (torch.float32,), (nq, h_idx), "w")
    _shape(q_seq, _I32, (nq,), "q_seq")
    _shape(q_vis, _I32, (nq,), "q_vis")
    _shape(out_idx, _I32, (nq, k), "out_idx")
    _shape(out_cnt, _I32, (nq,), "out_cnt")
    if out_idx is None:
        out_idx = torch.empty((nq, k), dtype=torch.int32, device=q_idx.device)
    if out_cnt is None:
        out_cnt = torch.empty(nq, dtype=torch.int32, device=q_idx.device)
    name = "csa2_prefill_index_topk" if dense else "csa2_index_topk"
    L.check(name, getattr(L.load(), name)(
        ctypes.byref(cache.view), _ptr(q_idx), _ptr(w), _ptr(q_seq), _ptr(q_vis), nq, h_idx, k, max_vis,
        _ptr(out_idx), _ptr(out_cnt), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_cnt


def csa2_pool_workspace(nq: int, p: int, device="cuda") -> torch.Tensor:
    """Workspace for csa2_pool_index_topk (no initial state)."""
    return torch.empty(int(L.load().csa2_pool_workspace_bytes(nq, p)), dtype=torch.uint8, device=device)


def csa2_pool_index_topk(cache: Cache, q_idx: torch.Tensor, w: torch.Tensor, q_seq: torch.Tensor,
                         pool: torch.Tensor, pool_cnt: torch.Tensor, k: int, ws: Optional[torch.Tensor] = None,
                         out_idx: Optional[torch.Tensor] = None, out_cnt: Optional[torch.Tensor] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Hierarchical indexer: Top-k of each query among its pool [nq][P]."""
    nq, h_idx = q_idx.shape[0], q_idx.shape[1]
    p = pool.shape[1]
    _shape(q_idx, (torch.uint8,), (nq, h_idx, D_INDEX), "q_idx")
    _shape(w, (torch.float32,), (nq, h_idx), "w")
    _shape(q_seq, _I32, (nq,), "q_seq")
    _shape(pool, _I32, (nq, p), "pool")
    _shape(pool_cnt, _I32, (nq,), "pool_cnt")
    _shape(out_idx, _I32, (nq, k), "out_idx")
    _shape(out_cnt, _I32, (nq,), "out_cnt")
    if ws is None:
        ws = csa2_pool_workspace(nq, p, device=q_idx.device)
    if out_idx is None:
        out_idx = torch.empty((nq, k), dtype=torch.int32, device=q_idx.device)
    if out_cnt is None:
        out_cnt = torch.empty(nq, dtype=torch.int32, device=q_idx.device)
    L.check("csa2_pool_index_topk", L.load().csa2_pool_index_topk(
        ctypes.byref(cache.view), _ptr(q_idx), _ptr(w), _ptr(q_seq), _ptr(pool), _ptr(pool_cnt), nq, h_idx, p, k,
        _ptr(out_idx), _ptr(out_cnt), _ptr(ws), ws.numel(), _stream(stream)))
    return out_idx, out_cnt


def csa2_sparse_attn(cache: Cache, q: torch.Tensor, q_seq: torch.Tensor, idx: torch.Tensor, cnt: torch.Tensor,
                     sm_scale: float, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     with_lse: bool = True, ws: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    nq, h = q.shape[0], q.shape[1]
    k = idx.shape[1]
    _shape(q, _BF16, (nq, h, D_LATENT), "q")
    _shape(q_seq, _I32, (nq,), "q_seq")
    _shape(idx, _I32, (nq, k), "idx")
    _shape(cnt, _I32, (nq,), "cnt")
    _shape(out, (torch.float32,), (nq, h, D_LATENT), "out")
    _shape(lse, (torch.float32,), (nq, h), "lse")
    if out is None:
        out = torch.empty((nq, h, D_LATENT), dtype=torch.float32, device=q.device)
    if lse is None and with_lse:
        lse = torch.empty((nq, h), dtype=torch.float32, device=q.device)
    L.check("csa2_sparse_attn", L.load().csa2_sparse_attn(
        ctypes.byref(cache.view), _ptr(q), _ptr(q_seq), _ptr(idx), _ptr(cnt), nq, h, k, float(sm_scale),
        _ptr(out), _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
    return out, lse


class LayerCall:
    """Prepared arguments of one csa2_layer_step call (pointers fixed at
    construction, so repeated launches cost one ctypes call each)."""

    def __init__(self, mode: int, cache: Cache, q: torch.Tensor, q_seq: torch.Tensor, q_vis: torch.Tensor,
                 k: int, max_vis: int, sm_scale: float, idx: torch.Tensor, cnt: torch.Tensor,
                 out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                 q_idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None,
                 new_slots: Optional[torch.Tensor] = None, new_kv: Optional[torch.Tensor] = None,
                 new_idxk: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 dense: bool = False, pool: Optional[torch.Tensor] = None, pool_cnt: Optional[torch.Tensor] = None,
                 dense_cand_factor: int = 0, attn_per_head_group: bool = False,
                 timing: Optional["Timing"] = None, seed: Optional[torch.Tensor] = None,
                 seed_cnt: Optional[torch.Tensor] = None):
        """pool / pool_cnt ([nq][P], [nq] int32): hierarchical indexer; a Full
        layer writes its Top-P there, a Reindex layer scores only those.
        dense_cand_factor: the dense indexer's candidate factor (0 default,
        L.DENSE_RESCORE_ALL rescores every query).  attn_per_head_group: one
        attention workgroup per 16-head group even where the shared-row form
        applies.  timing: device timestamps of this call's kernels.
        seed / seed_cnt ([nq][k], [nq] int32): block-level pruning of the
        indexer (needs a cache with bounds); the seed may be idx itself."""
        self.mode = mode
        self.cache = cache
        nq, h = q.shape[0], q.shape[1]
        _shape(q, _BF16, (nq, h, D_LATENT), "q")
        _shape(q_seq, _I32, (nq,), "q_seq")
        _shape(q_vis, _I32, (nq,), "q_vis")
        _shape(idx, _I32, (nq, k), "idx")
        _shape(cnt, _I32, (nq,), "cnt")
        _shape(out, (torch.float32,), (nq, h, D_LATENT), "out")
        _shape(lse, (torch.float32,), (nq, h), "lse")
        if mode in (FULL, REINDEX):
            _shape(q_idx, (torch.uint8,), (nq, q_idx.shape[1], D_INDEX), "q_idx")
            _shape(w, (torch.float32,), (nq, q_idx.shape[1]), "w")
        if mode == FULL and new_slots is not None:
            n_new = new_slots.numel()
            _shape(new_slots, _I32, (n_new,), "new_slots")
            _shape(new_kv, _BF16, (n_new, D_LATENT), "new_kv")
            _shape(new_idxk, _BF16, (n_new, D_INDEX), "new_idxk")
        if pool is not None:
            _shape(pool, _I32, (nq, pool.shape[1]), "pool")
            _shape(pool_cnt, _I32, (nq,), "pool_cnt")
        if seed is not None:
            _shape(seed, _I32, (nq, k), "seed")
            _shape(seed_cnt, _I32, (nq,), "seed_cnt")
        self._keep = (q, q_seq, q_vis, idx, cnt, out, lse, q_idx, w, new_slots, new_kv, new_idxk, ws, pool, pool_cnt,
                      seed, seed_cnt)
        a = L.StepArgs()
        a.cache = ctypes.pointer(cache.view)
        if mode == FULL and new_slots is not None and new_slots.numel() > 0:
            a.new_slots, a.new_kv, a.new_idxk, a.n_new = _ptr(new_slots), _ptr(new_kv), _ptr(new_idxk), new_slots.numel()
        if mode in (FULL, REINDEX):
            a.q_idx, a.w, a.h_idx = _ptr(q_idx), _ptr(w), q_idx.shape[1]
        if ws is not None:
            a.ws, a.ws_bytes = _ptr(ws), ws.numel()
        a.q, a.h, a.sm_scale = _ptr(q), q.shape[1], float(sm_scale)
        a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = _ptr(q_seq), _ptr(q_vis), q.shape[0], k, max_vis
        a.idx, a.cnt, a.out, a.lse = _ptr(idx), _ptr(cnt), _ptr(out), _ptr(lse)
        a.flags = L.STEP_DENSE_INDEX if dense else 0
        if attn_per_head_group:
            a.flags |= L.STEP_ATTN_PER_HEAD_GROUP
        a.dense_cand_factor = int(dense_cand_factor)
        if pool is not None:
            a.flags |= L.STEP_POOL
            a.pool, a.pool_cnt, a.pool_k = _ptr(pool), _ptr(pool_cnt), pool.shape[1]
        if seed is not None:
            a.flags |= L.STEP_PRUNE
            a.seed, a.seed_cnt = _ptr(seed), _ptr(seed_cnt)
        self.args = a
        self.timing = None
        self.set_timing(timing)
        self._ref = ctypes.byref(a)
        self._fn = L.load().csa2_layer_step

    def set_timing(self, timing: Optional["Timing"]) -> None:
        """Attach (or with None detach) device timestamps to later calls."""
        self.timing = timing
        self.args.timing = ctypes.pointer(timing.struct) if timing is not None else None

    def __call__(self, stream=None) -> None:
        st = self._fn(self.mode, self._ref, _stream(stream))
        if st:
            L.check("csa2_layer_step", st)


def csa2_layer_step(mode: int, cache: Cache, q: torch.Tensor, q_seq: torch.Tensor, q_vis: torch.Tensor, k: int,
                    max_vis: int, sm_scale: float, idx: torch.Tensor, cnt: torch.Tensor, out: torch.Tensor,
                    lse: Optional[torch.Tensor] = None, q_idx=None, w=None, new_slots=None, new_kv=None,
                    new_idxk=None, ws=None, stream=None, dense: bool = False, pool=None, pool_cnt=None) -> None:
    LayerCall(mode, cache, q, q_seq, q_vis, k, max_vis, sm_scale, idx, cnt, out, lse, q_idx, w,
              new_slots, new_kv, new_idxk, ws, dense, pool, pool_cnt)(stream)


def csa2_lse_merge(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, stream=None):
    """Merge of two attention branches' (O, LSE) over disjoint key sets (see
    csa2_lse_merge in include/csa2.h).  O tensors [..., dim] fp32, LSEs [...]
    fp32; returns (out, lse), allocating them when not given."""
    for t, n in ((o_a, "o_a"), (o_b, "o_b"), (lse_a, "lse_a"), (lse_b, "lse_b")):
        _need(t, (torch.float32,), n)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dim = o_a.shape[-1]
    rows = o_a.numel() // dim if dim else 0
    if o_b.shape != o_a.shape or lse_a.numel() != rows or lse_b.numel() != rows:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty_like(o_a)
    if lse is None:
        lse = torch.empty_like(lse_a)
    L.check("csa2_lse_merge", L.load().csa2_lse_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), rows, dim,
                                                      _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


def csa2_fake_quant_fp4(x: torch.Tensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """FP4 quantise-dequantise of x (fp32 or bf16, contiguous, numel a multiple
    of 32, blocks of 32 consecutive values) with the main-KV rules (see
    csa2_fake_quant_fp4 in include/csa2.h)."""
    if x.dtype == torch.float32:
        dt = L.DTYPE_F32
    elif x.dtype == torch.bfloat16:
        dt = L.DTYPE_BF16
    else:
        raise ValueError("x must be float32 or bfloat16")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    if out.dtype != x.dtype or out.numel() != x.numel():
        raise ValueError("out must match x")
    L.check("csa2_fake_quant_fp4", L.load().csa2_fake_quant_fp4(_ptr(x), _ptr(out), x.numel(), dt, _stream(stream)))
    return out


class FakeQuantFP4(torch.autograd.Function):
    """Quantization-aware training op: forward csa2_fake_quant_fp4, backward
    the straight-through gradient (identity; the scale rule never clips)."""

    @staticmethod
    def forward(ctx, x):
        return csa2_fake_quant_fp4(x.contiguous())

    @staticmethod
    def backward(ctx, grad):
        return grad


class GroupCall:
    """Prepared csa2_group_step over LayerCalls: appends and indexer scans on
    the calling stream, selects and attentions on n_aux auxiliary streams
    (default priority) with caller-owned events (see include/csa2.h).  With
    n_aux = 0 the layers run in order on the calling stream."""

    def __init__(self, calls, n_aux: int = 2, event_sets: int = 4):
        lib = L.load()
        n = len(calls)
        self.calls = list(calls)
        self.modes = (ctypes.c_int32 * n)(*[c.mode for c in calls])
        self.args = (L.StepArgs * n)()
        for i, c in enumerate(calls):
            ctypes.memmove(ctypes.byref(self.args[i]), ctypes.byref(c.args), ctypes.sizeof(L.StepArgs))
        # Several event sets, used in turn: re-recording an event whose last
        # record the device has not reached yet would hold the host back, so
        # rotating sets lets the host enqueue a few groups ahead.
        self.exs = []
        if n_aux > 0:
            self.streams = [torch.cuda.Stream() for _ in range(n_aux)]
            ne = lib.csa2_group_events(n, n_aux)
            if ne < 0:
                raise ValueError("group too large")
            self.events, self._ev = [], []
            for _ in range(max(1, event_sets)):
                evs = [torch.cuda.Event() for _ in range(ne)]
                for e in evs:              # materialise the hipEvent handles
                    e.record()
                self.events.append(evs)
                arr = (ctypes.c_void_p * ne)(*[0] * ne)
                self._ev.append(arr)
            torch.cuda.synchronize()
            for evs, arr in zip(self.events, self._ev):
                for i, e in enumerate(evs):
                    arr[i] = e.cuda_event
                ex = L.GroupExec()
                for j, st in enumerate(self.streams):
                    ex.aux[j] = st.cuda_stream
                ex.n_aux = n_aux
                ex.events = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
                ex.n_events = ne
                self.exs.append(ex)
        self._turn = 0
        self._n = n
        self._fn = lib.csa2_group_step

    def set_timing(self, timing: Optional["Timing"]) -> None:
        """Attach (or detach) device timestamps to every layer of later calls."""
        for i, c in enumerate(self.calls):
            c.set_timing(timing)
            self.args[i].timing = c.args.timing

    def __call__(self, stream=None) -> None:
        ex = None
        if self.exs:
            ex = ctypes.byref(self.exs[self._turn])
            self._turn = (self._turn + 1) % len(self.exs)
        st = self._fn(self._n, self.modes, self.args, _stream(stream), ex)
        if st:
            L.check("csa2_group_step", st)


# Timing events skip the system-scope fence of a plain event: they only
# measure, and read after a device synchronisation, and the fence's cache
# write-back would otherwise slow the work being timed.
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvent:
    """A timing hipEvent created without the system-scope fence (see
    hipEventDisableSystemFence in hip_runtime_api.h)."""

    def __init__(self):
        self.lib = L.load()
        self.handle = ctypes.c_void_p()
        if self.lib.hipEventCreateWithFlags(ctypes.byref(self.handle), _HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream=None) -> None:
        if self.lib.hipEventRecord(self.handle, ctypes.c_void_p(_stream(stream))) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            self.lib.hipEventDestroy(self.handle)
        except Exception:
            pass


class TimingRing:
    """Device-event ring for one kernel class: start/stop hipEvent pairs that
    the library records through the launches of calls carrying it."""

    def __init__(self, capacity: int):
        self.events = [(HipEvent(), HipEvent()) for _ in range(capacity)]
        self._start = (ctypes.c_void_p * capacity)(*[a.handle.value for a, _ in self.events])
        self._stop = (ctypes.c_void_p * capacity)(*[b.handle.value for _, b in self.events])
        self.ring = L.TimingRing(ctypes.cast(self._start, ctypes.POINTER(ctypes.c_void_p)),
                                 ctypes.cast(self._stop, ctypes.POINTER(ctypes.c_void_p)), capacity, 0)

    def durations_ms(self):
        torch.cuda.synchronize()
        return [a.elapsed_ms(b) for a, b in self.events[:self.ring.count]]


class Timing:
    """Per-call device timing (csa2_timing): one ring per kernel class named
    in capacities ({kernel class: capacity}); attach it to LayerCalls with
    set_timing (or the timing argument) before building a GroupCall on them."""

    def __init__(self, capacities: dict):
        self.rings = {cls: TimingRing(cap) for cls, cap in capacities.items()}
        self.struct = L.Timing()
        for cls, r in self.rings.items():
            self.struct.ring[cls] = ctypes.pointer(r.ring)

    def reset(self) -> None:
        for r in self.rings.values():
            r.ring.count = 0

    def durations_ms(self, cls: int):
        return self.rings[cls].durations_ms()
