"""Plain fp64 CPU oracle of one CSA2 layer step.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The GPU library never
calls it, and it shares no code, table or constant generator with the GPU
sources: every format here is decoded from its bit fields and every encoder
picks the nearest representable value by search over its own value table.

What is computed, and where it comes from:

* The three static layer modes (Full, Reindex, Reuse) and the Top-512
  selection: "Unlocking Extreme Context Scaling with DeepSeek-V4.1-Flash",
  section "Compressed Sparse Attention 2 (CSA2)"; the same three modes in
  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", Method.
* The main KV stored in the E2M1 FP4 format: "DeepSeek-V4.1-Flash" (aiany.app
  item), "What Sets It Apart"; FP4 main-KV caching at about half the bytes of
  FP8: "Unlocking Extreme Context Scaling ...", "Deployment and
  Infrastructure".
* The pages give no formula, block size, scale format, indexer format or
  tie rule.  The readings used here (each a plain choice the rest supports):
  - main KV: one 512-wide latent row per entry, shared by all heads as both
    key and value; E2M1 codes with one E8M0 scale per 32 consecutive
    elements; scale = smallest power of two 2^e with amax <= 6 * 2^e; codes
    by round-to-nearest, ties to the even code, sign bit kept (so -0 is a
    code); row bytes = 256 code bytes (even element in the low nibble) then
    16 scale bytes;
  - indexer-K and indexer-Q: OCP FP8 E4M3FN, 128 wide; the K rows are encoded
    from bf16 by round-to-nearest-even with saturation to +-448;
  - indexer score of entry t for one query: sum over indexer heads h of
    w_h * max(0, q_h . k_t), a zero score is taken as +0;
  - Top-K: the first min(k, V) entries under the order (score descending,
    index ascending), returned in ascending index order, padded with -1;
  - attention: softmax(sm_scale * q_h . X_t) over the selected rows, output
    sum_j p_j X_tj per head, plus the natural-log LSE.
* Hierarchical Sparse Indexer: later indexers are restricted to a shared
  candidate pool chosen by an earlier indexer ("DeepSeek-V4.1-Flash: Pushing
  the Limits of KV Cache Compression", Method).  The pool's size and the way it
  is chosen are not given; the reading used: the earlier (Full) layer's own
  Top-P under the same order (P >= k), and a later (Reindex) layer scores only
  the pool's entries and keeps its Top-k among them (pool_index_topk).
* Block-level pruning, the other half of the hierarchical indexer: the
  indexer it is informed by scores token-level entries and prunes them by
  block-level representations ("DeepSeek-V4.1-Flash: Pushing the Limits of
  KV Cache Compression", Related Work).  No block summary or pruning rule is
  given; the reading used keeps the Top-K exact: a block is 64 consecutive
  cache rows, its representation the per-dimension maximum and minimum of
  its indexer-K (block_bounds), which bounds every score in the block from
  above (block_score_bound); a query's threshold is the k-th largest score
  among k or more distinct entries it has scored already (a seed, such as
  its previous Top-K), and blocks whose bound lies below the threshold are
  never scored (pruned_index_topk), which cannot change the Top-K.
* FP4 for the global KV during training, by quantization-aware training:
  "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression".  The
  fake-quantization forward (fake_quant_e2m1) applies the cache's own E2M1 +
  E8M0 rules to every 32-element block; the pages name no gradient rule, and
  since the scale rule never clips (every |x| / 2^e <= 6) the plain
  straight-through gradient (identity) is taken.
* The global (CSA2) branch sits beside a local sliding-window branch: "DeepSeek-
  V4.1-Flash: Pushing the Limits of KV Cache Compression" (global attention
  over the full context together with local sliding-window attention) and the
  research-podcast summary (global context decoupled from local
  sliding-window attention).  No combination formula is given; the reading
  used is one softmax over the union of the two branches' keys, which the two
  branches' (output, LSE) pairs give exactly (lse_merge).

All arithmetic is float64.  Parity pins live in the tests (closed-form format
tables, brute-force selection, a textbook dense attention, exact integer
arithmetic); the numeric attention values on N(0,1) inputs are otherwise
pinned only by those invariants.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np

D_LATENT = 512
D_INDEX = 128
BLOCK = 32
N_BLOCKS = D_LATENT // BLOCK          # 16 scales per row
CODE_BYTES = D_LATENT // 2            # 256
KV_ROW_BYTES = CODE_BYTES + N_BLOCKS  # 272
E2M1_MAX = 6.0
E4M3_MAX = 448.0

FULL, REINDEX, REUSE = 0, 1, 2


# ---------------------------------------------------------------------------
# number formats (decoded from their bit fields)
# ---------------------------------------------------------------------------

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (any 16-bit integer dtype) -> float64 (exact)."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def e2m1_decode(code) -> np.ndarray:
    """E2M1 nibble -> value.  Bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (0 or 0.5)."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def e8m0_decode(code) -> np.ndarray:
    """E8M0 byte -> 2^(code - 127); 0xFF is NaN."""
    c = np.asarray(code).astype(np.int64)
    return np.where(c == 0xFF, np.nan, np.exp2(c - 127.0))


def e4m3fn_decode(code) -> np.ndarray:
    """OCP E4M3FN byte -> value.  Bit 7 sign, bits 6..3 exponent (bias 7),
    bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
    there is no infinity."""
    c = np.asarray(code).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _nearest_even_code(a: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index into the ascending value grid of the nearest value to each a >= 0
    (a <= grid[-1]); an exact tie goes to the even index."""
    i = np.searchsorted(grid, a, side="left")            # grid[i-1] < a <= grid[i]
    i = np.clip(i, 0, len(grid) - 1)
    lo = np.clip(i - 1, 0, len(grid) - 1)
    d_hi = grid[i] - a
    d_lo = a - grid[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    pick_lo &= (i > 0) & (grid[i] != a)
    return np.where(pick_lo, lo, i)


_E2M1_GRID = e2m1_decode(np.arange(8))                   # 0, .5, 1, 1.5, 2, 3, 4, 6
_E4M3_GRID = e4m3fn_decode(np.arange(0x7F))              # codes 0x00..0x7E, ascending


def e2m1_encode(r) -> np.ndarray:
    """Value (already divided by its block scale) -> E2M1 nibble: nearest of
    the 8 magnitudes, ties to the even code, magnitudes above 6 saturate; the
    sign bit is copied from the input, so a negative input that rounds to zero
    gives code 0x8."""
    r = np.asarray(r, dtype=np.float64)
    assert not np.isnan(r).any()
    a = np.minimum(np.abs(r), E2M1_MAX)
    code = _nearest_even_code(a, _E2M1_GRID)
    return (code | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


def e4m3fn_encode(x) -> np.ndarray:
    """Value -> E4M3FN byte: nearest finite value, ties to the even code,
    magnitudes above 448 saturate to 448; the sign bit is copied."""
    x = np.asarray(x, dtype=np.float64)
    assert not np.isnan(x).any()
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = _nearest_even_code(a, _E4M3_GRID)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Smallest integer e with amax <= 6 * 2^e (the block max divided by 6,
    rounded up to a power of two), clamped to the E8M0 range [-127, 127];
    an all-zero block takes -127."""
    amax = np.asarray(amax, dtype=np.float64)
    pos = amax > 0
    safe = np.where(pos, amax, 1.0)
    e = np.ceil(np.log2(safe / 6.0)).astype(np.int64)
    # make the defining inequality hold exactly (6 * 2^e is exact in fp64)
    for _ in range(2):
        e = np.where(safe > 6.0 * np.exp2(e.astype(np.float64)), e + 1, e)
        e = np.where(safe <= 6.0 * np.exp2((e - 1).astype(np.float64)), e - 1, e)
    e = np.where(pos, e, -127)
    return np.clip(e, -127, 127)


# ---------------------------------------------------------------------------
# row encodings
# ---------------------------------------------------------------------------

def quantize_kv_rows(x) -> np.ndarray:
    """[n][512] values -> [n][272] bytes: per 32-block scale and E2M1 codes."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, N_BLOCKS, BLOCK)
    e = block_exponent(np.abs(x).max(axis=2))                         # [n][16]
    r = x / np.exp2(e.astype(np.float64))[:, :, None]                 # exact
    codes = e2m1_encode(r).reshape(-1, D_LATENT).astype(np.uint8)     # [n][512]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    scales = (e + 127).astype(np.uint8)
    return np.concatenate([packed, scales], axis=1)


def fake_quant_e2m1(x) -> np.ndarray:
    """Quantise-dequantise of values [..., d] (d a multiple of 32) with the
    main-KV rules: per 32-element block the scale 2^e of block_exponent, the
    E2M1 code of x / 2^e, decoded back to E2M1(code) * 2^e (sign kept, so a
    negative value that rounds to zero gives -0)."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % BLOCK == 0
    b = x.reshape(-1, BLOCK)
    e = block_exponent(np.abs(b).max(axis=1)).astype(np.float64)
    codes = e2m1_encode(b / np.exp2(e)[:, None])
    return (e2m1_decode(codes) * np.exp2(e)[:, None]).reshape(x.shape)


def dequantize_kv_rows(b) -> np.ndarray:
    """[n][272] bytes -> [n][512] values: X[32j+i] = E2M1(code) * 2^(S_j - 127)."""
    b = np.asarray(b, dtype=np.uint8).reshape(-1, KV_ROW_BYTES)
    packed = b[:, :CODE_BYTES]
    codes = np.empty((b.shape[0], D_LATENT), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    scale = e8m0_decode(b[:, CODE_BYTES:])                            # [n][16]
    return (e2m1_decode(codes).reshape(-1, N_BLOCKS, BLOCK) * scale[:, :, None]).reshape(-1, D_LATENT)


def quantize_idxk_rows(x) -> np.ndarray:
    """[n][128] values -> [n][128] E4M3FN bytes."""
    return e4m3fn_encode(np.asarray(x, dtype=np.float64)).reshape(-1, D_INDEX)


# ---------------------------------------------------------------------------
# the paged cache
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Cache:
    """One Full layer's global cache.  Logical entry t of sequence s sits at
    page page_table[s][t // page_size], offset t % page_size."""
    kv: np.ndarray          # [num_pages][page_size][272] uint8
    idx_k: np.ndarray       # [num_pages][page_size][128] uint8
    page_table: np.ndarray  # [num_seqs][max_pages] int32
    seq_lens: np.ndarray    # [num_seqs] int32

    @property
    def page_size(self) -> int:
        return self.kv.shape[1]

    @staticmethod
    def empty(num_pages: int, page_size: int, page_table, seq_lens) -> "Cache":
        return Cache(np.zeros((num_pages, page_size, KV_ROW_BYTES), np.uint8),
                     np.zeros((num_pages, page_size, D_INDEX), np.uint8),
                     np.asarray(page_table, np.int32).copy(), np.asarray(seq_lens, np.int32).copy())

    def locate(self, seq: int, t) -> Tuple[np.ndarray, np.ndarray]:
        t = np.asarray(t, dtype=np.int64)
        return self.page_table[seq, t // self.page_size].astype(np.int64), t % self.page_size

    def kv_rows(self, seq: int, t) -> np.ndarray:
        p, o = self.locate(seq, t)
        return self.kv[p, o]

    def idxk_rows(self, seq: int, t) -> np.ndarray:
        p, o = self.locate(seq, t)
        return self.idx_k[p, o]


def append_quant_fp4(cache: Cache, slots, kv_bits, idxk_bits) -> None:
    """Quantize-on-append: row i is encoded and written at physical slot
    slots[i] = page * page_size + offset (both the main-KV row and the
    indexer-K row).  Later rows win if a slot repeats."""
    slots = np.asarray(slots, dtype=np.int64)
    if slots.size == 0:
        return
    kv = quantize_kv_rows(bf16_to_f64(kv_bits))
    ik = quantize_idxk_rows(bf16_to_f64(idxk_bits))
    ps = cache.page_size
    cache.kv[slots // ps, slots % ps] = kv
    cache.idx_k[slots // ps, slots % ps] = ik


# ---------------------------------------------------------------------------
# indexer, Top-K, attention
# ---------------------------------------------------------------------------

def index_scores(cache: Cache, seq: int, vis: int, qi_bytes, w, chunk: int = 1 << 16) -> np.ndarray:
    """Scores of entries 0..vis-1 of one sequence for one query:
    s_t = sum_h w_h * max(0, sum_d QI[h,d] * KI[t,d]); -0 becomes +0."""
    qi = e4m3fn_decode(np.asarray(qi_bytes, np.uint8)).reshape(-1, D_INDEX)   # [H_I][128]
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    assert qi.shape[0] == w.shape[0]
    out = np.empty(vis, dtype=np.float64)
    for t0 in range(0, vis, chunk):             # independent entries; chunked only to bound memory
        t = np.arange(t0, min(vis, t0 + chunk))
        k = e4m3fn_decode(cache.idxk_rows(seq, t))                              # [n][128]
        dots = k @ qi.T                                                         # [n][H_I]
        out[t0:t0 + len(t)] = np.maximum(dots, 0.0) @ w
    out = out + 0.0                             # IEEE: -0 + +0 = +0
    assert not np.isnan(out).any()
    return out


def select_topk(scores, k: int) -> Tuple[np.ndarray, int]:
    """First min(k, V) entries under (score descending, index ascending),
    returned ascending by index and padded with -1 to length k."""
    s = np.asarray(scores, dtype=np.float64)
    v = s.shape[0]
    kp = min(k, v)
    order = np.lexsort((np.arange(v), -s))      # primary: -score, secondary: index
    chosen = np.sort(order[:kp]).astype(np.int32)
    out = np.full(k, -1, dtype=np.int32)
    out[:kp] = chosen
    return out, kp


def index_topk(cache: Cache, q_idx, w, q_seq, q_vis, k: int):
    """Per query: scores over its visible entries, then Top-K.
    q_idx [nq][H_I][128] E4M3 bytes, w [nq][H_I] -> idx [nq][k], cnt [nq]."""
    q_idx = np.asarray(q_idx, np.uint8)
    w = np.asarray(w, np.float64)
    nq = len(q_seq)
    idx = np.full((nq, k), -1, dtype=np.int32)
    cnt = np.zeros(nq, dtype=np.int32)
    for i in range(nq):
        s = index_scores(cache, int(q_seq[i]), int(q_vis[i]), q_idx[i], w[i])
        idx[i], cnt[i] = select_topk(s, k)
    return idx, cnt


def pool_index_topk(cache: Cache, q_idx, w, q_seq, pool, pool_cnt, k: int):
    """Hierarchical indexer: per query, the scores of the entries of its pool
    only (pool [nq][P] entry indices, ascending, the first pool_cnt valid),
    then the first min(k, pool_cnt) of them under (score descending, entry
    index ascending), returned ascending by index and padded with -1."""
    q_idx = np.asarray(q_idx, np.uint8)
    w = np.asarray(w, np.float64)
    pool = np.asarray(pool, np.int64)
    nq = len(q_seq)
    idx = np.full((nq, k), -1, dtype=np.int32)
    cnt = np.zeros(nq, dtype=np.int32)
    for i in range(nq):
        t = pool[i, :int(pool_cnt[i])]
        qi = e4m3fn_decode(q_idx[i]).reshape(-1, D_INDEX)
        kt = e4m3fn_decode(cache.idxk_rows(int(q_seq[i]), t))                  # [n][128]
        s = np.maximum(kt @ qi.T, 0.0) @ w[i] + 0.0                            # -0 -> +0
        kp = min(k, t.size)
        order = np.lexsort((t, -s))
        idx[i, :kp] = np.sort(t[order[:kp]])
        cnt[i] = kp
    return idx, cnt


PRUNE_BLOCK = 64                        # cache rows per block-level representation


def block_bounds(cache: Cache) -> Tuple[np.ndarray, np.ndarray]:
    """Block-level representation of the indexer-K: for every block of 64
    consecutive physical rows, the per-dimension maximum and minimum of the
    decoded E4M3 values -> ([n_blocks][128], [n_blocks][128])."""
    k = e4m3fn_decode(cache.idx_k.reshape(-1, PRUNE_BLOCK, D_INDEX))
    return k.max(axis=1), k.min(axis=1)


def block_score_bound(qi_bytes, w, bmax, bmin) -> np.ndarray:
    """An upper bound of s_t = sum_h w_h * max(0, q_h . k_t) over every k_t
    with bmin <= k_t <= bmax in every dimension ([..., 128] boxes -> [...]).
    q_h . k lies in [lo_h, hi_h], hi_h = sum_d max(q_hd bmax_d, q_hd bmin_d),
    lo_h = sum_d min(q_hd bmax_d, q_hd bmin_d); max(0, x) never decreases, so
    w_h max(0, q_h . k) <= w_h max(0, hi_h) when w_h >= 0 and
    <= w_h max(0, lo_h) when w_h < 0."""
    qi = e4m3fn_decode(np.asarray(qi_bytes, np.uint8)).reshape(-1, D_INDEX)   # [H_I][128]
    w = np.asarray(w, dtype=np.float64).reshape(-1)
    bmax = np.asarray(bmax, np.float64)
    bmin = np.asarray(bmin, np.float64)
    total = np.zeros(bmax.shape[:-1], dtype=np.float64)
    for h in range(qi.shape[0]):
        a, b = qi[h] * bmax, qi[h] * bmin
        hi = np.maximum(a, b).sum(axis=-1)
        lo = np.minimum(a, b).sum(axis=-1)
        total += w[h] * np.maximum(hi if w[h] >= 0 else lo, 0.0)
    return total


def prune_threshold(cache: Cache, seq: int, vis: int, qi_bytes, w, seed_row, k: int) -> float:
    """The k-th largest score among the distinct entries of seed_row inside
    [0, vis) (negative or out-of-range entries ignored), or -inf when fewer
    than k such entries are given: at least k visible entries score at or
    above it, so it never exceeds the k-th largest score of the query."""
    t = np.unique(np.asarray(seed_row, np.int64))
    t = t[(t >= 0) & (t < vis)]
    if t.size < k:
        return -np.inf
    qi = e4m3fn_decode(np.asarray(qi_bytes, np.uint8)).reshape(-1, D_INDEX)
    kt = e4m3fn_decode(cache.idxk_rows(seq, t))
    s = np.maximum(kt @ qi.T, 0.0) @ np.asarray(w, np.float64).reshape(-1) + 0.0
    return float(np.sort(s)[::-1][k - 1])


def pruned_index_topk(cache: Cache, q_idx, w, q_seq, q_vis, seed, seed_cnt, k: int):
    """index_topk with block-level pruning: per query the threshold T of its
    seed (prune_threshold over seed[i][:seed_cnt[i]]); the logical 64-entry
    blocks of its visible range whose bound (block_score_bound over the
    block's physical rows) lies below T are not scored, and the Top-K is
    taken over the entries of the other blocks.  Returns idx, cnt and the
    per-query boolean mask of pruned logical blocks."""
    q_idx = np.asarray(q_idx, np.uint8)
    w = np.asarray(w, np.float64)
    bmax, bmin = block_bounds(cache)
    ps = cache.page_size
    nq = len(q_seq)
    idx = np.full((nq, k), -1, dtype=np.int32)
    cnt = np.zeros(nq, dtype=np.int32)
    masks = []
    for i in range(nq):
        s, v = int(q_seq[i]), int(q_vis[i])
        thr = prune_threshold(cache, s, v, q_idx[i], w[i], np.asarray(seed[i])[:int(seed_cnt[i])], k)
        nb = (v + PRUNE_BLOCK - 1) // PRUNE_BLOCK
        first = np.arange(nb, dtype=np.int64) * PRUNE_BLOCK               # logical first entry of each block
        phys = (cache.page_table[s, first // ps].astype(np.int64) * ps + first % ps) // PRUNE_BLOCK
        ub = block_score_bound(q_idx[i], w[i], bmax[phys], bmin[phys])
        pruned = ub < thr
        sc = index_scores(cache, s, v, q_idx[i], w[i])
        keep = ~np.repeat(pruned, PRUNE_BLOCK)[:v]
        t = np.nonzero(keep)[0]
        kp = min(k, t.size)
        order = np.lexsort((t, -sc[t]))
        idx[i, :kp] = np.sort(t[order[:kp]])
        cnt[i] = kp
        masks.append(pruned)
    return idx, cnt, masks


def attend(cache: Cache, seq: int, q_bits, idx_row, cnt: int, sm_scale: float):
    """Softmax attention of one query (all heads) over its selected rows.
    K = V = the dequantised latent.  Returns O [H][512], LSE [H]."""
    q = bf16_to_f64(q_bits).reshape(-1, D_LATENT)                 # [H][512]
    t = np.asarray(idx_row[:cnt], dtype=np.int64)
    if cnt == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    x = dequantize_kv_rows(cache.kv_rows(seq, t))                 # [cnt][512]
    logits = sm_scale * (q @ x.T)                                 # [H][cnt]
    m = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - m)
    z = p.sum(axis=1, keepdims=True)
    o = (p @ x) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def sparse_attn(cache: Cache, q, q_seq, idx, cnt, sm_scale: float):
    """O [nq][H][512] and LSE [nq][H] for every query."""
    q = np.asarray(q)
    nq = len(q_seq)
    h = q.shape[1]
    out = np.zeros((nq, h, D_LATENT))
    lse = np.zeros((nq, h))
    for i in range(nq):
        out[i], lse[i] = attend(cache, int(q_seq[i]), q[i], idx[i], int(cnt[i]), sm_scale)
    return out, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Output and LSE of one softmax over the union of two disjoint key sets,
    from each set's own softmax output O [..][d] and natural-log LSE [..]
    (the global branch and the local sliding-window branch).  Exactly: with
    Z = e^lse_a + e^lse_b, O = (e^lse_a O_a + e^lse_b O_b) / Z and LSE = ln Z.
    A side with no keys has LSE = -inf and counts for nothing; both empty
    gives O = 0 and LSE = -inf, the convention of attend()."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    empty = np.isneginf(m)
    ms = np.where(empty, 0.0, m)
    wa = np.where(np.isneginf(la), 0.0, np.exp(la - ms))
    wb = np.where(np.isneginf(lb), 0.0, np.exp(lb - ms))
    z = wa + wb
    zs = np.where(empty, 1.0, z)
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / zs[..., None]
    lse = np.where(empty, -np.inf, ms + np.log(zs))
    return o, lse


def layer_step(mode: int, cache: Cache, q, q_seq, q_vis, k: int, sm_scale: float,
               q_idx=None, w=None, new_slots=None, new_kv=None, new_idxk=None,
               idx: Optional[np.ndarray] = None, cnt: Optional[np.ndarray] = None):
    """One CSA2 layer.

    Full: append the new rows into this layer's own cache, score and select
    afresh, attend.  Reindex: score a new indexer query against the given
    (earlier Full layer's) cache, select, attend.  Reuse: attend with the
    given indices of an earlier layer.  Returns (idx, cnt, O, LSE).
    """
    if mode == FULL:
        if new_slots is not None:
            append_quant_fp4(cache, new_slots, new_kv, new_idxk)
    if mode in (FULL, REINDEX):
        idx, cnt = index_topk(cache, q_idx, w, q_seq, q_vis, k)
    elif mode == REUSE:
        assert idx is not None and cnt is not None
    else:
        raise ValueError(mode)
    o, lse = sparse_attn(cache, q, q_seq, idx, cnt, sm_scale)
    return idx, cnt, o, lse
