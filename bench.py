"""CSA2 layer-step benchmark on one MI355X.

Decode workloads (default: workload 1).  One step = one CSA2 layer group over
a decode batch, as one csa2_layer_step call per layer in layer order: in a
model each layer's queries depend on the previous layer's output, so this is
the schedule a real decode step runs.  Inputs are synthetic, seeded and
resident in HBM when timing starts.

The graded (headline) timing is cache-scrubbed: before every step a 512 MiB
read evicts the 256 MB Infinity Cache and the L2 (in a model the layers in
between would), and each step is bracketed by device events on the stream
the layers run on.  The same steps back to back, with the indexer-K partly
served from the Infinity Cache, are reported beside it as cache-assisted.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --config 1   # 32 x (65,536 + 1 appended), Full/Reindex/Reuse/Reuse (default)
    python bench.py --config 3   # 8 x 1,048,576 entries, Full only
    python bench.py --config 4   # 64 ragged sequences (4K..1M, <= 2^24 entries), 64-entry shuffled pages
    python bench.py --config 2   # causal prefill of 4,096 rows against 65,536 cached (dense FP8 indexer)
    python bench.py --only-timed # the timed region alone (for profiler runs)
    python bench.py --copy-calibration   # plain device copies of known size, for scaling
                                         # rocprofv3 FETCH_SIZE / WRITE_SIZE readings
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
METRICS = {
    1: "CSA2 decode tokens/s (B=32, 64K ctx) + % of HBM roofline",
    2: "CSA2 prefill tokens/s (4,096 rows vs 64K ctx) + % of FP8 MFMA roofline (dense indexer)",
    3: "CSA2 decode tokens/s (B=8, 1M ctx, Full layer) + % of HBM roofline",
    4: "CSA2 decode tokens/s (64 ragged sequences, 4K-1M ctx, paged) + % of HBM roofline",
}
COPY_BYTES = 1 << 30
SCRUB_BYTES = 512 << 20


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def scan_bytes(spec) -> int:
    """Algorithmic bytes of one indexer-scan launch: every visible indexer-K
    row (128 B) of every query, plus each query's indexer query (h_idx x 128 B)
    and head weights (h_idx x 4 B)."""
    vis = spec.q_vis()
    return int(vis.sum()) * 128 + spec.nq * spec.h_idx * (128 + 4)


def dense_flops(spec) -> int:
    """Algorithmic FLOP of the dense prefill indexer: every causal
    (query, visible entry) pair costs h_idx dot products of length 128."""
    return int(spec.q_vis().sum()) * 2 * spec.h_idx * 128


def attn_bytes(spec) -> int:
    """Algorithmic bytes of one attention layer: min(k, V) gathered rows
    (272 B) and their indices per query, bf16 Q, fp32 O and LSE."""
    rows = sum(min(spec.k, int(v)) for v in spec.q_vis())
    return rows * (272 + 4) + spec.nq * (spec.h * 512 * 2 + spec.h * 512 * 4 + spec.h * 4)


def append_bytes(spec) -> int:
    """Algorithmic bytes of the Full layer's append: bf16 rows in, encoded
    rows and slots out."""
    return spec.num_seqs * spec.n_new * (1024 + 256 + 272 + 128 + 4) if not spec.prefill else \
        spec.n_new * (1024 + 256 + 272 + 128 + 4)


def group_bytes(spec) -> int:
    """Algorithmic bytes of one layer group: the scans of its Full and Reindex
    layers, every layer's attention, the append."""
    from fp4_kv_cache_layer_amd import ops
    n_scan = sum(1 for m in spec.modes if m != ops.REUSE)
    return n_scan * scan_bytes(spec) + len(spec.modes) * attn_bytes(spec) + append_bytes(spec)


def merge_bytes(rows: int, dim: int = 512) -> int:
    """Algorithmic bytes of one branch merge: both branches' outputs and LSEs
    in, the merged output and LSE out."""
    return rows * (3 * dim * 4 + 3 * 4)


def pool_scan_bytes(nq: int, pool_k: int, h_idx: int) -> int:
    """Algorithmic bytes of one pool-scoring launch: each query's pool indices
    (4 B) and gathered indexer-K rows (128 B), its indexer query and weights,
    and the pool scores written (4 B each)."""
    return nq * (pool_k * (4 + 128 + 4) + h_idx * (128 + 4))


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def percentiles(xs) -> dict:
    """p10 / p50 / p90 of per-step durations (ms)."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {f"p{p}": round(float(np.percentile(a, p)), 5) for p in (10, 50, 90)}


def _avg_us(xs):
    return round(statistics.mean(xs) * 1e3, 2) if xs else None


def event_avg_ms(launch, reps: int) -> float:
    """Mean duration of `reps` back-to-back launches on the current stream,
    bracketed by one pair of device events (for single-kernel calls)."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    launch()
    torch.cuda.synchronize()
    e0, e1 = ops.HipEvent(), ops.HipEvent()
    e0.record()
    for _ in range(reps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_ms(e1) / reps


class Scrubber:
    """A read of SCRUB_BYTES on the current stream, enough to evict the
    256 MB Infinity Cache and every L2."""

    def __init__(self):
        import torch
        self.buf = torch.ones(SCRUB_BYTES // 8, dtype=torch.int64, device="cuda")
        self.sink = torch.zeros((), dtype=torch.int64, device="cuda")

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def scrubbed_steps(step, n: int, scrub) -> list:
    """n steps, each after a cache scrub and bracketed by device events on
    the current stream (timing events without the system-scope fence, whose
    cache write-back would slow the step they bracket); returns the step
    durations in ms."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    evs = [(ops.HipEvent(), ops.HipEvent()) for _ in range(n)]
    for e0, e1 in evs:
        scrub()
        e0.record()
        step()
        e1.record()
    torch.cuda.synchronize()
    return [a.elapsed_ms(b) for a, b in evs]


def time_lse_merge(o_a, lse_a, reps: int = 20):
    """csa2_lse_merge of the CSA2 output with a synthetic local-branch output
    of the same shape: mean duration of back-to-back launches."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    g = torch.Generator(device="cuda").manual_seed(5)
    o_b = torch.randn(o_a.shape, generator=g, device="cuda", dtype=torch.float32)
    lse_b = torch.randn(lse_a.shape, generator=g, device="cuda", dtype=torch.float32) * 4
    out, lse = torch.empty_like(o_a), torch.empty_like(lse_a)
    avg_s = event_avg_ms(lambda: ops.csa2_lse_merge(o_a, lse_a, o_b, lse_b, out, lse), reps) / 1e3
    rows = lse_a.numel()
    b = merge_bytes(rows, o_a.shape[-1])
    return {"kernel": "lse_merge_kernel", "rows": rows, "dim": int(o_a.shape[-1]), "bytes": b,
            "avg_us": round(avg_s * 1e6, 2), "GBps": round(b / avg_s / 1e9, 1),
            "hbm_frac": round(b / avg_s / 1e9 / HBM_PEAK_GBS, 4)}


def time_fake_quant(x, reps: int = 10):
    """csa2_fake_quant_fp4 on x; algorithmic bytes = x read once and its
    quantised copy written once."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    out = torch.empty_like(x)
    avg_s = event_avg_ms(lambda: ops.csa2_fake_quant_fp4(x, out), reps) / 1e3
    b = 2 * x.numel() * x.element_size()
    return {"kernel": "fake_quant_" + ("bf16" if x.element_size() == 2 else "f32") + "_kernel",
            "values": x.numel(), "bytes": b, "avg_us": round(avg_s * 1e6, 2), "GBps": round(b / avg_s / 1e9, 1),
            "hbm_frac": round(b / avg_s / 1e9 / HBM_PEAK_GBS, 4)}


def measured_hbm_read(nbytes: int):
    """Measured streaming-read rates (GB/s) of a plain kernel over nbytes:
    cold (successive slices of a buffer far larger than the 256 MB
    Infinity Cache) and warm (the same buffer every launch)."""
    import torch

    from fp4_kv_cache_layer_amd import probe
    nb = (min(nbytes, 1 << 30) + 15) // 16 * 16
    rot = max(2, (2 << 30) // nb)
    buf = torch.ones(rot * nb, dtype=torch.uint8, device="cuda")
    warm = probe.stream_read_gbps(buf, nb, rotate=1)
    cold = probe.stream_read_gbps(buf, nb, rotate=rot)
    del buf
    torch.cuda.empty_cache()
    return cold, warm


def measured_mfma_fp8():
    """Measured dense FP8 MFMA rates (TFLOP/s): the bare instruction stream,
    and the same stream with the indexer's minimal per-score epilogue (ReLU
    and head-weight multiply-add per output, one add) sharing the SIMD."""
    from fp4_kv_cache_layer_amd import probe
    return probe.mfma_fp8_tflops(epilogue=False), probe.mfma_fp8_tflops(epilogue=True)


def source_hash(name: str) -> str:
    """Hash of a kernel source file: a stored counter reading applies only to
    the kernel it was taken on."""
    src = os.path.join(ROOT, "fp4_kv_cache_layer_amd", "csrc", name)
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def stored_traffic(path: str, workload: str, src_name: str):
    """HBM bytes per launch from a stored rocprofv3 FETCH_SIZE/WRITE_SIZE
    reading (one entry per workload), or None when it is missing or was
    taken on other source."""
    try:
        entries = json.load(open(path))
        if isinstance(entries, dict):
            entries = [entries]
        for tr in entries:
            if tr.get("workload") == workload and tr.get("kernel_source_sha256_16") == source_hash(src_name):
                return tr.get("bytes_per_launch")
    except Exception:
        pass
    return None


def copy_calibration(reps: int = 4) -> int:
    """Device-to-device copies of exactly COPY_BYTES each (torch's copy
    kernel): FETCH_SIZE and WRITE_SIZE of these launches give the factor that
    turns counter readings into bytes."""
    import torch
    src = torch.full((COPY_BYTES // 4,), 1.0, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": reps}), flush=True)
    return 0


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def _threads():
    import threadpoolctl
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()]
    return max(blas) if blas else 1


def cpu_baseline_decode(spec, dc, seqs, budget_s: float = 10.0):
    """The fp64 oracle timed on this host on the decode workload: whole layer
    groups (append, scoring over every visible entry, Top-K, attention) for
    the sequences in `seqs`, once with every core and once on a single
    thread.  When `seqs` is every sequence of the workload the step is timed
    in full, one pass each; otherwise the sample is repeated until the budget
    is spent.  Set-up (the oracle's encoding of the cached indexer-K rows, and
    of the main-KV rows the group selects, found by an untimed pass) is
    outside the timing, as the GPU's resident cache is."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import csa2_oracle as O

    layer_in = [tuple(x.cpu().numpy() for x in li) for li in dc.inputs]
    cases = []
    for s in seqs:
        vis = spec.seq_len_after(s)
        c = spec.cached[s]
        ps = 64
        npg = (vis + ps - 1) // ps
        cache = O.Cache.empty(npg, ps, np.arange(npg, dtype=np.int32)[None], [vis])
        ik = W.idxk_rows(spec, s, "cuda").cpu().numpy().view(np.uint16)
        flat = cache.idx_k.reshape(-1, 128)
        for a in range(0, vis, 1 << 18):
            b = min(vis, a + (1 << 18))
            flat[a:b] = O.quantize_idxk_rows(O.bf16_to_f64(ik[a:b]))
        kv_all = W.kv_rows(spec, s, "cuda")
        new_kv = kv_all[c:c + spec.n_new].cpu().numpy().view(np.uint16)
        new_ik = ik[c:c + spec.n_new]
        # untimed pass: the rows the group selects get their main-KV rows
        rows = set(range(c, c + spec.n_new))
        for li, mode in enumerate(spec.modes):
            if mode == O.REUSE:
                continue
            qi, w, _ = layer_in[li]
            sc = O.index_scores(cache, 0, vis, qi[s], w[s])
            sel, cnt = O.select_topk(sc, spec.k)
            rows |= set(sel[:cnt].tolist())
        rows = np.array(sorted(rows), dtype=np.int64)
        cache.kv.reshape(-1, 272)[rows] = O.quantize_kv_rows(
            O.bf16_to_f64(kv_all[torch_index(rows, kv_all.device)].cpu().numpy().view(np.uint16)))
        cases.append((s, cache, new_kv, new_ik, c, vis))
    del kv_all

    def one_group(s, cache, new_kv, new_ik, c, vis):
        idx = cnt = None
        for li, mode in enumerate(spec.modes):
            qi, w, q = layer_in[li]
            if mode == O.REUSE:
                args = dict(idx=idx, cnt=cnt)
            else:
                args = dict(q_idx=qi[s:s + 1], w=w[s:s + 1])
            if mode == O.FULL and spec.n_new:
                args.update(new_slots=np.arange(c, c + spec.n_new), new_kv=new_kv, new_idxk=new_ik)
            i2, c2, _, _ = O.layer_step(mode, cache, q[s:s + 1].view(np.uint16), [0], [vis], spec.k,
                                        spec.sm_scale, **args)
            if mode == O.FULL:
                idx, cnt = i2, c2

    full = len(seqs) == spec.num_seqs

    def timed(limit):
        with threadpoolctl.threadpool_limits(limit):
            threads = _threads()
            tokens = 0
            t0 = time.perf_counter()
            while True:
                for case in cases:
                    one_group(*case)
                    tokens += max(1, spec.n_new)
                el = time.perf_counter() - t0
                if full or el >= budget_s:
                    return tokens / el, tokens, el, threads

    v_all, n_all, t_all, th_all = timed(None)
    v_one, n_one, t_one, _ = timed(1)
    lens = [spec.seq_len_after(s) for s in seqs]
    mean_len = sum(spec.seq_len_after(s) for s in range(spec.num_seqs)) / spec.num_seqs
    what = (f"the whole step: all {spec.num_seqs} sequences (visible entries {min(lens)}..{max(lens)}) x the "
            f"{len(spec.modes)}-layer group, one pass" if full else
            f"sequences {list(seqs)} of {spec.num_seqs} (visible entries {lens}; workload mean {mean_len:.0f}) x "
            f"the whole {len(spec.modes)}-layer group")
    return {"value": v_all, "unit": "tokens/s", "cores": int(th_all), "kind": "oracle",
            "sample": f"{what}, {n_all} sequence-steps in {t_all:.1f} s (fp64 NumPy, host cores "
                      f"{len(os.sched_getaffinity(0))})",
            "single_thread": {"value": v_one, "unit": "tokens/s", "cores": 1,
                              "sample": f"the same, {n_one} sequence-steps in {t_one:.1f} s"}}


def torch_index(rows, device):
    import torch
    return torch.from_numpy(rows).to(device)


def cpu_baseline_prefill(spec, dc, budget_s: float = 10.0):
    """The fp64 oracle on a bounded sample of the prefill step: the append of
    all new rows once, then index + select + attend for evenly spaced query
    rows (first and last included) until the budget is spent; the step time
    is extrapolated linearly to every row.  Every core, then one thread."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import csa2_oracle as O

    vis_all = spec.q_vis()
    ps = 64
    npg = (int(vis_all.max()) + ps - 1) // ps
    cache = O.Cache.empty(npg, ps, np.arange(npg, dtype=np.int32)[None], [spec.seq_len_after(0)])
    c = spec.cached[0]
    kv = W.kv_rows(spec, 0, "cuda").cpu().numpy().view(np.uint16)
    ik = W.idxk_rows(spec, 0, "cuda").cpu().numpy().view(np.uint16)
    O.append_quant_fp4(cache, np.arange(c), kv[:c], ik[:c])
    qi, w, q = (x.cpu().numpy() for x in dc.inputs[0])
    q = q.view(np.uint16)
    rows = np.unique(np.linspace(0, spec.nq - 1, 64).round().astype(np.int64))

    def timed(limit):
        with threadpoolctl.threadpool_limits(limit):
            threads = _threads()
            t0 = time.perf_counter()
            O.append_quant_fp4(cache, np.arange(c, c + spec.n_new), kv[c:], ik[c:])
            t_append = time.perf_counter() - t0
            done = 0
            t0 = time.perf_counter()
            while True:
                i = int(rows[done % len(rows)])
                O.layer_step(O.REINDEX, cache, q[i:i + 1], [0], [int(vis_all[i])], spec.k, spec.sm_scale,
                             q_idx=qi[i:i + 1], w=w[i:i + 1])
                done += 1
                el = time.perf_counter() - t0
                if el >= budget_s and done >= len(rows):
                    break
            step_s = t_append + el / done * spec.nq
            return spec.nq / step_s, t_append, done, el, threads

    v_all, ta, d_all, e_all, th = timed(None)
    v_one, ta1, d_one, e_one, _ = timed(1)
    return {"value": v_all, "unit": "tokens/s", "cores": int(th), "kind": "oracle",
            "sample": f"append of all {spec.n_new} rows ({ta:.2f} s) + {d_all} query rows of {spec.nq} "
                      f"(64 evenly spaced incl. first and last) in {e_all:.1f} s, extrapolated linearly to "
                      f"{spec.nq} rows (fp64 NumPy, host cores {len(os.sched_getaffinity(0))})",
            "single_thread": {"value": v_one, "unit": "tokens/s", "cores": 1,
                              "sample": f"the same: append {ta1:.2f} s + {d_one} rows in {e_one:.1f} s, "
                                        f"extrapolated"}}


# ---------------------------------------------------------------------------
# decode workloads
# ---------------------------------------------------------------------------

def time_hierarchical(dc, pool_k: int, steps: int):
    """The decode group with the hierarchical indexer: the Full layer keeps its
    Top-pool_k as the pool and the Reindex layer scores only the pool
    (per-layer calls, device timestamps on the pool kernels).  Also reports
    how much of each Reindex layer's exhaustive Top-k the pooled one keeps."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    from fp4_kv_cache_layer_amd import _lib as L
    spec = dc.spec
    reindex = [li for li, m in enumerate(spec.modes) if m == ops.REINDEX]
    dc.run_layers()
    torch.cuda.synchronize()
    exhaustive = {li: (dc.outputs[li]["idx"].cpu().numpy(), dc.outputs[li]["cnt"].cpu().numpy()) for li in reindex}
    pool, pool_cnt = dc.new_pool(pool_k)
    calls = [dc.make_call(li, dc.ws, pool, pool_cnt) for li in range(len(spec.modes))]

    def step():
        for c in calls:
            c()
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    n_pool = len(reindex) + 1
    tm = ops.Timing({L.KCLASS_POOL_SCAN: steps * n_pool, L.KCLASS_POOL_SELECT: steps * n_pool,
                     L.KCLASS_SCAN: steps, L.KCLASS_SELECT: steps})
    for c in calls:
        c.set_timing(tm)
    for _ in range(steps):
        step()
    for c in calls:
        c.set_timing(None)
    kept = []
    for li in reindex:
        ei, ec = exhaustive[li]
        gi, gc = dc.outputs[li]["idx"].cpu().numpy(), dc.outputs[li]["cnt"].cpu().numpy()
        inter = sum(len(set(a[:x].tolist()) & set(b[:y].tolist())) for a, x, b, y in zip(ei, ec, gi, gc))
        kept.append(round(inter / max(1, int(ec.sum())), 4))
    scan_us = statistics.mean(tm.durations_ms(L.KCLASS_POOL_SCAN)) * 1e3
    pb = pool_scan_bytes(spec.nq, pool_k, spec.h_idx)
    return {"pool_k": pool_k, "execution": "one csa2_layer_step call per layer, back to back (cache-assisted)",
            "ms_per_step": round(ms, 5),
            "tokens_per_s": round(spec.num_seqs * spec.n_new / (ms / 1e3), 1),
            "kernels_avg_us": {"scan_full": _avg_us(tm.durations_ms(L.KCLASS_SCAN)),
                               "select_full_top_pool_k": _avg_us(tm.durations_ms(L.KCLASS_SELECT)),
                               "pool_scan": round(scan_us, 2),
                               "pool_select": _avg_us(tm.durations_ms(L.KCLASS_POOL_SELECT))},
            "pool_scan_bytes_per_launch": pb, "pool_scan_GBps": round(pb / (scan_us / 1e6) / 1e9, 1),
            "reindex_topk_kept_vs_exhaustive": kept,
            "entries_scored_per_query": {"exhaustive": int(spec.q_vis().max()), "pool": pool_k}}


def time_block_pruning(spec, steps: int, scrub):
    """Block-level pruning (CSA2_STEP_PRUNE) on the decode group: the bench's
    own N(0,1) inputs and the same shape with clustered indexer-K rows (each
    64-entry block near a centre of its own).  Each Full and Reindex layer's
    seed is its selection of the previous step (same queries: the most a seed
    can prune).  Scrubbed steps, per-layer calls, with and without the flag;
    the selections must be identical."""
    import dataclasses

    import torch

    from fp4_kv_cache_layer_amd import ops, runner
    from fp4_kv_cache_layer_amd import _lib as L
    n_scan = sum(1 for m in spec.modes if m != ops.REUSE)
    res = {"seed": "each Full / Reindex layer's own selection of the previous step (same queries)",
           "execution": "one csa2_layer_step call per layer, a 512 MiB cache scrub before every step"}
    for name, sp in (("bench_inputs", spec), ("clustered_inputs", dataclasses.replace(spec, clustered=True))):
        row = {}
        sel = {}
        for prune in (False, True):
            dc = runner.DeviceCase(sp, gen_device="cuda", prune=prune)
            dc.run_layers()                                  # first step: empty seeds, nothing pruned
            scrubbed_steps(dc.run_layers, 2, scrub)
            tm = ops.Timing({L.KCLASS_SCAN: steps * n_scan})
            dc.set_timing(tm)
            ms = statistics.mean(scrubbed_steps(dc.run_layers, steps, scrub))
            dc.set_timing(None)
            scan = tm.durations_ms(L.KCLASS_SCAN)
            entry = {"ms_per_step": round(ms, 5), "scan_us": _avg_us(scan),
                     "scan_full_us": _avg_us(scan[0::n_scan]),
                     "scan_reindex_us": _avg_us(scan[1::n_scan]) if n_scan > 1 else None}
            if prune:
                fr = []
                for li, c in enumerate(dc.calls):             # one more step, masks read after each indexer layer
                    c()
                    if sp.modes[li] != ops.REUSE:
                        fr.append(round(ops.pruned_block_fraction(ops.workspace_prune_masks(dc.ws, sp.nq, dc.max_vis),
                                                                  sp.q_vis()), 4))
                entry["pruned_block_fraction"] = fr
                entry["scan_includes"] = "prune_mask_kernel + index_scan_kernel"
            torch.cuda.synchronize()
            sel[prune] = [o["idx"].cpu() for o in dc.outputs]
            row["pruned" if prune else "plain"] = entry
            del dc
            torch.cuda.empty_cache()
        row["identical_selection"] = all(torch.equal(a, b) for a, b in zip(sel[False], sel[True]))
        row["step_speedup"] = round(row["plain"]["ms_per_step"] / row["pruned"]["ms_per_step"], 3)
        res[name] = row
    return res


def cpu_sample_seqs(spec, n: int):
    """Sequences for the CPU baseline: the n whose lengths are closest to the
    workload's mean length (all equal for the uniform workloads)."""
    lens = [spec.seq_len_after(s) for s in range(spec.num_seqs)]
    mean = sum(lens) / len(lens)
    return sorted(sorted(range(spec.num_seqs), key=lambda s: (abs(lens[s] - mean), s))[:n])


def bench_decode(args, cfg, spec) -> int:
    import torch

    import workloads as W  # noqa: F401
    from fp4_kv_cache_layer_amd import ops, runner
    from fp4_kv_cache_layer_amd import _lib as L

    print(f"[bench] building {spec.name}", file=sys.stderr, flush=True)
    multi = len(spec.modes) > 1
    dc = runner.DeviceCase(spec, gen_device="cuda", group=1 if multi else 0)
    step = dc.run_layers
    n_scan = sum(1 for m in spec.modes if m != ops.REUSE)
    n_layers = len(spec.modes)
    scrub = Scrubber()
    torch.cuda.synchronize()

    # warm-up steps, scrubbed like the timed ones
    scrubbed_steps(step, args.warmup, scrub)

    # ---- timed region (graded): K scrubbed steps, scan launches timestamped ----
    tm = ops.Timing({L.KCLASS_SCAN: args.steps * n_scan})
    dc.set_timing(tm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = scrubbed_steps(step, args.steps, scrub)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    dc.set_timing(None)
    scan_ms = tm.durations_ms(L.KCLASS_SCAN)

    ms = statistics.mean(step_ms)
    tokens = spec.num_seqs * max(1, spec.n_new)
    value = tokens / (ms / 1e3)
    sbytes = scan_bytes(spec)
    scan_avg_s = statistics.mean(scan_ms) / 1e3
    achieved = sbytes / scan_avg_s / 1e9
    gb = group_bytes(spec)
    modes = ",".join(W_MODE[m] for m in spec.modes)
    out = {
        "metric": METRICS[cfg],
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "global_batch": spec.num_seqs,
                   "seq_len": (spec.cached[0] + spec.n_new) if len(set(spec.cached)) == 1 else "ragged",
                   "visible_entries_total": int(spec.q_vis().sum()), "modes": modes, "topk": spec.k,
                   "heads": spec.h, "indexer_heads": spec.h_idx, "page_size": spec.page_size,
                   "execution": "one csa2_layer_step call per layer, a 512 MiB cache scrub before every step",
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "index_scan_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(args.traffic, spec.name, "index_scan.hip"),
                     "bytes_per_launch": sbytes, "avg_launch_us": round(scan_avg_s * 1e6, 2),
                     "launches": len(scan_ms),
                     "scan_full_us": _avg_us(scan_ms[0::n_scan]),
                     "scan_reindex_us": _avg_us(scan_ms[1::n_scan]) if n_scan > 1 else None},
        "group_bytes": gb,
        "group_hbm_frac": round(gb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "timed_region_wall_ms": round(wall_ms, 3),
        "step_ms_percentiles": percentiles(step_ms),
    }
    if args.only_timed:
        out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return 0

    # ---- cache-assisted: the same steps back to back ----
    tmw = ops.Timing({L.KCLASS_SCAN: args.steps * n_scan})
    dc.set_timing(tmw)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_warm = (time.perf_counter() - t0) * 1e3 / args.steps
    dc.set_timing(None)
    warm_scan = tmw.durations_ms(L.KCLASS_SCAN)
    out["cache_assisted"] = {
        "note": "back-to-back steps: the Infinity Cache still holds part of the indexer-K",
        "ms_per_step": round(ms_warm, 5), "tokens_per_s": round(tokens / (ms_warm / 1e3), 1),
        "scan_avg_us": _avg_us(warm_scan),
        "scan_frac": round(sbytes / (statistics.mean(warm_scan) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "group_hbm_frac": round(gb / (ms_warm / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- breakdown (scrubbed): every kernel class timestamped ----
    tmb = ops.Timing({L.KCLASS_APPEND: args.steps, L.KCLASS_SCAN: args.steps * n_scan,
                      L.KCLASS_SELECT: args.steps * n_scan, L.KCLASS_ATTN: args.steps * n_layers})
    dc.set_timing(tmb)
    scrubbed_steps(step, args.steps, scrub)
    dc.set_timing(None)
    sel = tmb.durations_ms(L.KCLASS_SELECT)
    att = tmb.durations_ms(L.KCLASS_ATTN)
    out["kernels_avg_us"] = {"append": _avg_us(tmb.durations_ms(L.KCLASS_APPEND)),
                             "scan": _avg_us(tmb.durations_ms(L.KCLASS_SCAN)),
                             "select": _avg_us(sel), "attn": _avg_us(att)}
    ab = attn_bytes(spec)
    out["attention"] = {"bytes_per_layer": ab, "avg_us": _avg_us(att),
                        "hbm_frac": round(ab / (statistics.mean(att) / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- the whole group captured in one HIP graph, replayed per step (scrubbed) ----
    dc.capture_graph()
    scrubbed_steps(dc.replay_graph, 2, scrub)
    g_ms = statistics.mean(scrubbed_steps(dc.replay_graph, args.steps, scrub))
    out["graph"] = {"execution": "one HIP graph replay per step (the per-layer calls captured in order)",
                    "ms_per_step": round(g_ms, 5), "tokens_per_s": round(tokens / (g_ms / 1e3), 1)}

    # ---- group step: Reuse attentions on an auxiliary stream (independent inputs only) ----
    if multi:
        for _ in range(3):
            dc.run_group()
        gs = statistics.mean(scrubbed_steps(dc.run_group, args.steps, scrub))
        out["group_step"] = {"execution": "csa2_group_step, Reuse attentions on 1 auxiliary stream "
                                          "(valid only for independent layer inputs)",
                             "ms_per_step": round(gs, 5), "tokens_per_s": round(tokens / (gs / 1e3), 1)}

    cold, warm = measured_hbm_read(sbytes)
    out["roofline"].update({"peak_measured": round(cold, 1), "frac_of_measured": round(achieved / cold, 4),
                            "measured_by": "csa2_probe_stream_read: plain streaming read of the same byte count "
                                           "over successive slices of a 2 GiB buffer (cold)",
                            "stream_read_warm_GBps": round(warm, 1)})
    out["lse_merge"] = time_lse_merge(dc.outputs[0]["out"], dc.outputs[0]["lse"])
    if args.pool_k and ops.REINDEX in spec.modes and cfg == 1:
        out["hierarchical_indexer"] = time_hierarchical(dc, args.pool_k, args.steps)
    if args.prune and cfg == 1:
        print("[bench] block pruning variant", file=sys.stderr, flush=True)
        out["block_pruning"] = time_block_pruning(spec, args.steps, scrub)
    if not args.no_cpu_baseline:
        # the 64K decode group in full (about 10 s of oracle work per pass);
        # the 1M and ragged workloads (minutes per pass) on a bounded sample
        seqs = list(range(spec.num_seqs)) if cfg == 1 else cpu_sample_seqs(spec, 1 if cfg == 3 else 2)
        print(f"[bench] timing the CPU oracle on {len(seqs)} of {spec.num_seqs} sequences", file=sys.stderr,
              flush=True)
        out["cpu_baseline"] = cpu_baseline_decode(spec, dc, seqs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


W_MODE = {0: "full", 1: "reindex", 2: "reuse"}


# ---------------------------------------------------------------------------
# prefill workload
# ---------------------------------------------------------------------------

def bench_prefill(args, spec) -> int:
    """One step = one Full layer over the prefill chunk: append of the new
    rows, dense indexer, Top-K, attention.  The dominant contraction is the
    dense indexer's candidate kernel (FP8 MFMA); the roofline is reported on it."""
    import torch

    from fp4_kv_cache_layer_amd import ops, runner
    from fp4_kv_cache_layer_amd import _lib as L

    print(f"[bench] building {spec.name}", file=sys.stderr, flush=True)
    dc = runner.DeviceCase(spec, gen_device="cuda")
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        dc.run_layers()
    tm = ops.Timing({L.KCLASS_DENSE: args.steps})
    dc.set_timing(tm)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dc.run_layers()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dc.set_timing(None)
    prod_ms = tm.durations_ms(L.KCLASS_DENSE)
    flops = dense_flops(spec)
    prod_avg_s = statistics.mean(prod_ms) / 1e3
    achieved = flops / prod_avg_s / 1e12
    out = {
        "metric": METRICS[2],
        "value": round(spec.nq / (ms / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+bf16",
        "data": "synthetic",
        "config": {"workload": spec.name, "global_batch": 1, "seq_len": spec.cached[0] + spec.n_new,
                   "prefill_rows": spec.nq, "modes": "full", "topk": spec.k, "heads": spec.h,
                   "indexer_heads": spec.h_idx, "parallelism": "single-gpu"},
        "roofline": {"bound": "mfma", "kernel": "prefill_scan_kernel", "achieved": round(achieved, 1),
                     "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic(os.path.join(ROOT, "profiles", "prefill_scan_traffic.json"),
                                               spec.name, "prefill_scan.hip"),
                     "flop_per_launch": flops, "avg_launch_us": round(prod_avg_s * 1e6, 2)},
    }
    if args.only_timed:
        out["cpu_baseline"] = None
        print(json.dumps(out), flush=True)
        return 0
    classes = (L.KCLASS_APPEND, L.KCLASS_SCAN, L.KCLASS_SELECT, L.KCLASS_ATTN, L.KCLASS_DENSE)
    tmb = ops.Timing({c: args.steps for c in classes})
    dc.set_timing(tmb)
    for _ in range(args.steps):
        dc.run_layers()
    dc.set_timing(None)
    index_s = statistics.mean(tmb.durations_ms(L.KCLASS_SCAN)) / 1e3
    attn_s = statistics.mean(tmb.durations_ms(L.KCLASS_ATTN)) / 1e3
    ab = attn_bytes(spec)
    mf_peak, mf_epi = measured_mfma_fp8()
    out["roofline"].update({
        "peak_measured": round(mf_peak, 1), "frac_of_measured": round(achieved / mf_peak, 4),
        "measured_by": "csa2_probe_mfma_fp8: back-to-back 16x16x128 FP8 MFMAs, 4 waves per SIMD",
        "epilogue_ceiling": {"achieved": round(mf_epi, 1), "frac": round(mf_epi / FP8_PEAK_TFLOPS, 4),
                             "measured_by": "csa2_probe_mfma_fp8 with the per-score ReLU, head-weight fma and "
                                            "add beside each MFMA"}})
    out["indexer_all_kernels"] = {"avg_us": round(index_s * 1e6, 2),
                                  "mfma_frac": round(flops / index_s / 1e12 / FP8_PEAK_TFLOPS, 4)}
    out["attention"] = {"avg_us": round(attn_s * 1e6, 2), "bytes": ab, "GBps": round(ab / attn_s / 1e9, 1),
                        "hbm_frac": round(ab / attn_s / 1e9 / HBM_PEAK_GBS, 4)}
    out["kernels_avg_us"] = {"append": _avg_us(tmb.durations_ms(L.KCLASS_APPEND)),
                             "indexer": _avg_us(tmb.durations_ms(L.KCLASS_SCAN)),
                             "indexer_product": _avg_us(tmb.durations_ms(L.KCLASS_DENSE)),
                             "select": _avg_us(tmb.durations_ms(L.KCLASS_SELECT)),
                             "attn": _avg_us(tmb.durations_ms(L.KCLASS_ATTN))}
    out["lse_merge"] = time_lse_merge(dc.outputs[0]["out"], dc.outputs[0]["lse"])
    # the QAT forward on the chunk's attention output (fp32) and on its bf16 copy
    out["fake_quant_f32"] = time_fake_quant(dc.outputs[0]["out"])
    out["fake_quant_bf16"] = time_fake_quant(dc.outputs[0]["out"].to(torch.bfloat16))
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_prefill(spec, dc)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=(1, 2, 3, 4))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-timed", action="store_true",
                    help="run the warm-up and the timed region only (no breakdown, variants or baseline)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "scan_traffic.json"),
                    help="HBM traffic per scan launch measured with rocprofv3 counters (optional)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pool-k", type=int, default=2048,
                    help="pool width of the hierarchical-indexer variant timed beside workload 1 (0: skip)")
    ap.add_argument("--no-prune", dest="prune", action="store_false",
                    help="skip the block-pruning variant timed beside workload 1")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        return 2
    if args.copy_calibration:
        return copy_calibration()

    import torch

    import workloads as W
    from fp4_kv_cache_layer_amd import _lib

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    _lib.load()
    spec = W.config(args.config)
    if spec.prefill:
        return bench_prefill(args, spec)
    return bench_decode(args, args.config, spec)


if __name__ == "__main__":
    sys.exit(main())
