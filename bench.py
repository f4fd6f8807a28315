"""CSA2 decode benchmark on one MI355X.

One step = one CSA2 layer group (Full, Reindex, Reuse, Reuse) over a batch of
32 decode sequences with 65,536 cached entries each plus one entry appended
by quantize-on-append (indexer 8 x 128 FP8, 64 heads over the 512-wide FP4
latent, Top-512), as one csa2_layer_step call per layer in layer order: in a
model each layer's queries depend on the previous layer's output, so this is
the schedule a real decode step can run (the group step, which overlaps the
Reuse layers' attention with the next layers, is timed beside it).  Inputs
are synthetic, seeded, and already resident in HBM when timing starts.
Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --config 2             # causal prefill of 4,096 rows against
                                           # 65,536 cached: one Full layer, dense
                                           # FP8 indexer, MFMA roofline
    python bench.py --copy-calibration     # plain device copy of known size, for
                                           # scaling rocprofv3 FETCH_SIZE/WRITE_SIZE
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
METRIC = "CSA2 decode tokens/s (B=32, 64K ctx) + % of HBM roofline"
PREFILL_METRIC = "CSA2 prefill tokens/s (4,096 rows vs 64K ctx) + % of FP8 MFMA roofline (dense indexer)"


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
    """Algorithmic bytes of one attention layer: k gathered rows (272 B) and
    their indices per query, bf16 Q, fp32 O and LSE."""
    return spec.nq * (spec.k * 272 + spec.k * 4 + spec.h * 512 * 2 + spec.h * 512 * 4 + spec.h * 4)


def merge_bytes(rows: int, dim: int = 512) -> int:
    """Algorithmic bytes of one branch merge: both branches' outputs and LSEs
    in, the merged output and LSE out."""
    return rows * (3 * dim * 4 + 3 * 4)


def time_lse_merge(o_a, lse_a, reps: int = 20):
    """Times csa2_lse_merge of the CSA2 output with a synthetic local-branch
    output of the same shape (device timestamps of the merge's dispatches)."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    from fp4_kv_cache_layer_amd import _lib as L
    g = torch.Generator(device="cuda").manual_seed(5)
    o_b = torch.randn(o_a.shape, generator=g, device="cuda", dtype=torch.float32)
    lse_b = torch.randn(lse_a.shape, generator=g, device="cuda", dtype=torch.float32) * 4
    out, lse = torch.empty_like(o_a), torch.empty_like(lse_a)
    for _ in range(3):
        ops.csa2_lse_merge(o_a, lse_a, o_b, lse_b, out, lse)
    ring = ops.TimingRing(L.KCLASS_MERGE, reps)
    ring.install()
    for _ in range(reps):
        ops.csa2_lse_merge(o_a, lse_a, o_b, lse_b, out, lse)
    ring.uninstall()
    avg_s = statistics.mean(ring.durations_ms()) / 1e3
    rows = lse_a.numel()
    b = merge_bytes(rows, o_a.shape[-1])
    return {"kernel": "lse_merge_kernel", "rows": rows, "dim": int(o_a.shape[-1]), "bytes": b,
            "avg_us": round(avg_s * 1e6, 2), "GBps": round(b / avg_s / 1e9, 1),
            "hbm_frac": round(b / avg_s / 1e9 / HBM_PEAK_GBS, 4)}


def time_fake_quant(x, reps: int = 10):
    """Times csa2_fake_quant_fp4 on x (device timestamps of its dispatches);
    algorithmic bytes = x read once and its quantised copy written once."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    from fp4_kv_cache_layer_amd import _lib as L
    out = torch.empty_like(x)
    for _ in range(2):
        ops.csa2_fake_quant_fp4(x, out)
    ring = ops.TimingRing(L.KCLASS_QUANT, reps)
    ring.install()
    for _ in range(reps):
        ops.csa2_fake_quant_fp4(x, out)
    ring.uninstall()
    avg_s = statistics.mean(ring.durations_ms()) / 1e3
    b = 2 * x.numel() * x.element_size()
    return {"kernel": "fake_quant_" + ("bf16" if x.element_size() == 2 else "f32") + "_kernel",
            "values": x.numel(), "bytes": b, "avg_us": round(avg_s * 1e6, 2), "GBps": round(b / avg_s / 1e9, 1),
            "hbm_frac": round(b / avg_s / 1e9 / HBM_PEAK_GBS, 4)}


def pool_scan_bytes(nq: int, pool_k: int, h_idx: int) -> int:
    """Algorithmic bytes of one pool-scoring launch: each query's pool indices
    (4 B) and gathered indexer-K rows (128 B), its indexer query and weights,
    and the pool scores written (4 B each)."""
    return nq * (pool_k * (4 + 128 + 4) + h_idx * (128 + 4))


def time_hierarchical(dc, pool_k: int, steps: int):
    """The decode group with the hierarchical indexer: the Full layer keeps its
    Top-pool_k as the pool and the Reindex layer scores only the pool
    (per-layer calls, device timestamps on the pool kernels).  Also reports
    how much of each Reindex layer's exhaustive Top-k the pooled one keeps."""
    import numpy as np
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
    rings = {c: ops.TimingRing(c, steps * n_pool) for c in (L.KCLASS_POOL_SCAN, L.KCLASS_POOL_SELECT)}
    rings[L.KCLASS_SCAN] = ops.TimingRing(L.KCLASS_SCAN, steps)
    rings[L.KCLASS_SELECT] = ops.TimingRing(L.KCLASS_SELECT, steps)
    for r in rings.values():
        r.install()
    for _ in range(steps):
        step()
    for r in rings.values():
        r.uninstall()
    dur = {c: r.durations_ms() for c, r in rings.items()}
    group_ms = None
    if dc.group_ws is not None:
        # the same group as one csa2_group_step, Reuse attentions on an auxiliary stream
        gcall = ops.GroupCall([dc.make_call(li, dc.group_ws[li], pool, pool_cnt) for li in range(len(spec.modes))],
                              n_aux=1)
        for _ in range(3):
            gcall()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            gcall()
        torch.cuda.synchronize()
        group_ms = (time.perf_counter() - t0) * 1e3 / steps
    kept = []
    for li in reindex:
        ei, ec = exhaustive[li]
        gi, gc = dc.outputs[li]["idx"].cpu().numpy(), dc.outputs[li]["cnt"].cpu().numpy()
        inter = sum(len(set(a[:x].tolist()) & set(b[:y].tolist())) for a, x, b, y in zip(ei, ec, gi, gc))
        kept.append(round(inter / max(1, int(ec.sum())), 4))
    scan_us = statistics.mean(dur[L.KCLASS_POOL_SCAN]) * 1e3
    pb = pool_scan_bytes(spec.nq, pool_k, spec.h_idx)
    return {"pool_k": pool_k, "execution": "one csa2_layer_step call per layer",
            "ms_per_step_no_events": round(ms, 5),
            "tokens_per_s": round(spec.num_seqs * spec.n_new / (ms / 1e3), 1),
            "group_step": (None if group_ms is None else
                           {"execution": "csa2_group_step, Reuse attentions on 1 auxiliary stream",
                            "ms_per_step_no_events": round(group_ms, 5),
                            "tokens_per_s": round(spec.num_seqs * spec.n_new / (group_ms / 1e3), 1)}),
            "kernels_avg_us": {"scan_full": round(statistics.mean(dur[L.KCLASS_SCAN]) * 1e3, 2),
                               "select_full_top_pool_k": round(statistics.mean(dur[L.KCLASS_SELECT]) * 1e3, 2),
                               "pool_scan": round(scan_us, 2),
                               "pool_select": round(statistics.mean(dur[L.KCLASS_POOL_SELECT]) * 1e3, 2)},
            "pool_scan_bytes_per_launch": pb, "pool_scan_GBps": round(pb / (scan_us / 1e6) / 1e9, 1),
            "reindex_topk_kept_vs_exhaustive": kept,
            "entries_scored_per_query": {"exhaustive": int(spec.q_vis().max()), "pool": pool_k}}


def measured_hbm_read(nbytes: int):
    """Measured HBM read rates (GB/s) of a plain streaming-read kernel over
    nbytes: warm (the same buffer every launch, as the timed region reads the
    same indexer-K every step) and cold (successive slices of a buffer far
    larger than the 256 MB last-level cache)."""
    import torch

    from fp4_kv_cache_layer_amd import probe

    nb = (nbytes + 15) // 16 * 16
    rot = 8
    buf = torch.ones(rot * nb, dtype=torch.uint8, device="cuda")
    warm = probe.stream_read_gbps(buf, nb, rotate=1)
    cold = probe.stream_read_gbps(buf, nb, rotate=rot)
    del buf
    torch.cuda.empty_cache()
    return warm, cold


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


def scan_source_hash() -> str:
    return source_hash("index_scan.hip")


def stored_traffic(path: str, workload: str, src_name: str):
    """HBM bytes per launch from a stored rocprofv3 FETCH_SIZE/WRITE_SIZE
    reading, or None when it is missing or was taken on other source."""
    try:
        tr = json.load(open(path))
        if tr.get("workload") == workload and tr.get("kernel_source_sha256_16") == source_hash(src_name):
            return tr.get("bytes_per_launch")
    except Exception:
        pass
    return None


COPY_BYTES = 1 << 30
SCRUB_BYTES = 512 << 20


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


def cpu_baseline(spec, dc, budget_s: float = 12.0):
    """The fp64 oracle timed on this host on a bounded sample of the same
    workload: whole layer groups for a few sequences, repeated until the
    budget is spent.  Cache encoding is set-up, outside the timing, as the
    GPU's resident cache is."""
    import numpy as np
    import threadpoolctl

    import workloads as W
    from oracle import csa2_oracle as O

    seqs = [0, 1]
    caches = {}
    for s in seqs:
        vis = spec.seq_len_after(s)
        ps = 64
        npg = (vis + ps - 1) // ps
        cache = O.Cache.empty(npg, ps, np.arange(npg, dtype=np.int32)[None], [vis])
        c = spec.cached[s]
        kv = W.kv_rows(spec, s, "cuda").cpu().numpy().view(np.uint16)
        ik = W.idxk_rows(spec, s, "cuda").cpu().numpy().view(np.uint16)
        O.append_quant_fp4(cache, np.arange(c), kv[:c], ik[:c])
        caches[s] = (cache, kv[c:c + spec.n_new], ik[c:c + spec.n_new], c)
    layer_in = [tuple(x.cpu().numpy() for x in li) for li in dc.inputs]
    tokens = 0
    t0 = time.perf_counter()
    while True:
        for s in seqs:
            cache, nkv, nik, c = caches[s]
            idx = cnt = None
            for li, mode in enumerate(spec.modes):
                qi, w, q = layer_in[li]
                args = dict(q_idx=qi[s:s + 1], w=w[s:s + 1]) if mode != O.REUSE else dict(idx=idx, cnt=cnt)
                if mode == O.FULL:
                    args.update(new_slots=np.arange(c, c + spec.n_new), new_kv=nkv, new_idxk=nik)
                i2, c2, _, _ = O.layer_step(mode, cache, q[s:s + 1].view(np.uint16), [0], [spec.seq_len_after(s)],
                                            spec.k, spec.sm_scale, **args)
                if mode == O.FULL:
                    idx, cnt = i2, c2
            tokens += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()]
    cores = max(blas) if blas else 1
    return {"value": tokens / el, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(seqs)} of {spec.num_seqs} sequences x full 4-layer group, {tokens} sequence-steps "
                      f"in {el:.1f} s (fp64 NumPy, host cores {len(os.sched_getaffinity(0))})"}


def cpu_baseline_prefill(spec, dc, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample of the prefill step: the append of
    all new rows once, then index + select + attend for evenly spaced query
    rows (first and last included) until the budget is spent; the step time is
    extrapolated linearly to every row."""
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
    t0 = time.perf_counter()
    O.append_quant_fp4(cache, np.arange(c, c + spec.n_new), kv[c:], ik[c:])
    t_append = time.perf_counter() - t0
    rows = np.unique(np.linspace(0, spec.nq - 1, 64).round().astype(np.int64))
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
    per_row = el / done
    step_s = t_append + per_row * spec.nq
    blas = [p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()]
    cores = max(blas) if blas else 1
    return {"value": spec.nq / step_s, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"append of all {spec.n_new} rows ({t_append:.2f} s) + {done} query rows of {spec.nq} "
                      f"(64 evenly spaced incl. first and last) in {el:.1f} s, extrapolated linearly to "
                      f"{spec.nq} rows (fp64 NumPy, host cores {len(os.sched_getaffinity(0))})"}


def bench_prefill(args, spec, dc) -> int:
    """One step = one Full layer over the prefill chunk: append of the new
    rows, dense indexer, Top-K, attention.  The dominant contraction is the
    dense indexer's candidate kernel (FP8 MFMA); the roofline is reported on it."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    from fp4_kv_cache_layer_amd import _lib as L

    for _ in range(args.warmup):
        dc.run_group()
    torch.cuda.synchronize()
    ring = ops.TimingRing(L.KCLASS_DENSE, args.steps)
    ring.install()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dc.run_group()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ring.uninstall()
    prod_ms = ring.durations_ms()

    classes = (L.KCLASS_APPEND, L.KCLASS_SCAN, L.KCLASS_SELECT, L.KCLASS_ATTN, L.KCLASS_DENSE)
    rings = {k: ops.TimingRing(k, args.steps) for k in classes}
    for r in rings.values():
        r.install()
    for _ in range(args.steps):
        dc.run_group()
    for r in rings.values():
        r.uninstall()
    dur = {k: r.durations_ms() for k, r in rings.items()}

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dc.run_group()
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / args.steps

    def avg(xs):
        return round(statistics.mean(xs) * 1e3, 2) if xs else None

    mf_peak, mf_epi = measured_mfma_fp8()
    flops = dense_flops(spec)
    prod_avg_s = statistics.mean(prod_ms) / 1e3
    achieved = flops / prod_avg_s / 1e12
    index_s = statistics.mean(dur[L.KCLASS_SCAN]) / 1e3
    ab = attn_bytes(spec)
    attn_s = statistics.mean(dur[L.KCLASS_ATTN]) / 1e3
    out = {
        "metric": PREFILL_METRIC,
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
                     "traffic": stored_traffic(os.path.join(ROOT, "profiles", "prefill_scan_traffic.json"), spec.name,
                                               "prefill_scan.hip"),
                     "flop_per_launch": flops, "avg_launch_us": round(prod_avg_s * 1e6, 2),
                     "peak_measured": round(mf_peak, 1), "frac_of_measured": round(achieved / mf_peak, 4),
                     "measured_by": "csa2_probe_mfma_fp8: back-to-back 16x16x128 FP8 MFMAs, 4 waves per SIMD",
                     "epilogue_ceiling": {"achieved": round(mf_epi, 1), "frac": round(mf_epi / FP8_PEAK_TFLOPS, 4),
                                          "measured_by": "csa2_probe_mfma_fp8 with the per-score ReLU, "
                                                         "head-weight fma and add beside each MFMA"}},
        "indexer_all_kernels": {"avg_us": round(index_s * 1e6, 2),
                                "mfma_frac": round(flops / index_s / 1e12 / FP8_PEAK_TFLOPS, 4)},
        "attention": {"avg_us": round(attn_s * 1e6, 2), "bytes": ab,
                      "GBps": round(ab / attn_s / 1e9, 1), "hbm_frac": round(ab / attn_s / 1e9 / HBM_PEAK_GBS, 4)},
        "kernels_avg_us": {"append": avg(dur[L.KCLASS_APPEND]), "indexer": avg(dur[L.KCLASS_SCAN]),
                           "indexer_product": avg(dur[L.KCLASS_DENSE]), "select": avg(dur[L.KCLASS_SELECT]),
                           "attn": avg(dur[L.KCLASS_ATTN])},
        "ms_per_step_no_events": round(ms_plain, 5),
        "lse_merge": time_lse_merge(dc.outputs[0]["out"], dc.outputs[0]["lse"]),
        # the QAT forward on the chunk's attention output (fp32) and on its bf16 copy
        "fake_quant_f32": time_fake_quant(dc.outputs[0]["out"]),
        "fake_quant_bf16": time_fake_quant(dc.outputs[0]["out"].to(torch.bfloat16)),
    }
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
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--aux-streams", type=int, default=0,
                    help="run the timed multi-layer group as one csa2_group_step with this many auxiliary "
                         "streams (0: one csa2_layer_step call per layer); the other mode is timed too")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "scan_traffic.json"),
                    help="HBM traffic per scan launch measured with rocprofv3 counters (optional)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pool-k", type=int, default=2048,
                    help="pool width of the hierarchical-indexer variant timed beside the headline (0: skip)")
    args = ap.parse_args()
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1).", file=sys.stderr)
        return 2

    import torch

    import workloads as W
    from fp4_kv_cache_layer_amd import ops, runner
    from fp4_kv_cache_layer_amd import _lib as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    spec = W.config(args.config)
    print(f"[bench] building {spec.name}", file=sys.stderr, flush=True)
    aux = args.aux_streams if len(spec.modes) > 1 else 0
    # the case carries one workspace per layer, so both execution modes can run on it
    dc = runner.DeviceCase(spec, gen_device="cuda", group=max(aux, 1) if len(spec.modes) > 1 else 0)
    step = dc.run_group if aux else dc.run_layers
    torch.cuda.synchronize()
    if spec.prefill:
        return bench_prefill(args, spec, dc)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps; the dominant kernel (indexer scan) carries
    # device timestamps in its dispatches.
    n_scan = sum(1 for m in spec.modes if m != ops.REUSE)
    n_attn = len(spec.modes)
    scan_ring = ops.TimingRing(L.KCLASS_SCAN, args.steps * n_scan)
    scan_ring.install()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_events = (time.perf_counter() - t0) * 1e3 / args.steps
    scan_ring.uninstall()
    scan_ms = scan_ring.durations_ms()

    # Breakdown pass (not the timed region): every kernel class timed.
    rings = {L.KCLASS_SCAN: ops.TimingRing(L.KCLASS_SCAN, args.steps * n_scan),
             L.KCLASS_SELECT: ops.TimingRing(L.KCLASS_SELECT, args.steps * n_scan),
             L.KCLASS_ATTN: ops.TimingRing(L.KCLASS_ATTN, args.steps * n_attn),
             L.KCLASS_APPEND: ops.TimingRing(L.KCLASS_APPEND, args.steps)}
    for r in rings.values():
        r.install()
    for _ in range(args.steps):
        step()
    for r in rings.values():
        r.uninstall()
    dur = {k: r.durations_ms() for k, r in rings.items()}

    # Scrubbed pass: a 512 MiB read between steps evicts the 256 MB
    # Infinity Cache and the L2, so no step starts with the cache warm;
    # each step is bracketed by its own device events.
    scrub = torch.ones(SCRUB_BYTES // 8, dtype=torch.int64, device="cuda")
    sink = torch.zeros((), dtype=torch.int64, device="cuda")
    sring = ops.TimingRing(L.KCLASS_SCAN, args.steps * n_scan)
    sring.install()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in step_ev:
        torch.sum(scrub, dim=0, out=sink)
        e0.record()
        step()
        e1.record()
    sring.uninstall()
    torch.cuda.synchronize()
    scrubbed_steps = [a.elapsed_time(b) for a, b in step_ev]
    scrubbed_scan = sring.durations_ms()
    del scrub

    # the same K steps with no timestamps, for comparison
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_plain = (time.perf_counter() - t0) * 1e3 / args.steps

    # the other execution mode, no timestamps: one csa2_group_step per step
    # (Reuse attentions on an auxiliary stream beside the next layers) or
    # per-layer calls
    other = dc.run_layers if aux else dc.run_group
    for _ in range(3):
        other()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        other()
    torch.cuda.synchronize()
    ms_other = (time.perf_counter() - t0) * 1e3 / args.steps

    ms = ms_events
    value = spec.num_seqs * spec.n_new / (ms / 1e3) if spec.n_new else spec.nq / (ms / 1e3)
    scan_avg = statistics.mean(scan_ms)
    sbytes = scan_bytes(spec)
    achieved = sbytes / (scan_avg / 1e3) / 1e9
    traffic = stored_traffic(args.traffic, spec.name, "index_scan.hip")

    def avg(xs):
        return round(statistics.mean(xs) * 1e3, 2) if xs else None

    hbm_warm, hbm_cold = measured_hbm_read(sbytes)
    out = {
        "metric": METRIC,
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
        "config": {"workload": spec.name, "global_batch": spec.num_seqs, "seq_len": spec.cached[0] + spec.n_new,
                   "modes": "full,reindex,reuse,reuse", "topk": spec.k, "heads": spec.h, "indexer_heads": spec.h_idx,
                   "execution": (f"csa2_group_step, Reuse attentions on {aux} auxiliary stream(s)" if aux
                                 else "one csa2_layer_step call per layer"),
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "index_scan_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": sbytes, "avg_launch_us": round(scan_avg * 1e3, 2),
                     "peak_measured": round(hbm_warm, 1), "frac_of_measured": round(achieved / hbm_warm, 4),
                     "measured_by": "csa2_probe_stream_read over the same byte count, same buffer every launch"},
        "kernels_avg_us": {"append": avg(dur[L.KCLASS_APPEND]), "scan_full": avg(dur[L.KCLASS_SCAN][0::n_scan]),
                           "scan_reindex": avg(dur[L.KCLASS_SCAN][1::n_scan]) if n_scan > 1 else None,
                           "select": avg(dur[L.KCLASS_SELECT]), "attn": avg(dur[L.KCLASS_ATTN])},
        "cache_scrubbed": {"ms_per_step_median": round(statistics.median(scrubbed_steps), 5),
                           "scan_avg_us": avg(scrubbed_scan),
                           "scan_full_us": avg(scrubbed_scan[0::n_scan]),
                           "scan_reindex_us": avg(scrubbed_scan[1::n_scan]) if n_scan > 1 else None,
                           "scan_frac": round(sbytes / (statistics.mean(scrubbed_scan) / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                           "stream_read_cold_GBps": round(hbm_cold, 1),
                           "scan_frac_of_measured_cold": round(
                               sbytes / (statistics.mean(scrubbed_scan) / 1e3) / 1e9 / hbm_cold, 4)},
        "ms_per_step_no_events": round(ms_plain, 5),
        "other_execution": {"execution": ("one csa2_layer_step call per layer" if aux else
                                          "csa2_group_step, Reuse attentions on 1 auxiliary stream"),
                            "ms_per_step_no_events": round(ms_other, 5),
                            "tokens_per_s": round(spec.num_seqs * spec.n_new / (ms_other / 1e3), 1)},
        "group_hbm_frac": None,
        "lse_merge": time_lse_merge(dc.outputs[0]["out"], dc.outputs[0]["lse"]),
        "hierarchical_indexer": (time_hierarchical(dc, args.pool_k, args.steps)
                                 if args.pool_k and ops.REINDEX in spec.modes else None),
    }
    # whole-group algorithmic bytes: scans + gathered rows + Q + O + LSE + append
    attn_b = attn_bytes(spec)
    group_b = n_scan * sbytes + n_attn * attn_b + spec.num_seqs * spec.n_new * (1024 + 256 + 272 + 128 + 4)
    out["group_hbm_frac"] = round(group_b / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(spec, dc)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
