"""Device-side set-up and execution of one workload's CSA2 layer group.

Builds the paged cache by bulk quantize-on-append of the workload's cached
rows, prepares every layer's inputs and outputs, and runs the layers in group
order: Reindex and Reuse layers read the Full layer's cache, Reuse layers
read the Full layer's indices.  All compute goes through libcsa2.so.
"""
from __future__ import annotations

from typing import List, Optional

import torch

import workloads as W
from . import ops

APPEND_CHUNK = 1 << 20          # rows per bulk append call


class _null:
    def __enter__(self):
        return self

    def __exit__(self, *a):
        return False


class DeviceCase:
    """dense: None -> the dense prefill indexer for prefill workloads (all
    queries in one sequence), the per-query scan otherwise.  group: 0 runs
    the layers as separate csa2_layer_step calls; n > 0 runs them as one
    csa2_group_step with n auxiliary streams, with a workspace of their own
    for the Reuse layers so they overlap the layers after them.
    cand_factor / attn_per_head_group are the layer calls' dense-indexer
    candidate factor and attention-form flag (see ops.LayerCall)."""

    def __init__(self, spec: W.CaseSpec, gen_device: str = "cpu", device: str = "cuda",
                 dense: Optional[bool] = None, group: int = 0, shared_ws: bool = False,
                 cand_factor: int = 0, attn_per_head_group: bool = False, poison_ws: bool = False,
                 prune: bool = False):
        """poison_ws: before every layer call, fill the workspace bytes that
        carry no state between calls with 0xFF (a check that no kernel reads
        what the same call did not write).  prune: the cache keeps its
        block-level representation and every Full and Reindex layer prunes
        its indexer with its own previous selection as the seed (the first
        call, with empty outputs, prunes nothing)."""
        self.spec = spec
        self.poison_ws = poison_ws
        self.cand_factor = cand_factor if (spec.prefill if dense is None else dense) else 0
        self.attn_per_head_group = attn_per_head_group
        self.graph = None
        self.dense = spec.prefill if dense is None else dense
        self.group_aux = group
        self.shared_ws = shared_ws
        self.device = device
        self.gen_device = gen_device
        pt = torch.from_numpy(W.page_table(spec))
        seq_lens = torch.tensor([spec.seq_len_after(s) for s in range(spec.num_seqs)], dtype=torch.int32)
        self.page_table = pt
        self.prune = prune
        self.cache = ops.Cache(spec.total_pages(), spec.page_size, pt, seq_lens, device=device, bounds=prune)
        self.q_seq = torch.from_numpy(spec.q_seq()).to(device)
        self.q_vis = torch.from_numpy(spec.q_vis()).to(device)
        self.max_vis = int(spec.q_vis().max()) if spec.nq else 0
        self._fill_cache()
        if prune:
            self.cache.build_bounds()
        self._layers()

    # -- cache fill: cached entries written by bulk append; new rows kept for the Full layer --
    def _fill_cache(self):
        spec, dev = self.spec, self.device
        new_s, new_kv, new_ik = [], [], []
        pt_np = self.page_table.numpy()
        for s in range(spec.num_seqs):
            kv = W.kv_rows(spec, s, self.gen_device)
            ik = W.idxk_rows(spec, s, self.gen_device)
            c = spec.cached[s]
            for a in range(0, c, APPEND_CHUNK):
                b = min(c, a + APPEND_CHUNK)
                slots = torch.from_numpy(W.slots_for(spec, pt_np, s, a, b)).to(dev)
                ops.csa2_append_quant_fp4(self.cache, slots, kv[a:b].to(dev).contiguous(), ik[a:b].to(dev).contiguous())
            if spec.n_new:
                new_s.append(torch.from_numpy(W.slots_for(spec, pt_np, s, c, c + spec.n_new)))
                new_kv.append(kv[c:c + spec.n_new].to(dev))
                new_ik.append(ik[c:c + spec.n_new].to(dev))
            del kv, ik
        if spec.n_new:
            self.new_slots = torch.cat(new_s).to(dev).contiguous()
            self.new_kv = torch.cat(new_kv).contiguous()
            self.new_ik = torch.cat(new_ik).contiguous()
        else:
            self.new_slots = self.new_kv = self.new_ik = None

    def _layers(self):
        spec, dev = self.spec, self.device
        nq, k = spec.nq, spec.k
        self.ws = ops.workspace(ops.FULL, nq, self.max_vis, spec.h_idx, spec.h, k, device=dev)
        # Per-layer calls share one workspace.  A group step runs Full and
        # Reindex layers in order on the calling stream, so they keep sharing
        # it, while each Reuse layer, which runs beside them, gets its own.
        self.group_ws = [self.ws if (mode != ops.REUSE or self.shared_ws) else
                         ops.workspace(ops.REUSE, nq, self.max_vis, spec.h_idx, spec.h, k, device=dev)
                         for li, mode in enumerate(spec.modes)] if self.group_aux > 0 else None
        self.inputs = []
        self.outputs = []
        # hierarchical indexer: the Full layer's Top-pool_k, scored again by the Reindex layers
        self.pool = self.pool_cnt = None
        if spec.pool_k:
            self.pool, self.pool_cnt = self.new_pool(spec.pool_k)
        full_idx = full_cnt = None
        for li, mode in enumerate(spec.modes):
            qi, w, q = W.layer_queries(spec, li, self.gen_device)
            qi, w, q = qi.to(dev).contiguous(), w.to(dev).contiguous(), q.to(dev).contiguous()
            self.inputs.append((qi, w, q))
            out = torch.empty((nq, spec.h, 512), dtype=torch.float32, device=dev)
            lse = torch.empty((nq, spec.h), dtype=torch.float32, device=dev)
            if mode == ops.REUSE:
                idx, cnt = full_idx, full_cnt
            else:
                idx = torch.full((nq, k), -1, dtype=torch.int32, device=dev)
                cnt = torch.zeros(nq, dtype=torch.int32, device=dev)
                if mode == ops.FULL:
                    full_idx, full_cnt = idx, cnt
            self.outputs.append(dict(idx=idx, cnt=cnt, out=out, lse=lse))
        self.calls: List[ops.LayerCall] = [self.make_call(li, self.ws) for li in range(len(spec.modes))]
        group_calls = ([self.make_call(li, self.group_ws[li]) for li in range(len(spec.modes))]
                       if self.group_ws is not None else [])

        self.group = ops.GroupCall(group_calls, n_aux=self.group_aux) if self.group_aux > 0 else None

    def new_pool(self, pool_k: int):
        """Pool buffers [nq][pool_k], [nq] for a hierarchical-indexer variant."""
        nq = self.spec.nq
        return (torch.empty((nq, pool_k), dtype=torch.int32, device=self.device),
                torch.empty(nq, dtype=torch.int32, device=self.device))

    def make_call(self, li: int, ws, pool=None, pool_cnt=None) -> ops.LayerCall:
        """csa2_layer_step arguments of layer li on workspace ws; pool (default:
        the case's own) switches on the hierarchical indexer for Full and
        Reindex layers."""
        spec, k = self.spec, self.spec.k
        mode = spec.modes[li]
        qi, w, q = self.inputs[li]
        o = self.outputs[li]
        if pool is None:
            pool, pool_cnt = self.pool, self.pool_cnt
        common = (self.cache, q, self.q_seq, self.q_vis, k, self.max_vis, spec.sm_scale, o["idx"], o["cnt"],
                  o["out"], o["lse"])
        opts = dict(attn_per_head_group=self.attn_per_head_group)
        if mode == ops.REUSE:
            return ops.LayerCall(mode, *common, ws=ws, **opts)
        opts.update(dense=self.dense, pool=pool, pool_cnt=pool_cnt, dense_cand_factor=self.cand_factor)
        if self.prune:
            opts.update(seed=o["idx"], seed_cnt=o["cnt"])
        if mode == ops.FULL:
            return ops.LayerCall(mode, *common, q_idx=qi, w=w, new_slots=self.new_slots, new_kv=self.new_kv,
                                 new_idxk=self.new_ik, ws=ws, **opts)
        return ops.LayerCall(mode, *common, q_idx=qi, w=w, ws=ws, **opts)

    def set_timing(self, timing) -> None:
        """Attach an ops.Timing (or None) to the per-layer calls and the group step."""
        for c in self.calls:
            c.set_timing(timing)
        if self.group is not None:
            self.group.set_timing(timing)

    def _poison(self, ws, stream=None) -> None:
        z = ops.workspace_state_bytes(self.spec.nq)
        with torch.cuda.stream(stream) if stream is not None else _null():
            ws[z:].fill_(0xFF)

    def run_group(self, stream=None) -> None:
        if self.group is not None:
            if self.poison_ws:
                for ws in {id(w): w for w in self.group_ws}.values():
                    self._poison(ws, stream)
            self.group(stream)
            return
        self.run_layers(stream)

    def run_layers(self, stream=None) -> None:
        """The layers as separate csa2_layer_step calls, whatever `group` is."""
        for c in self.calls:
            if self.poison_ws:
                self._poison(self.ws, stream)
            c(stream)

    def capture_graph(self) -> None:
        """Captures one step's per-layer calls (in layer order, on one stream)
        into a HIP graph; replay_graph() then launches the whole group with one
        call.  The captured kernels read and write the same buffers as the
        eager calls, so a replay gives exactly their results.  Calls must not
        carry timing while captured."""
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.run_layers()
        torch.cuda.synchronize()
        self.graph = g

    def replay_graph(self) -> None:
        self.graph.replay()

    def results_host(self) -> List[dict]:
        torch.cuda.synchronize()
        return [{key: (v.cpu().numpy() if v is not None else None) for key, v in o.items()} for o in self.outputs]
