// C ABI of the CSA2 layer step (declared in include/csa2.h): host-side
// argument validation, workspace sizing and kernel dispatch.  Nothing here
// allocates device memory or synchronises a stream.
#include "csa2.h"
#include "csa2_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

using namespace csa2;

// Workspace of csa2_layer_step_static: a fixed array in device memory, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never uses the name itself (on the host it is only a stand-in for the
// symbol); it uses the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[CSA2_STATIC_SCRATCH_BYTES];

namespace {

// Takes the next slot of a kernel class's timing ring, if the call carries
// one; the launch records the slot's events as part of its dispatches.
struct TimedLaunch {
  csa2_timing_ring* ring;
  int slot;
  KEvents ev;
  TimedLaunch(const csa2_timing* tm, int cls) : ring(tm ? tm->ring[cls] : nullptr), slot(-1) {
    if (ring && ring->start && ring->stop && ring->count >= 0 && ring->count < ring->capacity) {
      slot = ring->count;
      ev.start = ring->start[slot];
      ev.stop = ring->stop[slot];
    }
  }
  ~TimedLaunch() {
    if (slot >= 0) ring->count = slot + 1;
  }
};

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The value of an enum argument as an integer.  A caller may pass any int
// (the header is C, where enums are ints); read as the C++ enum type, a value
// outside its range would be undefined, so its bytes are copied instead.
template <typename E>
int32_t enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int32_t), "C enums are int-sized");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

int ilog2_pow2(int x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

csa2_status check_cache(const csa2_cache_view* c, CacheArgs* out) {
  if (!c || !c->kv || !c->idx_k || !c->page_table) return CSA2_ERR_INVALID_ARG;
  if (!aligned(c->kv, 16) || !aligned(c->idx_k, 16) || !aligned(c->page_table, 4)) return CSA2_ERR_INVALID_ARG;
  if (c->num_pages < 1 || c->num_seqs < 1 || c->max_pages < 1) return CSA2_ERR_INVALID_ARG;
  const int lg = ilog2_pow2(c->page_size);
  if (lg < 0 || c->page_size < CSA2_MIN_PAGE_SIZE) return CSA2_ERR_INVALID_ARG;
  if ((int64_t)c->max_pages * c->page_size > INT32_MAX) return CSA2_ERR_UNSUPPORTED;
  out->kv = c->kv;
  out->idx_k = c->idx_k;
  out->page_table = c->page_table;
  out->max_pages = c->max_pages;
  out->lg_page = lg;
  out->num_pages = c->num_pages;
  return CSA2_OK;
}

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

csa2_status validate_index(const csa2_cache_view* c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                           const int32_t* q_vis, int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis,
                           const int32_t* out_idx, const int32_t* out_cnt, const void* ws, size_t ws_bytes,
                           CacheArgs* ca) {
  if (nq < 0 || h_idx < 1 || h_idx > CSA2_MAX_H_IDX || k < 1 || k > CSA2_MAX_K || max_vis < 0)
    return CSA2_ERR_INVALID_ARG;
  csa2_status st = check_cache(c, ca);
  if (st != CSA2_OK) return st;
  if ((int64_t)max_vis > (int64_t)c->max_pages * c->page_size) return CSA2_ERR_INVALID_ARG;
  if (nq == 0) return CSA2_OK;
  if (!q_idx || !w || !q_seq || !q_vis || !out_idx || !out_cnt || !ws) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(q_seq, 4) || !aligned(q_vis, 4) ||
      !aligned(out_idx, 16) || !aligned(out_cnt, 4) || !aligned(ws, 16))
    return CSA2_ERR_INVALID_ARG;
  if (ws_bytes < zero_state_bytes(nq) + index_score_bytes(nq, max_vis)) return CSA2_ERR_WORKSPACE;
  return CSA2_OK;
}

csa2_status validate_attn(const csa2_cache_view* c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                          const int32_t* cnt, int32_t nq, int32_t h, int32_t k, float sm_scale, const float* out,
                          const float* lse, CacheArgs* ca) {
  if (nq < 0 || h < 1 || h > CSA2_MAX_H || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_INVALID_ARG;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return CSA2_ERR_INVALID_ARG;
  csa2_status st = check_cache(c, ca);
  if (st != CSA2_OK) return st;
  if (nq == 0) return CSA2_OK;
  if (!q || !q_seq || !idx || !cnt || !out) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(q_seq, 4) || !aligned(idx, 4) || !aligned(cnt, 4) || !aligned(out, 16) ||
      (lse && !aligned(lse, 4)))
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

csa2_status validate_append(const csa2_cache_view* c, const int32_t* slots, const uint16_t* kv_rows,
                            const uint16_t* idxk_rows, int32_t n, CacheArgs* ca) {
  if (n < 0) return CSA2_ERR_INVALID_ARG;
  csa2_status st = check_cache(c, ca);
  if (st != CSA2_OK) return st;
  if (n == 0) return CSA2_OK;
  if (!slots || !kv_rows || !idxk_rows) return CSA2_ERR_INVALID_ARG;
  if (!aligned(slots, 4) || !aligned(kv_rows, 16) || !aligned(idxk_rows, 16)) return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

IndexWs index_ws(void* ws, int32_t nq, int32_t max_vis, size_t score_off, bool dense, bool prune) {
  IndexWs r;
  r.vis_cap = max_vis;
  uint8_t* p = reinterpret_cast<uint8_t*>(ws);
  r.cand_cnt = reinterpret_cast<uint32_t*>(p);
  r.tau = reinterpret_cast<float*>(p + (size_t)nq * 4);
  r.cnt2 = reinterpret_cast<uint32_t*>(p + (size_t)nq * 8);
  r.vstride = index_vstride(max_vis);
  r.cand = reinterpret_cast<int32_t*>(p + score_off);
  r.ckey = reinterpret_cast<uint32_t*>(p + score_off + (size_t)nq * (size_t)r.vstride * 4);
  r.fstride = (max_vis + kScanChunk - 1) / kScanChunk;
  r.floor = dense ? nullptr : reinterpret_cast<uint32_t*>(p + score_off + 2 * (size_t)nq * (size_t)r.vstride * 4);
  r.prune = prune ? reinterpret_cast<uint32_t*>(p + score_off + 2 * (size_t)nq * (size_t)r.vstride * 4 +
                                                (size_t)nq * (size_t)r.fstride * 4)
                  : nullptr;
  r.bmax = dense ? nullptr : reinterpret_cast<uint32_t*>(p + score_off + 2 * (size_t)nq * (size_t)r.vstride * 4 +
                                                        2 * (size_t)nq * (size_t)r.fstride * 4);
  return r;
}

csa2_status run_index(const CacheArgs& ca, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                      const int32_t* q_vis, int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis, int32_t* out_idx,
                      int32_t* out_cnt, const IndexWs& iw, bool dense, hipStream_t s) {
  // both indexers leave a candidate list: the final select completes the Top-k
  if (max_vis > 0) {
    csa2_status st =
        dense ? hip_status(launch_prefill_scan(ca, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, iw,
                                               kDefaultCandFactor, s))
              : hip_status(launch_index_scan(ca, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, iw, s));
    if (st != CSA2_OK) return st;
  }
  return hip_status(launch_topk_final(iw, ScanArgs{ca, q_idx, w, q_seq, h_idx}, q_vis, nq, k, out_idx, out_cnt, s));
}

// One layer of a step, validated, split into the stages that the group
// scheduler places on streams: append, indexer scan, Top-K select, attention.
struct Step {
  csa2_mode mode;
  const csa2_step_args* a;
  CacheArgs ca;
  bool dense;
  bool pool;                 // hierarchical indexer (Full: writes the pool; Reindex: reads it)
  bool prune;                // block-level pruning of the per-query indexer
  bool share_heads;          // attention: shared-row form for large 64-head batches
  int cand_factor;           // dense indexer candidate factor
  const csa2_timing* tm;     // nullable
  IndexWs iw;
  float* pool_sc;            // pool scores, in the workspace's score region
};

csa2_status validate_pool(const int32_t* pool, const int32_t* pool_cnt, int32_t nq, int32_t p, int32_t k,
                          const int32_t* out_idx, const int32_t* out_cnt) {
  if (nq < 0 || p < 1 || p > CSA2_MAX_K || k < 1 || k > CSA2_MAX_K) return CSA2_ERR_INVALID_ARG;
  if (nq == 0) return CSA2_OK;
  if (!pool || !pool_cnt || !out_idx || !out_cnt) return CSA2_ERR_INVALID_ARG;
  if (!aligned(pool, 16) || !aligned(pool_cnt, 4) || !aligned(out_idx, 4) || !aligned(out_cnt, 4))
    return CSA2_ERR_INVALID_ARG;
  return CSA2_OK;
}

// Every check of csa2_layer_step, before anything is launched.
csa2_status prepare_step(int32_t mode_value, const csa2_step_args* a, Step* p) {
  if (!a || (mode_value != CSA2_FULL && mode_value != CSA2_REINDEX && mode_value != CSA2_REUSE))
    return CSA2_ERR_INVALID_ARG;
  const csa2_mode mode = static_cast<csa2_mode>(mode_value);
  if (a->flags & ~(CSA2_STEP_DENSE_INDEX | CSA2_STEP_POOL | CSA2_STEP_ATTN_PER_HEAD_GROUP | CSA2_STEP_PRUNE))
    return CSA2_ERR_INVALID_ARG;
  const bool prune = (a->flags & CSA2_STEP_PRUNE) != 0;
  if (prune) {
    if (mode == CSA2_REUSE || (a->flags & (CSA2_STEP_DENSE_INDEX | CSA2_STEP_POOL))) return CSA2_ERR_INVALID_ARG;
    if (!a->cache || !a->cache->idxk_bounds || !aligned(a->cache->idxk_bounds, 16)) return CSA2_ERR_INVALID_ARG;
    if (a->nq > 0 && (!a->seed || !a->seed_cnt || !aligned(a->seed, 4) || !aligned(a->seed_cnt, 4)))
      return CSA2_ERR_INVALID_ARG;
  } else if (a->seed || a->seed_cnt) {
    return CSA2_ERR_INVALID_ARG;
  }
  if (a->flags & CSA2_STEP_DENSE_INDEX) {
    if (a->dense_cand_factor < CSA2_DENSE_RESCORE_ALL || a->dense_cand_factor > 64) return CSA2_ERR_INVALID_ARG;
  } else if (a->dense_cand_factor != 0) {
    return CSA2_ERR_INVALID_ARG;
  }
  const bool pool = (a->flags & CSA2_STEP_POOL) != 0;
  if (pool) {
    if (mode == CSA2_REUSE || a->pool_k < a->k) return CSA2_ERR_INVALID_ARG;
    csa2_status st = validate_pool(a->pool, a->pool_cnt, a->nq, a->pool_k, a->k, a->idx, a->cnt);
    if (st != CSA2_OK) return st;
    if (a->nq > 0 && (a->pool == a->idx || a->pool_cnt == a->cnt)) return CSA2_ERR_INVALID_ARG;
  } else if (a->pool || a->pool_cnt || a->pool_k != 0) {
    return CSA2_ERR_INVALID_ARG;
  }
  csa2_status st;
  if (mode == CSA2_FULL) {
    st = validate_append(a->cache, a->new_slots, a->new_kv, a->new_idxk, a->n_new, &p->ca);
    if (st != CSA2_OK) return st;
  } else if (a->n_new != 0 || a->new_slots || a->new_kv || a->new_idxk) {
    return CSA2_ERR_INVALID_ARG;
  }
  if (mode != CSA2_REUSE) {
    // a Full pool layer's indexer writes its Top-pool_k into the pool
    const bool to_pool = pool && mode == CSA2_FULL;
    st = validate_index(a->cache, a->q_idx, a->w, a->q_seq, a->q_vis, a->nq, a->h_idx, to_pool ? a->pool_k : a->k,
                        a->max_vis, to_pool ? a->pool : a->idx, to_pool ? a->pool_cnt : a->cnt, a->ws, a->ws_bytes,
                        &p->ca);
    if (st != CSA2_OK) return st;
  } else if (a->q_idx || a->w || a->h_idx != 0) {
    return CSA2_ERR_INVALID_ARG;
  }
  st = validate_attn(a->cache, a->q, a->q_seq, a->idx, a->cnt, a->nq, a->h, a->k, a->sm_scale, a->out, a->lse, &p->ca);
  if (st != CSA2_OK) return st;
  p->mode = mode;
  p->a = a;
  p->dense = (a->flags & CSA2_STEP_DENSE_INDEX) != 0;
  p->pool = pool;
  p->prune = prune;
  p->share_heads = (a->flags & CSA2_STEP_ATTN_PER_HEAD_GROUP) == 0;
  p->cand_factor = a->dense_cand_factor == 0 ? kDefaultCandFactor
                   : a->dense_cand_factor == CSA2_DENSE_RESCORE_ALL ? 0 : a->dense_cand_factor;
  p->tm = a->timing;
  p->iw = IndexWs{};
  p->pool_sc = nullptr;
  if (a->nq == 0) return CSA2_OK;
  const size_t z = zero_state_bytes(a->nq);
  if (mode != CSA2_REUSE) {
    // the pool scores reuse the candidate region (dead once the pool is selected)
    const size_t need = std::max(index_score_bytes(a->nq, a->max_vis), pool ? pool_score_bytes(a->nq, a->pool_k) : 0);
    if (a->ws_bytes < z + need) return CSA2_ERR_WORKSPACE;
    p->iw = index_ws(a->ws, a->nq, a->max_vis, z, p->dense, prune);
    if (pool) p->pool_sc = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(a->ws) + z);
  } else if (a->ws && !aligned(a->ws, 16)) {
    return CSA2_ERR_INVALID_ARG;
  }
  return CSA2_OK;
}

// A Full layer's few appended rows ride in the scan launch (one launch less):
// per-query scan, no pool, no block-level representation to refresh.
bool append_in_scan(const Step& p) {
  const csa2_step_args* a = p.a;
  return p.mode == CSA2_FULL && a->n_new > 0 && a->n_new <= kMaxFusedAppend && a->nq > 0 && a->max_vis > 0 &&
         !p.dense && !p.pool && !p.prune && a->cache->idxk_bounds == nullptr;
}

csa2_status stage_append(const Step& p, hipStream_t s) {
  const csa2_step_args* a = p.a;
  if (p.mode != CSA2_FULL || a->n_new == 0 || append_in_scan(p)) return CSA2_OK;
  TimedLaunch t(p.tm, CSA2_KCLASS_APPEND);
  uint8_t* const bounds = a->cache->idxk_bounds;
  if (!bounds)
    return hip_status(launch_append_quant(p.ca.kv, p.ca.idx_k, a->new_slots, a->new_kv, a->new_idxk, a->n_new, s, t.ev));
  // the appended rows' blocks get their representation recomputed
  csa2_status st = hip_status(launch_append_quant(p.ca.kv, p.ca.idx_k, a->new_slots, a->new_kv, a->new_idxk, a->n_new,
                                                  s, t.ev.first()));
  if (st != CSA2_OK) return st;
  return hip_status(launch_idxk_bounds(p.ca.idx_k, bounds, a->new_slots, 0, a->n_new,
                                       (int64_t)p.ca.num_pages << p.ca.lg_page, s, t.ev.last()));
}

csa2_status stage_scan(const Step& p, hipStream_t s) {
  const csa2_step_args* a = p.a;
  if (p.mode == CSA2_REUSE || a->nq == 0 || a->max_vis == 0) return CSA2_OK;
  if (p.pool && p.mode == CSA2_REINDEX) return CSA2_OK;     // the pool is scored in stage_select
  if (p.dense) {
    TimedLaunch t(p.tm, CSA2_KCLASS_SCAN), tp(p.tm, CSA2_KCLASS_DENSE);
    return hip_status(launch_prefill_scan(p.ca, a->q_idx, a->w, a->q_seq, a->q_vis, a->nq, a->h_idx,
                                          p.pool ? a->pool_k : a->k, a->max_vis, p.iw, p.cand_factor, s, t.ev,
                                          tp.ev));
  }
  TimedLaunch t(p.tm, CSA2_KCLASS_SCAN);
  if (p.prune) {
    csa2_status st = hip_status(launch_prune_mask(p.ca, a->cache->idxk_bounds, a->q_idx, a->w, a->q_seq, a->q_vis,
                                                  a->seed, a->seed_cnt, a->nq, a->h_idx, a->k, p.iw, s, t.ev.first()));
    if (st != CSA2_OK) return st;
    return hip_status(launch_index_scan(p.ca, a->q_idx, a->w, a->q_seq, a->q_vis, a->nq, a->h_idx, a->k, a->max_vis,
                                        p.iw, s, t.ev.last()));
  }
  if (append_in_scan(p)) {
    const AppendArgs ap{p.ca.kv, p.ca.idx_k, a->new_slots, a->new_kv, a->new_idxk, a->n_new};
    return hip_status(launch_index_scan(p.ca, a->q_idx, a->w, a->q_seq, a->q_vis, a->nq, a->h_idx, a->k,
                                        a->max_vis, p.iw, s, t.ev, &ap));
  }
  return hip_status(launch_index_scan(p.ca, a->q_idx, a->w, a->q_seq, a->q_vis, a->nq, a->h_idx,
                                      p.pool ? a->pool_k : a->k, a->max_vis, p.iw, s, t.ev));
}

csa2_status run_pool(const Step& p, hipStream_t s) {
  const csa2_step_args* a = p.a;
  TimedLaunch ts(p.tm, CSA2_KCLASS_POOL_SCAN), tl(p.tm, CSA2_KCLASS_POOL_SELECT);
  return hip_status(launch_pool_index(p.ca, a->q_idx, a->w, a->q_seq, a->pool, a->pool_cnt, a->nq, a->h_idx,
                                      a->pool_k, a->k, a->idx, a->cnt, p.pool_sc, s, ts.ev, tl.ev));
}

// Full and Reindex: Top-k of the scores.  With a pool, a Full layer selects
// its Top-pool_k into the pool and then its Top-k among the pool (the same
// set: the order is total) from the scores it already has, a Reindex layer
// scores and selects in the pool.
csa2_status stage_select(const Step& p, hipStream_t s) {
  const csa2_step_args* a = p.a;
  if (p.mode == CSA2_REUSE || a->nq == 0) return CSA2_OK;
  if (p.pool && p.mode == CSA2_REINDEX) return run_pool(p, s);
  const bool to_pool = p.pool;
  int32_t* idx = to_pool ? a->pool : a->idx;
  int32_t* cnt = to_pool ? a->pool_cnt : a->cnt;
  const int32_t k = to_pool ? a->pool_k : a->k;
  csa2_status st;
  {
    TimedLaunch t(p.tm, CSA2_KCLASS_SELECT);
    st = hip_status(launch_topk_final(p.iw, ScanArgs{p.ca, a->q_idx, a->w, a->q_seq, a->h_idx}, a->q_vis, a->nq, k,
                                      idx, cnt, s, t.ev));
  }
  if (st != CSA2_OK || !to_pool) return st;
  return run_pool(p, s);                      // the indexers keep no score rows: score the pool again
}

csa2_status stage_attn(const Step& p, hipStream_t s) {
  const csa2_step_args* a = p.a;
  if (a->nq == 0) return CSA2_OK;
  TimedLaunch t(p.tm, CSA2_KCLASS_ATTN);
  return hip_status(launch_sparse_attn(p.ca, a->q, a->q_seq, a->idx, a->cnt, a->nq, a->h, a->k, a->sm_scale, a->out,
                                       a->lse, p.share_heads, s, t.ev));
}

csa2_status run_step(const Step& p, hipStream_t s) {
  csa2_status st = stage_append(p, s);
  if (st == CSA2_OK) st = stage_scan(p, s);
  if (st == CSA2_OK) st = stage_select(p, s);
  if (st == CSA2_OK) st = stage_attn(p, s);
  return st;
}

// Layer j must not overlap layer i (i < j) when they share memory that
// either writes: a workspace, index/count buffers one of them writes, an
// output, or (a Full layer j appending) a cache that layer i reads.
bool layers_conflict(const Step& i, const Step& j) {
  const csa2_step_args *a = i.a, *b = j.a;
  auto same = [](const void* x, const void* y) { return x != nullptr && x == y; };
  if (same(a->ws, b->ws)) return true;
  if (same(a->out, b->out) || same(a->lse, b->lse)) return true;
  const bool iw = i.mode != CSA2_REUSE, jw = j.mode != CSA2_REUSE;   // writes idx/cnt
  if ((iw || jw) && (same(a->idx, b->idx) || same(a->cnt, b->cnt))) {
    // the one case ordered by stream placement: j reuses what i selected
    if (!(iw && !jw)) return true;
  }
  if (j.mode == CSA2_FULL && b->n_new > 0 && same(i.ca.kv, j.ca.kv)) return true;
  // pool buffers: any overlap with the other layer's buffers, unless both only read them
  auto touches = [&](const csa2_step_args* x, const void* ptr) {
    return same(x->ws, ptr) || same(x->out, ptr) || same(x->lse, ptr) || same(x->idx, ptr) || same(x->cnt, ptr);
  };
  const bool iwp = i.pool && i.mode == CSA2_FULL, jwp = j.pool && j.mode == CSA2_FULL;
  for (const void* ptr : {a->pool, a->pool_cnt})
    if (i.pool && (touches(b, ptr) || (j.pool && (iwp || jwp) && (same(b->pool, ptr) || same(b->pool_cnt, ptr)))))
      return true;
  for (const void* ptr : {b->pool, b->pool_cnt})
    if (j.pool && touches(a, ptr)) return true;
  return false;
}

}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status st) {
  switch (enum_value(st)) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_INVALID_ARG: return "invalid argument";
    case CSA2_ERR_UNSUPPORTED: return "unsupported request";
    case CSA2_ERR_WORKSPACE: return "workspace too small";
    case CSA2_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t csa2_workspace_bytes(csa2_mode mode_arg, int32_t nq, int32_t max_vis, int32_t h_idx, int32_t h, int32_t k) {
  const int32_t mode = enum_value(mode_arg);
  (void)h_idx; (void)k;
  if (nq <= 0 || max_vis < 0 || h < 1 || h > CSA2_MAX_H || k < 1 || k > CSA2_MAX_K) return 0;
  size_t b = zero_state_bytes(nq);
  if (mode != CSA2_REUSE) b += std::max(index_score_bytes(nq, max_vis), pool_score_bytes(nq, CSA2_MAX_K));
  return b;
}

csa2_status csa2_idxk_bounds_build(const csa2_cache_view* c, int32_t first_block, int32_t n_blocks, hipStream_t s) {
  CacheArgs ca;
  csa2_status st = check_cache(c, &ca);
  if (st != CSA2_OK) return st;
  if (!c->idxk_bounds || !aligned(c->idxk_bounds, 16)) return CSA2_ERR_INVALID_ARG;
  const int64_t nblocks = ((int64_t)c->num_pages << ca.lg_page) / CSA2_PRUNE_BLOCK;
  if (first_block < 0 || n_blocks < 0 || (int64_t)first_block + n_blocks > nblocks) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_idxk_bounds(ca.idx_k, c->idxk_bounds, nullptr, first_block, n_blocks,
                                       (int64_t)c->num_pages << ca.lg_page, s));
}

size_t csa2_pool_workspace_bytes(int32_t nq, int32_t p) {
  if (nq <= 0 || p < 1 || p > CSA2_MAX_K) return 0;
  return pool_score_bytes(nq, p);
}

csa2_status csa2_workspace_init(void* ws, size_t ws_bytes, hipStream_t s) {
  if (ws_bytes == 0) return CSA2_OK;
  if (!ws || !aligned(ws, 16)) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_fill_zero(ws, ws_bytes, s));
}

csa2_status csa2_append_quant_fp4(const csa2_cache_view* c, const int32_t* slots, const uint16_t* kv_rows,
                                  const uint16_t* idxk_rows, int32_t n, hipStream_t s) {
  CacheArgs ca;
  csa2_status st = validate_append(c, slots, kv_rows, idxk_rows, n, &ca);
  if (st != CSA2_OK || n == 0) return st;
  return hip_status(launch_append_quant(ca.kv, ca.idx_k, slots, kv_rows, idxk_rows, n, s));
}

csa2_status csa2_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                            const int32_t* q_vis, int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis,
                            int32_t* out_idx, int32_t* out_cnt, void* ws, size_t ws_bytes, hipStream_t s) {
  CacheArgs ca;
  csa2_status st = validate_index(c, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, out_idx, out_cnt, ws, ws_bytes, &ca);
  if (st != CSA2_OK || nq == 0) return st;
  return run_index(ca, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, out_idx, out_cnt,
                   index_ws(ws, nq, max_vis, zero_state_bytes(nq), false, false), false, s);
}

csa2_status csa2_prefill_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w, const int32_t* q_seq,
                                    const int32_t* q_vis, int32_t nq, int32_t h_idx, int32_t k, int32_t max_vis,
                                    int32_t* out_idx, int32_t* out_cnt, void* ws, size_t ws_bytes, hipStream_t s) {
  CacheArgs ca;
  csa2_status st = validate_index(c, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, out_idx, out_cnt, ws, ws_bytes, &ca);
  if (st != CSA2_OK || nq == 0) return st;
  return run_index(ca, q_idx, w, q_seq, q_vis, nq, h_idx, k, max_vis, out_idx, out_cnt,
                   index_ws(ws, nq, max_vis, zero_state_bytes(nq), true, false), true, s);
}

csa2_status csa2_pool_index_topk(const csa2_cache_view* c, const uint8_t* q_idx, const float* w,
                                 const int32_t* q_seq, const int32_t* pool, const int32_t* pool_cnt, int32_t nq,
                                 int32_t h_idx, int32_t p, int32_t k, int32_t* out_idx, int32_t* out_cnt, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  if (nq < 0 || h_idx < 1 || h_idx > CSA2_MAX_H_IDX) return CSA2_ERR_INVALID_ARG;
  csa2_status st = validate_pool(pool, pool_cnt, nq, p, k, out_idx, out_cnt);
  if (st != CSA2_OK) return st;
  CacheArgs ca;
  st = check_cache(c, &ca);
  if (st != CSA2_OK || nq == 0) return st;
  if (!q_idx || !w || !q_seq || !ws) return CSA2_ERR_INVALID_ARG;
  if (!aligned(q_idx, 16) || !aligned(w, 4) || !aligned(q_seq, 4) || !aligned(ws, 16)) return CSA2_ERR_INVALID_ARG;
  if (ws_bytes < pool_score_bytes(nq, p)) return CSA2_ERR_WORKSPACE;
  return hip_status(launch_pool_index(ca, q_idx, w, q_seq, pool, pool_cnt, nq, h_idx, p, k, out_idx, out_cnt,
                                     reinterpret_cast<float*>(ws), s));
}

csa2_status csa2_sparse_attn(const csa2_cache_view* c, const uint16_t* q, const int32_t* q_seq, const int32_t* idx,
                             const int32_t* cnt, int32_t nq, int32_t h, int32_t k, float sm_scale, float* out,
                             float* lse, void* ws, size_t ws_bytes, hipStream_t s) {
  CacheArgs ca;
  csa2_status st = validate_attn(c, q, q_seq, idx, cnt, nq, h, k, sm_scale, out, lse, &ca);
  if (st != CSA2_OK || nq == 0) return st;
  if (ws && !aligned(ws, 16)) return CSA2_ERR_INVALID_ARG;
  (void)ws_bytes;
  return hip_status(launch_sparse_attn(ca, q, q_seq, idx, cnt, nq, h, k, sm_scale, out, lse, true, s));
}

csa2_status csa2_layer_step(csa2_mode mode, const csa2_step_args* a, hipStream_t s) {
  Step p;
  csa2_status st = prepare_step(enum_value(mode), a, &p);
  if (st != CSA2_OK) return st;
  return run_step(p, s);
}

csa2_status csa2_layer_step_static(csa2_mode mode, const csa2_step_args* a, hipStream_t s) {
  // The scratch array's address on the current device, looked up once per
  // device with that device current.
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  if (!a) return CSA2_ERR_INVALID_ARG;
  if (a->ws || a->ws_bytes) return CSA2_ERR_INVALID_ARG;     // the workspace is the library's own
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CSA2_ERR_HIP;
  void* ptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {
      void* p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CSA2_ERR_HIP;
      dev_ptr[dev] = p;
    }
    ptr = dev_ptr[dev];
  }
  csa2_step_args b = *a;
  b.ws = ptr;
  b.ws_bytes = CSA2_STATIC_SCRATCH_BYTES;
  Step p;
  csa2_status st = prepare_step(enum_value(mode), &b, &p);   // CSA2_ERR_WORKSPACE: the shape needs more
  if (st != CSA2_OK || b.nq == 0) return st;
  // the state-carrying head of the workspace starts at zero (a fill kernel,
  // which a graph capture may record; no memset node)
  st = hip_status(launch_fill_zero(ptr, zero_state_bytes(b.nq), s));
  if (st != CSA2_OK) return st;
  return run_step(p, s);
}

csa2_status csa2_lse_merge(const float* o_a, const float* lse_a, const float* o_b, const float* lse_b,
                           int32_t rows, int32_t dim, float* o, float* lse, hipStream_t s) {
  if (rows < 0 || dim < 4 || dim % 4 != 0) return CSA2_ERR_INVALID_ARG;
  if (rows == 0) return CSA2_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o) return CSA2_ERR_INVALID_ARG;
  if (!aligned(o_a, 16) || !aligned(o_b, 16) || !aligned(o, 16) || !aligned(lse_a, 4) || !aligned(lse_b, 4) ||
      (lse && !aligned(lse, 4)))
    return CSA2_ERR_INVALID_ARG;
  if (lse && (lse == lse_a || lse == lse_b)) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_lse_merge(o_a, lse_a, o_b, lse_b, rows, dim, o, lse, s));
}

csa2_status csa2_fake_quant_fp4(const void* x, void* y, int64_t n, int32_t dtype, hipStream_t s) {
  if (n < 0 || n % 32 != 0 || (dtype != CSA2_DTYPE_F32 && dtype != CSA2_DTYPE_BF16)) return CSA2_ERR_INVALID_ARG;
  if (n == 0) return CSA2_OK;
  if (!x || !y || !aligned(x, 16) || !aligned(y, 16)) return CSA2_ERR_INVALID_ARG;
  return hip_status(launch_fake_quant(x, y, n, dtype == CSA2_DTYPE_BF16, s));
}

int32_t csa2_group_events(int32_t n_layers, int32_t n_aux) {
  if (n_layers < 0 || n_layers > CSA2_GROUP_MAX_LAYERS || n_aux < 0 || n_aux > CSA2_GROUP_MAX_AUX) return -1;
  return 1 + 3 * n_layers + n_aux;
}

csa2_status csa2_group_step(int32_t n, const csa2_mode* modes, const csa2_step_args* layers, hipStream_t s,
                            const csa2_group_exec* ex) {
  if (n < 0 || n > CSA2_GROUP_MAX_LAYERS) return CSA2_ERR_INVALID_ARG;
  if (n == 0) return CSA2_OK;
  if (!modes || !layers) return CSA2_ERR_INVALID_ARG;
  const int n_aux = ex ? ex->n_aux : 0;
  if (n_aux < 0 || n_aux > CSA2_GROUP_MAX_AUX) return CSA2_ERR_INVALID_ARG;
  if (n_aux > 0) {
    if (!ex->events || ex->n_events < csa2_group_events(n, n_aux)) return CSA2_ERR_INVALID_ARG;
    for (int j = 0; j < n_aux; ++j) {
      if (!ex->aux[j] || ex->aux[j] == s) return CSA2_ERR_INVALID_ARG;
      for (int j2 = 0; j2 < j; ++j2)
        if (ex->aux[j2] == ex->aux[j]) return CSA2_ERR_INVALID_ARG;
    }
    for (int e = 0; e < csa2_group_events(n, n_aux); ++e)
      if (!ex->events[e]) return CSA2_ERR_INVALID_ARG;
  }
  Step steps[CSA2_GROUP_MAX_LAYERS];
  for (int i = 0; i < n; ++i) {
    csa2_status st = prepare_step(enum_value(modes[i]), &layers[i], &steps[i]);
    if (st != CSA2_OK) return st;
  }
  if (n_aux == 0) {
    for (int i = 0; i < n; ++i) {
      csa2_status st = run_step(steps[i], s);
      if (st != CSA2_OK) return st;
    }
    return CSA2_OK;
  }

  // Full and Reindex layers run whole on s, in layer order.  A Reuse layer
  // (attention only) runs on an auxiliary stream, round-robin, as soon as
  // the select it reuses is done, beside the layers after it on s.  Events
  // carry the cross-stream order, and only the edges that stream order does
  // not already imply are enqueued (each record or wait costs host time).
  hipEvent_t* const ev = ex->events;
  auto ev_sel = [&](int i) { return ev[1 + i]; };
  auto ev_done = [&](int i) { return ev[1 + n + i]; };
  auto ev_append = [&](int i) { return ev[1 + 2 * n + i]; };
  auto ev_aux = [&](int j) { return ev[1 + 3 * n + j]; };
  auto hip = [](hipError_t e) { return e == hipSuccess; };

  int aux_of[CSA2_GROUP_MAX_LAYERS], src_of[CSA2_GROUP_MAX_LAYERS], app_of[CSA2_GROUP_MAX_LAYERS];
  bool need_sel[CSA2_GROUP_MAX_LAYERS] = {}, need_done[CSA2_GROUP_MAX_LAYERS] = {};
  bool need_append[CSA2_GROUP_MAX_LAYERS] = {};
  int rr = 0;
  for (int i = 0; i < n; ++i) {
    const Step& p = steps[i];
    src_of[i] = -1;
    app_of[i] = -1;                                   // latest in-group append to this layer's cache before it
    for (int j = i - 1; j >= 0 && app_of[i] < 0; --j)
      if (steps[j].mode == CSA2_FULL && steps[j].a->n_new > 0 && steps[j].ca.kv == p.ca.kv) app_of[i] = j;
    if (p.mode == CSA2_REUSE) {
      for (int j = i - 1; j >= 0 && src_of[i] < 0; --j)
        if (steps[j].mode != CSA2_REUSE && steps[j].a->idx == p.a->idx && steps[j].a->cnt == p.a->cnt) src_of[i] = j;
      aux_of[i] = rr++ % n_aux;
      if (src_of[i] >= 0) need_sel[src_of[i]] = true;
      // the source's select comes after the append on s, else wait for it
      if (app_of[i] >= 0 && !(src_of[i] >= app_of[i])) need_append[app_of[i]] = true;
    } else {
      aux_of[i] = -1;
    }
    // conflicts that stream order does not cover
    for (int j = 0; j < i; ++j)
      if ((aux_of[j] >= 0 || aux_of[i] >= 0) && aux_of[j] != aux_of[i] && layers_conflict(steps[j], p))
        need_done[j] = true;
  }

  // s-side events are numbered in record order; an auxiliary stream that has
  // waited on event m is ordered after everything on s up to m
  int s_seq = 0;
  int aux_seen[CSA2_GROUP_MAX_AUX];
  bool aux_used[CSA2_GROUP_MAX_AUX] = {};
  for (int j = 0; j < n_aux; ++j) aux_seen[j] = 0;
  int seq_of_sel[CSA2_GROUP_MAX_LAYERS], seq_of_done[CSA2_GROUP_MAX_LAYERS], seq_of_append[CSA2_GROUP_MAX_LAYERS];
  bool start_recorded = false;
  auto record_s = [&](hipEvent_t e, int* seq) {
    *seq = 2 + s_seq++;
    return hip(hipEventRecord(e, s));
  };
  auto wait_s_event = [&](int x, hipEvent_t e, int seq) {
    if (aux_seen[x] >= seq) return true;
    aux_seen[x] = seq;
    return hip(hipStreamWaitEvent(ex->aux[x], e, 0));
  };
  auto ensure_start = [&](int x) {                   // x after the work on s before the call
    if (aux_seen[x] > 0) return true;
    if (!start_recorded) {
      if (!hip(hipEventRecord(ev[0], s))) return false;
      start_recorded = true;
    }
    aux_seen[x] = 1;
    return hip(hipStreamWaitEvent(ex->aux[x], ev[0], 0));
  };
  // A Reuse layer on its auxiliary stream (every event it waits on has been
  // recorded earlier in this call).
  auto enqueue_reuse = [&](int i) {
    const Step& p = steps[i];
    const int x = aux_of[i];
    hipStream_t ls = ex->aux[x];
    aux_used[x] = true;
    if (src_of[i] >= 0 && !wait_s_event(x, ev_sel(src_of[i]), seq_of_sel[src_of[i]])) return CSA2_ERR_HIP;
    const int ap = app_of[i];
    if (ap >= 0 && need_append[ap] && !wait_s_event(x, ev_append(ap), seq_of_append[ap])) return CSA2_ERR_HIP;
    if (!ensure_start(x)) return CSA2_ERR_HIP;
    for (int j = 0; j < i; ++j) {
      if (aux_of[j] == x || !need_done[j] || !layers_conflict(steps[j], p)) continue;
      const bool ok = aux_of[j] < 0 ? wait_s_event(x, ev_done(j), seq_of_done[j])
                                    : hip(hipStreamWaitEvent(ls, ev_done(j), 0));
      if (!ok) return CSA2_ERR_HIP;
    }
    csa2_status st = stage_attn(p, ls);
    if (st != CSA2_OK) return st;
    if (need_done[i] && !hip(hipEventRecord(ev_done(i), ls))) return CSA2_ERR_HIP;
    return CSA2_OK;
  };
  for (int i = 0; i < n; ++i) {
    const Step& p = steps[i];
    csa2_status st = CSA2_OK;
    if (aux_of[i] < 0) {
      for (int j = 0; j < i; ++j)                    // earlier auxiliary layers it conflicts with
        if (aux_of[j] >= 0 && need_done[j] && layers_conflict(steps[j], p) &&
            !hip(hipStreamWaitEvent(s, ev_done(j), 0)))
          return CSA2_ERR_HIP;
      // the append is done after stage_append, or after stage_scan when the
      // scan launch carries it
      const bool in_scan = append_in_scan(p);
      st = stage_append(p, s);
      if (st == CSA2_OK && need_append[i] && !in_scan && !record_s(ev_append(i), &seq_of_append[i])) st = CSA2_ERR_HIP;
      if (st == CSA2_OK) st = stage_scan(p, s);
      if (st == CSA2_OK && need_append[i] && in_scan && !record_s(ev_append(i), &seq_of_append[i])) st = CSA2_ERR_HIP;
      if (st == CSA2_OK) st = stage_select(p, s);
      if (st == CSA2_OK && need_sel[i] && !record_s(ev_sel(i), &seq_of_sel[i])) st = CSA2_ERR_HIP;
      if (st == CSA2_OK) st = stage_attn(p, s);
      if (st == CSA2_OK && need_done[i] && !record_s(ev_done(i), &seq_of_done[i])) st = CSA2_ERR_HIP;
      if (st != CSA2_OK) return st;
      continue;
    }
    st = enqueue_reuse(i);
    if (st != CSA2_OK) return st;
  }
  for (int j = 0; j < n_aux; ++j) {
    if (!aux_used[j]) continue;
    if (!hip(hipEventRecord(ev_aux(j), ex->aux[j])) || !hip(hipStreamWaitEvent(s, ev_aux(j), 0)))
      return CSA2_ERR_HIP;
  }
  return CSA2_OK;
}

}  // extern "C"
