// Pool set-up, residency updates, error reporting and the C ABI entry
// points of libhisparse.
//
// The pool follows the tiered layout of [P2] "vLLM GLM 5.3 优化：混合 HiSparse
// 卸载" §"混合 HiSparse 的技术实现" (per-page residency, per-request hot buffer)
// and §"关键架构细节" (hot buffers are pool pages leased to the request, 2x
// top-K rows by default).
#include <hip/hip_runtime.h>

#include <new>
#include <string.h>

#include "hs_internal.h"

namespace hs {

static thread_local int32_t g_last_hip_error = 0;

hs_status set_hip_error(hipError_t e) {
  g_last_hip_error = static_cast<int32_t>(e);
  return HS_ERR_HIP;
}

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// Validate a descriptor and derive all sizes and offsets.
static hs_status plan_layout(const hs_pool_desc* d, hs_pool_sizes* sz, hs_state_layout* lay,
                             Offsets* off) {
  if (!d || !sz) return HS_ERR_INVALID_ARGUMENT;
  const int ps = d->page_size;
  if (ps < 1 || ps > 1024 || (ps & (ps - 1))) return HS_ERR_INVALID_ARGUMENT;
  if (d->num_pool_pages < 1 || d->max_requests < 1 || d->max_context < 1) return HS_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->max_context > (int64_t)kTkChunk * kTkMaxChunks) return HS_ERR_CAPACITY;
  if (d->nope_dim != 512 || d->rope_dim != 64) return HS_ERR_UNSUPPORTED;
  if (d->kv_dtype != HS_F32 && d->kv_dtype != HS_BF16 && d->kv_dtype != HS_FP8_E4M3) return HS_ERR_UNSUPPORTED;
  if (d->top_k < 1 || d->top_k > kMaxTopK) return HS_ERR_INVALID_ARGUMENT;
  if (d->max_batch < 1 || d->max_batch > d->max_requests) return HS_ERR_INVALID_ARGUMENT;
  if (d->max_q_rows < 1 || d->select_q < 0 || d->select_q > kMaxSelectQ || d->host_rows < 1)
    return HS_ERR_INVALID_ARGUMENT;
  if ((int64_t)d->num_pool_pages * ps > (int64_t)INT32_MAX) return HS_ERR_CAPACITY;
  const int S = d->hot_rows == 0 ? 2 * d->top_k : d->hot_rows;
  if (S < d->top_k || S > kMaxHotRows) return HS_ERR_CAPACITY;
  if (S % ps != 0) return HS_ERR_INVALID_ARGUMENT;

  const size_t rb = d->kv_dtype == HS_F32 ? 4 * kRowDim : d->kv_dtype == HS_BF16 ? 2 * kRowDim : kRowDim;
  const int64_t pool_rows = (int64_t)d->num_pool_pages * ps;
  const int ppr = (d->max_context + ps - 1) / ps;
  const size_t R = (size_t)d->max_requests, B = (size_t)d->max_batch;
  const size_t K = (size_t)d->top_k;

  sz->row_bytes = rb;
  sz->pool_bytes = rb * (size_t)pool_rows;
  sz->pool_scale_bytes = d->kv_dtype == HS_FP8_E4M3 ? 4 * (size_t)pool_rows : 0;
  sz->hot_rows = S;
  sz->pages_per_request = ppr;
  // an fp8 host row carries its fp32 scale after the 576 code bytes (one
  // read per miss), padded to a multiple of 16 bytes
  sz->host_row_stride = d->kv_dtype == HS_FP8_E4M3 ? kHostRowStrideFp8 : rb;
  sz->host_store_bytes = sz->host_row_stride * (size_t)d->host_rows;

  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes, 256);
    return at;
  };
  hs_state_layout L{};
  L.ctx_len = take(4 * R);
  L.host_base = take(8 * R);
  L.page_table = take(4 * R * ppr);
  L.hot_pages = take(4 * R * (S / ps));
  L.rev = take(4 * R * (size_t)d->max_context);
  L.slot_tag = take(4 * R * S);
  L.slot_stamp = take(4 * R * S);
  L.lru_order = take(4 * R * S);
  L.step = take(4 * R);
  L.counters = take(8 * 3 * R);
  L.error = take(16);
  L.page_stamp = take(4 * R * ppr);
  L.host_valid = take(R * ppr);
  L.scratch = o;
  Offsets of{};
  of.zero_row = take(4 * kRowDim);
  const size_t max_chunks = ((size_t)d->max_context + kTkChunk - 1) / kTkChunk;
  const size_t SQ = d->select_q > 1 ? (size_t)d->select_q : 1;  // score rows per request
  of.sel_q = (int32_t)SQ;
  of.tk_count = take(4 * B * SQ * max_chunks);
  of.tk_max = take(4 * B * SQ * max_chunks);
  of.tk_cand = take(8 * B * SQ * max_chunks * kTkChunk);
  of.tk_bound = take(4 * R * SQ);
  of.rs_mdst = take(8 * B * (size_t)K);
  of.rs_mslot = take(4 * B * (size_t)K);
  of.rs_mold = take(4 * B * (size_t)K);
  of.rs_ticket = take(16 * B);  // per batch position: ticket, sequence, done
  of.ru_list = take(8 * B * (size_t)kRuMaxList);
  of.ru_ncopy = take(4 * B);
  of.at_part_rows = (int64_t)B * d->max_q_rows * kAttSplitCap;
  if (of.at_part_rows < kAttMinPartRows) of.at_part_rows = kAttMinPartRows;
  of.at_part_o = take(4 * (size_t)of.at_part_rows * kNope);
  of.at_part_lse = take(4 * (size_t)of.at_part_rows);
  L.total = o;
  sz->state_bytes = o;
  if (lay) *lay = L;
  if (off) *off = of;
  return HS_OK;
}

StateView make_view(const hs_pool* p) {
  StateView v{};
  uint8_t* s = p->state;
  v.ctx_len = reinterpret_cast<int32_t*>(s + p->lay.ctx_len);
  v.host_base = reinterpret_cast<int64_t*>(s + p->lay.host_base);
  v.page_table = reinterpret_cast<int32_t*>(s + p->lay.page_table);
  v.hot_pages = reinterpret_cast<int32_t*>(s + p->lay.hot_pages);
  v.rev = reinterpret_cast<int32_t*>(s + p->lay.rev);
  v.slot_tag = reinterpret_cast<int32_t*>(s + p->lay.slot_tag);
  v.slot_stamp = reinterpret_cast<int32_t*>(s + p->lay.slot_stamp);
  v.lru_order = reinterpret_cast<int32_t*>(s + p->lay.lru_order);
  v.step = reinterpret_cast<int32_t*>(s + p->lay.step);
  v.counters = reinterpret_cast<int64_t*>(s + p->lay.counters);
  v.error = reinterpret_cast<uint32_t*>(s + p->lay.error);
  v.page_stamp = reinterpret_cast<int32_t*>(s + p->lay.page_stamp);
  v.host_valid = s + p->lay.host_valid;
  v.max_requests = p->d.max_requests;
  v.max_context = p->d.max_context;
  v.pages_per_req = p->sz.pages_per_request;
  v.hot_rows = p->sz.hot_rows;
  v.hot_pages_per_req = p->sz.hot_rows / p->d.page_size;
  v.page_size = p->d.page_size;
  v.log2_ps = p->log2_ps;
  v.num_pool_pages = p->d.num_pool_pages;
  v.top_k = p->d.top_k;
  return v;
}

// ---------------------------------------------------------------- kernels
__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__global__ void k_iota_rows(int32_t* __restrict__ p, int rows, int cols) {
  const size_t n = (size_t)rows * cols;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = (int32_t)(i % cols);
}

// One request's residency update. One workgroup; every thread handles its
// own pages and slots, so no barrier is needed.
__global__ void k_set_residency(StateView v, int32_t req, int32_t ctx, int64_t base,
                                int32_t first_page, int32_t num_pages,
                                const int32_t* __restrict__ gpu_pages,
                                const int32_t* __restrict__ hot_page_ids, uint32_t flags) {
  const int tid = threadIdx.x;
  const int ps = v.page_size;
  int32_t* stamp = v.page_stamp + (size_t)req * v.pages_per_req;
  uint8_t* hv = v.host_valid + (size_t)req * v.pages_per_req;
  const bool fresh = (flags & HS_RESET_PAGES) != 0;
  const int old_pages = fresh ? 0 : (v.ctx_len[req] + ps - 1) / ps;
  const int new_pages = (ctx + ps - 1) / ps;
  const int n = v.step[req];
  __syncthreads();  // every thread has read the old context length
  if (tid == 0) {
    v.ctx_len[req] = ctx;
    v.host_base[req] = base;
  }
  if (fresh) {
    for (int p = tid; p < v.pages_per_req; p += blockDim.x) {
      stamp[p] = 0;
      hv[p] = 0;
    }
    __syncthreads();
  }
  // pages entering the context take the current step as their stamp
  for (int p = old_pages + tid; p < new_pages; p += blockDim.x) stamp[p] = n;
  int32_t* pt = v.page_table + (size_t)req * v.pages_per_req;
  for (int i = tid; i < num_pages; i += blockDim.x) {
    int32_t g = gpu_pages[i];
    if (g >= v.num_pool_pages || g < -1) {
      raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)req, (uint32_t)(first_page + i));
      g = -1;
    }
    pt[first_page + i] = g;
    hv[first_page + i] = (g < 0 || (flags & HS_HOST_COPY_VALID)) ? 1 : 0;
  }
  if (hot_page_ids) {
    int32_t* hp = v.hot_pages + (size_t)req * v.hot_pages_per_req;
    for (int i = tid; i < v.hot_pages_per_req; i += blockDim.x) {
      int32_t g = hot_page_ids[i];
      if (g < 0 || g >= v.num_pool_pages) {
        raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)req, (uint32_t)i);
        g = -1;
      }
      hp[i] = g;
    }
  }
  if (flags & HS_RESET_HOT) {
    const size_t so = (size_t)req * v.hot_rows;
    int32_t* rev = v.rev + (size_t)req * v.max_context;
    for (int s = tid; s < v.hot_rows; s += blockDim.x) {
      const int32_t t = v.slot_tag[so + s];
      if (t >= 0 && t < v.max_context) rev[t] = -1;
      v.slot_tag[so + s] = -1;
      v.slot_stamp[so + s] = 0;
      v.lru_order[so + s] = s;
    }
  }
}

__global__ void k_clear_error(uint32_t* err) {
  if (threadIdx.x < 4) err[threadIdx.x] = 0;
}

static void fill(uint8_t* base, size_t off, size_t bytes, uint32_t v, hipStream_t s) {
  const size_t n = bytes / 4;
  if (n == 0) return;
  const int blocks = (int)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096);
  k_fill_u32<<<blocks, 256, 0, s>>>(reinterpret_cast<uint32_t*>(base + off), n, v);
}

}  // namespace hs

using namespace hs;

extern "C" {

hs_status hs_pool_requirements(const hs_pool_desc* desc, hs_pool_sizes* out) {
  if (!desc || !out) return HS_ERR_INVALID_ARGUMENT;
  hs_pool_sizes sz{};
  hs_status st = plan_layout(desc, &sz, nullptr, nullptr);
  if (st == HS_OK) *out = sz;
  return st;
}

hs_status hs_init_pool(const hs_pool_desc* desc, void* pool_rows, float* pool_scales, void* state,
                       size_t state_bytes, hipStream_t stream, hs_pool** out) {
  if (!desc || !out || !pool_rows || !state) return HS_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  hs_pool_sizes sz{};
  hs_state_layout lay{};
  Offsets off{};
  hs_status st = plan_layout(desc, &sz, &lay, &off);
  if (st != HS_OK) return st;
  if (state_bytes < sz.state_bytes || (reinterpret_cast<uintptr_t>(state) & 255)) return HS_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(pool_rows) & 15)) return HS_ERR_INVALID_ARGUMENT;
  if (desc->kv_dtype == HS_FP8_E4M3 && !pool_scales) return HS_ERR_INVALID_ARGUMENT;

  hs_pool* p = new (std::nothrow) hs_pool{};
  if (!p) return HS_ERR_OUT_OF_MEMORY;
  p->d = *desc;
  p->d.hot_rows = sz.hot_rows;
  p->sz = sz;
  p->lay = lay;
  p->off = off;
  p->log2_ps = ilog2(desc->page_size);
  p->pool_rows_n = (int64_t)desc->num_pool_pages * desc->page_size;
  p->pool_rows = static_cast<uint8_t*>(pool_rows);
  p->pool_scales = desc->kv_dtype == HS_FP8_E4M3 ? pool_scales : nullptr;
  p->state = static_cast<uint8_t*>(state);
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return set_hip_error(e);
  }
  // device address of this device's no-alloc scratch array (resolved once
  // per device, with the device current)
  st = static_scratch_address(p->device, &p->static_scratch);
  if (st != HS_OK) {
    delete p;
    return st;
  }
  // Pinned host store, mapped into the device address space so that the
  // resolve kernel reads single rows directly over PCIe.
  void* h = nullptr;
  e = hipHostMalloc(&h, sz.host_store_bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess || !h) {
    delete p;
    g_last_hip_error = (int32_t)e;
    return HS_ERR_OUT_OF_MEMORY;
  }
  p->host_rows = h;
  p->host_scales = desc->kv_dtype == HS_FP8_E4M3
                       ? reinterpret_cast<float*>(static_cast<uint8_t*>(h) + kRowDim)
                       : nullptr;

  // State initialisation: everything zero, then the -1 tables and the
  // identity LRU order (all stamps 0, so ascending slot number).
  uint8_t* s8 = p->state;
  fill(s8, 0, sz.state_bytes, 0u, stream);
  const size_t R = desc->max_requests;
  fill(s8, lay.page_table, 4 * R * sz.pages_per_request, 0xFFFFFFFFu, stream);
  fill(s8, lay.hot_pages, 4 * R * (sz.hot_rows / desc->page_size), 0xFFFFFFFFu, stream);
  fill(s8, lay.rev, 4 * R * (size_t)desc->max_context, 0xFFFFFFFFu, stream);
  fill(s8, lay.slot_tag, 4 * R * sz.hot_rows, 0xFFFFFFFFu, stream);
  k_iota_rows<<<1024, 256, 0, stream>>>(reinterpret_cast<int32_t*>(s8 + lay.lru_order),
                                         desc->max_requests, sz.hot_rows);
  e = hipGetLastError();
  if (e != hipSuccess) {
    (void)hipHostFree(p->host_rows);
    delete p;
    return set_hip_error(e);
  }
  *out = p;
  return HS_OK;
}

hs_status hs_host_rows(hs_pool* pool, void** rows, float** scales) {
  if (!pool || !rows) return HS_ERR_INVALID_ARGUMENT;
  *rows = pool->host_rows;
  if (scales) *scales = pool->host_scales;
  return HS_OK;
}

hs_status hs_set_residency(hs_pool* pool, int32_t req, int32_t context_len, int64_t host_row_base,
                           int32_t first_page, int32_t num_pages, const int32_t* gpu_page_ids,
                           const int32_t* hot_page_ids, uint32_t flags, hipStream_t stream) {
  if (!pool) return HS_ERR_INVALID_ARGUMENT;
  const hs_pool_desc& d = pool->d;
  if (req < 0 || req >= d.max_requests) return HS_ERR_INVALID_ARGUMENT;
  if (context_len < 0 || context_len > d.max_context) return HS_ERR_INVALID_ARGUMENT;
  if (host_row_base < 0 || host_row_base + context_len > d.host_rows) return HS_ERR_INVALID_ARGUMENT;
  if (first_page < 0 || num_pages < 0 || first_page + num_pages > pool->sz.pages_per_request)
    return HS_ERR_INVALID_ARGUMENT;
  if (num_pages > 0 && !gpu_page_ids) return HS_ERR_INVALID_ARGUMENT;
  if (flags & ~(uint32_t)(HS_RESET_HOT | HS_HOST_COPY_VALID | HS_RESET_PAGES)) return HS_ERR_INVALID_ARGUMENT;
  k_set_residency<<<1, 1024, 0, stream>>>(make_view(pool), req, context_len, host_row_base,
                                          first_page, num_pages, gpu_page_ids, hot_page_ids, flags);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

hs_status hs_update_residency(hs_pool* pool, const int32_t* req_ids, int32_t n_req,
                              const int32_t* budget_pages, int32_t max_copy_pages,
                              int32_t max_demote_pages, int32_t* freed_out, int32_t* counts_out,
                              hipStream_t stream) {
  if (!pool || !req_ids || n_req < 0) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if (max_copy_pages < 0 || max_copy_pages > kRuMaxList) return HS_ERR_INVALID_ARGUMENT;
  if (max_demote_pages < 0 || max_demote_pages > kRuMaxList) return HS_ERR_INVALID_ARGUMENT;
  if (max_demote_pages > 0 && !freed_out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req == 0) return HS_OK;
  return launch_update_residency(pool, req_ids, n_req, budget_pages, max_copy_pages, max_demote_pages,
                                 freed_out, counts_out, stream);
}

hs_status hs_select_topk(hs_pool* pool, const float* scores, int64_t score_stride,
                         const int32_t* req_ids, int32_t n_req, int32_t* idx_out, hipStream_t stream) {
  if (!pool || !scores || !req_ids || !idx_out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if (score_stride < pool->d.max_context || (score_stride & 3)) return HS_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(scores) & 15) return HS_ERR_INVALID_ARGUMENT;
  if (n_req == 0) return HS_OK;
  return launch_topk(pool, scores, score_stride, req_ids, n_req, 1, pool->d.top_k, idx_out, stream);
}

hs_status hs_select_topk_union(hs_pool* pool, const float* scores, int64_t score_stride,
                               const int32_t* req_ids, int32_t n_req, int32_t q_per_req,
                               int32_t k_per_token, int32_t* idx_out, int32_t* union_out,
                               int32_t* upos_out, hipStream_t stream) {
  if (!pool || !scores || !req_ids || !idx_out || !union_out || !upos_out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0 || q_per_req < 1 || k_per_token < 1) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch || q_per_req > pool->off.sel_q) return HS_ERR_CAPACITY;
  if ((int64_t)q_per_req * k_per_token > pool->d.top_k) return HS_ERR_CAPACITY;
  if (score_stride < pool->d.max_context || (score_stride & 3)) return HS_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(scores) & 15) return HS_ERR_INVALID_ARGUMENT;
  if (n_req == 0) return HS_OK;
  hs_status st = launch_topk(pool, scores, score_stride, req_ids, n_req, q_per_req, k_per_token, idx_out, stream);
  if (st != HS_OK) return st;
  return launch_topk_union(pool, idx_out, n_req, q_per_req, k_per_token, union_out, upos_out, stream);
}

hs_status hs_select_resolve(hs_pool* pool, const float* scores, int64_t score_stride, const int32_t* req_ids,
                            int32_t n_req, int32_t* idx_out, int32_t* plan_out, int32_t* counts_out,
                            hipStream_t stream) {
  if (!pool || !scores || !req_ids || !idx_out || !plan_out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if (score_stride < pool->d.max_context || (score_stride & 3)) return HS_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(scores) & 15) return HS_ERR_INVALID_ARGUMENT;
  if (n_req == 0) return HS_OK;
  return launch_select_resolve(pool, scores, score_stride, req_ids, n_req, idx_out, plan_out, counts_out, stream);
}

hs_status hs_indexer_scores(hs_pool* pool, const void* iq, const float* iw, const void* ik, int64_t ik_stride,
                            int32_t n_heads, const int32_t* req_ids, int32_t n_req, float* scores,
                            int64_t score_stride, hipStream_t stream) {
  if (!pool || !iq || !iw || !ik || !req_ids || !scores) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0 || n_heads < 16 || n_heads > 64 || (n_heads % 16)) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if (ik_stride < pool->d.max_context || score_stride < pool->d.max_context) return HS_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(iq) | reinterpret_cast<uintptr_t>(ik)) & 15) return HS_ERR_INVALID_ARGUMENT;
  if (n_req == 0) return HS_OK;
  return hs::launch_indexer_scores(pool, iq, iw, ik, ik_stride, n_heads, req_ids, n_req, scores, score_stride,
                                   stream);
}

hs_status hs_resolve_rows(hs_pool* pool, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                          int32_t* plan_out, int32_t* counts_out, hipStream_t stream) {
  if (!pool || !idx || !req_ids || !plan_out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if (n_req == 0) return HS_OK;
  return launch_resolve(pool, idx, req_ids, n_req, plan_out, counts_out, stream);
}

hs_status hs_sparse_mla_decode(hs_pool* pool, const void* q, int32_t q_dtype, int32_t n_req,
                               int32_t q_per_req, int32_t n_heads, const int32_t* plan,
                               float sm_scale, float* out, float* lse_out, hipStream_t stream) {
  if (!pool || !q || !plan || !out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0 || q_per_req < 1 || n_heads < 1) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if ((int64_t)q_per_req * n_heads > pool->d.max_q_rows) return HS_ERR_CAPACITY;
  const int kv = pool->d.kv_dtype;
  const bool ok = (kv == HS_F32 && q_dtype == HS_F32) ||
                  ((kv == HS_BF16 || kv == HS_FP8_E4M3) && q_dtype == HS_BF16);
  if (!ok) return HS_ERR_UNSUPPORTED;
  if (n_req == 0) return HS_OK;
  return launch_attention(pool, q, q_dtype, n_req, q_per_req, n_heads, plan, nullptr, pool->d.top_k, 1, sm_scale,
                          out, lse_out, reinterpret_cast<float*>(pool->state + pool->off.at_part_o),
                          reinterpret_cast<float*>(pool->state + pool->off.at_part_lse), pool->off.at_part_rows,
                          stream);
}

hs_status hs_sparse_mla_decode_noalloc(hs_pool* pool, const void* q, int32_t q_dtype, int32_t n_req,
                                       int32_t q_per_req, int32_t n_heads, const int32_t* plan,
                                       float sm_scale, float* out, float* lse_out, hipStream_t stream) {
  if (!pool || !q || !plan || !out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0 || q_per_req < 1 || n_heads < 1) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if ((int64_t)q_per_req * n_heads > pool->d.max_q_rows) return HS_ERR_CAPACITY;
  const int kv = pool->d.kv_dtype;
  const bool ok = (kv == HS_F32 && q_dtype == HS_F32) ||
                  ((kv == HS_BF16 || kv == HS_FP8_E4M3) && q_dtype == HS_BF16);
  if (!ok) return HS_ERR_UNSUPPORTED;
  if (!pool->static_scratch) return HS_ERR_INVALID_ARGUMENT;
  int dev = -1;
  HS_HIP_CHECK(hipGetDevice(&dev));
  if (dev != pool->device) return HS_ERR_INVALID_ARGUMENT;  // the scratch address is per device
  if (n_req == 0) return HS_OK;
  float* part_o = reinterpret_cast<float*>(pool->static_scratch);
  float* part_lse = part_o + (size_t)kStaticPartRows * kNope;
  return launch_attention(pool, q, q_dtype, n_req, q_per_req, n_heads, plan, nullptr, pool->d.top_k, 1, sm_scale,
                          out, lse_out, part_o, part_lse, kStaticPartRows, stream);
}

hs_status hs_sparse_mla_decode_union(hs_pool* pool, const void* q, int32_t q_dtype, int32_t n_req,
                                     int32_t q_per_req, int32_t n_heads, const int32_t* plan,
                                     const int32_t* upos, int32_t k_per_token, float sm_scale, float* out,
                                     float* lse_out, hipStream_t stream) {
  if (!pool || !q || !plan || !upos || !out) return HS_ERR_INVALID_ARGUMENT;
  if (n_req < 0 || q_per_req < 1 || n_heads < 1 || k_per_token < 1) return HS_ERR_INVALID_ARGUMENT;
  if (n_req > pool->d.max_batch) return HS_ERR_CAPACITY;
  if ((int64_t)q_per_req * n_heads > pool->d.max_q_rows) return HS_ERR_CAPACITY;
  if ((int64_t)q_per_req * k_per_token > pool->d.top_k) return HS_ERR_CAPACITY;
  const int kv = pool->d.kv_dtype;
  const bool ok = (kv == HS_F32 && q_dtype == HS_F32) ||
                  ((kv == HS_BF16 || kv == HS_FP8_E4M3) && q_dtype == HS_BF16);
  if (!ok) return HS_ERR_UNSUPPORTED;
  if (n_req == 0) return HS_OK;
  // query token t of request i is query row group i * q_per_req + t: its
  // n_heads rows ([n_req][q_per_req][n_heads][576] is [n_req * q_per_req]
  // [n_heads][576]) read the union plan row i through upos row i * q_per_req + t
  return launch_attention(pool, q, q_dtype, n_req * q_per_req, 1, n_heads, plan, upos, k_per_token, q_per_req,
                          sm_scale, out, lse_out, reinterpret_cast<float*>(pool->state + pool->off.at_part_o),
                          reinterpret_cast<float*>(pool->state + pool->off.at_part_lse), pool->off.at_part_rows,
                          stream);
}

hs_status hs_get_state_layout(const hs_pool* pool, hs_state_layout* out) {
  if (!pool || !out) return HS_ERR_INVALID_ARGUMENT;
  *out = pool->lay;
  return HS_OK;
}

hs_status hs_get_device_error(hs_pool* pool, uint32_t code[4], hipStream_t stream) {
  if (!pool || !code) return HS_ERR_INVALID_ARGUMENT;
  HS_HIP_CHECK(hipStreamSynchronize(stream));
  HS_HIP_CHECK(hipMemcpy(code, pool->state + pool->lay.error, 16, hipMemcpyDeviceToHost));
  return code[0] ? HS_ERR_DEVICE : HS_OK;
}

hs_status hs_clear_device_error(hs_pool* pool, hipStream_t stream) {
  if (!pool) return HS_ERR_INVALID_ARGUMENT;
  k_clear_error<<<1, 64, 0, stream>>>(reinterpret_cast<uint32_t*>(pool->state + pool->lay.error));
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

int32_t hs_last_hip_error(void) { return g_last_hip_error; }

const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "ok";
    case HS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case HS_ERR_CAPACITY: return "exceeds pool capacity";
    case HS_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case HS_ERR_HIP: return "HIP runtime error";
    case HS_ERR_OUT_OF_MEMORY: return "out of host memory";
    case HS_ERR_DEVICE: return "device-side data error";
  }
  return "unknown status";
}

hs_status hs_destroy_pool(hs_pool* pool) {
  if (!pool) return HS_OK;
  hipError_t e = hipDeviceSynchronize();
  if (pool->host_rows) (void)hipHostFree(pool->host_rows);
  delete pool;
  if (e != hipSuccess) return set_hip_error(e);
  return HS_OK;
}

}  // extern "C"
