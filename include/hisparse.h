/*
 * hisparse.h — C ABI of the tiered sparse-MLA decode step (libhisparse.so).
 *
 * One decode step of one sparse-MLA layer over a latent KV cache whose pages
 * live either in GPU memory or only in pinned host memory:
 *   hs_indexer_scores   per-token indexer scores (upstream of the step);
 *   hs_select_topk      the indexer's top-K over per-token scores;
 *   hs_resolve_rows     one fused pass that turns each selected token into a
 *                       physical pool row: read in place when its page is on
 *                       the GPU, read from the request's hot buffer (and its
 *                       LRU entry refreshed) when it is hot, or, on a miss,
 *                       copy that single row from pinned host memory into
 *                       the least-recently-used hot slot;
 *   hs_sparse_mla_decode absorbed-MLA decode attention over only those rows.
 * Around the step, hs_update_residency copies completed GPU pages to the
 * host store ahead of need and, under a GPU page budget, moves a request's
 * coldest pages back to host memory.
 *
 * Multi-layer steps ([P2] §"关键架构细节", lightweight execution: the
 * sparse-MLA work of all layers is issued once per step, in the model's
 * stream order). A request slot is the unit of state (page table, hot
 * buffer, LRU state, top-K bound), so one pool holds the slots of every
 * (layer, request) pair — numbered layer-major, slot = layer * R + r — with
 * their rows in the shared page pool and host store, as the hot buffers are
 * ordinary blocks leased from one shared pool. One call of each per-step
 * entry point with req_ids listing the slots of every layer then selects,
 * resolves and attends all layers in one launch per stage; inputs and
 * outputs are indexed by position in req_ids (scores [n][stride], queries
 * [n][Q][H][576], plans [n][K], outputs [n][Q][H][512]).
 *
 * Pages describing the method (cited by title and section):
 *   [P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" (agentlenshq.com)
 *   [P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈" (kongchang.com)
 *
 * Conventions shared by every call
 *   - Every call returns an hs_status; nothing throws across the ABI.
 *   - The per-step calls (select_topk, resolve_rows, sparse_mla_decode) and
 *     set_residency only enqueue kernels on the given stream. They never
 *     allocate, never synchronise and never read device memory from the
 *     host, so a caller may capture them in a hipGraph. Their arguments are
 *     validated on the host before anything is enqueued; on an error return
 *     nothing was enqueued.
 *   - Data errors that only the device can see (a selected index past the
 *     context length, a page id outside the pool, a plan row outside the
 *     pool) set a sticky device error word (first error wins) and the
 *     offending entry is treated as absent. Read it with
 *     hs_get_device_error (not capturable).
 *   - Ownership: the caller allocates every device buffer (pool rows, fp8
 *     scales, the state workspace, inputs and outputs) and keeps it alive
 *     until hs_destroy_pool. The library owns only its host-side handle and
 *     the pinned host row store, which it allocates in hs_init_pool.
 *   - A pool handle is not thread-safe; calls on one pool must be ordered
 *     on one stream (or synchronised by the caller across streams).
 *   - All element indices are int32 unless stated; host store rows int64.
 */
#ifndef HISPARSE_H_
#define HISPARSE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;  /* HIP stream handle (NULL = null stream) */
typedef struct hs_pool hs_pool;            /* opaque pool handle */

typedef enum hs_status {
  HS_OK = 0,
  HS_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or out-of-range id */
  HS_ERR_CAPACITY = 2,         /* exceeds what the pool was built for (e.g. hot_rows < top_k) */
  HS_ERR_UNSUPPORTED = 3,      /* dtype or shape combination not implemented */
  HS_ERR_HIP = 4,              /* a HIP runtime call failed; see hs_last_hip_error */
  HS_ERR_OUT_OF_MEMORY = 5,    /* the pinned host store could not be allocated */
  HS_ERR_DEVICE = 6            /* hs_get_device_error found a device-side data error */
} hs_status;

typedef enum hs_dtype {
  HS_F32 = 0,       /* IEEE fp32 */
  HS_BF16 = 1,      /* bfloat16 */
  HS_FP8_E4M3 = 2   /* OCP FP8 E4M3 ("fn", max 448), with one fp32 scale per row */
} hs_dtype;

/* Device error word codes (hs_get_device_error). */
enum {
  HS_DEV_OK = 0,
  HS_DEV_INDEX_RANGE = 1,  /* a selected token >= the request's context length */
  HS_DEV_PAGE_RANGE = 2,   /* a page-table or hot-page id >= num_pool_pages */
  HS_DEV_PLAN_RANGE = 3,   /* an attention plan row >= the pool's row count */
  HS_DEV_REQUEST_RANGE = 4, /* a req_ids entry outside [0, max_requests) */
  HS_DEV_TIMEOUT = 5       /* a bounded wait inside hs_resolve_rows gave up (info: batch position and
                              plan position of the copy wave, or 0xFFFFFFFF for the end-of-launch wait);
                              the positions of that wave were not copied, so the plan of that call must
                              not be used; the next call starts clean */
};

/* hs_set_residency flags */
enum {
  HS_RESET_HOT = 1u,        /* empty the request's hot buffer (nothing hot) */
  HS_HOST_COPY_VALID = 2u,  /* the host store already holds the rows of the GPU pages given */
  HS_RESET_PAGES = 4u       /* a new request: page stamps and host-copy marks start from zero */
};

/*
 * Pool description. The latent row layout is MLA's: nope_dim (512) dims that
 * serve as the value and nope_dim + rope_dim (576) dims that serve as the key
 * ([P3] §"稀疏MLA的核心思想", MLA note). Tokens are grouped in pages of
 * page_size rows ([P3] PagedAttention note). Each request's hot buffer is
 * hot_rows slots made of ordinary pool pages leased to it
 * ([P2] §"关键架构细节", first bullet; [P3] §"复用现有内存池"); hot_rows = 0
 * selects the default 2 x top_k.
 */
typedef struct hs_pool_desc {
  int32_t page_size;      /* tokens per page: power of two in [1, 1024] */
  int32_t num_pool_pages; /* device pool pages (resident pages + leased hot pages) */
  int32_t max_requests;   /* request ids are 0 .. max_requests-1 */
  int32_t max_context;    /* most tokens any request holds: 1 .. 4,194,304 (the top-K
                             filter's 2,048 chunks of 2,048 scores) */
  int32_t nope_dim;       /* must be 512 */
  int32_t rope_dim;       /* must be 64 */
  int32_t kv_dtype;       /* hs_dtype of the stored rows */
  int32_t top_k;          /* K: 1 .. 4096 */
  int32_t hot_rows;       /* S per request; 0 -> 2*top_k; must be >= top_k,
                             <= 8192 and a multiple of page_size */
  int32_t max_batch;      /* most requests in one per-step call, 1 .. max_requests */
  int32_t max_q_rows;     /* most q_per_req * n_heads in one sparse_mla_decode call */
  int32_t select_q;       /* most query tokens per request with a selection of their own
                             (hs_select_topk_union): 0 or 1 (plain steps only) .. 8 */
  int64_t host_rows;      /* rows in the pinned host store, >= 1 */
} hs_pool_desc;

/* Sizes the caller must provide, derived from a descriptor. */
typedef struct hs_pool_sizes {
  size_t row_bytes;          /* bytes of one stored row payload: 2304 f32, 1152 bf16, 576 fp8 */
  size_t pool_bytes;         /* device pool rows: num_pool_pages * page_size * row_bytes */
  size_t pool_scale_bytes;   /* fp8 only: 4 * pool rows (one fp32 scale per row); else 0 */
  size_t state_bytes;        /* device state workspace (tables, LRU state, scratch) */
  size_t host_store_bytes;   /* pinned host memory hs_init_pool allocates */
  int32_t hot_rows;          /* resolved S */
  int32_t pages_per_request; /* ceil(max_context / page_size) */
  size_t host_row_stride;    /* bytes between consecutive rows of the host store: row_bytes, or
                                640 for fp8 (576 code bytes, the fp32 row scale at byte 576, then
                                60 unused bytes), so that a missed row and its scale are one read
                                of 37 16-byte chunks starting on a 128-byte boundary */
} hs_pool_sizes;

/* Byte offsets of the state arrays inside the caller's workspace, so that a
 * caller can inspect (never write) the residency and LRU state. */
typedef struct hs_state_layout {
  size_t ctx_len;     /* int32 [max_requests]: context length L_r */
  size_t host_base;   /* int64 [max_requests]: host store row of token 0 */
  size_t page_table;  /* int32 [max_requests][pages_per_request]: pool page or -1 (host only) */
  size_t hot_pages;   /* int32 [max_requests][hot_rows/page_size]: leased pool pages */
  size_t rev;         /* int32 [max_requests][max_context]: hot slot holding token t, or -1 */
  size_t slot_tag;    /* int32 [max_requests][hot_rows]: token in slot s, or -1 */
  size_t slot_stamp;  /* int32 [max_requests][hot_rows]: step of last hit or fill, 0 = never */
  size_t lru_order;   /* int32 [max_requests][hot_rows]: slots by ascending (stamp, slot) */
  size_t step;        /* int32 [max_requests]: resolves done so far */
  size_t counters;    /* int64 [max_requests][3]: cumulative resident, hot, miss */
  size_t error;       /* uint32 [4]: code, request, index, 0 */
  size_t page_stamp;  /* int32 [max_requests][pages_per_request]: last step whose top-K
                         selected a token of the page, or the step at which the page
                         entered the context; 0 = neither */
  size_t host_valid;  /* uint8 [max_requests][pages_per_request]: 1 when the host store
                         holds the page's rows (always for host-only pages) */
  size_t scratch;     /* start of internal scratch */
  size_t total;       /* == hs_pool_sizes.state_bytes */
} hs_state_layout;

/* Derive buffer sizes from a descriptor. Pure host computation.
 * Errors: INVALID_ARGUMENT (null or malformed descriptor), CAPACITY
 * (hot_rows < top_k or > 8192, max_context > 4,194,304, more than 2^31 - 1
 * pool rows), UNSUPPORTED (dims other than 512 + 64, unknown kv_dtype). */
hs_status hs_pool_requirements(const hs_pool_desc* desc, hs_pool_sizes* out);

/* Create a pool over caller-owned device memory.
 *   pool_rows    device, >= pool_bytes, row r at byte offset r * row_bytes;
 *                physical row r = page * page_size + offset-in-page
 *   pool_scales  device fp32 [pool rows] for HS_FP8_E4M3, else NULL
 *   state        device workspace, >= state_bytes, 256-byte aligned
 * Allocates the pinned host row store (host_rows rows of host_row_stride
 * bytes; an fp8 row carries its fp32 scale), mapped for direct device reads
 * over PCIe, and
 * enqueues the state initialisation on `stream` (every page host-only, every
 * hot buffer empty, counters and the error word zero). *out receives the
 * handle. Errors: those of hs_pool_requirements, INVALID_ARGUMENT (null or
 * misaligned pointer, state_bytes too small), OUT_OF_MEMORY, HIP. */
hs_status hs_init_pool(const hs_pool_desc* desc, void* pool_rows, float* pool_scales,
                       void* state, size_t state_bytes, hipStream_t stream, hs_pool** out);

/* Pinned host store of the pool ([P2] §"混合 HiSparse 的技术实现", state 2:
 * misses are copied from pinned host memory). *rows: host_rows rows, row r
 * at byte r * host_row_stride, its first row_bytes bytes the row; *scales:
 * for fp8 pools the fp32 scale of row 0 (row r's at byte r * host_row_stride
 * of *scales), else NULL. The caller
 * fills it (the store keeps a copy of every row, so any page can be
 * demoted at any time). Errors: INVALID_ARGUMENT. */
hs_status hs_host_rows(hs_pool* pool, void** rows, float** scales);

/* Set request `req`'s context length and page residency (stream-ordered).
 *   context_len    L_r, 0 .. max_context
 *   host_row_base  host store row holding token 0; tokens 0..L_r-1 map to
 *                  rows host_row_base .. host_row_base + L_r - 1
 *   first_page, num_pages, gpu_page_ids
 *                  device int32 [num_pages]: the pool page holding logical
 *                  page first_page + i, or -1 when it lives only on host
 *                  ([P2] §"混合 HiSparse 的技术实现": residency is tracked
 *                  per page). num_pages may be 0 (gpu_page_ids then unused).
 *   hot_page_ids   device int32 [hot_rows/page_size]: pool pages leased as the
 *                  request's hot buffer, or NULL to keep the current lease
 *                  (must be given once before the first resolve)
 *   flags          HS_RESET_HOT empties the hot buffer ([P2] state 3: a
 *                  request that starts host-only loads rows only on demand);
 *                  HS_HOST_COPY_VALID: the host store already holds the rows
 *                  of the GPU pages given here (else they count as not yet
 *                  copied; host-only pages always hold a host copy);
 *                  HS_RESET_PAGES: clear the request's page stamps and
 *                  host-copy marks first (a new request in this slot)
 * Pages that enter the context (from ceil(old L / page_size) up to
 * ceil(L_r / page_size)) take the request's current step as page stamp.
 * No hot invalidation is needed when pages move: a page that is back on GPU
 * is read in place before any stale hot copy. Errors: INVALID_ARGUMENT. */
hs_status hs_set_residency(hs_pool* pool, int32_t req, int32_t context_len,
                           int64_t host_row_base, int32_t first_page, int32_t num_pages,
                           const int32_t* gpu_page_ids, const int32_t* hot_page_ids,
                           uint32_t flags, hipStream_t stream);

/* Indexer top-K ([P3] §"稀疏MLA的核心思想": decode attends only to the
 * top-K tokens; [P2] §"解决 KV 缓存内存压力"). For each i < n_req, with
 * r = req_ids[i] (device int32 [n_req]) and L = L_r read on the device:
 * writes idx_out[i][0..top_k) (device int32) = the min(top_k, L) token
 * indices with the largest scores[i * score_stride + t], t < L; equal scores
 * keep the lower index; -0.0 equals +0.0; listed in ascending index order,
 * padded with -1. NaN scores are not supported. scores: device fp32, 16-byte
 * aligned, row i valid over its first L entries; score_stride >= max_context
 * and a multiple of 4.
 * Errors: INVALID_ARGUMENT, CAPACITY (n_req > max_batch). */
hs_status hs_select_topk(hs_pool* pool, const float* scores, int64_t score_stride,
                         const int32_t* req_ids, int32_t n_req, int32_t* idx_out,
                         hipStream_t stream);

/* Top-K of a speculative step, one selection per query token, and their
 * union ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" §"与 vLLM 栈的集成",
 * speculative decoding: one resolve plan per step serves every query token
 * of a request, which share its hot state). Query token t of request
 * r = req_ids[i] has its own indexer scores and its own survivor bound.
 *   scores     device fp32 [n_req][q_per_req][score_stride] (16-byte aligned,
 *              score_stride >= max_context and a multiple of 4): row
 *              i * q_per_req + t, valid over its first L_r entries
 *   idx_out    device int32 [n_req][q_per_req][k_per_token]: the min(k, L_r)
 *              selected tokens of each query token, as hs_select_topk
 *   union_out  device int32 [n_req][top_k]: the distinct tokens of a
 *              request's selections, ascending, -1 padded (the input of
 *              hs_resolve_rows, whose plan then covers every query token)
 *   upos_out   device int32 [n_req][q_per_req][k_per_token]: the union
 *              position of each selected token (-1 for padding), the map
 *              hs_sparse_mla_decode_union reads the plan through
 * q_per_req <= select_q and q_per_req * k_per_token <= top_k (so every union
 * fits). Errors: INVALID_ARGUMENT, CAPACITY; a request id out of range raises
 * HS_DEV_REQUEST_RANGE and its rows are all -1. */
hs_status hs_select_topk_union(hs_pool* pool, const float* scores, int64_t score_stride,
                               const int32_t* req_ids, int32_t n_req, int32_t q_per_req,
                               int32_t k_per_token, int32_t* idx_out, int32_t* union_out,
                               int32_t* upos_out, hipStream_t stream);

/* Indexer scores, the input of hs_select_topk ([P3] §"稀疏MLA的核心思想": the
 * indexer picks the tokens that enter attention; [P2] §"与 vLLM 栈的集成",
 * indexer KV item: the indexer keeps a per-token key cache of its own). The
 * pages give no formula; the one computed (the lightning-indexer form) is,
 * for each i < n_req, r = req_ids[i] (device int32) and t < L_r (read on the
 * device):
 *     scores[i * score_stride + t] = sum_j iw[i][j] * max(0, <iq[i][j], ik_r[t]>)
 * over heads j < n_heads, in fp32 (exact bf16 products, fp32 sums).
 *   iq      device bf16 [n_req][n_heads][128], 16-byte aligned
 *   iw      device fp32 [n_req][n_heads]
 *   ik      device bf16, 16-byte aligned: token t of request slot r at
 *           ik + (r * ik_stride + t) * 128 (elements); ik_stride >= max_context
 *           rows; rows of tokens < L_r must be valid
 *   n_heads 16, 32, 48 or 64
 *   scores  device fp32, row i at scores + i * score_stride (score_stride >=
 *           max_context); entries t >= L_r are left untouched
 * Graph-capturable like the per-step calls. Errors: INVALID_ARGUMENT,
 * CAPACITY (n_req > max_batch); a req_ids entry outside [0, max_requests)
 * raises HS_DEV_REQUEST_RANGE and that row is not written. */
hs_status hs_indexer_scores(hs_pool* pool, const void* iq, const float* iw, const void* ik,
                            int64_t ik_stride, int32_t n_heads, const int32_t* req_ids,
                            int32_t n_req, float* scores, int64_t score_stride,
                            hipStream_t stream);

/* Fused resolve ([P2] §"混合 HiSparse 的技术实现", state 2: one fused kernel
 * handles the top-K results — resident rows read in place, hot rows read and
 * their LRU entry refreshed, a miss copies the single row from pinned host
 * memory into the LRU slot; [P3] §"融合内核与CUDA图兼容"). For each i < n_req
 * (request r = req_ids[i]), over idx[i][0..top_k) (device int32, ascending,
 * -1 padded, as hs_select_topk writes it):
 *   - classify each token t: RESIDENT if its page is on GPU, else HOT if a
 *     hot slot holds it, else MISS;
 *   - every HOT slot gets stamp n (this request's n-th resolve);
 *   - the misses, in ascending token order, take the slots not touched this
 *     step in ascending (stamp, slot) order; an evicted token loses its slot;
 *     each miss's row (and fp8 scale) is copied from the host store into its
 *     slot's pool row;
 *   - plan_out[i][j] (device int32 [n_req][top_k]) = the physical pool row
 *     holding token idx[i][j] (page * page_size + offset for RESIDENT, the
 *     slot's leased row otherwise), -1 for padding;
 *   - counts_out[i] (device int32 [n_req][3], may be NULL) = resident, hot,
 *     miss counts; they sum to min(top_k, L_r).
 * Each request's step counter advances by one. A request must appear at most
 * once per call. Errors: INVALID_ARGUMENT, CAPACITY.
 * A copy workgroup waits for its request's plan with a bounded number of
 * polls (2^20, at least 0.1 s; the environment variable
 * HS_RESOLVE_SPIN_LIMIT, read at each call, overrides it for tests). A wait
 * that gives up raises HS_DEV_TIMEOUT and copies nothing for its positions:
 * that call's plan and the hot buffers of its requests are then unusable;
 * after hs_clear_device_error and HS_RESET_HOT on those requests the next
 * call is exact (a destination published late by the call that gave up
 * carries that call's epoch and is never taken by a later call). */
hs_status hs_resolve_rows(hs_pool* pool, const int32_t* idx, const int32_t* req_ids,
                          int32_t n_req, int32_t* plan_out, int32_t* counts_out,
                          hipStream_t stream);

/* hs_select_topk followed by hs_resolve_rows in fewer launches: the top-K
 * filter kernel, then one kernel in which each request's bookkeeping
 * workgroup first selects its top-K and keeps the selection for the resolve
 * ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" §"混合 HiSparse 的技术实现": the
 * fused kernel handles the top-K results; [P3] §"融合内核与CUDA图兼容"). The
 * same arguments as the two calls (scores as hs_select_topk, idx_out then
 * holds the selection, plan_out and counts_out as hs_resolve_rows) and the
 * same results, bit for bit; the device state advances as after the two
 * calls. Errors: those of the two calls (HS_DEV_TIMEOUT also covers a copy
 * workgroup's bounded wait for the selection), and UNSUPPORTED when one
 * workgroup's LDS (160 KiB) cannot hold the select's tables, the
 * bookkeeping tables and the selection together (only with a very small
 * page size and many hot rows; the two calls work there). */
hs_status hs_select_resolve(hs_pool* pool, const float* scores, int64_t score_stride,
                            const int32_t* req_ids, int32_t n_req, int32_t* idx_out,
                            int32_t* plan_out, int32_t* counts_out, hipStream_t stream);

/* Sparse MLA decode attention over the resolved rows ([P3] §"稀疏MLA的核心思想"
 * and its MLA note; [P2] §"与 vLLM 栈的集成", speculative decoding: one
 * resolve plan is replayed for all query tokens of a request).
 *   q        device [n_req][q_per_req][n_heads][576], q_dtype HS_F32 (pool
 *            HS_F32) or HS_BF16 (pool HS_BF16 or HS_FP8_E4M3)
 *   plan     device int32 [n_req][top_k] from hs_resolve_rows (-1 = absent)
 *   out      device fp32 [n_req][q_per_req][n_heads][512]:
 *            out = sum_j softmax_j(sm_scale * <q, row_j>) * row_j[0:512]
 *            over the present rows j (fp8 rows are code * row scale)
 *   lse_out  device fp32 [n_req][q_per_req][n_heads] = log sum_j exp(...), or NULL
 * With no present rows the output is 0 and lse is -inf.
 * The launch shape (query rows per workgroup, plan tiles per workgroup) is
 * chosen from the batch size; two environment variables read at the first
 * call override it for tuning: HS_ATTN_QB (2 or 4 blocks of 16 query rows)
 * and HS_ATTN_TILES_PER_SPLIT (32-row tiles per workgroup). Results agree
 * to rounding under any shape.
 * Errors: INVALID_ARGUMENT, CAPACITY (n_req > max_batch or
 * q_per_req * n_heads > max_q_rows), UNSUPPORTED (dtype combination). */
hs_status hs_sparse_mla_decode(hs_pool* pool, const void* q, int32_t q_dtype,
                               int32_t n_req, int32_t q_per_req, int32_t n_heads,
                               const int32_t* plan, float sm_scale, float* out,
                               float* lse_out, hipStream_t stream);

/* hs_sparse_mla_decode for callers that cannot allocate (code under hipGraph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments, results to rounding and errors, but the split partials of the
 * attention kernels live in a fixed device array of the library, 16 MiB per
 * GPU (8,176 partial rows of 512 fp32 values plus one fp32 each), held from
 * the first hs_init_pool on that GPU until the process ends, instead of in
 * the pool's workspace. The call allocates nothing (no hipMalloc, no
 * allocating library routine). A batch whose smallest split needs more than
 * 8,176 partial rows (n_req * q_per_req * n_heads * ceil(top_k / 2048) with
 * top_k > 2048; with top_k <= 2048 no partials are needed) returns
 * HS_ERR_CAPACITY and enqueues nothing (fp32 pools split their plans only
 * as far as the array holds, so they never get this error). Every call on one GPU shares that
 * GPU's array, so calls whose kernels overlap on one GPU (other streams,
 * other pools, other threads) race; calls on one stream do not. The array
 * needs no clearing: every partial a call reads was written by that call.
 * The current device must be the pool's (else INVALID_ARGUMENT). */
hs_status hs_sparse_mla_decode_noalloc(hs_pool* pool, const void* q, int32_t q_dtype,
                                       int32_t n_req, int32_t q_per_req, int32_t n_heads,
                                       const int32_t* plan, float sm_scale, float* out,
                                       float* lse_out, hipStream_t stream);

/* Sparse MLA decode attention of a speculative step: query token t of
 * request i attends over its own k_per_token selected rows only, read
 * through the union's plan ([P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文
 * 显存瓶颈" §"稀疏MLA的核心思想": only the selected rows enter attention;
 * [P2] §"与 vLLM 栈的集成": one plan per step).
 *   q     device [n_req][q_per_req][n_heads][576] bf16 (fp32 for HS_F32 pools)
 *   plan  device int32 [n_req][top_k]: hs_resolve_rows of union_out
 *   upos  device int32 [n_req][q_per_req][k_per_token]: from
 *         hs_select_topk_union; query token t reads plan row i at
 *         upos[i][t][j] (-1 = absent)
 *   out   device fp32 [n_req][q_per_req][n_heads][512], lse_out as
 *         hs_sparse_mla_decode (per query token, over its own rows)
 * A upos entry >= top_k raises HS_DEV_PLAN_RANGE and is treated as absent.
 * Errors: INVALID_ARGUMENT, CAPACITY (n_req > max_batch, q_per_req * n_heads
 * > max_q_rows or q_per_req * k_per_token > top_k), UNSUPPORTED. */
hs_status hs_sparse_mla_decode_union(hs_pool* pool, const void* q, int32_t q_dtype,
                                     int32_t n_req, int32_t q_per_req, int32_t n_heads,
                                     const int32_t* plan, const int32_t* upos,
                                     int32_t k_per_token, float sm_scale, float* out,
                                     float* lse_out, hipStream_t stream);

/* Residency manager ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载"
 * §"混合 HiSparse 的技术实现": fully resident requests have their completed
 * prefix pages copied to host memory ahead of need, hybrid requests keep
 * the tail on GPU and older pages on host; §"关键架构细节", proactive copy:
 * the copies let GPU pages be released at once under pressure; [P3]
 * §"分级内存的运作机制": under memory pressure a request releases its
 * coldest pages to host memory). For each i < n_req, request r = req_ids[i]:
 *   1. proactive copy: of the GPU pages entirely inside the context that
 *      have no host copy, the lowest-numbered max_copy_pages are copied
 *      (rows, and fp8 scales) from the pool into the host store over PCIe
 *      and marked host-valid;
 *   2. demotion: while the request holds more GPU pages (pages below
 *      ceil(L_r / page_size) with a pool page) than budget_pages[i], its
 *      coldest demotable pages leave the GPU (page table -1), at most
 *      max_demote_pages per call. Demotable: entirely inside the context
 *      and host-valid (after step 1). Coldest: ascending (page stamp, page)
 *      (page stamps: hs_state_layout).
 *   budget_pages    device int32 [n_req], >= 0; NULL = no demotion
 *   freed_out       device int32 [n_req][max_demote_pages]: pool pages given
 *                   back, in ascending logical page order, -1 padded (the
 *                   caller owns pool pages and may reuse them); NULL only
 *                   when max_demote_pages = 0
 *   counts_out      device int32 [n_req][2]: pages copied, pages demoted;
 *                   may be NULL
 * max_copy_pages, max_demote_pages: 0 .. 1024. Graph-capturable.
 * Errors: INVALID_ARGUMENT, CAPACITY (n_req > max_batch). */
hs_status hs_update_residency(hs_pool* pool, const int32_t* req_ids, int32_t n_req,
                              const int32_t* budget_pages, int32_t max_copy_pages,
                              int32_t max_demote_pages, int32_t* freed_out, int32_t* counts_out,
                              hipStream_t stream);

/* Byte offsets of the state arrays in the workspace. Errors: INVALID_ARGUMENT. */
hs_status hs_get_state_layout(const hs_pool* pool, hs_state_layout* out);

/* Synchronise `stream`, then read the sticky device error word into
 * code[0..3] (code, request, index, 0). Returns HS_ERR_DEVICE when code[0] != 0.
 * Not capturable. Errors: INVALID_ARGUMENT, HIP, DEVICE. */
hs_status hs_get_device_error(hs_pool* pool, uint32_t code[4], hipStream_t stream);

/* Clear the sticky device error word (stream-ordered). */
hs_status hs_clear_device_error(hs_pool* pool, hipStream_t stream);

/* The hipError_t value of the last failing HIP call on this thread. */
int32_t hs_last_hip_error(void);

/* Static text for a status code. */
const char* hs_status_string(hs_status status);

/* Free the pinned host store and the handle. Device buffers stay the
 * caller's. Synchronises the device first. NULL is a no-op. */
hs_status hs_destroy_pool(hs_pool* pool);

#ifdef __cplusplus
}
#endif
#endif /* HISPARSE_H_ */
