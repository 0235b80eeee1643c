// Internal declarations of libhisparse: the pool handle, the workspace
// layout, device-side helpers shared by the kernels, and the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hs {

// ---------------------------------------------------------------- constants
constexpr int kRowDim = 576;       // 512 nope + 64 rope
constexpr int kNope = 512;
constexpr int kMaxTopK = 4096;
constexpr int kMaxHotRows = 8192;
// fp8 host row: 576 code bytes, the fp32 scale, 60 unused bytes. Rows start
// on 128-byte boundaries (as bf16 and fp32 rows do), which PCIe gathers of
// whole rows read ~8% faster than rows at 16-byte alignment.
constexpr int kHostRowStrideFp8 = 640;

// top-K: one filter workgroup scans one chunk of kTkChunk scores
constexpr int kTkChunk = 2048;
constexpr int kTkThreads = 256;
constexpr int kTkBins = 4096;      // 12-bit radix digits
constexpr int kTkMaxChunks = 2048; // => max_context <= 4,194,304
constexpr int kTkStage = 8192;     // survivors staged in LDS by the select workgroup
constexpr int kMaxSelectQ = 8;     // query tokens per request with a selection of their own

// resolve
constexpr int kRsThreads = 1024;

// residency manager
constexpr int kRuThreads = 1024;
constexpr int kRuMaxList = 1024;   // most pages copied or demoted per call

// attention
constexpr int kAttSplitCap = 4;    // partial rows reserved per (request, query row)
constexpr int kAttMinPartRows = 16384;  // at least this many partial rows (32 MiB)
constexpr int kAttMaxTilesPerSplit = 64;
// Split partials of hs_sparse_mla_decode_noalloc: a file-scope device array
// of this many bytes (one per GPU the library runs on), holding
// kStaticPartRows rows of 512 fp32 partial outputs followed by as many fp32
// partial log-sum-exps.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int64_t kStaticPartRows = 8176;
static_assert(kStaticPartRows * 4 * 512 % 256 == 0, "lse partials start 256-byte aligned");
static_assert(kStaticPartRows * 4 * 513 <= (int64_t)kStaticScratchBytes, "partials fit the array");

// ---------------------------------------------------------------- the handle
struct Offsets {
  size_t zero_row;  // kRowDim * 4 bytes of zeros, never written after init
  size_t tk_count, tk_max, tk_cand, tk_bound;
  size_t rs_mdst, rs_mslot, rs_mold, rs_ticket;
  size_t ru_list, ru_ncopy;  // residency manager: pages to copy [B][kRuMaxList][2], their count [B]
  size_t at_part_o, at_part_lse;
  int64_t at_part_rows;  // capacity of partial rows
  int32_t sel_q;         // top-K scratch rows and survivor bounds per request (select_q, at least 1)
};

}  // namespace hs

struct hs_pool {
  hs_pool_desc d;
  hs_pool_sizes sz;
  hs_state_layout lay;
  hs::Offsets off;
  int device;
  int log2_ps;
  int64_t pool_rows_n;        // num_pool_pages * page_size
  uint8_t* pool_rows;         // device
  float* pool_scales;         // device (fp8) or null
  uint8_t* state;             // device workspace
  uint8_t* static_scratch;    // device address of this device's no-alloc scratch array
  void* host_rows;            // pinned, mapped
  float* host_scales;         // fp8: the scale of host row 0 (row r's at byte r * host_row_stride), or null
};

namespace hs {

// Typed views of the workspace, passed by value to kernels.
struct StateView {
  int32_t* ctx_len;
  int64_t* host_base;
  int32_t* page_table;
  int32_t* hot_pages;
  int32_t* rev;
  int32_t* slot_tag;
  int32_t* slot_stamp;
  int32_t* lru_order;
  int32_t* step;
  int64_t* counters;
  uint32_t* error;
  int32_t* page_stamp;
  uint8_t* host_valid;
  int32_t max_requests, max_context, pages_per_req, hot_rows, hot_pages_per_req;
  int32_t page_size, log2_ps, num_pool_pages, top_k;
};

StateView make_view(const hs_pool* p);
hs_status set_hip_error(hipError_t e);

#define HS_HIP_CHECK(expr)                         \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return hs::set_hip_error(e_); \
  } while (0)

// Top-K of k tokens for each of the qsel score rows of each request (row
// i * qsel + t of `scores` and of idx_out [n_req * qsel][k]); qsel = 1 and
// k = top_k for a plain step.
hs_status launch_topk(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                      int32_t n_req, int32_t qsel, int32_t k, int32_t* idx_out, hipStream_t s);
// The filter kernel of launch_topk alone (one score row per request).
hs_status launch_topk_filter(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                             int32_t n_req, int32_t k, hipStream_t s);
// Select and resolve in one launch after the filter kernel: idx_out as
// launch_topk, then plan_out / counts_out as launch_resolve.
hs_status launch_select_resolve(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                                int32_t n_req, int32_t* idx_out, int32_t* plan_out, int32_t* counts_out,
                                hipStream_t s);
// Union of the qsel selections of each request (idx [n_req][qsel][k]):
// union_out [n_req][top_k] ascending, -1 padded; upos_out [n_req][qsel][k]
// the union position of each selected token (-1 for padding).
hs_status launch_topk_union(hs_pool* p, const int32_t* idx, int32_t n_req, int32_t qsel, int32_t k,
                            int32_t* union_out, int32_t* upos_out, hipStream_t s);
hs_status launch_resolve(hs_pool* p, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                         int32_t* plan_out, int32_t* counts_out, hipStream_t s);
hs_status launch_update_residency(hs_pool* p, const int32_t* req_ids, int32_t n_req,
                                  const int32_t* budget, int32_t max_copy, int32_t max_demote,
                                  int32_t* freed_out, int32_t* counts_out, hipStream_t s);
hs_status launch_indexer_scores(hs_pool* p, const void* iq, const float* iw, const void* ik, int64_t ik_stride,
                                int32_t n_heads, const int32_t* req_ids, int32_t n_req, float* scores,
                                int64_t score_stride, hipStream_t s);
// Attention of n_req groups of q_per_req * n_heads query rows; group i reads
// k_plan plan entries of plan row i / plan_div (rows of top_k entries),
// through upos [n_req][k_plan] when given. Split partials: part_o
// [part_rows][512] and part_lse [part_rows] fp32.
hs_status launch_attention(hs_pool* p, const void* q, int32_t q_dtype, int32_t n_req,
                           int32_t q_per_req, int32_t n_heads, const int32_t* plan, const int32_t* upos,
                           int32_t k_plan, int32_t plan_div, float sm_scale, float* out, float* lse_out,
                           float* part_o, float* part_lse, int64_t part_rows, hipStream_t s);
// Device address of the no-alloc scratch array on the current device
// (resolved once per device; the device must be current).
hs_status static_scratch_address(int device, uint8_t** out);

// ---------------------------------------------------------------- device helpers
// Sticky device error word: the first error wins; later ones are dropped.
__device__ inline void raise_error(uint32_t* err, uint32_t code, uint32_t a, uint32_t b) {
  if (atomicCAS(err, 0u, code) == 0u) {
    err[1] = a;
    err[2] = b;
  }
}

// Exclusive prefix count of a per-thread flag over the whole block, in
// thread order. `tmp` holds one int per wave (blockDim.x / 64 entries) plus
// one; the block total is returned in `total`. Contains two barriers.
__device__ inline int block_excl_count(bool f, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  const unsigned long long m = __ballot(f);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[wave] = __popcll(m);
  __syncthreads();
  int pre = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = tmp[w];
    pre += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return pre + below;
}

// Exclusive prefix sum of a per-thread int over the block, in thread order.
__device__ inline int block_excl_sum(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int pre = 0, tot = 0;
  for (int w = 0; w < nw; ++w) {
    const int c = tmp[w];
    pre += (w < wave) ? c : 0;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return pre + x - v;
}

}  // namespace hs
