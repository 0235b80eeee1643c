// Residency manager ([P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载"
// §"混合 HiSparse 的技术实现": fully resident requests have completed prefix
// pages copied to host memory ahead of need, hybrid requests keep the tail on
// GPU and older pages on host; §"关键架构细节", proactive copy: with the copy
// made in advance, GPU pages can be released at once when pressure comes;
// [P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈" §"分级内存的运作机制":
// under memory pressure a request releases its coldest pages to host memory).
//
// k_update_residency: one 1,024-thread workgroup per request.
//   1. One ordered pass over the request's pages counts its GPU pages and
//      lists, in page order, the complete GPU pages without a host copy; the
//      first max_copy of them are marked host-valid and written to a list
//      that k_residency_copy then copies (rows and fp8 scales) from the pool
//      into the mapped host store with many workgroups, 16 bytes per thread
//      and access. Because the copies take the lowest pending pages, a
//      pending page counts as copied exactly when it is not above the last
//      listed one.
//   2. If the request holds more GPU pages than its budget, d = min(excess,
//      max_demote) of its demotable pages (complete and host-valid) leave the
//      GPU: the d smallest by (page stamp, page). The stamp threshold comes
//      from a 12 + 12 + 8-bit radix select over the candidates' stamps (LDS
//      histograms); candidates at the threshold stamp are taken in page
//      order. A final ordered pass writes page table -1 and reports the pool
//      pages in ascending page order.
// Page stamps are written by resolve (the last step whose top-K selected a
// token of the page) and by set_residency (the step at which a page entered
// the context).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "hs_internal.h"

namespace hs {

typedef uint32_t ru_u32x4 __attribute__((ext_vector_type(4)));

struct RuArgs {
  const int32_t* req_ids;
  const int32_t* budget;  // [n_req] or null
  int max_copy, max_demote;
  const uint8_t* pool_rows;
  const float* pool_scales;
  uint8_t* host_rows;
  int row_bytes;
  int host_stride;  // bytes between host rows (fp8: the row's scale follows its codes)
  int32_t* freed_out;   // [n_req][max_demote] or null
  int32_t* counts_out;  // [n_req][2] or null
  int32_t* list;        // [n_req][kRuMaxList][2] pages to copy: (logical page, pool page)
  int32_t* ncopy;       // [n_req] entries of list
};

__device__ inline int ru_wave_incl_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// Ascending search of a 4,096-bin histogram: the bin b with below(b) < need
// <= below(b) + h[b], and below(b), for 1 <= need <= total. Every thread
// gets the result; contains three barriers.
__device__ void ru_find(const uint32_t* h, int need, int* wtot, int* res, int& b_out, int& below_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lo = 4 * tid;  // this thread's bins lo .. lo + 3
  const uint4 q = *reinterpret_cast<const uint4*>(h + lo);
  const int c4 = (int)(q.x + q.y + q.z + q.w);
  const int incl_w = ru_wave_incl_sum(c4);
  if (lane == 63) wtot[wave] = incl_w;
  __syncthreads();
  int pre = 0;
#pragma unroll
  for (int w = 0; w < kRuThreads / 64; ++w) pre += w < wave ? wtot[w] : 0;
  const int incl = pre + incl_w, excl = incl - c4;
  if (excl < need && need <= incl) {
    const int cnt[4] = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
    int below = excl, bb = lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (bb == lo + e && below + cnt[e] < need) {
        below += cnt[e];
        bb = lo + e + 1;
      }
    }
    res[0] = bb;
    res[1] = below;
  }
  __syncthreads();
  b_out = res[0];
  below_out = res[1];
  __syncthreads();
}

__global__ __launch_bounds__(kRuThreads) void k_update_residency(RuArgs a, StateView v) {
  __shared__ __align__(16) uint32_t hist[kTkBins];
  __shared__ int list_p[kRuMaxList];
  __shared__ int list_g[kRuMaxList];
  __shared__ int tmp[kRuThreads / 64 + 1];
  __shared__ int res[2];
  const int i = blockIdx.x, tid = threadIdx.x;
  int32_t* freed = a.freed_out ? a.freed_out + (size_t)i * a.max_demote : nullptr;
  const int r = a.req_ids[i];
  if (r < 0 || r >= v.max_requests) {
    if (freed)
      for (int j = tid; j < a.max_demote; j += kRuThreads) freed[j] = -1;
    if (tid == 0) {
      raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)r);
      if (a.counts_out) a.counts_out[2 * i] = a.counts_out[2 * i + 1] = 0;
    }
    return;
  }
  const int L = v.ctx_len[r], ps = v.page_size;
  const int npg = (L + ps - 1) / ps, full = L / ps;
  int32_t* pt = v.page_table + (size_t)r * v.pages_per_req;
  const int32_t* st = v.page_stamp + (size_t)r * v.pages_per_req;
  uint8_t* hv = v.host_valid + (size_t)r * v.pages_per_req;

  // 1. GPU pages held, pending copies (in page order), demotion candidates
  int pend_total = 0, my_gpu = 0;
  for (int base = 0; base < npg; base += kRuThreads) {
    const int p = base + tid;
    const int g = p < npg ? pt[p] : -1;
    const bool pending = g >= 0 && p < full && hv[p] == 0;
    int tot;
    const int rank = pend_total + block_excl_count(pending, tmp, tot);
    if (pending && rank < a.max_copy) {
      list_p[rank] = p;
      list_g[rank] = g;
    }
    pend_total += tot;
    my_gpu += g >= 0 ? 1 : 0;
  }
  int gpu_total;
  (void)block_excl_sum(my_gpu, tmp, gpu_total);
  const int ncopy = min(pend_total, a.max_copy);
  const int last_copied = ncopy > 0 ? list_p[ncopy - 1] : -1;  // (the scans' barriers published the list)
  auto candidate = [&](int p, int& key) -> bool {
    const int g = pt[p];
    const bool ok = g >= 0 && p < full && (hv[p] != 0 || p <= last_copied);
    key = ok ? st[p] : 0;
    return ok;
  };

  // the pages to copy, for k_residency_copy
  for (int k = tid; k < ncopy; k += kRuThreads) {
    a.list[((size_t)i * kRuMaxList + k) * 2] = list_p[k];
    a.list[((size_t)i * kRuMaxList + k) * 2 + 1] = list_g[k];
  }
  if (tid == 0) a.ncopy[i] = ncopy;

  // 2. demotion: the d smallest (stamp, page) among the candidates
  int d = 0;
  if (a.budget) d = min(max(gpu_total - a.budget[i], 0), a.max_demote);
  int ndemoted = 0;
  if (d > 0) {
    int my_cand = 0;
    for (int p = tid; p < npg; p += kRuThreads) {
      int key;
      my_cand += candidate(p, key) ? 1 : 0;
    }
    int cand_total;
    (void)block_excl_sum(my_cand, tmp, cand_total);
    d = min(d, cand_total);
    uint32_t T = 0xFFFFFFFFu;  // every candidate with stamp < T is taken ...
    int take_eq = 0;            // ... and the first take_eq with stamp == T
    if (d > 0 && d < cand_total) {
      uint32_t pre = 0u;
      int below_all = 0;
      const int shifts[3] = {20, 8, 0}, widths[3] = {12, 12, 8};
#pragma unroll
      for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass];
        const uint32_t mask = (1u << widths[pass]) - 1u;
        for (int b = tid; b < kTkBins; b += kRuThreads) hist[b] = 0u;
        __syncthreads();
        for (int p = tid; p < npg; p += kRuThreads) {
          int key;
          if (!candidate(p, key)) continue;
          const uint32_t k = (uint32_t)key;
          const bool in = pass == 0 || (k >> (sh + widths[pass])) == pre;
          if (in) atomicAdd(&hist[(k >> sh) & mask], 1u);
        }
        __syncthreads();
        int b, below;
        ru_find(hist, d - below_all, tmp, res, b, below);
        pre = (pre << widths[pass]) | (uint32_t)b;
        below_all += below;
      }
      T = pre;
      take_eq = d - below_all;
    }
    // ordered pass: take, write the page table, report the pool pages
    int eq_run = 0, pos_run = 0;
    for (int base = 0; base < npg; base += kRuThreads) {
      const int p = base + tid;
      int key = 0;
      const bool c = p < npg && candidate(p, key);
      const bool eq = c && (uint32_t)key == T;
      int tot_eq;
      const int eq_rank = eq_run + block_excl_count(eq, tmp, tot_eq);
      const bool take = c && ((uint32_t)key < T || (eq && eq_rank < take_eq) || T == 0xFFFFFFFFu);
      int tot_take;
      const int pos = pos_run + block_excl_count(take, tmp, tot_take);
      if (take) {
        freed[pos] = pt[p];
        pt[p] = -1;
      }
      eq_run += tot_eq;
      pos_run += tot_take;
    }
    ndemoted = pos_run;
  }
  // -1 padding of the report (entries not written above), host-valid marks
  // of the copied pages (after the scans that read them)
  if (freed)
    for (int j = ndemoted + tid; j < a.max_demote; j += kRuThreads) freed[j] = -1;
  __syncthreads();
  for (int k = tid; k < ncopy; k += kRuThreads) hv[list_p[k]] = 1;
  if (tid == 0 && a.counts_out) {
    a.counts_out[2 * i] = ncopy;
    a.counts_out[2 * i + 1] = ndemoted;
  }
}

// Copy of the listed pages into the host store: request blockIdx.y, the
// grid's x workgroups stride over its pages 64 bytes per thread, then over
// its fp8 scales (each written after its row's codes). Writes go over PCIe
// into the mapped pinned store.
__global__ __launch_bounds__(256) void k_residency_copy(RuArgs a, StateView v) {
  const int i = blockIdx.y;
  const int r = a.req_ids[i];
  if (r < 0 || r >= v.max_requests) return;
  const int n = a.ncopy[i];
  const int ps = v.page_size, lps = v.log2_ps;
  const int CH = a.row_bytes / 16;
  const int per_page = ps * CH;
  const int64_t hbase = v.host_base[r];
  const int32_t* lst = a.list + (size_t)i * kRuMaxList * 2;
  const int stride = gridDim.x * 256;
  // 4 consecutive 16-byte chunks of one row per thread (a row is a multiple
  // of 4 chunks: 64 B per lane in flight, 4 KiB per wave)
  for (int x = (blockIdx.x * 256 + threadIdx.x) * 4; x < n * per_page; x += stride * 4) {
    const int k = x / per_page, rem = x - k * per_page;
    const int row = rem / CH, c = rem - row * CH;
    const int lp = lst[2 * k], gp = lst[2 * k + 1];
    const ru_u32x4* src = reinterpret_cast<const ru_u32x4*>(a.pool_rows + (int64_t)gp * ps * a.row_bytes) + rem;
    ru_u32x4* dst =
        reinterpret_cast<ru_u32x4*>(a.host_rows + (hbase + (int64_t)lp * ps + row) * a.host_stride) + c;
    const ru_u32x4 t0 = src[0], t1 = src[1], t2 = src[2], t3 = src[3];
    dst[0] = t0;
    dst[1] = t1;
    dst[2] = t2;
    dst[3] = t3;
  }
  if (a.pool_scales)
    for (int x = blockIdx.x * 256 + threadIdx.x; x < n * ps; x += stride) {
      const int k = x >> lps, o = x & (ps - 1);
      *reinterpret_cast<float*>(a.host_rows + (hbase + (int64_t)lst[2 * k] * ps + o) * a.host_stride + a.row_bytes) =
          a.pool_scales[(int64_t)lst[2 * k + 1] * ps + o];
    }
}

hs_status launch_update_residency(hs_pool* p, const int32_t* req_ids, int32_t n_req, const int32_t* budget,
                                  int32_t max_copy, int32_t max_demote, int32_t* freed_out, int32_t* counts_out,
                                  hipStream_t s) {
  RuArgs a;
  a.req_ids = req_ids;
  a.budget = budget;
  a.max_copy = max_copy;
  a.max_demote = max_demote;
  a.pool_rows = p->pool_rows;
  a.pool_scales = p->pool_scales;
  a.host_rows = static_cast<uint8_t*>(p->host_rows);
  a.row_bytes = (int)p->sz.row_bytes;
  a.host_stride = (int)p->sz.host_row_stride;
  a.freed_out = freed_out;
  a.counts_out = counts_out;
  a.list = reinterpret_cast<int32_t*>(p->state + p->off.ru_list);
  a.ncopy = reinterpret_cast<int32_t*>(p->state + p->off.ru_ncopy);
  k_update_residency<<<n_req, kRuThreads, 0, s>>>(a, make_view(p));
  if (max_copy > 0) {
    // enough workgroups to keep many PCIe writes in flight, sized for the
    // largest copy allowed; surplus workgroups exit at once
    const int64_t quads = (int64_t)max_copy * p->d.page_size * (p->sz.row_bytes / 16) / 4;
    const int per_req = (int)std::max<int64_t>(1, std::min<int64_t>((quads + 255) / 256, std::max(1, 2048 / n_req)));
    k_residency_copy<<<dim3(per_req, n_req), 256, 0, s>>>(a, make_view(p));
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
