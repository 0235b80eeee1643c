// Resolve of the selected tokens into physical pool rows ([P2] "vLLM GLM 5.3
// 优化：混合 HiSparse 卸载" §"混合 HiSparse 的技术实现", residency state 2: one
// fused pass reads a resident row in place, reads a hot row and refreshes its
// LRU entry, or on a miss copies the single row from pinned host memory into
// the LRU slot; [P3] §"融合内核与CUDA图兼容": the pass is graph-capturable).
//
// k_resolve        one workgroup per request. Classifies the K tokens
//                  (resident > hot > miss), stamps the hit slots, picks the
//                  victims and rewrites the LRU order with two ordered
//                  compactions, updates tags / stamps / reverse map, writes
//                  the plan, the counts and the list of rows to copy.
// k_copy_misses    many workgroups: each wave copies whole rows from the
//                  mapped host store over PCIe into their hot slots.
//
// LRU order. lru_order lists all S slots in ascending (stamp, slot). With U
// the slots hit this step and M misses, the victims are the first M slots of
// lru_order \ U, and the new order is (lru_order \ U \ victims) followed by
// (U and victims) in ascending slot number: all of those now carry the
// newest stamp, and equal stamps order by slot. That equals choosing victims
// by sorting the untouched slots by (stamp, slot).
#include <hip/hip_runtime.h>

#include "hs_internal.h"

namespace hs {

struct RsScratch {
  int32_t* miss_count;  // [batch]
  int64_t* miss_src;    // [batch][K] host store row
  int32_t* miss_dst;    // [batch][K] pool row (-1 = skip)
};

enum : int { kPad = 0, kRes = 1, kHot = 2, kMiss = 3 };
constexpr int kRsMaxIt = kMaxTopK / kRsThreads;  // top-K entries per thread

__global__ __launch_bounds__(kRsThreads) void k_resolve(const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ req_ids,
                                                        StateView v, RsScratch sc,
                                                        int32_t* __restrict__ plan_out,
                                                        int32_t* __restrict__ counts_out) {
  __shared__ int32_t lru[kMaxHotRows];
  __shared__ int32_t comp[kMaxHotRows];
  __shared__ uint8_t flag[kMaxHotRows];  // bit0: hit this step, bit1: victim
  __shared__ int tmp[kRsThreads / 64 + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int K = v.top_k, S = v.hot_rows, ps = v.page_size, lps = v.log2_ps;
  const int32_t* sel = idx + (size_t)i * K;
  int32_t* plan = plan_out + (size_t)i * K;
  const int r0 = req_ids[i];
  if (r0 < 0 || r0 >= v.max_requests) {
    if (tid == 0) {
      raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)r0);
      sc.miss_count[i] = 0;
      if (counts_out) counts_out[3 * i] = counts_out[3 * i + 1] = counts_out[3 * i + 2] = 0;
    }
    for (int j = tid; j < K; j += kRsThreads) plan[j] = -1;
    return;
  }
  const int r = r0;
  const int L = v.ctx_len[r];
  const int n = v.step[r] + 1;
  const int32_t* pt = v.page_table + (size_t)r * v.pages_per_req;
  const int32_t* hp = v.hot_pages + (size_t)r * v.hot_pages_per_req;
  int32_t* rev = v.rev + (size_t)r * v.max_context;
  int32_t* tag = v.slot_tag + (size_t)r * S;
  int32_t* stamp = v.slot_stamp + (size_t)r * S;
  int32_t* order = v.lru_order + (size_t)r * S;

  for (int s = tid; s < S; s += kRsThreads) {
    flag[s] = 0;
    lru[s] = order[s];
  }
  __syncthreads();

  // 1. classify, stamp the hits, rank the misses in token order
  int kind[kRsMaxIt], tok[kRsMaxIt], prow[kRsMaxIt], mrank[kRsMaxIt];
  int M = 0, n_res = 0, n_hot = 0;
#pragma unroll
  for (int it = 0; it < kRsMaxIt; ++it) {
    kind[it] = kPad;
    tok[it] = -1;
    prow[it] = -1;
    mrank[it] = 0;
    if (it * kRsThreads >= K) continue;  // uniform across the block
    const int j = it * kRsThreads + tid;
    if (j < K) {
      const int t = sel[j];
      tok[it] = t;
      if (t >= L) {
        raise_error(v.error, HS_DEV_INDEX_RANGE, (uint32_t)r, (uint32_t)t);
      } else if (t >= 0) {
        const int g = pt[t >> lps];
        if (g >= 0) {
          kind[it] = kRes;
          prow[it] = g * ps + (t & (ps - 1));
        } else {
          const int slot = rev[t];
          if (slot >= 0) {
            const int hpg = hp[slot >> lps];
            if (hpg >= 0) {
              kind[it] = kHot;
              flag[slot] = 1;
              stamp[slot] = n;
              prow[it] = hpg * ps + (slot & (ps - 1));
            } else {
              raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)slot);
            }
          } else {
            kind[it] = kMiss;
          }
        }
      }
    }
    int tot;
    mrank[it] = M + block_excl_count(kind[it] == kMiss, tmp, tot);
    M += tot;
    n_res += __syncthreads_count(kind[it] == kRes);
    n_hot += __syncthreads_count(kind[it] == kHot);
  }
  // (the counting barriers above also publish the hit flags)

  // 2. untouched slots in LRU order -> comp[0 .. S - |U|)
  int kept = 0;
  for (int base = 0; base < S; base += kRsThreads) {
    const int s = base + tid < S ? lru[base + tid] : -1;
    const bool keep = s >= 0 && !(flag[s] & 1);
    int tot;
    const int pos = kept + block_excl_count(keep, tmp, tot);
    if (keep) comp[pos] = s;
    kept += tot;
  }
  __syncthreads();
  // 3. the first M untouched slots are the victims
  for (int x = tid; x < M; x += kRsThreads) flag[comp[x]] |= 2;
  __syncthreads();
  // 4. new LRU order: remaining untouched slots, then hit and victim slots
  //    in ascending slot number
  for (int x = tid; x < kept - M; x += kRsThreads) order[x] = comp[M + x];
  int fresh = kept - M;
  for (int base = 0; base < S; base += kRsThreads) {
    const int s = base + tid;
    const bool f = s < S && flag[s] != 0;
    int tot;
    const int pos = fresh + block_excl_count(f, tmp, tot);
    if (f) order[pos] = s;
    fresh += tot;
  }
  // 5. fill the victims with the misses (i-th miss -> i-th victim)
  const int64_t hbase = v.host_base[r];
#pragma unroll
  for (int it = 0; it < kRsMaxIt; ++it) {
    if (kind[it] != kMiss) continue;
    const int t = tok[it];
    const int slot = comp[mrank[it]];
    const int old = tag[slot];
    if (old >= 0 && old < v.max_context) rev[old] = -1;
    tag[slot] = t;
    rev[t] = slot;
    stamp[slot] = n;
    const int hpg = hp[slot >> lps];
    int dst = -1;
    if (hpg >= 0) {
      dst = hpg * ps + (slot & (ps - 1));
    } else {
      raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)slot);
    }
    prow[it] = dst;
    sc.miss_src[(size_t)i * K + mrank[it]] = hbase + t;
    sc.miss_dst[(size_t)i * K + mrank[it]] = dst;
  }
  // 6. plan, counts, step
#pragma unroll
  for (int it = 0; it < kRsMaxIt; ++it) {
    const int j = it * kRsThreads + tid;
    if (j < K) plan[j] = prow[it];
  }
  if (tid == 0) {
    sc.miss_count[i] = M;
    if (counts_out) {
      counts_out[3 * i] = n_res;
      counts_out[3 * i + 1] = n_hot;
      counts_out[3 * i + 2] = M;
    }
    v.counters[3 * r] += n_res;
    v.counters[3 * r + 1] += n_hot;
    v.counters[3 * r + 2] += M;
    v.step[r] = n;
  }
}

// Copy the missed rows. Wave w of the grid takes misses w, w + W, ... of the
// flattened (request, miss) list; each wave copies one whole row with 16-byte
// loads from the mapped host store.
template <int ROW_BYTES, bool FP8>
__global__ __launch_bounds__(kCopyThreads) void k_copy_misses(int n_req, int K, RsScratch sc,
                                                              const uint8_t* __restrict__ host_rows,
                                                              const float* __restrict__ host_scales,
                                                              uint8_t* __restrict__ pool_rows,
                                                              float* __restrict__ pool_scales) {
  constexpr int CH = ROW_BYTES / 16;
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * (kCopyThreads / 64);
  int f = blockIdx.x * (kCopyThreads / 64) + (threadIdx.x >> 6);
  int acc = 0;
  for (int i = 0; i < n_req; ++i) {
    const int M = sc.miss_count[i];
    for (; f < acc + M; f += W) {
      const int m = f - acc;
      const int64_t src = sc.miss_src[(size_t)i * K + m];
      const int dst = sc.miss_dst[(size_t)i * K + m];
      if (dst < 0) continue;
      const uint4* s4 = reinterpret_cast<const uint4*>(host_rows + src * ROW_BYTES);
      uint4* d4 = reinterpret_cast<uint4*>(pool_rows + (int64_t)dst * ROW_BYTES);
      uint4 x[(CH + 63) / 64];
#pragma unroll
      for (int c = 0; c < (CH + 63) / 64; ++c)
        if (lane + 64 * c < CH) x[c] = s4[lane + 64 * c];
#pragma unroll
      for (int c = 0; c < (CH + 63) / 64; ++c)
        if (lane + 64 * c < CH) d4[lane + 64 * c] = x[c];
      if (FP8 && lane == 0) pool_scales[dst] = host_scales[src];
    }
    acc += M;
  }
}

hs_status launch_resolve(hs_pool* p, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                         int32_t* plan_out, int32_t* counts_out, hipStream_t s) {
  StateView v = make_view(p);
  RsScratch sc;
  sc.miss_count = reinterpret_cast<int32_t*>(p->state + p->off.rs_miss_count);
  sc.miss_src = reinterpret_cast<int64_t*>(p->state + p->off.rs_miss_src);
  sc.miss_dst = reinterpret_cast<int32_t*>(p->state + p->off.rs_miss_dst);
  k_resolve<<<n_req, kRsThreads, 0, s>>>(idx, req_ids, v, sc, plan_out, counts_out);
  // enough waves for one row each in the worst case, capped
  const int64_t rows = (int64_t)n_req * p->d.top_k;
  int blocks = (int)((rows + 3) / 4);
  if (blocks > 1024) blocks = 1024;
  const uint8_t* hr = static_cast<const uint8_t*>(p->host_rows);
  switch (p->d.kv_dtype) {
    case HS_F32:
      k_copy_misses<2304, false><<<blocks, kCopyThreads, 0, s>>>(n_req, p->d.top_k, sc, hr, nullptr,
                                                                 p->pool_rows, nullptr);
      break;
    case HS_BF16:
      k_copy_misses<1152, false><<<blocks, kCopyThreads, 0, s>>>(n_req, p->d.top_k, sc, hr, nullptr,
                                                                 p->pool_rows, nullptr);
      break;
    default:
      k_copy_misses<576, true><<<blocks, kCopyThreads, 0, s>>>(n_req, p->d.top_k, sc, hr, p->host_scales,
                                                               p->pool_rows, p->pool_scales);
      break;
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
