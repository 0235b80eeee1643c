// Resolve of the selected tokens into physical pool rows ([P2] "vLLM GLM 5.3
// 优化：混合 HiSparse 卸载" §"混合 HiSparse 的技术实现", residency state 2: one
// fused pass reads a resident row in place, reads a hot row and refreshes its
// LRU entry, or on a miss copies the single row from pinned host memory into
// the LRU slot; [P3] §"融合内核与CUDA图兼容": the pass is graph-capturable).
//
// One kernel, two kinds of workgroup, roles handed out by a device ticket
// counter in the order workgroups start:
//   bookkeeper (tickets 0 .. n_req-1), one per request: classifies the K
//     tokens (resident > hot > miss), stamps the hit slots, picks the victims
//     and rewrites the LRU order with ordered compactions in LDS, updates
//     tags / stamps / reverse map, writes the plan and the counts, and
//     publishes the plan with a per-request flag;
//   copy workgroup (request i, part c), one per 64 plan positions: reads the
//     page table and reverse map itself to guess which of its tokens miss
//     and starts reading those rows from the mapped host store over PCIe
//     right away, then waits for the flag and writes the rows the
//     bookkeeper actually classified as misses into their hot slots (rows it
//     did not guess are read then). The guess only decides how early the
//     PCIe reads start; which rows are written comes from the bookkeeper.
// A copy workgroup holds a later ticket than its bookkeeper, which is
// therefore running and never waits, so the wait always ends; it is also
// bounded (a device error is raised past the bound and the copy skipped).
// Counters and flags are left cleared for the next call.
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

// Native 16-byte vector: arrays of it stay in registers (HIP's uint4 struct
// made the prefetch arrays go through scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RsScratch {
  unsigned long long* miss_mask;  // [batch][parts] miss bits of 64 plan positions
  uint32_t* flag;                 // [batch] 1 once request i's plan is published
  uint32_t* exit_cnt;             // [batch] copy workgroups of request i done
  uint32_t* ticket;               // [2] roles handed out, workgroups exited
  int words;                      // ceil(K / 64) mask words per request
  int parts;                      // ceil(K / kRsPart) copy workgroups per request
};

enum : int { kPad = 0, kRes = 1, kHot = 2, kMiss = 3 };
constexpr int kRsMaxIt = kMaxTopK / kRsThreads;  // top-K entries per thread
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kSpinLimit = 1 << 20;  // polls of the flag (>= 0.1 s) before giving up
constexpr int kRsPart = 64;          // plan positions per copy workgroup (divides 64)

struct RsArgs {
  const int32_t* idx;
  const int32_t* req_ids;
  int n_req;
  int32_t* plan_out;
  int32_t* counts_out;
  const uint8_t* host_rows;
  const float* host_scales;
  uint8_t* pool_rows;
  float* pool_scales;
};

struct RsShared {
  int32_t lru[kMaxHotRows];
  int32_t comp[kMaxHotRows];
  uint8_t flag[kMaxHotRows];  // bit0: hit this step, bit1: victim
  int tmp[kRsWaves + 1];
  int32_t tok[64];            // copy role: token of each position, -1 = not guessed
  int8_t gpos[64];            // copy role: positions of the guessed misses, in order
  int n_guess;
  int role;
  int go;
};

__device__ __forceinline__ void bookkeep(const RsArgs& a, const StateView& v, const RsScratch& sc, RsShared& sh, int i) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = v.top_k, S = v.hot_rows, ps = v.page_size, lps = v.log2_ps;
  const int32_t* sel = a.idx + (size_t)i * K;
  int32_t* plan = a.plan_out + (size_t)i * K;
  const int r0 = a.req_ids[i];
  auto publish = [&]() {
    __threadfence();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&sc.flag[i], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (r0 < 0 || r0 >= v.max_requests) {
    if (tid == 0) {
      raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)r0);
      if (a.counts_out) a.counts_out[3 * i] = a.counts_out[3 * i + 1] = a.counts_out[3 * i + 2] = 0;
    }
    for (int j = tid; j < K; j += kRsThreads) plan[j] = -1;
    for (int w = tid; w < sc.words; w += kRsThreads) sc.miss_mask[(size_t)i * sc.words + w] = 0ull;
    publish();
    return;
  }
  const int r = r0;
  const int L = v.ctx_len[r];
  const int n = v.step[r] + 1;
  const int32_t* pt = v.page_table + (size_t)r * v.pages_per_req;
  int32_t* rev = v.rev + (size_t)r * v.max_context;
  int32_t* tag = v.slot_tag + (size_t)r * S;
  int32_t* stamp = v.slot_stamp + (size_t)r * S;
  int32_t* order = v.lru_order + (size_t)r * S;
  const int32_t* hp = v.hot_pages + (size_t)r * v.hot_pages_per_req;
  for (int s = tid; s < S; s += kRsThreads) {
    sh.flag[s] = 0;
    sh.lru[s] = order[s];
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
      const bool ok = t >= 0 && t < L;
      if (t >= L) raise_error(v.error, HS_DEV_INDEX_RANGE, (uint32_t)r, (uint32_t)t);
      // both lookups issued before either is used
      const int g = ok ? pt[t >> lps] : -1;
      const int slot = ok ? rev[t] : -1;
      if (ok) {
        if (g >= 0) {
          kind[it] = kRes;
          prow[it] = g * ps + (t & (ps - 1));
        } else if (slot >= 0) {
          const int hpg = hp[slot >> lps];
          if (hpg >= 0) {
            kind[it] = kHot;
            sh.flag[slot] = 1;
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
    const unsigned long long mb = __ballot(kind[it] == kMiss);
    if (lane == 0 && it * kRsThreads + 64 * wave < K) sc.miss_mask[(size_t)i * sc.words + it * kRsWaves + wave] = mb;
    int tot;
    mrank[it] = M + block_excl_count(kind[it] == kMiss, sh.tmp, tot);
    M += tot;
    n_res += __syncthreads_count(kind[it] == kRes);
    n_hot += __syncthreads_count(kind[it] == kHot);
  }
  // (the counting barriers above also publish the hit flags)

  // 2. untouched slots in LRU order -> comp[0 .. S - |U|)
  int kept = 0;
  for (int base = 0; base < S; base += kRsThreads) {
    const int s = base + tid < S ? sh.lru[base + tid] : -1;
    const bool keep = s >= 0 && !(sh.flag[s] & 1);
    int tot;
    const int pos = kept + block_excl_count(keep, sh.tmp, tot);
    if (keep) sh.comp[pos] = s;
    kept += tot;
  }
  __syncthreads();
  // 3. the first M untouched slots are the victims
  for (int x = tid; x < M; x += kRsThreads) sh.flag[sh.comp[x]] |= 2;
  __syncthreads();
  // 4. new LRU order: remaining untouched slots, then hit and victim slots
  //    in ascending slot number
  for (int x = tid; x < kept - M; x += kRsThreads) order[x] = sh.comp[M + x];
  int fresh = kept - M;
  for (int base = 0; base < S; base += kRsThreads) {
    const int s = base + tid;
    const bool f = s < S && sh.flag[s] != 0;
    int tot;
    const int pos = fresh + block_excl_count(f, sh.tmp, tot);
    if (f) order[pos] = s;
    fresh += tot;
  }
  // 5. fill the victims with the misses (i-th miss -> i-th victim)
#pragma unroll
  for (int it = 0; it < kRsMaxIt; ++it) {
    if (kind[it] != kMiss) continue;
    const int t = tok[it];
    const int slot = sh.comp[mrank[it]];
    const int old = tag[slot];
    if (old >= 0 && old < v.max_context) rev[old] = -1;
    tag[slot] = t;
    rev[t] = slot;
    stamp[slot] = n;
    const int hpg = hp[slot >> lps];
    if (hpg >= 0) {
      prow[it] = hpg * ps + (slot & (ps - 1));
    } else {
      raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)slot);
    }
  }
  // 6. plan; publish it to the copy workgroups; counts and step
#pragma unroll
  for (int it = 0; it < kRsMaxIt; ++it) {
    const int j = it * kRsThreads + tid;
    if (j < K) plan[j] = prow[it];
  }
  publish();
  if (tid == 0) {
    if (a.counts_out) {
      a.counts_out[3 * i] = n_res;
      a.counts_out[3 * i + 1] = n_hot;
      a.counts_out[3 * i + 2] = M;
    }
    v.counters[3 * r] += n_res;
    v.counters[3 * r + 1] += n_hot;
    v.counters[3 * r + 2] += M;
    v.step[r] = n;
  }
}

// Copy the missed rows of plan positions [c kRsPart, (c + 1) kRsPart) of request i.
template <int ROW_BYTES, bool FP8>
__device__ __forceinline__ void copy_part(const RsArgs& a, const StateView& v, const RsScratch& sc, RsShared& sh, int i,
                          int c) {
  constexpr int CH = ROW_BYTES / 16;           // 16-byte chunks per row
  constexpr int CPL = (CH + 63) / 64;          // chunks per lane
  constexpr int RPW = (kRsPart + kRsWaves - 1) / kRsWaves;  // guessed rows per wave (at most)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = v.top_k, lps = v.log2_ps;
  const int j0 = kRsPart * c;
  const int r0 = a.req_ids[i];
  const bool valid_req = r0 >= 0 && r0 < v.max_requests;
  const int r = valid_req ? r0 : 0;
  const int L = valid_req ? v.ctx_len[r] : 0;
  const int64_t hbase = v.host_base[r];
  // Guess the misses from the current tables. The bookkeeper may be
  // updating them meanwhile (atomic reads, any outcome is harmless): the
  // guess only decides which host reads start before the plan is known.
  if (wave == 0) {
    const int j = j0 + lane;
    const int t = lane < kRsPart && j < K ? a.idx[(size_t)i * K + j] : -1;
    bool guess = false;
    if (t >= 0 && t < L) {
      const int g = v.page_table[(size_t)r * v.pages_per_req + (t >> lps)];
      const int slot =
          __hip_atomic_load(&v.rev[(size_t)r * v.max_context + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      guess = g < 0 && slot < 0;
    }
    const unsigned long long m = __ballot(guess);
    sh.tok[lane] = guess ? t : -1;
    if (guess) sh.gpos[__popcll(m & ((1ull << lane) - 1ull))] = (int8_t)lane;
    if (lane == 0) sh.n_guess = __popcll(m);
  }
  __syncthreads();
  const int ng = sh.n_guess;
  // wave w reads guessed rows w, w + kRsWaves, ... into registers
  u32x4 x[RPW][CPL];
  int pos_of[RPW];
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int rank = k * kRsWaves + wave;
    pos_of[k] = rank < ng ? sh.gpos[rank] : -1;
    if (pos_of[k] >= 0) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + sh.tok[pos_of[k]]) * ROW_BYTES);
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) x[k][u] = s4[lane + 64 * u];
    }
  }
  // wait for the bookkeeper: poll with plain device-coherent loads (an
  // acquire per poll would invalidate the caches each time), one acquire
  // fence once the flag is seen
  if (tid == 0) {
    int spins = 0;
    while (__hip_atomic_load(&sc.flag[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
      if (++spins > kSpinLimit) break;
      __builtin_amdgcn_s_sleep(4);
    }
    sh.go = spins <= kSpinLimit;
    if (spins > kSpinLimit) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, 0xFFFFFFFFu);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (!sh.go) return;
  const unsigned long long part_bits = ~0ull >> (64 - kRsPart);
  const unsigned long long am = (sc.miss_mask[(size_t)i * sc.words + (j0 >> 6)] >> (j0 & 63)) & part_bits;
  unsigned long long gm = 0ull;
  for (int k = 0; k < ng; ++k) gm |= 1ull << sh.gpos[k];
  const int32_t* plan = a.plan_out + (size_t)i * K + j0;
  // rows that were guessed and are misses: from registers
#pragma unroll
  for (int k = 0; k < RPW; ++k) {
    const int pos = pos_of[k];
    const int dst = pos >= 0 && ((am >> pos) & 1ull) ? plan[pos] : -1;
    if (dst >= 0) {
      u32x4* d4 = reinterpret_cast<u32x4*>(a.pool_rows + (int64_t)dst * ROW_BYTES);
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) d4[lane + 64 * u] = x[k][u];
    }
  }
  // misses that were not guessed (rare): read now
  {
    unsigned long long m = am & ~gm;
    for (int rank = 0; m; ++rank) {
      const int pos = __ffsll((long long)m) - 1;
      m &= m - 1ull;
      if (rank % kRsWaves != wave) continue;
      const int dst = plan[pos];
      if (dst < 0) continue;
      const int t = a.idx[(size_t)i * K + j0 + pos];
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + t) * ROW_BYTES);
      u32x4* d4 = reinterpret_cast<u32x4*>(a.pool_rows + (int64_t)dst * ROW_BYTES);
      u32x4 y[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) y[u] = s4[lane + 64 * u];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) d4[lane + 64 * u] = y[u];
    }
  }
  if (FP8 && tid < kRsPart) {  // one fp8 scale per missed row
    const int pos = tid;
    if ((am >> pos) & 1ull) {
      const int dst = plan[pos];
      const int t = a.idx[(size_t)i * K + j0 + pos];
      if (dst >= 0) a.pool_scales[dst] = a.host_scales[hbase + t];
    }
  }
}

template <int ROW_BYTES, bool FP8>
__global__ __launch_bounds__(kRsThreads) void k_resolve(RsArgs a, StateView v, RsScratch sc) {
  __shared__ RsShared sh;
  const int tid = threadIdx.x;
  if (tid == 0) sh.role = (int)atomicAdd(&sc.ticket[0], 1u);
  __syncthreads();
  const int role = sh.role;
  if (role < a.n_req) {
    bookkeep(a, v, sc, sh, role);
  } else {
    const int q = role - a.n_req;
    const int i = q / sc.parts, c = q - i * sc.parts;
    copy_part<ROW_BYTES, FP8>(a, v, sc, sh, i, c);
    __syncthreads();
    if (tid == 0 && atomicAdd(&sc.exit_cnt[i], 1u) == (uint32_t)(sc.parts - 1)) {
      sc.flag[i] = 0;  // every copy workgroup of request i has seen the flag
      sc.exit_cnt[i] = 0;
    }
  }
  __syncthreads();
  if (tid == 0 && atomicAdd(&sc.ticket[1], 1u) == gridDim.x - 1) {
    sc.ticket[0] = 0;  // every workgroup has taken its role
    sc.ticket[1] = 0;
  }
}

hs_status launch_resolve(hs_pool* p, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                         int32_t* plan_out, int32_t* counts_out, hipStream_t s) {
  StateView v = make_view(p);
  RsScratch sc;
  sc.miss_mask = reinterpret_cast<unsigned long long*>(p->state + p->off.rs_miss_mask);
  sc.flag = reinterpret_cast<uint32_t*>(p->state + p->off.rs_flag);
  sc.exit_cnt = reinterpret_cast<uint32_t*>(p->state + p->off.rs_exit);
  sc.ticket = reinterpret_cast<uint32_t*>(p->state + p->off.rs_ticket);
  sc.words = (p->d.top_k + 63) / 64;
  sc.parts = (p->d.top_k + kRsPart - 1) / kRsPart;
  RsArgs a{idx, req_ids, n_req, plan_out, counts_out, static_cast<const uint8_t*>(p->host_rows),
           p->host_scales, p->pool_rows, p->pool_scales};
  const int grid = n_req * (1 + sc.parts);
  switch (p->d.kv_dtype) {
    case HS_F32:
      k_resolve<2304, false><<<grid, kRsThreads, 0, s>>>(a, v, sc);
      break;
    case HS_BF16:
      k_resolve<1152, false><<<grid, kRsThreads, 0, s>>>(a, v, sc);
      break;
    default:
      k_resolve<576, true><<<grid, kRsThreads, 0, s>>>(a, v, sc);
      break;
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
