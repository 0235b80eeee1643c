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
//   copy workgroup (request i, part c), one per 16 plan positions (4 per
//     wave): reads the page table and reverse map itself to guess which of
//     its tokens miss and starts reading those rows from the mapped host
//     store over PCIe right away, then waits for the flag and writes the
//     rows the bookkeeper actually classified as misses into their hot
//     slots (rows it did not guess are read then). The guess only decides
//     how early the PCIe reads start; which rows are written comes from the
//     bookkeeper.
// Bookkeeper thread t owns plan positions [tP, tP + P) and LRU positions
// [tQ, tQ + Q) (P, Q powers of two), so each ordered compaction is one
// block-wide scan; every table lookup of a phase is issued before any is
// used.
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
  unsigned long long* miss_mask;  // [batch][words] miss bits of 64 plan positions
  uint32_t* flag;                 // [batch] 1 once request i's plan is published
  uint32_t* exit_cnt;             // [batch] copy workgroups of request i done
  uint32_t* ticket;               // [2] roles handed out, workgroups exited
  int words;                      // ceil(K / 64) mask words per request
  int parts;                      // ceil(K / kRsPart) copy workgroups per request
};

enum : int { kPad = 0, kRes = 1, kHot = 2, kMiss = 3 };
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kRsPos = kMaxTopK / kRsThreads;      // plan positions per bookkeeper thread, at most
constexpr int kRsSlots = kMaxHotRows / kRsThreads;  // LRU positions per bookkeeper thread, at most
constexpr int kRsPart = 4 * kRsWaves;              // plan positions per copy workgroup
constexpr int kSpinLimit = 1 << 20;                // polls of the flag (>= 0.1 s) before giving up

struct RsArgs {
  const int32_t* idx;
  const int32_t* req_ids;
  int n_req;
  int P, Q;  // plan and LRU positions per bookkeeper thread
  int32_t* plan_out;
  int32_t* counts_out;
  const uint8_t* host_rows;
  const float* host_scales;
  uint8_t* pool_rows;
  float* pool_scales;
};

struct RsStatic {
  int tmp[kRsWaves + 1];
  unsigned long long mword[kMaxTopK / 64];
  int n_res, n_hot;
  int role;
  int go;
};

// Dynamic LDS of a bookkeeper: lru[S] (reused for the victims), tag[S] and
// hot_pages[S / page_size] int32, flag[S] uint8 (bit0: hit this step, bit1:
// victim).
__host__ __device__ inline size_t rs_dyn_bytes(int S, int HP) {
  return 8 * (size_t)S + 4 * (size_t)HP + (size_t)S;
}

// The bookkeeper issues every global load before its first global store:
// the vector memory counter counts stores too, so a load waited for after
// a store would also wait for that store to complete.
__device__ __forceinline__ void bookkeep(const RsArgs& a, const StateView& v, const RsScratch& sc, RsStatic& st,
                                         unsigned char* dyn, int i) {
  const int tid = threadIdx.x;
  const int K = v.top_k, S = v.hot_rows, ps = v.page_size, lps = v.log2_ps, HP = v.hot_pages_per_req;
  const int P = a.P, Q = a.Q;
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
  const int32_t* hp_g = v.hot_pages + (size_t)r * HP;
  int32_t* lru = reinterpret_cast<int32_t*>(dyn);
  int32_t* vic = lru;  // the victims, once every thread holds its LRU slice
  int32_t* tag_l = lru + S;
  int32_t* hp = tag_l + S;
  uint8_t* flag = reinterpret_cast<uint8_t*>(hp + HP);

  // 0. loads: LRU order, slot tags, hot pages (to LDS); this thread's
  //    selected tokens, then their page-table and reverse-map entries
  for (int s = tid; s < S; s += kRsThreads) {
    lru[s] = order[s];
    tag_l[s] = tag[s];
    flag[s] = 0;
  }
  for (int p = tid; p < HP; p += kRsThreads) hp[p] = hp_g[p];
  for (int w = tid; w < sc.words; w += kRsThreads) st.mword[w] = 0ull;
  if (tid == 0) st.n_res = st.n_hot = 0;
  int tok[kRsPos], code[kRsPos];  // code: pool row, -1 nothing, -2 miss
  int M, mbase;
  {
    int g[kRsPos], slot[kRsPos];
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      const int j = tid * P + e;
      tok[e] = (e < P && j < K) ? sel[j] : -1;
    }
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      const int t = tok[e];
      const int tt = (t >= 0 && t < L) ? t : 0;  // in-range address either way
      g[e] = pt[tt >> lps];
      slot[e] = rev[tt];
    }
    __syncthreads();  // LDS tables ready
    // 1. classify: resident > hot > miss (hit flags in LDS, no stores yet)
    int nm = 0, nr = 0, nh = 0;
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      code[e] = -1;
      const int j = tid * P + e;
      const int t = tok[e];
      if (!(e < P && j < K) || t < 0) continue;
      if (t >= L) {
        raise_error(v.error, HS_DEV_INDEX_RANGE, (uint32_t)r, (uint32_t)t);
      } else if (g[e] >= 0) {
        code[e] = g[e] * ps + (t & (ps - 1));
        ++nr;
      } else if (slot[e] >= 0) {
        const int sl = slot[e];
        const int hpg = sl < S ? hp[sl >> lps] : -1;
        if (hpg >= 0) {
          flag[sl] = 1;
          code[e] = hpg * ps + (sl & (ps - 1));
          ++nh;
        } else {
          raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)sl);
        }
      } else {
        code[e] = -2;
        atomicOr(&st.mword[j >> 6], 1ull << (j & 63));
        ++nm;
      }
    }
    if (nr) atomicAdd(&st.n_res, nr);
    if (nh) atomicAdd(&st.n_hot, nh);
    mbase = block_excl_sum(nm, st.tmp, M);  // misses rank in token order
  }
  // 2. untouched slots in LRU order; the first M of them are the victims
  int my[kRsSlots];
  int kc = 0;
#pragma unroll
  for (int e = 0; e < kRsSlots; ++e) {
    const int x = tid * Q + e;
    const int s = (e < Q && x < S) ? lru[x] : -1;
    my[e] = (s >= 0 && !(flag[s] & 1)) ? s : -1;
    kc += my[e] >= 0 ? 1 : 0;
  }
  int kept;
  const int kbase = block_excl_sum(kc, st.tmp, kept);  // (its barriers end the reads of lru)
  {
    int kpos = kbase;
#pragma unroll
    for (int e = 0; e < kRsSlots; ++e) {
      if (my[e] >= 0) {
        if (kpos < M) {
          vic[kpos] = my[e];
          flag[my[e]] |= 2;
        }
        ++kpos;
      }
    }
  }
  __syncthreads();
  // 3. stores. New LRU order: the untouched non-victims in their order,
  //    then the hit and victim slots in ascending slot number, which all
  //    take stamp n. Victims lose their old token.
  {
    int kpos = kbase;
#pragma unroll
    for (int e = 0; e < kRsSlots; ++e) {
      if (my[e] >= 0) {
        if (kpos >= M) {
          order[kpos - M] = my[e];
        } else {
          const int old = tag_l[my[e]];
          if (old >= 0 && old < v.max_context) rev[old] = -1;
        }
        ++kpos;
      }
    }
  }
  int fc = 0;
#pragma unroll
  for (int e = 0; e < kRsSlots; ++e) {
    const int s = tid * Q + e;
    fc += (e < Q && s < S && flag[s] != 0) ? 1 : 0;
  }
  int ftot;
  int fpos = (kept - M) + block_excl_sum(fc, st.tmp, ftot);
#pragma unroll
  for (int e = 0; e < kRsSlots; ++e) {
    const int s = tid * Q + e;
    if (e < Q && s < S && flag[s] != 0) {
      order[fpos++] = s;
      stamp[s] = n;
    }
  }
  // fill the victims with the misses (i-th miss -> i-th victim)
  int mr = mbase;
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) {
    if (code[e] != -2) continue;
    const int t = tok[e];
    const int vs = vic[mr++];
    tag[vs] = t;
    rev[t] = vs;
    const int hpg = hp[vs >> lps];
    if (hpg >= 0) {
      code[e] = hpg * ps + (vs & (ps - 1));
    } else {
      code[e] = -1;
      raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)vs);
    }
  }
  // 4. plan and miss words; publish them to the copy workgroups; counts
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) {
    const int j = tid * P + e;
    if (e < P && j < K) plan[j] = code[e] < 0 ? -1 : code[e];
  }
  for (int w = tid; w < sc.words; w += kRsThreads) sc.miss_mask[(size_t)i * sc.words + w] = st.mword[w];
  publish();
  if (tid == 0) {
    const int n_res = st.n_res, n_hot = st.n_hot;
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

// Copy the missed rows of plan positions [c kRsPart, (c + 1) kRsPart) of
// request i; wave w takes 4 of them.
template <int ROW_BYTES, bool FP8>
__device__ __forceinline__ void copy_part(const RsArgs& a, const StateView& v, const RsScratch& sc, RsStatic& st,
                                          int i, int c) {
  constexpr int CH = ROW_BYTES / 16;   // 16-byte chunks per row
  constexpr int CPL = (CH + 63) / 64;  // chunks per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = v.top_k, lps = v.log2_ps;
  const int j0 = kRsPart * c + 4 * wave;
  const int r0 = a.req_ids[i];
  const bool valid_req = r0 >= 0 && r0 < v.max_requests;
  const int r = valid_req ? r0 : 0;
  const int L = valid_req ? v.ctx_len[r] : 0;
  const int64_t hbase = v.host_base[r];
  // Guess the misses from the current tables. The bookkeeper may be
  // updating them meanwhile (atomic reads, any outcome is harmless): the
  // guess only decides which host reads start before the plan is known.
  int t = -1;
  bool guess = false;
  if (lane < 4) {
    const int j = j0 + lane;
    t = j < K ? a.idx[(size_t)i * K + j] : -1;
    if (t >= 0 && t < L) {
      const int g = v.page_table[(size_t)r * v.pages_per_req + (t >> lps)];
      const int slot =
          __hip_atomic_load(&v.rev[(size_t)r * v.max_context + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      guess = g < 0 && slot < 0;
    }
  }
  const unsigned gb = (unsigned)(__ballot(guess) & 0xFull);
  int tk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tk[k] = __shfl(t, k, 64);
  u32x4 x[4][CPL];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((gb >> k) & 1u) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + tk[k]) * ROW_BYTES);
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
    st.go = spins <= kSpinLimit;
    if (spins > kSpinLimit) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, 0xFFFFFFFFu);
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (!st.go) return;
  // (j0 is a multiple of 4, so the 4 bits lie in one mask word)
  const unsigned am = (unsigned)((sc.miss_mask[(size_t)i * sc.words + (j0 >> 6)] >> (j0 & 63)) & 0xFull);
  const int32_t* plan = a.plan_out + (size_t)i * K + j0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (!((am >> k) & 1u)) continue;
    const int dst = plan[k];
    if (dst < 0) continue;
    u32x4* d4 = reinterpret_cast<u32x4*>(a.pool_rows + (int64_t)dst * ROW_BYTES);
    if ((gb >> k) & 1u) {
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) d4[lane + 64 * u] = x[k][u];
    } else {  // a miss that was not guessed (rare): read it now
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + tk[k]) * ROW_BYTES);
      u32x4 y[CPL];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) y[u] = s4[lane + 64 * u];
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < CH) d4[lane + 64 * u] = y[u];
    }
  }
  if (FP8 && lane < 4 && ((am >> lane) & 1u)) {  // one fp8 scale per missed row
    const int dst = plan[lane];
    if (dst >= 0) a.pool_scales[dst] = a.host_scales[hbase + t];
  }
}

template <int ROW_BYTES, bool FP8>
__global__ __launch_bounds__(kRsThreads) void k_resolve(RsArgs a, StateView v, RsScratch sc) {
  __shared__ RsStatic st;
  extern __shared__ __align__(16) unsigned char rs_dyn[];
  const int tid = threadIdx.x;
  if (tid == 0) st.role = (int)atomicAdd(&sc.ticket[0], 1u);
  __syncthreads();
  const int role = st.role;
  if (role < a.n_req) {
    bookkeep(a, v, sc, st, rs_dyn, role);
  } else {
    const int q = role - a.n_req;
    const int i = q / sc.parts, c = q - i * sc.parts;
    copy_part<ROW_BYTES, FP8>(a, v, sc, st, i, c);
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

static int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
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
  RsArgs a{idx, req_ids, n_req,
           pow2_at_least((p->d.top_k + kRsThreads - 1) / kRsThreads),
           pow2_at_least((v.hot_rows + kRsThreads - 1) / kRsThreads),
           plan_out, counts_out, static_cast<const uint8_t*>(p->host_rows),
           p->host_scales, p->pool_rows, p->pool_scales};
  const size_t dyn = (rs_dyn_bytes(v.hot_rows, v.hot_pages_per_req) + 15) & ~(size_t)15;
  const int grid = n_req * (1 + sc.parts);
  switch (p->d.kv_dtype) {
    case HS_F32:
      k_resolve<2304, false><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
    case HS_BF16:
      k_resolve<1152, false><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
    default:
      k_resolve<576, true><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
