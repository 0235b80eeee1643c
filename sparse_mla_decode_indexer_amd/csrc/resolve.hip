// Resolve of the selected tokens into physical pool rows ([P2] "vLLM GLM 5.3
// 优化：混合 HiSparse 卸载" §"混合 HiSparse 的技术实现", residency state 2: one
// fused pass reads a resident row in place, reads a hot row and refreshes its
// LRU entry, or on a miss copies the single row from pinned host memory into
// the LRU slot; [P3] §"融合内核与CUDA图兼容": the pass is graph-capturable).
//
// One kernel, two kinds of workgroup. Workgroup b serves batch position
// i = b mod n_req; the workgroups of one position take roles from that
// position's ticket counter in the order they start:
//   bookkeeper (ticket 0), one per request: classifies the K
//     tokens (resident > hot > miss), stamps the hit slots, picks the victims
//     and rewrites the LRU order with ordered compactions in LDS, writes the
//     plan and the counts, and for every plan position the hot slot and that
//     slot's old token (misses) and last the copy destination: the pool row
//     a miss is copied to, or -1, tagged with the launch's epoch;
//   copy workgroup (ticket 1 + c: part c), one per 64 plan positions (4 per
//     wave): reads the page table and reverse map itself to guess which of
//     its tokens miss and starts reading those rows from the mapped host
//     store over PCIe right away; each wave then waits until its four copy
//     destinations are published (a wave whose four positions are padding
//     or on resident pages cannot hold a miss and ends at once), writes the
//     rows the bookkeeper actually
//     classified as misses into their hot slots (rows it did not guess are
//     read then) and moves the slots' tags and reverse-map entries from the
//     old tokens to the new. The guess only decides how early the PCIe reads
//     start; which rows are written comes from the bookkeeper.
// Bookkeeper thread t owns plan positions t + 1024 e (e < P), so wave w
// holds plan positions 1024 e + 64 w .. + 63 and the token-order rank of a
// miss comes from a ballot and per-wave counts. It owns
// LRU positions [tQ, tQ + Q) (P, Q powers of two, Q >= 4), so each ordered
// compaction of the LRU order is one block-wide scan. The request's page
// table is staged in LDS when it fits (kRsPtLds entries), so that only the
// reverse-map lookups are scattered global loads.
// A copy workgroup holds a later ticket than its bookkeeper, which is
// therefore running and never waits, so the wait always ends; it is also
// bounded (HS_DEV_TIMEOUT is raised past the bound and the copy skipped).
// Epochs. Every workgroup reads its position's launch sequence number
// before it takes its ticket, and counts itself done at its end; the last
// workgroup of the position to be done advances the sequence and clears the
// position's ticket and done counters, so all workgroups of one launch and
// position share one epoch, the next launch has another and starts from
// cleared counters, and nothing waits for the end of a launch. The counters
// are per batch position, so no atomic is contended by more than one
// request's workgroups.
// A destination entry is a 64-bit (epoch, pool row) pair, and a copy wave
// takes an entry as published only when it carries its own launch's epoch.
// An entry left from an earlier launch therefore never passes for this
// launch's, even when that launch timed out before its copy waves read it,
// and no entry has to be put back to "pending" after use. (The sequence is
// 32 bits; an entry is rewritten by every launch that covers its batch
// position, so only one unwritten for 2^32 - 1 launches could alias.)
//
// Select and resolve in one launch (hs_select_resolve). The bookkeeper
// workgroup first runs the request's top-K select (the filter kernel ran
// before) in the LDS it then reuses, keeps the selection in LDS for the
// bookkeeping, writes it to idx_out and publishes it by storing the launch's
// epoch in the position's selection flag once those stores have completed.
// Copy workgroups wait for that flag (bounded, like their other wait)
// before they read the selection, with device-coherent loads. This saves
// the kernel boundary between the two steps and the bookkeeper's reload of
// the selection.
//
// LRU order. lru_order lists all S slots in ascending (stamp, slot). With U
// the slots hit this step and M misses, the victims are the first M slots of
// lru_order \ U, and the new order is (lru_order \ U \ victims) followed by
// (U and victims) in ascending slot number: all of those now carry the
// newest stamp, and equal stamps order by slot. That equals choosing victims
// by sorting the untouched slots by (stamp, slot).
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include "topk_select.h"

namespace hs {

// Native 16-byte vector: arrays of it stay in registers (HIP's uint4 struct
// made the prefetch arrays go through scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RsScratch {
  uint64_t* mdst;                 // [batch][K] (epoch << 32) | pool row a missed position is copied to, else -1
  int32_t* mslot;                 // [batch][K] hot slot a missed position takes, else -1
  int32_t* mold;                  // [batch][K] token that slot held before (or -1)
  uint32_t* ctl;                  // [batch][4]: roles handed out, launch sequence (epoch - 1), workgroups done,
                                  // selection published (epoch; select-and-resolve only)
  int parts;                      // ceil(K / kRsPart) copy workgroups per request
};

enum : int { kPad = 0, kRes = 1, kHot = 2, kMiss = 3 };
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kRsPos = kMaxTopK / kRsThreads;      // plan positions per bookkeeper thread, at most
constexpr int kRsSlots = kMaxHotRows / kRsThreads;  // LRU positions per bookkeeper thread, at most
constexpr int kRsPart = 4 * kRsWaves;              // plan positions per copy workgroup
constexpr int kSpinLimit = 1 << 20;                // polls of a destination (>= 0.1 s) before giving up
constexpr uint32_t kRsSeqWrap = 0xFFFFFFFFu;        // sequence values 0 .. 2^32 - 2: epochs 1 .. 2^32 - 1

// A published destination: the launch's epoch (never 0, the workspace's
// initial value) above the pool row (or -1).
__device__ __forceinline__ uint64_t rs_entry(uint32_t epoch, int32_t dst) {
  return ((uint64_t)epoch << 32) | (uint32_t)dst;
}

struct RsArgs {
  const int32_t* idx;             // the selection (select-and-resolve: written by this launch)
  const int32_t* req_ids;
  int n_req;
  int P, Q;    // plan and LRU positions per bookkeeper thread
  int pt_lds;  // page-table entries staged in LDS (0: look up in global memory)
  int spin_limit;  // polls of a destination before a copy wave gives up
  int32_t* plan_out;
  int32_t* counts_out;
  const uint8_t* host_rows;  // fp8 rows carry their scale (host row stride kHostRowStrideFp8)
  uint8_t* pool_rows;
  float* pool_scales;
  // select-and-resolve only: the scores, the top-K scratch and the LDS
  // offset of the selection (past both the select's and the bookkeeper's LDS)
  const float* scores;
  int64_t score_stride;
  TkScratch tk;
  int sel_off;
};

constexpr int kRsPtLds = 8192;  // page-table entries a bookkeeper stages in LDS, at most
// dynamic LDS of a select-and-resolve workgroup, at most: 160 KiB per
// workgroup less 4 KiB for the static LDS (RsStatic and the select's tables)
constexpr size_t kRsFusedMaxDyn = (size_t)156 << 10;

struct RsStatic {
  int tmp[kRsWaves + 1];
  int wmiss[kRsPos * kRsWaves];      // misses per (e, wave), then their exclusive prefix
  int n_res, n_hot;
  int role;
  uint32_t epoch;
};

// Dynamic LDS of a bookkeeper, with Spad = 1024 Q >= S: lru[Spad] and
// tag[Spad] int32 (padded with -1), victims[K] int32, hot_pages[HP] int32,
// page table[PT] int32, flag[Spad] uint8 (bit0: hit this step, bit1:
// victim).
__host__ __device__ inline size_t rs_dyn_bytes(int Spad, int K, int HP, int PT) {
  return 8 * (size_t)Spad + 4 * (size_t)K + 4 * (size_t)HP + 4 * (size_t)PT + (size_t)Spad;
}

// The bookkeeper issues every global load before its first global store
// (the vector memory counter counts stores too, so a load waited for after
// a store would also wait for that store), and keeps its loops free of
// per-lane conditions: loop bounds are uniform, LDS tables are padded, and
// each phase issues all of its LDS reads before using them.
__device__ __forceinline__ void bookkeep(const RsArgs& a, const StateView& v, const RsScratch& sc, RsStatic& st,
                                         unsigned char* dyn, int i, const int32_t* sel) {
  const int tid = threadIdx.x;
  const int K = v.top_k, S = v.hot_rows, ps = v.page_size, lps = v.log2_ps, HP = v.hot_pages_per_req;
  const int P = a.P, Q = a.Q, Spad = Q * kRsThreads;
  int32_t* plan = a.plan_out + (size_t)i * K;
  // this thread's selected tokens: read together with the request id (their
  // addresses do not depend on it)
  int tok[kRsPos];
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) {
    if (e < P) {
      const int j = e * kRsThreads + tid;
      const int t = sel[min(j, K - 1)];
      tok[e] = j < K ? t : -1;
    }
  }
  const int r0 = a.req_ids[i];
  // What the copy workgroups read (slot, old token, destination) is written
  // with device-coherent stores; a position's destination goes out (from
  // the thread that owns the position) once that thread's other stores have
  // completed, so a copy wave that sees it also sees the rest. The LRU
  // state is written afterwards: no copy workgroup reads it.
  auto put = [](int32_t* p, int x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
  const uint32_t epoch = st.epoch;
  auto publish = [epoch](uint64_t* p, int32_t dst) {
    __hip_atomic_store(p, rs_entry(epoch, dst), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  uint64_t* mdst = sc.mdst + (size_t)i * K;
  int32_t* mslot = sc.mslot + (size_t)i * K;
  int32_t* mold = sc.mold + (size_t)i * K;
  auto stores_done = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);  // this thread's stores have completed
    asm volatile("" ::: "memory");
  };
  if (r0 < 0 || r0 >= v.max_requests) {
    if (tid == 0) {
      raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)r0);
      if (a.counts_out) a.counts_out[3 * i] = a.counts_out[3 * i + 1] = a.counts_out[3 * i + 2] = 0;
    }
    for (int j = tid; j < K; j += kRsThreads) {
      put(&plan[j], -1);
      put(&mslot[j], -1);
    }
    stores_done();
    for (int j = tid; j < K; j += kRsThreads) publish(&mdst[j], -1);
    return;
  }
  const int r = r0;
  const int L = v.ctx_len[r];
  const int n = v.step[r] + 1;
  int cnt0[3];  // running counters, loaded before the first store
#pragma unroll
  for (int k = 0; k < 3; ++k) cnt0[k] = tid == 0 ? v.counters[3 * r + k] : 0;
  const int32_t* pt = v.page_table + (size_t)r * v.pages_per_req;
  int32_t* rev = v.rev + (size_t)r * v.max_context;
  int32_t* tag = v.slot_tag + (size_t)r * S;
  int32_t* stamp = v.slot_stamp + (size_t)r * S;
  int32_t* order = v.lru_order + (size_t)r * S;
  const int32_t* hp_g = v.hot_pages + (size_t)r * HP;
  int32_t* lru = reinterpret_cast<int32_t*>(dyn);
  int32_t* tag_l = lru + Spad;
  int32_t* vic = tag_l + Spad;
  int32_t* hp = vic + K;
  int32_t* ptl = hp + HP;
  uint8_t* flag = reinterpret_cast<uint8_t*>(ptl + a.pt_lds);
  const int npg = (L + ps - 1) >> lps;  // pages of the context
  // The request's whole page table is staged when it fits (a.pt_lds is then
  // pages_per_req), so that neither the staging nor the reverse-map lookups
  // below wait for the context length: lookups are clamped to the request's
  // rows of the tables, and the length only enters the classification.
  const bool pt_in_lds = a.pt_lds > 0;

  // 0. loads: LRU order and slot tags (coalesced, then to LDS), hot pages;
  //    this thread's selected tokens, then their page-table and reverse-map
  //    entries
  {
    int ov[kRsSlots], tv[kRsSlots];
#pragma unroll
    for (int e = 0; e < kRsSlots; ++e) {
      if (e < Q) {
        const int x = min(e * kRsThreads + tid, S - 1);
        ov[e] = order[x];
        tv[e] = tag[x];
      }
    }
#pragma unroll
    for (int e = 0; e < kRsSlots; ++e) {
      if (e < Q) {
        const int x = e * kRsThreads + tid;
        lru[x] = x < S ? ov[e] : -1;
        tag_l[x] = x < S ? tv[e] : -1;
        flag[x] = 0;
      }
    }
  }
  // this thread's slot stamps, updated in place at the end (whole 16 bytes)
  const bool stamp4 = (S & 3) == 0;
  int4 st4[kRsSlots / 4];
#pragma unroll
  for (int e4 = 0; e4 < kRsSlots / 4; ++e4) {
    const int x = tid * Q + 4 * e4;
    if (4 * e4 < Q && stamp4 && x < S) st4[e4] = reinterpret_cast<const int4*>(stamp)[x >> 2];
  }
  for (int p = tid; p < HP; p += kRsThreads) hp[p] = hp_g[p];
  if (pt_in_lds)
    for (int p = tid; p < a.pt_lds; p += kRsThreads) ptl[p] = pt[p];
  if (tid == 0) st.n_res = st.n_hot = 0;
  const int lane = tid & 63, wave = tid >> 6;
  const unsigned long long below = (1ull << lane) - 1ull;
  int code[kRsPos];  // code: pool row, -1 nothing, -2 miss
  uint32_t missbits = 0u;  // bit e: position e of this thread is a miss
  unsigned long long mb[kRsPos];  // miss bits of this wave's 64 positions of each e
  int M;
  {
    int g[kRsPos], sl[kRsPos];
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P) {
        const int t = tok[e];
        const int tt = (t >= 0 && t < v.max_context) ? t : 0;  // an address inside the request's rows
        if (!pt_in_lds) g[e] = pt[tt >> lps];
        sl[e] = rev[tt];
      }
    }
    __syncthreads();  // LDS tables ready
    // keep the counter loads here, ahead of every store (not sunk to their use)
    asm volatile("" : "+v"(cnt0[0]), "+v"(cnt0[1]), "+v"(cnt0[2]));
    // 1. classify: resident > hot > miss (hit flags in LDS, no stores yet)
    int hpg[kRsPos];
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P) {
        const int t = tok[e];
        const int tt = (t >= 0 && t < v.max_context) ? t : 0;
        if (pt_in_lds) g[e] = ptl[tt >> lps];
        hpg[e] = hp[min(max(sl[e], 0), S - 1) >> lps];
      }
    }
    int bad_tok = -1, bad_slot = -1;  // first offending entry of this thread
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P) {
        const int j = e * kRsThreads + tid;
        const int t = tok[e];
        const bool ok = t >= 0 && t < L;
        const bool res = ok && g[e] >= 0;
        const bool cand = ok && g[e] < 0 && sl[e] >= 0;
        const bool hot = cand && sl[e] < S && hpg[e] >= 0;
        const bool miss = ok && g[e] < 0 && sl[e] < 0;
        bad_tok = (bad_tok < 0 && j < K && t >= L) ? t : bad_tok;
        bad_slot = (bad_slot < 0 && cand && !hot) ? sl[e] : bad_slot;
        if (hot) flag[sl[e]] = 1;
        missbits |= miss ? (1u << e) : 0u;
        code[e] = res ? g[e] * ps + (t & (ps - 1)) : hot ? hpg[e] * ps + (sl[e] & (ps - 1)) : miss ? -2 : -1;
        mb[e] = __ballot(miss);
        const int nr = __popcll(__ballot(res)), nh = __popcll(__ballot(hot));
        if (lane == 0) {
          st.wmiss[e * kRsWaves + wave] = __popcll(mb[e]);
          if (nr) atomicAdd(&st.n_res, nr);
          if (nh) atomicAdd(&st.n_hot, nh);
        }
      }
    }
    if (bad_tok >= 0) raise_error(v.error, HS_DEV_INDEX_RANGE, (uint32_t)r, (uint32_t)bad_tok);
    if (bad_slot >= 0) raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)bad_slot);
    __syncthreads();
    // token-order rank base of each (e, wave): exclusive prefix over e-major
    // (e, wave) of the per-wave miss counts (wave 0; P * 16 <= 64 entries)
    if (wave == 0) {
      const int c = lane < P * kRsWaves ? st.wmiss[lane] : 0;
      int x = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane < P * kRsWaves) st.wmiss[lane] = x - c;
      if (lane == 63) st.tmp[0] = x;
    }
    __syncthreads();
    M = st.tmp[0];
  }
  // A request whose selected tokens are all resident touches no slot: its
  // LRU order, tags and stamps stay as they are, so steps 2 and 3 and the
  // LRU part of step 5 are skipped (a uniform branch). Without misses the
  // victim slots are not looked up either.
  const bool touched = M > 0 || st.n_hot > 0;
  // 2. untouched slots in LRU order (thread t holds LRU positions [tQ, tQ+Q));
  //    the first M of them are the victims
  int my[kRsSlots];
  uint32_t km = 0u;  // bit e: my[e] is untouched
  uint32_t fm = 0u;  // bit e: slot tQ + e is fresh (hit or victim)
  int kept = 0, kbase = 0, fbase = 0;
  if (touched) {
#pragma unroll
    for (int e4 = 0; e4 < kRsSlots / 4; ++e4) {
      if (4 * e4 < Q) {
        const int4 x = reinterpret_cast<const int4*>(lru + tid * Q)[e4];
        my[4 * e4] = x.x;
        my[4 * e4 + 1] = x.y;
        my[4 * e4 + 2] = x.z;
        my[4 * e4 + 3] = x.w;
      }
    }
    {
      int fl[kRsSlots];
#pragma unroll
      for (int e = 0; e < kRsSlots; ++e) {
        if (e < Q) {
          const int s = max(my[e], 0);
          fl[e] = flag[s];
        }
      }
#pragma unroll
      for (int e = 0; e < kRsSlots; ++e) {
        if (e < Q) {
          km |= (my[e] >= 0 && !(fl[e] & 1)) ? (1u << e) : 0u;
        }
      }
    }
    kbase = block_excl_sum(__popc(km), st.tmp, kept);
    // 3. victims (LDS)
    {
      int kpos = kbase;
#pragma unroll
      for (int e = 0; e < kRsSlots; ++e) {
        if (e < Q) {
          if ((km >> e) & 1u) {
            if (kpos < M) {
              vic[kpos] = my[e];
              flag[my[e]] |= 2;
            }
            ++kpos;
          }
        }
      }
    }
    __syncthreads();
    // fresh slots (hit or victim) of this thread's slot range [tQ, tQ + Q)
#pragma unroll
    for (int e4 = 0; e4 < kRsSlots / 4; ++e4) {
      if (4 * e4 < Q) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(flag + tid * Q)[e4];
        fm |= ((w & 0xFFu) ? 1u : 0u) << (4 * e4);
        fm |= ((w & 0xFF00u) ? 1u : 0u) << (4 * e4 + 1);
        fm |= ((w & 0xFF0000u) ? 1u : 0u) << (4 * e4 + 2);
        fm |= ((w & 0xFF000000u) ? 1u : 0u) << (4 * e4 + 3);
      }
    }
    int ftot;
    fbase = (kept - M) + block_excl_sum(__popc(fm), st.tmp, ftot);
  }  // touched
  // the i-th miss takes the i-th victim
  int vs[kRsPos];
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) vs[e] = -1;
  if (M > 0) {
    int hv[kRsPos];
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P) {
        const int mr = st.wmiss[e * kRsWaves + wave] + __popcll(mb[e] & below);  // misses before j
        vs[e] = vic[min(mr, max(M - 1, 0))];
      }
    }
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P) hv[e] = hp[max(vs[e], 0) >> lps];
    }
    int bad_vic = -1;
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P && code[e] == -2) {
        bad_vic = (bad_vic < 0 && hv[e] < 0) ? vs[e] : bad_vic;
        code[e] = hv[e] >= 0 ? hv[e] * ps + (vs[e] & (ps - 1)) : -1;
      }
    }
    if (bad_vic >= 0) raise_error(v.error, HS_DEV_PAGE_RANGE, (uint32_t)r, (uint32_t)bad_vic);
  }
  // 4. plan, slots and old tokens, then the copy destinations
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) {
    const int j = e * kRsThreads + tid;
    if (e < P && j < K) {
      const bool miss = (missbits >> e) & 1u;
      put(&plan[j], code[e] >= 0 ? code[e] : -1);
      put(&mslot[j], miss ? vs[e] : -1);
      if (miss) put(&mold[j], tag_l[vs[e]]);
    }
  }
  stores_done();
#pragma unroll
  for (int e = 0; e < kRsPos; ++e) {
    const int j = e * kRsThreads + tid;
    if (e < P && j < K) publish(&mdst[j], ((missbits >> e) & 1u) && code[e] >= 0 ? code[e] : -1);
  }
  // 5. LRU state: the untouched non-victims keep their order at the front,
  //    then the hit and victim slots in ascending slot number, all with
  //    stamp n; victims lose their old token and take the missed one. The
  //    new order is assembled in LDS (the old one there is no longer read)
  //    and written out with coalesced 16-byte stores.
  {
    if (touched) {
      int kpos = kbase;
#pragma unroll
      for (int e = 0; e < kRsSlots; ++e) {
        if (e < Q) {
          if ((km >> e) & 1u) {
            if (kpos >= M) lru[kpos - M] = my[e];
            ++kpos;
          }
        }
      }
      int fpos = fbase;
#pragma unroll
      for (int e = 0; e < kRsSlots; ++e) {
        if (e < Q && ((fm >> e) & 1u)) {
          const int s = tid * Q + e;
          lru[fpos++] = s;
          if (!stamp4) stamp[s] = n;
        }
      }
#pragma unroll
      for (int e4 = 0; e4 < kRsSlots / 4; ++e4) {
        const int x = tid * Q + 4 * e4;
        if (4 * e4 < Q && stamp4 && x < S) {
          int4 w = st4[e4];
          const uint32_t f = fm >> (4 * e4);
          w.x = (f & 1u) ? n : w.x;
          w.y = (f & 2u) ? n : w.y;
          w.z = (f & 4u) ? n : w.z;
          w.w = (f & 8u) ? n : w.w;
          reinterpret_cast<int4*>(stamp)[x >> 2] = w;
        }
      }
    }  // touched
    // (the victims' tags and the reverse map are updated by the copy
    // workgroups, which hold each miss's token, slot and the slot's old token)
    // page recency for the residency manager: every page the indexer
    // selected a token of this step takes stamp n. With the page table in
    // LDS (no longer read) the selected pages are marked there and stamped
    // in one coalesced pass instead of one scattered store per token.
    int32_t* pstamp = v.page_stamp + (size_t)r * v.pages_per_req;
    constexpr int kTouched = INT32_MIN;
#pragma unroll
    for (int e = 0; e < kRsPos; ++e) {
      if (e < P && tok[e] >= 0 && tok[e] < L) {
        if (pt_in_lds)
          ptl[tok[e] >> lps] = kTouched;
        else
          pstamp[tok[e] >> lps] = n;
      }
    }
    __syncthreads();  // new order and page marks in LDS
    if (!touched) {
      // (the LRU order is unchanged)
    } else if ((S & 3) == 0) {
      for (int x = tid; x < S / 4; x += kRsThreads)
        reinterpret_cast<int4*>(order)[x] = reinterpret_cast<const int4*>(lru)[x];
    } else {
      for (int x = tid; x < S; x += kRsThreads) order[x] = lru[x];
    }
    if (pt_in_lds)
      for (int p = tid; p < npg; p += kRsThreads)
        if (ptl[p] == kTouched) pstamp[p] = n;
  }
  if (tid == 0) {
    const int n_res = st.n_res, n_hot = st.n_hot;
    if (a.counts_out) {
      a.counts_out[3 * i] = n_res;
      a.counts_out[3 * i + 1] = n_hot;
      a.counts_out[3 * i + 2] = M;
    }
    v.counters[3 * r] = cnt0[0] + n_res;
    v.counters[3 * r + 1] = cnt0[1] + n_hot;
    v.counters[3 * r + 2] = cnt0[2] + M;
    v.step[r] = n;
  }
}

// Copy the missed rows of plan positions [c kRsPart, (c + 1) kRsPart) of
// request i; wave w takes 4 of them.
template <int ROW_BYTES, bool FP8, bool FUSED>
__device__ __forceinline__ void copy_part(const RsArgs& a, const StateView& v, const RsScratch& sc,
                                          int i, int c, uint32_t epoch) {
  constexpr int CH = ROW_BYTES / 16;        // 16-byte chunks of a pool row
  constexpr int HCH = FP8 ? CH + 1 : CH;    // ... read of a host row (fp8: then the chunk holding the scale)
  constexpr int HSTRIDE = FP8 ? kHostRowStrideFp8 : ROW_BYTES;  // host row stride
  static_assert(16 * HCH <= HSTRIDE && HSTRIDE % 128 == 0, "host rows hold their chunks, 128-byte aligned");
  constexpr int CPL = (HCH + 63) / 64;      // chunks per lane
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = v.top_k, lps = v.log2_ps;
  const int j0 = kRsPart * c + 4 * wave;
  const int r0 = a.req_ids[i];
  const bool valid_req = r0 >= 0 && r0 < v.max_requests;
  const int r = valid_req ? r0 : 0;
  const int L = valid_req ? v.ctx_len[r] : 0;
  const int64_t hbase = v.host_base[r];
  if constexpr (FUSED) {  // wait until this launch's selection of position i is published
    const uint32_t* flag = sc.ctl + 4 * (size_t)i + 3;
    int spins = 0;
    while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch) {
      if (++spins > a.spin_limit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (spins > a.spin_limit) {
      if (lane == 0) raise_error(v.error, HS_DEV_TIMEOUT, (uint32_t)i, (uint32_t)j0);
      return;
    }
  }
  // Guess the misses from the current tables. The bookkeeper may be
  // updating them meanwhile (atomic reads, any outcome is harmless): the
  // guess only decides which host reads start before the plan is known.
  int t = -1;
  bool guess = false;
  bool settled = true;  // this position is certainly no miss: padding, out of range or on a resident page
  if (lane < 4) {
    const int j = j0 + lane;
    t = j >= K ? -1
        : FUSED ? __hip_atomic_load(&a.idx[(size_t)i * K + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                : a.idx[(size_t)i * K + j];
    if (t >= 0 && t < L) {
      const int g = v.page_table[(size_t)r * v.pages_per_req + (t >> lps)];
      const int slot =
          __hip_atomic_load(&v.rev[(size_t)r * v.max_context + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      guess = g < 0 && slot < 0;
      settled = g >= 0;
    }
  }
  // The page table does not change during a call, so the bookkeeper
  // classifies a position on a resident page (and padding) exactly as this
  // wave does: no copy. A wave with nothing but such positions is done
  // without waiting for the plan.
  if ((__ballot(settled) & 0xFull) == 0xFull) return;
  const unsigned gb = (unsigned)(__ballot(guess) & 0xFull);
  int tk[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) tk[k] = __shfl(t, k, 64);
  u32x4 x[4][CPL];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if ((gb >> k) & 1u) {
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + tk[k]) * HSTRIDE);
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < HCH) x[k][u] = s4[lane + 64 * u];  // (fp8: the scale comes with the row)
    }
  }
  // wait for the bookkeeper (each wave on its own): lanes 0..3 poll their
  // positions' destinations with device-coherent loads until each carries
  // this launch's epoch
  const bool mine = lane < 4 && j0 + lane < K;
  const size_t jj = (size_t)i * K + j0 + (lane & 3);
  int md = -1;
  int spins = 0;
  for (;;) {
    bool pending = false;
    if (mine) {
      const uint64_t w = __hip_atomic_load(&sc.mdst[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pending = (uint32_t)(w >> 32) != epoch;
      md = (int32_t)(uint32_t)w;
    }
    if (!__any(pending)) break;  // (loop condition uniform per wave)
    if (++spins > a.spin_limit) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (spins > a.spin_limit) {  // nothing of this wave's positions is written
    if (lane == 0) raise_error(v.error, HS_DEV_TIMEOUT, (uint32_t)i, (uint32_t)j0);
    return;
  }
  // A miss destination for a token outside [0, L) can only come from a
  // selection this wave did not see as the bookkeeper did: raise an error and
  // copy nothing for it rather than read outside the request's host rows.
  if (mine && md >= 0 && (t < 0 || t >= L)) {
    raise_error(v.error, HS_DEV_INDEX_RANGE, (uint32_t)r, (uint32_t)t);
    md = -1;
  }
  int ms = -1, mo = -1;
  if (mine) {
    if (md >= 0) {
      ms = __hip_atomic_load(&sc.mslot[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      mo = __hip_atomic_load(&sc.mold[jj], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  int dsts[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) dsts[k] = __shfl(md, k, 64);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int dst = dsts[k];
    if (dst < 0) continue;
    u32x4* d4 = reinterpret_cast<u32x4*>(a.pool_rows + (int64_t)dst * ROW_BYTES);
    u32x4 y[CPL];
    if ((gb >> k) & 1u) {
#pragma unroll
      for (int u = 0; u < CPL; ++u) y[u] = x[k][u];
    } else {  // a miss that was not guessed (rare): read it now
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.host_rows + (hbase + tk[k]) * HSTRIDE);
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        if (lane + 64 * u < HCH) y[u] = s4[lane + 64 * u];
    }
#pragma unroll
    for (int u = 0; u < CPL; ++u)
      if (lane + 64 * u < CH) __builtin_nontemporal_store(y[u], d4 + lane + 64 * u);  // (streaming)
    if constexpr (FP8) {  // the row's scale: first word of host chunk CH
      const uint32_t sbits = (uint32_t)__shfl((int)y[CH / 64][0], CH % 64, 64);
      if (lane == k) a.pool_scales[dst] = __uint_as_float(sbits);
    }
  }
  // LRU tables of every miss: the slot's old token leaves the reverse map,
  // the missed token takes the slot (a missed token is in no slot, so it is
  // never another miss's old token: these stores do not collide)
  // (other copy workgroups' guesses may read these entries meanwhile; a
  // guess only decides which reads start early)
  if (lane < 4 && ms >= 0) {
    if (mo >= 0 && mo < v.max_context) v.rev[(size_t)r * v.max_context + mo] = -1;
    v.slot_tag[(size_t)r * v.hot_rows + ms] = t;
    v.rev[(size_t)r * v.max_context + t] = ms;
  }
}

template <int ROW_BYTES, bool FP8, bool FUSED>
__global__ __launch_bounds__(kRsThreads) void k_resolve(RsArgs a, StateView v, RsScratch sc) {
  __shared__ RsStatic st;
  extern __shared__ __align__(16) unsigned char rs_dyn[];
  const int tid = threadIdx.x;
  const int i = (int)(blockIdx.x % (unsigned)a.n_req);  // batch position served
  uint32_t* ctl = sc.ctl + 4 * (size_t)i;
  if (tid == 0) {
    const uint32_t seq = __hip_atomic_load(&ctl[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the ticket is taken only after the sequence load has returned, so the
    // sequence cannot advance before this workgroup has read it
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    st.epoch = seq + 1u;
    st.role = (int)atomicAdd(&ctl[0], 1u);
  }
  __syncthreads();
  const int role = st.role;
  if (role == 0) {
    if constexpr (FUSED) {
      const int K = v.top_k;
      int32_t* sel_lds = reinterpret_cast<int32_t*>(rs_dyn + a.sel_off);
      select_row<true>(a.scores, a.score_stride, a.req_ids, v, a.tk, K, const_cast<int32_t*>(a.idx), i, rs_dyn,
                       sel_lds);
      // publish the selection once every thread's idx stores have completed
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0);
      asm volatile("" ::: "memory");
      __syncthreads();  // (also: the select's LDS is free for the bookkeeping)
      if (tid == 0) __hip_atomic_store(&ctl[3], st.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      bookkeep(a, v, sc, st, rs_dyn, i, sel_lds);
    } else {
      bookkeep(a, v, sc, st, rs_dyn, i, a.idx + (size_t)i * v.top_k);
    }
  } else {
    copy_part<ROW_BYTES, FP8, FUSED>(a, v, sc, i, role - 1, st.epoch);
  }
  // The last workgroup of this position to finish (every other one has
  // taken its ticket and read the sequence by then) prepares the next launch.
  __syncthreads();
  if (tid == 0) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    asm volatile("" ::: "memory");
    if (atomicAdd(&ctl[2], 1u) == (uint32_t)sc.parts) {
      const uint32_t next = st.epoch == kRsSeqWrap ? 0u : st.epoch;  // sequence + 1, wrapped
      __hip_atomic_store(&ctl[1], next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctl[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&ctl[2], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Polls before a copy wave gives up: kSpinLimit, or HS_RESOLVE_SPIN_LIMIT
// when set (read at each call; a test hook that makes the wait give up).
static int spin_limit() {
  const char* s = getenv("HS_RESOLVE_SPIN_LIMIT");
  if (!s) return kSpinLimit;
  const int v = atoi(s);
  return v >= 0 ? v : kSpinLimit;
}

static int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <bool FUSED>
static hs_status launch_resolve_impl(hs_pool* p, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                                     int32_t* plan_out, int32_t* counts_out, const float* scores,
                                     int64_t score_stride, hipStream_t s) {
  StateView v = make_view(p);
  RsScratch sc;
  sc.mdst = reinterpret_cast<uint64_t*>(p->state + p->off.rs_mdst);
  sc.mslot = reinterpret_cast<int32_t*>(p->state + p->off.rs_mslot);
  sc.mold = reinterpret_cast<int32_t*>(p->state + p->off.rs_mold);
  sc.ctl = reinterpret_cast<uint32_t*>(p->state + p->off.rs_ticket);
  sc.parts = (p->d.top_k + kRsPart - 1) / kRsPart;
  RsArgs a{idx, req_ids, n_req,
           pow2_at_least((p->d.top_k + kRsThreads - 1) / kRsThreads),
           max(4, pow2_at_least((v.hot_rows + kRsThreads - 1) / kRsThreads)),
           v.pages_per_req <= kRsPtLds ? v.pages_per_req : 0, spin_limit(),
           plan_out, counts_out, static_cast<const uint8_t*>(p->host_rows),
           p->pool_rows, p->pool_scales, scores, score_stride, make_tk_scratch(p, 1), 0};
  size_t dyn = (rs_dyn_bytes(a.Q * kRsThreads, p->d.top_k, v.hot_pages_per_req, a.pt_lds) + 15) & ~(size_t)15;
  if (FUSED) {  // the select's LDS (the bookkeeping reuses it), then the selection
    if (dyn < kTkSelLdsBytes) dyn = kTkSelLdsBytes;
    a.sel_off = (int)dyn;
    dyn += 4 * (size_t)p->d.top_k;
    if (dyn > kRsFusedMaxDyn) return HS_ERR_UNSUPPORTED;  // (page size too small for one workgroup's LDS)
  }
  const int grid = n_req * (1 + sc.parts);
  switch (p->d.kv_dtype) {
    case HS_F32:
      k_resolve<2304, false, FUSED><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
    case HS_BF16:
      k_resolve<1152, false, FUSED><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
    default:
      k_resolve<576, true, FUSED><<<grid, kRsThreads, dyn, s>>>(a, v, sc);
      break;
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

hs_status launch_resolve(hs_pool* p, const int32_t* idx, const int32_t* req_ids, int32_t n_req,
                         int32_t* plan_out, int32_t* counts_out, hipStream_t s) {
  return launch_resolve_impl<false>(p, idx, req_ids, n_req, plan_out, counts_out, nullptr, 0, s);
}

hs_status launch_select_resolve(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                                int32_t n_req, int32_t* idx_out, int32_t* plan_out, int32_t* counts_out,
                                hipStream_t s) {
  hs_status st = launch_topk_filter(p, scores, stride, req_ids, n_req, p->d.top_k, s);
  if (st != HS_OK) return st;
  return launch_resolve_impl<true>(p, idx_out, req_ids, n_req, plan_out, counts_out, scores, stride, s);
}

}  // namespace hs
