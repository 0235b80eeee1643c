// Deterministic indexer top-K ([P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文
// 显存瓶颈" §"稀疏MLA的核心思想": decode attends only to the top-K tokens the
// indexer picks). Per request: the min(K, L) largest scores, equal scores
// keeping the lower token index, output in ascending token order.
//
// Scores map to order-preserving 32-bit keys (-0.0 folded onto +0.0). A
// token is selected when key > T, or key == T and it is among the first
// (K - #{key > T}) tokens with key T in token order, where T is the exact
// K-th largest key.
//
// Two kernels per call (each score row is one request's, or, for a
// speculative step, one query token's of a request, with a bound of its own):
//   k_topk_filter  workgroup (c, i) reads scores [2048c, 2048c + 2048) of
//                  score row i, keeps every key >= the row's bound, in
//                  token order, in its slice of a candidate buffer (ballot
//                  ranks, no LDS tables, no atomics) and writes the slice's
//                  count and largest key. Many small workgroups per CU.
//   k_topk_select  one 1024-thread workgroup per request: stages the
//                  survivors in LDS in token order, finds T by a radix
//                  select over (key - bound) whose digit widths follow the
//                  survivors' key range (usually two 12-bit digits), writes
//                  the selected tokens in order and sets the next bound.
// The bound carried from call to call only decides how much work is done;
// the result is exact in every case. The next bound is the lower edge of the
// first-digit bin holding the survivor of rank 5K/4, so that about 1.25K
// scores pass next time when scores move little between steps; with fewer
// than 5K/4 survivors it is lowered instead. If fewer than K scores pass (a
// bound too high) the select runs over the raw scores; if more pass than
// LDS holds (e.g. the first call, bound 0) it reads them from the candidate
// buffer. Grids are fixed and no scratch needs clearing, so the pair
// replays under a hipGraph without host input.
#include <hip/hip_runtime.h>

#include "topk_select.h"

namespace hs {

__global__ __launch_bounds__(kTkThreads) void k_topk_filter(const float* __restrict__ scores, int64_t stride,
                                                            const int32_t* __restrict__ req_ids, StateView v,
                                                            TkScratch sc, int K) {
  constexpr int NW = kTkThreads / 64;
  constexpr int PER_WAVE = kTkChunk / NW;  // 512 scores per wave
  constexpr int NU = PER_WAVE / 256;       // float4 loads per lane
  __shared__ int wcount[NW];
  __shared__ uint32_t wmax[NW];
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = i / sc.qsel, qt = i - qi * sc.qsel;  // request position, query token
  const int r = request_of(req_ids, qi, v);
  if (r < 0) return;
  const int L = v.ctx_len[r];
  if (L <= K) return;
  const int nch = (L + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  const float* s = scores + (size_t)i * stride;
  const uint32_t thr = sc.bound[(size_t)r * sc.bound_q + qt];
  const int beg = c * kTkChunk + wave * PER_WAVE, end = min(L, beg + PER_WAVE);
  float4 x[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = beg + 256 * u + 4 * lane;
    if (t + 4 <= end) {
      x[u] = *reinterpret_cast<const float4*>(s + t);
    } else {
      x[u].x = t < end ? s[t] : 0.f;
      x[u].y = t + 1 < end ? s[t + 1] : 0.f;
      x[u].z = t + 2 < end ? s[t + 2] : 0.f;
      x[u].w = 0.f;
    }
  }
  uint32_t k[NU][4];
  unsigned long long b[NU][4];
  int run = 0;
  uint32_t mx = 0u;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = beg + 256 * u + 4 * lane;
    k[u][0] = score_key(x[u].x);
    k[u][1] = score_key(x[u].y);
    k[u][2] = score_key(x[u].z);
    k[u][3] = score_key(x[u].w);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool f = t + e < end && k[u][e] >= thr;
      b[u][e] = __ballot(f);
      run += __popcll(b[u][e]);
      mx = f ? max(mx, k[u][e]) : mx;
    }
  }
  mx = wave_max_u32(mx);
  if (lane == 0) {
    wcount[wave] = run;
    wmax[wave] = mx;
  }
  __syncthreads();
  int before = 0, total = 0;
  uint32_t cmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    before += w < wave ? wcount[w] : 0;
    total += wcount[w];
    cmax = max(cmax, wmax[w]);
  }
  // token order inside the wave: t = beg + 256u + 4 lane + e, so the rank of
  // element (u, e) of this lane counts all of u' < u, then lanes below this
  // one over every e, then e' < e of this lane
  uint2* dst = sc.cand + ((size_t)i * sc.max_chunks + c) * kTkChunk + before;
  const unsigned long long below = (1ull << lane) - 1ull;
  int pos = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int t = beg + 256 * u + 4 * lane;
    int p = pos + __popcll(b[u][0] & below) + __popcll(b[u][1] & below) + __popcll(b[u][2] & below) +
            __popcll(b[u][3] & below);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((b[u][e] >> lane) & 1ull) dst[p++] = make_uint2(k[u][e], (uint32_t)(t + e));
    pos += __popcll(b[u][0]) + __popcll(b[u][1]) + __popcll(b[u][2]) + __popcll(b[u][3]);
  }
  if (tid == 0) {
    sc.count[(size_t)i * sc.max_chunks + c] = total;
    sc.maxk[(size_t)i * sc.max_chunks + c] = cmax;
  }
}

__global__ __launch_bounds__(kTkSelThreads) void k_topk_select(const float* __restrict__ scores, int64_t stride,
                                                               const int32_t* __restrict__ req_ids, StateView v,
                                                               TkScratch sc, int K, int32_t* __restrict__ idx_out) {
  extern __shared__ __align__(16) unsigned char tk_dyn[];
  select_row<false>(scores, stride, req_ids, v, sc, K, idx_out, blockIdx.x, tk_dyn, nullptr);
}

hs_status launch_topk_filter(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                             int32_t n_req, int32_t k, hipStream_t s) {
  StateView v = make_view(p);
  TkScratch sc = make_tk_scratch(p, 1);
  k_topk_filter<<<dim3(sc.max_chunks, n_req), kTkThreads, 0, s>>>(scores, stride, req_ids, v, sc, k);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

hs_status launch_topk(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                      int32_t n_req, int32_t qsel, int32_t k, int32_t* idx_out, hipStream_t s) {
  StateView v = make_view(p);
  TkScratch sc = make_tk_scratch(p, qsel);
  const int rows = n_req * qsel;
  k_topk_filter<<<dim3(sc.max_chunks, rows), kTkThreads, 0, s>>>(scores, stride, req_ids, v, sc, k);
  k_topk_select<<<rows, kTkSelThreads, kTkSelLdsBytes, s>>>(scores, stride, req_ids, v, sc, k, idx_out);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

// Union of the selections of a request's query tokens (one workgroup per
// request). Each selection is ascending with its valid entries first. An
// entry is the owner of its token when no earlier list holds the token, so
// every distinct token has one owner; the union position of a token x is the
// number of distinct tokens below x, the sum over the lists of their owners
// below x: an exclusive count of owners in list order, read at each list's
// lower bound of x. Owners write the union; every entry writes its position.
constexpr int kUnThreads = 1024;
constexpr int kUnRounds = kMaxTopK / kUnThreads;

__global__ __launch_bounds__(kUnThreads) void k_topk_union(const int32_t* __restrict__ idx, int qsel, int K, int cap,
                                                           int32_t* __restrict__ union_out,
                                                           int32_t* __restrict__ upos_out) {
  __shared__ int lst[kMaxTopK];
  __shared__ int opre[kMaxTopK + 1];
  __shared__ int mcount[kMaxSelectQ];
  __shared__ int wtot[kUnThreads / 64 + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int n = qsel * K;  // <= cap <= kMaxTopK
  const int32_t* src = idx + (size_t)i * n;
  for (int x = tid; x < n; x += kUnThreads) lst[x] = src[x];
  if (tid < kMaxSelectQ) mcount[tid] = 0;
  __syncthreads();
  for (int x = tid; x < n; x += kUnThreads)
    if (lst[x] >= 0) atomicAdd(&mcount[x / K], 1);
  __syncthreads();
  int lbs[kUnRounds][kMaxSelectQ];  // lower bound of each entry's token in every list
  bool own[kUnRounds];
  int base = 0;
#pragma unroll
  for (int e = 0; e < kUnRounds; ++e) {
    own[e] = false;
    const int x = e * kUnThreads + tid;
    if (e * kUnThreads < n) {  // uniform
      if (x < n) {
        const int t = x / K, j = x - t * K;
        const int tok = lst[x];
        if (j < mcount[t]) {
          own[e] = true;
#pragma unroll
          for (int q = 0; q < kMaxSelectQ; ++q) {
            if (q < qsel) {
              int lo = 0, hi = mcount[q];
              if (q == t) {
                lo = j;
              } else {
                while (lo < hi) {
                  const int mid = (lo + hi) >> 1;
                  if (lst[q * K + mid] < tok) lo = mid + 1; else hi = mid;
                }
                if (q < t && lo < mcount[q] && lst[q * K + lo] == tok) own[e] = false;
              }
              lbs[e][q] = lo;
            }
          }
        }
      }
      int tot;
      const int pre = block_excl_count(own[e], wtot, tot);
      if (x < n) opre[x] = base + pre;
      base += tot;
    }
  }
  if (tid == 0) opre[n] = base;
  __syncthreads();
  int32_t* uo = union_out + (size_t)i * cap;
#pragma unroll
  for (int e = 0; e < kUnRounds; ++e) {
    const int x = e * kUnThreads + tid;
    if (x < n) {
      const int t = x / K, j = x - t * K;
      int pos = -1;
      if (j < mcount[t]) {
        pos = 0;
#pragma unroll
        for (int q = 0; q < kMaxSelectQ; ++q)
          if (q < qsel) pos += opre[q * K + lbs[e][q]] - opre[q * K];
        if (own[e]) uo[pos] = lst[x];
      }
      upos_out[(size_t)i * n + x] = pos;
    }
  }
  for (int x = base + tid; x < cap; x += kUnThreads) uo[x] = -1;
}

// The same union through a bitmap of the token space (pools whose
// max_context fits it in LDS): every valid entry sets its token's bit; the
// union position of token x is the number of set bits below x, from an
// exclusive prefix of the words' popcounts (16 bits each: a union holds at
// most kMaxTopK tokens); each thread emits the set bits of its own run of
// words at their positions, so the union comes out ascending. No search,
// three barriers.
constexpr size_t kUnBitmapMaxLds = (size_t)150 << 10;
__host__ __device__ inline size_t union_bitmap_lds(int words) { return 4 * (size_t)words + 2 * (size_t)((words + 1) & ~1); }

__global__ __launch_bounds__(kUnThreads) void k_topk_union_bitmap(const int32_t* __restrict__ idx, int qsel, int K,
                                                                  int cap, int words, int32_t* __restrict__ union_out,
                                                                  int32_t* __restrict__ upos_out) {
  extern __shared__ __align__(16) uint32_t un_dyn[];
  uint32_t* bm = un_dyn;                                  // [words]
  uint16_t* wpre = reinterpret_cast<uint16_t*>(bm + words);  // [words] set bits in the words before
  __shared__ int wtot[kUnThreads / 64 + 1];
  const int i = blockIdx.x, tid = threadIdx.x;
  const int n = qsel * K;  // <= cap <= kMaxTopK
  const int32_t* src = idx + (size_t)i * n;
  for (int w = tid; w < words; w += kUnThreads) bm[w] = 0u;
  int tok[kUnRounds];
#pragma unroll
  for (int e = 0; e < kUnRounds; ++e) {
    const int x = e * kUnThreads + tid;
    const int t = x < n ? src[x] : -1;
    tok[e] = (t >= 0 && t < 32 * words) ? t : -1;  // (padding is -1; every selected token is below max_context)
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kUnRounds; ++e)
    if (tok[e] >= 0) atomicOr(&bm[tok[e] >> 5], 1u << (tok[e] & 31));
  __syncthreads();
  // this thread's run of words [w0, w1)
  const int per = (words + kUnThreads - 1) / kUnThreads;
  const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
  int cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
  int total;
  int run = block_excl_sum(cnt, wtot, total);
  for (int w = w0; w < w1; ++w) {
    wpre[w] = (uint16_t)run;
    run += __popc(bm[w]);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < kUnRounds; ++e) {
    const int x = e * kUnThreads + tid;
    if (x < n) {
      const int t = tok[e];
      upos_out[(size_t)i * n + x] = t >= 0 ? (int)wpre[t >> 5] + __popc(bm[t >> 5] & ((1u << (t & 31)) - 1u)) : -1;
    }
  }
  int32_t* uo = union_out + (size_t)i * cap;
  for (int w = w0; w < w1; ++w) {
    uint32_t b = bm[w];
    int p = wpre[w];
    while (b) {
      uo[p++] = 32 * w + __builtin_ctz(b);
      b &= b - 1u;
    }
  }
  for (int x = total + tid; x < cap; x += kUnThreads) uo[x] = -1;
}

hs_status launch_topk_union(hs_pool* p, const int32_t* idx, int32_t n_req, int32_t qsel, int32_t k,
                            int32_t* union_out, int32_t* upos_out, hipStream_t s) {
  const int words = (p->d.max_context + 31) / 32;
  const size_t lds = union_bitmap_lds(words);
  if (lds <= kUnBitmapMaxLds)
    k_topk_union_bitmap<<<n_req, kUnThreads, lds, s>>>(idx, qsel, k, p->d.top_k, words, union_out, upos_out);
  else  // (contexts beyond ~800K tokens: the search form)
    k_topk_union<<<n_req, kUnThreads, 0, s>>>(idx, qsel, k, p->d.top_k, union_out, upos_out);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
