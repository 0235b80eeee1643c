// Deterministic indexer top-K ([P3] "vLLM Hybrid HiSparse：稀疏MLA破解长上下文
// 显存瓶颈" §"稀疏MLA的核心思想": decode attends only to the top-K tokens the
// indexer picks). Per request: the min(K, L) largest scores, equal scores
// keeping the lower token index, output in ascending token order.
//
// Scores map to order-preserving 32-bit keys (-0.0 folded onto +0.0). The
// exact K-th largest key T is found by a radix select over 12 + 12 + 8 bits;
// a token is selected when key > T, or key == T and it is among the first
// (K - #{key > T}) tokens with key T in index order.
//
//   k_topk_hist    many workgroups per request: histogram of the top 12 key
//                  bits; the last workgroup to finish finds the digit b1 of
//                  the K-th largest key and clears the histogram.
//   k_topk_filter  the same workgroups: keep every key whose top digit is
//                  >= b1, compacted in index order into the chunk's slice of
//                  a candidate buffer (about K + a few thousand survive).
//   k_topk_final   one workgroup per request: the survivors are staged in LDS
//                  (when they fit); two more radix passes over them give T,
//                  then an ordered compaction writes the selected token ids.
// Every kernel has a fixed grid and leaves its scratch cleared, so the
// sequence replays under a hipGraph without host input.
#include <hip/hip_runtime.h>

#include "hs_internal.h"

namespace hs {

struct TkScratch {
  uint32_t* hist;   // [batch][kTkBins]
  uint32_t* done;   // [batch]
  int32_t* sel;     // [batch][4]: b1, #keys with top digit > b1
  int32_t* count;   // [batch][max_chunks]
  uint2* cand;      // [batch][max_chunks * kTkChunk] (key, token)
  int32_t max_chunks;
};

__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Scan the histogram h[0..nbins) from the top bin down and find the bin b
// with above(b) < need <= above(b) + h[b], where above(b) = sum of bins > b.
// Every thread gets (b, above(b)). nbins must be a multiple of blockDim.x.
__device__ inline void find_digit(const uint32_t* h, int nbins, int need, int* tmp, int* res,
                                  int& b_out, int& above_out) {
  const int per = nbins / blockDim.x;
  const int hi = nbins - per * threadIdx.x;  // this thread owns bins [hi-per, hi)
  int mine = 0;
  for (int b = hi - 1; b >= hi - per; --b) mine += (int)h[b];
  int tot;
  int above = block_excl_sum(mine, tmp, tot);
  for (int b = hi - 1; b >= hi - per; --b) {
    const int c = (int)h[b];
    if (above < need && above + c >= need) {
      res[0] = b;
      res[1] = above;
    }
    above += c;
  }
  __syncthreads();
  b_out = res[0];
  above_out = res[1];
  __syncthreads();
}

__device__ inline int request_of(const int32_t* req_ids, int i, const StateView& v) {
  const int r = req_ids[i];
  return (r >= 0 && r < v.max_requests) ? r : -1;
}

__global__ __launch_bounds__(kTkThreads) void k_topk_hist(const float* __restrict__ scores,
                                                          int64_t stride,
                                                          const int32_t* __restrict__ req_ids,
                                                          StateView v, TkScratch sc) {
  __shared__ uint32_t h[kTkBins];
  __shared__ int tmp[kTkThreads / 64 + 1];
  __shared__ int res[2];
  __shared__ int last;
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int r = request_of(req_ids, i, v);
  if (r < 0) {
    if (c == 0 && tid == 0) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)req_ids[i]);
    return;
  }
  const int L = v.ctx_len[r], K = v.top_k;
  if (L <= K) return;
  const int nch = (L + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  for (int b = tid; b < kTkBins; b += kTkThreads) h[b] = 0;
  __syncthreads();
  const float* s = scores + (size_t)i * stride;
  const int base = c * kTkChunk;
#pragma unroll
  for (int e = 0; e < kTkChunk / kTkThreads; ++e) {
    const int t = base + e * kTkThreads + tid;
    if (t < L) atomicAdd(&h[score_key(s[t]) >> 20], 1u);
  }
  __syncthreads();
  uint32_t* gh = sc.hist + (size_t)i * kTkBins;
  for (int b = tid; b < kTkBins; b += kTkThreads) {
    const uint32_t x = h[b];
    if (x) atomicAdd(&gh[b], x);
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) last = (atomicAdd(&sc.done[i], 1u) == (uint32_t)(nch - 1));
  __syncthreads();
  if (!last) return;
  // Last workgroup of this request: the acquire fence makes every other
  // workgroup's additions visible to plain loads. All 16 loads of a thread
  // are issued before any is used; the totals are cleared for next time.
  __threadfence();
  constexpr int PER = kTkBins / kTkThreads;
  uint32_t cnt[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) cnt[k] = gh[k * kTkThreads + tid];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    h[k * kTkThreads + tid] = cnt[k];
    gh[k * kTkThreads + tid] = 0;
  }
  __syncthreads();
  int b1, above;
  find_digit(h, kTkBins, K, tmp, res, b1, above);
  if (tid == 0) {
    sc.sel[4 * i + 0] = b1;
    sc.sel[4 * i + 1] = above;
    sc.done[i] = 0;
  }
}

__global__ __launch_bounds__(kTkThreads) void k_topk_filter(const float* __restrict__ scores,
                                                            int64_t stride,
                                                            const int32_t* __restrict__ req_ids,
                                                            StateView v, TkScratch sc) {
  __shared__ int tmp[kTkThreads / 64 + 1];
  const int i = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int r = request_of(req_ids, i, v);
  if (r < 0) return;
  const int L = v.ctx_len[r], K = v.top_k;
  if (L <= K) return;
  const int nch = (L + kTkChunk - 1) / kTkChunk;
  if (c >= nch) return;
  const uint32_t b1 = (uint32_t)sc.sel[4 * i];
  constexpr int EPT = kTkChunk / kTkThreads;  // consecutive scores per thread
  const int t0 = c * kTkChunk + tid * EPT;
  const float* s = scores + (size_t)i * stride;
  uint32_t key[EPT];
  int keep = 0;
  if (t0 + EPT <= L) {
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      const float4 x = *reinterpret_cast<const float4*>(s + t0 + e);
      key[e] = score_key(x.x);
      key[e + 1] = score_key(x.y);
      key[e + 2] = score_key(x.z);
      key[e + 3] = score_key(x.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) key[e] = (t0 + e < L) ? score_key(s[t0 + e]) : 0u;
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) keep += (t0 + e < L && (key[e] >> 20) >= b1) ? 1 : 0;
  int total;
  int pos = block_excl_sum(keep, tmp, total);
  uint2* out = sc.cand + ((size_t)i * sc.max_chunks + c) * kTkChunk;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (t0 + e < L && (key[e] >> 20) >= b1) out[pos++] = make_uint2(key[e], (uint32_t)(t0 + e));
  }
  if (tid == 0) sc.count[(size_t)i * sc.max_chunks + c] = total;
}

// Locate survivor v (0-based, in index order) among the chunk slices.
__device__ inline uint2 survivor(const uint2* cand, const int* off, int nch, int v) {
  int lo = 0, hi = nch;  // off[lo] <= v < off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= v) lo = mid; else hi = mid;
  }
  return cand[(size_t)lo * kTkChunk + (v - off[lo])];
}

__global__ __launch_bounds__(kTkFinalThreads) void k_topk_final(const int32_t* __restrict__ req_ids,
                                                                StateView v, TkScratch sc,
                                                                int32_t* __restrict__ idx_out) {
  __shared__ uint32_t h[kTkBins];
  __shared__ int off[kTkMaxChunks + 1];
  __shared__ uint2 surv[kTkFinalStage];
  __shared__ int tmp[kTkFinalThreads / 64 + 1];
  __shared__ int res[2];
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = v.top_k;
  int32_t* out = idx_out + (size_t)i * K;
  const int r = request_of(req_ids, i, v);
  const int L = r < 0 ? 0 : v.ctx_len[r];
  if (L <= K) {  // every token is selected
    for (int j = tid; j < K; j += kTkFinalThreads) out[j] = j < L ? j : -1;
    return;
  }
  const int nch = (L + kTkChunk - 1) / kTkChunk;
  // chunk offsets of the survivors (exclusive prefix over chunk counts)
  int run = 0;
  for (int base = 0; base < nch; base += kTkFinalThreads) {
    const int c = base + tid;
    const int x = c < nch ? sc.count[(size_t)i * sc.max_chunks + c] : 0;
    int tot;
    const int e = block_excl_sum(x, tmp, tot);
    if (c < nch) off[c] = run + e;
    run += tot;
  }
  if (tid == 0) off[nch] = run;
  __syncthreads();
  const int total = run;
  const uint2* cand = sc.cand + (size_t)i * sc.max_chunks * kTkChunk;
  // Survivors in index order: staged in LDS when they fit (one wave copies
  // one chunk slice), otherwise read from the chunk slices in place.
  const bool staged = total <= kTkFinalStage;
  if (staged) {
    for (int c = wave; c < nch; c += kTkFinalThreads / 64) {
      const int o = off[c], n = off[c + 1] - o;
      for (int j = lane; j < n; j += 64) surv[o + j] = cand[(size_t)c * kTkChunk + j];
    }
    __syncthreads();
  }
  auto get = [&](int x) -> uint2 { return staged ? surv[x] : survivor(cand, off, nch, x); };
  const uint32_t b1 = (uint32_t)sc.sel[4 * i];
  const int need1 = K - sc.sel[4 * i + 1];
  // pass 2: bits 19..8 of the keys whose top digit is b1
  for (int b = tid; b < kTkBins; b += kTkFinalThreads) h[b] = 0;
  __syncthreads();
  for (int x = tid; x < total; x += kTkFinalThreads) {
    const uint2 kv = get(x);
    if ((kv.x >> 20) == b1) atomicAdd(&h[(kv.x >> 8) & 0xFFFu], 1u);
  }
  __syncthreads();
  int b2, above2;
  find_digit(h, kTkBins, need1, tmp, res, b2, above2);
  const int need2 = need1 - above2;
  // pass 3: bits 7..0 of the keys whose top 24 bits are (b1, b2)
  const uint32_t pre24 = (b1 << 12) | (uint32_t)b2;
  for (int b = tid; b < kTkBins; b += kTkFinalThreads) h[b] = 0;
  __syncthreads();
  for (int x = tid; x < total; x += kTkFinalThreads) {
    const uint2 kv = get(x);
    if ((kv.x >> 8) == pre24) atomicAdd(&h[kv.x & 0xFFu], 1u);
  }
  __syncthreads();
  int b3, above3;
  find_digit(h, kTkBins, need2, tmp, res, b3, above3);
  const int ties = need2 - above3;  // how many keys equal to T are taken
  const uint32_t T = (pre24 << 8) | (uint32_t)b3;
  // ordered compaction of the selected survivors
  int sel_run = 0, tie_run = 0;
  for (int base = 0; base < total; base += kTkFinalThreads) {
    const int x = base + tid;
    uint2 kv = make_uint2(0u, 0u);
    if (x < total) kv = get(x);
    const bool eq = x < total && kv.x == T;
    int eq_tot;
    const int tie_rank = tie_run + block_excl_count(eq, tmp, eq_tot);
    const bool sel = x < total && (kv.x > T || (eq && tie_rank < ties));
    int sel_tot;
    const int pos = sel_run + block_excl_count(sel, tmp, sel_tot);
    if (sel) out[pos] = (int32_t)kv.y;
    sel_run += sel_tot;
    tie_run += eq_tot;
  }
}

hs_status launch_topk(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                      int32_t n_req, int32_t* idx_out, hipStream_t s) {
  StateView v = make_view(p);
  TkScratch sc;
  sc.hist = reinterpret_cast<uint32_t*>(p->state + p->off.tk_hist);
  sc.done = reinterpret_cast<uint32_t*>(p->state + p->off.tk_done);
  sc.sel = reinterpret_cast<int32_t*>(p->state + p->off.tk_sel);
  sc.count = reinterpret_cast<int32_t*>(p->state + p->off.tk_count);
  sc.cand = reinterpret_cast<uint2*>(p->state + p->off.tk_cand);
  sc.max_chunks = (p->d.max_context + kTkChunk - 1) / kTkChunk;
  const dim3 grid(sc.max_chunks, n_req);
  k_topk_hist<<<grid, kTkThreads, 0, s>>>(scores, stride, req_ids, v, sc);
  k_topk_filter<<<grid, kTkThreads, 0, s>>>(scores, stride, req_ids, v, sc);
  k_topk_final<<<n_req, kTkFinalThreads, 0, s>>>(req_ids, v, sc, idx_out);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
