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

#include "hs_internal.h"

namespace hs {

constexpr int kTkSelThreads = 1024;
constexpr int kTkSelWaves = kTkSelThreads / 64;

struct TkScratch {
  int32_t* count;   // [score rows][max_chunks] survivors per chunk
  uint32_t* maxk;   // [score rows][max_chunks] largest surviving key per chunk
  uint2* cand;      // [score rows][max_chunks * kTkChunk] (key, token), chunk slices
  uint32_t* bound;  // [max_requests][bound_q] survivor bound for the next call
  int32_t max_chunks;
  int32_t qsel;     // score rows per request in this call (row i * qsel + t)
  int32_t bound_q;  // bounds per request (the pool's select_q, at least 1)
};

__device__ inline uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  u = (u == 0x80000000u) ? 0u : u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int request_of(const int32_t* req_ids, int i, const StateView& v) {
  const int r = req_ids[i];
  return (r >= 0 && r < v.max_requests) ? r : -1;
}

__device__ inline uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, o, 64));
  return x;
}

__device__ inline int wave_incl_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

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

// Block-wide search of a 4096-bin histogram from the top bin down: for each
// of two needs (1 <= need <= total), the bin b with above(b) < need <=
// above(b) + h[b], and above(b). Every thread gets the results.
struct FindOut {
  int b[2];
  int above[2];
};
__device__ void hist_find2(const uint32_t* h, int need0, int need1, int* wtot, FindOut* res, FindOut& out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi = kTkBins - 1 - 4 * tid;  // this thread's bins hi, hi-1, hi-2, hi-3
  const uint4 q = *reinterpret_cast<const uint4*>(h + hi - 3);
  const int c4 = (int)(q.x + q.y + q.z + q.w);
  const int incl_w = wave_incl_sum(c4);
  if (lane == 63) wtot[wave] = incl_w;
  __syncthreads();
  int pre = 0;
#pragma unroll
  for (int w = 0; w < kTkSelWaves; ++w) pre += w < wave ? wtot[w] : 0;
  const int incl = pre + incl_w, excl = incl - c4;
  const int need[2] = {need0, need1};
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    if (excl < need[z] && need[z] <= incl) {
      const int cnt[4] = {(int)q.w, (int)q.z, (int)q.y, (int)q.x};  // bins hi .. hi-3
      int above = excl, bb = hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (bb == hi - e && above + cnt[e] < need[z]) {
          above += cnt[e];
          bb = hi - e - 1;
        }
      }
      res->b[z] = bb;
      res->above[z] = above;
    }
  }
  __syncthreads();
  out = *res;
}

__global__ __launch_bounds__(kTkSelThreads) void k_topk_select(const float* __restrict__ scores, int64_t stride,
                                                               const int32_t* __restrict__ req_ids, StateView v,
                                                               TkScratch sc, int K, int32_t* __restrict__ idx_out) {
  constexpr int NW = kTkSelWaves;
  __shared__ __align__(16) uint32_t hist[3][kTkBins];
  __shared__ int off[kTkMaxChunks + 1];
  __shared__ int off2[kTkMaxChunks + 1];
  __shared__ uint2 surv[kTkStage];
  __shared__ int wtot[NW];
  __shared__ int weq[NW];
  __shared__ uint32_t wmax[NW];
  __shared__ FindOut fres;
  const int i = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = i / sc.qsel, qt = i - qi * sc.qsel;  // request position, query token
  int32_t* out = idx_out + (size_t)i * K;
  const int r = request_of(req_ids, qi, v);
  if (r < 0) {
    if (tid == 0) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)qi, (uint32_t)req_ids[qi]);
    for (int j = tid; j < K; j += kTkSelThreads) out[j] = -1;
    return;
  }
  const int L = v.ctx_len[r];
  if (L <= K) {  // every token is selected
    for (int j = tid; j < K; j += kTkSelThreads) out[j] = j < L ? j : -1;
    return;
  }
  const int nch = (L + kTkChunk - 1) / kTkChunk;
  const float* s = scores + (size_t)i * stride;
  const uint2* cand = sc.cand + (size_t)i * sc.max_chunks * kTkChunk;
  const int32_t* cnt = sc.count + (size_t)i * sc.max_chunks;
  const uint32_t* cmx = sc.maxk + (size_t)i * sc.max_chunks;
  uint32_t* bound = sc.bound + (size_t)r * sc.bound_q + qt;
  const uint32_t thr = *bound;

  // Speculative preload (contexts of up to NW * kPreSlots chunks): the
  // first 64 * kPreU survivors of each of this wave's chunks (chunks wave,
  // wave + NW, ...), issued with the chunk counts so that both arrive in one
  // round trip; entries past a chunk's count are never used.
  constexpr int kPreSlots = 4, kPreU = 2;
  const bool preload = nch <= NW * kPreSlots;
  uint2 pv[kPreSlots][kPreU];
  if (preload) {
#pragma unroll
    for (int q = 0; q < kPreSlots; ++q) {
      const int c = min(wave + NW * q, nch - 1);
#pragma unroll
      for (int u = 0; u < kPreU; ++u) pv[q][u] = cand[(size_t)c * kTkChunk + lane + 64 * u];
    }
  }

  // 1. chunk offsets of the survivors, their count and largest key
  for (int b = tid; b < 3 * kTkBins; b += kTkSelThreads) (&hist[0][0])[b] = 0u;
  int run = 0;
  uint32_t mx = 0u;
  for (int base = 0; base < nch; base += kTkSelThreads) {
    const int cc = base + tid;
    const int x = cc < nch ? cnt[cc] : 0;
    mx = max(mx, cc < nch ? cmx[cc] : 0u);
    int tot;
    const int e = block_excl_sum(x, wtot, tot);
    if (cc < nch) off[cc] = run + e;
    run += tot;
  }
  mx = wave_max_u32(mx);
  if (lane == 0) wmax[wave] = mx;
  if (tid == 0) off[nch] = run;
  __syncthreads();
  uint32_t kmax = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) kmax = max(kmax, wmax[w]);
  const int total = run;
  const bool raw = total < K;  // fewer than K passed: select over the raw scores
  bool staged = !raw && total <= kTkStage;
  bool narrowed = false;
  int n = raw ? L : total;
  uint32_t base = raw ? 0u : thr;

  // Too many survivors for LDS (e.g. the first call, bound 0): find a cut
  // key, the lower edge of a digit bin of (key - bound), with K <= #{key >=
  // cut} <= kTkStage by histogram passes that read the chunk slices in
  // order (coalesced, UN loads in flight per lane), then stage the survivors
  // >= cut in token order. nb0 is the lower edge of the first pass's bin
  // holding rank 5K/4, the next call's bound when fewer than 5K/4 are staged.
  uint32_t nb0 = thr;
  if (!raw && !staged) {
    constexpr int UN = 8;
    // f(u, key, valid) for every slot of this wave's chunks, all lanes together
    auto sweep = [&](auto&& f, auto&& chunk_begin, auto&& chunk_end) {
      for (int c = wave; c < nch; c += NW) {
        const int m = off[c + 1] - off[c];
        const uint2* src = cand + (size_t)c * kTkChunk;
        chunk_begin(c);
        for (int j0 = 0; j0 < m; j0 += 64 * UN) {
          uint2 e[UN];
#pragma unroll
          for (int u = 0; u < UN; ++u) {
            const int j = j0 + 64 * u + lane;
            e[u] = j < m ? src[j] : make_uint2(0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < UN; ++u) f(e[u], j0 + 64 * u + lane < m);
        }
        chunk_end(c);
      }
    };
    auto none = [](int) {};
    const uint32_t range0 = kmax - thr;
    const int B0 = range0 == 0u ? 0 : 32 - __clz(range0);
    int shc = B0 > 12 ? B0 - 12 : 0;  // shift of the digit found last
    uint32_t pre = 0u;                // digits found so far
    int above = 0, cnt_ge = n;
    for (int pass = 0; pass < 3; ++pass) {
      const int w = pass == 0 ? 0 : min(12, shc);
      const int sn = shc - w;
      if (pass > 0 && (cnt_ge <= kTkStage || shc == 0)) break;  // uniform
      uint32_t* h = hist[pass];
      const uint32_t dmask = (1u << w) - 1u;
      sweep([&](uint2 e, bool ok) {
        const uint32_t rel = e.x - thr;
        if (ok && pass == 0) atomicAdd(&h[rel >> shc], 1u);
        if (ok && pass > 0 && (rel >> shc) == pre) atomicAdd(&h[(rel >> sn) & dmask], 1u);
      }, none, none);
      __syncthreads();
      FindOut g;
      hist_find2(h, K - above, pass == 0 ? min(n, K + K / 4) : K - above, wtot, &fres, g);
      if (pass == 0) nb0 = thr + ((uint32_t)g.b[1] << shc);
      cnt_ge = above + g.above[0] + (int)h[g.b[0]];
      pre = pass == 0 ? (uint32_t)g.b[0] : ((pre << w) | (uint32_t)g.b[0]);
      above += g.above[0];
      if (pass > 0) shc = sn;
      __syncthreads();  // h is read above by every thread
    }
    if (cnt_ge <= kTkStage) {
      const uint32_t cut = thr + (pre << shc);
      // survivors >= cut per chunk, then their offsets
      int k = 0;
      sweep([&](uint2 e, bool ok) { k += __popcll(__ballot(ok && e.x >= cut)); }, [&](int) { k = 0; },
            [&](int c) {
              if (lane == 0) off2[c] = k;
            });
      __syncthreads();
      int run2 = 0;
      for (int b0 = 0; b0 < nch; b0 += kTkSelThreads) {
        const int cc = b0 + tid;
        const int x = cc < nch ? off2[cc] : 0;
        int tot;
        const int e = block_excl_sum(x, wtot, tot);
        if (cc < nch) off2[cc] = run2 + e;
        run2 += tot;
      }
      __syncthreads();
      // stage in token order: ballot ranks inside each chunk slice
      const unsigned long long below = (1ull << lane) - 1ull;
      int pos = 0;
      sweep([&](uint2 e, bool ok) {
        const bool keep = ok && e.x >= cut;
        const unsigned long long bk = __ballot(keep);
        if (keep) surv[pos + __popcll(bk & below)] = e;
        pos += __popcll(bk);
      }, [&](int c) { pos = off2[c]; }, none);
      for (int b = tid; b < 3 * kTkBins; b += kTkSelThreads) (&hist[0][0])[b] = 0u;
      __syncthreads();
      n = run2;
      base = cut;
      staged = true;
      narrowed = true;
    } else {  // (only with more than kTkStage keys equal to the K-th)
      for (int b = tid; b < 3 * kTkBins; b += kTkSelThreads) (&hist[0][0])[b] = 0u;
      __syncthreads();
    }
  }
  const uint32_t range = raw ? 0xFFFFFFFFu : kmax - base;
  const int B = range == 0u ? 0 : 32 - __clz(range);  // bits of (key - base)
  const int s1 = B > 12 ? B - 12 : 0;

  // survivor x (0 <= x < n) in token order
  auto get = [&](int x) -> uint2 {
    if (staged) return surv[x];
    if (raw) return make_uint2(score_key(s[x]), (uint32_t)x);
    int lo = 0, hi = nch;  // off[lo] <= x < off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= x) lo = mid; else hi = mid;
    }
    return cand[(size_t)lo * kTkChunk + (x - off[lo])];
  };

  // 2. first digit (bits s1 .. B-1 of key - base), staging into LDS on the way
  if (staged && !narrowed && preload) {  // from the preloaded registers, chunk by chunk
#pragma unroll
    for (int q = 0; q < kPreSlots; ++q) {
      const int c = wave + NW * q;
      if (c < nch) {  // uniform per wave
        const int o = off[c], m = off[c + 1] - o;
#pragma unroll
        for (int u = 0; u < kPreU; ++u) {
          const int j = lane + 64 * u;
          if (j < m) {
            surv[o + j] = pv[q][u];
            atomicAdd(&hist[0][(pv[q][u].x - base) >> s1], 1u);
          }
        }
        for (int j = 64 * kPreU + lane; j < m; j += 64) {  // (a chunk with more survivors)
          const uint2 e = cand[(size_t)c * kTkChunk + j];
          surv[o + j] = e;
          atomicAdd(&hist[0][(e.x - base) >> s1], 1u);
        }
      }
    }
  } else if (staged && !narrowed) {
    constexpr int U = 4;
    for (int x0 = tid; x0 < n; x0 += U * kTkSelThreads) {
      uint2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = x0 + u * kTkSelThreads;
        if (x < n) {
          int lo = 0, hi = nch;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= x) lo = mid; else hi = mid;
          }
          e[u] = cand[(size_t)lo * kTkChunk + (x - off[lo])];
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = x0 + u * kTkSelThreads;
        if (x < n) {
          surv[x] = e[u];
          atomicAdd(&hist[0][(e[u].x - base) >> s1], 1u);
        }
      }
    }
  } else {
    for (int x = tid; x < n; x += kTkSelThreads) atomicAdd(&hist[0][(get(x).x - base) >> s1], 1u);
  }
  __syncthreads();
  FindOut f;
  hist_find2(hist[0], K, min(n, K + K / 4), wtot, &fres, f);
  uint32_t pre = (uint32_t)f.b[0];
  int need = K - f.above[0];
  const int bn = f.b[1];
  // 3. lower digits (at most two more: 12 + 12 + 8 bits)
  int sh = s1;
  for (int pass = 1; sh > 0; ++pass) {
    const int w = sh > 12 ? 12 : sh;
    const int sn = sh - w;
    const uint32_t mask = (1u << w) - 1u;
    uint32_t* h = hist[pass];
    for (int x = tid; x < n; x += kTkSelThreads) {
      const uint32_t rel = get(x).x - base;
      if ((rel >> sh) == pre) atomicAdd(&h[(rel >> sn) & mask], 1u);
    }
    __syncthreads();
    FindOut g;
    hist_find2(h, need, need, wtot, &fres, g);
    pre = (pre << w) | (uint32_t)g.b[0];
    need -= g.above[0];
    sh = sn;
  }
  const uint32_t T = base + pre;
  const int ties = need;  // keys equal to T that are taken
  // 4. ordered output: wave w walks survivors [w q, (w + 1) q) in order
  const int q = (n + NW - 1) / NW;
  const int beg = min(n, wave * q), end = min(n, beg + q);
  int gt = 0, eq = 0;
  for (int x0 = beg; x0 < end; x0 += 64) {
    const int x = x0 + lane;
    const uint32_t kv = x < end ? get(x).x : 0u;
    gt += __popcll(__ballot(x < end && kv > T));
    eq += __popcll(__ballot(x < end && kv == T));
  }
  __syncthreads();  // wtot is reused
  if (lane == 0) {
    wtot[wave] = gt;
    weq[wave] = eq;
  }
  __syncthreads();
  int gt_before = 0, eq_before = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    gt_before += w < wave ? wtot[w] : 0;
    eq_before += w < wave ? weq[w] : 0;
  }
  int pos = gt_before + min(eq_before, ties);
  int tie_run = eq_before;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int x0 = beg; x0 < end; x0 += 64) {
    const int x = x0 + lane;
    uint2 e = make_uint2(0u, 0u);
    if (x < end) e = get(x);
    const bool is_eq = x < end && e.x == T;
    const unsigned long long beq = __ballot(is_eq);
    const int tie_rank = tie_run + __popcll(beq & below);
    const bool sel = x < end && (e.x > T || (is_eq && tie_rank < ties));
    const unsigned long long bs = __ballot(sel);
    const int at = pos + __popcll(bs & below);
    if (sel && at < K) out[at] = (int32_t)e.y;
    pos += __popcll(bs);
    tie_run += __popcll(beq);
  }
  // 5. the bound for the next call
  if (tid == 0) {
    uint32_t nb;
    if (n >= K + K / 4) {
      nb = base + ((uint32_t)bn << s1);
    } else if (narrowed) {
      nb = nb0;
    } else {
      const uint32_t d = (T - base) + (1u << s1);
      nb = base > d ? base - d : 0u;
    }
    *bound = nb;
  }
}

hs_status launch_topk(hs_pool* p, const float* scores, int64_t stride, const int32_t* req_ids,
                      int32_t n_req, int32_t qsel, int32_t k, int32_t* idx_out, hipStream_t s) {
  StateView v = make_view(p);
  TkScratch sc;
  sc.count = reinterpret_cast<int32_t*>(p->state + p->off.tk_count);
  sc.maxk = reinterpret_cast<uint32_t*>(p->state + p->off.tk_max);
  sc.cand = reinterpret_cast<uint2*>(p->state + p->off.tk_cand);
  sc.bound = reinterpret_cast<uint32_t*>(p->state + p->off.tk_bound);
  sc.max_chunks = (p->d.max_context + kTkChunk - 1) / kTkChunk;
  sc.qsel = qsel;
  sc.bound_q = p->off.sel_q;
  const int rows = n_req * qsel;
  k_topk_filter<<<dim3(sc.max_chunks, rows), kTkThreads, 0, s>>>(scores, stride, req_ids, v, sc, k);
  k_topk_select<<<rows, kTkSelThreads, 0, s>>>(scores, stride, req_ids, v, sc, k, idx_out);
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

hs_status launch_topk_union(hs_pool* p, const int32_t* idx, int32_t n_req, int32_t qsel, int32_t k,
                            int32_t* union_out, int32_t* upos_out, hipStream_t s) {
  k_topk_union<<<n_req, kUnThreads, 0, s>>>(idx, qsel, k, p->d.top_k, union_out, upos_out);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
