// Top-K select of one score row by one workgroup, shared by the top-K
// kernels and the select-and-resolve kernel (see topk.hip for the method).
#pragma once

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

// LDS of one select: three 4,096-bin histograms, two chunk-offset tables
// and the staged survivors (16-byte aligned regions).
constexpr int kTkOffEntries = kTkMaxChunks + 4;  // kTkMaxChunks + 1, rounded up to 16 bytes
constexpr size_t kTkSelHistBytes = 3 * (size_t)kTkBins * 4;
constexpr size_t kTkSelLdsBytes = kTkSelHistBytes + 8 * (size_t)kTkOffEntries + 8 * (size_t)kTkStage;

// Views of the top-K scratch of a pool for a call with qsel score rows per
// request (host side).
inline TkScratch make_tk_scratch(const hs_pool* p, int qsel) {
  TkScratch sc;
  sc.count = reinterpret_cast<int32_t*>(p->state + p->off.tk_count);
  sc.maxk = reinterpret_cast<uint32_t*>(p->state + p->off.tk_max);
  sc.cand = reinterpret_cast<uint2*>(p->state + p->off.tk_cand);
  sc.bound = reinterpret_cast<uint32_t*>(p->state + p->off.tk_bound);
  sc.max_chunks = (p->d.max_context + kTkChunk - 1) / kTkChunk;
  sc.qsel = qsel;
  sc.bound_q = p->off.sel_q;
  return sc;
}

// COHERENT: the store is device-coherent (agent scope), for a selection
// that workgroups of the same launch read (plain stores reach only this
// XCD's L2 until the kernel ends).
template <bool COHERENT>
__device__ inline void out_store(int32_t* idx_out, int i, int K, int j, int32_t tok) {
  int32_t* p = idx_out + (size_t)i * K + j;
  if constexpr (COHERENT)
    __hip_atomic_store(p, tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = tok;
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

// Select of score row i (one 1,024-thread workgroup). `lds` is
// kTkSelLdsBytes of LDS, 16-byte aligned; sel_lds, when given, receives
// the selected tokens as idx_out does (K entries). COHERENT: idx_out is
// written with device-coherent stores (read by other workgroups of the
// same launch).
template <bool COHERENT>
__device__ __forceinline__ void select_row(const float* __restrict__ scores, int64_t stride,
                                           const int32_t* __restrict__ req_ids, const StateView& v,
                                           const TkScratch& sc, int K, int32_t* __restrict__ idx_out, int i,
                                           unsigned char* lds, int32_t* sel_lds) {
  constexpr int NW = kTkSelWaves;
  uint32_t(*hist)[kTkBins] = reinterpret_cast<uint32_t(*)[kTkBins]>(lds);
  int* off = reinterpret_cast<int*>(lds + kTkSelHistBytes);
  int* off2 = off + kTkOffEntries;
  uint2* surv = reinterpret_cast<uint2*>(lds + kTkSelHistBytes + 8 * kTkOffEntries);
  __shared__ int wtot[NW];
  __shared__ int weq[NW];
  __shared__ uint32_t wmax[NW];
  __shared__ FindOut fres;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto put = [&](int j, int32_t tok) {
    out_store<COHERENT>(idx_out, i, K, j, tok);
    if (sel_lds) sel_lds[j] = tok;
  };
  const int qi = i / sc.qsel, qt = i - qi * sc.qsel;  // request position, query token
  const int r = request_of(req_ids, qi, v);
  if (r < 0) {
    if (tid == 0) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)qi, (uint32_t)req_ids[qi]);
    for (int j = tid; j < K; j += kTkSelThreads) put(j, -1);
    return;
  }
  const int L = v.ctx_len[r];
  if (L <= K) {  // every token is selected
    for (int j = tid; j < K; j += kTkSelThreads) put(j, j < L ? j : -1);
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
    // The chunk of every survivor from a table that one lane per chunk
    // fills (in the third histogram, unused until the lower digits and
    // cleared again below: n <= kTkStage entries of 16 bits), instead of a
    // binary search over the chunk offsets per survivor.
    static_assert(kTkStage * 2 <= kTkBins * 4 && kTkMaxChunks <= 65536, "chunk table fits a histogram");
    uint16_t* owner = reinterpret_cast<uint16_t*>(hist[2]);
    for (int c = tid; c < nch; c += kTkSelThreads)
      for (int x = off[c]; x < off[c + 1]; ++x) owner[x] = (uint16_t)c;
    __syncthreads();
    constexpr int U = 4;
    for (int x0 = tid; x0 < n; x0 += U * kTkSelThreads) {
      uint2 e[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int x = x0 + u * kTkSelThreads;
        if (x < n) {
          const int c = owner[x];
          e[u] = cand[(size_t)c * kTkChunk + (x - off[c])];
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
    __syncthreads();  // every owner entry has been read
    for (int b = tid; b < kTkBins; b += kTkSelThreads) hist[2][b] = 0u;
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
    if (sel && at < K) put(at, (int32_t)e.y);
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

}  // namespace hs
