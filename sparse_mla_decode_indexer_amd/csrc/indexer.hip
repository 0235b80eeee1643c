// Indexer scores upstream of top-K. The indexer picks the top-K tokens of a
// decode step from a per-token key cache of its own, the indexer KV ([P3]
// "vLLM Hybrid HiSparse：稀疏MLA破解长上下文显存瓶颈" §"稀疏MLA的核心思想";
// [P2] "vLLM GLM 5.3 优化：混合 HiSparse 卸载" §"解决 KV 缓存内存压力" and
// §"与 vLLM 栈的集成", indexer KV item). The pages give no formula; the
// reading taken is the lightning-indexer form: H heads of dimension 128, per
// request and step a query q (H x 128, bf16) and head weights w (H, fp32),
// per token t a key k_t (128, bf16);
//
//     score_t = sum_j w_j * max(0, <q_j, k_t>).
//
// k_indexer_scores: a workgroup of 4 waves takes 128 tokens per pass of one
// request (two 16-token groups per wave: fewer registers, more waves per
// SIMD; plain loads, so that L2 merges the two 64-byte halves of each key
// line that two k-steps' loads request: both measured ~6% faster than
// four groups with streaming loads). Per 16 tokens a wave computes the 16 x H dot products with
// 16x16x32 bf16 MFMAs (the keys as the A operand straight from global memory,
// 16 bytes per lane and k-step; the queries as the B operand, read once per
// workgroup into LDS and kept in registers by each wave), applies max(0, .) and the head weights in
// fp32 and sums over heads within the lane (head blocks) and across the 16
// lanes that hold one token's heads. Bound by HBM: 256 bytes of keys per
// token against 4 bytes of score.
#include <hip/hip_runtime.h>

#include "hs_internal.h"

namespace hs {

namespace {
typedef __bf16 ix_bf16x8_t __attribute__((ext_vector_type(8)));
typedef float ix_f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t ix_u32x4_t __attribute__((ext_vector_type(4)));
}  // namespace

constexpr int kIxDim = 128;
constexpr int kIxThreads = 256;                       // 4 waves
constexpr int kIxGroups = 2;                          // 16-token groups per wave and pass
constexpr int kIxPassTokens = (kIxThreads / 64) * kIxGroups * 16;  // 128 tokens per pass

__device__ inline ix_f32x4_t ix_mfma(ix_u32x4_t a, ix_u32x4_t b, ix_f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ix_bf16x8_t, a),
                                                 __builtin_bit_cast(ix_bf16x8_t, b), c, 0, 0, 0);
}

// HB = heads / 16. Grid (ceil(max_context / (256 * passes)), n_req).
template <int HB>
__global__ __launch_bounds__(kIxThreads) __attribute__((amdgpu_waves_per_eu(4))) void k_indexer_scores(const uint16_t* __restrict__ iq,
                                                              const float* __restrict__ iw,
                                                              const uint16_t* __restrict__ ik,
                                                              int64_t ik_stride, const int32_t* __restrict__ req_ids,
                                                              StateView v, int passes, float* __restrict__ scores,
                                                              int64_t score_stride) {
  const int i = blockIdx.y;
  const int rq = req_ids[i];
  if (rq < 0 || rq >= v.max_requests) {
    if (blockIdx.x == 0 && threadIdx.x == 0) raise_error(v.error, HS_DEV_REQUEST_RANGE, (uint32_t)i, (uint32_t)rq);
    return;
  }
  const int L = v.ctx_len[rq];
  const int t_wg = blockIdx.x * passes * kIxPassTokens;
  if (t_wg >= L) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kg = lane >> 4, ln = lane & 15;

  // The request's queries (16 * HB heads x 128 dims, bf16) are read once per
  // workgroup into LDS, then each wave takes its B operands from there: head
  // block hb, k-step kk: head 16hb + ln, dims 32kk + 8kg .. +8.
  constexpr int kQChunks = 16 * HB * kIxDim / 8;  // 16-byte chunks
  __shared__ ix_u32x4_t q_s[kQChunks];
  {
    const ix_u32x4_t* qr = reinterpret_cast<const ix_u32x4_t*>(iq + (size_t)i * (16 * HB) * kIxDim);
    for (int c = threadIdx.x; c < kQChunks; c += kIxThreads) q_s[c] = qr[c];
  }
  float wv[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) wv[hb] = iw[(size_t)i * 16 * HB + 16 * hb + ln];
  const uint16_t* kr = ik + (size_t)rq * ik_stride * kIxDim;
  float* out = scores + (size_t)i * score_stride;
  // A operands: lane (kg, ln) holds token t0 + 16g + ln (clamped into the
  // context: tokens past it are computed on the last token and not
  // written), dims 32kk + 8kg .. +8. The first pass's keys are requested
  // before the barrier, so that they load together with the queries.
  ix_u32x4_t ka[kIxGroups][4];
  auto load_keys = [&](int t0) {
#pragma unroll
    for (int g = 0; g < kIxGroups; ++g) {
      const int t = min(t0 + 16 * g + ln, L - 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ka[g][kk] = *reinterpret_cast<const ix_u32x4_t*>(kr + (size_t)t * kIxDim + 32 * kk + 8 * kg);
    }
  };
  load_keys(t_wg + wave * (kIxGroups * 16));
  __syncthreads();
  ix_u32x4_t qop[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qop[hb][kk] = q_s[((16 * hb + ln) * kIxDim + 32 * kk + 8 * kg) / 8];
  }

  for (int p = 0; p < passes; ++p) {
    const int t0 = t_wg + p * kIxPassTokens + wave * (kIxGroups * 16);
    if (t0 >= L) break;
    if (p > 0) load_keys(t0);
#pragma unroll
    for (int g = 0; g < kIxGroups; ++g) {
      // D[token][head]: lane (kg, ln) holds head 16hb + ln of tokens
      // t0 + 16g + 4kg + e, e = 0..3
      float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        ix_f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) d = ix_mfma(ka[g][kk], qop[hb][kk], d);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += fmaxf(d[e], 0.f) * wv[hb];
      }
      // sum over the 16 heads held by the lanes of group kg
#pragma unroll
      for (int m = 1; m < 16; m <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] += __shfl_xor(s[e], m, 64);
      }
      if (ln < 4) {
        const int t = t0 + 16 * g + 4 * kg + ln;
        const float val = ln == 0 ? s[0] : ln == 1 ? s[1] : ln == 2 ? s[2] : s[3];
        if (t < L) out[t] = val;
      }
    }
  }
}

hs_status launch_indexer_scores(hs_pool* p, const void* iq, const float* iw, const void* ik, int64_t ik_stride,
                                int32_t n_heads, const int32_t* req_ids, int32_t n_req, float* scores,
                                int64_t score_stride, hipStream_t s) {
  const int64_t maxc = p->d.max_context;
  const int64_t chunks = (maxc + kIxPassTokens - 1) / kIxPassTokens;
  // about 2 workgroups per CU or more: fewer passes per workgroup when the
  // batch is small, up to 4 when it is large (the queries are loaded once
  // per wave and pass group)
  int passes = 1;
  while (passes < 4 && (int64_t)n_req * ((chunks + 2 * passes - 1) / (2 * passes)) >= 1024) passes *= 2;
  const dim3 grid((unsigned)((chunks + passes - 1) / passes), (unsigned)n_req);
  const StateView v = make_view(p);
  const uint16_t* q16 = static_cast<const uint16_t*>(iq);
  const uint16_t* k16 = static_cast<const uint16_t*>(ik);
#define HS_IX(HB) \
  k_indexer_scores<HB><<<grid, kIxThreads, 0, s>>>(q16, iw, k16, ik_stride, req_ids, v, passes, scores, score_stride)
  switch (n_heads / 16) {
    case 1: HS_IX(1); break;
    case 2: HS_IX(2); break;
    case 3: HS_IX(3); break;
    default: HS_IX(4); break;
  }
#undef HS_IX
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
