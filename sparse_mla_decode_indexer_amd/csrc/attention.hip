// Sparse MLA decode attention over the resolved rows ([P3] "vLLM Hybrid
// HiSparse：稀疏MLA破解长上下文显存瓶颈" §"稀疏MLA的核心思想" and its MLA note:
// each token caches one latent row that serves as key (576 dims) and value
// (first 512 dims); only the top-K rows enter attention. [P2] "vLLM GLM 5.3
// 优化：混合 HiSparse 卸载" §"与 vLLM 栈的集成": speculative decoding replays one
// resolve plan for every query token of a request).
//
// For query row (request i, query token, head) -> q (576 dims):
//   out = sum_j softmax_j(sm_scale * <q, row_j>) * row_j[0:512]
//
// k_attn_mfma (bf16 or fp8 rows, bf16 queries). A workgroup of 4 waves
// takes 64 query rows of one request and a contiguous split of its plan.
// Rows are gathered 32 at a time into LDS (fp8 codes are widened to bf16 on
// the way, which is exact); all four waves read the staged tile, each for
// its own 16 query rows, so each row is fetched once per workgroup.
//   S^T (32 rows x 16 q) = K_tile (32 x 576) . Q^T     16x16x32 bf16 MFMA
//   O^T (512 x 16 q)    += V^T (512 x 32) . P^T        16x16x32 bf16 MFMA
// Q^T stays in registers for the whole split. The scores land with each lane
// holding 8 rows of one query row, which is exactly the B operand layout of
// P^T, so P never leaves registers; V^T operands come from 8x8 register
// transposes of row-major LDS reads. P is split as p = hi + lo, two bf16
// terms (two MFMAs), keeping ~16 significant bits of each probability; a
// single bf16 P would cost up to 2^-8 relative error per weight. For fp8
// rows the per-row scale multiplies the logit and p in fp32.
// Softmax is online (running max and sum in fp32, base 2). With more than
// one split, each split writes a normalised partial output and its
// log-sum-exp; k_attn_combine merges them.
//
// k_attn_f32 (fp32 rows and queries): plain fp32 arithmetic on the vector
// units, one workgroup per query row.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdlib.h>

#include "hs_internal.h"

namespace hs {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kAttThreads = 256;       // 4 waves
constexpr int kQPerWave = 16;
constexpr int kQPerWG = 64;
constexpr int kTile = 32;              // rows per staged tile
constexpr int kLdsRow = 2 * kRowDim + 16;  // bf16 row + 16 bytes of padding
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ inline bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

__device__ inline f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Two floats -> one dword of two bf16 made of their upper halves
// (truncation; exact when the values are representable in bf16).
__device__ inline uint32_t pack_hi(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// 4 OCP e4m3 codes -> 4 bf16 (exact): decode to fp32 in hardware, keep the
// upper halves.
__device__ inline void fp8x4_to_bf16(uint32_t w, uint32_t* o) {
  const auto f01 = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const auto f23 = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  o[0] = pack_hi(f01[0], f01[1]);
  o[1] = pack_hi(f23[0], f23[1]);
}

// Row of the tile held in position e (0..7) of a lane's P^T / V^T k-vector:
// the scores of rows 4*kg + 0..3 and 16 + 4*kg + 0..3 land in lane group kg.
__device__ inline int krow(int kg, int e) { return (e < 4) ? 4 * kg + e : 16 + 4 * kg + (e - 4); }

template <bool FP8>
__global__ __launch_bounds__(kAttThreads) void k_attn_mfma(
    const uint16_t* __restrict__ q, int QR, const int32_t* __restrict__ plan, int K,
    const uint8_t* __restrict__ pool, const float* __restrict__ pool_scales, int64_t pool_rows_n,
    float c2, int tiles_per_split, int n_splits, float* __restrict__ out, float* __restrict__ lse_out,
    float* __restrict__ part_o, float* __restrict__ part_lse, uint32_t* __restrict__ err) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTile * kLdsRow];
  __shared__ float kvs[kTile];
  __shared__ int prow_s[kTile];

  const int sp = blockIdx.x, hg = blockIdx.y, i = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, ln = lane & 15;
  const int qh = hg * kQPerWG + wave * kQPerWave + ln;
  const bool qvalid = qh < QR;
  const int32_t* pl = plan + (size_t)i * K;

  // Q^T operand: lane holds query row qh, dims 32*kk + 8*kg .. +8
  u32x4_t qop[kRowDim / 32];
  {
    const uint16_t* qr = q + ((size_t)i * QR + (qvalid ? qh : 0)) * kRowDim;
#pragma unroll
    for (int kk = 0; kk < kRowDim / 32; ++kk) {
      u32x4_t x = *reinterpret_cast<const u32x4_t*>(qr + 32 * kk + 8 * kg);
      qop[kk] = qvalid ? x : u32x4_t{0, 0, 0, 0};
    }
  }
  f32x4_t acc[4][8];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_tiles = (K + kTile - 1) / kTile;
  const int t_begin = sp * tiles_per_split;
  const int t_end = min(n_tiles, t_begin + tiles_per_split);
  for (int tt = t_begin; tt < t_end; ++tt) {
    if (tid < kTile) {
      const int j = tt * kTile + tid;
      int pr = j < K ? pl[j] : -1;
      if (pr >= pool_rows_n) {
        raise_error(err, HS_DEV_PLAN_RANGE, (uint32_t)i, (uint32_t)j);
        pr = -1;
      }
      prow_s[tid] = pr;
      kvs[tid] = FP8 ? (pr >= 0 ? pool_scales[pr] : 0.f) : 1.f;
    }
    __syncthreads();
    if (!FP8) {
      constexpr int CH = 2 * kRowDim / 16;  // 72 chunks of 16 B per row
      for (int c = tid; c < kTile * CH; c += kAttThreads) {
        const int r = c / CH, ch = c - r * CH;
        const int pr = prow_s[r];
        u32x4_t x = u32x4_t{0, 0, 0, 0};
        if (pr >= 0) x = *reinterpret_cast<const u32x4_t*>(pool + (size_t)pr * (2 * kRowDim) + ch * 16);
        *reinterpret_cast<u32x4_t*>(tile + r * kLdsRow + ch * 16) = x;
      }
    } else {
      constexpr int CH = kRowDim / 16;  // 36 chunks of 16 codes per row
      for (int c = tid; c < kTile * CH; c += kAttThreads) {
        const int r = c / CH, ch = c - r * CH;
        const int pr = prow_s[r];
        u32x4_t x = u32x4_t{0, 0, 0, 0};
        if (pr >= 0) x = *reinterpret_cast<const u32x4_t*>(pool + (size_t)pr * kRowDim + ch * 16);
        uint32_t w[8];
        fp8x4_to_bf16(x[0], w);
        fp8x4_to_bf16(x[1], w + 2);
        fp8x4_to_bf16(x[2], w + 4);
        fp8x4_to_bf16(x[3], w + 6);
        *reinterpret_cast<u32x4_t*>(tile + r * kLdsRow + ch * 32) = u32x4_t{w[0], w[1], w[2], w[3]};
        *reinterpret_cast<u32x4_t*>(tile + r * kLdsRow + ch * 32 + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
      }
    }
    __syncthreads();

    // S^T = K_tile . Q^T, two 16-row blocks
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < kRowDim / 32; ++kk) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(tile + (16 * rb + ln) * kLdsRow + (32 * kk + 8 * kg) * 2);
        sacc[rb] = mfma16(a, qop[kk], sacc[rb]);
      }
    }
    // base-2 logits of this lane's 8 rows, masked rows at -inf
    float s[8], rs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = krow(kg, e);
      rs[e] = kvs[row];
      const float raw = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      s[e] = prow_s[row] >= 0 ? raw * (c2 * rs[e]) : -INFINITY;
    }
    float tmax = s[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = __builtin_amdgcn_exp2f(s[e] - m_use);
      psum += p[e];
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[g][c] *= alpha;
    // P^T operand as hi + lo bf16 parts; fp8 rows carry their scale in p
    u32x4_t phi, plo;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = FP8 ? p[2 * d] * rs[2 * d] : p[2 * d];
      const float b = FP8 ? p[2 * d + 1] * rs[2 * d + 1] : p[2 * d + 1];
      const float ah = __uint_as_float(__float_as_uint(a) & 0xFFFF0000u);
      const float bh = __uint_as_float(__float_as_uint(b) & 0xFFFF0000u);
      phi[d] = pack_hi(a, b);
      plo[d] = pack_hi(a - ah, b - bh);
    }
    // O^T += V^T . P^T, four groups of 128 value dims
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x4_t R[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        R[e] = *reinterpret_cast<const u32x4_t*>(tile + krow(kg, e) * kLdsRow + (128 * g + 8 * ln) * 2);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        u32x4_t A0, A1;  // dims 8*ln + 2w and 8*ln + 2w + 1
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t x = R[2 * d][w], y = R[2 * d + 1][w];
          A0[d] = (x & 0xFFFFu) | (y << 16);
          A1[d] = (x >> 16) | (y & 0xFFFF0000u);
        }
        acc[g][2 * w] = mfma16(A0, phi, acc[g][2 * w]);
        acc[g][2 * w + 1] = mfma16(A1, phi, acc[g][2 * w + 1]);
        acc[g][2 * w] = mfma16(A0, plo, acc[g][2 * w]);
        acc[g][2 * w + 1] = mfma16(A1, plo, acc[g][2 * w + 1]);
      }
    }
    __syncthreads();
  }

  if (!qvalid) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : -INFINITY;
  float* dst;
  if (n_splits == 1) {
    dst = out + ((size_t)i * QR + qh) * kNope;
    if (lse_out && kg == 0) lse_out[(size_t)i * QR + qh] = lse2 * kLn2;
  } else {
    const size_t prow = ((size_t)i * n_splits + sp) * QR + qh;
    dst = part_o + prow * kNope;
    if (kg == 0) part_lse[prow] = lse2;
  }
  // lane holds dims 128g + 32kg + 8v + c, c = 0..7, for v = 0..3
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float* o = dst + 128 * g + 32 * kg + 8 * v;
      *reinterpret_cast<float4*>(o) = make_float4(acc[g][0][v] * inv, acc[g][1][v] * inv,
                                                  acc[g][2][v] * inv, acc[g][3][v] * inv);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[g][4][v] * inv, acc[g][5][v] * inv,
                                                      acc[g][6][v] * inv, acc[g][7][v] * inv);
    }
}

// Merge split partials: lse = log2 sum_s 2^lse_s, out = sum_s 2^(lse_s - lse) o_s.
__global__ __launch_bounds__(256) void k_attn_combine(int n_rows, int QR, int n_splits,
                                                      const float* __restrict__ part_o,
                                                      const float* __restrict__ part_lse,
                                                      float* __restrict__ out, float* __restrict__ lse_out) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  const int i = row / QR, qh = row - i * QR;
  float M = -INFINITY;
  for (int s = 0; s < n_splits; ++s) M = fmaxf(M, part_lse[((size_t)i * n_splits + s) * QR + qh]);
  float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float W = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const size_t pr = ((size_t)i * n_splits + s) * QR + qh;
      const float w = __builtin_amdgcn_exp2f(part_lse[pr] - M);
      W += w;
      const float4 a = *reinterpret_cast<const float4*>(part_o + pr * kNope + 8 * lane);
      const float4 b = *reinterpret_cast<const float4*>(part_o + pr * kNope + 8 * lane + 4);
      o[0] += w * a.x; o[1] += w * a.y; o[2] += w * a.z; o[3] += w * a.w;
      o[4] += w * b.x; o[5] += w * b.y; o[6] += w * b.z; o[7] += w * b.w;
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  float* d = out + (size_t)row * kNope + 8 * lane;
  *reinterpret_cast<float4*>(d) = make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  *reinterpret_cast<float4*>(d + 4) = make_float4(o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv);
  if (lse_out && lane == 0) lse_out[row] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
}

// fp32 rows and queries: one workgroup per query row, vector-unit fp32.
__global__ __launch_bounds__(256) void k_attn_f32(const float* __restrict__ q, int QR,
                                                  const int32_t* __restrict__ plan, int K,
                                                  const float* __restrict__ pool, int64_t pool_rows_n,
                                                  float sm_scale, float* __restrict__ out,
                                                  float* __restrict__ lse_out, uint32_t* __restrict__ err) {
  __shared__ float qs[kRowDim];
  __shared__ float pb[kMaxTopK];
  __shared__ int pr_s[kMaxTopK];
  __shared__ float red[4];
  const int qh = blockIdx.x, i = blockIdx.y, tid = threadIdx.x;
  const float* qr = q + ((size_t)i * QR + qh) * kRowDim;
  for (int d = tid; d < kRowDim; d += 256) qs[d] = qr[d];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = tid; j < K; j += 256) {
    int pr = plan[(size_t)i * K + j];
    if (pr >= pool_rows_n) {
      raise_error(err, HS_DEV_PLAN_RANGE, (uint32_t)i, (uint32_t)j);
      pr = -1;
    }
    pr_s[j] = pr;
    float s = -INFINITY;
    if (pr >= 0) {
      const float4* row = reinterpret_cast<const float4*>(pool + (size_t)pr * kRowDim);
      float a = 0.f;
      for (int d = 0; d < kRowDim / 4; ++d) {
        const float4 x = row[d];
        a += x.x * qs[4 * d] + x.y * qs[4 * d + 1] + x.z * qs[4 * d + 2] + x.w * qs[4 * d + 3];
      }
      s = a * sm_scale;
    }
    pb[j] = s;
    mx = fmaxf(mx, s);
  }
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < K; j += 256) {
    const float p = pb[j] == -INFINITY ? 0.f : expf(pb[j] - m);
    pb[j] = p;
    sum += p;
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  const float l = red[0] + red[1] + red[2] + red[3];
  float* dst = out + ((size_t)i * QR + qh) * kNope;
  for (int d = tid; d < kNope; d += 256) {
    float a = 0.f;
    for (int j = 0; j < K; ++j) {
      const float p = pb[j];
      if (p != 0.f) a += p * pool[(size_t)pr_s[j] * kRowDim + d];
    }
    dst[d] = l > 0.f ? a / l : 0.f;
  }
  if (lse_out && tid == 0) lse_out[(size_t)i * QR + qh] = l > 0.f ? m + logf(l) : -INFINITY;
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}

hs_status launch_attention(hs_pool* p, const void* q, int32_t q_dtype, int32_t n_req,
                           int32_t q_per_req, int32_t n_heads, const int32_t* plan, float sm_scale,
                           float* out, float* lse_out, hipStream_t s) {
  (void)q_dtype;
  const int K = p->d.top_k;
  const int QR = q_per_req * n_heads;
  uint32_t* err = reinterpret_cast<uint32_t*>(p->state + p->lay.error);
  if (p->d.kv_dtype == HS_F32) {
    k_attn_f32<<<dim3(QR, n_req), 256, 0, s>>>(static_cast<const float*>(q), QR, plan, K,
                                                reinterpret_cast<const float*>(p->pool_rows),
                                                p->pool_rows_n, sm_scale, out, lse_out, err);
    HS_HIP_CHECK(hipGetLastError());
    return HS_OK;
  }
  const int n_tiles = (K + kTile - 1) / kTile;
  const int n_hg = (QR + kQPerWG - 1) / kQPerWG;
  // Split the plan so that the grid covers the chip; a split is at least
  // two tiles so that a workgroup's partial output stays below its row bytes.
  static const int forced = env_int("HS_ATTN_TILES_PER_SPLIT", 0);
  int tps;
  if (forced > 0) {
    tps = forced;
  } else {
    const int base = n_req * n_hg;
    int splits = (512 + base - 1) / base;
    tps = (n_tiles + splits - 1) / splits;
    if (tps < 2) tps = 2;
  }
  if (tps > n_tiles) tps = n_tiles;
  int splits = (n_tiles + tps - 1) / tps;
  while (splits > 1 && (int64_t)n_req * QR * splits > p->off.at_part_rows) {
    ++tps;
    splits = (n_tiles + tps - 1) / tps;
  }
  float* part_o = reinterpret_cast<float*>(p->state + p->off.at_part_o);
  float* part_lse = reinterpret_cast<float*>(p->state + p->off.at_part_lse);
  const float c2 = sm_scale * kLog2e;
  const dim3 grid(splits, n_hg, n_req);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  if (p->d.kv_dtype == HS_BF16)
    k_attn_mfma<false><<<grid, kAttThreads, 0, s>>>(q16, QR, plan, K, p->pool_rows, nullptr, p->pool_rows_n,
                                                    c2, tps, splits, out, lse_out, part_o, part_lse, err);
  else
    k_attn_mfma<true><<<grid, kAttThreads, 0, s>>>(q16, QR, plan, K, p->pool_rows, p->pool_scales,
                                                   p->pool_rows_n, c2, tps, splits, out, lse_out, part_o,
                                                   part_lse, err);
  if (splits > 1) {
    const int rows = n_req * QR;
    k_attn_combine<<<(rows + 3) / 4, 256, 0, s>>>(rows, QR, splits, part_o, part_lse, out, lse_out);
  }
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
