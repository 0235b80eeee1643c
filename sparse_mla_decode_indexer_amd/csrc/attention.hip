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
// k_attn_mfma (bf16 or fp8 rows, bf16 queries). A workgroup of 8 waves
// takes 64 query rows (4 blocks of 16; or 4 waves and 32 rows when only a
// few requests are decoded) of one request and a contiguous split of its
// plan, 32 rows (a tile) at a time:
//   - rows are fetched straight from the pool into LDS (buffer_load ... lds,
//     or global_load_lds for pools over 4 GB; no registers), through a ring
//     of three buffers: tiles t+1 and t+2 are in flight while tile t is
//     computed, and the queries load under the first gathers; fp8 codes
//     land raw and are widened to fp16 in registers after each operand
//     read (exact); absent rows read zeros; rows sit 73 (bf16) or 37
//     (fp8) chunks of 16 bytes apart in LDS (one pad chunk), so the MFMA
//     operand reads of 16 rows at one column spread over the banks and
//     operand addresses are a base plus an immediate offset;
//   - wave (q block, half) computes the partial scores of its 16 queries over
//     all 32 rows of the tile and its half (288) of the key dims,
//     S^T (32 x 16 q) += K (32 x 288) . Q^T, with 16x16x32 bf16 MFMAs (its
//     half of Q^T stays in registers); the two halves meet in LDS, so both
//     waves of a q block then hold the full scores;
//   - the scores land with each lane holding 8 rows of one query, exactly
//     the B operand of P^T: p stays in registers, split as hi + lo bf16
//     terms for bf16 rows (~16 significant bits per weight; a single bf16
//     term would cost up to 2^-8 relative error per weight); fp8 rows fold
//     their scale into the logit and into p in fp32;
//   - fp8 rows run both contractions in fp16 (codes widen to fp16 exactly;
//     each query half is scaled by a power of two so that its largest
//     magnitude lies in [2^14, 2^15), and the partial scores are scaled
//     back exactly), so p enters as a single fp16 term (11 significant
//     bits, round to nearest even) of p * row scale / the split's largest
//     row scale: 16 PV MFMAs per tile instead of 32;
//   - PV: O^T (256 dims x 16 q) += V^T . P^T; V^T operands come from LDS
//     transpose loads of the row-major tile (16-bit elements for bf16 rows;
//     8-bit codes, then widened, for fp8), in the same row order as P^T;
//   - two workgroup barriers per tile: tile landed / previous tile retired,
//     and the partial-score exchange; the gather of tile t + 2 is issued one
//     DMA at a time between the QK MFMAs of tile t;
//   - output rows leave through LDS so that each store writes whole lines.
// Softmax is online (fp32, base 2): a reference maximum that moves only
// when a score passes it by more than 2^8, and a running sum. With more than
// one split, each split writes a normalised partial output and its
// log-sum-exp; k_attn_combine merges them.
//
// k_attn_f32 (fp32 rows and queries): plain fp32 arithmetic on the vector
// units, one workgroup per (query row, split of the plan), the splits
// merged by k_attn_combine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include <math.h>
#include <stdlib.h>

#include "hs_internal.h"

namespace hs {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// A workgroup takes QB blocks of 16 query rows with 2 waves per block
// (launched with QB = 4, or 2 for a few requests).
constexpr int kTile = 32;              // rows per tile
constexpr int kChunks = 2 * kRowDim / 16;        // 72 chunks of 16 B per bf16 row
constexpr int kRowChunks = kChunks + 1;          // LDS row stride: 73 chunks (one pad chunk)
constexpr int kRawChunks = kRowDim / 16;         // 36 chunks per fp8 row
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazyMax = 8.f;  // see the online softmax in k_attn_mfma
// Tile gathers. When the pool spans at most kBufMaxBytes, rows are read
// through a raw buffer view of the pool (buffer_load ... lds, 32-bit
// offsets): absent rows and pad chunks take an offset past the view's end
// and read zeros. Larger pools use global_load_lds with 64-bit addresses and
// a zero row. The buffer form also keeps the compiler's LDS waits exact:
// with a global_load_lds in flight it treats the LDS counter as unordered
// and waits for every LDS read to finish before using any of them.
constexpr uint64_t kBufMaxBytes = 0xFFFF0000ull;
constexpr uint32_t kBufOob = 0xFFFF0000u;  // offset past any buffer view
constexpr int kBufWord3 = 0x00020000;      // descriptor word 3: 32-bit data format
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedVmemRead = 0x020;
constexpr int kQkAhead = 3;  // K operand steps loaded ahead of their MFMAs

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ inline bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// LDS transpose load of 4 x 16 bits (ds_read_b64_tr_b16): within each group
// of 16 lanes, output lane j receives element j % 4 of the 8 bytes addressed
// by lanes j / 4, 4 + j / 4, 8 + j / 4 and 12 + j / 4, in that order.
__device__ inline u32x2_t tr_load(const uint8_t* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
  const i16x4_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, r);
}

// LDS transpose load of 8 x 8 bits (ds_read_b64_tr_b8): within each group
// of 16 lanes, output lane j receives byte j % 8 of the 8 bytes addressed by
// lanes 2e + j / 8 of the group, as its byte e (e = 0..7).
__device__ inline u32x2_t tr8_load(const uint8_t* p) {
  typedef int i32x2_t __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)(p)));
}

// 8 OCP e4m3 codes (bytes 0..7) -> 8 fp16 in order (exact: every e4m3 value
// is an fp16 value; the hardware conversion with scale 1).
__device__ inline u32x4_t fp8x8_to_f16(u32x2_t w) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.f, true))};
}

__device__ inline f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ inline f32x4_t mfma16h(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                  c, 0, 0, 0);
}

// Two floats -> one dword of two fp16, round to nearest even.
__device__ inline uint32_t pack_f16(float a, float b) {
  const f16x2_t h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// s_waitcnt immediate: vmcnt(n) (6 bits, split over bits 3:0 and 15:14),
// expcnt and lgkmcnt left at their maximum (no wait).
constexpr int vmcnt_imm(int n) { return 0xF70 | (n & 0xF) | ((n & 0x30) << 10); }
static_assert(vmcnt_imm(0) == 0xF70 && vmcnt_imm(5) == 0xF75 && vmcnt_imm(38) == 0x8F76, "vmcnt encoding");

// Two floats -> one dword of two bf16 made of their upper halves
// (truncation; exact when the values are representable in bf16).
__device__ inline uint32_t pack_hi(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

// Workgroup barrier for LDS exchanges that leaves the tile prefetch in
// flight: wait for this wave's own LDS accesses (lgkmcnt 0 only), then
// s_barrier, with compiler-level memory barriers on both sides. A release
// fence (as in __syncthreads) would also wait for the global->LDS DMA of the
// next tile, since that DMA is an LDS write of this wave.
__device__ inline void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row of the tile in position e (0..7) of a lane's k-vector: the scores of
// rows 4*kg + 0..3 and 16 + 4*kg + 0..3 land in lane group kg = lane / 16.
__device__ inline int krow(int kg, int e) { return (e < 4) ? 4 * kg + e : 16 + 4 * kg + (e - 4); }

// Reductions over the 4 lanes l, l^16, l^32, l^48 that hold one query:
// each swap returns {x[l], x[l^32]} (or l^16) as a pair, in some order.
__device__ inline float max_across_kg(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_across_kg(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The plan rows of query row group (request) i: plan[(i / div) * stride + j]
// for j < K, or, with a union position map (speculative steps, where query
// token t of a request reads its own selection through the union's plan),
// plan[(i / div) * stride + upos[i * K + j]] (upos -1: absent).
struct PlanRef {
  const int32_t* plan;
  const int32_t* upos;  // or null
  int K, stride, div;
};

__device__ inline int plan_entry(const PlanRef& p, int i, int j, uint32_t* err) {
  const int32_t* pl = p.plan + (size_t)(i / p.div) * p.stride;
  if (!p.upos) return pl[j];
  const int u = p.upos[(size_t)i * p.K + j];
  if (u >= p.stride) {
    raise_error(err, HS_DEV_PLAN_RANGE, (uint32_t)i, (uint32_t)j);
    return -1;
  }
  return u >= 0 ? pl[u] : -1;
}

template <bool FP8, int QB, bool BUF>
__global__ __launch_bounds__(128 * QB) void k_attn_mfma(
    const uint16_t* __restrict__ q, int QR, PlanRef plan,
    const uint8_t* __restrict__ pool, const float* __restrict__ pool_scales, int64_t pool_rows_n,
    uint32_t pool_bytes, const uint8_t* __restrict__ zero_row, float c2, int tiles_per_split, int n_splits,
    float* __restrict__ out, float* __restrict__ lse_out, float* __restrict__ part_o,
    float* __restrict__ part_lse, uint32_t* __restrict__ err) {
  // A ring of three distinct LDS buffers (not one indexed array) so that
  // the compiler can tell the DMA into one from the reads of another and
  // does not wait for the prefetch before computing. Each holds a tile plus
  // the landing area of the padding DMAs (see issue below).
  // LDS row stride in 16-byte chunks: bf16 rows 72 + 1 pad, raw fp8 rows
  // 36 + 1 pad (the pad chunks read zeros), so that operand reads of 16
  // rows at one column spread over the banks
  constexpr int kRowChunksT = FP8 ? kRawChunks + 1 : kRowChunks;
  constexpr int kRowBytesT = 16 * kRowChunksT;
  constexpr int kPos = kTile * kRowChunksT;  // chunk positions of a tile
  constexpr int kIssue = (kPos + 128 * QB - 1) / (128 * QB);  // DMAs per thread and tile
  constexpr int kBufBytes = kIssue * 128 * QB * 16;
  __shared__ __attribute__((aligned(16))) uint8_t bufA[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bufB[kBufBytes];
  __shared__ __attribute__((aligned(16))) uint8_t bufC[kBufBytes];
  __shared__ int prow_s[kAttMaxTilesPerSplit * kTile];
  // Per-row softmax factors of the split: a row's base-2 logit is
  // raw * f[0] + f[1] (f[1] = -inf for an absent row) and its weight
  // p * f[2]; fp8: f = {c2 * scale, 0 or -inf, scale / sref}; bf16 rows
  // keep only the absent-row term (f[0] = c2, f[2] = 1).
  __shared__ f32x4_t rowf_s[FP8 ? kAttMaxTilesPerSplit * kTile : 1];
  __shared__ float rmask_s[FP8 ? 1 : kAttMaxTilesPerSplit * kTile];
  __shared__ f32x4_t sbuf[2][QB][2][64];  // partial scores [key half][q block][row block][lane]
  __shared__ float smax_s[2 * QB];        // fp8: largest row scale seen by each wave
  constexpr int kAttThreads = 128 * QB;
  constexpr int kQPerWG = 16 * QB;

  // Grid (splits, requests, query-row groups): the hardware deals
  // consecutive workgroups round-robin to the 8 XCDs, so when splits x
  // requests is a multiple of 8 the query-row groups of one (request,
  // split), which gather the same rows, all run on one XCD and share its L2.
  const int sp = blockIdx.x, i = blockIdx.y, hg = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = lane >> 4, ln = lane & 15;
  const int qb = wave % QB, half = wave / QB;  // query block; key-dim half (QK) and value-dim half (PV)
  const int qh = hg * kQPerWG + qb * 16 + ln;
  const bool qvalid = qh < QR;
  const int K = plan.K;
  const int n_tiles = (K + kTile - 1) / kTile;
  const int t_begin = sp * tiles_per_split;
  const int nt = min(n_tiles, t_begin + tiles_per_split) - t_begin;

  // plan rows (and fp8 scales) of this split; the query loads below stay in
  // flight across the barrier and the first gathers
  for (int j = tid; j < nt * kTile; j += kAttThreads) {
    const int jj = t_begin * kTile + j;
    int pr = jj < K ? plan_entry(plan, i, jj, err) : -1;
    if (pr >= pool_rows_n) {
      raise_error(err, HS_DEV_PLAN_RANGE, (uint32_t)i, (uint32_t)jj);
      pr = -1;
    }
    prow_s[j] = pr;
    if (FP8) rowf_s[j][0] = pr >= 0 ? pool_scales[pr] : 0.f;  // (the scale, until sref is known)
  }
  if constexpr (FP8) {  // the split's largest row scale (the fp16 weights are relative to it)
    float mx = 0.f;
    for (int j = tid; j < nt * kTile; j += kAttThreads) mx = fmaxf(mx, rowf_s[j][0]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
    if (lane == 0) smax_s[wave] = mx;
  }
  // Q^T operand for key dims 288*half .. +288: lane holds query row qh,
  // dims 288*half + 32*kk + 8*kg .. +8. Lanes past the last query row
  // compute on row 0 and write nothing. The registers are first read by the
  // first tile's QK, so the loads overlap the first gathers.
  constexpr int kKSteps = kRowDim / 64;  // 9
  u32x4_t qop[kKSteps];
  {
    const uint16_t* qr = q + ((size_t)i * QR + (qvalid ? qh : 0)) * kRowDim + 288 * half;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) qop[kk] = *reinterpret_cast<const u32x4_t*>(qr + 32 * kk + 8 * kg);
  }
  lds_sync();
  float sref = 1.f, inv_sref = 1.f;  // fp8: weights are p * scale / sref
  if constexpr (FP8) {
    float mx = 0.f;
#pragma unroll
    for (int w = 0; w < 2 * QB; ++w) mx = fmaxf(mx, smax_s[w]);
    if (mx > 0.f) {
      sref = mx;
      inv_sref = 1.f / mx;
    }
  }
  // the rows' softmax factors (each thread its own entries; the first tile's
  // barrier publishes them)
  for (int j = tid; j < nt * kTile; j += kAttThreads) {
    const bool present = prow_s[j] >= 0;
    if constexpr (FP8) {
      const float sc = rowf_s[j][0];
      rowf_s[j] = f32x4_t{present ? c2 * sc : 0.f, present ? 0.f : -INFINITY, sc * inv_sref, 0.f};
    } else {
      rmask_s[j] = present ? 0.f : -INFINITY;
    }
  }
  int q_shift = 0;  // fp8: this wave's query half was scaled by 2^q_shift

  // Gather of a tile into LDS (wave-contiguous LDS targets). This thread's
  // chunk positions p = k * threads + tid are the same in every tile; their
  // plan rows are read from LDS one tile ahead of the DMA, off the critical
  // path. Every wave issues exactly kIssue DMAs per tile, with every lane
  // active: positions past the tile, pad chunks, absent rows and tiles past
  // the split read the zero row. With a fixed count per tile the wait for a
  // tile is a constant vmcnt, and the compiler, which counts the same
  // instructions, sees that the tile is complete and adds no wait of its own.
  // tile-invariant per position: the tile row and the byte offset in the
  // row (-1: pad chunk or past the tile), from one division, then stepped
  int rowk[kIssue], coff[kIssue];
  {
    int r = tid / kRowChunksT, c = tid - r * kRowChunksT;
    constexpr int kStepR = kAttThreads / kRowChunksT, kStepC = kAttThreads % kRowChunksT;
#pragma unroll
    for (int k = 0; k < kIssue; ++k) {
      rowk[k] = min(r, kTile - 1);
      coff[k] = (r < kTile && c < (FP8 ? kRawChunks : kChunks)) ? c * 16 : -1;
      c += kStepC;
      r += kStepR;
      if (c >= kRowChunksT) {
        c -= kRowChunksT;
        ++r;
      }
    }
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  auto rows_of = [&](int t, int* rr) {
#pragma unroll
    for (int k = 0; k < kIssue; ++k) rr[k] = t < nt ? prow_s[t * kTile + rowk[k]] : -1;
  };
  const __amdgpu_buffer_rsrc_t pool_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)pool, 0, (int)pool_bytes, kBufWord3);
  auto issue = [&](const int* rr, uint8_t* dst) {
#pragma unroll
    for (int k = 0; k < kIssue; ++k) {
      constexpr int rb = FP8 ? kRowDim : 2 * kRowDim;
      const bool real = (rr[k] | coff[k]) >= 0;
      lds_void_t* ld = (lds_void_t*)(dst + (k * kAttThreads + wave_s * 64) * 16);
      if constexpr (BUF) {
        const uint32_t off = real ? (uint32_t)rr[k] * rb + (uint32_t)coff[k] : kBufOob;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(pool_rs, ld, 16, off, 0, 0, 0);
      } else {
        const uint8_t* src = real ? pool + (size_t)rr[k] * rb + coff[k] : zero_row;
        __builtin_amdgcn_global_load_lds(src, ld, 16, 0, 0);
      }
    }
  };
  constexpr int kWaitOne = vmcnt_imm(kIssue);      // all but the last tile issued
  constexpr int kWaitTwo = vmcnt_imm(2 * kIssue);  // all but the last two tiles issued

  // O^T accumulators: block b holds dims 256*half + 16b + 4kg + v (v = 0..3)
  // of query ln
  f32x4_t acc[16];
#pragma unroll
  for (int b = 0; b < 16; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // V^T operand reads (LDS transpose loads): in each 16-lane group, source
  // lane 4i + c reads dims 4c .. 4c+3 of row krow(kg, i) (first load) or
  // krow(kg, 4 + i) (second), and lane ln of the group receives dim ln of
  // those four rows: the A operand of 16 dims over rows krow(kg, 0..7).
  // Raw fp8 rows (8-bit transpose loads): source lane 2e + h of a group
  // reads dims 16b + 8h .. +8 of row krow(kg, e), and lane ln of the group
  // receives dim ln of the rows krow(kg, 0..7), as 8 codes widened in
  // registers.
  const int tr_i = (lane & 15) >> 2, tr_c = lane & 3;
  const int v_off0 = FP8 ? krow(kg, (lane & 15) >> 1) * kRowBytesT + 256 * half + 8 * (lane & 1)
                         : krow(kg, tr_i) * kRowBytesT + (256 * half + 4 * tr_c) * 2;
  const int v_off1 = krow(kg, 4 + tr_i) * kRowBytesT + (256 * half + 4 * tr_c) * 2;  // (bf16 only)
  // K operand reads (QK): lane (kg, ln) reads key dims 288*half + 32*kk +
  // 8*kg .. +8 of tile row 16*rb + ln (16 bytes of bf16, or 8 fp8 codes
  // widened in registers)
  const int k_off = ln * kRowBytesT + (FP8 ? 288 * half + 8 * kg : (288 * half + 8 * kg) * 2);
  float m_run = -INFINITY, lpart = 0.f;

  // One tile: wait for it, start the gather of tile t + 2 into `nxt` (the
  // buffer of tile t - 1), compute on `cur`. Tiles t and t + 1 are in flight
  // on entry (the latter possibly a padding gather).
  int rows_next[kIssue];
  auto tile = [&](int t, const uint8_t* cur, uint8_t* nxt) {
    __builtin_amdgcn_s_waitcnt(kWaitOne);  // this wave's part of tile t has landed
    lds_sync();                            // all of tile t is in LDS; tile t-1 is done
    const uint8_t* T = cur;
    // The gather of tile t + 2 goes out between the QK MFMAs below (one
    // DMA per key step): the CU's texture path moves a tile in about as
    // long as the QK phase takes, and DMAs issued all at once, by every
    // wave after the barrier, stalled the issuing waves until it drained.
    issue(rows_next, nxt);
    // QK partial over key dims 288*half .. +288, all 32 rows of the tile
    // (operand addresses: one per-lane base plus constant offsets)
    f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    const uint8_t* Tk = T + k_off;
    u32x4_t ka[kKSteps][2];
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if constexpr (FP8)
          ka[kk][rb] = fp8x8_to_f16(*reinterpret_cast<const u32x2_t*>(Tk + 16 * rb * kRowBytesT + 32 * kk));
        else
          ka[kk][rb] = *reinterpret_cast<const u32x4_t*>(Tk + 16 * rb * kRowBytesT + 64 * kk);
      }
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        sacc[rb] = FP8 ? mfma16h(ka[kk][rb], qop[kk], sacc[rb]) : mfma16(ka[kk][rb], qop[kk], sacc[rb]);
    // loads kQkAhead key steps ahead of their MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * kQkAhead, 0);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
      if (kk + kQkAhead < kKSteps) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      if (kk < kIssue) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    rows_of(t + 3, rows_next);
    if constexpr (FP8) {  // undo the query half's power-of-two scale (exact)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int v = 0; v < 4; ++v) sacc[rb][v] = ldexpf(sacc[rb][v], -q_shift);
    }
    sbuf[half][qb][0][lane] = sacc[0];
    sbuf[half][qb][1][lane] = sacc[1];
    lds_sync();
    sacc[0] += sbuf[half ^ 1][qb][0][lane];
    sacc[1] += sbuf[half ^ 1][qb][1][lane];
    // base-2 logits; lane holds rows krow(kg, e) of query ln
    float s[8], ws[8];
    float pm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = t * kTile + krow(kg, e);
      const float raw = e < 4 ? sacc[0][e] : sacc[1][e - 4];
      if constexpr (FP8) {
        const f32x4_t f = rowf_s[row];
        s[e] = fmaf(raw, f[0], f[1]);
        ws[e] = f[2];
      } else {
        s[e] = fmaf(raw, c2, rmask_s[row]);
      }
      pm = fmaxf(pm, s[e]);
    }
    pm = max_across_kg(pm);
    // The reference maximum moves only when a score passes it by more than
    // kLazyMax (base-2 units), so the accumulators are rarely rescaled; the
    // weights then stay below 2^kLazyMax, far inside fp32 and bf16 range.
    const bool grow = pm > m_run + kLazyMax;  // also the first finite maximum
    const bool rescale = grow && m_run != -INFINITY;
    const float m_new = grow ? pm : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m_run - m_new) : (grow ? 0.f : 1.f);
    m_run = m_new;
    u32x4_t bhi, blo;  // P^T operand (hi and lo parts; fp8: one fp16 term), rows krow(kg, 0..7)
    {
      float psum = 0.f, a[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(s[e] - m_use);
        psum += pe;
        a[e] = FP8 ? pe * ws[e] : pe;
        lo[e] = a[e] - __uint_as_float(__float_as_uint(a[e]) & 0xFFFF0000u);
      }
      lpart = lpart * alpha + psum;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if constexpr (FP8) {
          bhi[d] = pack_f16(a[2 * d], a[2 * d + 1]);
        } else {
          bhi[d] = pack_hi(a[2 * d], a[2 * d + 1]);
          blo[d] = pack_hi(lo[2 * d], lo[2 * d + 1]);
        }
      }
    }

    // PV: dims 256*half .. +256 of this wave's 16 queries, 16 at a time
    if (__any(rescale)) {  // the reference max moved for some query of this wave
#pragma unroll
      for (int b = 0; b < 16; ++b) acc[b] *= alpha;
    }
    u32x4_t va[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if constexpr (FP8) {
        va[b] = fp8x8_to_f16(tr8_load(T + v_off0 + 16 * b));
      } else {
        const u32x2_t x = tr_load(T + v_off0 + 32 * b);
        const u32x2_t y = tr_load(T + v_off1 + 32 * b);
        va[b] = u32x4_t{x[0], x[1], y[0], y[1]};
      }
    }
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      if constexpr (FP8) {
        acc[b] = mfma16h(va[b], bhi, acc[b]);
      } else {
        acc[b] = mfma16(va[b], bhi, acc[b]);
        acc[b] = mfma16(va[b], blo, acc[b]);
      }
    }
    // Instruction order: the operand loads run kPvAhead blocks ahead of
    // their MFMAs, so LDS latency overlaps the MFMAs of earlier blocks.
    constexpr int kPvMfma = FP8 ? 1 : 2;   // MFMAs per value block
    constexpr int kPvLoads = FP8 ? 1 : 2;  // transpose loads per value block
    // V^T operand blocks loaded ahead of their MFMAs: fp8 operands also wait
    // for their widening, so they go further ahead (6 was 2% faster than 3
    // on the fp8 workloads; bf16 is best at 3)
    constexpr int kPvAhead = FP8 ? 6 : 3;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPvLoads * kPvAhead, 0);
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPvMfma, 0);
      if (b + kPvAhead < 16) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPvLoads, 0);
    }
  };

  {
    int rr[kIssue];
    rows_of(0, rr);
    issue(rr, bufA);
    rows_of(1, rr);
    issue(rr, bufB);
    rows_of(2, rows_next);
  }
  __builtin_amdgcn_s_waitcnt(kWaitTwo);  // the query loads (issued before the gathers)
  if constexpr (FP8) {
    // Query half -> fp16, scaled by the power of two 2^q_shift that puts its
    // largest magnitude in [2^14, 2^15): exact for every element within 2^24
    // of that largest one (smaller ones contribute below 2^-24 of it).
    float m = 0.f;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        m = fmaxf(m, fabsf(__uint_as_float(qop[kk][d] << 16)));
        m = fmaxf(m, fabsf(__uint_as_float(qop[kk][d] & 0xFFFF0000u)));
      }
    m = max_across_kg(m);
    const int ex = (int)((__float_as_uint(m) >> 23) & 0xFF);
    q_shift = m > 0.f ? 141 - (ex == 0 ? 1 : ex) : 0;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
      for (int d = 0; d < 4; ++d)
        qop[kk][d] = pack_f16(ldexpf(__uint_as_float(qop[kk][d] << 16), q_shift),
                              ldexpf(__uint_as_float(qop[kk][d] & 0xFFFF0000u), q_shift));
  }
  // Full turns of the ring, then the 0-2 remaining tiles: every path issues
  // the same number of gathers per tile, so the compiler's count of pending
  // loads matches the waits above at every tile.
  int t = 0;
  for (; t + 3 <= nt; t += 3) {
    tile(t, bufA, bufC);
    tile(t + 1, bufB, bufA);
    tile(t + 2, bufC, bufB);
  }
  if (t < nt) {
    tile(t, bufA, bufC);
    if (t + 1 < nt) tile(t + 1, bufB, bufA);
  }
  // the two padding gathers issued by the last tiles land before the wave
  // ends (they were issued a tile earlier, so this rarely waits)
  __builtin_amdgcn_s_waitcnt(0xF70);

  // softmax denominator: sum over the 4 lanes (row groups) of each query
  const float l = sum_across_kg(lpart);
  lds_sync();  // every wave is past its last tile: the tile buffers are free
  const float inv = l > 0.f ? sref / l : 0.f;  // (sref = 1 for bf16 rows)
  const float lse2 = l > 0.f ? m_run + __log2f(l) : -INFINITY;
  if (qvalid && kg == 0 && half == 0) {
    if (n_splits == 1) {
      if (lse_out) lse_out[(size_t)i * QR + qh] = lse2 * kLn2;
    } else {
      part_lse[((size_t)i * n_splits + sp) * QR + qh] = lse2;
    }
  }
  // Output rows go out through this wave's own LDS region, 64 dims at a
  // time: lane (kg, ln) deposits dims 16b + 4kg .. +4 of query ln, then each
  // lane takes 16 contiguous bytes of one query, so that every store
  // instruction writes 256 contiguous bytes (whole cache lines) of each of
  // 4 rows. Streaming stores: the rows are read once, by the merge kernel
  // or the caller.
  constexpr int kStgRow = 272;  // a query's 64 dims (256 bytes) + 16 (LDS banks)
  constexpr int kStgPerBuf = kBufBytes / (16 * kStgRow);  // waves whose staging fits one ring buffer
  static_assert(2 * kStgPerBuf >= 2 * QB, "staging fits two ring buffers");
  uint8_t* stg = (wave < kStgPerBuf ? bufA + wave * 16 * kStgRow : bufB + (wave - kStgPerBuf) * 16 * kStgRow);
  const size_t row0 = n_splits == 1 ? (size_t)i * QR : ((size_t)i * n_splits + sp) * QR;
  float* const dst = n_splits == 1 ? out : part_o;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      const f32x4_t x = acc[4 * p + bb];
      *reinterpret_cast<f32x4_t*>(stg + ln * kStgRow + (16 * bb + 4 * kg) * 4) =
          f32x4_t{x[0] * inv, x[1] * inv, x[2] * inv, x[3] * inv};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ql = 4 * r + (lane >> 4);  // query of this lane's 16 bytes
      const f32x4_t y = *reinterpret_cast<const f32x4_t*>(stg + ql * kStgRow + (lane & 15) * 16);
      const int qh2 = hg * kQPerWG + qb * 16 + ql;
      if (qh2 < QR)
        __builtin_nontemporal_store(
            y, reinterpret_cast<f32x4_t*>(dst + (row0 + qh2) * kNope + 256 * half + 64 * p + 4 * (lane & 15)));
    }
  }
}

// Merge split partials: lse = log2 sum_s 2^lse_s, out = sum_s 2^(lse_s - lse) o_s.
// Thread (row, 4 dims): kBatch partial loads are in flight together; kBatch
// is the power of two >= the split count (2 to 32), so one round trip
// covers the usual split counts without many padding loads. One-wave
// workgroups: a single request's 128 query rows (16K threads) then spread
// over every CU instead of a quarter of them.
constexpr int kCombineThreads = 64;
template <int kBatch>
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(int n_rows, int QR, int n_splits,
                                                                  const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_lse,
                                                                  float* __restrict__ out,
                                                                  float* __restrict__ lse_out) {
  const int g = blockIdx.x * kCombineThreads + threadIdx.x;
  const int row = g / (kNope / 4), d4 = g - row * (kNope / 4);
  if (row >= n_rows) return;
  const int i = row / QR, qh = row - i * QR;
  const size_t base = (size_t)i * n_splits * QR + qh;  // partial row of split s: base + s * QR
  // One pass: the log-sum-exps and partial outputs of a batch of splits are
  // loaded together, the sums are rescaled when the running maximum moves.
  float M = -INFINITY;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float W = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += kBatch) {
    float w[kBatch];
    float4 x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int s = min(s0 + u, n_splits - 1);  // padding entries reload the last split
      const size_t pr = base + (size_t)s * QR;
      w[u] = s0 + u < n_splits ? part_lse[pr] : -INFINITY;
      const f32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(part_o + pr * kNope) + d4);
      x[u] = make_float4(t[0], t[1], t[2], t[3]);  // (read once: streaming load)
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mb = fmaxf(mb, w[u]);
    if (mb == -INFINITY) continue;  // nothing attended so far
    const float f = __builtin_amdgcn_exp2f(M - mb);  // 0 while M is -inf
    W *= f;
    o.x *= f; o.y *= f; o.z *= f; o.w *= f;
    M = mb;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float e = __builtin_amdgcn_exp2f(w[u] - M);  // 0 for empty splits and padding
      W += e;
      o.x += e * x[u].x; o.y += e * x[u].y; o.z += e * x[u].z; o.w += e * x[u].w;
    }
  }
  const float inv = W > 0.f ? 1.f / W : 0.f;
  __builtin_nontemporal_store(f32x4_t{o.x * inv, o.y * inv, o.z * inv, o.w * inv},
                              reinterpret_cast<f32x4_t*>(out + (size_t)row * kNope) + d4);
  if (lse_out && d4 == 0) lse_out[row] = W > 0.f ? (M + __log2f(W)) * kLn2 : -INFINITY;
}

// fp32 rows and queries: one workgroup per (query row, split of the plan),
// fp32 on the vector units. Scores: wave w takes rows w, w + 4, ... of the
// split; the 64 lanes read a row's 576 values together (9 each,
// coalesced), 16 rows in flight per wave, and sum across lanes. Weighted
// sum: thread t owns output dims t and t + 256 and walks the split's rows
// in plan order, 32 rows' loads in flight; absent rows read the zero row.
// With more than one split each writes its normalised partial output and
// base-2 log-sum-exp for k_attn_combine.
constexpr int kF32Threads = 256;
constexpr int kF32MinRowsPerSplit = 32;
__global__ __launch_bounds__(kF32Threads) void k_attn_f32(const float* __restrict__ q, int QR,
                                                         PlanRef plan,
                                                         const float* __restrict__ pool, int64_t pool_rows_n,
                                                         const float* __restrict__ zero_row, float sm_scale,
                                                         int rows_per_split, int n_splits,
                                                         float* __restrict__ out, float* __restrict__ lse_out,
                                                         float* __restrict__ part_o, float* __restrict__ part_lse,
                                                         uint32_t* __restrict__ err) {
  constexpr int kPerLane = kRowDim / 64;  // 9
  constexpr int kWaves = kF32Threads / 64;
  __shared__ float qs[kRowDim];
  __shared__ float pb[kMaxTopK];
  __shared__ int pr_s[kMaxTopK];
  __shared__ float red[kWaves];
  const int qh = blockIdx.x, i = blockIdx.y, sp = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j_begin = sp * rows_per_split;
  const int K = max(0, min(plan.K, j_begin + rows_per_split) - j_begin);  // this split's rows
  const float* qr = q + ((size_t)i * QR + qh) * kRowDim;
  for (int d = tid; d < kRowDim; d += kF32Threads) qs[d] = qr[d];
  for (int j = tid; j < K; j += kF32Threads) {
    int pr = plan_entry(plan, i, j_begin + j, err);
    if (pr >= pool_rows_n) {
      raise_error(err, HS_DEV_PLAN_RANGE, (uint32_t)i, (uint32_t)(j_begin + j));
      pr = -1;
    }
    pr_s[j] = pr;
  }
  __syncthreads();
  float qv[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) qv[u] = qs[lane + 64 * u];
  auto row_of = [&](int j) -> const float* {
    const int pr = j < K ? pr_s[j] : -1;
    return pr >= 0 ? pool + (size_t)pr * kRowDim : zero_row;
  };

  constexpr int kRowsInFlight = 16;
  float mx = -INFINITY;
  for (int j0 = wave; j0 < K; j0 += kWaves * kRowsInFlight) {
    float x[kRowsInFlight][kPerLane];
#pragma unroll
    for (int r = 0; r < kRowsInFlight; ++r) {
      const float* row = row_of(j0 + kWaves * r);
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) x[r][u] = row[lane + 64 * u];
    }
#pragma unroll
    for (int r = 0; r < kRowsInFlight; ++r) {
      float a = 0.f;
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) a += x[r][u] * qv[u];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) a += __shfl_xor(a, o, 64);
      const int j = j0 + kWaves * r;
      if (j < K) {
        const float sj = pr_s[j] >= 0 ? a * sm_scale : -INFINITY;
        if (lane == 0) pb[j] = sj;
        mx = fmaxf(mx, sj);
      }
    }
  }
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float m = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int j = tid; j < K; j += kF32Threads) {
    const float p = pb[j] == -INFINITY ? 0.f : expf(pb[j] - m);
    pb[j] = p;
    sum += p;
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  float l = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) l += red[w];

  constexpr int kPvInFlight = 32;
  float a0 = 0.f, a1 = 0.f;  // dims tid and tid + 256
  for (int j0 = 0; j0 < K; j0 += kPvInFlight) {
    float v0[kPvInFlight], v1[kPvInFlight];
#pragma unroll
    for (int u = 0; u < kPvInFlight; ++u) {
      const float* row = row_of(j0 + u);
      v0[u] = row[tid];
      v1[u] = row[tid + kF32Threads];
    }
#pragma unroll
    for (int u = 0; u < kPvInFlight; ++u) {
      const float p = j0 + u < K ? pb[j0 + u] : 0.f;
      a0 += p * v0[u];
      a1 += p * v1[u];
    }
  }
  if (n_splits == 1) {
    float* dst = out + ((size_t)i * QR + qh) * kNope;
    dst[tid] = l > 0.f ? a0 / l : 0.f;
    dst[tid + kF32Threads] = l > 0.f ? a1 / l : 0.f;
    if (lse_out && tid == 0) lse_out[(size_t)i * QR + qh] = l > 0.f ? m + logf(l) : -INFINITY;
  } else {  // partials as the merge kernel takes them (log-sum-exp in base 2)
    const size_t prow = ((size_t)i * n_splits + sp) * QR + qh;
    float* dst = part_o + prow * kNope;
    dst[tid] = l > 0.f ? a0 / l : 0.f;
    dst[tid + kF32Threads] = l > 0.f ? a1 / l : 0.f;
    if (tid == 0) part_lse[prow] = l > 0.f ? (m + logf(l)) * kLog2e : -INFINITY;
  }
}

// Split partials of hs_sparse_mla_decode_noalloc (kStaticScratchBytes per
// GPU, held until the process ends). Host code never uses this name as an
// address: it uses the device address static_scratch_address returns.
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

hs_status static_scratch_address(int device, uint8_t** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint8_t* ptrs[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices || !out) return HS_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return set_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol);
    ptrs[device] = static_cast<uint8_t*>(ptr);
  }
  *out = ptrs[device];
  return HS_OK;
}

static int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}

// The merge of n_splits partials for each of `rows` query rows.
static void launch_combine(int rows, int QR, int n_splits, const float* part_o, const float* part_lse, float* out,
                           float* lse_out, hipStream_t s) {
  const int64_t threads = (int64_t)rows * (kNope / 4);
  const int nb = (int)((threads + kCombineThreads - 1) / kCombineThreads);
#define HS_COMBINE(B) k_attn_combine<B><<<nb, kCombineThreads, 0, s>>>(rows, QR, n_splits, part_o, part_lse, out, lse_out)
  if (n_splits <= 2)
    HS_COMBINE(2);
  else if (n_splits <= 4)
    HS_COMBINE(4);
  else if (n_splits <= 8)
    HS_COMBINE(8);
  else if (n_splits <= 16)
    HS_COMBINE(16);
  else
    HS_COMBINE(32);
#undef HS_COMBINE
}

hs_status launch_attention(hs_pool* p, const void* q, int32_t q_dtype, int32_t n_req,
                           int32_t q_per_req, int32_t n_heads, const int32_t* plan, const int32_t* upos,
                           int32_t k_plan, int32_t plan_div, float sm_scale, float* out, float* lse_out,
                           float* part_o, float* part_lse, int64_t part_rows, hipStream_t s) {
  (void)q_dtype;
  const int K = k_plan;
  const PlanRef pref{plan, upos, k_plan, p->d.top_k, plan_div};
  const int QR = q_per_req * n_heads;
  uint32_t* err = reinterpret_cast<uint32_t*>(p->state + p->lay.error);
  if (p->d.kv_dtype == HS_F32) {
    // splits of at least kF32MinRowsPerSplit rows, enough for ~512
    // workgroups, within the partial rows
    int splits = (int)std::min<int64_t>((K + kF32MinRowsPerSplit - 1) / kF32MinRowsPerSplit,
                                        std::max<int64_t>(1, 512 / std::max<int64_t>(1, (int64_t)n_req * QR)));
    splits = (int)std::max<int64_t>(1, std::min<int64_t>(splits, part_rows / std::max<int64_t>(1, (int64_t)n_req * QR)));
    const int rps = (K + splits - 1) / splits;
    k_attn_f32<<<dim3(QR, n_req, splits), kF32Threads, 0, s>>>(
        static_cast<const float*>(q), QR, pref, reinterpret_cast<const float*>(p->pool_rows), p->pool_rows_n,
        reinterpret_cast<const float*>(p->state + p->off.zero_row), sm_scale, rps, splits, out, lse_out, part_o,
        part_lse, err);
    if (splits > 1) launch_combine(n_req * QR, QR, splits, part_o, part_lse, out, lse_out, s);
    HS_HIP_CHECK(hipGetLastError());
    return HS_OK;
  }
  const int n_tiles = (K + kTile - 1) / kTile;
  const uint8_t* zero_row = p->state + p->off.zero_row;
  // Split the plan so that about one workgroup per CU is busy, with a floor
  // on the tiles per split so that the fixed cost per workgroup (plan,
  // queries, partial output) is amortised. Workgroups take 4 blocks of 16
  // query rows (8 waves), or 2 blocks (4 waves) when even the smallest
  // splits of 4-block workgroups leave most CUs idle (a few requests: twice
  // the workgroups, each with half the LDS traffic per tile).
  static const int forced = env_int("HS_ATTN_TILES_PER_SPLIT", 0);
  static const int forced_qb = env_int("HS_ATTN_QB", 0);
  constexpr int min_tps = 2;
  const int64_t wg4 = (int64_t)n_req * ((QR + 63) / 64) * ((n_tiles + min_tps - 1) / min_tps);
  const int qb = (forced_qb == 2 || forced_qb == 4) ? forced_qb : (wg4 < 256 ? 2 : 4);
  const int q_per_wg = 16 * qb;
  const int n_hg = (QR + q_per_wg - 1) / q_per_wg;
  int tps;
  if (forced > 0) {
    tps = forced;
  } else {
    const int base = n_req * n_hg;
    const int want = (256 + base - 1) / base;
    tps = (n_tiles + want - 1) / want;
    if (tps < min_tps) tps = min_tps;
  }
  if (tps > n_tiles) tps = n_tiles;
  if (tps > kAttMaxTilesPerSplit) tps = kAttMaxTilesPerSplit;
  int splits = (n_tiles + tps - 1) / tps;
  while (splits > 1 && (int64_t)n_req * QR * splits > part_rows) {
    ++tps;
    splits = (n_tiles + tps - 1) / tps;
  }
  // more tiles per workgroup than the kernel takes: the partial buffer is
  // too small for this batch (nothing is enqueued)
  if (tps > kAttMaxTilesPerSplit) return HS_ERR_CAPACITY;
  const float c2 = sm_scale * kLog2e;
  const dim3 grid(splits, n_req, n_hg);
  const uint16_t* q16 = static_cast<const uint16_t*>(q);
  const bool fp8 = p->d.kv_dtype != HS_BF16;
  const float* sc = fp8 ? p->pool_scales : nullptr;
  const uint64_t pool_bytes = (uint64_t)p->pool_rows_n * (fp8 ? kRowDim : 2 * kRowDim);
  const bool buf = pool_bytes <= kBufMaxBytes;
  const uint32_t pb32 = buf ? (uint32_t)pool_bytes : 0u;
#define HS_ATTN_LAUNCH(F, B, U)                                                                           \
  k_attn_mfma<F, B, U><<<grid, 128 * (B), 0, s>>>(q16, QR, pref, p->pool_rows, sc, p->pool_rows_n, pb32, \
                                                  zero_row, c2, tps, splits, out, lse_out, part_o, part_lse, err)
#define HS_ATTN_LAUNCH_QB(F, U) \
  if (qb == 4)                  \
    HS_ATTN_LAUNCH(F, 4, U);    \
  else                          \
    HS_ATTN_LAUNCH(F, 2, U)
  if (fp8 && buf) {
    HS_ATTN_LAUNCH_QB(true, true);
  } else if (fp8) {
    HS_ATTN_LAUNCH_QB(true, false);
  } else if (buf) {
    HS_ATTN_LAUNCH_QB(false, true);
  } else {
    HS_ATTN_LAUNCH_QB(false, false);
  }
#undef HS_ATTN_LAUNCH_QB
#undef HS_ATTN_LAUNCH
  if (splits > 1) launch_combine(n_req * QR, QR, splits, part_o, part_lse, out, lse_out, s);
  HS_HIP_CHECK(hipGetLastError());
  return HS_OK;
}

}  // namespace hs
