// Measurement probes (libhsprobe): the measured PCIe host-read, HBM and
// bf16 MFMA rates that the decode step's roofline fractions are given
// against, beside the published peaks. See include/hsprobe.h.
#include <hip/hip_runtime.h>
#include <string.h>

#include "hsprobe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                   // 16-byte loads in flight per lane
constexpr uint32_t kNever = 0x9E3779B9u;     // a pattern the buffers never hold

// Grid-stride read of n16 16-byte words; each lane keeps kUnroll loads in
// flight. Works for host (mapped, read over PCIe) and device pointers.
__global__ __launch_bounds__(kThreads) void k_read(const u32x4* __restrict__ src, size_t n16,
                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == kNever) sink[blockIdx.x] = x;
}

__global__ __launch_bounds__(kThreads) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// One wave per row: the row's 16-byte words spread over the wave's lanes.
__global__ __launch_bounds__(kThreads) void k_gather(const uint8_t* __restrict__ src, int64_t src_rows,
                                                     int64_t row_bytes, int64_t row_stride,
                                                     const int64_t* __restrict__ rows,
                                                     int n_rows, uint8_t* __restrict__ dst) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kThreads / 64) + wave;
  if (j >= n_rows) return;
  const int64_t r = rows[j];
  if (r < 0 || r >= src_rows) return;
  const int w16 = (int)(row_bytes >> 4);
  const u32x4* s = reinterpret_cast<const u32x4*>(src + r * row_stride);
  u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)j * row_bytes);
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < w16) v[u] = s[lane + 64 * u];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (lane + 64 * u < w16) __builtin_nontemporal_store(v[u], d + lane + 64 * u);
}

template <int CHAINS>
__global__ void k_mfma(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = (__bf16)(float)((threadIdx.x + k) & 7);
    b[k] = (__bf16)(float)((threadIdx.x * 3 + k) & 7);
  }
  f32x4 c[CHAINS];
#pragma unroll
  for (int k = 0; k < CHAINS; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < CHAINS; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < CHAINS; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  if (s == -1.f) sink[blockIdx.x] = s;  // sums of products of non-negative values: never -1
}

}  // namespace

extern "C" {

int32_t hsp_alloc_pinned(size_t bytes, void** out) {
  if (!out || bytes == 0) return (int32_t)hipErrorInvalidValue;
  *out = nullptr;
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocMapped | hipHostMallocPortable);
  if (e != hipSuccess) return (int32_t)e;
  memset(p, 0x5A, bytes);
  *out = p;
  return 0;
}

int32_t hsp_free_pinned(void* p) {
  if (!p) return 0;
  return (int32_t)hipHostFree(p);
}

int32_t hsp_host_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || (bytes & 15) || blocks < 1) return (int32_t)hipErrorInvalidValue;
  k_read<<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
  return (int32_t)hipGetLastError();
}

int32_t hsp_device_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream) {
  return hsp_host_read(src, bytes, blocks, sink, stream);
}

int32_t hsp_host_gather(const void* src, int64_t src_rows, int64_t row_bytes, int64_t row_stride,
                        const int64_t* rows, int32_t n_rows, void* dst, hipStream_t stream) {
  if (!src || !rows || !dst || n_rows < 0 || src_rows < 1 || row_bytes < 16 || row_bytes > 4096 ||
      (row_bytes & 15) || row_stride < row_bytes || (row_stride & 15))
    return (int32_t)hipErrorInvalidValue;
  if (n_rows == 0) return 0;
  const int blocks = (n_rows + kThreads / 64 - 1) / (kThreads / 64);
  k_gather<<<blocks, kThreads, 0, stream>>>(static_cast<const uint8_t*>(src), src_rows, row_bytes, row_stride, rows,
                                            n_rows, static_cast<uint8_t*>(dst));
  return (int32_t)hipGetLastError();
}

int32_t hsp_device_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream) {
  if (!src || !dst || (bytes & 15) || blocks < 1) return (int32_t)hipErrorInvalidValue;
  k_copy<<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return (int32_t)hipGetLastError();
}

int32_t hsp_mfma_bf16(int32_t blocks, int32_t waves, int32_t iters, int32_t chains, float* sink,
                      hipStream_t stream) {
  if (!sink || blocks < 1 || waves < 1 || waves > 16 || iters < 1) return (int32_t)hipErrorInvalidValue;
  const dim3 g(blocks), b(64 * waves);
  switch (chains) {
    case 4: k_mfma<4><<<g, b, 0, stream>>>(iters, sink); break;
    case 8: k_mfma<8><<<g, b, 0, stream>>>(iters, sink); break;
    case 16: k_mfma<16><<<g, b, 0, stream>>>(iters, sink); break;
    default: return (int32_t)hipErrorInvalidValue;
  }
  return (int32_t)hipGetLastError();
}

}  // extern "C"
