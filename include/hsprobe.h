/* libhsprobe: measurement probes that give the roofline denominators of the
 * decode step their measured values on the GPU at hand, beside the published
 * peaks. Not part of the decode path; nothing in libhisparse uses them.
 *
 *   host read  the link the miss copy of hs_resolve_rows reads over: rows of
 *              the pinned host store are read in place by the GPU over PCIe
 *              ("vLLM GLM 5.3 优化：混合 HiSparse 卸载", section "混合 HiSparse
 *              的技术实现", residency state 2: a missing row is copied from
 *              host memory into the hot buffer);
 *   HBM        a plain device copy and a plain device read;
 *   MFMA       independent chains of the bf16 16x16x32 MFMA that
 *              hs_sparse_mla_decode contracts with.
 *
 * Conventions: every call returns 0 on success, else a hipError_t value.
 * Calls only enqueue work on `stream` (none allocates or synchronises,
 * except hsp_alloc_pinned / hsp_free_pinned). Device pointers are the
 * caller's; the pinned buffer is the library's, from hsp_alloc_pinned.
 */
#ifndef HSPROBE_H
#define HSPROBE_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Pinned, device-mapped host memory of `bytes` bytes (hipHostMalloc with
 * the mapped and portable flags, as the pool's host store), filled with a
 * byte pattern by the host. *out receives the pointer the GPU reads through
 * (the same address on the host). Freed with hsp_free_pinned. */
int32_t hsp_alloc_pinned(size_t bytes, void** out);
int32_t hsp_free_pinned(void* p);

/* Zero-copy coalesced read of `bytes` (a multiple of 16) of pinned host
 * memory at `src` by `blocks` workgroups of 256 threads, each lane reading
 * 16-byte words in a grid-stride loop with 8 loads in flight. `sink`
 * (device, `blocks` uint32) receives a value only for a data pattern that
 * never occurs; it keeps the loads from being dropped. */
int32_t hsp_host_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream);

/* Zero-copy read of `n_rows` rows of `row_bytes` bytes (a multiple of 16,
 * at most 4096) at host row indices `rows` (device int64) of the `src_rows`
 * rows at `src`, `row_stride` bytes apart (>= row_bytes, a multiple of 16),
 * one wave per row, written to device memory `dst` (n_rows x row_bytes):
 * the access pattern of the miss copy. An index outside [0, src_rows) is
 * skipped (its destination row is not written); the caller keeps
 * src_rows * row_stride within the buffer. */
int32_t hsp_host_gather(const void* src, int64_t src_rows, int64_t row_bytes, int64_t row_stride,
                        const int64_t* rows, int32_t n_rows, void* dst, hipStream_t stream);

/* Device copy of `bytes` (a multiple of 16) from `src` to `dst` (both
 * device memory), 16-byte words, grid-stride over `blocks` x 256 threads. */
int32_t hsp_device_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream);

/* Device read of `bytes` (a multiple of 16) at `src`, as hsp_host_read. */
int32_t hsp_device_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream);

/* `blocks` workgroups of `waves` waves (1..16), each wave running `iters`
 * iterations of `chains` (4, 8 or 16) independent bf16 16x16x32 MFMAs on
 * register operands, counted as
 * blocks * waves * iters * chains * 16384 FLOP. `sink` (device, `blocks`
 * floats) receives a value only for a sum that never occurs. */
int32_t hsp_mfma_bf16(int32_t blocks, int32_t waves, int32_t iters, int32_t chains, float* sink,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSPROBE_H */
