/*
 * pkv_ref.h -- measurement reference shipped beside the attention library
 * (libpkv.so).  Not part of the attention path: the benchmark uses it to
 * measure the device's plain streaming-read rate over the same byte counts
 * the decode calls read, the floor the decode kernels are compared with.
 *
 * Status codes are those of pkv.h.
 */
#ifndef PKV_REF_H
#define PKV_REF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words the sink of a pkv_ref_stream_read launch of `blocks` workgroups
 * needs (one uint32 per wavefront); 0 for blocks <= 0. */
size_t pkv_ref_stream_sink_words(int32_t blocks);

/*
 * pkv_ref_stream_read -- read `bytes` of device memory at `src` once,
 * contiguously: `blocks` workgroups of 256 threads, each reading its own
 * contiguous span in 16-byte loads, eight in flight per thread.  Each
 * wavefront XORs what it read into one word and stores it to
 * sink[wavefront], so every byte is really loaded.
 *
 *   src    : device pointer, 16-byte aligned; bytes a multiple of 16
 *   blocks : 1 .. 2^20
 *   sink   : device, at least pkv_ref_stream_sink_words(blocks) uint32,
 *            caller-owned; overwritten
 *   stream : hipStream_t (NULL = the null stream)
 *
 * Returns PKV_EINVAL for a bad argument (nothing launched), PKV_EHIP if the
 * launch fails; bytes == 0 is a no-op.
 */
int pkv_ref_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink,
                        void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_REF_H */
