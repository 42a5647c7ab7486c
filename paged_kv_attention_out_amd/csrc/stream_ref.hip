// HBM read-rate reference: a plain streaming read of a contiguous buffer,
// the floor against which the decode kernels' byte rate is compared.  It is
// not part of the attention path; the benchmark times it over the same byte
// counts the decode calls read.
//
// Block b reads its own contiguous span of the buffer (the spans tile the
// buffer in order), 256 threads x 16 bytes per load, UNROLL loads issued
// before any is used; each wave folds what it read into one word (XOR) and
// stores it, so no load can be dropped.

#include "pkv_common.h"
#include "pkv_ref.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* src, int64_t n16,
                                                              int64_t span, uint32_t* sink) {
  const int64_t begin = (int64_t)blockIdx.x * span;
  const int64_t end = begin + span < n16 ? begin + span : n16;
  uint32_t acc = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = src[i + k * kThreads];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < end; i += kThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if ((threadIdx.x & 63) == 0) sink[(int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

extern "C" size_t pkv_ref_stream_sink_words(int32_t blocks) {
  return blocks > 0 ? (size_t)blocks * (kThreads / 64) : 0;
}

extern "C" int pkv_ref_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink,
                                   void* stream) {
  if (blocks <= 0 || blocks > (1 << 20)) return PKV_EINVAL;
  if (bytes == 0) return PKV_OK;
  if (!src || !sink || !pkv_host::aligned16(src) || bytes % 16 != 0) return PKV_EINVAL;
  const int64_t n16 = (int64_t)(bytes / 16);
  // spans are whole multiples of one unrolled pass
  const int64_t pass = (int64_t)kThreads * kUnroll;
  const int64_t span = ((n16 + blocks - 1) / blocks + pass - 1) / pass * pass;
  const uint4* s = static_cast<const uint4*>(src);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), s, n16, span, sink);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}
