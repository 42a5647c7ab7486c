// Device-side step metadata: the per-step arrays the engine otherwise builds
// on the host and copies over before every forward pass.
//
// * Prefill (miniVLLM "Engine Architecture", ModelRunner / prepare_prefill):
//   the batch holds only the tokens after each sequence's cached prefix;
//   cu_seqlens_q are the cumulative counts of those new tokens (the pages'
//   example: [0, 5, 8, 12]), and slot_mapping gives each new token the
//   physical cache slot it is written to.
// * Decode (prepare_decode): each sequence contributes one token, its most
//   recent; context_lens counts every token so far, so the new token sits at
//   position context_len - 1 and slot_mapping holds that one slot.
//
// A token at logical position t of request r lives in physical page
// page_table[r, t / page_size] at row t % page_size: slot = page *
// page_size + t % page_size (mini-sglang "Engine Class", Key Attributes:
// page_table; miniVLLM allocate_kv_cache for the pool layout).

#include <algorithm>

#include "pkv_common.h"

namespace {

struct PrefillMetaParams {
  const int32_t* seq_lens;
  const int32_t* prefix_lens;
  const int32_t* page_table;
  int32_t* cu_seqlens;
  int32_t* out_loc;
  int32_t num_seqs;
  int32_t pt_stride;
  int32_t page_size;
  int32_t max_tokens;
};

struct DecodeMetaParams {
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t* out_loc;
  int32_t num_seqs;
  int32_t pt_stride;
  int32_t page_size;
};

// New tokens of request r: seq_len - cached prefix, never negative.
__device__ __forceinline__ int new_tokens(const PrefillMetaParams& p, int r) {
  const int n = p.seq_lens[r];
  const int c = max(p.prefix_lens[r], 0);
  return (int)max((int64_t)n - c, (int64_t)0);
}

// Slot of logical position t of a request, or -1 when the position falls
// outside the page-table row.  Only page ids are read; the pool is not.
__device__ __forceinline__ int32_t slot_of(const int32_t* row, int pt_stride, int page_size,
                                           int64_t t) {
  const int64_t i = t / page_size;
  if (t < 0 || i >= pt_stride) return -1;
  const int64_t s = (int64_t)row[i] * page_size + t % page_size;
  return (s < 0 || s > INT32_MAX) ? -1 : (int32_t)s;
}

// Sum of two token counts, both >= 0, saturated at INT32_MAX: lengths are
// device values the host does not check, and saturated prefix sums stay
// non-negative and non-decreasing however large they are.
__device__ __forceinline__ int sat_add(int a, int b) {
  return (int)min((int64_t)a + b, (int64_t)INT32_MAX);
}

// cu_seqlens by one workgroup: the requests go in chunks of 1024, each
// chunk scanned in LDS (inclusive, Hillis-Steele) and offset by the total of
// the chunks before it.  Linear in the number of requests.
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kScanThreads) void prefill_cu_kernel(PrefillMetaParams p) {
  __shared__ int buf[2][kScanThreads];
  const int tid = threadIdx.x;
  int carry = 0;
  if (tid == 0) p.cu_seqlens[0] = 0;
  for (int r0 = 0; r0 < p.num_seqs; r0 += kScanThreads) {
    const int r = r0 + tid;
    int cur = 0;
    buf[0][tid] = r < p.num_seqs ? new_tokens(p, r) : 0;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
      const int v = sat_add(buf[cur][tid], tid >= off ? buf[cur][tid - off] : 0);
      buf[cur ^ 1][tid] = v;
      cur ^= 1;
      __syncthreads();
    }
    if (r < p.num_seqs) p.cu_seqlens[r + 1] = sat_add(carry, buf[cur][tid]);
    carry = sat_add(carry, buf[cur][kScanThreads - 1]);
    __syncthreads();  // every thread has read the chunk total before the next chunk
  }
}

// Batches of up to kScanThreads requests in one launch.  Every workgroup
// scans the counts as above and keeps each request's end offset and first
// position in LDS; then the grid strides over the batch's new tokens, each
// thread finding its token's request by binary search over the offsets, so
// the slots of one long request are spread over the whole grid instead of
// one wave's serial loop.  Workgroup 0 writes cu_seqlens.
constexpr int kMetaBlocks = 64;  // grid bound of the small-batch builder

__global__ __launch_bounds__(kScanThreads) void prefill_meta_small_kernel(PrefillMetaParams p) {
  __shared__ int buf[2][kScanThreads];
  __shared__ int first_pos[kScanThreads];
  const int tid = threadIdx.x;
  const int r = tid;
  const int cnt = r < p.num_seqs ? new_tokens(p, r) : 0;
  first_pos[tid] = r < p.num_seqs ? max(p.prefix_lens[r], 0) : 0;
  int cur = 0;
  buf[0][tid] = cnt;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = sat_add(buf[cur][tid], tid >= off ? buf[cur][tid - off] : 0);
    buf[cur ^ 1][tid] = v;
    cur ^= 1;
    __syncthreads();
  }
  // end[q]: new tokens of requests 0..q (saturated), non-decreasing, so for
  // t < end[num_seqs - 1] the search below lands on a request of the batch
  const int* end = buf[cur];
  if (blockIdx.x == 0) {
    if (tid == 0) p.cu_seqlens[0] = 0;
    if (r < p.num_seqs) p.cu_seqlens[r + 1] = end[tid];
  }
  const int total = min(end[kScanThreads - 1], p.max_tokens);
  for (int64_t t = blockIdx.x * kScanThreads + tid; t < total; t += gridDim.x * kScanThreads) {
    // the first request whose end offset exceeds t
    int q = 0;
#pragma unroll
    for (int step = kScanThreads / 2; step >= 1; step >>= 1)
      if (end[q + step - 1] <= t) q += step;
    q = min(q, p.num_seqs - 1);
    const int start = q == 0 ? 0 : end[q - 1];
    const int32_t* row = p.page_table + (int64_t)q * p.pt_stride;
    p.out_loc[t] = slot_of(row, p.pt_stride, p.page_size, (int64_t)first_pos[q] + (t - start));
  }
}

// One 256-thread block per request: its new tokens start at cu_seqlens[r]
// (written by prefill_cu_kernel, earlier on the same stream); the block
// writes their slots.
__global__ __launch_bounds__(256) void prefill_slots_kernel(PrefillMetaParams p) {
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int start = p.cu_seqlens[r];  // >= 0: saturated sums
  const int len = new_tokens(p, r);
  if (start < 0) return;
  const int32_t* row = p.page_table + (int64_t)r * p.pt_stride;
  const int first = max(p.prefix_lens[r], 0);
  const int n = min(len, p.max_tokens - start);  // tokens that land inside out_loc
  for (int64_t i = tid; i < n; i += 256)
    p.out_loc[start + i] = slot_of(row, p.pt_stride, p.page_size, first + i);
}

__global__ __launch_bounds__(256) void decode_meta_kernel(DecodeMetaParams p) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= p.num_seqs) return;
  const int n = p.seq_lens[r];
  p.out_loc[r] = n <= 0 ? -1
                        : slot_of(p.page_table + (int64_t)r * p.pt_stride, p.pt_stride,
                                  p.page_size, n - 1);
}

}  // namespace

extern "C" int pkv_prefill_metadata(const int32_t* seq_lens, const int32_t* prefix_lens,
                                    int32_t num_seqs, const int32_t* page_table,
                                    int32_t page_table_stride, int32_t page_size,
                                    int32_t max_tokens, int32_t* cu_seqlens_q,
                                    int32_t* out_loc, void* stream) {
  using namespace pkv_host;
  if (num_seqs < 0 || max_tokens < 0) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_lens || !prefix_lens || !page_table || !cu_seqlens_q) return PKV_EINVAL;
  if (max_tokens > 0 && !out_loc) return PKV_EINVAL;
  if (page_table_stride <= 0 || page_size <= 0) return PKV_EINVAL;
  PrefillMetaParams p;
  p.seq_lens = seq_lens;
  p.prefix_lens = prefix_lens;
  p.page_table = page_table;
  p.cu_seqlens = cu_seqlens_q;
  p.out_loc = out_loc;
  p.num_seqs = num_seqs;
  p.pt_stride = page_table_stride;
  p.page_size = page_size;
  p.max_tokens = max_tokens;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (num_seqs <= kScanThreads) {
    const int blocks = (int)std::min<int64_t>(
        std::max<int64_t>(((int64_t)max_tokens + kScanThreads - 1) / kScanThreads, 1),
        kMetaBlocks);
    return launch(prefill_meta_small_kernel, dim3((unsigned)blocks), dim3(kScanThreads), s, p);
  }
  const int st = launch(prefill_cu_kernel, dim3(1), dim3(kScanThreads), s, p);
  if (st != PKV_OK || max_tokens == 0) return st;
  return launch(prefill_slots_kernel, dim3((unsigned)num_seqs), dim3(256), s, p);
}

extern "C" int pkv_decode_metadata(const int32_t* seq_lens, int32_t num_seqs,
                                   const int32_t* page_table, int32_t page_table_stride,
                                   int32_t page_size, int32_t* out_loc, void* stream) {
  using namespace pkv_host;
  if (num_seqs < 0) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_lens || !page_table || !out_loc) return PKV_EINVAL;
  if (page_table_stride <= 0 || page_size <= 0) return PKV_EINVAL;
  DecodeMetaParams p;
  p.seq_lens = seq_lens;
  p.page_table = page_table;
  p.out_loc = out_loc;
  p.num_seqs = num_seqs;
  p.pt_stride = page_table_stride;
  p.page_size = page_size;
  return launch(decode_meta_kernel, dim3((unsigned)((num_seqs + 255) / 256)), dim3(256),
                static_cast<hipStream_t>(stream), p);
}
