// KV scatter: copy each new token's K and V rows into its pool slot.
//
// The write that mini-sglang's "Engine Class" (forward_batch) calls out_loc
// and miniVLLM's "Engine Architecture" (prepare_prefill / prepare_decode)
// calls slot_mapping.  A slot row is num_kv_heads * head_dim bf16 values,
// contiguous in both the source and the pool, so every thread moves one
// 16-byte piece; a block covers 256 consecutive pieces, K in grid.y = 0 and
// V in grid.y = 1.  Pure HBM streaming: 2 * row bytes read and written per
// token and tensor, no arithmetic on the data.

#include "pkv_common.h"

namespace {

struct StoreParams {
  const uint4* k_new;
  const uint4* v_new;
  const int32_t* out_loc;
  uint4* k_cache;
  uint4* v_cache;
  int64_t num_pieces;   // num_tokens * pieces_per_row
  int64_t num_slots;
  int32_t pieces_per_row;
};

__global__ __launch_bounds__(256) void store_kv_kernel(StoreParams p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= p.num_pieces) return;
  const int64_t t = i / p.pieces_per_row;
  const int64_t c = i - t * p.pieces_per_row;
  const int64_t slot = p.out_loc[t];
  if (slot < 0 || slot >= p.num_slots) return;  // out-of-range slots are skipped
  const uint4* src = blockIdx.y ? p.v_new : p.k_new;
  uint4* dst = blockIdx.y ? p.v_cache : p.k_cache;
  dst[slot * p.pieces_per_row + c] = src[i];
}

}  // namespace

extern "C" int pkv_store_kv(const void* k_new, const void* v_new, const int32_t* out_loc,
                            int64_t num_tokens, void* k_cache, void* v_cache,
                            int64_t num_slots, int32_t num_kv_heads, int32_t head_dim,
                            void* stream) {
  using namespace pkv_host;
  if (num_tokens < 0 || num_slots <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return PKV_EINVAL;
  if (head_dim % 8 != 0) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !out_loc || !k_cache || !v_cache) return PKV_EINVAL;
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return PKV_EINVAL;
  const int64_t pieces_per_row = (int64_t)num_kv_heads * head_dim / 8;
  if (pieces_per_row > INT32_MAX || num_tokens > INT64_MAX / pieces_per_row) return PKV_EINVAL;
  const int64_t num_pieces = num_tokens * pieces_per_row;
  const int64_t blocks = (num_pieces + 255) / 256;
  if (blocks > INT32_MAX) return PKV_EINVAL;
  StoreParams p;
  p.k_new = (const uint4*)k_new;
  p.v_new = (const uint4*)v_new;
  p.out_loc = out_loc;
  p.k_cache = (uint4*)k_cache;
  p.v_cache = (uint4*)v_cache;
  p.num_pieces = num_pieces;
  p.num_slots = num_slots;
  p.pieces_per_row = (int32_t)pieces_per_row;
  return launch(store_kv_kernel, dim3((unsigned)blocks, 2), dim3(256), (hipStream_t)stream, p);
}

extern "C" const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "success";
    case PKV_EINVAL: return "invalid argument";
    case PKV_EUNSUPPORTED: return "unsupported shape (head_dim, page_size or head grouping)";
    case PKV_ENOSPACE: return "workspace too small";
    case PKV_EHIP: return "HIP runtime error while launching";
    default: return "unknown status";
  }
}

extern "C" const char* pkv_version(void) { return "pkv 0.1.0 gfx950"; }
