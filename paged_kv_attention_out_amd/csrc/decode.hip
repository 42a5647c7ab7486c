// Paged decode attention: one query token per request over its whole
// context, read through the page table (miniVLLM "Engine Architecture",
// prepare_decode: context_lens + block_tables; mini-sglang "Engine Class",
// Key Attributes: page_table).  The same kernels serve multi-token decode
// (a few draft tokens per request, causal among themselves: the verification
// step of speculative decoding, zero-to-sglang Part II Ch.1 section 4).
//
// Two kernels on the caller's stream:
//
// decode_split_kernel -- one wavefront per (request r, KV head kvh, split s),
//   two of them (adjacent KV heads of one split) per workgroup when Hkv is
//   even.  A split is `split` consecutive tokens; a request with n tokens has
//   ceil(n/split) splits.  The wave walks its tokens 16 at a time ("groups"):
//   * S^T = K Q^T on MFMA 16x16x32 bf16: each lane's K loads (8 dims of its
//     token's row per 32-dim block) are the A operand as loaded; the B
//     columns hold the (query token, query head) pairs of the KV head -- g
//     heads x LQ tokens, replicated to fill 16 columns.
//   * Softmax: base 2 with scale * log2(e) folded in, lazy rescaling (only
//     when a score exceeds the running max by more than kTau, so p <= 2^kTau;
//     the function is unchanged, only the reference point moves).
//   * O += P V on MFMA 16x16x32 per pair of groups: P straight from the S^T
//     registers (bf16), V staged row-major in LDS and read key-contiguous
//     with ds_read_b64_tr_b16.
//   * K/V rows of a chunk of groups are loaded together, then computed.
//   * A request with one split writes bf16 output directly; otherwise the
//     split writes (m, l, un-normalised o) to the workspace.
// decode_combine_kernel -- one wavefront per (r, query token, query head) with >= 2
//   splits merges the partials (flash-decoding): M = max m_s,
//   L = sum l_s 2^(m_s-M), out = sum o_s 2^(m_s-M) / L.
//
// Bandwidth: every K/V byte of the context is read once; partials add
// splits * g * (D + 2) * 4 bytes written and read per (r, kvh).

#include <algorithm>
#include <atomic>
#include <mutex>
#include <new>

#include "pkv_common.h"
#include "prefix_pass.h"

#ifndef PKV_DECODE_NBUF_D64
#define PKV_DECODE_NBUF_D64 8
#endif
#ifndef PKV_DECODE_NBUF_D128
#define PKV_DECODE_NBUF_D128 4
#endif

namespace {

using namespace pkv;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  uint16_t* out;
  // Fused step (pkv_decode_step): the new token of request r (position
  // seq_lens[r] - 1, slot out_loc[r]) is read from k_new/v_new [B, Hkv, d]
  // and written to the pools; null for a plain decode call.
  const uint16_t* k_new;
  const uint16_t* v_new;
  const int32_t* out_loc;
  uint16_t* k_pool;  // the pools, writable (same memory as k_cache / v_cache)
  uint16_t* v_pool;
  int64_t num_slots;
  float* ws_m;  // [B * Hkv * n_split_max * g]
  float* ws_l;
  float* ws_o;  // [B * Hkv * n_split_max * g * D]
  int32_t* ws_split;  // the split the split kernel used (read by the combine)
  // Balanced launch (decode_balanced_kernel): partial rows of its pieces and
  // per (request, KV head) the first row and the row count; null when the
  // workspace does not hold them.
  float* bal_m;
  float* bal_l;
  float* bal_o;
  int32_t* bal_table;
  int32_t auto_split;  // the split is the automatic one (a caller's split is kept)
  int64_t num_pages;
  int32_t page_size;
  int32_t page_shift;
  int32_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_seq_len;
  int32_t split;        // host split (tokens); the device may pick a longer one
  int32_t n_split_max;  // partial slots per (request, KV head): shared-prefix splits (if
                        // any), then the splits per request at the host split
  int32_t n_unit_splits;  // splits per request at the host split (sizes the grid)
  int32_t round_units;  // units per KV head and query slice that one round of resident
                        // waves holds; 0 = use `split` as given
  int32_t q_len;     // query tokens per request (1 for plain decode)
  int32_t q_slices;  // units per (request, KV head, split): each takes LQ query tokens
  int32_t heads_per_block;  // waves per workgroup, one per KV head (1, 2, 4 or 8)
  float scale_log2;  // softmax_scale * log2(e)
  // Shared prefixes (pkv_paged_attn_decode_shared): request r's first
  // skip[r] tokens (rounded down to 16) are attended by the shared-prefix
  // pass, whose partials fill slots 0 .. ceil(skip / ksplit) - 1 of (r, KV
  // head); the splits here cover the rest of the context and take the slots
  // after them.  Null: no request skips anything.
  const int32_t* skip;
  int32_t ksplit;
  int32_t max_skip;  // max_shared_len: the pass's slots are sized for at most this many
};

// Tokens of request r attended by the shared-prefix pass (0 without one),
// a multiple of 16 above neither n nor max_shared_len, and the partial slots
// that pass fills.
__device__ __forceinline__ int skip_tokens(const DecodeParams& p, int skip_raw, int n) {
  return p.skip == nullptr ? 0 : min(max(skip_raw, 0), min(max(n, 0), p.max_skip)) & ~15;
}
__device__ __forceinline__ int prefix_slots(const DecodeParams& p, int skip) {
  return skip == 0 ? 0 : (skip + p.ksplit - 1) / p.ksplit;
}

constexpr float kTau = 8.0f;

// DPP lane exchanges inside a row of 16 lanes.  After the two quad steps
// every lane of a quad holds the quad's total; row_half_mirror pairs quad 0
// with quad 1 (and 2 with 3), row_mirror pairs the two halves of the row.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp<kQuadXor1>(v));
  v = fmaxf(v, dpp<kQuadXor2>(v));
  v = fmaxf(v, dpp<kHalfMirror>(v));
  v = fmaxf(v, dpp<kRowMirror>(v));
  return v;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<kQuadXor1>(v);
  v += dpp<kQuadXor2>(v);
  v += dpp<kHalfMirror>(v);
  v += dpp<kRowMirror>(v);
  return v;
}

// Sum over the wavefront: DPP sums inside each row of 16 lanes, then the
// four row totals read as scalars (no LDS permutes).
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xf, 0xf, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xf, 0xf, false);  // row_mirror
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
         __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

// Inclusive prefix sum over the 64 lanes: inside each row of 16 lanes by
// shifts of 1, 2, 4 and 8 (lanes shifted in from outside the row add 0),
// then row 0's total is added to row 1 and row 2's to row 3 (row_bcast:15),
// and the total of rows 0-1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
  return v;
}

// Request lengths of the first 256 requests, 64 per chunk (lane = request
// within the chunk), clamped to [0, max_seq_len]; -1 where there is no
// request.
struct Lens4 {
  int v[4];
};

// Split length of a call whose split is chosen on the device.  Work units
// are (request, split) pairs, and the call time follows how they fill
// rounds of the waves that are resident at once: for a batch that needs few
// rounds, a split just long enough that all units fit one round beats a
// shorter split that leaves a partial last round (measured on the
// Llama-shaped, shared-prefix and speculative batches).  The host enables
// this (round_units > 0) only for batches of at most 256 requests that need
// at most 4 rounds at its split even at the longest length, and then
// launches one round of workgroups.  The split kernel takes a multiple of 16
// at or above the host split whose units fit that round (always possible:
// every request is one unit at split >= its length, and num_seqs <=
// round_units): the estimate from units(s) ~ tokens/s + num_seqs/2 when its
// exact count fits, else the smallest fitting one above it.
__device__ int device_split(const DecodeParams& p, const Lens4& lens) {
  const int T = p.round_units;
  if (T <= 0) return p.split;
  const int* len = lens.v;  // -1: no request
  const int nk = (p.num_seqs + 63) >> 6;  // chunks of 64 requests that exist
  auto units = [&](int x) {  // max(ceil(n / x), 1) per request, summed (exact)
    const float inv = __builtin_amdgcn_rcpf((float)x);  // the integer corrections below absorb its error
    int u = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (k < nk && len[k] >= 0) {
        // ceil(n / x) from a float quotient corrected by integer products
        int q = (int)((float)len[k] * inv);
        q += q * x < len[k];
        q += q * x < len[k];
        q -= q > 0 && (q - 1) * x >= len[k];
        u += max(q, 1);
      }
    }
    return wave_sum(u);
  };
  // (the host's gate keeps tokens <= 4 * T * split, far below 2^31)
  int tokens = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) tokens += max(len[k], 0);
  tokens = wave_sum(tokens);
  const int denom = max(T - p.num_seqs / 2, 1);
  const int est = max(p.split, ((tokens + denom - 1) / denom + 15) & ~15);
  // Otherwise gallop up from the estimate to a bracket (bad, good] --
  // units(bad) > T >= units(good) -- and bisect it; units() does not increase
  // with the split, and at split >= the longest request it is num_seqs <= T,
  // so the gallop ends.
  int good, bad, step = 16;
  if (units(est) <= T) {
    return est;
  } else {
    bad = est;
    good = est + step;
    while (units(good) > T) {
      bad = good;
      step *= 2;
      good = bad + step;
    }
  }
  while (good - bad > 16) {
    const int mid = bad + (((good - bad) >> 1) & ~15);
    if (units(mid) <= T) good = mid; else bad = mid;
  }
  return good;
}

#ifdef PKV_DECODE_WAVES_PER_EU
#define PKV_DECODE_OCC __attribute__((amdgpu_waves_per_eu(PKV_DECODE_WAVES_PER_EU)))
#else
#define PKV_DECODE_OCC
#endif

template <int D, int G>
struct DecodeTraits {
  // groups of 16 tokens per load chunk (even: PV consumes groups in pairs)
  static constexpr int NBUF = D == 64 ? PKV_DECODE_NBUF_D64 : PKV_DECODE_NBUF_D128;
  static_assert(NBUF % 2 == 0, "chunks hold pairs of groups");
};

// Per-split kernel, one wavefront per (request, KV head, split).
//
// One piece of a balanced launch (decode_balanced_kernel): tokens
// [t0, t1) of request r's KV head kvh (n tokens in all), partial row `id`.
struct Piece {
  int r, kvh, n, t0, t1, id;
};

// Per group of 16 tokens (lane l: token l%16 of the group, c = l/16):
//   S^T = K Q^T on MFMA 16x16x32: A = the K rows as loaded (lane l holds 8
//   dims 32kk+8c.. of token l%16), B = Q^T (column n = query head n % G,
//   so the G heads are replicated over the 16 columns).  Lane l receives
//   the scores of tokens 4c..4c+3 for query head (l%16) % G.
// Per pair of groups (32 tokens), O += P V on MFMA 16x16x32:
//   A = P: row = query head column, key slot (c, i) = token 4c+i of the
//   first group (i < 4) or of the second (i >= 4) -- exactly the S^T
//   registers this lane already holds, rounded to bf16.
//   B = V with the same key order: the V rows are staged row-major in LDS
//   and read back key-contiguous with ds_read_b64_tr_b16, which, within
//   each 16-lane group, hands lane 4q+e element e of the 8-byte chunks that
//   lanes q, q+4, q+8, q+12 point at; pointing lane L at row k0 + L/4,
//   column 4*(L%4) gives every lane 4 consecutive keys of one dim.
//   O (16 head rows x D dims) lives in D/16 accumulators of 4 registers;
//   row 4c+i is query head i % G.
// SKIP: requests may skip their shared-prefix tokens (p.skip); compiled
// out of the kernels of plain decode.
// BAL: the unit is the given piece of a balanced launch (LQ == 1, no
// skipped tokens) instead of the one `bid` selects.
template <int D, int G, int LQ, bool SKIP, bool BAL = false>
__device__ __forceinline__ void decode_split_unit(const DecodeParams& p, const uint32_t bid,
                                                  uint16_t* vlds_block,
                                                  const Piece* piece = nullptr) {
  constexpr int KCH = D / 32;  // 16-byte pieces per lane per row == QK MFMAs per group
  constexpr int NT = D / 16;   // 16-dim tiles of the output == PV MFMAs per pair
  constexpr int NBUF = DecodeTraits<D, G>::NBUF;
  constexpr int VPITCH = D + 8;  // LDS row pitch (bf16): conflict-free rows
  constexpr int NC = G * LQ;     // distinct query columns: (query token, query head)
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "query heads per KV head");
  static_assert(NC <= 16 && (16 % NC) == 0, "the 16 MFMA columns hold whole copies of the columns");
  // LDS: NBUF * 16 * VPITCH values per wave, sized at launch.
  // A workgroup holds heads_per_block waves, one per KV head of the same
  // unit: adjacent heads' slices of every token row are then read by one
  // CU at the same time.
  const int wv = (int)(threadIdx.x >> 6);
  uint16_t* vlds = vlds_block + wv * (NBUF * 16 * VPITCH);

  const int lane = threadIdx.x & 63;
  // Block -> unit: rank = block / (Hkv * slices) walks the (request, split) pairs that
  // exist -- each request has max(ceil(n / split), 1) splits; the full-length
  // ones come first, request-major, then each request's short last split --
  // so every block of the grid past the last pair sits at its end and the
  // dispatcher starts real units first.  The KV head is the fastest
  // index: the heads of one (request, split) sweep the same pages together.
  // It rotates from one rank to the next because blocks land on the 8 XCDs
  // round-robin: every XCD then sees every head's offset within the page rows.
  // With several query slices (multi-token queries wider than the 16 MFMA
  // columns) the slices of one unit are Hkv / heads_per_block blocks apart:
  // with that a multiple of 8 they share an XCD, so the second slice reads
  // K/V from L2.
  static_assert(!BAL || (LQ == 1 && !SKIP), "balanced pieces are single-token decode");
  const uint32_t hblocks = (uint32_t)(p.num_kv_heads / p.heads_per_block);  // blocks per unit
  const uint32_t u = bid / hblocks;
  const uint32_t rank = LQ == 1 ? u : u / (uint32_t)p.q_slices;
  const int tq0 = LQ == 1 ? 0 : (int)(u % (uint32_t)p.q_slices) * LQ;  // first query token
  const int QL = LQ == 1 ? 1 : p.q_len;
  const int kvh = BAL ? piece->kvh : (int)((bid + rank) % hblocks) * p.heads_per_block + wv;
  // The first 256 request lengths: four loads at clamped indices, issued
  // together (one memory round trip; the empty asm keeps the compiler from
  // moving each load into a branch of its own).  Then, not waited for with
  // them, one 256-byte piece of the page table per wave: the waves of an
  // XCD together bring the rows of a small table into its L2 while the unit
  // is being found, so the window read below hits there.
  // With shared prefixes a request's work is the rest of its context after
  // the skipped tokens; a request whose whole context is shared has no unit
  // here (-1, as a missing request).
  Lens4 lens;
  int skv[4] = {0, 0, 0, 0};
  int pf = 0;
  if constexpr (!BAL) {
    int x[4], y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = p.seq_lens[min(64 * k + lane, p.num_seqs - 1)];
    if (SKIP) {
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = p.skip[min(64 * k + lane, p.num_seqs - 1)];
    }
    const int64_t pt_entries = (int64_t)p.num_seqs * p.pt_stride;
    pf = p.page_table[min(((int64_t)(bid >> 3) * p.heads_per_block + wv) * 64 + lane,
                          pt_entries - 1)];
    asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = min(max(x[k], 0), p.max_seq_len);
      skv[k] = SKIP ? skip_tokens(p, y[k], n) : 0;
      const int w = n - skv[k];
      lens.v[k] = 64 * k + lane < p.num_seqs && (skv[k] == 0 || w > 0) ? w : -1;
    }
  }
  const int sl = BAL ? 0 : device_split(p, lens);  // tokens per split
  if (!BAL && p.ws_split != nullptr && bid == 0 && threadIdx.x == 0) *p.ws_split = sl;
  int r = -1, split = 0, n = 0, skip = 0;  // n: work tokens after the skipped ones
  if constexpr (BAL) {
    r = piece->r;
    n = piece->n;
  } else {
    // Units in two parts: first every full-length split of every request
    // (request-major), then the short last split of each request whose
    // length is not a multiple of the split (and the one unit of an empty
    // request), so that the grid ends with its shortest units and the last
    // round of a multi-round launch drains quickly.
    int chunk_skip = 0;  // this lane's skipped tokens in the current chunk
    auto chunk_len = [&](int c0) -> int {  // work tokens; -1: no request (or no work)
      const int k = c0 >> 6;
      if (k < 4) {
        chunk_skip = k == 0 ? skv[0] : k == 1 ? skv[1] : k == 2 ? skv[2] : skv[3];
        return k == 0 ? lens.v[0] : k == 1 ? lens.v[1] : k == 2 ? lens.v[2] : lens.v[3];
      }
      const int rr = c0 + lane;
      if (rr >= p.num_seqs) return -1;
      const int n = min(max(p.seq_lens[rr], 0), p.max_seq_len);
      chunk_skip = SKIP ? skip_tokens(p, p.skip[rr], n) : 0;
      return chunk_skip == 0 || n > chunk_skip ? n - chunk_skip : -1;
    };
    int target = (int)rank;
    for (int part = 0; part < 2 && r < 0; ++part) {
      int base = 0;  // units of the requests before this chunk of 64
      for (int c0 = 0; c0 < p.num_seqs; c0 += 64) {
        const int len = chunk_len(c0);
        const int full = len < 0 ? 0 : len / sl;
        const int cnt = part == 0 ? full : (len == 0 || (len > 0 && len != full * sl)) ? 1 : 0;
        const int inc = wave_incl_scan(cnt);
        const int total = __builtin_amdgcn_readlane(inc, 63);
        if (target < base + total) {
          const int rel = target - base;
          const uint64_t hit = __ballot(rel >= inc - cnt && rel < inc);
          if (hit == 0) break;  // (cannot happen: the unit lies in this chunk)
          const int lr = (int)__builtin_ctzll(hit);
          r = c0 + lr;
          split = part == 0 ? rel - __builtin_amdgcn_readlane(inc - cnt, lr)
                            : __builtin_amdgcn_readlane(full, lr);
          n = __builtin_amdgcn_readlane(len, lr);
          skip = SKIP ? __builtin_amdgcn_readlane(chunk_skip, lr) : 0;
          break;
        }
        base += total;
      }
      target -= base;
    }
  }
  if (r < 0) return;  // past the last pair
  const int64_t rk = (int64_t)r * p.num_kv_heads + kvh;
  const int slot0 = prefix_slots(p, skip);  // partial slots of the shared-prefix pass
  const int j = lane & 15;  // token within the group / score column
  const int c = lane >> 4;  // 16-byte piece within each 64-byte block / token quad
  const int col = j % NC;   // logical column of this lane: query token col / G, head col % G
  const int hcol = col % G;
  // Query token of the column; columns past the last token repeat it and
  // are never written.
  const int tq = min(tq0 + col / G, QL - 1);
  const int t_begin = BAL ? piece->t0 : skip + split * sl;

  // Q^T fragments (B operand): column j holds query token tq of head
  // kvh*G + hcol (the NC columns repeat over the 16 MFMA columns).
  bf16x8 qb[KCH];
  {
    const uint16_t* qp =
        p.q + (((int64_t)r * QL + tq) * p.num_q_heads + (int64_t)kvh * G + hcol) * D + 8 * c;
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) qb[kk] = as_bf16x8(ld16(qp + 32 * kk));
  }

  // Page ids, one window of up to 64 logical pages at a time (lane i holds
  // page base + i), so the streaming loop below issues no loads other than
  // K/V rows and needs no branches to find a page.  Entries past the
  // request's last page may be read but are never used.
  const int32_t* pt = p.page_table + (int64_t)r * p.pt_stride;
  int ptv = 0, lp_base = 0;
  auto load_window = [&](int base) {
    lp_base = base;
    const int i0 = base + lane;
    const int v = i0 < p.pt_stride ? pt[i0] : 0;
    ptv = (v < 0 || (int64_t)v >= p.num_pages) ? 0 : v;  // keep accesses in the pool
  };
  load_window(t_begin >> p.page_shift);
  if (!BAL) asm volatile("" ::"v"(pf));  // keeps the prefetch; its wait comes with the window's

  if (n <= 0) {
    if (split == 0) {
#pragma unroll
      for (int t = tq0; t < tq0 + LQ; ++t) {
        if (t >= QL) break;
        uint16_t* row = p.out + (((int64_t)r * QL + t) * p.num_q_heads + (int64_t)kvh * G) * D;
        for (int i = lane; i < G * D / 8; i += 64)
          reinterpret_cast<uint4*>(row)[i] = make_uint4(0, 0, 0, 0);
      }
    }
    return;
  }
  const int ns = BAL ? 0 : (n + sl - 1) / sl;
  const int t_end = BAL ? piece->t1 : min(skip + n, t_begin + sl);
  // The output is written directly only when this split is the request's
  // one partial; otherwise partials go to the workspace.
  const bool direct = BAL ? piece->t0 == 0 && piece->t1 == n : ns == 1 && slot0 == 0;
  const bool last = BAL ? t_end == n : split == ns - 1;  // holds the newest token

  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  // Fused step: the request's last split writes this head's slice of the
  // new token's K/V rows to slot out_loc[r] (out-of-range slots are
  // skipped).  No wave of this call reads that slot from the pool.
  if (LQ == 1 && p.k_new != nullptr && last && lane < D / 8) {
    const int64_t slot = p.out_loc[r];
    if (slot >= 0 && slot < p.num_slots) {
      const int64_t src = ((int64_t)r * p.num_kv_heads + kvh) * D + 8 * lane;
      const int64_t dst = slot * row_elems + (int64_t)kvh * D + 8 * lane;
      *reinterpret_cast<uint4*>(p.k_pool + dst) = ld16(p.k_new + src);
      *reinterpret_cast<uint4*>(p.v_pool + dst) = ld16(p.v_new + src);
    }
  }
  const int64_t page_elems = row_elems << p.page_shift;
  const int lane_off = (j * p.num_kv_heads + kvh) * D + 8 * c;

  auto group_offset = [&](int t0) -> int64_t {
    const int i = uniform((t0 >> p.page_shift) - lp_base);  // < 64 inside a window
    const int page = __builtin_amdgcn_readlane(ptv, i);
    return (int64_t)page * page_elems + (int64_t)(t0 & (p.page_size - 1)) * row_elems;
  };

  // Fused step: the lane whose token is the new one (position n - 1) reads
  // its row from k_new / v_new instead of the pool.
  const int t_new = LQ == 1 && p.k_new != nullptr ? skip + n - 1 : -1;
  const int64_t new_off = ((int64_t)r * p.num_kv_heads + kvh) * D + 8 * c;

  uint4 kb[NBUF][KCH], vb[NBUF][KCH];
  auto load_group = [&](int t0, int loff, int row, int buf) {
    const int64_t goff = group_offset(t0) + loff;
    const bool fresh = t0 + row == t_new;
    const uint16_t* kp = fresh ? p.k_new + new_off : p.k_cache + goff;
    const uint16_t* vp = fresh ? p.v_new + new_off : p.v_cache + goff;
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      if (b == buf) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk) kb[b][kk] = ld16(kp + 32 * kk);
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk) vb[b][kk] = ld16(vp + 32 * kk);
      }
    }
  };
  // K rows of a group -> S^T scores (4 tokens per lane)
  auto scores = [&](int buf) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
      if (b == buf) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb[b][kk]), qb[kk], acc, 0, 0,
                                                        0);
      }
    return acc;
  };
  // V rows of a group -> LDS slot (16 rows), row-major
  auto stage_v = [&](int buf, int slot) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b)
      if (b == buf) {
#pragma unroll
        for (int kk = 0; kk < KCH; ++kk)
          *reinterpret_cast<uint4*>(&vlds[(slot * 16 + j) * VPITCH + 32 * kk + 8 * c]) = vb[b][kk];
      }
  };
  auto zero_v = [&](int slot) {
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk)
      *reinterpret_cast<uint4*>(&vlds[(slot * 16 + j) * VPITCH + 32 * kk + 8 * c]) =
          make_uint4(0, 0, 0, 0);
  };

  f32x4 o[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_own = kNegInf;  // running max of this lane's column (equal in all its lanes)
  float l_own = 0.f;      // this lane's share of the row sum of its column
  // Query token tq sits at position n - QL + tq and sees keys up to there;
  // lim_lo is the lowest limit among this block's columns.
  const int lim = skip + n - QL + tq;
  const int lim_lo = skip + n - QL + tq0;

  const int trq = j & 3, trj = j >> 2;  // transpose-read lane roles

  // One pair of groups: softmax of the 32 scores, then O += P V.
  // va / vbv: valid tokens of each group (0 = absent group); ta / tb: the
  // groups' first positions (for the causal limit of multi-token queries).
  auto pv_pair = [&](f32x4 sa, f32x4 sb, int va, int vbv, int slot_a, int slot_b, int ta,
                     int tb) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = sa[i] * p.scale_log2;
      x[4 + i] = sb[i] * p.scale_log2;
    }
    if (va < 16 || vbv < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = 4 * c + i < va ? x[i] : kNegInf;
        x[4 + i] = 4 * c + i < vbv ? x[4 + i] : kNegInf;
      }
    }
    if (LQ > 1 && tb + 15 > lim_lo) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = ta + 4 * c + i <= lim ? x[i] : kNegInf;
        x[4 + i] = tb + 4 * c + i <= lim ? x[4 + i] : kNegInf;
      }
    }
    float lm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) lm = fmaxf(lm, x[i]);
    if (__any(lm > m_own + kTau)) {
      // New running max of each column: over the lanes that hold it -- the
      // four token quads (lane ^ 16, ^ 32) and the copies of the column
      // among the 16 MFMA columns (lane ^ NC, ^ 2NC, ...).
      float v = fmaxf(lm, __shfl_xor(lm, 16));
      v = fmaxf(v, __shfl_xor(v, 32));
#pragma unroll
      for (int off = NC; off < 16; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
      const float mn = fmaxf(m_own, v);
      const float a_own = mn == kNegInf ? 0.f : fast_exp2(m_own - mn);
      m_own = mn;
      l_own *= a_own;
      // O row 4c+i is column (4c+i) % NC, whose factor lane (4c+i) % NC holds.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ar = __shfl(a_own, (4 * c + i) % NC);
#pragma unroll
        for (int t = 0; t < NT; ++t) o[t][i] *= ar;
      }
    }
    // A multi-token column with no visible key yet keeps m = -inf: subtract
    // 0 instead so its probabilities come out 0, not NaN.
    const float m_sub = LQ > 1 && m_own == kNegInf ? 0.f : m_own;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = fast_exp2(x[i] - m_sub);
      l_own += e[i];
    }
    uint4 pw;
    pw.x = pack_bf16x2(e[0], e[1]);
    pw.y = pack_bf16x2(e[2], e[3]);
    pw.z = pack_bf16x2(e[4], e[5]);
    pw.w = pack_bf16x2(e[6], e[7]);
    const bf16x8 pa = as_bf16x8(pw);
    const int ra = (slot_a * 16 + 4 * c + trj) * VPITCH + 4 * trq;
    const int rb = (slot_b * 16 + 4 * c + trj) * VPITCH + 4 * trq;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const s16x4 lo = lds_read_tr16(vlds + ra + 16 * t);
      const s16x4 hi = lds_read_tr16(vlds + rb + 16 * t);
      const s16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8, vv), o[t], 0,
                                                     0, 0);
    }
  };

  // Main loop over windows of up to 64 pages.  A window ends at the end of
  // its 64th page (or of the split), never inside a 65th: a split need not
  // start on a page boundary (split lengths are multiples of 16, pages may
  // be longer), and the next window then starts at the page boundary.
  // Inside a window the groups go in chunks of NBUF: every K/V load of a
  // chunk is issued first, then the pairs of groups are computed in order,
  // each waiting only for its own rows.  No load is pending across a loop
  // back-edge, so the wait counts the compiler derives are exact.
  for (int w0 = t_begin, w_end; w0 < t_end; w0 = w_end) {
    if (w0 != t_begin) load_window(w0 >> p.page_shift);
    w_end = (int)min((int64_t)t_end, (int64_t)(lp_base + 64) << p.page_shift);
    const int len = w_end - w0;
    const int tail = len & 15;
    const int nfull = len >> 4;
    int g = 0;
    for (; g + NBUF <= nfull; g += NBUF) {
#pragma unroll
      for (int b = 0; b < NBUF; ++b) load_group(w0 + 16 * (g + b), lane_off, j, b);
      __builtin_amdgcn_sched_barrier(0);  // every load of the chunk issues first
#pragma unroll
      for (int b = 0; b < NBUF; b += 2) {
        const f32x4 sa = scores(b), sb = scores(b + 1);
        stage_v(b, b);
        stage_v(b + 1, b + 1);
        pv_pair(sa, sb, 16, 16, b, b + 1, w0 + 16 * (g + b), w0 + 16 * (g + b + 1));
      }
    }
    // Remaining full groups and the tail, two groups at a time; an absent
    // second group contributes zero probabilities against zero rows.
    const int ng = nfull + (tail ? 1 : 0);
    for (; g < ng; g += 2) {
      const int va = g < nfull ? 16 : tail;
      const int vbv = g + 1 < nfull ? 16 : (g + 1 == nfull ? tail : 0);
      const int ja = j < va ? j : va - 1;  // rows past the end repeat the last valid row
      load_group(w0 + 16 * g, (ja * p.num_kv_heads + kvh) * D + 8 * c, ja, 0);
      f32x4 sb = {0.f, 0.f, 0.f, 0.f};
      if (vbv > 0) {
        const int jb = j < vbv ? j : vbv - 1;
        load_group(w0 + 16 * (g + 1), (jb * p.num_kv_heads + kvh) * D + 8 * c, jb, 1);
        sb = scores(1);
        stage_v(1, 1);
      } else {
        zero_v(1);
      }
      const f32x4 sa = scores(0);
      stage_v(0, 0);
      pv_pair(sa, sb, va, vbv, 0, 1, w0 + 16 * g, w0 + 16 * (g + 1));
    }
  }

  // Row sums: a column's keys are spread over the four token quads.
  float l_tot = l_own + __shfl_xor(l_own, 16);
  l_tot += __shfl_xor(l_tot, 32);
  // O row x = 4c + i (query column x % NC) sits in lanes 16c .. 16c+15, dim
  // 16t + lane % 16; lane x holds column x's max and sum.
  if (4 * c >= NC) return;  // rows 4c.. hold no column of their own
  const int dl = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = 4 * c + i;
    const float Lx = __shfl(l_tot, x % NC);
    const float Mx = __shfl(m_own, x % NC);
    const int h = x % G, tx = tq0 + x / G;
    if (x >= NC || tx >= QL) continue;
    if (direct) {
      // (a multi-token row with no visible key has L = 0 and gets zeros)
      const float inv = LQ > 1 && Lx == 0.f ? 0.f : 1.f / Lx;
      uint16_t* o_row =
          p.out + (((int64_t)r * QL + tx) * p.num_q_heads + (int64_t)kvh * G + h) * D;
#pragma unroll
      for (int t = 0; t < NT; ++t) o_row[16 * t + dl] = to_bf16(o[t][i] * inv);
    } else {
      // Partial (m, l, un-normalised o) of this split for column (tx, h)
      // among the QL * G columns of the request's KV head.
      const int64_t base =
          (BAL ? (int64_t)piece->id : rk * p.n_split_max + slot0 + split) * (QL * G) + tx * G + h;
      float* dst = p.ws_o + base * D + dl;
#pragma unroll
      for (int t = 0; t < NT; ++t) dst[16 * t] = o[t][i];
      if (dl == 0) {
        p.ws_m[base] = Mx;
        p.ws_l[base] = Lx;
      }
    }
  }
}

template <int D, int G, int LQ, bool SKIP = false>
__global__ __launch_bounds__(512, 2) PKV_DECODE_OCC void decode_split_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t vlds_block[];
  decode_split_unit<D, G, LQ, SKIP>(p, blockIdx.x, vlds_block);
}

// Balanced decode of a batch that needs several rounds of units.  With one
// block per (request, split) the dispatcher starts units as slots free up,
// and the launch ends with a last round of long units draining one by one
// (on the Qwen-shaped batch the slots are busy 85% of the time).  Here one
// round of workgroups shares the work exactly: the batch is one sequence of
// 16-token blocks -- request by request, block by block (a request's last
// block may be partial) -- of total H, and workgroup g of W takes blocks
// [g Q, (g + 1) Q), Q = ceil(H / W), with one wave per KV head, so a
// workgroup reads whole token rows as a plain streaming read would.  Its
// range covers the end of one request, whole requests and the start of
// another; each such piece starts on a 16-token boundary (as every unit
// does: a group of 16 tokens never crosses a page) and is attended as a
// unit by every wave for its head, leaving a partial, or the output itself
// when the piece is the whole request.  A piece starting at block a of
// request r has partial row r + floor(a / Q) (per KV head): rows rise
// through the batch, a request's rows are consecutive, and its first piece
// records the first row and the row count for the merge.  At most 256
// requests (their lengths stay in registers) and 8 KV heads.
constexpr int kBalMaxSeqs = 256;
constexpr int kBalMaxWaves = 4096;  // waves at most (partial rows kept for the cut points)

template <int D, int G>
__global__ __launch_bounds__(512, 2) PKV_DECODE_OCC void decode_balanced_kernel(DecodeParams p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t vlds_block[];
  const int lane = threadIdx.x & 63;
  const int kvh = (int)(threadIdx.x >> 6);  // one wave per KV head
  const uint32_t W = gridDim.x;
  const int hkv = p.num_kv_heads;
  // Lengths (lane = request within a chunk of 64) and their 16-token blocks,
  // scanned per chunk; base[k]: blocks before chunk k.
  int len[4], inc[4];
  uint32_t base[5];
  {
    int x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = p.seq_lens[min(64 * k + lane, p.num_seqs - 1)];
    base[0] = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      len[k] = 64 * k + lane < p.num_seqs ? min(max(x[k], 0), p.max_seq_len) : 0;
      inc[k] = wave_incl_scan((len[k] + 15) >> 4);
      base[k + 1] = base[k] + (uint32_t)__builtin_amdgcn_readlane(inc[k], 63);
    }
  }
  const uint32_t H = base[4];
  if (H == 0) return;  // no keys at all: the merge writes the zero rows
  const uint32_t Q = (H + W - 1) / W;
  uint32_t a = blockIdx.x * Q;
  const uint32_t e = min(a + Q, H);
  while (a < e) {
    // the request holding block a: its chunk, then its lane
    const int k = a < base[1] ? 0 : a < base[2] ? 1 : a < base[3] ? 2 : 3;
    const int lk = k == 0 ? len[0] : k == 1 ? len[1] : k == 2 ? len[2] : len[3];
    const int ik = k == 0 ? inc[0] : k == 1 ? inc[1] : k == 2 ? inc[2] : inc[3];
    const uint32_t bk = k == 0 ? base[0] : k == 1 ? base[1] : k == 2 ? base[2] : base[3];
    const uint64_t hit = __ballot((uint32_t)ik > a - bk);
    const int lr = (int)__builtin_ctzll(hit);
    const int n = __builtin_amdgcn_readlane(lk, lr);  // > 0: block a lies in it
    const uint32_t nb = (uint32_t)((n + 15) >> 4);
    const uint32_t rbase = bk + (uint32_t)__builtin_amdgcn_readlane(ik, lr) - nb;
    const uint32_t send = min(e, rbase + nb);
    const int r = 64 * k + lr;
    const int row = (int)((uint32_t)r + a / Q);
    Piece pc;
    pc.r = r;
    pc.kvh = kvh;
    pc.n = n;
    pc.t0 = (int)(a - rbase) * 16;
    pc.t1 = min((int)(send - rbase) * 16, n);
    pc.id = row * hkv + kvh;
    if (pc.t0 == 0 && threadIdx.x == 0) {
      p.bal_table[2 * r] = row;
      p.bal_table[2 * r + 1] = (int)((rbase + nb - 1) / Q - rbase / Q + 1);
    }
    decode_split_unit<D, G, 1, false, true>(p, 0, vlds_block, &pc);
    a = send;
  }
}

// The merge of a balanced launch: one wave per (request, query head).  A
// request without keys gets a zero row; a sequence that was one piece was
// written by it; otherwise its rows (first, count) are merged as in
// decode_combine_kernel.
template <int D, int G>
__global__ __launch_bounds__(256) void decode_combine_balanced_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;
  constexpr int KB = 16;  // rows whose o is in flight together
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (int64_t)p.num_seqs * p.num_q_heads) return;
  const int r = (int)(rh / p.num_q_heads);
  const int qh = (int)(rh % p.num_q_heads);
  const int kvh = qh / G, hc = qh % G;
  const int32_t* t = p.bal_table + 2 * (int64_t)r;
  int n = p.seq_lens[r];
  int first = t[0], count = t[1];
  n = uniform(n);
  uint16_t* out = p.out + ((int64_t)r * p.num_q_heads + qh) * D;
  if (min(n, p.max_seq_len) <= 0) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[lane + 64 * i] = 0;
    return;
  }
  const int ns = uniform(count);
  if (ns <= 1) return;  // written by its one piece
  // rows first .. first + count - 1, this KV head's partials of each
  const int64_t row0 = (int64_t)uniform(first) * p.num_kv_heads + kvh;
  const int64_t stride = (int64_t)p.num_kv_heads * G;  // floats between rows (m, l)
  const float* om = p.bal_m + row0 * G + hc;
  const float* ol = p.bal_l + row0 * G + hc;
  const float* oo = p.bal_o + (row0 * G + hc) * D + lane;
  float M = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float y = s0 + lane < ns ? om[(int64_t)(s0 + lane) * stride] : kNegInf;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) y = fmaxf(y, __shfl_xor(y, off));
    M = fmaxf(M, y);
  }
  float L = 0.f, acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int sidx = s0 + lane;
    const float w = sidx < ns ? fast_exp2(om[(int64_t)sidx * stride] - M) : 0.f;
    float tl = sidx < ns ? ol[(int64_t)sidx * stride] * w : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tl += __shfl_xor(tl, off);
    L += tl;
    const int cnt = min(64, ns - s0);
    for (int k0 = 0; k0 < cnt; k0 += KB) {
      float v[KB][DPL];
#pragma unroll
      for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int i = 0; i < DPL; ++i)
          v[k][i] = k0 + k < cnt ? oo[(int64_t)(s0 + k0 + k) * stride * D + 64 * i] : 0.f;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (k0 + k < cnt) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k0 + k));
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[i] = fmaf(v[k][i], wk, acc[i]);
        }
      }
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < DPL; ++i) out[lane + 64 * i] = to_bf16(acc[i] * inv);
}

// The split kernel for batches with shared prefixes: the grid's first
// x.items workgroups run the shared-prefix pass (one item each), the rest
// the units of each request's remaining tokens, four KV heads per
// workgroup.  Both kinds are in flight together, and their partials go to
// disjoint slots of the workspace.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void decode_split_prefix_kernel(DecodeParams p,
                                                                     pkv_prefix::Params x) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_block[];
  if (blockIdx.x < (uint32_t)x.items) {
    pkv_prefix::prefix_item<D, D == 64 ? 2 : 1, G>(x, blockIdx.x, lds_block, (int)threadIdx.x);
    return;
  }
  decode_split_unit<D, G, 1, true>(p, blockIdx.x - (uint32_t)x.items, lds_block);
}

// The shared-prefix pass alone (for KV head counts the combined kernel's
// four-head workgroups do not fit), before the split kernel on one stream.
template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefix_pass_kernel(pkv_prefix::Params x) {
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_block[];
  pkv_prefix::prefix_item<D, D == 64 ? 2 : 1, G>(x, blockIdx.x, lds_block, (int)threadIdx.x);
}

// The loads of a batch of splits do not depend on the request length: the
// partials of a batch of KB splits are read at once (in bounds of the
// workspace; stale entries past the request's last split are never used),
// so a request of up to KB splits costs one memory round trip, not a chain
// of them.  KB is 16, or 64 when the host bound allows more than 16 splits
// (long requests): fewer, larger batches keep more bytes in flight for the
// few waves such batches have.
template <int D, int G, int KB>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  constexpr int DPL = D / 64;  // output dims per lane
  const int QL = p.q_len;
  const int NC = G * QL;  // partial columns per (request, KV head, split)
  const int lane = threadIdx.x & 63;
  // one wave per (request, query token, query head)
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (int64_t)p.num_seqs * QL * p.num_q_heads) return;
  const int r = (int)(rh / ((int64_t)QL * p.num_q_heads));
  const int rem = (int)(rh % ((int64_t)QL * p.num_q_heads));
  const int tq = rem / p.num_q_heads;
  const int qh = rem % p.num_q_heads;
  const int kvh = qh / G, h = qh % G;
  const int x = tq * G + h;  // column
  const int nsm = p.n_split_max;
  const int64_t sbase = ((int64_t)r * p.num_kv_heads + kvh) * nsm;  // split 0
  const float* om = p.ws_m + sbase * NC + x;
  const float* ol = p.ws_l + sbase * NC + x;
  const float* oo = p.ws_o + (sbase * NC + x) * D + lane;

  int n = p.seq_lens[r];
  int skip_raw = p.skip != nullptr ? p.skip[r] : 0;
  // First batch of partials, issued together with the length.  With a
  // device-chosen split the units fit one round, so requests have few
  // splits: only 8 are fetched ahead (the bound nsm, from the host split,
  // can be far above the real count), the rest once the count is known.
  const int pre = min(nsm, p.round_units > 0 ? 8 : KB);
  float mv = lane < nsm ? om[(int64_t)lane * NC] : kNegInf;
  float lv = lane < nsm ? ol[(int64_t)lane * NC] : 0.f;
  float v[KB][DPL];
#pragma unroll
  for (int k = 0; k < KB; ++k)
#pragma unroll
    for (int i = 0; i < DPL; ++i) v[k][i] = k < pre ? oo[(int64_t)k * NC * D + 64 * i] : 0.f;

  n = uniform(n);
  n = n > p.max_seq_len ? p.max_seq_len : n;
  if (n <= 0) return;
  const int skip = skip_tokens(p, uniform(skip_raw), n);
  const int sl = p.round_units > 0 ? uniform(*p.ws_split) : p.split;  // as the split kernel used
  // partials: those of the shared-prefix pass, then one per split of the rest
  const int ns = prefix_slots(p, skip) + (n - skip + sl - 1) / sl;
  if (ns == 1 && skip == 0) return;  // written by the split kernel

  // Global max over the splits (lane s holds split s, 64 at a time).
  float M = kNegInf;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    float y = s0 + lane < ns ? (s0 == 0 ? mv : om[(int64_t)(s0 + lane) * NC]) : kNegInf;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) y = fmaxf(y, __shfl_xor(y, off));
    M = fmaxf(M, y);
  }
  // (a multi-token row with no visible key: every m is -inf, every l is 0)
  if (M == kNegInf) M = 0.f;
  float L = 0.f, acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int s = s0 + lane;
    const float ms = s < ns ? (s0 == 0 ? mv : om[(int64_t)s * NC]) : kNegInf;
    const float w = s < ns ? fast_exp2(ms - M) : 0.f;
    float t = s < ns ? (s0 == 0 ? lv : ol[(int64_t)s * NC]) * w : 0.f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off);
    L += t;
    // lane = output dim; the weights of the 64 splits are broadcast by readlane
    const int cnt = min(64, ns - s0);
    for (int k0 = 0; k0 < cnt; k0 += KB) {
      // later batches load now; the first came with the length, unless it
      // holds more splits than were fetched ahead (then it is read again)
      if (s0 + k0 != 0 || min(cnt, KB) > pre) {
#pragma unroll
        for (int k = 0; k < KB; ++k)
#pragma unroll
          for (int i = 0; i < DPL; ++i)
            v[k][i] = k0 + k < cnt ? oo[(int64_t)(s0 + k0 + k) * NC * D + 64 * i] : 0.f;
      }
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        if (k0 + k < cnt) {
          const float wk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), k0 + k));
#pragma unroll
          for (int i = 0; i < DPL; ++i) acc[i] = fmaf(v[k][i], wk, acc[i]);
        }
      }
    }
  }
  uint16_t* out = p.out + (((int64_t)r * QL + tq) * p.num_q_heads + qh) * D;
  const float inv = L == 0.f ? 0.f : 1.f / L;
#pragma unroll
  for (int i = 0; i < DPL; ++i) out[lane + 64 * i] = to_bf16(acc[i] * inv);
}

// ---- host side -------------------------------------------------------------

// Automatic split: halve from one split per request until there are at
// least kTargetUnits (request, KV head, split) units or splits reach
// kMinAutoSplit tokens -- enough waves to keep HBM busy through the tail.
constexpr int64_t kTargetUnits = 16384;
constexpr int kMinAutoSplit = 128;

int32_t choose_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                     int32_t split_tokens) {
  if (split_tokens != 0) return split_tokens;
  int64_t s = ((int64_t)max_seq_len + 15) / 16 * 16;
  const int64_t rk = (int64_t)num_seqs * num_kv_heads;
  while (s > kMinAutoSplit && rk * (((int64_t)max_seq_len + s - 1) / s) < kTargetUnits)
    s = (s / 2 + 15) / 16 * 16;
  return (int32_t)std::min<int64_t>(s, (int64_t)1 << 30);
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Layout of the balanced launch's partial rows (decode_balanced_kernel) in
// the same workspace as the split layout (a call uses one of the two),
// after the first 256 bytes: B + kBalMaxWaves / Hkv rows of Hkv x g
// columns, then the (first row, count) table per request.  Only for batches of at
// most kBalMaxSeqs requests and 8 KV heads whose tokens count well below
// 2^31.
struct BalLayout {
  size_t m, l, o, table, total;
};
bool bal_eligible(int64_t num_seqs, int64_t num_q_heads, int64_t num_kv_heads, int64_t head_dim,
                  int64_t max_seq_len) {
  return num_seqs >= 1 && num_seqs <= kBalMaxSeqs && num_kv_heads <= 8 &&
         num_q_heads <= 8 * num_kv_heads && head_dim <= 128 &&
         num_seqs * max_seq_len + 16 * (int64_t)kBalMaxWaves < ((int64_t)1 << 31);
}
BalLayout bal_layout(int64_t num_seqs, int64_t num_kv_heads, int64_t g, int64_t d) {
  const int64_t rows = num_seqs * num_kv_heads + kBalMaxWaves;
  BalLayout b;
  b.m = 256;
  b.l = b.m + align256(rows * g * sizeof(float));
  b.o = b.l + align256(rows * g * sizeof(float));
  b.table = b.o + align256(rows * g * d * sizeof(float));
  b.total = b.table + align256(num_seqs * 2 * sizeof(int32_t));
  return b;
}

struct WsLayout {
  size_t m, l, o, split, total;
};

// ncols = query columns per (request, KV head): g * q_len.  total == 0
// when the partials would take more than 2^46 bytes (no such call is valid).
WsLayout ws_layout(int64_t rk, int64_t nsm, int64_t ncols, int d) {
  WsLayout w = {};
  const __int128 o_bytes = (__int128)rk * nsm * ncols * d * (int64_t)sizeof(float);
  if (rk < 0 || nsm < 0 || ncols < 0 || d < 0 || o_bytes > ((__int128)1 << 46)) return w;
  w.split = 0;  // first 256 bytes: the split the split kernel used
  w.m = 256;
  w.l = w.m + align256(rk * nsm * ncols * sizeof(float));
  w.o = w.l + align256(rk * nsm * ncols * sizeof(float));
  w.total = w.o + align256(rk * nsm * ncols * d * sizeof(float));
  return w;
}

// Query tokens per request handled by one multi-token launch; longer query
// runs are prefill's shape.
constexpr int kMaxQueryLen = 16;

// Query tokens per block for q_len tokens and g heads per KV head: the
// smallest power of two >= q_len, capped so that g * LQ fits the 16 MFMA
// columns.
int query_tile(int q_len, int g) {
  int lq = 1;
  while (lq < q_len) lq *= 2;
  return lq * g > 16 ? 16 / g : lq;
}

bool decode_shape_ok(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t max_seq_len, int32_t split_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_seq_len <= 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  if (head_dim <= 0) return false;
  if (split_tokens != 0 && (split_tokens < 16 || split_tokens > 65536 || split_tokens % 16))
    return false;
  return true;
}

// Waves of decode_split_kernel<D, G, LQ> resident on the current device at
// once with hpb waves per workgroup (occupancy x CUs, cached per device).
template <int D, int G, int LQ, bool BALANCED = false>
int resident_waves(int hpb) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices][4];  // by log2(hpb)
  const void* kernel = BALANCED ? reinterpret_cast<const void*>(decode_balanced_kernel<D, G>)
                                : reinterpret_cast<const void*>(decode_split_kernel<D, G, LQ>);
  constexpr size_t kWaveLds = (size_t)DecodeTraits<D, G>::NBUF * 16 * (D + 8) * sizeof(uint16_t);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  const int slot = hpb >= 8 ? 3 : hpb >= 4 ? 2 : hpb - 1;
  if (dev < kMaxDevices) {
    const int c = cache[dev][slot].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * hpb, kWaveLds * hpb) !=
      hipSuccess)
    return 0;
  const int n = cus * per_cu * hpb;
  if (n > 0 && dev < kMaxDevices) cache[dev][slot].store(n, std::memory_order_relaxed);
  return n;
}

// Resident waves of decode_split_prefix_kernel<D, G> (four-wave workgroups)
// on the current device, cached per device.
template <int D, int G>
int resident_waves_shared() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  constexpr size_t kWaveLds = (size_t)DecodeTraits<D, G>::NBUF * 16 * (D + 8) * sizeof(uint16_t);
  const size_t lds = std::max(kWaveLds * 4, pkv_prefix::item_lds_bytes<D>());
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(decode_split_prefix_kernel<D, G>), 256, lds) !=
      hipSuccess)
    return 0;
  const int n = cus * per_cu * 4;
  if (n > 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// With `x` (a shared-prefix pass, single-token queries, Hkv a multiple of
// four) the split kernel is decode_split_prefix_kernel: x->items workgroups
// of the pass ahead of the units, four KV heads per workgroup.
template <int D, int G, int LQ>
int launch_decode(DecodeParams p, int64_t waves, hipStream_t s,
                  const pkv_prefix::Params* x = nullptr) {
  constexpr size_t kWaveLds = (size_t)DecodeTraits<D, G>::NBUF * 16 * (D + 8) * sizeof(uint16_t);
  // KV heads per workgroup: adjacent heads' slices of every token row are
  // read by one CU at the same time.  Four when Hkv allows; eight when one
  // round of workgroups covers every unit (no workgroup then waits for a
  // CU, so none is held back by a slow wave of a large workgroup), while
  // with several rounds eight per workgroup is slower than four.
  const int hkv = p.num_kv_heads;
  const bool shared = LQ == 1 && x != nullptr;
  int hpb = hkv % 4 == 0 ? 4 : hkv % 2 == 0 ? 2 : 1;
  int64_t blocks = waves / hpb;
  if (p.round_units < 0) {
    // Units per KV head and query slice that one round of resident waves
    // holds.  Use the device's split choice only when even max-length
    // requests need at most 4 rounds at the host split; then one round of
    // workgroups covers every unit it can produce.
    const int hpb1 = hkv % 8 == 0 && !shared ? 8 : hpb;
    const int64_t per_unit = (int64_t)hkv * (LQ == 1 ? 1 : p.q_slices);
    const int64_t T =
        (shared ? resident_waves_shared<D, G>() : resident_waves<D, G, LQ>(hpb1)) / per_unit;
    const int64_t worst = (int64_t)p.num_seqs * p.n_unit_splits;  // units per head, host split
    if (T > 0 && p.num_seqs <= T && worst <= 4 * T) {
      p.round_units = (int32_t)T;
      hpb = hpb1;
      blocks = std::min<int64_t>(waves / hpb, T * per_unit / hpb);
    } else {
      p.round_units = 0;
    }
  }
  if (blocks > INT32_MAX) return PKV_EINVAL;
  p.heads_per_block = hpb;
  int st;
  if constexpr (LQ == 1) {
    if (shared) {
      if (hpb != 4 || blocks + x->items > INT32_MAX) return PKV_EINVAL;
      const size_t lds = std::max(kWaveLds * 4, pkv_prefix::item_lds_bytes<D>());
      DecodeParams pp = p;
      pkv_prefix::Params xx = *x;
      void* args[] = {&pp, &xx};
      st = hipLaunchKernel(reinterpret_cast<const void*>(decode_split_prefix_kernel<D, G>),
                           dim3((unsigned)(blocks + x->items)), dim3(256), args, lds, s) ==
                   hipSuccess
               ? PKV_OK
               : PKV_EHIP;
    } else if (p.skip != nullptr) {
      st = pkv_host::launch(decode_split_kernel<D, G, 1, true>, dim3((unsigned)blocks),
                            dim3(64 * p.heads_per_block), s, p, kWaveLds * p.heads_per_block);
    } else if (p.auto_split && p.round_units == 0 && p.bal_table != nullptr && hkv <= 8 &&
               !(hkv & (hkv - 1)) &&
               resident_waves<D, G, 1, true>(hkv) > 0 &&
               blocks * hpb > resident_waves<D, G, 1, true>(hkv)) {
      // several rounds of units: one round of workgroups (a wave per KV
      // head) sharing the work exactly
      DecodeParams pb = p;
      pb.ws_m = p.bal_m;
      pb.ws_l = p.bal_l;
      pb.ws_o = p.bal_o;
      pb.heads_per_block = hkv;
      const int64_t nblk = std::min(resident_waves<D, G, 1, true>(hkv), kBalMaxWaves) / hkv;
      st = pkv_host::launch(decode_balanced_kernel<D, G>, dim3((unsigned)nblk),
                            dim3(64 * hkv), s, pb, kWaveLds * hkv);
      if (st != PKV_OK) return st;
      const int64_t cb = ((int64_t)p.num_seqs * p.num_q_heads + 3) / 4;
      return pkv_host::launch(decode_combine_balanced_kernel<D, G>, dim3((unsigned)cb), dim3(256),
                              s, pb);
    } else {
      st = pkv_host::launch(decode_split_kernel<D, G, LQ>, dim3((unsigned)blocks),
                            dim3(64 * p.heads_per_block), s, p, kWaveLds * p.heads_per_block);
    }
  } else {
    st = pkv_host::launch(decode_split_kernel<D, G, LQ>, dim3((unsigned)blocks),
                          dim3(64 * p.heads_per_block), s, p, kWaveLds * p.heads_per_block);
  }
  if (st != PKV_OK || p.n_split_max <= 1) return st;
  const int64_t cblocks = ((int64_t)p.num_seqs * p.q_len * p.num_q_heads + 3) / 4;
  if (p.n_split_max > 16)
    return pkv_host::launch(decode_combine_kernel<D, G, 64>, dim3((unsigned)cblocks), dim3(256),
                            s, p);
  return pkv_host::launch(decode_combine_kernel<D, G, 16>, dim3((unsigned)cblocks), dim3(256), s,
                          p);
}

template <int D, int G>
int launch_decode_lq(const DecodeParams& p, int lq, int64_t waves, hipStream_t s,
                     const pkv_prefix::Params* x = nullptr) {
  switch (lq) {
    case 1: return launch_decode<D, G, 1>(p, waves, s, x);
    case 2: return launch_decode<D, G, 2>(p, waves, s);
    case 4:
      if constexpr (G <= 4) return launch_decode<D, G, 4>(p, waves, s);
      break;
    case 8:
      if constexpr (G <= 2) return launch_decode<D, G, 8>(p, waves, s);
      break;
    case 16:
      if constexpr (G == 1) return launch_decode<D, G, 16>(p, waves, s);
      break;
  }
  return PKV_EUNSUPPORTED;
}

}  // namespace

extern "C" int32_t pkv_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t max_seq_len, int32_t split_tokens) {
  if (num_seqs < 0 || num_kv_heads <= 0 || max_seq_len <= 0) return 0;
  if (split_tokens != 0 && (split_tokens < 16 || split_tokens > 65536 || split_tokens % 16))
    return 0;
  return choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim,
                                             int32_t max_seq_len, int32_t split_tokens) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       split_tokens))
    return 0;
  const int32_t s = choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
  const int64_t nsm = ((int64_t)max_seq_len + s - 1) / s;
  if (nsm <= 1 || num_seqs == 0) return 0;
  const size_t split_total =
      ws_layout((int64_t)num_seqs * num_kv_heads, nsm, num_q_heads / num_kv_heads, head_dim)
          .total;
  if (split_total == 0 ||
      !bal_eligible(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len))
    return split_total;
  return std::max(split_total, bal_layout(num_seqs, num_kv_heads, num_q_heads / num_kv_heads,
                                          head_dim)
                                   .total);
}

extern "C" size_t pkv_decode_multi_workspace_bytes(int32_t num_seqs, int32_t q_len,
                                                   int32_t num_q_heads, int32_t num_kv_heads,
                                                   int32_t head_dim, int32_t max_seq_len,
                                                   int32_t split_tokens) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       split_tokens))
    return 0;
  if (q_len < 1 || q_len > kMaxQueryLen) return 0;
  const int32_t s = choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
  const int64_t nsm = ((int64_t)max_seq_len + s - 1) / s;
  if (nsm <= 1 || num_seqs == 0) return 0;
  return ws_layout((int64_t)num_seqs * num_kv_heads, nsm,
                   (int64_t)q_len * (num_q_heads / num_kv_heads), head_dim)
      .total;
}

// ---- decode step without a caller workspace ----------------------------------
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops): the split partials live in a fixed array
// of this library instead of a caller workspace.  Each GPU the library runs
// on holds its own copy until the process ends.  Its address is looked up
// once per device with that device current and kept; the array's name is a
// host-side stand-in and is never passed to a kernel.

constexpr size_t kScratchBytes = size_t(32) << 20;  // 32 MiB per device
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of this device's copy of `scratch` (null if it cannot be
// found).  Looked up on the first call on each device.
void* scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = ptrs[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  ptrs[dev].store(p, std::memory_order_release);  // every thread finds the same address
  return p;
}

}  // namespace

namespace {

// Requests grouped by shared cached prefix (pkv_paged_attn_decode_shared).
struct SharedGroups {
  const int32_t* cu_groups;    // [num_groups + 1]
  const int32_t* shared_lens;  // [num_seqs]
  int32_t num_groups;
  int32_t max_group_size;
  int32_t max_shared_len;
};

template <int D, int G>
int launch_prefix_kernel(const pkv_prefix::Params& x, hipStream_t s) {
  pkv_prefix::Params xx = x;
  void* args[] = {&xx};
  return hipLaunchKernel(reinterpret_cast<const void*>(prefix_pass_kernel<D, G>),
                         dim3((unsigned)x.items), dim3(256), args,
                         pkv_prefix::item_lds_bytes<D>(), s) == hipSuccess
             ? PKV_OK
             : PKV_EHIP;
}

int launch_prefix_pass(const pkv_prefix::Params& x, int head_dim, int g, hipStream_t s) {
  if (head_dim == 64) {
    if (g == 1) return launch_prefix_kernel<64, 1>(x, s);
    if (g == 2) return launch_prefix_kernel<64, 2>(x, s);
    if (g == 4) return launch_prefix_kernel<64, 4>(x, s);
    return launch_prefix_kernel<64, 8>(x, s);
  }
  if (g == 1) return launch_prefix_kernel<128, 1>(x, s);
  if (g == 2) return launch_prefix_kernel<128, 2>(x, s);
  if (g == 4) return launch_prefix_kernel<128, 4>(x, s);
  return launch_prefix_kernel<128, 8>(x, s);
}

int decode_impl(const void* q, const void* k_new, const void* v_new, const int32_t* out_loc,
                const void* k_cache, const void* v_cache, int32_t page_size, int64_t num_pages,
                const int32_t* page_table, int32_t page_table_stride, const int32_t* seq_lens,
                int32_t num_seqs, int32_t q_len, int32_t max_seq_len, int32_t num_q_heads,
                int32_t num_kv_heads,
                int32_t head_dim, float softmax_scale, int32_t split_tokens, void* out,
                void* workspace, size_t workspace_bytes, void* stream,
                bool use_scratch = false, const SharedGroups* groups = nullptr) {
  using namespace pkv_host;
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       split_tokens))
    return PKV_EINVAL;
  if (!finite_positive(softmax_scale)) return PKV_EINVAL;
  if (q_len < 1 || q_len > kMaxQueryLen) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out) return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PKV_EINVAL;
  const bool fused = k_new != nullptr || v_new != nullptr || out_loc != nullptr;
  if (fused && (q_len != 1 || !k_new || !v_new || !out_loc || !aligned16(k_new) ||
                !aligned16(v_new)))
    return PKV_EINVAL;
  if (num_pages <= 0 || page_table_stride <= 0) return PKV_EINVAL;
  if (!is_pow2_page(page_size)) return PKV_EUNSUPPORTED;
  if ((int64_t)page_table_stride * page_size < max_seq_len) return PKV_EINVAL;
  const int g = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (g != 1 && g != 2 && g != 4 && g != 8) return PKV_EUNSUPPORTED;

  const int32_t split = choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
  const int64_t nsm = ((int64_t)max_seq_len + split - 1) / split;
  // partial slots of the shared-prefix pass, ahead of the splits
  const int64_t nks = groups == nullptr ? 0
                                        : ((int64_t)(groups->max_shared_len & ~15) +
                                           pkv_prefix::kSplit - 1) / pkv_prefix::kSplit;
  const int64_t slots = nks + nsm;
  const int64_t rk = (int64_t)num_seqs * num_kv_heads;
  const int lq = query_tile(q_len, g);
  const int slices = (q_len + lq - 1) / lq;
  DecodeParams p = {};
  if (slots > 1) {
    const WsLayout w = ws_layout(rk, slots, (int64_t)g * q_len, head_dim);
    if (w.total == 0) return PKV_EINVAL;  // partials beyond any device memory
    if (use_scratch) {  // the library's fixed scratch instead of a caller workspace
      workspace_bytes = kScratchBytes;
      if (workspace_bytes < w.total) return PKV_ENOSPACE;
      workspace = scratch_on_current_device();
      if (workspace == nullptr) return PKV_EHIP;
    }
    if (workspace_bytes < w.total) return PKV_ENOSPACE;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return PKV_EINVAL;
    char* ws = static_cast<char*>(workspace);
    p.ws_m = reinterpret_cast<float*>(ws + w.m);
    p.ws_l = reinterpret_cast<float*>(ws + w.l);
    p.ws_o = reinterpret_cast<float*>(ws + w.o);
    p.ws_split = reinterpret_cast<int32_t*>(ws + w.split);
    if (q_len == 1 && groups == nullptr &&
        bal_eligible(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len)) {
      const BalLayout b = bal_layout(num_seqs, num_kv_heads, g, head_dim);
      if (workspace_bytes >= b.total) {
        p.bal_m = reinterpret_cast<float*>(ws + b.m);
        p.bal_l = reinterpret_cast<float*>(ws + b.l);
        p.bal_o = reinterpret_cast<float*>(ws + b.o);
        p.bal_table = reinterpret_cast<int32_t*>(ws + b.table);
      }
    }
  }
  // One wave per (request, split) pair, KV head and query slice: at most
  // this many waves, those past the pairs that exist exit at once.
  const int64_t waves = rk * nsm * slices;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.out = static_cast<uint16_t*>(out);
  if (fused) {
    p.k_new = static_cast<const uint16_t*>(k_new);
    p.v_new = static_cast<const uint16_t*>(v_new);
    p.out_loc = out_loc;
    p.k_pool = const_cast<uint16_t*>(p.k_cache);
    p.v_pool = const_cast<uint16_t*>(p.v_cache);
    p.num_slots = num_pages * page_size;
  }
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.page_shift = log2_exact(page_size);
  p.pt_stride = page_table_stride;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_seq_len = max_seq_len;
  p.split = split;
  p.n_split_max = (int32_t)slots;
  p.n_unit_splits = (int32_t)nsm;
  // Device-chosen split (see device_split): only for the automatic split and
  // batches that need few rounds even at the longest length.
  p.round_units = split_tokens == 0 && num_seqs <= 256 ? -1 : 0;
  p.auto_split = split_tokens == 0;
  p.q_len = q_len;
  p.q_slices = slices;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  pkv_prefix::Params x = {};
  const pkv_prefix::Params* xp = nullptr;
  if (groups != nullptr) {
    // The shared-prefix pass fills slots 0 .. nks-1; the units of each
    // request's remaining tokens the slots after them.  With four or more
    // KV heads (a multiple of four) both run in one launch of the combined
    // split kernel, else the pass runs first as a kernel of its own.  (The
    // pass alone on a second stream, forked and joined with events,
    // measured slower than one stream: 51.8 against 37.7 us on the
    // shared-prefix batch.)
    p.skip = groups->shared_lens;
    p.ksplit = pkv_prefix::kSplit;
    // A shared length above max_shared_len (a device value, not checked on
    // the host) is cut to it, so a request's partial slots stay among the
    // nks + nsm sized above.
    p.max_skip = groups->max_shared_len;
    if (nks > 0) {
      const int nb = head_dim == 64 ? 2 : 1;
      const int qtile = 128 * nb / g;
      const int64_t page_bytes = (int64_t)page_size * num_kv_heads * head_dim * 2;
      if (page_bytes >= ((int64_t)1 << 32)) return PKV_EUNSUPPORTED;
      x.q = p.q;
      x.cu_groups = groups->cu_groups;
      x.shared_lens = groups->shared_lens;
      x.k_cache = p.k_cache;
      x.v_cache = p.v_cache;
      x.page_table = page_table;
      x.ws_m = p.ws_m;
      x.ws_l = p.ws_l;
      x.ws_o = p.ws_o;
      x.num_groups = groups->num_groups;
      x.num_seqs = num_seqs;
      x.max_group_size = groups->max_group_size;
      x.max_shared_len = groups->max_shared_len;
      x.page_size = page_size;
      x.page_shift = p.page_shift;
      x.pt_stride = page_table_stride;
      x.num_q_heads = num_q_heads;
      x.num_kv_heads = num_kv_heads;
      x.n_qtiles = (groups->max_group_size + qtile - 1) / qtile;
      x.ksplit = pkv_prefix::kSplit;
      x.slots = (int32_t)slots;
      const int64_t items = nks * x.n_qtiles * (int64_t)groups->num_groups * num_kv_heads;
      if (items > INT32_MAX / 2) return PKV_EINVAL;
      x.items = (int32_t)items;
      x.num_pages_u32 = (uint32_t)std::min<int64_t>(num_pages, INT32_MAX);
      x.page_bytes = (uint32_t)page_bytes;
      x.row_bytes = (uint32_t)(num_kv_heads * head_dim * 2);
      x.scale_log2 = p.scale_log2;
      if (num_kv_heads % 4 == 0) {
        xp = &x;
      } else if (x.items > 0) {
        const int st = launch_prefix_pass(x, head_dim, g, s);
        if (st != PKV_OK) return st;
      }
    }
  }
  if (head_dim == 64) {
    if (g == 1) return launch_decode_lq<64, 1>(p, lq, waves, s, xp);
    if (g == 2) return launch_decode_lq<64, 2>(p, lq, waves, s, xp);
    if (g == 4) return launch_decode_lq<64, 4>(p, lq, waves, s, xp);
    return launch_decode_lq<64, 8>(p, lq, waves, s, xp);
  }
  if (g == 1) return launch_decode_lq<128, 1>(p, lq, waves, s, xp);
  if (g == 2) return launch_decode_lq<128, 2>(p, lq, waves, s, xp);
  if (g == 4) return launch_decode_lq<128, 4>(p, lq, waves, s, xp);
  return launch_decode_lq<128, 8>(p, lq, waves, s, xp);
}

}  // namespace

extern "C" int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                     int32_t page_size, int64_t num_pages,
                                     const int32_t* page_table, int32_t page_table_stride,
                                     const int32_t* seq_lens, int32_t num_seqs,
                                     int32_t max_seq_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     float softmax_scale, int32_t split_tokens, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, nullptr, nullptr, nullptr, k_cache, v_cache, page_size, num_pages,
                     page_table, page_table_stride, seq_lens, num_seqs, 1, max_seq_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale, split_tokens, out,
                     workspace, workspace_bytes, stream);
}

extern "C" int pkv_decode_step(const void* q, const void* k_new, const void* v_new,
                               const int32_t* out_loc, void* k_cache, void* v_cache,
                               int32_t page_size, int64_t num_pages, const int32_t* page_table,
                               int32_t page_table_stride, const int32_t* seq_lens,
                               int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, float softmax_scale,
                               int32_t split_tokens, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !out_loc)) return PKV_EINVAL;
  return decode_impl(q, k_new, v_new, out_loc, k_cache, v_cache, page_size, num_pages,
                     page_table, page_table_stride, seq_lens, num_seqs, 1, max_seq_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale, split_tokens, out,
                     workspace, workspace_bytes, stream);
}

extern "C" int pkv_paged_attn_decode_multi(const void* q, int32_t q_len, const void* k_cache,
                                           const void* v_cache, int32_t page_size,
                                           int64_t num_pages, const int32_t* page_table,
                                           int32_t page_table_stride, const int32_t* seq_lens,
                                           int32_t num_seqs, int32_t max_seq_len,
                                           int32_t num_q_heads, int32_t num_kv_heads,
                                           int32_t head_dim, float softmax_scale,
                                           int32_t split_tokens, void* out, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return decode_impl(q, nullptr, nullptr, nullptr, k_cache, v_cache, page_size, num_pages,
                     page_table, page_table_stride, seq_lens, num_seqs, q_len, max_seq_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale, split_tokens, out,
                     workspace, workspace_bytes, stream);
}

extern "C" size_t pkv_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int pkv_decode_step_noalloc(const void* q, const void* k_new, const void* v_new,
                                       const int32_t* out_loc, void* k_cache, void* v_cache,
                                       int32_t page_size, int64_t num_pages,
                                       const int32_t* page_table, int32_t page_table_stride,
                                       const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t max_seq_len, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       float softmax_scale, int32_t split_tokens, void* out,
                                       void* stream) {
  // Validated exactly as pkv_decode_step; the scratch's address is looked up
  // only once every argument has passed and the partials fit.
  if (num_seqs > 0 && (!k_new || !v_new || !out_loc)) return PKV_EINVAL;
  return decode_impl(q, k_new, v_new, out_loc, k_cache, v_cache, page_size, num_pages,
                     page_table, page_table_stride, seq_lens, num_seqs, 1, max_seq_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale, split_tokens, out,
                     nullptr, 0, stream, /*use_scratch=*/true);
}

// ---- decode-step graphs, one per batch-size bucket ---------------------------
//
// The engines capture the decode step once per batch-size bucket and, at
// every step, replay the smallest captured graph that holds the batch, with
// the batch copied into the first rows of fixed buffers and the rows past it
// padded by a dummy request (miniVLLM "Engine Architecture", CUDA graph
// capture and run_model; mini-sglang "Engine Class", CUDA graph batch sizes
// and the dummy request).  Here a graph holds one pkv_decode_step (or one
// pkv_paged_attn_decode) over the first `bucket` rows of the caller's fixed
// buffers; every bucket shares one workspace, sized for the bucket that
// needs most, or the library's fixed scratch.

struct pkv_decode_graphs {
  int device;
  int count;
  int32_t bucket[64];         // ascending
  hipGraphExec_t exec[64];
};

namespace {

constexpr int kMaxGraphBuckets = 64;

// Occupancy queries are made (and cached) before capture, so nothing but
// kernel launches happens while the capture stream records.
template <int D, int G>
void prime_decode_occupancy() {
  for (int hpb : {1, 2, 4, 8}) (void)resident_waves<D, G, 1>(hpb);
}

void prime_occupancy(int head_dim, int g) {
  if (head_dim == 64) {
    if (g == 1) prime_decode_occupancy<64, 1>();
    else if (g == 2) prime_decode_occupancy<64, 2>();
    else if (g == 4) prime_decode_occupancy<64, 4>();
    else if (g == 8) prime_decode_occupancy<64, 8>();
  } else if (head_dim == 128) {
    if (g == 1) prime_decode_occupancy<128, 1>();
    else if (g == 2) prime_decode_occupancy<128, 2>();
    else if (g == 4) prime_decode_occupancy<128, 4>();
    else if (g == 8) prime_decode_occupancy<128, 8>();
  }
}

void destroy_graphs(pkv_decode_graphs* g) {
  if (g == nullptr) return;
  for (int i = 0; i < g->count; ++i)
    if (g->exec[i] != nullptr) (void)hipGraphExecDestroy(g->exec[i]);
  delete g;
}

}  // namespace

extern "C" size_t pkv_decode_graphs_workspace_bytes(const int32_t* buckets, int32_t num_buckets,
                                                    int32_t num_q_heads, int32_t num_kv_heads,
                                                    int32_t head_dim, int32_t max_seq_len) {
  if (buckets == nullptr || num_buckets <= 0 || num_buckets > kMaxGraphBuckets) return 0;
  size_t need = 0;
  for (int i = 0; i < num_buckets; ++i) {
    if (buckets[i] <= 0) return 0;  // as pkv_decode_graphs_create rejects it
    for (int j = 0; j < i; ++j)
      if (buckets[j] == buckets[i]) return 0;
    need = std::max(need, pkv_decode_workspace_bytes(buckets[i], num_q_heads, num_kv_heads,
                                                     head_dim, max_seq_len, 0));
  }
  return need;
}

extern "C" int pkv_decode_graphs_create(
    const int32_t* buckets, int32_t num_buckets, const void* q, const void* k_new,
    const void* v_new, const int32_t* out_loc, void* k_cache, void* v_cache, int32_t page_size,
    int64_t num_pages, const int32_t* page_table, int32_t page_table_stride,
    const int32_t* seq_lens, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
    pkv_decode_graphs** graphs) {
  if (graphs == nullptr) return PKV_EINVAL;
  *graphs = nullptr;
  if (buckets == nullptr || num_buckets <= 0 || num_buckets > kMaxGraphBuckets) return PKV_EINVAL;
  int32_t sorted[kMaxGraphBuckets];
  std::copy(buckets, buckets + num_buckets, sorted);
  std::sort(sorted, sorted + num_buckets);
  for (int i = 0; i < num_buckets; ++i)
    if (sorted[i] <= 0 || (i > 0 && sorted[i] == sorted[i - 1])) return PKV_EINVAL;
  const bool fused = k_new != nullptr || v_new != nullptr || out_loc != nullptr;
  if (fused && (!k_new || !v_new || !out_loc)) return PKV_EINVAL;
  if (!decode_shape_ok(sorted[num_buckets - 1], num_q_heads, num_kv_heads, head_dim,
                       max_seq_len, 0))
    return PKV_EINVAL;
  // One workspace for every bucket: the caller's, or the fixed scratch.
  const size_t need = pkv_decode_graphs_workspace_bytes(sorted, num_buckets, num_q_heads,
                                                        num_kv_heads, head_dim, max_seq_len);
  const bool use_scratch = workspace == nullptr && need > 0;
  if (use_scratch) {
    if (need > kScratchBytes) return PKV_ENOSPACE;
    if (scratch_on_current_device() == nullptr) return PKV_EHIP;
  } else if (need > 0 && workspace_bytes < need) {
    return PKV_ENOSPACE;
  }
  // Every argument check of the call, on the largest bucket, before capture.
  const int g = num_kv_heads > 0 ? num_q_heads / num_kv_heads : 0;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  prime_occupancy(head_dim, g);

  pkv_decode_graphs* set = new (std::nothrow) pkv_decode_graphs{};
  if (set == nullptr) return PKV_EHIP;
  set->device = dev;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
    delete set;
    return PKV_EHIP;
  }
  int status = PKV_OK;
  // Largest first, as the engines capture them.
  for (int i = num_buckets - 1; i >= 0 && status == PKV_OK; --i) {
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
      status = PKV_EHIP;
      break;
    }
    const int st = decode_impl(q, k_new, v_new, out_loc, k_cache, v_cache, page_size, num_pages,
                               page_table, page_table_stride, seq_lens, sorted[i], 1,
                               max_seq_len, num_q_heads, num_kv_heads, head_dim, softmax_scale,
                               0, out, workspace, use_scratch ? 0 : workspace_bytes, cs,
                               use_scratch);
    hipGraph_t graph = nullptr;
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    if (st != PKV_OK || e != hipSuccess || graph == nullptr) {
      status = st != PKV_OK ? st : PKV_EHIP;
      if (graph != nullptr) (void)hipGraphDestroy(graph);
      break;
    }
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (ei != hipSuccess || exec == nullptr) {
      status = PKV_EHIP;
      break;
    }
    set->bucket[i] = sorted[i];
    set->exec[i] = exec;
  }
  (void)hipStreamDestroy(cs);
  set->count = num_buckets;
  if (status != PKV_OK) {
    destroy_graphs(set);
    return status;
  }
  *graphs = set;
  return PKV_OK;
}

extern "C" int pkv_decode_graphs_replay(pkv_decode_graphs* graphs, int32_t num_seqs,
                                        void* stream, int32_t* bucket_used) {
  if (bucket_used != nullptr) *bucket_used = 0;
  if (graphs == nullptr || num_seqs < 0) return PKV_EINVAL;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PKV_EHIP;
  if (dev != graphs->device) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  int i = 0;
  while (i < graphs->count && graphs->bucket[i] < num_seqs) ++i;
  if (i == graphs->count) return PKV_EINVAL;  // larger than the largest bucket
  if (hipGraphLaunch(graphs->exec[i], static_cast<hipStream_t>(stream)) != hipSuccess)
    return PKV_EHIP;
  if (bucket_used != nullptr) *bucket_used = graphs->bucket[i];
  return PKV_OK;
}

extern "C" void pkv_decode_graphs_destroy(pkv_decode_graphs* graphs) { destroy_graphs(graphs); }

// ---- decode with shared prefixes read once per group ---------------------------

extern "C" size_t pkv_paged_attn_decode_shared_workspace_bytes(
    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    int32_t max_seq_len, int32_t max_shared_len, int32_t split_tokens) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       split_tokens) ||
      num_seqs == 0 || max_shared_len < 0 || max_shared_len > max_seq_len)
    return 0;
  const int32_t s = choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
  const int64_t slots = ((int64_t)(max_shared_len & ~15) + pkv_prefix::kSplit - 1) /
                            pkv_prefix::kSplit +
                        ((int64_t)max_seq_len + s - 1) / s;
  if (slots <= 1) return 0;
  return ws_layout((int64_t)num_seqs * num_kv_heads, slots, num_q_heads / num_kv_heads, head_dim)
      .total;
}

extern "C" int pkv_paged_attn_decode_shared(
    const void* q, const void* k_new, const void* v_new, const int32_t* out_loc, void* k_cache,
    void* v_cache, int32_t page_size, int64_t num_pages, const int32_t* page_table,
    int32_t page_table_stride, const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
    const int32_t* cu_groups, const int32_t* shared_lens, int32_t num_groups,
    int32_t max_group_size, int32_t max_shared_len, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float softmax_scale, int32_t split_tokens, void* out, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!cu_groups || !shared_lens)) return PKV_EINVAL;
  if (num_groups < 0 || (num_seqs > 0 && num_groups == 0) || num_groups > num_seqs)
    return PKV_EINVAL;
  if (max_group_size < 0 || max_group_size > num_seqs) return PKV_EINVAL;
  if (max_shared_len < 0 || max_shared_len > max_seq_len) return PKV_EINVAL;
  const SharedGroups groups = {cu_groups, shared_lens, num_groups, max_group_size,
                               max_shared_len};
  return decode_impl(q, k_new, v_new, out_loc, k_cache, v_cache, page_size, num_pages,
                     page_table, page_table_stride, seq_lens, num_seqs, 1, max_seq_len,
                     num_q_heads, num_kv_heads, head_dim, softmax_scale, split_tokens, out,
                     workspace, workspace_bytes, stream, false, &groups);
}
