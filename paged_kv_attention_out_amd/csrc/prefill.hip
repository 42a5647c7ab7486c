// Causal prefill attention with a cached prefix over a paged KV cache.
//
// Prefill feeds only the tokens after each request's cached prefix, as one
// flat ragged batch indexed by cu_seqlens_q (miniVLLM "Engine Architecture",
// prepare_prefill; zero-to-sglang Ch.1 section 3.3: extend length =
// sequence length - cached length).  New token i of request r is at
// absolute position P_r + i and sees keys 0 .. P_r + i.
//
// Work item = (query tile, request, KV head).  The block's 128*NB "columns"
// are (query head of the group, position) pairs, head-major, so the g query
// heads that share a KV head reuse every K/V tile staged in LDS; each wave
// owns NB blocks of 32 columns.
//
// The grid is persistent: as many 256-thread blocks as fit on the device at
// once, each pulling items from a counter in the caller's workspace, the
// longest key ranges first.  The hardware dispatcher starts
// blocks strictly in grid order, so a grid of one block per item leaves CUs
// idle behind long-running blocks; pulling keeps every resident block busy
// until the items run out.  A block draws its next ticket as the last tile
// of its current item ends, so the last (shortest) items go to the blocks
// that free up first.  The block that draws the last ticket puts the
// counter back to zero, ready for the next call on the same workspace.
//
// Per 64-key tile:
//   * K and V rows are fetched through the page table into registers three
//     tiles ahead (buffer loads at 32-bit offsets when a pool is at most
//     2 GiB) and written to LDS (row-major) one tile ahead, while the step's
//     QK^T MFMAs run.
//   * S^T = K Q^T with MFMA 32x32x16 bf16 (A = K from LDS, B = Q resident in
//     registers); lane l owns column l % 32, 32 keys of it per 32x32 block.
//   * Online softmax per column in base 2.  The first tile sets the
//     reference point; later tiles compute P against it speculatively and
//     are redone exactly only when a probability may exceed 2^kTau.  Tiles
//     left of the block's diagonal skip the mask.
//   * P (rounded to bf16, round-to-nearest-even) stays in registers: the
//     accumulator layout of S^T is already the B operand layout of
//     O^T += V^T P^T, with the key order permuted identically on both sides.
// Arithmetic per visible (query, key) pair: 4 * head_dim flops on MFMA.

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "pkv_common.h"

namespace {

using namespace pkv;

struct PrefillParams {
  const uint16_t* q;
  const int32_t* cu_seqlens;
  const int32_t* prefix_lens;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  uint16_t* out;
  uint32_t* counter;  // work-item counter (zero on entry, zero again on exit)
  int64_t num_pages;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_q_len;
  int32_t max_seq_len;
  int32_t page_size;
  int32_t page_shift;
  int32_t pt_stride;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t n_qtiles;
  int32_t n_items;
  int32_t longest_first;  // 1: tickets map to (request, query tile) pairs longest first
  uint32_t num_pages_u32;  // min(num_pages, 2^31 - 1); larger page numbers read its last page
  uint32_t page_bytes;     // bytes per page of one pool (K or V)
  uint32_t pool_bytes;     // bytes of one pool when they fit 32 bits (buffer loads), else 0
  uint32_t row_bytes;      // bytes per token row (all KV heads)
  float scale_log2;
};

constexpr size_t kPrefillWorkspaceBytes = 256;  // one counter, padded
constexpr float kTau = 8.0f;
// 2^kTau: a lane's row sum over a tile above it may hold a P above 2^kTau.
constexpr float kPmax = 256.0f;
static_assert(kPmax == (float)(1 << (int)kTau), "kPmax is 2^kTau");
constexpr int kKeys = 64;  // keys per tile
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle.
constexpr int kBufferFlags = 0x00020000;

// fmax over lanes l and l ^ 32 (the two halves of one 32x32 accumulator column).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of one column's 64 scores in a tile (both 32-key halves, both
// lane halves), as two v_max3 chains.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) {
    a = fmaxf(fmaxf(a, s[0][v]), s[0][v + 1]);
    b = fmaxf(fmaxf(b, s[1][v]), s[1][v + 1]);
  }
  return max_xor32(fmaxf(a, b));
}

// Request r's new tokens [s0, s0 + L) and cached prefix length P, clamped
// so every access stays inside the buffers.
__device__ __forceinline__ void request_geometry(const PrefillParams& p, int r, int& s0, int& L,
                                                 int& P) {
  int a = p.cu_seqlens[r], b = p.cu_seqlens[r + 1];
  a = min(max(a, 0), p.num_tokens);
  b = min(max(b, a), p.num_tokens);
  s0 = a;
  L = min(min(b - a, p.max_q_len), p.max_seq_len);
  P = min(max(p.prefix_lens[r], 0), p.max_seq_len - L);
}

template <int D, int NB, int G, bool BUF, typename KV>
__device__ __forceinline__ bool attend_item(const PrefillParams& p, int qt, int r, int kvh,
                                            int tid, int lane, int wave, KV& kv,
                                            uint32_t& next, const int (&geo)[3][64]);

// BUF: the pools are below 4 GiB and their pages and page numbers below 2^24,
// so rows are fetched by buffer loads at 32-bit offsets from the pool bases
// (one 24-bit multiply-add per row instead of 64-bit address arithmetic).
// A page id outside the pool is not clamped on this path: its offset, taken
// modulo 2^32 from the id's low 24 bits, either lies past the pool, where
// the load's range check returns zeros, or on other rows of the same pool.
template <int D, int NB, int G, bool BUF>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  constexpr int QT = 128 * NB / G;
  constexpr int TILE = kKeys * (D + 8);
  static_assert(QT >= 16 && QT % 16 == 0, "each 16-lane group stays within one query head");

  // [buffer][K or V][row * pitch + dim]: two tiles in flight, one barrier per tile.
  __shared__ __attribute__((aligned(16))) uint16_t kv[2][2][TILE];
  __shared__ uint32_t item_slot[2];
  __shared__ int geo[3][64];  // longest-first: first new token, new tokens, prefix per request

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rk_all = p.num_seqs * p.num_kv_heads;

  // Longest-first order (at most 64 requests, one per lane): query tile qt of
  // request r reads P_r + QT*(qt+1) keys, so it is put on level
  // P_r / QT + qt, and tickets walk the levels from the top; a level holds at
  // most one tile per request, taken in request order, each for every KV head
  // (consecutive tickets).  Without it, tickets go query tile by query tile
  // from the last, which leaves the tiles of long prefixes for the end.
  int lv_b = 0, lv_n = 0;     // this lane's request: first level, tile count
  int level = -1, below = 0;  // walk state: current level, tickets above it
  // Tickets at or past n_end end a block.  In longest-first order every
  // ticket below the tile count times the KV heads is a real item, so the
  // blocks stop there rather than draw the empty query tiles one by one.
  uint32_t n_end = (uint32_t)p.n_items;
  // Wave 0 also puts every request's geometry in LDS, so an item reads it
  // there instead of making a round trip to memory.
  if (p.longest_first) {
    if (lane < p.num_seqs) {
      int s0r, Lr, Pr;
      request_geometry(p, lane, s0r, Lr, Pr);
      if (wave == 0) {
        geo[0][lane] = s0r;
        geo[1][lane] = Lr;
        geo[2][lane] = Pr;
      }
      lv_b = Pr / QT;
      lv_n = (Lr + QT - 1) / QT;
    }
    int top = lv_n > 0 ? lv_b + lv_n - 1 : -1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) top = max(top, __shfl_xor(top, off));
    level = uniform(top);
    int tot = lv_n;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
    n_end = (uint32_t)uniform(tot) * (uint32_t)p.num_kv_heads;
  }

  // Tickets are compared unsigned, so even a counter left non-zero by a
  // misuse only ever yields item numbers inside [0, n_end).
  if (tid == 0) item_slot[0] = atomicAdd(p.counter, 1u);
  __syncthreads();
  int par = 0;
  // readfirstlane: the item is block-uniform, so its geometry stays scalar.
  for (uint32_t item = uniform(item_slot[0]);; item = uniform(item_slot[par])) {
    if (item >= n_end) {
      // Every block draws exactly one ticket past the end; the last such
      // ticket is drawn after all others, so its holder resets the counter.
      if (tid == 0 && item - n_end == gridDim.x - 1) atomicExch(p.counter, 0u);
      break;
    }
    int qt, r, kvh;
    if (p.longest_first) {
      const int t = (int)item / p.num_kv_heads;
      kvh = (int)item % p.num_kv_heads;
      uint64_t on = 0;
      while (level >= 0) {
        on = __ballot(lv_n > 0 && lv_b <= level && level < lv_b + lv_n);
        const int cnt = __popcll(on);
        if (t < below + cnt) break;
        below += cnt;
        --level;
      }
      if (level >= 0) {
        // the request of the (t - below)-th set bit of `on`
        const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(on >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)on, 0));
        const uint64_t pick = __ballot(((on >> lane) & 1) && rank == t - below);
        r = uniform(__builtin_ctzll(pick));
        qt = level - __builtin_amdgcn_readlane(lv_b, r);
      } else {
        qt = -1;  // past the last tile: nothing to do
        r = 0;
      }
    } else {
      qt = p.n_qtiles - 1 - (int)item / rk_all;
      r = (int)item % rk_all / p.num_kv_heads;
      kvh = (int)item % p.num_kv_heads;
    }
    // The next ticket is drawn inside the item, after its last tile (thread
    // 0 only); an item with no positions draws it here.
    uint32_t next = 0;
    const bool drawn = qt >= 0 && attend_item<D, NB, G, BUF>(p, qt, r, kvh, tid, lane, wave, kv, next,
                                                                 geo);
    if (tid == 0) item_slot[par ^ 1] = drawn ? next : atomicAdd(p.counter, 1u);
    par ^= 1;
    __syncthreads();  // LDS tiles free; the next item number is visible
  }
}

// Returns false (drawing nothing) for an item with no positions; else thread
// 0 has drawn the block's next ticket into `next`.
template <int D, int NB, int G, bool BUF, typename KV>
__device__ __forceinline__ bool attend_item(const PrefillParams& p, int qt, int r, int kvh,
                                            int tid, int lane, int wave, KV& kv,
                                            uint32_t& next, const int (&geo)[3][64]) {
  constexpr int QT = 128 * NB / G;        // positions per item
  constexpr int KS = D / 16;              // 16-dim steps of QK^T
  constexpr int DB = D / 32;              // 32-dim blocks of the output
  constexpr int PITCH = D + 8;            // LDS row pitch of K and V (bf16)
  constexpr int PIECES = D / 8;           // 16-byte pieces per K/V row
  constexpr int ROWS = 256 / PIECES;      // rows one pass of the block fetches
  constexpr int LOADS = kKeys / ROWS;     // passes per tile

  int s0, L, P;
  if (p.longest_first) {
    s0 = uniform(geo[0][r]);
    L = uniform(geo[1][r]);
    P = uniform(geo[2][r]);
  } else {
    request_geometry(p, r, s0, L, P);
  }
  const int q0 = qt * QT;
  if (q0 >= L) return false;
  const int qlast = min(q0 + QT, L) - 1;
  const int kend = P + qlast + 1;   // keys [0, kend) are read
  const int kfull = P + q0 + 1;     // keys [0, kfull) are visible to every column
  const int ntiles = (kend + kKeys - 1) / kKeys;

  // This lane's columns: NB blocks of 32 (query head, position) pairs, head-major.
  // Lanes l and l ^ 32 share a column and split its keys.
  const int half = lane >> 5;
  const int col = lane & 31;
  bf16x8 qb[NB][KS];
  int lim[NB], hb[NB], pos[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c = wave * 32 * NB + nb * 32 + col;
    hb[nb] = c / QT;
    pos[nb] = q0 + c % QT;
    const bool valid = pos[nb] <= qlast;
    lim[nb] = P + (valid ? pos[nb] : qlast);
    const uint16_t* qp =
        p.q + ((int64_t)(s0 + (valid ? pos[nb] : qlast)) * p.num_q_heads + kvh * G + hb[nb]) * D +
        8 * half;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = ld16(qp + 16 * ks);
      if (!valid) v = make_uint4(0, 0, 0, 0);
      qb[nb][ks] = as_bf16x8(v);
    }
  }

  // Tile fetch: thread -> (row lrow + ROWS * it, 16-byte piece lpc).  Rows
  // past the last key read are clamped onto it (always a valid row of the
  // request; those keys are masked), so every load is unconditional.  Page
  // numbers are fetched a tile before the rows they locate and checked only
  // where they are used, so their loads never hold up the wave.
  // The empty asm makes lrow opaque per item, so the compiler does not hoist
  // item-invariant address arithmetic of the first tiles out of the item loop
  // (where it would stay live through the whole tile loop and spill).
  int lrow = tid / PIECES;
  asm volatile("" : "+v"(lrow));
  const int lpc = tid % PIECES;
  const int32_t* pt = p.page_table + (int64_t)r * p.pt_stride;
  const char* kbase = reinterpret_cast<const char*>(p.k_cache) + (kvh * D + lpc * 8) * 2;
  const int64_t v_minus_k = reinterpret_cast<const char*>(p.v_cache) -
                            reinterpret_cast<const char*>(p.k_cache);
  const int klast = kend - 1;
  const int pmask = p.page_size - 1;
  int pg[LOADS];
  uint4 kr[2][LOADS], vr[2][LOADS];  // rows of two tiles in flight
  // With pages of at most 64 rows, a row slot keeps its place inside its page
  // from tile to tile and its page index advances by 64 / page_size, so tiles
  // that lie wholly before the last key need no per-row clamp or offset
  // arithmetic (the last tile of an item takes the general path).
  const bool small_pages = p.page_size <= kKeys;
  const int pstep = kKeys >> p.page_shift;
  // kin: row addresses (BUF: byte offsets) within a page, per row slot
  std::conditional_t<BUF, uint32_t, const char*> kin[LOADS];
  int pidx0[LOADS];
  const uint32_t hoff = (uint32_t)(kvh * D + lpc * 8) * 2u;  // BUF: the head's slice
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int r0 = lrow + ROWS * it;
    if constexpr (BUF)
      kin[it] = hoff + __umul24(r0 & pmask, p.row_bytes);
    else
      kin[it] = kbase + __umul24(r0 & pmask, p.row_bytes);
    pidx0[it] = r0 >> p.page_shift;
  }
  // BUF: 16 bytes of pool `pool` (K or V) at a byte offset
  auto bload = [&](const uint16_t* pool, uint32_t off) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(pool), (short)0, (int)p.pool_bytes, kBufferFlags);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
  };
  auto whole = [&](int kt) { return small_pages && kt * kKeys + kKeys - 1 <= klast; };
  auto fetch_pages = [&](int kt) {
    if (whole(kt)) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) pg[it] = pt[pidx0[it] + kt * pstep];
    } else {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int kg = min(kt * kKeys + lrow + ROWS * it, klast);
        pg[it] = pt[kg >> p.page_shift];
      }
    }
  };
  // Register set `set` (a constant at every call) holds the rows of tile kt.
  // With 64-bit addresses, page numbers at or past num_pages read the last
  // page (never unowned memory; such a table is invalid input).
  auto fetch_rows = [&](int kt, auto set_c) {
    constexpr int set = decltype(set_c)::value;
    if (whole(kt)) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        if constexpr (BUF) {
          const uint32_t off = __umul24((uint32_t)pg[it], p.page_bytes) + kin[it];
          kr[set][it] = bload(p.k_cache, off);
          vr[set][it] = bload(p.v_cache, off);
        } else {
          const uint32_t page = min((uint32_t)pg[it], p.num_pages_u32 - 1u);
          const char* kp = kin[it] + (uint64_t)page * p.page_bytes;
          kr[set][it] = ld16(kp);
          vr[set][it] = ld16(kp + v_minus_k);
        }
      }
    } else {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int kg = min(kt * kKeys + lrow + ROWS * it, klast);
        if constexpr (BUF) {
          const uint32_t off = __umul24((uint32_t)pg[it], p.page_bytes) + hoff +
                               __umul24(kg & pmask, p.row_bytes);
          kr[set][it] = bload(p.k_cache, off);
          vr[set][it] = bload(p.v_cache, off);
        } else {
          const uint32_t page = min((uint32_t)pg[it], p.num_pages_u32 - 1u);
          const char* kp =
              kbase + (uint64_t)page * p.page_bytes + __umul24(kg & pmask, p.row_bytes);
          kr[set][it] = ld16(kp);
          vr[set][it] = ld16(kp + v_minus_k);
        }
      }
    }
  };
  auto stash = [&](int buf, auto set_c) {
    constexpr int set = decltype(set_c)::value;
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int o = (lrow + ROWS * it) * PITCH + lpc * 8;
      *reinterpret_cast<uint4*>(&kv[buf][0][o]) = kr[set][it];
      *reinterpret_cast<uint4*>(&kv[buf][1][o]) = vr[set][it];
    }
  };
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;

  f32x16 oacc[DB][NB];
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = kNegInf;
    l[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[db][nb][v] = 0.f;
  }
  const float c = p.scale_log2;
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);

  // Offsets of this lane's operand reads inside one tile (elements).
  const int k_off = col * PITCH + 8 * half;
  const int l16 = lane & 15;
  const int v_off = (4 * half + (l16 >> 2)) * PITCH + 16 * ((lane >> 4) & 1) + 4 * (l16 & 3);

  // Tile t's rows sit in register set t & 1 from their fetch (three tiles
  // ahead) until they are staged in LDS buffer t & 1 (one tile ahead).
  fetch_pages(0);
  fetch_rows(0, Set0{});
  stash(0, Set0{});
  if (ntiles > 1) {
    fetch_pages(1);
    fetch_rows(1, Set1{});
    if (ntiles > 2) {
      fetch_pages(2);
      fetch_rows(2, Set0{});
      if (ntiles > 3) fetch_pages(3);
    }
  }

  auto tile = [&](int kt, auto par_c) {
    constexpr int par = decltype(par_c)::value;  // kt & 1
    constexpr int nxt = 1 - par;                 // register set of tiles kt + 1 and kt + 3
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt - 1
    const uint16_t* Kt = kv[kt & 1][0];
    const uint16_t* Vt = kv[kt & 1][1];

    // S^T tile: rows = 64 keys (two 32-key halves), columns = this wave's.
    f32x16 sacc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[nb][kh][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const bf16x8 a = as_bf16x8(ld16(&Kt[kh * 32 * PITCH + k_off + 16 * ks]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb][kh] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[nb][ks], sacc[nb][kh], 0, 0, 0);
      }
    }

    // Stage tile kt + 1 and fetch tile kt + 3 while the QK^T MFMAs run: the
    // address arithmetic and LDS writes issue from the VALU and LDS pipes
    // beside the matrix core.
    if (kt + 1 < ntiles) stash(nxt, std::integral_constant<int, nxt>{});
    if (kt + 3 < ntiles) {
      fetch_rows(kt + 3, std::integral_constant<int, nxt>{});
      if (kt + 4 < ntiles) fetch_pages(kt + 4);
    }

    // Causal mask, only on tiles that reach past the block's first column:
    // accumulator slot (kh, v) holds key kt*64 + 4*half + kh*32 + 8(v/4) + v%4,
    // so each slot compares a compile-time offset with a per-lane threshold.
    const bool diag = (kt + 1) * kKeys > kfull;
    auto mask = [&](f32x16& acc, int nb, int kh) {
      const int thr = lim[nb] - kt * kKeys - 4 * half;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = kh * 32 + (v >> 2) * 8 + (v & 3);
        acc[v] = off <= thr ? acc[v] : kNegInf;
      }
    };
    if (diag) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) mask(sacc[nb][kh], nb, kh);
    }

    // Reference point of the exponentials.  The first tile sets it to the
    // column maxima (every column sees key 0, so they are finite).  Later
    // tiles keep it and compute P speculatively: if a lane's row sum over
    // the tile shows a probability above 2^kTau (a score more than kTau above
    // the reference), the tile's scores are recomputed from the K tile still
    // in LDS, the reference moves to their column maxima, O and l are
    // rescaled and P is recomputed, all before any P of the tile enters O.
    // Every P is therefore <= 2^kTau, and tiles whose scores stay near the
    // running maximum cost no max reduction.
    if (kt == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) m[nb] = tile_max(sacc[nb]) * c;
    }

    // P = 2^(s * c - m) in bf16 (the B operands of O^T += V^T P^T, one per
    // (kh, u) step and column block) and this lane's row sums of the same
    // rounded values.
    bf16x8 pb[2][2][NB];
    float ts[NB];
    auto probs = [&](const f32x16 (&src)[NB][2]) {
      bool over = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float nm = -m[nb];
        float t[2] = {0.f, 0.f};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float e0 = fast_exp2(__builtin_fmaf(src[nb][kh][8 * u + 2 * j], c, nm));
              const float e1 = fast_exp2(__builtin_fmaf(src[nb][kh][8 * u + 2 * j + 1], c, nm));
              w[j] = pack_bf16x2(e0, e1);
              t[kh] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[j]), ones,
                                                      t[kh], false);
            }
            pb[kh][u][nb] = as_bf16x8(make_uint4(w[0], w[1], w[2], w[3]));
          }
        ts[nb] = t[0] + t[1];
        over |= ts[nb] > kPmax;
      }
      return over;
    };
    if (__any(probs(sacc))) {
      // Rare: recompute the tile's scores (the exponentials consumed them),
      // move the reference, rescale, recompute P.
      f32x16 rs[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int v = 0; v < 16; ++v) rs[nb][kh][v] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const bf16x8 a = as_bf16x8(ld16(&Kt[kh * 32 * PITCH + k_off + 16 * ks]));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            rs[nb][kh] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[nb][ks], rs[nb][kh], 0, 0, 0);
        }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (diag) {
          mask(rs[nb][0], nb, 0);
          mask(rs[nb][1], nb, 1);
        }
        const float mn = fmaxf(m[nb], tile_max(rs[nb]) * c);
        const float al = fast_exp2(m[nb] - mn);
        l[nb] *= al;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][nb][v] *= al;
        m[nb] = mn;
      }
      probs(rs);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) l[nb] += ts[nb];

    // Operand slot (half, i) of step (kh, u) holds key
    // kh*32 + 16u + 8(i/4) + 4*half + i%4 on both sides; the V^T operand
    // comes from two transposing LDS reads of 4 rows each.
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint16_t* vrow = Vt + (kh * 32 + 16 * u) * PITCH + v_off;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const s16x4 lo = lds_read_tr16(vrow + 32 * db);
          const s16x4 hi = lds_read_tr16(vrow + 8 * PITCH + 32 * db);
          const s16x8 a8 = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const bf16x8 a = __builtin_bit_cast(bf16x8, a8);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kh][u][nb], oacc[db][nb], 0, 0, 0);
        }
      }
  };
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile(kt, Set0{});
    if (kt + 1 < ntiles) tile(kt + 1, Set1{});
  }

  // The block's next ticket, drawn as its last tile ends: the last tickets
  // go to the blocks that free up first.  The result is stored to LDS only
  // after the output below, so the round trip overlaps it; the opaque zero
  // keeps the address lane-varying in the compiler's eyes, since a
  // uniform-address atomic is rewritten as a wave reduction that waits for
  // its result (and every older load) right where it is issued.
  if (tid == 0) {
    int zero = 0;
    asm volatile("" : "+v"(zero));
    next = atomicAdd(p.counter + zero, 1u);
  }

  // Normalise and write the output.  A lane holds dims
  // db*32 + 8*(v/4) + 4*half + v%4 of its column, so a direct store writes
  // 8 bytes to each of 32 rows.  At head_dim 128 every wave instead stages
  // its columns in LDS as rows of D values (the K/V buffers are free once
  // every wave is past its last tile) and reads back whole 16-byte pieces,
  // so each store writes contiguous output rows; at 64 the extra barrier
  // costs more than the wider stores gain (A/B: -2% at 128, +1% at 64).
  if constexpr (D == 128) {
    __syncthreads();  // every wave is done with the last tile's K and V
    uint16_t* stage = &kv[0][0][0] + wave * (32 * NB * PITCH);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = l[nb] + __shfl_xor(l[nb], 32);
      const float inv = 1.f / lt;  // (columns past the last position are staged, never stored)
      uint16_t* srow = stage + (nb * 32 + col) * PITCH;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          uint2 w;
          w.x = pack_bf16x2(oacc[db][nb][4 * v4] * inv, oacc[db][nb][4 * v4 + 1] * inv);
          w.y = pack_bf16x2(oacc[db][nb][4 * v4 + 2] * inv, oacc[db][nb][4 * v4 + 3] * inv);
          *reinterpret_cast<uint2*>(srow + db * 32 + 8 * v4 + 4 * half) = w;
        }
    }
    // A wave's LDS operations complete in order, so its reads below see
    // every lane's writes above.
    constexpr int ROW_PIECES = D / 8;                    // 16-byte pieces per output row
    constexpr int PER_LANE = 32 * NB * ROW_PIECES / 64;  // pieces per lane
#pragma unroll
    for (int k = 0; k < PER_LANE; ++k) {
      const int idx = k * 64 + lane;
      const int lc = idx / ROW_PIECES;  // the wave's column
      const int pc = idx % ROW_PIECES;
      const int c = wave * 32 * NB + lc;
      const int pos_c = q0 + c % QT;
      if (pos_c <= qlast) {
        const uint4 v = *reinterpret_cast<const uint4*>(stage + lc * PITCH + pc * 8);
        *reinterpret_cast<uint4*>(
            p.out + ((int64_t)(s0 + pos_c) * p.num_q_heads + kvh * G + c / QT) * D + pc * 8) = v;
      }
    }
  } else {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = l[nb] + __shfl_xor(l[nb], 32);
      if (pos[nb] > qlast) continue;
      const float inv = 1.f / lt;
      uint16_t* op = p.out + ((int64_t)(s0 + pos[nb]) * p.num_q_heads + kvh * G + hb[nb]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          uint2 w;
          w.x = pack_bf16x2(oacc[db][nb][4 * v4] * inv, oacc[db][nb][4 * v4 + 1] * inv);
          w.y = pack_bf16x2(oacc[db][nb][4 * v4 + 2] * inv, oacc[db][nb][4 * v4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + db * 32 + 8 * v4 + 4 * half) = w;
        }
    }
  }
  return true;
}

// Resident blocks per CU of one instantiation times the CU count of the
// current device, computed once per (device, instantiation).
template <int D, int NB, int G, bool BUF>
int resident_blocks() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
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
          &per_cu, reinterpret_cast<const void*>(prefill_kernel<D, NB, G, BUF>), 256, 0) !=
      hipSuccess)
    return 0;
  const int n = cus * per_cu;
  if (n > 0 && dev < kMaxDevices) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, int NB, int G, bool BUF>
int launch_prefill_as(PrefillParams& p, hipStream_t s) {
  const int resident = resident_blocks<D, NB, G, BUF>();
  if (resident <= 0) return PKV_EHIP;
  const int grid = (int)std::min<int64_t>(p.n_items, resident);
  return pkv_host::launch(prefill_kernel<D, NB, G, BUF>, dim3((unsigned)grid), dim3(256), s, p);
}

template <int D, int NB, int G>
int launch_prefill(PrefillParams& p, hipStream_t s) {
  return p.pool_bytes != 0 ? launch_prefill_as<D, NB, G, true>(p, s)
                           : launch_prefill_as<D, NB, G, false>(p, s);
}

}  // namespace

extern "C" size_t pkv_prefill_workspace_bytes(void) { return kPrefillWorkspaceBytes; }

extern "C" int pkv_paged_attn_prefill(const void* q, const int32_t* cu_seqlens_q,
                                      const int32_t* prefix_lens, int32_t num_seqs,
                                      int32_t num_tokens, int32_t max_q_len,
                                      int32_t max_seq_len, const void* k_cache,
                                      const void* v_cache, int32_t page_size,
                                      int64_t num_pages, const int32_t* page_table,
                                      int32_t page_table_stride, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      float softmax_scale, void* out, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  using namespace pkv_host;
  if (num_seqs < 0 || num_tokens < 0) return PKV_EINVAL;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return PKV_EINVAL;
  if (!finite_positive(softmax_scale)) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (num_seqs == 0 || max_q_len <= 0 || max_seq_len <= 0) return PKV_EINVAL;
  if (!q || !cu_seqlens_q || !prefix_lens || !k_cache || !v_cache || !page_table || !out ||
      !workspace)
    return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
      !aligned16(workspace))
    return PKV_EINVAL;
  if (num_pages <= 0 || page_table_stride <= 0) return PKV_EINVAL;
  if (!is_pow2_page(page_size)) return PKV_EUNSUPPORTED;
  if ((int64_t)page_table_stride * page_size < max_seq_len) return PKV_EINVAL;
  const int g = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  const int nb = head_dim == 64 ? 2 : 1;
  if (!(g == 1 || g == 2 || g == 4 || g == 8)) return PKV_EUNSUPPORTED;
  if (workspace_bytes < kPrefillWorkspaceBytes) return PKV_ENOSPACE;
  const int qtile = 128 * nb / g;
  const int64_t n_qtiles = ((int64_t)max_q_len + qtile - 1) / qtile;
  const int64_t n_items = n_qtiles * num_seqs * num_kv_heads;
  if (n_items >= INT32_MAX / 2) return PKV_EINVAL;
  // Row addresses are formed from a 32-bit page size and a 24-bit in-page
  // offset: pages of one pool must stay below 4 GiB.
  const int64_t page_bytes = (int64_t)page_size * num_kv_heads * head_dim * 2;
  if (page_bytes >= ((int64_t)1 << 32) || (int64_t)num_kv_heads * head_dim * 2 >= (1 << 24))
    return PKV_EUNSUPPORTED;

  PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.cu_seqlens = cu_seqlens_q;
  p.prefix_lens = prefix_lens;
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.out = static_cast<uint16_t*>(out);
  p.counter = static_cast<uint32_t*>(workspace);
  p.num_pages = num_pages;
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.max_q_len = max_q_len;
  p.max_seq_len = max_seq_len;
  p.page_size = page_size;
  p.page_shift = log2_exact(page_size);
  p.pt_stride = page_table_stride;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.n_qtiles = (int32_t)n_qtiles;
  p.n_items = (int32_t)n_items;
  // Longest-first tickets need one request per lane, and every block walks
  // the levels once (at most max_seq_len / qtile + n_qtiles of them).
  p.longest_first = num_seqs <= 64 && (int64_t)max_seq_len / qtile + n_qtiles <= 1024;
  p.num_pages_u32 = (uint32_t)std::min<int64_t>(num_pages, INT32_MAX);
  p.row_bytes = (uint32_t)(num_kv_heads * head_dim * 2);
  p.page_bytes = (uint32_t)page_bytes;
  // Buffer loads need the pool within 32-bit offsets and 24-bit page numbers
  // and page sizes for the multiply.
  const bool buf = num_pages < (1 << 24) && page_bytes < (1 << 24) &&
                   num_pages * page_bytes <= (int64_t)INT32_MAX;
  p.pool_bytes = buf ? (uint32_t)(num_pages * page_bytes) : 0u;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64) {
    if (g == 1) return launch_prefill<64, 2, 1>(p, s);
    if (g == 2) return launch_prefill<64, 2, 2>(p, s);
    if (g == 4) return launch_prefill<64, 2, 4>(p, s);
    return launch_prefill<64, 2, 8>(p, s);
  }
  if (g == 1) return launch_prefill<128, 1, 1>(p, s);
  if (g == 2) return launch_prefill<128, 1, 2>(p, s);
  if (g == 4) return launch_prefill<128, 1, 4>(p, s);
  return launch_prefill<128, 1, 8>(p, s);
}
