// The shared-prefix pass of decode over requests grouped by shared cached
// prefixes: for every group, the queries of all its members (all query
// heads of a KV head, as the MFMA columns) against one split of the group's
// shared prefix keys, read once through the group's first member's page
// table, with un-normalised partial results (reference point m in base 2,
// row sum l, o) written to the decode workspace's slots 0.. of every
// (member, KV head); the decode split kernel fills the slots after them
// from each request's remaining tokens, and the split merge combines all.
// The tile loop is that of the prefill kernel (MFMA 32x32x16 bf16 for QK^T
// and PV, 64-key tiles double-buffered in LDS, speculative softmax reference
// point redone exactly when a probability may exceed 2^kTau), with no causal
// mask: the split lies inside the prefix every member sees.
#pragma once

#include <type_traits>

#include "pkv_common.h"

namespace pkv_prefix {

using namespace pkv;

struct Params {
  const uint16_t* q;           // [num_seqs, num_q_heads, head_dim]
  const int32_t* cu_groups;    // [num_groups + 1]
  const int32_t* shared_lens;  // [num_seqs]
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  float* ws_m;
  float* ws_l;
  float* ws_o;
  int32_t num_groups;
  int32_t num_seqs;
  int32_t max_group_size;
  int32_t max_shared_len;
  int32_t page_size;
  int32_t page_shift;
  int32_t pt_stride;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t n_qtiles;   // query tiles per group (host bound)
  int32_t ksplit;     // keys per split (kSplit)
  int32_t slots;      // partial slots per (request, KV head)
  int32_t items;      // n_ksplits * n_qtiles * num_groups * num_kv_heads
  uint32_t num_pages_u32;
  uint32_t page_bytes;
  uint32_t row_bytes;
  float scale_log2;
};

constexpr float kTau = 8.0f;
constexpr float kPmax = 256.0f;  // 2^kTau
constexpr int kKeys = 64;        // keys per tile
// Keys per split of a shared prefix (one item, two tiles).  Longer items
// leave fewer partials for the merge to read, shorter ones more parallel
// items: 128 measured 1% faster than 64 on a 64-request batch sharing 1,024
// tokens, and 256 no faster than 64.
constexpr int kSplit = 128;

// LDS bytes of one item (two K and two V tiles).
template <int D>
constexpr size_t item_lds_bytes() {
  return (size_t)2 * 2 * kKeys * (D + 8) * sizeof(uint16_t);
}

// fmax over lanes l and l ^ 32 (the two halves of one 32x32 accumulator column).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum of one column's 64 scores in a tile.
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
  float a = fmaxf(s[0][0], s[0][1]), b = fmaxf(s[1][0], s[1][1]);
#pragma unroll
  for (int v = 2; v < 16; v += 2) {
    a = fmaxf(fmaxf(a, s[0][v]), s[0][v + 1]);
    b = fmaxf(fmaxf(b, s[1][v]), s[1][v + 1]);
  }
  return max_xor32(fmaxf(a, b));
}

// One item, by a workgroup of 256 threads (4 waves, NB blocks of 32
// columns each) with item_lds_bytes<D>() of LDS at `lds`:
// item = ((key split * query tiles + query tile) * groups + group) * KV heads + KV head.
template <int D, int NB, int G>
__device__ __forceinline__ void prefix_item(const Params& p, uint32_t item, uint16_t* lds, int tid) {
  constexpr int TILE = kKeys * (D + 8);
  auto& kv = *reinterpret_cast<uint16_t(*)[2][2][TILE]>(lds);
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = (int)(item % (uint32_t)p.num_kv_heads);
  uint32_t rest = item / (uint32_t)p.num_kv_heads;
  const int grp = (int)(rest % (uint32_t)p.num_groups);
  rest /= (uint32_t)p.num_groups;
  const int qt = (int)(rest % (uint32_t)p.n_qtiles);
  const int split = (int)(rest / (uint32_t)p.n_qtiles);
  constexpr int QT = 128 * NB / G;        // members per item
  constexpr int KS = D / 16;              // 16-dim steps of QK^T
  constexpr int DB = D / 32;              // 32-dim blocks of the output
  constexpr int PITCH = D + 8;            // LDS row pitch of K and V (bf16)
  constexpr int PIECES = D / 8;           // 16-byte pieces per K/V row
  constexpr int ROWS = 256 / PIECES;      // rows one pass of the block fetches
  constexpr int LOADS = kKeys / ROWS;     // passes per tile

  // The group's members are rows s0 .. s0 + L - 1 of q (clamped into the
  // batch); they share the first P tokens (rounded down to 16).
  const int s0 = min(max(p.cu_groups[grp], 0), p.num_seqs);
  const int L = min(min(max(p.cu_groups[grp + 1], s0), p.num_seqs) - s0, p.max_group_size);
  const int q0 = qt * QT;
  if (q0 >= L) return;
  const int P = min(max(p.shared_lens[s0], 0), p.max_shared_len) & ~15;
  const int qlast = min(q0 + QT, L) - 1;
  // Keys [kbeg, kend) of this split are read, and every member (column)
  // sees all of them.
  const int kbeg = split * p.ksplit;
  if (kbeg >= P) return;
  const int kend = min(P, kbeg + p.ksplit);
  const int kfull = kend;
  // first tile; buffers and register sets alternate with the tile's
  // parity relative to it
  const int kt0 = kbeg / kKeys;
  const int ntiles = (kend + kKeys - 1) / kKeys;

  // This lane's columns: NB blocks of 32 (query head, member) pairs, head-major.
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
    lim[nb] = kend - 1;
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
  // prefix; those keys are masked), so every load is unconditional.  Page
  // numbers are fetched a tile before the rows they locate and checked only
  // where they are used.  The empty asm keeps lrow opaque, so the compiler
  // does not hoist address arithmetic of later tiles into long-lived
  // registers.
  int lrow = tid / PIECES;
  asm volatile("" : "+v"(lrow));
  const int lpc = tid % PIECES;
  // the group's first member's page-table row
  const int32_t* pt = p.page_table + (int64_t)s0 * p.pt_stride;
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
  const char* kin[LOADS];
  int pidx0[LOADS];
#pragma unroll
  for (int it = 0; it < LOADS; ++it) {
    const int r0 = lrow + ROWS * it;
    kin[it] = kbase + __umul24(r0 & pmask, p.row_bytes);
    pidx0[it] = r0 >> p.page_shift;
  }
  auto whole = [&](int kt) { return small_pages && kt * kKeys + kKeys - 1 <= klast; };
  auto fetch_pages_into = [&](int kt, int (&dst)[LOADS]) {
    if (whole(kt)) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) dst[it] = pt[pidx0[it] + kt * pstep];
    } else {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int kg = min(kt * kKeys + lrow + ROWS * it, klast);
        dst[it] = pt[kg >> p.page_shift];
      }
    }
  };
  auto fetch_pages = [&](int kt) { fetch_pages_into(kt, pg); };
  // Register set `set` (a constant at every call) holds the rows of tile kt.
  // Page numbers at or past num_pages read the last page (never unowned
  // memory; such a table is invalid input).
  auto fetch_rows_from = [&](int kt, auto set_c, const int (&pgs)[LOADS]) {
    constexpr int set = decltype(set_c)::value;
    if (whole(kt)) {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const uint32_t page = min((uint32_t)pgs[it], p.num_pages_u32 - 1u);
        const char* kp = kin[it] + (uint64_t)page * p.page_bytes;
        kr[set][it] = ld16(kp);
        vr[set][it] = ld16(kp + v_minus_k);
      }
    } else {
#pragma unroll
      for (int it = 0; it < LOADS; ++it) {
        const int kg = min(kt * kKeys + lrow + ROWS * it, klast);
        const uint32_t page = min((uint32_t)pgs[it], p.num_pages_u32 - 1u);
        const char* kp =
            kbase + (uint64_t)page * p.page_bytes + __umul24(kg & pmask, p.row_bytes);
        kr[set][it] = ld16(kp);
        vr[set][it] = ld16(kp + v_minus_k);
      }
    }
  };
  auto fetch_rows = [&](int kt, auto set_c) { fetch_rows_from(kt, set_c, pg); };
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

  // Tile kt0 + t's rows sit in register set t & 1 from their fetch (three
  // tiles ahead) until they are staged in LDS buffer t & 1 (one tile
  // ahead).  Items are short (one key split, two tiles): both tiles' page
  // numbers are fetched together, then their rows, so the item starts
  // after two memory round trips, not four.
  int pg1[LOADS];
  fetch_pages_into(kt0, pg);
  if (ntiles > kt0 + 1) fetch_pages_into(kt0 + 1, pg1);
  fetch_rows_from(kt0, Set0{}, pg);
  if (ntiles > kt0 + 1) fetch_rows_from(kt0 + 1, Set1{}, pg1);
  stash(0, Set0{});
  if (ntiles > kt0 + 2) {
    fetch_pages(kt0 + 2);
    fetch_rows(kt0 + 2, Set0{});
    if (ntiles > kt0 + 3) fetch_pages(kt0 + 3);
  }

  auto tile = [&](int kt, auto par_c) {
    constexpr int par = decltype(par_c)::value;  // (kt - kt0) & 1
    constexpr int nxt = 1 - par;                 // register set of tiles kt + 1 and kt + 3
    __syncthreads();  // tile kt is in LDS; every wave is done with tile kt - 1
    const uint16_t* Kt = kv[(kt - kt0) & 1][0];
    const uint16_t* Vt = kv[(kt - kt0) & 1][1];

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

    // Mask of the keys past the split's end, only on a split's partial last
    // tile: accumulator slot (kh, v) holds key kt*64 + 4*half + kh*32 +
    // 8(v/4) + v%4, so each slot compares a compile-time offset with a
    // per-lane threshold.
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
    // column maxima (every column sees every key of the split, so they are
    // finite).  Later
    // tiles keep it and compute P speculatively: if a lane's row sum over
    // the tile shows a probability above 2^kTau (a score more than kTau above
    // the reference), the tile's scores are recomputed from the K tile still
    // in LDS, the reference moves to their column maxima, O and l are
    // rescaled and P is recomputed, all before any P of the tile enters O.
    // Every P is therefore <= 2^kTau, and tiles whose scores stay near the
    // running maximum cost no max reduction.
    if (kt == kt0) {
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
  for (int kt = kt0; kt < ntiles; kt += 2) {
    tile(kt, Set0{});
    if (kt + 1 < ntiles) tile(kt + 1, Set1{});
  }

  // Un-normalised partial of this key split for column (member, head): the
  // reference point m (base 2, scaled), the row sum l and o, in the decode
  // workspace's slot `split` of (member, KV head).
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = l[nb] + __shfl_xor(l[nb], 32);
    if (pos[nb] > qlast) continue;
    const int64_t base =
        (((int64_t)(s0 + pos[nb]) * p.num_kv_heads + kvh) * p.slots + split) * G + hb[nb];
    float* op = p.ws_o + base * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *reinterpret_cast<f32x4*>(op + db * 32 + 8 * v4 + 4 * half) =
            f32x4{oacc[db][nb][4 * v4], oacc[db][nb][4 * v4 + 1], oacc[db][nb][4 * v4 + 2],
                  oacc[db][nb][4 * v4 + 3]};
    if (half == 0) {
      p.ws_m[base] = m[nb];
      p.ws_l[base] = lt;
    }
  }
}

}  // namespace pkv_prefix
