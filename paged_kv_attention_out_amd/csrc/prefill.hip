// Causal prefill attention with a cached prefix over a paged KV cache.
//
// Prefill feeds only the tokens after each request's cached prefix, as one
// flat ragged batch indexed by cu_seqlens_q (miniVLLM "Engine Architecture",
// prepare_prefill; zero-to-sglang Ch.1 section 3.3: extend length =
// sequence length - cached length).  New token i of request r is at
// absolute position P_r + i and sees keys 0 .. P_r + i.
//
// Work unit = one 256-thread block per (request, KV head, query tile).  The
// block's 128*NB "columns" are (query head of the group, position) pairs,
// head-major, so the g query heads that share a KV head reuse every K/V tile
// staged in LDS; each wave owns NB blocks of 32 columns.
//
// Per 64-key tile:
//   * K and V rows are fetched through the page table into registers one
//     tile ahead, then written to LDS: K row-major, V transposed (dim-major)
//     so that PV operands are key-contiguous.
//   * S^T = K Q^T with MFMA 32x32x16 bf16 (A = K from LDS, B = Q resident in
//     registers); lane l owns column l % 32, 32 keys of it per 32x32 block.
//   * Online softmax per column in base 2 with lazy rescaling (threshold
//     kTau); tiles left of the block's diagonal skip the mask.
//   * P (rounded to bf16, round-to-nearest-even) stays in registers: the
//     accumulator layout of S^T is already the B operand layout of
//     O^T += V^T P^T, with the key order permuted identically on both sides.
// Arithmetic per visible (query, key) pair: 4 * head_dim flops on MFMA.

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
  float scale_log2;
};

constexpr float kTau = 8.0f;
constexpr int kKeys = 64;  // keys per tile

template <int D, int NB, int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int QT = 128 * NB / G;        // positions per block
  constexpr int KS = D / 16;              // 16-dim steps of QK^T
  constexpr int DB = D / 32;              // 32-dim blocks of the output
  constexpr int KPITCH = D + 8;           // LDS row pitch of K (bf16)
  constexpr int VPITCH = kKeys + 4;       // LDS row pitch of V^T (bf16)
  constexpr int PIECES = D / 8;           // 16-byte pieces per K/V row
  constexpr int LOADS = kKeys * PIECES / 256;
  static_assert(QT >= 32 && QT % 32 == 0, "a 32-column block must stay within one head");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKeys * KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rk_all = p.num_seqs * p.num_kv_heads;
  const int qt = p.n_qtiles - 1 - (int)(blockIdx.x / rk_all);  // longest tiles first
  const int rk = (int)(blockIdx.x % rk_all);
  const int kvh = rk % p.num_kv_heads;
  const int r = rk / p.num_kv_heads;

  // Request geometry, clamped so every access stays inside the buffers.
  int s0 = p.cu_seqlens[r], s1 = p.cu_seqlens[r + 1];
  s0 = min(max(s0, 0), p.num_tokens);
  s1 = min(max(s1, s0), p.num_tokens);
  const int L = min(min(s1 - s0, p.max_q_len), p.max_seq_len);
  const int P = min(max(p.prefix_lens[r], 0), p.max_seq_len - L);
  const int q0 = qt * QT;
  if (q0 >= L) return;
  const int qlast = min(q0 + QT, L) - 1;
  const int kend = P + qlast + 1;   // keys [0, kend) are read
  const int kfull = P + q0 + 1;     // keys [0, kfull) are visible to every column
  const int ntiles = (kend + kKeys - 1) / kKeys;

  // This wave's columns: NB blocks of 32 (query head hb, positions pos0..).
  const int half = lane >> 5;
  const int col = lane & 31;
  bf16x8 qb[NB][KS];
  int lim[NB], hb[NB], pos[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int c0 = wave * 32 * NB + nb * 32;
    hb[nb] = c0 / QT;
    pos[nb] = q0 + c0 % QT + col;
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

  const int32_t* pt = p.page_table + (int64_t)r * p.pt_stride;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  uint4 kreg[LOADS], vreg[LOADS];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int piece = tid + 256 * it;
      const int key = piece / PIECES;
      const int pc = piece % PIECES;
      const int kg = kt * kKeys + key;
      if (kg < kend) {
        int page = pt[kg >> p.page_shift];
        page = (page < 0 || (int64_t)page >= p.num_pages) ? 0 : page;
        const int64_t off =
            ((int64_t)page * p.page_size + (kg & (p.page_size - 1))) * row_elems + kvh * D + pc * 8;
        kreg[it] = ld16(p.k_cache + off);
        vreg[it] = ld16(p.v_cache + off);
      } else {
        kreg[it] = make_uint4(0, 0, 0, 0);
        vreg[it] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int it = 0; it < LOADS; ++it) {
      const int piece = tid + 256 * it;
      const int key = piece / PIECES;
      const int pc = piece % PIECES;
      *reinterpret_cast<uint4*>(&Ks[key * KPITCH + pc * 8]) = kreg[it];
      const uint32_t w[4] = {vreg[it].x, vreg[it].y, vreg[it].z, vreg[it].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Vt[(pc * 8 + 2 * e) * VPITCH + key] = (uint16_t)(w[e] & 0xffffu);
        Vt[(pc * 8 + 2 * e + 1) * VPITCH + key] = (uint16_t)(w[e] >> 16);
      }
    }
  };

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

  load_tile(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < ntiles) load_tile(kt + 1);
    const bool need_mask = (kt + 1) * kKeys > kfull;

    // S^T tile: rows = 64 keys (two 32-key halves), columns = this wave's.
    f32x16 sacc[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) sacc[nb][kh][v] = 0.f;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const uint4*>(&Ks[(kh * 32 + col) * KPITCH + 16 * ks + 8 * half]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb][kh] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[nb][ks], sacc[nb][kh], 0, 0, 0);
      }
    }

    // Scale, mask, tile max per column (the column's 64 keys are split
    // between lanes l and l ^ 32).
    bool grow = false;
    float mt[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mx = kNegInf;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[nb][kh][v] * p.scale_log2;
          if (need_mask) {
            const int key = kt * kKeys + kh * 32 + (v >> 2) * 8 + half * 4 + (v & 3);
            x = key <= lim[nb] ? x : kNegInf;
          }
          sacc[nb][kh][v] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mt[nb] = mx;
      grow |= mx > m[nb] + kTau;
    }
    if (__any(grow)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mn = fmaxf(m[nb], mt[nb]);
        const float a = mn == kNegInf ? 0.f : fast_exp2(m[nb] - mn);
        l[nb] *= a;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[db][nb][v] *= a;
        m[nb] = mn;
      }
    }

    // P = 2^(x - m) as bf16 B operands; one per (32-key half, 16-key step).
    bf16x8 pb[NB][2][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float e[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            e[i] = fast_exp2(sacc[nb][kh][8 * u + i] - m[nb]);
            l[nb] += e[i];
          }
          uint4 w;
          w.x = pack_bf16x2(e[0], e[1]);
          w.y = pack_bf16x2(e[2], e[3]);
          w.z = pack_bf16x2(e[4], e[5]);
          w.w = pack_bf16x2(e[6], e[7]);
          pb[nb][kh][u] = as_bf16x8(w);
        }

    // O^T += V^T P^T.  Operand slot (half, i) of step (kh, u) holds key
    // kh*32 + 16u + 8*(i/4) + 4*half + i%4 on both sides.
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int koff = kh * 32 + 16 * u + 4 * half;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint16_t* vrow = &Vt[(db * 32 + col) * VPITCH + koff];
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const bf16x8 a = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nb][kh][u], oacc[db][nb], 0, 0, 0);
        }
      }
  }

  // Normalise and write the valid columns: lane holds dims
  // db*32 + 8*(v/4) + 4*half + v%4 of its column.
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

template <int D, int NB, int G>
int launch_prefill(const PrefillParams& p, int64_t blocks, hipStream_t s) {
  return pkv_host::launch(prefill_kernel<D, NB, G>, dim3((unsigned)blocks), dim3(256), s, p);
}

}  // namespace

extern "C" int pkv_paged_attn_prefill(const void* q, const int32_t* cu_seqlens_q,
                                      const int32_t* prefix_lens, int32_t num_seqs,
                                      int32_t num_tokens, int32_t max_q_len,
                                      int32_t max_seq_len, const void* k_cache,
                                      const void* v_cache, int32_t page_size,
                                      int64_t num_pages, const int32_t* page_table,
                                      int32_t page_table_stride, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim,
                                      float softmax_scale, void* out, void* stream) {
  using namespace pkv_host;
  if (num_seqs < 0 || num_tokens < 0) return PKV_EINVAL;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads) return PKV_EINVAL;
  if (!finite_positive(softmax_scale)) return PKV_EINVAL;
  if (num_tokens == 0) return PKV_OK;
  if (num_seqs == 0 || max_q_len <= 0 || max_seq_len <= 0) return PKV_EINVAL;
  if (!q || !cu_seqlens_q || !prefix_lens || !k_cache || !v_cache || !page_table || !out)
    return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PKV_EINVAL;
  if (num_pages <= 0 || page_table_stride <= 0) return PKV_EINVAL;
  if (!is_pow2_page(page_size)) return PKV_EUNSUPPORTED;
  if ((int64_t)page_table_stride * page_size < max_seq_len) return PKV_EINVAL;
  const int g = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  const int nb = head_dim == 64 ? 2 : 1;
  if (!(g == 1 || g == 2 || g == 4 || (g == 8 && nb == 2))) return PKV_EUNSUPPORTED;
  const int qtile = 128 * nb / g;
  const int64_t n_qtiles = (max_q_len + qtile - 1) / qtile;
  const int64_t blocks = n_qtiles * num_seqs * num_kv_heads;
  if (blocks > INT32_MAX || (int64_t)num_seqs * num_kv_heads > INT32_MAX) return PKV_EINVAL;

  PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.cu_seqlens = cu_seqlens_q;
  p.prefix_lens = prefix_lens;
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.out = static_cast<uint16_t*>(out);
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
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64) {
    if (g == 1) return launch_prefill<64, 2, 1>(p, blocks, s);
    if (g == 2) return launch_prefill<64, 2, 2>(p, blocks, s);
    if (g == 4) return launch_prefill<64, 2, 4>(p, blocks, s);
    return launch_prefill<64, 2, 8>(p, blocks, s);
  }
  if (g == 1) return launch_prefill<128, 1, 1>(p, blocks, s);
  if (g == 2) return launch_prefill<128, 1, 2>(p, blocks, s);
  return launch_prefill<128, 1, 4>(p, blocks, s);
}
