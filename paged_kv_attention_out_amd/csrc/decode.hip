// Paged decode attention: one query token per request over its whole
// context, read through the page table (miniVLLM "Engine Architecture",
// prepare_decode: context_lens + block_tables; mini-sglang "Engine Class",
// Key Attributes: page_table).
//
// Work unit = one wavefront per (request r, KV head kvh, split s).  A split
// is `split` consecutive tokens; a request with n tokens has ceil(n/split)
// splits.  The wave walks its tokens 16 at a time ("groups"):
//
//   * K rows: lane l holds token (l % 16) of the group and the 16-byte
//     pieces [c*D/4, (c+1)*D/4) of its row, c = l / 16.  Those are exactly
//     the B operands of D/32 MFMA 16x16x32 bf16 instructions that compute
//     S = Q K^T for the group; each piece is a 16-byte global load and one
//     group of one page reads whole 128/256-byte rows.
//   * Q: the A operand has 16 rows; row m holds query head kvh*g + m % g,
//     so the g heads are replicated and every lane receives the scores of
//     all g heads for its own token (g = 1, 2, 4).
//   * Softmax: each lane keeps its own running max / sum per head (base-2,
//     scale * log2(e) folded in) and rescales lazily: only when some lane's
//     score exceeds its max by more than kTau, so p <= 2^kTau.  The result
//     is the same function; only the reference point of the exponentials
//     moves.
//   * PV: the V rows come in the same layout as K; each lane accumulates
//     p * v for its token into o[g][D/4] in fp32 (VALU FMAs).
//   * End of split: lanes holding the same dims are merged (max, rescale,
//     sum); a request with one split writes bf16 output directly, otherwise
//     the split writes (m, l, o) to the workspace and the last wave of the
//     (r, kvh) to finish -- found with one device-scope atomic counter --
//     merges the splits (flash-decoding) and resets the counter to zero.
//
// Bandwidth: every K/V byte of the context is read once; partials add
// splits * g * (D + 2) * 4 bytes per (r, kvh).

#include "pkv_common.h"

namespace {

using namespace pkv;

struct DecodeParams {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  const int32_t* seq_lens;
  uint16_t* out;
  int32_t* counters;  // [B * Hkv], zero between calls
  float* ws_m;        // [B * Hkv * n_split_max * g]
  float* ws_l;
  float* ws_o;        // [B * Hkv * n_split_max * g * D]
  int64_t num_pages;
  int32_t page_size;
  int32_t page_shift;
  int32_t pt_stride;
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t max_seq_len;
  int32_t split;
  int32_t n_split_max;
  float scale_log2;  // softmax_scale * log2(e)
};

constexpr float kTau = 8.0f;

__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 1));
  v = fmaxf(v, __shfl_xor(v, 2));
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  return v;
}

__device__ __forceinline__ float sum16(float v) {
  v += __shfl_xor(v, 1);
  v += __shfl_xor(v, 2);
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  return v;
}

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
  constexpr int KCH = D / 32;  // 16-byte pieces per lane per row == MFMAs per group
  constexpr int DL = D / 4;    // dims per lane

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * 4 + wave;
  const int split = (int)(unit % p.n_split_max);
  const int64_t rk = unit / p.n_split_max;
  if (rk >= (int64_t)p.num_seqs * p.num_kv_heads) return;
  const int kvh = (int)(rk % p.num_kv_heads);
  const int r = (int)(rk / p.num_kv_heads);
  const int j = lane & 15;  // token within the group
  const int c = lane >> 4;  // dim quarter

  uint16_t* out_rk = p.out + ((int64_t)r * p.num_q_heads + (int64_t)kvh * G) * D;
  int n = uniform(p.seq_lens[r]);
  n = n > p.max_seq_len ? p.max_seq_len : n;
  if (n <= 0) {
    if (split == 0)
      for (int i = lane; i < G * D / 8; i += 64)
        reinterpret_cast<uint4*>(out_rk)[i] = make_uint4(0, 0, 0, 0);
    return;
  }
  const int ns = (n + p.split - 1) / p.split;
  if (split >= ns) return;
  const int t_begin = split * p.split;
  const int t_end = min(n, t_begin + p.split);

  // Q fragments (A operand): row j holds head kvh*G + j % G.
  bf16x8 qa[KCH];
  {
    const uint16_t* qp =
        p.q + ((int64_t)r * p.num_q_heads + (int64_t)kvh * G + (j % G)) * D + c * DL;
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) qa[kk] = as_bf16x8(ld16(qp + 8 * kk));
  }

  // Page ids of the split, 64 logical pages per window (lane i holds one).
  const int32_t* pt = p.page_table + (int64_t)r * p.pt_stride;
  const int lp_last = (t_end - 1) >> p.page_shift;
  int lp_base = t_begin >> p.page_shift;
  auto load_window = [&](int base) {
    const int idx = base + lane;
    int v = idx <= lp_last ? pt[idx] : 0;
    return (v < 0 || (int64_t)v >= p.num_pages) ? 0 : v;  // keep accesses in the pool
  };
  int ptv = load_window(lp_base);

  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  const int64_t page_elems = row_elems << p.page_shift;
  const int lane_off = (j * p.num_kv_heads + kvh) * D + c * DL;

  auto group_offset = [&](int t0) -> int64_t {
    const int lp = t0 >> p.page_shift;
    if (lp - lp_base >= 64) {
      lp_base = lp;
      ptv = load_window(lp_base);
    }
    const int page = __builtin_amdgcn_readlane(ptv, lp - lp_base);
    return (int64_t)page * page_elems + (int64_t)(t0 & (p.page_size - 1)) * row_elems;
  };
  auto load_kv = [&](int64_t goff, int loff, uint4 (&kb)[KCH], uint4 (&vb)[KCH]) {
    const uint16_t* kp = p.k_cache + goff + loff;
    const uint16_t* vp = p.v_cache + goff + loff;
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) kb[kk] = ld16(kp + 8 * kk);
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) vb[kk] = ld16(vp + 8 * kk);
  };

  float o[G][DL];
  float m[G], l[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int i = 0; i < DL; ++i) o[h][i] = 0.f;
  }

  auto process = [&](const uint4 (&kb)[KCH], const uint4 (&vb)[KCH], int valid) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[kk], as_bf16x8(kb[kk]), acc, 0, 0, 0);
    float x[G];
    bool grow = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      x[h] = acc[h] * p.scale_log2;
      if (valid < 16) x[h] = j < valid ? x[h] : kNegInf;
      grow |= x[h] > m[h] + kTau;
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], x[h]);
        const float a = mn == kNegInf ? 0.f : fast_exp2(m[h] - mn);
        l[h] *= a;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[h][i] *= a;
        m[h] = mn;
      }
    }
    float pr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      pr[h] = fast_exp2(x[h] - m[h]);
      if (valid < 16) pr[h] = j < valid ? pr[h] : 0.f;
      l[h] += pr[h];
    }
    float v[DL];
#pragma unroll
    for (int kk = 0; kk < KCH; ++kk) {
      const uint32_t w[4] = {vb[kk].x, vb[kk].y, vb[kk].z, vb[kk].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[8 * kk + 2 * e] = bf16_lo(w[e]);
        v[8 * kk + 2 * e + 1] = bf16_hi(w[e]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < DL; ++i) o[h][i] = fmaf(pr[h], v[i], o[h][i]);
  };

  // Main loop: double-buffered register prefetch of whole groups.
  const int len = t_end - t_begin;
  const int tail = len & 15;
  const int nfull = len >> 4;
  uint4 kA[KCH], vA[KCH], kB[KCH], vB[KCH];
  int g = 0;
  if (nfull > 0) load_kv(group_offset(t_begin), lane_off, kA, vA);
  for (; g + 1 < nfull; g += 2) {
    load_kv(group_offset(t_begin + 16 * (g + 1)), lane_off, kB, vB);
    process(kA, vA, 16);
    if (g + 2 < nfull) load_kv(group_offset(t_begin + 16 * (g + 2)), lane_off, kA, vA);
    process(kB, vB, 16);
  }
  if (g < nfull) process(kA, vA, 16);
  if (tail) {
    // rows past the end are replaced by the last valid row (finite data),
    // and their probabilities are forced to zero
    const int jr = j < tail ? j : tail - 1;
    load_kv(group_offset(t_begin + 16 * nfull), (jr * p.num_kv_heads + kvh) * D + c * DL, kA,
            vA);
    process(kA, vA, tail);
  }

  // Merge the 16 token lanes that hold the same dims.
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float M = max16(m[h]);
    const float a = m[h] == kNegInf ? 0.f : fast_exp2(m[h] - M);
    m[h] = M;
    l[h] = sum16(l[h] * a);
#pragma unroll
    for (int i = 0; i < DL; ++i) o[h][i] = sum16(o[h][i] * a);
  }

  if (ns == 1) {
    if (j == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = 1.f / l[h];
        uint4* dst = reinterpret_cast<uint4*>(out_rk + h * D + c * DL);
#pragma unroll
        for (int q4 = 0; q4 < DL / 8; ++q4) {
          uint4 w;
          w.x = pack_bf16x2(o[h][8 * q4 + 0] * inv, o[h][8 * q4 + 1] * inv);
          w.y = pack_bf16x2(o[h][8 * q4 + 2] * inv, o[h][8 * q4 + 3] * inv);
          w.z = pack_bf16x2(o[h][8 * q4 + 4] * inv, o[h][8 * q4 + 5] * inv);
          w.w = pack_bf16x2(o[h][8 * q4 + 6] * inv, o[h][8 * q4 + 7] * inv);
          dst[q4] = w;
        }
      }
    }
    return;
  }

  // Partial (m, l, un-normalised o) of this split.
  const int64_t base = (rk * p.n_split_max + split) * G;
  if (j == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float4* dst = reinterpret_cast<float4*>(p.ws_o + (base + h) * D + c * DL);
#pragma unroll
      for (int q4 = 0; q4 < DL / 4; ++q4)
        dst[q4] = make_float4(o[h][4 * q4], o[h][4 * q4 + 1], o[h][4 * q4 + 2], o[h][4 * q4 + 3]);
    }
    if (c == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        p.ws_m[base + h] = m[h];
        p.ws_l[base + h] = l[h];
      }
    }
  }
  __threadfence();  // release the partial before counting this split as done
  int prev = 0;
  if (lane == 0) prev = atomicAdd(p.counters + rk, 1);
  prev = __shfl(prev, 0);
  if (prev != ns - 1) return;
  __threadfence();  // acquire every other split's partial

  // Last split of (r, kvh): merge all partials into the bf16 output.
  const int64_t rbase = rk * p.n_split_max * G;
#pragma unroll
  for (int it = 0; it < (G * D + 63) / 64; ++it) {
    const int idx = lane + 64 * it;
    if (idx < G * D) {
      const int h = idx / D;
      const int d = idx - h * D;
      float M = kNegInf;
      for (int s = 0; s < ns; ++s) M = fmaxf(M, p.ws_m[rbase + s * G + h]);
      float L = 0.f, O = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float w = fast_exp2(p.ws_m[rbase + s * G + h] - M);
        L = fmaf(p.ws_l[rbase + s * G + h], w, L);
        O = fmaf(p.ws_o[(rbase + s * G + h) * D + d], w, O);
      }
      out_rk[h * D + d] = to_bf16(O / L);
    }
  }
  if (lane == 0) p.counters[rk] = 0;
}

// ---- host side -------------------------------------------------------------

constexpr int64_t kTargetUnits = 8192;
constexpr int kMinAutoSplit = 256;

int32_t choose_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_seq_len,
                     int32_t split_tokens) {
  if (split_tokens != 0) return split_tokens;
  int32_t s = (max_seq_len + 15) / 16 * 16;
  const int64_t rk = (int64_t)num_seqs * num_kv_heads;
  while (s > kMinAutoSplit && rk * ((max_seq_len + s - 1) / s) < kTargetUnits)
    s = (s / 2 + 15) / 16 * 16;
  return s;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

struct WsLayout {
  size_t counters, m, l, o, total;
};

WsLayout ws_layout(int64_t rk, int64_t nsm, int g, int d) {
  WsLayout w;
  w.counters = 0;
  w.m = align256(rk * sizeof(int32_t));
  w.l = w.m + align256(rk * nsm * g * sizeof(float));
  w.o = w.l + align256(rk * nsm * g * sizeof(float));
  w.total = w.o + align256(rk * nsm * g * d * sizeof(float));
  return w;
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

template <int D, int G>
int launch_decode(const DecodeParams& p, int64_t blocks, hipStream_t s) {
  return pkv_host::launch(decode_kernel<D, G>, dim3((unsigned)blocks), dim3(256), s, p);
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
  const int64_t nsm = (max_seq_len + s - 1) / s;
  if (nsm <= 1 || num_seqs == 0) return 0;
  return ws_layout((int64_t)num_seqs * num_kv_heads, nsm, num_q_heads / num_kv_heads, head_dim)
      .total;
}

extern "C" int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                     int32_t page_size, int64_t num_pages,
                                     const int32_t* page_table, int32_t page_table_stride,
                                     const int32_t* seq_lens, int32_t num_seqs,
                                     int32_t max_seq_len, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     float softmax_scale, int32_t split_tokens, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv_host;
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                       split_tokens))
    return PKV_EINVAL;
  if (!finite_positive(softmax_scale)) return PKV_EINVAL;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !page_table || !seq_lens || !out) return PKV_EINVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PKV_EINVAL;
  if (num_pages <= 0 || page_table_stride <= 0) return PKV_EINVAL;
  if (!is_pow2_page(page_size)) return PKV_EUNSUPPORTED;
  if ((int64_t)page_table_stride * page_size < max_seq_len) return PKV_EINVAL;
  const int g = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128) return PKV_EUNSUPPORTED;
  if (g != 1 && g != 2 && g != 4) return PKV_EUNSUPPORTED;

  const int32_t split = choose_split(num_seqs, num_kv_heads, max_seq_len, split_tokens);
  const int64_t nsm = (max_seq_len + split - 1) / split;
  const int64_t rk = (int64_t)num_seqs * num_kv_heads;
  DecodeParams p = {};
  if (nsm > 1) {
    const WsLayout w = ws_layout(rk, nsm, g, head_dim);
    if (workspace_bytes < w.total) return PKV_ENOSPACE;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u)) return PKV_EINVAL;
    char* ws = static_cast<char*>(workspace);
    p.counters = reinterpret_cast<int32_t*>(ws + w.counters);
    p.ws_m = reinterpret_cast<float*>(ws + w.m);
    p.ws_l = reinterpret_cast<float*>(ws + w.l);
    p.ws_o = reinterpret_cast<float*>(ws + w.o);
  }
  const int64_t units = rk * nsm;
  const int64_t blocks = (units + 3) / 4;
  if (blocks > INT32_MAX) return PKV_EINVAL;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.page_table = page_table;
  p.seq_lens = seq_lens;
  p.out = static_cast<uint16_t*>(out);
  p.num_pages = num_pages;
  p.page_size = page_size;
  p.page_shift = log2_exact(page_size);
  p.pt_stride = page_table_stride;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.max_seq_len = max_seq_len;
  p.split = split;
  p.n_split_max = (int32_t)nsm;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 64) {
    if (g == 1) return launch_decode<64, 1>(p, blocks, s);
    if (g == 2) return launch_decode<64, 2>(p, blocks, s);
    return launch_decode<64, 4>(p, blocks, s);
  }
  if (g == 1) return launch_decode<128, 1>(p, blocks, s);
  if (g == 2) return launch_decode<128, 2>(p, blocks, s);
  return launch_decode<128, 4>(p, blocks, s);
}
