// Host-side checks of the C ABI, built together with the library's host code
// under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
// Every call here either is a pure host computation (sizes, split choice,
// status strings) or fails argument validation before anything is enqueued,
// so no GPU is needed; the fake device pointers are never dereferenced.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <limits>
#include <vector>

#include "pkv.h"
#include "pkv_ref.h"

static int failures = 0, checks = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    ++checks;                                                           \
    if (!(cond)) {                                                      \
      ++failures;                                                       \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
    }                                                                   \
  } while (0)

static void* const F = reinterpret_cast<void*>(uintptr_t(1) << 20);  // aligned, never read
static const int32_t* const FI = reinterpret_cast<const int32_t*>(uintptr_t(1) << 20);
static int32_t* const FO = reinterpret_cast<int32_t*>(uintptr_t(1) << 20);
static uint32_t* const FU = reinterpret_cast<uint32_t*>(uintptr_t(1) << 20);

int main() {
  const int32_t I32MAX = std::numeric_limits<int32_t>::max();

  for (int s = -2; s < 8; ++s) CHECK(pkv_strerror(s) != nullptr && strlen(pkv_strerror(s)) > 0);
  CHECK(strstr(pkv_version(), "gfx950") != nullptr);

  // Size and split queries over ordinary and extreme shapes: results must be
  // consistent (0 for invalid shapes) and the host arithmetic must not
  // overflow (UBSan aborts on signed overflow).
  const int32_t seqs[] = {0, 1, 7, 64, 1000, 1 << 20, I32MAX};
  const int32_t heads[][2] = {{32, 8}, {16, 8}, {8, 8}, {64, 8}, {4, 1}, {30, 8}, {I32MAX, 1}};
  const int32_t dims[] = {64, 128, 96, 0};
  const int32_t lens[] = {1, 15, 16, 2048, 131072, 1 << 24, I32MAX};
  const int32_t splits[] = {0, 16, 320, 65536, 65552, -16, 40};
  for (int32_t b : seqs)
    for (const auto& h : heads)
      for (int32_t d : dims)
        for (int32_t n : lens)
          for (int32_t sp : splits) {
            const size_t ws = pkv_decode_workspace_bytes(b, h[0], h[1], d, n, sp);
            const int32_t s = pkv_decode_split_tokens(b, h[1], n, sp);
            CHECK(s == 0 || (s >= 16 && s % 16 == 0));
            if (sp != 0 && s != 0) CHECK(s == sp);
            if (b == 0) CHECK(ws == 0);
            for (int32_t ql : {1, 4, 16, 17}) {
              const size_t wm = pkv_decode_multi_workspace_bytes(b, ql, h[0], h[1], d, n, sp);
              if (ql == 17) CHECK(wm == 0);
              if (ql == 1) CHECK(wm <= ws);  // plain decode may also hold balanced partials
            }
            for (int32_t shared : {0, 64, 1000}) {
              const size_t wsh =
                  pkv_paged_attn_decode_shared_workspace_bytes(b, h[0], h[1], d, n, shared, sp);
              if (shared > n) CHECK(wsh == 0);
            }
          }
  {
    const int32_t buckets[] = {1, 2, 4, 8, 16, 32, 64};
    CHECK(pkv_decode_graphs_workspace_bytes(buckets, 7, 32, 8, 64, 2048) >=
          pkv_decode_workspace_bytes(64, 32, 8, 64, 2048, 0));
    CHECK(pkv_decode_graphs_workspace_bytes(buckets, 0, 32, 8, 64, 2048) == 0);
    CHECK(pkv_decode_graphs_workspace_bytes(nullptr, 3, 32, 8, 64, 2048) == 0);
    const int32_t bad[] = {4, -1};
    CHECK(pkv_decode_graphs_workspace_bytes(bad, 2, 32, 8, 64, 2048) == 0);
  }
  CHECK(pkv_prefill_workspace_bytes() >= 4);
  CHECK(pkv_decode_step_noalloc_max_bytes() > 0);
  CHECK(pkv_ref_stream_sink_words(0) == 0 && pkv_ref_stream_sink_words(3) == 12);

  // Argument validation: each call fails before anything is enqueued.
  CHECK(pkv_store_kv(nullptr, F, FI, 4, F, F, 64, 8, 64, nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(F, F, FI, -1, F, F, 64, 8, 64, nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(F, F, FI, 4, F, F, 64, 8, 12, nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(F, F, FI, 4, F, F, 0, 8, 64, nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(nullptr, nullptr, nullptr, 0, F, F, 64, 8, 64, nullptr) == PKV_OK);
  // sizes whose piece or block counts overflow are rejected, not wrapped
  CHECK(pkv_store_kv(F, F, FI, std::numeric_limits<int64_t>::max() / 2, F, F, 64, 1 << 20, 128,
                     nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(F, F, FI, int64_t(1) << 40, F, F, 64, 8, 64, nullptr) == PKV_EINVAL);
  CHECK(pkv_store_kv(F, F, FI, 4, F, F, 64, I32MAX, 128, nullptr) == PKV_EINVAL);

  auto decode = [&](int32_t ps, int32_t stride, int32_t b, int32_t maxlen, int32_t hq, int32_t hkv,
                    int32_t d, float scale, int32_t split, void* ws, size_t wsb) {
    return pkv_paged_attn_decode(F, F, F, ps, 100, FI, stride, FI, b, maxlen, hq, hkv, d, scale,
                                 split, F, ws, wsb, nullptr);
  };
  CHECK(decode(16, 128, 4, 2048, 32, 8, 64, 0.125f, 0, nullptr, 0) == PKV_ENOSPACE);
  CHECK(decode(16, 128, 4, 2048, 30, 8, 64, 0.125f, 0, nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, 4, 2048, 32, 8, 96, 0.125f, 0, nullptr, 0) != PKV_OK);
  CHECK(decode(24, 128, 4, 2048, 32, 8, 64, 0.125f, 0, nullptr, 0) == PKV_EUNSUPPORTED);
  CHECK(decode(16, 8, 4, 2048, 32, 8, 64, 0.125f, 0, nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, 4, 2048, 32, 8, 64, -1.f, 0, nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, 4, 2048, 32, 8, 64, std::numeric_limits<float>::infinity(), 0, nullptr,
               0) == PKV_EINVAL);
  CHECK(decode(16, 128, 4, 2048, 32, 8, 64, std::numeric_limits<float>::quiet_NaN(), 0,
               nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, 4, 2048, 32, 8, 64, 0.125f, 40, nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, -1, 2048, 32, 8, 64, 0.125f, 0, nullptr, 0) == PKV_EINVAL);
  CHECK(decode(16, 128, 0, 2048, 32, 8, 64, 0.125f, 0, nullptr, 0) == PKV_OK);
  {
    const size_t need = pkv_decode_workspace_bytes(4, 32, 8, 64, 2048, 0);
    void* misaligned = reinterpret_cast<void*>((uintptr_t(1) << 20) + 16);
    CHECK(decode(16, 128, 4, 2048, 32, 8, 64, 0.125f, 0, misaligned, need) == PKV_EINVAL);
    CHECK(need > 256);
    CHECK(decode(16, 128, 4, 2048, 32, 8, 64, 0.125f, 0, F, 256) == PKV_ENOSPACE);
  }
  CHECK(pkv_decode_step(F, nullptr, F, FI, F, F, 16, 100, FI, 128, FI, 4, 2048, 32, 8, 64,
                        0.125f, 0, F, nullptr, 0, nullptr) == PKV_EINVAL);
  CHECK(pkv_decode_step_noalloc(F, F, F, FI, F, F, 16, 100, FI, 128, FI, 4, 2048, 30, 8, 64,
                                0.125f, 0, F, nullptr) == PKV_EINVAL);
  CHECK(pkv_paged_attn_decode_multi(F, 17, F, F, 16, 100, FI, 128, FI, 4, 2048, 32, 8, 64,
                                    0.125f, 0, F, nullptr, 0, nullptr) == PKV_EINVAL);
  CHECK(pkv_paged_attn_decode_multi(F, 0, F, F, 16, 100, FI, 128, FI, 4, 2048, 32, 8, 64, 0.125f,
                                    0, F, nullptr, 0, nullptr) == PKV_EINVAL);
  CHECK(pkv_paged_attn_decode_shared(F, nullptr, nullptr, nullptr, F, F, 16, 100, FI, 128, FI, 4,
                                     2048, nullptr, FI, 1, 4, 64, 32, 8, 64, 0.125f, 0, F,
                                     nullptr, 0, nullptr) == PKV_EINVAL);
  CHECK(pkv_paged_attn_decode_shared(F, nullptr, nullptr, nullptr, F, F, 16, 100, FI, 128, FI, 4,
                                     2048, FI, FI, 5, 4, 64, 32, 8, 64, 0.125f, 0, F, nullptr, 0,
                                     nullptr) == PKV_EINVAL);
  CHECK(pkv_paged_attn_decode_shared(F, nullptr, nullptr, nullptr, F, F, 16, 100, FI, 128, FI, 4,
                                     2048, FI, FI, 1, 4, 4096, 32, 8, 64, 0.125f, 0, F, nullptr,
                                     0, nullptr) == PKV_EINVAL);

  auto prefill = [&](int32_t b, int32_t t, int32_t maxq, int32_t maxlen, int32_t ps,
                     int32_t stride, int32_t hq, int32_t hkv, int32_t d, float scale, void* ws,
                     size_t wsb) {
    return pkv_paged_attn_prefill(F, FI, FI, b, t, maxq, maxlen, F, F, ps, 100, FI, stride, hq,
                                  hkv, d, scale, F, ws, wsb, nullptr);
  };
  CHECK(prefill(4, 100, 50, 1000, 16, 64, 32, 8, 64, 0.125f, F, 0) == PKV_ENOSPACE);
  CHECK(prefill(4, 100, 50, 1000, 16, 64, 32, 8, 64, 0.f, F, 256) == PKV_EINVAL);
  CHECK(prefill(4, 100, 50, 1000, 16, 8, 32, 8, 64, 0.125f, F, 256) == PKV_EINVAL);
  CHECK(prefill(4, 100, 50, 1000, 16, 64, 32, 8, 80, 0.125f, F, 256) != PKV_OK);
  CHECK(prefill(4, 100, 50, 1000, 48, 64, 32, 8, 64, 0.125f, F, 256) != PKV_OK);
  CHECK(prefill(-1, 100, 50, 1000, 16, 64, 32, 8, 64, 0.125f, F, 256) == PKV_EINVAL);
  CHECK(prefill(4, 0, 50, 1000, 16, 64, 32, 8, 64, 0.125f, nullptr, 0) == PKV_OK);
  // work-item counts beyond the ticket range are rejected (after the size
  // arithmetic, which must not overflow)
  CHECK(prefill(1 << 20, 1 << 30, I32MAX, I32MAX, 16, (1 << 27), 32, 8, 64, 0.125f, F, 256) ==
        PKV_EINVAL);
  CHECK(prefill(I32MAX, I32MAX, I32MAX, I32MAX, 256, (1 << 23), 8, 8, 128, 0.125f, F, 256) ==
        PKV_EINVAL);
  CHECK(prefill(4, 100, 50, 1000, 256, 64, 65536, 65536, 128, 0.125f, F, 256) ==
        PKV_EUNSUPPORTED);  // pages of 4 GiB

  CHECK(pkv_prefill_metadata(FI, FI, -1, FI, 8, 16, 10, FO, FO, nullptr) == PKV_EINVAL);
  CHECK(pkv_prefill_metadata(FI, FI, 4, FI, 0, 16, 10, FO, FO, nullptr) == PKV_EINVAL);
  CHECK(pkv_prefill_metadata(FI, FI, 4, FI, 8, 16, 10, FO, nullptr, nullptr) == PKV_EINVAL);
  CHECK(pkv_prefill_metadata(FI, FI, 0, FI, 8, 16, 10, FO, FO, nullptr) == PKV_OK);
  CHECK(pkv_decode_metadata(FI, 4, FI, 8, 0, FO, nullptr) == PKV_EINVAL);
  CHECK(pkv_decode_metadata(nullptr, 4, FI, 8, 16, FO, nullptr) == PKV_EINVAL);
  CHECK(pkv_decode_metadata(FI, 0, FI, 8, 16, FO, nullptr) == PKV_OK);

  {
    const int32_t buckets[] = {8, 4};
    pkv_decode_graphs* g = reinterpret_cast<pkv_decode_graphs*>(F);
    CHECK(pkv_decode_graphs_create(buckets, 0, F, F, F, FI, F, F, 16, 100, FI, 128, FI, 2048, 32,
                                   8, 64, 0.125f, F, nullptr, 0, &g) == PKV_EINVAL);
    CHECK(pkv_decode_graphs_create(buckets, 2, F, F, F, FI, F, F, 16, 100, FI, 128, FI, 2048, 30,
                                   8, 64, 0.125f, F, nullptr, 0, &g) == PKV_EINVAL);
    CHECK(pkv_decode_graphs_replay(nullptr, 4, nullptr, nullptr) == PKV_EINVAL);
    pkv_decode_graphs_destroy(nullptr);
  }
  CHECK(pkv_ref_stream_read(F, 1 << 20, 0, FU, nullptr) == PKV_EINVAL);
  CHECK(pkv_ref_stream_read(F, (1 << 20) + 8, 64, FU, nullptr) == PKV_EINVAL);
  CHECK(pkv_ref_stream_read(nullptr, 0, 64, nullptr, nullptr) == PKV_OK);

  printf("%d checks, %d failed\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
