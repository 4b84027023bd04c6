// Drives the C ABI's host code (argument validation, size arithmetic, the
// workspace protocol) with ordinary and extreme arguments, for a build under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// Pointers are fake, 256-byte-aligned addresses that validation never
// dereferences; every call returns before any launch (a device check fails
// first), so the statuses expected below are the host checks' own.
// Exit status 0 when every status matches.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/kvattn.h"

namespace {

int failures = 0, checks = 0;

void expect(int got, int want, const char* what, int line) {
  ++checks;
  if (got != want) {
    std::fprintf(stderr, "abi_driver.cpp:%d: %s -> %d, want %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

uint8_t* const P8 = reinterpret_cast<uint8_t*>(uintptr_t(1) << 20);
float* const PF = reinterpret_cast<float*>(P8);
int32_t* const PI = reinterpret_cast<int32_t*>(P8);

constexpr int OK = KVATTN_OK, INV = KVATTN_E_INVALID, UNS = KVATTN_E_UNSUPPORTED,
              WSP = KVATTN_E_WORKSPACE, DEV = KVATTN_E_DEVICE;

kvattn_geom geom(int32_t n_kv = 4, int32_t gqa = 6, int32_t n_phys = 64, int32_t v_type = 0,
                 int32_t k_type = 0) {
  return kvattn_geom{n_kv, gqa, KVATTN_HEAD_DIM, KVATTN_PAGE_TOKENS, n_phys, v_type, k_type};
}

int decode_query(const kvattn_geom& g, int32_t n_q_tok, int32_t n_logical, int64_t kv_len,
                 int32_t n_splits, size_t* bytes, const int32_t* blocks = nullptr,
                 int32_t n_blk = 0) {
  *bytes = 0;
  return kvattn_decode(&g, PF, n_q_tok, P8, P8, PI, n_logical, blocks, n_blk, kv_len, 0.0625f, PF,
                       PF, n_splits, nullptr, bytes, nullptr);
}

}  // namespace

int main() {
  // status strings and the selection count
  for (int s = -3; s < 8; ++s) EXPECT(kvattn_status_string(s) != nullptr, 1);
  EXPECT(kvattn_select_count(INT32_MAX, INT32_MAX, INT32_MAX), INT32_MAX);
  EXPECT(kvattn_select_count(INT32_MAX, 0, INT32_MAX), INT32_MAX);
  EXPECT(kvattn_select_count(INT32_MAX, 1, INT32_MAX), INT32_MAX);
  EXPECT(kvattn_select_count(0, 0, 0), -1);
  EXPECT(kvattn_select_count(5, INT32_MIN, 1), -1);

  // geometry
  size_t nb = 0;
  kvattn_geom g = geom();
  EXPECT(kvattn_decode(nullptr, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000, 0.0625f, PF, PF, 0,
                       nullptr, &nb, nullptr), INV);
  EXPECT(decode_query(geom(0), 1, 8, 1000, 0, &nb), INV);
  EXPECT(decode_query(geom(INT32_MAX, INT32_MAX), 1, 8, 1000, 0, &nb), INV);
  EXPECT(decode_query(geom(INT32_MAX, 1, INT32_MAX), 1, 8, 1000, 0, &nb), INV);
  EXPECT(decode_query(geom(4, 6, 64, 9), 1, 8, 1000, 0, &nb), UNS);
  EXPECT(decode_query(geom(4, 6, 64, 0, 9), 1, 8, 1000, 0, &nb), UNS);
  kvattn_geom bad = g;
  bad.head_dim = 128;
  EXPECT(decode_query(bad, 1, 8, 1000, 0, &nb), UNS);
  bad = g;
  bad.page_tokens = INT32_MIN;
  EXPECT(decode_query(bad, 1, 8, 1000, 0, &nb), UNS);

  // decode: the rows limit, kv_len bounds, workspace sizes at the extremes
  EXPECT(decode_query(g, INT32_MAX, 8, 1000, 0, &nb), UNS);         // n_q_tok * gqa overflows int32
  EXPECT(decode_query(geom(1, INT32_MAX, 1), 1, 8, 1000, 0, &nb), INV);  // n_kv * gqa > 2^20
  EXPECT(decode_query(g, 1, 8, INT64_MAX, 0, &nb), INV);
  EXPECT(decode_query(g, 1, 8, INT64_MIN, 0, &nb), INV);
  EXPECT(decode_query(g, 1, INT32_MAX, (int64_t)INT32_MAX * 128, 0, &nb), OK);
  EXPECT(nb > 0, 1);
  EXPECT(decode_query(g, 4, INT32_MAX, (int64_t)INT32_MAX * 128, INT32_MAX, &nb), OK);
  EXPECT(nb >= (size_t)INT32_MAX * 96 * 1028, 1);
  EXPECT(decode_query(g, 1, 8, 1000, -1, &nb), INV);
  EXPECT(decode_query(g, 1, 8, 1000, 0, &nb, PI, 0), INV);             // sparse with no blocks
  EXPECT(decode_query(g, 1, 8, 1000, 0, &nb, PI, INT32_MAX), OK);
  nb = 16;
  EXPECT(kvattn_decode(&g, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000, 0.0625f, PF, PF, 8, P8, &nb,
                       nullptr), WSP);
  EXPECT(kvattn_decode(&g, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000, __builtin_inff(), PF, PF, 0,
                       nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_decode_splits(&g, INT32_MAX) >= 1, 1);
  EXPECT(kvattn_decode_splits(&g, 0) >= 0, 1);
  EXPECT(kvattn_decode_partials(&g, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000, 0.0625f, 0, PF, PF,
                                nullptr), INV);
  EXPECT(kvattn_decode_partials(&g, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000, 0.0625f, INT32_MAX,
                                PF, PF, nullptr), DEV);

  // append + decode, with and without a workspace
  EXPECT(kvattn_append_decode(&g, PF, PF, INT32_MAX, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000,
                              0.0625f, nullptr, PF, PF, 0, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_append_decode(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0, INT64_MIN,
                              0.0625f, nullptr, PF, PF, 0, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_append_decode(&g, PF, PF, 4, PF, 4, P8, P8, PI, 8, nullptr, 0, 1000, 0.0625f, PF,
                              PF, PF, 0, nullptr, &nb, nullptr), OK);
  // append + partials, no merge
  EXPECT(kvattn_append_decode_partials(&g, PF, PF, INT32_MAX, PF, 1, P8, P8, PI, 8, nullptr, 0,
                                       1000, 0.0625f, nullptr, 8, PF, PF, nullptr), INV);
  EXPECT(kvattn_append_decode_partials(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0,
                                       INT64_MIN, 0.0625f, nullptr, 8, PF, PF, nullptr), INV);
  EXPECT(kvattn_append_decode_partials(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, PI, INT32_MAX,
                                       INT64_MAX, 0.0625f, nullptr, 8, PF, PF, nullptr), INV);
  EXPECT(kvattn_append_decode_partials(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000,
                                       0.0625f, nullptr, INT32_MIN, PF, PF, nullptr), INV);
  EXPECT(kvattn_append_decode_partials(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000,
                                       0.0625f, PF, INT32_MAX, PF, PF, nullptr), DEV);
  kvattn_geom big = geom(1 << 14, 8, 1 << 16);
  EXPECT(kvattn_append_decode_noalloc(&big, PF, PF, 1, PF, 4, P8, P8, PI, 1 << 16, nullptr, 0,
                                      (int64_t)128 << 16, 0.0625f, nullptr, PF, PF, 64, nullptr),
         WSP);
  EXPECT(kvattn_append_decode_noalloc(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000,
                                      0.0625f, nullptr, PF, PF, 0, nullptr), DEV);
  EXPECT(kvattn_append_decode_noalloc(&g, PF, PF, 1, PF, 1, P8, P8, PI, 8, nullptr, 0, 1000,
                                      0.0625f, nullptr, PF, PF, 8, nullptr), DEV);

  // quantisation: position bounds at the int64 extremes
  EXPECT(kvattn_quantize_pages(&g, PF, PF, INT64_MAX, 1, PI, 8, P8, P8, nullptr, nullptr), INV);
  EXPECT(kvattn_quantize_pages(&g, PF, PF, INT64_MAX, INT32_MAX, PI, INT32_MAX, P8, P8, nullptr,
                               nullptr), INV);
  EXPECT(kvattn_quantize_pages(&g, PF, PF, -1, 1, PI, 8, P8, P8, nullptr, nullptr), INV);
  EXPECT(kvattn_quantize_pages(&g, PF, PF, (int64_t)INT32_MAX * 128 - 1, 1, PI, INT32_MAX, P8, P8,
                               PF, nullptr), DEV);

  // selection
  EXPECT(kvattn_select_blocks(&g, PF, PF, INT32_MAX, INT32_MAX, INT32_MAX, INT32_MAX, PI, nullptr,
                              &nb, nullptr), OK);
  EXPECT(kvattn_select_blocks(&g, PF, PF, 8, 9, 0, 1, PI, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_select_blocks(&g, PF, PF, 8, 8, -1, 1, PI, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_select_blocks(&g, PF, PF, INT32_MAX, INT32_MAX, 0, 1, PI, nullptr, &nb, nullptr),
         OK);
  EXPECT(nb >= (size_t)INT32_MAX * 4 * 8, 1);

  // prefill: position bounds, group counts
  EXPECT(kvattn_prefill_chunk(&g, PF, INT32_MAX, P8, P8, PI, INT32_MAX, INT64_MAX, 0.0625f, PF,
                              PF, 0, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_prefill_chunk(&g, PF, 1, P8, P8, PI, 8, INT64_MAX, 0.0625f, PF, PF, 0, nullptr,
                              &nb, nullptr), INV);
  EXPECT(kvattn_prefill_chunk(&g, PF, 512, P8, P8, PI, INT32_MAX, (int64_t)INT32_MAX * 128 - 512,
                              0.0625f, PF, PF, 0, nullptr, &nb, nullptr), OK);
  // partials beyond any memory (2^24 groups x 2^35 rows x 1 KB): rejected
  EXPECT(kvattn_prefill_chunk(&g, PF, INT32_MAX, P8, P8, PI, INT32_MAX, 0, 0.0625f, PF, PF,
                              INT32_MAX, nullptr, &nb, nullptr), INV);
  EXPECT(kvattn_prefill_partials(&g, PF, 1, P8, P8, PI, 8, INT64_MAX, 0.0625f, 1, PF, PF,
                                 nullptr), INV);
  EXPECT(kvattn_prefill_range_partials(&g, PF, 512, P8, P8, PI, INT32_MAX,
                                       (int64_t)INT32_MAX * 128 - 512, 0.0625f, 0, INT32_MAX, 1,
                                       PF, PF, nullptr), DEV);
  EXPECT(kvattn_prefill_range_partials(&g, PF, 1, P8, P8, PI, 8, INT64_MAX, 0.0625f, 0, 1, 1,
                                       PF, PF, nullptr), INV);
  EXPECT(kvattn_prefill_range_partials(&g, PF, 100, P8, P8, PI, 16, 1000, 0.0625f, INT32_MIN, 2,
                                       1, PF, PF, nullptr), INV);
  EXPECT(kvattn_prefill_groups(&g, INT32_MAX, INT64_MAX) >= 0, 1);
  EXPECT(kvattn_prefill_groups(&g, 512, (int64_t)1 << 40) >= 1, 1);
  EXPECT(kvattn_prefill_groups(&g, 0, 0), 0);

  // merge, rotation, gather, prefetch
  EXPECT(kvattn_merge_lse(1, INT64_MAX, 256, PF, PF, PF, PF, nullptr), INV);
  EXPECT(kvattn_merge_lse(INT32_MAX, 1, INT32_MAX, PF, PF, PF, PF, nullptr), DEV);
  EXPECT(kvattn_merge_lse(0, 1, 256, PF, PF, PF, PF, nullptr), INV);
  EXPECT(kvattn_rotate_rows(PF, INT64_MAX, nullptr), INV);
  EXPECT(kvattn_rotate_rows(PF, -1, nullptr), INV);
  EXPECT(kvattn_rotate_rows(nullptr, 0, nullptr), DEV);
  EXPECT(kvattn_gather_blocks(&g, P8, P8, PI, 8, PI, 4, 5, P8, P8, PI, nullptr), INV);
  EXPECT(kvattn_gather_blocks(&g, P8, P8, PI, 8, PI, INT32_MAX, INT32_MAX, P8, P8, PI, nullptr),
         DEV);
  const int32_t pages_ok[3] = {0, 1, 63}, pages_bad[2] = {0, 64}, pages_neg[1] = {INT32_MIN};
  EXPECT(kvattn_prefetch_pages(&g, P8, P8, P8, P8, pages_bad, 2, nullptr), INV);
  EXPECT(kvattn_prefetch_pages(&g, P8, P8, P8, P8, pages_neg, 1, nullptr), INV);
  EXPECT(kvattn_prefetch_pages(&g, P8, P8, P8, P8, nullptr, 0, nullptr), OK);
  EXPECT(kvattn_prefetch_pages(&g, P8, P8, P8, P8, pages_ok, 3, nullptr), DEV);

  std::printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
