// C ABI of libkvattn: argument validation, device checks, workspace sizing
// and kernel launches. The operations and the pool layout are specified in
// include/kvattn.h; every check here runs on the host before anything is
// enqueued, and no path falls back to the CPU.
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/kvattn.h"
#include "launch.hpp"

using namespace kvattn;

// Scratch of kvattn_append_decode_noalloc: the split-K partials of the entry
// point that allocates nothing live in this file-scope array, one copy per
// GPU at its own address, held until the process ends. In host code `scratch`
// names a host-side stand-in, never the device memory: it is used only
// through the per-device address that hipGetSymbolAddress returns. Calls on
// one GPU share the array; calls that overlap on one GPU (other streams,
// other threads) race.
static __device__ __align__(256) uint8_t scratch[KVATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr float kLog2e = 1.4426950408889634f;  // softmax runs in base 2 on the device

struct DeviceInfo {
  std::atomic<int> state{0};  // 0 unknown, 1 gfx950, 2 other arch
  int n_cu = 0;
};
DeviceInfo g_devices[kMaxDevices];

// Checks (once per device) that the current device is gfx950: a code object
// for another architecture is never silently used (the KVMem report,
// section on the HIP general-protection fault, shows a missing gfx target
// crashing without an error).
kvattn_status current_device(int* n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return KVATTN_E_DEVICE;
  }
  DeviceInfo& info = g_devices[dev];
  int s = info.state.load(std::memory_order_acquire);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return KVATTN_E_DEVICE;
    }
    info.n_cu = prop.multiProcessorCount;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    info.state.store(s, std::memory_order_release);
  }
  if (s != 1) return KVATTN_E_UNSUPPORTED;
  if (n_cu) *n_cu = info.n_cu > 0 ? info.n_cu : 256;
  return KVATTN_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The address a kernel reads `p` through: device memory as is, pinned host
// memory (hipHostMalloc) through its device mapping. Pageable host memory and
// unknown pointers are rejected, so a kernel never dereferences them.
kvattn_status device_view(const void* p, const void** out) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return KVATTN_E_INVALID;
  }
  if (a.type == hipMemoryTypeDevice) {
    *out = p;
    return KVATTN_OK;
  }
  if (a.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || !d) {
      (void)hipGetLastError();
      return KVATTN_E_INVALID;
    }
    *out = d;
    return KVATTN_OK;
  }
  return KVATTN_E_INVALID;
}

kvattn_status check_geom(const kvattn_geom* g) {
  if (!g) return KVATTN_E_INVALID;
  if (g->n_kv_heads < 1 || g->gqa < 1 || g->n_phys_pages < 1) return KVATTN_E_INVALID;
  if (g->head_dim != KVATTN_HEAD_DIM || g->page_tokens != KVATTN_PAGE_TOKENS)
    return KVATTN_E_UNSUPPORTED;
  if ((int64_t)g->n_kv_heads * g->gqa > (1 << 20)) return KVATTN_E_INVALID;
  if ((int64_t)g->n_phys_pages * g->n_kv_heads > INT32_MAX) return KVATTN_E_INVALID;  // record index
  if (g->v_type != KVATTN_V_Q4_0 && g->v_type != KVATTN_V_Q8_0) return KVATTN_E_UNSUPPORTED;
  if (g->k_type != KVATTN_K_Q8_0 && g->k_type != KVATTN_K_Q4_0 && g->k_type != KVATTN_K_Q5_1)
    return KVATTN_E_UNSUPPORTED;
  return KVATTN_OK;
}

// Bytes of one (page, KV head) key record for the geometry's key type.
size_t k_record_bytes(const kvattn_geom* g) {
  return g->k_type == KVATTN_K_Q4_0   ? KVATTN_K4_RECORD_BYTES
         : g->k_type == KVATTN_K_Q5_1 ? KVATTN_K5_RECORD_BYTES
                                      : KVATTN_K_RECORD_BYTES;
}

// Bytes of one (page, KV head) value record for the geometry's value type.
size_t v_record_bytes(const kvattn_geom* g) {
  return g->v_type == KVATTN_V_Q8_0 ? KVATTN_V8_RECORD_BYTES : KVATTN_V_RECORD_BYTES;
}

kvattn_status check_pools(const kvattn_geom* g, const uint8_t* k_pool, const uint8_t* v_pool) {
  if (!k_pool || !v_pool || !aligned(k_pool, 256) || !aligned(v_pool, 256))
    return KVATTN_E_INVALID;
  return KVATTN_OK;
}

size_t round_up(size_t x) { return (x + 255) & ~size_t(255); }

// a * b * c rounded up to 256, or 0 when the product does not fit in half of
// size_t (the caller rejects such a call as invalid).
size_t checked_bytes(uint64_t a, uint64_t b, uint64_t c) {
  uint64_t ab = 0, abc = 0;
  if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc) ||
      abc > (uint64_t)(SIZE_MAX >> 1))
    return 0;
  return round_up((size_t)abc);
}

// Whether positions [pos0, pos0 + n) fit in n_logical_pages pages, with no
// overflow for any pos0 >= 0 and n >= 1.
bool fits_pages(int64_t pos0, int64_t n, int32_t n_logical_pages) {
  return pos0 <= (int64_t)n_logical_pages * KVATTN_PAGE_TOKENS - n;
}

// Every workspace starts with kSyncBytes of counters: zero before the first
// call that uses the workspace, and left zero by every call. Word 0 is the
// error word (bit 0: a prefill launch's bounded waits gave up).
constexpr size_t kSyncBytes = 2048;


kvattn_status launched(hipError_t e) {
  if (e != hipSuccess) return KVATTN_E_DEVICE;
  if (hipGetLastError() != hipSuccess) return KVATTN_E_DEVICE;
  return KVATTN_OK;
}

// Workspace protocol shared by every entry point that needs one.
kvattn_status workspace_check(void* workspace, size_t* workspace_bytes, size_t need,
                              bool* query_only) {
  *query_only = false;
  if (!workspace_bytes) return KVATTN_E_INVALID;
  if (!workspace) {
    *workspace_bytes = need;
    *query_only = true;
    return KVATTN_OK;
  }
  if (*workspace_bytes < need) return KVATTN_E_WORKSPACE;
  if (!aligned(workspace, 256)) return KVATTN_E_INVALID;
  return KVATTN_OK;
}

}  // namespace

extern "C" {

const char* kvattn_status_string(kvattn_status s) {
  switch (s) {
    case KVATTN_OK: return "ok";
    case KVATTN_E_INVALID: return "invalid argument";
    case KVATTN_E_UNSUPPORTED: return "unsupported shape or device";
    case KVATTN_E_WORKSPACE: return "workspace too small";
    case KVATTN_E_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

int32_t kvattn_select_count(int32_t n_blocks, int32_t n_recent, int32_t k_top) {
  if (n_blocks < 1 || n_recent < 0 || k_top < 0) return -1;
  const int32_t r = n_recent < n_blocks ? n_recent : n_blocks;
  const int32_t cand = n_blocks - r;
  return (k_top < cand ? k_top : cand) + r;
}

kvattn_status kvattn_quantize_pages(const kvattn_geom* geom, const float* k, const float* v,
                                    int64_t pos0, int32_t n_tok, const int32_t* page_table,
                                    int32_t n_logical_pages, uint8_t* k_pool, uint8_t* v_pool,
                                    float* k_summary, void* stream) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if ((st = check_pools(geom, k_pool, v_pool))) return st;
  if (!k || !v || !page_table || !aligned(k, 16) || !aligned(v, 16)) return KVATTN_E_INVALID;
  if (k_summary && !aligned(k_summary, 16)) return KVATTN_E_INVALID;
  if (pos0 < 0 || n_tok < 1 || n_logical_pages < 1) return KVATTN_E_INVALID;
  if (!fits_pages(pos0, n_tok, n_logical_pages)) return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launched(launch_quantize(k, v, pos0, n_tok, geom->n_kv_heads, page_table,
                                geom->n_phys_pages, k_pool, v_pool,
                                geom->v_type == KVATTN_V_Q8_0, geom->k_type, s));
  if (st || !k_summary) return st;
  const int64_t first = pos0 / KVATTN_PAGE_TOKENS;
  const int64_t last_full = (pos0 + n_tok) / KVATTN_PAGE_TOKENS - 1;
  if (last_full < first) return KVATTN_OK;
  return launched(launch_summarize(k_pool, page_table, geom->n_kv_heads, geom->n_phys_pages,
                                   n_logical_pages, (int32_t)first,
                                   (int32_t)(last_full - first + 1), k_summary,
                                   geom->k_type, s));
}

kvattn_status kvattn_select_blocks(const kvattn_geom* geom, const float* q,
                                   const float* k_summary, int32_t n_logical_pages,
                                   int32_t n_blocks, int32_t n_recent, int32_t k_top,
                                   int32_t* out_blocks, void* workspace,
                                   size_t* workspace_bytes, void* stream) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if (n_blocks < 1 || n_blocks > n_logical_pages || n_recent < 0 || k_top < 0)
    return KVATTN_E_INVALID;
  if (!q || !k_summary || !out_blocks || !aligned(q, 16) || !aligned(k_summary, 16))
    return KVATTN_E_INVALID;
  const int32_t r = n_recent < n_blocks ? n_recent : n_blocks;
  const int32_t n_cand = n_blocks - r;
  const int32_t k_sel = k_top < n_cand ? k_top : n_cand;
  const int32_t n_out = k_sel + r;
  const size_t need =
      kSyncBytes + round_up(sizeof(double) * (size_t)geom->n_kv_heads * (size_t)n_cand);
  bool query_only = false;
  if ((st = workspace_check(workspace, workspace_bytes, need, &query_only))) return st;
  if (query_only) return KVATTN_OK;
  if ((st = current_device(nullptr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  double* scores = reinterpret_cast<double*>(static_cast<uint8_t*>(workspace) + kSyncBytes);
  if (k_sel > 0 && k_sel < n_cand) {
    if ((st = launched(launch_score(q, k_summary, geom->n_kv_heads, geom->gqa, n_logical_pages,
                                    n_cand, scores, s))))
      return st;
  }
  return launched(launch_topk(k_sel > 0 && k_sel < n_cand ? scores : nullptr, geom->n_kv_heads,
                              n_cand, k_sel, r, n_out, out_blocks, s));
}

}  // extern "C"

namespace {

kvattn_status check_scale(float scale) {
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return KVATTN_E_INVALID;
  return KVATTN_OK;
}

// Validation shared by kvattn_decode and kvattn_decode_partials; n_units is
// the number of pages (dense) or listed blocks (sparse) the splits divide.
kvattn_status check_decode(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                           const uint8_t* k_pool, const uint8_t* v_pool,
                           const int32_t* page_table, int32_t n_logical_pages,
                           const int32_t* blocks, int32_t n_blk, int64_t kv_len, float scale,
                           int32_t* n_units) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if ((st = check_pools(geom, k_pool, v_pool))) return st;
  if (!q || !page_table || !aligned(q, 16)) return KVATTN_E_INVALID;
  if (n_q_tok < 1 || n_logical_pages < 1) return KVATTN_E_INVALID;
  if ((int64_t)n_q_tok * geom->gqa > KVATTN_MAX_QUERY_ROWS) return KVATTN_E_UNSUPPORTED;
  if (kv_len < n_q_tok || kv_len > (int64_t)n_logical_pages * KVATTN_PAGE_TOKENS)
    return KVATTN_E_INVALID;
  if (blocks && n_blk < 1) return KVATTN_E_INVALID;
  if ((st = check_scale(scale))) return st;
  *n_units = blocks ? n_blk : (int32_t)((kv_len + KVATTN_PAGE_TOKENS - 1) / KVATTN_PAGE_TOKENS);
  return KVATTN_OK;
}

// Splits per KV head chosen by the library: two resident workgroups per CU
// (the decode kernel is built for two waves per SIMD), spread over the KV
// heads, at most one per unit.
int32_t auto_decode_splits(int32_t n_kv, int32_t n_units, int n_cu) {
  int32_t splits = (DECODE_WGS_PER_CU * n_cu + n_kv - 1) / n_kv;
  if (splits > n_units) splits = n_units;
  return splits < 1 ? 1 : splits;
}

// The tokens kvattn_append_decode quantises inside the decode launch.
struct AppendArgs {
  const float* k_new;
  const float* v_new;
  uint8_t* k_pool;
  uint8_t* v_pool;
  int32_t n_new;
  float* k_summary;  // when not NULL: the summary of a page the append completes
};

kvattn_status launch_decode_partials(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                                     const uint8_t* k_pool, const uint8_t* v_pool,
                                     const int32_t* page_table, int32_t n_logical_pages,
                                     const int32_t* blocks, int32_t n_blk, int64_t kv_len,
                                     float scale, int32_t n_units, int32_t splits, float* o_part,
                                     float* lse_part, hipStream_t s,
                                     const AppendArgs* app = nullptr) {
  DecodeParams p;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.page_table = page_table;
  p.blocks = blocks;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.kv_len = kv_len;
  p.n_units = n_units;
  p.n_splits = splits;
  p.n_kv = geom->n_kv_heads;
  p.gqa = geom->gqa;
  p.n_q_tok = n_q_tok;
  p.n_logical = n_logical_pages;
  p.n_phys = geom->n_phys_pages;
  p.n_blk = blocks ? n_blk : 0;
  p.qscale = scale * kLog2e;
  p.k_new = app ? app->k_new : nullptr;
  p.v_new = app ? app->v_new : nullptr;
  p.k_pool_w = app ? app->k_pool : nullptr;
  p.v_pool_w = app ? app->v_pool : nullptr;
  p.n_new = app ? app->n_new : 0;
  p.v_q8 = geom->v_type == KVATTN_V_Q8_0;
  p.k_type = geom->k_type;
  // the appended positions kv_len - n_new .. kv_len - 1 (n_new <= 32 < 128)
  // complete at most one page: the one ending at a multiple of 128 among them
  p.sum_page = -1;
  p.k_summary = app ? app->k_summary : nullptr;
  if (app && app->k_summary && kv_len / KVATTN_PAGE_TOKENS > (kv_len - app->n_new) / KVATTN_PAGE_TOKENS)
    p.sum_page = (int32_t)(kv_len / KVATTN_PAGE_TOKENS - 1);
  return launched(launch_decode(p, s));
}

kvattn_status check_prefill(const kvattn_geom* geom, const float* q, int32_t chunk,
                            const uint8_t* k_pool, const uint8_t* v_pool,
                            const int32_t* page_table, int32_t n_logical_pages, int64_t pos0,
                            float scale) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if ((st = check_pools(geom, k_pool, v_pool))) return st;
  if (!q || !page_table || !aligned(q, 16)) return KVATTN_E_INVALID;
  if (chunk < 1 || pos0 < 0 || n_logical_pages < 1) return KVATTN_E_INVALID;
  if (!fits_pages(pos0, chunk, n_logical_pages)) return KVATTN_E_INVALID;
  return check_scale(scale);
}

// Page groups chosen by the library: about three rounds of the grid, at most
// one group per page.
int32_t auto_prefill_groups(const kvattn_geom* geom, int32_t chunk, int64_t pos0, int n_cu) {
  // ceil((pos0 + chunk) / 128) without forming pos0 + chunk
  const int64_t n_pages = pos0 / KVATTN_PAGE_TOKENS +
                          (pos0 % KVATTN_PAGE_TOKENS + chunk + KVATTN_PAGE_TOKENS - 1) /
                              KVATTN_PAGE_TOKENS;
  const int64_t rows_per_head = (int64_t)chunk * geom->gqa;
  const int64_t tiles =
      geom->n_kv_heads * ((rows_per_head + prefill_rows_per_tile() - 1) / prefill_rows_per_tile());
  int64_t gr = (3 * (int64_t)n_cu + tiles - 1) / tiles;
  if (gr > n_pages) gr = n_pages;
  return gr < 1 ? 1 : (int32_t)gr;
}

kvattn_status launch_prefill_partials(const kvattn_geom* geom, const float* q, int32_t chunk,
                                      const uint8_t* k_pool, const uint8_t* v_pool,
                                      const int32_t* page_table, int32_t n_logical_pages,
                                      int64_t pos0, float scale, int32_t groups, float* o_part,
                                      float* lse_part, hipStream_t s, uint32_t* flag = nullptr,
                                      int32_t pg_begin = 0, int32_t pg_end = -1) {
  PrefillParams p;
  p.pg_begin = pg_begin;
  p.pg_end = pg_end >= 0 ? pg_end
                         : (int32_t)((pos0 + chunk + KVATTN_PAGE_TOKENS - 1) / KVATTN_PAGE_TOKENS);
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.page_table = page_table;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.pos0 = pos0;
  p.chunk = chunk;
  p.n_groups = groups;
  p.n_kv = geom->n_kv_heads;
  p.gqa = geom->gqa;
  p.n_logical = n_logical_pages;
  p.n_phys = geom->n_phys_pages;
  p.qscale = scale * kLog2e;
  p.v_q8 = geom->v_type == KVATTN_V_Q8_0;
  p.k_type = geom->k_type;
  p.flag = flag;
  return launched(launch_prefill(p, s));
}

}  // namespace

extern "C" {

int32_t kvattn_decode_splits(const kvattn_geom* geom, int32_t n_units) {
  if (check_geom(geom) != KVATTN_OK || n_units < 1) return 0;
  int n_cu = 256;
  if (current_device(&n_cu) != KVATTN_OK) n_cu = 256;
  return auto_decode_splits(geom->n_kv_heads, n_units, n_cu);
}

}  // extern "C"

namespace {

// Split count, rows and partial sizes of one decode call.
struct DecodePlan {
  int32_t n_units = 0, splits = 0;
  int64_t rows = 0;
  size_t o_bytes = 0, lse_bytes = 0;
};

// Validates a decode call and sizes its partials. `need_device`: the split
// count must come from the current device's CU count (a launch); otherwise
// (a workspace query) a machine without a device sizes for 256 CUs, and the
// launch recomputes with the real count, so query and launch must run on the
// same device.
kvattn_status decode_plan(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                          const uint8_t* k_pool, const uint8_t* v_pool,
                          const int32_t* page_table, int32_t n_logical_pages,
                          const int32_t* blocks, int32_t n_blk, int64_t kv_len, float scale,
                          float* out, float* lse, int32_t n_splits, bool need_device,
                          DecodePlan* plan) {
  kvattn_status st = check_decode(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                  blocks, n_blk, kv_len, scale, &plan->n_units);
  if (st) return st;
  if (!out || !lse || !aligned(out, 16) || n_splits < 0) return KVATTN_E_INVALID;
  int32_t splits = n_splits;
  if (splits == 0) {
    int n_cu = 256;
    if (need_device && (st = current_device(&n_cu))) return st;
    if (!need_device && current_device(&n_cu) != KVATTN_OK) n_cu = 256;
    splits = auto_decode_splits(geom->n_kv_heads, plan->n_units, n_cu);
  }
  if (splits > plan->n_units) splits = plan->n_units;
  plan->splits = splits;
  plan->rows = (int64_t)n_q_tok * geom->n_kv_heads * geom->gqa;
  plan->o_bytes = checked_bytes(splits, plan->rows, sizeof(float) * KVATTN_HEAD_DIM);
  plan->lse_bytes = checked_bytes(splits, plan->rows, sizeof(float));
  if (!plan->o_bytes || !plan->lse_bytes) return KVATTN_E_INVALID;  // beyond any memory
  return KVATTN_OK;
}

// The decode kernel into o_part / lse_part, then the merge.
kvattn_status decode_launch(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                            const uint8_t* k_pool, const uint8_t* v_pool,
                            const int32_t* page_table, int32_t n_logical_pages,
                            const int32_t* blocks, int32_t n_blk, int64_t kv_len, float scale,
                            float* out, float* lse, const DecodePlan& plan, float* o_part,
                            float* lse_part, void* stream, const AppendArgs* app) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kvattn_status st =
      launch_decode_partials(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                             blocks, n_blk, kv_len, scale, plan.n_units, plan.splits, o_part,
                             lse_part, s, app);
  if (st) return st;
  return launched(launch_merge(plan.splits, plan.rows, KVATTN_HEAD_DIM, o_part, lse_part, out,
                               lse, s));
}

// kvattn_decode, with the fused append when `app` is given.
kvattn_status decode_impl(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                          const uint8_t* k_pool, const uint8_t* v_pool,
                          const int32_t* page_table, int32_t n_logical_pages,
                          const int32_t* blocks, int32_t n_blk, int64_t kv_len, float scale,
                          float* out, float* lse, int32_t n_splits, void* workspace,
                          size_t* workspace_bytes, void* stream, const AppendArgs* app) {
  DecodePlan plan;
  kvattn_status st = decode_plan(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                 blocks, n_blk, kv_len, scale, out, lse, n_splits,
                                 workspace != nullptr, &plan);
  if (st) return st;
  const size_t need = kSyncBytes + plan.o_bytes + plan.lse_bytes;
  bool query_only = false;
  if ((st = workspace_check(workspace, workspace_bytes, need, &query_only))) return st;
  if (query_only) return KVATTN_OK;
  if ((st = current_device(nullptr))) return st;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  return decode_launch(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages, blocks,
                       n_blk, kv_len, scale, out, lse, plan,
                       reinterpret_cast<float*>(ws + kSyncBytes),
                       reinterpret_cast<float*>(ws + kSyncBytes + plan.o_bytes), stream, app);
}

// The current device's copy of `scratch` (above), found once per device.
struct ScratchAddress {
  std::atomic<uint8_t*> ptr{nullptr};
  std::mutex init;
};
ScratchAddress g_scratch[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current) on its first use.
kvattn_status scratch_address(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return KVATTN_E_DEVICE;
  }
  ScratchAddress& a = g_scratch[dev];
  uint8_t* p = a.ptr.load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(a.init);
    p = a.ptr.load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        (void)hipGetLastError();
        return KVATTN_E_DEVICE;
      }
      p = static_cast<uint8_t*>(addr);
      a.ptr.store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVATTN_OK;
}

}  // namespace

extern "C" {

kvattn_status kvattn_decode(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                            const uint8_t* k_pool, const uint8_t* v_pool,
                            const int32_t* page_table, int32_t n_logical_pages,
                            const int32_t* blocks, int32_t n_blk, int64_t kv_len, float scale,
                            float* out, float* lse, int32_t n_splits, void* workspace,
                            size_t* workspace_bytes, void* stream) {
  return decode_impl(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages, blocks, n_blk,
                     kv_len, scale, out, lse, n_splits, workspace, workspace_bytes, stream, nullptr);
}

kvattn_status kvattn_append_decode(const kvattn_geom* geom, const float* k_new, const float* v_new,
                                   int32_t n_new, const float* q, int32_t n_q_tok,
                                   uint8_t* k_pool, uint8_t* v_pool, const int32_t* page_table,
                                   int32_t n_logical_pages, const int32_t* blocks, int32_t n_blk,
                                   int64_t kv_len, float scale, float* k_summary, float* out,
                                   float* lse, int32_t n_splits, void* workspace,
                                   size_t* workspace_bytes, void* stream) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVATTN_E_INVALID;
  if (n_new < 1 || n_new > KVATTN_MAX_APPEND_TOKENS || n_new > kv_len) return KVATTN_E_INVALID;
  if (k_summary && !aligned(k_summary, 16)) return KVATTN_E_INVALID;
  // the summary of a page the append completes is written by the decode
  // launch itself, from the updated pool
  const AppendArgs app{k_new, v_new, k_pool, v_pool, n_new, k_summary};
  return decode_impl(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages, blocks, n_blk,
                     kv_len, scale, out, lse, n_splits, workspace, workspace_bytes, stream, &app);
}

kvattn_status kvattn_append_decode_noalloc(const kvattn_geom* geom, const float* k_new,
                                           const float* v_new, int32_t n_new, const float* q,
                                           int32_t n_q_tok, uint8_t* k_pool, uint8_t* v_pool,
                                           const int32_t* page_table, int32_t n_logical_pages,
                                           const int32_t* blocks, int32_t n_blk, int64_t kv_len,
                                           float scale, float* k_summary, float* out, float* lse,
                                           int32_t n_splits, void* stream) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVATTN_E_INVALID;
  if (n_new < 1 || n_new > KVATTN_MAX_APPEND_TOKENS || n_new > kv_len) return KVATTN_E_INVALID;
  if (k_summary && !aligned(k_summary, 16)) return KVATTN_E_INVALID;
  DecodePlan plan;
  kvattn_status st = decode_plan(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                 blocks, n_blk, kv_len, scale, out, lse, n_splits, true, &plan);
  if (st) return st;
  // every partial is written by the decode kernel before the merge reads it,
  // so nothing in the scratch needs clearing between calls
  if (plan.o_bytes + plan.lse_bytes > KVATTN_NOALLOC_SCRATCH_BYTES) return KVATTN_E_WORKSPACE;
  if ((st = current_device(nullptr))) return st;
  uint8_t* base = nullptr;
  if ((st = scratch_address(&base))) return st;
  const AppendArgs app{k_new, v_new, k_pool, v_pool, n_new, k_summary};
  return decode_launch(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages, blocks,
                       n_blk, kv_len, scale, out, lse, plan, reinterpret_cast<float*>(base),
                       reinterpret_cast<float*>(base + plan.o_bytes), stream, &app);
}

kvattn_status kvattn_decode_partials(const kvattn_geom* geom, const float* q, int32_t n_q_tok,
                                     const uint8_t* k_pool, const uint8_t* v_pool,
                                     const int32_t* page_table, int32_t n_logical_pages,
                                     const int32_t* blocks, int32_t n_blk, int64_t kv_len,
                                     float scale, int32_t n_splits, float* o_part,
                                     float* lse_part, void* stream) {
  int32_t n_units = 0;
  kvattn_status st = check_decode(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                  blocks, n_blk, kv_len, scale, &n_units);
  if (st) return st;
  if (!o_part || !lse_part || !aligned(o_part, 16) || n_splits < 1) return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  return launch_decode_partials(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                blocks, n_blk, kv_len, scale, n_units, n_splits, o_part, lse_part,
                                static_cast<hipStream_t>(stream));
}

kvattn_status kvattn_append_decode_partials(const kvattn_geom* geom, const float* k_new,
                                            const float* v_new, int32_t n_new, const float* q,
                                            int32_t n_q_tok, uint8_t* k_pool, uint8_t* v_pool,
                                            const int32_t* page_table, int32_t n_logical_pages,
                                            const int32_t* blocks, int32_t n_blk, int64_t kv_len,
                                            float scale, float* k_summary, int32_t n_splits,
                                            float* o_part, float* lse_part, void* stream) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return KVATTN_E_INVALID;
  if (n_new < 1 || n_new > KVATTN_MAX_APPEND_TOKENS || n_new > kv_len) return KVATTN_E_INVALID;
  if (k_summary && !aligned(k_summary, 16)) return KVATTN_E_INVALID;
  int32_t n_units = 0;
  kvattn_status st = check_decode(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                  blocks, n_blk, kv_len, scale, &n_units);
  if (st) return st;
  if (!o_part || !lse_part || !aligned(o_part, 16) || n_splits < 1) return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  const AppendArgs app{k_new, v_new, k_pool, v_pool, n_new, k_summary};
  return launch_decode_partials(geom, q, n_q_tok, k_pool, v_pool, page_table, n_logical_pages,
                                blocks, n_blk, kv_len, scale, n_units, n_splits, o_part, lse_part,
                                static_cast<hipStream_t>(stream), &app);
}

int32_t kvattn_prefill_groups(const kvattn_geom* geom, int32_t chunk, int64_t pos0) {
  if (check_geom(geom) != KVATTN_OK || chunk < 1 || pos0 < 0) return 0;
  int n_cu = 256;
  if (current_device(&n_cu) != KVATTN_OK) n_cu = 256;
  return auto_prefill_groups(geom, chunk, pos0, n_cu);
}

kvattn_status kvattn_prefill_chunk(const kvattn_geom* geom, const float* q, int32_t chunk,
                                   const uint8_t* k_pool, const uint8_t* v_pool,
                                   const int32_t* page_table, int32_t n_logical_pages,
                                   int64_t pos0, float scale, float* out, float* lse,
                                   int32_t n_groups, void* workspace, size_t* workspace_bytes,
                                   void* stream) {
  kvattn_status st =
      check_prefill(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages, pos0, scale);
  if (st) return st;
  if (!out || !lse || !aligned(out, 16) || n_groups < 0) return KVATTN_E_INVALID;
  const int32_t n_pages = (int32_t)((pos0 + chunk + KVATTN_PAGE_TOKENS - 1) / KVATTN_PAGE_TOKENS);
  const int64_t rows = (int64_t)chunk * geom->n_kv_heads * geom->gqa;
  int32_t groups = n_groups;
  if (groups == 0) {
    int n_cu = 256;
    if (workspace && (st = current_device(&n_cu))) return st;
    if (!workspace && current_device(&n_cu) != KVATTN_OK) n_cu = 256;
    groups = auto_prefill_groups(geom, chunk, pos0, n_cu);
  }
  if (groups > n_pages) groups = n_pages;
  const size_t o_bytes = checked_bytes(groups, rows, sizeof(float) * KVATTN_HEAD_DIM);
  const size_t lse_bytes = checked_bytes(groups, rows, sizeof(float));
  if (!o_bytes || !lse_bytes) return KVATTN_E_INVALID;  // beyond any memory
  const size_t need = kSyncBytes + o_bytes + lse_bytes;
  bool query_only = false;
  if ((st = workspace_check(workspace, workspace_bytes, need, &query_only))) return st;
  if (query_only) return KVATTN_OK;
  if ((st = current_device(nullptr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* o_part = reinterpret_cast<float*>(ws + kSyncBytes);
  float* lse_part = reinterpret_cast<float*>(ws + kSyncBytes + o_bytes);
  if ((st = launch_prefill_partials(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages,
                                    pos0, scale, groups, o_part, lse_part, s,
                                    reinterpret_cast<uint32_t*>(ws))))
    return st;
  return launched(launch_merge(groups, rows, KVATTN_HEAD_DIM, o_part, lse_part, out, lse, s));
}

kvattn_status kvattn_prefill_partials(const kvattn_geom* geom, const float* q, int32_t chunk,
                                      const uint8_t* k_pool, const uint8_t* v_pool,
                                      const int32_t* page_table, int32_t n_logical_pages,
                                      int64_t pos0, float scale, int32_t n_groups, float* o_part,
                                      float* lse_part, void* stream) {
  kvattn_status st =
      check_prefill(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages, pos0, scale);
  if (st) return st;
  if (!o_part || !lse_part || !aligned(o_part, 16) || n_groups < 1) return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  return launch_prefill_partials(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages, pos0,
                                 scale, n_groups, o_part, lse_part,
                                 static_cast<hipStream_t>(stream));
}

kvattn_status kvattn_prefill_range_partials(const kvattn_geom* geom, const float* q,
                                            int32_t chunk, const uint8_t* k_pool,
                                            const uint8_t* v_pool, const int32_t* page_table,
                                            int32_t n_logical_pages, int64_t pos0, float scale,
                                            int32_t page_begin, int32_t page_end,
                                            int32_t n_groups, float* o_part, float* lse_part,
                                            void* stream) {
  kvattn_status st =
      check_prefill(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages, pos0, scale);
  if (st) return st;
  if (!o_part || !lse_part || !aligned(o_part, 16) || n_groups < 1) return KVATTN_E_INVALID;
  const int64_t n_pages = (pos0 + chunk + KVATTN_PAGE_TOKENS - 1) / KVATTN_PAGE_TOKENS;
  if (page_begin < 0 || page_end <= page_begin || page_end > n_pages) return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  return launch_prefill_partials(geom, q, chunk, k_pool, v_pool, page_table, n_logical_pages, pos0,
                                 scale, n_groups, o_part, lse_part,
                                 static_cast<hipStream_t>(stream), nullptr, page_begin, page_end);
}

kvattn_status kvattn_merge_lse(int32_t n_parts, int64_t rows, int32_t head_dim,
                               const float* o_parts, const float* lse_parts, float* out,
                               float* lse, void* stream) {
  if (n_parts < 1 || rows < 1 || head_dim < 1) return KVATTN_E_INVALID;
  if (!o_parts || !lse_parts || !out || !lse) return KVATTN_E_INVALID;
  if (!aligned(o_parts, 4) || !aligned(lse_parts, 4) || !aligned(out, 4) || !aligned(lse, 4))
    return KVATTN_E_INVALID;
  if (rows > (int64_t)1 << 31) return KVATTN_E_INVALID;
  kvattn_status st = current_device(nullptr);
  if (st) return st;
  return launched(launch_merge(n_parts, rows, head_dim, o_parts, lse_parts, out, lse,
                               static_cast<hipStream_t>(stream)));
}


kvattn_status kvattn_rotate_rows(float* x, int64_t n_rows, void* stream) {
  if (n_rows < 0 || (n_rows > 0 && (!x || !aligned(x, 16)))) return KVATTN_E_INVALID;
  if (n_rows > ((int64_t)1 << 33)) return KVATTN_E_INVALID;  // grid limit
  kvattn_status st = current_device(nullptr);
  if (st) return st;
  if (n_rows == 0) return KVATTN_OK;
  return launched(launch_rotate(x, n_rows, static_cast<hipStream_t>(stream)));
}

kvattn_status kvattn_gather_blocks(const kvattn_geom* geom, const uint8_t* src_k_pool,
                                   const uint8_t* src_v_pool, const int32_t* page_table,
                                   int32_t n_logical_pages, const int32_t* blocks, int32_t n_blk,
                                   int32_t n_sel, uint8_t* dst_k_pool, uint8_t* dst_v_pool,
                                   int32_t* dst_blocks, void* stream) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if (!src_k_pool || !src_v_pool || !dst_k_pool || !dst_v_pool || !page_table || !blocks ||
      !dst_blocks)
    return KVATTN_E_INVALID;
  if (n_logical_pages < 1 || n_blk < 1 || n_sel < 0 || n_sel > n_blk) return KVATTN_E_INVALID;
  if (!aligned(src_k_pool, 256) || !aligned(src_v_pool, 256) || !aligned(dst_k_pool, 256) ||
      !aligned(dst_v_pool, 256))
    return KVATTN_E_INVALID;
  if ((st = current_device(nullptr))) return st;
  if (n_sel == 0) return KVATTN_OK;
  const void *sk = nullptr, *sv = nullptr;
  if ((st = device_view(src_k_pool, &sk)) || (st = device_view(src_v_pool, &sv))) return st;
  return launched(launch_gather(static_cast<const uint8_t*>(sk), static_cast<const uint8_t*>(sv),
                                page_table, n_logical_pages, geom->n_phys_pages, blocks, n_blk,
                                n_sel, geom->n_kv_heads, dst_k_pool, dst_v_pool, dst_blocks,
                                geom->v_type == KVATTN_V_Q8_0, geom->k_type,
                                static_cast<hipStream_t>(stream)));
}

kvattn_status kvattn_prefetch_pages(const kvattn_geom* geom, const uint8_t* src_k_pool,
                                    const uint8_t* src_v_pool, uint8_t* dst_k_pool,
                                    uint8_t* dst_v_pool, const int32_t* pages, int32_t n_pages,
                                    void* stream) {
  kvattn_status st = check_geom(geom);
  if (st) return st;
  if (!src_k_pool || !src_v_pool || !dst_k_pool || !dst_v_pool || n_pages < 0)
    return KVATTN_E_INVALID;
  if (n_pages > 0 && !pages) return KVATTN_E_INVALID;
  for (int32_t i = 0; i < n_pages; ++i)
    if (pages[i] < 0 || pages[i] >= geom->n_phys_pages) return KVATTN_E_INVALID;
  if (n_pages == 0) return KVATTN_OK;
  if ((st = current_device(nullptr))) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // a physical page's records for all KV heads are contiguous in each pool;
  // runs of consecutive page indices go as one copy per pool
  const size_t k_page = (size_t)geom->n_kv_heads * k_record_bytes(geom);
  const size_t v_page = (size_t)geom->n_kv_heads * v_record_bytes(geom);
  int32_t i = 0;
  while (i < n_pages) {
    int32_t j = i + 1;
    while (j < n_pages && pages[j] == pages[j - 1] + 1) ++j;
    const size_t first = (size_t)pages[i], count = (size_t)(j - i);
    if (hipMemcpyAsync(dst_k_pool + first * k_page, src_k_pool + first * k_page, count * k_page,
                       hipMemcpyDefault, s) != hipSuccess ||
        hipMemcpyAsync(dst_v_pool + first * v_page, src_v_pool + first * v_page, count * v_page,
                       hipMemcpyDefault, s) != hipSuccess)
      return KVATTN_E_DEVICE;
    i = j;
  }
  return KVATTN_OK;
}

}  // extern "C"
