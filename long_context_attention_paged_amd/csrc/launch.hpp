// Internal launch interface between the C ABI (api.hip) and the kernel units.
// Every launcher assumes its arguments were validated by the caller and only
// enqueues work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace kvattn {

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per device (the attribute is per device). `done` is the caller's
// per-kernel set of devices already configured; thread-safe and idempotent.
inline hipError_t set_lds_limit(std::atomic<uint64_t>& done, const void* kernel, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = uint64_t(1) << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e =
      hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

hipError_t launch_quantize(const float* k, const float* v, int64_t pos0, int32_t n_tok,
                           int32_t n_kv, const int32_t* page_table, int32_t n_phys,
                           uint8_t* k_pool, uint8_t* v_pool, bool v_q8, int k_type,
                           hipStream_t stream);

hipError_t launch_summarize(const uint8_t* k_pool, const int32_t* page_table, int32_t n_kv,
                            int32_t n_phys, int32_t n_logical, int32_t first_page,
                            int32_t n_pages, float* k_summary, int k_type, hipStream_t stream);

hipError_t launch_score(const float* q, const float* k_summary, int32_t n_kv, int32_t gqa,
                        int32_t n_logical, int32_t n_cand, double* scores,
                        hipStream_t stream);

hipError_t launch_topk(const double* scores, int32_t n_kv, int32_t n_cand, int32_t k_sel,
                       int32_t n_recent, int32_t n_out, int32_t* out_blocks,
                       hipStream_t stream);

struct DecodeParams {
  const float* q;            // [n_q_tok][n_kv*gqa][256]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* page_table;
  const int32_t* blocks;     // [n_kv][n_blk] or nullptr (dense)
  float* o_part;             // [n_splits][n_q_tok*n_kv*gqa][256]
  float* lse_part;           // [n_splits][n_q_tok*n_kv*gqa]
  int64_t kv_len;
  int32_t n_units;           // pages (dense) or block-list entries (sparse)
  int32_t n_splits;
  int32_t n_kv;
  int32_t gqa;
  int32_t n_q_tok;
  int32_t n_logical;
  int32_t n_phys;
  int32_t n_blk;
  float qscale;              // softmax scale * log2(e)
  // Fused append (n_new > 0): positions kv_len - n_new .. kv_len - 1 are
  // quantised from k_new / v_new ([n_new][n_kv][256]) into the pools first.
  const float* k_new;
  const float* v_new;
  uint8_t* k_pool_w;         // k_pool / v_pool, writable
  uint8_t* v_pool_w;
  int32_t n_new;
  int32_t v_q8;              // value records hold Q8_0 codes (else Q4_0)
  int32_t k_type;            // key records: 0 Q8_0, 1 Q4_0, 2 Q5_1
  // Summary of the logical page the append completes (-1: none): written to
  // k_summary [n_kv][n_logical][256] by the workgroup whose units hold it.
  int32_t sum_page;
  float* k_summary;
};

// Wavefronts per decode workgroup. The kernel is sized for one workgroup of
// 8 (or two of 4) per CU; the default split count fills every CU once.
constexpr int DECODE_WAVES = 8;
constexpr int DECODE_WGS_PER_CU = 8 / DECODE_WAVES;

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

struct PrefillParams {
  const float* q;            // [chunk][n_kv*gqa][256]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* page_table;
  float* o_part;             // [n_groups][chunk*n_kv*gqa][256]
  float* lse_part;           // [n_groups][chunk*n_kv*gqa]
  int64_t pos0;
  int32_t chunk;
  int32_t n_groups;
  int32_t n_kv;
  int32_t gqa;
  int32_t n_logical;
  int32_t n_phys;
  float qscale;
  int32_t v_q8;              // value records hold Q8_0 codes (else Q4_0)
  int32_t k_type;            // key records: 0 Q8_0, 1 Q4_0, 2 Q5_1
  uint32_t* flag;            // workspace error word (bit 0: a wave's wait gave up) or nullptr
  int32_t pg_begin, pg_end;  // logical pages the groups split (keys outside are not read)
};

int32_t prefill_rows_per_tile();
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

hipError_t launch_gather(const uint8_t* src_k, const uint8_t* src_v, const int32_t* page_table,
                         int32_t n_logical, int32_t n_phys, const int32_t* blocks, int32_t n_blk,
                         int32_t n_sel, int32_t n_kv, uint8_t* dst_k, uint8_t* dst_v,
                         int32_t* dst_blocks, bool v_q8, int k_type, hipStream_t stream);

hipError_t launch_rotate(float* x, int64_t n_rows, hipStream_t stream);

hipError_t launch_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts,
                        const float* lse_parts, float* out, float* lse, hipStream_t stream);

}  // namespace kvattn
