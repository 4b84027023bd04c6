// KVMem host tier: the GPU pulls the blocks a selection kept from a pool in
// pinned host memory (the KVMem report, lcz.me topic 1972: history blocks in
// host RAM, budget/128 of them plus a recent window on the GPU; section
// 測試口徑). The block list stays on the device, so no host round trip sits
// between the selection and the copy.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int GATHER_THREADS = 256;

// grid (n_sel, n_kv); KREC, VREC the key and value record sizes (Q8_0,
// Q4_0 or Q5_1 keys, Q4_0 or Q8_0 values). Workgroup (i, h) copies the key and value records of
// logical page blocks[h][i] (row stride n_blk) into record i * n_kv + h of the
// destination pools and writes dst_blocks[h][i] (row stride n_sel) = i, or -1
// (nothing copied) when the entry or its physical page is out of range. Each
// thread requests all of its chunks (13 for the q8_0/q4_0 pair, at most 17) before
// storing any, so a record costs about one round trip over the host link.
template <int KREC, int VREC>
__global__ __launch_bounds__(GATHER_THREADS) void gather_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v,
    const int32_t* __restrict__ page_table, int32_t n_logical, int32_t n_phys,
    const int32_t* __restrict__ blocks, int32_t n_blk, int32_t n_kv, uint8_t* __restrict__ dst_k,
    uint8_t* __restrict__ dst_v, int32_t* __restrict__ dst_blocks) {
  constexpr int K_CHUNKS = KREC / 16;
  constexpr int V_CHUNKS = VREC / 16;
  constexpr int G_PER_THREAD = (K_CHUNKS + V_CHUNKS + GATHER_THREADS - 1) / GATHER_THREADS;
  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int32_t lp = blocks[(int64_t)h * n_blk + i];
  int32_t ph = -1;
  if (lp >= 0 && lp < n_logical) {
    ph = page_table[lp];
    if (ph >= n_phys) ph = -1;
  }
  if (tid == 0) dst_blocks[(int64_t)h * gridDim.x + i] = ph >= 0 ? i : -1;
  if (ph < 0) return;  // uniform across the workgroup
  const u32x4* ks = reinterpret_cast<const u32x4*>(src_k + ((int64_t)ph * n_kv + h) * KREC);
  const u32x4* vs = reinterpret_cast<const u32x4*>(src_v + ((int64_t)ph * n_kv + h) * VREC);
  u32x4* kd = reinterpret_cast<u32x4*>(dst_k + ((int64_t)i * n_kv + h) * KREC);
  u32x4* vd = reinterpret_cast<u32x4*>(dst_v + ((int64_t)i * n_kv + h) * VREC);
  u32x4 v[G_PER_THREAD];
#pragma unroll
  for (int k = 0; k < G_PER_THREAD; ++k) {
    const int c = tid + GATHER_THREADS * k;
    if (c < K_CHUNKS) v[k] = __builtin_nontemporal_load(ks + c);
    else if (c < K_CHUNKS + V_CHUNKS) v[k] = __builtin_nontemporal_load(vs + (c - K_CHUNKS));
  }
#pragma unroll
  for (int k = 0; k < G_PER_THREAD; ++k) {
    const int c = tid + GATHER_THREADS * k;
    if (c < K_CHUNKS) kd[c] = v[k];
    else if (c < K_CHUNKS + V_CHUNKS) vd[c - K_CHUNKS] = v[k];
  }
}

}  // namespace

hipError_t launch_gather(const uint8_t* src_k, const uint8_t* src_v, const int32_t* page_table,
                         int32_t n_logical, int32_t n_phys, const int32_t* blocks, int32_t n_blk,
                         int32_t n_sel, int32_t n_kv, uint8_t* dst_k, uint8_t* dst_v,
                         int32_t* dst_blocks, bool v_q8, int k_type, hipStream_t stream) {
  dim3 grid((unsigned)n_sel, (unsigned)n_kv);
  auto kern = k_type == 2   ? (v_q8 ? gather_kernel<K5_REC, V8_REC> : gather_kernel<K5_REC, V_REC>)
              : k_type == 1 ? (v_q8 ? gather_kernel<K4_REC, V8_REC> : gather_kernel<K4_REC, V_REC>)
                            : (v_q8 ? gather_kernel<K_REC, V8_REC> : gather_kernel<K_REC, V_REC>);
  hipLaunchKernelGGL(kern, grid, dim3(GATHER_THREADS), 0, stream, src_k, src_v,
                     page_table, n_logical, n_phys, blocks, n_blk, n_kv, dst_k, dst_v,
                     dst_blocks);
  return hipGetLastError();
}

}  // namespace kvattn
