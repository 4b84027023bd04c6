// a4: merge of partial attention results by log-sum-exp (the RX 9070 XT
// announcement on wqu.guru, bullet "Online Log-Sum-Exp prefill & pipelined
// prefetch": partial results over streamed pages are accumulated by online
// LSE). Per row: M = max lse_s; L = M + ln sum exp(lse_s - M);
// out = sum exp(lse_s - L) o_s; all-(-inf) rows give 0, -inf.
//
// Generic head_dim: grid (rows, ceil(head_dim / 64)); 256 threads = 4 waves.
// Each lane owns one output dim; the four waves take interleaved quarters of
// the parts and their partial sums are added in a fixed order in LDS, so
// results are deterministic. Part weights are computed once per workgroup
// into LDS. head_dim 256 (the decode and prefill partials) uses a float4 path.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int MERGE_THREADS = 256;
constexpr int MERGE_WCHUNK = 2048;  // part weights staged in LDS per pass

__device__ __forceinline__ float block_max(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return x;
}

__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  x = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return x;
}

__global__ __launch_bounds__(MERGE_THREADS) void merge_kernel(int32_t n_parts, int64_t rows,
                                                              int32_t head_dim,
                                                              const float* __restrict__ o_parts,
                                                              const float* __restrict__ lse_parts,
                                                              float* __restrict__ out,
                                                              float* __restrict__ lse) {
  __shared__ float w[MERGE_WCHUNK];
  __shared__ float red[4];
  __shared__ float acc_lds[4][64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int dim = blockIdx.y * 64 + lane;

  float m = neg_inf();
  for (int s = tid; s < n_parts; s += MERGE_THREADS) m = fmaxf(m, lse_parts[(int64_t)s * rows + r]);
  m = block_max(m, red);
  if (m == neg_inf()) {  // uniform across the workgroup
    if (wave == 0 && dim < head_dim) out[r * head_dim + dim] = 0.0f;
    if (tid == 0 && blockIdx.y == 0) lse[r] = neg_inf();
    return;
  }
  float se = 0.f;
  for (int s = tid; s < n_parts; s += MERGE_THREADS) se += expf(lse_parts[(int64_t)s * rows + r] - m);
  const float L = m + logf(block_sum(se, red));

  float acc = 0.f;
  for (int s0 = 0; s0 < n_parts; s0 += MERGE_WCHUNK) {
    const int cnt = min(MERGE_WCHUNK, n_parts - s0);
    for (int i = tid; i < cnt; i += MERGE_THREADS)
      w[i] = expf(lse_parts[(int64_t)(s0 + i) * rows + r] - L);
    __syncthreads();
    if (dim < head_dim) {
      const float* op = o_parts + ((int64_t)s0 * rows + r) * head_dim + dim;
      const int64_t stride = rows * head_dim;
#pragma unroll 4
      for (int i = wave; i < cnt; i += 4) {
        const float wi = w[i];
        if (wi != 0.0f) acc += wi * op[(int64_t)i * stride];  // -inf parts hold no data
      }
    }
    __syncthreads();
  }
  acc_lds[wave][lane] = acc;
  __syncthreads();
  if (wave == 0 && dim < head_dim)
    out[r * head_dim + dim] = (acc_lds[0][lane] + acc_lds[1][lane]) + (acc_lds[2][lane] + acc_lds[3][lane]);
  if (tid == 0 && blockIdx.y == 0) lse[r] = L;
}

// head_dim == 256: one workgroup of 16 waves per row; lane l owns dims
// 4l..4l+3 (one float4), so each part's row is one contiguous 1 KB read per
// wave. Wave w takes parts w, w+16, ... with up to eight loads in flight per
// lane; the 16 partial sums are added in a fixed order.
constexpr int M256_WAVES = 16;

__device__ __forceinline__ float block_reduce16(float x, float* red, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float t = red[0];
  for (int i = 1; i < M256_WAVES; ++i) t = is_max ? fmaxf(t, red[i]) : t + red[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(64 * M256_WAVES) void merge256_kernel(int32_t n_parts, int64_t rows,
                                                                   const float* __restrict__ o_parts,
                                                                   const float* __restrict__ lse_parts,
                                                                   float* __restrict__ out,
                                                                   float* __restrict__ lse) {
  constexpr int NT_ = 64 * M256_WAVES;
  __shared__ float w[MERGE_WCHUNK];
  __shared__ float red[M256_WAVES];
  __shared__ floatx4 acc_lds[M256_WAVES][64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  float m = neg_inf();
  for (int s = tid; s < n_parts; s += NT_) m = fmaxf(m, lse_parts[(int64_t)s * rows + r]);
  m = block_reduce16(m, red, true);
  if (m == neg_inf()) {
    if (wave == 0) reinterpret_cast<floatx4*>(out + r * 256)[lane] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tid == 0) lse[r] = neg_inf();
    return;
  }
  float se = 0.f;
  for (int s = tid; s < n_parts; s += NT_) se += expf(lse_parts[(int64_t)s * rows + r] - m);
  const float L = m + logf(block_reduce16(se, red, false));
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t stride4 = rows * 64;  // float4s between consecutive parts
  for (int s0 = 0; s0 < n_parts; s0 += MERGE_WCHUNK) {
    const int cnt = min(MERGE_WCHUNK, n_parts - s0);
    for (int i = tid; i < cnt; i += NT_) w[i] = expf(lse_parts[(int64_t)(s0 + i) * rows + r] - L);
    __syncthreads();
    const floatx4* op = reinterpret_cast<const floatx4*>(o_parts + ((int64_t)s0 * rows + r) * 256) + lane;
    int i = wave;
    for (; i + 7 * M256_WAVES < cnt; i += 8 * M256_WAVES) {
      floatx4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = op[(int64_t)(i + M256_WAVES * u) * stride4];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float wu = w[i + M256_WAVES * u];
        if (wu != 0.0f) acc += wu * v[u];  // a -inf part contributes nothing
      }
    }
    for (; i < cnt; i += M256_WAVES) {
      const float wi = w[i];
      if (wi != 0.0f) acc += wi * op[(int64_t)i * stride4];
    }
    __syncthreads();
  }
  acc_lds[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    floatx4 t = acc_lds[0][lane];
#pragma unroll
    for (int k = 1; k < M256_WAVES; ++k) t += acc_lds[k][lane];
    reinterpret_cast<floatx4*>(out + r * 256)[lane] = t;
  }
  if (tid == 0) lse[r] = L;
}

}  // namespace

hipError_t launch_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts,
                        const float* lse_parts, float* out, float* lse, hipStream_t stream) {
  if (head_dim == 256 && (reinterpret_cast<uintptr_t>(o_parts) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    hipLaunchKernelGGL(merge256_kernel, dim3((unsigned)rows), dim3(64 * M256_WAVES), 0, stream,
                       n_parts, rows, o_parts, lse_parts, out, lse);
    return hipGetLastError();
  }
  dim3 grid((unsigned)rows, (unsigned)((head_dim + 63) / 64));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(MERGE_THREADS), 0, stream, n_parts, rows, head_dim,
                     o_parts, lse_parts, out, lse);
  return hipGetLastError();
}

}  // namespace kvattn
