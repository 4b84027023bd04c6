// a4: merge of partial attention results by log-sum-exp (the RX 9070 XT
// announcement on wqu.guru, bullet "Online Log-Sum-Exp prefill & pipelined
// prefetch": partial results over streamed pages are accumulated by online
// LSE). Per row: M = max lse_s; L = M + ln sum exp(lse_s - M);
// out = sum exp(lse_s - L) o_s in ascending s; all-(-inf) rows give 0, -inf.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int MERGE_THREADS = 256;
constexpr int MERGE_WCHUNK = 1024;  // part weights staged in LDS per pass

// One workgroup per row; the threads stride over head_dim. Part weights are
// computed once per row into LDS (in chunks), then every output element is a
// fixed-order sum over the parts.
__global__ __launch_bounds__(MERGE_THREADS) void merge_kernel(int32_t n_parts, int64_t rows,
                                                              int32_t head_dim,
                                                              const float* __restrict__ o_parts,
                                                              const float* __restrict__ lse_parts,
                                                              float* __restrict__ out,
                                                              float* __restrict__ lse) {
  __shared__ float w[MERGE_WCHUNK];
  __shared__ float red[MERGE_THREADS / 64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  // M = max over parts
  float m = neg_inf();
  for (int s = tid; s < n_parts; s += MERGE_THREADS) m = fmaxf(m, lse_parts[(int64_t)s * rows + r]);
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  if (m == neg_inf()) {
    for (int n = tid; n < head_dim; n += MERGE_THREADS) out[r * head_dim + n] = 0.0f;
    if (tid == 0) lse[r] = neg_inf();
    return;
  }
  // L = M + ln sum_s exp(lse_s - M), the sum taken in ascending s by thread 0
  // over per-thread partial sums would reorder it; keep it serial and exact in
  // order: each thread sums a contiguous run of parts, runs are then combined
  // in thread order.
  const int per = (n_parts + MERGE_THREADS - 1) / MERGE_THREADS;
  float part = 0.0f;
  for (int s = tid * per; s < n_parts && s < (tid + 1) * per; ++s)
    part += __expf(lse_parts[(int64_t)s * rows + r] - m);
  __shared__ float runs[MERGE_THREADS];
  runs[tid] = part;
  __syncthreads();
  __shared__ float s_L;
  if (tid == 0) {
    float tot = 0.0f;
    for (int i = 0; i < MERGE_THREADS; ++i) tot += runs[i];
    s_L = m + __logf(tot);
  }
  __syncthreads();
  const float L = s_L;
  for (int n = tid; n < head_dim; n += MERGE_THREADS) out[r * head_dim + n] = 0.0f;
  // accumulate in chunks of MERGE_WCHUNK parts
  for (int s0 = 0; s0 < n_parts; s0 += MERGE_WCHUNK) {
    const int cnt = min(MERGE_WCHUNK, n_parts - s0);
    __syncthreads();
    for (int i = tid; i < cnt; i += MERGE_THREADS)
      w[i] = __expf(lse_parts[(int64_t)(s0 + i) * rows + r] - L);
    __syncthreads();
    for (int n = tid; n < head_dim; n += MERGE_THREADS) {
      float acc = out[r * head_dim + n];
      const float* op = o_parts + ((int64_t)s0 * rows + r) * head_dim + n;
      for (int i = 0; i < cnt; ++i) {
        const float wi = w[i];
        if (wi != 0.0f) acc += wi * op[(int64_t)i * rows * head_dim];
      }
      out[r * head_dim + n] = acc;
    }
  }
  if (tid == 0) lse[r] = L;
}

}  // namespace

hipError_t launch_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts,
                        const float* lse_parts, float* out, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)rows), dim3(MERGE_THREADS), 0, stream, n_parts,
                     rows, head_dim, o_parts, lse_parts, out, lse);
  return hipGetLastError();
}

}  // namespace kvattn
