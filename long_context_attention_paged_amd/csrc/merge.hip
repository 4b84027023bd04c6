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
// into LDS. head_dim 256 (the decode and prefill partials) has its own paths:
// one wavefront per row when there are few parts and many rows (prefill
// groups), one wavefront per 64 dims when there are at most 64 parts (decode
// splits), a 16-wave workgroup per row when there are more.
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
// wave. Wave w takes parts w, w+16, ... in passes of M256_DEPTH parts per
// wave; the 16 partial sums are added in a fixed order, so results are
// deterministic. Every load is unconditional (indices clamped, weights of
// absent or -inf parts zero, the select after the load), and the first
// pass's partial rows are requested before the lse reductions, so a row
// costs about one memory round trip when n_parts <= 16 * M256_DEPTH.
constexpr int M256_WAVES = 16;
constexpr int M256_THREADS = 64 * M256_WAVES;
constexpr int M256_DEPTH = 8;
constexpr int M256_PASS = M256_WAVES * M256_DEPTH;  // parts per pass

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

__global__ __launch_bounds__(M256_THREADS) void merge256_kernel(int32_t n_parts, int64_t rows,
                                                                const float* __restrict__ o_parts,
                                                                const float* __restrict__ lse_parts,
                                                                float* __restrict__ out,
                                                                float* __restrict__ lse) {
  __shared__ float w[M256_PASS];
  __shared__ float red[M256_WAVES];
  __shared__ floatx4 acc_lds[M256_WAVES][64];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int last = n_parts - 1;
  const int64_t stride4 = rows * 64;  // float4s between consecutive parts
  const floatx4* op = reinterpret_cast<const floatx4*>(o_parts + r * 256) + lane;
  auto load_pass = [&](int s0, floatx4 (&v)[M256_DEPTH]) {
#pragma unroll
    for (int u = 0; u < M256_DEPTH; ++u) {
      const int i = min(s0 + wave + M256_WAVES * u, last);
      v[u] = op[(int64_t)i * stride4];
    }
  };
  floatx4 v[M256_DEPTH];
  load_pass(0, v);  // in flight during the reductions below

  // this thread's first lse (part tid), later ones re-read (only when
  // n_parts exceeds the workgroup)
  const float my = lse_parts[(int64_t)min(tid, last) * rows + r];
  float m = tid < n_parts ? my : neg_inf();
  for (int s = tid + M256_THREADS; s < n_parts; s += M256_THREADS)
    m = fmaxf(m, lse_parts[(int64_t)s * rows + r]);
  m = block_reduce16(m, red, true);
  const bool empty = m == neg_inf();  // uniform: every part is -inf
  float se = 0.f;
  if (!empty) {
    se = tid < n_parts ? expf(my - m) : 0.f;
    for (int s = tid + M256_THREADS; s < n_parts; s += M256_THREADS)
      se += expf(lse_parts[(int64_t)s * rows + r] - m);
  }
  const float L = empty ? neg_inf() : m + logf(block_reduce16(se, red, false));

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_parts; s0 += M256_PASS) {
    if (s0 > 0) load_pass(s0, v);
    if (tid < M256_PASS) {  // weights of this pass; absent and -inf parts weigh 0
      const int s = s0 + tid;
      const float ls = s0 == 0 ? my : lse_parts[(int64_t)min(s, last) * rows + r];
      w[tid] = (s < n_parts && !empty && ls != neg_inf()) ? expf(ls - L) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < M256_DEPTH; ++u) {
      const float wu = w[wave + M256_WAVES * u];
      const floatx4 t = wu * v[u];
      // a zero weight contributes nothing, whatever the (unwritten) row holds
      acc[0] += wu != 0.f ? t[0] : 0.f;
      acc[1] += wu != 0.f ? t[1] : 0.f;
      acc[2] += wu != 0.f ? t[2] : 0.f;
      acc[3] += wu != 0.f ? t[3] : 0.f;
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

// head_dim == 256 with many rows and few parts (the prefill page groups):
// one wavefront per row, four rows per workgroup, no LDS and no barrier.
// Lane l owns dims 4l..4l+3; lane s holds lse of part s (passes of 64) for
// the max and the sum; the parts' rows are then added in ascending part
// order, MR_DEPTH rows in flight per lane.
constexpr int MR_DEPTH = 16;

__device__ __forceinline__ float wave_reduce(float x, bool is_max) {
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o);
    x = is_max ? fmaxf(x, y) : x + y;
  }
  return x;
}

__global__ __launch_bounds__(256) void merge_rows256_kernel(int32_t n_parts, int64_t rows,
                                                            const float* __restrict__ o_parts,
                                                            const float* __restrict__ lse_parts,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform across the wavefront
  const int last = n_parts - 1;
  const int64_t stride4 = rows * 64;  // float4s between consecutive parts
  const floatx4* op = reinterpret_cast<const floatx4*>(o_parts + r * 256) + lane;
  floatx4 v[MR_DEPTH];
  auto load_pass = [&](int s0) {
#pragma unroll
    for (int u = 0; u < MR_DEPTH; ++u) v[u] = op[(int64_t)min(s0 + u, last) * stride4];
  };
  load_pass(0);  // in flight during the reductions below

  const float my = lse_parts[(int64_t)min(lane, last) * rows + r];  // part `lane`
  float m = lane < n_parts ? my : neg_inf();
  for (int s = lane + 64; s < n_parts; s += 64) m = fmaxf(m, lse_parts[(int64_t)s * rows + r]);
  m = wave_reduce(m, true);
  const bool empty = m == neg_inf();  // every part is -inf
  float se = 0.f;
  if (!empty) {
    se = lane < n_parts ? expf(my - m) : 0.f;
    for (int s = lane + 64; s < n_parts; s += 64) se += expf(lse_parts[(int64_t)s * rows + r] - m);
  }
  const float L = empty ? neg_inf() : m + logf(wave_reduce(se, false));

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_parts; s0 += MR_DEPTH) {
    if (s0 > 0) load_pass(s0);
    // weight of part s0 + j sits in lane (s0 + j) % 64: this pass's weights
    float wl = 0.f;
    if (!empty) {
      const int s = (s0 & ~63) + lane;
      const float ls = s0 < 64 ? my : lse_parts[(int64_t)min(s, last) * rows + r];
      wl = (s < n_parts && ls != neg_inf()) ? expf(ls - L) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < MR_DEPTH; ++u) {
      const float wu = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), (s0 + u) & 63));
      const floatx4 t = wu * v[u];
      // a zero weight (absent or -inf part) contributes nothing, whatever the row holds
      acc[0] += wu != 0.f ? t[0] : 0.f;
      acc[1] += wu != 0.f ? t[1] : 0.f;
      acc[2] += wu != 0.f ? t[2] : 0.f;
      acc[3] += wu != 0.f ? t[3] : 0.f;
    }
  }
  reinterpret_cast<floatx4*>(out + r * 256)[lane] = acc;
  if (lane == 0) lse[r] = L;
}

// head_dim == 256 with at most 64 parts (the decode splits): one workgroup per
// row, wavefront qd owns dims 64qd..64qd+63 (lane l: dim 64qd + l). Every
// part's 256-byte slice is requested at once (one float per lane per part),
// lane s holds lse of part s, and the weights are broadcast with readlane:
// no LDS, no barrier, about one memory round trip per row. Parts are added
// in ascending order.
constexpr int MP_PARTS = 64;

__global__ __launch_bounds__(256) void merge_parts64_kernel(int32_t n_parts, int64_t rows,
                                                            const float* __restrict__ o_parts,
                                                            const float* __restrict__ lse_parts,
                                                            float* __restrict__ out,
                                                            float* __restrict__ lse) {
  const int lane = threadIdx.x & 63, qd = threadIdx.x >> 6;
  const int64_t r = blockIdx.x;
  const int last = n_parts - 1;
  const float* op = o_parts + r * 256 + 64 * qd + lane;
  const int64_t stride = rows * 256;  // floats between consecutive parts
  float v[MP_PARTS];
#pragma unroll
  for (int s = 0; s < MP_PARTS; ++s) v[s] = op[(int64_t)(s < last ? s : last) * stride];

  const float my = lse_parts[(int64_t)(lane < last ? lane : last) * rows + r];  // part `lane`
  const float m = wave_reduce(lane < n_parts ? my : neg_inf(), true);
  const bool empty = m == neg_inf();  // every part is -inf
  const float se = (!empty && lane < n_parts) ? expf(my - m) : 0.f;
  const float L = empty ? neg_inf() : m + logf(wave_reduce(se, false));
  const float wl = (!empty && lane < n_parts && my != neg_inf()) ? expf(my - L) : 0.f;
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < MP_PARTS; ++s) {
    const float ws = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wl), s));
    // a zero weight (absent or -inf part) contributes nothing, whatever the row holds
    acc += ws != 0.f ? ws * v[s] : 0.f;
  }
  out[r * 256 + 64 * qd + lane] = acc;
  if (threadIdx.x == 0) lse[r] = L;
}

}  // namespace

hipError_t launch_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts,
                        const float* lse_parts, float* out, float* lse, hipStream_t stream) {
  const bool vec4 = head_dim == 256 && (reinterpret_cast<uintptr_t>(o_parts) & 15) == 0 &&
                    (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  if (vec4 && n_parts <= 2 * MR_DEPTH && rows >= 1024) {
    hipLaunchKernelGGL(merge_rows256_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream,
                       n_parts, rows, o_parts, lse_parts, out, lse);
    return hipGetLastError();
  }
  if (head_dim == 256 && n_parts <= MP_PARTS) {
    hipLaunchKernelGGL(merge_parts64_kernel, dim3((unsigned)rows), dim3(256), 0, stream, n_parts,
                       rows, o_parts, lse_parts, out, lse);
    return hipGetLastError();
  }
  if (vec4) {
    hipLaunchKernelGGL(merge256_kernel, dim3((unsigned)rows), dim3(M256_THREADS), 0, stream,
                       n_parts, rows, o_parts, lse_parts, out, lse);
    return hipGetLastError();
  }
  dim3 grid((unsigned)rows, (unsigned)((head_dim + 63) / 64));
  hipLaunchKernelGGL(merge_kernel, grid, dim3(MERGE_THREADS), 0, stream, n_parts, rows, head_dim,
                     o_parts, lse_parts, out, lse);
  return hipGetLastError();
}

}  // namespace kvattn
