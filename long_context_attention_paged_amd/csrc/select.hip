// a2: KVMem-style block scoring and budgeted top-k selection.
//
// The KVMem report (lcz.me topic 1972) keeps budget/128 history blocks plus a
// reserved recent window on the GPU (section 測試口徑: --kvmem-budget 32768,
// --kvmem-gen-reserve 16384, 128-token blocks; section Recall 測試: 256 of 485
// blocks kept at budget 32768). Scoring as defined in include/kvattn.h:
// q_sel = RN32(binary64 sum of the group's query vectors), score = binary64
// sum over ascending dims of q_sel[n] * summary[n]; rank by (score desc,
// block asc). The summation orders are fixed so scores, and therefore the
// selected indices, are bit-exact.
#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace kvattn {
namespace {

constexpr int SCORE_BLOCKS = 64;   // candidate blocks scored per workgroup
constexpr int SCORE_THREADS = 256;  // all four waves stage, wave 0 sums
constexpr int SCORE_LD = SCORE_BLOCKS + 1;

// grid (ceil(n_cand / 64), n_kv), 256 threads. The 64 summaries (64 KB) are
// staged in LDS, transposed to [dim][block] (row stride 65 words), by all four
// waves with coalesced 16-byte loads (16 rows per wave, issued together);
// then lane t of wave 0 reads its column 32 dims at a time (independent,
// conflict-free reads) and runs block b0 + t's fixed-order binary64 sum over
// ascending dims.
__global__ __launch_bounds__(SCORE_THREADS) void score_kernel(const float* __restrict__ q,
                                                              const float* __restrict__ k_summary,
                                                              int32_t gqa, int32_t n_logical,
                                                              int32_t n_cand,
                                                              double* __restrict__ scores) {
  __shared__ float qs[D];
  __shared__ float sm[D * SCORE_LD];
  const int tid = threadIdx.x, t = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y;
  const int b0 = blockIdx.x * SCORE_BLOCKS;
  const float* base = k_summary + ((int64_t)h * n_logical + b0) * D;
  {
    // Row r is one coalesced 1 KB read (lane t: float4 t). Rows past the
    // candidates re-read the last candidate's row (a valid address, so the
    // loads need no branch) and store zeros.
    const int last = n_cand - 1 - b0;
    float4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = 16 * wave + k;
      v[k] = *reinterpret_cast<const float4*>(base + (int64_t)(row < last ? row : last) * D + 4 * t);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int row = 16 * wave + k;
      const float4 w = row <= last ? v[k] : float4{0.f, 0.f, 0.f, 0.f};
      sm[(4 * t + 0) * SCORE_LD + row] = w.x;
      sm[(4 * t + 1) * SCORE_LD + row] = w.y;
      sm[(4 * t + 2) * SCORE_LD + row] = w.z;
      sm[(4 * t + 3) * SCORE_LD + row] = w.w;
    }
  }
  {
    // q_sel[n], n = tid: the group's query vectors summed in ascending order;
    // the loads of eight members are issued together, the additions stay in
    // order (members past gqa re-read the last one and are not added)
    double acc = 0.0;
    for (int g0 = 0; g0 < gqa; g0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gg = g0 + j < gqa ? g0 + j : gqa - 1;
        v[j] = q[((int64_t)h * gqa + gg) * D + tid];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (g0 + j < gqa) acc = acc + (double)v[j];
    }
    qs[tid] = (float)acc;
  }
  __syncthreads();
  if (wave != 0) return;
  double acc = 0.0;
  for (int c0 = 0; c0 < D; c0 += 32) {
    float v[32];
#pragma unroll
    for (int n = 0; n < 32; ++n) v[n] = sm[(c0 + n) * SCORE_LD + t];
    // all 32 reads are in flight before the first is used
#pragma unroll
    for (int n = 0; n < 32; ++n) __asm__ __volatile__("" : "+v"(v[n]));
#pragma unroll
    for (int n = 0; n < 32; ++n) acc = acc + (double)qs[c0 + n] * (double)v[n];
  }
  if (b0 + t < n_cand) scores[(int64_t)h * n_cand + b0 + t] = acc;
}

// Order-preserving 64-bit key of a binary64 score (-0 is mapped to +0 first):
// larger score <=> larger key.
__device__ __forceinline__ uint64_t score_key(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t b = __builtin_bit_cast(uint64_t, s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

constexpr int TOPK_THREADS = 1024;

// Exclusive prefix sum of one flag per thread over the workgroup, in thread
// order; returns this thread's prefix and writes the total to *total.
__device__ int block_exclusive_scan(int flag, int* warp_sums, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t mask = __ballot(flag);
  const int before = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) warp_sums[wave] = __popcll(mask);
  __syncthreads();
  int off = 0, tot = 0;
  for (int w = 0; w < TOPK_THREADS / 64; ++w) {
    const int c = warp_sums[w];
    if (w < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + before;
}

constexpr int TOPK_LDS_KEYS = 6144;  // keys held in LDS (48 KB); more are re-read from scores

// One workgroup per KV head. Finds the k-th largest key by an 8-bit radix
// select over the 64-bit keys (held in LDS when they fit), stopping early once
// the digit bucket holding the k-th key is taken whole. Then marks the keys
// above it plus, among keys equal to it, the lowest block indices, and
// compacts the marked blocks in ascending block order; the recent window
// follows.
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const double* __restrict__ scores,
                                                            int32_t n_cand, int32_t k_sel,
                                                            int32_t n_recent, int32_t n_out,
                                                            int32_t* __restrict__ out_blocks) {
  __shared__ int hist[256];
  __shared__ int warp_sums[TOPK_THREADS / 64];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem, s_whole;
  __shared__ uint64_t skeys[TOPK_LDS_KEYS];
  const int tid = threadIdx.x;
  const int h = blockIdx.x;
  int32_t* out = out_blocks + (int64_t)h * n_out;
  for (int i = tid; i < n_recent; i += TOPK_THREADS) out[k_sel + i] = n_cand + i;
  if (!scores) {  // k_sel is 0 or every candidate: no ranking needed
    for (int i = tid; i < k_sel; i += TOPK_THREADS) out[i] = i;
    return;
  }
  const double* sc = scores + (int64_t)h * n_cand;
  const bool cached = n_cand <= TOPK_LDS_KEYS;  // uniform
  if (cached) {  // TOPK_LDS_KEYS / 1024 = 6 loads per thread, issued together
    double v[TOPK_LDS_KEYS / TOPK_THREADS];
#pragma unroll
    for (int k = 0; k < TOPK_LDS_KEYS / TOPK_THREADS; ++k) {
      const int i = tid + TOPK_THREADS * k;
      v[k] = sc[i < n_cand ? i : n_cand - 1];
    }
#pragma unroll
    for (int k = 0; k < TOPK_LDS_KEYS / TOPK_THREADS; ++k) {
      const int i = tid + TOPK_THREADS * k;
      if (i < n_cand) skeys[i] = score_key(v[k]);
    }
    __syncthreads();
  }
  auto key_at = [&](int i) -> uint64_t { return cached ? skeys[i] : score_key(sc[i]); };
  uint64_t prefix = 0, pmask = 0;
  int krem = k_sel;
  bool whole = false;
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n_cand; i += TOPK_THREADS) {
      const uint64_t key = key_at(i);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // Lane l owns digits 4l..4l+3. An inclusive suffix scan over lanes gives
      // the count of keys in digits above this lane's; the one lane in which
      // the running count from the top first reaches krem picks the digit.
      const int c0 = hist[4 * tid], c1 = hist[4 * tid + 1];
      const int c2 = hist[4 * tid + 2], c3 = hist[4 * tid + 3];
      const int s = c0 + c1 + c2 + c3;
      int incl = s;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(incl, o);
        if (tid + o < 64) incl += v;
      }
      int cum = incl - s;
      if (cum < krem && cum + s >= krem) {
        int digit, cnt;
        if (cum + c3 >= krem) {
          digit = 4 * tid + 3, cnt = c3;
        } else if ((cum += c3) + c2 >= krem) {
          digit = 4 * tid + 2, cnt = c2;
        } else if ((cum += c2) + c1 >= krem) {
          digit = 4 * tid + 1, cnt = c1;
        } else {
          cum += c1;
          digit = 4 * tid, cnt = c0;
        }
        s_krem = krem - cum;
        s_prefix = prefix | ((uint64_t)digit << shift);
        s_whole = cnt == krem - cum;  // the whole bucket is selected
      }
    }
    __syncthreads();
    prefix = s_prefix;
    pmask |= (uint64_t)255 << shift;
    krem = s_krem;
    whole = s_whole != 0;
    __syncthreads();
    if (whole) break;  // uniform
  }
  // Selected: keys whose digits so far are above the chosen ones, and every
  // key of the chosen bucket when it is taken whole; otherwise (prefix is the
  // exact k-th key) the first krem keys equal to it by block index.
  const uint64_t thr = prefix;
  int eq_seen = 0, written = 0;
  for (int base = 0; base < n_cand; base += TOPK_THREADS) {
    const int i = base + tid;
    const uint64_t key = i < n_cand ? key_at(i) : 0;
    int keep;
    if (whole) {
      keep = (i < n_cand) && (key & pmask) >= thr;
    } else {
      const int is_eq = (i < n_cand && key == thr) ? 1 : 0;
      int eq_total;
      const int eq_rank = eq_seen + block_exclusive_scan(is_eq, warp_sums, &eq_total);
      keep = (i < n_cand) && (key > thr || (is_eq && eq_rank < krem));
      eq_seen += eq_total;
    }
    int keep_total;
    const int pos = written + block_exclusive_scan(keep, warp_sums, &keep_total);
    if (keep) out[pos] = i;
    written += keep_total;
  }
}

}  // namespace

hipError_t launch_score(const float* q, const float* k_summary, int32_t n_kv, int32_t gqa,
                        int32_t n_logical, int32_t n_cand, double* scores, hipStream_t stream) {
  dim3 grid((unsigned)((n_cand + SCORE_BLOCKS - 1) / SCORE_BLOCKS), (unsigned)n_kv);
  hipLaunchKernelGGL(score_kernel, grid, dim3(SCORE_THREADS), 0, stream, q, k_summary, gqa, n_logical,
                     n_cand, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const double* scores, int32_t n_kv, int32_t n_cand, int32_t k_sel,
                       int32_t n_recent, int32_t n_out, int32_t* out_blocks,
                       hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)n_kv), dim3(TOPK_THREADS), 0, stream, scores,
                     n_cand, k_sel, n_recent, n_out, out_blocks);
  return hipGetLastError();
}

}  // namespace kvattn
