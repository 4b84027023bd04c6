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

constexpr int SCORE_BLOCKS = 64;  // candidate blocks scored per workgroup: one wavefront, a lane each
constexpr int SCORE_BATCH = 16;   // float4 loads per lane and buffer (64 dims)
#ifndef SCORE_BUFS
#define SCORE_BUFS 2              // buffers in flight: 128 of a lane's 256 dims
#endif

// acc = fma(q', x, acc) where q' is lane J of q's 16-lane row (DPP
// row_newbcast on the binary64 FMA): one rounding, as fma(). A DPP
// instruction may not read a VGPR written by a VALU op in the two wait states
// before it (here x and acc, written just before); the compiler cannot see
// into the asm, so the s_nop 1 in it provides them.
#define FMA_ROW_BCAST(J, acc, q, x)                                                     \
  __asm__("s_nop 1\n\tv_fmac_f64_dpp %0, %1, %2 row_newbcast:" #J                      \
          " row_mask:0xf bank_mask:0xf"                                                \
          : "+v"(acc)                                                                  \
          : "v"(q), "v"(x))

// grid (ceil(n_cand / 64), n_kv), 64 threads. Lane t scores block b0 + t,
// reading that block's summary itself, 64 dims (16 float4 loads) at a time
// with the next 64 in flight (each 128-byte line serves 8 consecutive loads
// of a lane). The query sum is staged once through LDS into registers, each
// 16-lane row holding all of it, and broadcast into the FMAs by DPP. A
// product of two binary32 values is exact in binary64, so the fused
// multiply-add acc + q * s rounds once, exactly as the separate product and
// sum do: the fixed-order sum is unchanged. The chain of 256 dependent FMAs
// is what a block's score costs once its summary has arrived.
__global__ __launch_bounds__(SCORE_BLOCKS) void score_kernel(const float* __restrict__ q,
                                                             const float* __restrict__ k_summary,
                                                             int32_t gqa, int32_t n_logical,
                                                             int32_t n_cand,
                                                             double* __restrict__ scores) {
  __shared__ double qd[D];
  const int t = threadIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.x * SCORE_BLOCKS + t;
  // q_sel[n], n = t + 64 r: the group's query vectors summed in ascending
  // order, rounded to binary32 (members past gqa re-read the last one and are
  // not added). Its loads go first: load counters retire in order, so loads
  // issued after the summaries' would wait for them.
  constexpr int QG = 8;  // group members loaded together
  const int n_pass = (gqa + QG - 1) / QG;
  float x[D / 64][QG];
#pragma unroll
  for (int r = 0; r < D / 64; ++r)
#pragma unroll
    for (int j = 0; j < QG; ++j) x[r][j] = q[((int64_t)h * gqa + (j < gqa ? j : gqa - 1)) * D + t + 64 * r];
  // lanes past the candidates re-read the last candidate (a valid address)
  const float4* row = reinterpret_cast<const float4*>(
      k_summary + ((int64_t)h * n_logical + (b < n_cand ? b : n_cand - 1)) * D);
  float4 v[SCORE_BUFS * SCORE_BATCH];  // buffer u: elements SCORE_BATCH * u ..
#pragma unroll
  for (int k = 0; k < SCORE_BUFS * SCORE_BATCH; ++k) v[k] = row[k];
#pragma unroll
  for (int r = 0; r < D / 64; ++r) {
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < QG; ++j)
      if (j < gqa) acc = acc + (double)x[r][j];
    for (int p = 1; p < n_pass; ++p) {  // groups of more than QG members
      for (int j = 0; j < QG; ++j) {
        const int gg = QG * p + j;
        if (gg < gqa) acc = acc + (double)q[((int64_t)h * gqa + gg) * D + t + 64 * r];
      }
    }
    qd[t + 64 * r] = (double)(float)acc;
  }
  __syncthreads();
  // Lane l keeps q_sel[16 m + (l & 15)], m = 0..15 (every 16-lane row holds
  // the whole vector); step n = 16 m + j of the chain takes lane j's value of
  // register m by a row broadcast (DPP row_newbcast) inside the FMA, so no
  // LDS read sits in the chain.
  double qrow[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) qrow[m] = qd[16 * m + (t & 15)];
  double acc = 0.0;
  constexpr int N_BATCH = D / (4 * SCORE_BATCH);
#pragma unroll
  for (int c = 0; c < N_BATCH; ++c) {
    const int e0 = SCORE_BATCH * (c % SCORE_BUFS);
#pragma unroll
    for (int mm = 0; mm < SCORE_BATCH / 4; ++mm) {  // dims 16 m .. 16 m + 15, m = 4 c + mm
      const double qm = qrow[4 * c + mm];
      const float4 y0 = v[e0 + 4 * mm], y1 = v[e0 + 4 * mm + 1];
      const float4 y2 = v[e0 + 4 * mm + 2], y3 = v[e0 + 4 * mm + 3];
      FMA_ROW_BCAST(0, acc, qm, (double)y0.x);
      FMA_ROW_BCAST(1, acc, qm, (double)y0.y);
      FMA_ROW_BCAST(2, acc, qm, (double)y0.z);
      FMA_ROW_BCAST(3, acc, qm, (double)y0.w);
      FMA_ROW_BCAST(4, acc, qm, (double)y1.x);
      FMA_ROW_BCAST(5, acc, qm, (double)y1.y);
      FMA_ROW_BCAST(6, acc, qm, (double)y1.z);
      FMA_ROW_BCAST(7, acc, qm, (double)y1.w);
      FMA_ROW_BCAST(8, acc, qm, (double)y2.x);
      FMA_ROW_BCAST(9, acc, qm, (double)y2.y);
      FMA_ROW_BCAST(10, acc, qm, (double)y2.z);
      FMA_ROW_BCAST(11, acc, qm, (double)y2.w);
      FMA_ROW_BCAST(12, acc, qm, (double)y3.x);
      FMA_ROW_BCAST(13, acc, qm, (double)y3.y);
      FMA_ROW_BCAST(14, acc, qm, (double)y3.z);
      FMA_ROW_BCAST(15, acc, qm, (double)y3.w);
    }
    if (c + SCORE_BUFS < N_BATCH) {  // this buffer takes batch c + SCORE_BUFS
#pragma unroll
      for (int k = 0; k < SCORE_BATCH; ++k) v[e0 + k] = row[SCORE_BATCH * (c + SCORE_BUFS) + k];
    }
  }
  if (b < n_cand) scores[(int64_t)h * n_cand + b] = acc;
}

// Order-preserving 64-bit key of a binary64 score (-0 is mapped to +0 first):
// larger score <=> larger key.
__device__ __forceinline__ uint64_t score_key(double s) {
  if (s == 0.0) s = 0.0;
  const uint64_t b = __builtin_bit_cast(uint64_t, s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

constexpr int TOPK_THREADS = 1024;
constexpr int TOPK_WAVES = TOPK_THREADS / 64;
constexpr int TOPK_AGG_ROUNDS = 4;  // ballot rounds per load in the first radix pass

// Inclusive prefix sum over the 64 lanes of a wavefront: row_shr:1, 2, 4, 8
// steps within each 16-lane row (a lane with no source adds 0), then the
// totals of the rows below.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31);
  const int r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

#ifndef TOPK_REG_THREADS
#define TOPK_REG_THREADS 512
#endif
constexpr int TOPK_REG_KEYS = 4096;  // candidates ranked from registers
constexpr int HIST_COPIES = 8;       // histogram copies, one per lane & 7
constexpr int HIST_LD = 257;         // copy stride: the copies of a digit sit in different banks

// Count of the set bits of a wavefront mask below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The same selection for at most TOPK_REG_KEYS candidates, one workgroup of
// THREADS per KV head: thread t holds the keys of candidates t + THREADS*j in
// registers. Lanes add into one of HIST_COPIES histogram copies, so a digit
// shared by most keys costs an 8-way rather than a 64-way conflict; the two
// buffers alternate, two barriers per pass. The kept blocks are written after
// one more barrier: within row j (candidates THREADS*j ..) a lane's position
// is the count of kept keys in earlier rows, in earlier wavefronts of the row,
// and in lower lanes (mbcnt of the row's ballot).
template <int THREADS>
__global__ __launch_bounds__(THREADS) void topk_reg_kernel(const double* __restrict__ scores,
                                                           int32_t n_cand, int32_t k_sel,
                                                           int32_t n_recent, int32_t n_out,
                                                           int32_t* __restrict__ out_blocks) {
  constexpr int KPT = TOPK_REG_KEYS / THREADS, WAVES = THREADS / 64;
  static_assert(KPT <= 64, "one lane per row in the compaction");
  __shared__ int hist[2][HIST_COPIES * HIST_LD];
  __shared__ int cnt[2][WAVES][KPT];  // per wavefront and row: keys above, keys equal
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem, s_whole;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  int32_t* out = out_blocks + (int64_t)h * n_out;
  for (int i = tid; i < n_recent; i += THREADS) out[k_sel + i] = n_cand + i;
  if (!scores) {  // k_sel is 0 or every candidate: no ranking needed
    for (int i = tid; i < k_sel; i += THREADS) out[i] = i;
    return;
  }
  const double* sc = scores + (int64_t)h * n_cand;
  uint64_t kr[KPT];
  {
    double v[KPT];  // all loads issued together
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int i = tid + THREADS * j;
      v[j] = sc[i < n_cand ? i : n_cand - 1];
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) kr[j] = score_key(v[j]);
  }
  for (int e = tid; e < HIST_COPIES * HIST_LD; e += THREADS) hist[0][e] = 0;
  __syncthreads();
  const int copy = (lane & (HIST_COPIES - 1)) * HIST_LD;
  uint64_t prefix = 0, pmask = 0;
  int krem = k_sel;
  bool whole = false;
  for (int pass = 0, shift = 56; shift >= 0; ++pass, shift -= 8) {
    int* hc = hist[pass & 1];
    int* hn = hist[(pass & 1) ^ 1];  // the next pass's histogram
    for (int e = tid; e < HIST_COPIES * HIST_LD; e += THREADS) hn[e] = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (tid + THREADS * j < n_cand && (kr[j] & pmask) == prefix)
        atomicAdd(&hc[copy + (int)((kr[j] >> shift) & 255)], 1);
    __syncthreads();
    if (tid < 64) {
      // Lane l owns digits 4l..4l+3 (each the sum of its copies); the prefix
      // sum over lanes gives the count of keys in digits above this lane's,
      // and the one lane in which the running count from the top first
      // reaches krem picks the digit.
      int c[4] = {0, 0, 0, 0};
      int part[HIST_COPIES][4];
#pragma unroll
      for (int k = 0; k < HIST_COPIES; ++k)
#pragma unroll
        for (int d = 0; d < 4; ++d) part[k][d] = hc[k * HIST_LD + 4 * tid + d];
#pragma unroll
      for (int k = 0; k < HIST_COPIES; ++k)
#pragma unroll
        for (int d = 0; d < 4; ++d) c[d] += part[k][d];
      const int s = c[0] + c[1] + c[2] + c[3];
      const int incl = wave_incl_scan(s);
      int cum = __builtin_amdgcn_readlane(incl, 63) - incl;
      if (cum < krem && cum + s >= krem) {
        int digit, cn;
        if (cum + c[3] >= krem) {
          digit = 4 * tid + 3, cn = c[3];
        } else if ((cum += c[3]) + c[2] >= krem) {
          digit = 4 * tid + 2, cn = c[2];
        } else if ((cum += c[2]) + c[1] >= krem) {
          digit = 4 * tid + 1, cn = c[1];
        } else {
          cum += c[1];
          digit = 4 * tid, cn = c[0];
        }
        s_krem = krem - cum;
        s_prefix = prefix | ((uint64_t)digit << shift);
        s_whole = cn == krem - cum;  // the whole bucket is selected
      }
    }
    __syncthreads();
    prefix = s_prefix;
    pmask |= (uint64_t)255 << shift;
    krem = s_krem;
    whole = s_whole != 0;
    if (whole) break;  // uniform
  }
  // Kept: keys whose digits so far are above the chosen ones, and every key
  // of the chosen bucket when it is taken whole; otherwise (prefix is the
  // exact k-th key) the first krem keys equal to it by block index.
  const uint64_t thr = prefix;
  uint64_t gm[KPT], em[KPT];
  int gcnt = 0, ecnt = 0;  // lane j: this wavefront's counts in row j
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool valid = tid + THREADS * j < n_cand;
    const bool gt = valid && (whole ? (kr[j] & pmask) >= thr : kr[j] > thr);
    const bool eq = valid && !whole && kr[j] == thr;
    gm[j] = __ballot(gt);
    em[j] = __ballot(eq);
    if (lane == j) gcnt = __popcll(gm[j]), ecnt = __popcll(em[j]);
  }
  if (lane < KPT) cnt[0][wave][lane] = gcnt, cnt[1][wave][lane] = ecnt;
  __syncthreads();
  // lane r < KPT: kept keys before row r's part of this wavefront
  int gt_tot = 0, eq_tot = 0, gt_pre = 0, eq_pre = 0;
  if (lane < KPT) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const int g = cnt[0][w][lane], e = cnt[1][w][lane];
      gt_tot += g, eq_tot += e;
      if (w < wave) gt_pre += g, eq_pre += e;
    }
  }
  const int gt_base = wave_incl_scan(gt_tot) - gt_tot + gt_pre;
  const int eq_base = wave_incl_scan(eq_tot) - eq_tot + eq_pre;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int i = tid + THREADS * j;
    const bool gt = (gm[j] >> lane) & 1, eq = (em[j] >> lane) & 1;
    const int gt_before = __builtin_amdgcn_readlane(gt_base, j) + lanes_below(gm[j]);
    const int eq_before = __builtin_amdgcn_readlane(eq_base, j) + lanes_below(em[j]);
    if (gt || (eq && eq_before < krem)) out[gt_before + min(eq_before, krem)] = i;
  }
}

constexpr int TOPK_LDS_KEYS = 6144;  // keys held in LDS (48 KB); more are re-read from scores

// One workgroup per KV head. Finds the k-th largest key by an 8-bit radix
// select over the 64-bit keys (held in LDS when they fit), stopping early once
// the digit bucket holding the k-th key is taken whole. Then keeps the keys
// above it plus, among keys equal to it, the lowest block indices, and writes
// the kept blocks in ascending block order; the recent window follows.
//
// The first pass's digit (sign and leading exponent bits) is shared by most
// keys, so its histogram is built from ballots: a wavefront adds each digit
// once with its lane count, for up to TOPK_AGG_ROUNDS digits per load, the
// rest by per-lane atomics. Histograms alternate between two buffers, so a
// pass needs two barriers. The kept blocks are written in one sweep: thread t
// owns a contiguous run of keys, and two prefix sums (keys above, keys equal)
// over the threads give every kept block its output position.
__global__ __launch_bounds__(TOPK_THREADS) void topk_kernel(const double* __restrict__ scores,
                                                            int32_t n_cand, int32_t k_sel,
                                                            int32_t n_recent, int32_t n_out,
                                                            int32_t* __restrict__ out_blocks) {
  __shared__ int hist[2][256];
  __shared__ int wsum[2][TOPK_WAVES];
  __shared__ uint64_t s_prefix;
  __shared__ int s_krem, s_whole;
  __shared__ uint64_t skeys[TOPK_LDS_KEYS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x;
  int32_t* out = out_blocks + (int64_t)h * n_out;
  for (int i = tid; i < n_recent; i += TOPK_THREADS) out[k_sel + i] = n_cand + i;
  if (!scores) {  // k_sel is 0 or every candidate: no ranking needed
    for (int i = tid; i < k_sel; i += TOPK_THREADS) out[i] = i;
    return;
  }
  const double* sc = scores + (int64_t)h * n_cand;
  const bool cached = n_cand <= TOPK_LDS_KEYS;  // uniform
  if (tid < 256) hist[0][tid] = 0;
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
  }
  __syncthreads();
  auto key_at = [&](int i) -> uint64_t { return cached ? skeys[i] : score_key(sc[i]); };
  uint64_t prefix = 0, pmask = 0;
  int krem = k_sel;
  bool whole = false;
  for (int pass = 0, shift = 56; shift >= 0; ++pass, shift -= 8) {
    int* hc = hist[pass & 1];
    if (tid < 256) hist[(pass & 1) ^ 1][tid] = 0;  // the next pass's histogram
    if (pass == 0) {
      for (int i0 = 0; i0 < n_cand; i0 += TOPK_THREADS) {  // uniform trip count
        const int i = i0 + tid;
        const bool valid = i < n_cand;
        const int d = valid ? (int)(key_at(i) >> 56) : 0;
        uint64_t act = __ballot(valid);
        for (int round = 0; act != 0; ++round) {  // act is uniform
          if (round == TOPK_AGG_ROUNDS) {
            if ((act >> lane) & 1) atomicAdd(&hc[d], 1);
            break;
          }
          const int leader = __builtin_ctzll(act);
          const int dl = __builtin_amdgcn_readlane(d, leader);
          const uint64_t m = __ballot(d == dl) & act;
          if (lane == leader) atomicAdd(&hc[dl], __popcll(m));
          act &= ~m;
        }
      }
    } else {
      for (int i = tid; i < n_cand; i += TOPK_THREADS) {
        const uint64_t key = key_at(i);
        if ((key & pmask) == prefix) atomicAdd(&hc[(key >> shift) & 255], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // Lane l owns digits 4l..4l+3. The prefix sum over lanes gives the count
      // of keys in digits above this lane's; the one lane in which the running
      // count from the top first reaches krem picks the digit.
      const int c0 = hc[4 * tid], c1 = hc[4 * tid + 1];
      const int c2 = hc[4 * tid + 2], c3 = hc[4 * tid + 3];
      const int s = c0 + c1 + c2 + c3;
      const int incl = wave_incl_scan(s);
      int cum = __builtin_amdgcn_readlane(incl, 63) - incl;
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
    if (whole) break;  // uniform
  }
  // Kept: keys whose digits so far are above the chosen ones, and every key
  // of the chosen bucket when it is taken whole; otherwise (prefix is the
  // exact k-th key) the first krem keys equal to it by block index.
  const uint64_t thr = prefix;
  const int per = (n_cand + TOPK_THREADS - 1) / TOPK_THREADS;
  const int i0 = tid * per;
  const int i1 = min(i0 + per, n_cand);
  int gt = 0, eq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint64_t key = key_at(i);
    if (whole) {
      gt += (key & pmask) >= thr;
    } else {
      gt += key > thr;
      eq += key == thr;
    }
  }
  const int gt_incl = wave_incl_scan(gt), eq_incl = wave_incl_scan(eq);
  if (lane == 63) wsum[0][wave] = gt_incl, wsum[1][wave] = eq_incl;
  __syncthreads();
  int gt_before = gt_incl - gt, eq_before = eq_incl - eq;
  for (int w = 0; w < wave; ++w) gt_before += wsum[0][w], eq_before += wsum[1][w];
  int pos = gt_before + min(eq_before, krem);
  for (int i = i0; i < i1; ++i) {
    const uint64_t key = key_at(i);
    bool keep;
    if (whole) {
      keep = (key & pmask) >= thr;
    } else {
      keep = key > thr;
      if (key == thr) keep = eq_before++ < krem;
    }
    if (keep) out[pos++] = i;
  }
}

}  // namespace

hipError_t launch_score(const float* q, const float* k_summary, int32_t n_kv, int32_t gqa,
                        int32_t n_logical, int32_t n_cand, double* scores, hipStream_t stream) {
  dim3 grid((unsigned)((n_cand + SCORE_BLOCKS - 1) / SCORE_BLOCKS), (unsigned)n_kv);
  hipLaunchKernelGGL(score_kernel, grid, dim3(SCORE_BLOCKS), 0, stream, q, k_summary, gqa, n_logical,
                     n_cand, scores);
  return hipGetLastError();
}

hipError_t launch_topk(const double* scores, int32_t n_kv, int32_t n_cand, int32_t k_sel,
                       int32_t n_recent, int32_t n_out, int32_t* out_blocks,
                       hipStream_t stream) {
  if (!scores || n_cand <= TOPK_REG_KEYS)
    hipLaunchKernelGGL(topk_reg_kernel<TOPK_REG_THREADS>, dim3((unsigned)n_kv),
                       dim3(TOPK_REG_THREADS), 0, stream, scores, n_cand, k_sel, n_recent, n_out,
                       out_blocks);
  else
    hipLaunchKernelGGL(topk_kernel, dim3((unsigned)n_kv), dim3(TOPK_THREADS), 0, stream, scores,
                       n_cand, k_sel, n_recent, n_out, out_blocks);
  return hipGetLastError();
}

}  // namespace kvattn
