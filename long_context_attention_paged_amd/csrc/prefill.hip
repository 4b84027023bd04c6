// a6: chunked-prefill attention over the paged Q8_0/Q4_0 cache.
//
// Source: the RX 9070 XT announcement (wqu.guru), bullet "Online Log-Sum-Exp
// prefill & pipelined prefetch": chunked prefill over pages with partial
// results accumulated by online LSE; micro-batch 512 from the Adaptive KV
// Streaming guide (alphalab.site, step ④: -ub 512). The kernel design is this
// library's.
//
// Grid (page groups, query tiles, KV heads); 256 threads = 4 wavefronts; a
// query tile is 128 rows (row = token * gqa + group member), 32 per wave.
// Each workgroup walks the pages of its group in 32-token sub-tiles. The
// quantised bytes stream into an LDS ring by direct global->LDS loads, two
// sub-tiles ahead; each wave loads and dequantises one quarter of a sub-tile
// (8 key rows, 64 value dims) into an f16 stage (keys [token][dim], values
// [dim][slot] in the pool's slot order, value scale applied). Every wave
// computes S^T = Khat . Q'^T and O^T += Vhat^T . P'^T with
// v_mfma_f32_16x16x32_f16 (rows in the N dimension, two N-tiles), with the
// online softmax in base 2 in between; the dequantisation of the next
// sub-tile is placed between the two products, so it overlaps the matrix
// cores. Each group writes a normalised partial (o, lse) per row; the LSE
// merge combines the groups.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int PF_PRODUCERS = 4;                 // waves that stream and dequantise
constexpr int PF_CONSUMERS = 4;                 // waves that multiply
constexpr int PF_THREADS = 64 * (PF_PRODUCERS + PF_CONSUMERS);
constexpr int PF_NT = 2;                        // 16-row N-tiles per consumer wave
constexpr int PF_ROWS = PF_CONSUMERS * 16 * PF_NT;  // rows per workgroup
constexpr int K_LDS_STRIDE = 264;               // halves per key row (256 + pad)
constexpr int V_LDS_STRIDE = 40;                // halves per value dim row (32 + pad)
constexpr int K_LDS_HALVES = 32 * K_LDS_STRIDE;
constexpr int V_LDS_HALVES = D * V_LDS_STRIDE;
constexpr int STAGE_HALVES = K_LDS_HALVES + V_LDS_HALVES;  // one f16 sub-tile
constexpr int N_STAGES = 3;  // f16 sub-tiles in LDS
constexpr float PF_RESCALE_MARGIN = 8.0f;
// Raw (quantised) sub-tile share of one producer wave: 8 key rows (2 KB), a
// quarter of the value words (1 KB), 128 B of key scales, 128 B of value
// scales. Two slots: sub-tile i+2 refills the slot sub-tile i came from.
constexpr int RAW_WAVE = 2048 + 1024 + 256;
constexpr int RAW_STAGE = PF_PRODUCERS * RAW_WAVE;
constexpr int RAW_DEPTH = 2;
constexpr int RAW_LOADS = 4;                    // direct loads per producer wave per sub-tile

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void dma16(const uint8_t* src, uint8_t* lds_dst) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_void*)(lds_dst), 16,
                                   0, 0);
}

// Wait until an LDS counter reaches target. The counters are raised by other
// waves of the workgroup, and every wait here is for work those waves do
// unconditionally: a producer waits for the consumers to release the stage's
// previous round (three sub-tiles back), a consumer for the producers to
// fill the current one, so no wait can close a cycle. The spin is capped all
// the same (2^20 sleeps, tens of milliseconds), so a broken invariant cannot hang the GPU.
__device__ __forceinline__ void wait_count(const int* c, int target) {
  for (int spin = 0; spin < (1 << 20); ++spin) {
    // an LDS read (a generic one would also wait for the raw tile loads)
    const volatile __attribute__((address_space(3))) int* lc =
        (const volatile __attribute__((address_space(3))) int*)(c);
    if (__builtin_amdgcn_readfirstlane(*lc) >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  __asm__ __volatile__("" ::: "memory");
}

// Publish this wave's LDS accesses before it: all of them have completed when
// the count is raised (lane 0 adds). The add is written as an instruction of
// its own: as an atomic the compiler would first wait for every raw tile load
// in flight, since those also write LDS.
__device__ __forceinline__ void signal_count(int* c, int lane) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  const uint32_t addr = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) int*)(c));
  if (lane == 0) __asm__ __volatile__("ds_add_u32 %0, %1" ::"v"(addr), "v"(1) : "memory");
}

template <int N>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __asm__ __volatile__("" ::: "memory");
}

// Producer wave w's share of sub-tile (group c of a page): key rows
// 8w..8w+7 of the group, the value words with q = w (dims 16*(4w+e)+d), and
// the scales both need. Key codes land in LDS as 16-byte chunks ordered
// (half, block, row): lane i of each load fetches row i%8, block i/8, so the
// dequantising lanes read and write without bank conflicts.
__device__ __forceinline__ void issue_raw(uint8_t* raw, const uint8_t* krec, const uint8_t* vrec,
                                          int c, int w, int lane) {
  const uint8_t* kc = krec + (c * 32 + 8 * w) * D + (lane & 7) * D + 32 * (lane >> 3);
  dma16(kc, raw);
  dma16(kc + 16, raw + 1024);
  dma16(vrec + (c * 1024 + w * 256) * 4 + lane * 16, raw + 2048);
  if (lane < 16) {
    const uint8_t* src = lane < 8 ? krec + K_SCALE_OFF + ((c * 32 + 8 * w) * 8) * 2 + lane * 16
                                  : vrec + V_SCALE_OFF + ((c * 8 + 2 * w) * 4) * 16 + (lane - 8) * 16;
    dma16(src, raw + 3072);
  }
}

// Dequantise producer wave w's raw share into an f16 stage. Only the first
// n_live slots of the sub-tile hold data (later slots are unwritten bytes
// past kv_len; n_live is 0 for a page the table does not map): their keys
// and value scales are replaced by zeros.
// Keys, lane l: row 8w + l%8, block l/8 (32 codes).
// Values, lane l: word quad l (4 dims, 8 slots each).
__device__ __forceinline__ void dequant_raw(const uint8_t* raw, _Float16* stage, int w, int lane,
                                            int n_live) {
  {
    const int u = 8 * w + (lane & 7), b = lane >> 3;
    const u32x4 k0 = *reinterpret_cast<const u32x4*>(raw + lane * 16);
    const u32x4 k1 = *reinterpret_cast<const u32x4*>(raw + 1024 + lane * 16);
    const uint32_t ks = *reinterpret_cast<const uint16_t*>(raw + 3072 + (lane & 7) * 16 + 2 * b);
    const half2_t d2 = as_h2(u < n_live ? (ks | (ks << 16)) : 0u);  // zero scale -> zeros
    _Float16* krow = stage + u * K_LDS_STRIDE + 32 * b;
    *reinterpret_cast<half8_t*>(krow + 0) = k_codes_to_f16(k0.x, k0.y, d2);
    *reinterpret_cast<half8_t*>(krow + 8) = k_codes_to_f16(k0.z, k0.w, d2);
    *reinterpret_cast<half8_t*>(krow + 16) = k_codes_to_f16(k1.x, k1.y, d2);
    *reinterpret_cast<half8_t*>(krow + 24) = k_codes_to_f16(k1.z, k1.w, d2);
  }
  {
    const int d = lane & 15, g = lane >> 4;
    const u32x4 words = *reinterpret_cast<const u32x4*>(raw + 2048 + lane * 16);
    uint32_t mk[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int u0 = 16 * ((2 * p) >> 2) + 4 * g + ((2 * p) & 3);
      const int u1 = 16 * ((2 * p + 1) >> 2) + 4 * g + ((2 * p + 1) & 3);
      mk[p] = (u0 < n_live ? 0x0000FFFFu : 0u) | (u1 < n_live ? 0xFFFF0000u : 0u);
    }
    _Float16* vbase = stage + K_LDS_HALVES;
    const uint32_t wv[4] = {words.x, words.y, words.z, words.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int dim = 16 * (4 * w + e) + d;
      // value scales of block 2w + e/2 for lane group g: 16 bytes
      const u32x4 sc = *reinterpret_cast<const u32x4*>(raw + 3072 + 128 + ((e >> 1) * 4 + g) * 16);
      const uint32_t scw[4] = {sc.x & mk[0], sc.y & mk[1], sc.z & mk[2], sc.w & mk[3]};
      half8_t val = v_codes_to_f16(wv[e]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const half2_t pr = {val[2 * p], val[2 * p + 1]};
        const half2_t r = pr * as_h2(scw[p]);
        val[2 * p] = r[0];
        val[2 * p + 1] = r[1];
      }
      *reinterpret_cast<half8_t*>(vbase + dim * V_LDS_STRIDE + 8 * g) = val;
    }
  }
}

struct SubTiles {
  int64_t pg0, pg1;  // this group's logical pages [pg0, pg1)
  int n_sub;         // 32-token sub-tiles to visit
};

// Page records of a group, 64 pages at a time in one VGPR (lane i holds the
// record index of page pg0 + first + i, or -1 when the table does not map
// it), read back with readlane: the loops then issue no page-table loads of
// their own, whose waits would also drain the raw tile stream.
struct PageWindow {
  int64_t first;
  int32_t rec;
  __device__ __forceinline__ void load(const PrefillParams& p, const SubTiles& t, int64_t f,
                                       int h, int lane) {
    first = f;
    const int64_t lp = t.pg0 + f + lane;
    int32_t r = -1;
    if (lp < t.pg1) {
      const int32_t ph = p.page_table[lp];
      if (ph >= 0 && ph < p.n_phys) r = ph * p.n_kv + h;
    }
    rec = r;
  }
  // record of sub-tile sub's page (-1: unmapped); the page must be in the window
  __device__ __forceinline__ int32_t record(int sub) const {
    return __builtin_amdgcn_readlane(rec, (int)((sub >> 2) - first));
  }
};

__global__ __launch_bounds__(PF_THREADS) void prefill_kernel(PrefillParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  _Float16* lds = reinterpret_cast<_Float16*>(lds_raw);                      // f16 stages
  uint8_t* raw_ring = lds_raw + N_STAGES * STAGE_HALVES * sizeof(_Float16);  // raw slots
  // Per stage: producer waves done writing it, consumer waves done reading
  // it (both counts only grow; round r of stage s is sub-tile 3r + s).
  __shared__ int counters[2 * N_STAGES];
  int* produced = counters;
  int* consumed = counters + N_STAGES;
  const int group = blockIdx.x, qtile = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_heads = p.n_kv * p.gqa;
  const int64_t rows_head = (int64_t)p.chunk * p.gqa;
  const int64_t kv_len = p.pos0 + p.chunk;
  const int64_t n_pages = (kv_len + PAGE - 1) / PAGE;

  // ---- this group's sub-tiles (32 tokens each) ------------------------------
  const int64_t tile_last_row = ((int64_t)qtile + 1) * PF_ROWS - 1 < rows_head
                                    ? ((int64_t)qtile + 1) * PF_ROWS - 1
                                    : rows_head - 1;
  const int64_t wg_max_pos = p.pos0 + tile_last_row / p.gqa;  // last key any row here sees
  SubTiles t;
  t.pg0 = n_pages * group / p.n_groups;
  t.pg1 = n_pages * (group + 1) / p.n_groups;
  if (t.pg1 > wg_max_pos / PAGE + 1) t.pg1 = wg_max_pos / PAGE + 1;
  t.n_sub = t.pg1 > t.pg0 ? (int)((t.pg1 - t.pg0) * 4) : 0;
  if (t.n_sub > 0) {  // drop trailing 32-token groups no row sees
    const int64_t last_tok0 = t.pg0 * PAGE + (int64_t)(t.n_sub - 1) * 32;
    if (last_tok0 > wg_max_pos) t.n_sub -= (int)((last_tok0 - wg_max_pos + 31) / 32);
  }
  const int n_sub = t.n_sub;
  PageWindow win;
  win.load(p, t, 0, h, lane);
  if (tid < 2 * N_STAGES) produced[tid] = 0;  // consumed follows produced
  __syncthreads();

  if (wave < PF_PRODUCERS) {
    // ======== producer: stream raw sub-tiles, dequantise into f16 stages ====
    const int w = wave;
    auto slot = [&](int sub) { return raw_ring + (sub % RAW_DEPTH) * RAW_STAGE + w * RAW_WAVE; };
    auto issue = [&](int sub) {
      const int32_t r = win.record(sub);
      const int64_t rec = r >= 0 ? r : 0;  // unmapped pages load record 0, then zero it
      issue_raw(slot(sub), p.k_pool + rec * K_REC, p.v_pool + rec * V_REC, r >= 0 ? (sub & 3) : 0,
                w, lane);
    };
    auto dequant = [&](int sub) {
      const int64_t left = kv_len - (t.pg0 * PAGE + (int64_t)sub * 32);
      const int n_live = win.record(sub) < 0 ? 0 : left >= 32 ? 32 : (int)left;
      dequant_raw(slot(sub), lds + (sub % N_STAGES) * STAGE_HALVES, w, lane, n_live);
    };
    if (n_sub > 0) issue(0);
    if (n_sub > 1) issue(1);
    for (int sub = 0; sub < n_sub; ++sub) {
      if (((sub + 2) >> 2) >= win.first + 64) {  // sub and sub + 2 stay in the window
        wait_loads<0>();
        win.load(p, t, sub >> 2, h, lane);
      }
      if (sub + 1 < n_sub) wait_loads<RAW_LOADS>(); else wait_loads<0>();  // raw sub-tile sub
      const int st = sub % N_STAGES, round = sub / N_STAGES;
      wait_count(consumed + st, PF_CONSUMERS * round);  // previous round read out
      dequant(sub);
      signal_count(produced + st, lane);  // also: this raw slot has been read
      if (sub + 2 < n_sub) issue(sub + 2);
    }
    return;
  }

  // ======== consumer: S^T = Khat . Q'^T, online softmax, O^T += Vhat^T . P'^T
  const int cw = wave - PF_PRODUCERS;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t row0 = (int64_t)qtile * PF_ROWS + cw * 16 * PF_NT;  // this wave's first row
  half8_t qb[PF_NT][8];
  int32_t limit[PF_NT];  // last visible key of the row, relative to pos0
#pragma unroll
  for (int nt = 0; nt < PF_NT; ++nt) {
    const int64_t r = row0 + nt * 16 + r16;
    if (r < rows_head) {
      const int64_t tq = r / p.gqa;
      const int gi = (int)(r - tq * p.gqa);
      const float* qp = p.q + (tq * n_heads + h * p.gqa + gi) * D + 64 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const float4 a = *reinterpret_cast<const float4*>(qp + 8 * ks);
        const float4 b = *reinterpret_cast<const float4*>(qp + 8 * ks + 4);
        qb[nt][ks] = half8_t{(_Float16)(a.x * p.qscale), (_Float16)(a.y * p.qscale),
                             (_Float16)(a.z * p.qscale), (_Float16)(a.w * p.qscale),
                             (_Float16)(b.x * p.qscale), (_Float16)(b.y * p.qscale),
                             (_Float16)(b.z * p.qscale), (_Float16)(b.w * p.qscale)};
      }
      limit[nt] = (int32_t)tq;
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qb[nt][ks] = half8_t{};
      limit[nt] = -64;  // below every key the mask is applied to
    }
  }
  // wave-uniform visibility bounds of this wave's rows
  const int64_t wr_lo = row0 < rows_head ? row0 : rows_head - 1;
  const int64_t wr_hi = (row0 + 16 * PF_NT - 1) < rows_head ? row0 + 16 * PF_NT - 1 : rows_head - 1;
  const int64_t wave_min_limit = p.pos0 + wr_lo / p.gqa;
  const int64_t wave_max_limit = p.pos0 + wr_hi / p.gqa;
  const bool wave_active = row0 < rows_head;

  float mrow[PF_NT], lrow[PF_NT];
  floatx4 o[PF_NT][16];
#pragma unroll
  for (int nt = 0; nt < PF_NT; ++nt) {
    mrow[nt] = neg_inf();
    lrow[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) o[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  for (int sub = 0; sub < n_sub; ++sub) {
    if ((sub >> 2) >= win.first + 64) win.load(p, t, sub >> 2, h, lane);
    const int st = sub % N_STAGES;
    wait_count(produced + st, PF_PRODUCERS * (sub / N_STAGES + 1));
    const _Float16* ks_lds = lds + st * STAGE_HALVES;
    const _Float16* vs_lds = ks_lds + K_LDS_HALVES;
    const int64_t cur_tok0 = t.pg0 * PAGE + (int64_t)sub * 32;
    const bool compute = win.record(sub) >= 0 && wave_active && cur_tok0 <= wave_max_limit;
    if (compute) {
      // The sub-tile's 32 operand fragments (16 of keys, then 16 of values)
      // go through a ring of FR registers, read FR fragments ahead, so LDS
      // latency is hidden behind the products and, for the first values,
      // behind the softmax.
      constexpr int FR = 6;
      int ln = lane;
      __asm__ __volatile__("" : "+v"(ln));  // recompute the offsets here, do not hold them
      const _Float16* kbase = ks_lds + (ln & 15) * K_LDS_STRIDE + 64 * (ln >> 4);
      const _Float16* vbase = vs_lds + (ln & 15) * V_LDS_STRIDE + 8 * (ln >> 4);
      auto frag = [&](int f) -> half8_t {
        return f < 16 ? *reinterpret_cast<const half8_t*>(kbase + 16 * (f & 1) * K_LDS_STRIDE +
                                                          8 * (f >> 1))
                      : *reinterpret_cast<const half8_t*>(vbase + 16 * (f - 16) * V_LDS_STRIDE);
      };
      half8_t ring[FR];
#pragma unroll
      for (int f = 0; f < FR; ++f) ring[f] = frag(f);
      floatx4 s[2][PF_NT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) s[m][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const int ks = f >> 1, m = f & 1;
        const half8_t a = ring[f % FR];
        if (f + FR < 32) ring[f % FR] = frag(f + FR);
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) s[m][nt] = mfma16(a, qb[nt][ks], s[m][nt]);
      }
      if (cur_tok0 + 31 > wave_min_limit) {  // then cur_tok0 - pos0 > -32
        const int32_t rel = (int32_t)(cur_tok0 - p.pos0) + 4 * g;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int nt = 0; nt < PF_NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (rel + 16 * m + i > limit[nt]) s[m][nt][i] = neg_inf();
      }
      half8_t pb[PF_NT];
#pragma unroll
      for (int nt = 0; nt < PF_NT; ++nt) {
        float mx = s[0][nt][0];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[m][nt][i]);
        mx = wave_max_xor_16_32(mx);
        if (mx > mrow[nt] + PF_RESCALE_MARGIN) {
          const float alpha = __builtin_amdgcn_exp2f(mrow[nt] - mx);
          lrow[nt] *= alpha;
#pragma unroll
          for (int mt = 0; mt < 16; ++mt) o[nt][mt] *= alpha;
          mrow[nt] = mx;
        }
        const float mref = mrow[nt] == neg_inf() ? 0.0f : mrow[nt];
        float pv[8];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[4 * m + i] = __builtin_amdgcn_exp2f(s[m][nt][i] - mref);
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += pv[j];
        lrow[nt] += sum;
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[nt][j] = (_Float16)pv[j];
      }
#pragma unroll
      for (int f = 16; f < 32; ++f) {
        const int mt = f - 16;
        const half8_t a = ring[f % FR];
        if (f + FR < 32) ring[f % FR] = frag(f + FR);
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) o[nt][mt] = mfma16(a, pb[nt], o[nt][mt]);
      }
    }
    signal_count(consumed + st, lane);
  }

  // ---- write this group's normalised partial ------------------------------
  const int64_t rows_total = (int64_t)p.chunk * n_heads;
#pragma unroll
  for (int nt = 0; nt < PF_NT; ++nt) {
    const float l = wave_sum_xor_16_32(lrow[nt]);
    const int64_t r = row0 + nt * 16 + r16;
    if (r < rows_head) {
      const int64_t tq = r / p.gqa;
      const int gi = (int)(r - tq * p.gqa);
      const int64_t rowg = tq * n_heads + h * p.gqa + gi;
      const float f = l > 0.f ? 1.0f / l : 0.f;
      float* op = p.o_part + ((int64_t)group * rows_total + rowg) * D + 4 * g;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt)
        *reinterpret_cast<floatx4*>(op + 16 * mt) = o[nt][mt] * f;
      if (g == 0)
        p.lse_part[(int64_t)group * rows_total + rowg] =
            l > 0.f ? (mrow[nt] + __log2f(l)) * LN2 : neg_inf();
    }
  }
}

}  // namespace

int32_t prefill_rows_per_tile() { return PF_ROWS; }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const size_t shmem = sizeof(_Float16) * N_STAGES * STAGE_HALVES + RAW_DEPTH * RAW_STAGE;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shmem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t rows_head = (int64_t)p.chunk * p.gqa;
  const unsigned n_qtiles = (unsigned)((rows_head + PF_ROWS - 1) / PF_ROWS);
  dim3 grid((unsigned)p.n_groups, n_qtiles, (unsigned)p.n_kv);
  hipLaunchKernelGGL(prefill_kernel, grid, dim3(PF_THREADS), shmem, stream, p);
  return hipGetLastError();
}

}  // namespace kvattn
