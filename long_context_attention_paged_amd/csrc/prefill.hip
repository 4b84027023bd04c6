// a6: chunked-prefill attention over the paged Q8_0/Q4_0 cache.
//
// Source: the RX 9070 XT announcement (wqu.guru), bullet "Online Log-Sum-Exp
// prefill & pipelined prefetch": chunked prefill over pages with partial
// results accumulated by online LSE; micro-batch 512 from the Adaptive KV
// Streaming guide (alphalab.site, step ④: -ub 512). The kernel design is this
// library's.
//
// Grid (page groups, query tiles, KV heads); 256 threads = 4 wavefronts; a
// query tile is 256 rows (row = token * gqa + group member), 64 per wave.
// Each workgroup walks the pages of its group in 32-token sub-tiles: all 256
// threads dequantise the sub-tile into LDS as f16 (keys [token][dim], values
// [dim][slot] in the pool's slot order, value scale applied), then every wave
// computes S^T = Khat . Q'^T and O^T += Vhat^T . P'^T with
// v_mfma_f32_16x16x32_f16 (rows in the N dimension, four N-tiles), with the
// online softmax in base 2 in between. Sub-tiles are double-buffered: the
// global loads of the next sub-tile are in flight while the current one is
// multiplied. Each group writes normalised partial (o, lse) per row; the LSE
// merge combines the groups. Group g's workgroups for every query tile share
// an XCD (group count is kept a multiple of 8 where possible), so the
// dequantised pages they all read come from the same L2.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int PF_THREADS = 256;
constexpr int PF_NT = 2;                        // 16-row N-tiles per wave
constexpr int PF_ROWS = 4 * 16 * PF_NT;         // rows per workgroup
constexpr int K_LDS_STRIDE = 264;               // halves per key row (256 + pad)
constexpr int V_LDS_STRIDE = 40;                // halves per value dim row (32 + pad)
constexpr int K_LDS_HALVES = 32 * K_LDS_STRIDE;
constexpr int V_LDS_HALVES = D * V_LDS_STRIDE;
constexpr int STAGE_HALVES = K_LDS_HALVES + V_LDS_HALVES;
constexpr float PF_RESCALE_MARGIN = 8.0f;

struct Staged {
  u32x4 k0, k1;     // 32 key codes: token u = tid/8, block tid%8
  uint32_t ks;      // that block's scale (low half)
  u32x4 v;          // four value words: dims 16(4q+e)+d, lane group g
  u32x4 vs0, vs1;   // value scales of blocks 2q and 2q+1 for the 8 slots of g
};

__device__ __forceinline__ void stage_load(Staged& s, const uint8_t* krec, const uint8_t* vrec,
                                           int c, int tid) {
  const int u = tid >> 3, b = tid & 7;
  const uint8_t* kp = krec + (c * 32 + u) * D + 32 * b;
  s.k0 = load16_nt(kp);
  s.k1 = load16_nt(kp + 16);
  s.ks = *reinterpret_cast<const uint16_t*>(krec + K_SCALE_OFF + ((c * 32 + u) * 8 + b) * 2);
  s.v = load16_nt(vrec + (c * 1024 + tid * 4) * 4);
  const int g = (tid >> 4) & 3, q = tid >> 6;
  s.vs0 = load16_nt(vrec + V_SCALE_OFF + (((c * 8 + 2 * q) * 4 + g) * 8) * 2);
  s.vs1 = load16_nt(vrec + V_SCALE_OFF + (((c * 8 + 2 * q + 1) * 4 + g) * 8) * 2);
}

// Dequantise the staged registers into one LDS stage. Slots at or past
// kv_len (unwritten bytes) are stored as zeros.
__device__ __forceinline__ void stage_store(const Staged& s, _Float16* stage, int tid,
                                            int64_t tok0, int64_t kv_len) {
  const int u = tid >> 3, b = tid & 7;
  _Float16* krow = stage + u * K_LDS_STRIDE + 32 * b;
  if (tok0 + u < kv_len) {
    const half2_t d2 = as_h2(s.ks | (s.ks << 16));
    *reinterpret_cast<half8_t*>(krow + 0) = k_codes_to_f16(s.k0.x, s.k0.y, d2);
    *reinterpret_cast<half8_t*>(krow + 8) = k_codes_to_f16(s.k0.z, s.k0.w, d2);
    *reinterpret_cast<half8_t*>(krow + 16) = k_codes_to_f16(s.k1.x, s.k1.y, d2);
    *reinterpret_cast<half8_t*>(krow + 24) = k_codes_to_f16(s.k1.z, s.k1.w, d2);
  } else {
    const half8_t z = {};
    *reinterpret_cast<half8_t*>(krow + 0) = z;
    *reinterpret_cast<half8_t*>(krow + 8) = z;
    *reinterpret_cast<half8_t*>(krow + 16) = z;
    *reinterpret_cast<half8_t*>(krow + 24) = z;
  }
  const int d = tid & 15, g = (tid >> 4) & 3, q = tid >> 6;
  uint32_t mk[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int j0 = 2 * p, j1 = 2 * p + 1;
    const int u0 = 16 * (j0 >> 2) + 4 * g + (j0 & 3);
    const int u1 = 16 * (j1 >> 2) + 4 * g + (j1 & 3);
    mk[p] = (tok0 + u0 < kv_len ? 0x0000FFFFu : 0u) | (tok0 + u1 < kv_len ? 0xFFFF0000u : 0u);
  }
  _Float16* vbase = stage + K_LDS_HALVES;
  const uint32_t words[4] = {s.v.x, s.v.y, s.v.z, s.v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int dim = 16 * (4 * q + e) + d;
    const u32x4 sc = (e < 2 ? s.vs0 : s.vs1);
    const uint32_t scw[4] = {sc.x & mk[0], sc.y & mk[1], sc.z & mk[2], sc.w & mk[3]};
    half8_t val = v_codes_to_f16(words[e]);
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

__global__ __launch_bounds__(PF_THREADS, 1) void prefill_kernel(PrefillParams p) {
  extern __shared__ _Float16 lds[];  // two stages
  const int group = blockIdx.x, qtile = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int n_heads = p.n_kv * p.gqa;
  const int64_t rows_head = (int64_t)p.chunk * p.gqa;
  const int64_t kv_len = p.pos0 + p.chunk;
  const int64_t n_pages = (kv_len + PAGE - 1) / PAGE;
  const int64_t row0 = (int64_t)qtile * PF_ROWS + wave * 16 * PF_NT;  // this wave's first row

  // ---- query operands, row limits ------------------------------------------
  half8_t qb[PF_NT][8];
  int64_t limit[PF_NT];
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
      limit[nt] = p.pos0 + tq;
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qb[nt][ks] = half8_t{};
      limit[nt] = -1;
    }
  }
  // wave-uniform visibility bounds of this wave's rows
  const int64_t wr_lo = row0 < rows_head ? row0 : rows_head - 1;
  const int64_t wr_hi = (row0 + 16 * PF_NT - 1) < rows_head ? row0 + 16 * PF_NT - 1 : rows_head - 1;
  const int64_t wave_min_limit = p.pos0 + wr_lo / p.gqa;
  const int64_t wave_max_limit = p.pos0 + wr_hi / p.gqa;
  const bool wave_active = row0 < rows_head;
  // workgroup-wide last visible position: skip sub-tiles beyond it
  const int64_t tile_last_row = ((int64_t)qtile + 1) * PF_ROWS - 1 < rows_head
                                    ? ((int64_t)qtile + 1) * PF_ROWS - 1
                                    : rows_head - 1;
  const int64_t wg_max_pos = p.pos0 + tile_last_row / p.gqa;

  float mrow[PF_NT], lrow[PF_NT];
  floatx4 o[PF_NT][16];
#pragma unroll
  for (int nt = 0; nt < PF_NT; ++nt) {
    mrow[nt] = neg_inf();
    lrow[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) o[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- this group's sub-tiles -----------------------------------------------
  const int64_t pg0 = n_pages * group / p.n_groups;
  int64_t pg1 = n_pages * (group + 1) / p.n_groups;
  const int64_t last_page = wg_max_pos / PAGE;
  if (pg1 > last_page + 1) pg1 = last_page + 1;
  const int64_t n_sub = pg1 > pg0 ? (pg1 - pg0) * 4 : 0;

  auto rec_of = [&](int64_t sub, const uint8_t*& krec, const uint8_t*& vrec, int64_t& tok0,
                    int& c) -> bool {
    const int64_t lp = pg0 + (sub >> 2);
    c = (int)(sub & 3);
    tok0 = lp * PAGE + c * 32;
    const int32_t ph = p.page_table[lp];
    if (ph < 0 || ph >= p.n_phys) return false;
    krec = p.k_pool + ((int64_t)ph * p.n_kv + h) * K_REC;
    vrec = p.v_pool + ((int64_t)ph * p.n_kv + h) * V_REC;
    return true;
  };

  Staged stg;
  int64_t cur_tok0 = 0, nxt_tok0 = 0;
  bool cur_ok = false, nxt_ok = false;
  if (n_sub > 0) {
    const uint8_t *kr, *vr;
    int c;
    cur_ok = rec_of(0, kr, vr, cur_tok0, c);
    if (cur_ok) {
      stage_load(stg, kr, vr, c, tid);
      stage_store(stg, lds, tid, cur_tok0, kv_len);
    }
  }
  __syncthreads();

  for (int64_t sub = 0; sub < n_sub; ++sub) {
    _Float16* stage = lds + (sub & 1) * STAGE_HALVES;
    _Float16* next_stage = lds + ((sub + 1) & 1) * STAGE_HALVES;
    const bool has_next = sub + 1 < n_sub;
    if (has_next) {
      const uint8_t *kr, *vr;
      int c;
      nxt_ok = rec_of(sub + 1, kr, vr, nxt_tok0, c);
      if (nxt_ok && nxt_tok0 <= wg_max_pos) stage_load(stg, kr, vr, c, tid);
    }
    // ---- compute on the current stage (waves whose rows see any of it) ----
    if (cur_ok && wave_active && cur_tok0 <= wave_max_limit) {
      const _Float16* ks_lds = stage;
      const _Float16* vs_lds = stage + K_LDS_HALVES;
      floatx4 s[2][PF_NT];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) s[m][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const half8_t a = *reinterpret_cast<const half8_t*>(
              ks_lds + (16 * m + r16) * K_LDS_STRIDE + 64 * g + 8 * ks);
#pragma unroll
          for (int nt = 0; nt < PF_NT; ++nt) s[m][nt] = mfma16(a, qb[nt][ks], s[m][nt]);
        }
      }
      if (cur_tok0 + 31 > wave_min_limit) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int nt = 0; nt < PF_NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (cur_tok0 + 16 * m + 4 * g + i > limit[nt]) s[m][nt][i] = neg_inf();
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
      for (int mt = 0; mt < 16; ++mt) {
        const half8_t a =
            *reinterpret_cast<const half8_t*>(vs_lds + (16 * mt + r16) * V_LDS_STRIDE + 8 * g);
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) o[nt][mt] = mfma16(a, pb[nt], o[nt][mt]);
      }
    }
    if (has_next && nxt_ok && nxt_tok0 <= wg_max_pos)
      stage_store(stg, next_stage, tid, nxt_tok0, kv_len);
    cur_ok = has_next && nxt_ok && nxt_tok0 <= wg_max_pos;
    cur_tok0 = nxt_tok0;
    __syncthreads();
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
  const size_t shmem = sizeof(_Float16) * 2 * STAGE_HALVES;
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
