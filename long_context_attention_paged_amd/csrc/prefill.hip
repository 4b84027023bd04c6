// a6: chunked-prefill attention over the paged Q8_0/Q4_0 cache.
//
// Source: the RX 9070 XT announcement (wqu.guru), bullet "Online Log-Sum-Exp
// prefill & pipelined prefetch": chunked prefill over pages with partial
// results accumulated by online LSE; micro-batch 512 from the Adaptive KV
// Streaming guide (alphalab.site, step ④: -ub 512). The kernel design is this
// library's.
//
// Grid (page groups, query tiles, KV heads); 512 threads = 8 wavefronts, two
// per SIMD; a query tile is 256 rows (row = token * gqa + group member), 32
// per wave. Each workgroup walks the pages of its group in 32-token
// sub-tiles. Every wave does two jobs per sub-tile:
//  - it streams one eighth of the quantised bytes of a later sub-tile into a
//    private LDS slot by direct global->LDS loads, and dequantises its eighth
//    (4 key rows; 64 value dims x 16 slots) into an f16 stage: keys
//    [token][dim], values [dim][slot] in the pool's slot order with the value
//    scale applied;
//  - it computes S^T = Khat . Q'^T and O^T += Vhat^T . P'^T for its 32 rows
//    with v_mfma_f32_16x16x32_f16 (rows in the N dimension, two N-tiles) and
//    the online softmax in base 2 in between.
// Three f16 stages rotate; waves synchronise through per-stage LDS counters
// (eighths written, waves done reading) rather than workgroup barriers, so
// the two waves of a SIMD drift apart and one's products overlap the other's
// LDS reads and vector work. Each group writes a normalised partial (o, lse)
// per row; the LSE merge combines the groups.
#include "common.hpp"
#include "launch.hpp"

namespace kvattn {
namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_NT = 2;                        // 16-row N-tiles per wave
constexpr int PF_ROWS = PF_WAVES * 16 * PF_NT;  // rows per workgroup
constexpr int K_LDS_STRIDE = 264;               // halves per key row (256 + pad)
// A value dim row holds 32 slots (64 bytes, no pad); its four 16-byte slot
// groups are stored in the order g ^ ((dim >> 2) & 3), so the 16 rows one
// matrix-core operand read touches fall on distinct banks.
constexpr int V_LDS_STRIDE = 32;                // halves per value dim row
__device__ __forceinline__ int v_group(int dim, int g) { return g ^ ((dim >> 2) & 3); }
constexpr int K_LDS_HALVES = 32 * K_LDS_STRIDE;
constexpr int V_LDS_HALVES = D * V_LDS_STRIDE;
constexpr int STAGE_HALVES = K_LDS_HALVES + V_LDS_HALVES;  // one f16 sub-tile
constexpr int N_STAGES = 3;
constexpr float PF_RESCALE_MARGIN = 8.0f;
// Raw (quantised) share of one wave per sub-tile: 4 key rows (1 KB), 128
// value words (512 B; with Q8_0 values, V8, 1 KB of value codes), 4 x 16 B
// of key scales, 4 x 16 B of value scales.
constexpr int RAW_K = 0, RAW_V = 1024;
template <bool V8> constexpr int RAW_KS = V8 ? 2048 : 1536;
template <bool V8> constexpr int RAW_VS = V8 ? 2112 : 1600;
// Q5_1 keys add the 4 rows' bytes of fifth bits (128 B, after the 512 B of
// nibbles) and 4 x 16 B of block minimums after the scales.
template <int KT, bool V8> constexpr int RAW_WAVE = (V8 ? 2176 : 1664) + (KT == 2 ? 64 : 0);
template <int KT, bool V8> constexpr int RAW_STAGE = PF_WAVES * RAW_WAVE<KT, V8>;
constexpr int RAW_DEPTH = 2;                    // sub-tile i+2 refills sub-tile i's slot
constexpr int RAW_LOADS = 4;                    // direct loads per wave per sub-tile

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a page record straight into LDS (lane l's bytes land
// at lds_dst + 16 l). Buffer loads with the record in scalar registers, not
// global ones: the compiler counts a global load into LDS against the LDS
// counter as well, which turns every wait for the operand reads of the
// products into a wait for all of them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rec, int off, uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rec, (lds_void*)(lds_dst), 16, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_loads() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __asm__ __volatile__("" ::: "memory");
}

// Wait until an LDS counter reaches target. The counters only grow, and each
// wait is for work that the awaited waves reach without waiting on the
// waiter (see the loop in prefill_kernel), so it ends. The poll has no sleep
// (each round trip to LDS paces it, and a sleeping wave wakes late); it is
// capped all the same (2^20 polls, tens of milliseconds), so a broken
// invariant cannot hang the GPU. Returns false if the cap was reached: the
// kernel then raises the workspace's error flag at its end.
__device__ __forceinline__ bool wait_count(const int* c, int target) {
  bool reached = false;
  for (int spin = 0; spin < (1 << 20); ++spin) {
    // an LDS read (a generic one would also wait for the raw tile loads)
    const volatile __attribute__((address_space(3))) int* lc =
        (const volatile __attribute__((address_space(3))) int*)(c);
    if (__builtin_amdgcn_readfirstlane(*lc) >= target) {
      reached = true;
      break;
    }
  }
  __asm__ __volatile__("" ::: "memory");
  return reached;
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

// Wave w's raw share of sub-tile (group c of a page), placed so that its
// dequantisation reads and writes LDS without bank conflicts:
//  - key codes: lane i fetches row 4w + i%4, block (i/4)%8, half i/32 (16 B);
//  - value words: q = w/2, lane groups g = 2(w%2), 2(w%2)+1: 128 consecutive
//    words (lanes 0-31); Q8_0 value codes: the same dims and lane groups are
//    blocks 2q, 2q+1, 512 consecutive bytes each (lanes 0-31, 32-63);
//  - scales (lanes 0-7): key rows 4w..4w+3 (16 B each), then value blocks
//    2q, 2q+1 for the two lane groups (16 B each).
// With Q4_0 keys (KT) lanes 0-31 fetch row 4w + i%4, block (i/4)%8 (16 B:
// the block's 32 nibbles).
template <int KT, bool V8>
__device__ __forceinline__ void issue_raw(uint8_t* raw, const uint8_t* krec, const uint8_t* vrec,
                                          int c, int w, int lane) {
  const int q = w >> 1, gh = w & 1;
  const __amdgpu_buffer_rsrc_t kr = rec_rsrc(krec, KREC_OF<KT>);
  const __amdgpu_buffer_rsrc_t vr = rec_rsrc(vrec, V8 ? V8_REC : V_REC);
  if constexpr (KT == 2) {  // lanes 32-39: the fifth bits of rows 4w..4w+3 (32 B each)
    const int off = lane < 32 ? (c * 32 + 4 * w + (lane & 3)) * (D / 2) + 16 * ((lane >> 2) & 7)
                              : K5_HI_OFF + (c * 32 + 4 * w + ((lane - 32) >> 1)) * 32 + 16 * (lane & 1);
    if (lane < 40) dma16(kr, off, raw + RAW_K);
  } else if constexpr (KT == 1) {
    if (lane < 32)
      dma16(kr, (c * 32 + 4 * w + (lane & 3)) * (D / 2) + 16 * ((lane >> 2) & 7), raw + RAW_K);
  } else {
    dma16(kr, (c * 32 + 4 * w + (lane & 3)) * D + 32 * ((lane >> 2) & 7) + 16 * (lane >> 5),
          raw + RAW_K);
  }
  if constexpr (V8)
    dma16(vr, c * 8192 + (2 * q + (lane >> 5)) * 1024 + 2 * gh * 256 + (lane & 31) * 16,
          raw + RAW_V);
  else if (lane < 32)
    dma16(vr, (((c * 4 + q) * 4 + 2 * gh) * 64) * 4 + lane * 16, raw + RAW_V);
  // scales, two loads (one per record): lanes 0-3 key rows 4w..4w+3, lanes
  // 8-11 their Q5_1 block minimums; lanes 4-7 value blocks 2q, 2q+1 of the two
  // lane groups
  if (lane < 4 || (KT == 2 && lane >= 8 && lane < 12)) {
    const int off = lane < 4 ? KSCALE_OF<KT> + (c * 32 + 4 * w + lane) * 16
                             : K5_M_OFF + (c * 32 + 4 * w + lane - 8) * 16;
    dma16(kr, off, raw + RAW_KS<V8>);
  }
  if (lane >= 4 && lane < 8) {
    const int vs_off = V8 ? K_SCALE_OFF : V_SCALE_OFF;
    dma16(vr, vs_off + ((c * 8 + 2 * q + ((lane - 4) >> 1)) * 4 + 2 * gh + (lane & 1)) * 16,
          raw + RAW_KS<V8>);
  }
}

// The raw share's bytes a lane needs, read in one block that also waits for
// them. Written as instructions of their own: as plain loads the compiler
// would first wait for every raw tile load in flight (those write LDS too),
// including the next sub-tile's, which is still meant to be in flight.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct RawIn {
  u32x4 k;      // 16 key codes
  u32x2 v;      // 2 value words
  u32x4 vs;     // 8 value scales
  uint32_t ks;  // key scale (low 16 bits)
};
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) uint8_t*)(p));
}
struct RawIn8 {
  u32x4 k;      // 16 key codes
  u32x4 v;      // 16 value codes: two dims x 8 slots
  u32x4 vs;     // 8 value scales
  uint32_t ks;  // key scale (low 16 bits)
};
__device__ __forceinline__ RawIn8 read_raw8(const uint8_t* k, const uint8_t* v, const uint8_t* vs,
                                            const uint8_t* ks) {
  RawIn8 r;
  __asm__ __volatile__(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_u16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.k), "=&v"(r.v), "=&v"(r.vs), "=&v"(r.ks)
      : "v"(lds_addr(k)), "v"(lds_addr(v)), "v"(lds_addr(vs)), "v"(lds_addr(ks))
      : "memory");
  return r;
}
__device__ __forceinline__ RawIn read_raw(const uint8_t* k, const uint8_t* v, const uint8_t* vs,
                                          const uint8_t* ks) {
  RawIn r;
  __asm__ __volatile__(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b64 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_u16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r.k), "=&v"(r.v), "=&v"(r.vs), "=&v"(r.ks)
      : "v"(lds_addr(k)), "v"(lds_addr(v)), "v"(lds_addr(vs)), "v"(lds_addr(ks))
      : "memory");
  return r;
}

// Dequantise wave w's raw share into an f16 stage. Only the first n_live
// slots of the sub-tile hold data (later slots are unwritten bytes past
// kv_len; n_live is 0 for a page the table does not map): their keys and
// value scales are replaced by zeros. ln is the lane index.
// Keys, lane (u, b, hh) = (l%4, (l/4)%8, l/32): 16 codes of row 4w + u.
// Values, lane (d, ep, gl) = (l%16, (l/16)%2, l/32): words e = 2ep, 2ep+1 of
// dim group q = w/2, lane group g = 2(w%2) + gl; with Q8_0 values the same
// dims are the lane's 16-byte piece (row d) of block 2q + ep.
template <int KT, bool V8>
__device__ __forceinline__ void dequant_raw(const uint8_t* raw, _Float16* stage, int w, int ln,
                                            int n_live) {
  const int u = ln & 3, b = (ln >> 2) & 7, hh = ln >> 5;
  const int q = w >> 1, d = ln & 15, ep = (ln >> 4) & 1, gl = ln >> 5;
  const int g = 2 * (w & 1) + gl;
  RawIn in;
  u32x4 v8 = {0u, 0u, 0u, 0u};
  // Q4_0 keys: the lane's block chunk (row u, block b) is lane l%32's load
  const int koff = KT != 0 ? (ln & 31) * 16 : ln * 16;
  if constexpr (V8) {
    const RawIn8 r8 = read_raw8(raw + RAW_K + koff, raw + RAW_V + (ep * 32 + gl * 16 + d) * 16,
                                raw + RAW_VS<V8> + (ep * 2 + gl) * 16,
                                raw + RAW_KS<V8> + u * 16 + 2 * b);
    in.k = r8.k;
    in.vs = r8.vs;
    in.ks = r8.ks;
    v8 = r8.v;
  } else {
    in = read_raw(raw + RAW_K + koff, raw + RAW_V + ((gl * 16 + d) * 4 + 2 * ep) * 4,
                  raw + RAW_VS<V8> + (ep * 2 + gl) * 16, raw + RAW_KS<V8> + u * 16 + 2 * b);
  }
  // n_live is wave-uniform and 32 on every sub-tile but a ragged last one
  const bool full = n_live >= 32;
  {
    const uint32_t ks = in.ks & 0xFFFFu;
    uint32_t dw = ks | (ks << 16);
    if (!full && 4 * w + u >= n_live) dw = 0u;  // zero scale -> zeros
    const half2_t d2 = as_h2(dw);
    _Float16* krow = stage + (4 * w + u) * K_LDS_STRIDE + 32 * b + 16 * hh;
    if constexpr (KT == 2) {  // as Q4_0, with the fifth bits and the block minimum
      uint32_t kh, km;
      __asm__ __volatile__(
          "ds_read_u16 %0, %2\n\t"
          "ds_read_u16 %1, %3\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(kh), "=&v"(km)
          : "v"(lds_addr(raw + RAW_K + 512 + u * 32 + 4 * b + 2 * hh)),
            "v"(lds_addr(raw + RAW_KS<V8> + 128 + u * 16 + 2 * b))
          : "memory");
      uint32_t mw = km & 0xFFFFu;
      if (!full && 4 * w + u >= n_live) mw = 0u;
      const half2_t m2 = as_h2(mw | (mw << 16));
      *reinterpret_cast<half8_t*>(krow + 0) = k5_codes_to_f16(hh ? in.k.z : in.k.x, kh & 0xFFu, d2, m2);
      *reinterpret_cast<half8_t*>(krow + 8) = k5_codes_to_f16(hh ? in.k.w : in.k.y, (kh >> 8) & 0xFFu, d2, m2);
    } else if constexpr (KT == 1) {  // words 4b + 2hh, +1: dims 32b + 16hh + 0..7, 8..15
      *reinterpret_cast<half8_t*>(krow + 0) = k4_codes_to_f16(hh ? in.k.z : in.k.x, NIB_LO, NIB_HI, d2);
      *reinterpret_cast<half8_t*>(krow + 8) = k4_codes_to_f16(hh ? in.k.w : in.k.y, NIB_LO, NIB_HI, d2);
    } else {
      *reinterpret_cast<half8_t*>(krow + 0) = k_codes_to_f16(in.k.x, in.k.y, d2);
      *reinterpret_cast<half8_t*>(krow + 8) = k_codes_to_f16(in.k.z, in.k.w, d2);
    }
  }
  {
    // scales of block 2q + ep for lane group g (in.vs), masked past n_live
    uint32_t scw[4] = {in.vs[0], in.vs[1], in.vs[2], in.vs[3]};
    if (!full) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int u0 = 16 * ((2 * p) >> 2) + 4 * g + ((2 * p) & 3);
        const int u1 = 16 * ((2 * p + 1) >> 2) + 4 * g + ((2 * p + 1) & 3);
        const uint32_t mk = (u0 < n_live ? 0x0000FFFFu : 0u) | (u1 < n_live ? 0xFFFF0000u : 0u);
        scw[p] &= mk;
      }
    }
    _Float16* vbase = stage + K_LDS_HALVES;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int dim = 16 * (4 * q + 2 * ep + i) + d;
      half8_t val;
      if constexpr (V8)
        val = v8_codes_to_f16(i ? v8.z : v8.x, i ? v8.w : v8.y);
      else
        val = v_codes_to_f16(in.v[i]);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const half2_t pr = {val[2 * p], val[2 * p + 1]};
        const half2_t r = pr * as_h2(scw[p]);
        val[2 * p] = r[0];
        val[2 * p + 1] = r[1];
      }
      *reinterpret_cast<half8_t*>(vbase + dim * V_LDS_STRIDE + 8 * v_group(dim, g)) = val;
    }
  }
}

struct SubTiles {
  int64_t pg0, pg1;  // this group's logical pages [pg0, pg1)
  int n_sub;         // 32-token sub-tiles to visit
};

// Page records of a group, 64 pages at a time in one VGPR (lane i holds the
// record index of page pg0 + first + i, or -1 when the table does not map
// it), read back with readlane: the loop then issues no page-table loads of
// its own, whose waits would also drain the raw tile stream.
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

template <int KT, bool V8>
__global__ __launch_bounds__(PF_THREADS) void prefill_kernel(PrefillParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
  _Float16* lds = reinterpret_cast<_Float16*>(lds_raw);                      // f16 stages
  uint8_t* raw_ring = lds_raw + N_STAGES * STAGE_HALVES * sizeof(_Float16);  // raw slots
  // Per stage: eighths written, waves done reading (both only grow; round r
  // of stage s is sub-tile 3r + s).
  __shared__ int counters[2 * N_STAGES];
  int* produced = counters;
  int* consumed = counters + N_STAGES;

  const int group = blockIdx.x, qtile = blockIdx.y, h = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int n_heads = p.n_kv * p.gqa;
  const int64_t rows_head = (int64_t)p.chunk * p.gqa;
  const int64_t kv_len = p.pos0 + p.chunk;

  // ---- this group's sub-tiles (32 tokens each) ------------------------------
  const int64_t tile_last_row = ((int64_t)qtile + 1) * PF_ROWS - 1 < rows_head
                                    ? ((int64_t)qtile + 1) * PF_ROWS - 1
                                    : rows_head - 1;
  const int64_t wg_max_pos = p.pos0 + tile_last_row / p.gqa;  // last key any row here sees
  SubTiles t;
  const int64_t span = p.pg_end - p.pg_begin;  // the groups split [pg_begin, pg_end)
  t.pg0 = p.pg_begin + span * group / p.n_groups;
  t.pg1 = p.pg_begin + span * (group + 1) / p.n_groups;
  if (t.pg1 > wg_max_pos / PAGE + 1) t.pg1 = wg_max_pos / PAGE + 1;
  t.n_sub = t.pg1 > t.pg0 ? (int)((t.pg1 - t.pg0) * 4) : 0;
  if (t.n_sub > 0) {  // drop trailing 32-token groups no row sees
    const int64_t last_tok0 = t.pg0 * PAGE + (int64_t)(t.n_sub - 1) * 32;
    if (last_tok0 > wg_max_pos) t.n_sub -= (int)((last_tok0 - wg_max_pos + 31) / 32);
  }
  const int n_sub = t.n_sub;
  PageWindow win;
  win.load(p, t, 0, h, lane);
  if (tid < 2 * N_STAGES) counters[tid] = 0;

  uint8_t* const my_raw = raw_ring + wave * RAW_WAVE<KT, V8>;
  auto issue = [&](int sub) {
    const int32_t r = win.record(sub);
    const int64_t rec = r >= 0 ? r : 0;  // unmapped pages load record 0, then zero it
    int ln = lane;
    __asm__ __volatile__("" : "+v"(ln));  // recompute lane offsets here, do not hold them
    issue_raw<KT, V8>(my_raw + (sub % RAW_DEPTH) * RAW_STAGE<KT, V8>, p.k_pool + rec * KREC_OF<KT>,
                  p.v_pool + rec * (V8 ? V8_REC : V_REC), r >= 0 ? (sub & 3) : 0, wave, ln);
  };
  auto dequant = [&](int sub) {
    const int64_t left = kv_len - (t.pg0 * PAGE + (int64_t)sub * 32);
    const int n_live = win.record(sub) < 0 ? 0 : left >= 32 ? 32 : (int)left;
    int ln = lane;
    __asm__ __volatile__("" : "+v"(ln));  // recompute lane offsets here, do not hold them
    dequant_raw<KT, V8>(my_raw + (sub % RAW_DEPTH) * RAW_STAGE<KT, V8>,
                    lds + (sub % N_STAGES) * STAGE_HALVES, wave, ln, n_live);
  };
  // start the raw stream before anything else
  if (n_sub > 0) issue(0);
  if (n_sub > 1) issue(1);

  // ---- query operands, row limits ------------------------------------------
  const int64_t row0 = (int64_t)qtile * PF_ROWS + wave * 16 * PF_NT;  // this wave's first row
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
  __syncthreads();  // counters cleared

  bool gave_up = false;  // a wait on another wave reached its cap (never expected)
  // Step i: multiply sub-tile i once all eighths of it are in, then
  // dequantise this wave's eighth of sub-tile i+1. The slowest wave never
  // waits on a faster one: what it needs (sub-tile i-2 read, sub-tile i
  // written) every other wave finished before step i.
  if (n_sub > 0) {
    if (n_sub > 1) wait_loads<RAW_LOADS>(); else wait_loads<0>();
    dequant(0);
    signal_count(produced + 0, lane);
    if (n_sub > 2) issue(2);
  }
  // Dequantise this wave's eighth of sub-tile nx into stage nx%3 (once every
  // wave has read sub-tile nx-3 from it), then refill the raw slot with
  // sub-tile nx+2.
  auto produce = [&](int nx) {
    if (nx < n_sub) {
      if (nx + 1 < n_sub) wait_loads<RAW_LOADS>(); else wait_loads<0>();  // raw sub-tile nx in
      if (nx >= N_STAGES)
        gave_up |= !wait_count(consumed + nx % N_STAGES, PF_WAVES * (nx / N_STAGES));
      // Every wave waits for all eighths of a stage, so a dequantising wave
      // holds up the workgroup: it outranks its SIMD partner's products
      // until its eighth is published.
      __builtin_amdgcn_s_setprio(2);
      dequant(nx);
      signal_count(produced + nx % N_STAGES, lane);  // also: raw slot of nx has been read
      __builtin_amdgcn_s_setprio(0);
      if (nx + 2 < n_sub) issue(nx + 2);
    }
  };
  // Every wave multiplies first and dequantises after; the waves of a SIMD
  // still drift apart, so one's dequantisation overlaps the other's
  // products. (Measured: taking the jobs in opposite orders on the two waves
  // of a SIMD, or dequantising first everywhere, is slower.)
  for (int sub = 0; sub < n_sub; ++sub) {
    if (((sub + 3) >> 2) >= win.first + 64) {  // sub .. sub + 3 stay in the window
      wait_loads<0>();
      win.load(p, t, sub >> 2, h, lane);
    }
    const int st = sub % N_STAGES;
    gave_up |= !wait_count(produced + st, PF_WAVES * (sub / N_STAGES + 1));
    const int64_t cur_tok0 = t.pg0 * PAGE + (int64_t)sub * 32;
    const bool compute = win.record(sub) >= 0 && wave_active && cur_tok0 <= wave_max_limit;
    if (compute) {
      // The sub-tile's 32 operand fragments (16 of keys, then 16 of values)
      // go through a ring of FR registers, read FR fragments ahead, so LDS
      // latency is hidden behind the products and, for the first values,
      // behind the softmax. A scheduling barrier after each refill keeps the
      // read ahead of the products: without it the compiler sinks every read
      // next to its first use, leaving two fragments in flight and a full
      // LDS round trip exposed every second fragment (measured: three
      // fragments ahead with the barriers is 2-3% faster per layer than the
      // ring of four without them; four ahead with them spills a query
      // fragment into the loop).
      constexpr int FR = 3;
      int ln = lane;
      __asm__ __volatile__("" : "+v"(ln));  // recompute lane offsets here, do not hold them
      const _Float16* kbase = lds + st * STAGE_HALVES + (ln & 15) * K_LDS_STRIDE + 64 * (ln >> 4);
      const _Float16* vbase =
          lds + st * STAGE_HALVES + K_LDS_HALVES + (ln & 15) * V_LDS_STRIDE +
          8 * v_group(ln & 15, ln >> 4);  // rows 16 (f - 16) + (ln & 15): same swizzle
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
        __builtin_amdgcn_sched_barrier(0);
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
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int nt = 0; nt < PF_NT; ++nt) o[nt][mt] = mfma16(a, pb[nt], o[nt][mt]);
      }
    }
    signal_count(consumed + st, lane);
    produce(sub + 1);
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
  if (gave_up && p.flag && lane == 0)  // wave-uniform
    __hip_atomic_fetch_or(p.flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int32_t prefill_rows_per_tile() { return PF_ROWS; }

template <int KT, bool V8>
hipError_t launch_prefill_v(const PrefillParams& p, hipStream_t stream) {
  const size_t shmem = sizeof(_Float16) * N_STAGES * STAGE_HALVES + RAW_DEPTH * RAW_STAGE<KT, V8>;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e =
      set_lds_limit(lds_set, reinterpret_cast<const void*>(&prefill_kernel<KT, V8>), shmem);
  if (e != hipSuccess) return e;
  const int64_t rows_head = (int64_t)p.chunk * p.gqa;
  const unsigned n_qtiles = (unsigned)((rows_head + PF_ROWS - 1) / PF_ROWS);
  dim3 grid((unsigned)p.n_groups, n_qtiles, (unsigned)p.n_kv);
  hipLaunchKernelGGL((prefill_kernel<KT, V8>), grid, dim3(PF_THREADS), shmem, stream, p);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  if (p.k_type == 2) return p.v_q8 ? launch_prefill_v<2, true>(p, stream) : launch_prefill_v<2, false>(p, stream);
  if (p.k_type == 1) return p.v_q8 ? launch_prefill_v<1, true>(p, stream) : launch_prefill_v<1, false>(p, stream);
  return p.v_q8 ? launch_prefill_v<0, true>(p, stream) : launch_prefill_v<0, false>(p, stream);
}

}  // namespace kvattn
