// a3/a5: decode and verify attention over the paged Q8_0/Q4_0 cache, split
// over pages; each split writes a partial (o, lse) that merge.hip combines by
// log-sum-exp.
//
// Sources: the RX 9070 XT announcement (wqu.guru), bullet "Stream-optimized
// speculative decoding": paged decode attention extended to verify batches;
// the Adaptive KV Streaming guide (alphalab.site), step ④: flash attention
// over Q8_0 K / Q4_0 V. The kernel design below is this library's.
//
// Work decomposition. Grid (splits, KV heads); 512 threads = 8 wavefronts,
// one workgroup per CU. A split owns a contiguous run of pages (or block-list
// entries); wavefront w handles 32-token group w % 4 of the pages of one
// part of the run (waves 4-7 the first 12/32 of it, waves 0-3 the rest), so
// four waves stream the four quarters of one page together. A CU-sized
// split halves the partials written per layer against two 4-wave workgroups
// per CU. Every page-record load is a buffer load straight into LDS whose
// base sits in scalar registers.
// Per 32-token group a wave computes
//   S^T (32 tokens x R rows) = Khat (32 x 256) . Q'^T      (16 mfma per N-tile)
//   O^T (256 dims x R rows) += Vhat^T (256 x 32) . P'^T    (16 mfma per N-tile)
// with v_mfma_f32_16x16x32_f16, R = query rows (n_q_tok * gqa) padded to 16
// (NT = 1) or 32 (NT = 2). Query rows ride in the N dimension so the row-wise
// softmax needs only the 4-lane-group reduction of one column, and the
// S^T accumulator layout is exactly the B-operand layout of the PV product,
// so probabilities never leave registers.
//
// Dequantisation happens in registers: K bytes -> f16 via the 0x64 exponent
// trick and one f16 multiply by the block scale; V nibbles -> exact f16
// (code - 8), with the per-(token, block) V scale folded into P' instead.
// Q' = q * scale * log2(e) in f16; softmax runs in base 2 with a lazily
// updated reference max (rescale only when a tile max exceeds it by 8), so
// P' <= 256 fits f16 and the O accumulators are rarely touched.
#include "common.hpp"
#include "launch.hpp"
#include "qround.hpp"

namespace kvattn {
namespace {

// The lazy reference max lets P' reach 2^RESCALE_MARGIN before a rescale.
// The value scale is folded into P' in f16, so |P' * d_V| <= 2^3 * 8188 =
// 65504 for every value block whose scale a finite |v| <= 65504 gives
// (Q4_0: |d_V| <= 65504 / 8): the products stay finite in f16.
constexpr float RESCALE_MARGIN = 3.0f;  // log2 units

constexpr int SLOW_SHARE = 12;          // 32nds of a split's units for waves 4-7
// One 32-token tile of one KV head in LDS:
//   [0, 8320)      key codes: 8 loads of 4 whole token rows (1 KB contiguous in
//                  the page); load i lands at kbase(i) with its 16-byte chunks
//                  rotated by 4 per row, so the matrix-core operand reads
//                  (16 rows x one 16-byte column each) hit 16 distinct bank groups;
//   [8320, 8832)   key scales;
//   [8832, 12928)  value words (4 x 1 KB, lane-ordered: each lane reads its own);
//   [12928, 13440) value scales.
// With Q8_0 values the value codes take 8 x 1 KB (lane-ordered the same way),
// the scales follow at 17024 and a slot is 17536 bytes. With Q4_0 keys (KT)
// the key codes take 4 loads of 8 token rows (128 B each) placed at
// k4base(i), 4288 bytes in all, and everything after moves down.
constexpr int SLOT_K = 0;
// With Q5_1 keys (KT 2) the 32 rows' bytes of fifth bits (1 KB) follow the
// nibbles at 4288, the scales d sit at 5312 and the minimums m after them.
constexpr int SLOT_KH = 4288;
template <int KT> constexpr int SLOT_KS = KT == 0 ? 8320 : KT == 1 ? 4288 : 5312;
template <int KT> constexpr int SLOT_V = SLOT_KS<KT> + (KT == 2 ? 1024 : 512);
template <int KT, bool V8> constexpr int SLOT_VS = SLOT_V<KT> + (V8 ? 8192 : 4096);
template <int KT, bool V8> constexpr int SLOT_BYTES = SLOT_VS<KT, V8> + 512;
constexpr int Q_LDS_STRIDE = 264;       // halves per query row in LDS (256 + pad)

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer (one page record) straight into LDS: the
// record base lives in scalar registers, the lane part is a 32-bit offset.
// The loads are marked non-temporal (cache policy NT): every KV byte is read
// once per launch, so keeping it in the caches only evicts what is reused
// (measured: 6% off verify-262k and 11% off decode-131k per layer).
constexpr int LOAD_NT = 2;
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rec, int lane_off, int wave_off,
                                      uint8_t* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rec, (lds_void*)(lds_dst), 16, lane_off, wave_off, 0,
                                           LOAD_NT);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t record(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}

// A copy of the lane id the compiler cannot see through, so per-lane offsets
// derived from it are recomputed where used rather than held across the loop.
__device__ __forceinline__ int opaque_lane() {
  int ln = __lane_id();
  __asm__ volatile("" : "+v"(ln));
  return ln;
}

// Wait until at most n direct-to-LDS loads of this wave are outstanding
// (vmcnt counts them in issue order), then fence the compiler.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __asm__ __volatile__("" ::: "memory");
}

// Direct loads of one tile (32-token group c of a page record) into an LDS
// slot, in two parts so each can be refilled as soon as it is consumed:
//   keys   (9 loads): 8 x 1 KB codes + 512 B scales (lanes 0..31);
//   values (5 loads): 4 x 1 KB words + 512 B scales (lanes 0..31);
//            9 loads with Q8_0 values (8 x 1 KB codes + scales).
// Lane (r16, g) brings exactly the 16-byte code chunks it will feed to the
// matrix cores, so those LDS reads are lane-local and conflict-free.
template <int KT> constexpr int K_LOADS = KT == 0 ? 9 : KT == 1 ? 5 : 7;
template <bool V8> constexpr int V_LOADS = V8 ? 9 : 5;

// LDS base of key load i (4 token rows): 1 KB apart plus a 16-byte shift per
// row quad (i % 4) and 64 bytes per M-tile (i / 4), so loads never overlap.
__device__ __forceinline__ int kbase(int i) { return i * 1024 + 16 * (i & 3) + 64 * (i >> 2); }
// Position (16-byte unit) inside a key load of chunk s (0..15) of row a (0..3).
__device__ __forceinline__ int kpos(int a, int s) { return 16 * a + ((s + 4 * a) & 15); }

// Q4_0 keys: load i (tokens 8i..8i+7 of the group) lands at k4base(i); lane
// p brings 16-byte chunk s = (p%8) ^ (a/2) of row a = p/8, so chunk s of row
// a sits at k4pos(a, s). The 64-byte step per load and the XOR spread the 16
// rows one matrix-core operand read touches over distinct banks.
__device__ __forceinline__ int k4base(int i) { return i * 1088; }
__device__ __forceinline__ int k4pos(int a, int s) { return a * 128 + 16 * (s ^ (a >> 1)); }

template <int KT>
__device__ __forceinline__ void issue_keys(uint8_t* slot, const uint8_t* krec, int c) {
  if constexpr (KT != 0) {
    const __amdgpu_buffer_rsrc_t r = record(krec, KREC_OF<KT>);
    const int lane = opaque_lane();
    const int a = lane >> 3, s = (lane & 7) ^ (a >> 1);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(r, a * 128 + 16 * s, (c * 32 + 8 * i) * 128, slot + SLOT_K + k4base(i));
    if constexpr (KT == 2) dma16(r, lane * 16, K5_HI_OFF + c * 1024, slot + SLOT_KH);
    if (lane < 32) dma16(r, lane * 16, KSCALE_OF<KT> + c * 512, slot + SLOT_KS<KT>);
    if constexpr (KT == 2)
      if (lane < 32) dma16(r, lane * 16, K5_M_OFF + c * 512, slot + SLOT_KS<KT> + 512);
    return;
  }
  const __amdgpu_buffer_rsrc_t r = record(krec, K_REC);
  // lane p of load i brings chunk s = (p%16 - 4a) & 15 of row a = p/16
  const int lane = opaque_lane();
  const int a = lane >> 4, s = ((lane & 15) - 4 * a) & 15;
#pragma unroll
  for (int i = 0; i < 8; ++i) dma16(r, a * D + 16 * s, (c * 32 + 4 * i) * D, slot + SLOT_K + kbase(i));
  if (lane < 32) dma16(r, lane * 16, K_SCALE_OFF + c * 512, slot + SLOT_KS<0>);
}

template <int KT, bool V8>
__device__ __forceinline__ void issue_values(uint8_t* slot, const uint8_t* vrec, int c) {
  constexpr int NQ = V8 ? 8 : 4;
  const __amdgpu_buffer_rsrc_t r = record(vrec, V8 ? V8_REC : V_REC);
  // value codes are stored lane-ordered: load q of group c is 1 KB at (NQ*c + q) KB
  const int lane = opaque_lane();
#pragma unroll
  for (int q = 0; q < NQ; ++q) dma16(r, lane * 16, (c * NQ + q) * 1024, slot + SLOT_V<KT> + q * 1024);
  if (lane < 32)
    dma16(r, lane * 16, (V8 ? K_SCALE_OFF : V_SCALE_OFF) + c * 512, slot + SLOT_VS<KT, V8>);
}


template <int NT>
struct State {
  const _Float16* q_lds;  // q' = q * scale * log2(e) in f16, [NT*16 rows][264]
  int64_t limit[NT];      // last visible key position of this lane's row
  float m[NT];            // reference max (log2 units) of this lane's row
  float l[NT];            // this lane's share of the row's sum of P'
  floatx4 o[NT][16];      // O^T accumulators: dims 16mt + 4g + i, row nt*16 + r16
};

template <int NT, int KT, bool V8, typename MidFn>
__device__ __forceinline__ void compute_tile(State<NT>& st, uint8_t* slot, int64_t tok0,
                                             int64_t kv_len, int64_t min_limit, int lane, int r16,
                                             int g, uint32_t nib_lo, uint32_t nib_hi, MidFn&& after_keys) {
  // ---- S^T = Khat . Q'^T --------------------------------------------------
  // Both 16-token halves (m) share each q' operand read.
  floatx4 s[2][NT];
  half2_t dlo[2], dhi[2], mlo[2], mhi[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const uint32_t sw = *reinterpret_cast<const uint32_t*>(slot + SLOT_KS<KT> + (16 * m + r16) * 16 + 4 * g);
    dlo[m] = as_h2((sw & 0xFFFFu) | (sw << 16));
    dhi[m] = as_h2((sw >> 16) | (sw & 0xFFFF0000u));
    if constexpr (KT == 2) {  // block minimums, laid out as the scales
      const uint32_t mw =
          *reinterpret_cast<const uint32_t*>(slot + SLOT_KS<KT> + 512 + (16 * m + r16) * 16 + 4 * g);
      mlo[m] = as_h2((mw & 0xFFFFu) | (mw << 16));
      mhi[m] = as_h2((mw >> 16) | (mw & 0xFFFF0000u));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[m][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // lane offsets recomputed per tile from an opaque copy of the lane id, so
  // they are not kept live across the loop
  int ln = lane;
  __asm__ volatile("" : "+v"(ln));
  const int kr16 = ln & 15, kg = ln >> 4;
  // Each step's LDS operands (key words, fifth bits, query fragments) are read
  // one step ahead, before the previous step is converted and multiplied, so
  // their latency hides behind that work; the scheduling barrier at the end
  // of a step keeps the reads there.
  auto qfrag = [&](int ks, int nt) -> half8_t {
    return *reinterpret_cast<const half8_t*>(st.q_lds + (nt * 16 + r16) * Q_LDS_STRIDE + 64 * g +
                                             8 * ks);
  };
  if constexpr (KT != 0) {
    // dims 64g + 8ks .. +7 are word 8g + ks of the row: chunk 2g + ks/4, word ks%4
    auto kword = [&](int ks, int m) -> uint32_t {
      return *reinterpret_cast<const uint32_t*>(slot + SLOT_K + k4base(2 * m + (kr16 >> 3)) +
                                                k4pos(kr16 & 7, 2 * kg + (ks >> 2)) + 4 * (ks & 3));
    };
    auto kfifth = [&](int ks, int m) -> uint32_t {
      return slot[SLOT_KH + (16 * m + kr16) * 32 + 8 * kg + ks];
    };
    uint32_t wc[2], ec[2] = {0u, 0u};
    half8_t qc[NT];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      wc[m] = kword(0, m);
      if constexpr (KT == 2) ec[m] = kfifth(0, m);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qc[nt] = qfrag(0, nt);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int hh = ks >> 2;
      uint32_t wn[2] = {0u, 0u}, en[2] = {0u, 0u};
      half8_t qn[NT];
      if (ks < 7) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          wn[m] = kword(ks + 1, m);
          if constexpr (KT == 2) en[m] = kfifth(ks + 1, m);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) qn[nt] = qfrag(ks + 1, nt);
      }
      half8_t a[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        if constexpr (KT == 2) {
          a[m] = k5_codes_to_f16(wc[m], ec[m], nib_lo, nib_hi, hh ? dhi[m] : dlo[m],
                                 hh ? mhi[m] : mlo[m]);
        } else {
          a[m] = k4_codes_to_f16(wc[m], nib_lo, nib_hi, hh ? dhi[m] : dlo[m]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int m = 0; m < 2; ++m) s[m][nt] = mfma16(a[m], qc[nt], s[m][nt]);
      __builtin_amdgcn_sched_barrier(0);
      if (ks < 7) {
#pragma unroll
        for (int m = 0; m < 2; ++m) wc[m] = wn[m], ec[m] = en[m];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) qc[nt] = qn[nt];
      }
    }
  } else {
    // bytes 64g + 16j of token 16m + r16: load 4m + r16/4, row r16%4, chunk 4g + j
    auto kwords = [&](int j, int m) -> u32x4 {
      return *reinterpret_cast<const u32x4*>(slot + SLOT_K + kbase(4 * m + (kr16 >> 2)) +
                                             16 * kpos(kr16 & 3, 4 * kg + j));
    };
    u32x4 w4[2];
    half8_t qc[NT];
#pragma unroll
    for (int m = 0; m < 2; ++m) w4[m] = kwords(0, m);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) qc[nt] = qfrag(0, nt);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 w4n[2];
      if (j < 3) {
#pragma unroll
        for (int m = 0; m < 2; ++m) w4n[m] = kwords(j + 1, m);
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int ks = 2 * j + h2;
        half8_t qn[NT];
        if (ks < 7) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) qn[nt] = qfrag(ks + 1, nt);
        }
        half8_t a[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
          a[m] = k_codes_to_f16(h2 ? w4[m].z : w4[m].x, h2 ? w4[m].w : w4[m].y,
                                ks < 4 ? dlo[m] : dhi[m]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int m = 0; m < 2; ++m) s[m][nt] = mfma16(a[m], qc[nt], s[m][nt]);
        __builtin_amdgcn_sched_barrier(0);
        if (ks < 7) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) qc[nt] = qn[nt];
        }
      }
      if (j < 3) {
#pragma unroll
        for (int m = 0; m < 2; ++m) w4[m] = w4n[m];
      }
    }
  }
  // the key half of the slot has been read: let the caller refill it
  after_keys();
  // ---- masks: causal rows, tokens past kv_len ------------------------------
  if (__builtin_expect(tok0 + 31 > min_limit, 0)) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tok0 + 16 * m + 4 * g + i > st.limit[nt]) s[m][nt][i] = neg_inf();
    // Slots past kv_len hold unwritten bytes: their V scales are zeroed in
    // this wave's slot (the values have landed; only this wave reads the
    // slot, and its LDS accesses complete in order), so the PV loop reads the
    // scales as they are. Scale word k (block k / 16, slot group (k / 4) % 4,
    // pair k % 4) holds slots 2(k % 4) and 2(k % 4) + 1 of that group.
    if (tok0 + 32 > kv_len) {  // uniform
      uint32_t* vs = reinterpret_cast<uint32_t*>(slot + SLOT_VS<KT, V8>);
#pragma unroll
      for (int k0 = 0; k0 < 128; k0 += 64) {
        const int k = k0 + lane, gg = (k >> 2) & 3, j0 = 2 * (k & 3), j1 = j0 + 1;
        const int u0 = 16 * (j0 >> 2) + 4 * gg + (j0 & 3);
        const int u1 = 16 * (j1 >> 2) + 4 * gg + (j1 & 3);
        const uint32_t mk =
            (tok0 + u0 < kv_len ? 0x0000FFFFu : 0u) | (tok0 + u1 < kv_len ? 0xFFFF0000u : 0u);
        vs[k] &= mk;
      }
    }
  }
  // ---- online softmax (base 2, lazy reference max) ------------------------
  half8_t pb[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float mx = s[0][nt][0];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[m][nt][i]);
    mx = wave_max_xor_16_32(mx);
    if (mx > st.m[nt] + RESCALE_MARGIN) {
      const float alpha = __builtin_amdgcn_exp2f(st.m[nt] - mx);
      st.l[nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt) st.o[nt][mt] *= alpha;
      st.m[nt] = mx;
    }
    const float mref = st.m[nt] == neg_inf() ? 0.0f : st.m[nt];
    float p[8];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * m + i] = __builtin_amdgcn_exp2f(s[m][nt][i] - mref);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sum += p[j];
    st.l[nt] += sum;
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[nt][j] = (_Float16)p[j];
  }
  // ---- O^T += Vhat^T . (P' * d_V)^T ----------------------------------------
  // Q4_0: four words per lane hold all 16 dim tiles; Q8_0: 16 bytes per
  // block b (two dim tiles), read one block ahead.
  u32x4 vw[4];
  if constexpr (V8) {
    vw[0] = *reinterpret_cast<const u32x4*>(slot + SLOT_V<KT> + lane * 16);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      vw[q] = *reinterpret_cast<const u32x4*>(slot + SLOT_V<KT> + q * 1024 + lane * 16);
  }
  // the value scales of block b are read one block ahead, as the operands above
  auto vscale = [&](int b) -> u32x4 {
    return *reinterpret_cast<const u32x4*>(slot + SLOT_VS<KT, V8> + (b * 4 + g) * 16);
  };
  u32x4 scn = vscale(0);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    u32x4 v8cur;
    if constexpr (V8) {
      v8cur = vw[0];
      if (b < 7) vw[0] = *reinterpret_cast<const u32x4*>(slot + SLOT_V<KT> + (b + 1) * 1024 + lane * 16);
    }
    const u32x4 sc = scn;
    if (b < 7) scn = vscale(b + 1);
    const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
    half8_t bb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2) {
        const half2_t pr = {pb[nt][2 * p2], pb[nt][2 * p2 + 1]};
        const half2_t r = pr * as_h2(scw[p2]);
        bb[nt][2 * p2] = r[0];
        bb[nt][2 * p2 + 1] = r[1];
      }
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2) {
      const int mt = 2 * b + e2;
      half8_t a;
      if constexpr (V8) {
        a = v8_codes_to_f16(e2 ? v8cur.z : v8cur.x, e2 ? v8cur.w : v8cur.y);
      } else {
        const u32x4 vq = vw[mt >> 2];
        const uint32_t w = (mt & 3) == 0 ? vq.x : (mt & 3) == 1 ? vq.y : (mt & 3) == 2 ? vq.z : vq.w;
        a = v_codes_to_f16_m(w, nib_lo, nib_hi);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) st.o[nt][mt] = mfma16(a, bb[nt], st.o[nt][mt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- fused append ------------------------------------------------------------
// The newest n_new tokens are quantised into the pools by the wavefront that
// streams the tile holding them, before it loads that tile (it waits for its
// own stores first), so no other wavefront or workgroup depends on them. One
// wavefront handles one slot at a time: lane (b, s) = (lane / 8, lane % 8)
// takes elements 4s..4s+3 of 32-dim block b, and the block's largest
// magnitude (keys) and lowest-index element of largest magnitude (values)
// are reduced over its eight lanes. The lane's value dims n0..n0+3
// (n0 = 32b + 4s) share (q, e) and take d = n0 % 16 .. +3, so each slot group
// g gives the lane four words to merge. Q8_0 values are plain bytes: the
// lane stores its four codes where the value record places them.
struct AppendTile {
  int64_t tok;        // first position of the tile (32-token group c of its page)
  int64_t rec;        // record index of the page and KV head
  int ub, ue;         // new slots [ub, ue) of the tile
  uint32_t newmask[4];  // per slot group g: bit j set when slot t(c, g, j) is new
  uint32_t old[4][4];   // words (g, i) whose other slots keep their codes
  float4 x[4], y[4];    // inputs of up to four slots in flight
};

__device__ __forceinline__ uint32_t slots_mask(uint32_t newmask) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (newmask & (1u << j)) m |= 0xFu << v_slot_bit(j);
  return m;
}

// Word index (within the V record) of the lane's dim n0 + i in slot group g.
__device__ __forceinline__ int append_word(int c, int g, int lane, int i) {
  const int b = lane >> 3, s = lane & 7;
  const int q = b >> 1, e = (2 * b + (s >> 2)) & 3, d = 4 * (s & 3) + i;
  return c * 1024 + (((q * 4 + g) * 16 + d) * 4 + e);
}

__device__ __forceinline__ void append_load(const DecodeParams& p, const AppendTile& a, int h,
                                            int64_t first_new, int u0, int lane, float4 (&x)[4],
                                            float4 (&y)[4]) {
  const int b = lane >> 3, s = lane & 7;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (u0 + k < a.ue) {  // uniform
      const int64_t row = ((a.tok + u0 + k - first_new) * p.n_kv + h) * D + 32 * b + 4 * s;
      x[k] = *reinterpret_cast<const float4*>(p.k_new + row);
      y[k] = *reinterpret_cast<const float4*>(p.v_new + row);
    }
  }
}

// Requests the first slots' inputs and the old words of partly new V words.
template <int KT, bool V8>
__device__ __forceinline__ void append_issue(const DecodeParams& p, AppendTile& a, int h, int c,
                                             int64_t first_new, int lane) {
  a.ub = (int)(first_new > a.tok ? first_new - a.tok : 0);
  a.ue = (int)(p.kv_len - a.tok < 32 ? p.kv_len - a.tok : 32);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u_lo = 4 * g + k, u_hi = 16 + 4 * g + k;  // slots j = k and j = 4 + k
      if (u_lo >= a.ub && u_lo < a.ue) m |= 1u << k;
      if (u_hi >= a.ub && u_hi < a.ue) m |= 1u << (4 + k);
    }
    a.newmask[g] = m;
  }
  append_load(p, a, h, first_new, a.ub, lane, a.x, a.y);
  if constexpr (V8) return;
  const uint32_t* vw = reinterpret_cast<const uint32_t*>(p.v_pool_w + a.rec * V_REC);
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a.old[g][i] = (a.newmask[g] != 0 && a.newmask[g] != 0xFFu) ? vw[append_word(c, g, lane, i)] : 0u;
}

// Quantises every new slot of the tile and writes codes, scales and words.
template <int KT, bool V8>
__device__ __forceinline__ void append_finish(const DecodeParams& p, AppendTile& a, int h, int c,
                                              int64_t first_new, int lane) {
  const int b = lane >> 3, s = lane & 7;
  uint8_t* krec = p.k_pool_w + a.rec * (KREC_OF<KT>);
  uint8_t* vrec = p.v_pool_w + a.rec * (V8 ? V8_REC : V_REC);
  uint32_t acc[4][4] = {};
  for (int u0 = a.ub; u0 < a.ue; u0 += 4) {
    if (u0 != a.ub) append_load(p, a, h, first_new, u0, lane, a.x, a.y);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = u0 + k;
      if (u >= a.ue) break;  // uniform
      const int t = c * 32 + u;
      const float xe[4] = {a.x[k].x, a.x[k].y, a.x[k].z, a.x[k].w};
      const float ye[4] = {a.y[k].x, a.y[k].y, a.y[k].z, a.y[k].w};
      if constexpr (KT == 2) {  // keys: Q5_1 from the block's extremes
        float mn = fminf(fminf(xe[0], xe[1]), fminf(xe[2], xe[3]));
        float mx = fmaxf(fmaxf(xe[0], xe[1]), fmaxf(xe[2], xe[3]));
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          mn = fminf(mn, peer8(mn, o));
          mx = fmaxf(mx, peer8(mx, o));
        }
        const _Float16 d16 = q5_scale(mx, mn), m16 = (_Float16)mn;
        const float dk = (float)d16, mk = (float)m16;
        const bool live = dk != 0.0f;
        const float inv = live ? 1.0f / dk : 0.0f;
        uint32_t part = 0u, hpart = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t code = live ? q5_code(xe[j], mk, inv) : 0u;
          const int k = 4 * (s & 1) + j;
          part |= (code & 0xFu) << v_slot_bit(k);
          hpart |= (code >> 4) << k5_hi_bit(k);
        }
        const uint32_t word = part | peer8(part, 1);
        const uint32_t hbyte = hpart | peer8(hpart, 1);
        const int wi = 4 * b + (s >> 1);
        if ((s & 1) == 0) {
          *reinterpret_cast<uint32_t*>(krec + t * (D / 2) + 4 * wi) = word;
          krec[K5_HI_OFF + t * 32 + wi] = (uint8_t)hbyte;
        }
        if (s == 0) {
          *reinterpret_cast<uint16_t*>(krec + K5_D_OFF + (t * 8 + b) * 2) =
              live ? __builtin_bit_cast(uint16_t, d16) : (uint16_t)0;
          *reinterpret_cast<uint16_t*>(krec + K5_M_OFF + (t * 8 + b) * 2) =
              __builtin_bit_cast(uint16_t, m16);
        }
      } else if constexpr (KT == 1) {  // keys: Q4_0, the value rule
        float ak = fabsf(xe[0]), mk = xe[0];
        int ik = 4 * s;
#pragma unroll
        for (int j = 1; j < 4; ++j)
          if (fabsf(xe[j]) > ak) {
            ak = fabsf(xe[j]);
            mk = xe[j];
            ik = 4 * s + j;
          }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) {
          const float ak2 = peer8(ak, o), mk2 = peer8(mk, o);
          const int ik2 = peer8(ik, o);
          if (ak2 > ak || (ak2 == ak && ik2 < ik)) {
            ak = ak2;
            mk = mk2;
            ik = ik2;
          }
        }
        const _Float16 dk16 = q4_scale(mk);
        const float dk = (float)dk16;
        const bool live = ak != 0.0f && dk != 0.0f;
        const float inv = live ? 1.0f / dk : 0.0f;
        // dims 32b + 4s + j are dims 4(s%2) + j of word 4b + s/2; lane pairs share a word
        uint32_t part = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          part |= (live ? q4_code(xe[j], inv) : 8u) << v_slot_bit(4 * (s & 1) + j);
        const uint32_t word = part | peer8(part, 1);
        if ((s & 1) == 0)
          *reinterpret_cast<uint32_t*>(krec + t * (D / 2) + 4 * (4 * b + (s >> 1))) = word;
        if (s == 0)
          *reinterpret_cast<uint16_t*>(krec + K4_SCALE_OFF + (t * 8 + b) * 2) =
              live ? __builtin_bit_cast(uint16_t, dk16) : (uint16_t)0;
      } else {
      // keys: Q8_0
      float amax = fmaxf(fmaxf(fabsf(xe[0]), fabsf(xe[1])), fmaxf(fabsf(xe[2]), fabsf(xe[3])));
      amax = fmaxf(amax, peer8(amax, 1));
      amax = fmaxf(amax, peer8(amax, 2));
      amax = fmaxf(amax, peer8(amax, 4));
      const _Float16 d16 = q8_scale(amax);
      const float d = (float)d16;
      uint32_t kw = 0u;
      if (d != 0.0f) {
        const float inv = 1.0f / d;
#pragma unroll
        for (int j = 0; j < 4; ++j) kw |= q8_code(xe[j], inv) << (8 * j);
      }
      *reinterpret_cast<uint32_t*>(krec + t * D + 32 * b + 4 * s) = kw;
      if (s == 0)
        *reinterpret_cast<uint16_t*>(krec + K_SCALE_OFF + (t * 8 + b) * 2) =
            d != 0.0f ? __builtin_bit_cast(uint16_t, d16) : (uint16_t)0;
      }
      if constexpr (V8) {  // values: Q8_0, the key rule
        float vmax = fmaxf(fmaxf(fabsf(ye[0]), fabsf(ye[1])), fmaxf(fabsf(ye[2]), fabsf(ye[3])));
        vmax = fmaxf(vmax, peer8(vmax, 1));
        vmax = fmaxf(vmax, peer8(vmax, 2));
        vmax = fmaxf(vmax, peer8(vmax, 4));
        const _Float16 dq16 = q8_scale(vmax);
        const float dq = (float)dq16;
        const float inv = dq != 0.0f ? 1.0f / dq : 0.0f;
        const int g = (u & 15) >> 2, j = 4 * (u >> 4) + (u & 3);
        // dim 32b + 4s + i sits in half s/4, row 4(s%4) + i of block b's piece
        uint8_t* dst = vrec + c * 8192 + b * 1024 + (16 * g + 4 * (s & 3)) * 16 + 8 * (s >> 2) + j;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[16 * i] = dq != 0.0f ? (uint8_t)q8_code(ye[i], inv) : (uint8_t)0;
        if (s == 0)
          *reinterpret_cast<uint16_t*>(vrec + K_SCALE_OFF + 2 * (((c * 8 + b) * 4 + g) * 8 + j)) =
              dq != 0.0f ? __builtin_bit_cast(uint16_t, dq16) : (uint16_t)0;
        continue;
      }
      // values: Q4_0, the lowest-index element of largest magnitude sets the scale
      float am = fabsf(ye[0]), m = ye[0];
      int idx = 4 * s;
#pragma unroll
      for (int j = 1; j < 4; ++j)
        if (fabsf(ye[j]) > am) {
          am = fabsf(ye[j]);
          m = ye[j];
          idx = 4 * s + j;
        }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        const float am2 = peer8(am, o), m2 = peer8(m, o);
        const int idx2 = peer8(idx, o);
        if (am2 > am || (am2 == am && idx2 < idx)) {
          am = am2;
          m = m2;
          idx = idx2;
        }
      }
      const _Float16 dv16 = q4_scale(m);
      const float dv = (float)dv16;
      uint32_t code[4] = {8u, 8u, 8u, 8u};
      uint16_t bits4 = 0;
      if (am != 0.0f && dv != 0.0f) {
        const float inv = 1.0f / dv;
#pragma unroll
        for (int j = 0; j < 4; ++j) code[j] = q4_code(ye[j], inv);
        bits4 = __builtin_bit_cast(uint16_t, dv16);
      }
      const int g = (u & 15) >> 2, j = 4 * (u >> 4) + (u & 3);
      if (s == 0)
        *reinterpret_cast<uint16_t*>(vrec + V_SCALE_OFF + 2 * (((c * 8 + b) * 4 + g) * 8 + j)) = bits4;
      const int bit = v_slot_bit(j);
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
        if (gg == g)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[gg][i] |= code[i] << bit;
    }
  }
  if constexpr (V8) return;
  uint32_t* vw = reinterpret_cast<uint32_t*>(vrec);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (a.newmask[g] == 0) continue;  // uniform
    const uint32_t keep = a.newmask[g] == 0xFFu ? 0u : ~slots_mask(a.newmask[g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[append_word(c, g, lane, i)] = (a.old[g][i] & keep) | acc[g][i];
  }
}

// ---- summary of the page an append completes ---------------------------------
// summary[n] = RN32((binary64 sum over slots t = 0..127, ascending, of the
// dequantised key K[t][n]) / 128), as quantize.hip's summarize_kernel. Every
// dequantised key is a multiple of 2^-24 (a binary16 scale times an integer
// code, plus a binary16 minimum for Q5_1). While the terms' magnitudes add up
// to less than 2^29, every partial sum, in any order, is a multiple of 2^-24
// below 2^29 and so exact in binary64: the ascending sum equals a sum in any
// order, here fused multiply-adds of code and scale. Q4_0 keys (|K| <= 8 x
// 65504) and Q5_1 keys (|d c| + |m| <= 32 x 65504) always stay below that
// bound over 128 slots; for Q8_0 keys the bound 127 x (sum of the 128 scales'
// magnitudes) is checked per 32-dim block, and where it is reached (scales
// near the binary16 limit) the ascending sum is run as written. The workgroup
// whose units hold the page computes it once its own appended bytes are in
// place: thread (tg = tid / 64, lane) sums dims 4 lane .. +3 over slots tg,
// tg + 8, ..., tg + 120.

// The ascending binary64 sum for dim n of a Q8_0 key record.
__device__ __noinline__ float summary_sequential_q8(const uint8_t* krec, int n) {
  double acc = 0.0;
  for (int t = 0; t < PAGE; ++t) {
    const float d = f16_value(reinterpret_cast<const uint16_t*>(krec + KSCALE_OF<0>)[t * 8 + n / 32]);
    const float kh = d * (float)(int8_t)krec[t * D + n];  // exact in binary32
    acc = acc + (double)kh;
  }
  return (float)(acc / 128.0);
}

// The page's key codes and scales this thread sums, in registers.
struct SummaryLoads {
  uint32_t w[16], sc[16], hi[16], mm[16];
};

template <int KT>
__device__ __forceinline__ void summary_issue(const uint8_t* krec, SummaryLoads& L) {
  const int lane = threadIdx.x & 63, tg = threadIdx.x >> 6;
  const int n4 = 4 * lane;
#pragma unroll
  for (int j = 0; j < 16; ++j) {  // every load in flight at once
    const int t = tg + 8 * j;
    const int sidx = t * 8 + n4 / 32;
    L.sc[j] = reinterpret_cast<const uint16_t*>(krec + KSCALE_OF<KT>)[sidx];
    if constexpr (KT == 0) {
      L.w[j] = *reinterpret_cast<const uint32_t*>(krec + t * D + n4);
    } else {
      L.w[j] = reinterpret_cast<const uint32_t*>(krec)[t * 32 + n4 / 8];
    }
    if constexpr (KT == 2) {
      L.hi[j] = krec[K5_HI_OFF + t * 32 + n4 / 8];
      L.mm[j] = reinterpret_cast<const uint16_t*>(krec + K5_M_OFF)[sidx];
    }
  }
}

template <int KT, int THREADS>
__device__ __forceinline__ void summary_finish(const uint8_t* krec, const SummaryLoads& L,
                                               float* out, uint8_t* lds) {
  static_assert(THREADS == 512, "eight slot groups of 64 lanes");
  const int tid = threadIdx.x, lane = tid & 63, tg = tid >> 6;
  const int n4 = 4 * lane;
  double S[4] = {0.0, 0.0, 0.0, 0.0};
  double B = 0.0;  // sum of |d| over this thread's slots (Q8_0 keys)
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double d = (double)f16_value(L.sc[j]);
    if constexpr (KT == 0) B += __builtin_fabs(d);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (KT == 0) {
        S[e] = __builtin_fma((double)(int)(int8_t)(L.w[j] >> (8 * e)), d, S[e]);
      } else {
        const int k = (n4 & 7) + e;  // dim 8w + k of the word
        const int code = (int)((L.w[j] >> v_slot_bit(k)) & 0xFu);
        if constexpr (KT == 1) {
          S[e] = __builtin_fma((double)(code - 8), d, S[e]);
        } else {
          const int c5 = code | (int)(((L.hi[j] >> k5_hi_bit(k)) & 1u) << 4);
          S[e] = __builtin_fma((double)c5, d, S[e]) + (double)f16_value(L.mm[j]);
        }
      }
    }
  }
  double* Ssh = reinterpret_cast<double*>(lds);
  double* Bsh = Ssh + 8 * D;
#pragma unroll
  for (int e = 0; e < 4; ++e) Ssh[tg * D + n4 + e] = S[e];
  if constexpr (KT == 0) Bsh[tg * 64 + lane] = B;
  __syncthreads();
  if (tid < D) {
    double s = 0.0, b = 0.0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      s += Ssh[g * D + tid];
      if constexpr (KT == 0) b += Bsh[g * 64 + tid / 4];
    }
    const float exact = (float)(s * 0x1p-7);
    if constexpr (KT == 0) {
      out[tid] = 127.0 * b < 0x1p29 ? exact : summary_sequential_q8(krec, tid);
    } else {
      out[tid] = exact;
    }
  }
}

// WAVES: wavefronts per workgroup (4 or 8); either way two wavefronts share
// a SIMD (two 4-wave workgroups or one 8-wave workgroup per CU), so every
// lane may hold up to 256 VGPRs. With 8 waves, waves 4-7 stream the first
// SLOW_SHARE/32 of the split's units and waves 0-3 the rest. V8: Q8_0 values.
template <int NT, int WAVES, int KT, bool V8>
__global__ __launch_bounds__(64 * WAVES, 2) void decode_kernel(DecodeParams p) {
  constexpr int THREADS = 64 * WAVES;
  constexpr int NH = WAVES / 4;  // halves of the workgroup streaming a split
  // LDS: [q' rows | one tile slot per wave] during the loop, then the
  // combine buffer [WAVES][16 rows][260] floats.
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_raw[];
  float* smem = reinterpret_cast<float*>(smem_raw);
  __shared__ float s_m[WAVES][32], s_l[WAVES][32];
  __shared__ int s_rowg[32];
  const int h = blockIdx.y, split = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, g = lane >> 4;
  const int R = p.n_q_tok * p.gqa;
  const int n_heads = p.n_kv * p.gqa;
  constexpr int Q_BYTES = ((NT * 16 * Q_LDS_STRIDE * 2) + 1023) / 1024 * 1024;
  constexpr int VREC = V8 ? V8_REC : V_REC;
  constexpr int KREC = KREC_OF<KT>;
  uint8_t* slots = smem_raw + Q_BYTES + wave * SLOT_BYTES<KT, V8>;

  _Float16* q_lds = reinterpret_cast<_Float16*>(smem_raw);
  State<NT> st;
  st.q_lds = q_lds;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + r16;
    // padding rows see every key (harmless, never written out)
    st.limit[nt] = r < R ? p.kv_len - p.n_q_tok + r / p.gqa : p.kv_len - 1;
    st.m[nt] = neg_inf();
    st.l[nt] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 16; ++mt) st.o[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const int64_t min_limit = p.kv_len - p.n_q_tok;
  // the nibble masks are kept in VGPRs so each pair unpacks with one
  // v_and_or_b32 (its exponent bits from an SGPR)
  uint32_t nib_lo, nib_hi;
  __asm__ volatile("v_mov_b32 %0, 0x000f000f" : "=v"(nib_lo));
  __asm__ volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(nib_hi));

  const int64_t u0 = (int64_t)p.n_units * split / p.n_splits;
  const int64_t u1 = (int64_t)p.n_units * (split + 1) / p.n_splits;
  // With two halves, waves 4-7 take the split's first SLOW_SHARE/32 units and
  // waves 0-3 the rest: the SIMDs favour the older waves 0-3, which get
  // through their tiles faster while both run, so they take the larger share
  // and both halves finish together (measured best at 12/32: about 5% off
  // the layer against an even split). Waves 0-3 also take the split's last
  // unit, the page that an append writes.
  const int n_all = (int)(u1 - u0);
  const int n_slow = NH == 1 ? 0 : (n_all * SLOW_SHARE + 16) / 32;
  const bool slow_half = NH != 1 && (wave >> 2) != 0;
  const int64_t ubase = slow_half ? u0 : u0 + n_slow;  // this wave's units: [ubase, uend)
  const int64_t uend = slow_half ? u0 + n_slow : u1;
  const int n_tiles = (int)(uend - ubase);
  const int c = wave & 3;  // 32-token group of every page handled by this wave

  // Page lookups for 64 upcoming units at a time, one per lane, read back
  // with readlane so every address is wavefront-uniform. Invalid tiles still
  // issue their 13 loads (from record 0) so the wait counts stay constant.
  int lp_vec = -1, ph_vec = -1;
  auto refill = [&](int i0) {
    const int64_t u = ubase + (int64_t)(i0 + lane);
    int lp = -1, ph = -1;
    if (u < uend) {
      lp = p.blocks ? p.blocks[(int64_t)h * p.n_blk + u] : (int)u;
      if (lp >= 0 && lp < p.n_logical && (int64_t)lp * PAGE + c * 32 < p.kv_len) {
        ph = p.page_table[lp];
        if (ph < 0 || ph >= p.n_phys) ph = -1;
      }
    }
    lp_vec = lp;
    ph_vec = ph;
  };
  // Tile i's record; invalid tiles (skipped pages, tokens past kv_len) still
  // load from record 0 so every wait count below is a constant.
  int sum_ph = -1;  // physical page of the page to summarise, once this wave streams it
  auto locate = [&](int i, int64_t& tok, bool& valid, int64_t& rec) {
    if (i % 64 == 0) refill(i);
    const int lp = __builtin_amdgcn_readlane(lp_vec, i % 64);
    const int ph = __builtin_amdgcn_readlane(ph_vec, i % 64);
    valid = ph >= 0;
    tok = (int64_t)lp * PAGE + c * 32;
    rec = valid ? (int64_t)ph * p.n_kv + h : 0;
    if (valid && lp == p.sum_page) sum_ph = ph;
  };

  // One LDS slot per wave with separately refilled key and value halves:
  // keys of tile i+1 load while tile i's softmax and PV run, values of tile
  // i+1 load while tile i+1's QK runs.
  uint8_t* slot = slots;
  int64_t tok = 0, rec = 0, tok_n = 0, rec_n = 0;
  bool valid = false, valid_n = false;
  // Fused append: the one tile of this wave that holds new tokens, if any
  // (n_new <= 32, and a wave keeps one 32-token group c of every page). Its
  // inputs and old words are requested before the first tile's loads; the
  // codes are computed and stored after the q' staging, while the first
  // tile's loads fly. The loop's first iteration then waits with vmcnt(0)
  // (app_pending, i == 0), which covers those stores, so every later tile
  // load of this wave sees them. When the first tile is the appended one, it
  // is loaded only after the stores complete. Within a launch only this wave
  // reads the appended tile, except when a sparse list repeats its page: then
  // another wave or workgroup may read the tile while it is being written,
  // which is harmless only because every writer of those bytes stores the
  // same values (each wave whose list holds the page quantises the same
  // tokens); the header states this.
  const int64_t first_new = p.kv_len - p.n_new;
  bool app = false, app_pending = false;
  AppendTile at;
  if (n_tiles > 0) {
    locate(0, tok, valid, rec);
    if (p.n_new > 0) {
      int i0 = 0;
      for (; i0 < n_tiles; i0 += 64) {
        if (i0 > 0) refill(i0);
        const bool hit = ph_vec >= 0 && (int64_t)lp_vec * PAGE + c * 32 + 32 > first_new;
        const uint64_t m = __ballot(hit);
        if (m) {
          const int l = (int)__builtin_ctzll(m);
          at.tok = (int64_t)__builtin_amdgcn_readlane(lp_vec, l) * PAGE + c * 32;
          at.rec = (int64_t)__builtin_amdgcn_readlane(ph_vec, l) * p.n_kv + h;
          app = true;
          break;
        }
      }
      if (n_tiles > 64 && i0 > 0) refill(0);  // the loop starts from the first 64 units
      if (app) append_issue<KT, V8>(p, at, h, c, first_new, lane);
    }
    const bool first_new_tile = app && valid && tok + 32 > first_new;
    if (!first_new_tile) {
      issue_keys<KT>(slot, p.k_pool + rec * KREC, valid ? c : 0);
      issue_values<KT, V8>(slot, p.v_pool + rec * VREC, valid ? c : 0);
    }
    if (first_new_tile) {
      append_finish<KT, V8>(p, at, h, c, first_new, lane);
      wait_loads<0>();  // this wave's stores have completed
      issue_keys<KT>(slot, p.k_pool + rec * KREC, c);
      issue_values<KT, V8>(slot, p.v_pool + rec * VREC, c);
    }
    app_pending = app && !first_new_tile;
  }
  // The first tile is in flight: stage q' rows (f16) into LDS, shared by all
  // waves (padding rows are zero). Row r of this KV head is query token
  // r / gqa, query head h*gqa + r % gqa; its global row goes to s_rowg.
  __shared__ int s_sum_ph;  // 1 + physical page to summarise (0: none here)
  if (threadIdx.x == 0) s_sum_ph = 0;
  if (threadIdx.x < NT * 16) {
    const int r = threadIdx.x;
    const int tq = r / p.gqa, gi = r - tq * p.gqa;
    s_rowg[r] = r < R ? tq * n_heads + h * p.gqa + gi : -1;
  }
  __syncthreads();
  {
    constexpr int PER = NT * 16 * (D / 4) / THREADS;  // float4s per thread
    float4 qv[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = threadIdx.x + THREADS * k;
      const int r = idx >> 6, d4 = idx & 63;
      const int rowg = s_rowg[r];
      qv[k] = rowg >= 0 ? reinterpret_cast<const float4*>(p.q + (int64_t)rowg * D)[d4]
                        : float4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int idx = threadIdx.x + THREADS * k;
      const int r = idx >> 6, d4 = idx & 63;
      const half2_t lo = {(_Float16)(qv[k].x * p.qscale), (_Float16)(qv[k].y * p.qscale)};
      const half2_t hi = {(_Float16)(qv[k].z * p.qscale), (_Float16)(qv[k].w * p.qscale)};
      *reinterpret_cast<uint2*>(q_lds + r * Q_LDS_STRIDE + 4 * d4) = uint2{as_u32(lo), as_u32(hi)};
    }
  }
  __syncthreads();
  if (app_pending) append_finish<KT, V8>(p, at, h, c, first_new, lane);
  for (int i = 0; i < n_tiles; ++i) {
    const bool more = i + 1 < n_tiles;
    if (more) locate(i + 1, tok_n, valid_n, rec_n);
    if (app_pending && i == 0) {
      wait_loads<0>();  // the appended tokens' stores (and all of tile 0) have completed
    } else {
      wait_loads<V_LOADS<V8>>();  // keys of tile i have landed (its values may still fly)
    }
    auto refill_keys = [&] {
      if (more) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): key reads of this slot are done
        issue_keys<KT>(slot, p.k_pool + rec_n * KREC, valid_n ? c : 0);
        wait_loads<K_LOADS<KT>>();  // values of tile i have landed
      } else {
        wait_loads<0>();
      }
    };
    if (valid) {
      compute_tile<NT, KT, V8>(st, slot, tok, p.kv_len, min_limit, lane, r16, g, nib_lo, nib_hi,
                               refill_keys);
    } else {
      refill_keys();
    }
    if (more) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): value reads of this slot are done
      issue_values<KT, V8>(slot, p.v_pool + rec_n * VREC, valid_n ? c : 0);
    }
    tok = tok_n;
    rec = rec_n;
    valid = valid_n;
  }

  // ---- combine the wavefronts, write this split's partial --------------------
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) st.l[nt] = wave_sum_xor_16_32(st.l[nt]);
  // The page the append completes is summarised by the workgroup whose units
  // hold it: a unit is a whole page, whose four 32-token groups are streamed
  // by four waves of one workgroup (group c by a wave with wave % 4 == c),
  // including the wave that wrote the page's new tokens. The waves of a
  // workgroup share one vector L1; the explicit wait (vmcnt, expcnt and
  // lgkmcnt all zero) has that wave's stores complete
  // before the barrier, so the summary's reads, issued after it and in
  // flight while the partial is combined, see them.
  if (p.sum_page >= 0) {
    if (sum_ph >= 0) s_sum_ph = sum_ph + 1;
    __builtin_amdgcn_s_waitcnt(0);
  }
  if (g == 0) {  // each wave's row maxima and sums, for the weights below
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      s_m[wave][nt * 16 + r16] = st.m[nt];
      s_l[wave][nt * 16 + r16] = st.l[nt];
    }
  }
  __syncthreads();  // every wave is done with the LDS ring and q_lds
  const int sum_ph1 = p.sum_page >= 0 ? s_sum_ph : 0;  // uniform
  const uint8_t* sum_rec = p.k_pool + ((int64_t)(sum_ph1 - 1) * p.n_kv + h) * KREC;
  SummaryLoads sl;
  if (sum_ph1 != 0) summary_issue<KT>(sum_rec, sl);
  constexpr int RS = 260;  // padded row stride of the combine buffer
  const int64_t rows_total = (int64_t)p.n_q_tok * n_heads;
  // Wave w's weight for row r, exp2(m_w - M) / L, and the row's lse, from
  // eight consecutive lanes per row (lane w of the eight holds wave w's max
  // and sum; the butterflies give every lane of the group the same M and L).
  // The lse is written here, while the waves dump their rows below.
  static_assert(WAVES == 8, "one row per eight lanes");
  __shared__ float s_f[WAVES][32];
  if (threadIdx.x < WAVES * NT * 16) {
    const int row = threadIdx.x >> 3, w = threadIdx.x & 7;
    const float mw = s_m[w][row];
    const float M = group8_max(mw);
    const float e = mw != neg_inf() ? __builtin_amdgcn_exp2f(mw - M) : 0.f;
    const float L = group8_sum(s_l[w][row] * e);
    s_f[w][row] = L > 0.f ? e / L : 0.f;
    if (w == 0 && row < R)
      p.lse_part[(int64_t)split * rows_total + s_rowg[row]] =
          L > 0.f ? (M + __log2f(L)) * LN2 : neg_inf();
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // every wave dumps its unnormalised rows (padding rows are never read);
    // the threads that add them up apply the weights
    if (s_rowg[nt * 16 + r16] >= 0) {
      float* buf = smem + (size_t)wave * 16 * RS;
#pragma unroll
      for (int mt = 0; mt < 16; ++mt)
        *reinterpret_cast<floatx4*>(buf + r16 * RS + 16 * mt + 4 * g) = st.o[nt][mt];
    }
    __syncthreads();
    // 16 rows x 64 float4 columns: the waves' weighted rows, added pairwise
    // in a fixed order (products rounded before the sums)
#pragma unroll
    for (int k = 0; k < 16 * 64 / THREADS; ++k) {
#pragma clang fp contract(off)
      const int idx = threadIdx.x + THREADS * k;
      const int rr = idx >> 6, c4 = idx & 63;
      const int rowg = s_rowg[nt * 16 + rr];
      if (rowg >= 0) {
        floatx4 v[WAVES];
#pragma unroll
        for (int w = 0; w < WAVES; ++w)
          v[w] = *reinterpret_cast<const floatx4*>(smem + (w * 16 + rr) * RS + 4 * c4) *
                 s_f[w][nt * 16 + rr];
#pragma unroll
        for (int step = 1; step < WAVES; step *= 2)
#pragma unroll
          for (int w = 0; w < WAVES; w += 2 * step) v[w] = v[w] + v[w + step];
        reinterpret_cast<floatx4*>(p.o_part + ((int64_t)split * rows_total + rowg) * D)[c4] = v[0];
      }
    }
    // the next round's dump, or the summary's partial sums, reuse the buffer
    if (nt + 1 < NT || sum_ph1 != 0) __syncthreads();
  }
  if (sum_ph1 != 0)  // the combine buffer is free after the partial's last barrier
    summary_finish<KT, THREADS>(sum_rec, sl, p.k_summary + ((int64_t)h * p.n_logical + p.sum_page) * D,
                                smem_raw);
}

template <int NT, int KT, bool V8>
hipError_t launch_nt(const DecodeParams& p, hipStream_t stream) {
  const size_t combine = sizeof(float) * DECODE_WAVES * 16 * 260;
  static_assert(sizeof(float) * DECODE_WAVES * 16 * 260 >= (8 * D + 8 * 64) * sizeof(double),
                "the page summary's partial sums fit the combine area");
  const size_t qbytes = ((NT * 16 * Q_LDS_STRIDE * 2) + 1023) / 1024 * 1024;
  const size_t loop = qbytes + DECODE_WAVES * SLOT_BYTES<KT, V8>;
  const size_t shmem = combine > loop ? combine : loop;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit(
      lds_set, reinterpret_cast<const void*>(&decode_kernel<NT, DECODE_WAVES, KT, V8>), shmem);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)p.n_splits, (unsigned)p.n_kv);
  hipLaunchKernelGGL((decode_kernel<NT, DECODE_WAVES, KT, V8>), grid, dim3(64 * DECODE_WAVES), shmem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  const int R = p.n_q_tok * p.gqa;
  if (p.k_type == 2) {
    if (p.v_q8) return R <= 16 ? launch_nt<1, 2, true>(p, stream) : launch_nt<2, 2, true>(p, stream);
    return R <= 16 ? launch_nt<1, 2, false>(p, stream) : launch_nt<2, 2, false>(p, stream);
  }
  if (p.k_type == 1) {
    if (p.v_q8) return R <= 16 ? launch_nt<1, 1, true>(p, stream) : launch_nt<2, 1, true>(p, stream);
    return R <= 16 ? launch_nt<1, 1, false>(p, stream) : launch_nt<2, 1, false>(p, stream);
  }
  if (p.v_q8) return R <= 16 ? launch_nt<1, 0, true>(p, stream) : launch_nt<2, 0, true>(p, stream);
  return R <= 16 ? launch_nt<1, 0, false>(p, stream) : launch_nt<2, 0, false>(p, stream);
}

}  // namespace kvattn
