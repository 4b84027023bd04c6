// a1: Q8_0 key / Q4_0 value quantisation into 128-token pages, and block
// summaries (mean dequantised key) of completed pages.
//
// Cache types from the Adaptive KV Streaming guide (alphalab.site, step ④:
// -ctk q8_0 -ctv q4_0) and the KVMem report (lcz.me topic 1972, 測試口徑:
// 128-token blocks); rounding chain and page layout as defined in
// include/kvattn.h. Every rounding step is an IEEE binary32 operation or a
// binary32 -> binary16 conversion, both round-to-nearest-even, so the bytes
// are reproducible bit for bit; nothing here may be contracted or reordered.
#include "common.hpp"
#include "launch.hpp"
#include "qround.hpp"

#pragma clang fp contract(off)

namespace kvattn {
namespace {

// One workgroup per (32-token group, KV head); thread (u, b) = (tid/8, tid%8)
// quantises the 32-dim block b of token slot u, so all tokens of the group
// are processed at once and each block's reductions stay in one thread.
// Value codes go through LDS to be packed into the group's V words (Q4_0) or
// reordered into the group's 16-byte lane pieces (Q8_0, V8 true).
template <bool V8, int KT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ k,
                                                       const float* __restrict__ v, int64_t pos0,
                                                       int32_t n_tok, int32_t n_kv,
                                                       const int32_t* __restrict__ page_table,
                                                       int32_t n_phys, uint8_t* __restrict__ k_pool,
                                                       uint8_t* __restrict__ v_pool) {
  __shared__ uint8_t vcodes[32][D];
  __shared__ uint16_t vscales[32][8];

  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t grp = pos0 / 32 + blockIdx.x;  // global 32-token group
  const int64_t gpos = grp * 32;
  const int64_t lp = gpos / PAGE;
  const int c = (int)((gpos % PAGE) / 32);
  const int32_t phys = page_table[lp];
  if (phys < 0 || phys >= n_phys) return;  // uniform across the workgroup
  uint8_t* krec = k_pool + ((int64_t)phys * n_kv + h) * (KREC_OF<KT>);
  uint8_t* vrec = v_pool + ((int64_t)phys * n_kv + h) * (V8 ? V8_REC : V_REC);
  uint32_t* vwords = reinterpret_cast<uint32_t*>(vrec) + c * 1024;
  const int64_t end = pos0 + n_tok;
  const bool whole = gpos >= pos0 && gpos + 32 <= end;  // uniform
  uint32_t old[4] = {0u, 0u, 0u, 0u};
  if (!V8 && !whole) {
#pragma unroll
    for (int q = 0; q < 4; ++q) old[q] = vwords[tid + 256 * q];
  }

  const int u = tid >> 3, b = tid & 7;
  const int64_t pos = gpos + u;
  const int t = c * 32 + u;  // slot in the page
  if (pos >= pos0 && pos < end) {
    const int64_t row = ((pos - pos0) * n_kv + h) * D + 32 * b;
    float x[32], y[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 a = reinterpret_cast<const float4*>(k + row)[i];
      const float4 e = reinterpret_cast<const float4*>(v + row)[i];
      x[4 * i] = a.x; x[4 * i + 1] = a.y; x[4 * i + 2] = a.z; x[4 * i + 3] = a.w;
      y[4 * i] = e.x; y[4 * i + 1] = e.y; y[4 * i + 2] = e.z; y[4 * i + 3] = e.w;
    }
    if constexpr (KT == 2) {  // Q5_1 keys: word i of the block holds the low bits of dims 8i..8i+7
      float mn = x[0], mx = x[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) {
        mn = fminf(mn, x[i]);
        mx = fmaxf(mx, x[i]);
      }
      const _Float16 dk16 = q5_scale(mx, mn), mk16 = (_Float16)mn;
      const float dk = (float)dk16, mk = (float)mk16;
      const bool live = dk != 0.0f;
      const float inv = live ? 1.0f / dk : 0.0f;
      uint32_t kw[4], hb = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t wv = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t code = live ? q5_code(x[8 * i + j], mk, inv) : 0u;
          wv |= (code & 0xFu) << v_slot_bit(j);
          hb |= (code >> 4) << (8 * i + k5_hi_bit(j));
        }
        kw[i] = wv;
      }
      *reinterpret_cast<uint4*>(krec + t * (D / 2) + 16 * b) = uint4{kw[0], kw[1], kw[2], kw[3]};
      *reinterpret_cast<uint32_t*>(krec + K5_HI_OFF + t * 32 + 4 * b) = hb;
      *reinterpret_cast<uint16_t*>(krec + K5_D_OFF + (t * 8 + b) * 2) =
          live ? __builtin_bit_cast(uint16_t, dk16) : (uint16_t)0;
      *reinterpret_cast<uint16_t*>(krec + K5_M_OFF + (t * 8 + b) * 2) = __builtin_bit_cast(uint16_t, mk16);
    } else if constexpr (KT == 1) {  // Q4_0 keys: the value rule; word i of the block holds dims 8i..8i+7
      float a = fabsf(x[0]), m = x[0];
#pragma unroll
      for (int i = 1; i < 32; ++i)
        if (fabsf(x[i]) > a) {
          a = fabsf(x[i]);
          m = x[i];
        }
      const _Float16 dk16 = q4_scale(m);
      const float dk = (float)dk16;
      const bool live = a != 0.0f && dk != 0.0f;
      const float inv = live ? 1.0f / dk : 0.0f;
      uint32_t kw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t wv = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) wv |= (live ? q4_code(x[8 * i + j], inv) : 8u) << v_slot_bit(j);
        kw[i] = wv;
      }
      *reinterpret_cast<uint4*>(krec + t * (D / 2) + 16 * b) = uint4{kw[0], kw[1], kw[2], kw[3]};
      *reinterpret_cast<uint16_t*>(krec + K4_SCALE_OFF + (t * 8 + b) * 2) =
          live ? __builtin_bit_cast(uint16_t, dk16) : (uint16_t)0;
    } else {
    // Q8_0: d = RN16(RN32(amax / 127)); codes with inv = RN32(1 / d).
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const _Float16 d16 = q8_scale(amax);
    const float d = (float)d16;
    uint32_t kw[8];
    if (d != 0.0f) {
      const float inv = 1.0f / d;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t wv = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) wv |= q8_code(x[4 * i + j], inv) << (8 * j);
        kw[i] = wv;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kw[i] = 0u;
    }
    uint4* kdst = reinterpret_cast<uint4*>(krec + t * D + 32 * b);
    kdst[0] = uint4{kw[0], kw[1], kw[2], kw[3]};
    kdst[1] = uint4{kw[4], kw[5], kw[6], kw[7]};
    *reinterpret_cast<uint16_t*>(krec + K_SCALE_OFF + (t * 8 + b) * 2) =
        d != 0.0f ? __builtin_bit_cast(uint16_t, d16) : (uint16_t)0;
    }

    if constexpr (V8) {  // Q8_0 values: the key rule
      float vmax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) vmax = fmaxf(vmax, fabsf(y[i]));
      const _Float16 dq16 = q8_scale(vmax);
      const float dq = (float)dq16;
      const float inv = dq != 0.0f ? 1.0f / dq : 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i)
        vcodes[u][32 * b + i] = dq != 0.0f ? (uint8_t)q8_code(y[i], inv) : (uint8_t)0;
      vscales[u][b] = dq != 0.0f ? __builtin_bit_cast(uint16_t, dq16) : (uint16_t)0;
    } else {
      // Q4_0: the lowest-index element of largest magnitude, signed, maps to -8.
      float a = fabsf(y[0]), m = y[0];
#pragma unroll
      for (int i = 1; i < 32; ++i)
        if (fabsf(y[i]) > a) {
          a = fabsf(y[i]);
          m = y[i];
        }
      uint16_t bits4 = 0;
      const _Float16 dv16 = q4_scale(m);
      const float dv = (float)dv16;
      if (a != 0.0f && dv != 0.0f) {
        const float inv = 1.0f / dv;
#pragma unroll
        for (int i = 0; i < 32; ++i) vcodes[u][32 * b + i] = (uint8_t)q4_code(y[i], inv);
        bits4 = __builtin_bit_cast(uint16_t, dv16);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) vcodes[u][32 * b + i] = 8;
      }
      vscales[u][b] = bits4;
    }
  }
  __syncthreads();

  if constexpr (V8) {
    // 16-byte piece i of the group (512 of them): bytes (half, j) hold dim
    // 32q + 16*half + r of slots 16*(j/4) + 4g + j%4; unwritten slots keep their bytes.
    uint8_t* vbytes = vrec + c * 8192;
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int i = tid + 256 * qq;
      const int r = i & 15, g = (i >> 4) & 3, q = i >> 6;
      uint32_t w[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        uint32_t wv = 0;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int half = x >> 1, j = 4 * (x & 1) + y;
          const int uu = 16 * (j >> 2) + 4 * g + (j & 3);
          wv |= (uint32_t)vcodes[uu][32 * q + 16 * half + r] << (8 * y);
        }
        w[x] = wv;
      }
      if (whole) {
        reinterpret_cast<uint4*>(vbytes)[i] = uint4{w[0], w[1], w[2], w[3]};
      } else {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int j = x & 7;
          const int64_t p = gpos + 16 * (j >> 2) + 4 * g + (j & 3);
          if (p >= pos0 && p < end) vbytes[16 * i + x] = (uint8_t)(w[x >> 2] >> (8 * (x & 3)));
        }
      }
    }
    {
      const int i = tid;
      const int j = i & 7, g = (i >> 3) & 3, bb = i >> 5;
      const int uu = 16 * (j >> 2) + 4 * g + (j & 3);
      const int64_t p = gpos + uu;
      if (p >= pos0 && p < end)
        reinterpret_cast<uint16_t*>(vrec + K_SCALE_OFF)[c * 256 + i] = vscales[uu][bb];
    }
    return;
  }

  // V words of this 32-slot group: word (q, g, d, e) holds dim 16*(4q+e)+d for
  // slots 16*(j/4) + 4g + j%4; slots outside the written range keep their bits.
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) {
    const int i = tid + 256 * qq;
    const int e = i & 3, d = (i >> 2) & 15, g = (i >> 6) & 3, q = i >> 8;
    const int dim = 16 * (4 * q + e) + d;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int uu = 16 * (j >> 2) + 4 * g + (j & 3);
      const int bit = v_slot_bit(j);
      const int64_t p = gpos + uu;
      const uint32_t nib = (whole || (p >= pos0 && p < end)) ? (uint32_t)vcodes[uu][dim]
                                                               : (old[qq] >> bit) & 0xFu;
      w |= nib << bit;
    }
    vwords[i] = w;
  }
  {
    const int i = tid;  // 8 blocks x 4 lane groups x 8 slots = 256 scales
    const int j = i & 7, g = (i >> 3) & 3, bb = i >> 5;
    const int uu = 16 * (j >> 2) + 4 * g + (j & 3);
    const int64_t p = gpos + uu;
    if (p >= pos0 && p < end)
      reinterpret_cast<uint16_t*>(vrec + V_SCALE_OFF)[c * 256 + i] = vscales[uu][bb];
  }
}

// summary[h][p][n] = RN32(binary64 sum over slots t = 0..127 ascending of
// d(t, n/32) * code(t, n), divided by 128). One workgroup per (page, head):
// the record's codes and scales are staged in LDS with 16-byte loads, then
// thread n sums its column in order. KT: Q4_0 key records.
template <int KT>
__global__ __launch_bounds__(256) void summarize_kernel(const uint8_t* __restrict__ k_pool,
                                                        const int32_t* __restrict__ page_table,
                                                        int32_t n_kv, int32_t n_phys,
                                                        int32_t n_logical, int32_t first_page,
                                                        float* __restrict__ k_summary) {
  __shared__ __attribute__((aligned(16))) uint8_t rec[K_REC];
  const int n = threadIdx.x;
  const int h = blockIdx.y;
  const int32_t lp = first_page + blockIdx.x;
  const int32_t phys = page_table[lp];
  if (phys < 0 || phys >= n_phys) return;  // uniform across the workgroup
  constexpr int REC = KREC_OF<KT>;
  constexpr int PIECES = (REC / 16 + 255) / 256;  // 9 (Q8_0 keys), 5 (Q4_0) or 6 (Q5_1)
  const uint8_t* krec = k_pool + ((int64_t)phys * n_kv + h) * REC;
  {  // the record's 16-byte pieces, PIECES per thread, issued together
    uint4 v[PIECES];
#pragma unroll
    for (int k = 0; k < PIECES; ++k) {
      const int i = n + 256 * k;
      v[k] = reinterpret_cast<const uint4*>(krec)[i < REC / 16 ? i : REC / 16 - 1];
    }
#pragma unroll
    for (int k = 0; k < PIECES; ++k) {
      const int i = n + 256 * k;
      if (i < REC / 16) reinterpret_cast<uint4*>(rec)[i] = v[k];
    }
  }
  __syncthreads();
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec + KSCALE_OF<KT>);
  double acc = 0.0;
  for (int t = 0; t < PAGE; ++t) {
    const float d = f16_value(sc[t * 8 + n / 32]);
    float code;
    if constexpr (KT == 2) {  // d * code + m in binary64, as the oracle's Q5_1 dequantisation
      const uint32_t w = reinterpret_cast<const uint32_t*>(rec)[t * 32 + n / 8];
      const uint32_t c5 = ((w >> v_slot_bit(n & 7)) & 0xFu) |
                          (((uint32_t)rec[K5_HI_OFF + t * 32 + n / 8] >> k5_hi_bit(n & 7)) & 1u) << 4;
      const double mk = (double)f16_value(reinterpret_cast<const uint16_t*>(rec + K5_M_OFF)[t * 8 + n / 32]);
      acc = acc + ((double)d * (double)c5 + mk);
      continue;
    } else if constexpr (KT == 1) {  // dim n = 8w + k: word w of row t, nibble at v_slot_bit(k)
      const uint32_t w = reinterpret_cast<const uint32_t*>(rec)[t * 32 + n / 8];
      code = (float)((int)((w >> v_slot_bit(n & 7)) & 0xFu) - 8);
    } else {
      code = (float)(int8_t)rec[t * D + n];
    }
    const float kh = d * code;  // exact in binary32
    acc = acc + (double)kh;
  }
  k_summary[((int64_t)h * n_logical + lp) * D + n] = (float)(acc / 128.0);
}

}  // namespace

hipError_t launch_quantize(const float* k, const float* v, int64_t pos0, int32_t n_tok,
                           int32_t n_kv, const int32_t* page_table, int32_t n_phys,
                           uint8_t* k_pool, uint8_t* v_pool, bool v_q8, int k_type,
                           hipStream_t stream) {
  const int64_t g0 = pos0 / 32, g1 = (pos0 + n_tok - 1) / 32;
  dim3 grid((unsigned)(g1 - g0 + 1), (unsigned)n_kv);
  auto kern = k_type == 2   ? (v_q8 ? quantize_kernel<true, 2> : quantize_kernel<false, 2>)
              : k_type == 1 ? (v_q8 ? quantize_kernel<true, 1> : quantize_kernel<false, 1>)
                            : (v_q8 ? quantize_kernel<true, 0> : quantize_kernel<false, 0>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, k, v, pos0, n_tok, n_kv,
                     page_table, n_phys, k_pool, v_pool);
  return hipGetLastError();
}

hipError_t launch_summarize(const uint8_t* k_pool, const int32_t* page_table, int32_t n_kv,
                            int32_t n_phys, int32_t n_logical, int32_t first_page,
                            int32_t n_pages, float* k_summary, int k_type, hipStream_t stream) {
  dim3 grid((unsigned)n_pages, (unsigned)n_kv);
  auto kern = k_type == 2 ? summarize_kernel<2> : k_type == 1 ? summarize_kernel<1> : summarize_kernel<0>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, k_pool, page_table, n_kv,
                     n_phys, n_logical, first_page, k_summary);
  return hipGetLastError();
}

}  // namespace kvattn
