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

#pragma clang fp contract(off)

namespace kvattn {
namespace {

// One workgroup per (32-token group, KV head); thread n owns dim n. A 32-dim
// quantisation block is one half of a wavefront, so block reductions are
// five xor-shuffles inside that half.
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ k,
                                                       const float* __restrict__ v, int64_t pos0,
                                                       int32_t n_tok, int32_t n_kv,
                                                       const int32_t* __restrict__ page_table,
                                                       int32_t n_phys, uint8_t* __restrict__ k_pool,
                                                       uint8_t* __restrict__ v_pool) {
  __shared__ uint8_t vcodes[32][D];
  __shared__ uint16_t vscales[32][8];

  const int n = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t grp = pos0 / 32 + blockIdx.x;  // global 32-token group
  const int64_t gpos = grp * 32;
  const int64_t lp = gpos / PAGE;
  const int c = (int)((gpos % PAGE) / 32);
  const int32_t phys = page_table[lp];
  if (phys < 0 || phys >= n_phys) return;  // uniform across the workgroup
  uint8_t* krec = k_pool + ((int64_t)phys * n_kv + h) * K_REC;
  uint8_t* vrec = v_pool + ((int64_t)phys * n_kv + h) * V_REC;
  const int lane = n & 63;
  const int half_base = lane & 32;  // first lane of this 32-dim block in the wave
  const int idx_in_block = lane & 31;

  for (int u = 0; u < 32; ++u) {
    const int64_t pos = gpos + u;
    if (pos < pos0 || pos >= pos0 + n_tok) continue;  // uniform
    const int64_t ti = pos - pos0;
    const int t = c * 32 + u;  // slot in the page
    const float xk = k[(ti * n_kv + h) * D + n];
    const float xv = v[(ti * n_kv + h) * D + n];

    // Q8_0: d = RN16(RN32(amax / 127)); codes with inv = RN32(1 / d).
    float amax = fabsf(xk);
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float d32 = amax / 127.0f;
    const _Float16 d16 = (_Float16)d32;
    const float d = (float)d16;
    int8_t code8 = 0;
    uint16_t bits8 = 0;
    if (d != 0.0f) {
      const float inv = 1.0f / d;
      float r = rintf(xk * inv);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      code8 = (int8_t)(int)r;
      bits8 = __builtin_bit_cast(uint16_t, d16);
    }
    krec[t * D + n] = (uint8_t)code8;
    if (idx_in_block == 0)
      *reinterpret_cast<uint16_t*>(krec + K_SCALE_OFF + (t * 8 + n / 32) * 2) = bits8;

    // Q4_0: the lowest-index element of largest magnitude, signed, maps to -8.
    float a = fabsf(xv);
    int ai = idx_in_block;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) {
      const float oa = __shfl_xor(a, o);
      const int oi = __shfl_xor(ai, o);
      if (oa > a || (oa == a && oi < ai)) {
        a = oa;
        ai = oi;
      }
    }
    const float m = __shfl(xv, half_base + ai);
    uint8_t code4 = 8;
    uint16_t bits4 = 0;
    if (a != 0.0f) {
      const float dv32 = (-m) / 8.0f;
      const _Float16 dv16 = (_Float16)dv32;
      const float dv = (float)dv16;
      if (dv != 0.0f) {
        const float inv = 1.0f / dv;
        float r = rintf(xv * inv);
        r = fminf(fmaxf(r, -8.0f), 7.0f);
        code4 = (uint8_t)((int)r + 8);
        bits4 = __builtin_bit_cast(uint16_t, dv16);
      }
    }
    vcodes[u][n] = code4;
    if (idx_in_block == 0) vscales[u][n / 32] = bits4;
  }
  __syncthreads();

  // V words of this 32-slot group: word (q, g, d, e) holds dim 16*(4q+e)+d for
  // slots 16*(j/4) + 4g + j%4; slots outside the written range keep their bits.
  uint32_t* vwords = reinterpret_cast<uint32_t*>(vrec) + c * 1024;
  for (int i = n; i < 1024; i += 256) {
    const int e = i & 3, d = (i >> 2) & 15, g = (i >> 6) & 3, q = i >> 8;
    const int dim = 16 * (4 * q + e) + d;
    const uint32_t old = vwords[i];
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int u = 16 * (j >> 2) + 4 * g + (j & 3);
      const int bit = 4 * (j >> 1) + 16 * (j & 1);
      const int64_t pos = gpos + u;
      const uint32_t nib = (pos >= pos0 && pos < pos0 + n_tok) ? (uint32_t)vcodes[u][dim]
                                                                : (old >> bit) & 0xFu;
      w |= nib << bit;
    }
    vwords[i] = w;
  }
  {
    const int i = n;  // 8 blocks x 4 lane groups x 8 slots = 256 scales
    const int j = i & 7, g = (i >> 3) & 3, b = i >> 5;
    const int u = 16 * (j >> 2) + 4 * g + (j & 3);
    const int64_t pos = gpos + u;
    if (pos >= pos0 && pos < pos0 + n_tok)
      reinterpret_cast<uint16_t*>(vrec + V_SCALE_OFF)[c * 256 + i] = vscales[u][b];
  }
}

// summary[h][p][n] = RN32(binary64 sum over slots t = 0..127 ascending of
// d(t, n/32) * code(t, n), divided by 128). One workgroup per (page, head).
__global__ __launch_bounds__(256) void summarize_kernel(const uint8_t* __restrict__ k_pool,
                                                        const int32_t* __restrict__ page_table,
                                                        int32_t n_kv, int32_t n_phys,
                                                        int32_t n_logical, int32_t first_page,
                                                        float* __restrict__ k_summary) {
  const int n = threadIdx.x;
  const int h = blockIdx.y;
  const int32_t lp = first_page + blockIdx.x;
  const int32_t phys = page_table[lp];
  if (phys < 0 || phys >= n_phys) return;
  const uint8_t* krec = k_pool + ((int64_t)phys * n_kv + h) * K_REC;
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(krec + K_SCALE_OFF);
  double acc = 0.0;
  for (int t = 0; t < PAGE; ++t) {
    const float d = f16_value(sc[t * 8 + n / 32]);
    const float kh = d * (float)(int8_t)krec[t * D + n];  // exact in binary32
    acc = acc + (double)kh;
  }
  k_summary[((int64_t)h * n_logical + lp) * D + n] = (float)(acc / 128.0);
}

}  // namespace

hipError_t launch_quantize(const float* k, const float* v, int64_t pos0, int32_t n_tok,
                           int32_t n_kv, const int32_t* page_table, int32_t n_phys,
                           uint8_t* k_pool, uint8_t* v_pool, hipStream_t stream) {
  const int64_t g0 = pos0 / 32, g1 = (pos0 + n_tok - 1) / 32;
  dim3 grid((unsigned)(g1 - g0 + 1), (unsigned)n_kv);
  hipLaunchKernelGGL(quantize_kernel, grid, dim3(256), 0, stream, k, v, pos0, n_tok, n_kv,
                     page_table, n_phys, k_pool, v_pool);
  return hipGetLastError();
}

hipError_t launch_summarize(const uint8_t* k_pool, const int32_t* page_table, int32_t n_kv,
                            int32_t n_phys, int32_t n_logical, int32_t first_page,
                            int32_t n_pages, float* k_summary, hipStream_t stream) {
  dim3 grid((unsigned)n_pages, (unsigned)n_kv);
  hipLaunchKernelGGL(summarize_kernel, grid, dim3(256), 0, stream, k_pool, page_table, n_kv,
                     n_phys, n_logical, first_page, k_summary);
  return hipGetLastError();
}

}  // namespace kvattn
