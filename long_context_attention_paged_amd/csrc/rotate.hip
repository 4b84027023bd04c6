// Hadamard rotation of 256-dim rows (key rows before quantisation, query rows
// before attention): the attention rotation that the Vulkan report (lcz.me
// topic 1398, section 沒踩到的坑：注意力旋轉) keeps on for its quantised KV
// caches. The transform is H_256 / 16 (Sylvester order) in a fixed binary32
// order, as defined in include/kvattn.h, so rotated keys quantise to the same
// bytes on every run.
#include "common.hpp"
#include "launch.hpp"

#pragma clang fp contract(off)

namespace kvattn {
namespace {

constexpr int ROT_THREADS = 256;  // four rows per workgroup, one per wavefront

// Lane l holds elements 4l..4l+3 of its row. Butterfly half-width h: 1 and 2
// pair elements inside a lane; 4..128 pair lane l with lane l ^ (h / 4), the
// lane with the bit clear keeping the sum and its partner the difference.
__global__ __launch_bounds__(ROT_THREADS) void rotate_rows_kernel(float* __restrict__ x,
                                                                  int64_t n_rows) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (ROT_THREADS / 64) + (threadIdx.x >> 6);
  if (row >= n_rows) return;  // uniform across the wavefront
  float4* p = reinterpret_cast<float4*>(x + row * D) + lane;
  const float4 v = *p;
  // h = 1: (0, 1), (2, 3)
  const float a0 = v.x + v.y, a1 = v.x - v.y, a2 = v.z + v.w, a3 = v.z - v.w;
  // h = 2: (0, 2), (1, 3)
  float e[4] = {a0 + a2, a1 + a3, a0 - a2, a1 - a3};
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float o = __shfl_xor(e[j], m);
      e[j] = upper ? o - e[j] : e[j] + o;
    }
  }
  *p = float4{e[0] * 0.0625f, e[1] * 0.0625f, e[2] * 0.0625f, e[3] * 0.0625f};
}

}  // namespace

hipError_t launch_rotate(float* x, int64_t n_rows, hipStream_t stream) {
  const int64_t per = ROT_THREADS / 64;
  hipLaunchKernelGGL(rotate_rows_kernel, dim3((unsigned)((n_rows + per - 1) / per)),
                     dim3(ROT_THREADS), 0, stream, x, n_rows);
  return hipGetLastError();
}

}  // namespace kvattn
