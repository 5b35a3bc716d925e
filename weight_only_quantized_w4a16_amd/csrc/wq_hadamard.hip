// wq_hadamard.hip -- online Hadamard rotation of the activations.
//
// The FLUTE page ("Maintenance & Community") lists Hadamard-transform support
// with no details.  Read as the rotation used with rotated weight-only
// quantisation: weights rotated offline (H W) and quantised, activations
// rotated at run time by the same orthonormal block-diagonal Walsh-Hadamard
// matrix, so (x H)(H W) = x W.  For block size b and every block of b
// consecutive elements of a row:
//     y[k0 + i] = b^(-1/2) * sum_j (-1)^popcount(i & j) * x[k0 + j].
//
// The transform is a fast Walsh-Hadamard butterfly: each lane holds 8
// consecutive elements (one 16-byte load), the first three butterfly levels
// run inside the lane, the remaining log2(b / 8) levels pair lanes whose
// index differs in one bit (cross-lane shuffles).  A block of up to 512
// elements therefore lives in one wave and the kernel is one streaming pass:
// 2 * M * K bytes read and written, fp32 arithmetic, one rounding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_common.hpp"
#include "wq_decode.hpp"

namespace wq {
namespace {

// LB = log2(block).  One thread per 8-element chunk; chunk c sits at position
// c % (b / 8) of its block and, since waves start at multiples of 64 chunks,
// that is lane % (b / 8) for every b <= 512.
// x and y may be the same buffer (in-place rotation): each thread reads its
// own 16 bytes before it writes them, so neither pointer is restrict.
template <int DT, int LB>
__global__ __launch_bounds__(256) void hadamard_kernel(const uint16_t* x, uint16_t* y, uint32_t chunks, float norm) {
  const uint32_t c = blockIdx.x * 256u + threadIdx.x;
  const int lane = threadIdx.x & 63;
  u32x4 raw = {0u, 0u, 0u, 0u};
  if (c < chunks) raw = *(const u32x4*)(x + (size_t)c * 8);
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint16_t lo = (uint16_t)(raw[q] & 0xFFFFu), hi = (uint16_t)(raw[q] >> 16);
    v[2 * q] = DT == F16 ? f16_to_f32(lo) : bf16_to_f32(lo);
    v[2 * q + 1] = DT == F16 ? f16_to_f32(hi) : bf16_to_f32(hi);
  }
  // butterfly levels on element-index bits 0..2 (inside the lane)
#pragma unroll
  for (int bit = 1; bit < 8 && bit < (1 << LB); bit <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e & bit) continue;
      const float a = v[e], b = v[e | bit];
      v[e] = a + b;
      v[e | bit] = a - b;
    }
  }
  // levels on element-index bits 3.. (lane bits 0..): the lane with the bit
  // set keeps partner - own, the other own + partner
#pragma unroll
  for (int d = 1; d < (1 << LB) / 8; d <<= 1) {
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = __shfl_xor(v[e], d, 64);
      v[e] = upper ? p - v[e] : v[e] + p;
    }
  }
  if (c < chunks) {
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = pack2<DT>(v[2 * q] * norm, v[2 * q + 1] * norm);
    *(u32x4*)(y + (size_t)c * 8) = out;
  }
}

template <int DT>
wq_status launch(const void* x, void* y, int M, int K, int lb, hipStream_t s) {
  const uint32_t chunks = (uint32_t)((size_t)M * K / 8);
  const dim3 grid((chunks + 255) / 256), block(256);
  const float norm = (float)(1.0 / __builtin_sqrt((double)(1 << lb)));
  const uint16_t* xi = (const uint16_t*)x;
  uint16_t* yo = (uint16_t*)y;
  bool ok = true;
  sfor<10>([&](auto lc) {
    constexpr int L = decltype(lc)::value;
    if constexpr (L >= 1) {
      if (L == lb) hipLaunchKernelGGL((hadamard_kernel<DT, L>), grid, block, 0, s, xi, yo, chunks, norm);
    } else {
      if (L == lb) ok = false;
    }
  });
  if (!ok) return WQ_EINVAL;
  return launch_status();
}

}  // namespace

wq_status launch_hadamard(const void* x, int dt, void* y, int M, int K, int lb, hipStream_t s) {
  return dt == F16 ? launch<F16>(x, y, M, K, lb, s) : launch<BF16>(x, y, M, K, lb, s);
}

}  // namespace wq
