// wq_common.hpp -- host-side helpers shared by the entry points.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "../../include/wq.h"
#include "wq_layout.hpp"

namespace wq {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0..N-1.
template <typename F, int... I>
__host__ __device__ inline void sfor_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__host__ __device__ inline void sfor(F&& f) {
  sfor_impl(f, std::make_integer_sequence<int, N>{});
}

// Validation shared by every entry point that reads a repacked layer.
inline wq_status check_layer(int K, int N, int bits, int group_size, int mode) {
  if (K <= 0 || N <= 0) return WQ_EINVAL;
  if (bits != 2 && bits != 3 && bits != 4) return WQ_EINVAL;
  if (mode < SYM || mode > ZFINE32) return WQ_EINVAL;
  if (group_size != -1 && (group_size <= 0 || K % group_size != 0)) return WQ_EINVAL;
  if (K > (1 << 24) || N > (1 << 24)) return WQ_EUNSUPPORTED;
  if (N % 16 != 0 || K % tile_k(bits) != 0) return WQ_EUNSUPPORTED;
  const int gsz = group_size == -1 ? K : group_size;
  if (gsz % 32 != 0) return WQ_EUNSUPPORTED;
  const int kt = tile_k(bits);
  if (gsz % kt != 0 && kt % gsz != 0) return WQ_EUNSUPPORTED;
  // every section of the repacked buffer must stay below 2 GiB (buffer offsets)
  if ((size_t)K * N * bits / 8 >= ((size_t)1 << 31) || (size_t)(K / gsz) * N * 2 >= ((size_t)1 << 31))
    return WQ_EUNSUPPORTED;
  return WQ_OK;
}

// K split of the large-M product.  A workgroup covers 256 columns and 64 rows
// when the grid is small, so a narrow layer at moderate M (fewer such
// workgroups than CUs) leaves most of the GPU idle; its K range is then split
// into as many slices as keep the grid within 512 workgroups (one round at two
// workgroups per CU: rounding up left a few workgroups for a second round,
// 18 % slower on the 70B table layer at M = 64), at least 4 k-tiles per
// slice.  The partial products go through an fp32 workspace.
inline int gemm_ksplit(int M, int N, int K, int bits) {
  const long nwg = (long)((M + 63) / 64) * ((N + 255) / 256);  // 64 x 256 workgroups
  if (nwg >= 256) return 1;
  const int ktiles = K / tile_k(bits);
  int s = (int)(512 / nwg);  // at most 512: one round at two workgroups per CU
  if (s > ktiles / 4) s = ktiles / 4;
  if (s <= 1) return 1;
  const int per = (ktiles + s - 1) / s;  // k-tiles per split; no split left empty
  return (ktiles + per - 1) / per;
}

inline wq_status launch_status() {
  return hipGetLastError() == hipSuccess ? WQ_OK : WQ_EHIP;
}

// Entry points of the product kernels (validated arguments only).
struct ProductArgs {
  const void* x;            // activations [M][K] (already permuted for act-order)
  int dt;
  const void* packed;
  int mode;
  const uint16_t* lut;
  void* y;
  int M, N, K, bits, group_size;
  int swiglu;               // 1: fused gate+up layer, y [M][N/2] = SiLU(gate) * up
  hipStream_t stream;
  int ksplit = 1;           // GEMM only: K split over this many workgroups
  void* part = nullptr;     // ksplit > 1: fp32 workspace [ksplit][M][N]
  // GEMV launch shape for measurements of the shape choice itself: waves per
  // workgroup and prefetch depth (0: the library's own choice, which every
  // entry point uses)
  int waves = 0, pf = 0;
};
#define WQ_CAT2(a, b) a##b
#define WQ_CAT(a, b) WQ_CAT2(a, b)
#define WQ_DECLARE_VARIANT(v)                      \
  wq_status launch_gemv_##v(const ProductArgs& a); \
  wq_status launch_gemm_##v(const ProductArgs& a);
WQ_DECLARE_VARIANT(f16_b2)
WQ_DECLARE_VARIANT(f16_b3)
WQ_DECLARE_VARIANT(f16_b4)
WQ_DECLARE_VARIANT(bf16_b2)
WQ_DECLARE_VARIANT(bf16_b3)
WQ_DECLARE_VARIANT(bf16_b4)
#undef WQ_DECLARE_VARIANT

// The kernel files are compiled once per variant with WQ_DT / WQ_BITS set.
#if defined(WQ_DT) && defined(WQ_BITS)
#if WQ_DT == 0 && WQ_BITS == 2
#define WQ_VARIANT f16_b2
#elif WQ_DT == 0 && WQ_BITS == 3
#define WQ_VARIANT f16_b3
#elif WQ_DT == 0 && WQ_BITS == 4
#define WQ_VARIANT f16_b4
#elif WQ_DT == 1 && WQ_BITS == 2
#define WQ_VARIANT bf16_b2
#elif WQ_DT == 1 && WQ_BITS == 3
#define WQ_VARIANT bf16_b3
#else
#define WQ_VARIANT bf16_b4
#endif
#endif

// Online Hadamard rotation (validated arguments; lb = log2(block), 1..9).
wq_status launch_hadamard(const void* x, int dt, void* y, int M, int K, int lb, hipStream_t s);

inline wq_status launch_product(bool gemm, const ProductArgs& a) {
#define WQ_PICK(v) return gemm ? launch_gemm_##v(a) : launch_gemv_##v(a)
  if (a.dt == F16) {
    if (a.bits == 2) WQ_PICK(f16_b2);
    if (a.bits == 3) WQ_PICK(f16_b3);
    WQ_PICK(f16_b4);
  }
  if (a.bits == 2) WQ_PICK(bf16_b2);
  if (a.bits == 3) WQ_PICK(bf16_b3);
  WQ_PICK(bf16_b4);
#undef WQ_PICK
}

}  // namespace wq
