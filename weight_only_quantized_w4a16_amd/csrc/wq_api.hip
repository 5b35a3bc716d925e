// wq_api.hip -- C entry points: validation, offline repack, debug dequant,
// act-order gather, dispatch of the product kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "wq_common.hpp"
#include "wq_decode.hpp"

using namespace wq;

// ---------------------------------------------------------------------------
// Repack kernels
// ---------------------------------------------------------------------------

// Code of row k of column n in the canonical layout (column = little-endian
// bit stream along K, word r at qweight[r][n]).
template <int BITS>
__device__ inline uint32_t canonical_code(const uint32_t* qw, int N, int n, int k) {
  const uint32_t bit = (uint32_t)BITS * (uint32_t)k;
  const uint32_t r = bit >> 5, sh = bit & 31;
  uint32_t v = qw[(size_t)r * N + n] >> sh;
  if (sh + BITS > 32) v |= qw[(size_t)(r + 1) * N + n] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// Place code q of element e, k-block kb into a lane's words (see wq_layout.hpp).
template <int BITS, bool TABLE_LAYOUT>
__device__ inline void place_code(uint32_t* w, int kb, int e, uint32_t q) {
  if (BITS == 4) {
    const int nib = TABLE_LAYOUT ? e : (e % 2) * 4 + e / 2;
    w[kb] |= q << (4 * nib);
  } else if (BITS == 2 && TABLE_LAYOUT) {
    // four codes byte-aligned: byte e % 4, bits 2 (2 (kb % 2) + e / 4)
    w[kb / 2] |= q << (8 * (e % 4) + 2 * (2 * (kb % 2) + e / 4));
  } else if (BITS == 2) {
    const int i = 4 * (kb % 2) + e / 2;
    w[kb / 2] |= q << (16 * (e % 2) + 2 * i);
  } else if (TABLE_LAYOUT) {
    // 3-bit table codes, four codes byte-aligned: group x = 2 kb + e / 4, byte e % 4
    const int x = 2 * kb + e / 4, b = e % 4;
    if (x < 6) {
      w[x / 2] |= q << (8 * b + 3 * (x % 2));
    } else {
      w[x - 6] |= (q & 3u) << (8 * b + 6);
      w[2] |= ((q >> 2) & 1u) << (8 * b + (x - 6) + 6);
    }
  } else {
    const int p = 4 * kb + e / 2;
    const int fb = 3 * (e % 2);  // bit offset of this code inside the 6-bit pair field
    if (p < 15) {
      w[p / 5] |= q << (6 * (p % 5) + fb);
    } else {
      for (int b = 0; b < 3; ++b) {
        const int fbit = fb + b;
        w[fbit / 2] |= ((q >> b) & 1u) << (30 + fbit % 2);
      }
    }
  }
}

// Source column tile of destination tile nt.  For a fused gate+up layer
// ([gate | up] along N) the tiles are interleaved gate, up, gate, up, ... so
// that the two halves of every output column sit in adjacent tiles.
__device__ inline int source_tile(int nt, int ntiles, int gate_up) {
  return gate_up ? ((nt & 1) ? ntiles / 2 + (nt >> 1) : (nt >> 1)) : nt;
}

// One thread per lane-slot of a tile: grid (ktiles, ntiles), block 64.
template <int BITS, bool TABLE_LAYOUT>
__global__ void repack_codes_kernel(const uint32_t* __restrict__ qw, const int32_t* __restrict__ perm,
                                    int N, int ktiles, int gate_up, uint32_t* __restrict__ out) {
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int KB = KT / 32;
  constexpr int WPL = BITS == 3 ? 3 : 4;
  const int lane = threadIdx.x, kt = blockIdx.x, nt = blockIdx.y;
  const int c = lane & 15, h = lane >> 4;
  const int n = source_tile(nt, (int)gridDim.y, gate_up) * 16 + c;
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int kb = 0; kb < KB; ++kb) {
    for (int e = 0; e < 8; ++e) {
      const int row = kt * KT + tile_row(kb, h, e);
      const int k = perm ? perm[row] : row;
      place_code<BITS, TABLE_LAYOUT>(w, kb, e, canonical_code<BITS>(qw, N, n, k));
    }
  }
  uint32_t* dst = out + (((size_t)nt * ktiles + kt) * 64 + lane) * WPL;
  for (int j = 0; j < WPL; ++j) dst[j] = w[j];
}

// Scale records: [G][N] (+ fp16 zero-points [G][N]) -> [N/16][R][16][GPU]
// (pairs (s, z) when zeros16 is given).  grid (R, ntiles), block 16 * gpu.
__global__ void repack_scales_kernel(const uint16_t* __restrict__ scales, const uint16_t* __restrict__ zeros16,
                                     int N, int nrec, int gpu, int gate_up, void* __restrict__ dst) {
  const int c = threadIdx.x / gpu, j = threadIdx.x % gpu, rec = blockIdx.x, nt = blockIdx.y;
  const int g = rec * gpu + j;
  const size_t src = (size_t)g * N + source_tile(nt, (int)gridDim.y, gate_up) * 16 + c;
  const size_t o = (((size_t)nt * nrec + rec) * 16 + c) * gpu + j;
  if (zeros16)
    ((uint32_t*)dst)[o] = (uint32_t)scales[src] | ((uint32_t)zeros16[src] << 16);
  else
    ((uint16_t*)dst)[o] = scales[src];
}

// Packed zero-points: canonical row g = bit stream along N of BITS-wide codes
// -> per (column tile, record, half, group in record) one word of 8 nibbles.
template <int BITS>
__global__ void repack_zeros_packed_kernel(const uint32_t* __restrict__ zp, int N, int nrec, int gpu, int ntiles,
                                           int gate_up, uint32_t* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // ((nt * nrec + rec) * 2 + half) * gpu + j
  if (i >= ntiles * nrec * 2 * gpu) return;
  const int j = i % gpu, half = (i / gpu) % 2, rec = (i / (2 * gpu)) % nrec, nt = i / (2 * gpu * nrec);
  const int g = rec * gpu + j;
  const size_t wpr = (size_t)N * BITS / 32;
  uint32_t word = 0;
  for (int c = 0; c < 8; ++c) {
    const uint32_t bit = (uint32_t)BITS * (uint32_t)(source_tile(nt, ntiles, gate_up) * 16 + 8 * half + c);
    const uint32_t r = bit >> 5, sh = bit & 31;
    uint32_t v = zp[g * wpr + r] >> sh;
    if (sh + BITS > 32) v |= zp[g * wpr + r + 1] << (32 - sh);
    word |= (v & ((1u << BITS) - 1u)) << (4 * c);
  }
  dst[i] = word;
}

// Fine zero-points: fp16 [K / zg][N] -> [N/16][K/128][16][128/zg] (layout in
// wq_layout.hpp).  One thread per entry.
__global__ void repack_zeros_fine_kernel(const uint16_t* __restrict__ zeros, int N, int K, int zg, int ntiles,
                                         int gate_up, uint16_t* __restrict__ dst) {
  const int per = fine_per_unit(zg);  // entries per column and unit
  const size_t total = (size_t)ntiles * (K / 128) * 16 * per;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int e = (int)(i % per), c = (int)((i / per) % 16);
  const size_t rest = i / (16 * per);
  const int u = (int)(rest % (K / 128)), nt = (int)(rest / (K / 128));
  dst[i] = zeros[(size_t)(u * per + e) * N + source_tile(nt, ntiles, gate_up) * 16 + c];
}

// ---------------------------------------------------------------------------
// Debug dequantisation: one wave per tile, exact path (the one the large-M
// product uses), written back in the original row order.
// ---------------------------------------------------------------------------
template <int BITS, int DT, int MODE>
__global__ __launch_bounds__(64) void dequant_debug_kernel(const uint8_t* __restrict__ packed, Layout L,
                                                          const uint16_t* __restrict__ lut,
                                                          const int32_t* __restrict__ perm,
                                                          uint16_t* __restrict__ w) {
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int KB = KT / 32;
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr bool LDS_TABLE = MODE == LUT && BITS == 4;
  __shared__ __attribute__((aligned(16))) uint32_t table[LDS_TABLE ? (32 << (2 * BITS)) : 4];
  const int lane = threadIdx.x, kt = blockIdx.x, nt = blockIdx.y;
  const int c = lane & 15, h = lane >> 4;
  if constexpr (LDS_TABLE) {
    fill_pair_table<BITS, false>(table, lut, lane, 64);
    __syncthreads();
  }
  // 2- and 3-bit tables: the values as pairs in registers (lane i loads T[i])
  uint32_t Tp[4] = {0u, 0u, 0u, 0u};
  if constexpr (MODE == LUT && BITS < 4) {
    const uint32_t tv = lane < (1 << BITS) ? lut[lane] : 0u;
    table_pairs_from_lanes<BITS>(tv, Tp);
  }
  const uint32_t* tab = table + (lane & 31);
  const DecodeConsts dk = make_decode_consts<DT>();
  const uint32_t* src = (const uint32_t*)(packed + L.codes_off) + (((size_t)nt * L.ktiles + kt) * 64 + lane) * WPL;
  uint32_t words[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < WPL; ++j) words[j] = src[j];
  const uint8_t* S = packed + L.scales_off;
  const uint32_t* Z = (const uint32_t*)(packed + L.zeros_off);
  const int n = nt * 16 + c;
  sfor<KB>([&](auto kbc) {
    constexpr int kb = decltype(kbc)::value;
    const int row0 = kt * KT + tile_row(kb, h, 0);
    const int unit = row0 / 128;
    const int rec = meta_record(unit, L.gsz);
    const int j = L.gpu > 1 ? (row0 % 128) / L.gsz : 0;  // group inside the record
    const size_t ri = (((size_t)nt * L.nrec + rec) * 16 + c) * L.gpu + j;
    float sv, zv;
    if (MODE == ZFINE) {
      sv = f16_to_f32(((const uint16_t*)S)[ri]);
      const int zg = fine_zero_group(L.mode);
      const size_t zi = (((size_t)nt * (L.K / 128) + unit) * 16 + c) * fine_per_unit(zg) + (row0 % 128) / zg;
      zv = f16_to_f32(((const uint16_t*)Z)[zi]);
    } else if (MODE == ZERO_F16) {
      const uint32_t w2 = ((const uint32_t*)S)[ri];
      sv = f16_to_f32((uint16_t)(w2 & 0xFFFFu));
      zv = f16_to_f32((uint16_t)(w2 >> 16));
    } else {
      sv = f16_to_f32(((const uint16_t*)S)[ri]);
      zv = MODE == ZERO_PACKED
               ? rec_zero_packed(Z + (((size_t)nt * L.nrec + rec) * 2 + (c >> 3)) * L.gpu, j, c)
               : (float)(1 << (BITS - 1));
    }
    ExactParams p;
    p.s = sv;
    p.s_h = h2s(p.s);
    p.sz = MODE == LUT ? 0.0f : p.s * zv;
    if constexpr (MODE == LUT && BITS < 4) p.rt = scaled_reg_table<BITS, DT>(Tp, p.s, dk);
    const u32x4 v = exact_frag<BITS, DT, MODE, kb>(words, p, tab, dk);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = row0 + e;
      const int k = perm ? perm[row] : row;
      const uint32_t pair = v[e / 2];
      w[(size_t)k * L.N + n] = (uint16_t)((e % 2) ? (pair >> 16) : (pair & 0xFFFFu));
    }
  });
}

// Act-order: xp[m][i] = x[m][perm[i]].  Eight consecutive i per thread: two
// 16-byte loads of perm, eight independent 2-byte loads of x, one 16-byte
// store (K % 8 == 0, perm and xp 16-byte aligned, M * K < 2^31: checked by
// the caller).
__global__ void gather_x8_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, int M, int K,
                                 uint16_t* __restrict__ xp) {
  const int k8 = K >> 3;
  const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (unsigned)M * (unsigned)k8) return;
  const unsigned m = t / (unsigned)k8, i = (t - m * (unsigned)k8) * 8u;
  const int4 p0 = *(const int4*)(perm + i), p1 = *(const int4*)(perm + i + 4);
  const uint16_t* xr = x + (size_t)m * K;
  uint4 v;
  v.x = (uint32_t)xr[p0.x] | ((uint32_t)xr[p0.y] << 16);
  v.y = (uint32_t)xr[p0.z] | ((uint32_t)xr[p0.w] << 16);
  v.z = (uint32_t)xr[p1.x] | ((uint32_t)xr[p1.y] << 16);
  v.w = (uint32_t)xr[p1.z] | ((uint32_t)xr[p1.w] << 16);
  *(uint4*)(xp + (size_t)m * K + i) = v;
}
// The same one element per thread (any alignment of perm).
__global__ void gather_x_kernel(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm, int M, int K,
                                uint16_t* __restrict__ xp) {
  const unsigned i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (unsigned)M * (unsigned)K) return;
  const unsigned m = i / (unsigned)K, k = i - m * (unsigned)K;
  xp[i] = x[(size_t)m * K + perm[k]];
}

// ---------------------------------------------------------------------------
// C entry points
// ---------------------------------------------------------------------------
extern "C" {

int wq_layout_version(void) { return WQ_LAYOUT_VERSION; }

const char* wq_status_str(wq_status s) {
  switch (s) {
    case WQ_OK: return "ok";
    case WQ_EINVAL: return "invalid argument";
    case WQ_EUNSUPPORTED: return "unsupported shape or configuration";
    case WQ_EHIP: return "HIP runtime error";
    case WQ_ENOSPACE: return "workspace too small";
  }
  return "unknown status";
}

size_t wq_packed_bytes(int K, int N, int bits, int group_size, wq_qmode mode) {
  if (check_layer(K, N, bits, group_size, mode) != WQ_OK) return 0;
  return make_layout(K, N, bits, group_size, mode).total;
}

// Workspace layout: [permuted x, M*K*2 bytes, when act-order] then, 256-byte
// aligned, [K-split partial products, ksplit*M*N*4 bytes, large-M product
// only].
static size_t perm_ws_bytes(int M, int K, int has_perm) { return has_perm ? align256((size_t)M * K * 2) : 0; }
static size_t split_ws_bytes(int M, int N, int K, int bits) {
  const int ks = gemm_ksplit(M, N, K, bits);
  return ks > 1 ? (size_t)ks * M * N * 4 : 0;
}

size_t wq_workspace_bytes(int M, int N, int K, int bits, int has_perm) {
  if (M <= 0 || K <= 0 || N <= 0) return 0;
  return perm_ws_bytes(M, K, has_perm) + split_ws_bytes(M, N, K, bits);
}

static wq_status repack(const uint32_t* qweight, const uint16_t* scales, const void* zeros, wq_qmode mode,
                        const int32_t* g_idx_host, int K, int N, int bits, int group_size, void* packed,
                        int32_t* perm, void* stream, int gate_up) {
  wq_status st = check_layer(K, N, bits, group_size, mode);
  if (st != WQ_OK) return st;
  if (gate_up && N % 32 != 0) return WQ_EUNSUPPORTED;
  if (!qweight || !scales || !packed) return WQ_EINVAL;
  if ((mode == ZERO_F16 || mode == ZERO_PACKED || fine_zero_group(mode)) && !zeros) return WQ_EINVAL;
  if (mode == ZERO_PACKED && ((long)N * bits) % 32 != 0) return WQ_EINVAL;
  if (g_idx_host && !perm) return WQ_EINVAL;
  // fine zero groups follow the original row order, which act-order breaks up
  if (g_idx_host && fine_zero_group(mode)) return WQ_EUNSUPPORTED;
  const Layout L = make_layout(K, N, bits, group_size, mode);
  hipStream_t s = (hipStream_t)stream;

  // Act-order: stable sort of rows by group; every group must hold gsz rows.
  std::vector<int32_t> host_perm;
  if (g_idx_host) {
    std::vector<int> count(L.G, 0);
    for (int k = 0; k < K; ++k) {
      const int g = g_idx_host[k];
      if (g < 0 || g >= L.G) return WQ_EINVAL;
      ++count[g];
    }
    for (int g = 0; g < L.G; ++g)
      if (count[g] != L.gsz) return WQ_EUNSUPPORTED;
    std::vector<int> next(L.G);
    for (int g = 0; g < L.G; ++g) next[g] = g * L.gsz;
    host_perm.resize(K);
    for (int k = 0; k < K; ++k) host_perm[next[g_idx_host[k]]++] = k;
    if (hipMemcpyAsync(perm, host_perm.data(), sizeof(int32_t) * K, hipMemcpyHostToDevice, s) != hipSuccess)
      return WQ_EHIP;
  }
  const int32_t* dperm = g_idx_host ? perm : nullptr;
  uint8_t* out = (uint8_t*)packed;
  const bool table_layout = mode == LUT;
  dim3 grid(L.ktiles, L.ntiles);
#define WQ_REPACK_CODES(B)                                                                              \
  if (table_layout)                                                                                     \
    hipLaunchKernelGGL((repack_codes_kernel<B, true>), grid, dim3(64), 0, s, qweight, dperm, N, L.ktiles, \
                       gate_up, (uint32_t*)(out + L.codes_off));                                        \
  else                                                                                                  \
    hipLaunchKernelGGL((repack_codes_kernel<B, false>), grid, dim3(64), 0, s, qweight, dperm, N, L.ktiles, \
                       gate_up, (uint32_t*)(out + L.codes_off));
  if (bits == 4) { WQ_REPACK_CODES(4) }
  else if (bits == 3) { WQ_REPACK_CODES(3) }
  else { WQ_REPACK_CODES(2) }
#undef WQ_REPACK_CODES
  hipLaunchKernelGGL(repack_scales_kernel, dim3(L.nrec, L.ntiles), dim3(16 * L.gpu), 0, s, scales,
                     mode == ZERO_F16 ? (const uint16_t*)zeros : nullptr, N, L.nrec, L.gpu, gate_up,
                     (void*)(out + L.scales_off));
  if (fine_zero_group(mode)) {
    const size_t n = L.zeros_bytes / 2;
    hipLaunchKernelGGL(repack_zeros_fine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)zeros, N, K, fine_zero_group(mode), L.ntiles, gate_up,
                       (uint16_t*)(out + L.zeros_off));
  }
  if (mode == ZERO_PACKED) {
    const int words = L.ntiles * L.nrec * 2 * L.gpu;
    dim3 g2((words + 255) / 256);
    if (bits == 4)
      hipLaunchKernelGGL(repack_zeros_packed_kernel<4>, g2, dim3(256), 0, s, (const uint32_t*)zeros, N, L.nrec,
                         L.gpu, L.ntiles, gate_up, (uint32_t*)(out + L.zeros_off));
    else if (bits == 3)
      hipLaunchKernelGGL(repack_zeros_packed_kernel<3>, g2, dim3(256), 0, s, (const uint32_t*)zeros, N, L.nrec,
                         L.gpu, L.ntiles, gate_up, (uint32_t*)(out + L.zeros_off));
    else
      hipLaunchKernelGGL(repack_zeros_packed_kernel<2>, g2, dim3(256), 0, s, (const uint32_t*)zeros, N, L.nrec,
                         L.gpu, L.ntiles, gate_up, (uint32_t*)(out + L.zeros_off));
  }
  st = launch_status();
  // host_perm is read by the copy above: wait before it goes out of scope,
  // also when a launch failed.
  const bool synced = hipStreamSynchronize(s) == hipSuccess;
  if (st != WQ_OK) return st;
  return synced ? WQ_OK : WQ_EHIP;
}

wq_status wq_repack(const uint32_t* qweight, const uint16_t* scales, const void* zeros, wq_qmode mode,
                    const int32_t* g_idx_host, int K, int N, int bits, int group_size, void* packed,
                    int32_t* perm, void* stream) {
  return repack(qweight, scales, zeros, mode, g_idx_host, K, N, bits, group_size, packed, perm, stream, 0);
}

wq_status wq_repack_gate_up(const uint32_t* qweight, const uint16_t* scales, const void* zeros, wq_qmode mode,
                            const int32_t* g_idx_host, int K, int N, int bits, int group_size, void* packed,
                            int32_t* perm, void* stream) {
  return repack(qweight, scales, zeros, mode, g_idx_host, K, N, bits, group_size, packed, perm, stream, 1);
}

wq_status wq_dequant_debug(const void* packed, wq_qmode mode, const uint16_t* lut, const int32_t* perm, int K,
                           int N, int bits, int group_size, wq_dtype out, void* w, void* stream) {
  wq_status st = check_layer(K, N, bits, group_size, mode);
  if (st != WQ_OK) return st;
  if (!packed || !w) return WQ_EINVAL;
  if (out != WQ_F16 && out != WQ_BF16) return WQ_EINVAL;
  if (mode == LUT && !lut) return WQ_EINVAL;
  if (perm && fine_zero_group(mode)) return WQ_EUNSUPPORTED;
  const Layout L = make_layout(K, N, bits, group_size, mode);
  hipStream_t s = (hipStream_t)stream;
  dim3 grid(L.ktiles, L.ntiles);
  bool launched = false;
  sfor<3>([&](auto bi) {
    constexpr int B = decltype(bi)::value + 2;
    if (B != bits) return;
    sfor<2>([&](auto di) {
      constexpr int D = decltype(di)::value;
      if (D != (int)out) return;
      sfor<5>([&](auto mi) {
        constexpr int MODE = decltype(mi)::value;
        if (MODE != kernel_mode((int)mode)) return;
        hipLaunchKernelGGL((dequant_debug_kernel<B, D, MODE>), grid, dim3(64), 0, s, (const uint8_t*)packed, L,
                           lut, perm, (uint16_t*)w);
        launched = true;
      });
    });
  });
  if (!launched) return WQ_EINVAL;
  return launch_status();
}

static wq_status product(bool gemm, bool swiglu, const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                         const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K, int bits,
                         int group_size, void* ws, size_t ws_bytes, void* stream) {
  wq_status st = check_layer(K, N, bits, group_size, mode);
  if (st != WQ_OK) return st;
  if (M < 0) return WQ_EINVAL;
  if (dt != WQ_F16 && dt != WQ_BF16) return WQ_EINVAL;
  if (!gemm && M > 32) return WQ_EUNSUPPORTED;
  if (swiglu && N % 32 != 0) return WQ_EUNSUPPORTED;
  if (M == 0) return WQ_OK;
  if (!x || !packed || !y) return WQ_EINVAL;
  if (mode == LUT && !lut) return WQ_EINVAL;
  if (perm && fine_zero_group(mode)) return WQ_EUNSUPPORTED;
  if (((uintptr_t)x | (uintptr_t)y | (uintptr_t)packed) & 15) return WQ_EUNSUPPORTED;
  if (M > (1 << 24)) return WQ_EUNSUPPORTED;
  if ((size_t)M * K * 2 >= ((size_t)1 << 31)) return WQ_EUNSUPPORTED;  // activation buffer offsets
  const int ksplit = gemm ? gemm_ksplit(M, N, K, bits) : 1;
  const size_t need = perm_ws_bytes(M, K, perm != nullptr) + (ksplit > 1 ? split_ws_bytes(M, N, K, bits) : 0);
  if (need && (!ws || ws_bytes < need)) return WQ_ENOSPACE;
  if (need && ((uintptr_t)ws & 15)) return WQ_EUNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const void* xin = x;
  if (perm) {
    const size_t total = (size_t)M * K;  // < 2^30 (activation buffer check above)
    if (K % 8 == 0 && ((uintptr_t)perm & 15) == 0)
      hipLaunchKernelGGL(gather_x8_kernel, dim3((unsigned)((total / 8 + 255) / 256)), dim3(256), 0, s,
                         (const uint16_t*)x, perm, M, K, (uint16_t*)ws);
    else
      hipLaunchKernelGGL(gather_x_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                         (const uint16_t*)x, perm, M, K, (uint16_t*)ws);
    if ((st = launch_status()) != WQ_OK) return st;
    xin = ws;
  }
  ProductArgs a{xin, (int)dt, packed, (int)mode, lut, y, M, N, K, bits, group_size, swiglu ? 1 : 0, s};
  a.ksplit = ksplit;
  a.part = ksplit > 1 ? (void*)((uint8_t*)ws + perm_ws_bytes(M, K, perm != nullptr)) : nullptr;
  return launch_product(gemm, a);
}

// ---------------------------------------------------------------------------
// Scratch for wq_gemm_noalloc: one static device array per GPU, the library's
// only device memory of its own.  Its host-side name is not a device address;
// the address comes from hipGetSymbolAddress, taken once per device (with
// that device current) and kept.  The K-split partial products never exceed
// 32 MiB (at most 512 slices x workgroups of 64 x 256 outputs, 4 bytes each);
// the other 32 MiB hold the act-order permuted activations.
// ---------------------------------------------------------------------------
static constexpr size_t kScratchBytes = WQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
static constexpr int kMaxDevices = 64;
static void* scratch_ptr[kMaxDevices];
static std::mutex scratch_mu;

// Device address of this GPU's scratch array (nullptr if it cannot be had).
static void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

wq_status wq_gemm_noalloc(const void* x, wq_dtype dt, const void* packed, wq_qmode mode, const uint16_t* lut,
                          const int32_t* perm, void* y, int M, int N, int K, int bits, int group_size,
                          void* stream) {
  wq_status st = check_layer(K, N, bits, group_size, mode);
  if (st != WQ_OK) return st;
  if (M < 0) return WQ_EINVAL;
  if (M == 0) return WQ_OK;
  if (M > (1 << 24)) return WQ_EUNSUPPORTED;
  // the same scratch wq_gemm would need, checked against the array's size
  const size_t need = wq_workspace_bytes(M, N, K, bits, perm != nullptr);
  if (need > kScratchBytes) return WQ_ENOSPACE;
  void* ws = need ? device_scratch() : nullptr;
  if (need && !ws) return WQ_EHIP;
  return product(true, false, x, dt, packed, mode, lut, perm, y, M, N, K, bits, group_size, ws,
                 need ? kScratchBytes : 0, stream);
}

wq_status wq_gemv(const void* x, wq_dtype dt, const void* packed, wq_qmode mode, const uint16_t* lut,
                  const int32_t* perm, void* y, int M, int N, int K, int bits, int group_size, void* ws,
                  size_t ws_bytes, void* stream) {
  return product(false, false, x, dt, packed, mode, lut, perm, y, M, N, K, bits, group_size, ws, ws_bytes, stream);
}

wq_status wq_gemm(const void* x, wq_dtype dt, const void* packed, wq_qmode mode, const uint16_t* lut,
                  const int32_t* perm, void* y, int M, int N, int K, int bits, int group_size, void* ws,
                  size_t ws_bytes, void* stream) {
  return product(true, false, x, dt, packed, mode, lut, perm, y, M, N, K, bits, group_size, ws, ws_bytes, stream);
}

wq_status wq_gemv_gate_up(const void* x, wq_dtype dt, const void* packed, wq_qmode mode, const uint16_t* lut,
                          const int32_t* perm, void* y, int M, int N, int K, int bits, int group_size, void* ws,
                          size_t ws_bytes, void* stream) {
  return product(false, true, x, dt, packed, mode, lut, perm, y, M, N, K, bits, group_size, ws, ws_bytes, stream);
}

wq_status wq_gemm_gate_up(const void* x, wq_dtype dt, const void* packed, wq_qmode mode, const uint16_t* lut,
                          const int32_t* perm, void* y, int M, int N, int K, int bits, int group_size, void* ws,
                          size_t ws_bytes, void* stream) {
  return product(true, true, x, dt, packed, mode, lut, perm, y, M, N, K, bits, group_size, ws, ws_bytes, stream);
}

wq_status wq_hadamard(const void* x, wq_dtype dt, void* y, int M, int K, int block, void* stream) {
  if (M < 0 || K <= 0) return WQ_EINVAL;
  if (dt != WQ_F16 && dt != WQ_BF16) return WQ_EINVAL;
  if (block < 2 || block > 512 || (block & (block - 1)) != 0 || K % block != 0) return WQ_EINVAL;
  if (K % 8 != 0) return WQ_EUNSUPPORTED;
  if ((size_t)M * K >= ((size_t)1 << 31)) return WQ_EUNSUPPORTED;
  if (M == 0) return WQ_OK;
  if (!x || !y) return WQ_EINVAL;
  if (((uintptr_t)x | (uintptr_t)y) & 15) return WQ_EUNSUPPORTED;
  // x and y either coincide (in place) or do not overlap
  const uintptr_t xb = (uintptr_t)x, yb = (uintptr_t)y, n = (uintptr_t)M * K * 2;
  if (xb != yb && xb < yb + n && yb < xb + n) return WQ_EINVAL;
  return launch_hadamard(x, (int)dt, y, M, K, __builtin_ctz((unsigned)block), (hipStream_t)stream);
}

}  // extern "C"
