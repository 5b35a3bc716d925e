// wq_gemv.hip -- y = x . dequant(W) for decode-sized M (1..16).
//
// Matrix-vector products are bound by memory bandwidth; the quantised kernel
// wins only by reading fewer weight bytes, while decoding costs extra
// arithmetic (exllama bandwidth discussion, GPTQ paper quote and turboderp's
// reply).  So this kernel is built around one stream of the packed weight:
//
//  * A workgroup owns TN column tiles (16 columns each) and the whole of K;
//    its WAVES waves split K and each streams its k-range of those tiles, PF
//    tiles ahead (128-bit coalesced loads, 1 KiB per wave per tile).
//  * Codes become MFMA B operands in registers (offset or table decode);
//    16x16x32 MFMAs do the multiply-accumulate, which leaves the vector ALUs
//    to the decode.
//  * Scales are applied after the MFMA, per 128-row unit of K, in fp32:
//    sum_k x*s*(q - z) = s*(sum_k x*B - c*sum_k x) with B the decoded operand
//    and c the zero-point correction; sum_k x comes from one more MFMA against
//    a B of ones.  No per-element scaling and no zero subtraction in fp16.
//  * M <= 4 packs (row m, k-block kb) into MFMA row 4m + kb, so one 128-bit
//    activation load feeds the 4 k-blocks of a unit; larger M uses one MFMA
//    row per activation row and one activation load per k-block.
//  * Waves reduce through LDS at the end; the output is rounded once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_common.hpp"
#include "wq_decode.hpp"

namespace wq {
namespace {

struct GemvArgs {
  const uint16_t* x;      // [M][K], sorted order under act-order
  const uint32_t* codes;  // tile layout
  const uint16_t* S;      // scales [N/16][G][16]
  const void* Z;          // zero-points (re-laid) or null
  const uint16_t* lut;    // fp16 [2^bits] (table mode)
  uint16_t* y;            // [M][N]
  int M, N, K, G, gsz, ktiles, kt_per_wave;
};

// Decode k-block KB of a tile into a B operand.
template <int BITS, int DT, int MODE, int KB>
__device__ inline u32x4 decode_frag(const uint32_t* w, const uint32_t* tab) {
  if constexpr (MODE == LUT)
    return table_frag<BITS, KB>(w, tab);
  else
    return offset_frag<BITS, DT, KB>(w);
}

// Zero-point correction c for (group, column): B - c == q - z (see offset_frag).
template <int DT, int MODE, int BITS>
__device__ inline float zero_corr(float z) {
  if constexpr (DT == F16) return z - (float)(1 << (BITS - 1));
  else return z + 128.0f;
}

template <int DT, int BITS, int MODE, int TN, int GPU, bool PACKED, int WAVES, int PF>
__global__ __launch_bounds__(WAVES * 64) void gemv_kernel(const GemvArgs a) {
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int UPT = KT / 128;                 // 128-row units per tile
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr int NXA = PACKED ? UPT : 4 * UPT;   // activation loads per tile
  constexpr int NS = UPT * GPU;                 // (scale, zero) pairs per tile per column tile
  constexpr int KBPG = 4 / GPU;                 // k-blocks per group inside a unit
  constexpr bool TABLE = MODE == LUT;
  constexpr bool HAS_Z = MODE == ZERO_F16 || MODE == ZERO_PACKED;
  constexpr bool XS = HAS_Z || (DT == BF16 && MODE != LUT);
  constexpr int NRED = PACKED ? 1 : 4;          // reduced values per lane per column tile

  __shared__ uint32_t table[TABLE ? (32 << (2 * BITS)) : 1];
  __shared__ float red[WAVES][TN][NRED][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, h = lane >> 4;
  const int nt0 = blockIdx.x * TN;

  if constexpr (TABLE) {
    fill_pair_table<BITS, DT == BF16>(table, a.lut, threadIdx.x, WAVES * 64);
    __syncthreads();
  }
  const uint32_t* tab = table + (lane & 31);

  // Activation row this lane feeds into the MFMA A operand.
  //   packed:   lane c -> (m = c / 4, k-block c % 4) ; standard: lane c -> m = c
  const int xm = PACKED ? (c >> 2) : c;
  const bool xok = xm < a.M;
  const uint16_t* xrow = a.x + (size_t)(xok ? xm : 0) * a.K + 8 * h + (PACKED ? 32 * (c & 3) : 0);

  float tot[TN][4];
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) tot[t][e] = 0.0f;

  struct Frame {
    uint32_t w[TN][WPL];
    u32x4 xa[NXA];
    uint16_t s[TN][NS];
    uint32_t z[TN][NS];
  };

  auto load = [&](Frame& f, int kt) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint32_t* p = a.codes + (((size_t)(nt0 + t) * a.ktiles + kt) * 64 + lane) * WPL;
      if constexpr (WPL == 4) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
        f.w[t][0] = v[0]; f.w[t][1] = v[1]; f.w[t][2] = v[2]; f.w[t][3] = v[3];
      } else {
#pragma unroll
        for (int j = 0; j < WPL; ++j) f.w[t][j] = __builtin_nontemporal_load(p + j);
      }
    }
#pragma unroll
    for (int i = 0; i < NXA; ++i) {
      // packed: unit i covers rows 128 i ..; standard: k-block i covers rows 32 i ..
      const int off = kt * KT + (PACKED ? 128 * i : 32 * i);
      f.xa[i] = xok ? *(const u32x4*)(xrow + off) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int g = (kt * KT + j * (128 / GPU)) / a.gsz;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const size_t mi = ((size_t)(nt0 + t) * a.G + g);
        f.s[t][j] = a.S[mi * 16 + c];
        if constexpr (MODE == ZERO_F16) f.z[t][j] = ((const uint16_t*)a.Z)[mi * 16 + c];
        else if constexpr (MODE == ZERO_PACKED) f.z[t][j] = ((const uint32_t*)a.Z)[mi * 2 + (c >> 3)];
        else f.z[t][j] = 0u;
      }
    }
  };

  auto zero_of = [&](uint32_t zraw) -> float {
    if constexpr (MODE == ZERO_F16) return f16_to_f32((uint16_t)zraw);
    else if constexpr (MODE == ZERO_PACKED) return (float)((zraw >> (4 * (c & 7))) & 0xFu);
    else return (float)(1 << (BITS - 1));
  };

  auto compute = [&](const Frame& f) {
    const f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    sfor<UPT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      if constexpr (PACKED) {
        // One A operand for the 4 k-blocks of the unit; accumulator kb keeps row 4m + kb.
        f4 acc[TN][4];
        sfor<4>([&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const u32x4 b = decode_frag<BITS, DT, MODE, 4 * u + kb>(f.w[t], tab);
            acc[t][kb] = mfma16<DT>(f.xa[u], b, zero4);
          }
        });
        f4 xs = zero4;
        if constexpr (XS) xs = mfma16<DT>(f.xa[u], ones_frag<DT>(), zero4);
        // element e of this lane = row 4m + e = k-block e of the unit
#pragma unroll
        for (int t = 0; t < TN; ++t) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = u * GPU + e / KBPG;
            const float s = f16_to_f32(f.s[t][j]);
            float v = acc[t][e][e];
            if constexpr (XS) v = __builtin_fmaf(-zero_corr<DT, MODE, BITS>(zero_of(f.z[t][j])), xs[e], v);
            tot[t][e] = __builtin_fmaf(s, v, tot[t][e]);
          }
        }
      } else {
        sfor<GPU>([&](auto gc) {
          constexpr int gi = decltype(gc)::value;
          f4 acc[TN];
#pragma unroll
          for (int t = 0; t < TN; ++t) acc[t] = zero4;
          f4 xs = zero4;
          sfor<KBPG>([&](auto kc) {
            constexpr int kb = 4 * u + gi * KBPG + decltype(kc)::value;  // k-block inside the tile
#pragma unroll
            for (int t = 0; t < TN; ++t) {
              const u32x4 b = decode_frag<BITS, DT, MODE, kb>(f.w[t], tab);
              acc[t] = mfma16<DT>(f.xa[kb], b, acc[t]);
            }
            if constexpr (XS) xs = mfma16<DT>(f.xa[kb], ones_frag<DT>(), xs);
          });
          const int j = u * GPU + gi;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const float s = f16_to_f32(f.s[t][j]);
            const float cz = XS ? zero_corr<DT, MODE, BITS>(zero_of(f.z[t][j])) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = acc[t][e];
              if constexpr (XS) v = __builtin_fmaf(-cz, xs[e], v);
              tot[t][e] = __builtin_fmaf(s, v, tot[t][e]);
            }
          }
        });
      }
    });
  };

  // Stream this wave's k-range, PF tiles ahead.
  const int kt0 = wave * a.kt_per_wave;
  const int kt1 = min(kt0 + a.kt_per_wave, a.ktiles);
  if (kt0 < kt1) {
    Frame fr[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (kt0 + p < kt1) load(fr[p], kt0 + p);
    for (int kt = kt0; kt < kt1; kt += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        if (kt + p < kt1) {
          compute(fr[p]);
          if (kt + p + PF < kt1) load(fr[p], kt + p + PF);
        }
      }
    }
  }

  // Cross-wave reduction and store.
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    if constexpr (PACKED) {
      red[wave][t][0][lane] = (tot[t][0] + tot[t][1]) + (tot[t][2] + tot[t][3]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][t][e][lane] = tot[t][e];
    }
  }
  __syncthreads();
  constexpr int SLOTS = TN * NRED * 64;
  for (int i = threadIdx.x; i < SLOTS; i += WAVES * 64) {
    const int l = i & 63, e = (i >> 6) % NRED, t = i / (64 * NRED);
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][t][e][l];
    // packed: lane l = 16 m + col ; standard: row 4 (l / 16) + e, col l % 16
    const int m = PACKED ? (l >> 4) : 4 * (l >> 4) + e;
    const int n = (nt0 + t) * 16 + (l & 15);
    if (m < a.M) a.y[(size_t)m * a.N + n] = DT == F16 ? f32_to_f16(v) : f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Launch-shape choice and dispatch.
// ---------------------------------------------------------------------------
template <int DT, int BITS, int MODE, int TN, int GPU, bool PACKED, int WAVES>
wq_status run(const GemvArgs& g, int grid, hipStream_t s) {
  constexpr int PF = (!PACKED && TN >= 2) ? 2 : 3;
  hipLaunchKernelGGL((gemv_kernel<DT, BITS, MODE, TN, GPU, PACKED, WAVES, PF>), dim3(grid), dim3(WAVES * 64), 0, s,
                     g);
  return launch_status();
}

template <int DT, int BITS, int MODE, int GPU>
wq_status pick_shape(const GemvArgs& g, hipStream_t s) {
  const int ntiles = g.N / 16;
  GemvArgs a = g;
  if (g.M <= 4) {
    // Packed activations, one column tile per workgroup; small layers get
    // 16 waves per workgroup so that every CU has enough loads in flight.
    const int grid = ntiles;
    const int waves = (grid < 512 && g.ktiles >= 16) ? 16 : 4;
    a.kt_per_wave = (g.ktiles + waves - 1) / waves;
    if (waves == 16) return run<DT, BITS, MODE, 1, GPU, true, 16>(a, grid, s);
    return run<DT, BITS, MODE, 1, GPU, true, 4>(a, grid, s);
  }
  // One activation row per MFMA row; two column tiles per workgroup share the
  // activation loads when the grid stays large enough.
  const int tn = (ntiles % 2 == 0 && ntiles / 2 >= 512) ? 2 : 1;
  const int grid = ntiles / tn;
  a.kt_per_wave = (g.ktiles + 7) / 8;
  if (tn == 2) return run<DT, BITS, MODE, 2, GPU, false, 8>(a, grid, s);
  return run<DT, BITS, MODE, 1, GPU, false, 8>(a, grid, s);
}

}  // namespace

// Compiled once per (activation dtype, code width): WQ_DT and WQ_BITS.
wq_status WQ_CAT(launch_gemv_, WQ_VARIANT)(const ProductArgs& p) {
  constexpr int D = WQ_DT, B = WQ_BITS;
  const Layout L = make_layout(p.K, p.N, p.bits, p.group_size, p.mode);
  GemvArgs g;
  g.x = (const uint16_t*)p.x;
  g.codes = (const uint32_t*)((const uint8_t*)p.packed + L.codes_off);
  g.S = (const uint16_t*)((const uint8_t*)p.packed + L.scales_off);
  g.Z = (const uint8_t*)p.packed + L.zeros_off;
  g.lut = p.lut;
  g.y = (uint16_t*)p.y;
  g.M = p.M; g.N = p.N; g.K = p.K; g.G = L.G; g.gsz = L.gsz; g.ktiles = L.ktiles; g.kt_per_wave = 0;
  const int gpu = L.gsz >= 128 ? 1 : 128 / L.gsz;  // groups per 128-row unit
  wq_status st = WQ_EINVAL;
  sfor<4>([&](auto mi) {
    constexpr int MODE = decltype(mi)::value;
    if (MODE != p.mode) return;
    if (gpu == 1) st = pick_shape<D, B, MODE, 1>(g, p.stream);
    else if (gpu == 2) st = pick_shape<D, B, MODE, 2>(g, p.stream);
    else st = pick_shape<D, B, MODE, 4>(g, p.stream);
  });
  return st;
}

}  // namespace wq
