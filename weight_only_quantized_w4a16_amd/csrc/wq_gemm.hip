// wq_gemm.hip -- y = x . dequant(W) for large M (prefill / long context).
//
// The matrix-matrix case the Triton GPTQ page targets ("How It Works": decode
// the weights on the fly before the multiply, no slowdown with context
// length).  On gfx950 the product runs on 16x16x32 MFMAs:
//
//  * workgroup tile BM x 128 (BM = 128 or 64), four waves in a 2 x 2 grid;
//  * the activation tile (BM rows x 128 k) is staged through LDS, double
//    buffered, 16-byte chunks XOR-swizzled by row so the MFMA A reads of 16
//    rows hit 16 different bank groups;
//  * each wave loads the packed codes of its 64 columns straight from global
//    memory -- the tile layout already is the MFMA B operand, one 128-bit load
//    per lane per tile -- and dequantises them in registers with the exact
//    decode (RN(s*(q - z)) or RN(s*T[q]) in the activation dtype), so the
//    product multiplies exactly the weights the debug dump writes;
//  * with one scale per column and fp16 symmetric codes, the scale moves to
//    the epilogue (the B operand is then the exact integer q - 8).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_common.hpp"
#include "wq_decode.hpp"

namespace wq {
namespace {

struct GemmArgs {
  const uint16_t* x;      // [M][K], sorted order under act-order
  const uint32_t* codes;
  const uint16_t* S;
  const void* Z;
  const uint16_t* lut;
  uint16_t* y;
  int M, N, K, nrec, upr, ktiles, ntiles, mtiles, ntiles_wg;  // upr: 128-row units per metadata record
};

template <int DT, int BITS, int MODE, int GPU, bool EPI_SCALE, int BM>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  constexpr int BN = 128;
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int UPT = KT / 128;
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr int MT = BM / 32;         // 16-row subtiles per wave (wave covers BM/2 rows)
  constexpr int NT = 4;               // 16-column tiles per wave (64 columns)
  constexpr int KBPG = 4 / GPU;
  constexpr bool TABLE = MODE == LUT;
  constexpr int AROW_CHUNKS = 16;     // 128 halves per LDS row = 16 chunks of 16 B
  constexpr int A_LOADS = BM * AROW_CHUNKS / 256;  // 16-byte chunks per thread per unit

  __shared__ uint32_t table[TABLE ? (32 << (2 * BITS)) : 1];
  __shared__ u32x4 As[2][BM * AROW_CHUNKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, h = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: consecutive workgroups (which land on different XCDs) walk
  // down M for one column block, so the weights of a column block are shared
  // through the last-level cache while the activation rows stream.
  const int bid = blockIdx.x;
  const int mt = bid % a.mtiles, nb = bid / a.mtiles;
  const int m0 = mt * BM;
  const int nt0 = nb * (BN / 16) + wn * NT;  // first 16-column tile of this wave

  if constexpr (TABLE) {
    fill_pair_table<BITS, false>(table, a.lut, tid, 256);
  }
  const uint32_t* tab = table + (lane & 31);
  const DecodeConsts dk = make_decode_consts<DT>();

  // ---- activation staging: thread -> (row, chunk) slots of the BM x 128 tile
  u32x4 areg[A_LOADS];
  auto a_load = [&](int unit) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int slot = tid + 256 * i;
      const int r = slot >> 4, ch = slot & 15;
      const int m = m0 + r;
      areg[i] = m < a.M ? *(const u32x4*)(a.x + (size_t)m * a.K + unit * 128 + ch * 8) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto a_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int slot = tid + 256 * i;
      const int r = slot >> 4, ch = slot & 15;
      As[buf][r * AROW_CHUNKS + (ch ^ (r & 15))] = areg[i];
    }
  };

  // ---- weight words and their scales / zero-points (per wave, its NT column
  //      tiles) for one tile; column tiles past N are clamped (never stored)
  constexpr bool Z16 = MODE == ZERO_F16;
  constexpr int REC = (Z16 ? 4 : 2) * GPU;   // scale record bytes per column
  constexpr int SW = REC < 4 ? 1 : REC / 4;  // words per scale record
  constexpr int ZW = MODE == ZERO_PACKED ? GPU : 1;
  uint32_t bw[NT][WPL];
  uint32_t srec[UPT][NT][SW];
  uint32_t zrec[UPT][NT][ZW];
  auto b_load = [&](int kt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int nt = min(nt0 + t, a.ntiles - 1);
      const uint32_t* p = a.codes + (((size_t)nt * a.ktiles + kt) * 64 + lane) * WPL;
      if constexpr (WPL == 4) {
        const u32x4 v = *(const u32x4*)p;
        bw[t][0] = v[0]; bw[t][1] = v[1]; bw[t][2] = v[2]; bw[t][3] = v[3];
      } else {
#pragma unroll
        for (int j = 0; j < WPL; ++j) bw[t][j] = p[j];
      }
    }
    if constexpr (!EPI_SCALE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int rec = (kt * UPT + u) / a.upr;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int nt = min(nt0 + t, a.ntiles - 1);
          const size_t ri = (size_t)nt * a.nrec + rec;
          const uint8_t* sp = (const uint8_t*)a.S + (ri * 16 + c) * REC;
          if constexpr (REC == 2) srec[u][t][0] = *(const uint16_t*)sp;
#pragma unroll
          for (int w = 0; w < (REC == 2 ? 0 : SW); ++w) srec[u][t][w] = ((const uint32_t*)sp)[w];
          if constexpr (MODE == ZERO_PACKED) {
            const uint32_t* zp = (const uint32_t*)a.Z + (ri * 2 + (c >> 3)) * GPU;
#pragma unroll
            for (int w = 0; w < GPU; ++w) zrec[u][t][w] = zp[w];
          }
        }
      }
    }
  };

  f4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int nunits = a.ktiles * UPT;
  a_load(0);
  b_load(0);
  a_store(0);
  __syncthreads();

  for (int kt = 0; kt < a.ktiles; ++kt) {
    uint32_t cw[NT][WPL];
    uint32_t cs[UPT][NT][SW];
    uint32_t cz[UPT][NT][ZW];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < WPL; ++j) cw[t][j] = bw[t][j];
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
#pragma unroll
        for (int w = 0; w < SW; ++w) cs[u][t][w] = srec[u][t][w];
#pragma unroll
        for (int w = 0; w < ZW; ++w) cz[u][t][w] = zrec[u][t][w];
      }
    }
    if (kt + 1 < a.ktiles) b_load(kt + 1);

    sfor<UPT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int unit = kt * UPT + u;
      const int buf = unit & 1;
      if (unit + 1 < nunits) a_load(unit + 1);

      sfor<GPU>([&](auto gc) {
        constexpr int gi = decltype(gc)::value;
        ExactParams prm[NT];
        if constexpr (!EPI_SCALE) {
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float s = rec_scale<Z16>(cs[u][t], gi);
            float z;
            if constexpr (MODE == ZERO_F16) z = rec_zero16(cs[u][t], gi);
            else if constexpr (MODE == ZERO_PACKED) z = rec_zero_packed(cz[u][t], gi, c);
            else z = (float)(1 << (BITS - 1));
            prm[t].s = s;
            prm[t].s_h = h2s(s);
            prm[t].sz = MODE == LUT ? 0.0f : s * z;
          }
        }
        sfor<KBPG>([&](auto kc) {
          constexpr int kbu = gi * KBPG + decltype(kc)::value;  // k-block inside the unit
          constexpr int kb = 4 * u + kbu;                        // k-block inside the tile
          u32x4 bf[NT];
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            if constexpr (EPI_SCALE)
              bf[t] = offset_frag<BITS, DT, kb>(cw[t], dk);
            else
              bf[t] = exact_frag<BITS, DT, MODE, kb>(cw[t], prm[t], tab, dk);
          }
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const int r = wm * (BM / 2) + 16 * i + c;
            const u32x4 af = As[buf][r * AROW_CHUNKS + ((4 * kbu + h) ^ (r & 15))];
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[i][t] = mfma16<DT>(af, bf[t], acc[i][t]);
          }
        });
      });

      if (unit + 1 < nunits) {
        // Buffer buf ^ 1 was last read in the previous unit, which every wave
        // finished before the barrier that ended it.
        a_store(buf ^ 1);
        __syncthreads();
      }
    });
  }

  // ---- epilogue: lane holds rows 4h + e of each 16-row subtile, column c
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (nt0 + t >= a.ntiles) continue;
    const int n = (nt0 + t) * 16 + c;
    float s = 1.0f;
    if constexpr (EPI_SCALE) s = f16_to_f32(a.S[(size_t)(nt0 + t) * 16 + c]);  // one record per column tile
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * (BM / 2) + 16 * i + 4 * h + e;
        if (m < a.M) {
          const float v = acc[i][t][e] * s;
          a.y[(size_t)m * a.N + n] = DT == F16 ? f32_to_f16(v) : f32_to_bf16(v);
        }
      }
    }
  }
}

template <int DT, int BITS, int MODE, int GPU, bool EPI>
wq_status run_gemm(GemmArgs g, hipStream_t s) {
  const int bm = g.M <= 64 ? 64 : 128;
  g.mtiles = (g.M + bm - 1) / bm;
  g.ntiles_wg = (g.N + 127) / 128;
  const int grid = g.mtiles * g.ntiles_wg;
  if (bm == 64)
    hipLaunchKernelGGL((gemm_kernel<DT, BITS, MODE, GPU, EPI, 64>), dim3(grid), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((gemm_kernel<DT, BITS, MODE, GPU, EPI, 128>), dim3(grid), dim3(256), 0, s, g);
  return launch_status();
}

}  // namespace

// Compiled once per (activation dtype, code width): WQ_DT and WQ_BITS.
wq_status WQ_CAT(launch_gemm_, WQ_VARIANT)(const ProductArgs& p) {
  constexpr int D = WQ_DT, B = WQ_BITS;
  const Layout L = make_layout(p.K, p.N, p.bits, p.group_size, p.mode);
  GemmArgs g;
  g.x = (const uint16_t*)p.x;
  g.codes = (const uint32_t*)((const uint8_t*)p.packed + L.codes_off);
  g.S = (const uint16_t*)((const uint8_t*)p.packed + L.scales_off);
  g.Z = (const uint8_t*)p.packed + L.zeros_off;
  g.lut = p.lut;
  g.y = (uint16_t*)p.y;
  g.M = p.M; g.N = p.N; g.K = p.K; g.nrec = L.nrec; g.upr = (L.gsz > 128 ? L.gsz : 128) / 128;
  g.ktiles = L.ktiles; g.ntiles = L.ntiles;
  g.mtiles = 0; g.ntiles_wg = 0;
  const int gpu = L.gsz >= 128 ? 1 : 128 / L.gsz;
  const bool epi = L.G == 1 && p.mode == SYM && D == F16;
  wq_status st = WQ_EINVAL;
  sfor<4>([&](auto mi) {
    constexpr int MODE = decltype(mi)::value;
    if (MODE != p.mode) return;
    if (gpu == 1) {
      if (epi) { if constexpr (MODE == SYM && D == F16) st = run_gemm<D, B, MODE, 1, true>(g, p.stream); }
      else st = run_gemm<D, B, MODE, 1, false>(g, p.stream);
    } else if (gpu == 2) {
      st = run_gemm<D, B, MODE, 2, false>(g, p.stream);
    } else {
      st = run_gemm<D, B, MODE, 4, false>(g, p.stream);
    }
  });
  return st;
}

}  // namespace wq
