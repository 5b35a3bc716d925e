// wq_gemm.hip -- y = x . dequant(W) for large M (prefill / long context).
//
// The matrix-matrix case the Triton GPTQ page targets ("How It Works": decode
// the weights on the fly before the multiply, no slowdown with context
// length).  On gfx950 the product runs on 16x16x32 MFMAs:
//
//  * workgroup tile BM x 256 (BM = 128, or 64 for small M), four waves side
//    by side along N: each wave owns 64 columns for all BM rows, so every
//    weight fragment is dequantised exactly once per workgroup and reused by
//    BM / 16 MFMAs;
//  * the activation tile (BM rows x 128 k) is staged through LDS by buffer
//    loads that write LDS directly (no staging registers), double buffered;
//    16-byte chunks are XOR-swizzled by row -- the swizzle is applied on the
//    source side, since a wave's load lands contiguously -- so the MFMA A
//    reads of 16 rows hit 16 different bank groups;
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
  uint32_t codes_bytes, s_bytes, z_bytes;
  int M, N, K, nrec, upr, ktiles, ntiles, mtiles, ntiles_wg;  // upr: 128-row units per metadata record
};

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int DT, int BITS, int MODE, int GPU, bool EPI_SCALE, int BM>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs a) {
  constexpr int BN = 256;
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int UPT = KT / 128;
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr int MT = BM / 16;         // 16-row subtiles per wave (a wave covers all BM rows)
  constexpr int NT = 4;               // 16-column tiles per wave (64 columns)
  constexpr int KBPG = 4 / GPU;
  constexpr bool TABLE = MODE == LUT;
  constexpr bool Z16 = MODE == ZERO_F16;
  constexpr int REC = (Z16 ? 4 : 2) * GPU;   // scale record bytes per column
  constexpr int SW = REC < 4 ? 1 : REC / 4;  // words per scale record
  constexpr int ZREC = 4 * GPU;              // packed-zero record bytes per column half
  constexpr int ZW = MODE == ZERO_PACKED ? GPU : 1;
  constexpr int AW = BM / 16;         // 1-KiB activation loads per wave per unit

  __shared__ uint32_t table[TABLE ? (32 << (2 * BITS)) : 1];
  // Two stages of the BM x 128 activation tile, 16-byte chunks, row r at
  // chunk (c ^ (r % 16)).  Separate arrays so each stage's reads and loads are
  // distinct objects.
  __shared__ __attribute__((aligned(16))) u32x4 As0[BM * 16];
  __shared__ __attribute__((aligned(16))) u32x4 As1[BM * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // -> 64-column slice
  const int c = lane & 15, h = lane >> 4;

  // Consecutive workgroups walk down M for one column block, so a column
  // block's weights are shared through the caches while activation rows stream.
  const int bid = blockIdx.x;
  const int mt = bid % a.mtiles, nb = bid / a.mtiles;
  const int m0 = mt * BM;
  const int nt0 = nb * (BN / 16) + wave * NT;  // first 16-column tile of this wave

  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * a.K * 2);
  const rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const rsrc_t rs = make_rsrc(a.S, a.s_bytes);
  const rsrc_t rz = make_rsrc(MODE == ZERO_PACKED ? a.Z : a.S, MODE == ZERO_PACKED ? a.z_bytes : 0u);

  if constexpr (TABLE) fill_pair_table<BITS, false>(table, a.lut, tid, 256);
  const uint32_t* tab = table + (lane & 31);
  const DecodeConsts dk = make_decode_consts<DT>();

  // ---- activations: wave issues AW LDS-destination loads of 1 KiB per unit.
  //      Load i of this wave fills rows 4j..4j+3 (j = wave + 4 i); lane L lands
  //      at row 4j + L / 16, physical chunk L % 16, so it fetches logical chunk
  //      (L % 16) ^ (row % 16).  Rows past M read as zero (out of range).
  uint32_t a_voff[AW];
#pragma unroll
  for (int i = 0; i < AW; ++i) {
    const int row = 4 * (wave + 4 * i) + (lane >> 4);
    const int lc = (lane & 15) ^ (row & 15);
    a_voff[i] = m0 + row < a.M ? (uint32_t)(((m0 + row) * a.K + 8 * lc) * 2) : kOutOfRange;
  }
  auto a_issue = [&](int unit, u32x4* stage) {
#pragma unroll
    for (int i = 0; i < AW; ++i)
      buffer_load_lds16(rx, stage + (wave + 4 * i) * 64, a_voff[i], (uint32_t)unit * 256);
  };

  // ---- weight words and metadata records of one tile (out of range past K);
  //      column tiles past N are clamped (never stored)
  uint32_t b_voff[NT], s_soff_t[NT], z_soff_t[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int nt = min(nt0 + t, a.ntiles - 1);
    b_voff[t] = (uint32_t)(nt * a.ktiles * 64 + lane) * WPL * 4;
    s_soff_t[t] = (uint32_t)(nt * a.nrec) * 16 * REC;
    z_soff_t[t] = (uint32_t)(nt * a.nrec) * 2 * ZREC;
  }
  uint32_t bw[NT][WPL];
  uint32_t srec[UPT][NT][SW];
  uint32_t zrec[UPT][NT][ZW];
  auto b_load = [&](int kt) {
    const bool ok = kt < a.ktiles;
    const int ktc = ok ? kt : 0;
    const uint32_t kofs = (uint32_t)ktc * 64 * WPL * 4;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t vo = ok ? b_voff[t] + kofs : kOutOfRange;
      if constexpr (WPL == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, 0, 0);
        bw[t][0] = v[0]; bw[t][1] = v[1]; bw[t][2] = v[2]; bw[t][3] = v[3];
      } else {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, vo, 0, 0);
        bw[t][0] = v[0]; bw[t][1] = v[1]; bw[t][2] = v[2];
      }
    }
    if constexpr (!EPI_SCALE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const uint32_t rec = (uint32_t)((ktc * UPT + u) / a.upr);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          load_record<REC>(rs, ok ? (uint32_t)c * REC : kOutOfRange, s_soff_t[t] + rec * 16 * REC, srec[u][t]);
          if constexpr (MODE == ZERO_PACKED)
            load_record<ZREC>(rz, ok ? (uint32_t)(c >> 3) * ZREC : kOutOfRange, z_soff_t[t] + rec * 2 * ZREC,
                              zrec[u][t]);
        }
      }
    }
  };

  f4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // One 128-row unit of K from stage `As`: 4 k-blocks of MT x NT MFMAs.
  auto compute_unit = [&](const u32x4* As, const uint32_t (&cw)[NT][WPL], const uint32_t (&cs)[NT][SW],
                          const uint32_t (&cz)[NT][ZW], auto uc) {
    constexpr int u = decltype(uc)::value;
    sfor<GPU>([&](auto gc) {
      constexpr int gi = decltype(gc)::value;
      ExactParams prm[NT];
      if constexpr (!EPI_SCALE) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float sv = rec_scale<Z16>(cs[t], gi);
          float z;
          if constexpr (MODE == ZERO_F16) z = rec_zero16(cs[t], gi);
          else if constexpr (MODE == ZERO_PACKED) z = rec_zero_packed(cz[t], gi, c);
          else z = (float)(1 << (BITS - 1));
          prm[t].s = sv;
          prm[t].s_h = h2s(sv);
          prm[t].sz = MODE == LUT ? 0.0f : sv * z;
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
          const int r = 16 * i + c;
          const u32x4 af = As[r * 16 + ((4 * kbu + h) ^ (r & 15))];
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[i][t] = mfma16<DT>(af, bf[t], acc[i][t]);
        }
      });
    });
  };

  const int nunits = a.ktiles * UPT;
  a_issue(0, As0);
  b_load(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
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
    sfor<UPT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int unit = kt * UPT + u;
      // the stage of a unit alternates; with UPT = 2 it follows u, else kt
      const bool odd = UPT == 2 ? (u == 1) : (kt & 1);
      // Next weights (once per tile), then the next unit's activations; both
      // stream while this unit computes.  The wait counter logic does not
      // see the LDS-destination loads, so the current weights were copied out
      // before any of them was issued and the unit ends with an explicit full
      // wait and a barrier.
      if constexpr (u == 0) b_load(kt + 1);
      if (unit + 1 < nunits) a_issue(unit + 1, odd ? As0 : As1);
      compute_unit(odd ? As1 : As0, cw, cs[u], cz[u], uc);
      if (unit + 1 < nunits) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
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
        const int m = m0 + 16 * i + 4 * h + e;
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
  g.ntiles_wg = (g.N + 255) / 256;
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
  g.codes_bytes = (uint32_t)L.codes_bytes;
  g.s_bytes = (uint32_t)L.scales_bytes;
  g.z_bytes = (uint32_t)L.zeros_bytes;
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
