// wq_gemv.hip -- y = x . dequant(W) for decode-sized M (1..32).
//
// Matrix-vector products are bound by memory bandwidth; the quantised kernel
// wins only by reading fewer weight bytes, while decoding costs extra
// arithmetic (exllama bandwidth discussion, GPTQ paper quote and turboderp's
// reply).  So this kernel is built around one stream of the packed weight:
//
//  * A workgroup owns TN column tiles (16 columns each) and the whole of K;
//    its waves (1..16; a few thousand over the grid, see the launch-shape
//    choice below) split K and each streams
//    its k-range of those tiles PF tiles ahead with 128-bit coalesced buffer
//    loads, 1 KiB per wave per tile.  Loads past the range are issued with an
//    out-of-range offset instead of a branch, so the code stays straight-line
//    and every wait on the memory counter is exact.
//  * Codes become MFMA B operands in registers (offset, table or exact decode);
//    16x16x32 MFMAs do the multiply-accumulate, which leaves the vector ALUs
//    to the decode.
//  * With fp16 activations scales are applied after the MFMA, per 128-row
//    unit of K, in fp32: sum_k x*s*(q - z) = s*(sum_k x*B - c*sum_k x) with
//    B = bias + q the decoded operand and c = bias + z; sum_k x comes from one
//    more MFMA against a B of ones.  No per-element float work at all: the
//    products x*B are exact in fp32 and the bias cancels in the correction.
//    With bf16 activations the operand is the dequantised weight itself
//    (exact product, one rounding to bf16), as in the large-M product.
//  * M <= 4 packs (row m, k-block kb) into MFMA row 4m + kb, so one 128-bit
//    activation load feeds the 4 k-blocks of a unit; M <= 8 packs 8 rows x 2
//    k-blocks the same way (two loads per unit); larger M uses one MFMA row
//    per activation row (blocks of 16 rows, two for M > 16), loading four
//    rows x 256 contiguous bytes per load, regrouped into fragments through a
//    per-wave LDS stage (the fragments themselves for table codes with four
//    column tiles per wave).
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
  uint32_t codes_bytes, s_bytes, z_bytes;
  int M, N, K, nrec, upr, ktiles, waves, kt_per_wave;  // upr: 128-row units per metadata record
  int ldy;                // row stride of y (N, or N / 2 for a fused gate+up layer)
  int force_waves, force_pf;  // launch-shape overrides (0: automatic)
};

// Whether the product multiplies the dequantised weights themselves (the
// exact decode, no scale after the MFMA).  With bf16 activations always: a
// bf16 operand keeps only 8 bits, so applying the scale after the MFMA would
// multiply other weights than the rounded ones the product is defined on --
// one further bf16 rounding per weight, which with the bf16 rounding of the
// output measured outside the tolerance on a 2048-row layer.  With fp16
// activations when a unit holds more than one scale group: the four quarters
// of every MFMA k-block then belong to different groups (the tile row map),
// so no single scale can follow the MFMA.
template <int DT, int GPU>
constexpr bool gemv_scaled() { return DT == BF16 || GPU > 1; }

// Decode k-block KB of a tile into a B operand.  SCALED: the dequantised
// weight RN(s * (q - z)) or RN(s * T[q]) in the activation dtype, exactly the
// bits of the debug dump (zbits: the k-block's fine zero-point).  Otherwise
// (fp16, one group per unit): the biased code bias + q (scale and zero-point
// follow the MFMA), the table value T[q], or, for fine zero-points, RN(q - z)
// (11 bits; the scale follows the MFMA).
template <int BITS, int DT, int MODE, int KB, bool SCALED>
__device__ inline u32x4 decode_frag(const uint32_t* w, const uint32_t* tab, const DecodeConsts& k, uint32_t zbits,
                                    const ExactParams& p) {
  if constexpr (SCALED) {
    if constexpr (MODE >= ZFINE) {
      ExactParams q = p;
      q.sz = p.s * f16_to_f32((uint16_t)zbits);
      return exact_frag<BITS, DT, ZFINE, KB>(w, q, tab, k);
    } else {
      return exact_frag<BITS, DT, MODE, KB>(w, p, tab, k);
    }
  } else if constexpr (MODE == LUT && BITS < 4) {
    return perm_table_frag<BITS, KB>(w, p.rt);  // the layer's T[q] (p.rt unscaled here)
  } else if constexpr (MODE == LUT) {
    return table_frag<BITS, KB>(w, tab);
  } else if constexpr (MODE >= ZFINE) {
    return fine_frag<BITS, DT, KB>(w, zbits, k);
  } else {
    return biased_frag<BITS, KB>(w, k);
  }
}

// Zero-point correction c for (group, column): B - c == q - z (see biased_frag).
template <int DT>
__device__ inline float zero_corr(float z) {
  return z + (DT == F16 ? 1024.0f : 128.0f);
}

// Waves per workgroup are chosen at launch: 1..16, or 1..8 for the variants
// whose frames need more than the 128 registers a 1024-thread workgroup
// leaves each lane (four column tiles per wave, 2-bit codes with their
// 256-row tiles, two column tiles with four groups per unit, two blocks of
// 16 activation rows).
template <int BITS, int TN, int GPU, int MR>
constexpr bool gemv_big_frames() { return TN >= 4 || BITS == 2 || (TN >= 2 && GPU >= 4) || MR >= 2; }

// LDS bytes per wave: the partial results of the cross-wave reduction, or,
// in the standard scheme, at least the 4 KiB activation stage (the same bytes
// serve both, one after the other).
template <int TN, int MR, int PK, bool STAGE>
constexpr int gemv_wave_lds() {
  constexpr int red = TN * MR * (PK == 4 ? 1 : PK == 8 ? 2 : 4) * 64 * 4;
  return STAGE && red < 4096 ? 4096 : red;
}

// MODE is the C ABI mode (fine zero-points keep their group: 4, 5, 6).
// SWIGLU: the layer is a fused gate+up layer repacked with interleaved column
// tiles (gate, up, gate, up, ...).  Workgroup p owns output tile p: its even
// waves stream gate tile 2p, its odd waves up tile 2p + 1 (TN = 1, each pair
// of waves shares one k-range), and the store writes SiLU(gate) * up.
// MR: blocks of 16 activation rows (standard scheme; M <= 16 MR).
// STAGE: standard scheme with contiguous activation loads regrouped through
// the wave's LDS stage (otherwise the fragments are loaded directly).
// PK: packed scheme with 4 rows x 4 k-blocks (PK = 4) or 8 rows x 2 k-blocks
// (PK = 8) in the 16 MFMA rows; 0: standard scheme.
template <int DT, int BITS, int MODE, int TN, int GPU, int PK, int PF, bool SWIGLU, int MR, bool STAGE>
__global__ __launch_bounds__((gemv_big_frames<BITS, TN, GPU, MR>() ? 512 : 1024)) void gemv_kernel(const GemvArgs a) {
  constexpr bool PACKED = PK != 0;
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int UPT = KT / 128;                 // 128-row units per tile
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr int NXA = PK == 4 ? UPT : PK == 8 ? 2 * UPT : 4 * UPT;  // activation loads per tile
  constexpr bool TABLE = MODE == LUT;
  constexpr bool LDS_TABLE = TABLE && BITS == 4;  // 4-bit: LDS pair table; 2/3-bit: register tables
  constexpr bool REG_TABLE = TABLE && BITS < 4;
  constexpr bool Z16 = MODE == ZERO_F16;
  constexpr bool FINE = MODE >= ZFINE;          // fp16 zero-points per ZG rows
  constexpr int ZG = fine_zero_group(MODE);
  constexpr int ZPL = FINE ? fine_per_lane(ZG) : 0;  // fine zero-points of a lane per unit
  constexpr int SB = Z16 ? 4 : 2;               // bytes of a lane's scale (+ zero) entry
  constexpr int REC = SB * GPU;                 // scale record bytes per column
  constexpr int ZREC = 4 * GPU;                 // packed-zero record bytes per column half
  constexpr bool SCALED = gemv_scaled<DT, GPU>();
  constexpr bool XS = !SCALED && MODE != LUT && !FINE;  // shared zero-points: remove bias + z via row sums
  constexpr int ZW = FINE ? (ZPL + 1) / 2 : 1;  // words of a lane's zero entry
  constexpr int NRED = PK == 4 ? 1 : PK == 8 ? 2 : 4;  // reduced values per lane per column tile

  __shared__ __attribute__((aligned(16))) uint32_t table[LDS_TABLE ? (32 << (2 * BITS)) : 4];
  // LDS of wave w at red + w * WSTRIDE: its activation stage (standard scheme,
  // 4 KiB) while it streams, then its partial results [TN][MR][NRED][64] for
  // the cross-wave reduction.
  extern __shared__ float red[];
  constexpr int WSTRIDE = gemv_wave_lds<TN, MR, PK, STAGE>() / 4;  // floats
  static_assert(!STAGE || !PACKED, "the packed scheme loads its fragments directly");
  static_assert(!PACKED || MR == 1, "the packed scheme holds at most 8 rows");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar arithmetic
  const int c = lane & 15, h = lane >> 4;
  const int nt0 = SWIGLU ? 2 * blockIdx.x + (wave & 1) : blockIdx.x * TN;  // first column tile of this wave
  const int kslot = SWIGLU ? wave >> 1 : wave;                             // k-range of this wave

  // table codes: lane i of every wave loads T[i] first of all (lanes past the
  // table read zero)
  uint32_t lut_lane = 0;
  if constexpr (TABLE)
    lut_lane = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(a.lut, 2u << BITS), (uint32_t)lane * 2u, 0, 0);
  __builtin_amdgcn_sched_barrier(0);  // keep it ahead of the weight loads
  const rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * a.K * 2);
  const rsrc_t rs = make_rsrc(a.S, a.s_bytes);
  const rsrc_t rz = make_rsrc(MODE == ZERO_PACKED || FINE ? a.Z : a.S,
                              MODE == ZERO_PACKED || FINE ? a.z_bytes : 0u);

  // Activation buffer offsets = per-lane vector part + per-tile scalar part;
  // the vector part is kOutOfRange for rows past M (those loads return zero).
  // The MFMA k-block kb of a unit pairs position 8 h' + e of its 32-long k
  // dimension with unit row 32 h' + 8 kb + e (the tile row map), so:
  //   packed:   lane c -> (m = c / 4, k-block c % 4), one load per 128-row unit;
  //   packed 8: lane c -> (m = c / 2, k-block 2 p + c % 2), load p = 0, 1 of a
  //             unit covering its k-blocks 2 p and 2 p + 1;
  //   standard: lane c -> m = 16 r + c, one load per k-block (the MFMA
  //             fragment itself: 16 rows, 16 bytes each, per load);
  //   staged:   load j of a unit and row block r reads rows 16 r + 4 j .. + 3,
  //             lane L -> row 16 r + 4 j + L / 16, 16 bytes at k = 8 (L % 16):
  //             four rows x 256 contiguous bytes per load, regrouped into
  //             MFMA fragments through the wave's LDS stage.
  constexpr int XJ = STAGE ? 4 : 1;
  uint32_t x_lane[MR][XJ];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int xm = PK == 4 ? (c >> 2) : PK == 8 ? (c >> 1) : STAGE ? 16 * r + 4 * j + h : 16 * r + c;
      const int xk = PK == 4 ? 32 * h + 8 * (c & 3) : PK == 8 ? 32 * h + 8 * (c & 1) : STAGE ? 8 * c : 32 * h;
      x_lane[r][j] = xm < a.M ? (uint32_t)(xm * a.K + xk) * 2u : kOutOfRange;
    }
  // LDS stage of this wave: row i (0..15) of the unit at 16 chunks of 16 bytes,
  // chunk q stored at position q ^ i (the fragment reads of 16 rows then hit
  // 16 different bank groups); the fragment of k-block kb reads chunk 4 h + kb
  u32x4* const stage = (u32x4*)(red + (size_t)wave * WSTRIDE);
  int st_w[XJ], st_r[4];
#pragma unroll
  for (int j = 0; j < XJ; ++j) st_w[j] = (4 * j + h) * 16 + (c ^ (4 * j + h));
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) st_r[kb] = c * 16 + ((4 * h + kb) ^ c);
  const uint32_t w_lane = (uint32_t)lane * WPL * 4;
  // metadata: the lane's own group of each unit
  const int jg = lane_group(h, GPU);
  const uint32_t s_lane = (uint32_t)(c * REC + jg * SB);
  const uint32_t zp_lane = (uint32_t)((c >> 3) * ZREC + 4 * jg);
  const uint32_t zf_lane = FINE ? (uint32_t)((c * fine_per_unit(ZG > 0 ? ZG : 32) + h * ZPL) * 2) : 0u;
  const int nunits = a.ktiles * UPT;

  const int kt0 = kslot * a.kt_per_wave;
  const int kt1 = min(kt0 + a.kt_per_wave, a.ktiles);
  const int kt_safe = min(kt0, a.ktiles - 1);  // an in-range tile for loads whose result is unused

  struct Frame {
    uint32_t w[TN][WPL];
    u32x4 xa[MR][NXA];
    uint32_t s[TN][UPT];                      // the lane's scale (with its fp16 zero-point when Z16)
    uint32_t z[TN][UPT][ZW];                  // the lane's packed or fine zero-points
  };

  // Loads of tile kt.  CHECK: kt may lie past the wave's range; its codes are
  // then loaded out of range (free), everything else from an in-range tile
  // (the frame is never computed).  Without CHECK, kt is in range.
  auto load = [&](Frame& f, int kt, auto check) __attribute__((always_inline)) {
    constexpr bool CHECK = decltype(check)::value;
    const bool ok = !CHECK || kt < kt1;
    const int ktc = ok ? kt : kt_safe;  // keeps the scalar offsets in range
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const uint32_t so = (uint32_t)(((nt0 + t) * a.ktiles + ktc) * 64 * WPL * 4);
      const uint32_t vo = CHECK ? (ok ? w_lane : kOutOfRange) : w_lane;
      if constexpr (WPL == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, so, kNontemporal);
        f.w[t][0] = v[0]; f.w[t][1] = v[1]; f.w[t][2] = v[2]; f.w[t][3] = v[3];
      } else {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, vo, so, kNontemporal);
        f.w[t][0] = v[0]; f.w[t][1] = v[1]; f.w[t][2] = v[2];
      }
    }
#pragma unroll
    for (int r = 0; r < MR; ++r) {
#pragma unroll
      for (int i = 0; i < NXA; ++i) {
        // packed: load i covers unit i; packed 8: k-blocks 2 (i % 2) + {0, 1}
        // of unit i / 2; standard: k-block i % 4 of unit i / 4; staged: load
        // j = i % 4 of unit i / 4
        const uint32_t koff =
            (uint32_t)(ktc * KT + (PK == 4 ? 128 * i : PK == 8 ? 128 * (i / 2) + 16 * (i % 2)
                                  : STAGE ? 128 * (i / 4) : 128 * (i / 4) + 8 * (i % 4))) * 2u;
        f.xa[r][i] = __builtin_amdgcn_raw_buffer_load_b128(rx, x_lane[r][STAGE ? i % 4 : 0], koff, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int rec = (ktc * UPT + u) / a.upr;
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const uint32_t ri = (uint32_t)((nt0 + t) * a.nrec + rec);
        load_record<SB>(rs, s_lane, ri * 16 * REC, &f.s[t][u]);
        if constexpr (MODE == ZERO_PACKED) load_record<4>(rz, zp_lane, ri * 2 * ZREC, f.z[t][u]);
        if constexpr (FINE)
          load_record<2 * ZPL>(rz, zf_lane, (uint32_t)((nt0 + t) * nunits + ktc * UPT + u) * 32u * fine_per_unit(ZG),
                               f.z[t][u]);
      }
    }
  };
  const auto checked = std::integral_constant<bool, true>{};
  const auto unchecked = std::integral_constant<bool, false>{};

  Frame fr[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load(fr[p], kt0 + p, checked);
    // packed scheme: frame by frame, in the order the loop reloads them, so
    // that every wait for a frame leaves the later frames in flight
    if constexpr (PACKED) __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (LDS_TABLE) {
    fill_pair_table_lanes<BITS>(table, lut_lane, threadIdx.x, a.waves * 64);  // fp16 values
    __syncthreads();
  }
  // 2- and 3-bit tables: the values as pairs, and (scale after the MFMA) the
  // layer's table itself as a register table
  uint32_t Tp[4] = {0u, 0u, 0u, 0u};
  RegTable rt_raw = {};
  if constexpr (REG_TABLE) {
    table_pairs_from_lanes<BITS>(lut_lane, Tp);
    if constexpr (!SCALED) rt_raw = reg_table<BITS>(Tp);
  }
  const uint32_t* tab = table + (lane & 31);
  const DecodeConsts dk = make_decode_consts<DT>();

  // Scale-after paths: running sums of the scaled unit results.  Exact-decode
  // paths: MFMA accumulators carried across the whole k-range (acc), summed
  // into tot at the end.
  float tot[MR][TN][4];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) tot[r][t][e] = 0.0f;
  constexpr int NACC = PACKED ? 4 : 1;  // accumulators per (row block, column tile)
  f4 acc[SCALED ? MR : 1][TN][SCALED ? NACC : 1];
  const f4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int r = 0; r < (SCALED ? MR : 1); ++r)
#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
      for (int i = 0; i < (SCALED ? NACC : 1); ++i) acc[r][t][i] = zero4;

  // the lane's zero-point of unit u of column tile t (shared-group modes)
  auto zero_of = [&](const Frame& f, int t, int u) __attribute__((always_inline)) -> float {
    if constexpr (MODE == ZERO_F16) return f16_to_f32((uint16_t)(f.s[t][u] >> 16));
    else if constexpr (MODE == ZERO_PACKED) return (float)((f.z[t][u][0] >> (4 * (c & 7))) & 0xFu);
    else return (float)(1 << (BITS - 1));
  };
  auto scale_of = [&](const Frame& f, int t, int u) __attribute__((always_inline)) -> float { return f16_to_f32((uint16_t)(f.s[t][u] & 0xFFFFu)); };
  // fp16 bits of the fine zero-point of k-block kb (0..3 inside the unit)
  auto fine_bits = [&](const Frame& f, int t, int u, int kb) __attribute__((always_inline)) -> uint32_t {
    if constexpr (FINE) {
      const int i = kb * ZPL / 4;
      return (f.z[t][u][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    } else {
      return 0u;
    }
  };
  // exact-decode parameters of unit u of column tile t
  auto params = [&](const Frame& f, int t, int u) __attribute__((always_inline)) {
    ExactParams p;
    p.s = scale_of(f, t, u);
    p.s_h = h2s(p.s);
    p.sz = (MODE == LUT || FINE) ? 0.0f : p.s * zero_of(f, t, u);
    p.nz_h = h2s(0.0f);
    return p;
  };

  auto compute = [&](const Frame& f) __attribute__((always_inline)) {
    sfor<UPT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      ExactParams prm[TN] = {};
      if constexpr (SCALED) {
#pragma unroll
        for (int t = 0; t < TN; ++t) {
          prm[t] = params(f, t, u);
          if constexpr (REG_TABLE) prm[t].rt = scaled_reg_table<BITS, DT>(Tp, prm[t].s, dk);
        }
      } else if constexpr (REG_TABLE) {
#pragma unroll
        for (int t = 0; t < TN; ++t) prm[t].rt = rt_raw;
      }
      if constexpr (PK == 8) {
        // Two A operands per unit (p = 0, 1: rows 2m + j hold k-block 2p + j);
        // accumulator kb keeps the rows 2m + kb % 2, i.e. the elements e with
        // e % 2 == kb % 2 (row 4h + e = 2m + j: m = 2h + e / 2, j = e % 2).
        f4 ua[TN][4];
        sfor<4>([&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const u32x4 b = decode_frag<BITS, DT, MODE, 4 * u + kb, SCALED>(f.w[t], tab, dk, fine_bits(f, t, u, kb),
                                                                             prm[t]);
            if constexpr (SCALED) acc[0][t][kb] = mfma16<DT>(f.xa[0][2 * u + kb / 2], b, acc[0][t][kb]);
            else ua[t][kb] = mfma16<DT>(f.xa[0][2 * u + kb / 2], b, zero4);
          }
        });
        if constexpr (!SCALED) {
          f4 xs[2] = {zero4, zero4};
          if constexpr (XS) {
#pragma unroll
            for (int p = 0; p < 2; ++p) xs[p] = mfma16<DT>(f.xa[0][2 * u + p], ones_frag<DT>(), zero4);
          }
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const float s = scale_of(f, t, u);
            const float cz = XS ? zero_corr<DT>(zero_of(f, t, u)) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
#pragma unroll
              for (int kb = e & 1; kb < 4; kb += 2) {
                float v = ua[t][kb][e];
                if constexpr (XS) v = __builtin_fmaf(-cz, xs[kb / 2][e], v);
                tot[0][t][e] = __builtin_fmaf(s, v, tot[0][t][e]);
              }
            }
          }
        }
      } else if constexpr (PACKED) {
        // One A operand for the 4 k-blocks of the unit; accumulator kb keeps row 4m + kb.
        f4 ua[TN][4];
        sfor<4>([&](auto kbc) {
          constexpr int kb = decltype(kbc)::value;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const u32x4 b = decode_frag<BITS, DT, MODE, 4 * u + kb, SCALED>(f.w[t], tab, dk, fine_bits(f, t, u, kb),
                                                                             prm[t]);
            if constexpr (SCALED) acc[0][t][kb] = mfma16<DT>(f.xa[0][u], b, acc[0][t][kb]);
            else ua[t][kb] = mfma16<DT>(f.xa[0][u], b, zero4);
          }
        });
        if constexpr (!SCALED) {
          f4 xs = zero4;
          if constexpr (XS) xs = mfma16<DT>(f.xa[0][u], ones_frag<DT>(), zero4);
          // element e of this lane = row 4m + e = k-block e of the unit
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const float s = scale_of(f, t, u);
            const float cz = XS ? zero_corr<DT>(zero_of(f, t, u)) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = ua[t][e][e];
              if constexpr (XS) v = __builtin_fmaf(-cz, xs[e], v);
              tot[0][t][e] = __builtin_fmaf(s, v, tot[0][t][e]);
            }
          }
        }
      } else {
        // the unit's activations as MFMA fragments (k-block kb: rows 16 r + c,
        // unit rows 32 h + 8 kb ..), regrouped through the LDS stage when staged
        u32x4 xf[MR][4];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          if constexpr (STAGE) {
#pragma unroll
            for (int j = 0; j < 4; ++j) stage[st_w[j]] = f.xa[r][4 * u + j];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) xf[r][kb] = stage[st_r[kb]];
          } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) xf[r][kb] = f.xa[r][4 * u + kb];
          }
        }
        f4 ua[MR][TN];
        f4 xs[MR];
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          xs[r] = zero4;
#pragma unroll
          for (int t = 0; t < TN; ++t) ua[r][t] = zero4;
        }
        sfor<4>([&](auto kc) {
          constexpr int kb = decltype(kc)::value;
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const u32x4 b = decode_frag<BITS, DT, MODE, 4 * u + kb, SCALED>(f.w[t], tab, dk, fine_bits(f, t, u, kb),
                                                                             prm[t]);
#pragma unroll
            for (int r = 0; r < MR; ++r) {
              if constexpr (SCALED) acc[r][t][0] = mfma16<DT>(xf[r][kb], b, acc[r][t][0]);
              else ua[r][t] = mfma16<DT>(xf[r][kb], b, ua[r][t]);
            }
          }
          if constexpr (XS)
#pragma unroll
            for (int r = 0; r < MR; ++r) xs[r] = mfma16<DT>(xf[r][kb], ones_frag<DT>(), xs[r]);
        });
        if constexpr (!SCALED) {
#pragma unroll
          for (int t = 0; t < TN; ++t) {
            const float s = scale_of(f, t, u);
            const float cz = XS ? zero_corr<DT>(zero_of(f, t, u)) : 0.0f;
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                float v = ua[r][t][e];
                if constexpr (XS) v = __builtin_fmaf(-cz, xs[r][e], v);
                tot[r][t][e] = __builtin_fmaf(s, v, tot[r][t][e]);
              }
          }
        }
      }
    });
  };

  // Stream this wave's k-range PF tiles ahead.  Inside the loops every frame
  // is a valid tile and every load unconditional; the first loop's reloads all
  // lie in range (no checks), the second (at most one iteration) reloads past
  // the range with checked loads, and the last group is computed after them.
  const int T = kt1 > kt0 ? kt1 - kt0 : 0;
  const int niter = (T + PF - 1) / PF;
  const int nfast = T >= PF ? T / PF - 1 : 0;
  auto step = [&](int it, auto check) __attribute__((always_inline)) {
    const int kt = kt0 + it * PF;
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      compute(fr[p]);
      // packed scheme: each frame's reload right after its compute (left
      // alone, the scheduler sinks every reload below the last compute and
      // the wave's stream drains every PF tiles): about 3 % at M = 2-4,
      // neutral at M = 1 and for the standard scheme, which keeps the
      // scheduler's order
      if constexpr (PACKED) __builtin_amdgcn_sched_barrier(0);
      load(fr[p], kt + p + PF, check);
      if constexpr (PACKED) __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int it = 0; it < nfast; ++it) step(it, unchecked);
  for (int it = nfast; it + 1 < niter; ++it) step(it, checked);
  if (niter > 0) {
    const int kt = kt0 + (niter - 1) * PF;
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (kt + p < kt1) compute(fr[p]);
  }
  if constexpr (SCALED) {
    // packed: element e is the diagonal row 4m + e (k-block e); packed 8:
    // rows 2m + e % 2 of the two accumulators of that parity
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          tot[r][t][e] = PK == 4 ? acc[r][t][PACKED ? e : 0][e]
                       : PK == 8 ? acc[r][t][PACKED ? (e & 1) : 0][e] + acc[r][t][PACKED ? (e & 1) + 2 : 0][e]
                                 : acc[r][t][0][e];
  }

  // Cross-wave reduction and store.
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      float* dst = red + (size_t)wave * WSTRIDE + (size_t)((t * MR + r) * NRED) * 64;
      if constexpr (PK == 8) {
        dst[lane] = tot[r][t][0] + tot[r][t][1];       // row 2h
        dst[64 + lane] = tot[r][t][2] + tot[r][t][3];  // row 2h + 1
      } else if constexpr (PACKED) {
        dst[lane] = (tot[r][t][0] + tot[r][t][1]) + (tot[r][t][2] + tot[r][t][3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e * 64 + lane] = tot[r][t][e];
      }
    }
  __syncthreads();
  static_assert(!SWIGLU || TN == 1, "gate and up tiles sit on different waves");
  constexpr int SLOTS = TN * MR * NRED * 64;
  for (int i = threadIdx.x; i < SLOTS; i += a.waves * 64) {
    const int l = i & 63, e = (i >> 6) % NRED, rb = (i / (64 * NRED)) % MR, t = i / (64 * NRED * MR);
    // sum over the waves w0, w0 + step, ... of tile t's partial results
    auto reduce = [&](int w0, int step) {
      float v = 0.0f;
      for (int w = w0; w < a.waves; w += step) v += red[(size_t)w * WSTRIDE + ((t * MR + rb) * NRED + e) * 64 + l];
      return v;
    };
    float v;
    if constexpr (SWIGLU) {
      const float g = reduce(0, 2), u = reduce(1, 2);
      v = g / (1.0f + expf(-g)) * u;
    } else {
      v = reduce(0, 1);
    }
    // packed: lane l = 16 m + col; packed 8: row 2 (l / 16) + e, col l % 16;
    // standard: row 16 rb + 4 (l / 16) + e, col l % 16
    const int m = PK == 4 ? (l >> 4) : PK == 8 ? 2 * (l >> 4) + e : 16 * rb + 4 * (l >> 4) + e;
    const int n = (SWIGLU ? (int)blockIdx.x : nt0 + t) * 16 + (l & 15);
    if (m < a.M) a.y[(size_t)m * a.ldy + n] = DT == F16 ? f32_to_f16(v) : f32_to_bf16(v);
  }
}

// ---------------------------------------------------------------------------
// Launch-shape choice and dispatch.
// ---------------------------------------------------------------------------
template <int DT, int BITS, int MODE, int TN, int GPU, int PK, int PF, bool SWIGLU, int MR, bool STAGE>
wq_status run(GemvArgs g, int grid, hipStream_t s) {
  const size_t lds = (size_t)g.waves * gemv_wave_lds<TN, MR, PK, STAGE>();
  hipLaunchKernelGGL((gemv_kernel<DT, BITS, MODE, TN, GPU, PK, PF, SWIGLU, MR, STAGE>), dim3(grid), dim3(g.waves * 64),
                     lds, s, g);
  return launch_status();
}

// Launch shape (measured on MI355X for the decode layer shapes): a few
// thousand waves over the grid (about 6144 for the packed schemes, 3072 for
// one block of 16 rows, 1536 for two, 12288 for table codes), each streaming
// an equal share of K; the prefetch depth is 2 except for workgroups of one
// or two waves with long k-ranges (see run_pf).
inline int pick_waves_auto(int grid, int ktiles, bool table, int wmax, long plain);
// The waves of a launch: the override when given (clamped to wmax), else the heuristic.
inline int pick_waves(const GemvArgs& g, int grid, bool table, int wmax, long plain = 3072L) {
  if (g.force_waves > 0) return g.force_waves < wmax ? g.force_waves : wmax;
  return pick_waves_auto(grid, g.ktiles, table, wmax, plain);
}
inline int pick_waves_auto(int grid, int ktiles, bool table, int wmax, long plain) {
  // about `plain` waves in flight (12288 when each workgroup fills an LDS code
  // table -- 4-bit table codes -- which caps the workgroups per CU), at most
  // 32 k-tiles per wave, at least 2
  const long target = table ? 12288L : plain;
  int w = 1;
  while (w < wmax && 2 * w <= ktiles && ((long)grid * w < target || ktiles > 32 * w)) w *= 2;
  return w;
}
template <int DT, int BITS, int MODE, int TN, int GPU, int PK, bool SWIGLU, int MR, bool STAGE = false>
wq_status run_pf(GemvArgs g, int grid, hipStream_t s) {
  const int tpw = g.kt_per_wave;
  if constexpr (PK != 0) {
    // Prefetch depth (tiles in flight per wave): deep only when a workgroup
    // has one or two waves, each streaming a long k-range; with four or more
    // waves two tiles ahead measured best or level on every decode shape
    // (16 waves at four ahead lost up to 30 %: the frames cost half the
    // occupancy), one wave per SIMD at four ahead gained up to 20 %.
    const int pf = g.force_pf ? g.force_pf : g.waves > 2 ? 2 : tpw >= 8 ? 4 : tpw >= 5 ? 3 : 2;
    if (pf >= 4) return run<DT, BITS, MODE, TN, GPU, PK, 4, SWIGLU, MR, false>(g, grid, s);
    if (pf == 3) return run<DT, BITS, MODE, TN, GPU, PK, 3, SWIGLU, MR, false>(g, grid, s);
  }
  return run<DT, BITS, MODE, TN, GPU, PK, 2, SWIGLU, MR, STAGE>(g, grid, s);
}

// Standard scheme (one activation row per MFMA row, MR blocks of 16 rows,
// more than 8 rows).  Activations go through the LDS stage (measured on the
// decode layer shapes: 5-38 % faster at 16 rows), except with four column
// tiles per wave and table codes, whose LDS table and stage together cost
// occupancy.
template <int DT, int BITS, int MODE, int TN, int GPU, bool SWIGLU, int MR>
wq_status run_standard(GemvArgs g, int grid, hipStream_t s) {
  constexpr bool stage = MR == 2 || !(MODE == LUT && BITS == 4 && TN == 4);
  if constexpr (!stage) return run_pf<DT, BITS, MODE, TN, GPU, 0, SWIGLU, MR, false>(g, grid, s);
  else return run_pf<DT, BITS, MODE, TN, GPU, 0, SWIGLU, MR, true>(g, grid, s);
}

template <int DT, int BITS, int MODE, int GPU, bool SWIGLU, int MR>
wq_status pick_standard(GemvArgs g, hipStream_t s) {
  const int ntiles = g.N / 16;
  if constexpr (SWIGLU) {
    // One workgroup per output tile, its waves split between the gate and up
    // tiles.  Half the waves per column tile of the plain product (each
    // streaming twice the k-range) keeps the workgroup at the plain product's
    // size; measured faster than matching its per-wave work with workgroups
    // twice as large.
    const int wmax = gemv_big_frames<BITS, 1, GPU, MR>() ? 8 : 16;
    const int kw = max(1, pick_waves(g, ntiles, MODE == LUT && BITS == 4, wmax) / 2);  // waves per column tile
    g.waves = 2 * kw;
    g.kt_per_wave = (g.ktiles + kw - 1) / kw;
    return run_standard<DT, BITS, MODE, 1, GPU, true, MR>(g, ntiles / 2, s);
  } else {
    // Each wave loads 16 activation rows per row block and k-tile -- up to four
    // times the weight bytes of a column tile -- so wide layers give a wave
    // four (or two) column tiles that share those loads; narrow layers keep one
    // so that enough workgroups run.
    // 2-bit frames hold 256 rows, and a second row block doubles the activation
    // frames: four tiles would not fit the registers (nor two, for 2-bit codes
    // with four groups per 128 rows)
    constexpr int TNMAX = (BITS == 2 && GPU == 4) ? 1 : (BITS == 2 || MR == 2) ? 2 : 4;
    int tn = ntiles >= 768 ? 4 : ntiles >= 512 ? 2 : 1;
    if (tn > TNMAX) tn = TNMAX;
    // Two column tiles instead of four when the workgroups then fill their
    // last round over the 256 CUs better (1376 tiles: 344 workgroups fill
    // 67 %, 688 fill 90 %): 12-25 % faster on the 22016-column layer at
    // M = 9-16, unchanged where both fill alike; table codes keep four (their
    // two-tile variant stages the activations beside the LDS table: 20 %
    // slower).
    if (!(MODE == LUT && BITS == 4) && tn == 4 && ntiles % 2 == 0) {
      const long g4 = ntiles / 4, g2 = ntiles / 2;
      if (g2 * ((g4 + 255) / 256) > g4 * ((g2 + 255) / 256)) tn = 2;
    }
    while (ntiles % tn != 0) tn /= 2;
    const int grid = ntiles / tn;
    const bool big = tn == 4 ? gemv_big_frames<BITS, 4, GPU, MR>()
                   : tn == 2 ? gemv_big_frames<BITS, 2, GPU, MR>() : gemv_big_frames<BITS, 1, GPU, MR>();
    // two row blocks: about half the waves, each streaming twice the k-range
    // (M = 32: 10-13 % faster on the 12288- and 22016-column layers, equal on
    // the others; at 16 rows the same target loses up to 10 %)
    g.waves = pick_waves(g, grid, MODE == LUT && BITS == 4, big ? 8 : 16, MR == 2 ? 1536L : 3072L);
    g.kt_per_wave = (g.ktiles + g.waves - 1) / g.waves;
    if constexpr (TNMAX >= 4)
      if (tn == 4) return run_standard<DT, BITS, MODE, 4, GPU, false, MR>(g, grid, s);
    if constexpr (TNMAX >= 2)
      if (tn == 2) return run_standard<DT, BITS, MODE, 2, GPU, false, MR>(g, grid, s);
    return run_standard<DT, BITS, MODE, 1, GPU, false, MR>(g, grid, s);
  }
}

template <int DT, int BITS, int MODE, int GPU, bool SWIGLU>
wq_status pick_shape(GemvArgs g, hipStream_t s) {
  const int ntiles = g.N / 16;
  if (g.M > 16) {
    if constexpr (BITS == 2) {
      // Two row blocks of 2-bit frames (256 rows) do not fit the registers:
      // rows 16.. go through a second launch (the weights are streamed twice).
      GemvArgs hi = g;
      hi.x += (size_t)16 * g.K;
      hi.y += (size_t)16 * g.ldy;
      hi.M = g.M - 16;
      g.M = 16;
      const wq_status st = pick_standard<DT, BITS, MODE, GPU, SWIGLU, 1>(g, s);
      return st != WQ_OK ? st : pick_standard<DT, BITS, MODE, GPU, SWIGLU, 1>(hi, s);
    } else {
      return pick_standard<DT, BITS, MODE, GPU, SWIGLU, 2>(g, s);
    }
  }
  if (g.M > 8) return pick_standard<DT, BITS, MODE, GPU, SWIGLU, 1>(g, s);
  // Packed scheme: M <= 4 rows x 4 k-blocks, or M <= 8 rows x 2 k-blocks, in
  // the 16 MFMA rows (8 rows: 8-35 % faster at M = 5-8 than the standard
  // scheme, whose MFMA rows are half empty there).
  const int wmax = gemv_big_frames<BITS, 1, GPU, 1>() ? 8 : 16;
  const bool pk8 = g.M > 4;
  if constexpr (SWIGLU) {
    const int kw = max(1, pick_waves(g, ntiles, MODE == LUT && BITS == 4, wmax) / 2);  // waves per column tile
    g.waves = 2 * kw;
    g.kt_per_wave = (g.ktiles + kw - 1) / kw;
    return pk8 ? run_pf<DT, BITS, MODE, 1, GPU, 8, true, 1>(g, ntiles / 2, s)
               : run_pf<DT, BITS, MODE, 1, GPU, 4, true, 1>(g, ntiles / 2, s);
  } else {
    // about 6144 waves (4096 measured 3-4 % slower on the 12288- and
    // 22016-column layers at M = 1, 3072 3-10 % slower on the 12288-, 24576-
    // and 28672-column layers, equal elsewhere)
    // (two column tiles per wave, sharing the activation loads and, for table
    // codes, the LDS table fill of half as many workgroups, measured 3-35 %
    // slower on every M = 1 layer of the workloads)
    g.waves = pick_waves(g, ntiles, MODE == LUT && BITS == 4, wmax, 6144L);
    g.kt_per_wave = (g.ktiles + g.waves - 1) / g.waves;
    return pk8 ? run_pf<DT, BITS, MODE, 1, GPU, 8, false, 1>(g, ntiles, s)
               : run_pf<DT, BITS, MODE, 1, GPU, 4, false, 1>(g, ntiles, s);
  }
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
  g.codes_bytes = (uint32_t)L.codes_bytes;
  g.s_bytes = (uint32_t)L.scales_bytes;
  g.z_bytes = (uint32_t)L.zeros_bytes;
  g.M = p.M; g.N = p.N; g.K = p.K; g.nrec = L.nrec; g.upr = (L.gsz > 128 ? L.gsz : 128) / 128;
  g.ktiles = L.ktiles;
  g.waves = 1; g.kt_per_wave = 0;
  g.force_waves = p.waves; g.force_pf = p.pf;
  g.ldy = p.swiglu ? p.N / 2 : p.N;
  const int gpu = L.gsz >= 128 ? 1 : 128 / L.gsz;  // groups per 128-row unit
  wq_status st = WQ_EINVAL;
  sfor<7>([&](auto mi) {  // the ABI mode itself: fine zero-points keep their group
    constexpr int MODE = decltype(mi)::value;
    if (MODE != p.mode) return;
    if (p.swiglu) {
      if (gpu == 1) st = pick_shape<D, B, MODE, 1, true>(g, p.stream);
      else if (gpu == 2) st = pick_shape<D, B, MODE, 2, true>(g, p.stream);
      else st = pick_shape<D, B, MODE, 4, true>(g, p.stream);
    } else {
      if (gpu == 1) st = pick_shape<D, B, MODE, 1, false>(g, p.stream);
      else if (gpu == 2) st = pick_shape<D, B, MODE, 2, false>(g, p.stream);
      else st = pick_shape<D, B, MODE, 4, false>(g, p.stream);
    }
  });
  return st;
}

}  // namespace wq
