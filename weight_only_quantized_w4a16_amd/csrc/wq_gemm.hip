// wq_gemm.hip -- y = x . dequant(W) for large M (prefill / long context).
//
// The matrix-matrix case the Triton GPTQ page targets ("How It Works": decode
// the weights on the fly before the multiply, no slowdown with context
// length).  On gfx950 the product runs on 16x16x32 MFMAs:
//
//  * workgroup tile BM x BN (128 x 256, 128 x 128 or 64 x 256, by the decode's
//    register needs and M), four waves side by side along N: each wave owns
//    BN / 4 columns for all BM rows, so every weight fragment is dequantised
//    exactly once per workgroup and reused by BM / 16 MFMAs;
//  * the activation tile (BM rows x 128 k) is staged through LDS by buffer
//    loads that write LDS directly (no staging registers), double buffered;
//    16-byte chunks are XOR-swizzled by row -- the swizzle is applied on the
//    source side, since a wave's load lands contiguously -- so the MFMA A
//    reads of 16 rows hit 16 different bank groups;
//  * each wave loads the packed codes of its columns straight from global
//    memory -- the tile layout already is the MFMA B operand, one 128-bit load
//    per lane per tile -- and dequantises them in registers.  The product
//    multiplies exactly the weights the debug dump writes (RN(s*(q - z)) or
//    RN(s*T[q]) in the activation dtype) for every decode but one: with fp16
//    activations and fp16 zero-points (shared or fine) q - z is formed in
//    fp16 first, RN(s*RN(q - z)), which differs only where q - z needs more
//    than 11 significant bits (never for zero-points in [8, 16); for those in
//    [4, 8) where |q - z| >= 8);
//  * with one scale per column and fp16 symmetric codes, the scale moves to
//    the epilogue (the weight operand is then the exact integer q - 8, and
//    (q - 8) * s is exact in fp32 before the output rounding);
//  * the weights are the MFMA A operand and the activations B, so each lane
//    ends with four consecutive outputs of one row: 8-byte stores.
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
  int swiglu;             // fused gate+up layer: y [M][N/2] = SiLU(gate) * up
  int ksplit, ktps;       // K split over ksplit workgroups of ktps k-tiles (1: no split)
  float* part;            // ksplit > 1: fp32 partial products [ksplit][M][N]
};

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int DT, int BITS, int MODE, int GPU, bool EPI_SCALE, int BM, int NT>
__global__ __launch_bounds__(256, 2) void gemm_kernel(const GemmArgs a) {
  constexpr int BN = 64 * NT;         // NT 16-column tiles per wave, four waves
  constexpr int KT = BITS == 2 ? 256 : 128;
  constexpr int UPT = KT / 128;
  constexpr int WPL = BITS == 3 ? 3 : 4;
  constexpr int MT = BM / 16;         // 16-row subtiles per wave (a wave covers all BM rows)
  constexpr bool TABLE = MODE == LUT;
  constexpr bool Z16 = MODE == ZERO_F16;
  constexpr bool FINE = MODE >= ZFINE;       // fp16 zero-points per ZG rows (MODE is the ABI mode)
  constexpr int ZG = fine_zero_group(MODE);
  constexpr int ZPL = FINE ? fine_per_lane(ZG) : 0;  // fine zero-points of a lane per unit
  constexpr int SB = Z16 ? 4 : 2;            // bytes of a lane's scale (+ zero) entry
  constexpr int REC = SB * GPU;              // scale record bytes per column
  constexpr int ZREC = 4 * GPU;              // packed-zero record bytes per column half
  constexpr int ZW = FINE ? (ZPL + 1) / 2 : 1;  // words of a lane's zero entry
  constexpr int AW = BM / 16;         // 1-KiB activation loads per wave per unit

  // Table columns: 32 (one per lane of a half-wave), 16 for 4-bit tables in
  // 128 x 128 tiles, whose 80 KiB of LDS (16 KiB table + two 32 KiB stages)
  // then leave room for two workgroups per CU.
  constexpr int COPIES = (TABLE && BITS == 4 && NT == 2) ? 16 : 32;
  constexpr bool LDS_TABLE = TABLE && BITS == 4;  // 2/3-bit tables: register tables per group and column
  // one-shift nibble decode (bf16) except in 128 x 256 tiles, where its two
  // extra registers per column tile would spill
  constexpr bool SPLIT4 = !(BM == 128 && NT == 4);
  __shared__ __attribute__((aligned(16))) uint32_t table[LDS_TABLE ? (COPIES << (2 * BITS)) : 4];
  // Two stages of the BM x 128 activation tile, 16-byte chunks, row r at
  // chunk (c ^ (r % 16)).  Separate arrays so each stage's reads and loads are
  // distinct objects.
  __shared__ __attribute__((aligned(16))) u32x4 As0[BM * 16];
  __shared__ __attribute__((aligned(16))) u32x4 As1[BM * 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // -> its BN / 4 columns
  const int c = lane & 15, h = lane >> 4;

  // Tile order: M fastest.  Workgroups are dispatched to the 8 XCDs
  // round-robin (id i -> XCD i % 8, each XCD with its own L2), so with a
  // multiple of 8 row tiles an XCD only ever sees 1/8 of the activation row
  // tiles (which stay in its L2) while the weight column blocks stream past,
  // each shared by the XCD's workgroups on the same block.
  const int bid = blockIdx.x;
  const int mt = bid % a.mtiles, nb = (bid / a.mtiles) % a.ntiles_wg, ks = bid / (a.mtiles * a.ntiles_wg);
  const int kt0 = ks * a.ktps, kt1 = min(kt0 + a.ktps, a.ktiles);  // this workgroup's k-tiles
  const int m0 = mt * BM;
  const int nt0 = nb * (BN / 16) + wave * NT;  // first 16-column tile of this wave

  const rsrc_t rx = make_rsrc(a.x, (uint32_t)a.M * a.K * 2);
  const rsrc_t rc = make_rsrc(a.codes, a.codes_bytes);
  const rsrc_t rs = make_rsrc(a.S, a.s_bytes);
  const rsrc_t rz = make_rsrc(MODE == ZERO_PACKED || FINE ? a.Z : a.S, MODE == ZERO_PACKED || FINE ? a.z_bytes : 0u);
  // metadata: the lane's own group of each unit (the tile row map gives lane
  // half h rows 32 h .. 32 h + 31 of every unit)
  const int jg = lane_group(h, GPU);
  const uint32_t s_lane = (uint32_t)(c * REC + jg * SB);
  const uint32_t zp_lane = (uint32_t)((c >> 3) * ZREC + 4 * jg);
  const uint32_t zf_lane = FINE ? (uint32_t)((c * fine_per_unit(ZG > 0 ? ZG : 32) + h * ZPL) * 2) : 0u;

  if constexpr (LDS_TABLE) fill_pair_table<BITS, false, COPIES>(table, a.lut, tid, 256);
  uint32_t Tp[4] = {0u, 0u, 0u, 0u};  // 2/3-bit tables: the values as pairs (lane i loads T[i])
  if constexpr (TABLE && !LDS_TABLE) {
    const uint32_t tv = __builtin_amdgcn_raw_buffer_load_b16(make_rsrc(a.lut, 2u << BITS), (uint32_t)lane * 2u, 0, 0);
    table_pairs_from_lanes<BITS>(tv, Tp);
  }
  const uint32_t* tab = table + (lane % COPIES);
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
    z_soff_t[t] = FINE ? (uint32_t)(nt * a.ktiles * UPT) * 32u * fine_per_unit(ZG > 0 ? ZG : 32)
                       : (uint32_t)(nt * a.nrec) * 2 * ZREC;
  }
  // Weight registers of one tile.
  struct BSet {
    uint32_t w[NT][WPL];
    uint32_t s[UPT][NT];       // the lane's scale (with its fp16 zero-point when Z16)
    uint32_t z[UPT][NT][ZW];   // the lane's packed or fine zero-points
  };
  // loads issued by one b_load (codes, scale records, packed-zero records)
  constexpr int NBL = NT * (1 + (EPI_SCALE ? 0 : UPT) + (MODE == ZERO_PACKED || FINE ? UPT : 0));
  auto b_load = [&](BSet& bs, int kt) {
    // Past K every offset gets 2^31 added (out of range, reads zero): a
    // scalar add instead of a select, so the code stays branch-free.
    const bool ok = kt < kt1;
    const int ktc = ok ? kt : 0;
    const uint32_t oob = ok ? 0u : kOutOfRange;
    const uint32_t kofs = (uint32_t)ktc * 64 * WPL * 4 + oob;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint32_t vo = b_voff[t] + kofs;
      if constexpr (WPL == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, vo, 0, 0);
        bs.w[t][0] = v[0]; bs.w[t][1] = v[1]; bs.w[t][2] = v[2]; bs.w[t][3] = v[3];
      } else {
        typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
        const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rc, vo, 0, 0);
        bs.w[t][0] = v[0]; bs.w[t][1] = v[1]; bs.w[t][2] = v[2];
      }
    }
    if constexpr (!EPI_SCALE) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const uint32_t rec = (uint32_t)((ktc * UPT + u) / a.upr);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          load_record<SB>(rs, s_lane + oob, s_soff_t[t] + rec * 16 * REC, &bs.s[u][t]);
          if constexpr (MODE == ZERO_PACKED)
            load_record<4>(rz, zp_lane + oob, z_soff_t[t] + rec * 2 * ZREC, bs.z[u][t]);
          if constexpr (FINE)
            load_record<2 * ZPL>(rz, zf_lane + oob,
                                 z_soff_t[t] + (uint32_t)(ktc * UPT + u) * 32u * fine_per_unit(ZG), bs.z[u][t]);
        }
      }
    }
  };

  f4 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  // A fragment (activation rows 16 i .. 16 i + 15, k-block kbu) from stage As:
  // lane half h takes unit rows 32 h + 8 kbu .. + 7 (the tile row map), i.e.
  // 16-byte chunk 4 h + kbu of the row.
  auto a_frag = [&](const u32x4* As, int kbu, int i) {
    const int r = 16 * i + c;
    return As[r * 16 + ((kbu + 4 * h) ^ (r & 15))];
  };
  // One 128-row unit of K from stage `As`: 4 k-blocks of MT x NT MFMAs, taken
  // as pairs of row subtiles.  With 128-row tiles the A fragments of the next
  // pair are read from LDS before the MFMAs of the current pair are issued, so
  // each read has the pair's 2 NT MFMAs to complete; with 64-row tiles the
  // extra registers would cost a wave per SIMD, so the reads stay next to
  // their MFMAs.
  constexpr bool LOOKAHEAD = BM == 128;
  auto compute_unit = [&](const u32x4* As, const uint32_t (&cw)[NT][WPL], const uint32_t (&cs)[NT],
                          const uint32_t (&cz)[NT][ZW], auto uc) {
    constexpr int u = decltype(uc)::value;
    constexpr int PAIRS = MT / 2;       // row-subtile pairs per k-block
    constexpr int STEPS = 4 * PAIRS;    // pairs per unit
    ExactParams prm[NT];
    u32x4 bf[NT];
    u32x4 f0, f1;
    if constexpr (LOOKAHEAD) {
      f0 = a_frag(As, 0, 0);
      f1 = a_frag(As, 0, 1);
    }
    sfor<STEPS>([&](auto sc) {
      constexpr int step = decltype(sc)::value;
      constexpr int kbu = step / PAIRS, ip = step % PAIRS;  // k-block inside the unit, pair
      constexpr int kb = 4 * u + kbu;                         // k-block inside the tile
      if constexpr (ip == 0) {
        if constexpr (!EPI_SCALE && kbu == 0) {  // the lane's group of this unit
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float sv = f16_to_f32((uint16_t)(cs[t] & 0xFFFFu));
            float z;
            if constexpr (MODE == ZERO_F16) z = f16_to_f32((uint16_t)(cs[t] >> 16));
            else if constexpr (MODE == ZERO_PACKED) z = (float)((cz[t][0] >> (4 * (c & 7))) & 0xFu);
            else z = (float)(1 << (BITS - 1));
            prm[t].s = sv;
            prm[t].s_h = h2s(sv);
            prm[t].sz = MODE == LUT ? 0.0f : sv * z;
            prm[t].nz_h = h2s(MODE == ZERO_PACKED ? -(1024.0f + z) : -z);
            if constexpr (TABLE && !LDS_TABLE) prm[t].rt = scaled_reg_table<BITS, DT>(Tp, sv, dk);
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if constexpr (EPI_SCALE) {
            bf[t] = offset_frag<BITS, DT, kb>(cw[t], dk);
          } else if constexpr (FINE) {
            // the k-block's own zero-point: entry kbu * ZPL / 4 of the lane's
            constexpr int zi = kbu * ZPL / 4;
            ExactParams pk = prm[t];
            const float zk = f16_to_f32((uint16_t)((cz[t][zi >> 1] >> (16 * (zi & 1))) & 0xFFFFu));
            pk.sz = pk.s * zk;
            pk.nz_h = h2s(-zk);
            bf[t] = product_frag<BITS, DT, ZFINE, kb, COPIES, SPLIT4>(cw[t], pk, tab, dk);
          } else {
            bf[t] = product_frag<BITS, DT, MODE, kb, COPIES, SPLIT4>(cw[t], prm[t], tab, dk);
          }
        }
      }
      u32x4 n0 = f0, n1 = f1;
      if constexpr (!LOOKAHEAD) {
        f0 = a_frag(As, kbu, 2 * ip);
        f1 = a_frag(As, kbu, 2 * ip + 1);
      } else {
        if constexpr (step + 1 < STEPS) {
          constexpr int nk = (step + 1) / PAIRS, ni = 2 * ((step + 1) % PAIRS);
          n0 = a_frag(As, nk, ni);
          n1 = a_frag(As, nk, ni + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[2 * ip][t] = mfma16<DT>(bf[t], f0, acc[2 * ip][t]);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[2 * ip + 1][t] = mfma16<DT>(bf[t], f1, acc[2 * ip + 1][t]);
      f0 = n0;
      f1 = n1;
    });
  };

  // Pipeline: weights are loaded two tiles ahead (two register sets, the
  // tile loop unrolled by two), activations one 128-row unit ahead into the
  // other LDS stage.  In each unit the activation loads are issued before the
  // weight loads, so the unit can end by waiting only until the activation
  // loads are done (at most NBL newer operations outstanding) while the next
  // weights keep streaming.  The compiler's wait tracking does not see the
  // LDS-destination loads, hence the explicit waits; a scheduling barrier
  // keeps the two groups of loads in program order.
  const int uend = kt1 * UPT;  // first unit past this workgroup's range
  BSet set0, set1;
  a_issue(kt0 * UPT, As0);
  b_load(set0, kt0);
  b_load(set1, kt0 + 1);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  auto tile = [&](int kt, BSet& cur) {
    BSet use = cur;  // copied out before this set is reloaded
    sfor<UPT>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int unit = kt * UPT + u;
      // the stage of a unit alternates; with UPT = 2 it follows u, else kt
      const bool odd = UPT == 2 ? (u == 1) : ((kt - kt0) & 1);
      if (unit + 1 < uend) a_issue(unit + 1, odd ? As0 : As1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (u == 0) b_load(cur, kt + 2);
      compute_unit(odd ? As1 : As0, use.w, use.s[u], use.z[u], uc);
      if (unit + 1 < uend) {
        // u == 0: the weight loads issued after the activation loads may stay
        // in flight; later units have no newer loads
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(u == 0 ? NBL : 0));
        __syncthreads();
      }
    });
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    tile(kt, set0);
    if (kt + 1 < kt1) tile(kt + 1, set1);
  }

  // ---- epilogue.  The MFMAs take the weights as the A operand and the
  //      activations as B, so they produce y transposed: lane (c, h) holds
  //      row m0 + 16 i + c, columns 4h .. 4h + 3 of column tile t -- four
  //      consecutive outputs, one 8-byte store.
  auto col_scales = [&](int t, float (&s)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) s[e] = 1.0f;
    if constexpr (EPI_SCALE) {  // one scale record per column tile
      typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
      const u16x4 sv = *(const u16x4*)(a.S + (size_t)(nt0 + t) * 16 + 4 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = f16_to_f32(sv[e]);
    }
  };
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if (a.ksplit > 1) {
    // Split K: this workgroup's fp32 partial sums (scaled when the scale sits
    // in the epilogue) go to its slice of the workspace; the reduction kernel
    // adds the slices in split order and applies the output stage.
    float* dst = a.part + (size_t)ks * a.M * a.N;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (nt0 + t >= a.ntiles) continue;
      const int n = (nt0 + t) * 16 + 4 * h;
      float s[4];
      col_scales(t, s);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + c;
        if (m < a.M)
          *(f4*)(dst + (size_t)m * a.N + n) =
              f4{acc[i][t][0] * s[0], acc[i][t][1] * s[1], acc[i][t][2] * s[2], acc[i][t][3] * s[3]};
      }
    }
    return;
  }
  if (a.swiglu) {
    // Fused gate+up layer: column tiles are interleaved (gate, up, ...), so
    // tiles 2p and 2p + 1 of the wave are the gate and up halves of output
    // tile nt0 / 2 + p (nt0 is a multiple of 4 and the tile count even).
#pragma unroll
    for (int p = 0; p < NT / 2; ++p) {
      if (nt0 + 2 * p >= a.ntiles) continue;
      float sg[4], su[4];
      col_scales(2 * p, sg);
      col_scales(2 * p + 1, su);
      const int n = (nt0 / 2 + p) * 16 + 4 * h;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int m = m0 + 16 * i + c;
        if (m < a.M) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = acc[i][2 * p][e] * sg[e];
            v[e] = g / (1.0f + expf(-g)) * (acc[i][2 * p + 1][e] * su[e]);
          }
          *(u32x2*)(a.y + (size_t)m * (a.N / 2) + n) = u32x2{pack2<DT>(v[0], v[1]), pack2<DT>(v[2], v[3])};
        }
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (nt0 + t >= a.ntiles) continue;
    const int n = (nt0 + t) * 16 + 4 * h;
    float s[4];
    col_scales(t, s);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int m = m0 + 16 * i + c;
      if (m < a.M) {
        const uint32_t lo = pack2<DT>(acc[i][t][0] * s[0], acc[i][t][1] * s[1]);
        const uint32_t hi = pack2<DT>(acc[i][t][2] * s[2], acc[i][t][3] * s[3]);
        *(u32x2*)(a.y + (size_t)m * a.N + n) = u32x2{lo, hi};
      }
    }
  }
}

// Sum of the K-split partial products, rounded once to the activation dtype
// (y [M][N]), or, for a fused gate+up layer, SiLU(gate) * up of the summed
// halves (y [M][N/2]; partial columns in the interleaved tile order).  Each
// group of 4 consecutive outputs has `rows` threads (1, 2, 4 or 8, more when
// there are few outputs): thread row r sums slices r, r + rows, ... (all its
// loads independent, so in flight together), then row 0 adds the row sums in
// order: a fixed summation order for a given shape.
template <int DT>
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(const float* __restrict__ part, int ksplit, int M, int N,
                                                            int swiglu, int rows, uint16_t* __restrict__ y) {
  __shared__ f4 red_g[256], red_u[256];
  const int ldy = swiglu ? N / 2 : N;
  const size_t quads = (size_t)M * ldy / 4;
  const int qw = 256 / rows;  // groups of 4 outputs per workgroup
  const int ql = threadIdx.x % qw, row = threadIdx.x / qw;
  const size_t q = (size_t)blockIdx.x * qw + ql;
  const size_t slice = (size_t)M * N;
  f4 g = {0.0f, 0.0f, 0.0f, 0.0f}, u = g;
  int m = 0, j = 0;
  if (q < quads) {
    m = (int)(q * 4 / ldy);
    j = (int)(q * 4 % ldy);  // first of 4 outputs (ldy % 16 == 0)
    const int col = swiglu ? (j / 16) * 32 + j % 16 : j;  // gate column; up is 16 further
    const float* p = part + (size_t)m * N + col;
    for (int k = row; k < ksplit; k += rows) {
      g += *(const f4*)(p + k * slice);
      if (swiglu) u += *(const f4*)(p + k * slice + 16);
    }
  }
  if (rows > 1) {
    red_g[threadIdx.x] = g;
    red_u[threadIdx.x] = u;
    __syncthreads();
    if (row != 0) return;
    for (int r = 1; r < rows; ++r) {
      g += red_g[r * qw + ql];
      u += red_u[r * qw + ql];
    }
  }
  if (q >= quads) return;
  if (swiglu) {
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] = g[e] / (1.0f + expf(-g[e])) * u[e];
  }
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  *(u32x2*)(y + (size_t)m * ldy + j) = u32x2{pack2<DT>(g[0], g[1]), pack2<DT>(g[2], g[3])};
}

template <int DT, int BITS, int MODE, int GPU, bool EPI>
wq_status run_gemm(GemmArgs g, hipStream_t s) {
  // Workgroup tile.  Each wave covers all BM rows of its columns, so a weight
  // is decoded once per BM rows; the accumulators (BM x 64 / 64 per lane at
  // four column tiles) and the weight registers must fit 256 per lane for
  // two workgroups per CU.
  //  * 128 x 256 (four column tiles per wave) for the decodes that fit it --
  //    symmetric 3- and 4-bit codes (4-bit with at most two groups per 128
  //    rows), fp16 zero-points with one group per 128 rows, 3-bit integer
  //    zero-points with one group per 128 rows, 3-bit tables -- when K is not
  //    split and the grid holds at least about two workgroups per CU.
  //    Measured gains at M = 2048-4096: 7-31 % on fp16 zero-points and 3-bit
  //    tables; 128 x 128 loses 0-11 % to it there.
  //  * otherwise above M = 64, 128 x 128 (two column tiles per wave): half
  //    the decode work of 64 x 256 per output for as many workgroups, with or
  //    without a K split.  The decodes that spill at 128 x 256 (more groups or
  //    zero-point records per tile, 2-bit codes, fine zero-points, 4-bit
  //    tables) always take it there.  Measured 5-40 % faster than 64 x 256
  //    at M = 80-4096 (the 16384 x 53248 bf16 packed-zero layer at M = 128:
  //    390 -> 279 us; 4096-column layers at M = 2048: 7-23 %; 4-bit tables,
  //    with their table in 16 columns, 10-25 %).  Not taken when the rows
  //    fill an odd number of 64-row blocks below 7 (M = 192: a padded half
  //    tile and a third more workgroups, 10 % slower), nor for the cheapest
  //    decode (fp16 symmetric codes, scale in the epilogue) when 64 x 256
  //    tiles more than fill two workgroups per CU: there the doubled LDS
  //    reads of the activations cost more than the decode saves (3-8 %
  //    slower at 768 and more workgroups; 7 % faster at 512).
  //  * 64 x 256 otherwise (M <= 64 among them), except for the one decode
  //    below that spills there.
  // The K split (chosen by the host for 64 x 256 workgroups) keeps its slice
  // count whichever tile runs.
  constexpr bool FIT128 = (MODE == SYM && BITS != 2 && (BITS == 3 || GPU <= 2)) ||
                          (MODE == ZERO_F16 && BITS != 2 && GPU == 1) ||
                          (MODE == ZERO_PACKED && BITS == 3 && GPU == 1) ||
                          (MODE == LUT && BITS == 3);
  // 2-bit codes with packed zero-points in groups of 32 rows spill even at
  // 64 x 256 (four zero-point words per column tile and unit): 128 x 128 at
  // every M, 25-90 % faster at M = 8-192 despite the padded rows.
  constexpr bool NO64 = MODE == ZERO_PACKED && BITS == 2 && GPU == 4;
  const int blocks64 = (g.M + 63) / 64;
  int bm = 64, nt = 4;
  if (FIT128 && g.ksplit == 1 && g.M > 64 && (long)((g.M + 127) / 128) * ((g.N + 255) / 256) >= 480) {
    bm = 128;
  } else if (NO64) {
    bm = 128;
    nt = 2;
  } else if (g.M > 64 && (blocks64 % 2 == 0 || blocks64 >= 7) &&
             !(EPI && (long)blocks64 * ((g.N + 255) / 256) * g.ksplit > 512)) {
    bm = 128;
    nt = 2;
  }
  g.ntiles_wg = (g.N + 64 * nt - 1) / (64 * nt);
  g.mtiles = (g.M + bm - 1) / bm;
  g.ktps = (g.ktiles + g.ksplit - 1) / g.ksplit;
  const int grid = g.mtiles * g.ntiles_wg * g.ksplit;
  if (bm == 64) {
    if constexpr (!NO64)
      hipLaunchKernelGGL((gemm_kernel<DT, BITS, MODE, GPU, EPI, 64, 4>), dim3(grid), dim3(256), 0, s, g);
  } else if (nt == 2) {
    hipLaunchKernelGGL((gemm_kernel<DT, BITS, MODE, GPU, EPI, 128, 2>), dim3(grid), dim3(256), 0, s, g);
  } else {
    if constexpr (FIT128)
      hipLaunchKernelGGL((gemm_kernel<DT, BITS, MODE, GPU, EPI, 128, 4>), dim3(grid), dim3(256), 0, s, g);
  }
  if (g.ksplit > 1) {
    const size_t quads = (size_t)g.M * (g.swiglu ? g.N / 2 : g.N) / 4;
    int rows = 1;  // threads per group of 4 outputs: about 2^18 threads in all
    while (rows < 8 && rows < g.ksplit && quads * rows < ((size_t)1 << 18)) rows *= 2;
    const size_t qw = 256 / rows;
    hipLaunchKernelGGL((ksplit_reduce_kernel<DT>), dim3((unsigned)((quads + qw - 1) / qw)), dim3(256), 0, s,
                       (const float*)g.part, g.ksplit, g.M, g.N, g.swiglu, rows, g.y);
  }
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
  g.swiglu = p.swiglu;
  g.ksplit = p.ksplit;
  g.part = (float*)p.part;
  g.ktps = L.ktiles;
  const int gpu = L.gsz >= 128 ? 1 : 128 / L.gsz;
  const bool epi = L.G == 1 && p.mode == SYM && D == F16;
  wq_status st = WQ_EINVAL;
  sfor<7>([&](auto mi) {  // the ABI mode itself: fine zero-points keep their group
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
