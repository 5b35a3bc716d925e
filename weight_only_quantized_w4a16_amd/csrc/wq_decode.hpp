// wq_decode.hpp -- in-register decoding of packed codes into MFMA B operands.
//
// Codes are turned into 16-bit floats in registers and fed straight to the
// matrix cores; nothing is written back (Triton GPTQ page, "How It Works";
// exllama bandwidth discussion, GPTQ paper quote).  Three decoders:
//
//  * offset decode (uniform modes): OR-ing a code into the mantissa of a float
//    whose exponent makes the unit in the last place 1 yields (bias + q)
//    exactly.  The biased form keeps that value (bias 1024 for fp16, 0x6400;
//    128 for bf16, 0x4300) and the decode-sized product with fp16 activations
//    removes bias + z after the MFMA with the row sums of x.  The offset form
//    (fp16) removes the bias with one packed fp16 add or fma, giving
//    q - 2^(bits-1) exactly; the fma may also scale a field sitting 4^i
//    higher by 4^-i, which saves shifts.
//  * table decode: two codes form an index into an LDS table of value pairs
//    (FLUTE page, "How It Works": value = table entry times scale).  The
//    table is replicated 32 times so that lane l always reads bank l%32 (16
//    times where LDS is short).
//  * exact decode (the large-M product, the debug dump, and the decode-sized
//    product with bf16 activations): the dequantised weight RN(s*(q - z)) or
//    RN(s*T[q]) in the activation dtype, one rounding of a value that is
//    exact in fp32 (s has 11 significant bits, q - z at most 13 for fp16
//    zero-points in the ranges used, T[q] 11).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq_layout.hpp"

namespace wq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

// Raw buffer resources: a load whose offset lies past num_records returns zero
// without touching memory, which lets prefetches past the end of a range stay
// unconditional (straight-line code keeps the wait counters exact).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // every buffer here is smaller than 2 GiB
__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr int kNontemporal = 2;  // cache policy of the streamed weight loads

// 16 bytes per lane from a buffer straight into LDS: lane L writes
// lds[L] (the wave's 1 KiB lands contiguously from `lds`, which must be
// wave-uniform).  A separate device function keeps the LDS address-space cast
// out of kernel bodies, which the host compilation pass must still accept.
__device__ inline void buffer_load_lds16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

__device__ inline uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ inline h2 h2s(float a) { return h2{(_Float16)a, (_Float16)a}; }

__device__ inline float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ inline uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
__device__ inline uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Round a pair of fp32 values to the activation dtype with
// round-to-nearest-even; lo in bits 0..15 (one v_cvt_pk_{f16,bf16}_f32).
template <int DT>
__device__ inline uint32_t pack2(float lo, float hi) {
  if constexpr (DT == F16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, h2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2){lo, hi}, bf2));
  }
}

template <int DT>
__device__ inline f4 mfma16(u32x4 a, u32x4 b, f4 c) {
  if constexpr (DT == F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8, a), __builtin_bit_cast(bf8, b), c, 0, 0, 0);
}

// 1.0 in every element: B operand that turns an MFMA into row sums of A.
template <int DT>
__device__ inline u32x4 ones_frag() {
  const uint32_t one = DT == F16 ? 0x3C003C00u : 0x3F803F80u;
  return u32x4{one, one, one, one};
}

constexpr uint32_t kMagicF16 = 0x64006400u;   // fp16 1024 in both halves
constexpr uint32_t kMagicBF16 = 0x43004300u;  // bf16 128 in both halves

// Operands of the offset decode, held in registers the compiler cannot see
// through.  gfx9 VOP3 encodings take no literal constants and at most one
// scalar operand; with the masks in scalar registers and the exponent pattern
// in a vector register, (w & mask) | magic becomes one v_and_or_b32 instead
// of an AND and an OR.  Built once per kernel (the empty asm emits nothing).
struct DecodeConsts {
  uint32_t m4lo, m4hi;  // 0x000F000F, 0x00F000F0
  uint32_t m2[5];       // 0x00030003 << 2i
  uint32_t magic;       // kMagicF16 or kMagicBF16
  uint32_t magic_h;     // kMagicF16 (exact bf16 decode: fp16 halves widened by v_fma_mix)
  float nzero;          // -0.0f, an addend the compiler cannot fold away
};

template <int DT>
__device__ inline DecodeConsts make_decode_consts() {
  DecodeConsts k;
  k.m4lo = 0x000F000Fu;
  k.m4hi = 0x00F000F0u;
#pragma unroll
  for (int i = 0; i < 5; ++i) k.m2[i] = 0x00030003u << (2 * i);
  k.magic = DT == F16 ? kMagicF16 : kMagicBF16;
  k.magic_h = kMagicF16;
  k.nzero = -0.0f;
  asm volatile("" : "+s"(k.m4lo));
  asm volatile("" : "+s"(k.m4hi));
#pragma unroll
  for (int i = 0; i < 5; ++i) asm volatile("" : "+s"(k.m2[i]));
  asm volatile("" : "+v"(k.magic));
  if constexpr (DT == BF16) {
    asm volatile("" : "+v"(k.magic_h));
    asm volatile("" : "+v"(k.nzero));
  }
  return k;
}

// ---------------------------------------------------------------------------
// Field extraction for the 3-bit layout: pair p (0..15) of a tile lane.
// ---------------------------------------------------------------------------
template <int P>
__device__ inline uint32_t pair6(const uint32_t* w) {
  if constexpr (P < 15) {
    return (w[P / 5] >> (6 * (P % 5))) & 0x3Fu;
  } else {
    return (w[0] >> 30) | ((w[1] >> 30) << 2) | ((w[2] >> 30) << 4);
  }
}

// ---------------------------------------------------------------------------
// Register tables of 2- and 3-bit table codes.  The 4 or 8 values of a table
// (the layer's T[q], or the dequantised RN(s * T[q]) of one group and column)
// are held as two byte planes: L[i] holds the low bytes and H[i] the high
// bytes of entries 4i .. 4i + 3.  One v_perm_b32 then looks up the low (or
// high) bytes of four codes at once (its selector bytes 0..7 pick bytes of
// {L[1], L[0]}), and two more interleave them into the two value pairs an MFMA
// operand register holds -- no LDS table, no per-pair index arithmetic.  The
// code layout of these modes keeps four codes byte-aligned (wq_layout.hpp).
// ---------------------------------------------------------------------------
struct RegTable {
  uint32_t L[2], H[2];
};

// From 16-bit values packed in pairs P[j] = v[2j] | v[2j+1] << 16.
template <int BITS>
__device__ inline RegTable reg_table(const uint32_t* P) {
  RegTable t;
  t.L[0] = __builtin_amdgcn_perm(P[1], P[0], 0x06040200u);
  t.H[0] = __builtin_amdgcn_perm(P[1], P[0], 0x07050301u);
  if constexpr (BITS == 3) {
    t.L[1] = __builtin_amdgcn_perm(P[3], P[2], 0x06040200u);
    t.H[1] = __builtin_amdgcn_perm(P[3], P[2], 0x07050301u);
  } else {
    t.L[1] = t.L[0];
    t.H[1] = t.H[0];
  }
  return t;
}

// Four codes of a 2- or 3-bit table layout, one per byte: elements
// 4 HALF .. 4 HALF + 3 of k-block KB (see wq_layout.hpp).
template <int BITS, int KB, int HALF>
__device__ inline uint32_t table_codes4(const uint32_t* w) {
  if constexpr (BITS == 2) {
    return (w[KB / 2] >> (2 * (2 * (KB % 2) + HALF))) & 0x03030303u;
  } else {
    constexpr int x = 2 * KB + HALF;
    if constexpr (x < 6) return (w[x / 2] >> (3 * (x % 2))) & 0x07070707u;
    else if constexpr (x == 6) return ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u);
    else return ((w[1] >> 6) & 0x03030303u) | ((w[2] >> 5) & 0x04040404u);
  }
}

// B operand of k-block KB from a register table: pair q = elements (2q, 2q+1).
template <int BITS, int KB>
__device__ inline u32x4 perm_table_frag(const uint32_t* w, const RegTable& t) {
  u32x4 r;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint32_t x = half == 0 ? table_codes4<BITS, KB, 0>(w) : table_codes4<BITS, KB, 1>(w);
    const uint32_t lo = __builtin_amdgcn_perm(t.L[1], t.L[0], x);
    const uint32_t hi = __builtin_amdgcn_perm(t.H[1], t.H[0], x);
    r[2 * half] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);      // elements 4 half, 4 half + 1
    r[2 * half + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // elements 4 half + 2, + 3
  }
  return r;
}

// Table values as pairs Tp[j] = T[2j] | T[2j+1] << 16 from lanes 0 .. 2^BITS - 1
// holding T[lane] in their low 16 bits (every lane of the wave active).
template <int BITS>
__device__ inline void table_pairs_from_lanes(uint32_t tval, uint32_t* Tp) {
#pragma unroll
  for (int j = 0; j < (1 << BITS) / 2; ++j)
    Tp[j] = ((uint32_t)__shfl((int)tval, 2 * j) & 0xFFFFu) | ((uint32_t)__shfl((int)tval, 2 * j + 1) << 16);
}

// ---------------------------------------------------------------------------
// Offset decode: B operand (8 values of one k-block) for uniform modes.
//   fp16: values are q - 2^(BITS-1)  (exact small integers)
//   bf16: values are 128 + q         (exact; caller subtracts 128 + z later)
// ---------------------------------------------------------------------------
template <int BITS, int DT, int KB>
__device__ inline u32x4 offset_frag(const uint32_t* w, const DecodeConsts& k) {
  u32x4 r;
  if constexpr (BITS == 4) {
    const uint32_t x = w[KB];
    if constexpr (DT == F16) {
      const float off = 1024.0f + 8.0f;
      const uint32_t x8 = x >> 8;
      r[0] = as_u32(as_h2((x & k.m4lo) | k.magic) - h2s(off));
      r[1] = as_u32(__builtin_elementwise_fma(as_h2((x & k.m4hi) | k.magic), h2s(1.0f / 16), h2s(-(64.0f + 8.0f))));
      r[2] = as_u32(as_h2((x8 & k.m4lo) | k.magic) - h2s(off));
      r[3] = as_u32(__builtin_elementwise_fma(as_h2((x8 & k.m4hi) | k.magic), h2s(1.0f / 16), h2s(-(64.0f + 8.0f))));
    } else {
      r[0] = (x & k.m4lo) | k.magic;
      r[1] = ((x >> 4) & k.m4lo) | k.magic;
      r[2] = ((x >> 8) & k.m4lo) | k.magic;
      r[3] = ((x >> 12) & k.m4lo) | k.magic;
    }
  } else if constexpr (BITS == 2) {
    const uint32_t x = w[KB / 2];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = 4 * (KB % 2) + q;  // pair index inside the word
      if constexpr (DT == F16) {
        const int ii = i < 5 ? i : i - 5;
        const uint32_t xs = i < 5 ? x : (x >> 10);
        const float sc = 1.0f / (float)(1 << (2 * ii));
        r[q] = as_u32(__builtin_elementwise_fma(as_h2((xs & k.m2[ii]) | k.magic), h2s(sc),
                                                h2s(-(1024.0f * sc + 2.0f))));
      } else {
        r[q] = ((x >> (2 * i)) & k.m2[0]) | k.magic;
      }
    }
  } else {  // BITS == 3
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t f;
      switch (4 * KB + q) {
        case 0: f = pair6<0>(w); break;   case 1: f = pair6<1>(w); break;
        case 2: f = pair6<2>(w); break;   case 3: f = pair6<3>(w); break;
        case 4: f = pair6<4>(w); break;   case 5: f = pair6<5>(w); break;
        case 6: f = pair6<6>(w); break;   case 7: f = pair6<7>(w); break;
        case 8: f = pair6<8>(w); break;   case 9: f = pair6<9>(w); break;
        case 10: f = pair6<10>(w); break; case 11: f = pair6<11>(w); break;
        case 12: f = pair6<12>(w); break; case 13: f = pair6<13>(w); break;
        case 14: f = pair6<14>(w); break; default: f = pair6<15>(w); break;
      }
      const uint32_t v = (f & 7u) | ((f & 0x38u) << 13);
      if constexpr (DT == F16)
        r[q] = as_u32(as_h2(v | k.magic) - h2s(1024.0f + 4.0f));
      else
        r[q] = v | k.magic;
    }
  }
  return r;
}

// ---------------------------------------------------------------------------
// Biased decode (decode-sized product): B = bias + q exactly for either dtype
// (bias 1024 for fp16, 128 for bf16), one shift and one AND-OR per register
// and no float arithmetic; the caller removes bias + z with the row sums of x.
// ---------------------------------------------------------------------------
// `magic` is k.magic (the activation dtype's bias) unless given.
template <int BITS, int KB>
__device__ inline u32x4 biased_frag(const uint32_t* w, const DecodeConsts& k, uint32_t magic) {
  u32x4 r;
  if constexpr (BITS == 4) {
    const uint32_t x = w[KB];
    r[0] = (x & k.m4lo) | magic;
    r[1] = ((x >> 4) & k.m4lo) | magic;
    r[2] = ((x >> 8) & k.m4lo) | magic;
    r[3] = ((x >> 12) & k.m4lo) | magic;
  } else if constexpr (BITS == 2) {
    const uint32_t x = w[KB / 2];
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = ((x >> (2 * (4 * (KB % 2) + q))) & k.m2[0]) | magic;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t f;
      switch (4 * KB + q) {
        case 0: f = pair6<0>(w); break;   case 1: f = pair6<1>(w); break;
        case 2: f = pair6<2>(w); break;   case 3: f = pair6<3>(w); break;
        case 4: f = pair6<4>(w); break;   case 5: f = pair6<5>(w); break;
        case 6: f = pair6<6>(w); break;   case 7: f = pair6<7>(w); break;
        case 8: f = pair6<8>(w); break;   case 9: f = pair6<9>(w); break;
        case 10: f = pair6<10>(w); break; case 11: f = pair6<11>(w); break;
        case 12: f = pair6<12>(w); break; case 13: f = pair6<13>(w); break;
        case 14: f = pair6<14>(w); break; default: f = pair6<15>(w); break;
      }
      r[q] = (f & 7u) | ((f & 0x38u) << 13) | magic;
    }
  }
  return r;
}
template <int BITS, int KB>
__device__ inline u32x4 biased_frag(const uint32_t* w, const DecodeConsts& k) {
  return biased_frag<BITS, KB>(w, k, k.magic);
}

// 4-bit codes as fp16 pairs with one shift per word: pairs 0 and 2 are
// 1024 + q (nibbles at bits 0-3 / 16-19 of x and of x >> 8), pairs 1 and 3
// are 1024 + 16 q (nibbles at bits 4-7 / 20-23 masked in place), both exact.
template <int KB>
__device__ inline u32x4 split4_frag(const uint32_t* w, const DecodeConsts& k) {
  const uint32_t x = w[KB], x8 = x >> 8;
  return u32x4{(x & k.m4lo) | k.magic_h, (x & k.m4hi) | k.magic_h, (x8 & k.m4lo) | k.magic_h,
               (x8 & k.m4hi) | k.magic_h};
}

// Fine zero-points, scale applied later: B operand RN_dt(q - z) for k-block KB,
// whose eight rows share one zero-point z (fp16 bits zbits).
//   fp16: (1024 + q) - 1024 is exact, one packed add of -z rounds once;
//   bf16: (128 + q) widened to fp32, minus (128 + z) (exact: both fit 24
//         bits), one rounding to bf16.
template <int BITS, int DT, int KB>
__device__ inline u32x4 fine_frag(const uint32_t* w, uint32_t zbits, const DecodeConsts& k) {
  const u32x4 o = biased_frag<BITS, KB>(w, k);
  u32x4 r;
  if constexpr (DT == F16) {
    const _Float16 z = __builtin_bit_cast(_Float16, (uint16_t)zbits);
    const h2 nz = h2{-z, -z};
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = as_u32((as_h2(o[q]) + h2s(-1024.0f)) + nz);
  } else {
    const float cz = 128.0f + f16_to_f32((uint16_t)zbits);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r[q] = pack2<BF16>(__uint_as_float(o[q] << 16) - cz, __uint_as_float(o[q] & 0xFFFF0000u) - cz);
  }
  return r;
}

// fp16 bits of the zero-point of k-block kbu (0..3) from a fine zero record
// (two words, four fp16 values, k-block order).
__device__ inline uint32_t fine_zero_bits(const uint32_t* zr, int kbu) {
  return (zr[kbu >> 1] >> (16 * (kbu & 1))) & 0xFFFFu;
}

// ---------------------------------------------------------------------------
// Table decode: B operand from an LDS pair table.  tab points at the table's
// column for this lane (base + lane % COPIES); entry idx sits at
// tab[idx * COPIES].
// ---------------------------------------------------------------------------
template <int BITS, int KB, int COPIES = 32>
__device__ inline u32x4 table_frag(const uint32_t* w, const uint32_t* tab) {
  static_assert(BITS == 4, "2- and 3-bit table codes use register tables");
  u32x4 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t idx;
    if constexpr (BITS == 4) {
      idx = (w[KB] >> (8 * q)) & 0xFFu;
    } else if constexpr (BITS == 2) {
      idx = (w[KB / 2] >> (4 * (4 * (KB % 2) + q))) & 0xFu;
    } else {
      switch (4 * KB + q) {
        case 0: idx = pair6<0>(w); break;   case 1: idx = pair6<1>(w); break;
        case 2: idx = pair6<2>(w); break;   case 3: idx = pair6<3>(w); break;
        case 4: idx = pair6<4>(w); break;   case 5: idx = pair6<5>(w); break;
        case 6: idx = pair6<6>(w); break;   case 7: idx = pair6<7>(w); break;
        case 8: idx = pair6<8>(w); break;   case 9: idx = pair6<9>(w); break;
        case 10: idx = pair6<10>(w); break; case 11: idx = pair6<11>(w); break;
        case 12: idx = pair6<12>(w); break; case 13: idx = pair6<13>(w); break;
        case 14: idx = pair6<14>(w); break; default: idx = pair6<15>(w); break;
      }
    }
    r[q] = tab[idx * COPIES];
  }
  return r;
}

// Fill an LDS pair table: entry idx = value[lo] | value[hi] << 16 with
// lo = idx & (2^BITS - 1), hi = idx >> BITS, replicated over COPIES columns.
// AS_BF16: store RN_bf16(T) instead of the fp16 T.  Each thread writes 16
// bytes (four copies of one entry) per step; consecutive threads write
// consecutive 16-byte chunks, so the writes of a wave hit every bank once.
// `table` must be 16-byte aligned.
template <int BITS, bool AS_BF16, int COPIES = 32>
__device__ inline void fill_pair_table(uint32_t* table, const uint16_t* lut, int tid, int nthreads) {
  static_assert(COPIES % 4 == 0, "copies come in 16-byte chunks");
  constexpr int n = 1 << (2 * BITS);
  constexpr int mask = (1 << BITS) - 1;
  constexpr int CPE = COPIES / 4;  // chunks per entry
  for (int i = tid; i < n * CPE; i += nthreads) {
    const int idx = i / CPE;
    uint16_t lo = lut[idx & mask], hi = lut[idx >> BITS];
    if (AS_BF16) {
      lo = f32_to_bf16(f16_to_f32(lo));
      hi = f32_to_bf16(f16_to_f32(hi));
    }
    const uint32_t v = (uint32_t)lo | ((uint32_t)hi << 16);
    *(u32x4*)(table + 4 * i) = u32x4{v, v, v, v};
  }
}

// The same table from values already in registers: lane i (< 2^BITS) of
// every wave holds T[i] in the low 16 bits of tval (one load per lane, issued
// before anything else, so its latency overlaps the first weight loads); the
// pairs are gathered with cross-lane shuffles.  Every lane of the workgroup
// calls this; `table` must be 16-byte aligned.
template <int BITS, int COPIES = 32>
__device__ inline void fill_pair_table_lanes(uint32_t* table, uint32_t tval, int tid, int nthreads) {
  static_assert(COPIES % 4 == 0, "copies come in 16-byte chunks");
  constexpr int n = 1 << (2 * BITS);
  constexpr int mask = (1 << BITS) - 1;
  constexpr int CPE = COPIES / 4;  // chunks per entry
  for (int base = 0; base < n * CPE; base += nthreads) {
    const int i = base + tid;
    const int idx = (i / CPE) & (n - 1);
    // shuffles with every lane active (the source lanes 0 .. 2^BITS - 1 always are)
    const uint32_t lo = (uint32_t)__shfl((int)tval, idx & mask), hi = (uint32_t)__shfl((int)tval, idx >> BITS);
    const uint32_t v = (lo & 0xFFFFu) | (hi << 16);
    if (i < n * CPE) *(u32x4*)(table + 4 * i) = u32x4{v, v, v, v};
  }
}

// Zero-point / table parameters of one (group, column) for the exact path.
struct ExactParams {
  float s;        // scale
  float sz;       // s * z (exact in fp32)
  h2 s_h;         // scale as an fp16 pair (fp16 fast paths)
  h2 nz_h;        // fp16 product path: -z (fp16 zero-points) or -(1024 + z) (integer zero-points)
  RegTable rt;    // 2- and 3-bit table codes: the dequantised RN(s * T[q]) (scaled_reg_table)
};

// The dequantised values RN_dt(s * T[q]) of one (group, column) as a register
// table, from the table pairs Tp: fp16 one packed product per pair (exact
// product rounded once); bf16 the product in fp32 (exact) rounded once.
template <int BITS, int DT>
__device__ inline RegTable scaled_reg_table(const uint32_t* Tp, float s, const DecodeConsts& k) {
  uint32_t P[(1 << BITS) / 2];
#pragma unroll
  for (int j = 0; j < (1 << BITS) / 2; ++j) {
    const h2 v = as_h2(Tp[j]);
    if constexpr (DT == F16)
      P[j] = as_u32(v * h2s(s));
    else
      P[j] = pack2<DT>(__builtin_fmaf((float)v[0], s, k.nzero), __builtin_fmaf((float)v[1], s, k.nzero));
  }
  return reg_table<BITS>(P);
}

// Exact dequantised B operand for k-block KB: RN_dt(s*(q - z)) or RN_dt(s*T[q]).
// tab: LDS fp16 pair table column for this lane (table mode only).
template <int BITS, int DT, int MODE, int KB, int COPIES = 32, bool SPLIT4 = true>
__device__ inline u32x4 exact_frag(const uint32_t* w, const ExactParams& p, const uint32_t* tab,
                                   const DecodeConsts& k) {
  u32x4 r;
  if constexpr (MODE == LUT && BITS < 4) {
    return perm_table_frag<BITS, KB>(w, p.rt);
  } else if constexpr (MODE == SYM && DT == F16) {
    // q - 2^(b-1) is exact in fp16; one fp16 multiply rounds s*(q-z) once.
    const u32x4 o = offset_frag<BITS, F16, KB>(w, k);
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = as_u32(as_h2(o[q]) * p.s_h);
  } else if constexpr (MODE == LUT && DT == F16) {
    const u32x4 t = table_frag<BITS, KB, COPIES>(w, tab);
#pragma unroll
    for (int q = 0; q < 4; ++q) r[q] = as_u32(as_h2(t[q]) * p.s_h);
  } else if constexpr (MODE == LUT) {
    // fp16 table values widened inside v_fma_mix: s * T exact in fp32 (adding
    // -0 keeps the product's sign), one rounding to bf16
    const u32x4 t = table_frag<BITS, KB, COPIES>(w, tab);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const h2 v = as_h2(t[q]);
      r[q] = pack2<DT>(__builtin_fmaf((float)v[0], p.s, k.nzero), __builtin_fmaf((float)v[1], p.s, k.nzero));
    }
  } else {
    // (bf16 activations, and fp16 activations with stored zero-points.)
    // Codes decoded as fp16 (1024 + q) pairs, widened inside v_fma_mix:
    //   integer zero-points: s * (1024 + q) - s * (1024 + z) = s * (q - z),
    //     every term exact in fp32 (at most 22 significant bits);
    //   fp16 zero-points: s * (1024 + q) - 1024 s = s * q exactly, then
    //     minus s * z (exact) rounds once to the exact s * (q - z);
    // then one rounding to bf16.
    constexpr bool INT_Z = MODE == SYM || MODE == ZERO_PACKED;
    const float c = INT_Z ? -__builtin_fmaf(1024.0f, p.s, p.sz) : -1024.0f * p.s;
    if constexpr (SPLIT4 && BITS == 4 && INT_Z) {
      // odd pairs hold 1024 + 16 q: (1024 + 16 q) * (s / 16) - s * (64 + z),
      // every term exact as above
      const u32x4 o = split4_frag<KB>(w, k);
      const float s16 = p.s * 0.0625f, c16 = -__builtin_fmaf(64.0f, p.s, p.sz);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const h2 v = as_h2(o[q]);
        const float sq = (q & 1) ? s16 : p.s, cq = (q & 1) ? c16 : c;
        r[q] = pack2<DT>(__builtin_fmaf((float)v[0], sq, cq), __builtin_fmaf((float)v[1], sq, cq));
      }
      return r;
    }
    const u32x4 o = biased_frag<BITS, KB>(w, k, k.magic_h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const h2 v = as_h2(o[q]);
      float lo = __builtin_fmaf((float)v[0], p.s, c), hi = __builtin_fmaf((float)v[1], p.s, c);
      if constexpr (!INT_Z) {
        lo -= p.sz;
        hi -= p.sz;
      }
      r[q] = pack2<DT>(lo, hi);
    }
  }
  return r;
}

// B operand of the large-M product for k-block KB.  With fp16 activations and
// stored zero-points the subtraction and the scale run as packed fp16
// arithmetic on the biased codes (1024 + q):
//   integer zero-points: (1024 + q) - (1024 + z) is exact, then one rounding
//     of s * (q - z): exactly RN(s * (q - z));
//   fp16 zero-points: q - z is formed in fp16 (exact unless it needs more than
//     11 significant bits) and then scaled: RN(s * RN(q - z)), at most one
//     extra rounding away from RN(s * (q - z));
// every other case takes the exact decode above.
template <int BITS, int DT, int MODE, int KB, int COPIES = 32, bool SPLIT4 = true>
__device__ inline u32x4 product_frag(const uint32_t* w, const ExactParams& p, const uint32_t* tab,
                                     const DecodeConsts& k) {
  if constexpr (DT == F16 && (MODE == ZERO_F16 || MODE == ZFINE || MODE == ZERO_PACKED)) {
    const u32x4 o = biased_frag<BITS, KB>(w, k);
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h2 d = as_h2(o[q]);
      if constexpr (MODE != ZERO_PACKED) d = d + h2s(-1024.0f);
      r[q] = as_u32((d + p.nz_h) * p.s_h);
    }
    return r;
  } else {
    return exact_frag<BITS, DT, MODE, KB, COPIES, SPLIT4>(w, p, tab, k);
  }
}

// ---------------------------------------------------------------------------
// Metadata records (see wq_layout.hpp).  A record is loaded as REC bytes
// into words; accessors pick group j of the record.
// ---------------------------------------------------------------------------
template <int BYTES>
__device__ inline void load_record(rsrc_t r, uint32_t voff, uint32_t soff, uint32_t* dst) {
  if constexpr (BYTES == 2) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  } else if constexpr (BYTES == 4) {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (BYTES == 8) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    dst[0] = v[0]; dst[1] = v[1];
  } else {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
  }
}

// Scale of group j from a scale record (interleaved with fp16 zero-points when Z16).
template <bool Z16>
__device__ inline float rec_scale(const uint32_t* w, int j) {
  const uint32_t v = Z16 ? (w[j] & 0xFFFFu) : ((w[j / 2] >> (16 * (j % 2))) & 0xFFFFu);
  return f16_to_f32((uint16_t)v);
}
// fp16 zero-point of group j from an interleaved record.
__device__ inline float rec_zero16(const uint32_t* w, int j) { return f16_to_f32((uint16_t)(w[j] >> 16)); }
// Packed zero-point of group j for column c from a packed-zero record.
__device__ inline float rec_zero_packed(const uint32_t* w, int j, int c) {
  return (float)((w[j] >> (4 * (c & 7))) & 0xFu);
}

}  // namespace wq
