// wq_layout.hpp -- geometry of the gfx950 tile layout of a repacked layer.
//
// The pages only say a kernel consumes weights in its own format, produced
// offline from whatever the quantiser wrote (Marlin zero-point issue,
// efrantar's reply).  This is that format for the MFMA-based kernels here.
//
// Codes.  The weight is cut into tiles of 16 columns x KT rows (KT = 128 for
// 3- and 4-bit codes, 256 for 2-bit codes).  Tiles are stored column-tile
// major ([N/16][K/KT]), so one wave streaming down K for one column tile
// reads contiguous memory.  Inside a tile, lane l (0..63) of a wave owns
// WPL consecutive 32-bit words (WPL = 4, or 3 for 3-bit codes): one 128-bit
// (96-bit) coalesced load per lane, 1 KiB (768 B) per wave.  Lane l = 16h + c
// holds column c of the tile.  Its codes form k-blocks kb of 8 elements e, one
// k-block per MFMA: element e of k-block kb is row
//     128 (kb / 4) + 32 h + 8 (kb % 4) + e
// of the tile, so the 8 rows a lane feeds one 16x16x32 MFMA are consecutive
// and the four lanes of a column (h = 0..3) hold the four 32-row quarters of
// every 128-row unit.  A lane therefore meets exactly one scale group per unit
// for every group size from 32 rows up (quarter h lies in group h * GPU / 4 of
// the unit, GPU = groups per unit).  The MFMA pairs A and B by position inside
// its 32-long k dimension, so the activation fragments are loaded with the
// same row map.  Rows are in act-order-sorted order when a permutation is used.
//
// Element e of k-block kb inside the lane's words:
//   4-bit uniform  word kb, nibble (e%2)*4 + e/2   (pairs (e, e+1) sit in the
//                  two 16-bit halves, so one AND/OR makes two fp16 values)
//   4-bit table    word kb, nibble e               (a byte is a code pair)
//   2-bit uniform  word kb/2, bits 16*(e%2) + 2*i,  i = 4*(kb%2) + e/2
//   2-bit table    word kb/2, bits 8*(e%4) + 2*(2*(kb%2) + e/4)
//                  (elements 4j .. 4j + 3 of a k-block sit in the four bytes
//                  at one shift: one AND isolates four codes, one per byte)
//   3-bit uniform  pair p = 4*kb + e/2 is the 6-bit field lo | hi << 3
//                  (lo = even element); pairs 0..14 at bits 6*(p%5) of word
//                  p/5, pair 15 split over bits 30..31 of words 0, 1, 2.
//   3-bit table    group x = 2*kb + e/4 of four codes, byte b = e%4: groups
//                  0..5 at bits 8b + 3*(x%2) of word x/2; groups 6 and 7 keep
//                  their low two bits at bits 8b + 6 of word x - 6 and their
//                  high bit at bit 8b + x of word 2 (four codes, one per
//                  byte, from one or two shifts and masks).
//
// Scales / zero-points.  With GPU = groups per 128-row unit (1 for groups of
// 128 rows or more, else 128 / group_size) and a record per (column tile,
// unit or group, column):
//   scale records   fp16 [N/16][R][16][GPU]          R = K / max(group, 128)
//                   or, with fp16 zero-points, (scale, zero) fp16 pairs
//                   [N/16][R][16][GPU][2] (one record holds both);
//   packed zeros    uint32 [N/16][R][2][GPU]: word j of half h holds the
//                   zero-points of columns 8h..8h+7 of group j as nibbles
//                   (whatever the code width).
// Record r covers unit r when groups are smaller than 128 rows, else group r.
// Lane (c, h) reads only entry j = h * GPU / 4 of its column's record.
//
// Fine zero-points (zero groups of ZG = 8, 16 or 32 rows, apart from the
// scale groups): fp16 [N/16][K/128][16][128/ZG], entry [nt][u][c][i] the zero
// of rows 128 u + ZG i .. + ZG - 1 of column 16 nt + c.  Lane (c, h) covers
// rows 32 h .. 32 h + 31 of the unit: entries ZPL h .. ZPL h + ZPL - 1 with
// ZPL = 32 / ZG (one 8-, 4- or 2-byte load), k-block kb using entry
// ZPL h + kb * ZPL / 4.
#pragma once
#include <stddef.h>
#include <stdint.h>

#define WQ_HD __host__ __device__ constexpr

namespace wq {

// Modes of the C ABI; 4..6 are fp16 zero-points per 8 / 16 / 32 rows, which
// the kernels handle as one mode (ZFINE) with the zero group as a value.
enum { SYM = 0, ZERO_F16 = 1, ZERO_PACKED = 2, LUT = 3, ZFINE = 4, ZFINE16 = 5, ZFINE32 = 6 };
WQ_HD int fine_zero_group(int mode) { return mode == ZFINE ? 8 : mode == ZFINE16 ? 16 : mode == ZFINE32 ? 32 : 0; }
WQ_HD int kernel_mode(int mode) { return mode >= ZFINE ? ZFINE : mode; }
enum { F16 = 0, BF16 = 1 };

WQ_HD int tile_k(int bits) { return bits == 2 ? 256 : 128; }
WQ_HD int words_per_lane(int bits) { return bits == 3 ? 3 : 4; }
WQ_HD int tile_bytes(int bits) { return 256 * words_per_lane(bits); }
WQ_HD int kblocks_per_tile(int bits) { return tile_k(bits) / 32; }

WQ_HD int groups_per_unit(int gsz) { return gsz >= 128 ? 1 : 128 / gsz; }
// Row of element e of k-block kb (within its tile) for lane half h.
WQ_HD int tile_row(int kb, int h, int e) { return 128 * (kb / 4) + 32 * h + 8 * (kb % 4) + e; }
// Group inside its unit that lane half h meets (gpu = groups per unit).
WQ_HD int lane_group(int h, int gpu) { return (h * gpu) >> 2; }
// Fine zero-points: entries per column and unit, and per lane.
WQ_HD int fine_per_unit(int zg) { return 128 / zg; }
WQ_HD int fine_per_lane(int zg) { return 32 / zg; }
// Metadata record of the 128-row unit `unit` (see above).
WQ_HD int meta_record(int unit, int gsz) { return (unit * 128) / (gsz > 128 ? gsz : 128); }

struct Layout {
  int K, N, bits, group_size, mode;
  int G;        // number of groups
  int gsz;      // rows per group (K for group_size == -1)
  int gpu;      // groups per 128-row unit
  int nrec;     // metadata records per column tile
  int rec_bytes;  // scale record bytes per column: 2*gpu, or 4*gpu with fp16 zero-points
  int ktiles;   // K / tile_k
  int ntiles;   // N / 16
  size_t codes_off, codes_bytes;
  size_t scales_off, scales_bytes;
  size_t zeros_off, zeros_bytes;
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Valid only for arguments the API has already validated.
inline Layout make_layout(int K, int N, int bits, int group_size, int mode) {
  Layout L;
  L.K = K; L.N = N; L.bits = bits; L.group_size = group_size; L.mode = mode;
  L.gsz = group_size == -1 ? K : group_size;
  L.G = K / L.gsz;
  L.gpu = groups_per_unit(L.gsz);
  L.nrec = K / (L.gsz > 128 ? L.gsz : 128);
  L.rec_bytes = (mode == ZERO_F16 ? 4 : 2) * L.gpu;
  L.ktiles = K / tile_k(bits);
  L.ntiles = N / 16;
  L.codes_off = 0;
  L.codes_bytes = (size_t)L.ntiles * L.ktiles * tile_bytes(bits);
  L.scales_off = align256(L.codes_bytes);
  L.scales_bytes = (size_t)L.ntiles * L.nrec * 16 * L.rec_bytes;
  L.zeros_off = align256(L.scales_off + L.scales_bytes);
  L.zeros_bytes = mode == ZERO_PACKED ? (size_t)L.ntiles * L.nrec * 2 * L.gpu * 4 : 0;
  if (fine_zero_group(mode)) L.zeros_bytes = (size_t)L.ntiles * (K / 128) * 16 * 2 * fine_per_unit(fine_zero_group(mode));
  L.total = align256(L.zeros_off + L.zeros_bytes);
  return L;
}

}  // namespace wq
