/*
 * wq.h -- C ABI of the weight-only quantized mixed-input matrix product
 *         y = x . dequant(W)   on AMD Instinct MI355X (gfx950)
 *
 * The operation (what every entry point below serves):
 *   - x is an M x K activation matrix in fp16 or bf16; W is a K x N weight
 *     matrix stored as 2-, 3- or 4-bit codes (FLUTE page, "How It Works");
 *   - a weight is decoded on the fly, inside the product, and never written
 *     back in full precision (Triton GPTQ page, "How It Works"; exllama
 *     bandwidth discussion, GPTQ paper quote on the quantized-matrix
 *     full-precision-vector product);
 *   - uniform modes: w = s * (q - z) with one fp16 scale s per (group, column)
 *     and a zero-point z that is fixed at 2^(bits-1) (symmetric), stored in
 *     fp16, or stored as a bits-wide integer (Marlin zero-point issue, replies
 *     by efrantar and mobicham); group_size -1 means one scale per column;
 *   - table mode: w = s * T[q] with a per-layer fp16 table T of 2^bits values
 *     (FLUTE page, "How It Works" and "Highlighted Details");
 *   - act-order: the group of input row k is g_idx[k] (Triton GPTQ page,
 *     "Limitations & Caveats");
 *   - fused QKV / gate+up are the same call on weights concatenated along N
 *     (Triton GPTQ page, "How It Works").
 * The dequantised weight is defined as one round-to-nearest-even of the exact
 * s*(q-z) or s*T[q] to the activation dtype (a reading: the pages give no
 * formula); wq_dequant_debug produces exactly those bits.  The products
 * multiply those weights (with fp16 activations and one scale group per 128
 * rows the decode-sized product applies s after the MFMA, which for one-hot
 * rows of x gives the same bits), except where fp16 activations meet fp16
 * zero-points in two places -- the large-M product (shared or fine zero-points)
 * and the decode-sized product with fine zero-points and one scale group per
 * 128 rows -- which multiply RN(s*RN(q-z)): different bits only where q - z
 * needs more than 11 significant bits.
 *
 * Conventions shared by every entry point:
 *   - Pointers named *_host are host memory; every other pointer is device
 *     memory of the current HIP device.  All buffers are owned by the caller;
 *     the library allocates nothing and frees nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; results are valid once the
 *     stream has been synchronised.  Only wq_repack synchronises (offline).
 *   - Errors are returned as wq_status, never thrown.  Arguments are fully
 *     validated before anything is launched; on any error nothing is written.
 *   - Shapes: N % 16 == 0; K % 128 == 0 (K % 256 == 0 for 2-bit codes);
 *     group_size is -1 or a multiple of 32 that divides K and either divides
 *     or is a multiple of the code tile depth (128 rows; 256 for 2-bit).
 *     Other shapes return WQ_EUNSUPPORTED.  M == 0 is a valid no-op.
 *   - Matrices are row-major: x [M][K], y [M][N], scales [G][N], fp16/bf16
 *     passed as their 16-bit patterns.  G = 1 if group_size == -1 else K/group_size.
 *
 * Canonical (input) weight format, read by wq_repack only:
 *   qweight uint32 [K*bits/32][N]: column n is a little-endian bit stream along
 *     K, code k at bit offset bits*k over qweight[0][n], qweight[1][n], ...
 *     (for 4 bits: word r holds rows 8r..8r+7, row 8r+i at bits 4i..4i+3);
 *   scales fp16 [G][N];
 *   zeros  fp16 [G][N] (WQ_ZERO_F16), uint32 [G][N*bits/32] (WQ_ZERO_PACKED,
 *          row g a little-endian bit stream along N), fp16 [K/zg][N]
 *          (WQ_ZERO_F16_G8/16/32, zg = 8/16/32); NULL otherwise;
 *   g_idx  int32 [K] (act-order) or NULL.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  WQ_OK = 0,
  WQ_EINVAL = 1,        /* malformed arguments (NULL where required, bad sizes, bad mode) */
  WQ_EUNSUPPORTED = 2,  /* well-formed but outside the shapes the kernels cover */
  WQ_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
  WQ_ENOSPACE = 4       /* workspace smaller than wq_workspace_bytes() */
} wq_status;

typedef enum { WQ_F16 = 0, WQ_BF16 = 1 } wq_dtype;

typedef enum {
  WQ_SYM = 0,           /* z = 2^(bits-1) */
  WQ_ZERO_F16 = 1,      /* fp16 zero-point per (group, column) */
  WQ_ZERO_PACKED = 2,   /* bits-wide integer zero-point per (group, column) */
  WQ_LUT = 3,           /* w = s * T[q], fp16 table of 2^bits entries */
  /* fp16 zero-points with a group of their own, 8 / 16 / 32 rows, apart from
   * the scales' group_size (Marlin zero-point issue, mobicham's reply: the
   * zero-point granularity matters most at low bit widths, e.g. per-column
   * scales with a zero-point every 8 rows).  Row k of column n uses
   * zeros[k / zg][n]; zeros fp16 [K / zg][N].  Not combinable with act-order
   * (WQ_EUNSUPPORTED): the zero groups follow the original row order. */
  WQ_ZERO_F16_G8 = 4,
  WQ_ZERO_F16_G16 = 5,
  WQ_ZERO_F16_G32 = 6
} wq_qmode;

/* Version of the repacked layout; a stored repacked buffer from another
 * version must be repacked again. */
#define WQ_LAYOUT_VERSION 3
int wq_layout_version(void);

const char* wq_status_str(wq_status s);

/*
 * Size in bytes of the repacked weight buffer (codes + scales + zero-points in
 * the gfx950 tile layout).  Returns 0 for unsupported arguments.
 */
size_t wq_packed_bytes(int K, int N, int bits, int group_size, wq_qmode mode);

/*
 * Scratch memory wq_gemv / wq_gemm (and their *_gate_up forms) need for a call
 * with these sizes: the permuted copy of x when act-order is used (M*K
 * activation elements, 2 bytes each, rounded up to 256 bytes), then, for
 * wq_gemm on problems too small to fill the GPU (fewer than 256 workgroups of
 * 64 rows x 256 columns), the fp32 partial products of a K split (S*M*N*4
 * bytes, S the number of K slices, a function of M, N, K and bits).  0 when
 * neither applies.
 */
size_t wq_workspace_bytes(int M, int N, int K, int bits, int has_perm);

/*
 * wq_repack -- offline conversion of one quantised layer from the canonical
 * format to the gfx950 tile layout.  The pages require a kernel-specific
 * format that any quantiser's output is converted to (Marlin zero-point issue,
 * efrantar's reply); this is that conversion for these kernels.
 *
 *   qweight, scales, zeros : canonical buffers (device), see above
 *   mode                   : quantisation mode (the code order inside a word
 *                            differs between uniform and table modes)
 *   g_idx_host             : act-order group of every row (host, int32 [K]) or
 *                            NULL.  Each group must hold exactly group_size
 *                            rows (WQ_EUNSUPPORTED otherwise); rows are stably
 *                            sorted by group
 *   packed                 : output, wq_packed_bytes(K, N, bits, group_size, mode)
 *   perm                   : output (device, int32 [K]) when g_idx_host is given:
 *                            perm[i] = original row at sorted position i; else
 *                            ignored (may be NULL)
 * Synchronises `stream` before returning (the act-order sort runs on the host).
 */
wq_status wq_repack(const uint32_t* qweight, const uint16_t* scales, const void* zeros,
                    wq_qmode mode, const int32_t* g_idx_host, int K, int N, int bits,
                    int group_size, void* packed, int32_t* perm, void* stream);

/*
 * wq_dequant_debug -- write the dequantised weight w [K][N] (rows in the
 * original order, activation dtype `out`) from a repacked buffer.  Test aid:
 * the result equals, bit for bit, one RNE rounding of s*(q-z) or s*T[q].
 *   lut  : device fp16 [2^bits] for WQ_LUT, else NULL
 *   perm : the permutation wq_repack wrote (act-order) or NULL
 */
wq_status wq_dequant_debug(const void* packed, wq_qmode mode, const uint16_t* lut,
                           const int32_t* perm, int K, int N, int bits, int group_size,
                           wq_dtype out, void* w, void* stream);

/*
 * wq_gemv -- y [M][N] = x [M][K] . dequant(W), for decode-sized M (1 <= M <= 32;
 * WQ_EUNSUPPORTED above).  Matrix-vector products are bound by memory
 * bandwidth and the gain comes from moving fewer weight bytes (exllama
 * bandwidth discussion, GPTQ paper quote and turboderp's reply); this entry
 * point streams the packed weight once, split along K inside each workgroup.
 *   x, y : device, activation dtype `dt` (y in the same dtype), row-major
 *   packed, lut, perm : as for wq_dequant_debug
 *   ws   : scratch of at least wq_workspace_bytes(M, N, K, bits, perm != NULL)
 *          bytes (may be NULL when that is 0)
 * fp32 accumulation; the output is rounded to `dt` once (RNE).
 */
wq_status wq_gemv(const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                  const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K,
                  int bits, int group_size, void* ws, size_t ws_bytes, void* stream);

/*
 * wq_gemm -- the same product for any M >= 1 (prefill, long context: the
 * matrix-matrix case the Triton GPTQ page targets, "How It Works"), on MFMA
 * matrix cores with the activation tile staged in LDS and the weight tile
 * dequantised in registers.  Same arguments as wq_gemv.
 */
wq_status wq_gemm(const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                  const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K,
                  int bits, int group_size, void* ws, size_t ws_bytes, void* stream);

/*
 * wq_gemm_noalloc -- wq_gemm without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The scratch wq_gemm takes from
 * `ws` (act-order permuted activations, K-split partial products) comes from
 * one static device array per GPU of WQ_NOALLOC_SCRATCH_BYTES, which the
 * library holds from its first use on that GPU until the process ends; this
 * entry point allocates and frees nothing.
 *   Arguments, limits and results as wq_gemm.  A call needing more scratch
 *   than the array holds (wq_workspace_bytes(M, N, K, bits, perm != NULL) >
 *   WQ_NOALLOC_SCRATCH_BYTES, e.g. act-order with M * K > 16 Mi) returns
 *   WQ_ENOSPACE and launches nothing.
 *   Every call on one GPU uses that GPU's one array: calls that overlap in
 *   time on one GPU (different streams, or different host threads without
 *   ordering) race on it and give undefined results.  Calls ordered on one
 *   stream are safe; nothing in the array needs to start at zero.
 */
#define WQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
wq_status wq_gemm_noalloc(const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                          const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K,
                          int bits, int group_size, void* stream);

/*
 * Activation-fused gate+up layer.  The Triton GPTQ page fuses the feed-forward
 * layers ("How It Works") without naming the activation; these entry points
 * read it as the gated SiLU of LLaMA-style blocks: for a weight W = [gate | up]
 * concatenated along N (N = 2I, each half quantised on its own, columns
 * 0..I-1 the gate, I..2I-1 the up projection)
 *     h [M][I] = SiLU(x . dequant(gate)) * (x . dequant(up)),  SiLU(v) = v / (1 + e^-v),
 * written once, so the two products are never stored and no second kernel
 * reads them back.
 *
 * wq_repack_gate_up -- the same conversion as wq_repack (same arguments, same
 *   canonical inputs, same wq_packed_bytes size), with N % 32 == 0 required,
 *   that interleaves the 16-column tiles of the two halves (gate tile j, then
 *   up tile j) so one workgroup owns both halves of an output tile.  Such a
 *   buffer is only meaningful to the *_gate_up products; wq_dequant_debug
 *   writes its columns in that interleaved order.
 * wq_gemv_gate_up / wq_gemm_gate_up -- h as above from a wq_repack_gate_up
 *   buffer; same arguments and limits as wq_gemv / wq_gemm, N is the full
 *   width 2I (N % 32 == 0, else WQ_EUNSUPPORTED) and y is h [M][N/2].  Gate
 *   and up are each accumulated in fp32 as in wq_gemv / wq_gemm; SiLU and the
 *   product are evaluated in fp32 and rounded to `dt` once (RNE).
 */
wq_status wq_repack_gate_up(const uint32_t* qweight, const uint16_t* scales, const void* zeros,
                            wq_qmode mode, const int32_t* g_idx_host, int K, int N, int bits,
                            int group_size, void* packed, int32_t* perm, void* stream);
wq_status wq_gemv_gate_up(const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                          const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K,
                          int bits, int group_size, void* ws, size_t ws_bytes, void* stream);
wq_status wq_gemm_gate_up(const void* x, wq_dtype dt, const void* packed, wq_qmode mode,
                          const uint16_t* lut, const int32_t* perm, void* y, int M, int N, int K,
                          int bits, int group_size, void* ws, size_t ws_bytes, void* stream);

/*
 * wq_hadamard -- online rotation of the activations before the product.  The
 * FLUTE page lists Hadamard-transform support ("Maintenance & Community")
 * without details; the reading: weights were rotated offline (H W) before
 * quantisation, and each activation row is rotated at run time by the same
 * orthonormal block-diagonal Walsh-Hadamard matrix H, so that (x H)(H W) = x W.
 * For every row and every block of `block` consecutive elements starting at k0:
 *     y[m][k0 + i] = block^(-1/2) * sum_j (-1)^popcount(i & j) * x[m][k0 + j]
 * The rotated rows feed wq_gemv / wq_gemm (or the *_gate_up products) as x.
 *   x, y  : device [M][K] in `dt`, 16-byte aligned; y == x rotates in place,
 *           other overlaps are WQ_EINVAL
 *   block : power of two, 2 <= block <= 512, K % block == 0 (else WQ_EINVAL);
 *           K % 8 == 0 (else WQ_EUNSUPPORTED)
 * fp32 arithmetic (fast Walsh-Hadamard butterflies), y rounded once to `dt`
 * (RNE).  M == 0 is a valid no-op.
 */
wq_status wq_hadamard(const void* x, wq_dtype dt, void* y, int M, int K, int block, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
