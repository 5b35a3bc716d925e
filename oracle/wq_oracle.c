/*
 * wq_oracle.c -- CPU oracle for the weight-only quantized mixed-input product
 *                y = x . dequant(W)
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark load this library.  The GPU library never
 * links, includes or calls it, and it shares no source with the GPU path.
 *
 * What it computes (and where the pages fix it):
 *   - the product is an ordinary matrix product with the weights decoded on
 *     the fly, never kept in full precision in the fast path (Triton GPTQ page,
 *     "How It Works"; exllama bandwidth discussion, the GPTQ paper quote on the
 *     quantized-matrix full-precision-vector kernel);
 *   - uniform codes with a scale per (group, column) and either a zero-point
 *     fixed at the middle of the code range (symmetric) or a stored zero-point,
 *     kept in fp16 or itself quantised (Marlin zero-point issue, replies by
 *     efrantar and mobicham);
 *   - lookup-table codes: a code selects a table value, which is multiplied by
 *     the scale (FLUTE page, "How It Works"); 2/3/4-bit codes (same section);
 *   - a column-wise scale (group size -1) or group-wise scales (Triton GPTQ
 *     page, "Highlighted Details"; Marlin zero-point issue, efrantar);
 *   - act-order: the group of an input row is looked up in g_idx rather than
 *     derived from its index (Triton GPTQ page, "Limitations & Caveats");
 *   - zero-points whose group size is chosen apart from the scales' (Marlin
 *     zero-point issue, mobicham's reply, the HQQ+ experiment).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   canonical packing = per column, a little-endian bit stream along K (code
 *   k at bit offset bits*k over words qweight[0][n], qweight[1][n], ...);
 *   packed zero-points = per group row, a little-endian bit stream along N;
 *   symmetric zero = 2^(bits-1); dequant = one round-to-nearest-even of the
 *   exact real s*(q-z) or s*T[q] to the activation dtype, subnormals kept,
 *   overflow to +-inf; the sum over k is exact-as-possible fp64, k ascending.
 *
 * Everything here is plain and slow on purpose: element-wise decode, fp64
 * arithmetic, a naive loop over (m, n, k).  OpenMP splits output columns over
 * host threads; it does not change what is computed.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status codes of the oracle (independent of the GPU library's). */
#define WQO_OK 0
#define WQO_EINVAL 1

/* Quantisation modes and dtypes, numbered as the public interface numbers them. */
#define WQO_SYM 0          /* zero-point fixed at 2^(bits-1)            */
#define WQO_ZERO_F16 1     /* fp16 zero-point per (group, column)         */
#define WQO_ZERO_PACKED 2  /* bits-wide integer zero-point per (group, column) */
#define WQO_LUT 3          /* w = s * T[q], fp16 table of 2^bits entries  */
/* fp16 zero-points with a group of their own, 8 / 16 / 32 rows, decoupled from
 * the scale group (Marlin zero-point issue, mobicham's reply: zero-point and
 * scale group sizes chosen separately, e.g. per-column scales with a
 * zero-point every 8 rows); zeros fp16 [K / zero group][N], indexed by the
 * row's original position. */
#define WQO_ZERO_F16_G8 4
#define WQO_ZERO_F16_G16 5
#define WQO_ZERO_F16_G32 6
#define WQO_F16 0
#define WQO_BF16 1

/* ------------------------------------------------------------------ */
/* Number formats.  Written from the IEEE-754 binary16 definition and   */
/* from bfloat16 = the top 16 bits of binary32.                         */
/* ------------------------------------------------------------------ */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double wqo_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);     /* (1.f) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double wqo_bf16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 7) & 0xff;
  int f = h & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
  } else if (e == 255) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(128 + f), e - 134);     /* (1.f) * 2^(e-127) */
  }
  return sign ? -v : v;
}

/*
 * Round a double to the nearest value of a binary format with `p` significand
 * bits (implicit bit included), minimum normal exponent `emin` and largest
 * finite exponent `emax`, ties to even, keeping subnormals.  Returns the rounded
 * value as a double (exactly representable in the target format), or +-inf on
 * overflow.  Direct from the double: no intermediate format, so one rounding.
 */
static double round_to_format(double v, int p, int emin, int emax) {
  if (v == 0.0 || isnan(v) || isinf(v)) return v;
  double a = fabs(v);
  int ex;
  frexp(a, &ex);                   /* a = m * 2^ex, m in [0.5, 1) */
  int e = ex - 1;                  /* a in [2^e, 2^(e+1)) */
  if (e < emin) e = emin;          /* subnormal range keeps the quantum of emin */
  double quantum = ldexp(1.0, e - (p - 1));
  double r = rint(a / quantum);    /* exact division by a power of two; rint = ties-to-even */
  double out = r * quantum;
  /* Largest finite value is (2 - 2^(1-p)) * 2^emax; anything that rounds to 2^(emax+1) overflows. */
  if (out >= ldexp(1.0, emax + 1)) out = INFINITY;
  return v < 0 ? -out : out;
}

uint16_t wqo_f64_to_f16(double v) {
  if (isnan(v)) return 0x7e00;
  double r = round_to_format(v, 11, -14, 15);
  uint16_t sign = (signbit(r) ? 0x8000 : 0);
  double a = fabs(r);
  if (isinf(a)) return sign | 0x7c00;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -14)) return sign | (uint16_t)ldexp(a, 24);   /* subnormal fraction */
  int ex;
  frexp(a, &ex);
  int e = ex - 1;                                                   /* a in [2^e, 2^(e+1)) */
  uint16_t frac = (uint16_t)(ldexp(a, 10 - e) - 1024.0);
  return sign | (uint16_t)((e + 15) << 10) | frac;
}

uint16_t wqo_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7fc0;
  double r = round_to_format(v, 8, -126, 127);
  uint16_t sign = (signbit(r) ? 0x8000 : 0);
  double a = fabs(r);
  if (isinf(a)) return sign | 0x7f80;
  if (a == 0.0) return sign;
  if (a < ldexp(1.0, -126)) return sign | (uint16_t)ldexp(a, 133);
  int ex;
  frexp(a, &ex);
  int e = ex - 1;
  uint16_t frac = (uint16_t)(ldexp(a, 7 - e) - 128.0);
  return sign | (uint16_t)((e + 127) << 7) | frac;
}

static double decode_act(uint16_t h, int dtype) {
  return dtype == WQO_BF16 ? wqo_bf16_to_f64(h) : wqo_f16_to_f64(h);
}

static uint16_t encode_act(double v, int dtype) {
  return dtype == WQO_BF16 ? wqo_f64_to_bf16(v) : wqo_f64_to_f16(v);
}

/* ------------------------------------------------------------------ */
/* Canonical packing (reading of the pages: the GPTQ convention of     */
/* codes packed along K into 32-bit words, generalised to 2 and 3 bits */
/* as a little-endian bit stream per column).                           */
/* ------------------------------------------------------------------ */

/* Code of row k in a bit stream whose word r sits at stream[r * stride]. */
static unsigned stream_code(const uint32_t* stream, size_t stride, long idx, int bits) {
  long bit = (long)bits * idx;
  long r = bit / 32;
  int sh = (int)(bit % 32);
  uint64_t two = (uint64_t)stream[(size_t)r * stride] >> sh;
  if (sh + bits > 32) two |= (uint64_t)stream[(size_t)(r + 1) * stride] << (32 - sh);
  return (unsigned)(two & ((1u << bits) - 1u));
}

static void stream_put(uint32_t* stream, size_t stride, long idx, int bits, unsigned code) {
  long bit = (long)bits * idx;
  long r = bit / 32;
  int sh = (int)(bit % 32);
  uint64_t mask = ((uint64_t)((1u << bits) - 1u)) << sh;
  uint64_t val = ((uint64_t)code << sh) & mask;
  uint32_t* w0 = &stream[(size_t)r * stride];
  *w0 = (uint32_t)((*w0 & ~(uint32_t)mask) | (uint32_t)val);
  if (sh + bits > 32) {
    uint32_t* w1 = &stream[(size_t)(r + 1) * stride];
    uint32_t m1 = (uint32_t)(mask >> 32), v1 = (uint32_t)(val >> 32);
    *w1 = (*w1 & ~m1) | v1;
  }
}

static int bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 4; }

/* qweight is uint32[K*bits/32][N]; codes is uint8[K][N]. */
int wqo_unpack_codes(const uint32_t* qweight, int K, int N, int bits, uint8_t* codes) {
  if (!bits_ok(bits) || K <= 0 || N <= 0 || ((long)K * bits) % 32) return WQO_EINVAL;
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      codes[(size_t)k * N + n] = (uint8_t)stream_code(qweight + n, (size_t)N, k, bits);
  return WQO_OK;
}

int wqo_pack_codes(const uint8_t* codes, int K, int N, int bits, uint32_t* qweight) {
  if (!bits_ok(bits) || K <= 0 || N <= 0 || ((long)K * bits) % 32) return WQO_EINVAL;
  memset(qweight, 0, sizeof(uint32_t) * ((size_t)K * bits / 32) * (size_t)N);
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k)
      stream_put(qweight + n, (size_t)N, k, bits, codes[(size_t)k * N + n] & ((1u << bits) - 1u));
  return WQO_OK;
}

/* Packed zero-points: uint32[G][N*bits/32]; row g is a bit stream along N. */
int wqo_unpack_zeros(const uint32_t* zp, int G, int N, int bits, uint8_t* z) {
  if (!bits_ok(bits) || G <= 0 || N <= 0 || ((long)N * bits) % 32) return WQO_EINVAL;
  size_t wpr = (size_t)N * bits / 32;
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      z[(size_t)g * N + n] = (uint8_t)stream_code(zp + (size_t)g * wpr, 1, n, bits);
  return WQO_OK;
}

int wqo_pack_zeros(const uint8_t* z, int G, int N, int bits, uint32_t* zp) {
  if (!bits_ok(bits) || G <= 0 || N <= 0 || ((long)N * bits) % 32) return WQO_EINVAL;
  size_t wpr = (size_t)N * bits / 32;
  memset(zp, 0, sizeof(uint32_t) * wpr * (size_t)G);
  for (int g = 0; g < G; ++g)
    for (int n = 0; n < N; ++n)
      stream_put(zp + (size_t)g * wpr, 1, n, bits, z[(size_t)g * N + n] & ((1u << bits) - 1u));
  return WQO_OK;
}

/* ------------------------------------------------------------------ */
/* Dequantisation of one weight.                                        */
/* ------------------------------------------------------------------ */

typedef struct {
  const uint32_t* qweight;
  const uint16_t* scales;   /* fp16 [G][N] */
  const void* zeros;        /* fp16 [G][N] or uint32 [G][N*bits/32] or NULL */
  int mode;
  const uint16_t* lut;      /* fp16 [2^bits] or NULL */
  const int32_t* g_idx;     /* int32 [K] or NULL */
  int K, N, bits, group_size, G, dtype;
} layer_t;

static int fine_zero_group(int mode);

static int layer_check(const layer_t* L) {
  if (!L->qweight || !L->scales) return WQO_EINVAL;
  if (!bits_ok(L->bits) || L->K <= 0 || L->N <= 0) return WQO_EINVAL;
  if (((long)L->K * L->bits) % 32) return WQO_EINVAL;
  if (L->dtype != WQO_F16 && L->dtype != WQO_BF16) return WQO_EINVAL;
  if (L->group_size != -1 && (L->group_size <= 0 || L->K % L->group_size)) return WQO_EINVAL;
  switch (L->mode) {
    case WQO_SYM: break;
    case WQO_ZERO_F16: if (!L->zeros) return WQO_EINVAL; break;
    case WQO_ZERO_F16_G8:
    case WQO_ZERO_F16_G16:
    case WQO_ZERO_F16_G32:
      if (!L->zeros || L->K % fine_zero_group(L->mode)) return WQO_EINVAL;
      break;
    case WQO_ZERO_PACKED:
      if (!L->zeros || ((long)L->N * L->bits) % 32) return WQO_EINVAL;
      break;
    case WQO_LUT: if (!L->lut) return WQO_EINVAL; break;
    default: return WQO_EINVAL;
  }
  if (L->g_idx)
    for (int k = 0; k < L->K; ++k)
      if (L->g_idx[k] < 0 || L->g_idx[k] >= L->G) return WQO_EINVAL;
  return WQO_OK;
}

/* Rows per zero-point group of the modes whose zero-points have their own,
 * finer group (0 for the other modes). */
static int fine_zero_group(int mode) {
  return mode == WQO_ZERO_F16_G8 ? 8 : mode == WQO_ZERO_F16_G16 ? 16 : mode == WQO_ZERO_F16_G32 ? 32 : 0;
}

static int group_of(const layer_t* L, int k) {
  if (L->g_idx) return L->g_idx[k];
  if (L->group_size == -1) return 0;
  return k / L->group_size;
}

/*
 * The exact real value s*(q - z) (uniform) or s*T[q] (table), every operand
 * exact in fp64 and the product exact too (at most 11+40 significant bits),
 * then a single round-to-nearest-even to the activation dtype.
 * Returns the dtype's bit pattern.
 */
static uint16_t dequant_one(const layer_t* L, int k, int n) {
  unsigned q = stream_code(L->qweight + n, (size_t)L->N, k, L->bits);
  int g = group_of(L, k);
  double s = wqo_f16_to_f64(L->scales[(size_t)g * L->N + n]);
  double e;
  if (L->mode == WQO_LUT) {
    e = s * wqo_f16_to_f64(L->lut[q]);
  } else {
    double z;
    if (L->mode == WQO_SYM) {
      z = (double)(1 << (L->bits - 1));
    } else if (L->mode == WQO_ZERO_F16) {
      z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)g * L->N + n]);
    } else if (fine_zero_group(L->mode)) {
      /* zero-point group of row k: k / zero-group rows (original row order) */
      z = wqo_f16_to_f64(((const uint16_t*)L->zeros)[(size_t)(k / fine_zero_group(L->mode)) * L->N + n]);
    } else {
      size_t wpr = (size_t)L->N * L->bits / 32;
      z = (double)stream_code((const uint32_t*)L->zeros + (size_t)g * wpr, 1, n, L->bits);
    }
    e = s * ((double)q - z);
  }
  return encode_act(e, L->dtype);
}

static int n_groups(int K, int group_size) { return group_size == -1 ? 1 : K / group_size; }

/* w (dtype bits) [K][N] = dequant(W), rows in their original order. */
int wqo_dequant(const uint32_t* qweight, const uint16_t* scales, const void* zeros, int mode,
                const uint16_t* lut, const int32_t* g_idx, int K, int N, int bits, int group_size,
                int dtype, uint16_t* w) {
  layer_t L = {qweight, scales, zeros, mode, lut, g_idx, K, N, bits, group_size, 0, dtype};
  if (bits_ok(bits) && K > 0 && (group_size == -1 || (group_size > 0 && K % group_size == 0)))
    L.G = n_groups(K, group_size);
  int rc = layer_check(&L);
  if (rc) return rc;
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n)
    for (int k = 0; k < K; ++k) w[(size_t)k * N + n] = dequant_one(&L, k, n);
  return WQO_OK;
}

/*
 * y[m][j] (fp64) = sum_k x[m][k] * w[k][cols[j]], with w the dequantised weight
 * (rounded to the activation dtype) and x decoded exactly.  k ascends.
 * cols == NULL means every column (ncols must then equal N).
 */
int wqo_linear(const uint16_t* x, int dtype, const uint32_t* qweight, const uint16_t* scales,
               const void* zeros, int mode, const uint16_t* lut, const int32_t* g_idx, int M, int N,
               int K, int bits, int group_size, const int32_t* cols, int ncols, double* y) {
  layer_t L = {qweight, scales, zeros, mode, lut, g_idx, K, N, bits, group_size, 0, dtype};
  if (bits_ok(bits) && K > 0 && (group_size == -1 || (group_size > 0 && K % group_size == 0)))
    L.G = n_groups(K, group_size);
  int rc = layer_check(&L);
  if (rc) return rc;
  if (M < 0 || ncols < 0 || !y || (M > 0 && !x)) return WQO_EINVAL;
  if (!cols && ncols != N) return WQO_EINVAL;
  if (cols)
    for (int j = 0; j < ncols; ++j)
      if (cols[j] < 0 || cols[j] >= N) return WQO_EINVAL;
  if (M == 0 || ncols == 0) return WQO_OK;

  double* xd = (double*)malloc(sizeof(double) * (size_t)M * K);
  if (!xd) return WQO_EINVAL;
  for (size_t i = 0; i < (size_t)M * K; ++i) xd[i] = decode_act(x[i], dtype);

  int bad = 0;
#pragma omp parallel
  {
    double* wcol = (double*)malloc(sizeof(double) * (size_t)K);
    if (!wcol) {
#pragma omp atomic write
      bad = 1;
    }
#pragma omp for schedule(dynamic, 8)
    for (int j = 0; j < ncols; ++j) {
      if (!wcol) continue;
      int n = cols ? cols[j] : j;
      for (int k = 0; k < K; ++k) {
        uint16_t h = dequant_one(&L, k, n);
        wcol[k] = dtype == WQO_BF16 ? wqo_bf16_to_f64(h) : wqo_f16_to_f64(h);
      }
      for (int m = 0; m < M; ++m) {
        const double* xr = xd + (size_t)m * K;
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += xr[k] * wcol[k];
        y[(size_t)m * ncols + j] = acc;
      }
    }
    free(wcol);
  }
  free(xd);
  return bad ? WQO_EINVAL : WQO_OK;
}

int wqo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Array forms of the format converters (for the tests' pins). */
void wqo_decode_array(const uint16_t* h, size_t n, int dtype, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = decode_act(h[i], dtype);
}

void wqo_encode_array(const double* v, size_t n, int dtype, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = encode_act(v[i], dtype);
}

/*
 * Activation-fused FFN input projection: h = SiLU(g) * u elementwise, with
 * g = x . W_gate and u = x . W_up the two halves of a fused gate+up product
 * (Triton GPTQ page, "How It Works": FFN layers fused).  The page does not
 * name the activation; SiLU(v) = v / (1 + exp(-v)) is the reading taken.
 * fp64 throughout.
 */
double wqo_silu(double v) { return v / (1.0 + exp(-v)); }

void wqo_swiglu(const double* g, const double* u, size_t n, double* h) {
  for (size_t i = 0; i < n; ++i) h[i] = wqo_silu(g[i]) * u[i];
}

/*
 * Online Hadamard rotation of the activations (FLUTE page, "Maintenance &
 * Community": Hadamard transform support).  The page gives no details; the
 * reading taken is the usual one for rotated weight-only quantisation: the
 * weights were rotated and quantised offline as H W, and at run time each
 * activation row is rotated by the same orthonormal, block-diagonal
 * Walsh-Hadamard matrix, so that (x H)(H W) = x W (H is symmetric and H H = I).
 *
 * With block size b (a power of two dividing K), for every row m and every
 * block start k0 = 0, b, 2b, ...:
 *     y[m][k0 + i] = b^(-1/2) * sum_j (-1)^popcount(i & j) * x[m][k0 + j]
 * (the Sylvester construction of the b x b Hadamard matrix, entry (i, j) =
 * (-1)^(number of bit positions where both i and j have a one)).
 * Direct O(b^2) sum per block, fp64.  Returns 0, or 1 for bad sizes.
 */
static int parity_of_and(unsigned i, unsigned j) {
  unsigned v = i & j;
  int p = 0;
  while (v) {
    p ^= (int)(v & 1u);
    v >>= 1;
  }
  return p;
}

int wqo_hadamard(const double* x, int M, int K, int b, double* y) {
  if (M < 0 || K <= 0 || b <= 0 || (b & (b - 1)) != 0 || K % b != 0) return 1;
  const double norm = 1.0 / sqrt((double)b);
  for (int m = 0; m < M; ++m) {
    for (int k0 = 0; k0 < K; k0 += b) {
      const double* xb = x + (size_t)m * K + k0;
      double* yb = y + (size_t)m * K + k0;
      for (int i = 0; i < b; ++i) {
        double s = 0.0;
        for (int j = 0; j < b; ++j) s += parity_of_and((unsigned)i, (unsigned)j) ? -xb[j] : xb[j];
        yb[i] = s * norm;
      }
    }
  }
  return 0;
}
