/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for the NVFP4 linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the package smoke check and the CPU leg of
 * the benchmark do.  It shares no source with the HIP kernels.
 *
 * Every function states the passage of the source pages it follows.  The
 * pages (news articles about NVIDIA's 4-bit pretraining recipe) are cited by
 * title and section:
 *   [P1] hyper.ai, "NVIDIA revolutioniert KI-Praetrainingsgeschwindigkeit mit
 *        4-Bit-Genauigkeit", body.
 *   [P3] aibuzzwire.news, "Thinking Machines ... End-to-End 4-Bit Training"
 *        article, sections "Warum weniger Bits ein schnelleres Training
 *        bedeuten", "Drei Formate, ein Trainingslauf", "Unterschiedliche
 *        Phasen, unterschiedliche Regeln".
 *   [P4] aisight.pl, "Koniec marnowania mocy. NVIDIA udowadnia, ze 4 bity
 *        wystarcza do trenowania gigantow", sections "Architektura NVFP4
 *        kontra ograniczenia mikroskalowania" and "Technologie stabilizujace
 *        proces treningowy".
 * Where the pages are silent the reading taken is stated at the function and
 * listed with the other readings in the design notes of the repository.
 *
 * Numerics: compiled with -ffp-contract=off and without -ffast-math, so every
 * float expression below is one IEEE binary32 operation rounded to nearest
 * even, subnormals kept.  Integer work on bit patterns is exact.
 *
 * Parity status per function (see tests/test_oracle_*.py for the pins):
 *   oracle_e2m1_value / oracle_e2m1_rne / oracle_e2m1_sr   pinned
 *   oracle_e4m3_value / oracle_e4m3_rne_sat                pinned
 *   oracle_philox4x32_10                                    pinned (rocRAND)
 *   oracle_rht16                                            pinned
 *   oracle_quantize / oracle_dequantize / oracle_decode_qs  pinned
 *   oracle_mx_scale_exp / oracle_mxfp4_quantize / _decode   pinned
 *   oracle_mx8_scale_exp / oracle_mxfp8_quantize / _decode  pinned
 *   oracle_mxfp8_trunc_bound (a tolerance checker)          worked cases
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Bit helpers                                                              */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bf16 is the upper half of a binary32; widening is exact. */
static float bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* Round a binary32 to bf16, nearest-even (NaN kept quiet). */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* ------------------------------------------------------------------------ */
/* E2M1 element format                                                      */
/* ------------------------------------------------------------------------ */

/* The 4-bit element: sign bit, then a 3-bit magnitude code whose values are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 (one sign, two exponent bits with bias 1, one
 * mantissa bit).  The pages only say "4 bit" ([P4] lede, [P1]); this value
 * set is the standard E2M1 element of NVFP4. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float oracle_e2m1_value(uint8_t code)
{
    double m = E2M1_MAG[code & 7];
    return (float)((code & 8) ? -m : m);
}

/* Round-to-nearest onto the E2M1 grid ([P3] "Warum weniger Bits ...": a
 * value is stored as the nearest representable one, the worked example
 * being 3.2 stored as 3 in a format that holds 3 and 4).  Ties go to the
 * even magnitude code (the code whose mantissa bit is 0); magnitudes above 6
 * saturate to 6 because E2M1 has no infinity.  Written as the definition: an
 * argmin of the distance over the eight magnitudes.  The sign bit of v is
 * kept, so -0.0 and negative values that round to zero give code 0x8. */
uint8_t oracle_e2m1_rne(float v)
{
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 8 : 0;
    /* Beyond the largest magnitude the nearest value is 6 (saturation); the
     * early exit also keeps the distances below exact in double. */
    if (a >= 6.0) return (uint8_t)(sign | 7);
    int best = 0;
    double best_d = fabs(a - E2M1_MAG[0]);
    for (int j = 1; j < 8; ++j) {
        double d = fabs(a - E2M1_MAG[j]);
        if (d < best_d || (d == best_d && (j & 1) == 0 && (best & 1) == 1)) {
            best = j;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/* Stochastic rounding onto the E2M1 grid ([P4] "Technologie stabilizujace
 * ...": stochastic rounding removes the systematic error of ordinary
 * rounding; [P3] "Unterschiedliche Phasen ...": the backward pass tolerates
 * noise but not bias).  Reading: the textbook definition -- add a uniform
 * random offset u in [0, 1) grid steps and truncate -- with u taken at the
 * midpoint of the 16-bit random value's interval, u = (r16 + 1/2) / 2^16.
 * With lo the largest grid magnitude <= |v|, hi the next one and
 * frac = (|v| - lo) / (hi - lo): round up iff frac + u >= 1.  Then
 * P(up) = floor(frac * 2^16 + 1/2) / 2^16, within 2^-17 of frac either
 * way.  |v| >= 6 saturates to 6; a value on the grid (frac = 0) never moves
 * because u < 1. */
uint8_t oracle_e2m1_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    uint8_t sign = signbit(v) ? 8 : 0;
    if (!(a < 6.0)) return (uint8_t)(sign | 7);
    int lo = 0;
    for (int j = 0; j < 8; ++j)
        if (E2M1_MAG[j] <= a) lo = j;
    double step = E2M1_MAG[lo + 1] - E2M1_MAG[lo];
    double frac = (a - E2M1_MAG[lo]) / step;          /* exact: step is a power of two */
    double u = ((double)(r16 & 0xFFFFu) + 0.5) / 65536.0;
    int code = (frac >= 1.0 - u) ? lo + 1 : lo;       /* frac + u >= 1, both sides exact */
    return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------------ */
/* E4M3 block-scale format                                                  */
/* ------------------------------------------------------------------------ */

/* [P4] "Architektura NVFP4 ...": the per-block scale is an E4M3 number
 * instead of a power of two.  Reading: the OCP E4M3FN encoding (bias 7,
 * three mantissa bits, subnormals with spacing 2^-9, largest finite 448,
 * no infinity, 0x7F/0xFF are NaN). */
float oracle_e4m3_value(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(8.0 + m, e - 10);
    return (float)(s ? -v : v);
}

/* Nearest E4M3 value to t >= 0, ties to even mantissa, saturating at 448
 * (reading: an E4M3 scale may never become NaN).  Negative, zero and NaN
 * inputs give 0 (they never occur: block maxima are >= 0). */
uint8_t oracle_e4m3_rne_sat(float t)
{
    double x = (double)t;
    if (!(x > 0.0)) return 0x00;
    if (x >= 448.0) return 0x7E;
    int e;
    frexp(x, &e);        /* x in [2^(e-1), 2^e) */
    e -= 1;              /* now x in [2^e, 2^(e+1)) */
    if (e < -6) e = -6;  /* subnormals share the spacing of the first binade */
    double step = ldexp(1.0, e - 3);
    double n = nearbyint(x / step);   /* x/step is exact; default mode is RNE */
    double r = n * step;
    if (r > 448.0) r = 448.0;
    /* encode r */
    if (r < ldexp(1.0, -6)) return (uint8_t)(int)(r / ldexp(1.0, -9));
    int er;
    frexp(r, &er);
    er -= 1;
    int mant = (int)(r / ldexp(1.0, er - 3)) - 8;
    return (uint8_t)(((er + 7) << 3) | mant);
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as  */
/* easy as 1, 2, 3", SC'11)                                                 */
/* ------------------------------------------------------------------------ */

/* Counter-based generator for stochastic rounding.  The pages do not name a
 * generator; Philox4x32 with ten rounds is taken from its publication: two
 * 32x32->64 multiplies per round with multipliers 0xD2511F53 and 0xCD9E8D57,
 * a Feistel-like permutation of the four words, and a key schedule that adds
 * the Weyl constants 0x9E3779B9 and 0xBB67AE85 between rounds. */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4])
{
    uint32_t c[4] = {ctr_in[0], ctr_in[1], ctr_in[2], ctr_in[3]};
    uint32_t k[2] = {key_in[0], key_in[1]};
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c[2];
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c[1] ^ k[0];
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c[3] ^ k[1];
        uint32_t n3 = lo0;
        c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    }
    out[0] = c[0]; out[1] = c[1]; out[2] = c[2]; out[3] = c[3];
}

/* The 16 random bits used for element i (index in the quantized [outer][K]
 * layout).  Reading: one Philox call serves 8 consecutive elements; the
 * counter is (lo32(i/8), hi32(i/8), lo32(offset), hi32(offset)), the key is
 * (lo32(seed), hi32(seed)); element i takes 16-bit half (i mod 2) (low half
 * first) of output word ((i mod 8) / 2). */
uint32_t oracle_sr_bits(uint64_t seed, uint64_t offset, uint64_t i)
{
    uint64_t g = i >> 3;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset,
                       (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    oracle_philox4x32_10(ctr, key, w);
    uint32_t word = w[(i & 7) >> 1];
    return (i & 1) ? (word >> 16) : (word & 0xFFFFu);
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform over 16 elements                               */
/* ------------------------------------------------------------------------ */

/* [P4] "Technologie stabilizujace ...": random Hadamard transforms spread
 * outliers of the weight gradients.  Reading: y = (1/4) H16 diag(s) x with
 * H16 the Sylvester Hadamard matrix, H[i][j] = (-1)^popcount(i & j), and s
 * the random sign vector (bit j of sign_mask set means s_j = -1).  Applied
 * as the fast Walsh-Hadamard butterfly in binary32 with stages h = 1, 2, 4,
 * 8; in each pair the lower index takes a + b and the upper a - b.  The sign
 * flip and the factor 1/4 are exact. */
void oracle_rht16(const float *x, uint32_t sign_mask, float *y)
{
    float t[16];
    for (int j = 0; j < 16; ++j)
        t[j] = ((sign_mask >> j) & 1u) ? -x[j] : x[j];
    for (int h = 1; h < 16; h <<= 1) {
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            float a = t[j], b = t[j + h];
            t[j] = a + b;
            t[j + h] = a - b;
        }
    }
    for (int j = 0; j < 16; ++j) y[j] = 0.25f * t[j];
}

/* ------------------------------------------------------------------------ */
/* Quantize                                                                 */
/* ------------------------------------------------------------------------ */

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_RNE = 0, OR_SR = 1 };

/* Element (o, k) of the quantization view: axis 1 takes rows as the outer
 * index and columns as K; axis 0 takes columns as the outer index and rows
 * as K (the GEMM reduction runs along K). */
static float view_get(const void *x, int dtype, int64_t rows, int64_t cols,
                      int axis, int64_t o, int64_t k)
{
    (void)rows;
    int64_t r = axis ? o : k;
    int64_t c = axis ? k : o;
    if (dtype == OR_BF16) return bf16_to_f32(((const uint16_t *)x)[r * cols + c]);
    return ((const float *)x)[r * cols + c];
}

/* Load the 16 values of block (o, b), applying the RHT when asked. */
static void load_block(const void *x, int dtype, int64_t rows, int64_t cols,
                       int axis, int rht, uint32_t sign_mask, int64_t o,
                       int64_t b, float *y)
{
    float raw[16];
    for (int j = 0; j < 16; ++j)
        raw[j] = view_get(x, dtype, rows, cols, axis, o, 16 * b + j);
    if (rht) oracle_rht16(raw, sign_mask, y);
    else memcpy(y, raw, sizeof raw);
}

/* The NVFP4 quantizer ([P4] "Architektura NVFP4 ..."): a per-tensor FP32
 * scale level, a per-16-element E4M3 block scale, 4-bit elements; optional
 * RHT ([P4] "Technologie stabilizujace ...") and stochastic rounding.
 *
 * Steps (readings where the pages are silent):
 *  1. view Y[o][k] (axis), K % 16 == 0; RHT per 16-chunk along K if asked.
 *  2. amax = max |Y| over the whole tensor, taken on the bit patterns of |Y|
 *     (exact and order free; NaN > Inf > finite).  Non-finite amax: meta is
 *     written and the codes/scales are left unspecified.
 *  3. amax == 0: s_enc = k = g = 0.  Otherwise s_enc = 2688/amax,
 *     k = 448/amax, g = amax/2688 (2688 = 6 * 448 maps the tensor maximum to
 *     the largest element times the largest scale).  meta = {amax, g}.
 *  4. per block b: amax_b = max_j |Y|; S_b = E4M3(amax_b * k) (RNE, sat);
 *     m_b = (S_b == 0) ? 0 : s_enc / S_b.
 *  5. per element v = Y * m_b, coded by RNE or SR (16 Philox bits).
 *  6. two codes per byte, even element in the low nibble.
 * Output layout: codes[o][K/2], scales[o][K/16], meta[2].
 * amax_in: NULL, or a supplied tensor amax that replaces step 2 (the scale
 * level the producer of x already knows; a smaller value than the true
 * maximum saturates: block scales at 448, codes at 6).
 * outer0: index of the first output row of x within a larger tensor (0 for
 * a whole tensor).  It only shifts the SR element index, i = (outer0 + o)*K
 * + k, so a slice of a tensor too large for this reference -- quantized
 * with that tensor's amax supplied -- gets the codes of its rows in the
 * whole tensor. */
int oracle_quantize(const void *x, int dtype, int64_t rows, int64_t cols,
                    int axis, int rounding, uint64_t seed, uint64_t offset,
                    int rht, uint32_t sign_mask, const float *amax_in,
                    int64_t outer0,
                    uint8_t *codes, uint8_t *scales, float *meta)
{
    if (rows < 0 || cols < 0 || outer0 < 0) return -2;
    int64_t outer = axis ? rows : cols;
    int64_t K = axis ? cols : rows;
    if (K % 16 != 0) return -2;
    int64_t nb = K / 16;

    /* step 2: tensor amax (unless supplied) */
    uint32_t amax_bits = 0;
#pragma omp parallel for reduction(max : amax_bits) schedule(static)
    for (int64_t o = 0; o < (amax_in ? 0 : outer); ++o) {
        for (int64_t b = 0; b < nb; ++b) {
            float y[16];
            load_block(x, dtype, rows, cols, axis, rht, sign_mask, o, b, y);
            for (int j = 0; j < 16; ++j) {
                uint32_t a = f32_bits(y[j]) & 0x7FFFFFFFu;
                if (a > amax_bits) amax_bits = a;
            }
        }
    }
    float amax = amax_in ? *amax_in : bits_f32(amax_bits);

    /* step 3: tensor scales */
    float s_enc, kk, g;
    if (amax == 0.0f) {
        s_enc = 0.0f; kk = 0.0f; g = 0.0f;
    } else {
        s_enc = 2688.0f / amax;
        kk = 448.0f / amax;
        g = amax / 2688.0f;
    }
    meta[0] = amax;
    meta[1] = g;
    if (!isfinite(amax)) return 0;

    /* steps 4-6 */
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t b = 0; b < nb; ++b) {
            float y[16];
            load_block(x, dtype, rows, cols, axis, rht, sign_mask, o, b, y);
            uint32_t bmax = 0;
            for (int j = 0; j < 16; ++j) {
                uint32_t a = f32_bits(y[j]) & 0x7FFFFFFFu;
                if (a > bmax) bmax = a;
            }
            float amax_b = bits_f32(bmax);
            uint8_t S = oracle_e4m3_rne_sat(amax_b * kk);
            float Sf = oracle_e4m3_value(S);
            float m = (S == 0) ? 0.0f : s_enc / Sf;
            scales[o * nb + b] = S;
            uint8_t q[16];
            for (int j = 0; j < 16; ++j) {
                float v = y[j] * m;
                if (rounding == OR_SR) {
                    uint64_t i = (uint64_t)(outer0 + o) * (uint64_t)K + (uint64_t)(16 * b + j);
                    q[j] = oracle_e2m1_sr(v, oracle_sr_bits(seed, offset, i));
                } else {
                    q[j] = oracle_e2m1_rne(v);
                }
            }
            for (int j = 0; j < 8; ++j)
                codes[o * (K / 2) + 8 * b + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantize and exact decode                                              */
/* ------------------------------------------------------------------------ */

/* Decoded value of element (o, k): (q * S_b) * g in binary32.  q * S_b is
 * exact (at most 6 significant bits); the product with g is one rounding.
 * y_dtype 0 writes f32, 1 writes bf16 (nearest-even of the f32 value). */
int oracle_dequantize(const uint8_t *codes, const uint8_t *scales,
                      const float *meta, int64_t outer, int64_t K,
                      int y_dtype, void *y)
{
    if (outer < 0 || K < 0 || K % 16 != 0) return -2;
    float g = meta[1];
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = codes[o * (K / 2) + k / 2];
            uint8_t q = (k & 1) ? (byte >> 4) : (byte & 15);
            float S = oracle_e4m3_value(scales[o * (K / 16) + k / 16]);
            float v = (oracle_e2m1_value(q) * S) * g;
            if (y_dtype == OR_BF16) ((uint16_t *)y)[o * K + k] = f32_to_bf16_rne(v);
            else ((float *)y)[o * K + k] = v;
        }
    }
    return 0;
}

/* q * S_b for the selected outer rows, as exact doubles.  The GEMM oracle
 * multiplies these matrices in double and applies g_A * g_B afterwards. */
int oracle_decode_qs(const uint8_t *codes, const uint8_t *scales, int64_t K,
                     const int64_t *rows_sel, int64_t n_sel, double *out)
{
    if (K < 0 || K % 16 != 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_sel; ++r) {
        int64_t o = rows_sel[r];
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = codes[o * (K / 2) + k / 2];
            uint8_t q = (k & 1) ? (byte >> 4) : (byte & 15);
            double S = (double)oracle_e4m3_value(scales[o * (K / 16) + k / 16]);
            out[r * K + k] = (double)oracle_e2m1_value(q) * S;
        }
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------- MXFP4 ----
 * The microscaling format the pages set NVFP4 against ([P4] "Architektura
 * NVFP4 kontra ograniczenia mikroskalowania": blocks of 32 elements sharing
 * a power-of-two scale; the comparison with MXFP4 in the same article's
 * closing section).  Elements are E2M1 as for NVFP4; each 32-block along K
 * carries one 8-bit biased exponent (E8M0: scale = 2^(code - 127)); there is
 * no tensor-level scale.
 * Readings (the pages give no formula): the block scale is the smallest
 * power of two X = 2^e with amax_b / X <= 6, so the block maximum is never
 * clipped, e clamped to [-127, 127]; an all-zero block takes e = -127.
 * Elements are the nearest-even E2M1 code of x / X (exact: X is a power of
 * two), codes packed two per byte as for NVFP4. */

/* Smallest e with amax <= 6 * 2^e, from the bit pattern of amax >= 0.
 * 6 * 2^e = 1.5 * 2^(e+2): for amax = m * 2^E (m in [1,2)) that is e = E - 2
 * when m <= 1.5, else e = E - 1.  Subnormal amax fits e = -127. */
int oracle_mx_scale_exp(uint32_t amax_bits)
{
    amax_bits &= 0x7FFFFFFFu;
    if (amax_bits < 0x00800000u) return -127;          /* zero or subnormal */
    int E = (int)(amax_bits >> 23) - 127;
    uint32_t mant = amax_bits & 0x7FFFFFu;
    int e = (mant <= 0x400000u) ? E - 2 : E - 1;        /* m <= 1.5 ? */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int oracle_mxfp4_quantize(const void *x, int dtype, int64_t rows, int64_t cols,
                          int axis, uint8_t *codes, uint8_t *scales)
{
    if (rows < 0 || cols < 0) return -2;
    int64_t outer = axis ? rows : cols;
    int64_t K = axis ? cols : rows;
    if (K % 32 != 0) return -2;
    int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t b = 0; b < nb; ++b) {
            float y[32];
            uint32_t bmax = 0;
            for (int j = 0; j < 32; ++j) {
                y[j] = view_get(x, dtype, rows, cols, axis, o, 32 * b + j);
                uint32_t a = f32_bits(y[j]) & 0x7FFFFFFFu;
                if (a > bmax) bmax = a;
            }
            int e = oracle_mx_scale_exp(bmax);
            scales[o * nb + b] = (uint8_t)(e + 127);
            uint8_t q[32];
            for (int j = 0; j < 32; ++j)
                q[j] = oracle_e2m1_rne((float)ldexp((double)y[j], -e));
            for (int j = 0; j < 16; ++j)
                codes[o * (K / 2) + 16 * b + j] = (uint8_t)(q[2 * j] | (q[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* Exact value q * 2^(code - 127) of the selected outer rows, as doubles. */
int oracle_mxfp4_decode(const uint8_t *codes, const uint8_t *scales, int64_t K,
                        const int64_t *rows_sel, int64_t n_sel, double *out)
{
    if (K < 0 || K % 32 != 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_sel; ++r) {
        int64_t o = rows_sel[r];
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = codes[o * (K / 2) + k / 2];
            uint8_t q = (k & 1) ? (byte >> 4) : (byte & 15);
            int e = (int)scales[o * (K / 32) + k / 32] - 127;
            out[r * K + k] = ldexp((double)oracle_e2m1_value(q), e);
        }
    }
    return 0;
}

/* ------------------------------------------------------------- MXFP8 ----
 * The 8-bit member of the microscaling family: one of the three number
 * formats of the training run in [P3] "Drei Formate, ein Trainingslauf"
 * (about 5 PFLOPS on GB300), and the block layout NVFP4 is contrasted with
 * in [P4] "Architektura NVFP4 kontra ograniczenia mikroskalowania" (blocks of
 * 32 elements sharing a power-of-two scale).  Elements are OCP E4M3FN (bias
 * 7, largest 448, subnormals down to 2^-9), one byte each; each 32-block
 * along K carries one E8M0 exponent (scale 2^(code - 127)); no tensor scale.
 * Readings, as for MXFP4: the block scale is the smallest power of two
 * X = 2^e with amax_b / X <= 448, so the block maximum is never clipped, e
 * clamped to [-127, 127], an all-zero block takes e = -127; each element is
 * the nearest-even E4M3 code of x / X with the sign of x kept (-0.0 and
 * negatives that round to zero give 0x80). */

/* Smallest e with amax <= 448 * 2^e, from the bit pattern of amax >= 0.
 * 448 * 2^e = 1.75 * 2^(e+8): for amax = m * 2^E (m in [1,2)) that is
 * e = E - 8 when m <= 1.75, else e = E - 7.  Zero and subnormal maxima fit
 * e = -127. */
int oracle_mx8_scale_exp(uint32_t amax_bits)
{
    amax_bits &= 0x7FFFFFFFu;
    if (amax_bits < 0x00800000u) return -127;
    int E = (int)(amax_bits >> 23) - 127;
    uint32_t mant = amax_bits & 0x7FFFFFu;
    int e = (mant <= 0x600000u) ? E - 8 : E - 7;        /* m <= 1.75 ? */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e;
}

int oracle_mxfp8_quantize(const void *x, int dtype, int64_t rows, int64_t cols,
                          int axis, uint8_t *codes, uint8_t *scales)
{
    if (rows < 0 || cols < 0) return -2;
    int64_t outer = axis ? rows : cols;
    int64_t K = axis ? cols : rows;
    if (K % 32 != 0) return -2;
    int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o) {
        for (int64_t b = 0; b < nb; ++b) {
            float y[32];
            uint32_t bmax = 0;
            for (int j = 0; j < 32; ++j) {
                y[j] = view_get(x, dtype, rows, cols, axis, o, 32 * b + j);
                uint32_t a = f32_bits(y[j]) & 0x7FFFFFFFu;
                if (a > bmax) bmax = a;
            }
            int e = oracle_mx8_scale_exp(bmax);
            scales[o * nb + b] = (uint8_t)(e + 127);
            for (int j = 0; j < 32; ++j) {
                /* x / 2^e is exact in double; its magnitude is <= 448, so the
                 * binary32 cast is exact down to 2^-149, far below half the
                 * smallest E4M3 step (2^-10) */
                float v = (float)ldexp((double)y[j], -e);
                uint8_t sign = signbit(v) ? 0x80 : 0x00;
                codes[o * K + 32 * b + j] = (uint8_t)(sign | oracle_e4m3_rne_sat(fabsf(v)));
            }
        }
    }
    return 0;
}

/* Exact value e4m3(code) * 2^(scale - 127) of the selected outer rows. */
int oracle_mxfp8_decode(const uint8_t *codes, const uint8_t *scales, int64_t K,
                        const int64_t *rows_sel, int64_t n_sel, double *out)
{
    if (K < 0 || K % 32 != 0) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n_sel; ++r) {
        int64_t o = rows_sel[r];
        for (int64_t k = 0; k < K; ++k) {
            int e = (int)scales[o * (K / 32) + k / 32] - 127;
            out[r * K + k] = ldexp((double)oracle_e4m3_value(codes[o * K + k]), e);
        }
    }
    return 0;
}

/* Checker (part of the tolerance, not of the method): the most the FP8
 * block-scaled MFMA can lose to its product truncation, per output element.
 * Reading of the instruction, from device measurements on MI355X: the 64
 * products of one instruction are summed in groups of 8 consecutive K
 * positions (aligned runs of 8); within a group every product is truncated
 * toward zero to a multiple of 2^(E - 13), where E is the largest
 * exponent(a) + exponent(b) over the group plus the two block-scale
 * exponents (exponent(x) = floor(log2|x|) for a normal E4M3 value, -6 for a
 * subnormal or zero); group results and the accumulator are then added and
 * rounded to binary32 once.  A product with exponent(a) + exponent(b) >= E - 7
 * has no bits below 2^(E - 13) and is exact; any other loses less than
 * min(|p|, 2^(E - 13)).  out[i][j] = the sum of those losses over all groups
 * of row rows_a[i] of A and row rows_b[j] of B (K % 32 == 0). */
static int e4m3_exponent(uint8_t c)
{
    int f = (c >> 3) & 15;
    return f == 0 ? -6 : f - 7;
}

int oracle_mxfp8_trunc_bound(const uint8_t *codes_a, const uint8_t *scales_a,
                             const uint8_t *codes_b, const uint8_t *scales_b, int64_t K,
                             const int64_t *rows_a, int64_t na,
                             const int64_t *rows_b, int64_t nb, double *out)
{
    if (K < 0 || K % 32 != 0) return -2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < na; ++i) {
        for (int64_t j = 0; j < nb; ++j) {
            const uint8_t *a = codes_a + rows_a[i] * K, *b = codes_b + rows_b[j] * K;
            const uint8_t *sa = scales_a + rows_a[i] * (K / 32), *sb = scales_b + rows_b[j] * (K / 32);
            double t = 0.0;
            for (int64_t g = 0; g < K / 8; ++g) {
                int s = ((int)sa[g / 4] - 127) + ((int)sb[g / 4] - 127);
                int ex[8], E = -1000;
                for (int q = 0; q < 8; ++q) {
                    ex[q] = e4m3_exponent(a[8 * g + q]) + e4m3_exponent(b[8 * g + q]);
                    if (ex[q] > E) E = ex[q];
                }
                double unit = ldexp(1.0, E + s - 13);
                for (int q = 0; q < 8; ++q) {
                    if (ex[q] >= E - 7) continue;
                    double p = fabs((double)oracle_e4m3_value(a[8 * g + q]) *
                                    (double)oracle_e4m3_value(b[8 * g + q])) * ldexp(1.0, s);
                    t += p < unit ? p : unit;
                }
            }
            out[i * nb + j] = t;
        }
    }
    return 0;
}
