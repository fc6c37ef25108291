// nvfp4_device.h -- gfx950 device helpers for the NVFP4 kernels.
//
// Format ([P4] aisight.pl "Koniec marnowania mocy ...", section "Architektura
// NVFP4 kontra ograniczenia mikroskalowania"): 4-bit E2M1 elements, one
// E4M3 scale per 16 elements along the reduction dimension, one FP32 scale
// per tensor.  Every helper here is written for CDNA4 and relies on four
// measured properties of gfx950:
//  * v_cvt_scalef32_pk_fp4_f32 with scale 1.0 rounds binary32 to E2M1
//    nearest-even (ties to the even code), saturates at 6 and keeps the sign
//    of zero;
//  * v_cvt_scalef32_pk_f16_fp4 with scale 1.0 decodes E2M1 exactly (its scale
//    operand only contributes its exponent, so the E4M3 block scale is
//    applied with a separate exact f16 multiply);
//  * v_cvt_scalef32_sr_pk_fp4_f32 with scale 1.0 rounds the first value of
//    its pair up iff rand >= (1 - frac) * 2^32 (add-and-truncate on the
//    discarded fraction), saturating at 6 and keeping the sign;
//  * v_cvt_f32_fp8 decodes OCP E4M3FN, binary32 denormals are kept and
//    __fdiv_rn is the correctly rounded quotient.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

// Tensor-level constants: 2688 = 6 * 448 maps the tensor maximum onto the
// largest element (6) times the largest block scale (448).
constexpr float kTensorRange = 2688.0f;
constexpr float kScaleMax = 448.0f;

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Load 16 consecutive elements (bf16 or f32) starting at p (16-byte aligned)
// as binary32 values.
template <typename T> struct Load16;
template <> struct Load16<uint16_t> {
  __device__ __forceinline__ static void run(const uint16_t *p, float *y) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 a = q[0], b = q[1];
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) { y[2 * i] = bf16_lo(w[i]); y[2 * i + 1] = bf16_hi(w[i]); }
  }
};
template <> struct Load16<float> {
  __device__ __forceinline__ static void run(const float *p, float *y) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v = q[i];
      y[4 * i] = v.x; y[4 * i + 1] = v.y; y[4 * i + 2] = v.z; y[4 * i + 3] = v.w;
    }
  }
};

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }

// ---------------------------------------------------------------- E4M3 ----
// Nearest-even E4M3FN code of t >= 0, saturating at 448.  Below 2^-6 the
// code is the count of 2^-9 steps: adding 2^14 (whose ulp is 2^-9) rounds t
// to that grid in one IEEE addition.  From 2^-6 up the binary32 pattern is
// rounded to three mantissa bits and the exponent is rebiased (127 -> 7).
__device__ __forceinline__ uint32_t e4m3_rne_sat(float t) {
  t = fminf(t, kScaleMax);
  if (t < 0x1p-6f) {
    float s = t + 16384.0f;
    return __float_as_uint(s) - 0x46800000u;  // 0x46800000 = bits of 2^14
  }
  uint32_t u = __float_as_uint(t);
  uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);
}

// E4M3FN code (0..0x7E) to binary32 (hardware OCP decode, exact).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// ---------------------------------------------------------------- E2M1 ----
// Two binary32 values to two E2M1 codes (nearest-even, saturating, sign of
// zero kept), written into byte `sel` of `old` (low nibble = first value).
#define NVFP4_PK_FP4(old, a, b, sel) __builtin_amdgcn_cvt_scalef32_pk_fp4_f32((old), (a), (b), 1.0f, (sel))

// Encode 8 values into one 32-bit word of nibbles (element 0 lowest).
__device__ __forceinline__ uint32_t encode8_rne(const float *v) {
  uint32_t w = 0;
  w = NVFP4_PK_FP4(w, v[0], v[1], 0);
  w = NVFP4_PK_FP4(w, v[2], v[3], 1);
  w = NVFP4_PK_FP4(w, v[4], v[5], 2);
  w = NVFP4_PK_FP4(w, v[6], v[7], 3);
  return w;
}

// Stochastic rounding ([P4] "Technologie stabilizujace ...": stochastic
// rounding removes the systematic error of ordinary rounding).  Rule: with
// frac the position of |v| between its two neighbouring grid values, round
// up iff frac + (r16 + 1/2) / 2^16 >= 1 -- add a uniform offset of
// (r16 + 1/2) / 2^16 grid steps, then truncate.  gfx950's
// v_cvt_scalef32_sr_pk_fp4_f32 (scale 1) computes, for the FIRST value of
// its pair, exactly "round up iff rand >= (1 - frac) * 2^32" (checked against
// the exact rational rule on 3.8 M (value, rand) pairs covering every
// binade, the saturation at 6, signs and tiny values), so rand =
// (r16 << 16) | 0x8000 gives the rule above.  The second value of a pair
// rounds with rand << 1 (checked bit for bit against the first-value form
// on 16.8 M (value, r16) cases), so one conversion of the pair (v[2j],
// v[2j+1]) with rand = R_even gives the even element's code in the low
// nibble, and one with rand = R_odd >> 1 (R_odd has bit 0 clear) the odd
// element's code in the high nibble; the other nibble of each is unused.
// Eight conversions, each writing one byte of a word (byte sel, the other
// bytes kept), build the even and odd words; one masked merge gives the 8
// codes.  Written as one asm block: the compiler's form of the byte-select
// conversion does not keep the destination's other bytes.  The two chains
// alternate, so no conversion reads a result of the instruction just before.
__device__ __forceinline__ uint32_t encode8_sr(const float *v, const uint32_t *w) {
  const float2_t p0 = {v[0], v[1]}, p1 = {v[2], v[3]}, p2 = {v[4], v[5]}, p3 = {v[6], v[7]};
  uint32_t re[4], ro[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    re[j] = (w[j] << 16) | 0x8000u;
    ro[j] = ((w[j] >> 1) & 0x7FFF8000u) | 0x4000u;     // ((w & 0xFFFF0000) | 0x8000) >> 1
  }
  uint32_t ev, od;
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %2, %6, 1.0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %2, %10, 1.0\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %3, %7, 1.0 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %3, %11, 1.0 op_sel:[0,0,1,0]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %4, %8, 1.0 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %4, %12, 1.0 op_sel:[0,0,0,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %0, %5, %9, 1.0 op_sel:[0,0,1,1]\n\t"
      "v_cvt_scalef32_sr_pk_fp4_f32 %1, %5, %13, 1.0 op_sel:[0,0,1,1]"
      : "=&v"(ev), "=&v"(od)
      : "v"(p0), "v"(p1), "v"(p2), "v"(p3), "v"(re[0]), "v"(re[1]), "v"(re[2]), "v"(re[3]), "v"(ro[0]),
        "v"(ro[1]), "v"(ro[2]), "v"(ro[3]));
  return (ev & 0x0F0F0F0Fu) | (od & 0xF0F0F0F0u);
}

// -------------------------------------------------------------- Philox ----
// Philox4x32-10 (Salmon et al., SC'11): ten rounds of two 32x32->64 products
// with the multipliers 0xD2511F53 / 0xCD9E8D57, word permutation, and a key
// schedule bumped by the Weyl constants 0x9E3779B9 / 0xBB67AE85.  Each
// product is one 64-bit multiply (v_mad_u64_u32 gives both halves; measured
// cheaper on gfx950 than a v_mul_hi_u32 / v_mul_lo_u32 pair) and each
// three-way XOR one v_bitop3_b32 (truth table 0x96).  The key words are wave-uniform (scalar).
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                   __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Philox output for the 8 elements with output indices 8g .. 8g+7: counter
// (lo(g), hi(g), lo(offset), hi(offset)), key (lo(seed), hi(seed)); element
// 8g+j takes half (j & 1) (low first) of word j >> 1.
__device__ __forceinline__ uint4 sr_words8(uint64_t g, uint64_t seed, uint64_t offset) {
  return philox4x32_10(make_uint4((uint32_t)g, (uint32_t)(g >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)),
                       (uint32_t)seed, (uint32_t)(seed >> 32));
}

// ----------------------------------------------------------------- RHT ----
// 16-point random Hadamard transform in registers ([P4] "Technologie
// stabilizujace ..."): sign flips from the mask, the Walsh-Hadamard
// butterfly with stages 1, 2, 4, 8 (lower index a+b, upper a-b), then the
// exact factor 1/4.
//
// The signs as factors +-1, one per element (wave-uniform).
struct RhtSigns {
  float s[16];
};
__device__ __forceinline__ RhtSigns rht_signs(uint32_t sign_mask) {
  RhtSigns r;
#pragma unroll
  for (int j = 0; j < 16; ++j) r.s[j] = ((sign_mask >> j) & 1u) ? -1.0f : 1.0f;
  return r;
}

// 4y, the transform without its factor 1/4.  The sign flips ride in the
// first stage: b = s_{j+1} x_{j+1} is an exact product, and fma(x_j, s_j, +-b)
// rounds s_j x_j +- b once, as the addition of the flipped values does, so
// every stage output is bit for bit the one of flip-then-butterfly (one
// multiply and two fused multiply-adds per pair instead of two flips and
// two additions).
__device__ __forceinline__ void rht16_x4(float *t, const RhtSigns &sg) {
#pragma unroll
  for (int j = 0; j < 16; j += 2) {
    const float b = t[j + 1] * sg.s[j + 1];
    const float a0 = __builtin_fmaf(t[j], sg.s[j], b);
    const float a1 = __builtin_fmaf(t[j], sg.s[j], -b);
    t[j] = a0;
    t[j + 1] = a1;
  }
#pragma unroll
  for (int h = 2; h < 16; h <<= 1) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j & h) continue;
      float a = t[j], b = t[j + h];
      t[j] = a + b;
      t[j + h] = a - b;
    }
  }
}

// The 1/4 of the transform moved out of the values.  amax: the maximum of
// |4y| taken as a bit pattern, then multiplied by 1/4 once (x -> x/4 is
// monotone, so this is the bit pattern of max |y| for any input; a NaN stays
// a NaN).  Encode of bf16 input: every value the butterfly forms is a
// multiple of 2^-133 (the bf16 grid): an exact sum of multiples is one, and
// a sum is rounded only from 2^-109 up, where the f32 grid is coarser.  So
// y = t/4, a multiple of 2^-135, is exact and t is exactly 4y; the block
// maximum times k/4 and the element times m/4 are then
// the same real products as y times k and m, and round the same, as long as
// k/4 and m/4 are exact: k >= 448/FLT_MAX always is, and every multiplier
// m >= s_enc/448 is when s_enc >= 2^-115 (amax below about 1.1e38).
__device__ __forceinline__ uint32_t quarter_bits(uint32_t bits) {
  return __float_as_uint(0.25f * __uint_as_float(bits));
}

// Largest |value| of 16 binary32 values as a bit pattern (exact, NaN > Inf).
__device__ __forceinline__ uint32_t absmax_bits16(const float *y) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  return m;
}

// The block maximum of an encode, 16 values as a bit pattern: eight
// v_max3_f32 with |.| source modifiers, against 16 masks and 8 integer
// maxima.  Equal to absmax_bits16 whenever no value is NaN (f32 denormals
// are kept, so subnormals compare exactly); a NaN comes only from a
// non-finite input, whose codes and scales are unspecified.  The tensor
// amax keeps the integer form, which orders NaN above Inf.  Written as asm:
// the compiler's float maximum would first quiet every operand it cannot
// prove canonical (converted bf16 values among them).
__device__ __forceinline__ float fmax3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, |%3|" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t block_absmax_bits16(const float *y) {
  float m = fmax3_abs(y[0], y[1], y[2]);
#pragma unroll
  for (int j = 3; j < 15; j += 2) m = fmax3_abs(m, y[j], y[j + 1]);
  m = fmax3_abs(m, y[15], y[15]);
  return __float_as_uint(m);
}

// ------------------------------------------------------ tensor scales ----
struct TensorScales {
  float s_enc;  // 2688 / amax
  float k;      // 448 / amax (block maxima -> E4M3 scale)
  float g;      // amax / 2688 (decode)
};

__device__ __forceinline__ TensorScales tensor_scales(float amax) {
  TensorScales s;
  if (amax == 0.0f) {
    s.s_enc = 0.0f; s.k = 0.0f; s.g = 0.0f;
  } else {
    s.s_enc = __fdiv_rn(kTensorRange, amax);
    s.k = __fdiv_rn(kScaleMax, amax);
    s.g = __fdiv_rn(amax, kTensorRange);
  }
  return s;
}

// Block scale code and element multiplier of one 16-block.
__device__ __forceinline__ uint32_t block_scale(uint32_t bmax_bits, const TensorScales &ts, float *m) {
  uint32_t S = e4m3_rne_sat(__uint_as_float(bmax_bits) * ts.k);
  *m = (S == 0u) ? 0.0f : __fdiv_rn(ts.s_enc, e4m3_to_f32(S));
  return S;
}

// The element multiplier of every block scale code (0 for code 0, codes
// past 0x7E unused): the same correctly rounded quotients block_scale
// computes, one division per code and workgroup instead of one per block.
// Threads [t0, t0 + 128) fill it; the caller puts a barrier before any use.
__device__ __forceinline__ void fill_scale_lut(float *lut, const TensorScales &ts, int t0) {
  const int i = (int)threadIdx.x - t0;
  if (i >= 0 && i < 128) lut[i] = (i == 0 || i > 0x7E) ? 0.0f : __fdiv_rn(ts.s_enc, e4m3_to_f32((uint32_t)i));
}

// The tensor scales for block values taken as 4y (the transform without its
// 1/4): k/4 and s_enc/4, so block scales and multipliers come out as for y
// (the multipliers as m/4).  Exact when s_enc >= 2^-115 (quarter_exact):
// then k/4, s_enc/4 and every s_enc/4 / e4m3(S) >= s_enc / 1792 are normal,
// and a quotient scaled by a power of two rounds the same.  g is kept.
__device__ __forceinline__ bool quarter_exact(const TensorScales &ts) { return ts.s_enc >= 0x1p-115f; }
__device__ __forceinline__ TensorScales quarter_scales(const TensorScales &ts) {
  TensorScales q = ts;
  q.k = 0.25f * ts.k;
  q.s_enc = 0.25f * ts.s_enc;
  return q;
}

__device__ __forceinline__ uint32_t block_scale_lut(uint32_t bmax_bits, const TensorScales &ts, const float *lut,
                                                    float *m) {
  const uint32_t S = e4m3_rne_sat(__uint_as_float(bmax_bits) * ts.k);
  *m = lut[S];
  return S;
}

// Quantize 16 values with their multiplier m; returns the 8 code bytes as
// two words.  RNE uses the hardware conversion, SR the Philox bits of the
// block (output indices 16*blk .. 16*blk+15 have counters 2*blk and 2*blk+1).
template <bool SR>
__device__ __forceinline__ uint2 encode16(const float *y, float m, uint64_t blk, uint64_t seed,
                                          uint64_t offset) {
  float v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = y[j] * m;
  if (!SR) {
    return make_uint2(encode8_rne(v), encode8_rne(v + 8));
  } else {
    const uint4 a = sr_words8(2 * blk, seed, offset), b = sr_words8(2 * blk + 1, seed, offset);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
    const uint32_t w0 = encode8_sr(v, wa), w1 = encode8_sr(v + 8, wb);
    return make_uint2(w0, w1);
  }
}

}  // namespace nvfp4
