// quantize.hip -- NVFP4 quantizer kernels for gfx950: tensor amax,
// block-scaled E2M1 encode (nearest-even or Philox stochastic rounding),
// optional fused 16-point random Hadamard transform, and dequantize.
//
// Format and recipe: [P4] aisight.pl "Koniec marnowania mocy ...", sections
// "Architektura NVFP4 kontra ograniczenia mikroskalowania" (16-element
// blocks, E4M3 block scale, FP32 tensor scale) and "Technologie
// stabilizujace proces treningowy" (random Hadamard transform, stochastic
// rounding); [P3] aibuzzwire.news "End-to-End 4-Bit Training" article,
// section "Warum weniger Bits ein schnelleres Training bedeuten" (rounding to
// the nearest representable value).
//
// Pass structure: the per-tensor scale needs the whole-tensor maximum before
// any block can be encoded, so a quantization is (1) a one-thread kernel that
// zeroes meta, (2) an amax kernel (integer max of |x| bit patterns, wave
// reduction, one atomicMax per workgroup), (3) the encode kernel, which
// re-reads the input.  Both passes are HBM-bound:
//  * the amax pass streams one contiguous chunk per workgroup with four
//    16-byte loads in flight per thread;
//  * the encode pass walks the tensor in the opposite order of the amax
//    pass, so its first part is still resident in the 256 MB MALL;
//  * axis 0 (K runs down the columns; the output is the transpose) gives
//    each thread two adjacent columns and four consecutive blocks: rows are
//    read as 1 KB contiguous runs per workgroup and each output row gets 32
//    code bytes and 4 scale bytes from one thread.
#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kQT = kQuantThreads;

// Wide stores are taken only where the destination address itself is
// aligned: output buffers need only the alignment of their element type.
__device__ __forceinline__ bool aligned_to(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Streaming (non-temporal) stores for outputs written as contiguous runs:
// the lines are not kept in the caches ahead of the input still to be read.
// Measured on the 32768 x 8192 bf16 tensor: the axis-1 quantizations 5-6 %
// faster; the axis-0 ones, whose output is 128-byte lines 16 KB apart, 7 %
// slower, so those keep ordinary stores.  Quantized codes are read next by
// a GEMM, which finds them in the last-level cache when they were stored
// the ordinary way: the axis-1 encode streams its output only for inputs
// larger than that cache (kStreamOutBytes), and the dual encode not at all.
typedef unsigned nt_u2 __attribute__((ext_vector_type(2)));
typedef unsigned nt_u4 __attribute__((ext_vector_type(4)));
// the MI355X last-level cache (MALL): 256 MB
constexpr int64_t kStreamOutBytes = (int64_t)256 << 20;
__device__ __forceinline__ void store_nt(uint2 *p, uint2 v) {
  __builtin_nontemporal_store((nt_u2){v.x, v.y}, reinterpret_cast<nt_u2 *>(p));
}
__device__ __forceinline__ void store_nt(uint4 *p, uint4 v) {
  __builtin_nontemporal_store((nt_u4){v.x, v.y, v.z, v.w}, reinterpret_cast<nt_u4 *>(p));
}
__device__ __forceinline__ void store_nt(float4 *p, float4 v) {
  __builtin_nontemporal_store((nt_u4){__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                                      __float_as_uint(v.w)},
                              reinterpret_cast<nt_u4 *>(p));
}
__device__ __forceinline__ void store_nt(uint32_t *p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store_nt(uint8_t *p, uint8_t v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Reduce a per-thread max over the workgroup and fold it into *dst.  Atomics
// on one address serialise in L2 (thousands of workgroups each issuing one
// cost tens of microseconds), so the current value is read first (relaxed,
// device scope: not from a stale L1 line) and the atomic is issued only when
// this workgroup can raise it.  The result is the same maximum: a skipped
// update was already dominated by a value in *dst, and *dst only grows.
__device__ __forceinline__ void block_max_atomic(uint32_t v, uint32_t *dst) {
  __shared__ uint32_t part[kQT / 64];
  v = wave_max(v);
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = part[0];
#pragma unroll
    for (int i = 1; i < kQT / 64; ++i) m = max(m, part[i]);
    const uint32_t cur = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m > cur) atomicMax(dst, m);
  }
}

// block_max_atomic for two maxima at once (one LDS round).
__device__ __forceinline__ void block_max2_atomic(uint32_t v0, uint32_t *dst0, uint32_t v1, uint32_t *dst1) {
  __shared__ uint32_t part2[2][kQT / 64];
  v0 = wave_max(v0);
  v1 = wave_max(v1);
  int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    part2[0][wave] = v0;
    part2[1][wave] = v1;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    const int t = threadIdx.x;
    uint32_t m = part2[t][0];
#pragma unroll
    for (int i = 1; i < kQT / 64; ++i) m = max(m, part2[t][i]);
    uint32_t *dst = t ? dst1 : dst0;
    const uint32_t cur = __hip_atomic_load(dst, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (m > cur) atomicMax(dst, m);
  }
}

__global__ void k_meta_init(float *meta) {
  if (threadIdx.x == 0) {
    meta[0] = 0.0f;
    meta[1] = 0.0f;
  }
}

// meta = {supplied amax, 0}: the encode pass reads meta[0] and writes meta[1].
__global__ void k_meta_set(float *meta, const float *amax) {
  if (threadIdx.x == 0) {
    meta[0] = amax[0];
    meta[1] = 0.0f;
  }
}

__global__ void k_zero1(float *v) {
  if (threadIdx.x == 0) v[0] = 0.0f;
}

__global__ void k_meta_init2(float *meta_a, float *meta_b) {
  if (threadIdx.x == 0) {
    meta_a[0] = 0.0f;
    meta_a[1] = 0.0f;
    meta_b[0] = 0.0f;
    meta_b[1] = 0.0f;
  }
}

// |x| bit-pattern maximum of one 16-byte vector of T (bf16: packed 16-bit
// maxima of the magnitudes, returned as the f32 bit pattern).
template <typename T> __device__ __forceinline__ uint32_t vec_absmax(uint4 v);
template <> __device__ __forceinline__ uint32_t vec_absmax<uint16_t>(uint4 v) {
  ushort2_t acc = __builtin_bit_cast(ushort2_t, v.x & 0x7FFF7FFFu);
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(ushort2_t, v.y & 0x7FFF7FFFu));
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(ushort2_t, v.z & 0x7FFF7FFFu));
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(ushort2_t, v.w & 0x7FFF7FFFu));
  return (uint32_t)max(acc.x, acc.y) << 16;
}
template <> __device__ __forceinline__ uint32_t vec_absmax<float>(uint4 v) {
  return max(max(v.x & 0x7FFFFFFFu, v.y & 0x7FFFFFFFu), max(v.z & 0x7FFFFFFFu, v.w & 0x7FFFFFFFu));
}

// --------------------------------------------------------------- amax ----

// Input reads of the single-pass-over-the-data loops (the flat amax and
// the three axis-0 column kernels) carry the nontemporal hint: each input
// line is read once per pass.  Measured on the 32768 x 8192 bf16 tensor,
// same GPU, bit-identical: axis-0 RNE 238.7 -> 214.4 us per quantization,
// axis-0 SR 240.6 -> 227.9, the other variants and the dual-layout
// quantization of dY within the spread.  (The axis-1 encodes read their
// 32-byte blocks with ordinary loads: the hint on those slowed the variants
// with the transform by 15 us.)
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  const nt_u4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Flat amax over n16 16-byte vectors (no transform; the axis does not
// matter).  Each workgroup streams one contiguous chunk with four loads in
// flight per thread (measured on MI355X: contiguous chunks per workgroup
// read ~15 % faster than a grid-wide stride, which spreads every wave's
// accesses over the whole tensor).
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_flat(const uint4 *x, int64_t n16, int64_t per_wg, uint32_t *amax_bits,
                                                  uint32_t *amax_bits2) {
  uint32_t m = 0;
  const int64_t beg = (int64_t)blockIdx.x * per_wg;
  const int64_t end = beg + per_wg < n16 ? beg + per_wg : n16;
  int64_t i = beg + threadIdx.x;
  for (; i + 3 * kQT < end; i += 4 * kQT) {
    const uint4 v0 = load_nt(x + i), v1 = load_nt(x + i + kQT), v2 = load_nt(x + i + 2 * kQT),
                v3 = load_nt(x + i + 3 * kQT);
    m = max(max(m, vec_absmax<T>(v0)), max(vec_absmax<T>(v1), max(vec_absmax<T>(v2), vec_absmax<T>(v3))));
  }
  for (; i < end; i += kQT) m = max(m, vec_absmax<T>(load_nt(x + i)));
  if (amax_bits2)   // the same maximum for a second tensor (dual-layout quantize)
    block_max2_atomic(m, amax_bits, m, amax_bits2);
  else
    block_max_atomic(m, amax_bits);
}

// amax of the transformed tensor, axis 1: 16-chunks of rows, one contiguous
// range of chunks per workgroup, two chunks in flight per thread.
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_rht_rows(const T *x, int64_t nchunks, int64_t per_wg, uint32_t sign_mask,
                                                      uint32_t *amax_bits) {
  const RhtSigns sg = rht_signs(sign_mask);
  uint32_t m = 0;                    // max |4y| (bit pattern)
  const int64_t beg = (int64_t)blockIdx.x * per_wg;
  const int64_t end = beg + per_wg < nchunks ? beg + per_wg : nchunks;
  int64_t c = beg + threadIdx.x;
  for (; c + kQT < end; c += 2 * kQT) {
    float y0[16], y1[16];
    Load16<T>::run(x + 16 * c, y0);
    Load16<T>::run(x + 16 * (c + kQT), y1);
    rht16_x4(y0, sg);
    rht16_x4(y1, sg);
    m = max(m, max(absmax_bits16(y0), absmax_bits16(y1)));
  }
  for (; c < end; c += kQT) {
    float y[16];
    Load16<T>::run(x + 16 * c, y);
    rht16_x4(y, sg);
    m = max(m, absmax_bits16(y));
  }
  block_max_atomic(quarter_bits(m), amax_bits);
}

// ------------------------------------------------------- axis 0 ----
//
// K runs down the columns.  A thread owns kCPT adjacent columns (two bf16
// columns share one 4-byte load, f32 takes one) and kNBT consecutive
// 16-row blocks, so a wave reads 256 contiguous bytes of each row, and each
// output row (= input column) receives kNBT code words (32 bytes) and kNBT
// scale bytes from one thread.  The encode's four waves share their columns
// and take consecutive block groups (one 128-byte output line per column);
// the amax pass of the RHT path uses 256 * kCPT columns x kNBT blocks per
// workgroup.
constexpr int kNBT = 4;

template <typename T>
struct ColPairs {
  static constexpr int kCPT = 4 / (int)sizeof(T);   // columns per thread
};

// The 16 values of block kb of columns c .. c + kCPT - 1 (binary32; columns
// past `cols` read as zero).  `fast`: one aligned 4-byte load per row, with
// the nontemporal hint (see load_nt).
template <typename T>
__device__ __forceinline__ void load_col_block(const T *x, int64_t cols, int64_t kb, int64_t c, bool fast,
                                               float (*y)[16]) {
  constexpr int CPT = ColPairs<T>::kCPT;
  const T *p = x + 16 * kb * cols + c;
  if (fast) {
    uint32_t w[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) w[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + j * cols));
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if constexpr (CPT == 2) {
        y[0][j] = bf16_lo(w[j]);
        y[1][j] = bf16_hi(w[j]);
      } else {
        y[0][j] = __uint_as_float(w[j]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < CPT; ++e)
#pragma unroll
      for (int j = 0; j < 16; ++j) y[e][j] = (c + e < cols) ? to_f32<T>(p[j * cols + e]) : 0.0f;
  }
}

// amax of the transformed tensor, axis 0 (16-row chunks of each column).
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_rht_cols(const T *x, int64_t rows, int64_t cols, uint32_t sign_mask,
                                                      uint32_t *amax_bits) {
  constexpr int CPT = ColPairs<T>::kCPT;
  const int64_t c = ((int64_t)blockIdx.x * kQT + threadIdx.x) * CPT;
  const int64_t nkb = rows / 16, kb0 = (int64_t)blockIdx.y * kNBT;
  const bool fast = (c + CPT <= cols) && (CPT == 1 || (cols % 2) == 0);
  const RhtSigns sg = rht_signs(sign_mask);
  uint32_t m = 0;                    // max |4y| (bit pattern)
  if (c < cols) {
#pragma unroll
    for (int i = 0; i < kNBT; ++i) {
      if (kb0 + i >= nkb) break;
      float y[CPT][16];
      load_col_block<T>(x, cols, kb0 + i, c, fast, y);
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        rht16_x4(y[e], sg);
        m = max(m, absmax_bits16(y[e]));
      }
    }
  }
  block_max_atomic(quarter_bits(m), amax_bits);
}

// Dual-layout amax: one read of x gives the plain maximum (for the axis-1
// output) and the maximum after the column transform (for the axis-0 RHT
// output).
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_dual_cols(const T *x, int64_t rows, int64_t cols, uint32_t sign_mask,
                                                       uint32_t *plain_bits, uint32_t *rht_bits) {
  constexpr int CPT = ColPairs<T>::kCPT;
  const int64_t c = ((int64_t)blockIdx.x * kQT + threadIdx.x) * CPT;
  const int64_t nkb = rows / 16, kb0 = (int64_t)blockIdx.y * kNBT;
  const bool fast = (c + CPT <= cols) && (CPT == 1 || (cols % 2) == 0);
  const RhtSigns sg = rht_signs(sign_mask);
  uint32_t mp = 0, mr = 0;           // max |x|, max |4y| (bit patterns)
  if (c < cols) {
#pragma unroll
    for (int i = 0; i < kNBT; ++i) {
      if (kb0 + i >= nkb) break;
      float y[CPT][16];
      load_col_block<T>(x, cols, kb0 + i, c, fast, y);
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        mp = max(mp, absmax_bits16(y[e]));
        rht16_x4(y[e], sg);
        mr = max(mr, absmax_bits16(y[e]));
      }
    }
  }
  block_max2_atomic(mp, plain_bits, quarter_bits(mr), rht_bits);
}

// ------------------------------------------------------------- encode ----

// axis 1: one thread per 16-block (o, b); codes are 8 contiguous bytes.  The
// blocks are visited from the end of the tensor backwards (the amax pass
// went forwards), so the most recently read part is encoded first.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(kQT) k_quant_rows(const T *x, int64_t nblocks, uint32_t sign_mask, uint64_t seed,
                                                   uint64_t offset, float *meta, uint2 *codes, uint8_t *scales,
                                                   bool stream_out) {
  const float amax = meta[0];
  const TensorScales ts = tensor_scales(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) meta[1] = ts.g;
  // with the transform on bf16 input, the blocks are taken as 4y and the
  // scales as k/4, s_enc/4 where that is exact (see quarter_scales)
  const bool fold = RHT && sizeof(T) == 2 && quarter_exact(ts);
  const TensorScales tb = fold ? quarter_scales(ts) : ts;
  const RhtSigns sg = rht_signs(sign_mask);
  // stochastic rounding walks several blocks per thread: their multipliers
  // come from a per-workgroup table
  __shared__ float lut[128];
  if constexpr (SR) {
    fill_scale_lut(lut, tb, 0);
    __syncthreads();
  }
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t i = (int64_t)blockIdx.x * kQT + threadIdx.x; i < nblocks; i += stride) {
    const int64_t b = nblocks - 1 - i;
    float y[16];
    Load16<T>::run(x + 16 * b, y);
    if (RHT) {
      rht16_x4(y, sg);
      if (!fold) {
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = 0.25f * y[j];
      }
    }
    float m;
    const uint32_t bmax = block_absmax_bits16(y);
    uint32_t S = SR ? block_scale_lut(bmax, tb, lut, &m) : block_scale(bmax, tb, &m);
    const uint2 cw = encode16<SR>(y, m, (uint64_t)b, seed, offset);
    if (stream_out) {
      store_nt(codes + b, cw);
      store_nt(scales + b, (uint8_t)S);
    } else {
      codes[b] = cw;
      scales[b] = (uint8_t)S;
    }
  }
}

// axis 0: output row o = input column, block kb = 16-row group; the blocks
// are visited in reverse order of the amax pass.  Stochastic rounding
// without the transform is held to five waves per SIMD (85 VGPRs instead of
// 138 at three): 32768 x 8192 bf16 227.8 -> 219.5 us per quantization on one
// GPU, bit-identical; the same bound spills in the other instances.
template <bool SR, bool RHT>
constexpr int kColsMinWaves = SR && !RHT ? 5 : 1;

template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(kQT) __attribute__((amdgpu_waves_per_eu(kColsMinWaves<SR, RHT>, 8))) k_quant_cols(const T *x, int64_t rows, int64_t cols, uint32_t sign_mask,
                                                   uint64_t seed, uint64_t offset, float *meta, uint2 *codes,
                                                   uint8_t *scales) {
  constexpr int CPT = ColPairs<T>::kCPT;
  const float amax = meta[0];
  const TensorScales ts = tensor_scales(amax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) meta[1] = ts.g;
  // The four waves of a workgroup take the same 64 * CPT columns and four
  // consecutive groups of kNBT blocks, so they write the four 32-byte pieces
  // of each 128-byte output line together: the line is complete in L2
  // before it is written back (pieces from different workgroups, possibly on
  // different XCDs, left L2 as partial lines: +25-45 % HBM write bytes).
  static_assert(kQT == 256, "four waves per workgroup");
  // with the transform on bf16 input, the blocks are taken as 4y and the
  // scales as k/4, s_enc/4 where that is exact (see quarter_scales)
  const bool fold = RHT && sizeof(T) == 2 && quarter_exact(ts);
  const TensorScales tb = fold ? quarter_scales(ts) : ts;
  const RhtSigns sg = rht_signs(sign_mask);
  __shared__ float lut[128];         // multipliers of the block scale codes
  fill_scale_lut(lut, tb, 0);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = ((int64_t)(gridDim.x - 1 - blockIdx.x) * 64 + lane) * CPT;
  const int64_t nkb = rows / 16, kb0 = ((int64_t)(gridDim.y - 1 - blockIdx.y) * 4 + wave) * kNBT;
  if (c >= cols || kb0 >= nkb) return;
  const bool fast = (c + CPT <= cols) && (CPT == 1 || (cols % 2) == 0);
  const int nb = (int)(nkb - kb0 < kNBT ? nkb - kb0 : kNBT);
  uint2 cw[CPT][kNBT];
  uint32_t sc[CPT] = {};
#pragma unroll
  for (int i = 0; i < kNBT; ++i) {
    if (i >= nb) break;
    float y[CPT][16];
    load_col_block<T>(x, cols, kb0 + i, c, fast, y);
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      if (RHT) {
        rht16_x4(y[e], sg);
        if (!fold) {
#pragma unroll
          for (int j = 0; j < 16; ++j) y[e][j] = 0.25f * y[e][j];
        }
      }
      float m;
      const uint32_t S = block_scale_lut(block_absmax_bits16(y[e]), tb, lut, &m);
      const int64_t blk = (c + e) * nkb + kb0 + i;   // block index in the [outer][K/16] layout
      cw[e][i] = encode16<SR>(y[e], m, (uint64_t)blk, seed, offset);
      sc[e] |= S << (8 * i);
    }
  }
  // A full workgroup tile (its 64 * CPT columns x 16 blocks all inside
  // the tensor) is 64 * CPT whole 128-byte code lines and as many 16-byte
  // scale runs: staged through LDS, so each store instruction writes 8
  // whole lines (the lanes' own 32-byte pieces went to 64 lines per
  // instruction).  Tiles at the edges store their pieces directly.
  constexpr int kCols = 64 * CPT;
  __shared__ __attribute__((aligned(16))) uint2 tile_codes[kCols][4 * kNBT + 2];   // 144-byte rows: no bank conflicts
  __shared__ __attribute__((aligned(16))) uint32_t tile_scales[kCols][kNBT];
  const int64_t c_wg = (int64_t)(gridDim.x - 1 - blockIdx.x) * kCols;
  const int64_t kb_wg = (int64_t)(gridDim.y - 1 - blockIdx.y) * 4 * kNBT;
  const bool whole = (c_wg + kCols <= cols) && (kb_wg + 4 * kNBT <= nkb) && (nkb % 2 == 0) &&
                     aligned_to(codes, 16) && aligned_to(scales, 16) && (nkb % 16 == 0);
  if (whole) {
    const int cl = lane * CPT;
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
#pragma unroll
      for (int i = 0; i < kNBT; ++i) tile_codes[cl + e][wave * kNBT + i] = cw[e][i];
      tile_scales[cl + e][wave] = sc[e];
    }
    __syncthreads();
    // codes: column q / 8, 16-byte piece q % 8 of its 128-byte line
#pragma unroll
    for (int r = 0; r < kCols * 8 / kQT; ++r) {
      const int q = r * kQT + (int)threadIdx.x, col = q >> 3, piece = q & 7;
      const uint4 v = *reinterpret_cast<const uint4 *>(&tile_codes[col][2 * piece]);
      *reinterpret_cast<uint4 *>(codes + (c_wg + col) * nkb + kb_wg + 2 * piece) = v;
    }
    // scales: one 16-byte run per column
    if (threadIdx.x < kCols) {
      const int col = threadIdx.x;
      *reinterpret_cast<uint4 *>(scales + (c_wg + col) * nkb + kb_wg) = *reinterpret_cast<const uint4 *>(tile_scales[col]);
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    if (c + e >= cols) break;
    const int64_t blk0 = (c + e) * nkb + kb0;
    if (nb == kNBT && aligned_to(codes + blk0, 16)) {
      uint4 *dst = reinterpret_cast<uint4 *>(codes + blk0);
      dst[0] = make_uint4(cw[e][0].x, cw[e][0].y, cw[e][1].x, cw[e][1].y);
      dst[1] = make_uint4(cw[e][2].x, cw[e][2].y, cw[e][3].x, cw[e][3].y);
    } else {
#pragma unroll
      for (int i = 0; i < kNBT; ++i)
        if (i < nb) codes[blk0 + i] = cw[e][i];
    }
    if (nb == kNBT && aligned_to(scales + blk0, 4)) {
      *reinterpret_cast<uint32_t *>(scales + blk0) = sc[e];
    } else {
#pragma unroll
      for (int i = 0; i < kNBT; ++i)
        if (i < nb) scales[blk0 + i] = (uint8_t)(sc[e] >> (8 * i));
    }
  }
}

// ---------------------------------------------------------- dequantize ----

// bf16 output: one thread per half block (8 elements, one 16-byte store),
// so the lanes of a wave store one contiguous 1 KB run per instruction;
// value = (e2m1 * S) * g in f32, rounded once to bf16.
__global__ void __launch_bounds__(kQT) k_dequant_bf16(const uint32_t *codes, const uint8_t *scales, const float *meta,
                                                     int64_t nhalves, uint16_t *y) {
  const float g = meta[1];
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t q = (int64_t)blockIdx.x * kQT + threadIdx.x; q < nhalves; q += stride) {
    const uint32_t w = codes[q];           // elements 8(q%2) .. +7 of block q/2: 4 code bytes
    const float S = e4m3_to_f32(scales[q >> 1]);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w >> (8 * i)) & 15u, 1.0f, 0);
      const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w >> (8 * i + 4)) & 15u, 1.0f, 0);
      // nearest-even bf16 of each f32 (NaN cannot occur for finite meta)
      uint32_t a = __float_as_uint(((float)lo[0] * S) * g), c = __float_as_uint(((float)hi[0] * S) * g);
      a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
      c = (c + 0x7FFFu + ((c >> 16) & 1u)) >> 16;
      o[i] = a | (c << 16);
    }
    store_nt(reinterpret_cast<uint4 *>(y + 8 * q), make_uint4(o[0], o[1], o[2], o[3]));
  }
}

// f32 output: one thread per quarter block (4 elements, one 16-byte store),
// so the lanes of a wave store one contiguous 1 KB run per instruction (a
// thread per block wrote 16-byte pieces 64 bytes apart: 32 % slower on a
// 1 GiB output).  Same arithmetic as the bf16 kernel.
__global__ void __launch_bounds__(kQT) k_dequant_f32(const uint16_t *codes, const uint8_t *scales, const float *meta,
                                                    int64_t nquarters, float *y) {
  const float g = meta[1];
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t q = (int64_t)blockIdx.x * kQT + threadIdx.x; q < nquarters; q += stride) {
    const uint32_t w = codes[q];           // elements 4(q%4) .. +3 of block q/4: 2 code bytes
    const float S = e4m3_to_f32(scales[q >> 2]);
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4((w >> (4 * j)) & 15u, 1.0f, 0);
      v[j] = ((float)h[0] * S) * g;
    }
    store_nt(reinterpret_cast<float4 *>(y + 4 * q), make_float4(v[0], v[1], v[2], v[3]));
  }
}

// ------------------------------------------------------ dual encode ----
//
// Both layouts of x from one read: a workgroup stages a 64-row x 256-column
// tile in LDS, then encodes it along the rows (axis-1 output: every thread
// four consecutive blocks of one row, so four adjacent threads write the
// tile's whole 128-byte code line of that row) and down the columns (axis-0
// output, optionally after the transform: every thread the four 16-row
// blocks of one column, 32 contiguous code bytes).  Bit-identical to the two
// single-layout encodes: the same block scales, multipliers and counter
// indices (block b of output o: elements 16b .. 16b+15 of the output
// layout).  Tiles are dealt to the XCDs in contiguous ranges, ordered so that
// the four row tiles sharing one 128-byte axis-0 output line (256 rows) are
// consecutive and so run together on one XCD: its L2 then merges their four
// 32-byte pieces into whole lines before writing them back.  Row tiles run
// from the end of x back (the amax pass went forwards).  The tile height is
// a parameter (32 or 64 rows); 32-row tiles double the occupancy (LDS-bound
// at 64: four workgroups per CU) but measured 5 % slower on dY for every
// rounding setting but both-SR-with-the-transform, where they tie.
constexpr int kDualRows = 64, kDualCols = 256;
constexpr int kDualB = kDualRows / 16;     // 16-row blocks per tile column = blocks per thread in each layout
static_assert(kDualB == 2 || kDualB == 4, "tile height");

template <typename T, bool SR1, bool SR0, bool RHT0>
__global__ void __launch_bounds__(kQT) k_quant_dual(const T *x, int64_t rows, int64_t cols, uint64_t seed1,
                                                   uint64_t offset1, float *meta1, uint2 *codes1, uint8_t *scales1,
                                                   uint32_t sign_mask0, uint64_t seed0, uint64_t offset0,
                                                   float *meta0, uint2 *codes0, uint8_t *scales0) {
  constexpr int E = 16 / (int)sizeof(T);                    // elements per 16-byte chunk
  constexpr int kPitch = kDualCols * (int)sizeof(T) + 16;   // LDS row pitch (bytes), padded
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDualRows * kPitch];
  const int t = threadIdx.x;
  const int tiles_r = (int)((rows + kDualRows - 1) / kDualRows), tiles_c = (int)((cols + kDualCols - 1) / kDualCols);
  int tr, tc;
  xcd_tile(blockIdx.x, tiles_r, tiles_c, 256 / kDualRows, tr, tc);
  const int64_t r0 = (int64_t)(tiles_r - 1 - tr) * kDualRows, c0 = (int64_t)tc * kDualCols;
  const TensorScales ts1 = tensor_scales(meta1[0]), ts0 = tensor_scales(meta0[0]);
  if (blockIdx.x == 0 && t == 0) {
    meta1[1] = ts1.g;
    meta0[1] = ts0.g;
  }
  // axis 0 with the transform on bf16 input: blocks taken as 4y, scales as
  // k/4, s_enc/4 where that is exact (see quarter_scales)
  const bool fold0 = RHT0 && sizeof(T) == 2 && quarter_exact(ts0);
  const TensorScales tb0 = fold0 ? quarter_scales(ts0) : ts0;
  const RhtSigns sg0 = rht_signs(sign_mask0);
  // multipliers of the block scale codes of each layout (the staging
  // barrier below orders these writes before their reads)
  __shared__ float lut1[128], lut0[128];
  fill_scale_lut(lut1, ts1, 0);
  fill_scale_lut(lut0, tb0, 128);
  // The body for one tile; W: the whole tile lies inside x (the bounds
  // checks fold away), which every tile but the last row and column of
  // tiles is.
  auto encode_tile = [&](auto whole) {
    constexpr bool W = decltype(whole)::value;
    // ---- stage the tile (rows past `rows` and chunks past `cols` skipped:
    // no block that reads them is encoded)
    constexpr int kChunksRow = kDualCols / E;
#pragma unroll
    for (int i = 0; i < kDualRows * kChunksRow / kQT; ++i) {
      const int q = i * kQT + t, row = q / kChunksRow, ch = q % kChunksRow;
      const int64_t gr = r0 + row, gc = c0 + (int64_t)ch * E;
      if (W || (gr < rows && gc < cols))
        *reinterpret_cast<uint4 *>(tile + row * kPitch + ch * 16) =
            *reinterpret_cast<const uint4 *>(x + gr * cols + gc);
    }
    __syncthreads();
    const int64_t nb1 = cols / 16, nb0 = rows / 16;
    // ---- axis 1: row t / (16 / kDualB), blocks kDualB * (t % (16 / kDualB)) .. of the tile
    {
      constexpr int kTpr = 16 / kDualB;    // threads per tile row
      const int row = t / kTpr, cb0 = kDualB * (t % kTpr);
      const int64_t gr = r0 + row;
      uint2 cw[kDualB];
      uint32_t sc = 0;
      int nvalid = 0;
#pragma unroll
      for (int i = 0; i < kDualB; ++i) {
        const int64_t gc = c0 + 16 * (cb0 + i);
        if (!W && (gr >= rows || gc >= cols)) break;
        float y[16];
        const T *src = reinterpret_cast<const T *>(tile + row * kPitch) + 16 * (cb0 + i);
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = to_f32<T>(src[j]);
        float m;
        const uint32_t S = block_scale_lut(block_absmax_bits16(y), ts1, lut1, &m);
        cw[i] = encode16<SR1>(y, m, (uint64_t)(gr * nb1 + gc / 16), seed1, offset1);
        sc |= S << (8 * i);
        nvalid = i + 1;
      }
      const int64_t b = gr * nb1 + (c0 / 16 + cb0);
      if ((W || nvalid == kDualB) && aligned_to(codes1 + b, 16)) {
        uint4 *dst = reinterpret_cast<uint4 *>(codes1 + b);
#pragma unroll
        for (int h = 0; h < kDualB / 2; ++h)
          dst[h] = make_uint4(cw[2 * h].x, cw[2 * h].y, cw[2 * h + 1].x, cw[2 * h + 1].y);
      } else {
#pragma unroll
        for (int i = 0; i < kDualB; ++i)
          if (i < nvalid) codes1[b + i] = cw[i];
      }
      if ((W || nvalid == kDualB) && aligned_to(scales1 + b, kDualB)) {
        if constexpr (kDualB == 4)
          *reinterpret_cast<uint32_t *>(scales1 + b) = sc;
        else
          *reinterpret_cast<uint16_t *>(scales1 + b) = (uint16_t)sc;
      } else {
#pragma unroll
        for (int i = 0; i < kDualB; ++i)
          if (i < nvalid) scales1[b + i] = (uint8_t)(sc >> (8 * i));
      }
    }
    // ---- axis 0: column t, the tile's kDualB 16-row blocks
    {
      const int64_t gc = c0 + t;
      uint2 cw[kDualB];
      uint32_t sc = 0;
      int nvalid = 0;
#pragma unroll
      for (int i = 0; i < kDualB; ++i) {
        const int64_t gr = r0 + 16 * i;
        if (!W && (gc >= cols || gr >= rows)) break;
        float y[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = to_f32<T>(*reinterpret_cast<const T *>(tile + (16 * i + j) * kPitch + t * (int)sizeof(T)));
        if (RHT0) {
          rht16_x4(y, sg0);
          if (!fold0) {
#pragma unroll
            for (int j = 0; j < 16; ++j) y[j] = 0.25f * y[j];
          }
        }
        float m;
        const uint32_t S = block_scale_lut(block_absmax_bits16(y), tb0, lut0, &m);
        cw[i] = encode16<SR0>(y, m, (uint64_t)(gc * nb0 + gr / 16), seed0, offset0);
        sc |= S << (8 * i);
        nvalid = i + 1;
      }
      const int64_t b = gc * nb0 + r0 / 16;
      if ((W || nvalid == kDualB) && aligned_to(codes0 + b, 16)) {
        uint4 *dst = reinterpret_cast<uint4 *>(codes0 + b);
#pragma unroll
        for (int h = 0; h < kDualB / 2; ++h)
          dst[h] = make_uint4(cw[2 * h].x, cw[2 * h].y, cw[2 * h + 1].x, cw[2 * h + 1].y);
      } else {
#pragma unroll
        for (int i = 0; i < kDualB; ++i)
          if (i < nvalid) codes0[b + i] = cw[i];
      }
      if ((W || nvalid == kDualB) && aligned_to(scales0 + b, kDualB)) {
        if constexpr (kDualB == 4)
          *reinterpret_cast<uint32_t *>(scales0 + b) = sc;
        else
          *reinterpret_cast<uint16_t *>(scales0 + b) = (uint16_t)sc;
      } else {
#pragma unroll
        for (int i = 0; i < kDualB; ++i)
          if (i < nvalid) scales0[b + i] = (uint8_t)(sc >> (8 * i));
      }
    }
  };
  if (r0 + kDualRows <= rows && c0 + kDualCols <= cols)
    encode_tile(std::true_type{});
  else
    encode_tile(std::false_type{});
}

// ------------------------------------------------------------ launches ----

inline unsigned grid_for(int64_t work, int64_t per_block = kQT, int64_t cap = 1 << 20) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

namespace {

// Pass 2 of a quantization (encode), reading amax from meta[0].
void launch_encode(const void *x, bool bf16, int64_t rows, int64_t cols, int axis, int rounding, uint64_t seed,
                   uint64_t offset, bool rht, uint32_t sign_mask, uint8_t *codes, uint8_t *scales, float *meta,
                   hipStream_t stream) {
  const int64_t n = rows * cols;
  const int64_t cpt = bf16 ? 2 : 1;
  const bool sr = (rounding == 1);
  const int64_t nblocks = n / 16;
  // Axis 1: with stochastic rounding the encode is ALU-bound, so each thread
  // walks four blocks (the tensor scales, three divisions, are computed once
  // per thread): 4-5 % faster than one block per thread, which stays the
  // faster choice for nearest rounding (memory-bound).
  unsigned g = grid_for(nblocks, sr ? kQT * 4 : kQT);
  // Axis 1 streams its output only when the input is larger than the
  // last-level cache, where the codes could not stay cached for their
  // reader anyway: the 512 MiB sweep tensor quantizes 5-6 % faster that
  // way, while the 40-50 MB operands of a layer step keep their codes for
  // the GEMM that follows (step -0.12 % on one GPU).
  const bool stream_out = n * (bf16 ? 2 : 4) > kStreamOutBytes;
  const dim3 qtiles((unsigned)((cols + 64 * cpt - 1) / (64 * cpt)), (unsigned)((rows / 16 + 4 * kNBT - 1) / (4 * kNBT)));
#define NVFP4_QROWS(T, S, R) hipLaunchKernelGGL((k_quant_rows<T, S, R>), dim3(g), dim3(kQT), 0, stream, (const T *)x, nblocks, sign_mask, seed, offset, meta, (uint2 *)codes, scales, stream_out)
#define NVFP4_QCOLS(T, S, R) hipLaunchKernelGGL((k_quant_cols<T, S, R>), qtiles, dim3(kQT), 0, stream, (const T *)x, rows, cols, sign_mask, seed, offset, meta, (uint2 *)codes, scales)
#define NVFP4_DISPATCH(MAC, T)                  \
  do {                                          \
    if (sr) { if (rht) MAC(T, true, true); else MAC(T, true, false); } \
    else { if (rht) MAC(T, false, true); else MAC(T, false, false); } \
  } while (0)
  if (axis == 1) {
    if (bf16) NVFP4_DISPATCH(NVFP4_QROWS, uint16_t);
    else NVFP4_DISPATCH(NVFP4_QROWS, float);
  } else {
    if (bf16) NVFP4_DISPATCH(NVFP4_QCOLS, uint16_t);
    else NVFP4_DISPATCH(NVFP4_QCOLS, float);
  }
#undef NVFP4_QROWS
#undef NVFP4_QCOLS
#undef NVFP4_DISPATCH
}

// Grid of the column-wise amax kernels: 256 * kCPT columns x kNBT blocks.
dim3 col_tiles(int64_t rows, int64_t cols, bool bf16) {
  const int64_t cpt = bf16 ? 2 : 1;
  return dim3((unsigned)((cols + kQT * cpt - 1) / (kQT * cpt)), (unsigned)((rows / 16 + kNBT - 1) / kNBT));
}

// Plain amax of all n elements into amax_bits (and amax_bits2 if given).
void launch_amax_flat(const void *x, bool bf16, int64_t n, uint32_t *amax_bits, uint32_t *amax_bits2,
                      hipStream_t stream) {
  const int64_t n16 = n * (bf16 ? 2 : 4) / 16;
  // 1024 workgroups, or 512 where a thread would have fewer than 16
  // vectors (tensors below 64 MiB): there the workgroups finish together
  // and their atomics queue on one address.  Measured on MI355X: the 40-50
  // MB layer operands quantize 3-7 us faster with 512, the 512 MiB sweep
  // tensor 5-8 us slower.
  const unsigned g = grid_for(n16, kQT * 4, n16 < (int64_t)kQT * 16 * 1024 ? 512 : 1024);
  const int64_t per = (n16 + g - 1) / g;
  if (bf16) hipLaunchKernelGGL(k_amax_flat<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint4 *)x, n16, per, amax_bits, amax_bits2);
  else hipLaunchKernelGGL(k_amax_flat<float>, dim3(g), dim3(kQT), 0, stream, (const uint4 *)x, n16, per, amax_bits, amax_bits2);
}

// Pass 1 of a quantization: the tensor amax (after the transform if rht)
// folded into *amax_bits, which must start at zero.
void launch_pass1(const void *x, bool bf16, int64_t rows, int64_t cols, int axis, bool rht, uint32_t sign_mask,
                  uint32_t *amax_bits, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (!rht) {
    launch_amax_flat(x, bf16, n, amax_bits, nullptr, stream);
  } else if (axis == 1) {
    const int64_t nch = n / 16;
    const unsigned g = grid_for(nch, kQT * 2, 2048);
    const int64_t per = (nch + g - 1) / g;
    if (bf16) hipLaunchKernelGGL(k_amax_rht_rows<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint16_t *)x, nch, per, sign_mask, amax_bits);
    else hipLaunchKernelGGL(k_amax_rht_rows<float>, dim3(g), dim3(kQT), 0, stream, (const float *)x, nch, per, sign_mask, amax_bits);
  } else {
    const dim3 tiles = col_tiles(rows, cols, bf16);
    if (bf16) hipLaunchKernelGGL(k_amax_rht_cols<uint16_t>, tiles, dim3(kQT), 0, stream, (const uint16_t *)x, rows, cols, sign_mask, amax_bits);
    else hipLaunchKernelGGL(k_amax_rht_cols<float>, tiles, dim3(kQT), 0, stream, (const float *)x, rows, cols, sign_mask, amax_bits);
  }
}

}  // namespace

hipError_t launch_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, bool rht,
                       uint32_t sign_mask, float *amax, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(64), 0, stream, amax);
  if (rows * cols == 0) return hipGetLastError();
  const bool bf16 = (x_dtype == 1);
  if (axis == 0 && col_tiles(rows, cols, bf16).y > 65535u) return hipErrorInvalidValue;
  launch_pass1(x, bf16, rows, cols, axis, rht, sign_mask, reinterpret_cast<uint32_t *>(amax), stream);
  return hipGetLastError();
}

hipError_t launch_quantize_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                                uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, const float *amax,
                                uint8_t *codes, uint8_t *scales, float *meta, hipStream_t stream) {
  hipLaunchKernelGGL(k_meta_set, dim3(1), dim3(64), 0, stream, meta, amax);
  if (rows * cols == 0) return hipGetLastError();
  const bool bf16 = (x_dtype == 1);
  if (axis == 0 && col_tiles(rows, cols, bf16).y > 65535u) return hipErrorInvalidValue;
  launch_encode(x, bf16, rows, cols, axis, rounding, seed, offset, rht, sign_mask, codes, scales, meta, stream);
  return hipGetLastError();
}

hipError_t launch_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                           uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, uint8_t *codes,
                           uint8_t *scales, float *meta, hipStream_t stream) {
  const int64_t n = rows * cols;
  uint32_t *amax_bits = reinterpret_cast<uint32_t *>(meta);
  hipLaunchKernelGGL(k_meta_init, dim3(1), dim3(64), 0, stream, meta);
  if (n == 0) return hipGetLastError();
  const bool bf16 = (x_dtype == 1);
  if (axis == 0 && col_tiles(rows, cols, bf16).y > 65535u) return hipErrorInvalidValue;
  // pass 1: amax
  launch_pass1(x, bf16, rows, cols, axis, rht, sign_mask, amax_bits, stream);
  // pass 2: encode
  launch_encode(x, bf16, rows, cols, axis, rounding, seed, offset, rht, sign_mask, codes, scales, meta, stream);
  return hipGetLastError();
}

hipError_t launch_quantize_dual(const void *x, int x_dtype, int64_t rows, int64_t cols, int rounding1,
                                uint64_t seed1, uint64_t offset1, uint8_t *codes1, uint8_t *scales1, float *meta1,
                                bool rht0, uint32_t sign_mask0, int rounding0, uint64_t seed0, uint64_t offset0,
                                uint8_t *codes0, uint8_t *scales0, float *meta0, hipStream_t stream) {
  const int64_t n = rows * cols;
  hipLaunchKernelGGL(k_meta_init2, dim3(1), dim3(64), 0, stream, meta1, meta0);
  if (n == 0) return hipGetLastError();
  const bool bf16 = (x_dtype == 1);
  const dim3 tiles = col_tiles(rows, cols, bf16);
  if (tiles.y > 65535u) return hipErrorInvalidValue;
  uint32_t *bits1 = reinterpret_cast<uint32_t *>(meta1), *bits0 = reinterpret_cast<uint32_t *>(meta0);
  // pass 1: both maxima from one read
  if (!rht0) {
    launch_amax_flat(x, bf16, n, bits1, bits0, stream);
  } else {
    if (bf16) hipLaunchKernelGGL(k_amax_dual_cols<uint16_t>, tiles, dim3(kQT), 0, stream, (const uint16_t *)x, rows, cols, sign_mask0, bits1, bits0);
    else hipLaunchKernelGGL(k_amax_dual_cols<float>, tiles, dim3(kQT), 0, stream, (const float *)x, rows, cols, sign_mask0, bits1, bits0);
  }
  // pass 2: both encodes from one read
  const int64_t ntiles = ((cols + kDualCols - 1) / kDualCols) * ((rows + kDualRows - 1) / kDualRows);
  if (ntiles > INT32_MAX) return hipErrorInvalidValue;
  const dim3 dtiles((unsigned)ntiles);
  const bool sr1 = rounding1 == 1, sr0 = rounding0 == 1;
#define NVFP4_QDUAL(T, S1, S0, R0)                                                                          \
  hipLaunchKernelGGL((k_quant_dual<T, S1, S0, R0>), dtiles, dim3(kQT), 0, stream, (const T *)x, rows, cols, seed1, \
                     offset1, meta1, (uint2 *)codes1, scales1, sign_mask0, seed0, offset0, meta0, (uint2 *)codes0,   \
                     scales0)
#define NVFP4_QDUAL_T(T)                                                                       \
  do {                                                                                         \
    if (sr1) {                                                                                 \
      if (sr0) { if (rht0) NVFP4_QDUAL(T, true, true, true); else NVFP4_QDUAL(T, true, true, false); }     \
      else { if (rht0) NVFP4_QDUAL(T, true, false, true); else NVFP4_QDUAL(T, true, false, false); }       \
    } else {                                                                                   \
      if (sr0) { if (rht0) NVFP4_QDUAL(T, false, true, true); else NVFP4_QDUAL(T, false, true, false); }   \
      else { if (rht0) NVFP4_QDUAL(T, false, false, true); else NVFP4_QDUAL(T, false, false, false); }     \
    }                                                                                          \
  } while (0)
  if (bf16) NVFP4_QDUAL_T(uint16_t);
  else NVFP4_QDUAL_T(float);
#undef NVFP4_QDUAL_T
#undef NVFP4_QDUAL
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *meta, int64_t outer,
                             int64_t k, void *y, int y_dtype, hipStream_t stream) {
  const int64_t nblocks = outer * (k / 16);
  if (nblocks == 0) return hipSuccess;
  if (y_dtype == 0)
    hipLaunchKernelGGL(k_dequant_f32, dim3(grid_for(4 * nblocks)), dim3(kQT), 0, stream, (const uint16_t *)codes,
                       scales, meta, 4 * nblocks, (float *)y);
  else
    hipLaunchKernelGGL(k_dequant_bf16, dim3(grid_for(2 * nblocks)), dim3(kQT), 0, stream, (const uint32_t *)codes,
                       scales, meta, 2 * nblocks, (uint16_t *)y);
  return hipGetLastError();
}

}  // namespace nvfp4
