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
//  * the amax pass keeps four 16-byte loads in flight per thread;
//  * the encode pass walks the tensor in the opposite order of the amax
//    pass, so its first part is still resident in the 256 MB MALL;
//  * axis 0 (K runs down the columns; the output is the transpose) stages a
//    512-row x 32-column tile in LDS with coalesced 16-byte loads, so each
//    thread reads its column's 16-element blocks from LDS and the codes and
//    scales of one output row are written as contiguous runs.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kQT = kQuantThreads;

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Reduce a per-thread max over the workgroup and fold it into *dst.
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
    if (m) atomicMax(dst, m);
  }
}

__global__ void k_meta_init(float *meta) {
  if (threadIdx.x == 0) {
    meta[0] = 0.0f;
    meta[1] = 0.0f;
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

// Flat amax over n16 16-byte vectors (no transform; the axis does not
// matter).  Four loads in flight per thread per iteration.
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_flat(const uint4 *x, int64_t n16, uint32_t *amax_bits) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kQT;
  int64_t i = (int64_t)blockIdx.x * kQT + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 v0 = x[i], v1 = x[i + stride], v2 = x[i + 2 * stride], v3 = x[i + 3 * stride];
    m = max(max(m, vec_absmax<T>(v0)), max(vec_absmax<T>(v1), max(vec_absmax<T>(v2), vec_absmax<T>(v3))));
  }
  for (; i < n16; i += stride) m = max(m, vec_absmax<T>(x[i]));
  block_max_atomic(m, amax_bits);
}

// amax of the transformed tensor, axis 1: one 16-chunk of a row per thread
// and iteration, two chunks in flight.
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_rht_rows(const T *x, int64_t nchunks, uint32_t sign_mask,
                                                      uint32_t *amax_bits) {
  uint32_t m = 0;
  const int64_t stride = (int64_t)gridDim.x * kQT;
  int64_t c = (int64_t)blockIdx.x * kQT + threadIdx.x;
  for (; c + stride < nchunks; c += 2 * stride) {
    float y0[16], y1[16];
    Load16<T>::run(x + 16 * c, y0);
    Load16<T>::run(x + 16 * (c + stride), y1);
    rht16(y0, sign_mask);
    rht16(y1, sign_mask);
    m = max(m, max(absmax_bits16(y0), absmax_bits16(y1)));
  }
  for (; c < nchunks; c += stride) {
    float y[16];
    Load16<T>::run(x + 16 * c, y);
    rht16(y, sign_mask);
    m = max(m, absmax_bits16(y));
  }
  block_max_atomic(m, amax_bits);
}

// ------------------------------------------------- axis-0 LDS tiles ----
//
// A tile is 32 columns x kTileBlocks 16-row blocks of the input (512 rows).
// LDS holds it row-major as 32-bit words with one 4-word pad after every
// 16 rows, so that the 16 threads reading the same row offset of 16
// different blocks hit 16 different bank groups.  Thread t handles the
// column pair cp = t / 16 (columns 2cp, 2cp+1) and blocks g = t % 16 and
// g + 16: sixteen consecutive threads then write one output row's 16
// consecutive code words (128 bytes) and scales.
constexpr int kTileCols = 32;
constexpr int kTileBlocks = 32;
constexpr int kTileRows = 16 * kTileBlocks;

template <typename T>
struct ColTile {
  static constexpr int kWordsPerRow = kTileCols * (int)sizeof(T) / 4;   // 16 (bf16) or 32 (f32)
  static constexpr int kWords = kTileRows * kWordsPerRow + 4 * kTileBlocks;
  __device__ static __forceinline__ int word(int row, int w) { return row * kWordsPerRow + w + 4 * (row >> 4); }
};

// Load rows [r0, r0 + 512) x columns [c0, c0 + 32) of x into the LDS tile;
// positions outside the matrix read as zero.
template <typename T>
__device__ __forceinline__ void load_col_tile(const T *x, int64_t rows, int64_t cols, int64_t r0, int64_t c0,
                                              uint32_t *tile) {
  using Tl = ColTile<T>;
  constexpr int kVecPerRow = Tl::kWordsPerRow / 4;   // 16-byte vectors per tile row
  constexpr int kVecs = kTileRows * kVecPerRow;
  const bool vec_ok = (c0 + kTileCols <= cols) && ((cols * (int64_t)sizeof(T)) % 16 == 0);
  if (vec_ok) {
#pragma unroll 4
    for (int u = threadIdx.x; u < kVecs; u += kQT) {
      const int row = u / kVecPerRow, q = u % kVecPerRow;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r0 + row < rows) v = *reinterpret_cast<const uint4 *>(x + (r0 + row) * cols + c0 + q * (16 / sizeof(T)));
      *reinterpret_cast<uint4 *>(tile + Tl::word(row, 4 * q)) = v;
    }
  } else {
    constexpr int kPerWord = 4 / (int)sizeof(T);
    for (int u = threadIdx.x; u < kTileRows * Tl::kWordsPerRow; u += kQT) {
      const int row = u / Tl::kWordsPerRow, w = u % Tl::kWordsPerRow;
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < kPerWord; ++e) {
        const int64_t c = c0 + w * kPerWord + e;
        if (r0 + row < rows && c < cols) {
          const T v = x[(r0 + row) * cols + c];
          word |= (uint32_t)__builtin_bit_cast(typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type, v)
                  << (16 * e * (sizeof(T) == 2));
        }
      }
      tile[Tl::word(row, w)] = word;
    }
  }
}

// The 16 values of column cc (0..31) in tile block blk, as binary32.
template <typename T>
__device__ __forceinline__ void tile_block(const uint32_t *tile, int blk, int cc, float *y) {
  using Tl = ColTile<T>;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int row = 16 * blk + j;
    if constexpr (sizeof(T) == 2) {
      const uint32_t w = tile[Tl::word(row, cc >> 1)];
      y[j] = (cc & 1) ? bf16_hi(w) : bf16_lo(w);
    } else {
      y[j] = __uint_as_float(tile[Tl::word(row, cc)]);
    }
  }
}

// amax of the transformed tensor, axis 0 (16-row chunks of each column).
template <typename T>
__global__ void __launch_bounds__(kQT) k_amax_rht_cols(const T *x, int64_t rows, int64_t cols, uint32_t sign_mask,
                                                      uint32_t *amax_bits) {
  __shared__ uint32_t tile[ColTile<T>::kWords];
  const int64_t c0 = (int64_t)blockIdx.x * kTileCols, r0 = (int64_t)blockIdx.y * kTileRows;
  load_col_tile<T>(x, rows, cols, r0, c0, tile);
  __syncthreads();
  const int cp = threadIdx.x >> 4, g = threadIdx.x & 15;
  uint32_t m = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float y[16];
      tile_block<T>(tile, g + 16 * h, 2 * cp + e, y);   // zero rows/columns stay zero
      rht16(y, sign_mask);
      m = max(m, absmax_bits16(y));
    }
  }
  block_max_atomic(m, amax_bits);
}

// ------------------------------------------------------------- encode ----

// axis 1: one thread per 16-block (o, b); codes are 8 contiguous bytes.  The
// blocks are visited from the end of the tensor backwards (the amax pass
// went forwards), so the most recently read part is encoded first.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(kQT) k_quant_rows(const T *x, int64_t nblocks, uint32_t sign_mask, uint64_t seed,
                                                   uint64_t offset, float *meta, uint2 *codes, uint8_t *scales) {
  const float amax = meta[0];
  const TensorScales ts = tensor_scales(amax);
  if (blockIdx.x == 0 && threadIdx.x == 0) meta[1] = ts.g;
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t i = (int64_t)blockIdx.x * kQT + threadIdx.x; i < nblocks; i += stride) {
    const int64_t b = nblocks - 1 - i;
    float y[16];
    Load16<T>::run(x + 16 * b, y);
    if (RHT) rht16(y, sign_mask);
    float m;
    uint32_t S = block_scale(absmax_bits16(y), ts, &m);
    codes[b] = encode16<SR>(y, m, (uint64_t)b, seed, offset);
    scales[b] = (uint8_t)S;
  }
}

// axis 0: one 512-row x 32-column tile per workgroup (see ColTile).  Output
// row o = column, block kb = 16-row group; the tiles are visited in reverse
// order of the amax pass.
template <typename T, bool SR, bool RHT>
__global__ void __launch_bounds__(kQT) k_quant_cols(const T *x, int64_t rows, int64_t cols, uint32_t sign_mask,
                                                   uint64_t seed, uint64_t offset, float *meta, uint2 *codes,
                                                   uint8_t *scales) {
  __shared__ uint32_t tile[ColTile<T>::kWords];
  const float amax = meta[0];
  const TensorScales ts = tensor_scales(amax);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) meta[1] = ts.g;
  const int64_t c0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * kTileCols;
  const int64_t r0 = (int64_t)(gridDim.y - 1 - blockIdx.y) * kTileRows;
  load_col_tile<T>(x, rows, cols, r0, c0, tile);
  __syncthreads();
  const int64_t nkb = rows / 16, kb0 = r0 / 16;
  const int cp = threadIdx.x >> 4, g = threadIdx.x & 15;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int64_t o = c0 + 2 * cp + e;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t kb = kb0 + g + 16 * h;
      if (o >= cols || kb >= nkb) continue;
      float y[16];
      tile_block<T>(tile, g + 16 * h, 2 * cp + e, y);
      if (RHT) rht16(y, sign_mask);
      float m;
      const uint32_t S = block_scale(absmax_bits16(y), ts, &m);
      const int64_t blk = o * nkb + kb;   // block index in the [outer][K/16] layout
      codes[blk] = encode16<SR>(y, m, (uint64_t)blk, seed, offset);
      scales[blk] = (uint8_t)S;
    }
  }
}

// ---------------------------------------------------------- dequantize ----

// One thread per 16-block: value = (e2m1 * S) * g, S applied exactly in f16.
template <typename TO>
__global__ void __launch_bounds__(kQT) k_dequant(const uint2 *codes, const uint8_t *scales, const float *meta,
                                                int64_t nblocks, TO *y) {
  const float g = meta[1];
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t b = (int64_t)blockIdx.x * kQT + threadIdx.x; b < nblocks; b += stride) {
    uint2 c = codes[b];
    float S = e4m3_to_f32(scales[b]);
    float v[16];
    uint32_t w[2] = {c.x, c.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t nib = (w[h] >> (4 * j)) & 15u;
        half2_t q = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(nib, 1.0f, 0);
        v[8 * h + j] = ((float)q[0] * S) * g;
      }
    }
    if constexpr (sizeof(TO) == 4) {
      float4 *dst = reinterpret_cast<float4 *>(y + 16 * b);
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
    } else {
      uint32_t o[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // nearest-even bf16 of each f32 (NaN cannot occur for finite meta)
        uint32_t lo = __float_as_uint(v[2 * i]), hi = __float_as_uint(v[2 * i + 1]);
        lo = (lo + 0x7FFFu + ((lo >> 16) & 1u)) >> 16;
        hi = (hi + 0x7FFFu + ((hi >> 16) & 1u)) >> 16;
        o[i] = lo | (hi << 16);
      }
      uint4 *dst = reinterpret_cast<uint4 *>(y + 16 * b);
      dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
      dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
  }
}

// ------------------------------------------------------------ launches ----

inline unsigned grid_for(int64_t work, int64_t per_block = kQT, int64_t cap = 1 << 20) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (unsigned)g;
}

}  // namespace

hipError_t launch_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                           uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, uint8_t *codes,
                           uint8_t *scales, float *meta, hipStream_t stream) {
  const int64_t n = rows * cols;
  uint32_t *amax_bits = reinterpret_cast<uint32_t *>(meta);
  hipLaunchKernelGGL(k_meta_init, dim3(1), dim3(64), 0, stream, meta);
  if (n == 0) return hipGetLastError();
  const bool bf16 = (x_dtype == 1);
  const dim3 tiles((unsigned)((cols + kTileCols - 1) / kTileCols), (unsigned)((rows + kTileRows - 1) / kTileRows));
  if (axis == 0 && tiles.y > 65535u) return hipErrorInvalidValue;
  // pass 1: amax
  if (!rht) {
    const int64_t n16 = n * (bf16 ? 2 : 4) / 16;
    unsigned g = grid_for(n16, kQT * 4, 2048);
    if (bf16) hipLaunchKernelGGL(k_amax_flat<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint4 *)x, n16, amax_bits);
    else hipLaunchKernelGGL(k_amax_flat<float>, dim3(g), dim3(kQT), 0, stream, (const uint4 *)x, n16, amax_bits);
  } else if (axis == 1) {
    const int64_t nch = n / 16;
    unsigned g = grid_for(nch, kQT * 2, 4096);
    if (bf16) hipLaunchKernelGGL(k_amax_rht_rows<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint16_t *)x, nch, sign_mask, amax_bits);
    else hipLaunchKernelGGL(k_amax_rht_rows<float>, dim3(g), dim3(kQT), 0, stream, (const float *)x, nch, sign_mask, amax_bits);
  } else {
    if (bf16) hipLaunchKernelGGL(k_amax_rht_cols<uint16_t>, tiles, dim3(kQT), 0, stream, (const uint16_t *)x, rows, cols, sign_mask, amax_bits);
    else hipLaunchKernelGGL(k_amax_rht_cols<float>, tiles, dim3(kQT), 0, stream, (const float *)x, rows, cols, sign_mask, amax_bits);
  }
  // pass 2: encode
  const bool sr = (rounding == 1);
  const int64_t nblocks = n / 16;
  unsigned g = grid_for(nblocks);
#define NVFP4_QROWS(T, S, R) hipLaunchKernelGGL((k_quant_rows<T, S, R>), dim3(g), dim3(kQT), 0, stream, (const T *)x, nblocks, sign_mask, seed, offset, meta, (uint2 *)codes, scales)
#define NVFP4_QCOLS(T, S, R) hipLaunchKernelGGL((k_quant_cols<T, S, R>), tiles, dim3(kQT), 0, stream, (const T *)x, rows, cols, sign_mask, seed, offset, meta, (uint2 *)codes, scales)
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
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *meta, int64_t outer,
                             int64_t k, void *y, int y_dtype, hipStream_t stream) {
  const int64_t nblocks = outer * (k / 16);
  if (nblocks == 0) return hipSuccess;
  unsigned g = grid_for(nblocks);
  if (y_dtype == 0)
    hipLaunchKernelGGL(k_dequant<float>, dim3(g), dim3(kQT), 0, stream, (const uint2 *)codes, scales, meta, nblocks, (float *)y);
  else
    hipLaunchKernelGGL(k_dequant<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint2 *)codes, scales, meta, nblocks, (uint16_t *)y);
  return hipGetLastError();
}

}  // namespace nvfp4
