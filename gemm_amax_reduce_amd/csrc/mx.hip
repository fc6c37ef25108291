// mx.hip -- MXFP4 quantizer and GEMM on gfx950's block-scaled MFMA.
//
// MXFP4 is the microscaling format the pages set NVFP4 against ([P4]
// aisight.pl "Koniec marnowania mocy ...", section "Architektura NVFP4
// kontra ograniczenia mikroskalowania": 32-element blocks sharing a
// power-of-two scale, where NVFP4 uses 16-element blocks with an E4M3 scale
// and a tensor-level FP32 scale).  Elements are E2M1; each 32-block along K
// carries an E8M0 exponent (scale 2^(code - 127)); there is no tensor scale.
// Block scale: the smallest power of two X = 2^e with amax_b / X <= 6, so
// the block maximum is never clipped (e clamped to [-127, 127]); elements
// are the nearest-even E2M1 codes of x / X.
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 takes FP4 operands with one E8M0
// scale per lane, and a lane of a 32x32x64 operand holds exactly one 32-
// element block of its row (lane l: row l % 32, K half l / 32), measured
// bit-exact against an fp64 reference: the codes feed the MFMA as they are,
// with no decode, at the FP4 rate (64 K per 32-cycle instruction, four times
// the f16 form's K).  (With FP8 operands the same instruction truncates its
// products within groups of 8 K positions; MXFP8 is in mx8.hip with the
// tolerance that follows from that.)
#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kQT = kQuantThreads;

// ------------------------------------------------------------ quantize ----

// Smallest e with amax <= 6 * 2^e for the bit pattern of amax >= 0:
// 6 * 2^e = 1.5 * 2^(e+2), so for amax = m * 2^E (m in [1, 2)) e = E - 2
// when m <= 1.5 and E - 1 otherwise; zero and subnormal maxima fit e = -127.
__device__ __forceinline__ int mx_exp(uint32_t amax_bits) {
  if (amax_bits < 0x00800000u) return -127;
  const int E = (int)(amax_bits >> 23) - 127;
  const int e = (amax_bits & 0x7FFFFFu) <= 0x400000u ? E - 2 : E - 1;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^n as binary32 for n in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float pow2f(int n) {
  return n >= -126 ? __uint_as_float((uint32_t)(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// Codes and scale of one 32-block held as binary32 values y[0..31].
__device__ __forceinline__ uint4 mx_encode32(const float *y, uint8_t *scale) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  const int e = mx_exp(m);
  *scale = (uint8_t)(e + 127);
  const float inv = pow2f(-e);       // exact: x * 2^-e is x / X rounded once
  float v[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = y[j] * inv;
  return make_uint4(encode8_rne(v), encode8_rne(v + 8), encode8_rne(v + 16), encode8_rne(v + 24));
}

// axis 1: one thread per 32-block of a row.
template <typename T>
__global__ void __launch_bounds__(kQT) k_mx_quant_rows(const T *x, int64_t nblocks, uint4 *codes, uint8_t *scales) {
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t b = (int64_t)blockIdx.x * kQT + threadIdx.x; b < nblocks; b += stride) {
    float y[32];
    Load16<T>::run(x + 32 * b, y);
    Load16<T>::run(x + 32 * b + 16, y + 16);
    uint8_t s;
    // ordinary stores: the codes stay in the last-level cache for the GEMM
    // that reads them next (streaming stores made this call 3 us faster
    // alone but the MXFP4 linear-layer step 0.4 % slower on one GPU)
    codes[b] = mx_encode32(y, &s);
    scales[b] = s;
  }
}

// axis 0 (K runs down the columns, output transposed): a thread takes two
// adjacent bf16 columns (one f32 column) and two consecutive 32-row blocks;
// the four waves of a workgroup share their columns and take consecutive
// block pairs, so each 128-byte output line is written by one workgroup.
// The column loads carry the nontemporal hint (each line is read once):
// dY 8192 x 20480 bf16 141 -> 125 us on one GPU; a 20480 x 5120 tensor
// quantized back to back ran 67 -> 72 us, losing the last-level cache
// reuse between calls.  Whole tiles stage their output lines in LDS (below):
// dY 124 -> 87.5 us.
template <typename T>
__global__ void __launch_bounds__(kQT) k_mx_quant_cols(const T *x, int64_t rows, int64_t cols, uint4 *codes,
                                                      uint8_t *scales) {
  constexpr int CPT = 4 / (int)sizeof(T);
  constexpr int kCols = 64 * CPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * CPT;
  const int64_t nkb = rows / 32, kb0 = ((int64_t)blockIdx.y * 4 + wave) * 2;
  // A workgroup tile wholly inside x (its kCols columns x 8 blocks, output
  // lines 128-byte aligned) goes out through LDS as whole lines, 8 per store
  // instruction, instead of one 16-byte piece per lane and line.
  const int64_t c_wg = (int64_t)blockIdx.x * kCols, kb_wg = (int64_t)blockIdx.y * 8;
  const bool whole = (c_wg + kCols <= cols) && (kb_wg + 8 <= nkb) && (nkb % 8 == 0) && (CPT == 1 || cols % 2 == 0) &&
                     ((uintptr_t)codes & 127) == 0 && ((uintptr_t)scales & 7) == 0;
  __shared__ __attribute__((aligned(16))) uint4 tile_codes[kCols][9];    // 144-byte rows: no bank conflicts
  __shared__ __attribute__((aligned(8))) uint8_t tile_scales[kCols][8];
  if (whole) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float y[CPT][32];
      const T *p = x + 32 * (kb0 + i) * cols + c;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + j * cols));
        if constexpr (CPT == 2) {
          y[0][j] = bf16_lo(w);
          y[1][j] = bf16_hi(w);
        } else {
          y[0][j] = __uint_as_float(w);
        }
      }
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        uint8_t sb;
        tile_codes[lane * CPT + e][2 * wave + i] = mx_encode32(y[e], &sb);
        tile_scales[lane * CPT + e][2 * wave + i] = sb;
      }
    }
    __syncthreads();
    // codes: column q / 8, 16-byte piece q % 8 of its line
#pragma unroll
    for (int r = 0; r < kCols * 8 / kQT; ++r) {
      const int q = r * kQT + (int)threadIdx.x, col = q >> 3, piece = q & 7;
      codes[(c_wg + col) * nkb + kb_wg + piece] = tile_codes[col][piece];
    }
    if (threadIdx.x < kCols) {
      const int col = threadIdx.x;
      *reinterpret_cast<uint2 *>(scales + (c_wg + col) * nkb + kb_wg) = *reinterpret_cast<const uint2 *>(tile_scales[col]);
    }
    return;
  }
  if (c >= cols) return;
  const bool fast = (c + CPT <= cols) && (CPT == 1 || (cols % 2) == 0);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t kb = kb0 + i;
    if (kb >= nkb) break;
    float y[CPT][32];
    const T *p = x + 32 * kb * cols + c;
    if (fast) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + j * cols));
        if constexpr (CPT == 2) {
          y[0][j] = bf16_lo(w);
          y[1][j] = bf16_hi(w);
        } else {
          y[0][j] = __uint_as_float(w);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < CPT; ++e)
#pragma unroll
        for (int j = 0; j < 32; ++j) y[e][j] = (c + e < cols) ? to_f32<T>(p[j * cols + e]) : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      if (c + e >= cols) break;
      uint8_t s;
      const uint4 w = mx_encode32(y[e], &s);
      codes[(c + e) * nkb + kb] = w;
      scales[(c + e) * nkb + kb] = s;
    }
  }
}

// ---------------------------------------------------------------- GEMM ----
//
// One 256-thread workgroup per 256 x BN tile (BN = 256, or 128 for the
// column remainder), four waves of 128 x BN/2.  K is consumed in groups of
// 256 (four 64-wide stages); each group's codes (one 128-byte line per row)
// come into LDS by DMA exactly as in the NVFP4 kernel (chunk c of row R in
// slot c ^ (R & 7)).  The scales of two groups (16 bytes per row, one per
// 32-block) come in one 16-byte DMA per row, 64 rows per instruction, into
// one of two pair buffers.  (Per group, two 4-byte DMAs per 64 rows touched
// one cache line per row and lane: a timing copy without them ran the dgrad
// shape 15 % faster.)  A stage is one MFMA step: lane (r, h) of fragment f
// reads chunk 2s'+h of its row (16 bytes = one 32-block) and that block's
// scale byte.  Requires K % 256 == 0.

constexpr int BM = 256;
constexpr int kThreads = 256;
constexpr int kGroupK = 256;
constexpr int kRowsMax = BM + 256;
constexpr int kCodeBytes = kRowsMax * 128;      // 64 KB
constexpr int kGroupBytes = kCodeBytes;         // a group buffer: codes only
constexpr int kScalePair = kRowsMax * 16;       // 8 KB: the scales of two groups
constexpr int kLdsBytes = 2 * kGroupBytes + 2 * kScalePair;
constexpr int kGroupM = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool OUT_BF16, int BN>
__device__ __forceinline__ void mx_gemm_tile(uint8_t *smem, int pid, const uint8_t *__restrict__ A,
                                             const uint8_t *__restrict__ SA, const uint8_t *__restrict__ B,
                                             const uint8_t *__restrict__ SB, int64_t M, int64_t N, int64_t K,
                                             void *__restrict__ C, int64_t ldc) {
  constexpr int NB = BN / 64;
  constexpr int NF = 4 + NB;
  constexpr int kRowsB = BN / 2;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, h = lane >> 5;

  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int tm, tn;
  xcd_tile(pid, tiles_m, tiles_n, kGroupM, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  // ---- DMA side (as in the NVFP4 kernel; rows past M or N read as zeros)
  const uint32_t rb = (uint32_t)(K / 2), rs = (uint32_t)(K / 32);
  const bool dma_b = wave >= 2;
  const int64_t drow0 = dma_b ? n0 + (int64_t)kRowsB * (wave - 2) : m0 + 128 * (int64_t)wave;
  const int64_t dlimit = dma_b ? N : M;
  const int64_t dbase = min<int64_t>(drow0, dlimit);
  const uint32_t dvalid = (uint32_t)min<int64_t>(dma_b ? kRowsB : 128, dlimit - dbase);
  const __amdgpu_buffer_rsrc_t dcodes = make_rsrc((dma_b ? B : A) + dbase * rb, dvalid * rb);
  const __amdgpu_buffer_rsrc_t dscales = make_rsrc((dma_b ? SB : SA) + dbase * rs, dvalid * rs);
  const int lds_row0 = dma_b ? BM + kRowsB * (wave - 2) : 128 * wave;
  const int spare_row0 = BM + 128 + 64 * (wave - 2);
  const uint32_t dv_code = (uint32_t)(lane >> 3) * rb + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t dv_scale = (uint32_t)lane * rs;
  const int ng = (int)(K / kGroupK);
  auto dma_part = [&](int g, int buf, int part) {
    uint8_t *gbuf = smem + buf * kGroupBytes;
    const bool gin = g < ng;
    const int q0 = part == 3 ? 0 : 5 * part + 5, q1 = part == 3 ? 5 : part == 2 ? 16 : q0 + 5;
#pragma unroll
    for (int qq = q0; qq < q1; ++qq) {
      const bool real = !(BN == 128 && dma_b && qq >= 8);
      const int lrow = real ? lds_row0 + 8 * qq : spare_row0 + 8 * (qq - 8);
      dma16(dcodes, gbuf + lrow * 128, dv_code, (gin && real) ? 128u * (uint32_t)g + 8u * qq * rb : kOutOfRange);
    }
    if (part == 2 && (g & 1) == 0) {   // scales of groups g, g+1: 128 or 64 rows per wave
      uint8_t *sbuf = smem + 2 * kGroupBytes + ((g >> 1) & 1) * kScalePair;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bool real = !(BN == 128 && dma_b && half >= 1);
        const int lrow = real ? lds_row0 + 64 * half : spare_row0;
        dma16(dscales, sbuf + lrow * 16, dv_scale, (gin && real) ? 8u * (uint32_t)g + 64u * half * rs : kOutOfRange);
      }
    }
  };

  // ---- read side: fragment f of stage sp: 16 code bytes (one 32-block)
  // and its scale byte
  const uint32_t a_row = 128 * wm + r, b_row = BM + (BN / 2) * wn + r;
  u32x4 codes[2][NF];
  int sc[2][NF];
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  u32x2 srow[NF];          // the fragment rows' 8 scale bytes of one group
  auto read_stage = [&](int cb, const uint8_t *gb, int sp) {
    const int c = 2 * sp + h;
    const uint32_t slot = (uint32_t)((c ^ (r & 7)) * 16);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t row = f < 4 ? a_row + 32 * f : b_row + 32 * (f - 4);
      codes[cb][f] = *reinterpret_cast<const u32x4 *>(gb + row * 128 + slot);
    }
  };
  // one 8-byte read per fragment row and group (a byte read per fragment
  // and stage cost 10 % of the dgrad shape in a timing copy)
  auto read_scales = [&](int g) {
    const uint8_t *sb = smem + 2 * kGroupBytes + ((g >> 1) & 1) * kScalePair + 8 * (g & 1);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t row = f < 4 ? a_row + 32 * f : b_row + 32 * (f - 4);
      srow[f] = *reinterpret_cast<const u32x2 *>(sb + row * 16);
    }
  };
  // fragment f's scale byte for stage sp: byte 2 sp + h of the group's 8
  auto pick_scale = [&](int cb, int f, int sp) {
    sc[cb][f] = (int)((srow[f][sp >> 1] >> (8 * ((2 * sp + h) & 3))) & 0xFFu);
  };

  float16_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

#pragma unroll
  for (int part = 0; part < 4; ++part) dma_part(0, 0, part);
  dma_part(1, 1, 3);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  read_stage(0, smem, 0);
  read_scales(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) pick_scale(0, f, 0);
  __builtin_amdgcn_s_waitcnt(0);

  // Stage s = 4g + P: read the next stage's operands (in the last stage of a
  // group, after the group barrier), issue one part of the prefetch DMA,
  // then the 4 x NB MFMAs of this stage in snake order.
  auto stage = [&](int g, auto phase) {
    constexpr int P = decltype(phase)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    const uint8_t *gb = smem + (g & 1) * kGroupBytes;
    const uint8_t *gn = smem + ((g + 1) & 1) * kGroupBytes;
    __builtin_amdgcn_sched_barrier(0);
    if (P == 3) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA of group g+1
      __syncthreads();
      read_stage(nxt, gn, 0);
      read_scales(g + 1);
      dma_part(g + 2, g & 1, 3);
    } else {
      read_stage(nxt, gb, P + 1);
      dma_part(g + 1, (g + 1) & 1, P);
    }
    // the next stage's scale bytes are taken from srow between the MFMAs
    constexpr int psp = P == 3 ? 0 : P + 1;
#pragma unroll
    for (int u = 0; u < 4 * NB; ++u) {
      const int mi = u / NB, mj = (mi & 1) ? NB - 1 - u % NB : u % NB;
      const u32x4 ca = codes[cur][mi], cbv = codes[cur][4 + mj];
      const v8i av = {(int)ca.x, (int)ca.y, (int)ca.z, (int)ca.w, 0, 0, 0, 0};
      const v8i bv = {(int)cbv.x, (int)cbv.y, (int)cbv.z, (int)cbv.w, 0, 0, 0, 0};
      acc[mi][mj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[mi][mj], 4, 4, 0, sc[cur][mi], 0,
                                                                   sc[cur][4 + mj]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = (u * NF) / (4 * NB); f < ((u + 1) * NF) / (4 * NB); ++f) pick_scale(nxt, f, psp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  for (int g = 0; g < ng; ++g) {
    stage(g, P0{});
    stage(g, P1{});
    stage(g, P2{});
    stage(g, P3{});
  }
  __builtin_amdgcn_sched_barrier(0);

  const int64_t row_l = m0 + wm * 128 + 4 * h, col_l = n0 + wn * (BN / 2) + r;
  const bool full_tile = (m0 + BM <= M) && (n0 + BN <= N);
  using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
  OutT *base = reinterpret_cast<OutT *>(C) + row_l * ldc + col_l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int roff = 32 * i + 8 * (e >> 2) + (e & 3);
      if (!full_tile && row_l + roff >= M) continue;
      OutT *prow = base + (int64_t)roff * ldc;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (!full_tile && col_l + 32 * j >= N) continue;
        if constexpr (OUT_BF16)
          __builtin_nontemporal_store(f32_to_bf16_rne(acc[i][j][e]), prow + 32 * j);   // streaming: C is written once
        else
          __builtin_nontemporal_store(acc[i][j][e], prow + 32 * j);
      }
    }
  }
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_mx_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const uint8_t *__restrict__ B,
          const uint8_t *__restrict__ SB, int64_t M, int64_t N, int64_t K, void *__restrict__ C, int64_t ldc,
          int n_big, int64_t n1) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  const int pid = blockIdx.x;
  if (pid < n_big) {
    mx_gemm_tile<OUT_BF16, 256>(smem, pid, A, SA, B, SB, M, n1, K, C, ldc);
  } else {
    using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
    mx_gemm_tile<OUT_BF16, 128>(smem, pid - n_big, A, SA, B + n1 * (K / 2), SB + n1 * (K / 32), M, N - n1, K,
                                reinterpret_cast<OutT *>(C) + n1, ldc);
  }
}

__global__ void k_mx_zero_c(void *C, int64_t M, int64_t N, int64_t ldc, int elem) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t rr = i / N, cc = i - rr * N;
    if (elem == 4) reinterpret_cast<float *>(C)[rr * ldc + cc] = 0.0f;
    else reinterpret_cast<uint16_t *>(C)[rr * ldc + cc] = 0;
  }
}

}  // namespace

hipError_t launch_mx_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const bool bf16 = (x_dtype == 1);
  if (axis == 1) {
    const int64_t nblocks = n / 32;
    const unsigned g = (unsigned)std::min<int64_t>((nblocks + kQT - 1) / kQT, 1 << 20);
    if (bf16) hipLaunchKernelGGL(k_mx_quant_rows<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint16_t *)x, nblocks, (uint4 *)codes, scales);
    else hipLaunchKernelGGL(k_mx_quant_rows<float>, dim3(g), dim3(kQT), 0, stream, (const float *)x, nblocks, (uint4 *)codes, scales);
  } else {
    const int64_t cpt = bf16 ? 2 : 1;
    const int64_t gy = (rows / 32 + 7) / 8;
    if (gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((cols + 64 * cpt - 1) / (64 * cpt)), (unsigned)gy);
    if (bf16) hipLaunchKernelGGL(k_mx_quant_cols<uint16_t>, grid, dim3(kQT), 0, stream, (const uint16_t *)x, rows, cols, (uint4 *)codes, scales);
    else hipLaunchKernelGGL(k_mx_quant_cols<float>, grid, dim3(kQT), 0, stream, (const float *)x, rows, cols, (uint4 *)codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_mx_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                          const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                          hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    const int64_t total = M * N;
    const unsigned g = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_mx_zero_c, dim3(g), dim3(256), 0, stream, c, M, N, ldc, c_dtype == 0 ? 4 : 2);
    return hipGetLastError();
  }
  if (K % kGroupK != 0 || (int64_t)128 * (K / 2) >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  // same column split as the NVFP4 GEMM: 256-wide tiles, then 128-wide ones
  const int64_t cus = device_cus();
  const int64_t tm = (M + BM - 1) / BM, tn = (N + 255) / 256;
  auto rounds = [&](int64_t t) { return (t + cus - 1) / cus; };
  int64_t best_n1 = N;
  double best = (double)rounds(tm * tn);
  for (int64_t t1 = 0; t1 < tn; ++t1) {
    const int64_t n1 = t1 * 256, rest = (N - n1 + 127) / 128;
    const double cost = (double)rounds(tm * t1) + 0.55 * (double)rounds(tm * rest);
    if (cost < best - 1e-9) { best = cost; best_n1 = n1; }
  }
  // best_n1 is a multiple of 256 or N itself (no split: the last tile
  // column may be ragged, so round up)
  const int64_t n_big = tm * ((best_n1 + 255) / 256), n_small = tm * ((N - best_n1 + 127) / 128);
  if (n_big + n_small > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(n_big + n_small));
  if (c_dtype == 0)
    hipLaunchKernelGGL((k_mx_gemm<false>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, b_codes, b_scales, M, N,
                       K, c, ldc, (int)n_big, best_n1);
  else
    hipLaunchKernelGGL((k_mx_gemm<true>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, b_codes, b_scales, M, N,
                       K, c, ldc, (int)n_big, best_n1);
  return hipGetLastError();
}

}  // namespace nvfp4
