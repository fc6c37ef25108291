// mx8.hip -- MXFP8 quantizer and GEMM on gfx950's block-scaled MFMA.
//
// MXFP8 is the 8-bit member of the microscaling family: one of the three
// number formats of the training run in [P3] aibuzzwire.news "End-to-End
// 4-Bit Training", section "Drei Formate, ein Trainingslauf" (about 5 PFLOPS
// on GB300), with the 32-element power-of-two-scaled blocks that [P4]
// aisight.pl "Koniec marnowania mocy ...", section "Architektura NVFP4 kontra
// ograniczenia mikroskalowania", sets NVFP4 against.  Elements are OCP
// E4M3FN bytes; each 32-block along K carries an E8M0 exponent (scale
// 2^(code - 127)); there is no tensor scale.  Block scale: the smallest power
// of two X = 2^e with amax_b / X <= 448 (the block maximum is never
// clipped), e clamped to [-127, 127]; elements are the nearest-even E4M3
// codes of x / X, sign kept.
//
// GEMM operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 with FP8 operands
// (measured on the device): of the 32 bytes a lane holds, bytes 0-15 belong
// to the instruction's first 32-block and bytes 16-31 to its second, in both
// lane halves; lane r passes the scale of the first block of row r and lane
// r + 32 that of the second.  So memory block b of a row (32 bytes) is split
// as its bytes 0-15 in lane r and bytes 16-31 in lane r + 32.  The
// instruction sums its products in aligned groups of 8 K positions, each
// product truncated to 13 bits below the group's largest exponent sum (the
// GEMM's tolerance is stated from that), so the K order within a lane keeps
// memory order: every group is 8 consecutive K positions of one block.
#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int kQT = kQuantThreads;

// ------------------------------------------------------------ quantize ----

// Smallest e with amax <= 448 * 2^e for the bit pattern of amax >= 0:
// 448 * 2^e = 1.75 * 2^(e+8), so for amax = m * 2^E (m in [1, 2)) e = E - 8
// when m <= 1.75 and E - 7 otherwise; zero and subnormal maxima fit e = -127.
__device__ __forceinline__ int mx8_exp(uint32_t amax_bits) {
  if (amax_bits < 0x00800000u) return -127;
  const int E = (int)(amax_bits >> 23) - 127;
  const int e = (amax_bits & 0x7FFFFFu) <= 0x600000u ? E - 8 : E - 7;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^n as binary32 for n in [-127, 127] (2^-127 is subnormal).
__device__ __forceinline__ float pow2f_mx8(int n) {
  return n >= -126 ? __uint_as_float((uint32_t)(n + 127) << 23) : __uint_as_float(0x00400000u);
}

// E4M3 code of v with |v| <= 448 (nearest even, sign of v kept).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  return ((__float_as_uint(v) >> 24) & 0x80u) | e4m3_rne_sat(fabsf(v));
}

// Codes (8 words, element j in byte j % 4 of word j / 4) and scale of one
// 32-block held as binary32 values y[0..31].
__device__ __forceinline__ void mx8_encode32(const float *y, uint32_t *w, uint8_t *scale) {
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = max(m, __float_as_uint(y[j]) & 0x7FFFFFFFu);
  const int e = mx8_exp(m);
  *scale = (uint8_t)(e + 127);
  const float inv = pow2f_mx8(-e);   // x * 2^-e is x / X rounded once (exact unless below 2^-126)
#pragma unroll
  for (int i = 0; i < 8; ++i)
    w[i] = e4m3_code(y[4 * i] * inv) | (e4m3_code(y[4 * i + 1] * inv) << 8) |
           (e4m3_code(y[4 * i + 2] * inv) << 16) | (e4m3_code(y[4 * i + 3] * inv) << 24);
}

// axis 1: one thread per 32-block of a row (64 B of bf16 in, 32 B of codes
// out in two 16-byte stores).
template <typename T>
__global__ void __launch_bounds__(kQT) k_mx8_quant_rows(const T *x, int64_t nblocks, uint4 *codes, uint8_t *scales) {
  const int64_t stride = (int64_t)gridDim.x * kQT;
  for (int64_t b = (int64_t)blockIdx.x * kQT + threadIdx.x; b < nblocks; b += stride) {
    float y[32];
    Load16<T>::run(x + 32 * b, y);
    Load16<T>::run(x + 32 * b + 16, y + 16);
    uint32_t w[8];
    uint8_t s;
    mx8_encode32(y, w, &s);
    codes[2 * b] = make_uint4(w[0], w[1], w[2], w[3]);
    codes[2 * b + 1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[b] = s;
  }
}

// axis 0 (K runs down the columns, output transposed): a thread takes two
// adjacent bf16 columns (one f32 column) and one 32-row block; the four
// waves of a workgroup share their columns and take consecutive blocks, so
// each 128-byte output line (four blocks of one column) is written by one
// workgroup.
template <typename T>
__global__ void __launch_bounds__(kQT) k_mx8_quant_cols(const T *x, int64_t rows, int64_t cols, uint4 *codes,
                                                       uint8_t *scales) {
  constexpr int CPT = 4 / (int)sizeof(T);
  constexpr int kCols = 64 * CPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c = ((int64_t)blockIdx.x * 64 + lane) * CPT;
  const int64_t nkb = rows / 32, kb = (int64_t)blockIdx.y * 4 + wave;
  // A workgroup tile wholly inside x (its kCols columns x 4 blocks, output
  // lines 128-byte aligned) goes out through LDS as whole lines, 8 per store
  // instruction, instead of two 16-byte pieces per lane and line.
  const int64_t c_wg = (int64_t)blockIdx.x * kCols, kb_wg = (int64_t)blockIdx.y * 4;
  const bool whole = (c_wg + kCols <= cols) && (kb_wg + 4 <= nkb) && (nkb % 4 == 0) && (CPT == 1 || cols % 2 == 0) &&
                     ((uintptr_t)codes & 127) == 0 && ((uintptr_t)scales & 3) == 0;
  __shared__ __attribute__((aligned(16))) uint4 tile_codes[kCols][9];    // 144-byte rows: no bank conflicts
  __shared__ __attribute__((aligned(4))) uint8_t tile_scales[kCols][4];
  if (whole) {
    float y[CPT][32];
    const T *p = x + 32 * kb * cols + c;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t wd = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + j * cols));
      if constexpr (CPT == 2) {
        y[0][j] = bf16_lo(wd);
        y[1][j] = bf16_hi(wd);
      } else {
        y[0][j] = __uint_as_float(wd);
      }
    }
#pragma unroll
    for (int e = 0; e < CPT; ++e) {
      uint32_t w[8];
      uint8_t sb;
      mx8_encode32(y[e], w, &sb);
      tile_codes[lane * CPT + e][2 * wave] = make_uint4(w[0], w[1], w[2], w[3]);
      tile_codes[lane * CPT + e][2 * wave + 1] = make_uint4(w[4], w[5], w[6], w[7]);
      tile_scales[lane * CPT + e][wave] = sb;
    }
    __syncthreads();
    // codes: column q / 8, 16-byte piece q % 8 of its line
#pragma unroll
    for (int r = 0; r < kCols * 8 / kQT; ++r) {
      const int q = r * kQT + (int)threadIdx.x, col = q >> 3, piece = q & 7;
      codes[2 * ((c_wg + col) * nkb + kb_wg) + piece] = tile_codes[col][piece];
    }
    if (threadIdx.x < kCols) {
      const int col = threadIdx.x;
      *reinterpret_cast<uint32_t *>(scales + (c_wg + col) * nkb + kb_wg) =
          *reinterpret_cast<const uint32_t *>(tile_scales[col]);
    }
    return;
  }
  if (c >= cols || kb >= nkb) return;
  const bool fast = (c + CPT <= cols) && (CPT == 1 || (cols % 2) == 0);
  float y[CPT][32];
  const T *p = x + 32 * kb * cols + c;
  if (fast) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t wd = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p + j * cols));
      if constexpr (CPT == 2) {
        y[0][j] = bf16_lo(wd);
        y[1][j] = bf16_hi(wd);
      } else {
        y[0][j] = __uint_as_float(wd);
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
    uint32_t w[8];
    uint8_t s;
    mx8_encode32(y[e], w, &s);
    const int64_t blk = (c + e) * nkb + kb;
    codes[2 * blk] = make_uint4(w[0], w[1], w[2], w[3]);
    codes[2 * blk + 1] = make_uint4(w[4], w[5], w[6], w[7]);
    scales[blk] = s;
  }
}

// ---------------------------------------------------------------- GEMM ----
//
// One 256-thread workgroup per 256 x BN tile (BN = 256, or 128 for the
// column remainder), four waves of 128 x BN/2.  K is consumed in groups of
// 128 (two 64-wide stages): a group is one 128-byte line per operand row,
// the same bytes per row and group as the FP4 kernels, so the DMA of codes
// into LDS is theirs (chunk c of row R in slot c ^ (R & 7)).  The scales of
// four groups (16 bytes per row) come in one 16-byte DMA per row, 64 rows
// per instruction, into one of two quad buffers (one 4-byte DMA per 64 rows
// and group touched a cache line per lane: the same change in the MXFP4
// kernel gained 3-5 %).  Per stage each fragment reads two 16-byte chunks
// (4s' + h and 4s' + 2 + h) and one scale byte (block 2s' + h), and one MFMA
// step covers 64 K.  Requires K % 128 == 0.

constexpr int BM = 256;
constexpr int kThreads = 256;
constexpr int kGroupK = 128;
constexpr int kRowsMax = BM + 256;
constexpr int kCodeBytes = kRowsMax * 128;      // 64 KB
constexpr int kGroupBytes = kCodeBytes;         // a group buffer: codes only
constexpr int kScaleQuad = kRowsMax * 16;       // 8 KB: the scales of four groups
constexpr int kLdsBytes = 2 * kGroupBytes + 2 * kScaleQuad;
constexpr int kGroupM = 8;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <bool OUT_BF16, int BN>
__device__ __forceinline__ void mx8_gemm_tile(uint8_t *smem, int pid, const uint8_t *__restrict__ A,
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

  // ---- DMA side (rows past M or N read as zeros)
  const uint32_t rb = (uint32_t)K, rs = (uint32_t)(K / 32);
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
  // Part `part` of the DMA of group g into buffer buf: the 16 code
  // instructions in three parts (0-4, 5-9, then 10-15 with the two scale
  // instructions).  A group past the last one gets offsets beyond every
  // view, so the prefetch needs no branch at the end of K.
  auto dma_part = [&](int g, int buf, int part) {
    uint8_t *gbuf = smem + buf * kGroupBytes;
    const bool gin = g < ng;
    const int q0 = part == 0 ? 0 : part == 1 ? 5 : 10, q1 = part == 0 ? 5 : part == 1 ? 10 : 16;
#pragma unroll
    for (int qq = q0; qq < q1; ++qq) {
      const bool real = !(BN == 128 && dma_b && qq >= 8);
      const int lrow = real ? lds_row0 + 8 * qq : spare_row0 + 8 * (qq - 8);
      dma16(dcodes, gbuf + lrow * 128, dv_code, (gin && real) ? 128u * (uint32_t)g + 8u * qq * rb : kOutOfRange);
    }
    if (part == 2 && (g & 3) == 0) {   // scales of groups g .. g+3
      uint8_t *sbuf = smem + 2 * kGroupBytes + ((g >> 2) & 1) * kScaleQuad;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bool real = !(BN == 128 && dma_b && half >= 1);
        const int lrow = real ? lds_row0 + 64 * half : spare_row0;
        dma16(dscales, sbuf + lrow * 16, dv_scale, (gin && real) ? 4u * (uint32_t)g + 64u * half * rs : kOutOfRange);
      }
    }
  };

  // ---- read side: fragment f of stage sp: chunks 4sp+h (block 2sp) and
  // 4sp+2+h (block 2sp+1), and the scale byte of block 2sp+h
  const uint32_t a_row = 128 * wm + r, b_row = BM + (BN / 2) * wn + r;
  u32x4 lo[2][NF], hi[2][NF];
  int sc[2][NF];
  uint32_t srow[NF];       // the fragment rows' 4 scale bytes of one group
  auto read_stage = [&](int cb, const uint8_t *gb, int sp) {
    const int c0 = 4 * sp + h, c1 = 4 * sp + 2 + h;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t row = f < 4 ? a_row + 32 * f : b_row + 32 * (f - 4);
      lo[cb][f] = *reinterpret_cast<const u32x4 *>(gb + row * 128 + (uint32_t)((c0 ^ (r & 7)) * 16));
      hi[cb][f] = *reinterpret_cast<const u32x4 *>(gb + row * 128 + (uint32_t)((c1 ^ (r & 7)) * 16));
    }
  };
  // one 4-byte read per fragment row and group (bytes 4 (g % 4) .. of the
  // row in the quad buffer), instead of a byte read per fragment and stage
  auto read_scales = [&](int g) {
    const uint8_t *sb = smem + 2 * kGroupBytes + ((g >> 2) & 1) * kScaleQuad + 4 * (g & 3);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t row = f < 4 ? a_row + 32 * f : b_row + 32 * (f - 4);
      srow[f] = *reinterpret_cast<const uint32_t *>(sb + row * 16);
    }
  };
  // fragment f's scale byte for stage sp: byte 2 sp + h of the group's 4
  auto pick_scale = [&](int cb, int f, int sp) { sc[cb][f] = (int)((srow[f] >> (8 * (2 * sp + h))) & 0xFFu); };

  float16_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

#pragma unroll
  for (int part = 0; part < 3; ++part) dma_part(0, 0, part);
  dma_part(1, 1, 0);
  dma_part(1, 1, 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  read_stage(0, smem, 0);
  read_scales(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) pick_scale(0, f, 0);
  __builtin_amdgcn_s_waitcnt(0);

  // Stage s = 2g + P: read the next stage's operands (in the last stage of
  // a group, after the group barrier), issue prefetch DMA, then the 4 x NB
  // MFMAs of this stage in snake order.  Group g+1 moves in three parts:
  // parts 0 and 1 right after the barrier of group g-1's last stage (its
  // buffer is free then), part 2 in stage 0 of group g; the last stage of
  // group g waits for all three before its barrier.
  auto stage = [&](int g, auto phase) {
    constexpr int P = decltype(phase)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    const uint8_t *gb = smem + (g & 1) * kGroupBytes;
    const uint8_t *gn = smem + ((g + 1) & 1) * kGroupBytes;
    __builtin_amdgcn_sched_barrier(0);
    if (P == 1) {
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA of group g+1
      __syncthreads();
      read_stage(nxt, gn, 0);
      read_scales(g + 1);
      dma_part(g + 2, g & 1, 0);
      dma_part(g + 2, g & 1, 1);
    } else {
      read_stage(nxt, gb, 1);
      dma_part(g + 1, (g + 1) & 1, 2);
    }
    // the next stage's scale bytes are taken from srow between the MFMAs
    constexpr int psp = P == 1 ? 0 : 1;
#pragma unroll
    for (int u = 0; u < 4 * NB; ++u) {
      const int mi = u / NB, mj = (mi & 1) ? NB - 1 - u % NB : u % NB;
      const u32x4 al = lo[cur][mi], ah = hi[cur][mi], bl = lo[cur][4 + mj], bh = hi[cur][4 + mj];
      const v8i av = {(int)al.x, (int)al.y, (int)al.z, (int)al.w, (int)ah.x, (int)ah.y, (int)ah.z, (int)ah.w};
      const v8i bv = {(int)bl.x, (int)bl.y, (int)bl.z, (int)bl.w, (int)bh.x, (int)bh.y, (int)bh.z, (int)bh.w};
      acc[mi][mj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[mi][mj], 0, 0, 0, sc[cur][mi], 0,
                                                                   sc[cur][4 + mj]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = (u * NF) / (4 * NB); f < ((u + 1) * NF) / (4 * NB); ++f) pick_scale(nxt, f, psp);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  for (int g = 0; g < ng; ++g) {
    stage(g, P0{});
    stage(g, P1{});
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);

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
k_mx8_gemm(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const uint8_t *__restrict__ B,
           const uint8_t *__restrict__ SB, int64_t M, int64_t N, int64_t K, void *__restrict__ C, int64_t ldc,
           int n_big, int64_t n1) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  const int pid = blockIdx.x;
  if (pid < n_big) {
    mx8_gemm_tile<OUT_BF16, 256>(smem, pid, A, SA, B, SB, M, n1, K, C, ldc);
  } else {
    using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
    mx8_gemm_tile<OUT_BF16, 128>(smem, pid - n_big, A, SA, B + n1 * K, SB + n1 * (K / 32), M, N - n1, K,
                                 reinterpret_cast<OutT *>(C) + n1, ldc);
  }
}

__global__ void k_mx8_zero_c(void *C, int64_t M, int64_t N, int64_t ldc, int elem) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t rr = i / N, cc = i - rr * N;
    if (elem == 4) reinterpret_cast<float *>(C)[rr * ldc + cc] = 0.0f;
    else reinterpret_cast<uint16_t *>(C)[rr * ldc + cc] = 0;
  }
}

}  // namespace

hipError_t launch_mx8_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, uint8_t *codes,
                               uint8_t *scales, hipStream_t stream) {
  const int64_t n = rows * cols;
  if (n == 0) return hipSuccess;
  const bool bf16 = (x_dtype == 1);
  if (axis == 1) {
    const int64_t nblocks = n / 32;
    const unsigned g = (unsigned)std::min<int64_t>((nblocks + kQT - 1) / kQT, 1 << 20);
    if (bf16) hipLaunchKernelGGL(k_mx8_quant_rows<uint16_t>, dim3(g), dim3(kQT), 0, stream, (const uint16_t *)x, nblocks, (uint4 *)codes, scales);
    else hipLaunchKernelGGL(k_mx8_quant_rows<float>, dim3(g), dim3(kQT), 0, stream, (const float *)x, nblocks, (uint4 *)codes, scales);
  } else {
    const int64_t cpt = bf16 ? 2 : 1;
    const int64_t gy = (rows / 32 + 3) / 4;
    if (gy > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((cols + 64 * cpt - 1) / (64 * cpt)), (unsigned)gy);
    if (bf16) hipLaunchKernelGGL(k_mx8_quant_cols<uint16_t>, grid, dim3(kQT), 0, stream, (const uint16_t *)x, rows, cols, (uint4 *)codes, scales);
    else hipLaunchKernelGGL(k_mx8_quant_cols<float>, grid, dim3(kQT), 0, stream, (const float *)x, rows, cols, (uint4 *)codes, scales);
  }
  return hipGetLastError();
}

hipError_t launch_mx8_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                           const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                           hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    const int64_t total = M * N;
    const unsigned g = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_mx8_zero_c, dim3(g), dim3(256), 0, stream, c, M, N, ldc, c_dtype == 0 ? 4 : 2);
    return hipGetLastError();
  }
  // 128 rows of K code bytes addressed by 32-bit buffer offsets below 2^31
  if (K % kGroupK != 0 || (int64_t)128 * K >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  // same column split as the other GEMMs: 256-wide tiles, then 128-wide ones
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
  const int64_t n_big = tm * ((best_n1 + 255) / 256), n_small = tm * ((N - best_n1 + 127) / 128);
  if (n_big + n_small > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(n_big + n_small));
  if (c_dtype == 0)
    hipLaunchKernelGGL((k_mx8_gemm<false>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, b_codes, b_scales, M,
                       N, K, c, ldc, (int)n_big, best_n1);
  else
    hipLaunchKernelGGL((k_mx8_gemm<true>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, b_codes, b_scales, M,
                       N, K, c, ldc, (int)n_big, best_n1);
  return hipGetLastError();
}

}  // namespace nvfp4
