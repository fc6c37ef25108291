// gemm.hip -- block-scaled NVFP4 GEMM with FP32 accumulation on gfx950 MFMA.
//
// [P1] hyper.ai "NVIDIA revolutioniert KI-Praetrainingsgeschwindigkeit mit
// 4-Bit-Genauigkeit" (body): the 4-bit recipe rests on accelerated GEMMs;
// [P4] aisight.pl "Koniec marnowania mocy ...", section "Architektura NVFP4
// kontra ograniczenia mikroskalowania": the operands carry an E4M3 scale per
// 16 elements and an FP32 scale per tensor.
//
//   C[m][n] = gA * gB * sum_k (qA * SA)[m][k] * (qB * SB)[n][k]
//
// Design for CDNA4: gfx950's block-scaled MFMA forms take power-of-two
// (E8M0) scales per 32 elements, which cannot represent an E4M3 scale per 16
// elements.  Each element is therefore decoded exactly in registers: the
// hardware FP4->F16 conversion gives q, and one packed f16 multiply by the
// block scale S gives q*S, which has at most 6 significant bits and lies in
// [2^-10, 2688], so it is exact in f16.  The exact products feed
// v_mfma_f32_32x32x16_f16 with f32 accumulators; every 16-block partial sum
// is exact, so the accumulation rounds once per 16-element step.
//
// Tiling: a 256-thread workgroup computes a 128x128 tile of C; each of its
// four waves owns a 64x64 sub-tile (2x2 MFMA tiles of 32x32).  The K loop
// stages 128 K-elements of packed codes (64 bytes per row) and their eight
// scales per row in LDS; each lane then reads 16 bytes (32 codes) of one row
// per 64-K half.  Lane l of an MFMA fragment holds K positions
// 64*kk + 32*(l/32) + 8*s + [0,8) for step s: a permutation of K applied
// identically to A and B, which leaves the sum unchanged.
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

namespace nvfp4 {

namespace {

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int BKB = BK / 2;        // code bytes per row per K tile
constexpr int BKS = BK / 16;       // scales per row per K tile
constexpr int LDSB = BKB + 16;     // padded LDS row stride of the code tiles
constexpr int kThreads = 256;

// 16 code bytes of row `row` starting at byte `kb` (K/2 bytes per row);
// zero outside the matrix.  The tail of a row may hold only 8 valid bytes.
__device__ __forceinline__ uint4 load_codes16(const uint8_t *p, int64_t rows, int64_t KB, int64_t row,
                                              int64_t kb, bool al16) {
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row >= rows) return v;
  const uint8_t *src = p + row * KB + kb;
  if (kb + 16 <= KB) {
    if (al16) {
      v = *reinterpret_cast<const uint4 *>(src);
    } else {
      uint2 a = *reinterpret_cast<const uint2 *>(src);
      uint2 b = *reinterpret_cast<const uint2 *>(src + 8);
      v = make_uint4(a.x, a.y, b.x, b.y);
    }
  } else if (kb + 8 <= KB) {
    uint2 a = *reinterpret_cast<const uint2 *>(src);
    v = make_uint4(a.x, a.y, 0, 0);
  }
  return v;
}

// 4 scale bytes of row `row` starting at scale index `ks`; zero outside.
__device__ __forceinline__ uint32_t load_scales4(const uint8_t *p, int64_t rows, int64_t KS, int64_t row,
                                                 int64_t ks) {
  uint32_t v = 0;
  if (row >= rows) return v;
  const uint8_t *src = p + row * KS;
#pragma unroll
  for (int t = 0; t < 4; ++t)
    if (ks + t < KS) v |= (uint32_t)src[ks + t] << (8 * t);
  return v;
}

// 8 E2M1 codes (one 32-bit word, element 0 in the low nibble) -> 8 exact
// f16 values of q * S.
__device__ __forceinline__ half8_t decode8(uint32_t w, _Float16 S) {
  half2_t s2 = {S, S};
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  half8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t b) { return (_Float16)e4m3_to_f32(b); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(kThreads) k_gemm_nvfp4(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                                                       const float *__restrict__ metaA, const uint8_t *__restrict__ B,
                                                       const uint8_t *__restrict__ SB, const float *__restrict__ metaB,
                                                       int64_t M, int64_t N, int64_t K, void *__restrict__ C,
                                                       int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[BM * LDSB];
  __shared__ __attribute__((aligned(16))) uint8_t sB[BN * LDSB];
  __shared__ __attribute__((aligned(16))) uint8_t sSA[BM * BKS];
  __shared__ __attribute__((aligned(16))) uint8_t sSB[BN * BKS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t KB = K / 2, KS = K / 16;
  const bool alA = (KB % 16 == 0) && (((uintptr_t)A & 15) == 0);
  const bool alB = (KB % 16 == 0) && (((uintptr_t)B & 15) == 0);

  float16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    uint4 ra[2], rb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, r = c >> 2, q = c & 3;
      ra[i] = load_codes16(A, M, KB, m0 + r, k0 / 2 + 16 * q, alA);
      rb[i] = load_codes16(B, N, KB, n0 + r, k0 / 2 + 16 * q, alB);
    }
    const int sr = tid >> 1, s4 = (tid & 1) * 4;
    const uint32_t rsa = load_scales4(SA, M, KS, m0 + sr, k0 / 16 + s4);
    const uint32_t rsb = load_scales4(SB, N, KS, n0 + sr, k0 / 16 + s4);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + kThreads * i, r = c >> 2, q = c & 3;
      *reinterpret_cast<uint4 *>(&sA[r * LDSB + 16 * q]) = ra[i];
      *reinterpret_cast<uint4 *>(&sB[r * LDSB + 16 * q]) = rb[i];
    }
    *reinterpret_cast<uint32_t *>(&sSA[sr * BKS + s4]) = rsa;
    *reinterpret_cast<uint32_t *>(&sSB[sr * BKS + s4]) = rsb;
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8_t af[2][4], bf[2][4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = wm * 64 + 32 * i + l32;
        const uint4 w = *reinterpret_cast<const uint4 *>(&sA[row * LDSB + kk * 32 + 16 * lh]);
        const _Float16 s0 = scale_f16(sSA[row * BKS + kk * 4 + 2 * lh]);
        const _Float16 s1 = scale_f16(sSA[row * BKS + kk * 4 + 2 * lh + 1]);
        af[i][0] = decode8(w.x, s0);
        af[i][1] = decode8(w.y, s0);
        af[i][2] = decode8(w.z, s1);
        af[i][3] = decode8(w.w, s1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = wn * 64 + 32 * j + l32;
        const uint4 w = *reinterpret_cast<const uint4 *>(&sB[col * LDSB + kk * 32 + 16 * lh]);
        const _Float16 s0 = scale_f16(sSB[col * BKS + kk * 4 + 2 * lh]);
        const _Float16 s1 = scale_f16(sSB[col * BKS + kk * 4 + 2 * lh + 1]);
        bf[j][0] = decode8(w.x, s0);
        bf[j][1] = decode8(w.y, s0);
        bf[j][2] = decode8(w.z, s1);
        bf[j][3] = decode8(w.w, s1);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: C = (acc * gA) * gB; lane holds column l32 and rows
  // 8*a + 4*lh + b of each 32x32 tile (register 4*a + b).
  const float gA = metaA[1], gB = metaB[1];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + 32 * j + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row >= M) continue;
        const float v = (acc[i][j][r] * gA) * gB;
        if (OUT_BF16)
          reinterpret_cast<uint16_t *>(C)[row * ldc + col] = f32_to_bf16_rne(v);
        else
          reinterpret_cast<float *>(C)[row * ldc + col] = v;
      }
    }
  }
}

__global__ void k_zero_c(void *C, int64_t M, int64_t N, int64_t ldc, int elem) {
  const int64_t total = M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    int64_t r = i / N, c = i - r * N;
    if (elem == 4) reinterpret_cast<float *>(C)[r * ldc + c] = 0.0f;
    else reinterpret_cast<uint16_t *>(C)[r * ldc + c] = 0;
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_meta,
                       const uint8_t *b_codes, const uint8_t *b_scales, const float *b_meta, int64_t M,
                       int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    int64_t total = M * N;
    unsigned g = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_zero_c, dim3(g), dim3(256), 0, stream, c, M, N, ldc, c_dtype == 0 ? 4 : 2);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (c_dtype == 0)
    hipLaunchKernelGGL(k_gemm_nvfp4<false>, grid, dim3(kThreads), 0, stream, a_codes, a_scales, a_meta, b_codes,
                       b_scales, b_meta, M, N, K, c, ldc);
  else
    hipLaunchKernelGGL(k_gemm_nvfp4<true>, grid, dim3(kThreads), 0, stream, a_codes, a_scales, a_meta, b_codes,
                       b_scales, b_meta, M, N, K, c, ldc);
  return hipGetLastError();
}

}  // namespace nvfp4
