// nvfp4_kernels.h -- host-side launch entry points of the gfx950 kernels
// (internal to the library; the public C ABI is include/nvfp4.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr int kQuantThreads = 256;

// Compute units of the current device (cached per device id).
int device_cus();

// Enqueue meta reset, amax and encode for one quantization.  Arguments are
// validated by the caller; x_dtype 0 = f32, 1 = bf16; rounding 0 = RNE,
// 1 = SR; rht selects the fused Hadamard transform.
hipError_t launch_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                           uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, uint8_t *codes,
                           uint8_t *scales, float *meta, hipStream_t stream);

// Pass 1 alone: amax[0] = the tensor amax (after the transform if rht).
hipError_t launch_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, bool rht,
                       uint32_t sign_mask, float *amax, hipStream_t stream);

// Pass 2 alone, with the tensor amax supplied in device memory.
hipError_t launch_quantize_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                                uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, const float *amax,
                                uint8_t *codes, uint8_t *scales, float *meta, hipStream_t stream);

// One input, two quantizations with one amax read: the axis-1 output (no
// transform) and the axis-0 output (with or without the RHT); each output is
// bit-identical to launch_quantize's.
hipError_t launch_quantize_dual(const void *x, int x_dtype, int64_t rows, int64_t cols, int rounding1,
                                uint64_t seed1, uint64_t offset1, uint8_t *codes1, uint8_t *scales1, float *meta1,
                                bool rht0, uint32_t sign_mask0, int rounding0, uint64_t seed0, uint64_t offset0,
                                uint8_t *codes0, uint8_t *scales0, float *meta0, hipStream_t stream);

// MXFP4 (32-element E2M1 blocks with E8M0 scales): quantize on axis 1 or 0,
// and C = A . B^T on the block-scaled FP4 MFMA (K % 256 == 0).
hipError_t launch_mx_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, uint8_t *codes,
                              uint8_t *scales, hipStream_t stream);
hipError_t launch_mx_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                          const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                          hipStream_t stream);

// MXFP8 (32-element E4M3 blocks with E8M0 scales): quantize on axis 1 or 0,
// and C = A . B^T on the block-scaled FP8 MFMA (K % 128 == 0).
hipError_t launch_mx8_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, uint8_t *codes,
                               uint8_t *scales, hipStream_t stream);
hipError_t launch_mx8_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                           const uint8_t *b_scales, int64_t M, int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc,
                           hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *codes, const uint8_t *scales, const float *meta, int64_t outer,
                             int64_t k, void *y, int y_dtype, hipStream_t stream);

// C[M][ldc] = gA gB * A (M x K) . B^T (N x K); out_dtype 0 = f32, 1 = bf16.
hipError_t launch_gemm(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_meta,
                       const uint8_t *b_codes, const uint8_t *b_scales, const float *b_meta, int64_t M,
                       int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, hipStream_t stream);

// The same product with the tiles left over after whole rounds of the CUs
// cut into K ranges (split tail), where that is faster; split tiles are
// combined in a fixed order through ws.  ws: gemm_split_workspace_bytes()
// bytes, 256-byte aligned, zero-filled before its first use; left
// zero-filled on completion.
int64_t gemm_split_workspace_bytes();
// The library-owned workspace of the current device (set up on the first
// call per device, its flags cleared by a kernel on `stream`), for the
// entry point that allocates nothing; gemm_scratch_bytes() bytes.
int64_t gemm_scratch_bytes();
hipError_t gemm_scratch(hipStream_t stream, void **ptr);
hipError_t launch_gemm_split(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_meta,
                          const uint8_t *b_codes, const uint8_t *b_scales, const float *b_meta, int64_t M,
                          int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, void *ws, hipStream_t stream);

}  // namespace nvfp4
