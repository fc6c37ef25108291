// api.hip -- the extern "C" boundary declared in include/nvfp4.h: argument
// validation (synchronous, before any launch) and kernel launches on the
// caller's stream.  Nothing here allocates or synchronises.
#include "nvfp4.h"
#include "nvfp4_kernels.h"

#include <stdint.h>

namespace {

// Size limits of the launch geometry (each documented in nvfp4.h).
// Quantization down the columns (axis 0) puts 16-row blocks on the grid's
// y dimension (at most 65535): 4 blocks per y step for NVFP4, 8 x 32 rows
// for MXFP4.
constexpr int64_t kMaxRowsAxis0 = 65535LL * 4 * 16;       // 4 194 240
constexpr int64_t kMaxRowsAxis0Mx = 65535LL * 8 * 32;     // 16 776 960
constexpr int64_t kMaxRowsAxis0Mx8 = 65535LL * 4 * 32;    // 8 388 480
// The MXFP8 GEMM addresses 128 operand rows of K code bytes with 32-bit
// buffer offsets below 2^31.
constexpr int64_t kMaxGemmKMx8 = (1LL << 24) - 128;
// The GEMMs address 128 operand rows of K/2 code bytes with 32-bit buffer
// offsets below 2^31, and launch at most INT32_MAX workgroups (tiles of
// 256 x 128 or larger).
constexpr int64_t kMaxGemmK = (1LL << 25) - 16;
// Element counts (rows x cols, outer x k, M x ldc) stay at or below 2^60, so
// every byte offset the kernels form fits in int64.
constexpr int64_t kMaxCount = 1LL << 60;

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline bool count_ok(int64_t a, int64_t b) { return a <= 0 || b <= kMaxCount / a; }

inline bool gemm_shape_ok(int64_t M, int64_t N, int64_t K) {
  if (K > kMaxGemmK) return false;
  // ceil(M/256) * ceil(N/128) <= INT32_MAX, without overflow
  const int64_t tm = M / 256 + (M % 256 != 0), tn = N / 128 + (N % 128 != 0);
  return tn == 0 || tm <= INT32_MAX / tn;
}

inline int hip_status(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

int check_tensor(const nvfp4_tensor *t) {
  if (!t || !t->meta) return NVFP4_ERR_NULL;
  if (t->outer < 0 || t->k < 0 || t->k % 16 != 0 || !count_ok(t->outer, t->k)) return NVFP4_ERR_SHAPE;
  if (t->outer > 0 && t->k > 0 && (!t->codes || !t->scales)) return NVFP4_ERR_NULL;
  if (!aligned(t->codes, 8) || !aligned(t->meta, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// Operands and output of an NVFP4 GEMM (shared by its entry points).
int check_gemm_args(const nvfp4_tensor *a, const nvfp4_tensor *b, const void *c, int c_dtype, int64_t ldc) {
  int st = check_tensor(a);
  if (st != NVFP4_OK) return st;
  st = check_tensor(b);
  if (st != NVFP4_OK) return st;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (a->k != b->k) return NVFP4_ERR_SHAPE;
  const int64_t M = a->outer, N = b->outer;
  if (ldc < N || !count_ok(M, ldc) || !gemm_shape_ok(M, N, a->k)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N > 0 && !c) return NVFP4_ERR_NULL;
  if (!aligned(c, c_dtype == NVFP4_F32 ? 4 : 2)) return NVFP4_ERR_ALIGN;
  // with K % 64 == 0 the kernels move the scale rows by DMA in whole dwords
  if (a->k % 64 == 0 && (!aligned(a->scales, 4) || !aligned(b->scales, 4))) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int quantize_common(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                    uint64_t seed, uint64_t offset, bool rht, uint32_t sign_mask, nvfp4_tensor *out,
                    void *hip_stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_ENUM;
  if (axis != 0 && axis != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  const int64_t outer = axis ? rows : cols;
  const int64_t k = axis ? cols : rows;
  if (k % 16 != 0) return NVFP4_ERR_SHAPE;
  if (out->outer != outer || out->k != k) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows > kMaxRowsAxis0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_ERR_NULL;
  int st = check_tensor(out);
  if (st != NVFP4_OK) return st;
  if (!aligned(x, 16)) return NVFP4_ERR_ALIGN;
  hipError_t e = nvfp4::launch_quantize(x, x_dtype, rows, cols, axis, rounding, seed, offset, rht, sign_mask,
                                        out->codes, out->scales, out->meta, (hipStream_t)hip_stream);
  return hip_status(e);
}

}  // namespace

extern "C" {

int nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding, uint64_t seed,
                   uint64_t offset, nvfp4_tensor *out, void *hip_stream) {
  return quantize_common(x, x_dtype, rows, cols, axis, rounding, seed, offset, false, 0u, out, hip_stream);
}

int nvfp4_rht_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                       uint64_t seed, uint64_t offset, uint16_t sign_mask, nvfp4_tensor *out, void *hip_stream) {
  return quantize_common(x, x_dtype, rows, cols, axis, rounding, seed, offset, true, sign_mask, out, hip_stream);
}

int nvfp4_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rht, uint16_t sign_mask,
               float *amax, void *hip_stream) {
  if (!amax) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (axis != 0 && axis != 1) return NVFP4_ERR_ENUM;
  if (rht != 0 && rht != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if ((axis ? cols : rows) % 16 != 0) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows > kMaxRowsAxis0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_amax(x, x_dtype, rows, cols, axis, rht != 0, sign_mask, amax,
                                       (hipStream_t)hip_stream));
}

int nvfp4_quantize_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rounding,
                        uint64_t seed, uint64_t offset, int rht, uint16_t sign_mask, const float *amax,
                        nvfp4_tensor *out, void *hip_stream) {
  if (!out || !amax) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (rounding != NVFP4_RNE && rounding != NVFP4_SR) return NVFP4_ERR_ENUM;
  if (axis != 0 && axis != 1) return NVFP4_ERR_ENUM;
  if (rht != 0 && rht != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  const int64_t outer = axis ? rows : cols;
  const int64_t k = axis ? cols : rows;
  if (k % 16 != 0) return NVFP4_ERR_SHAPE;
  if (out->outer != outer || out->k != k) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows > kMaxRowsAxis0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_ERR_NULL;
  int st = check_tensor(out);
  if (st != NVFP4_OK) return st;
  if (!aligned(x, 16) || !aligned(amax, 4)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_quantize_amax(x, x_dtype, rows, cols, axis, rounding, seed, offset, rht != 0,
                                                sign_mask, amax, out->codes, out->scales, out->meta,
                                                (hipStream_t)hip_stream));
}

int nvfp4_quantize_dual(const void *x, int x_dtype, int64_t rows, int64_t cols, int rounding1, uint64_t seed1,
                        uint64_t offset1, nvfp4_tensor *out1, int rht0, uint16_t sign_mask0, int rounding0,
                        uint64_t seed0, uint64_t offset0, nvfp4_tensor *out0, void *hip_stream) {
  if (!out1 || !out0) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if ((rounding1 != NVFP4_RNE && rounding1 != NVFP4_SR) || (rounding0 != NVFP4_RNE && rounding0 != NVFP4_SR))
    return NVFP4_ERR_ENUM;
  if (rht0 != 0 && rht0 != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || rows % 16 != 0 || cols % 16 != 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  if (out1->outer != rows || out1->k != cols || out0->outer != cols || out0->k != rows) return NVFP4_ERR_SHAPE;
  if (rows > kMaxRowsAxis0) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && !x) return NVFP4_ERR_NULL;
  int st = check_tensor(out1);
  if (st != NVFP4_OK) return st;
  st = check_tensor(out0);
  if (st != NVFP4_OK) return st;
  // each meta is two floats that the kernels write while other workgroups
  // read them: the two 8-byte ranges must not overlap
  if (out1->meta + 2 > out0->meta && out0->meta + 2 > out1->meta) return NVFP4_ERR_SHAPE;
  if (!aligned(x, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_quantize_dual(x, x_dtype, rows, cols, rounding1, seed1, offset1, out1->codes,
                                                out1->scales, out1->meta, rht0 != 0, sign_mask0, rounding0, seed0,
                                                offset0, out0->codes, out0->scales, out0->meta,
                                                (hipStream_t)hip_stream));
}

int mxfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, mxfp4_tensor *out,
                   void *hip_stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (axis != 0 && axis != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  const int64_t outer = axis ? rows : cols, k = axis ? cols : rows;
  if (k % 32 != 0 || out->outer != outer || out->k != k) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows > kMaxRowsAxis0Mx) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (!x || !out->codes || !out->scales)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out->codes, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_mx_quantize(x, x_dtype, rows, cols, axis, out->codes, out->scales,
                                              (hipStream_t)hip_stream));
}

int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, void *c, int c_dtype, int64_t ldc, void *hip_stream) {
  if (!a || !b) return NVFP4_ERR_NULL;
  if (a->outer < 0 || b->outer < 0 || a->k < 0 || a->k != b->k || a->k % 256 != 0) return NVFP4_ERR_SHAPE;
  if (!count_ok(a->outer, a->k) || !count_ok(b->outer, b->k)) return NVFP4_ERR_SHAPE;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  const int64_t M = a->outer, N = b->outer;
  if (ldc < N || !count_ok(M, ldc) || !gemm_shape_ok(M, N, a->k)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N > 0 && (!c || (a->k > 0 && (!a->codes || !a->scales || !b->codes || !b->scales))))
    return NVFP4_ERR_NULL;
  if (!aligned(c, c_dtype == NVFP4_F32 ? 4 : 2)) return NVFP4_ERR_ALIGN;
  // the kernel moves codes in 16-byte and scales in 4-byte pieces by DMA
  if (!aligned(a->codes, 16) || !aligned(b->codes, 16) || !aligned(a->scales, 4) || !aligned(b->scales, 4))
    return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_mx_gemm(a->codes, a->scales, b->codes, b->scales, M, N, a->k, c, c_dtype, ldc,
                                          (hipStream_t)hip_stream));
}

int mxfp8_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, mxfp8_tensor *out,
                   void *hip_stream) {
  if (!out) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_F32 && x_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (axis != 0 && axis != 1) return NVFP4_ERR_ENUM;
  if (rows < 0 || cols < 0 || !count_ok(rows, cols)) return NVFP4_ERR_SHAPE;
  const int64_t outer = axis ? rows : cols, k = axis ? cols : rows;
  if (k % 32 != 0 || out->outer != outer || out->k != k) return NVFP4_ERR_SHAPE;
  if (axis == 0 && rows > kMaxRowsAxis0Mx8) return NVFP4_ERR_SHAPE;
  if (rows > 0 && cols > 0 && (!x || !out->codes || !out->scales)) return NVFP4_ERR_NULL;
  if (!aligned(x, 16) || !aligned(out->codes, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_mx8_quantize(x, x_dtype, rows, cols, axis, out->codes, out->scales,
                                               (hipStream_t)hip_stream));
}

int mxfp8_gemm(const mxfp8_tensor *a, const mxfp8_tensor *b, void *c, int c_dtype, int64_t ldc, void *hip_stream) {
  if (!a || !b) return NVFP4_ERR_NULL;
  if (a->outer < 0 || b->outer < 0 || a->k < 0 || a->k != b->k || a->k % 128 != 0) return NVFP4_ERR_SHAPE;
  if (a->k > kMaxGemmKMx8 || !count_ok(a->outer, a->k) || !count_ok(b->outer, b->k)) return NVFP4_ERR_SHAPE;
  if (c_dtype != NVFP4_F32 && c_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  const int64_t M = a->outer, N = b->outer;
  if (ldc < N || !count_ok(M, ldc) || !gemm_shape_ok(M, N, 0)) return NVFP4_ERR_SHAPE;
  if (M > 0 && N > 0 && (!c || (a->k > 0 && (!a->codes || !a->scales || !b->codes || !b->scales))))
    return NVFP4_ERR_NULL;
  if (!aligned(c, c_dtype == NVFP4_F32 ? 4 : 2)) return NVFP4_ERR_ALIGN;
  // the kernel moves codes in 16-byte and scales in 4-byte pieces by DMA
  if (!aligned(a->codes, 16) || !aligned(b->codes, 16) || !aligned(a->scales, 4) || !aligned(b->scales, 4))
    return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_mx8_gemm(a->codes, a->scales, b->codes, b->scales, M, N, a->k, c, c_dtype, ldc,
                                           (hipStream_t)hip_stream));
}

int nvfp4_dequantize(const nvfp4_tensor *q, void *y, int y_dtype, void *hip_stream) {
  int st = check_tensor(q);
  if (st != NVFP4_OK) return st;
  if (y_dtype != NVFP4_F32 && y_dtype != NVFP4_BF16) return NVFP4_ERR_ENUM;
  if (q->outer > 0 && q->k > 0 && !y) return NVFP4_ERR_NULL;
  if (!aligned(y, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_dequantize(q->codes, q->scales, q->meta, q->outer, q->k, y, y_dtype,
                                              (hipStream_t)hip_stream));
}

int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype, int64_t ldc, void *hip_stream) {
  int st = check_gemm_args(a, b, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  return hip_status(nvfp4::launch_gemm(a->codes, a->scales, a->meta, b->codes, b->scales, b->meta, a->outer, b->outer, a->k, c,
                                       c_dtype, ldc, (hipStream_t)hip_stream));
}

int nvfp4_gemm_ws(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype, int64_t ldc, void *workspace,
                  int64_t workspace_bytes, void *hip_stream) {
  int st = check_gemm_args(a, b, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  if (!workspace) return NVFP4_ERR_NULL;
  if (workspace_bytes < nvfp4::gemm_split_workspace_bytes()) return NVFP4_ERR_SHAPE;
  if (!aligned(workspace, 256)) return NVFP4_ERR_ALIGN;
  return hip_status(nvfp4::launch_gemm_split(a->codes, a->scales, a->meta, b->codes, b->scales, b->meta, a->outer,
                                          b->outer, a->k, c, c_dtype, ldc, workspace, (hipStream_t)hip_stream));
}

int64_t nvfp4_gemm_workspace_bytes(void) { return nvfp4::gemm_split_workspace_bytes(); }

int nvfp4_gemm_noalloc(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype, int64_t ldc,
                       void *hip_stream) {
  int st = check_gemm_args(a, b, c, c_dtype, ldc);
  if (st != NVFP4_OK) return st;
  // the split launcher needs at most gemm_split_workspace_bytes() for any
  // shape; beyond the library's array the call is refused
  if (nvfp4::gemm_split_workspace_bytes() > nvfp4::gemm_scratch_bytes()) return NVFP4_ERR_SHAPE;
  void *ws = nullptr;
  hipError_t e = nvfp4::gemm_scratch((hipStream_t)hip_stream, &ws);
  if (e != hipSuccess) return NVFP4_ERR_HIP;
  return hip_status(nvfp4::launch_gemm_split(a->codes, a->scales, a->meta, b->codes, b->scales, b->meta, a->outer,
                                             b->outer, a->k, c, c_dtype, ldc, ws, (hipStream_t)hip_stream));
}

const char *nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "null pointer";
    case NVFP4_ERR_SHAPE: return "invalid shape";
    case NVFP4_ERR_ENUM: return "invalid enum value";
    case NVFP4_ERR_HIP: return "HIP launch failed";
    case NVFP4_ERR_ALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

}  // extern "C"
