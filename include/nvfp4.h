/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 linear-layer library.
 *
 * The library implements the 4-bit linear-layer path of NVIDIA's NVFP4
 * pretraining recipe as described on these pages:
 *   [P1] hyper.ai, "NVIDIA revolutioniert KI-Praetrainingsgeschwindigkeit mit
 *        4-Bit-Genauigkeit" (body: 4-bit pretraining with dynamic scaling on
 *        accelerated GEMMs).
 *   [P3] aibuzzwire.news, Thinking Machines "End-to-End 4-Bit Training"
 *        article; sections "Warum weniger Bits ein schnelleres Training
 *        bedeuten" (rounding to the nearest representable value) and
 *        "Unterschiedliche Phasen, unterschiedliche Regeln" (backward passes
 *        are sensitive to rounding bias).
 *   [P4] aisight.pl, "Koniec marnowania mocy. NVIDIA udowadnia, ze 4 bity
 *        wystarcza do trenowania gigantow"; sections "Architektura NVFP4
 *        kontra ograniczenia mikroskalowania" (16-element blocks, E4M3 block
 *        scale, extra FP32 per-tensor scale) and "Technologie stabilizujace
 *        proces treningowy" (random Hadamard transforms on weight gradients,
 *        stochastic rounding).
 *
 * Conventions shared by every entry point
 *  - Pointers named x, y, c and every pointer inside nvfp4_tensor are DEVICE
 *    pointers owned by the caller; the library never allocates, frees or
 *    retains them.  nvfp4_tensor structs themselves are HOST memory.
 *  - hip_stream is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it; calls return without synchronising.
 *  - Argument errors are reported synchronously, before anything is
 *    launched.  NVFP4_ERR_HIP reports a failed launch.
 *  - Sizes are int64_t and may be 0 (empty tensors are valid, see below).
 *    Limits of the launch geometry (NVFP4_ERR_SHAPE beyond them):
 *    quantization down the columns (axis 0, and the dual call) takes
 *    rows <= 4 194 240 (MXFP4: 16 776 960, MXFP8: 8 388 480); the NVFP4
 *    GEMMs take K <= 2^25 - 16 (MXFP8: K <= 2^24 - 128)
 *    and ceil(M/256) * ceil(N/128) <= INT32_MAX; every element count
 *    (rows * cols, outer * k, M * ldc) is at most 2^60.
 *  - Element types: NVFP4_F32 (binary32) or NVFP4_BF16 (bfloat16).
 *  - Thread safety: stateless; concurrent calls on different outputs are
 *    fine.  The calls keep no scratch memory between launches (the one
 *    workspace, of nvfp4_gemm_ws, belongs to the caller).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = -1,   /* a required pointer is NULL                      */
    NVFP4_ERR_SHAPE = -2,  /* negative size, K % 16 != 0, mismatched shapes,
                              size beyond a documented limit                */
    NVFP4_ERR_ENUM = -3,   /* unknown dtype / rounding / axis value           */
    NVFP4_ERR_HIP = -4,    /* a HIP launch failed                             */
    NVFP4_ERR_ALIGN = -5   /* a pointer or leading dimension is misaligned    */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1 } nvfp4_dtype;
typedef enum { NVFP4_RNE = 0, NVFP4_SR = 1 } nvfp4_rounding;

/*
 * An NVFP4 tensor in its quantized layout [outer][k], k being the GEMM
 * reduction length ([P4] "Architektura NVFP4 ..."):
 *  codes  : u8 [outer][k/2]; element 2j of a row in the low nibble of byte j,
 *           element 2j+1 in the high nibble.  A nibble is an E2M1 code:
 *           bit 3 sign, bits 0-2 the magnitude 0, .5, 1, 1.5, 2, 3, 4, 6.
 *           8-byte aligned.
 *  scales : u8 [outer][k/16]; the OCP E4M3FN block scale of each 16-element
 *           block along k (never NaN, at most 448).  4-byte aligned when k %
 *           64 == 0 and the tensor is a GEMM operand (whole scale dwords move
 *           by DMA then); any alignment otherwise.
 *  meta   : f32 [2]; meta[0] = amax (the tensor maximum magnitude after the
 *           optional transform), meta[1] = g = amax / 2688, the FP32 decode
 *           scale.  4-byte aligned.
 *  outer, k : k % 16 == 0.
 * The value of element (o, kk) is e2m1(code) * e4m3(scale) * g.
 */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    float *meta;
    int64_t outer;
    int64_t k;
} nvfp4_tensor;

/*
 * nvfp4_quantize -- quantize a row-major [rows][cols] matrix x to NVFP4
 * ([P4] "Architektura NVFP4 ..." for the format; [P3] "Warum weniger Bits
 * ..." for nearest rounding; [P4] "Technologie stabilizujace ..." for
 * stochastic rounding).
 *
 *  x        : device, x_dtype elements, row-major [rows][cols], 16-byte aligned.
 *  axis     : 1 -> outer = rows, k = cols (blocks run along rows of x);
 *             0 -> outer = cols, k = rows (blocks run down the columns of x;
 *             the output is the transpose, as needed for the K-major operand
 *             of a GEMM whose reduction runs over the rows of x).
 *  rounding : NVFP4_RNE (nearest, ties to the even code, saturate at 6) or
 *             NVFP4_SR (stochastic: with frac the position of |v| between
 *             its two neighbouring grid values, round up iff
 *             frac + (r16 + 1/2) / 2^16 >= 1, r16 being the 16 bits
 *             Philox4x32-10 assigns to the element; saturate at 6).
 *  seed, offset : Philox key = (lo32(seed), hi32(seed)); for the element with
 *             output index i = o*k + kk the counter is (lo32(i/8), hi32(i/8),
 *             lo32(offset), hi32(offset)) and r16 is half (i%2, low first) of
 *             output word (i%8)/2.  Ignored for NVFP4_RNE.
 *  out      : host struct; out->codes/scales/meta must point to buffers of
 *             the sizes above and out->outer, out->k must equal the view's.
 * Steps: amax over the whole tensor; s_enc = 2688/amax, per block
 * S = E4M3_rne_sat(blockmax * (448/amax)); element code of x * (s_enc / S).
 * amax == 0 gives all-zero scales and codes of +-0.  Non-finite input: meta[0]
 * becomes Inf/NaN and the codes and scales are unspecified.  An empty tensor
 * (outer == 0) writes meta = {0, 0} only.  Enqueues three kernels.
 */
int nvfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis,
                   int rounding, uint64_t seed, uint64_t offset, nvfp4_tensor *out,
                   void *hip_stream);

/*
 * nvfp4_rht_quantize -- as nvfp4_quantize, but each 16-element chunk along k
 * is first replaced by (1/4) H16 diag(s) chunk, the 16-point random Hadamard
 * transform ([P4] "Technologie stabilizujace ...": it spreads the outliers
 * of the weight gradients).  H16 is the Sylvester Hadamard matrix
 * H[i][j] = (-1)^popcount(i & j) and s_j = -1 where bit j of sign_mask is
 * set.  The butterfly runs in binary32 with stages 1, 2, 4, 8 (lower index
 * a+b, upper a-b).  amax and block maxima are those of the transformed
 * values.  Both operands of a weight-gradient GEMM must use the same
 * sign_mask along their shared reduction dimension; the transform then
 * cancels in the product.
 */
int nvfp4_rht_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis,
                       int rounding, uint64_t seed, uint64_t offset, uint16_t sign_mask,
                       nvfp4_tensor *out, void *hip_stream);

/*
 * nvfp4_amax -- the first pass of a quantization alone: *amax = the tensor
 * amax of x viewed on `axis` (after the 16-point transform along k when
 * rht == 1, with sign_mask as in nvfp4_rht_quantize), the maximum of |value|
 * taken on IEEE bit patterns (exact; NaN > Inf > finite).  0 for an empty
 * tensor.  amax: device, one f32, 4-byte aligned.  Enqueues two kernels.
 *
 * nvfp4_quantize_amax -- the second pass alone: as nvfp4_quantize (rht == 0)
 * or nvfp4_rht_quantize (rht == 1) with the tensor amax read from device
 * memory instead of computed, which saves the first read of x when the
 * producer of x already knows its maximum ([P4] "Architektura NVFP4 ...":
 * the FP32 tensor-level scale).  out->meta becomes {*amax, *amax / 2688}.
 * *amax must be finite and >= 0 (not checked): with the true maximum the
 * result equals nvfp4_quantize's bit for bit; a smaller value saturates
 * (block scales at 448, codes at 6), so the decoded values are clipped to
 * +-*amax.  Non-finite input values leave the codes and scales unspecified,
 * as in nvfp4_quantize.  Enqueues two kernels.
 */
int nvfp4_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis, int rht,
               uint16_t sign_mask, float *amax, void *hip_stream);
int nvfp4_quantize_amax(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis,
                        int rounding, uint64_t seed, uint64_t offset, int rht,
                        uint16_t sign_mask, const float *amax, nvfp4_tensor *out,
                        void *hip_stream);

/*
 * nvfp4_quantize_dual -- both layouts of one input with one amax read.  A
 * training step needs each of its tensors quantized along both of its
 * dimensions: dY along its columns for the data gradient and along its rows
 * for the weight gradient ([P4] "Technologie stabilizujace ...": stochastic
 * rounding of the gradients, the Hadamard transform for the weight
 * gradients).  Equivalent, bit for bit, to
 *   nvfp4_quantize(x, x_dtype, rows, cols, 1, rounding1, seed1, offset1, out1)
 * followed by nvfp4_quantize (rht0 == 0) or nvfp4_rht_quantize (rht0 == 1)
 * of x with axis 0, rounding0, seed0, offset0, sign_mask0 into out0, but
 * each of the two passes reads x once for both layouts: the amax pass takes
 * both maxima (the plain one, and the one after the column transform), the
 * encode pass writes both outputs from one tile of x staged in LDS.
 *  rows % 16 == 0 and cols % 16 == 0 (both layouts need whole blocks);
 *  out1: outer = rows, k = cols; out0: outer = cols, k = rows; the two meta
 *  pairs (8 bytes each) must not overlap (NVFP4_ERR_SHAPE otherwise) and the
 *  outputs must not overlap each other or x.  Enqueues three kernels.
 */
int nvfp4_quantize_dual(const void *x, int x_dtype, int64_t rows, int64_t cols,
                        int rounding1, uint64_t seed1, uint64_t offset1, nvfp4_tensor *out1,
                        int rht0, uint16_t sign_mask0, int rounding0, uint64_t seed0,
                        uint64_t offset0, nvfp4_tensor *out0, void *hip_stream);

/*
 * nvfp4_dequantize -- y[o][kk] = (e2m1(code) * e4m3(scale)) * g in binary32
 * (the first product is exact, the second rounds once); bf16 output is the
 * nearest-even rounding of that value.  y: device [q->outer][q->k] row-major
 * in the QUANTIZED layout (an axis-0 tensor comes back transposed), 16-byte
 * aligned.  Defines the values the GEMM multiplies ([P3] "Warum weniger Bits
 * ..." measures quantization error against these decoded values).
 */
int nvfp4_dequantize(const nvfp4_tensor *q, void *y, int y_dtype, void *hip_stream);

/*
 * nvfp4_gemm -- the block-scaled NVFP4 GEMM with FP32 accumulation
 * ([P1] body: accelerated 4-bit GEMMs; [P4] "Architektura NVFP4 ...").
 *
 *   C[m][n] = g_A * g_B * sum_k (qA*SA)[m][k] * (qB*SB)[n][k]
 *
 *  a : M x K NVFP4 tensor (a->outer = M), b : N x K (b->outer = N), a->k ==
 *      b->k.  Both operands are K-contiguous ("TN"): fprop Y = X W^T takes
 *      a = X (axis 1), b = W (axis 1); dgrad dX = dY W takes a = dY (axis 1),
 *      b = W quantized on axis 0; wgrad dW = X^T dY takes a = X (axis 0) and
 *      b = dY (axis 0).
 *  c : device, row-major [M][ldc], c_dtype NVFP4_F32 or NVFP4_BF16 (nearest
 *      even of the f32 result), ldc >= N, 4-byte aligned (f32) / 2-byte (bf16).
 * Accuracy: every decoded element q*S is exact in f16 and every product of
 * two is exact in f32.  Each MFMA adds one K step of 16 products -- 8 from
 * each of two different 16-blocks, with different block scales -- into the
 * f32 accumulator, so an output element goes through at least K/16 binary32
 * roundings and the worst-case error is of order
 * (K/16) * 2^-24 * g_A g_B sum_k |(qA SA)(qB SB)|: that guarantees the
 * 1e-5 * sum|ab| tolerance only up to K of about 2700.  Beyond, the
 * tolerance rests on successive rounding errors having independent signs
 * (error ~ sqrt(K/16) * 2^-24 * sum|ab|).  Measured worst |err| / sum|ab|:
 * zero-mean operands at the layer shapes (K = 5120 .. 20480) below 1e-6;
 * non-negative operands (the case where every partial sum grows) 2.5e-6 at
 * K = 20480, 6.9e-6 at K = 131072, and above the tolerance from K = 262144
 * (1.04e-5; 1.9e-4 at K = 2^25 - 256).  So for same-sign operands this call
 * meets 1e-5 for K <= 131072; nvfp4_gemm_ws splits long reductions of small
 * outputs (3.5e-7 at K = 2^25 - 256).
 * Deterministic: one kernel, no atomics, fixed summation order.  M == 0 or
 * N == 0: nothing is written; K == 0: C is set to zero.
 */
int nvfp4_gemm(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype,
               int64_t ldc, void *hip_stream);

/*
 * nvfp4_gemm_ws -- nvfp4_gemm with a caller-owned workspace, which lets it
 * balance the last, partly filled round of the CUs by splitting tiles along
 * K.  The data-parallel grid runs whole 256 x 256 output tiles, so when the
 * tile count is not a multiple of the CU count the last round leaves CUs
 * idle.  Two schedules use the workspace:
 *  - stream-K tail (at least one round of tiles, not a whole number of
 *    rounds, at least 4096 K positions per tile): all whole rounds but the
 *    last run data-parallel; the remaining tiles' K groups are dealt out in
 *    equal contiguous ranges to one round of workgroups, eight chunks (one
 *    per XCD) of whole tiles.  A tile is then the sum of at most two
 *    ranges: the workgroup holding its end adds the f32 partial of the one
 *    holding its start (kept in the workspace).
 *  - split tail (fewer tiles than one round): whole rounds run as before and
 *    each remaining tile is cut into up to CUs / tiles-left-over K ranges;
 *    the workgroup of the last range adds the others' partials.  Taken when
 *    fewer than half the CUs would get a tile or the ranges stay long (at
 *    least 4096 K positions).
 * Otherwise the call runs nvfp4_gemm's grid.  Partials add in a fixed order
 * -- deterministic for a given device, no atomics on the data.  Same
 * operands, output and accuracy contract as nvfp4_gemm; a split shortens
 * each f32 accumulation chain (the partials then add in binary32), which
 * keeps same-sign operands inside the tolerance at any K when the output
 * has few tiles.
 *  workspace       : device, at least nvfp4_gemm_workspace_bytes() bytes,
 *                    256-byte aligned, zero-filled before its FIRST use (the
 *                    kernel leaves it zero-filled again when it completes,
 *                    so it can be reused without clearing).  Calls that use
 *                    one workspace must not overlap in time (same stream,
 *                    or ordered by events).
 *  workspace_bytes : its size (NVFP4_ERR_SHAPE if smaller).
 * Errors as nvfp4_gemm, plus NVFP4_ERR_NULL for a NULL workspace and
 * NVFP4_ERR_ALIGN for a misaligned one.  Enqueues one kernel.
 */
int nvfp4_gemm_ws(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype,
                  int64_t ldc, void *workspace, int64_t workspace_bytes, void *hip_stream);

/*
 * nvfp4_gemm_noalloc -- nvfp4_gemm_ws with the library's own workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  It allocates
 * nothing: the workspace is a file-scope device array of
 * nvfp4_gemm_workspace_bytes() bytes (64 MiB + 64 KiB), one per GPU the
 * library runs on, held until the process ends; its address is looked up
 * and its flags cleared (by a kernel on hip_stream) on the first call on
 * each device.  Same arguments, results and errors as nvfp4_gemm_ws without
 * the workspace; the output is bit-identical to nvfp4_gemm_ws's.  Every
 * call on one GPU shares that array, so calls that overlap in time on one
 * GPU race (use one stream, or order them); it keeps the last call's
 * partials.  Enqueues one kernel (two on the first call on a device).
 */
int nvfp4_gemm_noalloc(const nvfp4_tensor *a, const nvfp4_tensor *b, void *c, int c_dtype,
                       int64_t ldc, void *hip_stream);

/* Workspace bytes nvfp4_gemm_ws needs (the same for every shape: 64 KiB of
 * flags plus one 256 KiB partial per persistent workgroup, at most 256). */
int64_t nvfp4_gemm_workspace_bytes(void);

/*
 * MXFP4 -- the microscaling format the pages set NVFP4 against ([P4]
 * "Architektura NVFP4 kontra ograniczenia mikroskalowania": 32-element
 * blocks sharing a power-of-two scale; no tensor-level scale).
 *  codes  : u8 [outer][k/2], E2M1 codes two per byte (element 2j low
 *           nibble), 16-byte aligned.
 *  scales : u8 [outer][k/32], E8M0 exponents: the block scale is
 *           2^(code - 127).  4-byte aligned for a GEMM operand.
 *  outer, k : k % 32 == 0.
 * The value of element (o, kk) is e2m1(code) * 2^(scale - 127).
 */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    int64_t outer;
    int64_t k;
} mxfp4_tensor;

/*
 * mxfp4_quantize -- x (row-major [rows][cols], x_dtype, 16-byte aligned)
 * viewed on `axis` as in nvfp4_quantize.  Per 32-block along k: the scale is
 * the smallest power of two 2^e with blockmax / 2^e <= 6 (e clamped to
 * [-127, 127]; an all-zero block takes e = -127), so the block maximum is
 * never clipped; each element is the nearest-even E2M1 code of x / 2^e.
 * Enqueues one kernel.
 */
int mxfp4_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis,
                   mxfp4_tensor *out, void *hip_stream);

/*
 * mxfp4_gemm -- C[m][n] = sum_k (qA * 2^eA)[m][k] * (qB * 2^eB)[n][k] with
 * FP32 accumulation on gfx950's block-scaled FP4 MFMA (the codes are not
 * decoded).  a: M x K, b: N x K, both K-contiguous; K % 256 == 0
 * (NVFP4_ERR_SHAPE otherwise).  c: row-major [M][ldc], f32 or bf16 (nearest
 * even).  Accuracy as nvfp4_gemm: within 1e-5 * sum_k |a b|.  Deterministic.
 */
int mxfp4_gemm(const mxfp4_tensor *a, const mxfp4_tensor *b, void *c, int c_dtype,
               int64_t ldc, void *hip_stream);

/*
 * MXFP8 -- the 8-bit microscaling format, one of the three number formats
 * of a training run in [P3] "Drei Formate, ein Trainingslauf" (the one
 * quoted at about 5 PFLOPS on GB300), with the 32-element power-of-two
 * blocks of [P4] "Architektura NVFP4 kontra ograniczenia mikroskalowania".
 *  codes  : u8 [outer][k], OCP E4M3FN bytes (bias 7, max 448), 16-byte
 *           aligned.
 *  scales : u8 [outer][k/32], E8M0 exponents: the block scale is
 *           2^(code - 127).  4-byte aligned for a GEMM operand.
 *  outer, k : k % 32 == 0.
 * The value of element (o, kk) is e4m3(code) * 2^(scale - 127).
 */
typedef struct {
    uint8_t *codes;
    uint8_t *scales;
    int64_t outer;
    int64_t k;
} mxfp8_tensor;

/*
 * mxfp8_quantize -- x (row-major [rows][cols], x_dtype, 16-byte aligned)
 * viewed on `axis` as in nvfp4_quantize.  Per 32-block along k: the scale is
 * the smallest power of two 2^e with blockmax / 2^e <= 448 (e clamped to
 * [-127, 127]; an all-zero block takes e = -127), so the block maximum is
 * never clipped; each element is the nearest-even E4M3 code of x / 2^e with
 * the sign of x (-0.0 gives 0x80).  Axis 0 takes rows <= 8 388 480.
 * Enqueues one kernel.
 */
int mxfp8_quantize(const void *x, int x_dtype, int64_t rows, int64_t cols, int axis,
                   mxfp8_tensor *out, void *hip_stream);

/*
 * mxfp8_gemm -- C[m][n] = sum_k (qA * 2^eA)[m][k] * (qB * 2^eB)[n][k] with
 * FP32 accumulation on gfx950's block-scaled FP8 MFMA (the codes are not
 * decoded).  a: M x K, b: N x K, both K-contiguous; K % 128 == 0 and
 * K <= 2^24 - 128 (NVFP4_ERR_SHAPE otherwise).  c: row-major [M][ldc], f32
 * or bf16 (nearest even).  Accuracy: the instruction sums its 64 products
 * per step in groups of 8 consecutive K positions and truncates each
 * product toward zero to 13 bits below the group's largest exponent sum
 * (measured on MI355X), so an element can lose up to
 * sum over groups of sum_k min(|a_k b_k|, 2^(E_group - 13)) on top of the
 * binary32 accumulation of about K/64 steps; every element lies within
 * that bound plus 1e-5 * sum_k |a b| of the exact value.  Deterministic.
 */
int mxfp8_gemm(const mxfp8_tensor *a, const mxfp8_tensor *b, void *c, int c_dtype,
               int64_t ldc, void *hip_stream);

/*
 * nvfp4_probe_mfma -- measurement helper, not part of the method: launches
 * 1024 workgroups of 256 threads that run `iters` x 32 v_mfma_f32_32x32x16_f16
 * per wave (one wave per SIMD, sixteen accumulators) on operands with the
 * values the NVFP4 GEMM multiplies (E2M1 codes times E4M3 block scales), with
 * no memory traffic, giving the ceiling of that MFMA on that data.  Work:
 * 1024 * 4 * iters * 32 * 32768 flop.  out: device, 1024 * 256 floats (the
 * per-thread sums, which keep the work live).
 */
int nvfp4_probe_mfma(int64_t iters, float *out, void *hip_stream);

/*
 * nvfp4_probe_philox -- measurement helper, not part of the method: runs the
 * stochastic-rounding random generator alone (Philox4x32-10, the same
 * routine the encodes use, counters 0 .. calls-1, one call per 8 elements)
 * with no memory traffic, over 4096 workgroups of 256 threads, giving the
 * floor the RNG contract puts under a stochastic-rounding encode of
 * 8 * calls elements.  out: device, 4096 * 256 words (per-thread XOR of the
 * outputs, which keeps the work live).
 */
int nvfp4_probe_philox(int64_t calls, uint32_t *out, void *hip_stream);

/* Human-readable name of a status code (static string). */
const char *nvfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
