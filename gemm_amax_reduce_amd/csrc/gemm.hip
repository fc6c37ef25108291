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
// Design for CDNA4.  gfx950's block-scaled MFMA forms take one power-of-two
// (E8M0) scale per 32 elements, which cannot represent an E4M3 scale per 16
// elements, so every element is decoded exactly: the hardware FP4->F16
// conversion gives q and one packed f16 multiply by the block scale gives
// q*S.  q*S has at most 6 significant bits and lies in [2^-10, 2688], so it
// is exact in f16 and every product of two is exact in f32.  One MFMA sums a
// K step of 16 products taken from two different 16-blocks (8 positions of
// each, see the K order below) into the f32 accumulator, so the rounding is
// that of about K/16 binary32 accumulations.
//
// Data movement.  A 256-thread workgroup computes a 256 x BN tile of C (BN =
// 256, or 128 for the column remainder) with four waves of 128 x BN/2.  K is
// consumed in groups of 256 (four 64-wide stages).  For each group the
// workgroup copies the packed codes of its 256 + BN operand rows -- one full
// 128-byte line per row -- and their 16 scale bytes into LDS with the
// buffer-load-to-LDS (DMA) form, double-buffered, so one load instruction
// covers 8 rows with whole lines.  (Loading per lane in MFMA operand order,
// lane l its own row, touches 32 lines per instruction; that line traffic
// measured costlier than the whole decode.)  Each wave then reads only its
// own operand rows from LDS (16 bytes = 32 codes per row and stage), decodes
// them per K step into MFMA operand registers, and interleaves that decode
// with the MFMAs of the previous K step.  Nothing decoded goes back to LDS,
// so LDS carries about 100 KB per 4-stage group instead of 768 KB when
// decoded operands are shared through it (LDS writes run at ~70 B/clk/CU).
//
// LDS image of a group: row R's 128 code bytes at R*128, its 16-byte chunk c
// (32 K positions) in slot c ^ (R & 7), so the rows read by one ds_read_b128
// fall on distinct banks; row R's 16 scale bytes at kCodeBytes + R*16.  A
// rows are LDS rows 0..255, B rows 256.. .
//
// K order inside an MFMA operand: lane l (row l%32, half h = l/32) of stage
// s' (0..3) of a group takes chunk 2s'+h, and K step ks its positions
// 8ks..8ks+7 -- the same for A and B, which is all the MFMA's sum over K
// requires.
//
// Grid: one workgroup per tile.  The launcher covers most columns with
// 256 x 256 tiles and the remainder with 256 x 128 tiles in the same launch,
// so the tile count fills whole rounds of the CUs.  Workgroups are dealt
// round-robin to the eight XCDs (pid % 8); the tile index is remapped so each
// XCD works on a contiguous range of tiles, ordered in groups of 8 tile rows,
// so the tiles resident on one XCD share A rows and B columns in its L2.
#include "gemm_common.h"
#include "nvfp4_device.h"
#include "nvfp4_kernels.h"

#include <atomic>
#include <type_traits>

namespace nvfp4 {

namespace {

constexpr int BM = 256;
constexpr int kThreads = 256;
constexpr int kGroupK = 256;                        // K positions per LDS group (4 stages)
constexpr int kRowsMax = BM + 256;                  // operand rows of the widest tile
constexpr int kCodeBytes = kRowsMax * 128;          // 64 KB of codes per group buffer
constexpr int kGroupBytes = kCodeBytes + kRowsMax * 16;
constexpr int kGroupM = 8;                          // tile rows per L2 group

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The f32 accumulators of one 256 x BN tile: wave (wm, wn) holds rows
// 128wm + 32i and columns (BN/2)wn + 32j of MFMA block [i][j].
template <int BN> using TileAcc = float16_t[4][BN / 64];

// acc = the unscaled sum over K groups [g0, g1) of the 256 x BN tile of
// C[M][N] = A.B^T at rows m0.., columns n0.. (B, N already restricted to
// this tile width's column range).  g1 > g0.  Every DMA this issues has
// completed when it returns, so the LDS buffers are free again once all
// waves are past a barrier.  With `flag` set, thread 0 stores 1 to it
// once the prologue's wait has seen every earlier memory access of the
// workgroup complete (the stores of a partial issued before the call).
template <bool SCALE_DMA, int BN>
__device__ __forceinline__ void tile_accumulate(uint8_t *smem, int64_t m0, int64_t n0, int g0, int g1,
                                                const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA,
                                                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                                                int64_t M, int64_t N, int64_t K, TileAcc<BN> &acc,
                                                unsigned *flag = nullptr) {
  constexpr int NB = BN / 64;          // B fragments (32 columns each) per wave
  constexpr int NF = 4 + NB;           // operand fragments decoded per wave and K step
  constexpr int NU = 4 * NB;           // MFMAs per wave and K step
  constexpr int kRowsB = BN / 2;       // B rows copied by each of waves 2 and 3
  static_assert(BN == 256 || BN == 128, "tile width");

  // The wave index is uniform across a wave; readfirstlane tells the
  // compiler so, which keeps every per-wave choice in scalar registers.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, h = lane >> 5;

  // ---- DMA side: waves 0 and 1 copy A rows 128w .. 128w+127, waves 2 and
  // 3 B rows kRowsB(w-2) ..; a view holds only rows inside the operand, so
  // rows past M or N read as zeros.
  const uint32_t rb = (uint32_t)(K / 2), rs = (uint32_t)(K / 16);
  const bool dma_b = wave >= 2;
  const int64_t drow0 = dma_b ? n0 + (int64_t)kRowsB * (wave - 2) : m0 + 128 * (int64_t)wave;
  const int64_t dlimit = dma_b ? N : M;
  const int64_t dbase = min<int64_t>(drow0, dlimit);
  const uint32_t dvalid = (uint32_t)min<int64_t>(dma_b ? kRowsB : 128, dlimit - dbase);
  const __amdgpu_buffer_rsrc_t dcodes = make_rsrc((dma_b ? B : A) + dbase * rb, dvalid * rb);
  const __amdgpu_buffer_rsrc_t dscales = make_rsrc((dma_b ? SB : SA) + dbase * rs, dvalid * rs);
  const int lds_row0 = dma_b ? BM + kRowsB * (wave - 2) : 128 * wave;
  // A 256 x 128 tile has 384 operand rows: its B waves copy 64 rows each and
  // send the rest of their 16 + 2 instructions, out of range (no memory
  // access), to the unused LDS rows 384..511, which keeps the instruction
  // stream the same for every wave (no branch in the main loop).
  const int spare_row0 = BM + 128 + 64 * (wave - 2);
  // code DMA instruction: 8 rows, lane l -> row l>>3, LDS slot l&7, which
  // holds the row's chunk (l&7) ^ (row&7)
  const uint32_t dv_code = (uint32_t)(lane >> 3) * rb + 16u * (uint32_t)((lane & 7) ^ (lane >> 3));
  const uint32_t dv_scale = (uint32_t)lane * rs;     // scale DMA: 64 rows, lane l -> row l
  // Part `part` of the DMA of group g into LDS buffer buf.  The 16 code and
  // 2 scale instructions of a group are spread over four stages (parts 3,
  // 0, 1, 2 in issue order: code instructions 0-4, 5-9, 10-14, then 15 and
  // the scales) instead of one burst.  A group past the last one gets
  // offsets beyond every view: the range check then drops all lanes, so the
  // DMA of the prefetch distance needs no branch at the end of K.
  auto dma_part = [&](int g, int buf, int part) {
    uint8_t *gbuf = smem + buf * kGroupBytes;
    const bool gin = g < g1;
    const int q0 = part == 3 ? 0 : 5 * part + 5, q1 = part == 3 ? 5 : part == 2 ? 16 : q0 + 5;
#pragma unroll
    for (int qq = q0; qq < q1; ++qq) {
      const bool real = !(BN == 128 && dma_b && qq >= 8);
      const int lrow = real ? lds_row0 + 8 * qq : spare_row0 + 8 * (qq - 8);
      dma16(dcodes, gbuf + lrow * 128, dv_code, (gin && real) ? 128u * (uint32_t)g + 8u * qq * rb : kOutOfRange);
    }
    if (SCALE_DMA && part == 2) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        const bool real = !(BN == 128 && dma_b && qq >= 1);
        const int lrow = real ? lds_row0 + 64 * qq : spare_row0;
        dma16(dscales, gbuf + kCodeBytes + lrow * 16, dv_scale,
              (gin && real) ? 16u * (uint32_t)g + 64u * qq * rs : kOutOfRange);
      }
    }
  };

  // ---- read side: A fragment i is LDS row 128wm + 32i + r, B fragment j
  // row BM + (BN/2)wn + 32j + r.
  const uint32_t a_row = 128 * wm + r, b_row = BM + (BN / 2) * wn + r;
  // Without scale DMA each lane loads its two scale bytes itself, from views
  // of this wave's A rows and B rows (byte loads: the range check is exact).
  __amdgpu_buffer_rsrc_t sview_a, sview_b;
  if constexpr (!SCALE_DMA) {
    const int64_t ar0 = min<int64_t>(m0 + 128 * wm, M), br0 = min<int64_t>(n0 + (BN / 2) * wn, N);
    sview_a = make_rsrc(SA + ar0 * rs, (uint32_t)min<int64_t>(128, M - ar0) * rs);
    sview_b = make_rsrc(SB + br0 * rs, (uint32_t)min<int64_t>(BN / 2, N - br0) * rs);
  }
  u32x4 codes[2][NF];      // [stage parity][fragment]: this lane's 32 codes
  uint32_t sraw[NF];       // their two E4M3 block scales (per-lane loads)
  u32x4 srow[NF];          // scale DMA: the fragment row's 16 scale bytes of the group, as read
  uint32_t sgrp[NF][2];    // ... this lane's two bytes of stages 0,1 and of stages 2,3
  // byte selector of v_perm_b32: bytes 2h, 2h+1 of two scale dwords
  const uint32_t ssel = h ? 0x07060302u : 0x05040100u;
  uint32_t keep = 0;       // which of those two scales lie inside K
  half2_t spair[NF];       // ... as an f16 pair
  half8_t opnd[2][NF];     // [K step parity][fragment]: decoded MFMA operands
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Codes and scales of stage sp of group g (LDS buffer gb) into codes[cb].
  // The scales of 16-blocks at or past K are zeroed, which zeroes those
  // products whatever codes the DMA left there (every E2M1 value is finite).
  // The mask is applied where the scales are converted, a few K steps
  // later: using the loaded values here would make the wave wait for the
  // LDS reads right after issuing them.
  const int k32 = (int)K;    // K < 2^25 (checked by the launcher)
  auto read_stage = [&](int cb, const uint8_t *gb, int g, int sp) {
    const int c = 2 * sp + h;
    const uint32_t slot = (uint32_t)((c ^ (r & 7)) * 16);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t row = f < 4 ? a_row + 32 * f : b_row + 32 * (f - 4);
      codes[cb][f] = *reinterpret_cast<const u32x4 *>(gb + row * 128 + slot);
      if constexpr (SCALE_DMA) {
        // all four stages' scales of the group in one conflict-free 16-byte
        // read per row (per-stage 2-byte reads put 32 rows on 8 banks)
        if (sp == 0) srow[f] = *reinterpret_cast<const u32x4 *>(gb + kCodeBytes + row * 16);
      } else {
        const __amdgpu_buffer_rsrc_t v = f < 4 ? sview_a : sview_b;
        const uint32_t vo = (uint32_t)r * rs + 2 * h;
        const uint32_t so = 16u * (uint32_t)g + 4u * sp + 32u * (uint32_t)(f < 4 ? f : f - 4) * rs;
        sraw[f] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(v, vo, so, 0) |
                  ((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(v, vo, so + 1, 0) << 8);
      }
    }
    const int kc = kGroupK * g + 32 * c;
    keep = (kc < k32 ? 0x00FFu : 0u) | (kc + 16 < k32 ? 0xFF00u : 0u);
  };
  // This lane's scale bytes of the group's four stages, a K step after the
  // 16-byte reads were issued.
  auto pick_scales = [&]() {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      sgrp[f][0] = __builtin_amdgcn_perm(srow[f].y, srow[f].x, ssel);
      sgrp[f][1] = __builtin_amdgcn_perm(srow[f].w, srow[f].z, ssel);
    }
  };
  // f16 pairs of the scales of stage sp (of the group last read).
  auto scale_pairs = [&](auto spc) {
    constexpr int sp = decltype(spc)::value;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if constexpr (SCALE_DMA)
        spair[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sgrp[f][sp >> 1] & (keep << (16 * (sp & 1))), 1.0f,
                                                            (sp & 1) != 0);
      else
        spair[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw[f] & keep, 1.0f, false);
    }
  };
  // Half `part` (bytes 2part, 2part+1 = 4 codes) of word ks of fragment f:
  // K step ks lies in 16-block ks/2 of the chunk.
  auto decode_half = [&](int cb, int ks, int f, int part, int db) {
    const u32x4 cw = codes[cb][f];
    const uint32_t w = ks == 0 ? cw.x : ks == 1 ? cw.y : ks == 2 ? cw.z : cw.w;
    const half2_t p = spair[f];
    const half2_t s = (ks >> 1) ? (half2_t){p[1], p[1]} : (half2_t){p[0], p[0]};
    const half2_t x0 = (part ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0)) * s;
    const half2_t x1 = (part ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)
                             : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1)) * s;
    half8_t &d = opnd[db][f];
    d[4 * part + 0] = x0[0];
    d[4 * part + 1] = x0[1];
    d[4 * part + 2] = x1[0];
    d[4 * part + 3] = x1[1];
  };

  // ---- prologue: group g0 and the first part of group g0+1 in flight
  // (the rest of group g0+1 follows in stages 0-2), stage 0 read, K step 0
  // decoded.  Group g lives in LDS buffer g & 1.
#pragma unroll
  for (int part = 0; part < 4; ++part) dma_part(g0, g0 & 1, part);
  dma_part(g0 + 1, (g0 + 1) & 1, 3);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (flag != nullptr && tid == 0) __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  read_stage(0, smem + (g0 & 1) * kGroupBytes, g0, 0);
  __builtin_amdgcn_s_waitcnt(0);     // nothing outstanding at loop entry
  if constexpr (SCALE_DMA) pick_scales();
  scale_pairs(std::integral_constant<int, 0>{});
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    decode_half(0, 0, f, 0, 0);
    decode_half(0, 0, f, 1, 0);
  }

  // Stage s = 4g + P.  K step ks: its NU MFMAs, each followed by its share
  // of the decode of the next K step (of this stage, or K step 0 of the next
  // stage), the order fixed by sched_barrier fences.  K step 0 reads the
  // next stage's codes from LDS and then issues one part of the DMA of
  // group g+1 (stages 0-2).  In the last stage of a group it first waits for
  // this wave's DMA of group g+1 and meets the other waves at the barrier --
  // after which group g+1 is in LDS and no wave reads group g any more --
  // reads stage 0 of group g+1 and starts the DMA of group g+2 into group
  // g's buffer.  The reads come before the DMA so that per-lane scale loads
  // do not queue behind it.
  auto stage = [&](int g, auto phase) {
    constexpr int P = decltype(phase)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    const uint8_t *gb = smem + (g & 1) * kGroupBytes;
    const uint8_t *gn = smem + ((g + 1) & 1) * kGroupBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int dcur = ks & 1, dnxt = dcur ^ 1;
      if (ks == 0) {
        if (P == 3) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's DMA of group g+1
          __syncthreads();
          read_stage(nxt, gn, g + 1, 0);
          dma_part(g + 2, g & 1, 3);
        } else {
          read_stage(nxt, gb, g, P + 1);
          dma_part(g + 1, (g + 1) & 1, P);
        }
      }
      if (SCALE_DMA && P == 3 && ks == 1) pick_scales();
      if (ks == 3) scale_pairs(std::integral_constant<int, (P + 1) & 3>{});
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        // snake order: the B fragment stays the same across the step to
        // the next A fragment (MFMA power, hence clock, follows operand
        // toggling)
        const int mi = u / NB, mj = (mi & 1) ? NB - 1 - u % NB : u % NB;
        acc[mi][mj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(opnd[dcur][mi], opnd[dcur][4 + mj], acc[mi][mj], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // decode halves [u*2NF/NU, (u+1)*2NF/NU) of the next K step
#pragma unroll
        for (int hv = (u * 2 * NF) / NU; hv < ((u + 1) * 2 * NF) / NU; ++hv) {
          if (ks < 3)
            decode_half(cur, ks + 1, hv >> 1, hv & 1, dnxt);
          else
            decode_half(nxt, 0, hv >> 1, hv & 1, dnxt);
        }
      }
    }
  };
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;
  for (int g = g0; g < g1; ++g) {
    stage(g, P0{});
    stage(g, P1{});
    stage(g, P2{});
    stage(g, P3{});
  }
  __builtin_amdgcn_sched_barrier(0);
  // the prefetch DMAs past g1 (out of range) are the only ones left
  __builtin_amdgcn_s_waitcnt(0);
}

constexpr int kDeviceScope = 0x10;     // cache-policy bits: sc1

// C tile = ((acc + P) * gA) * gB, P the unscaled f32 partial of a 256 x 256
// tile at `partial` (workspace layout: float4 q of thread tid at byte
// 16 * (256 q + tid)) or 0 when `partial` is null.  Lane holds column r and
// rows 8*(e/4) + 4*h + e%4 of each 32x32 block; row offsets are uniform, so
// the per-store address is one lane base plus a scalar offset.
//
// The partial goes through LDS, which must be free (every wave past the
// main loop and a barrier): each half (blocks of rows i = 0,1, then 2,3) is
// copied in by the DMA form -- all of a wave's loads in flight at once,
// each wave only its own threads' float4s (1 KB per index q), so no barrier
// between the copy and the reads -- and added block by block as the rows
// are stored.  The loads use the sc1 policy (see store_partial_data).
template <bool OUT_BF16, int BN>
__device__ __forceinline__ void tile_store(const TileAcc<BN> &acc, int64_t m0, int64_t n0, float gA, float gB,
                                           int64_t M, int64_t N, void *__restrict__ C, int64_t ldc,
                                           int tid = threadIdx.x, uint8_t *smem = nullptr,
                                           const uint8_t *partial = nullptr) {
  constexpr int NB = BN / 64;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, h = lane >> 5;
  const int64_t row_l = m0 + wm * 128 + 4 * h, col_l = n0 + wn * (BN / 2) + r;
  const bool full_tile = (m0 + BM <= M) && (n0 + BN <= N);
  using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
  OutT *base = reinterpret_cast<OutT *>(C) + row_l * ldc + col_l;
  __amdgpu_buffer_rsrc_t prsrc;
  if (BN == 256 && partial != nullptr) prsrc = make_rsrc(partial, (uint32_t)(BM * 256 * 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float16_t v[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) v[j] = acc[i][j];
    if constexpr (BN == 256) {
      if (partial != nullptr) {
        if ((i & 1) == 0) {
          // float4 q = 32 half + qq of every thread: 4 KB at 4096 q; this
          // wave's kilobyte of it at + 1024 wave, into LDS at 4096 qq + the same
          const int half = i >> 1;
          __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the previous half's reads are done
#pragma unroll
          for (int qq = 0; qq < 32; ++qq)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                prsrc, (__attribute__((address_space(3))) void *)(smem + 4096 * qq + 1024 * wave), 16,
                (uint32_t)(16 * lane), (uint32_t)(4096 * (32 * half + qq) + 1024 * wave), 0, kDeviceScope);
          __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this wave's copies are in LDS
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int b = (i & 1) * 4 + j;           // block (i, j) within its half
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const float4 p = *reinterpret_cast<const float4 *>(smem + 4096 * (4 * b + q4) + 16 * tid);
            v[j][4 * q4] += p.x;
            v[j][4 * q4 + 1] += p.y;
            v[j][4 * q4 + 2] += p.z;
            v[j][4 * q4 + 3] += p.w;
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int roff = 32 * i + 8 * (e >> 2) + (e & 3);
      if (!full_tile && row_l + roff >= M) continue;
      OutT *prow = base + (int64_t)roff * ldc;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (!full_tile && col_l + 32 * j >= N) continue;
        // streaming stores: C is written once, and its lines would
        // otherwise take cache space from the operand panels
        const float x = (v[j][e] * gA) * gB;
        if constexpr (OUT_BF16)
          __builtin_nontemporal_store(f32_to_bf16_rne(x), prow + 32 * j);
        else
          __builtin_nontemporal_store(x, prow + 32 * j);
      }
    }
  }
}

// One 256 x BN output tile: workgroup `pid` of the tiles of C[M][N] = A.B^T
// (B, C and N already restricted to this tile width's column range), placed
// XCD-contiguously and grouped by tile rows.
template <bool OUT_BF16, bool SCALE_DMA, int BN>
__device__ __forceinline__ void gemm_tile(uint8_t *smem, int pid, const uint8_t *__restrict__ A,
                                          const uint8_t *__restrict__ SA, const float *__restrict__ metaA,
                                          const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB,
                                          const float *__restrict__ metaB, int64_t M, int64_t N, int64_t K,
                                          void *__restrict__ C, int64_t ldc) {
  const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
  int tm, tn;
  xcd_tile(pid, tiles_m, tiles_n, kGroupM, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  TileAcc<BN> acc;
  tile_accumulate<SCALE_DMA, BN>(smem, m0, n0, 0, (int)((K + kGroupK - 1) / kGroupK), A, SA, B, SB, M, N, K, acc);
  tile_store<OUT_BF16, BN>(acc, m0, n0, metaA[1], metaB[1], M, N, C, ldc);
}

// The GEMM kernel: workgroups [0, n_big) compute the 256 x 256 tiles of
// columns [0, n1), the others the 256 x 128 tiles of columns [n1, N).  The
// branch is uniform per workgroup; LDS holds two group buffers sized for the
// wider tile (2 x 72 KB).
template <bool OUT_BF16, bool SCALE_DMA>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm_nvfp4(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ metaA,
             const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ metaB,
             int64_t M, int64_t N, int64_t K, void *__restrict__ C, int64_t ldc, int n_big, int64_t n1) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kGroupBytes];
  const int pid = blockIdx.x;
  if (pid < n_big) {
    gemm_tile<OUT_BF16, SCALE_DMA, 256>(smem, pid, A, SA, metaA, B, SB, metaB, M, n1, K, C, ldc);
  } else {
    using OutT = typename std::conditional<OUT_BF16, uint16_t, float>::type;
    gemm_tile<OUT_BF16, SCALE_DMA, 128>(smem, pid - n_big, A, SA, metaA, B + n1 * (K / 2), SB + n1 * (K / 16), metaB, M,
                             N - n1, K, reinterpret_cast<OutT *>(C) + n1, ldc);
  }
}

// ------------------------------------------------------- split tail ----
//
// The data-parallel grid runs whole tiles, so when the tile count is not a
// multiple of the CU count the last round leaves CUs idle.  For grids of
// fewer tiles than one round of the CUs (grids of at least one round take
// the stream-K tail below): the whole rounds run as before, and each of
// the remaining `rem` tiles is cut into `sp` equal K ranges (sp = CUs /
// rem, at least kMinSplitGroups K groups per range), one workgroup per
// range, so the CUs fill.
//
// Of the sp workgroups of a split tile, the last (highest-numbered) one
// finishes it: the others each write their unscaled f32 partial to their
// own workspace slot and raise its flag; the finisher waits for the flags,
// adds the partials in increasing range order to its own, and stores the
// tile.  The result does not depend on timing (deterministic).  Splitting
// the tail of a larger grid this way pays only where the ranges are long:
// on the layer shapes, a 2-way split of dgrad's 40-group ranges gained
// 1.5 %, 4-way splits of 5- and 8-group ranges (fprop, wgrad) lost 10 %
// and 1 % to the mixed 256/128-wide grid (a second wave of short
// workgroups, each with its own prologue, partial and wait).
//
// Progress: a finisher waits only for lower-numbered workgroups, which never
// wait themselves; workgroups of one dispatch start in increasing order (per
// XCD), so every wait ends.  The wait is bounded anyway: after about a
// second it gives up, counts the event in the workspace's error word and
// finishes the tile (that output is then wrong, but the kernel drains).
//
// Workspace: flags at bytes [0, 32 KB) (slot t's at 128 t), the error word
// at 32 KB, slot t's partial (256 x 256 f32, 256 KB) at 64 KB + 256 KB t.
// Flags are 0 between launches: the finisher clears each flag it consumed.
constexpr int kSplitMaxSlots = 256;
constexpr int64_t kSplitFlagBytes = 128;
constexpr int64_t kSplitErrOffset = 32 << 10;
constexpr int64_t kSplitSlot0 = 64 << 10;
constexpr int64_t kSplitSlotBytes = (int64_t)BM * 256 * 4;
constexpr unsigned kSplitSpinLimit = 1u << 20;        // polls of ~1000 clocks each

struct SplitSched {
  int tiles_m, tiles_n;     // 256 x 256 tiles of C, in row groups of kGroupM
  int n_dp;                 // whole tiles (the first n_dp in that order), one workgroup each
  int sp;                   // K ranges per remaining tile (1: no split)
};

// Tile u (0 .. tiles-1) in row groups of kGroupM tile rows.
__device__ __forceinline__ void grouped_tile(int u, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int per_group = kGroupM * tiles_n;
  const int first_m = (u / per_group) * kGroupM;
  const int gsz = min(tiles_m - first_m, kGroupM);
  tm = first_m + (u % per_group) % gsz;
  tn = (u % per_group) / gsz;
}

// Workgroup pid of n (dealt round-robin to the eight XCDs) -> its index in
// an XCD-contiguous order of n items.
__device__ __forceinline__ int xcd_logical(int pid, int n) {
  constexpr int kXcds = 8;
  const int xcd = pid % kXcds, local = pid / kXcds;
  const int q = n / kXcds, rq = n % kXcds;
  return (xcd < rq) ? xcd * (q + 1) + local : rq * (q + 1) + (xcd - rq) * q + local;
}

// Unscaled f32 partial of a 256 x 256 tile into a workspace slot, then the
// slot's flag.  Float4 q of thread tid at byte 16 * (256 q + tid): each
// wave's store or load instruction covers one contiguous kilobyte.  The
// stores write through this XCD's L2 (the sc1 cache policy) and the flag
// follows their completion, so a reader on another XCD that loads with the
// same policy after seeing the flag gets the stored values.
__device__ __forceinline__ void store_partial_data(const TileAcc<256> &acc, uint8_t *ws, int slot_idx) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t slot =
      make_rsrc(ws + kSplitSlot0 + (int64_t)slot_idx * kSplitSlotBytes, (uint32_t)kSplitSlotBytes);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        __builtin_amdgcn_raw_buffer_store_b128(
            (u32x4){__float_as_uint(acc[i][j][4 * c]), __float_as_uint(acc[i][j][4 * c + 1]),
                    __float_as_uint(acc[i][j][4 * c + 2]), __float_as_uint(acc[i][j][4 * c + 3])},
            slot, (uint32_t)(16 * (256 * ((i * 4 + j) * 4 + c) + tid)), 0, kDeviceScope);
}

__device__ __forceinline__ unsigned *slot_flag(uint8_t *ws, int slot_idx) {
  return reinterpret_cast<unsigned *>(ws + (int64_t)slot_idx * kSplitFlagBytes);
}

// The partial and then its flag, once every wave's stores have completed.
__device__ __forceinline__ void store_partial(const TileAcc<256> &acc, uint8_t *ws, int slot_idx) {
  store_partial_data(acc, ws, slot_idx);
  __builtin_amdgcn_s_waitcnt(0);     // this wave's partial stores have completed
  __syncthreads();                   // ... and every other wave's
  if (threadIdx.x == 0) __hip_atomic_store(slot_flag(ws, slot_idx), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (thread 0) for the flags of slots [c0, c1) and clear them; a wait
// that gives up counts in the error word.  Ends with a workgroup barrier.
__device__ __forceinline__ void wait_flags(uint8_t *ws, int c0, int c1) {
  if (threadIdx.x == 0) {
    for (int c = c0; c < c1; ++c) {
      unsigned *flag = reinterpret_cast<unsigned *>(ws + (int64_t)c * kSplitFlagBytes);
      unsigned n = 0;
      while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        if (++n >= kSplitSpinLimit) {
          atomicAdd(reinterpret_cast<unsigned *>(ws + kSplitErrOffset), 1u);
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
}

// acc += the partials of slots c0 .. c0 + n - 1 (n not known at compile
// time), in that order, one 32 x 32 block at a time: only that block's 16
// accumulators pass through the loop over contributors (a loop carrying all
// 256 would spill).
__device__ __forceinline__ void add_partials_n(TileAcc<256> &acc, const uint8_t *ws, int c0, int n) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t parts =
      make_rsrc(ws + kSplitSlot0 + (int64_t)c0 * kSplitSlotBytes, (uint32_t)(n * kSplitSlotBytes));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float16_t v = acc[i][j];
      for (int c = 0; c < n; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 p = __builtin_amdgcn_raw_buffer_load_b128(
              parts, (uint32_t)(16 * (256 * ((i * 4 + j) * 4 + q) + tid)), (uint32_t)(c * kSplitSlotBytes),
              kDeviceScope);
          v[4 * q] += __uint_as_float(p.x);
          v[4 * q + 1] += __uint_as_float(p.y);
          v[4 * q + 2] += __uint_as_float(p.z);
          v[4 * q + 3] += __uint_as_float(p.w);
        }
      }
      acc[i][j] = v;
    }
}

template <bool OUT_BF16, bool SCALE_DMA>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm_nvfp4_split(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ metaA,
                   const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ metaB,
                   int64_t M, int64_t N, int64_t K, void *__restrict__ C, int64_t ldc, uint8_t *__restrict__ ws,
                   SplitSched sc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kGroupBytes];
  const int pid = blockIdx.x;
  const int ng = (int)((K + kGroupK - 1) / kGroupK);
  int u, g0 = 0, g1 = ng, part = 0, t = 0;
  if (pid < sc.n_dp) {
    u = xcd_logical(pid, sc.n_dp);
  } else {
    t = pid - sc.n_dp;
    part = t % sc.sp;
    u = sc.n_dp + t / sc.sp;
    g0 = (int)((int64_t)part * ng / sc.sp);
    g1 = (int)((int64_t)(part + 1) * ng / sc.sp);
  }
  int tm, tn;
  grouped_tile(u, sc.tiles_m, sc.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * 256;
  TileAcc<256> acc;
  tile_accumulate<SCALE_DMA, 256>(smem, m0, n0, g0, g1, A, SA, B, SB, M, N, K, acc);
  if (pid >= sc.n_dp && part < sc.sp - 1) {
    store_partial(acc, ws, t);
    return;
  }
  if (pid >= sc.n_dp && sc.sp > 1) {
    // the finisher: ranges 0 .. sp-2 are slots t-part .. t-1
    wait_flags(ws, t - part, t);
    add_partials_n(acc, ws, t - part, part);
  }
  tile_store<OUT_BF16, 256>(acc, m0, n0, metaA[1], metaB[1], M, N, C, ldc);
}

// ------------------------------------------------- stream-K tail ----
//
// For grids of at least one round of 256 x 256 tiles.  All rounds but the
// last whole one run data-parallel (one tile per workgroup); the tiles left
// (between one and two rounds) are cut into eight chunks of whole tiles, one
// per XCD, and the chunk's K groups ("units", tile after tile in the grouped
// tile order) are dealt out in equal contiguous ranges to the XCD's
// workgroups.  Every range is at least one tile long, so a range is a head
// segment (the first K groups of a tile, whose tail the next workgroup of
// the XCD holds), whole tiles, and a tail segment (the rest of the tile
// whose head the previous workgroup holds).  Each workgroup works its range
// backwards: the head first -- its f32 partial goes to the workgroup's
// workspace slot and raises its flag -- then the whole tiles, then the tail,
// which it finishes by adding the previous workgroup's head partial (raised
// long before) and storing the tile.  Every tile is thus the sum of at most
// two ranges, added in one fixed order, and the last round fills the CUs:
// the fprop, dgrad and wgrad layers (1.25, 2.5 and 6.25 rounds of work) run
// it in as many round-times plus two segment starts.  Measured against the
// mixed 256/128-wide grid on the same GPU: fprop -9.7 %, dgrad -1.6 % (as
// the split tail), wgrad -0.8 % (that grid's partial last round of 256-wide
// tiles already overlaps its 128-wide ones).  What keeps the overhead small:
// the head's flag is raised by the next segment's prologue, whose wait for
// its first DMA also covers the partial's stores; the tail adds the partial
// from LDS, where each half of it arrives by DMA with all loads in flight
// (loading it into registers block by block serialised 64 round trips to
// memory and cost 9 % on fprop).
//
// Workgroups are dealt round-robin to the XCDs, so the XCD's workgroups are
// pid = xcd + 8 l in increasing local index l, and a finisher waits only
// for pid - 8 on its own XCD, which was dispatched before it and waits only
// for pid - 16; the chain ends at l = 0, whose range starts a chunk.  The
// wait is bounded as in the split kernel.  Workspace as for the split
// kernel; slot and flag s belong to stream-K workgroup s (pid - n_dp).
struct SkSched {
  int tiles_m, tiles_n;     // 256 x 256 tiles of C, in row groups of kGroupM
  int n_dp;                 // data-parallel tiles (the first n_dp), one workgroup each
  int t_sk;                 // tiles of the stream-K part (the rest), t_sk >= 8 w
  int w;                    // stream-K workgroups per XCD
};

template <bool OUT_BF16, bool SCALE_DMA>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
k_gemm_nvfp4_sk(const uint8_t *__restrict__ A, const uint8_t *__restrict__ SA, const float *__restrict__ metaA,
                const uint8_t *__restrict__ B, const uint8_t *__restrict__ SB, const float *__restrict__ metaB,
                int64_t M, int64_t N, int64_t K, void *__restrict__ C, int64_t ldc, uint8_t *__restrict__ ws,
                SkSched sc) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kGroupBytes];
  const int pid = blockIdx.x;
  const int ng = (int)((K + kGroupK - 1) / kGroupK);
  // this workgroup's units [v0, v1), unit v = K group v % ng of tile v / ng
  // (tiles * ng < 2^31, checked by the launcher)
  int v0, v1;
  int s = -1;                        // stream-K index (slot), -1 if data-parallel
  if (pid < sc.n_dp) {
    v0 = xcd_logical(pid, sc.n_dp) * ng;
    v1 = v0 + ng;
  } else {
    s = pid - sc.n_dp;
    const int xcd = s % 8, l = s / 8;
    const int c0 = (int)((int64_t)sc.t_sk * xcd / 8), c1 = (int)((int64_t)sc.t_sk * (xcd + 1) / 8);
    const int base = (sc.n_dp + c0) * ng;
    const int64_t units = (int64_t)(c1 - c0) * ng;
    v0 = base + (int)(units * l / sc.w);
    v1 = base + (int)(units * (l + 1) / sc.w);
  }
  const int t_hi = (v1 - 1) / ng, g_hi = v1 - t_hi * ng;     // last tile, its end group (1 .. ng)
  const int t_lo = v0 / ng, g_lo = v0 - t_lo * ng;           // first tile, its start group
  int t = t_hi;
  if (g_hi < ng) {
    // head segment (groups [0, g_hi) of tile t_hi): the next workgroup of
    // the XCD finishes the tile
    int tm, tn;
    grouped_tile(t, sc.tiles_m, sc.tiles_n, tm, tn);
    TileAcc<256> acc;
    tile_accumulate<SCALE_DMA, 256>(smem, (int64_t)tm * BM, (int64_t)tn * 256, 0, g_hi, A, SA, B, SB, M, N, K, acc);
    // the flag is raised by the next segment once these stores complete
    store_partial_data(acc, ws, s);
    --t;
  }
  unsigned *flag = g_hi < ng ? slot_flag(ws, s) : nullptr;
  const float gA = metaA[1], gB = metaB[1];
  for (; t >= t_lo; --t) {
    const int g0 = t == t_lo ? g_lo : 0;
    if (t != t_hi || g_hi < ng) __syncthreads();    // every wave is done with the previous segment's LDS
    int tm, tn;
    grouped_tile(t, sc.tiles_m, sc.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * 256;
    TileAcc<256> acc;
    tile_accumulate<SCALE_DMA, 256>(smem, m0, n0, g0, ng, A, SA, B, SB, M, N, K, acc, flag);
    flag = nullptr;
    // Opaque copies of what only the epilogue uses: keeps the compiler from
    // computing the epilogue's addressing before the loop and holding it in
    // registers across the main loop.
    int64_t ldc_s = ldc, m_s = M, n_s = N;
    int tid = threadIdx.x;
    asm volatile("" : "+s"(ldc_s), "+s"(m_s), "+s"(n_s), "+v"(tid));
    const uint8_t *partial = nullptr;
    if (g0 > 0) {                    // tail: add the head of the previous workgroup of the XCD
      wait_flags(ws, s - 8, s - 7);
      partial = ws + kSplitSlot0 + (int64_t)(s - 8) * kSplitSlotBytes;
    }
    tile_store<OUT_BF16, 256>(acc, m0, n0, gA, gB, m_s, n_s, C, ldc_s, tid, smem, partial);
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

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

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
  // The DMA views address 128 rows with 32-bit offsets below the
  // out-of-range marker 2^31 (this also keeps K below 2^25).
  if ((int64_t)128 * (K / 2) >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  // Balance the grid over the CUs.  Columns [0, n1) get 256 x 256 tiles and
  // the rest 256 x 128 tiles (half the work per tile; their per-flop cost is
  // taken as 1.1x); n1 minimises the modelled time
  //   rounds(256-wide tiles) + 0.55 * rounds(128-wide tiles),
  // rounds(t) = ceil(t / CUs).  The fprop, dgrad and wgrad layers would
  // otherwise run 1.25, 2.5 and 6.25 rounds of 256 x 256 tiles as 2, 3 and 7.
  // Both tile widths run in one launch; every output element is computed by
  // exactly one workgroup.
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
  // Scale rows go through the DMA only when they are whole dwords (K % 64
  // == 0): the range check of a view works per dword, and with a row pitch
  // of K/16 bytes not a multiple of 4 the dword holding a view's last scale
  // bytes reaches past the view and would be dropped whole.  Code rows
  // (K/2 bytes) are always a multiple of 8.
  const bool scale_dma = K % 64 == 0;
#define NVFP4_GEMM_LAUNCH(OB, SD)                                                                          \
  hipLaunchKernelGGL((k_gemm_nvfp4<OB, SD>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, a_meta, \
                     b_codes, b_scales, b_meta, M, N, K, c, ldc, (int)n_big, best_n1)
  if (c_dtype == 0) {
    if (scale_dma) NVFP4_GEMM_LAUNCH(false, true);
    else NVFP4_GEMM_LAUNCH(false, false);
  } else {
    if (scale_dma) NVFP4_GEMM_LAUNCH(true, true);
    else NVFP4_GEMM_LAUNCH(true, false);
  }
#undef NVFP4_GEMM_LAUNCH
  return hipGetLastError();
}

int64_t gemm_split_workspace_bytes() { return kSplitSlot0 + (int64_t)kSplitMaxSlots * kSplitSlotBytes; }

// ------------------------------------------- library-owned workspace ----
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid it): the split GEMM's workspace as a
// file-scope device array, one copy per GPU, held until the process ends.
// In host code `scratch` names a host-side stand-in, so its device address
// comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is passed to kernels.  Calls on one GPU
// share the array: calls that overlap in time on one GPU race.
constexpr int64_t kScratchBytes = kSplitSlot0 + (int64_t)kSplitMaxSlots * kSplitSlotBytes;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void k_zero_words(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0u;
}

int64_t gemm_scratch_bytes() { return kScratchBytes; }

hipError_t gemm_scratch(hipStream_t stream, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // The flags and the error word must start at zero; the kernel leaves
    // them at zero after every complete launch.  A fill kernel, ordered on
    // the caller's stream before the first GEMM (no memset: it may be
    // captured into a graph).
    hipLaunchKernelGGL(k_zero_words, dim3(64), dim3(256), 0, stream, (uint32_t *)p, kSplitSlot0 / 4);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_gemm_split(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_meta,
                          const uint8_t *b_codes, const uint8_t *b_scales, const float *b_meta, int64_t M,
                          int64_t N, int64_t K, void *c, int c_dtype, int64_t ldc, void *ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  if (K == 0) {
    int64_t total = M * N;
    unsigned g = (unsigned)std::min<int64_t>((total + 255) / 256, 65536);
    hipLaunchKernelGGL(k_zero_c, dim3(g), dim3(256), 0, stream, c, M, N, ldc, c_dtype == 0 ? 4 : 2);
    return hipGetLastError();
  }
  if ((int64_t)128 * (K / 2) >= (int64_t)kOutOfRange) return hipErrorInvalidValue;
  const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + 255) / 256, tiles = tiles_m * tiles_n;
  const int64_t ng = (K + kGroupK - 1) / kGroupK;
  const int64_t P = std::min<int64_t>(device_cus(), kSplitMaxSlots);
  const bool scale_dma = K % 64 == 0;
  // At least one round of tiles, not a whole number of rounds: the
  // stream-K tail over the last one to two rounds, on P rounded down to
  // whole XCDs, when tiles are long enough in K that a segment's start and
  // the partial's round trip are small against it (measured: at 8 groups
  // per tile the stream-K tail is 10 % slower than the mixed grid, at 20
  // and more it is faster).
  constexpr int64_t kSkMinGroups = 16;
  const int64_t p_sk = P / 8 * 8;
  if (p_sk >= 8 && tiles >= p_sk && tiles % p_sk != 0 && ng >= kSkMinGroups && tiles * ng <= INT32_MAX) {
    SkSched sk;
    sk.tiles_m = (int)tiles_m;
    sk.tiles_n = (int)tiles_n;
    sk.n_dp = (int)((tiles / p_sk - 1) * p_sk);
    sk.t_sk = (int)(tiles - sk.n_dp);
    sk.w = (int)(p_sk / 8);
    const dim3 grid((unsigned)(sk.n_dp + p_sk));
#define NVFP4_GEMM_SK_LAUNCH(OB, SD)                                                                               \
  hipLaunchKernelGGL((k_gemm_nvfp4_sk<OB, SD>), grid, dim3(kThreads), 0, stream, a_codes, a_scales, a_meta, b_codes, \
                     b_scales, b_meta, M, N, K, c, ldc, (uint8_t *)ws, sk)
    if (c_dtype == 0) {
      if (scale_dma) NVFP4_GEMM_SK_LAUNCH(false, true);
      else NVFP4_GEMM_SK_LAUNCH(false, false);
    } else {
      if (scale_dma) NVFP4_GEMM_SK_LAUNCH(true, true);
      else NVFP4_GEMM_SK_LAUNCH(true, false);
    }
#undef NVFP4_GEMM_SK_LAUNCH
    return hipGetLastError();
  }
  // whole rounds data-parallel; the rem remaining tiles split into sp K
  // ranges each, sp * rem <= P, at least kMinSplitGroups groups per range.
  // The split is taken when most CUs would idle without it (fewer than P/2
  // tiles) or when its ranges are long (at least kLongRangeGroups groups);
  // otherwise the mixed-width data-parallel grid of launch_gemm is faster.
  constexpr int64_t kMinSplitGroups = 4, kLongRangeGroups = 16;
  const int64_t rem = tiles % P;
  const int64_t sp = rem == 0 ? 1 : std::max<int64_t>(1, std::min<int64_t>(P / rem, ng / kMinSplitGroups));
  if (sp == 1 || (2 * tiles >= P && ng / sp < kLongRangeGroups))
    return launch_gemm(a_codes, a_scales, a_meta, b_codes, b_scales, b_meta, M, N, K, c, c_dtype, ldc, stream);
  const int64_t grid = (tiles - rem) + rem * sp;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  SplitSched sc;
  sc.tiles_m = (int)tiles_m;
  sc.tiles_n = (int)tiles_n;
  sc.n_dp = (int)(tiles - rem);
  sc.sp = (int)sp;
#define NVFP4_GEMM_SPLIT_LAUNCH(OB, SD)                                                                         \
  hipLaunchKernelGGL((k_gemm_nvfp4_split<OB, SD>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a_codes,     \
                     a_scales, a_meta, b_codes, b_scales, b_meta, M, N, K, c, ldc, (uint8_t *)ws, sc)
  if (c_dtype == 0) {
    if (scale_dma) NVFP4_GEMM_SPLIT_LAUNCH(false, true);
    else NVFP4_GEMM_SPLIT_LAUNCH(false, false);
  } else {
    if (scale_dma) NVFP4_GEMM_SPLIT_LAUNCH(true, true);
    else NVFP4_GEMM_SPLIT_LAUNCH(true, false);
  }
#undef NVFP4_GEMM_SPLIT_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
