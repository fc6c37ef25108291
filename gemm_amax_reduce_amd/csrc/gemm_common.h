// gemm_common.h -- pieces shared by the NVFP4 and MXFP4 GEMM kernels:
// range-checked buffer views, the buffer-load-to-LDS (DMA) form, the bf16
// output rounding and the XCD-aware tile order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

constexpr uint32_t kOutOfRange = 0x80000000u;       // buffer offset past every view

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  // 0x00020000: 32-bit data format word of a raw (stride 0) buffer on gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

// 16 bytes per lane from a buffer view into LDS at dst + 16 * lane (the
// gfx950 DMA form of buffer_load_dwordx4; dst must be wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t v, uint8_t *dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(v, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

// 4 bytes per lane into LDS at dst + 4 * lane (buffer_load_dword ... lds).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t v, uint8_t *dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(v, (__attribute__((address_space(3))) void *)dst, 4, voff, soff, 0, 0);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Tile (tm, tn) of workgroup pid among tiles_m x tiles_n tiles.  Workgroups
// are dealt round-robin to the eight XCDs (pid % 8); each XCD gets a
// contiguous range of tiles, ordered in groups of group_m tile rows, so the
// tiles resident on one XCD share A rows and B columns in its L2.
__device__ __forceinline__ void xcd_tile(int pid, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
  constexpr int kXcds = 8;
  const int ntiles = tiles_m * tiles_n;
  const int xcd = pid % kXcds, local = pid / kXcds;
  const int q = ntiles / kXcds, rq = ntiles % kXcds;
  const int logical = (xcd < rq) ? xcd * (q + 1) + local : rq * (q + 1) + (xcd - rq) * q + local;
  const int per_group = group_m * tiles_n;
  const int group = logical / per_group;
  const int first_m = group * group_m;
  const int gsz = min(tiles_m - first_m, group_m);
  tm = first_m + (logical % per_group) % gsz;
  tn = (logical % per_group) / gsz;
}

}  // namespace nvfp4
