// Device helpers shared by the MFMA partial-pass kernels (gfx950 only): LDS tile layout, direct
// global->LDS loads, lane-layout permutations and inline-asm MFMA forms.
#pragma once

#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kNst = 3;           // LDS ring stages
constexpr int kLatStride = 1056;  // bytes per latent row (bf16) or row pair (fp8): 1 KiB + 32 B pad
constexpr int kPbStride = 80;     // bytes per head row of the probability exchange buffer (64 + pad)

template <bool FP8>
struct Layout {
  static constexpr int kLatStage = FP8 ? 16 * kLatStride : 32 * kLatStride;
  static constexpr int kRopeOff = kLatStage;
  static constexpr int kScaleOff = kLatStage + 4096;
  static constexpr int kStage = kLatStage + 4096 + (FP8 ? 128 : 0);
};

// score-operand row for lane l (0..31): bits 2 and 3 swapped
__device__ __forceinline__ int pi_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// fp8 row offset inside a stage (two 512-byte rows per padded 1 KiB block)
__device__ __forceinline__ int fp8_row_off(int r) { return (r >> 1) * kLatStride + (r & 1) * 512; }

// Direct global->LDS loads (global_load_lds_dwordx4 / _dword): lane i writes bytes
// [lds + size*i, lds + size*(i+1)) from gbase + voff.  Issued through inline asm so that the
// compiler does not treat every later LDS read as dependent on them (it cannot tell the ring
// stages apart and would wait for all outstanding loads); completion is tracked explicitly with
// s_waitcnt vmcnt before the workgroup barrier that publishes a stage.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS void*)p;
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(uniform_ptr(gbase)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(uniform_ptr(gbase)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 8 E4M3 codes -> 8 bf16 (exact: every E4M3 value is a bf16 value); v_cvt_scalef32_pk_bf16_fp8
// with scale 1 converts two codes into one packed bf16 pair
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 v) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true))};
}

// uniform 32-bit load through the scalar data cache (s_load): keeps block-table lookups off the
// vector-memory counter that tracks the tile DMA loads
__device__ __forceinline__ int load_uniform_i32(const int32_t* p) {
  const uint64_t addr = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const __attribute__((address_space(4))) int32_t* q =
      (const __attribute__((address_space(4))) int32_t*)(((uint64_t)hi << 32) | lo);
  return *q;
}

constexpr int lgkmcnt_imm0() { return 15 | (3 << 14) | (7 << 4); }

// Score MFMAs with the accumulator in VGPRs (inline asm: the builtin would place it in AGPRs,
// which the output accumulator fills, forcing copies).  Back-to-back MFMAs accumulating into the
// same registers need no wait states; the caller adds the wait before VALU reads of the result.
__device__ __forceinline__ void mfma_v_first(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& d, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// s_waitcnt immediate waiting for vmcnt == 0 and lgkmcnt == 0 (tile loads landed, own LDS writes done)
constexpr int vm_lgkm_imm0() { return 7 << 4; }

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

}  // namespace mla
