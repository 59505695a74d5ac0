// Internal declarations shared by the HIP sources of the MLA decode library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla.h"

namespace mla {

// ----------------------------------------------------------------------------------------------
// Batch partition used by the partial and combine passes.
//
// Every sequence b is cut into tiles of kTile tokens (tiles_b = ceil(len_b / kTile)).  The tiles
// of all sequences are concatenated in sequence order (prefix P[b] = sum of tiles_b' for b' < b,
// NT = P[B]).  With Wp = min(W, NT) workgroups, workgroup w owns tiles
// [floor(w*NT/Wp), floor((w+1)*NT/Wp)), which is never empty.  The part of that range that falls
// in sequence b is one "segment"; it leaves one partial (m, l, acc) per head in workspace slot
// w + b.  Slots are unique because consecutive segments advance w, b, or both.
// ----------------------------------------------------------------------------------------------
constexpr int kTile = 32;
constexpr int kMaxB = 2048;
constexpr int kSmallMaxB = 256;   // batch limit of the small-batch partial kernel (tile prefix in LDS)

struct PartialArgs {
  const void* q_abs;            // [B, H, d_c]
  const void* q_R;              // [B, H, d_R]
  const void* latent;
  const void* rope;
  const float* lscale;
  const int32_t* block_table;
  int64_t lat_sb, lat_st, rope_sb, rope_st, scale_sb;
  int page_size, max_pages;
  const int32_t* seq_lens;
  int B, H, d_c, d_R;
  int W;                        // partial-pass workgroups requested
  float sl2;                    // softmax scale * log2(e)
  float* ws_acc;                // [slots, H, d_c] sums, float or bf16 (kPartF32 / kPartBF16)
  float* ws_ml;                 // [slots, H, 2]   (m in log2 units, l)
  int* ws_prefix;               // [B + 2] tile prefix sums, then the format of ws_acc (workgroup 0)
  int* ws_cnt;                  // [H] counters of the fused combine + uv pass, zeroed by workgroup 0
  const void* warm;             // optional: buffer to pull into the cache with the spare workgroups
  int64_t warm_bytes;
  int extra;                    // workgroups launched beyond W (only used for the warm-up)
  int hgroups;                  // MFMA pass: head groups (grid y); group g owns heads [g H/hgroups, ..)
  int small;                    // bf16: the small-batch kernel (one 32-head block per workgroup)
};

struct CombineArgs {
  const int32_t* seq_lens;
  int B, H, d_c;
  int W;
  const float* ws_acc;          // float or bf16 elements: ws_prefix[B + 1] says which
  const float* ws_ml;
  const int* ws_prefix;         // [B + 2] tile prefix sums and the sums' format, from the partial pass
  int* ws_cnt;                  // [H] fused combine + uv: finished quarters per head (0 on entry)
  float* ws_uv;                 // [min(B, 4), H, 4, 128] fused combine + uv: per-quarter outputs
  float* o_latent;              // [B, H, d_c]
  float* lse;                   // [B, H] or nullptr
};

// Element type of the partial sums in the acc block, recorded by the partial pass at
// ws_prefix[B + 1] for the combine: the large-batch MFMA kernel stores bf16 (half the bytes
// written and read back; the rounding is far below the bf16 operands' own), the fp32 and the
// small-batch kernels store float.
constexpr int kPartF32 = 0;
constexpr int kPartBF16 = 1;

// workspace layout (bytes): acc block, then (m, l) block, then the tile prefix sums, then the
// counters and per-quarter outputs of the fused combine + uv pass, each 256-byte aligned.  A slot
// of the acc block holds H x d_c floats, row-major [slot][H][d_c]: the partial pass writes whole
// 128-byte lines of a head's row, and a head's partial is contiguous for the combine.
inline size_t ws_slots(int W, int B) { return (size_t)W + (size_t)B - 1; }
inline size_t ws_acc_bytes(int W, int B, int H, int d_c) {
  size_t b = ws_slots(W, B) * (size_t)H * (size_t)d_c * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
inline size_t ws_ml_bytes(int W, int B, int H) {
  size_t b = ws_slots(W, B) * (size_t)H * 2 * sizeof(float);
  return (b + 255) & ~(size_t)255;
}
inline size_t ws_prefix_bytes(int B) { return (((size_t)B + 2) * sizeof(int) + 255) & ~(size_t)255; }
inline size_t ws_cnt_bytes(int H) { return ((size_t)H * sizeof(int) + 255) & ~(size_t)255; }
inline size_t ws_uv_bytes(int B, int H) {
  const size_t nb = B < 4 ? (size_t)B : 4;
  return (nb * (size_t)H * 4 * 128 * sizeof(float) + 255) & ~(size_t)255;
}
inline size_t ws_total_bytes(int W, int B, int H, int d_c) {
  return ws_acc_bytes(W, B, H, d_c) + ws_ml_bytes(W, B, H) + ws_prefix_bytes(B) + ws_cnt_bytes(H) + ws_uv_bytes(B, H);
}
// byte offsets of the regions after the acc block
inline size_t ws_ml_off(int W, int B, int H, int d_c) { return ws_acc_bytes(W, B, H, d_c); }
inline size_t ws_prefix_off(int W, int B, int H, int d_c) { return ws_ml_off(W, B, H, d_c) + ws_ml_bytes(W, B, H); }
inline size_t ws_cnt_off(int W, int B, int H, int d_c) { return ws_prefix_off(W, B, H, d_c) + ws_prefix_bytes(B); }
inline size_t ws_uv_off(int W, int B, int H, int d_c) { return ws_cnt_off(W, B, H, d_c) + ws_cnt_bytes(H); }

// launchers (return the launch error; host-side validation happens in mla_abi.cpp)
hipError_t launch_absorb_f32(const float* q, const float* w, float* out, int B, int H, int d_h, int d_c,
                             hipStream_t s);
hipError_t launch_absorb_bf16(const void* q, const void* w, void* out, int B, int H, hipStream_t s);
hipError_t launch_partial_f32(const PartialArgs& a, hipStream_t s);
hipError_t launch_partial_mfma(const PartialArgs& a, bool fp8, bool paged, hipStream_t s);
hipError_t launch_partial_small(const PartialArgs& a, bool paged, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);
hipError_t launch_uv_f32w(const float* o_lat, const float* w, float* out, int B, int H, int d_h, int d_c,
                          hipStream_t s);
hipError_t launch_uv_bf16w_generic(const float* o_lat, const void* w, float* out, int B, int H, int d_h,
                                   int d_c, hipStream_t s);
hipError_t launch_uv_bf16(const float* o_lat, const void* w, float* out, int B, int H, hipStream_t s);
hipError_t launch_combine_uv(const CombineArgs& a, const void* w, float* out, hipStream_t s);

}  // namespace mla

// ------------------------------------------------------------------------------------------------
// Device helpers (only visible to the HIP translation units)
// ------------------------------------------------------------------------------------------------
#if defined(__HIPCC__)
namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// four consecutive partial sums starting at element e (a multiple of 4) of the acc block, stored
// as float (BF = false) or bf16 (BF = true)
template <bool BF>
__device__ __forceinline__ float4 load_part4(const float* acc, int64_t e) {
  if constexpr (BF) {
    const u32x2 r = *(const u32x2*)((const uint16_t*)acc + e);
    return make_float4(__uint_as_float(r[0] << 16), __uint_as_float(r[0] & 0xffff0000u),
                       __uint_as_float(r[1] << 16), __uint_as_float(r[1] & 0xffff0000u));
  } else {
    return *(const float4*)(acc + e);
  }
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bfloat16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int tiles_of(int len) { return (len + kTile - 1) / kTile; }

// Builds P[0..B] (LDS) = prefix sums of tile counts, and L[0..B) = lengths (unless L is null).
// Ends with a barrier.
__device__ __forceinline__ void build_tile_prefix(const int32_t* __restrict__ lens, int B, int* P, int* L) {
  const int tid = threadIdx.x;
  for (int b = tid; b < B; b += blockDim.x) {
    int len = lens[b];
    if (L) L[b] = len;
    P[b + 1] = tiles_of(len);
  }
  if (tid == 0) P[0] = 0;
  __syncthreads();
  if (tid < 64) {
    int carry = 0;
    for (int base = 0; base < B; base += 64) {
      int i = base + tid;
      int v = (i < B) ? P[i + 1] : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        int u = __shfl_up(v, d, 64);
        if (tid >= d) v += u;
      }
      if (i < B) P[i + 1] = carry + v;
      carry += __shfl(v, 63, 64);
    }
  }
  __syncthreads();
}

// sequence that owns global tile t (P[b] <= t < P[b+1]); P has B+1 entries, t < P[B]
__device__ __forceinline__ int seq_of_tile(const int* P, int B, int t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (P[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace mla
#endif
