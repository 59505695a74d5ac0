// The two per-head projections around the attention pass, for the DeepSeek-V3 shape
// (d_h = 128, d_c = 512), on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
//   absorb:  q'[b,h,:]  = W_UK[h]^T q_C[b,h,:]   ([B x 128] . [128 x 512] per head)
//   uv:      o[b,h,:]   = W_UV[h] o_lat[b,h,:]   ([B x 512] . [512 x 128] per head)
//
// ("Grouped-query and latent attention", section "The absorption trick".)  Both read their weight
// once per launch for batches up to 128 (absorb) / 32 (uv) rows per workgroup; at B = 1 they are
// bandwidth-bound streams over the 16.8 MB weight.
#include "mla_internal.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// absorb.  Grid (H, 2 column halves, ceil(B/128)), 256 threads.  The workgroup stages its
// [128 x 256] slice of W_UK[h] in LDS; wave w computes rows b0 + 32w .. +31 of the output.
// MFMA operand A = q_C rows (k = i contiguous in memory), operand B = W_UK[h][i][col] read with
// the transposing LDS load ds_read_b64_tr_b16 (the reduction index i is the row index of W_UK).
// ---------------------------------------------------------------------------------------------
constexpr int kAbsStride = 256 + 16;  // LDS row stride (bf16 elements): 544 B = 8 dwords mod 64 banks

__global__ __launch_bounds__(256) void k_absorb_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int B, int H) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[128 * kAbsStride];
  const int h = blockIdx.x, half = blockIdx.y, bz = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const uint16_t* wsrc = w + (int64_t)h * 128 * 512 + half * 256;
#pragma unroll 4
  for (int c = tid; c < 128 * 32; c += 256) {
    const int row = c >> 5, ch = c & 31;
    const u32x4 v = *(const u32x4*)(wsrc + row * 512 + ch * 8);
    *(u32x4*)(&Ws[row * kAbsStride + ch * 8]) = v;
  }
  __syncthreads();

  const int b0 = bz * 128 + wave * 32;
  if (b0 >= B) return;
  const int brow = b0 + (lane & 31), kh = lane >> 5;
  u32x4 aq[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    if (brow < B) aq[ks] = *(const u32x4*)(q + ((int64_t)brow * H + h) * 128 + 16 * ks + 8 * kh);
    else aq[ks] = u32x4{0u, 0u, 0u, 0u};
  }
  const int G = lane >> 4, r4 = (lane & 15) >> 2, q4 = lane & 3;
  uint16_t* orow = out + (int64_t)h * 512 + half * 256 + (lane & 31);
#pragma unroll 1
  for (int cb = 0; cb < 8; ++cb) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const uint16_t* p0 = &Ws[(16 * ks + 8 * (G >> 1) + r4) * kAbsStride + 32 * cb + 16 * (G & 1) + 4 * q4];
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p0);
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 4 * kAbsStride));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      const u32x4 bop = {l2[0], l2[1], h2[0], h2[1]};
      acc = mfma32x32x16(aq[ks], bop, acc);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int b = b0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (b < B) orow[(int64_t)b * H * 512 + 32 * cb] = (uint16_t)(pack_bf16x2(acc[v], 0.f) & 0xffffu);
    }
  }
}

hipError_t launch_absorb_bf16(const void* q, const void* w, void* out, int B, int H, hipStream_t s) {
  dim3 grid(H, 2, (B + 127) / 128);
  hipLaunchKernelGGL(k_absorb_bf16, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w, (uint16_t*)out,
                     B, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// uv.  Grid (H, 2 halves of the 128 output rows, ceil(B/32)), 128 threads.  Wave w computes
// output rows i0 .. i0+31 (i0 = 64*half + 32w) for batch rows b0 .. b0+31.  Operand A = o_lat
// rows (fp32, split into bf16 hi + bf16 lo so the product keeps ~16 mantissa bits of o_lat),
// operand B = W_UV[h][i][k] rows straight from global memory (k contiguous).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void split_hi_lo(const float4& x0, const float4& x1, u32x4& hi, u32x4& lo) {
  const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h2 = pack_bf16x2(xs[2 * j], xs[2 * j + 1]);
    hi[j] = h2;
    lo[j] = pack_bf16x2(xs[2 * j] - __uint_as_float(h2 << 16), xs[2 * j + 1] - __uint_as_float(h2 & 0xffff0000u));
  }
}

__global__ __launch_bounds__(128) void k_uv_bf16(const float* __restrict__ o_lat, const uint16_t* __restrict__ w,
                                                 float* __restrict__ out, int B, int H) {
  const int h = blockIdx.x, ih = blockIdx.y, bz = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = ih * 64 + wave * 32;
  const int b0 = bz * 32;
  const int brow = b0 + (lane & 31), kh = lane >> 5;
  const bool bvalid = brow < B;
  const uint16_t* wr = w + ((int64_t)h * 128 + i0 + (lane & 31)) * 512 + 8 * kh;
  const float* xr = o_lat + ((int64_t)(bvalid ? brow : 0) * H + h) * 512 + 8 * kh;
  f32x16 acc = {};
#pragma unroll 8
  for (int ks = 0; ks < 32; ++ks) {
    const u32x4 bw = *(const u32x4*)(wr + 16 * ks);
    float4 x0 = make_float4(0.f, 0.f, 0.f, 0.f), x1 = x0;
    if (bvalid) {
      x0 = *(const float4*)(xr + 16 * ks);
      x1 = *(const float4*)(xr + 16 * ks + 4);
    }
    u32x4 hi, lo;
    split_hi_lo(x0, x1, hi, lo);
    acc = mfma32x32x16(hi, bw, acc);
    acc = mfma32x32x16(lo, bw, acc);
  }
  float* orow = out + (int64_t)h * 128 + i0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int b = b0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (b < B) orow[(int64_t)b * H * 128] = acc[v];
  }
}

hipError_t launch_uv_bf16(const float* o_lat, const void* w, float* out, int B, int H, hipStream_t s) {
  dim3 grid(H, 2, (B + 31) / 32);
  hipLaunchKernelGGL(k_uv_bf16, grid, dim3(128), 0, s, o_lat, (const uint16_t*)w, out, B, H);
  return hipGetLastError();
}

}  // namespace mla
