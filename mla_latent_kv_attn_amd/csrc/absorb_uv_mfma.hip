// The two per-head projections around the attention pass, for the DeepSeek-V3 shape
// (d_h = 128, d_c = 512), on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation.
//
//   absorb:  q'[b,h,:]  = W_UK[h]^T q_C[b,h,:]   ([B x 128] . [128 x 512] per head)
//   uv:      o[b,h,:]   = W_UV[h] o_lat[b,h,:]   ([B x 512] . [512 x 128] per head)
//
// ("Grouped-query and latent attention", section "The absorption trick".)  The MFMA kernels read
// the weight once per 128 (absorb) / 32 (uv) batch rows; for B <= 4 the streaming kernels below
// read it once, as plain bandwidth-bound passes over the 16.8 MB weight.
#include "lane_reduce.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// absorb.  Grid (H, 2 column halves, ceil(B/128)), 256 threads.  The workgroup stages its
// [128 x 256] slice of W_UK[h] in LDS; its (32-row block, 32-column block) output tiles are dealt
// to the four waves.
// MFMA operand A = q_C rows (k = i contiguous in memory), operand B = W_UK[h][i][col] read with
// the transposing LDS load ds_read_b64_tr_b16 (the reduction index i is the row index of W_UK).
// ---------------------------------------------------------------------------------------------
constexpr int kAbsStride = 256 + 16;  // LDS row stride (bf16 elements): 544 B = 8 dwords mod 64 banks

// (q is not __restrict__: an invariant load could be sunk below the LDS stores and the barrier,
// which costs a second memory round trip)
template <bool STG>
__global__ __launch_bounds__(256) void k_absorb_bf16(const uint16_t* q, const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int B, int H) {
  __shared__ __attribute__((aligned(16))) uint16_t Ws[128 * kAbsStride];
  __shared__ __attribute__((aligned(16))) uint8_t ostg[STG ? 4 : 1][32 * 144];   // per wave: 32 rows x 64 bf16 + pad
  const int h = blockIdx.x, half = blockIdx.y, bz = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Output tiles: (row block of 32 batch rows, column block of 32), nrb x 8 of them.  The waves
  // split evenly over the row blocks (4 / nrb waves each; with three row blocks the fourth wave
  // idles) and a row block's column blocks over its waves, so that every wave has MFMA work at
  // any batch size; a wave takes two adjacent column blocks at a time (two independent chains,
  // and 128-byte output rows).
  const int nrb = min(4, (B - bz * 128 + 31) / 32);
  const int wpr = nrb == 1 ? 4 : nrb == 2 ? 2 : 1;   // waves per row block
  const int rb = wave / wpr, cpw = 8 / wpr, cfirst = (wave % wpr) * cpw;

  // all 16 loads of the thread's share of the slice go out before the first LDS store (one memory
  // round trip, not one per group), and so do the q rows (rows past B read the last one; their
  // outputs are not stored)
  const uint16_t* wsrc = w + (int64_t)h * 128 * 512 + half * 256;
  const int brow = min(bz * 128 + 32 * rb + (lane & 31), B - 1), kh = lane >> 5;
  u32x4 aq[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) aq[ks] = *(const u32x4*)(q + ((int64_t)brow * H + h) * 128 + 16 * ks + 8 * kh);
  u32x4 wv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = tid + 256 * i, row = c >> 5, ch = c & 31;
    wv[i] = *(const u32x4*)(wsrc + row * 512 + ch * 8);
  }
  asm volatile("" ::: "memory");   // keeps every load above issued before the first store below
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = tid + 256 * i, row = c >> 5, ch = c & 31;
    *(u32x4*)(&Ws[row * kAbsStride + ch * 8]) = wv[i];
  }
  __syncthreads();
  if (rb >= nrb) return;
  const int G = lane >> 4, r4 = (lane & 15) >> 2, q4 = lane & 3;
  auto column_block = [&](int cb) __attribute__((always_inline)) -> f32x16 {
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
    return acc;
  };
  // lane l holds column l & 31 of rows 8 (v >> 2) + 4 (l >> 5) + (v & 3) of a block.  With a
  // 16-byte aligned output (STG) the pair of blocks (cb, cb + 1) goes through this wave's staging
  // rows and leaves as 16-byte pieces of 128-byte output rows, eight rows per store instruction;
  // otherwise each lane stores its bf16 values one by one.
  uint8_t* stg = ostg[STG ? wave : 0];
  auto store_pair = [&](const f32x16& acc1, const f32x16& acc2, int cb) __attribute__((always_inline)) {
    if constexpr (!STG) {
      uint16_t* ocol = out + (int64_t)h * 512 + half * 256 + 32 * cb + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int b = bz * 128 + 32 * rb + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (b < B) {
          ocol[(int64_t)b * H * 512] = (uint16_t)(pack_bf16x2(acc1[v], 0.f) & 0xffffu);
          ocol[(int64_t)b * H * 512 + 32] = (uint16_t)(pack_bf16x2(acc2[v], 0.f) & 0xffffu);
        }
      }
      return;
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      *(uint16_t*)(stg + row * 144 + 2 * (lane & 31)) = (uint16_t)(pack_bf16x2(acc1[v], 0.f) & 0xffffu);
      *(uint16_t*)(stg + row * 144 + 64 + 2 * (lane & 31)) = (uint16_t)(pack_bf16x2(acc2[v], 0.f) & 0xffffu);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = 8 * q + (lane >> 3), b = bz * 128 + 32 * rb + row;
      const u32x4 piece = *(const u32x4*)(stg + row * 144 + 16 * (lane & 7));
      if (b < B) *(u32x4*)(out + ((int64_t)b * H + h) * 512 + half * 256 + 32 * cb + 8 * (lane & 7)) = piece;
    }
  };
#pragma unroll 1
  for (int cb = cfirst; cb < cfirst + cpw; cb += 2) {
    const f32x16 acc1 = column_block(cb);
    const f32x16 acc2 = column_block(cb + 1);
    store_pair(acc1, acc2, cb);
  }
}

// ---------------------------------------------------------------------------------------------
// absorb, small batch (B <= 4): a plain stream over W_UK (no reuse to exploit).  Grid (H, 8
// column eighths), 256 threads.  Thread t owns columns 8 (t % 8) .. +7 of its eighth and rows
// t / 8 + 32 j (j = 0..3): four 16-byte weight loads in flight per thread, issued first.  The
// NB query rows of head h come through LDS; the 32 row groups are summed through LDS.
// ---------------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void k_absorb_gemv(const uint16_t* __restrict__ q, const uint16_t* __restrict__ w,
                                                     uint16_t* __restrict__ out, int B, int H) {
  constexpr int kRed = 64 + 4;
  __shared__ __attribute__((aligned(16))) float red[32 * NB * kRed];
  __shared__ __attribute__((aligned(16))) uint16_t qs[NB][128];
  const int h = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int cg = tid & 7, rg = tid >> 3;
  const uint16_t* wp = w + ((int64_t)h * 128 + rg) * 512 + part * 64 + cg * 8;
  u32x4 wv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wv[j] = *(const u32x4*)(wp + (int64_t)j * 32 * 512);
  if (tid < 16 * NB) {
    const int b = tid >> 4;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (b < B) v = *(const u32x4*)(q + ((int64_t)b * H + h) * 128 + 8 * (tid & 15));
    *(u32x4*)&qs[b][8 * (tid & 15)] = v;
  }
  __syncthreads();
  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[b][c] = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float qv[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) qv[b] = bf16_bits_to_f32(qs[b][rg + 32 * j]);
#pragma unroll
    for (int c2 = 0; c2 < 4; ++c2) {
      const float w0 = __uint_as_float(wv[j][c2] << 16), w1 = __uint_as_float(wv[j][c2] & 0xffff0000u);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        acc[b][2 * c2] = fmaf(qv[b], w0, acc[b][2 * c2]);
        acc[b][2 * c2 + 1] = fmaf(qv[b], w1, acc[b][2 * c2 + 1]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    float* r = &red[(rg * NB + b) * kRed + cg * 8];
    *(float4*)r = make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
    *(float4*)(r + 4) = make_float4(acc[b][4], acc[b][5], acc[b][6], acc[b][7]);
  }
  __syncthreads();
  for (int o = tid; o < NB * 64; o += 256) {
    const int b = o >> 6, col = o & 63;
    if (b >= B) break;
    float v = 0.f;
#pragma unroll
    for (int g = 0; g < 32; ++g) v += red[(g * NB + b) * kRed + col];
    out[((int64_t)b * H + h) * 512 + part * 64 + col] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
  }
}

hipError_t launch_absorb_bf16(const void* q, const void* w, void* out, int B, int H, hipStream_t s) {
  if (B <= 4) {
    const dim3 grid(H, 8);
    if (B == 1)
      hipLaunchKernelGGL(k_absorb_gemv<1>, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w,
                         (uint16_t*)out, B, H);
    else if (B == 2)
      hipLaunchKernelGGL(k_absorb_gemv<2>, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w,
                         (uint16_t*)out, B, H);
    else
      hipLaunchKernelGGL(k_absorb_gemv<4>, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w,
                         (uint16_t*)out, B, H);
    return hipGetLastError();
  }
  dim3 grid(H, 2, (B + 127) / 128);
  if (((uintptr_t)out & 15) == 0)
    hipLaunchKernelGGL(k_absorb_bf16<true>, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w,
                       (uint16_t*)out, B, H);
  else
    hipLaunchKernelGGL(k_absorb_bf16<false>, grid, dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)w,
                       (uint16_t*)out, B, H);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// uv.  Grid (H, ceil(B/32), RS), 256 threads.  With RS = 1 the workgroup computes all 128 output
// rows of head h for batch rows b0 .. b0+31: wave w takes output rows 32w .. 32w+31.  With RS = 2
// (fewer workgroups than CUs otherwise) workgroup (h, ., r) computes output rows 64r .. 64r+63:
// waves w and w + 2 take rows 64r + 32w .. +31 over the two halves of the k range, and wave w + 2
// hands its sum to wave w through LDS.  Operand A = o_lat rows,
// fp32 split into bf16 hi + bf16 lo (the product keeps ~16 mantissa bits of o_lat); the split is
// done once per workgroup into LDS (32 rows x 512 columns x 2 halves, 64 KiB), where every wave
// reads it.  Operand B = W_UV[h][i][k] rows straight from global memory (k contiguous).
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

constexpr int kUvRow = 1024 + 16;   // LDS bytes per o_lat row and half (512 bf16 + pad)

template <int RS>
__global__ __launch_bounds__(256) void k_uv_bf16(const float* __restrict__ o_lat, const uint16_t* __restrict__ w,
                                                 float* __restrict__ out, int B, int H) {
  constexpr int KS = 32 / RS;   // k-steps per wave
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][32 * kUvRow];   // [hi/lo][row][k]
  __shared__ f32x4 red[RS == 2 ? 2 * 4 * 64 : 1];   // RS = 2: the k-half partials of waves 2 and 3
  const int h = blockIdx.x, bz = blockIdx.y, rs = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b0 = bz * 32;
  const int i0 = RS == 1 ? wave * 32 : 64 * rs + 32 * (wave & 1);
  const int k0 = RS == 1 ? 0 : KS * (wave >> 1);
  const int kh = lane >> 5;
  // this wave's 32 weight rows for its KS k-steps, loaded before anything waits (one memory
  // round trip for the whole workgroup, together with the o_lat rows below)
  const uint16_t* wr = w + ((int64_t)h * 128 + i0 + (lane & 31)) * 512 + 8 * kh + 16 * k0;
  u32x4 bw[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) bw[ks] = *(const u32x4*)(wr + 16 * ks);
  // stage: thread t converts 8 consecutive columns (8 (t % 64) ..) of rows t / 64 + 4 j
  float4 xv[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 6) + 4 * j;
    // rows past B read the last token (their outputs are not stored)
    const float* src = o_lat + ((int64_t)min(b0 + r, B - 1) * H + h) * 512 + 8 * lane;
    xv[2 * j] = *(const float4*)src;
    xv[2 * j + 1] = *(const float4*)(src + 4);
  }
  asm volatile("" ::: "memory");   // keeps every load above issued before the first store below
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = (tid >> 6) + 4 * j;
    u32x4 hi, lo;
    split_hi_lo(xv[2 * j], xv[2 * j + 1], hi, lo);
    *(u32x4*)(xs[0] + r * kUvRow + 16 * lane) = hi;
    *(u32x4*)(xs[1] + r * kUvRow + 16 * lane) = lo;
  }
  __syncthreads();
  const uint8_t* ahi = xs[0] + (lane & 31) * kUvRow + 16 * kh + 32 * k0;
  const uint8_t* alo = xs[1] + (lane & 31) * kUvRow + 16 * kh + 32 * k0;
  f32x16 acc = {}, acc2 = {};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 hi = *(const u32x4*)(ahi + 32 * ks);
    const u32x4 lo = *(const u32x4*)(alo + 32 * ks);
    acc = mfma32x32x16(hi, bw[ks], acc);
    acc2 = mfma32x32x16(lo, bw[ks], acc2);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v) acc[v] += acc2[v];
  if constexpr (RS == 2) {
    // waves 2 and 3 hand their half of the k range to waves 0 and 1 (same output rows)
    if (wave >= 2) {
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        red[((wave - 2) * 4 + v4) * 64 + lane] = f32x4{acc[4 * v4], acc[4 * v4 + 1], acc[4 * v4 + 2], acc[4 * v4 + 3]};
    }
    __syncthreads();
    if (wave >= 2) return;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const f32x4 o = red[(wave * 4 + v4) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * v4 + e] += o[e];
    }
  }
  float* orow = out + (int64_t)h * 128 + i0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int b = b0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    if (b < B) orow[(int64_t)b * H * 128] = acc[v];
  }
}

// ---------------------------------------------------------------------------------------------
// uv, small batch (B <= 4): a plain stream over W_UV in fp32 arithmetic.  Grid (H, 4 quarters of
// the 128 output rows), 256 threads; wave v takes rows 32 q + 8 v .. +7 and lane l holds columns
// 8 l .. 8 l + 7 of those rows and of o_lat.  The NB x 8 dot products are summed over the 64 lanes
// by a halving exchange: at each step a lane keeps one half of its values and adds the partner's
// copy of that half, so K values need K - 1 + log2(64 / K) exchanges instead of 6 K.
// ---------------------------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void k_uv_gemv(const float* __restrict__ o_lat, const uint16_t* __restrict__ w,
                                                 float* __restrict__ out, int B, int H) {
  constexpr int K = NB * 8;                      // values per lane: index b * 8 + r
  constexpr int LK = NB == 1 ? 3 : NB == 2 ? 4 : 5;
  const int h = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i0 = blockIdx.y * 32 + wave * 8;
  const uint16_t* wp = w + ((int64_t)h * 128 + i0) * 512 + 8 * lane;
  u32x4 wv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) wv[r] = *(const u32x4*)(wp + r * 512);
  float x[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    // tokens past B read the last one (all loads in flight together; their outputs are not stored)
    const float* xp = o_lat + ((int64_t)min(b, B - 1) * H + h) * 512 + 8 * lane;
    const float4 x0 = *(const float4*)xp, x1 = *(const float4*)(xp + 4);
    x[b][0] = x0.x; x[b][1] = x0.y; x[b][2] = x0.z; x[b][3] = x0.w;
    x[b][4] = x1.x; x[b][5] = x1.y; x[b][6] = x1.z; x[b][7] = x1.w;
  }
  float v[K];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float s = 0.f;
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        s = fmaf(x[b][2 * c2], __uint_as_float(wv[r][c2] << 16), s);
        s = fmaf(x[b][2 * c2 + 1], __uint_as_float(wv[r][c2] & 0xffff0000u), s);
      }
      v[b * 8 + r] = s;
    }
  // halving exchange over lane bits 5, 4, ...: afterwards lane l holds value (l >> (6 - LK)) & (K - 1)
  const float t = lane_sum_halving<K>(v, lane);
  const int idx = (lane >> (6 - LK)) & (K - 1);
  const int b = idx >> 3, r = idx & 7;
  if ((lane & ((64 >> LK) - 1)) == 0 && b < B) out[((int64_t)b * H + h) * 128 + i0 + r] = t;
}

// ---------------------------------------------------------------------------------------------
// Combine + uv, small batch (B <= 4, d_h = 128, d_c = 512, row-major workspace).
// Grid (H, 4), 256 threads.  Workgroup (h, q) owns latent columns 128q .. 128q+127 of head h, so
// each one reads a quarter of the head's partial rows and of W_UV[h] (the per-CU load rate, not
// HBM, bounds this pass at small batch, so the work is spread over four times as many CUs):
//   1. per sequence b: the log-sum-exp merge of the segments' (m, l) and of the quarter's partial
//      columns into o_lat[b,h, quarter]: eight groups of 32 threads (one float4 column each) take
//      every eighth segment and are summed through LDS in group order; written to o_latent
//      (lse by the q = 0 workgroup);
//   2. y_q[b,i] = sum over the quarter's columns c of W_UV[h][i][c] o_lat[b,h,c], i = 0..127
//      (thread pair 2i, 2i+1 takes 64 columns each), stored to the workspace;
//   3. the last of the four workgroups of head h to finish adds the four quarters in the order
//      q = 0..3 and writes out[b,h,:].  The quarters are exchanged with device-coherent stores and
//      loads (agent-scope atomic accesses: they reach the coherence point without the whole-cache
//      write-back and invalidate of a device-scope fence), and the stores have completed
//      (s_waitcnt) before a device-scope counter is raised; the partial pass zeroes the counter
//      and the last workgroup resets it.  The summation order is fixed, so the result does not
//      depend on which workgroup finishes last.
// ---------------------------------------------------------------------------------------------
template <int NB, bool BF>
__device__ __forceinline__ void combine_uv(const CombineArgs& a, const uint16_t* __restrict__ w,
                                           float* __restrict__ out) {
  constexpr int kW = 1024;   // segment weights kept in LDS
  __shared__ __attribute__((aligned(16))) float olq[NB][128];
  __shared__ float4 part[7][32];
  __shared__ float wts[kW];
  __shared__ float rr[4];
  __shared__ int last_s;
  const int h = blockIdx.x, q = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int H = a.H;
  const int NT = a.ws_prefix[a.B];
  const int c4 = tid & 31, sg = tid >> 5;
  const int64_t sstride = (int64_t)H * 512;
  u32x4 wv[8];   // W_UV[h][tid >> 1][128q + 64 (tid & 1) .. +63], loaded after the first partial rows
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= a.B) break;
    const int Pb = a.ws_prefix[b], Pb1 = a.ws_prefix[b + 1];
    float* orow = a.o_latent + ((int64_t)b * H + h) * 512 + 128 * q;
    const bool empty = Pb1 == Pb;
    const int Wp = max(1, min(a.W, NT));
    const int w0 = empty ? 0 : (int)(((int64_t)(Pb + 1) * Wp + NT - 1) / NT) - 1;   // owner of tile t: ceil((t+1)Wp/NT)-1
    const int w1 = empty ? -1 : (int)(((int64_t)Pb1 * Wp + NT - 1) / NT) - 1;
    const int nseg = w1 - w0 + 1;
    const float2* ml = (const float2*)(a.ws_ml + ((int64_t)(w0 + b) * H + h) * 2);   // segment s at ml[s H]
    const int64_t src = ((int64_t)(w0 + b) * H + h) * 512 + 128 * q + 4 * c4;   // element + s H 512
    const float2 q0 = tid < nseg ? ml[(int64_t)tid * H] : make_float2(-INFINITY, 0.f);
    // the first 64 segments (8 per thread), all loads in flight together: segments past nseg read
    // the last one (weight 0 below), where a conditional or looped load would be waited on before
    // the next one is issued
    constexpr int kPre = 8;
    float4 x[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int su = min(sg + 8 * u, max(nseg - 1, 0));
      x[u] = load_part4<BF>(a.ws_acc, src + su * sstride);
    }
    if (b == 0) {
      const uint16_t* wp = w + ((int64_t)h * 128 + (tid >> 1)) * 512 + 128 * q + 64 * (tid & 1);
#pragma unroll
      for (int k = 0; k < 8; ++k) wv[k] = *(const u32x4*)(wp + 8 * k);
    }
    if (empty) {
      if (sg == 0) {
        *(float4*)&olq[b][4 * c4] = make_float4(0.f, 0.f, 0.f, 0.f);
        *(float4*)(orow + 4 * c4) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (a.lse && q == 0 && tid == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
      continue;
    }
    float mloc = q0.x;
    for (int s = tid + 256; s < nseg; s += 256) mloc = fmaxf(mloc, ml[(int64_t)s * H].x);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, d, 64));
    if (lane == 0) rr[wave] = mloc;
    __syncthreads();
    const float M = fmaxf(fmaxf(rr[0], rr[1]), fmaxf(rr[2], rr[3]));
    __syncthreads();
    float lloc = 0.f;
    for (int s = tid; s < nseg; s += 256) {
      const float2 mls = s == tid ? q0 : ml[(int64_t)s * H];
      const float f = exp2f(mls.x - M);
      if (s < kW) wts[s] = f;
      lloc += f * mls.y;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) lloc += __shfl_xor(lloc, d, 64);
    if (lane == 0) rr[wave] = lloc;
    __syncthreads();
    const float Ls = (rr[0] + rr[1]) + (rr[2] + rr[3]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int su = sg + 8 * u;
      const float f = su < nseg ? wts[su] : 0.f;
      o.x = fmaf(f, x[u].x, o.x);
      o.y = fmaf(f, x[u].y, o.y);
      o.z = fmaf(f, x[u].z, o.z);
      o.w = fmaf(f, x[u].w, o.w);
    }
    for (int s = sg + 8 * kPre; s < nseg; s += 8) {
      const float4 xs = load_part4<BF>(a.ws_acc, src + s * sstride);
      const float f = s < kW ? wts[s] : exp2f(ml[(int64_t)s * H].x - M);
      o.x = fmaf(f, xs.x, o.x);
      o.y = fmaf(f, xs.y, o.y);
      o.z = fmaf(f, xs.z, o.z);
      o.w = fmaf(f, xs.w, o.w);
    }
    if (sg > 0) part[sg - 1][c4] = o;
    __syncthreads();
    if (sg == 0) {
#pragma unroll
      for (int g = 0; g < 7; ++g) {
        const float4 u = part[g][c4];
        o.x += u.x;
        o.y += u.y;
        o.z += u.z;
        o.w += u.w;
      }
      const float inv = 1.f / Ls;
      const float4 r = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
      *(float4*)&olq[b][4 * c4] = r;
      *(float4*)(orow + 4 * c4) = r;
    }
    if (a.lse && q == 0 && tid == 0) a.lse[(int64_t)b * H + h] = (M + log2f(Ls)) * 0.69314718055994530942f;
    __syncthreads();   // part / rr / wts are reused by the next sequence
  }
  __syncthreads();
  // 2. this quarter's share of out[b, h, i], i = tid >> 1: 64 columns per thread, pair sum
  float* yq = a.ws_uv + (int64_t)h * 4 * 128;   // [b][h][q][i]
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    if (b >= a.B) break;
    const float* xo = &olq[b][64 * (tid & 1)];
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 xa = *(const float4*)(xo + 8 * k), xb = *(const float4*)(xo + 8 * k + 4);
      acc0 = fmaf(xa.x, __uint_as_float(wv[k][0] << 16), acc0);
      acc1 = fmaf(xa.y, __uint_as_float(wv[k][0] & 0xffff0000u), acc1);
      acc0 = fmaf(xa.z, __uint_as_float(wv[k][1] << 16), acc0);
      acc1 = fmaf(xa.w, __uint_as_float(wv[k][1] & 0xffff0000u), acc1);
      acc0 = fmaf(xb.x, __uint_as_float(wv[k][2] << 16), acc0);
      acc1 = fmaf(xb.y, __uint_as_float(wv[k][2] & 0xffff0000u), acc1);
      acc0 = fmaf(xb.z, __uint_as_float(wv[k][3] << 16), acc0);
      acc1 = fmaf(xb.w, __uint_as_float(wv[k][3] & 0xffff0000u), acc1);
    }
    float t = acc0 + acc1;
    t += __shfl_xor(t, 1, 64);
    // device-coherent store (agent-scope atomic store: written through to the coherence point,
    // so no cache write-back is needed before the counter below is raised)
    if ((tid & 1) == 0)
      __hip_atomic_store(yq + (int64_t)b * H * 512 + q * 128 + (tid >> 1), t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // 3. publish: every store of this workgroup has completed before the counter is raised; the
  // last workgroup of head h reads the four quarters with device-coherent loads and adds them in
  // order q = 0..3
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) last_s = __hip_atomic_fetch_add(a.ws_cnt + h, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 3;
  __syncthreads();
  if (!last_s) return;
  if (tid < 128) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b >= a.B) break;
      float* y = yq + (int64_t)b * H * 512 + tid;
      float yv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) yv[k] = __hip_atomic_load(y + 128 * k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      out[((int64_t)b * H + h) * 128 + tid] = ((yv[0] + yv[1]) + yv[2]) + yv[3];
    }
  }
  if (tid == 0) __hip_atomic_store(a.ws_cnt + h, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// the partial sums are float or bf16, as the partial pass recorded after the tile prefix sums
template <int NB>
__global__ __launch_bounds__(256) void k_combine_uv(CombineArgs a, const uint16_t* __restrict__ w,
                                                    float* __restrict__ out) {
  if (a.ws_prefix[a.B + 1] == kPartBF16)
    combine_uv<NB, true>(a, w, out);
  else
    combine_uv<NB, false>(a, w, out);
}

hipError_t launch_combine_uv(const CombineArgs& a, const void* w, float* out, hipStream_t s) {
  const dim3 grid(a.H, 4);
  if (a.B == 1)
    hipLaunchKernelGGL(k_combine_uv<1>, grid, dim3(256), 0, s, a, (const uint16_t*)w, out);
  else if (a.B == 2)
    hipLaunchKernelGGL(k_combine_uv<2>, grid, dim3(256), 0, s, a, (const uint16_t*)w, out);
  else
    hipLaunchKernelGGL(k_combine_uv<4>, grid, dim3(256), 0, s, a, (const uint16_t*)w, out);
  return hipGetLastError();
}

hipError_t launch_uv_bf16(const float* o_lat, const void* w, float* out, int B, int H, hipStream_t s) {
  if (B <= 4) {
    const dim3 grid(H, 4);
    if (B == 1)
      hipLaunchKernelGGL(k_uv_gemv<1>, grid, dim3(256), 0, s, o_lat, (const uint16_t*)w, out, B, H);
    else if (B == 2)
      hipLaunchKernelGGL(k_uv_gemv<2>, grid, dim3(256), 0, s, o_lat, (const uint16_t*)w, out, B, H);
    else
      hipLaunchKernelGGL(k_uv_gemv<4>, grid, dim3(256), 0, s, o_lat, (const uint16_t*)w, out, B, H);
    return hipGetLastError();
  }
  // with fewer workgroups than CUs, the output rows of a head are split over two workgroups, each
  // wave pair taking half of the k range (half the weight bytes per CU)
  const int nbz = (B + 31) / 32;
  if ((int64_t)H * nbz < 256) {
    hipLaunchKernelGGL(k_uv_bf16<2>, dim3(H, nbz, 2), dim3(256), 0, s, o_lat, (const uint16_t*)w, out, B, H);
  } else {
    hipLaunchKernelGGL(k_uv_bf16<1>, dim3(H, nbz, 1), dim3(256), 0, s, o_lat, (const uint16_t*)w, out, B, H);
  }
  return hipGetLastError();
}

}  // namespace mla
