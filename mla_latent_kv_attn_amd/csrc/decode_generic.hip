// Generic-dimension fp32 kernels (VALU): query absorption, split-N partial pass, and the W_UV
// product, plus the combine pass shared with the MFMA path.  These serve small or unusual
// shapes; the DeepSeek-V3 shapes run on the MFMA kernels.
#include "mla_internal.h"

namespace mla {

// ---------------------------------------------------------------------------------------------
// q'[b,h,k] = sum_i W_UK[h,i,k] q_C[b,h,i]      (fold W_UK into the query)
// ---------------------------------------------------------------------------------------------
__global__ void k_absorb_f32(const float* __restrict__ q, const float* __restrict__ w, float* __restrict__ out,
                             int B, int H, int d_h, int d_c) {
  const int64_t total = (int64_t)B * H * d_c;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int k = (int)(idx % d_c);
    const int64_t bh = idx / d_c;
    const int h = (int)(bh % H);
    const float* qr = q + bh * d_h;
    const float* wr = w + (int64_t)h * d_h * d_c + k;
    float acc = 0.f;
    for (int i = 0; i < d_h; ++i) acc = fmaf(wr[(int64_t)i * d_c], qr[i], acc);
    out[idx] = acc;
  }
}

hipError_t launch_absorb_f32(const float* q, const float* w, float* out, int B, int H, int d_h, int d_c,
                             hipStream_t s) {
  int64_t total = (int64_t)B * H * d_c;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_absorb_f32, dim3(blocks), dim3(256), 0, s, q, w, out, B, H, d_h, d_c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Partial pass, fp32 cache, any d_c <= 1024 and d_R <= 256.  Workgroup w walks the segments of its
// tile range; for each head it runs an online softmax over 32-token tiles and writes the partial
// (m, l, acc) into slot w + b.  Scores are kept in log2 units (s * scale * log2 e).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ const float* row_f32(const float* base, int64_t sb, int64_t st, const int32_t* bt,
                                                int page_size, int max_pages, int b, int tok) {
  if (bt) {
    int p = bt[(int64_t)b * max_pages + tok / page_size];
    return base + (int64_t)p * sb + (int64_t)(tok % page_size) * st;
  }
  return base + (int64_t)b * sb + (int64_t)tok * st;
}

__global__ __launch_bounds__(256) void k_partial_f32(PartialArgs a) {
  __shared__ int P[kMaxB + 1];
  __shared__ int L[kMaxB];
  __shared__ float qs[1024 + 256];
  __shared__ float ss[kTile];
  build_tile_prefix(a.seq_lens, a.B, P, L);
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_prefix[i] = P[i];  // for the combine pass
  const int NT = P[a.B];
  const int Wp = min(a.W, NT);
  const int w = blockIdx.x;
  if (w >= Wp) return;
  const int t_begin = (int)((int64_t)w * NT / Wp);
  const int t_end = (int)((int64_t)(w + 1) * NT / Wp);
  const int tid = threadIdx.x;
  const int d_c = a.d_c, d_R = a.d_R, H = a.H;
  const float* qa = (const float*)a.q_abs;
  const float* qr = (const float*)a.q_R;
  const float* lat = (const float*)a.latent;
  const float* rope = (const float*)a.rope;

  int t = t_begin;
  while (t < t_end) {
    const int b = seq_of_tile(P, a.B, t);
    const int seg_end = min(t_end, P[b + 1]);
    const int tok_lo = (t - P[b]) * kTile;
    const int tok_hi = min(L[b], (seg_end - P[b]) * kTile);
    const int slot = w + b;
    for (int h = 0; h < H; ++h) {
      __syncthreads();
      for (int k = tid; k < d_c; k += blockDim.x) qs[k] = qa[((int64_t)b * H + h) * d_c + k];
      for (int k = tid; k < d_R; k += blockDim.x) qs[d_c + k] = qr[((int64_t)b * H + h) * d_R + k];
      __syncthreads();
      float m = -INFINITY, l = 0.f;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int t0 = tok_lo; t0 < tok_hi; t0 += kTile) {
        const int n = min(kTile, tok_hi - t0);
        if (tid < n) {
          const float* cr = row_f32(lat, a.lat_sb, a.lat_st, a.block_table, a.page_size, a.max_pages, b, t0 + tid);
          const float* rr = row_f32(rope, a.rope_sb, a.rope_st, a.block_table, a.page_size, a.max_pages, b, t0 + tid);
          float s = 0.f;
          for (int k = 0; k < d_c; ++k) s = fmaf(qs[k], cr[k], s);
          for (int k = 0; k < d_R; ++k) s = fmaf(qs[d_c + k], rr[k], s);
          ss[tid] = s * a.sl2;
        }
        __syncthreads();
        float mx = -INFINITY;
        for (int j = 0; j < n; ++j) mx = fmaxf(mx, ss[j]);
        const float m_new = fmaxf(m, mx);
        const float alpha = exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] *= alpha;
        for (int j = 0; j < n; ++j) {
          const float p = exp2f(ss[j] - m_new);
          l += p;
          const float* cr = row_f32(lat, a.lat_sb, a.lat_st, a.block_table, a.page_size, a.max_pages, b, t0 + j);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = tid + i * 256;
            if (k < d_c) acc[i] = fmaf(p, cr[k], acc[i]);
          }
        }
        m = m_new;
        __syncthreads();
      }
      const int64_t o = ((int64_t)slot * H + h);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = tid + i * 256;
        if (k < d_c) a.ws_acc[o * d_c + k] = acc[i];
      }
      if (tid == 0) {
        a.ws_ml[o * 2 + 0] = m;
        a.ws_ml[o * 2 + 1] = l;
      }
    }
    t = seg_end;
  }
}

hipError_t launch_partial_f32(const PartialArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_partial_f32, dim3(a.W), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine pass: for (b, h) merge the partials of the segments of sequence b.
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  o = sum_s 2^(m_s - M) acc_s / L,
//   lse = (M + log2 L) * ln 2       (natural log).   No segment -> o = 0, lse = -inf.
// Grid (H, B), 256 threads; thread t owns columns 2t + 512 j.  The segments of sequence b are the
// partial-pass workgroups w0..w1 whose tile ranges meet b's tiles (prefix sums from the partial pass).
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float u = __shfl_xor(v, d, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) v = is_max ? fmaxf(v, red[i]) : v + red[i];
  return v;
}

__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d_c = a.d_c, H = a.H;
  const int Pb = a.ws_prefix[b], Pb1 = a.ws_prefix[b + 1], NT = a.ws_prefix[a.B];
  float* out = a.o_latent + ((int64_t)b * H + h) * d_c;
  if (Pb1 == Pb) {
    for (int k = 2 * tid; k < d_c; k += 512) *(float2*)(out + k) = make_float2(0.f, 0.f);
    if (a.lse && tid == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  const int Wp = min(a.W, NT);
  // workgroup that owns tile t: ceil((t+1)*Wp/NT) - 1
  const int w0 = (int)(((int64_t)(Pb + 1) * Wp + NT - 1) / NT) - 1;
  const int w1 = (int)(((int64_t)Pb1 * Wp + NT - 1) / NT) - 1;
  const int nseg = w1 - w0 + 1;
  const float* ml = a.ws_ml + ((int64_t)(w0 + b) * H + h) * 2;   // segment s at ml + 2 H s
  const int64_t mstride = 2 * (int64_t)H;

  float M = -INFINITY;
  for (int s = tid; s < nseg; s += blockDim.x) M = fmaxf(M, ml[s * mstride]);
  M = block_reduce(M, true, red);
  float Ls = 0.f;
  for (int s = tid; s < nseg; s += blockDim.x) Ls += exp2f(ml[s * mstride] - M) * ml[s * mstride + 1];
  Ls = block_reduce(Ls, false, red);
  const float inv = 1.f / Ls;

  const float* acc0 = a.ws_acc + ((int64_t)(w0 + b) * H + h) * d_c;   // segment s at acc0 + H d_c s
  const int64_t astride = (int64_t)H * d_c;
  for (int k = 2 * tid; k < d_c; k += 512) {
    float2 o = make_float2(0.f, 0.f);
    int s = 0;
    for (; s + 4 <= nseg; s += 4) {
      float2 v[4];
      float f[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v[u] = *(const float2*)(acc0 + (s + u) * astride + k);
        f[u] = ml[(s + u) * mstride];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = exp2f(f[u] - M);
        o.x = fmaf(wgt, v[u].x, o.x);
        o.y = fmaf(wgt, v[u].y, o.y);
      }
    }
    for (; s < nseg; ++s) {
      const float2 v = *(const float2*)(acc0 + s * astride + k);
      const float wgt = exp2f(ml[s * mstride] - M);
      o.x = fmaf(wgt, v.x, o.x);
      o.y = fmaf(wgt, v.y, o.y);
    }
    o.x *= inv;
    o.y *= inv;
    *(float2*)(out + k) = o;
  }
  if (a.lse && tid == 0) a.lse[(int64_t)b * H + h] = (M + log2f(Ls)) * 0.69314718055994530942f;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(a.H, a.B), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// out[b,h,i] = sum_k W_UV[h,i,k] o_lat[b,h,k]   (generic; one wave per output row)
// ---------------------------------------------------------------------------------------------
template <bool BF16W>
__global__ __launch_bounds__(256) void k_uv_generic(const float* __restrict__ o_lat, const void* __restrict__ wv,
                                                    float* __restrict__ out, int B, int H, int d_h, int d_c) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)B * H * d_h;
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < rows; r += (int64_t)gridDim.x * 4) {
    const int i = (int)(r % d_h);
    const int64_t bh = r / d_h;
    const int h = (int)(bh % H);
    const float* x = o_lat + bh * d_c;
    float acc = 0.f;
    for (int k = lane; k < d_c; k += 64) {
      float wk;
      if (BF16W) wk = bf16_bits_to_f32(((const uint16_t*)wv)[((int64_t)h * d_h + i) * d_c + k]);
      else wk = ((const float*)wv)[((int64_t)h * d_h + i) * d_c + k];
      acc = fmaf(wk, x[k], acc);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc += __shfl_xor(acc, d, 64);
    if (lane == 0) out[r] = acc;
  }
}

hipError_t launch_uv_f32w(const float* o_lat, const float* w, float* out, int B, int H, int d_h, int d_c,
                          hipStream_t s) {
  int64_t rows = (int64_t)B * H * d_h;
  int blocks = (int)((rows + 3) / 4);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_uv_generic<false>, dim3(blocks), dim3(256), 0, s, o_lat, (const void*)w, out, B, H, d_h, d_c);
  return hipGetLastError();
}

hipError_t launch_uv_bf16w_generic(const float* o_lat, const void* w, float* out, int B, int H, int d_h, int d_c,
                                   hipStream_t s) {
  int64_t rows = (int64_t)B * H * d_h;
  int blocks = (int)((rows + 3) / 4);
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_uv_generic<true>, dim3(blocks), dim3(256), 0, s, o_lat, w, out, B, H, d_h, d_c);
  return hipGetLastError();
}

}  // namespace mla
