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
// Partial pass, fp32 cache, any d_c <= 1024 and d_R <= 256.  Grid (W, H): workgroup (w, h) walks
// the segments of tile range w for head h, running an online softmax over 32-token tiles (8
// threads per token for the score, one column per thread for the weighted sum), and writes the
// partial (m, l, acc) into slot w + b.  Scores are kept in log2 units (s * scale * log2 e).
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
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_prefix[i] = P[i];
    if (threadIdx.x == 0) a.ws_prefix[a.B + 1] = kPartF32;
    for (int i = threadIdx.x; i < a.H; i += blockDim.x) a.ws_cnt[i] = 0;
  }
  const int NT = P[a.B];
  const int Wp = min(a.W, NT);
  const int w = blockIdx.x, h = blockIdx.y;
  if (w >= Wp) return;
  const int t_begin = (int)((int64_t)w * NT / Wp);
  const int t_end = (int)((int64_t)(w + 1) * NT / Wp);
  const int tid = threadIdx.x;
  const int tj = tid >> 3, tr = tid & 7;   // score phase: token tj of the tile, lane tr of its 8
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
    __syncthreads();
    for (int k = tid; k < d_c; k += blockDim.x) qs[k] = qa[((int64_t)b * H + h) * d_c + k];
    for (int k = tid; k < d_R; k += blockDim.x) qs[d_c + k] = qr[((int64_t)b * H + h) * d_R + k];
    __syncthreads();
    float m = -INFINITY, l = 0.f;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = tok_lo; t0 < tok_hi; t0 += kTile) {
      const int n = min(kTile, tok_hi - t0);
      // score of token tj: 8 lanes split the dot product, then a 3-step exchange
      float sc = 0.f;
      if (tj < n) {
        const float* cr = row_f32(lat, a.lat_sb, a.lat_st, a.block_table, a.page_size, a.max_pages, b, t0 + tj);
        const float* rr = row_f32(rope, a.rope_sb, a.rope_st, a.block_table, a.page_size, a.max_pages, b, t0 + tj);
        for (int k = tr; k < d_c; k += 8) sc = fmaf(qs[k], cr[k], sc);
        for (int k = tr; k < d_R; k += 8) sc = fmaf(qs[d_c + k], rr[k], sc);
      }
      sc += __shfl_xor(sc, 1, 64);
      sc += __shfl_xor(sc, 2, 64);
      sc += __shfl_xor(sc, 4, 64);
      if (tj < n && tr == 0) ss[tj] = sc * a.sl2;
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
    t = seg_end;
  }
}

hipError_t launch_partial_f32(const PartialArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_partial_f32, dim3(a.W, a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine pass: for (b, h) merge the partials of the segments of sequence b.
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  o = sum_s 2^(m_s - M) acc_s / L,
//   lse = (M + log2 L) * ln 2       (natural log).   No segment -> o = 0, lse = -inf.
// The segments of sequence b are the partial-pass workgroups w0..w1 whose tile ranges meet b's
// tiles (tile prefix sums left in the workspace by the partial pass, followed by the element
// type of its sums, float or bf16).
// Grid (H, B, ceil(d_c / 512)), 256 threads: the workgroup merges up to 512 columns of one row.
// The (m, l) pairs are reduced by the whole workgroup and the segment weights 2^(m_s - M) kept in
// LDS (the first kCombW of them); thread t takes float4 column group t % 128 and segments
// t / 128 + 2 i, sixteen loads in flight (the first sixteen issued before the reduction), and the
// two segment groups are summed through LDS.
// ---------------------------------------------------------------------------------------------
constexpr int kCombW = 1024;

__device__ __forceinline__ float block_reduce256(float v, bool is_max, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float u = __shfl_xor(v, d, 64);
    v = is_max ? fmaxf(v, u) : v + u;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = is_max ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

template <bool BF>
__device__ __forceinline__ void combine_rows(const CombineArgs& a, float4* red, float* wts, float* rr) {
  constexpr int NU = 16;   // segments per thread loaded before the (m, l) reduction (32 per row)
  const int h = blockIdx.x, b = blockIdx.y, cq = blockIdx.z, tid = threadIdx.x;
  const int d_c = a.d_c, H = a.H;
  const int c4 = tid & 127, sg = tid >> 7;
  const int col = cq * 512 + 4 * c4;
  const int Pb = a.ws_prefix[b], Pb1 = a.ws_prefix[b + 1], NT = a.ws_prefix[a.B];
  float* out = a.o_latent + ((int64_t)b * H + h) * d_c;
  if (Pb1 == Pb) {
    if (sg == 0 && col < d_c) *(float4*)(out + col) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse && tid == 0 && cq == 0) a.lse[(int64_t)b * H + h] = -INFINITY;
    return;
  }
  const int Wp = min(a.W, NT);
  // workgroup that owns tile t: ceil((t+1)*Wp/NT) - 1
  const int w0 = (int)(((int64_t)(Pb + 1) * Wp + NT - 1) / NT) - 1;
  const int w1 = (int)(((int64_t)Pb1 * Wp + NT - 1) / NT) - 1;
  const int nseg = w1 - w0 + 1;
  const float2* ml = (const float2*)(a.ws_ml + ((int64_t)(w0 + b) * H + h) * 2);   // segment s at ml + H s
  const int64_t e0 = ((int64_t)(w0 + b) * H + h) * d_c + col;   // segment s at element e0 + H d_c s
  const int64_t astride = (int64_t)H * d_c;
  // Thread t takes segments t / 128 + 2 u.  Its first NU do not depend on the weights: their loads
  // go out before the (m, l) reduction, so that both wait on one memory round trip.  Segments
  // past nseg read the last one and get weight 0 (a load per remaining segment would be waited on
  // one by one; skipping them behind a branch measured slower).
  const bool has_col = col < d_c;
  float4 v0[NU];
  if (has_col) {
#pragma unroll
    for (int u = 0; u < NU; ++u) v0[u] = load_part4<BF>(a.ws_acc, e0 + min(sg + 2 * u, nseg - 1) * astride);
  }
  // (m, l) of segment tid is kept in registers between the two reductions (segments past 256,
  // a rare case, are read again)
  const float2 ml_t = tid < nseg ? ml[(int64_t)tid * H] : make_float2(-INFINITY, 0.f);
  float mloc = ml_t.x;
  for (int s = tid + 256; s < nseg; s += 256) mloc = fmaxf(mloc, ml[(int64_t)s * H].x);
  const float M = block_reduce256(mloc, true, rr);
  float lloc = 0.f;
  for (int s = tid; s < nseg; s += 256) {
    const float2 v = s == tid ? ml_t : ml[(int64_t)s * H];
    const float f = exp2f(v.x - M);
    if (s < kCombW) wts[s] = f;
    lloc += f * v.y;
  }
  const float Ls = block_reduce256(lloc, false, rr);   // its barriers also publish wts
  auto weight = [&](int s) -> float { return s < kCombW ? wts[s] : exp2f(ml[(int64_t)s * H].x - M); };

  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (has_col) {
    auto accumulate = [&](const float4 (&v)[NU], int s) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const float f = s + 2 * u < nseg ? weight(s + 2 * u) : 0.f;
        o.x = fmaf(f, v[u].x, o.x);
        o.y = fmaf(f, v[u].y, o.y);
        o.z = fmaf(f, v[u].z, o.z);
        o.w = fmaf(f, v[u].w, o.w);
      }
    };
    accumulate(v0, sg);
    // further passes (more than 32 segments), all NU loads in flight together
    for (int s = sg + 2 * NU; s < nseg; s += 2 * NU) {
      float4 v[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) v[u] = load_part4<BF>(a.ws_acc, e0 + min(s + 2 * u, nseg - 1) * astride);
      accumulate(v, s);
    }
  }
  if (sg == 1) red[c4] = o;
  __syncthreads();
  if (sg == 0 && has_col) {
    const float4 u = red[c4];
    const float inv = 1.f / Ls;
    *(float4*)(out + col) = make_float4((o.x + u.x) * inv, (o.y + u.y) * inv, (o.z + u.z) * inv, (o.w + u.w) * inv);
  }
  if (a.lse && tid == 0 && cq == 0) a.lse[(int64_t)b * H + h] = (M + log2f(Ls)) * 0.69314718055994530942f;
}

__global__ __launch_bounds__(256) void k_combine_rows(CombineArgs a) {
  __shared__ float4 red[128];
  __shared__ float wts[kCombW];
  __shared__ float rr[4];
  if (a.ws_prefix[a.B + 1] == kPartBF16)
    combine_rows<true>(a, red, wts, rr);
  else
    combine_rows<false>(a, red, wts, rr);
}

constexpr int kCombWB = 128;   // segments whose weights are kept in LDS (the rest are recomputed)

// Combine for batches wide enough to fill the chip with one workgroup per (32-head block,
// sequence): grid (H/32, B), 256 threads.  The (m, l) reduction is done once per head block; the
// block's 32 partial rows are contiguous per segment (64 KiB as float, 32 KiB as bf16); thread t
// reads groups of four sums t + 256 i (i = 0..15: head 2i + t / 128, columns 4 (t % 128) ..),
// sixteen loads in flight, the first segment's during the reduction.  d_c must be 512.
template <bool BF>
__device__ __forceinline__ void combine_heads(const CombineArgs& a, float (*red)[32], float* Ms, float* Lsum,
                                              float (*wts)[32]) {
  constexpr int NI = 16;
  const int hb = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int H = a.H, d_c = a.d_c;
  const int hr = tid & 31, g = tid >> 5;                       // (m, l) phase: head hr, group g
  const int c4 = tid & 127, r0 = tid >> 7;                     // accumulate phase: heads r0 + 2i
  float* out = a.o_latent + ((int64_t)b * H + hb * 32) * d_c + 4 * c4;   // + (r0 + 2i) d_c
  const int Pb = a.ws_prefix[b], Pb1 = a.ws_prefix[b + 1], NT = a.ws_prefix[a.B];
  if (Pb1 == Pb) {
#pragma unroll
    for (int i = 0; i < NI; ++i) *(float4*)(out + (r0 + 2 * i) * d_c) = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse && tid < 32) a.lse[(int64_t)b * H + hb * 32 + tid] = -INFINITY;
    return;
  }
  const int Wp = min(a.W, NT);
  const int w0 = (int)(((int64_t)(Pb + 1) * Wp + NT - 1) / NT) - 1;   // owner of tile t: ceil((t+1)Wp/NT)-1
  const int w1 = (int)(((int64_t)Pb1 * Wp + NT - 1) / NT) - 1;
  const int nseg = w1 - w0 + 1;
  const float2* ml = (const float2*)(a.ws_ml + ((int64_t)(w0 + b) * H + hb * 32) * 2);   // (s, head) at ml[s H + head]
  const int64_t sstride = (int64_t)H * d_c;   // elements per slot
  const int64_t src = ((int64_t)(w0 + b) * H + hb * 32) * d_c + 4 * c4;   // element + (r0 + 2i) d_c + s sstride
  // the first segment's rows do not depend on the weights: load them during the (m, l) reduction
  float4 x0[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) x0[i] = load_part4<BF>(a.ws_acc, src + (r0 + 2 * i) * d_c);
  // (m, l) of segment g is kept in registers between the two reductions
  const float2 ml_g = g < nseg ? ml[(int64_t)g * H + hr] : make_float2(-INFINITY, 0.f);
  float mloc = ml_g.x;
  for (int s = g + 8; s < nseg; s += 8) mloc = fmaxf(mloc, ml[(int64_t)s * H + hr].x);
  red[g][hr] = mloc;
  __syncthreads();
  if (tid < 32) {
    float m = red[0][tid];
#pragma unroll
    for (int i = 1; i < 8; ++i) m = fmaxf(m, red[i][tid]);
    Ms[tid] = m;
  }
  __syncthreads();
  {
    const float M = Ms[hr];
    float lloc = 0.f;
    for (int s = g; s < nseg; s += 8) {
      const float2 q = s == g ? ml_g : ml[(int64_t)s * H + hr];
      const float f = exp2f(q.x - M);
      if (s < kCombWB) wts[s][hr] = f;
      lloc += f * q.y;
    }
    red[g][hr] = lloc;
  }
  __syncthreads();
  if (tid < 32) {
    float t = red[0][tid];
#pragma unroll
    for (int i = 1; i < 8; ++i) t += red[i][tid];
    Lsum[tid] = t;
  }
  __syncthreads();
  float4 o[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float f = wts[0][r0 + 2 * i];
    o[i] = make_float4(f * x0[i].x, f * x0[i].y, f * x0[i].z, f * x0[i].w);
  }
  for (int s = 1; s < nseg; ++s) {
    float4 x[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) x[i] = load_part4<BF>(a.ws_acc, src + s * sstride + (r0 + 2 * i) * d_c);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = r0 + 2 * i;
      const float f = s < kCombWB ? wts[s][r] : exp2f(ml[(int64_t)s * H + r].x - Ms[r]);
      o[i].x = fmaf(f, x[i].x, o[i].x);
      o[i].y = fmaf(f, x[i].y, o[i].y);
      o[i].z = fmaf(f, x[i].z, o[i].z);
      o[i].w = fmaf(f, x[i].w, o[i].w);
    }
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const float inv = 1.f / Lsum[r0 + 2 * i];
    *(float4*)(out + (r0 + 2 * i) * d_c) = make_float4(o[i].x * inv, o[i].y * inv, o[i].z * inv, o[i].w * inv);
  }
  if (a.lse && tid < 32)
    a.lse[(int64_t)b * H + hb * 32 + tid] = (Ms[tid] + log2f(Lsum[tid])) * 0.69314718055994530942f;
}

__global__ __launch_bounds__(256) void k_combine_heads(CombineArgs a) {
  __shared__ float red[8][32];
  __shared__ float Ms[32], Lsum[32];
  __shared__ float wts[kCombWB][32];
  if (a.ws_prefix[a.B + 1] == kPartBF16)
    combine_heads<true>(a, red, Ms, Lsum, wts);
  else
    combine_heads<false>(a, red, Ms, Lsum, wts);
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.H % 32 == 0 && a.d_c == 512 && (int64_t)(a.H / 32) * a.B >= 256)
    hipLaunchKernelGGL(k_combine_heads, dim3(a.H / 32, a.B), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_combine_rows, dim3(a.H, a.B, (a.d_c + 511) / 512), dim3(256), 0, s, a);
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
