// Same-dimension comparison: plain multi-head attention decode with an explicit per-head K/V cache
// at the DeepSeek-V3 head sizes (keys d_k = 128 + 64 = 192, values d_v = 128).  Per token and layer
// it stores H (d_k + d_v) = 40,960 values against the latent path's d_c + d_R = 576
// ("Grouped-query and latent attention", section "Multi-head latent attention (MLA)"; "The
// Journey to Multi-Head Latent Attention", section "The KV cache -- and why it exists at all").
// The pages ask for comparisons at the same dimensions and warn that smaller caches do not by
// themselves mean proportionally faster decoding ("DeepSeek MLA: ...", section "Memory savings do
// not automatically equal latency savings"); this kernel turns the ratio into measured time.
//
// Caches are head-major, [B, H, cap, d] bf16: each (sequence, head) stream is contiguous, the most
// favourable layout for this path.  Nothing is shared between heads, so the work is a bandwidth-
// bound dot product per cached row: fp32 VALU, no MFMA.
//
// k_mha_partial: grid (W splits, H, B), 256 threads.  The 64-token tiles of sequence b are split
// evenly over the W workgroups of head h.  Wave v takes tokens 16v .. 16v+15 of every tile; lane l
// takes token l >> 2 and quarter l & 3 (48 key / 32 value components).  Each wave keeps its own
// online softmax (maximum, sum, 32-value accumulator per lane) in log2 units; at the end the
// lanes of a wave and then the four waves are merged, and the split's (m, l, acc[128]) is written.
// k_mha_combine: grid (H, B), 128 threads: the log-sum-exp merge of the W splits.
#include "rows_internal.h"

namespace mla {

namespace {
constexpr int kDk = 192, kDv = 128, kT = 64;

__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f[2 * c] = __uint_as_float(v[c] << 16);
    f[2 * c + 1] = __uint_as_float(v[c] & 0xffff0000u);
  }
}
}  // namespace

size_t mha_ws_bytes(int B, int H, int W) { return (size_t)B * H * W * (kDv + 2) * sizeof(float); }

__global__ __launch_bounds__(256) void k_mha_partial(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                                                     const uint16_t* __restrict__ vc, const int32_t* __restrict__ lens,
                                                     int H, int64_t cap, float sl2, int W, float* __restrict__ ws) {
  __shared__ float sm[4][2];
  __shared__ __attribute__((aligned(16))) float sacc[4][kDv];
  const int w = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane >> 2, qd = lane & 3;
  const int len = lens[b];
  const int ntile = (len + kT - 1) / kT;
  const int t0 = (int)((int64_t)w * ntile / W), t1 = (int)((int64_t)(w + 1) * ntile / W);
  const int64_t head = (int64_t)b * H + h;
  const uint16_t* kbase = kc + head * cap * kDk + 48 * qd;
  const uint16_t* vbase = vc + head * cap * kDv + 32 * qd;

  float qf[48];
  {
    const uint16_t* qp = q + head * kDk + 48 * qd;
#pragma unroll
    for (int i = 0; i < 6; ++i) unpack8(*(const u32x4*)(qp + 8 * i), qf + 8 * i);
  }
  float m_run = -INFINITY, l_run = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;

  auto load = [&](int tile, u32x4* kv, u32x4* vv) __attribute__((always_inline)) {
    const int tok = min(tile * kT + 16 * wave + r, max(len - 1, 0));
#pragma unroll
    for (int i = 0; i < 6; ++i) kv[i] = *(const u32x4*)(kbase + (int64_t)tok * kDk + 8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = *(const u32x4*)(vbase + (int64_t)tok * kDv + 8 * i);
  };
  u32x4 kv[6], vv[4];
  if (t0 < t1) load(t0, kv, vv);
  for (int tile = t0; tile < t1; ++tile) {
    float kf[48], vf[32];
#pragma unroll
    for (int i = 0; i < 6; ++i) unpack8(kv[i], kf + 8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) unpack8(vv[i], vf + 8 * i);
    if (tile + 1 < t1) load(tile + 1, kv, vv);   // next tile's rows in flight during this one
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 48; ++i) s = fmaf(qf[i], kf[i], s);
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    const bool valid = tile * kT + 16 * wave + r < len;
    s = valid ? s * sl2 : -INFINITY;
    float mx = s;
#pragma unroll
    for (int d = 4; d < 64; d <<= 1) mx = fmaxf(mx, __shfl_xor(mx, d, 64));
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) continue;               // no valid token in this wave's rows yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float p = __builtin_amdgcn_exp2f(s - m_new);
    m_run = m_new;
    l_run = l_run * alpha + (qd == 0 ? p : 0.f);     // one lane per token adds its weight
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = fmaf(p, vf[i], acc[i] * alpha);
  }
  // merge the 16 token lanes of the wave (same quarter), then the four waves
#pragma unroll
  for (int d = 4; d < 64; d <<= 1) {
    l_run += __shfl_xor(l_run, d, 64);
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] += __shfl_xor(acc[i], d, 64);
  }
  if (lane == 0) {
    sm[wave][0] = m_run;
    sm[wave][1] = l_run;
  }
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) *(float4*)&sacc[wave][32 * qd + i] = make_float4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
  }
  __syncthreads();
  if (t < kDv) {
    const float M = fmaxf(fmaxf(sm[0][0], sm[1][0]), fmaxf(sm[2][0], sm[3][0]));
    float L = 0.f, o = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float f = __builtin_amdgcn_exp2f(sm[v][0] - M);   // 0 for a wave with no valid token
        L = fmaf(f, sm[v][1], L);
        o = fmaf(f, sacc[v][t], o);
      }
    }
    float* dst = ws + (head * W + w) * (kDv + 2);
    dst[2 + t] = o;
    if (t == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

__global__ __launch_bounds__(128) void k_mha_combine(const float* __restrict__ ws, int H, int W,
                                                     float* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int64_t head = (int64_t)b * H + h;
  const float* src = ws + head * W * (kDv + 2);
  float M = -INFINITY;
  for (int w = 0; w < W; ++w) M = fmaxf(M, src[w * (kDv + 2)]);
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int w = 0; w < W; ++w) {
      const float* s = src + w * (kDv + 2);
      const float f = exp2f(s[0] - M);
      L = fmaf(f, s[1], L);
      o = fmaf(f, s[2 + t], o);
    }
  }
  out[head * kDv + t] = M == -INFINITY ? 0.f : o / L;
  if (lse && t == 0) lse[head] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * 0.69314718055994530942f;
}

hipError_t launch_mha(const void* q, const void* kc, const void* vc, const int32_t* lens, int B, int H, int64_t cap,
                      float scale, int W, float* ws, float* out, float* lse, hipStream_t s) {
  hipLaunchKernelGGL(k_mha_partial, dim3(W, H, B), dim3(256), 0, s, (const uint16_t*)q, (const uint16_t*)kc,
                     (const uint16_t*)vc, lens, H, cap, scale * 1.4426950408889634f, W, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mha_combine, dim3(H, B), dim3(128), 0, s, ws, H, W, out, lse);
  return hipGetLastError();
}

}  // namespace mla
