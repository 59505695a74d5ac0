// Projections around the attention core: y[b, n] = sum_k W[n, k] x[b, k] for every token b, with
// W bf16 [N, K] row-major (a weight matrix in column-vector form, y = W x).  They serve
//  * the query side ("Grouped-query and latent attention", section "Multi-head latent attention
//    (MLA)"): c_q = W_DQ h, then [q_C ; q_R] = [W_UQ ; W_QR] c_q with the rotary key's rotation
//    applied per head to the q_R rows (section "Why a separate rotary key");
//  * the absorbed query projection folded offline, q' = W_QK c_q ("The Journey to Multi-Head
//    Latent Attention", section "The absorption trick (the magic)");
//  * the output projection W_O, or its fold with W_UV ("Grouped-query and latent attention",
//    section "The absorption trick").
//
// For the few tokens of a decode step every weight byte is used B times, so the work is a
// stream of the weights from HBM.  Two kernels:
//  * k_proj_gemv (B <= 8): one workgroup (4 waves) per 8 rows of W over the whole of K.  K is
//    cut into 512-element chunks; wave w takes chunks w, w + 4, ...  Lane l reads elements
//    8l .. 8l+7 of a chunk of each of the 8 rows (every load instruction is one contiguous KiB of
//    a row) and of each token's x, keeps 8 x NB fp32 products-sums, and the sums are reduced
//    over the 64 lanes (halving exchange) and then over the 4 waves through LDS.  No workspace.
//  * k_proj_mfma (B > 8): bf16 MFMA 32x32x16 with fp32 accumulation on 32-token x 32-row tiles,
//    split over K in chunks (grid z) so that a few rows still spread over many CUs; operands
//    come straight from global memory in the MFMA operand layout (16 contiguous bytes of a row
//    per lane); fp32 x is rounded to bf16 for the MFMA.  The chunks' partial sums go to the
//    workspace [chunk][token][N] and k_proj_reduce adds them in chunk order.
// Both end in the same epilogue on pairs of adjacent outputs (n, n + 1), n even: rows below
// n_split are scaled and stored to y (bf16 or fp32); rows from n_split on are the rotary rows
// (pairs (2i, 2i+1) of each 64-row head block turned by pos[b] * base^(-2i/64), angle and its
// sine and cosine in double precision) stored to y1 as bf16.
//
// k_fold: the per-head product of two weight matrices with fp32 accumulation and a bf16 result,
// C_h = A_h B_h (A_h [M, 128] and B_h [128, Nc], both through strides), used offline for
// W_QK_h = W_UK_h^T W_UQ_h and W_OV_h = W_O[:, h] W_UV_h.
#include "mla_internal.h"

namespace mla {

namespace {
constexpr int kChunk = 512;        // K elements per chunk (GEMV: one KiB per row per wave load)
constexpr int kRot = 64;           // rotary rows per head block

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// the epilogue of one output pair (n, n + 1) of token b
template <bool YBF16>
__device__ __forceinline__ void store_pair(const ProjArgs& a, int b, int n, float v0, float v1) {
  if (n < a.n_split) {
    v0 *= a.scale;
    v1 *= a.scale;
    if (YBF16)
      *(uint32_t*)((uint16_t*)a.y + (int64_t)b * a.ldy + n) = pack_bf16x2(v0, v1);
    else
      *(float2*)((float*)a.y + (int64_t)b * a.ldy + n) = make_float2(v0, v1);
  } else {
    const int n1 = n - a.n_split;
    const int i = (n1 % kRot) >> 1;                                  // pair index within the head
    const double th = (double)a.pos[b] * pow((double)a.rope_base, -2.0 * i / (double)kRot);
    double sn, cs;
    sincos(th, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    *(uint32_t*)((uint16_t*)a.y1 + (int64_t)b * a.ldy1 + n1) = pack_bf16x2(v0 * c - v1 * s, v0 * s + v1 * c);
  }
}

__device__ __forceinline__ const uint16_t* wrow(const ProjArgs& a, int n) {
  return n < a.n_split ? a.w0 + (int64_t)n * a.ldw : a.w1 + (int64_t)(n - a.n_split) * a.ldw;
}

// 8 x-elements k .. k+7 of token b as bf16 pairs (fp32 x is rounded, for the MFMA operand)
template <bool XF32>
__device__ __forceinline__ u32x4 load_x_bf16(const ProjArgs& a, int b, int k) {
  if (!XF32) return *(const u32x4*)((const uint16_t*)a.x + (int64_t)b * a.ldx + k);
  const float* p = (const float*)a.x + (int64_t)b * a.ldx + k;
  const float4 u = *(const float4*)p, v = *(const float4*)(p + 4);
  u32x4 r;
  r[0] = pack_bf16x2(u.x, u.y);
  r[1] = pack_bf16x2(u.z, u.w);
  r[2] = pack_bf16x2(v.x, v.y);
  r[3] = pack_bf16x2(v.z, v.w);
  return r;
}
}  // namespace

size_t proj_ws_bytes(int B, int N, int K) {
  if (B <= kProjGemvMaxB) return 0;
  return (size_t)proj_chunks(K) * (size_t)B * (size_t)N * sizeof(float);
}

// ------------------------------------------------------------------------------------------------
// GEMV, B <= 8.  grid (N / 8), 256 threads.
// ------------------------------------------------------------------------------------------------
template <int NB, bool XF32, bool YBF16>
__global__ __launch_bounds__(256) void k_proj_gemv(ProjArgs a) {
  constexpr int U = NB <= 2 ? 4 : (NB == 8 && XF32) ? 1 : 2;   // chunks whose loads are in flight together
  constexpr int XV = XF32 ? 8 : 4;            // x registers per token and chunk
  __shared__ float red[4][NB * 8];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = 8 * blockIdx.x;
  const int nch = a.K / kChunk;
  const uint16_t* rows[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) rows[r] = wrow(a, n0 + r) + 8 * lane;

  float acc[NB][8];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[b][r] = 0.f;

  for (int c0 = wave; c0 < nch; c0 += 4 * U) {
    u32x4 wv[U][8];
    uint32_t xv[U][NB][XV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = min(c0 + 4 * u, nch - 1);   // past the end: reload the last chunk, unused
#pragma unroll
      for (int r = 0; r < 8; ++r) wv[u][r] = *(const u32x4*)(rows[r] + (int64_t)c * kChunk);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int bb = min(b, a.B - 1);
        const int k = c * kChunk + 8 * lane;
        if (XF32) {
          const float* p = (const float*)a.x + (int64_t)bb * a.ldx + k;
          const u32x4 v0 = *(const u32x4*)p, v1 = *(const u32x4*)(p + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[u][b][j] = v0[j];
            xv[u][b][4 + j] = v1[j];
          }
        } else {
          const u32x4 v = *(const u32x4*)((const uint16_t*)a.x + (int64_t)bb * a.ldx + k);
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[u][b][j] = v[j];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + 4 * u < nch) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            float s = acc[b][r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x0 = XF32 ? __uint_as_float(xv[u][b][2 * j]) : lo_bf16(xv[u][b][j]);
              const float x1 = XF32 ? __uint_as_float(xv[u][b][2 * j + 1]) : hi_bf16(xv[u][b][j]);
              s = fmaf(x0, lo_bf16(wv[u][r][j]), s);
              s = fmaf(x1, hi_bf16(wv[u][r][j]), s);
            }
            acc[b][r] = s;
          }
      }
    }
  }

  // sum over the 64 lanes: each halving step halves the values a lane holds
  constexpr int KV = NB * 8;
  constexpr int LK = NB == 1 ? 3 : NB == 2 ? 4 : NB == 4 ? 5 : 6;   // log2 KV
  float v[KV];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 8; ++r) v[b * 8 + r] = acc[b][r];
#pragma unroll
  for (int step = 0; step < LK; ++step) {
    const int d = 32 >> step;
    const int half = KV >> (step + 1);
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? v[i] : v[i + half];
      const float keep = upper ? v[i + half] : v[i];
      v[i] = keep + __shfl_xor(send, d, 64);
    }
  }
  float s = v[0];
#pragma unroll
  for (int d = (32 >> (LK - 1)) >> 1; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const int idx = (lane >> (6 - LK)) & (KV - 1);
  if ((lane & ((64 >> LK) - 1)) == 0) red[wave][idx] = s;
  __syncthreads();
  if (t < NB * 4) {
    const int b = t >> 2, p = t & 3;
    if (b < a.B) {
      const int i0 = b * 8 + 2 * p;
      const float v0 = ((red[0][i0] + red[1][i0]) + red[2][i0]) + red[3][i0];
      const float v1 = ((red[0][i0 + 1] + red[1][i0 + 1]) + red[2][i0 + 1]) + red[3][i0 + 1];
      store_pair<YBF16>(a, b, n0 + 2 * p, v0, v1);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// MFMA, B > 8.  grid (N / 32, ceil(B / 32), chunks), 64 threads.  Chunk z covers K elements
// [z kc, (z + 1) kc), kc = K / chunks (a multiple of 256).
// ------------------------------------------------------------------------------------------------
template <bool XF32>
__global__ __launch_bounds__(64) void k_proj_mfma(ProjArgs a, int kc, float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int jb = blockIdx.x, tb = blockIdx.y, z = blockIdx.z;
  const int j = jb * 32 + (lane & 31);                    // W row (B operand column)
  const int tok = min(tb * 32 + (lane & 31), a.B - 1);   // token (A operand row); rows past B repeat
  const int k0 = z * kc + 8 * (lane >> 5);
  const uint16_t* w = wrow(a, j) + k0;
  f32x16 acc = {};
  for (int ks = 0; ks < kc; ks += 256) {
    u32x4 xa[16], wb[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      xa[s] = load_x_bf16<XF32>(a, tok, k0 + ks + 16 * s);
      wb[s] = *(const u32x4*)(w + ks + 16 * s);
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma32x32x16(xa[s], wb[s], acc);
  }
  // D layout: lane holds row j for tokens 8 (i / 4) + 4 (lane / 32) + i % 4
  float* dst = part + (int64_t)z * a.B * a.N + j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tt = tb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (tt < a.B) dst[(int64_t)tt * a.N] = acc[i];
  }
}

// grid (ceil(N / 512), B), 256 threads: thread t owns outputs 2t, 2t + 1 of its 512-row block
template <bool YBF16>
__global__ __launch_bounds__(256) void k_proj_reduce(ProjArgs a, int nz, const float* __restrict__ part) {
  const int b = blockIdx.y;
  const int n = blockIdx.x * 512 + 2 * threadIdx.x;
  if (n >= a.N) return;
  const float* p = part + (int64_t)b * a.N + n;
  const int64_t zs = (int64_t)a.B * a.N;
  float v0 = 0.f, v1 = 0.f;
  for (int z0 = 0; z0 < nz; z0 += 8) {                  // groups of 8 loads in flight, summed in order
    float2 u[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = *(const float2*)(p + min(z0 + i, nz - 1) * zs);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (z0 + i < nz) {
        v0 += u[i].x;
        v1 += u[i].y;
      }
  }
  store_pair<YBF16>(a, b, n, v0, v1);
}

// ------------------------------------------------------------------------------------------------
// Fold: C_h[m, n] = sum_{i < 128} A_h[m, i] B_h[i, n].  grid (Nc / 64, M / 64, H), 256 threads,
// each thread 4 x 4 outputs; A and B tiles of 32 inner elements through LDS (fp32).
// ------------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_fold(FoldArgs f) {
  __shared__ float As[32][65];
  __shared__ float Bs[32][65];
  const int t = threadIdx.x;
  const int h = blockIdx.z, m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const uint16_t* A = f.A + (int64_t)h * f.a_sh;
  const uint16_t* Bm = f.B + (int64_t)h * f.b_sh;
  const int tm = (t >> 4) * 4, tn = (t & 15) * 4;
  float acc[4][4] = {};
  for (int i0 = 0; i0 < f.inner; i0 += 32) {
    for (int e = t; e < 32 * 64; e += 256) {
      // consecutive threads walk A's unit-stride index (m or i)
      const int ii = f.a_si == 1 ? (e & 31) : (e >> 6), mm = f.a_si == 1 ? (e >> 5) : (e & 63);
      As[ii][mm] = bf16_bits_to_f32(A[(int64_t)(m0 + mm) * f.a_sm + (int64_t)(i0 + ii) * f.a_si]);
      Bs[e >> 6][e & 63] = bf16_bits_to_f32(Bm[(int64_t)(i0 + (e >> 6)) * f.b_si + (n0 + (e & 63))]);
    }
    __syncthreads();
#pragma unroll 8
    for (int ii = 0; ii < 32; ++ii) {
      float av[4], bv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        av[q] = As[ii][tm + q];
        bv[q] = Bs[ii][tn + q];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(av[x], bv[y], acc[x][y]);
    }
    __syncthreads();
  }
  uint16_t* C = f.C + (int64_t)h * f.c_sh;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    uint16_t* row = C + (int64_t)(m0 + tm + x) * f.c_sm + n0 + tn;
    *(uint32_t*)row = pack_bf16x2(acc[x][0], acc[x][1]);
    *(uint32_t*)(row + 2) = pack_bf16x2(acc[x][2], acc[x][3]);
  }
}

// ------------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------------
namespace {
template <bool XF32, bool YBF16>
hipError_t launch_gemv_nb(const ProjArgs& a, hipStream_t s) {
  const dim3 grid(a.N / 8), block(256);
  if (a.B <= 1)
    hipLaunchKernelGGL((k_proj_gemv<1, XF32, YBF16>), grid, block, 0, s, a);
  else if (a.B <= 2)
    hipLaunchKernelGGL((k_proj_gemv<2, XF32, YBF16>), grid, block, 0, s, a);
  else if (a.B <= 4)
    hipLaunchKernelGGL((k_proj_gemv<4, XF32, YBF16>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_proj_gemv<8, XF32, YBF16>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <bool XF32, bool YBF16>
hipError_t launch_proj_t(const ProjArgs& a, float* ws, hipStream_t s) {
  if (a.B <= kProjGemvMaxB) return launch_gemv_nb<XF32, YBF16>(a, s);
  const int nz = proj_chunks(a.K);
  hipLaunchKernelGGL((k_proj_mfma<XF32>), dim3(a.N / 32, (a.B + 31) / 32, nz), dim3(64), 0, s, a, a.K / nz, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_proj_reduce<YBF16>), dim3((a.N + 511) / 512, a.B), dim3(256), 0, s, a, nz,
                     (const float*)ws);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_proj(const ProjArgs& a, bool x_f32, bool y_bf16, float* ws, hipStream_t s) {
  if (x_f32) return y_bf16 ? launch_proj_t<true, true>(a, ws, s) : launch_proj_t<true, false>(a, ws, s);
  return y_bf16 ? launch_proj_t<false, true>(a, ws, s) : launch_proj_t<false, false>(a, ws, s);
}

hipError_t launch_fold(const FoldArgs& f, hipStream_t s) {
  hipLaunchKernelGGL(k_fold, dim3(f.Nc / 64, f.M / 64, f.H), dim3(256), 0, s, f);
  return hipGetLastError();
}

}  // namespace mla
