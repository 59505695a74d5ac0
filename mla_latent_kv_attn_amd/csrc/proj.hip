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
// stream of the weights from HBM.  Two kernels (the GEMV for up to 4 tokens, and for up to 8 when
// K >= 4096 and the weight has at most 32M elements; the MFMA path otherwise):
//  * k_proj_gemv: one workgroup (4 waves) per R rows of W (R = 2, 4 or 8 by batch) over
//    the whole of K.  K is cut into 512-element chunks; wave w takes chunks w, w + 4, ... with U
//    chunks' loads in flight together.  Lane l reads elements 8l .. 8l+7 of a chunk of each of the
//    R rows (every load instruction is one contiguous KiB of a row) and of each token's x, keeps
//    R x NB fp32 product sums, and the sums are reduced over the 64 lanes (halving exchange) and
//    then over the 4 waves through LDS.  No workspace.
//  * k_proj_mfma: bf16 MFMA 32x32x16 with fp32 accumulation on tiles of 128 rows x up
//    to 128 tokens (4 waves of 32 rows), split over K in chunks (grid z) so that the weights
//    stream from many CUs at once; x (fp32 rounded to bf16) is staged once per workgroup through
//    LDS, W comes straight from global memory in the MFMA operand layout (16 contiguous bytes of
//    a row per lane).  The chunks' partial sums go to the workspace [chunk][token][N] and
//    k_proj_reduce adds them in chunk order.
// Both end in the same epilogue on pairs of adjacent outputs (n, n + 1), n even: rows below
// n_split are scaled and stored to y (bf16 or fp32); rows from n_split on are the rotary rows
// (pairs (2i, 2i+1) of each 64-row head block turned by pos[b] * base^(-2i/64), angle and its
// sine and cosine in double precision) stored to y1 as bf16.  For the cache write (bf16 caches)
// both go straight into the new token's cache row at pos[b]: latent = W_DKV h, rope key =
// RoPE_pos(W_KR h) ("MLA storage: Representing KV with a small latent vector", section "Storing a
// positional key separately").
//
// k_fold: the per-head product of two weight matrices with fp32 accumulation and a bf16 result,
// C_h = A_h B_h (A_h [M, 128] and B_h [128, Nc], both through strides), used offline for
// W_QK_h = W_UK_h^T W_UQ_h and W_OV_h = W_O[:, h] W_UV_h.
#include "lane_reduce.h"
#include "rows_internal.h"

namespace mla {

namespace {
constexpr int kChunk = 512;        // K elements per chunk (GEMV: one KiB per row per wave load)
constexpr int kRot = 64;           // rotary rows per head block

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// rotation of the rotary pair that holds output n (n >= n_split) of token b: cos and sin of
// pos[b] * base^(-2i/64), i the pair index within the head, in double precision
__device__ __forceinline__ float2 rope_cs_pair(const ProjArgs& a, int b, int i) {
  const double th = (double)a.pos[b] * pow((double)a.rope_base, -2.0 * i / (double)kRot);
  double sn, cs;
  sincos(th, &sn, &cs);
  return make_float2((float)cs, (float)sn);
}
__device__ __forceinline__ float2 rope_cs(const ProjArgs& a, int b, int n) {
  return rope_cs_pair(a, b, ((n - a.n_split) % kRot) >> 1);
}

// the epilogue of one output pair (n, n + 1) of token b; cs is the pair's rotation when n >= n_split
template <bool YBF16>
__device__ __forceinline__ void store_pair(const ProjArgs& a, int b, int n, float v0, float v1, float2 cs) {
  if (a.dst_cache && n >= a.n_cache) {
    // the cache write: token b's new row at pos[b] (contiguous, or through the block table)
    const AppendArgs& c = a.cache;
    const int ps = a.pos[b];
    int64_t lrow, rrow;
    if (c.block_table) {
      const int page = c.block_table[(int64_t)b * c.max_pages + ps / c.page_size];
      const int slot = ps % c.page_size;
      lrow = (int64_t)page * c.lat_sb + (int64_t)slot * c.lat_st;
      rrow = (int64_t)page * c.rope_sb + (int64_t)slot * c.rope_st;
    } else {
      lrow = (int64_t)b * c.lat_sb + (int64_t)ps * c.lat_st;
      rrow = (int64_t)b * c.rope_sb + (int64_t)ps * c.rope_st;
    }
    if (n < a.n_split)
      *(uint32_t*)((uint16_t*)c.latent + lrow + (n - a.n_cache)) = pack_bf16x2(v0, v1);
    else
      *(uint32_t*)((uint16_t*)c.rope + rrow + (n - a.n_split)) =
          pack_bf16x2(v0 * cs.x - v1 * cs.y, v0 * cs.y + v1 * cs.x);
    return;
  }
  if (n < a.n_split) {
    v0 *= a.scale;
    v1 *= a.scale;
    if (YBF16)
      *(uint32_t*)((uint16_t*)a.y + (int64_t)b * a.ldy + n) = pack_bf16x2(v0, v1);
    else
      *(float2*)((float*)a.y + (int64_t)b * a.ldy + n) = make_float2(v0, v1);
  } else {
    *(uint32_t*)((uint16_t*)a.y1 + (int64_t)b * a.ldy1 + (n - a.n_split)) =
        pack_bf16x2(v0 * cs.x - v1 * cs.y, v0 * cs.y + v1 * cs.x);
  }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v >> 1); }

__device__ __forceinline__ const uint16_t* wrow(const ProjArgs& a, int n) {
  if (n >= a.n_split) return a.w1 + (int64_t)(n - a.n_split) * a.ldw;
  if (n >= a.n_cache) return a.wc + (int64_t)(n - a.n_cache) * a.ldw;
  return a.w0 + (int64_t)n * a.ldw;
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
  if (proj_uses_gemv(B, N, K)) return 0;
  return (size_t)proj_chunks(B, N, K) * (size_t)B * (size_t)N * sizeof(float);
}

// ------------------------------------------------------------------------------------------------
// GEMV, B <= 8.  grid (N / R), 256 threads; R rows per workgroup.
// ------------------------------------------------------------------------------------------------
template <int NB, int R, int U, bool XF32, bool YBF16>
__global__ __launch_bounds__(256) void k_proj_gemv(ProjArgs a) {
  constexpr int XV = XF32 ? 8 : 4;            // x registers per token and chunk
  constexpr int KV = NB * R;                  // lane partial sums
  constexpr int LK = ilog2(KV);
  static_assert((KV & (KV - 1)) == 0 && KV >= 2 && KV <= 64, "NB x R: a power of two in [2, 64]");
  __shared__ float red[4][KV];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n0 = R * blockIdx.x;
  const int nch = a.K / kChunk;
  const uint16_t* rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) rows[r] = wrow(a, n0 + r) + 8 * lane;
  // the epilogue pair of this thread (threads t < KV / 2 of wave 0): its rotation is computed
  // while the first loads are in flight
  const int eb = t / (R / 2), en = n0 + 2 * (t % (R / 2));
  const bool epi = t < KV / 2 && eb < a.B;
  float2 cs = make_float2(1.f, 0.f);

  float acc[NB][R];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[b][r] = 0.f;

  for (int c0 = wave; c0 < nch; c0 += 4 * U) {
    u32x4 wv[U][R];
    uint32_t xv[U][NB][XV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      if (c >= nch) break;                      // wave-uniform
#pragma unroll
      for (int r = 0; r < R; ++r) wv[u][r] = *(const u32x4*)(rows[r] + (int64_t)c * kChunk);
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
    if (c0 == wave && epi && en >= a.n_split) cs = rope_cs(a, eb, en);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + 4 * u < nch) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < R; ++r) {
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
  float v[KV];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < R; ++r) v[b * R + r] = acc[b][r];
  // lane l ends with the full sum of value index (l >> (6 - LK))
  const float s = lane_sum_halving<KV>(v, lane);
  const int idx = (lane >> (6 - LK)) & (KV - 1);
  if ((lane & ((64 >> LK) - 1)) == 0) red[wave][idx] = s;
  __syncthreads();
  if (epi) {
    const int i0 = eb * R + (en - n0);
    const float v0 = ((red[0][i0] + red[1][i0]) + red[2][i0]) + red[3][i0];
    const float v1 = ((red[0][i0 + 1] + red[1][i0 + 1]) + red[2][i0 + 1]) + red[3][i0 + 1];
    store_pair<YBF16>(a, eb, en, v0, v1, cs);
  }
}

// ------------------------------------------------------------------------------------------------
// MFMA, the batches the GEMV does not serve.  grid (ceil(N / 128), ceil(B / 128), chunks), 256
// threads.  The workgroup owns rows
// [128 x, 128 x + 128) (wave w: 32 of them) and tokens [128 y, 128 y + 32 NT) over chunk z of K
// (kc elements).  Per 64-element step of K the tokens' x (rounded to bf16) goes through LDS once
// for all four waves (double buffered, one barrier per step; x is read from L2 one step ahead),
// while each wave loads its rows' W straight into registers in the MFMA operand layout (lane:
// row lane % 32, 8 elements at 16 s + 8 (lane / 32)), two steps ahead through a ring of three
// register sets (the step loop is unrolled by three so that the ring indices are constants).
// A = x (tokens), B = W (rows), D[token][row] in fp32.
// ------------------------------------------------------------------------------------------------
template <int NT, bool XF32>
__global__ __launch_bounds__(256) void k_proj_mfma(ProjArgs a, int kc, float* __restrict__ part) {
  constexpr int kStep = 64, kRowB = kStep * 2 + 16;       // LDS row: 64 bf16 + 16 bytes of skew
  constexpr int TB = 32 * NT;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2][TB * kRowB];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int row0 = blockIdx.x * kProjRows + 32 * wave;
  const int tok0 = blockIdx.y * kProjToks;
  const int kbeg = blockIdx.z * kc;
  const bool active = row0 < a.N;                         // wave-uniform (N is a multiple of 32)
  const uint16_t* w = wrow(a, active ? row0 + (lane & 31) : 0) + kbeg + 8 * (lane >> 5);

  // x staging: TB tokens x 64 elements = TB * 8 pieces of 8 elements; thread t takes pieces t + 256 i
  constexpr int XP = TB * 8 / 256;                        // = NT
  u32x4 xr[XP];
  auto load_x = [&](int k) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int piece = t + 256 * i;
      const int tok = min(tok0 + (piece >> 3), a.B - 1);  // tokens past B repeat the last (discarded)
      xr[i] = load_x_bf16<XF32>(a, tok, k + 8 * (piece & 7));
    }
  };
  auto store_x = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const int piece = t + 256 * i;
      *(u32x4*)&xs[buf][(piece >> 3) * kRowB + 16 * (piece & 7)] = xr[i];
    }
  };
  // inactive waves (rows past N) read row 0 (in bounds) and store nothing
  u32x4 wr[3][4];
  auto load_w = [&](int k, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 4; ++s) dst[s] = *(const u32x4*)(w + (k - kbeg) + 16 * s);
  };

  f32x16 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) acc[i] = f32x16{};
  const int nsteps = kc / kStep;
  // Every load is unconditional (steps past the chunk's end reread its last step, from L2): a load
  // under a branch makes the compiler's wait counting fall back to waiting for all loads in flight
  // where the paths join, which would undo the prefetch.  Inactive waves compute on row 0 and
  // store nothing.
  load_x(kbeg);
  load_w(kbeg, wr[0]);
  load_w(kbeg + min(1, nsteps - 1) * kStep, wr[1]);
  for (int st0 = 0; st0 < nsteps; st0 += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int st = st0 + u;
      if (st >= nsteps) break;
      const int buf = st & 1;
      store_x(buf);
      __syncthreads();
      load_x(kbeg + min(st + 1, nsteps - 1) * kStep);
      load_w(kbeg + min(st + 2, nsteps - 1) * kStep, wr[(u + 2) % 3]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          const u32x4 xa = *(const u32x4*)&xs[buf][(32 * i + (lane & 31)) * kRowB + 32 * s + 16 * (lane >> 5)];
          acc[i] = mfma32x32x16(xa, wr[u][s], acc[i]);
        }
      }
    }
  }
  if (!active) return;
  // D layout: lane holds row row0 + lane % 32 for tokens 8 (e / 4) + 4 (lane / 32) + e % 4
  float* dst = part + (int64_t)blockIdx.z * a.B * a.N + row0 + (lane & 31);
#pragma unroll
  for (int i = 0; i < NT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int tt = tok0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      if (tt < a.B) dst[(int64_t)tt * a.N] = acc[i][e];
    }
}

// grid (ceil(N / 1024), B), 256 threads: thread t owns outputs 4t .. 4t + 3 (two pairs) of its
// 1024-row block (N % 4 == 0).  The chunks' partials are read G at a time (16 bytes each, every
// load unconditional: chunk indices past nz are clamped and their values not added) and summed in
// chunk order.
template <bool YBF16, int G>
__global__ __launch_bounds__(256) void k_proj_reduce(ProjArgs a, int nz, const float* __restrict__ part) {
  const int b = blockIdx.y;
  const int n = blockIdx.x * 1024 + 4 * threadIdx.x;
  // every head block of token b turns its rotary pairs by the same kRot / 2 angles: computed once
  // per workgroup (the same double-precision function as elsewhere, so the same values)
  __shared__ float2 cs_s[kRot / 2];
  const bool rot = a.N > a.n_split && (int)blockIdx.x * 1024 + 1024 > a.n_split;   // workgroup-uniform
  if (rot) {
    if (threadIdx.x < kRot / 2) cs_s[threadIdx.x] = rope_cs_pair(a, b, threadIdx.x);
    __syncthreads();
  }
  if (n >= a.N) return;
  const float* p = part + (int64_t)b * a.N + n;
  const int64_t zs = (int64_t)a.B * a.N;
  float v0 = 0.f, v1 = 0.f, v2 = 0.f, v3 = 0.f;
  for (int z0 = 0; z0 < nz; z0 += G) {
    f32x4 u[G];
#pragma unroll
    for (int i = 0; i < G; ++i) u[i] = *(const f32x4*)(p + min(z0 + i, nz - 1) * zs);
#pragma unroll
    for (int i = 0; i < G; ++i)
      if (z0 + i < nz) {
        v0 += u[i][0];
        v1 += u[i][1];
        v2 += u[i][2];
        v3 += u[i][3];
      }
  }
  const int i0 = n >= a.n_split ? ((n - a.n_split) % kRot) >> 1 : 0;
  const int i1 = n + 2 >= a.n_split ? ((n + 2 - a.n_split) % kRot) >> 1 : 0;
  store_pair<YBF16>(a, b, n, v0, v1, n >= a.n_split ? cs_s[i0] : make_float2(1.f, 0.f));
  store_pair<YBF16>(a, b, n + 2, v2, v3, n + 2 >= a.n_split ? cs_s[i1] : make_float2(1.f, 0.f));
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
template <int NB, bool XF32, bool YBF16, int RK = 0>
void launch_gemv_t(const ProjArgs& a, hipStream_t s) {
  // rows per workgroup R and chunks in flight per wave U, from a sweep at the V3 shapes: one token
  // streams best with few rows and a deep queue; from two tokens on the register budget (and so
  // the waves per SIMD) decides, and more rows share each x load
#ifdef PROJ_GEMV_R
  constexpr int R = PROJ_GEMV_R;
#else
  constexpr int R = RK ? RK : NB == 1 ? (XF32 ? 4 : 2) : NB == 2 ? 4 : NB == 4 ? (XF32 ? 8 : 4) : (XF32 ? 8 : 2);
#endif
#ifdef PROJ_GEMV_U
  constexpr int U = PROJ_GEMV_U;
#else
  constexpr int U = NB == 1 ? (XF32 ? 4 : 2) : NB == 2 ? (XF32 ? 2 : 1) : 1;
#endif
  hipLaunchKernelGGL((k_proj_gemv<NB, R, U, XF32, YBF16>), dim3(a.N / R), dim3(256), 0, s, a);
}

template <bool XF32, bool YBF16>
hipError_t launch_gemv_nb(const ProjArgs& a, hipStream_t s) {
  if (a.B <= 1) {
    // one token, bf16 x: short rows (K < 4096, 3 KiB) stream better with 4 rows per workgroup
    if (!XF32 && a.K < 4096)
      launch_gemv_t<1, XF32, YBF16, 4>(a, s);
    else
      launch_gemv_t<1, XF32, YBF16>(a, s);
  }
  else if (a.B <= 2)
    launch_gemv_t<2, XF32, YBF16>(a, s);
  else if (a.B <= 4)
    launch_gemv_t<4, XF32, YBF16>(a, s);
  else
    launch_gemv_t<8, XF32, YBF16>(a, s);
  return hipGetLastError();
}

template <bool XF32, bool YBF16>
hipError_t launch_proj_t(const ProjArgs& a, float* ws, hipStream_t s) {
  if (proj_uses_gemv(a.B, a.N, a.K)) return launch_gemv_nb<XF32, YBF16>(a, s);
  const int nz = proj_chunks(a.B, a.N, a.K);
  const dim3 grid((a.N + kProjRows - 1) / kProjRows, (a.B + kProjToks - 1) / kProjToks, nz);
  const int toks = a.B < kProjToks ? a.B : kProjToks;     // tokens of the widest workgroup
  if (toks <= 32)
    hipLaunchKernelGGL((k_proj_mfma<1, XF32>), grid, dim3(256), 0, s, a, a.K / nz, ws);
  else if (toks <= 64)
    hipLaunchKernelGGL((k_proj_mfma<2, XF32>), grid, dim3(256), 0, s, a, a.K / nz, ws);
  else
    hipLaunchKernelGGL((k_proj_mfma<4, XF32>), grid, dim3(256), 0, s, a, a.K / nz, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rg((a.N + 1023) / 1024, a.B);
  if (nz <= 2)
    hipLaunchKernelGGL((k_proj_reduce<YBF16, 2>), rg, dim3(256), 0, s, a, nz, (const float*)ws);
  else if (nz <= 4)
    hipLaunchKernelGGL((k_proj_reduce<YBF16, 4>), rg, dim3(256), 0, s, a, nz, (const float*)ws);
  else
    hipLaunchKernelGGL((k_proj_reduce<YBF16, 8>), rg, dim3(256), 0, s, a, nz, (const float*)ws);
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
