// Cache write of one decode step: the new token of every sequence gets its cache row
// ("MLA storage: Representing KV with a small latent vector", sections "Forming head-specific K
// and V from a small vector" and "Storing a positional key separately"; "Grouped-query and
// latent attention", section "Why a separate rotary key"):
//   latent   c_b   = W_DKV h_b               (d_c = 512 outputs)
//   rope key k_R,b = RoPE_pos_b(W_KR h_b)    (d_R = 64 outputs, pairs (2i, 2i+1) turned by
//                                             pos * base^(-2i/d_R))
// written at row pos[b] of sequence b, as bf16, or as OCP E4M3 codes with the per-token float32
// scale amax/448 (RNE of the clamped c/s), into the contiguous or paged layouts the decode path
// reads.
//
// bf16 caches, up to 8 tokens: one projection y = [W_DKV; W_KR] h through the projection GEMV
// (proj.hip), whose epilogue writes the row (and rotates the rope pairs) straight into the cache.
// E4M3 caches need the amax of the whole latent row before any code is chosen, and beyond 8
// tokens the 576 outputs are too few rows to spread a one-pass projection over the chip, so
// those take two passes:
//  * k_append_gemv (B <= 8): a streaming GEMV over coalesced weight rows, split over D in chunks
//    of 512 (see below);
//  * k_append_proj (B > 8): the projection [B x D] . [D x 576] on bf16 MFMA 32x32x16 with fp32
//    accumulation, split over D in chunks of 512 so that the 8.3 MB of weights stream from many
//    CUs at once even for one token.  One wave per workgroup computes a 32-token x 32-output tile
//    of one chunk; both operands come straight from global memory in the MFMA operand layout
//    (16 contiguous bytes of a row per lane).  Partial sums go to the workspace,
//    [chunk][token][576] float32.
//  * k_append_finalize: one workgroup per token adds the chunks in order, rotates the rope pairs
//    (angles in double precision), encodes, and stores the row.
#include "lane_reduce.h"
#include "rows_internal.h"

namespace mla {

namespace {
constexpr int kOut = 576;          // d_c + d_R outputs per token
constexpr int kKChunk = 512;       // D elements per projection chunk
}  // namespace

size_t append_ws_bytes(int B, int D) {
  // chunk partials of the two-pass form (the one-pass form needs none)
  return (size_t)(D / kKChunk) * (size_t)B * kOut * sizeof(float);
}

// grid (576 / 32 output blocks, ceil(B / 32) token blocks, D / 512 chunks), 64 threads
__global__ __launch_bounds__(64) void k_append_proj(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
                                                    const uint16_t* __restrict__ w_kr, int B, int D,
                                                    float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int jb = blockIdx.x, tb = blockIdx.y, ks = blockIdx.z;
  const int j = jb * 32 + (lane & 31);                     // this lane's output row (B operand column)
  const int tok = min(tb * 32 + (lane & 31), B - 1);      // this lane's token (A operand row); rows past B repeat the last
  const int k0 = ks * kKChunk + 8 * (lane >> 5);
  const uint16_t* wrow = (j < 512 ? w_dkv + (int64_t)j * D : w_kr + (int64_t)(j - 512) * D) + k0;
  const uint16_t* hrow = h + (int64_t)tok * D + k0;
  f32x16 acc = {};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x4 a[16], b[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      a[s] = *(const u32x4*)(hrow + 16 * (16 * half + s));
      b[s] = *(const u32x4*)(wrow + 16 * (16 * half + s));
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = mfma32x32x16(a[s], b[s], acc);
  }
  // D layout: lane holds output j for tokens 8 (i / 4) + 4 (lane / 32) + i % 4
  float* dst = part + ((int64_t)ks * B) * kOut + j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int t = tb * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (t < B) dst[(int64_t)t * kOut] = acc[i];
  }
}

// Few tokens (B <= 8): streaming GEMV.  Grid (576 / 8 row groups, D / 512 chunks), 64 threads.
// The wave reads rows 8g .. 8g+7 of [W_DKV; W_KR] over one 512-wide chunk (lane l: elements
// 8l .. 8l+7, so each load is one contiguous KiB of a row) and the matching chunk of every h row,
// then sums the NB x 8 lane products over the 64 lanes with a halving exchange (each step halves
// the values a lane holds and doubles the lanes summed into each).
template <int NB>
__global__ __launch_bounds__(64) void k_append_gemv(const uint16_t* __restrict__ h, const uint16_t* __restrict__ w_dkv,
                                                    const uint16_t* __restrict__ w_kr, int B, int D,
                                                    float* __restrict__ part) {
  const int lane = threadIdx.x;
  const int g = blockIdx.x, ks = blockIdx.y;
  const int k = ks * kKChunk + 8 * lane;
  u32x4 wv[8], hv[NB];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int j = 8 * g + r;
    wv[r] = *(const u32x4*)((j < 512 ? w_dkv + (int64_t)j * D : w_kr + (int64_t)(j - 512) * D) + k);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) hv[b] = *(const u32x4*)(h + (int64_t)min(b, B - 1) * D + k);
  constexpr int K = NB * 8;   // values per lane before the exchange: index b * 8 + r
  float v[K];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        acc = fmaf(__uint_as_float(hv[b][c] << 16), __uint_as_float(wv[r][c] << 16), acc);
        acc = fmaf(__uint_as_float(hv[b][c] & 0xffff0000u), __uint_as_float(wv[r][c] & 0xffff0000u), acc);
      }
      v[b * 8 + r] = acc;
    }
  constexpr int LK = NB == 1 ? 3 : NB == 2 ? 4 : NB == 4 ? 5 : 6;   // log2 K
  // lane l ends with the full sum of value index (l >> (6 - LK))
  const float t = lane_sum_halving<K>(v, lane);
  const int idx = (lane >> (6 - LK)) & (K - 1);
  const int b = idx >> 3, r = idx & 7;
  if ((lane & ((64 >> LK) - 1)) == 0 && b < B) part[((int64_t)ks * B + b) * kOut + 8 * g + r] = t;
}

namespace {
// float -> OCP E4M3 code, |y| <= 448 (clamped by the caller), round to nearest even:
// below 2^-6 the grid step is 2^-9 (subnormals), in [2^e, 2^(e+1)) it is 2^(e-3)
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = __float_as_uint(y) >> 31;
  const float a = fabsf(y);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);          // 0 .. 8 (8 is 2^-6, the first normal)
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;   // a is a normal float here
    const float m = __builtin_rintf((a * __builtin_ldexpf(1.0f, -e) - 1.0f) * 8.0f);   // 0 .. 8
    code = (uint32_t)((e + 7) << 3) + (uint32_t)m;           // m = 8 carries into the exponent
    code = min(code, 0x7Eu);
  }
  return code == 0 ? 0u : (code | (sign << 7));
}
}  // namespace

// grid (B), 256 threads.  Thread t owns latent outputs 2t, 2t+1; threads t < 32 also own rope
// pair t (outputs 512 + 2t, 513 + 2t).
template <bool FP8, bool PAGED>
__global__ __launch_bounds__(256) void k_append_finalize(const float* __restrict__ part, int nks, int B,
                                                         const int32_t* __restrict__ pos, AppendArgs a) {
  __shared__ float red[4];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* p = part + (int64_t)b * kOut;
  const int64_t kstride = (int64_t)B * kOut;
  float2 lat = make_float2(0.f, 0.f);
  float2 rp = make_float2(0.f, 0.f);
  // chunks in groups of 8: all loads of a group are in flight together, the sums keep chunk order
  for (int k0 = 0; k0 < nks; k0 += 8) {
    float2 v[8], r[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int ks = min(k0 + u, nks - 1);
      v[u] = *(const float2*)(p + ks * kstride + 2 * t);
      r[u] = t < 32 ? *(const float2*)(p + ks * kstride + 512 + 2 * t) : make_float2(0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < nks) {
        lat.x += v[u].x;
        lat.y += v[u].y;
        rp.x += r[u].x;
        rp.y += r[u].y;
      }
    }
  }
  const int ps = pos[b];
  int64_t lrow, rrow, srow;
  if (PAGED) {
    const int page = a.block_table[(int64_t)b * a.max_pages + ps / a.page_size];
    const int slot = ps % a.page_size;
    lrow = (int64_t)page * a.lat_sb + (int64_t)slot * a.lat_st;
    rrow = (int64_t)page * a.rope_sb + (int64_t)slot * a.rope_st;
    srow = (int64_t)page * a.scale_sb + slot;
  } else {
    lrow = (int64_t)b * a.lat_sb + (int64_t)ps * a.lat_st;
    rrow = (int64_t)b * a.rope_sb + (int64_t)ps * a.rope_st;
    srow = (int64_t)b * a.scale_sb + ps;
  }
  if (t < 32) {
    // pair t turns by pos * base^(-2t/64); the angle and its sine and cosine in double precision
    const double th = (double)ps * pow((double)a.rope_base, -2.0 * t / 64.0);
    double sn, cs;
    sincos(th, &sn, &cs);
    const float c = (float)cs, s = (float)sn;
    const float x0 = rp.x * c - rp.y * s;
    const float x1 = rp.x * s + rp.y * c;
    *(uint32_t*)((uint16_t*)a.rope + rrow + 2 * t) = pack_bf16x2(x0, x1);
  }
  if (!FP8) {
    *(uint32_t*)((uint16_t*)a.latent + lrow + 2 * t) = pack_bf16x2(lat.x, lat.y);
    return;
  }
  float m = fmaxf(fabsf(lat.x), fabsf(lat.y));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  const float y0 = fminf(fmaxf(lat.x / s, -448.0f), 448.0f);
  const float y1 = fminf(fmaxf(lat.y / s, -448.0f), 448.0f);
  *(uint16_t*)((uint8_t*)a.latent + lrow + 2 * t) = (uint16_t)(e4m3_code(y0) | (e4m3_code(y1) << 8));
  if (t == 0) a.latent_scale[srow] = s;
}

hipError_t launch_append(const void* h, const void* w_dkv, const void* w_kr, const int32_t* pos, int B, int D,
                         const AppendArgs& a, bool fp8, bool paged, float* ws, hipStream_t s) {
  // one pass only where the projection GEMV serves it (no workspace; the workspace of this call is
  // sized for the two-pass form)
  if (!fp8 && proj_uses_gemv(B, kOut, D)) {
    ProjArgs pa{};
    pa.w0 = (const uint16_t*)w_dkv;
    pa.wc = (const uint16_t*)w_dkv;
    pa.w1 = (const uint16_t*)w_kr;
    pa.n_cache = 0;
    pa.n_split = kOut - 64;
    pa.ldw = D;
    pa.x = h;
    pa.ldx = D;
    pa.B = B;
    pa.N = kOut;
    pa.K = D;
    pa.scale = 1.f;
    pa.pos = pos;
    pa.rope_base = a.rope_base;
    pa.dst_cache = 1;
    pa.cache = a;
    return launch_proj(pa, false, true, ws, s);
  }
  if (B <= 8) {
    const dim3 g0(kOut / 8, D / kKChunk);
#define MLA_GEMV(NB) hipLaunchKernelGGL(k_append_gemv<NB>, g0, dim3(64), 0, s, (const uint16_t*)h, \
                                        (const uint16_t*)w_dkv, (const uint16_t*)w_kr, B, D, ws)
    if (B == 1) MLA_GEMV(1);
    else if (B == 2) MLA_GEMV(2);
    else if (B <= 4) MLA_GEMV(4);
    else MLA_GEMV(8);
#undef MLA_GEMV
  } else {
    const dim3 g1(kOut / 32, (B + 31) / 32, D / kKChunk);
    hipLaunchKernelGGL(k_append_proj, g1, dim3(64), 0, s, (const uint16_t*)h, (const uint16_t*)w_dkv,
                       (const uint16_t*)w_kr, B, D, ws);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nks = D / kKChunk;
#define MLA_FIN(F, PG) hipLaunchKernelGGL((k_append_finalize<F, PG>), dim3(B), dim3(256), 0, s, ws, nks, B, pos, a)
  if (fp8) {
    if (paged) MLA_FIN(true, true); else MLA_FIN(true, false);
  } else {
    if (paged) MLA_FIN(false, true); else MLA_FIN(false, false);
  }
#undef MLA_FIN
  return hipGetLastError();
}

}  // namespace mla
