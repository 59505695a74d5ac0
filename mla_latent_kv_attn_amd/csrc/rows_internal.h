// Internal declarations of the rows around the decode path (cache write, projections, the
// same-dimension MHA comparison), shared by their HIP sources and the C ABI (gfx950 only).
#pragma once

#include "mla_internal.h"

namespace mla {

// cache write: destination rows (element strides as in mla_cache_desc)
struct AppendArgs {
  void* latent;
  void* rope;
  float* latent_scale;
  const int32_t* block_table;
  int64_t lat_sb, lat_st, rope_sb, rope_st, scale_sb;
  int page_size, max_pages;
  float rope_base;
};

// projections y[b, n] = sum_k W[n, k] x[b, k] (proj.hip).  Rows n < n_split come from w0 and are
// scaled and stored to y; rows n >= n_split come from w1 (row n - n_split) and are the rotary rows,
// turned per 64-row head block at pos[b] and stored to y1 as bf16.  With dst_cache, rows
// [n_cache, n_split) come from wc and both they and the rotary rows go into the new token's cache
// row instead.  N % 32 == 0, K % 512 == 0, segment boundaries even.
constexpr int kProjGemvMaxB = 8;   // the GEMV kernel serves at most this many tokens
// GEMV (no workspace) for up to 4 tokens, and for up to 8 when K is long (>= 4096) and the weight
// small (at most 32M elements: W_DQ, the cache write); otherwise the MFMA path (whose 32-token tile
// costs about the same from 1 to 32 tokens, with W two steps ahead) is faster
inline bool proj_uses_gemv(int B, int N, int K) {
  return B <= 4 || (B <= kProjGemvMaxB && K >= 4096 && (int64_t)N * K <= ((int64_t)32 << 20));
}
struct ProjArgs {
  const uint16_t* w0;
  const uint16_t* w1;
  int n_split;
  int64_t ldw;                  // row stride of w0 and w1 (elements)
  const void* x;                // [B, K] bf16 or fp32, row stride ldx
  int64_t ldx;
  int B, N, K;
  float scale;                  // applied to rows below n_split
  void* y;                      // [B, n_split] (row stride ldy), bf16 or fp32
  int64_t ldy;
  void* y1;                     // [B, N - n_split] bf16 (row stride ldy1), the rotated rows
  int64_t ldy1;
  const int32_t* pos;           // [B] positions of the rotary rows
  float rope_base;
  int dst_cache;                // 1: rows [n_cache, n_split) come from wc (row n - n_cache) and go to
  AppendArgs cache;             //    the cache latent row of token b at pos[b], the rotated rows to its
  const uint16_t* wc;           //    rope row (bf16; y1 unused); rows below n_cache still go to y
  int n_cache;                  // == n_split unless dst_cache
};
// MFMA path (otherwise): workgroup tiles of 128 rows x up to 128 tokens; K is split into
// proj_chunks(B, N, K) chunks, a divisor of K / 256, the fewest that give at least 224 workgroups
// and at most 4096 elements of K per chunk (with W two steps ahead in every workgroup, about one
// workgroup per CU keeps enough loads in flight; more chunks add partial sums without streaming
// faster, and longer chunks leave the chip's second workgroup slot idle on the long rows of the
// folded W_O W_UV)
constexpr int kProjRows = 128, kProjToks = 128;
inline int proj_chunks(int B, int N, int K) {
  const int64_t blocks = (int64_t)((N + kProjRows - 1) / kProjRows) * ((B + kProjToks - 1) / kProjToks);
  const int units = K / 256;
  for (int d = 1; d <= units; ++d)
    if (units % d == 0 && blocks * d >= 224 && K / d <= 4096) return d;
  return units;
}
size_t proj_ws_bytes(int B, int N, int K);

// per-head weight fold C_h[m, n] = sum_{i < inner} A_h[m, i] B_h[i, n] (bf16 in, fp32 sums, bf16 out)
struct FoldArgs {
  const uint16_t* A;
  int64_t a_sh, a_sm, a_si;
  const uint16_t* B;
  int64_t b_sh, b_si;           // column stride 1
  uint16_t* C;
  int64_t c_sh, c_sm;           // column stride 1
  int H, M, Nc, inner;          // M % 64 == 0, Nc % 64 == 0, inner % 32 == 0
};

size_t append_ws_bytes(int B, int D);
size_t mha_ws_bytes(int B, int H, int W);
hipError_t launch_mha(const void* q, const void* kc, const void* vc, const int32_t* lens, int B, int H, int64_t cap,
                      float scale, int W, float* ws, float* out, float* lse, hipStream_t s);
hipError_t launch_proj(const ProjArgs& a, bool x_f32, bool y_bf16, float* ws, hipStream_t s);
hipError_t launch_fold(const FoldArgs& f, hipStream_t s);
hipError_t launch_append(const void* h, const void* w_dkv, const void* w_kr, const int32_t* pos, int B, int D,
                         const AppendArgs& a, bool fp8, bool paged, float* ws, hipStream_t s);

}  // namespace mla
