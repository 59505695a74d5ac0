// Host side of the C ABI declared in include/mla.h: argument validation, path selection,
// workspace sizing and launches.  No device memory is allocated here.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "rows_internal.h"
#include "step_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  g_last_hip_error = (int)e;
  return MLA_ERR_HIP;
}

bool known_dtype(int d) { return d == MLA_F32 || d == MLA_BF16 || d == MLA_FP8_E4M3; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Batches of at most kSmallTiles 32-token tiles in total (bf16) take the small-batch partial
// kernel: one 32-head block per workgroup, so H/32 workgroups share each split.
constexpr int64_t kSmallTiles = 1024;

int64_t total_tiles_bound(int B, int max_len) { return (int64_t)B * ((max_len + mla::kTile - 1) / mla::kTile); }

// Partial-pass splits when the caller passes 0.
//  * small batches: about 8/3 tiles per split, ceil(3 T / 8), at most 64 splits (with the V3 head
//    count the four head blocks of 64 splits fill the 256 CUs).  Fewer splits mean fewer partials
//    for the combine pass to read and spare CUs for the weight warm-up; more splits shorten the
//    partial pass (measured at B = 1, N = 4096: 48 splits);
//  * otherwise about two tiles per split, at most one workgroup per CU (256).
int auto_splits(int B, int H, int max_len) {
  (void)H;
  const int64_t nt = total_tiles_bound(B, max_len);
  int64_t w = nt <= kSmallTiles ? std::min<int64_t>((3 * nt + 7) / 8, 64) : std::min<int64_t>((nt + 1) / 2, 256);
  if (w < 1) w = 1;
  return (int)w;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: invalid or inconsistent sizes";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown or invalid dtype combination";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for these arguments";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime or launch failure";
    default: return "unknown mla status";
  }
}

int mla_last_hip_error(void) { return g_last_hip_error; }

int mla_version(void) { return 10000; }

int mla_absorb_q(const void* q_C, const void* W_UK, void* q_abs, int in_dtype, int out_dtype, int B, int H,
                 int d_h, int d_c, void* stream) {
  if (B < 0 || H < 1 || d_h < 1 || d_c < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(in_dtype) || !known_dtype(out_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!q_C || !W_UK || !q_abs) return MLA_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (in_dtype == MLA_F32 && out_dtype == MLA_F32) {
    if (d_h > 1024 || d_c > 4096) return MLA_ERR_UNSUPPORTED;
    return hip_status(mla::launch_absorb_f32((const float*)q_C, (const float*)W_UK, (float*)q_abs, B, H, d_h, d_c, s));
  }
  if (in_dtype == MLA_BF16 && out_dtype == MLA_BF16) {
    if (d_h != 128 || d_c != 512) return MLA_ERR_UNSUPPORTED;
    if (!aligned16(q_C) || !aligned16(W_UK)) return MLA_ERR_UNSUPPORTED;
    return hip_status(mla::launch_absorb_bf16(q_C, W_UK, q_abs, B, H, s));
  }
  return MLA_ERR_UNSUPPORTED;
}

int mla_decode_auto_splits(int B, int H, int max_len) {
  if (B < 0 || H < 1 || max_len < 0) return 0;
  return auto_splits(B, H, max_len);
}

size_t mla_decode_workspace_bytes(int B, int H, int d_c, int max_len, int num_splits) {
  if (B < 1 || H < 1 || d_c < 1 || max_len < 0 || num_splits < 0) return 0;
  const int W = num_splits > 0 ? num_splits : auto_splits(B, H, max_len);
  return mla::ws_total_bytes(W, B, H, d_c);
}

}  // extern "C"

namespace {

// Validates the arguments of the partial pass and fills its argument block.  Returns MLA_OK or an
// error status; *fp8 / *generic report the selected kernel family.
int prepare_partial(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                    const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes, mla::PartialArgs* pa, bool* generic,
                    bool* fp8, bool* paged) {
  if (B < 0 || H < 1 || d_c < 4 || (d_c % 4) != 0 || d_R < 1 || max_len < 0 || num_splits < 0)
    return MLA_ERR_SHAPE;
  if (B > mla::kMaxB) return MLA_ERR_UNSUPPORTED;
  if (!known_dtype(q_dtype)) return MLA_ERR_DTYPE;
  if (!cache) return MLA_ERR_NULL;
  if (!known_dtype(cache->latent_dtype) || !known_dtype(cache->rope_dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(scale) || !(scale > 0.f)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_abs || !q_R || !seq_lens || !cache->latent || !cache->rope) return MLA_ERR_NULL;
  if (cache->latent_stride_tok < 1 || cache->rope_stride_tok < 1 || cache->latent_stride_b < 0 ||
      cache->rope_stride_b < 0)
    return MLA_ERR_SHAPE;
  *paged = cache->block_table != nullptr;
  if (*paged) {
    if (cache->page_size < 1 || cache->max_pages < 1) return MLA_ERR_SHAPE;
    if ((int64_t)cache->max_pages * cache->page_size < (int64_t)max_len) return MLA_ERR_SHAPE;
  }
  const int W = num_splits > 0 ? num_splits : auto_splits(B, H, max_len);
  if (W > 65535) return MLA_ERR_SHAPE;
  const size_t need = mla::ws_total_bytes(W, B, H, d_c);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_UNSUPPORTED;

  if (q_dtype == MLA_F32 && cache->latent_dtype == MLA_F32 && cache->rope_dtype == MLA_F32) {
    if (d_c > 1024 || d_R > 256 || H > 65535) return MLA_ERR_UNSUPPORTED;
    *generic = true;
    *fp8 = false;
  } else if (q_dtype == MLA_BF16 && (cache->latent_dtype == MLA_BF16 || cache->latent_dtype == MLA_FP8_E4M3) &&
             cache->rope_dtype == MLA_BF16) {
    *generic = false;
    *fp8 = cache->latent_dtype == MLA_FP8_E4M3;
    if (d_c != 512 || d_R != 64 || !(H == 32 || H == 64 || H == 128)) return MLA_ERR_UNSUPPORTED;
    if (*paged && (cache->page_size % mla::kTile) != 0) return MLA_ERR_UNSUPPORTED;
    if (*fp8 && !cache->latent_scale) return MLA_ERR_NULL;
    const int les = *fp8 ? 1 : 2;
    if (!aligned16(cache->latent) || !aligned16(cache->rope) || !aligned16(q_abs) || !aligned16(q_R) ||
        ((cache->latent_stride_tok * les) % 16) != 0 || ((cache->latent_stride_b * les) % 16) != 0 ||
        ((cache->rope_stride_tok * 2) % 16) != 0 || ((cache->rope_stride_b * 2) % 16) != 0 ||
        (*fp8 && (((uintptr_t)cache->latent_scale & 3u) != 0 || cache->scale_stride_b < 0)))
      return MLA_ERR_UNSUPPORTED;
  } else {
    return MLA_ERR_UNSUPPORTED;
  }

  pa->q_abs = q_abs;
  pa->q_R = q_R;
  pa->latent = cache->latent;
  pa->rope = cache->rope;
  pa->lscale = cache->latent_scale;
  pa->block_table = cache->block_table;
  pa->lat_sb = cache->latent_stride_b;
  pa->lat_st = cache->latent_stride_tok;
  pa->rope_sb = cache->rope_stride_b;
  pa->rope_st = cache->rope_stride_tok;
  pa->scale_sb = cache->scale_stride_b;
  pa->page_size = *paged ? cache->page_size : 1;
  pa->max_pages = *paged ? cache->max_pages : 0;
  pa->seq_lens = seq_lens;
  pa->B = B;
  pa->H = H;
  pa->d_c = d_c;
  pa->d_R = d_R;
  pa->W = W;
  pa->sl2 = scale * 1.4426950408889634f;
  pa->ws_acc = (float*)workspace;
  pa->ws_ml = (float*)((char*)workspace + mla::ws_ml_off(W, B, H, d_c));
  pa->ws_prefix = (int*)((char*)workspace + mla::ws_prefix_off(W, B, H, d_c));
  pa->ws_cnt = (int*)((char*)workspace + mla::ws_cnt_off(W, B, H, d_c));
  pa->warm = nullptr;
  pa->warm_bytes = 0;
  pa->extra = 0;
  // Small bf16 batches: the small-batch kernel, one workgroup per (split, 32-head block).
  // Otherwise, with few splits, the heads of the large-batch kernel are split into two groups of
  // workgroups, so that each workgroup loads and stores half as much per tile (its fixed costs
  // dominate there); two groups still fit on the chip for W <= 128.
  pa->small = (!*generic && !*fp8 && B <= mla::kSmallMaxB && total_tiles_bound(B, max_len) <= kSmallTiles) ? 1 : 0;
  pa->hgroups = pa->small ? H / 32 : (!*generic && H == 128 && W <= 128) ? 2 : 1;
  return MLA_OK;
}

// MI355X compute units (one partial-pass workgroup fills one), and the most workgroups a partial
// pass adds to warm a buffer (64 read a 16.8 MB weight well within a small-batch pass)
constexpr int kCUs = 256;
constexpr int kWarmWGs = 64;

int launch_partial(const mla::PartialArgs& pa, bool generic, bool fp8, bool paged, hipStream_t s) {
  if (generic) return hip_status(mla::launch_partial_f32(pa, s));
  if (pa.small) return hip_status(mla::launch_partial_small(pa, paged, s));
  return hip_status(mla::launch_partial_mfma(pa, fp8, paged, s));
}

int prepare_combine(const int32_t* seq_lens, int max_len, int B, int H, int d_c, int num_splits,
                    const void* workspace, size_t workspace_bytes, float* o_latent, float* lse,
                    mla::CombineArgs* ca) {
  if (B < 0 || H < 1 || d_c < 4 || (d_c % 4) != 0 || max_len < 0 || num_splits < 0) return MLA_ERR_SHAPE;
  if (B > mla::kMaxB) return MLA_ERR_UNSUPPORTED;
  if (B == 0) return MLA_OK;
  if (!seq_lens || !o_latent) return MLA_ERR_NULL;
  const int W = num_splits > 0 ? num_splits : auto_splits(B, H, max_len);
  if (W > 65535) return MLA_ERR_SHAPE;
  const size_t need = mla::ws_total_bytes(W, B, H, d_c);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(o_latent)) return MLA_ERR_UNSUPPORTED;
  ca->seq_lens = seq_lens;
  ca->B = B;
  ca->H = H;
  ca->d_c = d_c;
  ca->W = W;
  ca->ws_acc = (const float*)workspace;
  ca->ws_ml = (const float*)((const char*)workspace + mla::ws_ml_off(W, B, H, d_c));
  ca->ws_prefix = (const int*)((const char*)workspace + mla::ws_prefix_off(W, B, H, d_c));
  ca->ws_cnt = (int*)((char*)workspace + mla::ws_cnt_off(W, B, H, d_c));
  ca->ws_uv = (float*)((char*)workspace + mla::ws_uv_off(W, B, H, d_c));
  ca->o_latent = o_latent;
  ca->lse = lse;
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_decode_partial(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                       const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  mla::PartialArgs pa;
  bool generic = false, fp8 = false, paged = false;
  int st = prepare_partial(q_abs, q_R, q_dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale, num_splits,
                           workspace, workspace_bytes, &pa, &generic, &fp8, &paged);
  if (st != MLA_OK || B == 0) return st;
  return launch_partial(pa, generic, fp8, paged, (hipStream_t)stream);
}

int mla_decode_partial_warm(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                            const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                            int num_splits, void* workspace, size_t workspace_bytes, const void* warm,
                            size_t warm_bytes, void* stream) {
  mla::PartialArgs pa;
  bool generic = false, fp8 = false, paged = false;
  int st = prepare_partial(q_abs, q_R, q_dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale, num_splits,
                           workspace, workspace_bytes, &pa, &generic, &fp8, &paged);
  if (st != MLA_OK || B == 0) return st;
  if (warm_bytes > 0 && !warm) return MLA_ERR_NULL;
  if (warm_bytes > 0 && ((uintptr_t)warm & 3u) != 0) return MLA_ERR_UNSUPPORTED;
  // up to kWarmWGs extra workgroups on otherwise idle CUs warm the buffer; the fp32 kernel has none
  if (!generic && warm_bytes >= 4 && pa.W * pa.hgroups < kCUs) {
    pa.warm = warm;
    pa.warm_bytes = (int64_t)warm_bytes;
    pa.extra = std::min(kWarmWGs, kCUs - pa.W * pa.hgroups);
    // keep the block-index stride W + extra a multiple of 8 (one XCD per split in the
    // small-batch kernel) when that leaves a warm-up workgroup
    const int r = (pa.W + pa.extra) % 8;
    if (r != 0 && pa.extra > r) pa.extra -= r;
  }
  return launch_partial(pa, generic, fp8, paged, (hipStream_t)stream);
}

int mla_decode_combine(const int32_t* seq_lens, int max_len, int B, int H, int d_c, int num_splits,
                       const void* workspace, size_t workspace_bytes, float* o_latent, float* lse, void* stream) {
  mla::CombineArgs ca;
  int st = prepare_combine(seq_lens, max_len, B, H, d_c, num_splits, workspace, workspace_bytes, o_latent, lse, &ca);
  if (st != MLA_OK || B == 0) return st;
  return hip_status(mla::launch_combine(ca, (hipStream_t)stream));
}

int mla_decode_attn(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                    const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes, float* o_latent, float* lse,
                    void* stream) {
  mla::PartialArgs pa;
  mla::CombineArgs ca;
  bool generic = false, fp8 = false, paged = false;
  int st = prepare_partial(q_abs, q_R, q_dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale, num_splits,
                           workspace, workspace_bytes, &pa, &generic, &fp8, &paged);
  if (st != MLA_OK || B == 0) return st;
  st = prepare_combine(seq_lens, max_len, B, H, d_c, num_splits, workspace, workspace_bytes, o_latent, lse, &ca);
  if (st != MLA_OK) return st;
  st = launch_partial(pa, generic, fp8, paged, (hipStream_t)stream);
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_combine(ca, (hipStream_t)stream));
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// mla_decode_attn_noalloc: mla_decode_attn with its workspace in a device array of this file
// (each device holds its own copy; its address is taken once per device at the first call).
// ------------------------------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices];   // device address of `scratch` per device, null = not taken yet

// The device address of the current device's scratch array (hipGetSymbolAddress once per device,
// with that device current).  The array's name is a host-side stand-in in host code, never an
// address to pass to a kernel.
int current_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kScratchDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (!p) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace

extern "C" {

size_t mla_decode_attn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

int mla_decode_attn_noalloc_splits(int B, int H, int d_c, int max_len) {
  if (B < 1 || H < 1 || d_c < 1 || max_len < 0) return 0;
  int W = auto_splits(B, H, max_len);
  while (W > 1 && mla::ws_total_bytes(W, B, H, d_c) > kNoAllocScratchBytes) --W;
  return mla::ws_total_bytes(W, B, H, d_c) <= kNoAllocScratchBytes ? W : 0;
}

int mla_decode_attn_noalloc(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                            const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                            int num_splits, float* o_latent, float* lse, void* stream) {
  if (B < 0 || H < 1 || d_c < 4 || max_len < 0 || num_splits < 0) return MLA_ERR_SHAPE;
  if (B == 0) return mla_decode_attn(q_abs, q_R, q_dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale,
                                     num_splits, nullptr, 0, o_latent, lse, stream);
  int W = num_splits;
  if (W == 0) {
    W = mla_decode_attn_noalloc_splits(B, H, d_c, max_len);
    if (W == 0) return MLA_ERR_WORKSPACE;   // even one split needs more than the array holds
  }
  if (mla::ws_total_bytes(W, B, H, d_c) > kNoAllocScratchBytes) return MLA_ERR_WORKSPACE;
  void* ws = nullptr;
  const int st = current_scratch(&ws);
  if (st != MLA_OK) return st;
  return mla_decode_attn(q_abs, q_R, q_dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale, W, ws,
                         kNoAllocScratchBytes, o_latent, lse, stream);
}

int mla_uv_out(const float* o_latent, const void* W_UV, int w_dtype, float* out, int B, int H, int d_h, int d_c,
               void* stream) {
  if (B < 0 || H < 1 || d_h < 1 || d_c < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(w_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!o_latent || !W_UV || !out) return MLA_ERR_NULL;
  hipStream_t s = (hipStream_t)stream;
  if (w_dtype == MLA_F32) return hip_status(mla::launch_uv_f32w(o_latent, (const float*)W_UV, out, B, H, d_h, d_c, s));
  if (w_dtype == MLA_BF16) {
    if (d_h == 128 && d_c == 512 && aligned16(o_latent) && aligned16(W_UV))
      return hip_status(mla::launch_uv_bf16(o_latent, W_UV, out, B, H, s));
    return hip_status(mla::launch_uv_bf16w_generic(o_latent, W_UV, out, B, H, d_h, d_c, s));
  }
  return MLA_ERR_UNSUPPORTED;
}

int mla_decode_combine_uv(const int32_t* seq_lens, int max_len, int B, int H, int d_c, int num_splits,
                          const void* workspace, size_t workspace_bytes, const void* W_UV, int w_dtype, int d_h,
                          float* out, float* o_latent, float* lse, void* stream) {
  mla::CombineArgs ca;
  int st = prepare_combine(seq_lens, max_len, B, H, d_c, num_splits, workspace, workspace_bytes, o_latent, lse, &ca);
  if (st != MLA_OK) return st;
  if (d_h < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(w_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!W_UV || !out) return MLA_ERR_NULL;
  if (w_dtype == MLA_BF16 && d_h == 128 && d_c == 512 && B <= 4 && aligned16(W_UV))
    return hip_status(mla::launch_combine_uv(ca, W_UV, out, (hipStream_t)stream));
  st = hip_status(mla::launch_combine(ca, (hipStream_t)stream));
  if (st != MLA_OK) return st;
  return mla_uv_out(o_latent, W_UV, w_dtype, out, B, H, d_h, d_c, stream);
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// The whole decode step behind one call: the one-launch form for one bf16 sequence at the V3 head
// sizes, otherwise mla_absorb_q -> mla_decode_partial_warm -> mla_decode_combine_uv.
// ------------------------------------------------------------------------------------------------
namespace {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];   // compute units per device, 0 = not queried yet

int current_device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int c = __atomic_load_n(&g_cu_count[dev], __ATOMIC_RELAXED);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&g_cu_count[dev], c, __ATOMIC_RELAXED);
  }
  return c;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// data region of the multi-kernel form: q_abs (up to 4-byte elements), o_latent, decode workspace
size_t step_multi_data_bytes(int B, int H, int d_c, int max_len) {
  return round256((size_t)B * H * d_c * 4) + round256((size_t)B * H * d_c * 4) +
         mla_decode_workspace_bytes(B, H, d_c, max_len, 0);
}
size_t step_one_data_bytes() {
  return round256(mla::kStepQpBytes) + round256(mla::kStepMlBytes) + round256(mla::kStepAccBytes);
}

bool step_one_launch_fits(int dtype, const mla_cache_desc* c, int max_len, int B, int H, int d_h, int d_c, int d_R,
                          const void* q_C, const void* q_R, const void* W_UK, const void* W_UV, const void* q_abs,
                          const float* o_latent) {
  if (dtype != MLA_BF16 || c->latent_dtype != MLA_BF16 || c->rope_dtype != MLA_BF16) return false;
  if (B != 1 || H != 128 || d_h != 128 || d_c != 512 || d_R != 64) return false;
  if (max_len > mla::kStepSplits * mla::kStepTiles * mla::kTile) return false;
  if (c->block_table && (c->page_size % mla::kTile) != 0) return false;
  if (!aligned16(q_C) || !aligned16(q_R) || !aligned16(W_UK) || !aligned16(W_UV) || !aligned16(c->latent) ||
      !aligned16(c->rope) || ((c->latent_stride_tok * 2) % 16) != 0 || ((c->latent_stride_b * 2) % 16) != 0 ||
      ((c->rope_stride_tok * 2) % 16) != 0 || ((c->rope_stride_b * 2) % 16) != 0)
    return false;
  if ((q_abs && ((uintptr_t)q_abs & 3u) != 0) || (o_latent && !aligned16(o_latent))) return false;
  return current_device_cus() >= mla::kStepWGs;
}

}  // namespace

extern "C" {

size_t mla_decode_step_workspace_bytes(int B, int H, int d_c, int max_len) {
  if (B < 1 || H < 1 || d_c < 1 || max_len < 0) return 0;
  size_t data = step_multi_data_bytes(B, H, d_c, max_len);
  if (B == 1 && H == 128 && d_c == 512) data = std::max(data, step_one_data_bytes());
  return mla::kStepFlagBytes + data;
}

int mla_decode_step_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return MLA_ERR_NULL;
  if (workspace_bytes < mla::kStepFlagBytes) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_step_zero((int*)workspace, (int64_t)(mla::kStepFlagBytes / 4), (hipStream_t)stream));
}

int mla_decode_step(const void* q_C, const void* q_R, const void* W_UK, const void* W_UV, int dtype,
                    const mla_cache_desc* cache, const int32_t* seq_lens, int max_len, int B, int H, int d_h,
                    int d_c, int d_R, float scale, void* workspace, size_t workspace_bytes, void* q_abs,
                    float* o_latent, float* lse, float* out, void* stream) {
  if (B < 0 || H < 1 || d_h < 1 || d_c < 4 || d_R < 1 || max_len < 0) return MLA_ERR_SHAPE;
  if (B > mla::kMaxB) return MLA_ERR_UNSUPPORTED;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!cache) return MLA_ERR_NULL;
  if (!known_dtype(cache->latent_dtype) || !known_dtype(cache->rope_dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(scale) || !(scale > 0.f)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q_C || !q_R || !W_UK || !W_UV || !seq_lens || !out || !cache->latent || !cache->rope) return MLA_ERR_NULL;
  if (cache->latent_stride_tok < 1 || cache->rope_stride_tok < 1 || cache->latent_stride_b < 0 ||
      cache->rope_stride_b < 0)
    return MLA_ERR_SHAPE;
  if (cache->block_table && (cache->page_size < 1 || cache->max_pages < 1 ||
                             (int64_t)cache->max_pages * cache->page_size < (int64_t)max_len))
    return MLA_ERR_SHAPE;
  const size_t need = mla_decode_step_workspace_bytes(B, H, d_c, max_len);
  if (!workspace || workspace_bytes < need) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  char* data = ws + mla::kStepFlagBytes;
  if (step_one_launch_fits(dtype, cache, max_len, B, H, d_h, d_c, d_R, q_C, q_R, W_UK, W_UV, q_abs, o_latent)) {
    mla::StepArgs a;
    a.q_C = (const uint16_t*)q_C;
    a.q_R = (const uint16_t*)q_R;
    a.W_UK = (const uint16_t*)W_UK;
    a.W_UV = (const uint16_t*)W_UV;
    a.latent = cache->latent;
    a.rope = cache->rope;
    a.block_table = cache->block_table;
    a.lat_sb = cache->latent_stride_b;
    a.lat_st = cache->latent_stride_tok;
    a.rope_sb = cache->rope_stride_b;
    a.rope_st = cache->rope_stride_tok;
    a.page_size = cache->block_table ? cache->page_size : 1;
    a.seq_lens = seq_lens;
    a.sl2 = scale * 1.4426950408889634f;
    a.err = (int*)ws;
    a.fa = (int*)(ws + mla::kStepErrBytes);
    a.fb = a.fa + mla::kStepFaInts;
    a.qp = q_abs ? (uint16_t*)q_abs : (uint16_t*)data;
    a.part_ml = (float*)(data + round256(mla::kStepQpBytes));
    a.part_acc = (uint16_t*)(data + round256(mla::kStepQpBytes) + round256(mla::kStepMlBytes));
    a.out = out;
    a.o_latent = o_latent;
    a.lse = lse;
    return hip_status(mla::launch_step_b1(a, s));
  }
  // multi-kernel form
  const int qe = dtype == MLA_F32 ? 4 : 2;
  void* qa = q_abs ? q_abs : (void*)data;
  float* ol = o_latent ? o_latent : (float*)(data + round256((size_t)B * H * d_c * 4));
  char* dws = data + 2 * round256((size_t)B * H * d_c * 4);
  const size_t dws_bytes = mla_decode_workspace_bytes(B, H, d_c, max_len, 0);
  int st = mla_absorb_q(q_C, W_UK, qa, dtype, dtype, B, H, d_h, d_c, stream);
  if (st != MLA_OK) return st;
  st = mla_decode_partial_warm(qa, q_R, dtype, cache, seq_lens, max_len, B, H, d_c, d_R, scale, 0, dws, dws_bytes,
                               W_UV, (size_t)H * d_h * d_c * qe, stream);
  if (st != MLA_OK) return st;
  return mla_decode_combine_uv(seq_lens, max_len, B, H, d_c, 0, dws, dws_bytes, W_UV, dtype, d_h, out, ol, lse,
                               stream);
}

}  // extern "C"

extern "C" {

size_t mla_cache_append_workspace_bytes(int B, int D) {
  if (B < 1 || D < 512 || (D % 512) != 0) return 0;
  return mla::append_ws_bytes(B, D);
}

int mla_cache_append(const void* h, const void* W_DKV, const void* W_KR, int dtype, const int32_t* pos,
                     const mla_cache_desc* cache, int B, int D, int d_c, int d_R, float rope_base, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (B < 0 || D < 1 || d_c < 1 || d_R < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!cache) return MLA_ERR_NULL;
  if (!known_dtype(cache->latent_dtype) || !known_dtype(cache->rope_dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(rope_base) || !(rope_base > 0.f)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!h || !W_DKV || !W_KR || !pos || !cache->latent || !cache->rope) return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || cache->rope_dtype != MLA_BF16 ||
      !(cache->latent_dtype == MLA_BF16 || cache->latent_dtype == MLA_FP8_E4M3))
    return MLA_ERR_UNSUPPORTED;
  if (d_c != 512 || d_R != 64 || D < 512 || (D % 512) != 0 || B > 65535 || (int64_t)B * D * 2 >= ((int64_t)1 << 32))
    return MLA_ERR_UNSUPPORTED;
  const bool fp8 = cache->latent_dtype == MLA_FP8_E4M3;
  const bool paged = cache->block_table != nullptr;
  if (fp8 && !cache->latent_scale) return MLA_ERR_NULL;
  if (cache->latent_stride_tok < 1 || cache->rope_stride_tok < 1 || cache->latent_stride_b < 0 ||
      cache->rope_stride_b < 0 || (fp8 && cache->scale_stride_b < 0))
    return MLA_ERR_SHAPE;
  if (paged && (cache->page_size < 1 || cache->max_pages < 1)) return MLA_ERR_SHAPE;
  const int les = fp8 ? 1 : 2;
  if (!aligned16(h) || !aligned16(W_DKV) || !aligned16(W_KR) || !aligned16(cache->latent) ||
      !aligned16(cache->rope) || ((cache->latent_stride_tok * les) % 16) != 0 ||
      ((cache->latent_stride_b * les) % 16) != 0 || ((cache->rope_stride_tok * 2) % 16) != 0 ||
      ((cache->rope_stride_b * 2) % 16) != 0 || (fp8 && ((uintptr_t)cache->latent_scale & 3u) != 0))
    return MLA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < mla::append_ws_bytes(B, D)) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  mla::AppendArgs a;
  a.latent = const_cast<void*>(cache->latent);
  a.rope = const_cast<void*>(cache->rope);
  a.latent_scale = const_cast<float*>(cache->latent_scale);
  a.block_table = cache->block_table;
  a.lat_sb = cache->latent_stride_b;
  a.lat_st = cache->latent_stride_tok;
  a.rope_sb = cache->rope_stride_b;
  a.rope_st = cache->rope_stride_tok;
  a.scale_sb = cache->scale_stride_b;
  a.page_size = paged ? cache->page_size : 1;
  a.max_pages = paged ? cache->max_pages : 0;
  a.rope_base = rope_base;
  return hip_status(mla::launch_append(h, W_DKV, W_KR, pos, B, D, a, fp8, paged, (float*)workspace,
                                       (hipStream_t)stream));
}

}  // extern "C"

namespace {
// MHA comparison path: splits per (sequence, head) when the caller passes 0 -- about 1024
// workgroups over the batch, at most one per two 64-token tiles of the longest sequence
int mha_auto_splits(int B, int H, int max_len) {
  const int64_t tiles = ((int64_t)max_len + 63) / 64;
  int64_t w = std::min<int64_t>((tiles + 1) / 2, (1024 + (int64_t)B * H - 1) / ((int64_t)B * H));
  return (int)std::max<int64_t>(w, 1);
}
}  // namespace

extern "C" {

size_t mla_mha_decode_workspace_bytes(int B, int H, int max_len, int num_splits) {
  if (B < 1 || H < 1 || max_len < 0 || num_splits < 0) return 0;
  const int W = num_splits > 0 ? num_splits : mha_auto_splits(B, H, max_len);
  return mla::mha_ws_bytes(B, H, W);
}

int mla_mha_decode(const void* q, const void* k_cache, const void* v_cache, int dtype, const int32_t* seq_lens,
                   int max_len, int64_t cap, int B, int H, int d_k, int d_v, float scale, int num_splits,
                   void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream) {
  if (B < 0 || H < 1 || d_k < 1 || d_v < 1 || max_len < 0 || num_splits < 0 || cap < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(scale) || !(scale > 0.f)) return MLA_ERR_SHAPE;
  if ((int64_t)max_len > cap) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || d_k != 192 || d_v != 128) return MLA_ERR_UNSUPPORTED;
  if (B > 65535 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return MLA_ERR_UNSUPPORTED;
  const int W = num_splits > 0 ? num_splits : mha_auto_splits(B, H, max_len);
  if (W > 65535) return MLA_ERR_SHAPE;
  if (!workspace || workspace_bytes < mla::mha_ws_bytes(B, H, W)) return MLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  return hip_status(mla::launch_mha(q, k_cache, v_cache, seq_lens, B, H, cap, scale, W, (float*)workspace, out, lse,
                                    (hipStream_t)stream));
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// Projections around the attention core: the query side, the folded absorbed query projection,
// the output projection (and the offline folds that produce the folded weights).
// ------------------------------------------------------------------------------------------------
namespace {
bool proj_shape_ok(int N, int K) { return N >= 32 && (N % 32) == 0 && K >= 512 && (K % 512) == 0; }
// the MFMA projection addresses x with 32-bit byte offsets
bool proj_x_fits(int B, int K, int elem_bytes) { return (int64_t)B * K * elem_bytes < ((int64_t)1 << 32); }

mla::ProjArgs proj_args(const void* w0, const void* w1, int n_split, const void* x, int B, int N, int K) {
  mla::ProjArgs a{};
  a.w0 = (const uint16_t*)w0;
  a.w1 = (const uint16_t*)w1;
  a.n_split = n_split;
  a.n_cache = n_split;
  a.ldw = K;
  a.x = x;
  a.ldx = K;
  a.B = B;
  a.N = N;
  a.K = K;
  a.scale = 1.f;
  return a;
}
}  // namespace

extern "C" {

size_t mla_proj_workspace_bytes(int B, int N, int K) {
  if (B < 1 || N < 1 || K < 1) return 0;
  return mla::proj_ws_bytes(B, N, K);
}

size_t mla_query_workspace_bytes(int B, int D, int d_q, int H, int d_h, int d_R) {
  if (B < 1 || D < 1 || d_q < 1 || H < 1 || d_h < 1 || d_R < 1) return 0;
  const size_t a = mla::proj_ws_bytes(B, d_q, D);
  const size_t b = mla::proj_ws_bytes(B, H * (d_h + d_R), d_q);
  return a > b ? a : b;
}

int mla_query_proj(const void* h, const void* W_DQ, const void* W_UQ, const void* W_QR, int dtype,
                   const int32_t* pos, int B, int D, int d_q, int H, int d_h, int d_R, float rope_base, void* c_q,
                   void* q_C, void* q_R, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || D < 1 || d_q < 1 || H < 1 || d_h < 1 || d_R < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(rope_base) || !(rope_base > 0.f)) return MLA_ERR_SHAPE;
  if (B == 0) return MLA_OK;
  if (!h || !W_DQ || !W_UQ || !W_QR || !pos || !c_q || !q_C || !q_R) return MLA_ERR_NULL;
  if (dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  const int64_t n2 = (int64_t)H * (d_h + d_R);
  if (d_R != 64 || (d_h % 2) != 0 || ((H * d_h) % 8) != 0 || !proj_shape_ok(d_q, D) || n2 > (1 << 30) ||
      !proj_shape_ok((int)n2, d_q) || !proj_x_fits(B, D, 2))
    return MLA_ERR_UNSUPPORTED;
  if (!aligned16(h) || !aligned16(W_DQ) || !aligned16(W_UQ) || !aligned16(W_QR) || !aligned16(c_q) ||
      !aligned16(q_C) || !aligned16(q_R))
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla_query_workspace_bytes(B, D, d_q, H, d_h, d_R);
  if (need && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // c_q = W_DQ h, bf16
  mla::ProjArgs a = proj_args(W_DQ, W_DQ, d_q, h, B, d_q, D);
  a.y = c_q;
  a.ldy = d_q;
  hipError_t e = mla::launch_proj(a, false, true, (float*)workspace, s);
  if (e != hipSuccess) return hip_status(e);
  // [q_C ; q_R] = [W_UQ ; W_QR] c_q, the q_R rows rotated at pos
  mla::ProjArgs u = proj_args(W_UQ, W_QR, H * d_h, c_q, B, (int)n2, d_q);
  u.y = q_C;
  u.ldy = (int64_t)H * d_h;
  u.y1 = q_R;
  u.ldy1 = (int64_t)H * d_R;
  u.pos = pos;
  u.rope_base = rope_base;
  return hip_status(mla::launch_proj(u, false, true, (float*)workspace, s));
}

size_t mla_query_append_workspace_bytes(int B, int D, int d_q, int H, int d_h, int d_R, int d_c) {
  if (B < 1 || D < 1 || d_q < 1 || H < 1 || d_h < 1 || d_R < 1 || d_c < 1) return 0;
  const size_t a = mla::proj_ws_bytes(B, d_q + d_c + d_R, D);
  const size_t b = mla::proj_ws_bytes(B, H * (d_h + d_R), d_q);
  return a > b ? a : b;
}

int mla_query_proj_append(const void* h, const void* W_DQ, const void* W_UQ, const void* W_QR, const void* W_DKV,
                          const void* W_KR, int dtype, const int32_t* pos, const mla_cache_desc* cache, int B, int D,
                          int d_q, int H, int d_h, int d_R, int d_c, float rope_base, void* c_q, void* q_C, void* q_R,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || D < 1 || d_q < 1 || H < 1 || d_h < 1 || d_R < 1 || d_c < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!isfinite(rope_base) || !(rope_base > 0.f)) return MLA_ERR_SHAPE;
  if (!cache) return MLA_ERR_NULL;
  if (!known_dtype(cache->latent_dtype) || !known_dtype(cache->rope_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!h || !W_DQ || !W_UQ || !W_QR || !W_DKV || !W_KR || !pos || !c_q || !q_C || !q_R || !cache->latent ||
      !cache->rope)
    return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || cache->latent_dtype != MLA_BF16 || cache->rope_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  const int64_t n2 = (int64_t)H * (d_h + d_R);
  if (d_R != 64 || d_c != 512 || (d_h % 2) != 0 || ((H * d_h) % 8) != 0 || !proj_shape_ok(d_q, D) ||
      !proj_shape_ok(d_q + d_c + d_R, D) || n2 > (1 << 30) || !proj_shape_ok((int)n2, d_q) || !proj_x_fits(B, D, 2) ||
      B > 65535)
    return MLA_ERR_UNSUPPORTED;
  const bool paged = cache->block_table != nullptr;
  if (cache->latent_stride_tok < 1 || cache->rope_stride_tok < 1 || cache->latent_stride_b < 0 ||
      cache->rope_stride_b < 0)
    return MLA_ERR_SHAPE;
  if (paged && (cache->page_size < 1 || cache->max_pages < 1)) return MLA_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(W_DQ) || !aligned16(W_UQ) || !aligned16(W_QR) || !aligned16(W_DKV) ||
      !aligned16(W_KR) || !aligned16(c_q) || !aligned16(q_C) || !aligned16(q_R) || !aligned16(cache->latent) ||
      !aligned16(cache->rope) || ((cache->latent_stride_tok * 2) % 16) != 0 || ((cache->latent_stride_b * 2) % 16) != 0 ||
      ((cache->rope_stride_tok * 2) % 16) != 0 || ((cache->rope_stride_b * 2) % 16) != 0)
    return MLA_ERR_UNSUPPORTED;
  const size_t need = mla_query_append_workspace_bytes(B, D, d_q, H, d_h, d_R, d_c);
  if (need && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  // one pass over h: c_q = W_DQ h (to c_q), c = W_DKV h and RoPE_pos(W_KR h) (into the cache row)
  mla::ProjArgs a = proj_args(W_DQ, W_KR, d_q + d_c, h, B, d_q + d_c + d_R, D);
  a.y = c_q;
  a.ldy = d_q;
  a.pos = pos;
  a.rope_base = rope_base;
  a.dst_cache = 1;
  a.wc = (const uint16_t*)W_DKV;
  a.n_cache = d_q;
  a.cache.latent = const_cast<void*>(cache->latent);
  a.cache.rope = const_cast<void*>(cache->rope);
  a.cache.block_table = cache->block_table;
  a.cache.lat_sb = cache->latent_stride_b;
  a.cache.lat_st = cache->latent_stride_tok;
  a.cache.rope_sb = cache->rope_stride_b;
  a.cache.rope_st = cache->rope_stride_tok;
  a.cache.page_size = paged ? cache->page_size : 1;
  a.cache.max_pages = paged ? cache->max_pages : 0;
  a.cache.rope_base = rope_base;
  hipError_t e = mla::launch_proj(a, false, true, (float*)workspace, s);
  if (e != hipSuccess) return hip_status(e);
  // [q_C ; q_R] = [W_UQ ; W_QR] c_q, the q_R rows rotated at pos
  mla::ProjArgs u = proj_args(W_UQ, W_QR, H * d_h, c_q, B, (int)n2, d_q);
  u.y = q_C;
  u.ldy = (int64_t)H * d_h;
  u.y1 = q_R;
  u.ldy1 = (int64_t)H * d_R;
  u.pos = pos;
  u.rope_base = rope_base;
  return hip_status(mla::launch_proj(u, false, true, (float*)workspace, s));
}

int mla_absorb_q_folded(const void* c_q, const void* W_QK, int dtype, void* q_abs, int out_dtype, int B, int H,
                        int d_c, int d_q, void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || H < 1 || d_c < 1 || d_q < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype) || !known_dtype(out_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!c_q || !W_QK || !q_abs) return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || !(out_dtype == MLA_BF16 || out_dtype == MLA_F32)) return MLA_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)H * d_c;
  if (n > (1 << 30) || !proj_shape_ok((int)n, d_q) || !proj_x_fits(B, d_q, 2)) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(c_q) || !aligned16(W_QK) || !aligned16(q_abs)) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::proj_ws_bytes(B, (int)n, d_q);
  if (need && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  mla::ProjArgs a = proj_args(W_QK, W_QK, (int)n, c_q, B, (int)n, d_q);
  a.y = q_abs;
  a.ldy = n;
  return hip_status(mla::launch_proj(a, false, out_dtype == MLA_BF16, (float*)workspace, (hipStream_t)stream));
}

int mla_out_proj(const float* x, const void* W, int w_dtype, float* out, int B, int D, int K, void* workspace,
                 size_t workspace_bytes, void* stream) {
  if (B < 0 || D < 1 || K < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(w_dtype)) return MLA_ERR_DTYPE;
  if (B == 0) return MLA_OK;
  if (!x || !W || !out) return MLA_ERR_NULL;
  if (w_dtype != MLA_BF16 || !proj_shape_ok(D, K) || !proj_x_fits(B, K, 4)) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(W) || !aligned16(out)) return MLA_ERR_UNSUPPORTED;
  const size_t need = mla::proj_ws_bytes(B, D, K);
  if (need && (!workspace || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  if (need && !aligned16(workspace)) return MLA_ERR_UNSUPPORTED;
  mla::ProjArgs a = proj_args(W, W, D, x, B, D, K);
  a.y = out;
  a.ldy = D;
  return hip_status(mla::launch_proj(a, true, false, (float*)workspace, (hipStream_t)stream));
}

int mla_fold_q(const void* W_UQ, const void* W_UK, int dtype, void* W_QK, int H, int d_h, int d_c, int d_q,
               void* stream) {
  if (H < 1 || d_h < 1 || d_c < 1 || d_q < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!W_UQ || !W_UK || !W_QK) return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || (d_h % 32) != 0 || (d_c % 64) != 0 || (d_q % 64) != 0 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(W_UQ) || !aligned16(W_UK) || !aligned16(W_QK)) return MLA_ERR_UNSUPPORTED;
  mla::FoldArgs f{};
  f.A = (const uint16_t*)W_UK;           // A_h[m = k, i] = W_UK[h, i, k]
  f.a_sh = (int64_t)d_h * d_c;
  f.a_sm = 1;
  f.a_si = d_c;
  f.B = (const uint16_t*)W_UQ;           // B_h[i, n] = W_UQ[h d_h + i, n]
  f.b_sh = (int64_t)d_h * d_q;
  f.b_si = d_q;
  f.C = (uint16_t*)W_QK;                 // W_QK[h, k, n]
  f.c_sh = (int64_t)d_c * d_q;
  f.c_sm = d_q;
  f.H = H;
  f.M = d_c;
  f.Nc = d_q;
  f.inner = d_h;
  return hip_status(mla::launch_fold(f, (hipStream_t)stream));
}

int mla_fold_o(const void* W_O, const void* W_UV, int dtype, void* W_OV, int D, int H, int d_h, int d_c,
               void* stream) {
  if (D < 1 || H < 1 || d_h < 1 || d_c < 1) return MLA_ERR_SHAPE;
  if (!known_dtype(dtype)) return MLA_ERR_DTYPE;
  if (!W_O || !W_UV || !W_OV) return MLA_ERR_NULL;
  if (dtype != MLA_BF16 || (d_h % 32) != 0 || (d_c % 64) != 0 || (D % 64) != 0 || H > 65535) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(W_O) || !aligned16(W_UV) || !aligned16(W_OV)) return MLA_ERR_UNSUPPORTED;
  mla::FoldArgs f{};
  f.A = (const uint16_t*)W_O;            // A_h[m, i] = W_O[m, h d_h + i]
  f.a_sh = d_h;
  f.a_sm = (int64_t)H * d_h;
  f.a_si = 1;
  f.B = (const uint16_t*)W_UV;           // B_h[i, n] = W_UV[h, i, n]
  f.b_sh = (int64_t)d_h * d_c;
  f.b_si = d_c;
  f.C = (uint16_t*)W_OV;                 // W_OV[m, h d_c + n]
  f.c_sh = d_c;
  f.c_sm = (int64_t)H * d_c;
  f.H = H;
  f.M = D;
  f.Nc = d_c;
  f.inner = d_h;
  return hip_status(mla::launch_fold(f, (hipStream_t)stream));
}

}  // extern "C"
