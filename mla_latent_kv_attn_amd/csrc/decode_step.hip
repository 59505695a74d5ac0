// The whole absorbed decode step for one sequence in one launch (bf16, DeepSeek-V3 shape:
// H = 128, d_h = 128, d_c = 512, d_R = 64, at most 4096 cached tokens):
//
//   q'[h]    = W_UK[h]^T q_C[h]                                  (phase A, "the absorption trick")
//   s_j      = scale (q'[h] . c_j + q_R[h] . k_R,j),  a = softmax_j s   (phase B)
//   o_lat[h] = sum_j a_j c_j,   o[h] = W_UV[h] o_lat[h]          (phase B partials, phase C)
//
// ("Grouped-query and latent attention", sections "The absorption trick" and "Why a separate
// rotary key".)  At one sequence the step moves 33.5 MB of weights and 4.7 MB of cache, and each
// of the three separate passes is too short to get the memory system up to speed: a cold 16.8 MB
// stream over the whole chip takes about 6 us.  Here the three streams follow each other inside
// one launch and the phases hand their results to each other between workgroups.  Measured on
// the part, a CU fetching from HBM under full-chip load delivers only about 40 GB/s (each request
// waits the loaded latency and few are in flight per CU), so the work before the attention is
// spread by bytes per CU, not by workgroup count.
//
// Grid: 256 workgroups (one per CU; the LDS use forces that), 512 threads.  Waves 0-3 compute;
// waves 4-7 only move data into LDS and then take part in the workgroup's barriers, so no compute
// wave ever waits for a prefetch it did not need (s_waitcnt counts a wave's own memory operations
// in order).  Workgroup r sits on XCD r % 8; slot r / 8:
//  * slots 0-15: attention workgroup (split s = 4 (r % 8) + slot / 4 of the token tiles, head
//    block g = slot % 4 of 32 heads); the four head blocks of a split share an XCD and start on
//    different tiles, so a tile is read from HBM once and from that XCD's L2 three times;
//  * slots 16-31: projection workgroup for head h = 16 (r % 8) + slot - 16.
// Phase A: q' is cut into 1024 pieces (head, 64 latent columns), each from a 16 KB block of
// W_UK; an attention workgroup computes kPA of them (it also fetches 144 KB of tiles), a
// projection workgroup 8 - kPA.  The sums are rounded to bf16 and published.
// Phase B (attention): the split's (at most four) 32-token tiles are DMA'd into LDS by the loader
// waves, one 9 KB column slice per compute wave.  Wave w computes the partial scores of its
// latent columns 128 w .. + 127 and rope dimensions 16 w .. + 15 (9 MFMA 32x32x16 per tile), the
// four partials are added through LDS, the softmax of the split is exact (all of its scores are
// held at once: its maximum, then 2^(s - m)); compute wave w and loader wave 4 + w each multiply
// half of slice w's columns by the probabilities (4 MFMA per tile each).  The partial
// (m, l, acc / l) per head is published.
// Phase C (projection): W_UV[h] (128 KB) is DMA'd into LDS after the workgroup's absorb pieces
// (delayed and paced so that it leaves the fabric to the tiles); the 32 splits' partials of head h
// are merged (log-sum-exp) into o_lat[h] and multiplied by W_UV[h].
//
// Hand-over between workgroups: the producer writes its data with device-coherent stores (sc1),
// waits for them to complete (s_waitcnt vmcnt(0)), then sets one flag word per consumer (sc1
// store).  Each consumer polls only its own flag words (one vector load per poll), resets them
// after it has seen them all, and then reads the data with device-coherent loads.  There is no
// counter that many workgroups update or poll: measured on the box, 128 workgroups polling one
// counter saw it change about 5 us late.  Every wait gives up after 20 ms of wall-clock time
// (s_memrealtime) and records an error word, so every wave always reaches the end.  The flags
// must be zero before the first launch; every launch leaves them zero.
#include "partial_common.h"
#include "step_internal.h"

namespace mla {

namespace {
constexpr int kSSlice = 9216;                  // LDS bytes per tile and wave slice (latent 8 KB + rope 1 KB)
constexpr int kSRope = 8192;
constexpr int kRingBytes = kStepTiles * 4 * kSSlice;   // 147456
constexpr int kXBytes = 16384;                 // exchange buffer
constexpr int kLdsBytes = kRingBytes + kXBytes;        // 163840: the whole LDS of a CU
constexpr int kPRow = 272;                     // bytes per head row of the probabilities (128 tokens + pad)
constexpr int kLinvOff = 12288;                // exchange-buffer offset of the 1 / l array
constexpr unsigned kCoh = 16;                  // buffer cache policy: sc1 (device-coherent)
constexpr uint64_t kWaitTicks = 2000000;       // 20 ms at the 100 MHz s_memrealtime clock
#ifndef MLA_STEP_PACE
#define MLA_STEP_PACE 4
#endif
constexpr int kStepPace = MLA_STEP_PACE;       // s_sleep between the W_UV loads of a loader wave
#ifndef MLA_STEP_WUV_DELAY
#define MLA_STEP_WUV_DELAY 600
#endif
constexpr int kWuvDelay = MLA_STEP_WUV_DELAY;  // W_UV loads start this many 10 ns ticks after the workgroup
#ifndef MLA_STEP_STAGGER
#define MLA_STEP_STAGGER 1
#endif
constexpr bool kStagger = MLA_STEP_STAGGER != 0;  // head blocks of a split start on different tiles
#ifndef MLA_STEP_PA
#define MLA_STEP_PA 2
#endif
#ifndef MLA_STEP_TILES_AFTER_ABSORB
#define MLA_STEP_TILES_AFTER_ABSORB 1
#endif
// The absorb phase is cut into 1024 pieces (head, block of 64 latent columns); each attention
// workgroup takes kPA of them (one per compute wave), each projection workgroup 8 - kPA.
constexpr int kPA = MLA_STEP_PA;
constexpr bool kTilesAfterAbsorb = MLA_STEP_TILES_AFTER_ABSORB != 0;   // attention tiles after its pieces
static_assert(kPA >= 0 && kPA <= 4, "one piece per attention compute wave at most");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void coh_store4(const __amdgpu_buffer_rsrc_t& r, uint32_t off, const u32x4& v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kCoh);
}
__device__ __forceinline__ u32x4 coh_load4(const __amdgpu_buffer_rsrc_t& r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoh);
}
__device__ __forceinline__ u32x2 coh_load2(const __amdgpu_buffer_rsrc_t& r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCoh);
}
__device__ __forceinline__ void coh_store_i32(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Waits until the flag word of every active lane (lane < n) is nonzero, then clears them.
// Uniform; gives up after kWaitTicks and records the error.
__device__ __forceinline__ void wait_flags(int* flags, int lane, int n, int* err) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int* p = flags + (lane < n ? lane : 0);
  while (true) {
    const int v = lane < n ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 1;
    if (__builtin_amdgcn_ballot_w64(v == 0) == 0) break;
    if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
      if (lane == 0) coh_store_i32(err, 1);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (lane < n) coh_store_i32(p, 0);
  compiler_fence();
}

// Sum of 8 per-lane values over lane bits 5, 4, 3 (d = 32, 16, 8) by halving exchange; afterwards
// lane l holds the sum of value index (l >> 3) & 7.  (The pair passes through an empty asm so
// that the compiler keeps the selects as register selects.)
__device__ __forceinline__ float sum8_over_bits543(float (&v)[8], int lane) {
#pragma unroll
  for (int step = 0; step < 3; ++step) {
    const int d = 32 >> step;
    const int half = 4 >> step;
    const bool upper = (lane & d) != 0;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      float lo = v[i], hi = v[i + half];
      asm("" : "+v"(lo), "+v"(hi));
      const float send = upper ? lo : hi;
      const float keep = upper ? hi : lo;
      v[i] = keep + __shfl_xor(send, d, 64);
    }
  }
  return v[0];
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

}  // namespace

// DMA of column slice lw (latent columns 128 lw .. + 127, rope dimensions 16 lw .. + 15) of the
// 32-token tile t of the sequence into LDS at dst (9216 bytes): latent row q is 256 bytes with its
// 16-byte chunk c at position c ^ (q & 15), rope row q 32 bytes with chunk c at c ^ ((q >> 3) & 1).
// Rows past the sequence's end are loaded from its last row (finite data, masked later).
__device__ __forceinline__ void issue_tile(const StepArgs& a, int t, int len, int lw, uint8_t* dst) {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));
  const int tok0 = t * kTile;
  const int last = __builtin_amdgcn_readfirstlane(min(kTile, len - tok0) - 1);
  int64_t lrow0 = 0, rrow0 = 0;
  int tslot0 = tok0;
  if (a.block_table) {
    const int page = load_uniform_i32(a.block_table + tok0 / a.page_size);
    lrow0 = (int64_t)page * a.lat_sb;
    rrow0 = (int64_t)page * a.rope_sb;
    tslot0 = tok0 % a.page_size;
  }
  const uint8_t* lbase =
      (const uint8_t*)uniform_ptr((const uint8_t*)a.latent + (lrow0 + (int64_t)tslot0 * a.lat_st) * 2 + 256 * lw);
  const uint8_t* rbase =
      (const uint8_t*)uniform_ptr((const uint8_t*)a.rope + (rrow0 + (int64_t)tslot0 * a.rope_st) * 2 + 32 * lw);
  const uint32_t st = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  const uint32_t lstride = (uint32_t)a.lat_st * 2u;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int q = 4 * k + (ln >> 4);
    const uint32_t voff = (uint32_t)min(q, last) * lstride + 16u * (uint32_t)((ln & 15) ^ (q & 15));
    lds_dma16(lbase, voff, st + 1024 * k);
  }
  const int rq = ln >> 1;
  const uint32_t roff =
      (uint32_t)(min(rq, last) * (int)a.rope_st * 2) + 16u * (uint32_t)((ln & 1) ^ ((rq >> 3) & 1));
  lds_dma16(rbase, roff, st + kSRope);
}

// Phase A, one compute wave: pieces q0 .. q0 + NP - 1 of q', piece q = q'[hw][c0 .. c0 + 63] with
// hw = q / 8 and c0 = 64 (q % 8), from the 16 KB block of W_UK[hw] under those columns (all loads
// issued before any arithmetic).  Lane (rg, cc) sums rows 16 rg .. 16 rg + 15 of columns
// c0 + 8 cc .. + 7.  xq: NP * 256 bytes of LDS private to the wave.  The pieces are written with
// device-coherent stores, which complete before one flag per piece and consumer is set: compute
// wave (q % 8) / 2 of each of the 32 attention workgroups of head block hw / 32 (lane = split),
// flag index 2 (hw % 32) + q % 2 among that wave's 64 pieces.
template <int NP>
__device__ __forceinline__ void absorb_pieces(const StepArgs& a, int q0, int lane, uint8_t* xq) {
  const int rg = lane >> 3, cc = lane & 7;
  u32x4 qv[NP];
  u32x4 wv[NP][16];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int hw = (q0 + e) >> 3;
    qv[e] = u32x4{0u, 0u, 0u, 0u};
    if (lane < 16) qv[e] = *(const u32x4*)(a.q_C + hw * 128 + lane * 8);
  }
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int hw = (q0 + e) >> 3, c0 = ((q0 + e) & 7) * 64;
    const uint16_t* wp = a.W_UK + ((int64_t)hw * 128 + 16 * rg) * 512 + c0 + cc * 8;
#pragma unroll
    for (int k = 0; k < 16; ++k) wv[e][k] = *(const u32x4*)(wp + k * 512);
  }
#pragma unroll
  for (int e = 0; e < NP; ++e)
    if (lane < 16) *(u32x4*)(xq + e * 256 + lane * 16) = qv[e];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int hw = (q0 + e) >> 3, c0 = ((q0 + e) & 7) * 64;
    const u32x4 qa = *(const u32x4*)(xq + e * 256 + 32 * rg), qb = *(const u32x4*)(xq + e * 256 + 32 * rg + 16);
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t qw = k < 8 ? qa[(k & 7) >> 1] : qb[(k & 7) >> 1];
      const float q = (k & 1) ? bf16_hi(qw) : bf16_lo(qw);
#pragma unroll
      for (int c2 = 0; c2 < 4; ++c2) {
        acc[2 * c2] = fmaf(q, bf16_lo(wv[e][k][c2]), acc[2 * c2]);
        acc[2 * c2 + 1] = fmaf(q, bf16_hi(wv[e][k][c2]), acc[2 * c2 + 1]);
      }
    }
    // lane (rg, cc) now holds column c0 + 8 cc + rg; lanes with rg even store two columns
    const float s = sum8_over_bits543(acc, lane);
    const float s1 = __shfl_xor(s, 8, 64);
    if ((rg & 1) == 0)
      __hip_atomic_store((uint32_t*)(a.qp + hw * 512 + c0 + cc * 8 + rg), pack_bf16x2(s, s1), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  compiler_fence();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  compiler_fence();
  if (lane < kStepSplits) {
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      const int q = q0 + e, hw = q >> 3;
      coh_store_i32(a.fa + (((hw >> 5) * kStepSplits + lane) * 4 + ((q & 7) >> 1)) * 64 + 2 * (hw & 31) + (q & 1), 1);
    }
  }
}

// The pieces of compute wave `wave` of workgroup r: attention workgroups (r < 128) take pieces
// kPA r + wave for wave < kPA; projection workgroup r - 128 takes the 8 - kPA pieces after
// 128 kPA + (r - 128) (8 - kPA), spread over its four compute waves.
__device__ __forceinline__ void absorb_wave(const StepArgs& a, int r, int wave, int lane, uint8_t* xq) {
  if (r < 128) {
    if (wave < kPA) absorb_pieces<1>(a, kPA * r + wave, lane, xq);
    return;
  }
  constexpr int n = 8 - kPA;
  const int base = 128 * kPA + (r - 128) * n;
  const int cnt = n / 4 + (wave < n % 4 ? 1 : 0);
  const int q0 = base + wave * (n / 4) + min(wave, n % 4);
  if (cnt == 2) {
    absorb_pieces<2>(a, q0, lane, xq);
  } else if (cnt == 1) {
    absorb_pieces<1>(a, q0, lane, xq);
  }
}

// Value product of one wave over the split's tiles for latent column blocks cb0 and cb0 + 1 of
// slice cw (columns 128 cw + 32 cb .. + 31): acc[k] = O^T block (32 columns x 32 heads) of block
// cb0 + k.  Step 2 i + ks takes tokens 16 ks .. 16 ks + 15 of tile i, its operands read one step
// ahead (the probabilities from the head rows in xb, the latent operand through transposing LDS
// reads).
__device__ __forceinline__ void value_blocks(const uint8_t* lds, const uint8_t* xb, int cw, int cb0, int ntl, int lane,
                                             f32x16 (&acc)[2]) {
  const int hl = lane & 31, hf = lane >> 5;
  const int G = lane >> 4;
  const int vrow0 = 8 * (G >> 1) + ((lane & 15) >> 2);
  auto v_ops = [&](int stp, u32x4 (&av)[2], u32x4& pv) __attribute__((always_inline)) {
    const int i = min(stp >> 1, kStepTiles - 1), ks = stp & 1;
    const uint8_t* st = lds + (i * 4 + cw) * kSSlice;
    pv = *(const u32x4*)(xb + hl * kPRow + 2 * (kTile * i + 16 * ks + 8 * hf));
    const int R = 16 * ks + vrow0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int cch = 4 * (cb0 + k) + 2 * (G & 1) + ((lane & 3) >> 1);
      const uint8_t* pa = st + R * 256 + 16 * (cch ^ (R & 15)) + 8 * (lane & 1);
      const uint8_t* pb = st + (R + 4) * 256 + 16 * (cch ^ ((R + 4) & 15)) + 8 * (lane & 1);
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pa));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pb));
      const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
      av[k] = u32x4{l2[0], l2[1], h2[0], h2[1]};
    }
  };
  acc[0] = f32x16{};
  acc[1] = f32x16{};
  u32x4 ca[2], na[2], cp, np;
  v_ops(0, ca, cp);
#pragma unroll
  for (int stp = 0; stp < 2 * kStepTiles; ++stp) {
    if (stp + 1 < 2 * kStepTiles) v_ops(stp + 1, na, np);
    if ((stp >> 1) < ntl) {
      acc[0] = mfma32x32x16(ca[0], cp, acc[0]);
      acc[1] = mfma32x32x16(ca[1], cp, acc[1]);
    }
    ca[0] = na[0];
    ca[1] = na[1];
    cp = np;
  }
}

// The split's mean acc / l of blocks cb0, cb0 + 1 of slice cw as bf16 rows of the workspace: each
// 32 x 32 block is turned into head rows of 64 bytes through the LDS of tile 0's slice cw (free
// once every wave has passed the barrier after the value products; 16-byte chunk c of row n at
// position c ^ (n & 3)), then stored as 16-byte pieces of whole rows (a store of pieces scattered
// over 32 rows per lane pair issues far more slowly).
__device__ __forceinline__ void store_blocks(const StepArgs& a, uint8_t* lds, const uint8_t* xb, int cw, int cb0,
                                             int split, int g, int lane, const f32x16 (&acc)[2]) {
  const int hl = lane & 31, hf = lane >> 5;
  const float* linv = (const float*)(xb + kLinvOff);
  const float li = linv[hl];
  int ln = lane;
  asm volatile("" : "+v"(ln));
  uint8_t* tb = lds + cw * kSSlice;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      *(u32x2*)(tb + (cb0 + k) * 2048 + hl * 64 + 16 * (v4 ^ (hl & 3)) + 8 * hf) =
          u32x2{pack_bf16x2(acc[k][4 * v4] * li, acc[k][4 * v4 + 1] * li),
                pack_bf16x2(acc[k][4 * v4 + 2] * li, acc[k][4 * v4 + 3] * li)};
  const __amdgpu_buffer_rsrc_t pr = rsrc(a.part_acc);
  const int tc = ln & 3;
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int cb = cb0 + k;
      const int row = (ln >> 2) + 16 * ps;
      const u32x4 v = *(const u32x4*)(tb + cb * 2048 + row * 64 + 16 * (tc ^ (row & 3)));
      coh_store4(pr, (uint32_t)(((split * 128 + 32 * g + row) * 512 + 128 * cw + 32 * cb + 8 * tc) * 2), v);
    }
}

__global__ __launch_bounds__(512) void k_step_b1(StepArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];
  const int r = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int slot = r >> 3, xcd = r & 7;
  const bool attn = slot < 16;
  const int split = 4 * xcd + (slot >> 2);
  const int g = slot & 3;
  const int hproj = 16 * xcd + slot - 16;
  uint8_t* xb = lds + kRingBytes;
  const uint64_t t_entry = __builtin_amdgcn_s_memrealtime();

  // tile range of this split (attention): T tiles of the sequence cut evenly over kStepSplits
  auto tile_range = [&](int len, int& t0, int& ntl) __attribute__((always_inline)) {
    const int T = min(tiles_of(len), kStepSplits * kStepTiles);
    t0 = split * T / kStepSplits;
    ntl = (split + 1) * T / kStepSplits - t0;
  };

  // ------------------------------------------------------------------ loader waves
  if (wave >= 4) {
    const int lw = wave - 4;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // B0: the compute waves have published their q' pieces (workgroups that absorb)
    if (!attn || (kPA > 0 && kTilesAfterAbsorb)) lds_barrier();
    if (attn) {
      const int len = max(load_uniform_i32(a.seq_lens), 0);
      int t0, ntl;
      tile_range(len, t0, ntl);
      // the four head blocks of a split start on different tiles, so that only the first request for
      // a tile waits for HBM and the others find it in (or on its way into) the XCD's L2
      for (int k = 0; k < ntl; ++k) {
        const int i = kStagger ? (k + g) % ntl : k;
        issue_tile(a, t0 + i, len, lw, lds + (i * 4 + lw) * kSSlice);
      }
      if (kPA > 0 && !kTilesAfterAbsorb) lds_barrier();   // B0
    } else {
      // W_UV[h]: row i (1 KB) at LDS i * 1024, 16-byte chunk c at position c ^ (i & 63)
      const uint8_t* wbase = (const uint8_t*)a.W_UV + (int64_t)hproj * 128 * 1024;
      if (kWuvDelay > 0)
        while (__builtin_amdgcn_s_memrealtime() - t_entry < (uint64_t)kWuvDelay) __builtin_amdgcn_s_sleep(4);
      for (int k = 0; k < 32; ++k) {
        const int i = 32 * lw + k;
        lds_dma16(wbase + i * 1024, 16u * (uint32_t)(ln ^ (i & 63)),
                  __builtin_amdgcn_readfirstlane(lds_addr(lds + i * 1024)));
        if (kStepPace > 0) __builtin_amdgcn_s_sleep(kStepPace);
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    lds_barrier();   // B1: the prefetched data is in LDS
    // then the barriers the compute waves take after B1, so that every barrier of the workgroup
    // sees all eight waves: projection, three; attention, two per tile and the probabilities,
    // then this wave's half of the value product (V), its mean rows, and the published partials
    if (!attn) {
      for (int k = 0; k < 3; ++k) lds_barrier();
      return;
    }
    int t0, ntl;
    tile_range(max(load_uniform_i32(a.seq_lens), 0), t0, ntl);
    for (int k = 0; k < 2 * ntl + 1; ++k) lds_barrier();
    f32x16 acc[2];
    if (ntl > 0) value_blocks(lds, xb, lw, 2, ntl, lane, acc);
    lds_barrier();   // V
    if (ntl > 0) store_blocks(a, lds, xb, lw, 2, split, g, lane, acc);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compiler_fence();
    lds_barrier();   // the partial stores of every wave have completed
    return;
  }

  if (!attn || kPA > 0) {
    absorb_wave(a, r, wave, lane, xb + wave * 512);
    lds_barrier();   // B0
  }
  const int len = max(load_uniform_i32(a.seq_lens), 0);
  if (attn) {
    // ---------------------------------------------------------------- phase B: attention
    const int cw = wave;
    const int hl = lane & 31, hf = lane >> 5;
    int t0, ntl;
    tile_range(len, t0, ntl);
    // this wave's folded-query slice: latent k-steps 8 cw .. 8 cw + 7 (qf[0..7]) and rope k-step cw
    // after the flags of its producers
    wait_flags(a.fa + ((g * kStepSplits + split) * 4 + cw) * 64, lane, 64, a.err);
    const __amdgpu_buffer_rsrc_t qr = rsrc(a.qp);
    u32x4 qf[9];
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[j] = coh_load4(qr, (uint32_t)(((32 * g + hl) * 512 + 128 * cw + 16 * j + 8 * hf) * 2));
    qf[8] = *(const u32x4*)(a.q_R + (32 * g + hl) * 64 + 16 * cw + 8 * hf);
    lds_barrier();   // B1: tiles landed

    // scores: S[i] = partial S^T of tile i (32 tokens x 32 heads) over this wave's columns.  The
    // rows of a tile are read in a permuted order (bits 2 and 3 swapped) so that the softmax
    // layout below sees four consecutive tokens per lane.
    const int srow = pi_row(hl);
    const int sc_row = srow * 256, sc_x = srow & 15;
    const int rope_rd = kSRope + srow * 32 + 16 * (hf ^ ((srow >> 3) & 1));
    // The four tiles' chains advance together, one k-step at a time, with the next k-step's
    // operands read ahead (tiles past ntl read stale, in-bounds LDS; their scores are never used)
    f32x16 S[kStepTiles];
#pragma unroll
    for (int i = 0; i < kStepTiles; ++i) S[i] = f32x16{};
    auto a_op = [&](int i, int j) __attribute__((always_inline)) -> u32x4 {
      const uint8_t* st = lds + (i * 4 + cw) * kSSlice;
      return j < 8 ? *(const u32x4*)(st + sc_row + 16 * ((2 * j + hf) ^ sc_x)) : *(const u32x4*)(st + rope_rd);
    };
    {
      u32x4 cur[kStepTiles], nxt[kStepTiles];
#pragma unroll
      for (int i = 0; i < kStepTiles; ++i) cur[i] = a_op(i, 0);
#pragma unroll
      for (int j = 0; j < 9; ++j) {
        if (j < 8) {
#pragma unroll
          for (int i = 0; i < kStepTiles; ++i) nxt[i] = a_op(i, j + 1);
        }
#pragma unroll
        for (int i = 0; i < kStepTiles; ++i) S[i] = mfma32x32x16(cur[i], qf[j], S[i]);
#pragma unroll
        for (int i = 0; i < kStepTiles; ++i) cur[i] = nxt[i];
      }
    }
    // add the four waves' partials, one tile per round: wave w writes its block head-major (128 B
    // per head, chunk c of head n at position c ^ ((n >> 1) & 7)); then wave w reads heads
    // 8 w .. 8 w + 7, chunk sc (4 consecutive tokens) per lane
    const int sn = 8 * cw + (lane >> 3), sc = lane & 7;
    const int tok_c = 4 * ((sc >> 1) & 1) + 8 * (sc & 1) + 16 * (sc >> 2);
    f32x4 sv[kStepTiles];
#pragma unroll
    for (int i = 0; i < kStepTiles; ++i) {
      sv[i] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (i < ntl) {
        uint8_t* sb = xb + cw * 4096 + hl * 128;
        const int xs = (hl >> 1) & 7;
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *(f32x4*)(sb + 16 * ((2 * v4 + hf) ^ xs)) =
              f32x4{S[i][4 * v4], S[i][4 * v4 + 1], S[i][4 * v4 + 2], S[i][4 * v4 + 3]};
        lds_barrier();
        const uint8_t* rb = xb + sn * 128 + 16 * (sc ^ ((sn >> 1) & 7));
        f32x4 x = *(const f32x4*)rb;
#pragma unroll
        for (int q = 1; q < 4; ++q) x += *(const f32x4*)(rb + 4096 * q);
        const int tok = (t0 + i) * kTile + tok_c;
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[i][e] = tok + e < len ? x[e] * a.sl2 : -INFINITY;
        lds_barrier();
      }
    }
    // exact softmax over the split (base 2, scale folded in): max, probabilities, sum
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStepTiles; ++i)
      m = fmaxf(m, fmaxf(fmaxf(sv[i][0], sv[i][1]), fmaxf(sv[i][2], sv[i][3])));
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    m = fmaxf(m, __shfl_xor(m, 4, 64));
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < kStepTiles; ++i) {
      if (i < ntl) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(sv[i][e] - m);
        l += (p[0] + p[1]) + (p[2] + p[3]);
        *(u32x2*)(xb + sn * kPRow + 2 * (kTile * i + tok_c)) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      }
    }
    l += __shfl_xor(l, 1, 64);
    l += __shfl_xor(l, 2, 64);
    l += __shfl_xor(l, 4, 64);
    float* linv = (float*)(xb + kLinvOff);   // [32] 1 / l per head (0 for a split without tokens)
    if (sc == 0) linv[sn] = l > 0.f ? 1.f / l : 0.f;
    lds_barrier();   // the probabilities and 1 / l of all 32 heads are in LDS

    // value: compute wave cw takes latent column blocks 0, 1 of its slice, loader wave 4 + cw
    // blocks 2, 3; then, once no wave reads the tiles any more, both turn their blocks into the
    // split's mean rows
    f32x16 acc[2];
    if (ntl > 0) value_blocks(lds, xb, cw, 0, ntl, lane, acc);
    lds_barrier();   // V: the value products are done; the tile slices are free
    if (ntl > 0) store_blocks(a, lds, xb, cw, 0, split, g, lane, acc);
    if (sc == 0)
      __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(m), __float_as_uint(l)}, rsrc(a.part_ml),
                                            (int)((split * 128 + 32 * g + sn) * 8), 0, kCoh);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    compiler_fence();
    lds_barrier();   // every wave's partial stores have completed
    if (cw == 0 && lane < 32) coh_store_i32(a.fb + (32 * g + lane) * kStepSplits + split, 1);
    return;
  }

  // ------------------------------------------------------------------ phase C: merge + W_UV
  const int h = hproj;
  if (wave == 0) wait_flags(a.fb + h * kStepSplits, lane, kStepSplits, a.err);
  lds_barrier();   // B1: W_UV[h] in LDS, every split of head h published
  float* ws = (float*)(xb + 1024);        // [32] split weights
  uint16_t* olhi = (uint16_t*)(xb + 2048);   // [512] bf16 hi part of o_lat[h]
  uint16_t* ollo = (uint16_t*)(xb + 3072);   // [512] bf16 lo part
  float* half1 = (float*)(xb + 4096);     // [128] float4: the second half's sums
  float* stat = (float*)(xb + 8192);      // M, L
  // the partial rows of the 32 splits are loaded first (all in flight together), the splits'
  // (m, l) pairs by wave 0 just before them; the weights are ready before the rows have landed
  const int c4 = tid & 127, hs = tid >> 7;
  u32x2 ml = {0u, 0u};
  if (wave == 0 && lane < kStepSplits) ml = coh_load2(rsrc(a.part_ml), (uint32_t)((lane * 128 + h) * 8));
  const __amdgpu_buffer_rsrc_t pr = rsrc(a.part_acc);
  u32x2 x[kStepSplits / 2];
#pragma unroll
  for (int u = 0; u < kStepSplits / 2; ++u)
    x[u] = coh_load2(pr, (uint32_t)((((hs + 2 * u) * 128 + h) * 512 + 4 * c4) * 2));
  if (wave == 0) {
    const float ms = lane < kStepSplits ? __uint_as_float(ml[0]) : -INFINITY;
    const float ls = lane < kStepSplits ? __uint_as_float(ml[1]) : 0.f;
    float M = ms;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d, 64));
    const float w = (ms == -INFINITY || M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    float L = w * ls;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) L += __shfl_xor(L, d, 64);
    // split s contributes l_s 2^(m_s - M) / L times its mean acc_s / l_s
    if (lane < kStepSplits) ws[lane] = L > 0.f ? w * ls / L : 0.f;
    if (lane == 0) {
      stat[0] = M;
      stat[1] = L;
    }
  }
  lds_barrier();
  // o_latent and lse are stored at the very end: a store in flight before the MFMA work below
  // would make the compiler wait for it before reusing its registers
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  {
    // thread t: columns 4 (t % 128) .. + 3 over splits t / 128 + 2 u
#pragma unroll
    for (int u = 0; u < kStepSplits / 2; ++u) {
      const float w = ws[hs + 2 * u];
      const f32x4 xv = {bf16_lo(x[u][0]), bf16_hi(x[u][0]), bf16_lo(x[u][1]), bf16_hi(x[u][1])};
      // a split without tokens has weight 0 and never wrote its rows: select, do not multiply
      if (w != 0.f) o += w * xv;
    }
    if (hs == 1) *(f32x4*)(half1 + 4 * c4) = o;
    lds_barrier();
    if (hs == 0) {
      o += *(const f32x4*)(half1 + 4 * c4);

      // o_lat split into bf16 hi + lo parts for the W_UV product below
      const uint32_t h01 = pack_bf16x2(o[0], o[1]), h23 = pack_bf16x2(o[2], o[3]);
      const uint32_t l01 = pack_bf16x2(o[0] - bf16_lo(h01), o[1] - bf16_hi(h01));
      const uint32_t l23 = pack_bf16x2(o[2] - bf16_lo(h23), o[3] - bf16_hi(h23));
      *(u32x2*)(olhi + 4 * c4) = u32x2{h01, h23};
      *(u32x2*)(ollo + 4 * c4) = u32x2{l01, l23};
    }
    lds_barrier();
  }
  {
    // out[h][i] = sum_k W_UV[h][i][k] o_lat[k] on MFMA 16x16x32 (bf16): wave w takes rows
    // 32 w .. 32 w + 31 (two 16-row blocks).  A = W_UV rows from LDS (chunk c of row i at
    // position c ^ (i & 63)); B = o_lat split into bf16 hi (column 0) and lo (column 1) parts
    // (from LDS), zero elsewhere, so that out = D[:, 0] + D[:, 1] keeps about 16 bits of o_lat.
    const int n = lane & 15, kq = lane >> 4;
    const uint16_t* bsrc = n == 0 ? olhi : ollo;
    u32x4 bq[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const u32x4 v = *(const u32x4*)(bsrc + 32 * st + 8 * kq);
      bq[st] = n < 2 ? v : u32x4{0u, 0u, 0u, 0u};
    }
    f32x4 d0 = {0.f, 0.f, 0.f, 0.f}, d1 = {0.f, 0.f, 0.f, 0.f};
    const int i0 = 32 * wave + n, i1 = i0 + 16;
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int c = 4 * st + kq;
      const u32x4 w0 = *(const u32x4*)(lds + i0 * 1024 + 16 * (c ^ (i0 & 63)));
      const u32x4 w1 = *(const u32x4*)(lds + i1 * 1024 + 16 * (c ^ (i1 & 63)));
      d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w0), __builtin_bit_cast(bf16x8, bq[st]),
                                                   d0, 0, 0, 0);
      d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w1), __builtin_bit_cast(bf16x8, bq[st]),
                                                   d1, 0, 0, 0);
    }
    // lane (n, kq) holds rows 4 kq + e (e = 0..3) of each block, column n: add columns 0 and 1
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      d0[e] += __shfl_xor(d0[e], 1, 64);
      d1[e] += __shfl_xor(d1[e], 1, 64);
    }
    if (n == 0) {
      *(f32x4*)(a.out + h * 128 + 32 * wave + 4 * kq) = d0;
      *(f32x4*)(a.out + h * 128 + 32 * wave + 16 + 4 * kq) = d1;
    }
  }
  if (hs == 0 && a.o_latent) *(f32x4*)(a.o_latent + h * 512 + 4 * c4) = o;
  if (a.lse && tid == 0) {
    const float M = stat[0], L = stat[1];
    a.lse[h] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * 0.69314718055994530942f;
  }
}

// Zeroes the flag words (and the error word) of a step workspace: a plain fill kernel, so that it
// can be captured in a graph.
__global__ void k_step_zero(int* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_step_b1(const StepArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_step_b1, dim3(kStepWGs), dim3(512), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_step_zero(int* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(k_step_zero, dim3(blocks), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

}  // namespace mla
