// Partial pass of the absorbed decode for the DeepSeek-V3 shape (d_c = 512, d_R = 64), on
// gfx950 bf16 MFMA.  This is the kernel that streams the latent cache.
//
// Per token j of sequence b and head h the score is q'_h . c_j + q_R,h . k_R,j, scaled by
// 1/sqrt(d_h + d_R) ("Grouped-query and latent attention", sections "The absorption trick" and
// "Why a separate rotary key"); the output is the softmax-weighted latent sum sum_j a_j c_j, with
// W_UV applied later, once ("The absorption trick", value side).
//
// Design (one workgroup per CU, NWAVE = H/32 waves, wave w owns heads 32w .. 32w+31):
//  * The batch's token tiles (32 tokens) are split evenly over the workgroups (see
//    mla_internal.h).  A workgroup streams its tiles through a 3-stage LDS ring filled by
//    direct global->LDS loads (global_load_lds_dwordx4), without passing through registers:
//    while tile it is scored, tile it-1 is still being read by the value step and tile it+1 is
//    in flight.  Every tile is read from HBM once and shared by all heads of the workgroup.
//  * Software pipeline, one barrier per tile: score(it), value(it-1), softmax(it) form one basic
//    block, so the VALU work of the softmax overlaps the value MFMAs of the previous tile; the
//    probabilities, rescale factors and flags are double-buffered by tile parity.
//  * Score block per wave: S^T[32 tokens x 32 heads] = C_tile[32 x 576] . Qhat^T[576 x 32],
//    36 MFMA 32x32x16 steps.  Qhat = [q' ; q_R] of the wave's 32 heads stays in registers for the
//    whole segment.
//  * Online softmax in log2 units: each lane holds 16 scores of one head; the tile maximum needs
//    one cross-lane exchange (lane l <-> l^32).  The running maximum is only raised when a score
//    exceeds it by more than 2^8, which keeps every exp2 <= 256 and makes rescaling of the
//    accumulator rare; the partial (m, l, acc) stays exact in real arithmetic.
//  * Value block per wave: O^T[512 x 32 heads] += C_tile^T[512 x 32 tokens] . P[32 tokens x 32
//    heads].  The token order of the score MFMA's output rows is chosen (bits 2 and 3 of the row
//    index swapped when the tile is read) so that each lane's probabilities are directly the B
//    operand of the value MFMA; the latent operand comes from the same LDS tile through the
//    transposing reads ds_read_b64_tr_b16 (bf16) / ds_read_b64_tr_b8 (fp8).  No second copy.
//  * fp8 (OCP E4M3) latents stay 1 byte in LDS; they are widened to bf16 exactly after the LDS
//    read.  The per-token scale multiplies the latent part of the fp32 score and is folded into
//    the probabilities before the value MFMA, so the MFMA operands are the exact stored codes.
//  * Rows past a sequence's length in its last tile are loaded from the last valid row (finite
//    data) and masked to probability 0, so padding contents (even NaN) never reach the result.
#include <type_traits>

#include "partial_common.h"

namespace mla {


template <int NWAVE, bool FP8, bool PAGED>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_partial_mfma(PartialArgs a) {
  using LY = Layout<FP8>;
  constexpr int LPT = FP8 ? (16 + 4 + 4) / NWAVE : (32 + 4) / NWAVE;  // LDS-DMA loads per wave per tile
  static_assert(LPT < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNst * LY::kStage];
  __shared__ int P[kMaxB + 1];
  __shared__ __attribute__((aligned(16))) uint8_t qrs[NWAVE * 32 * 128];  // q_R of each wave's heads
  // fp8 variant: the last (32 - QREG) latent k-steps of Qhat live in LDS (its tiles are half the
  // size of bf16 tiles, which leaves room), freeing registers for the fp8 widening
  constexpr int QREG = FP8 ? (NWAVE == 1 ? 20 : 24) : 32;
  __shared__ __attribute__((aligned(16))) uint8_t qls[FP8 ? NWAVE * (32 - QREG) * 1024 : 16];
  // double-buffered by tile parity: tile it writes buffer it & 1 while tile it-1's is being read
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][NWAVE * 32 * kPbStride];  // bf16 probabilities
  __shared__ float alpha_s[2][NWAVE * 32];   // rescale factor of each head
  __shared__ __attribute__((aligned(16))) int flags_s[2][4];   // 1 if any of wave w's heads was rescaled

  if ((int)blockIdx.x >= a.W) {
    if (blockIdx.y != 0) return;
    // one of the a.extra warm-up workgroups: read one word of every 128-byte line of its share of
    // the warm-up buffer (the lines stay in the last-level cache for the next pass) and exit
    const int64_t nlines = (a.warm_bytes + 127) / 128;
    const int64_t per = (nlines + a.extra - 1) / a.extra;
    const int64_t l0 = (int64_t)(blockIdx.x - a.W) * per, l1 = min(nlines, l0 + per);
    const uint32_t* p = (const uint32_t*)a.warm;
    const int64_t last_word = a.warm_bytes / 4 - 1;
    uint32_t x = 0;
    for (int64_t l = l0 + threadIdx.x; l < l1; l += blockDim.x) x ^= p[min(l * 32, last_word)];
    asm volatile("" : : "v"(x));   // consume the loads
    return;
  }
  build_tile_prefix(a.seq_lens, a.B, P, nullptr);
  if (blockIdx.x == 0 && blockIdx.y == 0) {
    for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_prefix[i] = P[i];
    if (threadIdx.x == 0) a.ws_prefix[a.B + 1] = kPartBF16;
    for (int i = threadIdx.x; i < a.H; i += blockDim.x) a.ws_cnt[i] = 0;
  }
  const int NT = P[a.B];
  const int Wp = min(a.W, NT);
  const int w = blockIdx.x;
  if (w >= Wp) return;
  const int t_begin = (int)((int64_t)w * NT / Wp);
  const int t_end = (int)((int64_t)(w + 1) * NT / Wp);
  const int ntiles = t_end - t_begin;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H;
  const uint8_t* latent = (const uint8_t*)a.latent;
  const uint8_t* rope = (const uint8_t*)a.rope;

  // ---------------------------------------------------------------- loader: tile it -> stage
  // The loader walks the tiles in order with its own cursor (lb = sequence of the next tile to
  // load), two tiles ahead of the compute loop.
  // per-lane byte offsets of the DMA loads (16-byte chunk positions, XOR-swizzled)
  const uint32_t voff_x0 = (uint32_t)lane * 16u, voff_x1 = (uint32_t)(lane ^ 1) * 16u;
  const uint32_t voff_f8_0 = (uint32_t)((lane & 31)) * 16u, voff_f8_1 = (uint32_t)((lane & 31) ^ 1) * 16u;
  // Load cursor (uniform): the sequence lk_b of the next tile to load, its first tile lk_start,
  // the first tile of the sequence after it lk_next, and its length lk_len.
  int lk_b = seq_of_tile(P, a.B, t_begin);
  int lk_start = __builtin_amdgcn_readfirstlane(P[lk_b]);
  int lk_next = __builtin_amdgcn_readfirstlane(P[lk_b + 1]);
  int lk_len = load_uniform_i32(a.seq_lens + lk_b);
  // A tile's loads are LPT "jobs" per wave: latent rows (bf16) or row pairs (fp8), then the
  // fp8 scale rows, then the rope chunks.  advance() moves the cursor to the sequence of a tile
  // (a branch taken only at sequence ends); locate() computes where the tile lives (straight-line
  // code, so that its scalar loads can be scheduled under the MFMAs of the tile loop); job(k)
  // issues load k.
  constexpr int kLatJobs = FP8 ? 16 / NWAVE : 32 / NWAVE;
  constexpr int kScaleJobs = FP8 ? 4 / NWAVE : 0;
  struct TileSrc {
    const uint8_t* lbase;   // byte address of row 0 of the tile's latents
    const uint8_t* rbase;   // same for the rope keys
    const float* sbase;     // fp8: scale of row 0
    uint32_t st;            // LDS address of the stage
    int last;               // last valid row of the tile
  };
  auto advance = [&](int it) __attribute__((always_inline)) {
    const int t = t_begin + it;
    while (t >= lk_next) {
      ++lk_b;
      lk_start = lk_next;
      lk_next = __builtin_amdgcn_readfirstlane(P[lk_b + 1]);
      lk_len = load_uniform_i32(a.seq_lens + lk_b);
    }
  };
  auto locate = [&](int it) __attribute__((always_inline)) -> TileSrc {
    const int t = t_begin + it;
    const int b = __builtin_amdgcn_readfirstlane(lk_b);
    const int tok0 = (t - lk_start) * kTile;
    TileSrc ts;
    ts.last = min(kTile, lk_len - tok0) - 1;
    ts.st = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (it % kNst) * LY::kStage);
    int64_t lrow0, rrow0, srow0;  // element offsets of the page / sequence holding the tile
    int tslot0;                   // row of tok0 inside it
    if (PAGED) {
      const int page = load_uniform_i32(a.block_table + (int64_t)b * a.max_pages + tok0 / a.page_size);
      lrow0 = (int64_t)page * a.lat_sb;
      rrow0 = (int64_t)page * a.rope_sb;
      srow0 = (int64_t)page * a.scale_sb;
      tslot0 = tok0 % a.page_size;
    } else {
      lrow0 = (int64_t)b * a.lat_sb;
      rrow0 = (int64_t)b * a.rope_sb;
      srow0 = (int64_t)b * a.scale_sb;
      tslot0 = tok0;
    }
    ts.lbase = (const uint8_t*)uniform_ptr(latent + (lrow0 + (int64_t)tslot0 * a.lat_st) * (FP8 ? 1 : 2));
    ts.rbase = (const uint8_t*)uniform_ptr(rope + (rrow0 + (int64_t)tslot0 * a.rope_st) * 2);
    ts.sbase = FP8 ? (const float*)uniform_ptr(a.lscale + srow0 + tslot0) : nullptr;
    ts.last = __builtin_amdgcn_readfirstlane(ts.last);
    return ts;
  };
  auto prep = [&](int it) __attribute__((always_inline)) -> TileSrc {
    advance(it);
    return locate(it);
  };

  // vx0, vx1, vf0, vf1: opaque copies of the lane offsets (made by the caller), which keep them
  // from being folded into hoisted 64-bit pointers
  auto job = [&](const TileSrc& ts, int k, uint32_t vx0, uint32_t vx1, uint32_t vf0, uint32_t vf1) __attribute__((always_inline)) {
    const uint32_t lstride = (uint32_t)a.lat_st * (FP8 ? 1u : 2u);
    const int last = ts.last;
    if (k < kLatJobs) {
      if (!FP8) {
        // row r = wave + NWAVE k; since wave < NWAVE and NWAVE divides 8, bit 3 of r is bit 3 of
        // NWAVE k: the swizzle choice is a constant of the unrolled job
        // the row offset goes into the scalar base: the lane offset is then loop-invariant
        const int r = wave + NWAVE * k;
        const uint32_t roff = (uint32_t)min(r, last) * lstride;
        lds_dma16(ts.lbase + roff, (((NWAVE * k) >> 3) & 1) ? vx1 : vx0, ts.st + r * kLatStride);
      } else {
        const int pr = wave + NWAVE * k;       // row pair
        const uint32_t r0 = (uint32_t)min(2 * pr, last) * lstride;
        const uint32_t r1 = (uint32_t)min(2 * pr + 1, last) * lstride;
        lds_dma16(ts.lbase, (lane >> 5) ? r1 + vf1 : r0 + vf0, ts.st + pr * kLatStride);
      }
    } else if (k < kLatJobs + kScaleJobs) {
      const int q = wave + NWAVE * (k - kLatJobs);   // rows 8q .. 8q+7
      if (lane < 8) {
        const int dr = min(8 * q + lane, last);
        lds_dma4(ts.sbase, (uint32_t)dr * 4u, ts.st + LY::kScaleOff + 32 * q);
      }
    } else {
      // rope region is chunk-major: slot (c, r) = 32c + r holds bytes [16c, 16c+16) of row r;
      // job q writes chunks 2q and 2q+1 of all 32 rows
      const int q = wave + NWAVE * (k - kLatJobs - kScaleJobs);
      const int r = lane & 31;
      const int c = 2 * q + (lane >> 5);
      const int dr = min(r, last);
      lds_dma16(ts.rbase, (uint32_t)(dr * (int)a.rope_st * 2 + c * 16), ts.st + LY::kRopeOff + 1024 * q);
    }
  };
  auto issue_src = [&](TileSrc ts) __attribute__((always_inline)) {
    // opaque here: keeps the per-lane addresses derived from ts from being computed early and
    // held in registers across the tile loop
    asm volatile("" : "+s"(ts.lbase), "+s"(ts.rbase), "+s"(ts.sbase), "+s"(ts.st), "+s"(ts.last));
    uint32_t vx0 = voff_x0, vx1 = voff_x1, vf0 = voff_f8_0, vf1 = voff_f8_1;
    if constexpr (FP8) asm volatile("" : "+v"(vf0), "+v"(vf1));
#pragma unroll
    for (int k = 0; k < LPT; ++k) job(ts, k, vx0, vx1, vf0, vf1);
  };  auto issue = [&](int it) __attribute__((always_inline)) { issue_src(prep(it)); };


  // ---------------------------------------------------------------- per-lane constants
  constexpr int CPW = 16 / NWAVE;           // 32-column blocks of the latent owned by each wave
  const int hf = lane >> 5;                 // lane half
  const int h0 = blockIdx.y * 32 * NWAVE;   // first head of this workgroup's head group
  const int h = h0 + wave * 32 + (lane & 31);   // this lane's head in the score phase
  const int srow = pi_row(lane & 31);       // score-operand row (token within tile)
  const int G = lane >> 4;                  // 16-lane group
  // LDS read bases (bytes inside a stage); every k-step / column block adds an immediate offset
  //  score, bf16: row srow, chunk (2s + hf) ^ swz = 2s + (hf ^ swz)          -> base + 32 s
  //  score, fp8:  row srow, chunk s ^ (srow & 1), half hf                    -> even/odd bases + 16 s
  //  rope (chunk-major): slot 32 c + srow, c = 2q + hf                        -> base + 1024 q
  //  value, bf16: rows 16ks + vrow0 (+4), chunk 4cb + 2(G&1) + ((lane&3)>>1 ^ swz), +8 (lane&1)
  //                                                                           -> base + 16896 ks + 64 cb
  //  value, fp8:  rows 16ks + vrow0, chunk 2cb + ((G&1) ^ (vrow0&1)), +8 (lane&1) -> base + 8448 ks + 32 cb
  //  probabilities (pbuf): head row of 80 bytes, tokens 16ks + 8hf .. +7     -> base + 32 ks (+ 2560 hb)
  const int vrow0 = FP8 ? 8 * (G >> 1) + ((lane & 15) >> 1) : 8 * (G >> 1) + ((lane & 15) >> 2);
  int sc_base, sc_base_odd, val_base;
  if (!FP8) {
    sc_base = srow * kLatStride + 16 * (hf ^ ((srow >> 3) & 1));
    sc_base_odd = sc_base;
    val_base = vrow0 * kLatStride + 16 * (2 * (G & 1) + (((lane & 3) >> 1) ^ ((vrow0 >> 3) & 1))) + 8 * (lane & 1);
  } else {
    const int sw = srow & 1;
    sc_base = fp8_row_off(srow) + 16 * sw + 8 * hf;       // even s: chunk s + sw
    sc_base_odd = fp8_row_off(srow) - 16 * sw + 8 * hf;   // odd s:  chunk s - sw
    val_base = fp8_row_off(vrow0) + 16 * ((G & 1) ^ (vrow0 & 1)) + 8 * (lane & 1);
  }
  const int rope_base = LY::kRopeOff + 16 * (hf * 32 + srow);
  const int qr_base = 16 * (hf * 32 + (lane & 31));
  const int pb_base = (lane & 31) * kPbStride + 16 * hf;

  // ---------------------------------------------------------------- phases of one tile
  // score: S^T block of this wave's 32 heads for the tile in stage `st` (latent and rope parts
  // summed; fp8: the latent part multiplied by the per-token scale)
  u32x4 qf[QREG];
  using LatRaw = typename std::conditional<FP8, u32x2, u32x4>::type;
  auto widen = [&](const LatRaw& r) __attribute__((always_inline)) -> u32x4 {
    if constexpr (!FP8) return r;
    else return fp8x8_to_bf16x8(r);
  };
  // score(st, jobs, js): with jobs = true_type the loads of the tile described by js are issued
  // between the MFMAs (each load instruction takes tens of cycles to issue; there the MFMAs in
  // flight cover it)
  auto score = [&](const uint8_t* st, auto jobs, TileSrc js) __attribute__((always_inline)) -> f32x16 {
    constexpr bool kJobs = decltype(jobs)::value;
    if (kJobs) asm volatile("" : "+s"(js.lbase), "+s"(js.rbase), "+s"(js.sbase), "+s"(js.st), "+s"(js.last));
    f32x16 S = {}, S2 = {};
    // latent score operand: bf16 rows read as 16 bytes; fp8 rows read as 8 raw bytes and widened
    // to bf16 just before the MFMA that consumes them (keeps prefetched operands small)
    auto lat_op = [&](int s) __attribute__((always_inline)) -> LatRaw {
      if constexpr (!FP8) return *(const u32x4*)(st + sc_base + 32 * s);
      else return *(const u32x2*)(st + ((s & 1) ? sc_base_odd : sc_base) + 16 * s);
    };
    auto rope_op = [&](int q) __attribute__((always_inline)) -> u32x4 { return *(const u32x4*)(st + rope_base + 1024 * q); };
    auto q_lds = [&](int s) __attribute__((always_inline)) -> u32x4 {
      return *(const u32x4*)(qls + wave * (32 - QREG) * 1024 + qr_base + 1024 * (s - QREG));
    };
    // operands of k-steps s .. s + kPre - 1 are in flight while the MFMAs of step s issue
    constexpr int kPre = 4;
    LatRaw pre[kPre];
#pragma unroll
    for (int s = 0; s < kPre; ++s) pre[s] = lat_op(s);
#pragma unroll
    for (int s = 0; s < 32; s += 2) {
      const LatRaw a0 = pre[s % kPre], a1 = pre[(s + 1) % kPre];
      if (s + kPre < 32) {
        pre[s % kPre] = lat_op(s + kPre);
        pre[(s + 1) % kPre] = lat_op(s + kPre + 1);
      }
      asm volatile("" ::: "memory");
      // two accumulators: consecutive MFMAs are independent (a dependent 32x32x16 chain issues
      // at roughly 60% of the independent rate)
      const u32x4 q0 = (s < QREG) ? qf[s < QREG ? s : 0] : q_lds(s);
      const u32x4 q1 = (s + 1 < QREG) ? qf[s + 1 < QREG ? s + 1 : 0] : q_lds(s + 1);
      if constexpr (!FP8) {
        if (s == 0) {
          mfma_v_first(S, a0, q0);
          mfma_v_first(S2, a1, q1);
        } else {
          mfma_v(S, a0, q0);
          mfma_v(S2, a1, q1);
        }
      } else {
        S = mfma32x32x16(widen(a0), q0, S);
        S2 = mfma32x32x16(widen(a1), q1, S2);
      }
      if constexpr (kJobs) {
        const int k0 = (s / 2) * LPT / 16, k1 = (s / 2 + 1) * LPT / 16;   // constants after unrolling
        if (k0 < k1) {
          uint32_t vx0 = voff_x0, vx1 = voff_x1, vf0 = voff_f8_0, vf1 = voff_f8_1;
          if constexpr (FP8) asm volatile("" : "+v"(vf0), "+v"(vf1));
#pragma unroll
          for (int k = k0; k < k1; ++k) job(js, k, vx0, vx1, vf0, vf1);
        }
      }
    }
    {
      // rope k-steps: A = rope keys of the tile, B = q_R of the wave's heads (both LDS)
      const uint8_t* qrow = qrs + wave * 4096 + qr_base;
      const u32x4 b0 = *(const u32x4*)(qrow);
      const u32x4 b1 = *(const u32x4*)(qrow + 1024);
      const u32x4 b2 = *(const u32x4*)(qrow + 2048);
      const u32x4 b3 = *(const u32x4*)(qrow + 3072);
      const u32x4 r0 = rope_op(0), r1 = rope_op(1), r2 = rope_op(2), r3 = rope_op(3);
      if (FP8) {
        S += S2;  // latent part (scaled per token below); rope part accumulates in S2
        S2 = f32x16{};
        S2 = mfma32x32x16(r0, b0, S2);
        S2 = mfma32x32x16(r1, b1, S2);
        S2 = mfma32x32x16(r2, b2, S2);
        S2 = mfma32x32x16(r3, b3, S2);
      } else {
        mfma_v(S, r0, b0);
        mfma_v(S2, r1, b1);
        mfma_v(S, r2, b2);
        mfma_v(S2, r3, b3);
      }
    }
    if constexpr (!FP8) {
      // VALU reads of an MFMA result need 12 wait states after the MFMA that wrote it (what the
      // compiler itself inserts for this instruction); 16 here, tied to S and S2 so that no read
      // of them can be scheduled above it
      asm volatile("s_nop 15" : "+v"(S), "+v"(S2));
    } else {
      // keep the score block in VGPRs (the softmax works on it with VALU ops)
      asm volatile("" : "+v"(S), "+v"(S2));
    }
    const uint8_t* scl = st + LY::kScaleOff + 32 * hf;  // fp8 per-token scales of this lane's tokens
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float x = S[i];
      if (FP8) x *= *(const float*)(scl + 4 * (16 * (i >> 3) + (i & 7)));
      S[i] = x + S2[i];  // bf16: odd k-steps; fp8: rope part
    }
    return S;
  };

  // online softmax of one tile (log2 units); lane holds 16 tokens of head h: element i is token
  // 16 (i >> 3) + 8 hf + (i & 7) of the tile.  p_j = 2^(x_j * scale * log2e - m).  Writes the
  // bf16 probabilities, the head's rescale factor and the wave's rescale flag into buffer `pb`.
  // Branch-free (rows past nvalid are masked with selects; every lane stores), so that the
  // compiler can interleave it with the value MFMAs of the previous tile.
  float m_run = -INFINITY, l_run = 0.f;   // of head h (score phase)
  auto softmax = [&](f32x16 S, int nvalid, const uint8_t* st, int pb) __attribute__((always_inline)) {
    const int nv = nvalid - 8 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = (16 * (i >> 3) + (i & 7) < nv) ? S[i] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, S[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * a.sl2;
    const bool need = mx > m_run + 8.0f;
    const int any = __builtin_amdgcn_ballot_w64(need) != 0 ? 1 : 0;
    const float m_new = need ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 unless raised (m_run = -inf: 0)
    m_run = m_new;
    l_run *= alpha;
    alpha_s[pb][h - h0] = alpha;   // lanes l and l ^ 32 hold the same head and store the same value
    flags_s[pb][wave] = any;       // every lane stores the same value
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S[i] = __builtin_amdgcn_exp2f(fmaf(S[i], a.sl2, -m_run));
      l_run += S[i];
    }
    if (FP8) {
      const uint8_t* scl = st + LY::kScaleOff + 32 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i) S[i] *= *(const float*)(scl + 4 * (16 * (i >> 3) + (i & 7)));
    }
    const u32x4 pb0 = {pack_bf16x2(S[0], S[1]), pack_bf16x2(S[2], S[3]), pack_bf16x2(S[4], S[5]),
                       pack_bf16x2(S[6], S[7])};
    const u32x4 pb1 = {pack_bf16x2(S[8], S[9]), pack_bf16x2(S[10], S[11]), pack_bf16x2(S[12], S[13]),
                       pack_bf16x2(S[14], S[15])};
    uint8_t* pw = pbuf[pb] + wave * 32 * kPbStride + pb_base;
    *(u32x4*)(pw) = pb0;
    *(u32x4*)(pw + 32) = pb1;
  };

  // acc[hb * CPW + j]: O^T rows (latent columns) 32 * (wave * CPW + j) .. +31, heads 32 hb .. +31
  f32x16 acc[16];
  // rescale the accumulator blocks of every head block whose running maximum rose in the tile
  // that wrote buffer pb (in-place AGPR multiply, one register at a time)
  auto read_flags = [&](int pb) __attribute__((always_inline)) -> u32x4 { return *(const u32x4*)flags_s[pb]; };
  auto rescale_with = [&](const u32x4 fl, int pb) __attribute__((always_inline)) {
    uint32_t fany = 0;
#pragma unroll
    for (int hb = 0; hb < NWAVE; ++hb) fany |= fl[hb];
    if (__builtin_amdgcn_readfirstlane(fany) == 0) return;
#pragma unroll
    for (int hb = 0; hb < NWAVE; ++hb) {
      if (__builtin_amdgcn_readfirstlane(fl[hb])) {
        const float al = alpha_s[pb][hb * 32 + (lane & 31)];
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = acc[hb * CPW + j][v];
            float t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t) : "v"(al));
            acc[hb * CPW + j][v] = x;
          }
        }
      }
    }
  };  // one LDS read for the flags of every wave; usually none is set
  auto rescale = [&](int pb) __attribute__((always_inline)) { rescale_with(read_flags(pb), pb); };

  // value block: this wave's latent columns for all heads of the workgroup, from the tile in stage
  // st and the probabilities in buffer pb:  acc[hb][j] (O^T) += C^T . P
  auto value = [&](const uint8_t* st, int pb) __attribute__((always_inline)) {
    auto val_op = [&](int cb, int ks) __attribute__((always_inline)) -> LatRaw {
      if constexpr (!FP8) {
        const uint8_t* p0 = st + val_base + 16 * kLatStride * ks + 64 * cb;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 4 * kLatStride));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      } else {
        const uint8_t* p0 = st + val_base + 8 * kLatStride * ks + 32 * cb;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(p0));
        return __builtin_bit_cast(u32x2, v);
      }
    };
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 pbv[NWAVE];
#pragma unroll
      for (int hb = 0; hb < NWAVE; ++hb) pbv[hb] = *(const u32x4*)(pbuf[pb] + hb * 32 * kPbStride + pb_base + 32 * ks);
#pragma unroll
      for (int j0 = 0; j0 < CPW; j0 += 2) {
        const u32x4 av0 = widen(val_op(wave * CPW + j0, ks));
        const u32x4 av1 = widen(val_op(wave * CPW + j0 + 1, ks));
#pragma unroll
        for (int hb = 0; hb < NWAVE; ++hb) {
          acc[hb * CPW + j0] = mfma32x32x16(av0, pbv[hb], acc[hb * CPW + j0]);
          acc[hb * CPW + j0 + 1] = mfma32x32x16(av1, pbv[hb], acc[hb * CPW + j0 + 1]);
        }
      }
    }
  };
  // the output accumulator lives in AGPRs (pinned after the softmax that follows each value step,
  // which leaves the scheduler free to place the softmax between the value MFMAs)
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+a"(acc[i]));
  };

  // ---------------------------------------------------------------- pipeline
  // Tile it: wait for its loads, barrier (publishes the tile, the probabilities of tile it-1 and
  // frees the stage of tile it-2), issue the loads of tile it+1 into that stage, then
  //   score(it) ; value(it-1) ; softmax(it)
  // in one basic block, so that the softmax of tile it runs under the value MFMAs of tile it-1.
  // The first tile of a segment has no value step; the last one's value runs after the loop
  // (behind one more barrier), before the segment's partial is written.
  auto stage = [&](int i) __attribute__((always_inline)) -> const uint8_t* { return smem + (i % kNst) * LY::kStage; };
  issue(0);
  // source of tile it + 1, located during the previous tile (tile indices past the end are
  // clamped to the last tile: the lookup is then harmless and unused)
  TileSrc nsrc = prep(min(1, ntiles - 1));

  int it = 0;
  int cb_seq = seq_of_tile(P, a.B, t_begin);
  while (it < ntiles) {
    // ------------------------------------------------------------ one segment: sequence b
    while (t_begin + it >= P[cb_seq + 1]) ++cb_seq;
    const int b = __builtin_amdgcn_readfirstlane(cb_seq);
    const int it_end = min(ntiles, P[b + 1] - t_begin);
    const int len_b = load_uniform_i32(a.seq_lens + b);
    const int tok_base = (t_begin - P[b]) * kTile;   // token index of tile 0 of this workgroup in b

    {
      const uint16_t* qa = (const uint16_t*)a.q_abs + ((int64_t)b * H + h) * 512 + 8 * hf;
#pragma unroll
      for (int s = 0; s < QREG; ++s) qf[s] = *(const u32x4*)(qa + 16 * s);
      // k-steps QREG..31 -> this wave's LDS block, slot (2 (s - QREG) + hf) * 32 + head
#pragma unroll
      for (int s = QREG; s < 32; ++s)
        *(u32x4*)(qls + wave * (32 - QREG) * 1024 + 16 * ((2 * (s - QREG) + hf) * 32 + (lane & 31))) =
            *(const u32x4*)(qa + 16 * s);
      // q_R of head h -> this wave's LDS block, chunk-major (slot 32c + head)
      const uint16_t* qr = (const uint16_t*)a.q_R + ((int64_t)b * H + h) * 64;
#pragma unroll
      for (int c = hf; c < 8; c += 2) {
        const u32x4 v = *(const u32x4*)(qr + 8 * c);
        *(u32x4*)(qrs + wave * 4096 + 16 * (32 * c + (lane & 31))) = v;
      }
    }
    // Complete the folded-query loads (and the loads of tile it) here, once per segment, so that
    // no wait on them is left inside the tile loop.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;

    // first tile of the segment: score and softmax only
    {
      __builtin_amdgcn_s_waitcnt(lgkmcnt_imm0());   // q_R / folded-query LDS writes done
      lds_barrier();
      if (it + 1 < ntiles) issue_src(nsrc);
      const int nn = min(it + 2, ntiles - 1);
      advance(nn);
      nsrc = locate(nn);
      const int nvalid = min(kTile, len_b - (tok_base + it * kTile));
      const f32x16 S = score(stage(it), std::false_type{}, nsrc);
      softmax(S, nvalid, stage(it), it & 1);
      ++it;
    }
    // steady tiles that have a next tile to load: its loads are spread over the score MFMAs
    // (bf16; the fp8 variants issue them before the score, which keeps them free of spills)
    const int it_dma_end = min(it_end, ntiles - 1);
    for (; it < it_dma_end; ++it) {
      __builtin_amdgcn_s_waitcnt(vm_lgkm_imm0());   // tile it landed; this wave's probabilities written
      lds_barrier();
      // bf16: the flags are read here and acted on after the score MFMAs (the read's latency
      // hides under them); fp8: rescale first (fewer live registers across the score)
      u32x4 fl = {0u, 0u, 0u, 0u};
      if constexpr (FP8) {
        issue_src(nsrc);
        rescale((it - 1) & 1);
      } else {
        fl = read_flags((it - 1) & 1);
      }
      const TileSrc cur = nsrc;
      const int nn = min(it + 2, ntiles - 1);
      advance(nn);
      nsrc = locate(nn);
      const int nvalid = min(kTile, len_b - (tok_base + it * kTile));
      const f32x16 S = score(stage(it), std::integral_constant<bool, !FP8>{}, cur);
      if constexpr (!FP8) rescale_with(fl, (it - 1) & 1);
      value(stage(it - 1), (it - 1) & 1);
      softmax(S, nvalid, stage(it), it & 1);
      pin_acc();
    }
    // the workgroup's last tile, if it is in this segment (nothing left to load)
    if (it < it_end) {
      __builtin_amdgcn_s_waitcnt(vm_lgkm_imm0());
      lds_barrier();
      rescale((it - 1) & 1);
      const int nvalid = min(kTile, len_b - (tok_base + it * kTile));
      const f32x16 S = score(stage(it), std::false_type{}, nsrc);
      value(stage(it - 1), (it - 1) & 1);
      softmax(S, nvalid, stage(it), it & 1);
      pin_acc();
      ++it;
    }
    // value of the segment's last tile (its probabilities are published by this barrier)
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm0());
    lds_barrier();
    rescale((it - 1) & 1);
    value(stage(it - 1), (it - 1) & 1);
    pin_acc();

    // ------------------------------------------------------------ segment partial -> slot w + b
    {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      // opaque copy of the lane id: keeps these addresses from being hoisted out of the segment
      // loop (where they would occupy registers for the whole tile loop)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      // Row-major workspace of bf16 sums: each pair of 32x32 accumulator blocks (64 latent
      // columns of 32 heads) goes through this wave's part of the (now idle) probability buffers,
      // 144-byte rows, and leaves as 8 full 128-byte row segments per store instruction.  Every
      // wave has finished reading the probabilities once it passes this barrier.
      __builtin_amdgcn_s_waitcnt(lgkmcnt_imm0());
      lds_barrier();
      uint8_t* tb = &pbuf[0][0] + wave * 5120;
      const int trow = ln >> 3, tchunk = ln & 7;
      static_assert(CPW % 2 == 0 && 32 * 144 <= 5120, "store staging");
#pragma unroll
      for (int hb = 0; hb < NWAVE; ++hb) {
        uint16_t* dst = (uint16_t*)a.ws_acc + ((int64_t)(w + b) * H + h0 + hb * 32 + trow) * 512 +
                        32 * wave * CPW + 8 * tchunk;
#pragma unroll
        for (int j = 0; j < CPW; j += 2) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            // lane l holds latent columns 8 v4 + 4 (l >> 5) + 0..3 of block j + jj, head l & 31
            const f32x16& A = acc[hb * CPW + j + jj];
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
              *(u32x2*)(tb + (ln & 31) * 144 + (32 * jj + 8 * v4 + 4 * (ln >> 5)) * 2) =
                  u32x2{pack_bf16x2(A[4 * v4], A[4 * v4 + 1]), pack_bf16x2(A[4 * v4 + 2], A[4 * v4 + 3])};
          }
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *(u32x4*)(dst + (8 * q) * 512 + 32 * j) = *(const u32x4*)(tb + (8 * q + trow) * 144 + 16 * tchunk);
        }
      }
      if (ln < 32) *(f32x2*)(a.ws_ml + ((int64_t)(w + b) * H + h0 + wave * 32 + ln) * 2) = f32x2{m_run, l_tot};
    }
  }
}

hipError_t launch_partial_mfma(const PartialArgs& a, bool fp8, bool paged, hipStream_t s) {
  const int nw = a.H / 32 / a.hgroups;
#define MLA_LAUNCH(NW, F, PG)                                                              \
  hipLaunchKernelGGL((k_partial_mfma<NW, F, PG>), dim3(a.W + a.extra, a.hgroups), dim3(NW * 64), 0, s, a); \
  return hipGetLastError();
#define MLA_BY_NW(F, PG)            \
  if (nw == 4) { MLA_LAUNCH(4, F, PG) } \
  if (nw == 2) { MLA_LAUNCH(2, F, PG) } \
  if (nw == 1) { MLA_LAUNCH(1, F, PG) } \
  return hipErrorInvalidValue;
  if (fp8) {
    if (paged) { MLA_BY_NW(true, true) } else { MLA_BY_NW(true, false) }
  } else {
    if (paged) { MLA_BY_NW(false, true) } else { MLA_BY_NW(false, false) }
  }
#undef MLA_BY_NW
#undef MLA_LAUNCH
}

}  // namespace mla
