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
//    direct global->LDS loads (global_load_lds_dwordx4), so a tile arrives two tiles ahead of its
//    use without passing through registers.  Every tile is read from HBM once and shared by all
//    heads of the workgroup.
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
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kNst = 3;           // LDS ring stages
constexpr int kLatStride = 1056;  // bytes per LDS block of 1 KiB (+32 B pad: 8 dwords mod 64 banks)

template <bool FP8>
struct Layout {
  static constexpr int kLatStage = FP8 ? 16 * kLatStride : 32 * kLatStride;
  static constexpr int kRopeOff = kLatStage;
  static constexpr int kScaleOff = kLatStage + 4096;
  static constexpr int kStage = kLatStage + 4096 + (FP8 ? 128 : 0);
};

// score-operand row for lane l (0..31): bits 2 and 3 swapped
__device__ __forceinline__ int pi_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// rope chunk swizzle
__device__ __forceinline__ int rope_swz(int r) { return (r ^ (r >> 3)) & 7; }
// fp8 row offset inside a stage (two 512-byte rows per padded 1 KiB block)
__device__ __forceinline__ int fp8_row_off(int r) { return (r >> 1) * kLatStride + (r & 1) * 512; }

// Direct global->LDS loads (global_load_lds_dwordx4 / _dword): lane i writes bytes
// [lds + size*i, lds + size*(i+1)) from gbase + voff.  Issued through inline asm so that the
// compiler does not treat every later LDS read as dependent on them (it cannot tell the ring
// stages apart and would wait for all outstanding loads); completion is tracked explicitly with
// s_waitcnt vmcnt before the workgroup barrier that publishes a stage.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const MLA_LDS void*)p;
}
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(uniform_ptr(gbase)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void lds_dma4(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, %1" : : "v"(voff), "s"(uniform_ptr(gbase)),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 8 E4M3 codes -> 8 bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(u32x2 v) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(v[0], true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(v[1], true);
  // exact values: the bf16 bits are the high halves of the fp32 bits
  return u32x4{__builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(b[1]), __float_as_uint(b[0]), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(d[1]), __float_as_uint(d[0]), 0x07060302u)};
}

// uniform 32-bit load through the scalar data cache (s_load): keeps block-table lookups off the
// vector-memory counter that tracks the tile DMA loads
__device__ __forceinline__ int load_uniform_i32(const int32_t* p) {
  const uint64_t addr = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  const __attribute__((address_space(4))) int32_t* q =
      (const __attribute__((address_space(4))) int32_t*)(((uint64_t)hi << 32) | lo);
  return *q;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace

template <int NWAVE, bool FP8, bool PAGED>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_partial_mfma(PartialArgs a) {
  using LY = Layout<FP8>;
  constexpr int LPT = FP8 ? (16 + 4 + 4) / NWAVE : (32 + 4) / NWAVE;  // LDS-DMA loads per wave per tile
  static_assert(LPT < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kNst * LY::kStage];
  __shared__ int P[kMaxB + 1];
  __shared__ int L[kMaxB];
  __shared__ __attribute__((aligned(16))) uint8_t qrs[NWAVE * 32 * 128];  // q_R of each wave's heads

  build_tile_prefix(a.seq_lens, a.B, P, L);
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
  int lb = seq_of_tile(P, a.B, t_begin);
  auto issue = [&](int it) {
    // opaque copies: keep the 32-bit lane offsets from being folded into hoisted 64-bit pointers
    uint32_t vx0 = voff_x0, vx1 = voff_x1, vf0 = voff_f8_0, vf1 = voff_f8_1;
    asm volatile("" : "+v"(vx0), "+v"(vx1), "+v"(vf0), "+v"(vf1));
    const int t = t_begin + it;
    while (t >= P[lb + 1]) ++lb;
    const int b = __builtin_amdgcn_readfirstlane(lb);
    const int tok0 = (t - P[b]) * kTile;
    const int last = min(kTile, L[b] - tok0) - 1;  // last valid row of the tile
    const uint32_t st = __builtin_amdgcn_readfirstlane(lds_addr(smem) + (it % kNst) * LY::kStage);
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
    if (!FP8) {
#pragma unroll
      for (int i = 0; i < 32 / NWAVE; ++i) {
        const int r = wave + NWAVE * i;
        const int tok = tslot0 + min(r, last);
        const uint8_t* gb = latent + (lrow0 + (int64_t)tok * a.lat_st) * 2;
        lds_dma16(gb, ((r >> 3) & 1) ? vx1 : vx0, st + r * kLatStride);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16 / NWAVE; ++i) {
        const int pr = wave + NWAVE * i;       // row pair
        const int tok = tslot0 + min(2 * pr, last);
        const uint8_t* gb = latent + (lrow0 + (int64_t)tok * a.lat_st);
        const uint32_t second = (2 * pr + 1 <= last) ? (uint32_t)a.lat_st : 0u;  // row 2pr+1 (or 2pr again)
        lds_dma16(gb, (lane >> 5) ? second + vf1 : vf0, st + pr * kLatStride);
      }
#pragma unroll
      for (int i = 0; i < 4 / NWAVE; ++i) {
        const int q = wave + NWAVE * i;        // rows 8q .. 8q+7
        if (lane < 8) {
          const int tok_u = tslot0 + min(8 * q, last);
          const int dr = min(8 * q + lane, last) - min(8 * q, last);
          lds_dma4(a.lscale + srow0 + tok_u, (uint32_t)dr * 4u, st + LY::kScaleOff + 32 * q);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4 / NWAVE; ++i) {
      // rope region is chunk-major: slot (c, r) = 32c + r holds bytes [16c, 16c+16) of row r;
      // instruction q writes chunks 2q and 2q+1 of all 32 rows
      const int q = wave + NWAVE * i;
      const int r = lane & 31;
      const int c = 2 * q + (lane >> 5);
      const int dr = min(r, last);
      const uint8_t* gb = rope + (rrow0 + (int64_t)tslot0 * a.rope_st) * 2;
      lds_dma16(gb, (uint32_t)(dr * (int)a.rope_st * 2 + c * 16), st + LY::kRopeOff + 1024 * q);
    }
  };

  // ---------------------------------------------------------------- per-lane constants
  const int hf = lane >> 5;                 // lane half
  const int h = wave * 32 + (lane & 31);    // this lane's head
  const int srow = pi_row(lane & 31);       // score-operand row (token within tile)
  const int G = lane >> 4;                  // 16-lane group
  // LDS read bases (bytes inside a stage); every k-step / column block adds an immediate offset
  //  score, bf16: row srow, chunk (2s + hf) ^ swz = 2s + (hf ^ swz)          -> base + 32 s
  //  score, fp8:  row srow, chunk s ^ (srow & 1), half hf                    -> even/odd bases + 16 s
  //  rope (chunk-major): slot 32 c + srow, c = 2q + hf                        -> base + 1024 q
  //  value, bf16: rows 16ks + vrow0 (+4), chunk 4cb + 2(G&1) + ((lane&3)>>1 ^ swz), +8 (lane&1)
  //                                                                           -> base + 16896 ks + 64 cb
  //  value, fp8:  rows 16ks + vrow0, chunk 2cb + ((G&1) ^ (vrow0&1)), +8 (lane&1) -> base + 8448 ks + 32 cb
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

  issue(0);
  if (ntiles > 1) issue(1);

  int it = 0;
  int cb_seq = seq_of_tile(P, a.B, t_begin);
  while (it < ntiles) {
    // ------------------------------------------------------------ one segment: sequence b
    while (t_begin + it >= P[cb_seq + 1]) ++cb_seq;
    const int b = __builtin_amdgcn_readfirstlane(cb_seq);
    const int it_end = min(ntiles, P[b + 1] - t_begin);
    const int len_b = L[b];

    u32x4 qf[32];
    {
      const uint16_t* qa = (const uint16_t*)a.q_abs + ((int64_t)b * H + h) * 512 + 8 * hf;
#pragma unroll
      for (int s = 0; s < 32; ++s) qf[s] = *(const u32x4*)(qa + 16 * s);
      // q_R of head h -> this wave's LDS block, chunk-major (slot 32c + head)
      const uint16_t* qr = (const uint16_t*)a.q_R + ((int64_t)b * H + h) * 64;
#pragma unroll
      for (int c = hf; c < 8; c += 2) {
        const u32x4 v = *(const u32x4*)(qr + 8 * c);
        *(u32x4*)(qrs + wave * 4096 + 16 * (32 * c + (lane & 31))) = v;
      }
    }
    // Complete the folded-query loads here, once per segment (this also waits for the tiles in
    // flight), so that no wait on them is left inside the tile loop, where any vmcnt wait would
    // also drain the tile DMA pipeline.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    f32x16 acc[16];
#pragma unroll
    for (int cb = 0; cb < 16; ++cb) acc[cb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    for (; it < it_end; ++it) {
      if (it + 1 < ntiles) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_barrier();
      if (it + 2 < ntiles) issue(it + 2);

      const int nvalid = min(kTile, len_b - (t_begin + it - P[b]) * kTile);
      const uint8_t* st = smem + (it % kNst) * LY::kStage;

      // ---- score block: S^T[token rows][heads], 32 latent k-steps + 4 rope k-steps
      f32x16 S = {}, S2 = {};
      auto lat_op = [&](int s) -> u32x4 {
        if (!FP8) return *(const u32x4*)(st + sc_base + 32 * s);
        return fp8x8_to_bf16x8(*(const u32x2*)(st + ((s & 1) ? sc_base_odd : sc_base) + 16 * s));
      };
      auto rope_op = [&](int q) -> u32x4 { return *(const u32x4*)(st + rope_base + 1024 * q); };
      u32x4 a0 = lat_op(0), a1 = lat_op(1);
#pragma unroll
      for (int s = 0; s < 32; s += 2) {
        u32x4 n0, n1;
        if (s + 2 < 32) {
          n0 = lat_op(s + 2);
          n1 = lat_op(s + 3);
        } else {
          n0 = rope_op(0);
          n1 = rope_op(1);
        }
        asm volatile("" ::: "memory");
        S = mfma32x32x16(a0, qf[s], S);
        S = mfma32x32x16(a1, qf[s + 1], S);
        a0 = n0;
        a1 = n1;
      }
      {
        // rope k-steps: A = rope keys of the tile, B = q_R of the wave's heads (both LDS)
        const uint8_t* qrow = qrs + wave * 4096 + qr_base;
        const u32x4 b0 = *(const u32x4*)(qrow);
        const u32x4 b1 = *(const u32x4*)(qrow + 1024);
        const u32x4 b2 = *(const u32x4*)(qrow + 2048);
        const u32x4 b3 = *(const u32x4*)(qrow + 3072);
        const u32x4 n2 = rope_op(2);
        const u32x4 n3 = rope_op(3);
        if (FP8) {
          S2 = mfma32x32x16(a0, b0, S2);
          S2 = mfma32x32x16(a1, b1, S2);
          S2 = mfma32x32x16(n2, b2, S2);
          S2 = mfma32x32x16(n3, b3, S2);
        } else {
          S = mfma32x32x16(a0, b0, S);
          S = mfma32x32x16(a1, b1, S);
          S = mfma32x32x16(n2, b2, S);
          S = mfma32x32x16(n3, b3, S);
        }
      }

      // keep the score block in VGPRs (the softmax works on it with VALU ops)
      asm volatile("" : "+v"(S));
      if (FP8) asm volatile("" : "+v"(S2));

      // ---- online softmax (log2 units); lane holds 16 tokens of head h
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = 16 * (i >> 3) + 8 * hf + (i & 7);
        float x = S[i];
        if (FP8) x = x * *(const float*)(st + LY::kScaleOff + 4 * tl) + S2[i];
        S[i] = (tl < nvalid) ? x * a.sl2 : -INFINITY;
        mx = fmaxf(mx, S[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const bool need = mx > m_run + 8.0f;
      if (__builtin_amdgcn_ballot_w64(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
        // in-place AGPR rescale, one register at a time (keeps the accumulator resident in AGPRs)
#pragma unroll
        for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float x = acc[cb][v];
            float t;
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t) : "v"(alpha));
            acc[cb][v] = x;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        S[i] = __builtin_amdgcn_exp2f(S[i] - m_run);
        l_run += S[i];
      }
      if (FP8) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tl = 16 * (i >> 3) + 8 * hf + (i & 7);
          S[i] *= *(const float*)(st + LY::kScaleOff + 4 * tl);
        }
      }
      const u32x4 pb0 = {pack_bf16x2(S[0], S[1]), pack_bf16x2(S[2], S[3]), pack_bf16x2(S[4], S[5]),
                         pack_bf16x2(S[6], S[7])};
      const u32x4 pb1 = {pack_bf16x2(S[8], S[9]), pack_bf16x2(S[10], S[11]), pack_bf16x2(S[12], S[13]),
                         pack_bf16x2(S[14], S[15])};

      // ---- value block: acc[cb] (O^T rows 32cb..32cb+31 of head h) += C^T . P
      auto val_op = [&](int cb, int ks) -> u32x4 {
        if (!FP8) {
          const uint8_t* p0 = st + val_base + 16 * kLatStride * ks + 64 * cb;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(p0 + 4 * kLatStride));
          const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
          return u32x4{l2[0], l2[1], h2[0], h2[1]};
        }
        const uint8_t* p0 = st + val_base + 8 * kLatStride * ks + 32 * cb;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MLA_LDS i32x2*)(p0));
        return fp8x8_to_bf16x8(__builtin_bit_cast(u32x2, v));
      };
      u32x4 v0 = val_op(0, 0), v1 = val_op(0, 1);
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
        u32x4 w0 = v0, w1 = v1;
        if (cb + 1 < 16) { w0 = val_op(cb + 1, 0); w1 = val_op(cb + 1, 1); }
        asm volatile("" ::: "memory");
        acc[cb] = mfma32x32x16(v0, pb0, acc[cb]);
        acc[cb] = mfma32x32x16(v1, pb1, acc[cb]);
        asm volatile("" : "+a"(acc[cb]));  // the output accumulator lives in AGPRs
        v0 = w0; v1 = w1;
      }
    }

    // ------------------------------------------------------------ segment partial -> slot w + b
    {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      const int64_t o = (int64_t)(w + b) * H + h;
      float* dst = a.ws_acc + o * 512 + 4 * hf;
#pragma unroll
      for (int cb = 0; cb < 16; ++cb) {
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) {
          *(f32x4*)(dst + 32 * cb + 8 * v4) =
              f32x4{acc[cb][4 * v4], acc[cb][4 * v4 + 1], acc[cb][4 * v4 + 2], acc[cb][4 * v4 + 3]};
        }
      }
      if (lane < 32) *(f32x2*)(a.ws_ml + o * 2) = f32x2{m_run, l_tot};
    }
  }
}

hipError_t launch_partial_mfma(const PartialArgs& a, bool fp8, bool paged, hipStream_t s) {
  const int nw = a.H / 32;
#define MLA_LAUNCH(NW, F, PG)                                                              \
  hipLaunchKernelGGL((k_partial_mfma<NW, F, PG>), dim3(a.W), dim3(NW * 64), 0, s, a); \
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
