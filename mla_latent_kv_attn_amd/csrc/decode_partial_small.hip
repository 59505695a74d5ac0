// Partial pass of the absorbed decode for small batches (few 32-token tiles in total), bf16
// latents, DeepSeek-V3 shape (d_c = 512, d_R = 64).  Computes what the large-batch MFMA kernel
// computes ("Grouped-query and latent attention", sections "The absorption trick" and "Why a
// separate rotary key": per token the score q'_h . c_j + q_R,h . k_R,j scaled by 1/sqrt(d_h + d_R),
// and the softmax-weighted latent sum, W_UV applied later), with the work of one tile cut finer.
//
// With few tiles the large-batch kernel leaves most SIMDs idle: one wave owns all of a tile's
// work for 32 heads (68 MFMAs per tile in a row), and the many splits needed to fill the chip
// multiply the partial results written.  Here a workgroup owns one split of the tiles and one
// block of 32 heads, and its four waves (one per SIMD) share each tile.  Wave w owns latent
// columns 128w .. 128w+127 and rope dimensions 16w .. 16w+15 of every row:
//  * loads: each wave moves only its own slice of a tile into its own LDS area (direct
//    global->LDS loads, 3 stages, two tiles ahead), so no barrier is needed to publish a tile;
//  * score: wave w sums the eight k-steps of its latent columns and the k-step of its rope
//    dimensions (9 MFMA 32x32x16, a 36-register slice of Qhat) and writes the partial S^T block
//    (32 tokens x 32 heads, fp32) to LDS;
//  * online softmax, split over the waves: wave w adds the four partials (in wave order) for
//    heads 8w .. 8w+7, four scores per lane, keeps those heads' running maximum (raised only past
//    a threshold of 2^8, as in the large-batch kernel) and sum, and writes bf16 probabilities,
//    rescale factors and a flag to LDS;
//  * value: wave w multiplies its columns by the probabilities of all 32 heads (8 MFMA per tile
//    into 64 accumulator registers; transposing LDS reads give the latent operand).
// Software pipeline, one barrier per tile: iteration i runs score(i+1), value(i-1), softmax(i),
// with the MFMAs of the first two issued before the VALU work of the softmax; the barrier
// publishes the score partials of tile i and the probabilities of tile i-1.  The
// four head-block workgroups of a split sit on one XCD (block index stride a multiple of 8), so
// a tile comes from HBM once and from that XCD's L2 for the other three.
#include "partial_common.h"

namespace mla {

namespace {
constexpr int kSlice = 9216;      // LDS bytes per wave and stage: 32 rows x 256 B latent + 32 x 32 B rope
constexpr int kSRope = 8192;      // rope part of a slice
constexpr int kPb = 80;           // bytes per head row of the probability buffer (64 + pad)
}  // namespace

template <bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_partial_small(PartialArgs a) {
  constexpr int NWAVE = 4;
  constexpr int LPT = 9;          // direct loads per wave per tile: 8 latent (4 rows each) + 1 rope
  __shared__ __attribute__((aligned(1024))) uint8_t ring[kNst * NWAVE * kSlice];
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2][NWAVE * 4096];   // score partials / flush
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][32 * kPb];        // bf16 probabilities
  __shared__ float alpha_s[2][32];
  __shared__ __attribute__((aligned(16))) int flags_s[2][4];
  __shared__ int P[kSmallMaxB + 1];
  __shared__ int Ls[kSmallMaxB];

  if ((int)blockIdx.x >= a.W) {
    if (blockIdx.y != 0) return;
    // warm-up workgroup: read one word of every 128-byte line of its share of the warm-up buffer
    const int64_t nlines = (a.warm_bytes + 127) / 128;
    const int64_t per = (nlines + a.extra - 1) / a.extra;
    const int64_t l0 = (int64_t)(blockIdx.x - a.W) * per, l1 = min(nlines, l0 + per);
    const uint32_t* p = (const uint32_t*)a.warm;
    const int64_t last_word = a.warm_bytes / 4 - 1;
    uint32_t x = 0;
    for (int64_t l = l0 + threadIdx.x; l < l1; l += blockDim.x) x ^= p[min(l * 32, last_word)];
    asm volatile("" : : "v"(x));
    return;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = a.H;
  const int h0 = blockIdx.y * 32;
  const int hf = lane >> 5;
  const int hl = lane & 31;        // head of this lane in the score and value layouts
  const int sn = 8 * wave + (lane >> 3);   // head of this lane in the softmax layout
  const int sc = lane & 7;                 // its 4-score chunk: rows 4 sc .. 4 sc + 3 of S^T

  // folded query slice of this wave for sequence b: latent k-steps 8 wave .. 8 wave + 7 (qf[0..7])
  // and rope k-step `wave` (qf[8]); lane half hf holds k 8 hf .. 8 hf + 7 of each step
  u32x4 qf[9];
  auto load_q = [&](int b) __attribute__((always_inline)) {
    const uint16_t* qa = (const uint16_t*)a.q_abs + ((int64_t)b * H + h0 + hl) * 512 + 8 * hf + 128 * wave;
#pragma unroll
    for (int j = 0; j < 8; ++j) qf[j] = *(const u32x4*)(qa + 16 * j);
    const uint16_t* qr = (const uint16_t*)a.q_R + ((int64_t)b * H + h0 + hl) * 64 + 8 * hf + 16 * wave;
    qf[8] = *(const u32x4*)(qr);
  };

  // ---------------------------------------------------------------- tile prefix
  // One sequence: its length comes through the scalar cache (not queued behind the query loads)
  // and the prefix is built without a workgroup barrier.
  int NT;
  if (a.B == 1) {
    const int len = load_uniform_i32(a.seq_lens);
    load_q(0);
    NT = tiles_of(len);
    if (lane == 0) {   // every wave writes the same values and reads only its own
      P[0] = 0;
      P[1] = NT;
      Ls[0] = len;
    }
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      if (threadIdx.x == 0) {
        a.ws_prefix[0] = 0;
        a.ws_prefix[1] = NT;
        a.ws_prefix[2] = kPartF32;
      }
      for (int i = threadIdx.x; i < H; i += blockDim.x) a.ws_cnt[i] = 0;
    }
  } else {
    build_tile_prefix(a.seq_lens, a.B, P, Ls);
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      for (int i = threadIdx.x; i <= a.B; i += blockDim.x) a.ws_prefix[i] = P[i];
      if (threadIdx.x == 0) a.ws_prefix[a.B + 1] = kPartF32;
      for (int i = threadIdx.x; i < H; i += blockDim.x) a.ws_cnt[i] = 0;
    }
    NT = P[a.B];
  }
  const int Wp = min(a.W, NT);
  const int w = blockIdx.x;
  if (w >= Wp) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    return;
  }
  const int t_begin = (int)((int64_t)w * NT / Wp);
  const int t_end = (int)((int64_t)(w + 1) * NT / Wp);
  const int ntiles = t_end - t_begin;
  auto seq_of = [&](int it) __attribute__((always_inline)) -> int {
    return a.B == 1 ? 0 : seq_of_tile(P, a.B, t_begin + it);
  };
  if (a.B != 1) load_q(seq_of(0));   // the first segment's query goes out before the tile loads

  // ---------------------------------------------------------------- loader (tile it -> stage it % 3)
  const uint8_t* latent = (const uint8_t*)a.latent;
  const uint8_t* rope = (const uint8_t*)a.rope;
  uint8_t* my_ring = ring + wave * kSlice;   // + stage * NWAVE * kSlice
  int lk_b = seq_of(0);
  int lk_start = __builtin_amdgcn_readfirstlane(P[lk_b]);
  int lk_next = __builtin_amdgcn_readfirstlane(P[lk_b + 1]);
  int lk_len = __builtin_amdgcn_readfirstlane(Ls[lk_b]);
  // Latent: row r of a slice is 256 contiguous bytes in LDS; its 16-byte chunk c sits at position
  // c ^ (r & 15) (conflict-free score reads).  Load k fills rows 4k .. 4k+3: lane i writes
  // position i & 15 of row 4k + (i >> 4).  Rope: row r is 32 bytes, chunk c at position
  // c ^ ((r >> 3) & 1); lane i writes position i & 1 of row i >> 1.  Rows past the sequence's end
  // are loaded from its last row (finite data, masked later).
  auto issue = [&](int it) __attribute__((always_inline)) {
    const int t = t_begin + it;
    while (t >= lk_next) {
      ++lk_b;
      lk_start = lk_next;
      lk_next = __builtin_amdgcn_readfirstlane(P[lk_b + 1]);
      lk_len = __builtin_amdgcn_readfirstlane(Ls[lk_b]);
    }
    const int b = __builtin_amdgcn_readfirstlane(lk_b);
    const int tok0 = (t - lk_start) * kTile;
    const int last = __builtin_amdgcn_readfirstlane(min(kTile, lk_len - tok0) - 1);
    int64_t lrow0, rrow0;
    int tslot0;
    if (PAGED) {
      const int page = load_uniform_i32(a.block_table + (int64_t)b * a.max_pages + tok0 / a.page_size);
      lrow0 = (int64_t)page * a.lat_sb;
      rrow0 = (int64_t)page * a.rope_sb;
      tslot0 = tok0 % a.page_size;
    } else {
      lrow0 = (int64_t)b * a.lat_sb;
      rrow0 = (int64_t)b * a.rope_sb;
      tslot0 = tok0;
    }
    const uint8_t* lbase = (const uint8_t*)uniform_ptr(latent + (lrow0 + (int64_t)tslot0 * a.lat_st) * 2 + 256 * wave);
    const uint8_t* rbase = (const uint8_t*)uniform_ptr(rope + (rrow0 + (int64_t)tslot0 * a.rope_st) * 2 + 32 * wave);
    const uint32_t st = __builtin_amdgcn_readfirstlane(lds_addr(my_ring + (it % kNst) * NWAVE * kSlice));
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint32_t lstride = (uint32_t)a.lat_st * 2u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = 4 * k + (ln >> 4);
      const uint32_t voff = (uint32_t)min(r, last) * lstride + 16u * (uint32_t)((ln & 15) ^ (r & 15));
      lds_dma16(lbase, voff, st + 1024 * k);
    }
    const int rr = ln >> 1;
    const uint32_t roff = (uint32_t)(min(rr, last) * (int)a.rope_st * 2) + 16u * (uint32_t)((ln & 1) ^ ((rr >> 3) & 1));
    lds_dma16(rbase, roff, st + kSRope);
  };

  // ---------------------------------------------------------------- per-lane LDS offsets
  const int srow = pi_row(hl);   // score-operand row (token within the tile)
  const int G = lane >> 4;
  const int vrow0 = 8 * (G >> 1) + ((lane & 15) >> 2);
  // score A operand, latent k-step j: row srow, chunk 2j + hf
  const int sc_row = srow * 256;
  const int sc_x = srow & 15;
  const int rope_rd = kSRope + srow * 32 + 16 * (hf ^ ((srow >> 3) & 1));

  // score partial of this wave for the tile in stage st -> sbuf[par] (head-major rows of 128 B,
  // 16-byte chunk c of head n at position c ^ ((n >> 1) & 7))
  // (score_mfma issues the MFMAs; score_store, later, writes the result: the MFMAs run while the
  // wave does other work)
  auto score_mfma = [&](int stg, f32x16& S0, f32x16& S1) __attribute__((always_inline)) {
    const uint8_t* st = my_ring + stg * NWAVE * kSlice;
    u32x4 av[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) av[j] = *(const u32x4*)(st + sc_row + 16 * ((2 * j + hf) ^ sc_x));
    const u32x4 rv = *(const u32x4*)(st + rope_rd);
    mfma_v_first(S0, av[0], qf[0]);
    mfma_v_first(S1, av[1], qf[1]);
#pragma unroll
    for (int j = 2; j < 8; j += 2) {
      mfma_v(S0, av[j], qf[j]);
      mfma_v(S1, av[j + 1], qf[j + 1]);
    }
    mfma_v(S0, rv, qf[8]);
  };
  auto score_store = [&](f32x16& S0, f32x16& S1, int par) __attribute__((always_inline)) {
    asm volatile("s_nop 15" : "+v"(S0), "+v"(S1));
    const f32x16 S = S0 + S1;
    uint8_t* sb = sbuf[par] + wave * 4096 + hl * 128;
    const int xs = (hl >> 1) & 7;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4)
      *(f32x4*)(sb + 16 * ((2 * v4 + hf) ^ xs)) = f32x4{S[4 * v4], S[4 * v4 + 1], S[4 * v4 + 2], S[4 * v4 + 3]};
  };

  // online softmax of heads 8 wave .. 8 wave + 7 (log2 units), tile in sbuf[par]
  float m_run = -INFINITY, l_part = 0.f;
  const int tok_c = 4 * ((sc >> 1) & 1) + 8 * (sc & 1) + 16 * (sc >> 2);   // token of row 4 sc
  auto softmax = [&](int par, int nvalid) __attribute__((always_inline)) {
    const uint8_t* sb = sbuf[par] + sn * 128 + 16 * (sc ^ ((sn >> 1) & 7));
    f32x4 x = *(const f32x4*)(sb);
#pragma unroll
    for (int q = 1; q < NWAVE; ++q) x += *(const f32x4*)(sb + 4096 * q);
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (tok_c + r < nvalid) ? x[r] : -INFINITY;
    float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    mx *= a.sl2;
    const bool need = mx > m_run + 8.0f;
    // a segment's first tile raises every maximum from -inf, but its accumulator is still zero:
    // no rescale needed (alpha is 0 there)
    const int any = __builtin_amdgcn_ballot_w64(need && m_run != -INFINITY) != 0 ? 1 : 0;
    const float m_new = need ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 1 unless raised (m_run = -inf: 0)
    m_run = m_new;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(x[r], a.sl2, -m_run));
    l_part = fmaf(l_part, alpha, (p[0] + p[1]) + (p[2] + p[3]));
    *(u32x2*)(pbuf[par] + sn * kPb + 2 * tok_c) = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
    if (sc == 0) alpha_s[par][sn] = alpha;
    flags_s[par][wave] = any;
  };

  // value: acc[cb] (O^T rows = latent columns 128 wave + 32 cb .. +31, columns = the 32 heads)
  f32x16 acc[4];
  auto value = [&](int stg, int par) __attribute__((always_inline)) {
    const uint8_t* st = my_ring + stg * NWAVE * kSlice;
    const u32x4 fl = *(const u32x4*)flags_s[par];
    const u32x4 p0 = *(const u32x4*)(pbuf[par] + hl * kPb + 16 * hf);
    const u32x4 p1 = *(const u32x4*)(pbuf[par] + hl * kPb + 32 + 16 * hf);
    if (__builtin_amdgcn_readfirstlane(fl[0] | fl[1] | fl[2] | fl[3]) != 0) {
      const float al = alpha_s[par][hl];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] *= al;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 av[4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // rows R and R + 4 (R = 16 ks + vrow0), column chunk 4 cb + 2 (G & 1) + ((lane & 3) >> 1)
        const int R = 16 * ks + vrow0;
        const int cc = 4 * cb + 2 * (G & 1) + ((lane & 3) >> 1);
        const uint8_t* pa = st + R * 256 + 16 * (cc ^ (R & 15)) + 8 * (lane & 1);
        const uint8_t* pb = st + (R + 4) * 256 + 16 * (cc ^ ((R + 4) & 15)) + 8 * (lane & 1);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pa));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)(pb));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        av[cb] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[cb] = mfma32x32x16(av[cb], ks ? p1 : p0, acc[cb]);
    }
  };

  // partial of the segment of sequence b -> workspace slot w + b: flush_ml writes the (m, l) pairs
  // of this wave's softmax heads, flush the accumulator.  The accumulator blocks are transposed
  // through LDS: the last segment uses this wave's ring slices (no tile is in flight any more; all
  // four blocks at once), an earlier one this wave's part of sbuf[par] (free at this point; one
  // block at a time).
  auto flush_ml = [&](int b) __attribute__((always_inline)) {
    float l_tot = l_part;
    l_tot += __shfl_xor(l_tot, 1, 64);
    l_tot += __shfl_xor(l_tot, 2, 64);
    l_tot += __shfl_xor(l_tot, 4, 64);
    if (sc == 0) *(f32x2*)(a.ws_ml + ((int64_t)(w + b) * H + h0 + sn) * 2) = f32x2{m_run, l_tot};
  };
  auto flush = [&](int b, int par, bool final_seg) __attribute__((always_inline)) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int trow = ln >> 3, tch = ln & 7;
    const int xs = ((ln & 31) >> 1) & 7;
    float* dst = a.ws_acc + ((int64_t)(w + b) * H + h0 + trow) * 512 + 128 * wave + 4 * tch;
    auto put = [&](uint8_t* tb, int cb) __attribute__((always_inline)) {
      const f32x16& A = acc[cb];
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4)
        *(f32x4*)(tb + (ln & 31) * 128 + 16 * ((2 * v4 + (ln >> 5)) ^ xs)) =
            f32x4{A[4 * v4], A[4 * v4 + 1], A[4 * v4 + 2], A[4 * v4 + 3]};
    };
    auto get = [&](const uint8_t* tb, int cb) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 8 * q + trow;
        *(f32x4*)(dst + (8 * q) * 512 + 32 * cb) = *(const f32x4*)(tb + row * 128 + 16 * (tch ^ ((row >> 1) & 7)));
      }
    };
    if (final_seg) {
      // blocks 0, 1 in stage 0's slice, 2, 3 in stage 1's (4 KiB each, within the 9 KiB slices)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) put(my_ring + (cb >> 1) * NWAVE * kSlice + (cb & 1) * 4096, cb);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) get(my_ring + (cb >> 1) * NWAVE * kSlice + (cb & 1) * 4096, cb);
    } else {
      uint8_t* tb = sbuf[par] + wave * 4096;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        put(tb, cb);
        get(tb, cb);
      }
    }
  };


  // ---------------------------------------------------------------- pipeline
  issue(0);
  if (ntiles > 1) issue(1);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
  // score(0): the query and tile 0 have landed once only tile 1's loads are outstanding (the
  // compiler, which does not see the tile loads, adds its own wait for the query loads here)
  if (ntiles > 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
  else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  {
    f32x16 S0, S1;
    score_mfma(0, S0, S1);
    if (ntiles > 2) issue(2);   // after the query wait the compiler put before the MFMAs
    score_store(S0, S1, 0);
  }
  // Segment bookkeeping (uniform, in registers): the sequence of the tile whose value step comes
  // next and the first tile of the sequence after it; the same for the softmax step, with the
  // token index of that tile and the sequence length.  LDS lookups happen only at segment ends.
  int b_val = seq_of(0);
  int val_next = __builtin_amdgcn_readfirstlane(P[b_val + 1]);
  int b_sm = b_val, sm_next = val_next;
  int sm_tok = __builtin_amdgcn_readfirstlane((t_begin - P[b_sm]) * kTile);
  int sm_len = __builtin_amdgcn_readfirstlane(Ls[b_sm]);
  // Iteration it: the score MFMAs of tile it + 1 and the value MFMAs of tile it - 1 are issued
  // first, then the loads of tile it + 2 (into the stage tile it - 1 just left); the softmax of
  // tile it (VALU and LDS work) runs while the MFMAs execute; then the end of a segment is written
  // out and the score partial of tile it + 1 is stored.
  for (int it = 0; it <= ntiles; ++it) {
    __builtin_amdgcn_s_waitcnt(lgkmcnt_imm0());
    lds_barrier();
    if (it < ntiles && t_begin + it >= sm_next) {   // the softmax enters a new sequence
      while (t_begin + it >= sm_next) sm_next = __builtin_amdgcn_readfirstlane(P[++b_sm + 1]);
      sm_tok = 0;
      sm_len = __builtin_amdgcn_readfirstlane(Ls[b_sm]);
    }
    const bool do_score = it + 1 < ntiles;
    f32x16 S0, S1;
    if (do_score) {
      // tile it + 1 has landed once only tile 2's loads may be outstanding (issued before the
      // loop); a new sequence first loads its folded query
      if (t_begin + it + 1 >= sm_next) {
        load_q(seq_of(it + 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      } else if (it == 0 && ntiles > 2) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
      } else {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      }
      score_mfma((it + 1) % kNst, S0, S1);
    }
    bool seg_end = false;
    if (it >= 1) {
      value((it - 1) % kNst, (it - 1) & 1);
      if (it + 2 < ntiles) issue(it + 2);
      seg_end = it == ntiles || t_begin + it >= val_next;
      if (seg_end) {
        flush_ml(b_val);
        m_run = -INFINITY;
        l_part = 0.f;
      }
    }
    if (it < ntiles) {
      softmax(it & 1, min(kTile, sm_len - sm_tok));
      sm_tok += kTile;
    }
    if (seg_end) {
      flush(b_val, (it - 1) & 1, it == ntiles);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
      if (it < ntiles) {
        while (t_begin + it >= val_next) val_next = __builtin_amdgcn_readfirstlane(P[++b_val + 1]);
      }
    }
    if (do_score) score_store(S0, S1, (it + 1) & 1);
  }
}

hipError_t launch_partial_small(const PartialArgs& a, bool paged, hipStream_t s) {
  if (a.B > kSmallMaxB) return hipErrorInvalidValue;
  const dim3 grid(a.W + a.extra, a.H / 32);
  if (paged) hipLaunchKernelGGL((k_partial_small<true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_partial_small<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mla
