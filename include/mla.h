/*
 * mla.h -- C ABI of the MI355X (gfx950) library for the absorbed decode step of
 * Multi-Head Latent Attention.
 *
 * One decode step, per sequence b and head h (column-vector notation of
 * "Grouped-query and latent attention", sections "Multi-head latent attention
 * (MLA)", "The absorption trick" and "Why a separate rotary key"):
 *
 *   q'[b,h]    = W_UK[h]^T q_C[b,h]                                  mla_absorb_q
 *   s[b,h,j]   = scale * (q'[b,h] . c[b,j]  +  q_R[b,h] . k_R[b,j])   j < len[b]
 *   a[b,h,:]   = softmax_j s[b,h,:]
 *   o_lat[b,h] = sum_j a[b,h,j] c[b,j]                                mla_decode_attn
 *   o[b,h]     = W_UV[h] o_lat[b,h]                                   mla_uv_out
 *
 * c[b,j] is the cached d_c-wide latent of token j and k_R[b,j] the cached,
 * already rotated d_R-wide rope key shared by all heads ("MLA storage:
 * Representing KV with a small latent vector", section "Storing a positional
 * key separately").  scale is 1/sqrt(d_h + d_R).  Full keys and values are
 * never formed.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *    every buffer.  Tensors are dense row-major with the shapes given, except
 *    the cache, which is described by mla_cache_desc.
 *  - Calls only enqueue work on `stream` (a hipStream_t; NULL = the default
 *    stream) and return without synchronising.  They allocate no memory.
 *  - Host-side argument checks run before anything is enqueued and return a
 *    status other than MLA_OK; nothing is launched in that case.  A failed
 *    launch returns MLA_ERR_HIP and mla_last_hip_error() gives the hipError_t
 *    (per calling thread).
 *  - Values held in device memory (sequence lengths, block-table entries) are
 *    not validated: a length above max_len or outside the cache capacity, or a
 *    page id outside the pool, is undefined behaviour.
 *  - Results are bitwise reproducible for fixed arguments: every sum is taken in a fixed order.
 *    Some kernels exchange data between workgroups of one launch (mla_decode_combine_uv at
 *    small batch, mla_decode_step's one-launch form): the producers write with device-coherent (agent-scope) stores, wait until
 *    those stores have completed (s_waitcnt vmcnt(0)), then raise an agent-scope counter with
 *    an integer atomic add (mla_decode_step: set one flag word per consumer); a consumer reads
 *    the data with device-coherent loads only after it has seen the counter's final value (its
 *    flags), and adds the parts in a fixed order, so the result does
 *    not depend on which workgroup finished last.  No floating-point atomics are used.
 *  - Calls on different streams are independent; the library keeps no state
 *    other than the per-thread last HIP error.
 */
#ifndef MLA_AMD_MLA_H
#define MLA_AMD_MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,         /* a required pointer is NULL                       */
  MLA_ERR_SHAPE = 2,        /* a size is negative, zero where not allowed, or inconsistent */
  MLA_ERR_DTYPE = 3,        /* unknown dtype or unsupported dtype combination    */
  MLA_ERR_UNSUPPORTED = 4,  /* valid arguments that this build has no kernel for */
  MLA_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than required           */
  MLA_ERR_HIP = 6           /* a HIP runtime call or kernel launch failed        */
} mla_status;

typedef enum {
  MLA_F32 = 0,              /* IEEE binary32                                    */
  MLA_BF16 = 1,             /* bfloat16                                         */
  MLA_FP8_E4M3 = 2          /* OCP FP8 E4M3 (bias 7, max 448, no infinities, S.1111.111 = NaN) */
} mla_dtype;

/*
 * One layer's latent + rope-key cache.  Row j of sequence b:
 *   contiguous (block_table == NULL):
 *     latent row  = latent + b*latent_stride_b + j*latent_stride_tok      (elements of latent_dtype)
 *     rope row    = rope   + b*rope_stride_b   + j*rope_stride_tok        (elements of rope_dtype)
 *     scale       = latent_scale[b*scale_stride_b + j]                    (FP8 latents only)
 *   paged (block_table != NULL): with p = block_table[b*max_pages + j/page_size]
 *   and s = j % page_size, the *_stride_b fields are page strides:
 *     latent row  = latent + p*latent_stride_b + s*latent_stride_tok
 *     rope row    = rope   + p*rope_stride_b   + s*rope_stride_tok
 *     scale       = latent_scale[p*scale_stride_b + s]
 * The rows of a latent and of a rope key must each be contiguous (unit
 * element stride).  Latent and rope may live in one packed row [c ; k_R]
 * (the two stored parts of one illustrated cache row in "MLA storage:
 * Representing KV with a small latent vector") or in separate buffers.
 * An FP8 latent c is latent_scale * decode(code).
 */
typedef struct mla_cache_desc {
  const void* latent;
  const void* rope;
  const float* latent_scale;   /* FP8 latents only, else NULL */
  const int32_t* block_table;  /* NULL = contiguous; else [B, max_pages] int32 physical page ids */
  int32_t latent_dtype;        /* MLA_F32, MLA_BF16 or MLA_FP8_E4M3 */
  int32_t rope_dtype;          /* MLA_F32 or MLA_BF16 */
  int64_t latent_stride_b;
  int64_t latent_stride_tok;
  int64_t rope_stride_b;
  int64_t rope_stride_tok;
  int64_t scale_stride_b;
  int32_t page_size;           /* paged only: tokens per page */
  int32_t max_pages;           /* paged only: columns of block_table */
} mla_cache_desc;

/* Human-readable name of a status code (static string). */
const char* mla_status_string(int status);

/* hipError_t of the last MLA_ERR_HIP returned on the calling thread (0 if none). */
int mla_last_hip_error(void);

/* Library version as 10000*major + 100*minor + patch. */
int mla_version(void);

/*
 * mla_absorb_q -- fold W_UK into the query ("Grouped-query and latent
 * attention", section "The absorption trick": q' = W_UK^T q_C, computed once
 * for the new token).
 *   q_C    [B, H, d_h]   in_dtype
 *   W_UK   [H, d_h, d_c] in_dtype   (W_UK[h] maps a latent to head h's content key)
 *   q_abs  [B, H, d_c]   out_dtype  (written)
 * Dtypes: in MLA_F32 -> out MLA_F32 (any d_h <= 1024, d_c <= 4096), or
 *         in MLA_BF16 -> out MLA_BF16 (d_h == 128, d_c == 512; fp32 accumulation,
 *         one round-to-nearest-even to bf16 at the end).
 * B == 0 is a no-op.
 */
int mla_absorb_q(const void* q_C, const void* W_UK, void* q_abs, int in_dtype, int out_dtype,
                 int B, int H, int d_h, int d_c, void* stream);

/*
 * Workspace (device bytes) mla_decode_attn needs for these sizes.  num_splits
 * is the number of partial-pass workgroups over the whole batch (0 = the
 * library's choice for (B, H, max_len), the same choice mla_decode_attn makes).
 * With W workgroups the workspace holds (W + B - 1) partial slots of H x d_c
 * float sums (bf16 sums, in the first half of the region, where the large-batch
 * kernel runs: E4M3 caches, and bf16 caches with B x ceil(max_len / 32) above
 * 1024 or B above 256) and H (max, sum) pairs, then B + 1 int32
 * tile prefix sums and one int32 naming the sums' element type, then H
 * int32 counters and min(B, 4) x H x 4 x 128 floats used by the one-kernel form
 * of mla_decode_combine_uv; each of the five regions is rounded up to a multiple
 * of 256 bytes.  Returns 0 for invalid sizes.
 */
size_t mla_decode_workspace_bytes(int B, int H, int d_c, int max_len, int num_splits);

/* The number of partial-pass splits mla_decode_attn uses when num_splits == 0, from the tile
 * count bound T = B * ceil(max_len / 32): for T <= 1024, min(ceil(3 T / 8), 64); otherwise
 * about two tiles per split, min(ceil(T / 2), 256); at least 1. */
int mla_decode_auto_splits(int B, int H, int max_len);

/*
 * mla_decode_attn -- scores of the folded query against the cached latents
 * plus the rope term, scaled softmax over j < seq_lens[b], and the weighted
 * latent sum ("Grouped-query and latent attention", sections "The absorption
 * trick" and "Why a separate rotary key"; the attention row of the newest
 * token only, "The Journey to Multi-Head Latent Attention", section "The KV
 * cache -- and why it exists at all").
 *
 * Two passes on `stream`: a partial pass splits the concatenated token tiles of
 * the batch evenly over num_splits workgroups, each writing a running
 * (max, sum, weighted latent sum) per head for every sequence it touches into
 * the workspace; a combine pass merges those partials per (b, h).
 *   q_abs     [B, H, d_c]  q_dtype   folded queries (output of mla_absorb_q)
 *   q_R       [B, H, d_R]  q_dtype   rotated rope queries
 *   cache     host pointer to the descriptor (read during the call only)
 *   seq_lens  [B] int32 device: tokens cached per sequence, 0 <= len <= max_len
 *   max_len   host: an upper bound on every seq_lens[b]
 *   scale     softmax scale, positive and finite, normally 1/sqrt(d_h + d_R)
 *   workspace device buffer of at least mla_decode_workspace_bytes(...) bytes,
 *             16-byte aligned, any contents; overwritten
 *   o_latent  [B, H, d_c] float32, 16-byte aligned (written): sum_j a_j c_j
 *   lse       [B, H] float32 (written unless NULL): natural-log log-sum-exp of
 *             the scaled scores
 * A sequence with len 0 gives o_latent = 0 and lse = -inf.
 * Supported: q_dtype MLA_F32 with an MLA_F32 cache (d_c <= 1024, d_R <= 256);
 *            q_dtype MLA_BF16 with an MLA_BF16 or MLA_FP8_E4M3 latent and MLA_BF16
 *            rope (d_c == 512, d_R == 64, H a multiple of 32 up to 128;
 *            paged: page_size a multiple of 32).  B <= 2048.
 */
int mla_decode_attn(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                    const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                    int num_splits, void* workspace, size_t workspace_bytes, float* o_latent, float* lse,
                    void* stream);

/*
 * The two passes of mla_decode_attn as separate calls (same arguments, same workspace contract),
 * for callers that schedule or time them individually.  mla_decode_attn(...) is exactly
 * mla_decode_partial(...) followed by mla_decode_combine(...) on the same stream with the same
 * B, H, d_c, max_len, num_splits and workspace.
 *   mla_decode_partial: writes one (max, sum, weighted latent sum) partial per head for every
 *     (workgroup, sequence) segment into the workspace.
 *   mla_decode_combine: merges the partials of each (b, h) into o_latent and lse (the
 *     log-sum-exp merge: M = max m_s, L = sum 2^(m_s-M) l_s, o = sum 2^(m_s-M) acc_s / L).
 *     It reads the segment layout (tile prefix sums of seq_lens) that the partial pass left
 *     in the workspace, so it must follow a partial pass over the same seq_lens.
 */
int mla_decode_partial(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                       const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                       int num_splits, void* workspace, size_t workspace_bytes, void* stream);
/*
 * mla_decode_partial_warm -- mla_decode_partial (same arguments, same result) that also pulls
 * [warm, warm + warm_bytes) into the device's last-level cache: when the pass has fewer
 * workgroups than the GPU has compute units (small batches), the spare workgroups read one word
 * of every 128-byte line of that buffer and exit.  A decode step passes W_UV here so that the
 * W_UV product after the combine reads it from the cache.  Nothing is written; results never
 * depend on it.  warm: device pointer, 4-byte aligned (NULL with warm_bytes == 0 = no warm-up).
 */
int mla_decode_partial_warm(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                            const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                            int num_splits, void* workspace, size_t workspace_bytes, const void* warm,
                            size_t warm_bytes, void* stream);
int mla_decode_combine(const int32_t* seq_lens, int max_len, int B, int H, int d_c, int num_splits,
                       const void* workspace, size_t workspace_bytes, float* o_latent, float* lse, void* stream);

/*
 * mla_decode_combine_uv -- the combine pass followed by mla_uv_out, as one call: the same
 * arguments as mla_decode_combine (o_latent and lse are written exactly as there) plus W_UV
 * [H, d_h, d_c] in w_dtype and out [B, H, d_h] float32 (written), with the semantics of
 * mla_uv_out.  For a bf16 W_UV with d_h == 128, d_c == 512 and B <= 4 it is one kernel: four
 * workgroups per head each merge a quarter of the latent columns and multiply it with the
 * matching quarter of W_UV, and the last of the four to finish adds the four products in a
 * fixed order (a device-scope counter in the workspace, which the partial pass zeroes, so this
 * form must follow a partial pass on the same workspace); otherwise it launches the two passes.
 * Results are the same whichever workgroup finishes last.  Errors as for mla_decode_combine
 * and mla_uv_out; nothing is launched when validation fails.
 */
int mla_decode_combine_uv(const int32_t* seq_lens, int max_len, int B, int H, int d_c, int num_splits,
                          const void* workspace, size_t workspace_bytes, const void* W_UV, int w_dtype, int d_h,
                          float* out, float* o_latent, float* lse, void* stream);

/*
 * mla_decode_attn_noalloc -- mla_decode_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments and results without the workspace, which is instead a fixed array of
 * mla_decode_attn_noalloc_max_bytes() bytes (64 MiB) that the library holds on each device it
 * runs on until the process ends.  No memory is allocated by the call.
 *   num_splits 0 = the library's choice, mla_decode_attn_noalloc_splits(B, H, d_c, max_len): the
 *              split count mla_decode_attn would use, lowered until its workspace fits the array;
 *              an explicit count is used as given.
 * Returns MLA_ERR_WORKSPACE when the workspace of these sizes and split count exceeds the array
 * (with the V3 head count, slots = splits + B - 1 of 256 KB each, so at most 256 slots), other
 * errors as for mla_decode_attn.  The first call on a device looks up the array's address on that
 * device (hipGetSymbolAddress); a failure there returns MLA_ERR_HIP.
 * Every call on one device uses that device's one array, which keeps the last call's contents
 * (the decode passes need no particular initial contents): calls that overlap in time on one
 * device, for example on two streams, race and give undefined results.
 * Results are those of mla_decode_attn with the same split count.
 */
size_t mla_decode_attn_noalloc_max_bytes(void);
int mla_decode_attn_noalloc_splits(int B, int H, int d_c, int max_len);
int mla_decode_attn_noalloc(const void* q_abs, const void* q_R, int q_dtype, const mla_cache_desc* cache,
                            const int32_t* seq_lens, int max_len, int B, int H, int d_c, int d_R, float scale,
                            int num_splits, float* o_latent, float* lse, void* stream);

/*
 * mla_uv_out -- apply W_UV once to the weighted latent sum ("Grouped-query and
 * latent attention", section "The absorption trick": sum_j a_j W_UV c_j =
 * W_UV sum_j a_j c_j).
 *   o_latent [B, H, d_c]  float32
 *   W_UV     [H, d_h, d_c] w_dtype (MLA_F32, or MLA_BF16 with d_h == 128, d_c == 512)
 *   out      [B, H, d_h]  float32 (written), fp32 accumulation
 * B == 0 is a no-op.
 */
int mla_uv_out(const float* o_latent, const void* W_UV, int w_dtype, float* out, int B, int H, int d_h,
               int d_c, void* stream);

/*
 * mla_decode_step -- the whole absorbed decode step in one call: mla_absorb_q, mla_decode_attn and
 * mla_uv_out of the same arguments ("Grouped-query and latent attention", sections "The
 * absorption trick" and "Why a separate rotary key"):
 *   out[b,h] = W_UV[h] sum_j a[b,h,j] c[b,j],  a = softmax_j scale (q'[b,h] . c[b,j] + q_R[b,h] . k_R[b,j]),
 *   q'[b,h]  = W_UK[h]^T q_C[b,h]
 *   q_C [B,H,d_h], q_R [B,H,d_R], W_UK and W_UV [H,d_h,d_c], all in `dtype` (MLA_F32 or MLA_BF16);
 *   cache, seq_lens, max_len, scale: as for mla_decode_attn
 *   out      [B,H,d_h] float32 (written)
 *   q_abs    [B,H,d_c] in `dtype`, o_latent [B,H,d_c] float32, lse [B,H] float32: written when not
 *            NULL (the intermediate results of the three calls; NULL = not needed)
 *   workspace at least mla_decode_step_workspace_bytes(B, H, d_c, max_len) bytes, 16-byte aligned.
 *            Its first mla-defined bytes are a flag region that must be ZERO before the first call
 *            (zero-filled memory, or mla_decode_step_init); every call leaves it zero.  The int32
 *            at byte 0 is a sticky error word: nonzero after a one-launch call in which a wait
 *            between workgroups gave up (after 20 ms; results of that call are invalid, and the
 *            workspace must be re-initialised with mla_decode_step_init).
 * One launch when: dtype and both cache parts MLA_BF16, B == 1, H == 128, d_h == 128, d_c == 512,
 * d_R == 64, max_len <= 4096, paged page_size a multiple of 32, 16-byte aligned inputs, cache rows
 * and o_latent, 4-byte aligned q_abs, and at least 256 compute units on the current device.  That
 * kernel keeps one workgroup on each of 256 compute units, and its workgroups wait for each other:
 * do not run it concurrently with other work that occupies compute units for a long time (a wait
 * that cannot complete gives up after 20 ms and sets the error word).  Otherwise the step is the
 * three calls, mla_absorb_q -> mla_decode_partial_warm (W_UV warmed) -> mla_decode_combine_uv,
 * with the automatic split count, their buffers carved from the workspace.
 * Errors as for those calls; nothing is launched when validation fails.  B == 0 is a no-op.
 */
size_t mla_decode_step_workspace_bytes(int B, int H, int d_c, int max_len);
int mla_decode_step_init(void* workspace, size_t workspace_bytes, void* stream);
int mla_decode_step(const void* q_C, const void* q_R, const void* W_UK, const void* W_UV, int dtype,
                    const mla_cache_desc* cache, const int32_t* seq_lens, int max_len, int B, int H, int d_h,
                    int d_c, int d_R, float scale, void* workspace, size_t workspace_bytes, void* q_abs,
                    float* o_latent, float* lse, float* out, void* stream);

/*
 * Workspace (device bytes) mla_cache_append needs: (D / 512) x B x 576 float32 partial sums of
 * the projection.  Returns 0 for unsupported sizes (B < 1, D not a positive multiple of 512).
 */
size_t mla_cache_append_workspace_bytes(int B, int D);

/*
 * mla_cache_append -- write each sequence's new token into its cache row, the step before the
 * attention pass ("MLA storage: Representing KV with a small latent vector", sections "Forming
 * head-specific K and V from a small vector" and "Storing a positional key separately";
 * "Grouped-query and latent attention", section "Why a separate rotary key"):
 *   latent   c_b   = W_DKV h_b
 *   rope key k_R,b = RoPE_pos[b](W_KR h_b): pair (2i, 2i+1) turned by pos[b] * rope_base^(-2i/d_R)
 * stored at row pos[b] of sequence b in the cache described by `cache` (the same descriptor the
 * attention pass reads; its latent, rope and latent_scale buffers are WRITTEN, only at that row).
 *   h        [B, D] bf16      hidden states of the new tokens
 *   W_DKV    [d_c, D] bf16    (row i maps h to latent component i)
 *   W_KR     [d_R, D] bf16
 *   dtype    MLA_BF16 (the dtype of h and both weights)
 *   pos      [B] int32 device: row index (0-based position) of each new token; must lie inside
 *            the cache (contiguous: below its per-sequence capacity; paged: a valid block-table
 *            entry).  Not validated (that would need a host sync).
 *   workspace device buffer of at least mla_cache_append_workspace_bytes(B, D) bytes,
 *            16-byte aligned, any contents; overwritten
 * fp32 accumulation; rope angles in double precision.  Storage: MLA_BF16 latent and rope are
 * rounded to nearest even; an MLA_FP8_E4M3 latent stores OCP E4M3 codes RNE(clamp(c/s, +-448))
 * with the float32 scale s = amax/448 over the row (s = 1 when the row is zero) in latent_scale.
 * Supported: d_c == 512, d_R == 64, D a multiple of 512, rope MLA_BF16, latent MLA_BF16 or
 * MLA_FP8_E4M3, contiguous or paged, 16-byte aligned pointers and rows, B <= 65535, B D < 2^31.
 * B == 0 is a no-op.  Deterministic.  Up to 8 tokens a bf16 cache row is written by the
 * projection itself (one kernel); otherwise, and for E4M3 (which needs the row's amax first), the
 * projection's chunk partials are finished by a second kernel.
 */
int mla_cache_append(const void* h, const void* W_DKV, const void* W_KR, int dtype, const int32_t* pos,
                     const mla_cache_desc* cache, int B, int D, int d_c, int d_R, float rope_base, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Same-dimension comparison path (not part of the latent path): plain multi-head attention decode
 * with an explicit per-head K/V cache at the V3 head sizes, keys d_k = 192 (128 content + 64 rope
 * components), values d_v = 128 -- H (d_k + d_v) values per token and layer against the latent
 * path's d_c + d_R ("Grouped-query and latent attention", section "Multi-head latent attention
 * (MLA)"; the pages ask for comparisons at the same dimensions, "DeepSeek MLA: ...", section
 * "Memory savings do not automatically equal latency savings").
 *
 * mla_mha_decode_workspace_bytes: workspace for these sizes (num_splits 0 = the library's choice,
 * the same one mla_mha_decode makes); 0 for invalid sizes.
 *
 * mla_mha_decode: out[b,h] = sum_j a_j V[b,h,j] with a = softmax_j(scale q[b,h] . K[b,h,j]) over
 * j < seq_lens[b]; lse as for mla_decode_attn.
 *   q        [B, H, d_k] bf16
 *   k_cache  [B, H, cap, d_k] bf16, v_cache [B, H, cap, d_v] bf16 (head-major rows)
 *   seq_lens [B] int32 device, 0 <= len <= max_len <= cap (max_len checked on the host)
 *   out      [B, H, d_v] float32 (written); lse [B, H] float32 or NULL
 *   workspace at least mla_mha_decode_workspace_bytes(B, H, max_len, num_splits) bytes, 16-byte
 *            aligned, any contents; overwritten
 * Supported: dtype MLA_BF16, d_k == 192, d_v == 128, 16-byte aligned pointers.  fp32 arithmetic.
 * A sequence with len 0 gives out = 0 and lse = -inf.  Two kernel launches on `stream`.
 */
size_t mla_mha_decode_workspace_bytes(int B, int H, int max_len, int num_splits);
int mla_mha_decode(const void* q, const void* k_cache, const void* v_cache, int dtype, const int32_t* seq_lens,
                   int max_len, int64_t cap, int B, int H, int d_k, int d_v, float scale, int num_splits,
                   void* workspace, size_t workspace_bytes, float* out, float* lse, void* stream);

/*
 * Projections around the attention core.  Each is y[b, n] = sum_k W[n, k] x[b, k] over a bf16
 * weight W [N, K] (row n maps x to output n, the column-vector form y = W x) with fp32
 * accumulation.  Up to 4 tokens, or up to 8 tokens when K >= 4096 and N * K <= 32M: a streaming GEMV, no
 * workspace needed.  Otherwise: bf16 MFMA (fp32 x is rounded to bf16 for it) split over K, partial sums in
 * the workspace, added in a fixed order.  Deterministic.
 *
 * mla_proj_workspace_bytes: workspace of one projection with B tokens, N outputs, K inputs
 * (0 when the GEMV serves it); mla_query_workspace_bytes: workspace of mla_query_proj (the larger
 * of its two projections).  0 for invalid sizes.
 */
size_t mla_proj_workspace_bytes(int B, int N, int K);
size_t mla_query_workspace_bytes(int B, int D, int d_q, int H, int d_h, int d_R);

/*
 * mla_query_proj -- the query side of a decode step ("Grouped-query and latent attention",
 * sections "Multi-head latent attention (MLA)" and "Why a separate rotary key"):
 *   c_q = W_DQ h,   q_C = W_UQ c_q,   q_R = RoPE_pos(W_QR c_q) per head
 *   h     [B, D] bf16            hidden states of the new tokens
 *   W_DQ  [d_q, D] bf16          W_UQ [H d_h, d_q] bf16 (head h: rows h d_h ..)
 *   W_QR  [H d_R, d_q] bf16      (head h: rows h d_R ..)
 *   pos   [B] int32 device       position of each new token (the rotation the cache write gives
 *                                its key: pair (2i, 2i+1) of each head turned by
 *                                pos * rope_base^(-2i/d_R), angles in double precision)
 *   c_q   [B, d_q] bf16 written  (also the input of mla_absorb_q_folded)
 *   q_C   [B, H, d_h] bf16 written (the input of mla_absorb_q), q_R [B, H, d_R] bf16 written
 *         (the input of mla_decode_attn)
 *   workspace at least mla_query_workspace_bytes(...) bytes (NULL allowed when that is 0),
 *         16-byte aligned, any contents; overwritten
 * c_q is rounded to bf16 before the second projection reads it.  No normalisation is applied.
 * Supported: dtype MLA_BF16, d_R == 64, d_h even, H d_h a multiple of 8, D and d_q multiples of
 * 512, d_q and H (d_h + d_R) multiples of 32, B D < 2^31, 16-byte aligned pointers.  B == 0 is a no-op.  Two projections
 * on `stream` (one kernel each on the GEMV path, two on the MFMA path).
 */
int mla_query_proj(const void* h, const void* W_DQ, const void* W_UQ, const void* W_QR, int dtype,
                   const int32_t* pos, int B, int D, int d_q, int H, int d_h, int d_R, float rope_base, void* c_q,
                   void* q_C, void* q_R, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_query_proj_append -- mla_query_proj and mla_cache_append of the same new tokens in two
 * projections instead of three: W_DQ, W_DKV and W_KR all project h, so one pass over the stacked
 * rows [W_DQ; W_DKV; W_KR] writes c_q and the new cache row (latent, and the rope key turned at
 * pos) together; the second pass is mla_query_proj's.  Arguments as for those two calls; the
 * cache must be bf16 (latent and rope; E4M3 caches need the row's amax first: use the two
 * calls).  workspace: at least mla_query_append_workspace_bytes(B, D, d_q, H, d_h, d_R, d_c)
 * bytes (NULL allowed when 0).  Up to 8 tokens the results are bitwise those of the two separate
 * calls (the same per-row kernel); beyond, every output is the same sums split into other K
 * chunks (the stacked rows are a different projection shape), equal up to rounding.
 * Supported: dtype MLA_BF16, d_c == 512, d_R == 64, and mla_query_proj's shape rules.
 */
size_t mla_query_append_workspace_bytes(int B, int D, int d_q, int H, int d_h, int d_R, int d_c);
int mla_query_proj_append(const void* h, const void* W_DQ, const void* W_UQ, const void* W_QR, const void* W_DKV,
                          const void* W_KR, int dtype, const int32_t* pos, const mla_cache_desc* cache, int B, int D,
                          int d_q, int H, int d_h, int d_R, int d_c, float rope_base, void* c_q, void* q_C, void* q_R,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_fold_q -- the absorbed query projection, folded once when the weights are loaded
 * ("The Journey to Multi-Head Latent Attention", section "The absorption trick (the magic)"):
 *   W_QK[h] = W_UK[h]^T W_UQ[h d_h : (h+1) d_h, :]      [H, d_c, d_q] bf16 written
 *   W_UQ [H d_h, d_q] bf16, W_UK [H, d_h, d_c] bf16 (the layout mla_absorb_q takes)
 * fp32 sums of the exact bf16 products, rounded to bf16 once.  Supported: dtype MLA_BF16, d_h a
 * multiple of 32, d_c and d_q multiples of 64, 16-byte aligned pointers.  One kernel on `stream`.
 *
 * mla_absorb_q_folded -- q'[b, h] = W_QK[h] c_q[b]: the same absorbed query mla_absorb_q makes
 * from q_C, computed from c_q with the folded weights.
 *   c_q [B, d_q] bf16, W_QK [H, d_c, d_q] bf16, q_abs [B, H, d_c] written, MLA_BF16 or MLA_F32
 *   workspace at least mla_proj_workspace_bytes(B, H d_c, d_q) bytes (NULL allowed when 0)
 * Supported: dtype MLA_BF16, d_q a multiple of 512, H d_c a multiple of 32, B d_q < 2^31,
 * 16-byte aligned pointers.  B == 0 is a no-op.
 */
int mla_fold_q(const void* W_UQ, const void* W_UK, int dtype, void* W_QK, int H, int d_h, int d_c, int d_q,
               void* stream);
int mla_absorb_q_folded(const void* c_q, const void* W_QK, int dtype, void* q_abs, int out_dtype, int B, int H,
                        int d_c, int d_q, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_out_proj -- the output projection after the heads ("The Journey to Multi-Head Latent
 * Attention", section "The absorption trick (the magic)"): out[b] = W x[b] with
 *   x   [B, K] float32: the heads' outputs o [B, H, d_h] of mla_uv_out (K = H d_h, W = W_O), or
 *       the latent outputs [B, H, d_c] of mla_decode_attn (K = H d_c, W = W_OV from mla_fold_o)
 *   W   [D, K] bf16, out [B, D] float32 written
 *   workspace at least mla_proj_workspace_bytes(B, D, K) bytes (NULL allowed when 0)
 * Supported: w_dtype MLA_BF16, D a multiple of 32, K a multiple of 512, B K < 2^30, 16-byte
 * aligned pointers.  B == 0 is a no-op.
 *
 * mla_fold_o -- W_UV merged into W_O once when the weights are loaded ("Grouped-query and latent
 * attention", section "The absorption trick"):
 *   W_OV[:, h d_c : (h+1) d_c] = W_O[:, h d_h : (h+1) d_h] W_UV[h]     [D, H d_c] bf16 written
 *   W_O [D, H d_h] bf16, W_UV [H, d_h, d_c] bf16 (the layout mla_uv_out takes)
 * fp32 sums, rounded to bf16 once.  Supported: dtype MLA_BF16, d_h a multiple of 32, d_c and D
 * multiples of 64, 16-byte aligned pointers.  One kernel on `stream`.
 */
int mla_out_proj(const float* x, const void* W, int w_dtype, float* out, int B, int D, int K, void* workspace,
                 size_t workspace_bytes, void* stream);
int mla_fold_o(const void* W_O, const void* W_UV, int dtype, void* W_OV, int D, int H, int d_h, int d_c,
               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_AMD_MLA_H */
