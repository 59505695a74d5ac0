// Internal declarations of the one-launch decode step (gfx950 only).
#pragma once

#include "mla_internal.h"

namespace mla {

constexpr int kStepWGs = 256;      // workgroups of the one-launch step (one per CU)
constexpr int kStepSplits = 32;    // token splits of the attention phase
constexpr int kStepTiles = 4;      // 32-token tiles per split held in LDS: at most 4096 tokens

struct StepArgs {
  const uint16_t* q_C;          // [128, 128] bf16
  const uint16_t* q_R;          // [128, 64] bf16
  const uint16_t* W_UK;         // [128, 128, 512] bf16
  const uint16_t* W_UV;         // [128, 128, 512] bf16
  const void* latent;           // bf16 latent rows of the sequence (or page pool)
  const void* rope;             // bf16 rope rows
  const int32_t* block_table;   // null = contiguous
  int64_t lat_sb, lat_st, rope_sb, rope_st;
  int page_size;
  const int32_t* seq_lens;      // [1]
  float sl2;                    // softmax scale * log2(e)
  uint16_t* qp;                 // [128, 512] bf16 folded query (written, then read by other workgroups)
  float* part_ml;               // [kStepSplits, 128, 2]
  uint16_t* part_acc;           // [kStepSplits, 128, 512] bf16 acc / l of each split
  int* fa;                      // [4, kStepSplits, 4, 64] flags: q' pieces
  int* fb;                      // [128, kStepSplits] flags: split partials
  int* err;                     // sticky error word: a wait gave up
  float* out;                   // [128, 128]
  float* o_latent;              // [128, 512] or null
  float* lse;                   // [128] or null
};

// workspace of the step: the flag region (must be zero before the first launch; every launch
// leaves it zero), then the data region (shared with the multi-kernel form)
constexpr size_t kStepErrBytes = 256;
constexpr size_t kStepFaInts = (size_t)4 * kStepSplits * 4 * 64;
constexpr size_t kStepFbInts = (size_t)128 * kStepSplits;
constexpr size_t kStepFlagBytes = kStepErrBytes + (kStepFaInts + kStepFbInts) * 4;
constexpr size_t kStepQpBytes = (size_t)128 * 512 * 2;
constexpr size_t kStepMlBytes = (size_t)kStepSplits * 128 * 2 * 4;
constexpr size_t kStepAccBytes = (size_t)kStepSplits * 128 * 512 * 2;

hipError_t launch_step_b1(const StepArgs& a, hipStream_t s);
hipError_t launch_step_zero(int* p, int64_t n, hipStream_t s);

}  // namespace mla
