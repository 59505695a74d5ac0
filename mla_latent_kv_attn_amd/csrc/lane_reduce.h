// Cross-lane sum of K per-lane values over a 64-lane wave by halving exchange (gfx950 only).
#pragma once

#include "mla_internal.h"

namespace mla {

// Each step exchanges half of the values a lane still holds with the lane d = 32, 16, ... away
// and adds, so K values need K - 1 + log2(64 / K) exchanges instead of 6 K.  Afterwards lane l
// holds the full sum of value index (l >> (6 - log2 K)) & (K - 1); the lanes sharing that index
// (the low 6 - log2 K lane bits) all hold it.
//
// The pair (v[i], v[i + half]) passes through an empty asm statement before the select: without
// it the compiler turns "upper ? v[i] : v[i + half]" into one load from a computed index of the
// array, which it then emulates with compare/select chains over all K registers (O(K^2) VALU).
template <int K>
__device__ __forceinline__ float lane_sum_halving(float (&v)[K], int lane) {
  static_assert(K >= 2 && K <= 64 && (K & (K - 1)) == 0, "K: a power of two in [2, 64]");
  constexpr int LK = K == 2 ? 1 : K == 4 ? 2 : K == 8 ? 3 : K == 16 ? 4 : K == 32 ? 5 : 6;
#pragma unroll
  for (int step = 0; step < LK; ++step) {
    const int d = 32 >> step;
    const int half = K >> (step + 1);
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
  float t = v[0];
#pragma unroll
  for (int d = (32 >> (LK - 1)) >> 1; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
  return t;
}

}  // namespace mla
