// Per-token router top-k shared by the routing kernels: one wavefront routes
// one token.  Lane l holds logits l, l+64, ... as order-preserving 32-bit keys
// (-0.0 mapped to +0.0).  Each of the k rounds takes the lane-local maximum,
// a DPP wave maximum, then the lowest expert index holding that key (ballot
// over the lane's slots in index order: index e = lane + 64*slot).  The owner
// clears the winner; lane j < k keeps round j's winner and finally the
// softmax over the k selected logits (or the full-softmax value).
#pragma once

#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0.0 ranks equal to +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Route one token with the calling wave; lane j < k returns (id_j, w_j).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int renorm,
                                            int lane, int& my_id, float& my_w) {
  uint32_t key[VPL];
  float val[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    val[i] = (e < E) ? row[e] : 0.0f;
    key[i] = (e < E) ? order_key(val[i]) : 0u;
  }
  my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint32_t best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    const uint32_t g = wave_max_u32(best);
    int win = -1;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const uint64_t b = __ballot(key[i] == g);
      if (win < 0 && b) {
        const int wl = (int)__builtin_ctzll(b);
        win = wl + 64 * i;
        if (lane == wl) key[i] = 0u;
      }
    }
    if (win >= E || win < 0) win = E - 1;  // only reachable with NaN logits
    if (lane == r) {
      my_id = win;
      my_val = key_value(g);
    }
  }
  const float v0 = __shfl(my_val, 0, 64);
  const float z = (lane < k) ? expf(my_val - v0) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum_f32(z);
  } else {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) s += expf(val[i] - v0);
    denom = wave_sum_f32(s);
  }
  my_w = z / denom;
}

inline int vpl_of(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

}  // namespace moe
