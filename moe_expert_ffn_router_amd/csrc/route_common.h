// Per-token router top-k shared by the routing kernels: one wavefront routes
// one token.  Lane l holds logits l, l+64, ... as order-preserving 32-bit keys
// (-0.0 mapped to +0.0), each packed with its complemented index.  Each of
// the k rounds takes the lane-local maximum and a DPP wave maximum of the
// packed values: the largest key, lowest index first among equal keys.  The
// owner clears the winner; lane j < k keeps round j's winner and finally the
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

// Logits of one token into the calling wave's lanes (slot i = index lane + 64i).
template <int VPL>
__device__ __forceinline__ void route_load(const float* __restrict__ row, int E, int lane,
                                           float (&val)[VPL]) {
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    val[i] = (e < E) ? row[e] : 0.0f;
  }
}

// Top-k of loaded logits with the calling wave; lane j < k returns (id_j, w_j).
// Each slot is packed as (key << 32 | ~index): one 64-bit wave maximum gives
// the largest key and, among equal keys, the lowest index; the owning lane
// clears it with selects (no branches).  Slots past E are 0, below any logit.
template <int VPL>
__device__ __forceinline__ void route_select(const float (&val)[VPL], int E, int k, int renorm,
                                             int lane, int& my_id, float& my_w) {
  uint64_t pk[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    pk[i] = (e < E) ? ((uint64_t)order_key(val[i]) << 32) | (uint32_t)~e : 0ull;
  }
  my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = pk[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = pk[i] > best ? pk[i] : best;
    const uint64_t g = wave_max_u64(best);
    const int win = (int)~(uint32_t)g;
#pragma unroll
    for (int i = 0; i < VPL; ++i) pk[i] = (lane + 64 * i == win) ? 0ull : pk[i];
    if (lane == r) {
      my_id = win;
      my_val = key_value((uint32_t)(g >> 32));
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

// Route one token with the calling wave; lane j < k returns (id_j, w_j).
template <int VPL>
__device__ __forceinline__ void route_token(const float* __restrict__ row, int E, int k, int renorm,
                                            int lane, int& my_id, float& my_w) {
  float val[VPL];
  route_load<VPL>(row, E, lane, val);
  route_select<VPL>(val, E, k, renorm, lane, my_id, my_w);
}

inline int vpl_of(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

}  // namespace moe
