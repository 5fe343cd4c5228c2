// Per-token router top-k shared by the routing kernels: one wavefront routes
// one token.  Lane l holds logits l, l+64, ... as order-preserving 32-bit keys
// (-0.0 mapped to +0.0); each lane first sorts its own keys (largest first,
// lower index first among equal keys).  Each of the k rounds is a 32-bit DPP
// wave maximum over the lanes' heads; a ballot of the lanes whose head equals
// it finds the owner (when several lanes tie, a wave minimum of their indices
// picks the lowest index), and the owner pops its head.  Lane j < k keeps
// round j's winner and finally the softmax over the k selected logits (or the
// full-softmax value).
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

// Lane-local state of one token's top-k selection: the lane's remaining keys
// and indices, largest first, and round r's winner (index, key) held by lane r.
template <int VPL>
struct TopK {
  uint32_t key[VPL], idx[VPL];
  int id_r, key_r;
};

// Sort the lane's own logits by (key desc, index asc): the packed value
// (key << 32 | ~index) orders exactly that way.  Slots past E hold key 0 and
// index 0xffffffff, below every logit.
template <int VPL>
__device__ __forceinline__ void topk_begin(const float (&val)[VPL], int E, int lane, TopK<VPL>& s) {
  uint64_t pk[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    pk[i] = (e < E) ? ((uint64_t)order_key(val[i]) << 32) | (uint32_t)~e : 0ull;
  }
#pragma unroll
  for (int p = 0; p < VPL; ++p)
#pragma unroll
    for (int i = p & 1; i + 1 < VPL; i += 2) {
      const uint64_t hi = pk[i] > pk[i + 1] ? pk[i] : pk[i + 1];
      const uint64_t lo = pk[i] > pk[i + 1] ? pk[i + 1] : pk[i];
      pk[i] = hi;
      pk[i + 1] = lo;
    }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    s.key[i] = (uint32_t)(pk[i] >> 32);
    s.idx[i] = ~(uint32_t)pk[i];
  }
  s.id_r = 0;
  s.key_r = 0;
}

// Round r: the largest remaining key over the wave (lowest index among equal
// keys) is popped from its lane and kept by lane r.
template <int VPL>
__device__ __forceinline__ void topk_round(TopK<VPL>& s, int r, int lane) {
  const uint32_t top = wave_max_u32(s.key[0]);
  const uint64_t tied = __builtin_amdgcn_ballot_w64(s.key[0] == top);
  uint32_t win = (uint32_t)__builtin_amdgcn_readlane((int)s.idx[0], (int)__builtin_ctzll(tied));
  if (__builtin_expect(__builtin_popcountll(tied) != 1, 0))  // equal keys in several lanes
    win = wave_min_u32(s.key[0] == top ? s.idx[0] : 0xffffffffu);
  const bool pop = lane == (int)(win & 63u);
#pragma unroll
  for (int i = 0; i + 1 < VPL; ++i) {
    s.key[i] = pop ? s.key[i + 1] : s.key[i];
    s.idx[i] = pop ? s.idx[i + 1] : s.idx[i];
  }
  s.key[VPL - 1] = pop ? 0u : s.key[VPL - 1];
  s.idx[VPL - 1] = pop ? 0xffffffffu : s.idx[VPL - 1];
  s.id_r = lane == r ? (int)win : s.id_r;
  s.key_r = lane == r ? (int)top : s.key_r;
}

// After k rounds: lane j < k returns w_j, the softmax over the k selected
// logits (renorm) or the full-softmax value.
template <int VPL>
__device__ __forceinline__ float topk_weight(const TopK<VPL>& s, const float (&val)[VPL], int E,
                                             int k, int renorm, int lane) {
  const float my_val = key_value((uint32_t)s.key_r);
  const float v0 = __shfl(my_val, 0, 64);
  const float z = (lane < k) ? expf(my_val - v0) : 0.0f;
  float denom;
  if (renorm) {
    denom = wave_sum_f32(z);
  } else {
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (lane + 64 * i < E) sum += expf(val[i] - v0);
    denom = wave_sum_f32(sum);
  }
  return z / denom;
}

// Top-k of loaded logits with the calling wave; lane j < k returns (id_j, w_j).
template <int VPL>
__device__ __forceinline__ void route_select(const float (&val)[VPL], int E, int k, int renorm,
                                             int lane, int& my_id, float& my_w) {
  TopK<VPL> s;
  topk_begin<VPL>(val, E, lane, s);
  for (int r = 0; r < k; ++r) topk_round<VPL>(s, r, lane);
  my_id = s.id_r;
  my_w = topk_weight<VPL>(s, val, E, k, renorm, lane);
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
