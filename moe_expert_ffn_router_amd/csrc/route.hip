// Router: top-k experts per token with renormalised softmax weights.
//
// One wavefront per token.  Lane l holds logits l, l+64, ... of its token as
// 64-bit keys (order-preserving map of the fp32 value in the high half, the
// complement of the expert index in the low half), so a single unsigned
// max picks the largest logit and, among equal logits, the lowest index.
// Each of the k rounds is a lane-local max plus a 6-step butterfly; the
// winner's key is cleared in its owner lane.  Lane j < k keeps round j's
// winner and finally computes exp(l_j - l_0) / sum.
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

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = __shfl_xor(v, m, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int renorm, int* __restrict__ ids,
                                                    float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  unsigned long long key[VPL];
  float val[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    val[i] = (e < E) ? row[e] : 0.0f;
    key[i] = (e < E) ? (((unsigned long long)order_key(val[i]) << 32) | (uint32_t)(~(uint32_t)e))
                     : 0ull;
  }

  int my_id = 0;
  float my_val = 0.0f;
  for (int r = 0; r < k; ++r) {
    unsigned long long best = key[0];
#pragma unroll
    for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    const unsigned long long g = wave_max_u64(best);
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (key[i] == g) key[i] = 0ull;
    if (lane == r) {
      my_id = (int)(~(uint32_t)g);
      my_val = key_value((uint32_t)(g >> 32));
    }
  }

  const float v0 = __shfl(my_val, 0, 64);
  float z = (lane < k) ? expf(my_val - v0) : 0.0f;
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
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    wts[(size_t)t * k + lane] = z / denom;
  }
}

}  // namespace moe

extern "C" int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                         int32_t* topk_ids, float* topk_w, moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "moe_route: need T>=0, 1<=E<=%d, 1<=k<=min(E,%d) "
                     "(T=%d E=%d k=%d)", kMaxE, kMaxK, T, E, k);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_w)
    return set_error(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
  if (!aligned16(logits) || !aligned16(topk_ids) || !aligned16(topk_w))
    return set_error(MOE_ERR_INVALID_ARG, "moe_route: pointers must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, renorm, topk_ids, topk_w);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, renorm, topk_ids, topk_w);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, renorm, topk_ids, topk_w);
  else if (E <= 512)
    route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, renorm, topk_ids, topk_w);
  else
    route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, renorm, topk_ids, topk_w);
  return check_launch("moe_route");
}
