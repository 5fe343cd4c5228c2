// Weighted combine: y[t] = sum_j w[t,j] * y_perm[inv[t*k+j]] (+ y_shared[t]),
// fp32 sum in j order, one rounding to bf16.  Pure gather + streaming: each
// thread owns 8 consecutive columns (one 16-byte load per source row), a
// workgroup owns one token row and loops over the columns.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_perm,
                                                      const int* __restrict__ inv_idx,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int H,
                                                      const uint16_t* __restrict__ y_shared,
                                                      uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  __shared__ int src[kMaxK];
  __shared__ float wt[kMaxK];
  if (threadIdx.x < k) {
    src[threadIdx.x] = dbg_clamp(inv_idx[(size_t)t * k + threadIdx.x], T * k, kDbgInv);
    wt[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    for (int j = 0; j < k; ++j) {
      const uint4 v = *reinterpret_cast<const uint4*>(y_perm + (size_t)src[j] * H + c);
      const float w = wt[j];
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(w, __uint_as_float(q[i] << 16), acc[2 * i]);
        acc[2 * i + 1] = fmaf(w, __uint_as_float(q[i] & 0xffff0000u), acc[2 * i + 1]);
      }
    }
    if (y_shared) {
      const uint4 v = *reinterpret_cast<const uint4*>(y_shared + (size_t)t * H + c);
      const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += __uint_as_float(q[i] << 16);
        acc[2 * i + 1] += __uint_as_float(q[i] & 0xffff0000u);
      }
    }
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(y + (size_t)t * H + c) = o;
  }
}

#ifdef MOE_DEBUG
uint32_t dbg_take_combine() { return dbg_take_unit(); }
#endif

}  // namespace moe

extern "C" int moe_combine(const uint16_t* y_perm, const int32_t* inv_idx, const float* topk_w,
                           int32_t T, int32_t k, int32_t H, const uint16_t* y_shared, uint16_t* y,
                           moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || k < 1 || k > kMaxK || H < 8 || H % 8)
    return set_error(MOE_ERR_INVALID_ARG, "moe_combine: need T>=0, 1<=k<=%d, H multiple of 8",
                     kMaxK);
  if (T == 0) return MOE_OK;
  if (!y_perm || !inv_idx || !topk_w || !y)
    return set_error(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  if (!aligned16(y_perm) || !aligned16(inv_idx) || !aligned16(topk_w) || !aligned16(y) ||
      (y_shared && !aligned16(y_shared)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_combine: pointers must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  combine_kernel<<<T, 256, 0, s>>>(y_perm, inv_idx, topk_w, T, k, H, y_shared, y);
  return check_launch("moe_combine");
}
