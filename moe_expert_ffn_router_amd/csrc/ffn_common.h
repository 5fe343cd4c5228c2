// Device pieces shared by the expert-FFN kernels: argument block, the K
// mapping of a 128-wide chunk onto MFMA lanes, raw weight loads and their
// in-register decode to bf16.
#pragma once

#include "moe_internal.h"

namespace moe {

constexpr int KC = 128;          // K chunk
constexpr int A_PITCH = KC + 8;  // LDS row pitch in bf16 (16-byte pad: no bank conflicts)

struct FfnArgs {
  int E, H, I, k, A;
  const uint8_t* base;
  int64_t stride;
  const int* slot_of;
  int64_t off_w13, off_w13s, off_w2, off_w2s, off_ts;
  const uint16_t* x;
  const int* counts;
  const int* offsets;
  const int* sorted_idx;
  uint16_t* hbuf;
  uint16_t* y_perm;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// weight loads: raw bytes first (so many can be in flight), decode later
// ---------------------------------------------------------------------------
template <int FMT>
struct BRaw {
  uint4 q[FMT == MOE_W_BF16 ? 4 : FMT == MOE_W_FP8_B128 ? 2 : 1];
  uint32_t s;   // MX: E8M0 byte; NV: two E4M3 bytes
  float bs;     // FP8: block scale
};

// Raw bytes of the 32 consecutive K values [k0, k0+32) of weight row `row`.
template <int FMT>
__device__ __forceinline__ void load_b_raw(const uint8_t* __restrict__ w,
                                           const uint8_t* __restrict__ sc, int row, int K, int k0,
                                           BRaw<FMT>& r) {
  if constexpr (FMT == MOE_W_MXFP4) {
    r.q[0] = *reinterpret_cast<const uint4*>(w + (((size_t)row * K + k0) >> 1));
    r.s = sc[(size_t)row * (K / 32) + k0 / 32];
  } else if constexpr (FMT == MOE_W_NVFP4) {
    r.q[0] = *reinterpret_cast<const uint4*>(w + (((size_t)row * K + k0) >> 1));
    r.s = *reinterpret_cast<const uint16_t*>(sc + (size_t)row * (K / 16) + k0 / 16);
  } else if constexpr (FMT == MOE_W_FP8_B128) {
    const uint4* p = reinterpret_cast<const uint4*>(w + (size_t)row * K + k0);
    r.q[0] = p[0];
    r.q[1] = p[1];
    r.bs = reinterpret_cast<const float*>(sc)[(size_t)(row / 128) * (K / 128) + k0 / 128];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(w + ((size_t)row * K + k0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.q[i] = p[i];
  }
}

template <int FMT>
__device__ __forceinline__ void decode_b(const BRaw<FMT>& r, bf16x8 (&b)[4]) {
  if constexpr (FMT == MOE_W_MXFP4) {
    const float s = e8m0_to_f32(r.s);
    b[0] = fp4x8_to_bf16(r.q[0].x, s); b[1] = fp4x8_to_bf16(r.q[0].y, s);
    b[2] = fp4x8_to_bf16(r.q[0].z, s); b[3] = fp4x8_to_bf16(r.q[0].w, s);
  } else if constexpr (FMT == MOE_W_NVFP4) {
    const float s0 = e4m3_to_f32(r.s & 0xffu), s1 = e4m3_to_f32((r.s >> 8) & 0xffu);
    b[0] = fp4x8_to_bf16_mul(r.q[0].x, s0); b[1] = fp4x8_to_bf16_mul(r.q[0].y, s0);
    b[2] = fp4x8_to_bf16_mul(r.q[0].z, s1); b[3] = fp4x8_to_bf16_mul(r.q[0].w, s1);
  } else if constexpr (FMT == MOE_W_FP8_B128) {
    b[0] = fp8x8_to_bf16(r.q[0].x, r.q[0].y); b[1] = fp8x8_to_bf16(r.q[0].z, r.q[0].w);
    b[2] = fp8x8_to_bf16(r.q[1].x, r.q[1].y); b[3] = fp8x8_to_bf16(r.q[1].z, r.q[1].w);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = bits_to_bf16x8(r.q[i].x, r.q[i].y, r.q[i].z, r.q[i].w);
  }
}

template <int FMT>
__device__ __forceinline__ float block_scale(const BRaw<FMT>& r) {
  if constexpr (FMT == MOE_W_FP8_B128) return r.bs;
  return 1.0f;
}

__device__ __forceinline__ const uint8_t* record_of(const FfnArgs& a, int e) {
  const int slot = a.slot_of ? a.slot_of[e] : e;
  return a.base + (size_t)slot * a.stride;
}

}  // namespace moe
