// Device pieces shared by the expert-FFN kernels: argument block, the K
// mapping of a 128-wide chunk onto MFMA lanes, the block-scaled MFMA, the
// split of bf16 activation rows into E4M3 hi + lo with E8M0 scales (as a pass
// and as the gate/up epilogue), raw weight loads and their in-register
// decode to bf16.
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
  // block-scaled prefill: the A operand (x rows for gate/up, h rows for down)
  // split into E4M3 hi and lo bytes in A order ([rows][K] each) and one E8M0
  // scale per 32 along K ([rows][K/32])
  const uint8_t* aq_hi;
  const uint8_t* aq_lo;
  const uint8_t* aq_sc;
  // block-scaled prefill, gate/up: h written split as the down GEMM's A
  // operand (same layout as aq_*), in place of bf16 h
  uint8_t* hq_hi = nullptr;
  uint8_t* hq_lo = nullptr;
  uint8_t* hq_sc = nullptr;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Block-scaled MFMA (CDNA4 v_mfma_scale_f32_16x16x128_f8f6f4), A in E4M3 and
// B in E2M1, one E8M0 scale per 32 consecutive K of each row (A) and column
// (B).  Operand layouts (checked on the device against a CPU model):
//  * E2M1 B: lane (g, i) holds column i, K [32g, 32g+32) of the 128-chunk,
//    low nibble first (the weights' memory order); its scale register holds
//    that block's E8M0 byte (byte 0 is used).
//  * E4M3 A: lane (g, i) holds row i, K [16g, 16g+16) in bytes 0..15 and
//    K [64+16g, 64+16g+16) in bytes 16..31; the scale for row i's 32-block s
//    comes from lane (s, i).
//  * C: lane (g, i) element r is C[4g + r][i], as for the other 16x16 shapes.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

__device__ __forceinline__ f32x4 mfma_mx(i32x8 a, i32x4 b, int sa, int sb, f32x4 c) {
  const i32x8 bb = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bb, c, 0, 4, 0, sa, 0, sb);
}

// Both operands E4M3 (same lane layout for B as for A); B's scale is 1.
__device__ __forceinline__ f32x4 mfma_f8(i32x8 a, i32x8 b, int sa, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127);
}

// Pins an accumulator at this point of the program: an MFMA chain whose result
// is only read at the end would otherwise be sunk there as a whole, keeping
// every chunk's operands live at once.
__device__ __forceinline__ void pin(f32x4& acc) { asm volatile("" : "+v"(acc)); }
// The same, keeping the accumulator in accumulation registers (AGPRs).
__device__ __forceinline__ void pin_a(f32x4& acc) { asm volatile("" : "+a"(acc)); }

// Byte offset of element r of a row in the E4M3 A order (rows of K bytes).
__device__ __forceinline__ int a_order(int r) {
  const int rr = r & 127;
  return (r & ~127) + ((rr & 63) >> 4) * 32 + (rr >> 6) * 16 + (rr & 15);
}

// Four floats -> E4M3 bytes of their RNE values (hw) and of the residuals (lw).
__device__ __forceinline__ void e4m3_hi_lo(float a0, float a1, float a2, float a3, int& hw,
                                           int& lw) {
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  hw = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, hw, true);
  const float r0 = a0 - __builtin_amdgcn_cvt_f32_fp8(hw, 0);
  const float r1 = a1 - __builtin_amdgcn_cvt_f32_fp8(hw, 1);
  const float r2 = a2 - __builtin_amdgcn_cvt_f32_fp8(hw, 2);
  const float r3 = a3 - __builtin_amdgcn_cvt_f32_fp8(hw, 3);
  lw = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
  lw = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, lw, true);
}

// bf16 rows [rows][K] (row pitch src_pitch elements) -> E4M3 hi and lo bytes
// in A order ([rows][K] each) and one E8M0 scale per 32 consecutive K
// ([rows][K/32]), by NT threads (thread index `tid`).  The block scale 2^e
// puts the block's largest magnitude in [128, 256); hi = RNE_e4m3(x / 2^e)
// and lo = RNE_e4m3(x / 2^e - hi).  hi takes the top 4 significant bits of
// the bf16 value and the residual at most 4 more, so hi + lo equals x / 2^e
// whenever that residual is a multiple of 2^-9 (the E4M3 subnormal step),
// i.e. for |x / 2^e| >= 1/4; smaller elements (more than 2^9 below the block
// maximum) lose the bits under 2^-9, an error of at most 2^-10 * 2^e, at most
// 2^-17 of the block's largest magnitude.  Work goes in
// rounds of NT*4 16-byte pieces: prep_a_mx_load issues one round's loads,
// prep_a_mx_store converts and stores them, so the loads of the first round
// can be issued early and other loads issued behind them.
template <int NT>
__device__ __forceinline__ void prep_a_mx_load(const uint16_t* __restrict__ src, int rows, int K,
                                               int src_pitch, int i0, int tid, uint4 (&v)[4]) {
  const int per_row = K / 8, n = rows * per_row;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int i = i0 + b * NT + tid;
    v[b] = uint4{0u, 0u, 0u, 0u};
    if (i < n) {
      const int row = i / per_row, r = (i - row * per_row) * 8;
      v[b] = *reinterpret_cast<const uint4*>(src + (size_t)row * src_pitch + r);
    }
  }
}

template <int NT>
__device__ __forceinline__ void prep_a_mx_store(const uint4 (&v)[4], int rows, int K, int i0,
                                                int tid, uint8_t* hi, uint8_t* lo, uint8_t* sc) {
  const int per_row = K / 8, n = rows * per_row;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int i = i0 + b * NT + tid;
    const uint32_t w[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
    float f[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = __uint_as_float(w[q] << 16);
      f[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
    }
    uint32_t am = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t m = __float_as_uint(f[q]) & 0x7fffffffu;
      am = m > am ? m : am;
    }
    // the 4 threads of a 32-block are lanes 4j..4j+3 of one quad
    am = max(am, (uint32_t)dpp_i32<0xB1>((int)am, (int)am));
    am = max(am, (uint32_t)dpp_i32<0x4E>((int)am, (int)am));
    int e = am ? (int)(am >> 23) - 127 - 7 : 0;
    e = e < -127 ? -127 : e;
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    int h0, h1, l0, l1;
    e4m3_hi_lo(f[0] * inv, f[1] * inv, f[2] * inv, f[3] * inv, h0, l0);
    e4m3_hi_lo(f[4] * inv, f[5] * inv, f[6] * inv, f[7] * inv, h1, l1);
    if (i < n) {
      const int row = i / per_row, r = (i - row * per_row) * 8;
      const size_t o = (size_t)row * K + a_order(r);
      *reinterpret_cast<uint2*>(hi + o) = uint2{(uint32_t)h0, (uint32_t)h1};
      *reinterpret_cast<uint2*>(lo + o) = uint2{(uint32_t)l0, (uint32_t)l1};
      if ((r & 31) == 0) sc[(size_t)row * (K / 32) + r / 32] = (uint8_t)(127 + e);
    }
  }
}

// Max over the 16 lanes of each DPP row; every lane receives its row's value.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t x) {
  int v = (int)x;
  auto mx = [](int a, int b) { return (int)((uint32_t)a > (uint32_t)b ? (uint32_t)a : (uint32_t)b); };
  v = mx(v, dpp_i32<0xB1>(0, v));   // quad_perm [1,0,3,2]
  v = mx(v, dpp_i32<0x4E>(0, v));   // quad_perm [2,3,0,1]
  v = mx(v, dpp_i32<0x141>(0, v));  // row_half_mirror
  v = mx(v, dpp_i32<0x140>(0, v));  // row_mirror
  return (uint32_t)v;
}

// Gate/up epilogue of the block-scaled prefill kernels: one row's 32-column
// block of h, held by the 16 lanes of one DPP row as (lane l16, half j) =
// column 16 j + l16 of the block starting at column c0.  Rounds the values to
// bf16 and writes the E4M3 hi / lo bytes (A order) and the E8M0 scale that
// prep_a_mx_store makes from those bf16 values, the down GEMM's A operand.
// Every lane of the row takes part (the maximum crosses lanes); `store` must
// be the same for all 16.
__device__ __forceinline__ void h32_split_store(float h0, float h1, bool store, int l16, int c0,
                                                uint8_t* hi_row, uint8_t* lo_row,
                                                uint8_t* sc_row) {
  const float f0 = bf16_to_f32(f32_to_bf16_rne(h0)), f1 = bf16_to_f32(f32_to_bf16_rne(h1));
  const uint32_t m0 = __float_as_uint(f0) & 0x7fffffffu, m1 = __float_as_uint(f1) & 0x7fffffffu;
  const uint32_t am = row16_max_u32(m0 > m1 ? m0 : m1);
  int e = am ? (int)(am >> 23) - 127 - 7 : 0;
  e = e < -127 ? -127 : e;
  const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
  int hw, lw;
  e4m3_hi_lo(f0 * inv, f1 * inv, 0.0f, 0.0f, hw, lw);
  if (store) {
    const int o0 = a_order(c0 + l16), o1 = a_order(c0 + 16 + l16);
    hi_row[o0] = (uint8_t)hw;
    lo_row[o0] = (uint8_t)lw;
    hi_row[o1] = (uint8_t)(hw >> 8);
    lo_row[o1] = (uint8_t)(lw >> 8);
    if (l16 == 0) sc_row[c0 / 32] = (uint8_t)(127 + e);
  }
}

template <int NT>
__device__ __forceinline__ void prep_a_mx(const uint16_t* __restrict__ src, int rows, int K,
                                          int src_pitch, uint8_t* hi, uint8_t* lo, uint8_t* sc,
                                          int tid = threadIdx.x) {
  const int n = rows * (K / 8);
  for (int i0 = 0; i0 < n; i0 += NT * 4) {
    uint4 v[4];
    prep_a_mx_load<NT>(src, rows, K, src_pitch, i0, tid, v);
    prep_a_mx_store<NT>(v, rows, K, i0, tid, hi, lo, sc);
  }
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
  const int slot = a.slot_of ? dbg_clamp(a.slot_of[e], a.E, kDbgSlot) : e;
  return a.base + (size_t)slot * a.stride;
}

}  // namespace moe
