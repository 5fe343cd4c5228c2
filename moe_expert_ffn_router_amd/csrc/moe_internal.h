// Internal declarations shared by the library's translation units.
// gfx950 (CDNA4) only: wave64, MFMA bf16 16x16x32, OCP FP8/FP4 conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_layer.h"

namespace moe {

// ---------------------------------------------------------------------------
// host-side status plumbing
// ---------------------------------------------------------------------------
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);  // hipGetLastError after a launch

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr int kChunk = 1024;  // assignments per permutation block

// Record layout (host); mirrors the header's description.
struct Layout {
  int64_t w13, w13s, w2, w2s, ts, payload, stride;
};
bool layout_of(int fmt, int H, int I, Layout* out);

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// fp32 -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// E8M0 byte -> fp32 scale 2^(b-127).  b = 0 gives the fp32 subnormal 2^-127;
// b = 255 (NaN) gives NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  if (b == 0) return __uint_as_float(0x00400000u);
  if (b == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(b << 23);
}

// OCP E4M3 byte -> fp32, decoded from its bit fields (bias 7, subnormals kept,
// S.1111.111 = NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0) {
    mag = (float)m * 0.001953125f;  // m/8 * 2^-6 = m * 2^-9
  } else if (e == 15 && m == 7) {
    mag = __uint_as_float(0x7fc00000u);
  } else {
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1+m/8) * 2^(e-7)
  }
  return s ? -mag : mag;
}

// E2M1 code -> fp32 from its bit fields (bias 1, no Inf/NaN).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  const uint32_t s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
  float mag = (e == 0) ? 0.5f * (float)m : __uint_as_float(((e + 126u) << 23) | (m << 22));
  return s ? -mag : mag;
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  i32x4 v = {(int)a, (int)b, (int)c, (int)d};
  return __builtin_bit_cast(bf16x8, v);
}

// 8 E2M1 codes of one dword (element 2i = low nibble of byte i) -> 8 bf16,
// each multiplied by `scale`, which must be a power of two (an E8M0 scale):
// the CDNA4 scaled FP4 -> bf16 conversion applies only the scale's exponent.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16(uint32_t w, float scale) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// 8 E2M1 codes -> 8 bf16 times an arbitrary fp32 scale `s` whose products
// with the E2M1 values are exact in bf16 (an E4M3 block scale: at most 6
// significant bits).  The scaled conversion instructions use only the
// exponent of their scale operand, so the product is formed in fp32 (exact)
// and its upper half taken (exact, no rounding needed).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16_mul(uint32_t w, float s) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  auto hi2 = [s](float a, float b) {
    return __builtin_amdgcn_perm(__float_as_uint(b * s), __float_as_uint(a * s), 0x07060302u);
  };
  return bits_to_bf16x8(hi2(p0[0], p0[1]), hi2(p1[0], p1[1]), hi2(p2[0], p2[1]),
                        hi2(p3[0], p3[1]));
}

// 8 E4M3 bytes (two dwords, byte i = element i) -> 8 bf16 (exact).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}


// ---------------------------------------------------------------------------
// wave64 primitives on DPP lane moves (no LDS round trip).  gfx9 DPP controls:
// quad_perm, row_shr:n (0x110+n), row_mirror, row_half_mirror, row_bcast15,
// row_bcast31.  Results that end in lane 63 are broadcast with readlane.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ int dpp_i32(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

// Wave maximum / minimum: the DPP source operand's "old" value is the
// operation's identity, so each step compiles to one v_max/v_min with a DPP
// modifier (lanes without a source lane keep their value).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  auto mx = [](int a, int b) { return (int)((uint32_t)a > (uint32_t)b ? (uint32_t)a : (uint32_t)b); };
  v = mx(v, dpp_i32<0xB1>(0, v));         // quad_perm [1,0,3,2]
  v = mx(v, dpp_i32<0x4E>(0, v));         // quad_perm [2,3,0,1]
  v = mx(v, dpp_i32<0x141>(0, v));        // row_half_mirror
  v = mx(v, dpp_i32<0x140>(0, v));        // row_mirror
  v = mx(v, dpp_i32<0x142, 0xA>(0, v));   // row_bcast15 into rows 1, 3
  v = mx(v, dpp_i32<0x143, 0xC>(0, v));   // row_bcast31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  int v = (int)x;
  auto mn = [](int a, int b) { return (int)((uint32_t)a < (uint32_t)b ? (uint32_t)a : (uint32_t)b); };
  v = mn(v, dpp_i32<0xB1>(-1, v));
  v = mn(v, dpp_i32<0x4E>(-1, v));
  v = mn(v, dpp_i32<0x141>(-1, v));
  v = mn(v, dpp_i32<0x140>(-1, v));
  v = mn(v, dpp_i32<0x142, 0xA>(-1, v));
  v = mn(v, dpp_i32<0x143, 0xC>(-1, v));
  return (uint32_t)__builtin_amdgcn_readlane(v, 63);
}

// Sum over the wave in a fixed order (identical result in every lane).
__device__ __forceinline__ float wave_sum_f32(float x) {
  int v = __float_as_int(x);
  auto add = [](int a, int b) { return __float_as_int(__int_as_float(a) + __int_as_float(b)); };
  v = add(v, dpp_i32<0xB1>(v, v));
  v = add(v, dpp_i32<0x4E>(v, v));
  v = add(v, dpp_i32<0x141>(v, v));
  v = add(v, dpp_i32<0x140>(v, v));
  v = add(v, dpp_i32<0x142, 0xA>(0, v));
  v = add(v, dpp_i32<0x143, 0xC>(0, v));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i32<0x111, 0xF, true>(0, v);   // row_shr:1
  v += dpp_i32<0x112, 0xF, true>(0, v);   // row_shr:2
  v += dpp_i32<0x114, 0xF, true>(0, v);   // row_shr:4
  v += dpp_i32<0x118, 0xF, true>(0, v);   // row_shr:8
  v += dpp_i32<0x142, 0xA>(0, v);         // row_bcast15
  v += dpp_i32<0x143, 0xC>(0, v);         // row_bcast31
  return v;
}

__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Exclusive scan over E <= kMaxE ints in LDS by all NT threads of the
// workgroup (each owns kMaxE/NT consecutive entries); returns the total.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int* v, int E, int* wave_tot) {
  static_assert(NT % 64 == 0 && kMaxE % NT == 0 && NT / 64 <= 16, "scan shape");
  constexpr int PER = kMaxE / NT, NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int loc[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    loc[i] = (e < E) ? v[e] : 0;
    sum += loc[i];
  }
  const int incl = wave_incl_scan(sum);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = wave_tot[w];
    base += (w < wave) ? t : 0;
    total += t;
  }
  int run = base + incl - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    if (e < E) v[e] = run;
    run += loc[i];
  }
  __syncthreads();
  return total;
}

__device__ __forceinline__ int block_exclusive_scan_256(int* v, int E, int* wave_tot) {
  return block_exclusive_scan<256>(v, E, wave_tot);
}

// Exclusive scan over n <= 1024 ints in LDS with 1024 threads (one each).
__device__ __forceinline__ int block_exclusive_scan_1024(int* v, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int x = tid < n ? v[tid] : 0;
  const int incl = wave_incl_scan(x);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const int t = wave_tot[w];
    base += (w < wave) ? t : 0;
    total += t;
  }
  if (tid < n) v[tid] = base + incl - x;
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// Bounds-checked build (-DMOE_DEBUG).  Every index a kernel takes from a
// caller's array — slot table entries, sorted and inverse indices, the row
// segment an expert's offset and count describe — passes through dbg_clamp /
// dbg_segment: an out-of-range value sets a bit in this translation unit's
// flag word and is replaced by an in-range one, so the kernel stays inside
// its buffers (the results are then meaningless, the flag says so).
// moe_debug_take() returns and clears the flags of every translation unit.
// Release builds compile the checks away.
// ---------------------------------------------------------------------------
enum : uint32_t { kDbgSlot = 1u, kDbgSorted = 2u, kDbgSegment = 4u, kDbgInv = 8u };
#ifdef MOE_DEBUG
static __device__ uint32_t g_dbg_flags;
__device__ __forceinline__ int dbg_clamp(int v, int hi, uint32_t bit) {  // expects 0 <= v < hi
  if (v < 0 || v >= hi) {
    atomicOr(&g_dbg_flags, bit);
    return v < 0 || hi < 1 ? 0 : hi - 1;
  }
  return v;
}
// An expert's rows [seg0, seg0 + rows) must lie in [0, A); else no rows.
__device__ __forceinline__ void dbg_segment(int& seg0, int& rows, int A) {
  if (seg0 < 0 || rows < 0 || (int64_t)seg0 + rows > A) {
    atomicOr(&g_dbg_flags, kDbgSegment);
    seg0 = 0;
    rows = 0;
  }
}
// The flags of the calling translation unit, cleared (host; synchronizes the device).
static inline uint32_t dbg_take_unit() {
  uint32_t v = 0, z = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dbg_flags), sizeof(v)) != hipSuccess ||
      hipMemcpyToSymbol(HIP_SYMBOL(g_dbg_flags), &z, sizeof(z)) != hipSuccess)
    return 0x80000000u;  // the read failed: reported as a flag of its own
  return v;
}
uint32_t dbg_take_ffn();
uint32_t dbg_take_decode();
uint32_t dbg_take_combine();
#else
__device__ __forceinline__ int dbg_clamp(int v, int, uint32_t) { return v; }
__device__ __forceinline__ void dbg_segment(int&, int&, int) {}
#endif

}  // namespace moe
