// Per-expert SwiGLU FFN over the permuted rows: a grouped GEMM on the bf16
// MFMA (V_MFMA_F32_16X16X32_BF16), one launch for gate/up (+ SiLU*mul
// epilogue) and one for down.
//
// Work unit = (m-tile of one expert's rows, block of output columns).  The
// m-tile list is built on the device from `counts` (no host sync), so the
// whole call can be captured into a graph.
//
// Operands.  A = activations, bf16 rows gathered by token (gate/up) or the
// contiguous h rows (down), staged through LDS one 128-wide K chunk at a
// time.  B = expert weights, read straight from HBM into registers in their
// stored format and decoded there to bf16 (CDNA4 scaled FP4/FP8 -> bf16
// conversions; every MXFP4 value, NVFP4 E2M1 x E4M3 product and E4M3 value
// is exact in bf16).  FP8 block scales and NVFP4 tensor scales multiply fp32
// partial sums.
//
// K mapping.  For a 128-wide chunk, lane group g = lane/16 owns the 32
// consecutive K values [32g, 32g+32) of its row; MFMA step s consumes values
// [32g+8s, 32g+8s+8).  A and B use the same mapping, so each output is the
// full dot product regardless of the instruction's internal K order.
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
  const int* tile_info;  // [0] = n_tiles, [1..] expert of tile, then m0 of tile
  int max_tiles;
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32 consecutive K values [k0, k0+32) of weight row `row` -> 4 x bf16x8.
// For FP8 also returns the row's 128x128 block scale in `bs`.
template <int FMT>
__device__ __forceinline__ void load_b(const uint8_t* __restrict__ w, const uint8_t* __restrict__ sc,
                                       int row, int K, int k0, bf16x8 (&b)[4], float& bs) {
  if constexpr (FMT == MOE_W_MXFP4) {
    const uint4 q = *reinterpret_cast<const uint4*>(w + (((size_t)row * K + k0) >> 1));
    const float s = e8m0_to_f32(sc[(size_t)row * (K / 32) + k0 / 32]);
    b[0] = fp4x8_to_bf16(q.x, s); b[1] = fp4x8_to_bf16(q.y, s);
    b[2] = fp4x8_to_bf16(q.z, s); b[3] = fp4x8_to_bf16(q.w, s);
    bs = 1.0f;
  } else if constexpr (FMT == MOE_W_NVFP4) {
    const uint4 q = *reinterpret_cast<const uint4*>(w + (((size_t)row * K + k0) >> 1));
    const uint32_t s2 = *reinterpret_cast<const uint16_t*>(sc + (size_t)row * (K / 16) + k0 / 16);
    const float s0 = e4m3_to_f32(s2 & 0xffu), s1 = e4m3_to_f32(s2 >> 8);
    b[0] = fp4x8_to_bf16_mul(q.x, s0); b[1] = fp4x8_to_bf16_mul(q.y, s0);
    b[2] = fp4x8_to_bf16_mul(q.z, s1); b[3] = fp4x8_to_bf16_mul(q.w, s1);
    bs = 1.0f;
  } else if constexpr (FMT == MOE_W_FP8_B128) {
    const uint4* p = reinterpret_cast<const uint4*>(w + (size_t)row * K + k0);
    const uint4 q0 = p[0], q1 = p[1];
    b[0] = fp8x8_to_bf16(q0.x, q0.y); b[1] = fp8x8_to_bf16(q0.z, q0.w);
    b[2] = fp8x8_to_bf16(q1.x, q1.y); b[3] = fp8x8_to_bf16(q1.z, q1.w);
    bs = reinterpret_cast<const float*>(sc)[(size_t)(row / 128) * (K / 128) + k0 / 128];
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(w + ((size_t)row * K + k0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 q = p[i];
      b[i] = bits_to_bf16x8(q.x, q.y, q.z, q.w);
    }
    bs = 1.0f;
  }
}

// Tile list: m-tiles of BM rows for every expert with rows, in expert order.
__global__ __launch_bounds__(256) void build_tiles_kernel(const int* __restrict__ counts, int E,
                                                          int BM, int max_tiles,
                                                          int* __restrict__ info) {
  __shared__ int pre[kMaxE];
  __shared__ int wave_tot[4];
  for (int e = threadIdx.x; e < E; e += 256) pre[e] = (counts[e] + BM - 1) / BM;
  __syncthreads();
  const int total = block_exclusive_scan_256(pre, E, wave_tot);
  const int n = total < max_tiles ? total : max_tiles;
  for (int t = threadIdx.x; t < n; t += 256) {
    int lo = 0, hi = E;  // last e with pre[e] <= t
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid] <= t) lo = mid; else hi = mid;
    }
    info[1 + t] = lo;
    info[1 + max_tiles + t] = (t - pre[lo]) * BM;
  }
  if (threadIdx.x == 0) info[0] = n;
}

template <int FMT, bool GATED, int MSUB, int NSUB>
__global__ __launch_bounds__(256) void ffn_tile_kernel(FfnArgs a) {
  constexpr int BM = MSUB * 16;
  constexpr int NH = GATED ? NSUB / 2 : NSUB;  // output column subtiles per wave
  constexpr int NCOL_W = NH * 16;
  constexpr int NCOL = 4 * NCOL_W;
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I;
  const int nnb = N_out / NCOL;
  const int tile = blockIdx.x / nnb, nb = blockIdx.x - tile * nnb;
  if (tile >= a.tile_info[0]) return;
  const int e = a.tile_info[1 + tile];
  const int m0 = a.tile_info[1 + a.max_tiles + tile];
  const int seg0 = a.offsets[e] + m0;
  const int rows = min(BM, a.counts[e] - m0);
  const int slot = a.slot_of ? a.slot_of[e] : e;
  const uint8_t* rec = a.base + (size_t)slot * a.stride;
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * A_PITCH];
  __shared__ int src_row[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  for (int r = tid; r < BM; r += 256) {
    int v = -1;
    if (r < rows) v = GATED ? a.sorted_idx[seg0 + r] / a.k : seg0 + r;
    src_row[r] = v;
  }
  const int ncol0 = nb * NCOL + wave * NCOL_W;
  int brow[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    if constexpr (GATED)
      brow[j] = (j < NH) ? ncol0 + j * 16 + l16 : a.I + ncol0 + (j - NH) * 16 + l16;
    else
      brow[j] = ncol0 + j * 16 + l16;
  }
  f32x4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const uint16_t* Asrc = GATED ? a.x : a.hbuf;
  for (int kc = 0; kc < K; kc += KC) {
    for (int q = tid; q < BM * 16; q += 256) {
      const int r = q >> 4, c = (q & 15) * 8;
      uint4 v = {0u, 0u, 0u, 0u};
      const int sr = src_row[r];
      if (sr >= 0) v = *reinterpret_cast<const uint4*>(Asrc + (size_t)sr * K + kc + c);
      *reinterpret_cast<uint4*>(&As[r * A_PITCH + c]) = v;
    }
    bf16x8 b[NSUB][4];
    float bs[NSUB];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) load_b<FMT>(w, sc, brow[j], K, kc + g * 32, b[j], bs[j]);
    __syncthreads();
    if constexpr (FMT == MOE_W_FP8_B128) {
#pragma unroll
      for (int i = 0; i < MSUB; ++i) {
        f32x4 t[NSUB];
#pragma unroll
        for (int j = 0; j < NSUB; ++j) t[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(&As[(i * 16 + l16) * A_PITCH + g * 32 + s * 8]);
#pragma unroll
          for (int j = 0; j < NSUB; ++j) t[j] = mfma16(av, b[j][s], t[j]);
        }
#pragma unroll
        for (int j = 0; j < NSUB; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(bs[j], t[j][r], acc[i][j][r]);
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
          const bf16x8 av =
              *reinterpret_cast<const bf16x8*>(&As[(i * 16 + l16) * A_PITCH + g * 32 + s * 8]);
#pragma unroll
          for (int j = 0; j < NSUB; ++j) acc[i][j] = mfma16(av, b[j][s], acc[i][j]);
        }
      }
    }
    __syncthreads();
  }

  // epilogue: lane holds column l16 of each subtile, rows 4g..4g+3 of each m-subtile
  if constexpr (GATED) {
    float tsg = 1.0f, tsu = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4) {
      const float* ts = reinterpret_cast<const float*>(rec + a.off_ts);
      tsg = ts[0];
      tsu = ts[1];
    }
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NH; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + g * 4 + r;
          if (m < rows) {
            const float gv = acc[i][j][r] * tsg, uv = acc[i][j + NH][r] * tsu;
            const float hv = gv / (1.0f + expf(-gv)) * uv;
            a.hbuf[(size_t)(seg0 + m) * a.I + ncol0 + j * 16 + l16] = f32_to_bf16_rne(hv);
          }
        }
  } else {
    float tsd = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4) tsd = reinterpret_cast<const float*>(rec + a.off_ts)[2];
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + g * 4 + r;
          if (m < rows)
            a.y_perm[(size_t)(seg0 + m) * a.H + ncol0 + j * 16 + l16] =
                f32_to_bf16_rne(acc[i][j][r] * tsd);
        }
  }
}

// Decode one expert record to fp32 with the same decoders as the GEMM.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ rec, FfnArgs a,
                                                      float* __restrict__ w13,
                                                      float* __restrict__ w2) {
  // one thread = 32 consecutive K values of one row; rows of w13 then w2
  const int rows13 = 2 * a.I, K13 = a.H, K2 = a.I;
  const long n13 = (long)rows13 * (K13 / 32), n2 = (long)a.H * (K2 / 32);
  for (long u = blockIdx.x * 256L + threadIdx.x; u < n13 + n2; u += (long)gridDim.x * 256) {
    const bool first = u < n13;
    const long v = first ? u : u - n13;
    const int K = first ? K13 : K2;
    const int row = (int)(v / (K / 32)), k0 = (int)(v % (K / 32)) * 32;
    const uint8_t* w = rec + (first ? a.off_w13 : a.off_w2);
    const uint8_t* sc = rec + (first ? a.off_w13s : a.off_w2s);
    bf16x8 b[4];
    float bs;
    load_b<FMT>(w, sc, row, K, k0, b, bs);
    float ts = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4) {
      const float* t = reinterpret_cast<const float*>(rec + a.off_ts);
      ts = first ? (row < a.I ? t[0] : t[1]) : t[2];
    }
    float* out = (first ? w13 : w2) + (size_t)row * K + k0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i) out[s * 8 + i] = (float)b[s][i] * bs * ts;
  }
}

static int64_t max_tiles_for(int64_t A, int E, int BM) {
  const int64_t touched = A < E ? A : E;
  return (A + touched * (BM - 1)) / BM;
}

static int check_experts(const moe_experts* W, Layout* L, const char* who) {
  if (!W) return set_error(MOE_ERR_INVALID_ARG, "%s: W is NULL", who);
  if (W->E < 1 || W->E > kMaxE) return set_error(MOE_ERR_INVALID_ARG, "%s: E=%d", who, W->E);
  if (!layout_of(W->fmt, W->H, W->I, L))
    return set_error(MOE_ERR_UNSUPPORTED, "%s: fmt=%d H=%d I=%d unsupported", who, W->fmt, W->H,
                     W->I);
  if (!W->base || !aligned16(W->base)) return set_error(MOE_ERR_INVALID_ARG, "%s: base", who);
  if (W->stride < L->stride || W->stride % 256)
    return set_error(MOE_ERR_INVALID_ARG, "%s: stride %lld (need >= %lld, multiple of 256)", who,
                     (long long)W->stride, (long long)L->stride);
  return MOE_OK;
}

static void fill_args(FfnArgs& a, const moe_experts* W, const Layout& L) {
  a.E = W->E; a.H = W->H; a.I = W->I;
  a.base = static_cast<const uint8_t*>(W->base);
  a.stride = W->stride;
  a.off_w13 = L.w13; a.off_w13s = L.w13s < 0 ? 0 : L.w13s;
  a.off_w2 = L.w2; a.off_w2s = L.w2s < 0 ? 0 : L.w2s;
  a.off_ts = L.ts < 0 ? 0 : L.ts;
}

constexpr int kBMSmall = 16, kBMLarge = 64;

template <int FMT, int MSUB>
static void launch_ffn(const FfnArgs& a, hipStream_t s) {
  constexpr int BM = MSUB * 16;
  const int n_gu = (a.I / 128) * a.max_tiles;  // gate/up: 4 waves x 2 h-subtiles = 128 columns
  const int n_dn = (a.H / 128) * a.max_tiles;  // down: 4 waves x 2 subtiles = 128 columns
  build_tiles_kernel<<<1, 256, 0, s>>>(a.counts, a.E, BM, a.max_tiles, const_cast<int*>(a.tile_info));
  ffn_tile_kernel<FMT, true, MSUB, 4><<<n_gu, 256, 0, s>>>(a);
  ffn_tile_kernel<FMT, false, MSUB, 2><<<n_dn, 256, 0, s>>>(a);
}

template <int MSUB>
static void launch_fmt(int fmt, const FfnArgs& a, hipStream_t s) {
  switch (fmt) {
    case MOE_W_BF16: launch_ffn<MOE_W_BF16, MSUB>(a, s); break;
    case MOE_W_MXFP4: launch_ffn<MOE_W_MXFP4, MSUB>(a, s); break;
    case MOE_W_NVFP4: launch_ffn<MOE_W_NVFP4, MSUB>(a, s); break;
    default: launch_ffn<MOE_W_FP8_B128, MSUB>(a, s); break;
  }
}

}  // namespace moe

using namespace moe;

static size_t ws_h_bytes(int64_t A, int I) { return (size_t)((A * I * 2 + 255) / 256 * 256); }

extern "C" size_t moe_expert_ffn_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W || T < 0 || k < 1 || W->E < 1) return 0;
  const int64_t A = (int64_t)T * k;
  const int64_t mt = max_tiles_for(A, W->E, kBMSmall);
  return ws_h_bytes(A, W->I) + (size_t)((4 * (1 + 2 * mt) + 255) / 256 * 256);
}

extern "C" int moe_expert_ffn(const moe_experts* W, const int32_t* slot_of_expert,
                              const uint16_t* x, int32_t T, int32_t k, const int32_t* counts,
                              const int32_t* offsets, const int32_t* sorted_idx, uint16_t* y_perm,
                              int32_t variant, void* ws, size_t ws_bytes, moe_stream_t stream) {
  Layout L;
  int st = check_experts(W, &L, "moe_expert_ffn");
  if (st) return st;
  if (T < 0 || k < 1 || k > W->E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: need T>=0, 1<=k<=min(E,%d)", kMaxK);
  if (variant < 0 || variant > 2)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: variant %d", variant);
  const int64_t A = (int64_t)T * k;
  if (A > (1 << 28)) return set_error(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: T*k too large");
  if (T == 0) return MOE_OK;
  if (!x || !counts || !offsets || !sorted_idx || !y_perm || !ws)
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: null pointer");
  if (!aligned16(x) || !aligned16(counts) || !aligned16(offsets) || !aligned16(sorted_idx) ||
      !aligned16(y_perm) || !aligned16(ws) || (slot_of_expert && !aligned16(slot_of_expert)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_expert_ffn: pointers must be 16-byte aligned");
  const size_t need = moe_expert_ffn_workspace(W, T, k);
  if (ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace %zu < %zu bytes", ws_bytes, need);

  const bool small = variant == 1 || (variant == 0 && A <= 2 * (int64_t)W->E);
  const int BM = small ? kBMSmall : kBMLarge;
  FfnArgs a;
  fill_args(a, W, L);
  a.k = k;
  a.A = (int)A;
  a.slot_of = slot_of_expert;
  a.x = x;
  a.counts = counts;
  a.offsets = offsets;
  a.sorted_idx = sorted_idx;
  a.hbuf = static_cast<uint16_t*>(ws);
  a.y_perm = y_perm;
  a.tile_info = reinterpret_cast<const int*>(static_cast<uint8_t*>(ws) + ws_h_bytes(A, W->I));
  a.max_tiles = (int)max_tiles_for(A, W->E, BM);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (small) launch_fmt<1>(W->fmt, a, s);
  else launch_fmt<4>(W->fmt, a, s);
  return check_launch("moe_expert_ffn");
}

extern "C" int moe_dequant_expert(const moe_experts* W, int32_t expert, float* w13, float* w2,
                                  moe_stream_t stream) {
  Layout L;
  int st = check_experts(W, &L, "moe_dequant_expert");
  if (st) return st;
  if (expert < 0 || expert >= W->E)
    return set_error(MOE_ERR_INVALID_ARG, "moe_dequant_expert: expert %d", expert);
  if (!w13 || !w2 || !aligned16(w13) || !aligned16(w2))
    return set_error(MOE_ERR_INVALID_ARG, "moe_dequant_expert: outputs");
  FfnArgs a;
  fill_args(a, W, L);
  const uint8_t* rec = a.base + (size_t)expert * W->stride;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (W->fmt) {
    case MOE_W_BF16: dequant_kernel<MOE_W_BF16><<<256, 256, 0, s>>>(rec, a, w13, w2); break;
    case MOE_W_MXFP4: dequant_kernel<MOE_W_MXFP4><<<256, 256, 0, s>>>(rec, a, w13, w2); break;
    case MOE_W_NVFP4: dequant_kernel<MOE_W_NVFP4><<<256, 256, 0, s>>>(rec, a, w13, w2); break;
    default: dequant_kernel<MOE_W_FP8_B128><<<256, 256, 0, s>>>(rec, a, w13, w2); break;
  }
  return check_launch("moe_dequant_expert");
}
