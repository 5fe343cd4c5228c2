// The always-on shared expert: a dense SwiGLU FFN over every token, with no
// routing or permutation — two dense bf16 products on the 32x32x16 bf16 MFMA
// with fp32 accumulation:
//   gate/up:  h[T][I] = bf16( SiLU(x W_gate^T) * (x W_up^T) )   (fused epilogue)
//   down:     y[T][H] = bf16( h W2^T )
// x [T][H], W13 [2I][H] (gate rows, then up rows), W2 [H][I]: every operand is
// K-major, so both GEMMs are C[M][N] = A[M][K] . B[N][K]^T.
//
// Tiling (gfx950, 160 KB LDS per CU): 256 output rows x 256 weight rows per
// workgroup of kSgWaves waves, 2 along the rows x kSgWaves/2 along the weight
// rows (default 8 waves, two per SIMD: each wave 128 x 64 outputs as 4 x 2
// blocks of 32 x 32, accumulators in AGPRs).  Operands are copied from global
// memory straight into LDS (global_load_lds_dwordx4) in K steps of kSgBK
// (kSgStages stages, default two of 64: the next kSgStages-1 chunks are in
// flight while one is computed), one barrier per chunk.  Gate/up tiles take
// 128 h columns: each wave column group's weight rows are 16*kSgNJ gate rows
// followed by the matching 16*kSgNJ up rows, so SiLU(gate) * up is formed in
// registers.  Workgroups are mapped to
// rectangles of tiles per XCD (consecutive workgroups of one XCD share their
// A rows or weight rows in its L2).
//   32x32x16 operands: lane l holds row (A) / column (B) l % 32 and the 8
//   consecutive K at 8 * (l / 32) of the step's 16; result value v of lane l
//   is D[8 * (v / 4) + 4 * (l / 32) + v % 4][l % 32].  The weights are the
//   first operand (D = W X^T): a lane's values are output columns of one
//   token row, four consecutive per group (one 8-byte store).
#include "lds_copy.h"
#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSgBM = 256;     // output rows per workgroup
constexpr int kSgBN = 256;     // weight rows per workgroup
#ifndef MOE_SG_BK
#define MOE_SG_BK 64
#endif
#ifndef MOE_SG_STAGES
#define MOE_SG_STAGES 2
#endif
constexpr int kSgBK = MOE_SG_BK;          // K per stage (32: 64-byte rows, 64: 128-byte rows)
constexpr int kSgStages = MOE_SG_STAGES;  // kSgStages * (kSgBM + kSgBN) * kSgBK * 2 <= 160 KB
constexpr int kSgRowB = kSgBK * 2;        // bytes of one row of a stage
constexpr int kSgUnits = kSgRowB / 16;    // 16-byte units per row
#ifndef MOE_SG_WAVES
#define MOE_SG_WAVES 8
#endif
#ifndef MOE_SG_SCHED
#define MOE_SG_SCHED 1
#endif
constexpr int kSgWaves = MOE_SG_WAVES;     // 4: one wave per SIMD; 8: two
constexpr int kSgWN = kSgWaves / 2;        // waves along the weight rows (2 along M)
constexpr int kSgNJ = kSgBN / kSgWN / 32;  // 32-column blocks per wave (4 or 2)
constexpr int kSgCopies = kSgBM * kSgRowB / 1024 / kSgWaves;  // 1 KB copies of A (and of B) per wave
static_assert(kSgStages * (kSgBM + kSgBN) * kSgRowB <= 160 * 1024, "LDS");
static_assert(kSgStages >= 2 && kSgStages <= 5, "waits are written for 2..5 stages");

// unit swizzle of a stage row (64-byte rows: b_swz, 128-byte rows: a_swz)
__device__ __forceinline__ int sg_swz(int r) { return kSgUnits == 4 ? b_swz(r) : a_swz(r); }

struct SgStage {
  uint8_t a[kSgBM * kSgRowB];  // [row][kSgRowB], 16-byte unit u stored at u ^ sg_swz(row)
  uint8_t b[kSgBN * kSgRowB];
};

struct SgArgs {
  const uint8_t* a;  // bf16 [M][K]
  const uint8_t* w;  // bf16 [N][K]
  uint16_t* out;     // bf16: gated h [M][I], else y [M][N]
  int M, K, N, I;    // N: weight rows (gated: 2I)
  int tm, tn;        // tiles along M and along the output columns
  int rm, rn, nrn;   // tile rectangle worked on by one XCD at a time; rectangles along N
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <bool GATED>
__global__ __launch_bounds__(64 * kSgWaves) void shared_gemm_kernel(SgArgs p) {
  __shared__ SgStage st[kSgStages];
  // block -> (XCD-contiguous index) -> rectangle -> tile
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int v = (b & 7) * (G >> 3) + (b >> 3);  // G is a multiple of 8
  const int per = p.rm * p.rn;
  const int rect = v / per, pos = v - rect * per;
  const int rect_m = rect / p.nrn, rect_n = rect - rect_m * p.nrn;
  const int tmi = rect_m * p.rm + pos / p.rn, tni = rect_n * p.rn + pos % p.rn;
  if (tmi >= p.tm || tni >= p.tn) return;

  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave / kSgWN, nh = wave % kSgWN;
  const int K = p.K, nch = K / kSgBK;
  const int m0 = tmi * kSgBM;

  // this wave's copies: 1 KB each, local rows (1024 / kSgRowB) n + lane / kSgUnits
  // (n = wave*kSgCopies + q), unit lane % kSgUnits
  const uint8_t* abase = p.a + (size_t)m0 * K * 2;
  const uint8_t* wbase = GATED ? p.w : p.w + (size_t)tni * kSgBN * K * 2;
  const int last_row = p.M - 1 - m0;  // rows past M read the last row (outputs discarded)
  uint32_t ao[kSgCopies], wo[kSgCopies];
#pragma unroll
  for (int q = 0; q < kSgCopies; ++q) {
    const int lr = (wave * kSgCopies + q) * (1024 / kSgRowB) + lane / kSgUnits;
    const int ar = lr < last_row ? lr : last_row;
    const uint32_t unit = (uint32_t)(((lane % kSgUnits) ^ sg_swz(lr)) * 16);
    ao[q] = (uint32_t)ar * (uint32_t)(K * 2) + unit;
    int wr;
    if constexpr (GATED) {
      // per wave column group: 16*NJ gate rows, then the matching 16*NJ up rows
      const int grp = lr / (32 * kSgNJ), j = (lr >> 5) % kSgNJ, l = lr & 31;
      const int col = tni * 128 + grp * (16 * kSgNJ) + (j % (kSgNJ / 2)) * 32 + l;
      wr = j < kSgNJ / 2 ? col : p.I + col;
    } else {
      const int rows_left = p.N - 1 - tni * kSgBN;
      wr = lr < rows_left ? lr : rows_left;
    }
    wo[q] = (uint32_t)wr * (uint32_t)(K * 2) + unit;
  }
  auto issue = [&](int c, SgStage& S) {
    const uint32_t kb = (uint32_t)(c * kSgRowB);
#pragma unroll
    for (int q = 0; q < kSgCopies; ++q) {
      const int n = wave * kSgCopies + q;
      dma16(abase, ao[q] + kb, S.a + n * 1024);
      dma16(wbase, wo[q] + kb, S.b + n * 1024);
    }
  };

  f32x16 acc[4][kSgNJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kSgNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragments of K step s (16 K: unit 2s + hh of each row)
  auto load_frags = [&](const SgStage& S, int s, bf16x8 (&af)[4], bf16x8 (&bfr)[kSgNJ]) {
    const int u = 2 * s + hh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mh * 128 + i * 32 + l32;
      af[i] = *reinterpret_cast<const bf16x8*>(S.a + r * kSgRowB + ((u ^ sg_swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < kSgNJ; ++j) {
      const int r = nh * (32 * kSgNJ) + j * 32 + l32;
      bfr[j] = *reinterpret_cast<const bf16x8*>(S.b + r * kSgRowB + ((u ^ sg_swz(r)) * 16));
    }
  };
  // Per K step: the next step's fragments are read while this step's MFMAs
  // issue (one LDS read between consecutive MFMAs), so the LDS latency hides
  // behind MFMA work instead of stalling before each group.
  auto compute = [&](const SgStage& S) {
    constexpr int NSTEP = kSgBK / 16;
    bf16x8 af[2][4], bfr[2][kSgNJ];
    load_frags(S, 0, af[0], bfr[0]);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (s + 1 < NSTEP) load_frags(S, s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
#if MOE_SG_SCHED
      __builtin_amdgcn_sched_barrier(0);  // the reads stay ahead of this step's MFMAs
#endif
      // weights as the MFMA's first operand: the result's rows are output columns,
      // so each lane ends with 4 consecutive columns of one row per value group
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < kSgNJ; ++j) acc[i][j] = mfma32(bfr[s & 1][j], af[s & 1][i], acc[i][j]);
#if MOE_SG_SCHED
      __builtin_amdgcn_sched_barrier(0);
#endif
    }
  };


  // prologue: chunks 0..2 in flight
#pragma unroll
  for (int c = 0; c < kSgStages - 1; ++c)
    if (c < nch) issue(c, st[c]);
  for (int c = 0; c < nch; ++c) {
    // chunk c's copies done (the later in-flight chunks may still be pending),
    // every wave's reads of chunk c-1 done
    // chunks issued after chunk c that may still be in flight: min(stages - 2, nch - 1 - c)
    const int ahead = nch - 1 - c < kSgStages - 2 ? nch - 1 - c : kSgStages - 2;
    if (ahead >= 3) MOE_DMA_SYNC(6 * kSgCopies);
    else if (ahead == 2) MOE_DMA_SYNC(4 * kSgCopies);
    else if (ahead == 1) MOE_DMA_SYNC(2 * kSgCopies);
    else MOE_DMA_SYNC(0);
    if (c + kSgStages - 1 < nch) issue(c + kSgStages - 1, st[(c + kSgStages - 1) % kSgStages]);
    compute(st[c % kSgStages]);
  }

  // lane: row m0 + mh*128 + 32i + l32; value v of block j: column 32j + 8(v/4) + 4hh + v%4
  // of the wave's 128 weight rows, so values 4q..4q+3 are 4 consecutive columns
  const int row_l = m0 + mh * 128 + l32;
  if constexpr (GATED) {
    const int col0 = tni * 128 + nh * (16 * kSgNJ) + 4 * hh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row_l + i * 32;
      if (row >= p.M) continue;
      uint16_t* dst = p.out + (size_t)row * p.I + col0;
#pragma unroll
      for (int jj = 0; jj < kSgNJ / 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint16_t hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[i][jj][4 * q + r], uv = acc[i][jj + kSgNJ / 2][4 * q + r];
            hv[r] = f32_to_bf16_rne(g / (1.0f + expf(-g)) * uv);
          }
          *reinterpret_cast<uint2*>(dst + jj * 32 + 8 * q) =
              uint2{(uint32_t)hv[0] | ((uint32_t)hv[1] << 16), (uint32_t)hv[2] | ((uint32_t)hv[3] << 16)};
        }
    }
  } else {
    const int col0 = tni * kSgBN + nh * (32 * kSgNJ) + 4 * hh;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row_l + i * 32;
      if (row >= p.M) continue;
      uint16_t* dst = p.out + (size_t)row * p.N + col0;
#pragma unroll
      for (int j = 0; j < kSgNJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = col0 + j * 32 + 8 * q;  // the 4 columns lie on one side of N (N % 128 == 0)
          if (col >= p.N) continue;
          const uint32_t b0 = f32_to_bf16_rne(acc[i][j][4 * q]);
          const uint32_t b1 = f32_to_bf16_rne(acc[i][j][4 * q + 1]);
          const uint32_t b2 = f32_to_bf16_rne(acc[i][j][4 * q + 2]);
          const uint32_t b3 = f32_to_bf16_rne(acc[i][j][4 * q + 3]);
          *reinterpret_cast<uint2*>(dst + j * 32 + 8 * q) = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
        }
    }
  }
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// Launch one dense product: tiles (tm x tn) walked as rectangles of up to 32
// tiles per XCD round (rn tiles along N).
template <bool GATED>
int launch_gemm(SgArgs p, hipStream_t s, const char* what) {
  p.tm = (p.M + kSgBM - 1) / kSgBM;
  p.tn = GATED ? p.I / 128 : (p.N + kSgBN - 1) / kSgBN;
  p.rn = p.tn >= 8 ? 8 : p.tn >= 4 ? 4 : p.tn >= 2 ? 2 : 1;
  while (p.rn > 1 && p.tn % p.rn && p.tn % (p.rn / 2) == 0) p.rn /= 2;
  p.rm = 32 / p.rn;
  p.nrn = (p.tn + p.rn - 1) / p.rn;
  const int nrm = (p.tm + p.rm - 1) / p.rm;
  const int64_t blocks = (int64_t)nrm * p.nrn * p.rm * p.rn;
  const int64_t grid = (blocks + 7) / 8 * 8;
  if (grid > (int64_t)1 << 30) return set_error(MOE_ERR_UNSUPPORTED, "%s: too many tiles", what);
  shared_gemm_kernel<GATED><<<(unsigned)grid, 64 * kSgWaves, 0, s>>>(p);
  return check_launch(what);
}

}  // namespace
}  // namespace moe

using namespace moe;

// Workspace: h bf16 [T][I].
extern "C" size_t moe_shared_ffn_workspace(const moe_experts* W, int32_t T) {
  if (!W || T < 0) return 0;
  return align256((size_t)T * W->I * 2);
}

extern "C" int moe_shared_ffn(const moe_experts* W, const uint16_t* x, int32_t T, uint16_t* y,
                              void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (!W) return set_error(MOE_ERR_INVALID_ARG, "moe_shared_ffn: W is NULL");
  Layout Lo;
  if (W->fmt != MOE_W_BF16 || W->E < 1 || !layout_of(W->fmt, W->H, W->I, &Lo))
    return set_error(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: needs BF16 weights (fmt=%d H=%d I=%d)",
                     W->fmt, W->H, W->I);
  if (T < 0) return set_error(MOE_ERR_INVALID_ARG, "moe_shared_ffn: T < 0");
  if (T == 0) return MOE_OK;
  if (!W->base || !aligned16(W->base) || !x || !aligned16(x) || !y || !aligned16(y) || !ws ||
      !aligned16(ws))
    return set_error(MOE_ERR_INVALID_ARG, "moe_shared_ffn: null or misaligned pointer");
  if (ws_bytes < moe_shared_ffn_workspace(W, T))
    return set_error(MOE_ERR_WORKSPACE, "moe_shared_ffn: workspace %zu too small", ws_bytes);
  const int H = W->H, I = W->I;
  // offsets inside one 256-row tile and inside a weight matrix are 32-bit
  if ((int64_t)2 * I * H * 2 >= ((int64_t)1 << 32))
    return set_error(MOE_ERR_UNSUPPORTED, "moe_shared_ffn: weights of %d x %d too large", H, I);
  const uint8_t* rec = static_cast<const uint8_t*>(W->base);  // expert 0
  uint16_t* hb = static_cast<uint16_t*>(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  SgArgs g{};
  g.a = reinterpret_cast<const uint8_t*>(x);
  g.w = rec + Lo.w13;
  g.out = hb;
  g.M = T; g.K = H; g.N = 2 * I; g.I = I;
  int st = launch_gemm<true>(g, s, "moe_shared_ffn gate/up");
  if (st) return st;
  SgArgs d{};
  d.a = reinterpret_cast<const uint8_t*>(hb);
  d.w = rec + Lo.w2;
  d.out = y;
  d.M = T; d.K = I; d.N = H; d.I = I;
  return launch_gemm<false>(d, s, "moe_shared_ffn down");
}
