// Per-expert SwiGLU FFN over the permuted rows (grouped GEMMs on MFMA): one
// launch for gate/up with the SiLU*mul epilogue, one for down (plus, on the
// block-scaled prefill path, one pass that splits x).
//
// Work unit = (m-tile of one expert's rows, block of output columns).  Each
// workgroup finds its (expert, first row) from `counts` itself (a wave-wide
// prefix sum of per-expert tile counts), so no extra launch or host sync is
// needed and the whole call can be captured into a graph.
//
// Operands.  A = activations: bf16 rows gathered by token (gate/up) or the
// contiguous h rows (down); on the block-scaled paths (MXFP4, FP8) each row
// is split once into E4M3 hi + lo with one E8M0 scale per 32.  B = expert
// weights in their stored format: fed to the block-scaled MFMA as stored
// (E2M1 with its E8M0 scales, E4M3 with a unit scale), or decoded in
// registers to bf16 for the bf16 MFMA (every MXFP4 value, NVFP4 E2M1 x E4M3
// product and E4M3 value is exact in bf16); FP8 block scales and NVFP4
// tensor scales multiply fp32 partial sums.
//
// K mapping of the 16x16x32 bf16 kernels.  For a 128-wide K chunk, lane
// group g = lane/16 owns the 32 consecutive K values [32g, 32g+32) of its
// row; MFMA step s consumes values [32g+8s, 32g+8s+8).  A and B use the same
// mapping, so each output is the full dot product whatever the instruction's
// internal K order.
//
// Kernel families:
//  * decode (few rows per expert): m-tile = 16 rows; the 4 waves of a
//    workgroup split K (chunks w, w+4, ...), each wave issues the loads of
//    up to 4 chunks before consuming any (16 KB in flight per wave), and the
//    4 partial sums are added in wave order through LDS (deterministic).
//    Bandwidth-bound: each touched expert's weights are read once.
//  * prefill, register-staged (BF16, FP8, and the MXFP4 / NVFP4 shapes the
//    copy kernels do not take): m-tile = 64 rows, the A chunk staged in LDS,
//    the weight chunk raw in registers one chunk ahead.
//  * prefill, copy pipeline (MXFP4: 128-row tiles on 8 waves; NVFP4: 64-row
//    tiles on 4 waves): every operand byte copied from global memory into
//    LDS by global_load_lds, two K chunks deep, so no registers hold loads in
//    flight.
#include "ffn_common.h"
#include "lds_copy.h"

namespace moe {

// ---------------------------------------------------------------------------
// tile lookup: the `tile`-th m-tile of BM rows, experts in ascending order
// ---------------------------------------------------------------------------
struct TileInfo {
  int e, m0, rows, seg0;
};

// Called by one whole wave; returns false (in every lane) if `tile` is past
// the last tile.  E <= 1024: lane l owns experts [l*EPL, l*EPL + EPL).  The
// counts and offsets of a lane's experts are loaded together (one round trip).
template <int BM>
__device__ __forceinline__ bool find_tile(const int* __restrict__ counts,
                                          const int* __restrict__ offsets, int E, int tile,
                                          int lane, TileInfo& ti) {
  const int epl = (E + 63) >> 6;
  const int e0 = lane * epl;
  int c[16], o[16];
  int tl = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool ok = i < epl && e0 + i < E;
    c[i] = ok ? counts[e0 + i] : 0;
    o[i] = ok ? offsets[e0 + i] : 0;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) tl += (c[i] + BM - 1) / BM;
  const int incl = wave_incl_scan(tl);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (tile >= total) return false;
  const int excl = incl - tl;
  const uint64_t own = __ballot(excl <= tile && tile < incl);
  const int ol = (int)__builtin_ctzll(own);
  int e = 0, m0 = 0, cnt = 0, off = 0;
  if (lane == ol) {
    int t = tile - excl;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int n = (c[i] + BM - 1) / BM;
      if (cnt == 0 && t < n) {
        e = e0 + i;
        m0 = t * BM;
        cnt = c[i];
        off = o[i];
      }
      t -= n;
    }
  }
  ti.e = __builtin_amdgcn_readlane(e, ol);
  ti.m0 = __builtin_amdgcn_readlane(m0, ol);
  ti.rows = min(BM, __builtin_amdgcn_readlane(cnt, ol) - ti.m0);
  ti.seg0 = __builtin_amdgcn_readlane(off, ol) + ti.m0;
  return true;
}

// ---------------------------------------------------------------------------
// decode family (few rows per expert, bandwidth-bound)
//   SPLIT = 4: the 4 waves of a workgroup share NSUB weight subtiles and split
//              K (chunks w, w+4, ...); partial sums meet in LDS in wave order.
//   SPLIT = 1: each wave owns NSUB subtiles over the whole K (no LDS).
// Every wave looks its tile up itself and issues the weight loads of U chunks
// before it needs the activation rows, so HBM requests start right away.
// ---------------------------------------------------------------------------
template <int FMT, bool GATED, int NSUB, int SPLIT, int U>
__device__ __forceinline__ void ffn_decode_body(const FfnArgs& a) {
  static_assert(!GATED || NSUB % 2 == 0, "gate/up subtiles come in pairs");
  constexpr int WAVE_COLS = (GATED ? NSUB / 2 : NSUB) * 16;     // output columns per wave
  constexpr int NCOL = SPLIT == 4 ? WAVE_COLS : 4 * WAVE_COLS;  // per workgroup
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I;
  const int nnb = N_out / NCOL;
  const int tile = blockIdx.x / nnb, nb = blockIdx.x - tile * nnb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;

  TileInfo ti;
  if (!find_tile<16>(a.counts, a.offsets, a.E, tile, lane, ti)) return;  // uniform per block
  dbg_segment(ti.seg0, ti.rows, a.A);
  const uint8_t* rec = record_of(a, ti.e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);

  const int n0 = nb * NCOL + (SPLIT == 4 ? 0 : wave * WAVE_COLS);
  int brow[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    if constexpr (GATED)
      brow[j] = (j < NSUB / 2 ? n0 : a.I + n0) + (j % (NSUB / 2)) * 16 + l16;
    else
      brow[j] = n0 + j * 16 + l16;
  }
  const int nchunks = K / KC;
  const int c_first = SPLIT == 4 ? wave : 0;
  constexpr int CSTEP = SPLIT;  // chunk stride of one wave

  f32x4 acc[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the row index is requested first: waits on it then leave the weight loads in flight
  int tok = -1;
  if (l16 < ti.rows) tok = GATED ? dbg_clamp(a.sorted_idx[ti.seg0 + l16], a.A, kDbgSorted) : ti.seg0 + l16;
  const uint16_t* arow = nullptr;
  bool have_row = false;
  for (int c0 = c_first; c0 < nchunks; c0 += CSTEP * U) {
    BRaw<FMT> raw[U][NSUB];
    uint4 araw[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + CSTEP * u;
      if (c < nchunks) {
#pragma unroll
        for (int j = 0; j < NSUB; ++j) load_b_raw<FMT>(w, sc, brow[j], K, c * KC + g * 32, raw[u][j]);
      }
    }
    if (!have_row) {  // activation row of this lane, resolved after the weight loads are out
      have_row = true;
      if (tok >= 0)
        arow = GATED ? a.x + (size_t)(tok / a.k) * a.H : a.hbuf + (size_t)tok * a.I;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + CSTEP * u;
      if (c < nchunks) {
        if (arow) {
          const uint4* ap = reinterpret_cast<const uint4*>(arow + c * KC + g * 32);
#pragma unroll
          for (int s = 0; s < 4; ++s) araw[u][s] = ap[s];
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) araw[u][s] = uint4{0u, 0u, 0u, 0u};
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c0 + CSTEP * u < nchunks) {
        bf16x8 av[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
          av[s] = bits_to_bf16x8(araw[u][s].x, araw[u][s].y, araw[u][s].z, araw[u][s].w);
#pragma unroll
        for (int j = 0; j < NSUB; ++j) {
          bf16x8 b[4];
          decode_b<FMT>(raw[u][j], b);
          if constexpr (FMT == MOE_W_FP8_B128) {
            f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) t = mfma16(av[s], b[s], t);
            const float bs = block_scale<FMT>(raw[u][j]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(bs, t[r], acc[j][r]);
          } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[j] = mfma16(av[s], b[s], acc[j]);
          }
        }
      }
    }
  }

  if constexpr (SPLIT == 4) {
    __shared__ f32x4 red[4][NSUB][64];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) red[wave][j][lane] = acc[j];
    __syncthreads();
    // wave q sums subtile(s) in wave order 0..3 (deterministic)
    constexpr int NOUT = GATED ? NSUB / 2 : NSUB;
    if (wave >= NOUT) return;
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      if (GATED ? (j % (NSUB / 2) == wave) : (j == wave)) {
        f32x4 sum = red[0][j][lane];
#pragma unroll
        for (int q = 1; q < 4; ++q) {
          const f32x4 v = red[q][j][lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[r] += v[r];
        }
        acc[j] = sum;
      }
    }
  }

  // lane holds column l16 of a subtile, rows 4g..4g+3 of the m-tile
  const int subs_here = GATED ? NSUB / 2 : NSUB;
#pragma unroll
  for (int jo = 0; jo < subs_here; ++jo) {
    if (SPLIT == 4 && jo != wave) continue;
    if constexpr (GATED) {
      float tsg = 1.0f, tsu = 1.0f;
      if constexpr (FMT == MOE_W_NVFP4) {
        const float* ts = reinterpret_cast<const float*>(rec + a.off_ts);
        tsg = ts[0];
        tsu = ts[1];
      }
      const f32x4 gs = acc[jo], us = acc[jo + NSUB / 2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = g * 4 + r;
        if (m < ti.rows) {
          const float gv = gs[r] * tsg, uv = us[r] * tsu;
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          a.hbuf[(size_t)(ti.seg0 + m) * a.I + n0 + jo * 16 + l16] = f32_to_bf16_rne(hv);
        }
      }
    } else {
      float tsd = 1.0f;
      if constexpr (FMT == MOE_W_NVFP4) tsd = reinterpret_cast<const float*>(rec + a.off_ts)[2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = g * 4 + r;
        if (m < ti.rows)
          a.y_perm[(size_t)(ti.seg0 + m) * a.H + n0 + jo * 16 + l16] =
              f32_to_bf16_rne(acc[jo][r] * tsd);
      }
    }
  }
}

#ifndef MOE_GU_NSUB
#define MOE_GU_NSUB 4
#define MOE_GU_SPLIT 4
#define MOE_GU_U 2
#endif
#ifndef MOE_DN_NSUB
#define MOE_DN_NSUB 2
#define MOE_DN_SPLIT 1
#define MOE_DN_U 4
#endif
// gate/up: 4 waves split K over NSUB/2 x 16 h-columns per workgroup
constexpr int kGuNsub = MOE_GU_NSUB, kGuSplit = MOE_GU_SPLIT, kGuU = MOE_GU_U;
// down: each wave owns NSUB x 16 output rows over the whole (short) K
constexpr int kDnNsub = MOE_DN_NSUB, kDnSplit = MOE_DN_SPLIT, kDnU = MOE_DN_U;
constexpr int kGuCols = (kGuSplit == 4 ? 1 : 4) * kGuNsub / 2 * 16;
constexpr int kDnCols = (kDnSplit == 4 ? 1 : 4) * kDnNsub * 16;

template <int FMT>
__global__ __launch_bounds__(256) void ffn_gateup_decode_kernel(FfnArgs a) {
  ffn_decode_body<FMT, true, kGuNsub, kGuSplit, kGuU>(a);
}
template <int FMT>
__global__ __launch_bounds__(256) void ffn_down_decode_kernel(FfnArgs a) {
  ffn_decode_body<FMT, false, kDnNsub, kDnSplit, kDnU>(a);
}

// ---------------------------------------------------------------------------
// prefill family: 64-row m-tiles staged in LDS
// ---------------------------------------------------------------------------
template <int FMT, bool GATED, int MSUB, int NSUB>
__device__ __forceinline__ void ffn_tile_body(const FfnArgs& a) {
  constexpr int BM = MSUB * 16;
  constexpr int NH = GATED ? NSUB / 2 : NSUB;  // output column subtiles per wave
  constexpr int NCOL_W = NH * 16;
  constexpr int NCOL = 4 * NCOL_W;
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I;
  const int nnb = N_out / NCOL;
  const int tile = blockIdx.x / nnb, nb = blockIdx.x - tile * nnb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * A_PITCH];
  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (wave == 0) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) {
        dbg_segment(ti.seg0, ti.rows, a.A);
        s_ti = ti;
      }
    }
  }
  __syncthreads();
  if (!s_valid) return;
  const TileInfo ti = s_ti;
  const int seg0 = ti.seg0, rows = ti.rows;
  const uint8_t* rec = record_of(a, ti.e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);

  for (int r = tid; r < BM; r += 256) {
    int v = -1;
    if (r < rows) v = GATED ? dbg_clamp(a.sorted_idx[seg0 + r], a.A, kDbgSorted) / a.k : seg0 + r;
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
    BRaw<FMT> raw[NSUB];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) load_b_raw<FMT>(w, sc, brow[j], K, kc + g * 32, raw[j]);
    __syncthreads();
    bf16x8 b[NSUB][4];
#pragma unroll
    for (int j = 0; j < NSUB; ++j) decode_b<FMT>(raw[j], b[j]);
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
        for (int j = 0; j < NSUB; ++j) {
          const float bs = block_scale<FMT>(raw[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(bs, t[j][r], acc[i][j][r]);
        }
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

constexpr int kPreMSUB = 4;  // 64-row m-tiles
template <int FMT>
__global__ __launch_bounds__(256) void ffn_gateup_tile_kernel(FfnArgs a) {
  ffn_tile_body<FMT, true, kPreMSUB, 4>(a);
}
template <int FMT>
__global__ __launch_bounds__(256) void ffn_down_tile_kernel(FfnArgs a) {
  ffn_tile_body<FMT, false, kPreMSUB, 2>(a);
}

// ----------------------------------------------------------------------------
// Prefill grouped GEMM, pipelined.  A block owns BM = 16*MSUB rows of one
// expert tile and 256 weight rows (4 waves x 4 subtiles of 16; gate/up pairs
// them as 2 gate + 2 up subtiles per wave, so 128 h-columns per block).  K
// goes in chunks of 128: the A chunk is staged in LDS (two buffers), the B
// chunk stays raw in registers (two named buffers used alternately, so no
// register holding a pending load is copied).  While chunk c is computed the
// loads of chunk c+1 are in flight; one barrier per chunk.  K/128 must be
// even (the last prefetch re-reads the last chunk).  Blocks walk super-tiles
// of 8 m-tiles column block by column block, each super-tile on one XCD
// (tile_of_block).
// ----------------------------------------------------------------------------
constexpr int kSuperM = 8;  // m-tiles per super-tile (prefill block order), bf16 kernels

// Block b -> (m-tile, column block) for the prefill grids.  The grid holds
// whole super-tiles (SM m-tiles x nnb column blocks, walked column block by
// column block, so that the blocks an XCD runs at a time share the A rows of
// a few m-tiles and the weights of a few column blocks in its L2), a multiple
// of 8 of them.  Hardware block b runs on XCD b % 8, and super-tile s is
// served by XCD s % 8: the grid is sized from an upper bound on the m-tiles,
// the ones that hold rows come first, and this keeps them spread over all
// eight XCDs (a contiguous range of super-tiles per XCD would leave most
// XCDs with only empty tiles when the bound is loose).
template <int SM>
__device__ __forceinline__ void tile_of_block(int b, int nnb, int& tile, int& nb) {
  const int S = SM * nnb;                  // blocks per super-tile
  const int x = b & 7, j = b >> 3;         // XCD, index among that XCD's blocks
  const int sl = j / S, gi = j - sl * S;   // super-tile of this XCD, block inside it
  tile = (sl * 8 + x) * SM + gi % SM;
  nb = gi / SM;
}
// m-tiles of a grid: the bound rounded up to whole groups of 8 super-tiles
// of SM m-tiles
static int64_t grid_m_tiles(int64_t bound, int SM) { return (bound + 8 * SM - 1) / (8 * SM) * (8 * SM); }

template <int FMT, bool GATED, int MSUB, int MH>
__device__ __forceinline__ void ffn_pipe_body(const FfnArgs& a) {
  // MH row groups of MSUB*16 rows; 4*MH waves: wave = (row group, column quarter)
  constexpr int NT = 256 * MH, WM = MSUB * 16, BM = WM * MH, NSUB = 4, NH = GATED ? 2 : 4;
  constexpr int NCOLB = GATED ? 128 : 256;  // output columns per block
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I, nch = K / KC;
  const int nnb = N_out / NCOLB;
  const int b = (int)blockIdx.x;
  // super-tiles of kSuperM m-tiles, walked column block by column block (as
  // in the block-scaled kernels)
  int tile, nb;
  tile_of_block<kSuperM>(b, nnb, tile, nb);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = (tid >> 6) & 3, mh = tid >> 8;  // column quarter, row group

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_PITCH];
  // NVFP4: the chunk's 8 E4M3 block-scale bytes of each of the block's 256
  // weight rows, staged with the A chunk (one 8-byte load per thread instead
  // of one 2-byte load per lane and subtile)
  constexpr bool SNV = FMT == MOE_W_NVFP4 && MH == 1;
  __shared__ uint2 Bs[2][SNV ? 256 : 1];
  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (tid < 64) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) {
        dbg_segment(ti.seg0, ti.rows, a.A);
        s_ti = ti;
      }
    }
  }
  __syncthreads();
  if (!s_valid) return;
  const TileInfo ti = s_ti;
  const int seg0 = ti.seg0, rows = ti.rows;
  const uint8_t* rec = record_of(a, ti.e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);
  // rows past the tile read its first row: valid memory, outputs discarded
  for (int r = tid; r < BM; r += NT) {
    const int rr = r < rows ? r : 0;
    src_row[r] = GATED ? dbg_clamp(a.sorted_idx[seg0 + rr], a.A, kDbgSorted) / a.k : seg0 + rr;
  }
  const int ncol0 = nb * NCOLB + wave * (NH * 16);
  int brow[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    if constexpr (GATED)
      brow[j] = (j < NH) ? ncol0 + j * 16 + l16 : a.I + ncol0 + (j - NH) * 16 + l16;
    else
      brow[j] = ncol0 + j * 16 + l16;
  }
  // the weight row whose scales thread tid stages: block-local row tid =
  // (wave tid/64, subtile (tid/16)%4, lane row tid%16)
  size_t bso = 0;
  if constexpr (SNV) {
    const int sw = tid >> 6, sj = (tid >> 4) & 3, sl = tid & 15;
    const int c0 = nb * NCOLB + sw * (NH * 16);
    int row;
    if constexpr (GATED)
      row = (sj < NH) ? c0 + sj * 16 + sl : a.I + c0 + (sj - NH) * 16 + sl;
    else
      row = c0 + sj * 16 + sl;
    bso = (size_t)row * (K / 16);
  }
  uint2 bsv = uint2{0u, 0u};
  f32x4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  const uint16_t* Asrc = GATED ? a.x : a.hbuf;
  uint4 av[MSUB];  // this thread's share of one A chunk: BM*16 uint4 over NT threads
  auto a_issue = [&](int c) {
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      const int q = tid + NT * i, r = q >> 4, col = (q & 15) * 8;
      av[i] = *reinterpret_cast<const uint4*>(Asrc + (size_t)src_row[r] * K + c * KC + col);
    }
    if constexpr (SNV) bsv = *reinterpret_cast<const uint2*>(sc + bso + (size_t)c * 8);
  };
  auto a_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      const int q = tid + NT * i, r = q >> 4, col = (q & 15) * 8;
      *reinterpret_cast<uint4*>(&As[buf][r * A_PITCH + col]) = av[i];
    }
    if constexpr (SNV) Bs[buf][tid] = bsv;
  };
  auto b_issue = [&](int c, BRaw<FMT> (&r)[NSUB]) {
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      if constexpr (SNV)  // codes only; the scales come through LDS (Bs)
        r[j].q[0] = *reinterpret_cast<const uint4*>(w + (((size_t)brow[j] * K + c * KC + g * 32) >> 1));
      else
        load_b_raw<FMT>(w, sc, brow[j], K, c * KC + g * 32, r[j]);
    }
  };
  // A fragments of the chunk come to registers once; then each B subtile is
  // decoded right before its MFMAs, so the decode of subtile j+1 can overlap
  // the MFMAs of subtile j.
  auto compute = [&](int buf, const BRaw<FMT> (&r)[NSUB]) {
    const uint16_t* Ab = As[buf] + mh * WM * A_PITCH;  // this wave's row group
    bf16x8 af[MSUB][4];
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        af[i][s] = *reinterpret_cast<const bf16x8*>(&Ab[(i * 16 + l16) * A_PITCH + g * 32 + s * 8]);
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      bf16x8 bv[4];
      if constexpr (SNV) {
        BRaw<FMT> rj = r[j];
        rj.s = reinterpret_cast<const uint16_t*>(&Bs[buf][wave * 64 + j * 16 + l16])[g];
        decode_b<FMT>(rj, bv);
      } else {
        decode_b<FMT>(r[j], bv);
      }
      if constexpr (FMT == MOE_W_FP8_B128) {
        const float bs = block_scale<FMT>(r[j]);
#pragma unroll
        for (int i = 0; i < MSUB; ++i) {
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < 4; ++s) t = mfma16(af[i][s], bv[s], t);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(bs, t[q], acc[i][j][q]);
        }
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < MSUB; ++i) acc[i][j] = mfma16(af[i][s], bv[s], acc[i][j]);
      }
    }
  };

  BRaw<FMT> rx[NSUB], ry[NSUB];
  a_issue(0);
  b_issue(0, rx);
  a_store(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    a_issue(c + 1);
    b_issue(c + 1, ry);
    compute(0, rx);
    a_store(1);
    __syncthreads();
    const int c2 = c + 2 < nch ? c + 2 : nch - 1;
    a_issue(c2);
    b_issue(c2, rx);
    compute(1, ry);
    a_store(0);  // the last iteration stores a re-read chunk nobody uses
    __syncthreads();
  }

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
          const int m = mh * WM + i * 16 + g * 4 + r;
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
          const int m = mh * WM + i * 16 + g * 4 + r;
          if (m < rows)
            a.y_perm[(size_t)(seg0 + m) * a.H + ncol0 + j * 16 + l16] =
                f32_to_bf16_rne(acc[i][j][r] * tsd);
        }
  }
}

template <int FMT, int MSUB, int MH>
__global__ __launch_bounds__(256 * MH) void ffn_gateup_pipe_kernel(FfnArgs a) {
  ffn_pipe_body<FMT, true, MSUB, MH>(a);
}
template <int FMT, int MSUB, int MH>
__global__ __launch_bounds__(256 * MH) void ffn_down_pipe_kernel(FfnArgs a) {
  ffn_pipe_body<FMT, false, MSUB, MH>(a);
}

// ----------------------------------------------------------------------------
// Prefill grouped GEMM on the block-scaled MFMA (MXFP4 and FP8 weights).
// Same tiling and pipeline as ffn_pipe_body (64 rows x 256 weight rows per
// block, K chunks of 128, A double-buffered in LDS, B raw in two register
// buffers; blocks walk super-tiles of 8 m-tiles), but nothing is decoded: the
// A operand arrives split into E4M3 hi + lo with E8M0 scales
// (quant_rows_kernel), and each 16x16x128 product is two
// v_mfma_scale_f32_16x16x128_f8f6f4 (hi, lo) on the raw weight bytes — E2M1
// with their E8M0 bytes, or E4M3 with scale 1 and the fp32 block scale
// applied to the chunk's partial sums.
//   LDS per buffer: hi and lo rows of 128 bytes at a 144-byte pitch (lane
//   (g, i) reads 32 bytes of row i at 32g: 16 rows land on distinct banks),
//   4 A-scale bytes per row, and the chunk's weight scales (MXFP4: 4 E8M0
//   bytes per weight row; FP8: the two fp32 block scales), staged with A.
// ----------------------------------------------------------------------------
constexpr int QP = KC;  // LDS row pitch of the hi / lo bytes (16-byte units XOR-swizzled by a_swz)

// A lane's raw weight bytes of one chunk in the MFMA's B order: E2M1, K
// [32g, 32g+32) (16 bytes); E4M3, K [16g, 16g+16) and [64+16g, 64+16g+16)
// (2 x 16 bytes).  Their scales are staged through LDS.
// m-tiles per super-tile of the register-staged block-scaled kernels (4: FP8
// hit path 0.79 -> 0.74 ms against 8; 2 measured 0.75)
constexpr int kMxSuperM = 4;
template <int FMT>
struct QRaw {
  uint4 q[FMT == MOE_W_FP8_B128 ? 2 : 1];
};

template <int FMT, bool GATED>
__device__ __forceinline__ void ffn_mx_pipe_body(const FfnArgs& a) {
  static_assert(FMT == MOE_W_MXFP4 || FMT == MOE_W_FP8_B128, "block-scaled formats only");
  // 4 waves; each owns 4 subtiles of 16 weight rows over all 64 rows
  constexpr int MSUB = 4, NT = 256, BM = 64, NSUB = 4, NH = GATED ? 2 : 4;
  constexpr int NCOLB = GATED ? 128 : 256;  // output columns per block
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I, nch = K / KC;
  const int nnb = N_out / NCOLB;
  const int b = (int)blockIdx.x;
  // super-tiles of kMxSuperM m-tiles x all column blocks, walked column
  // block by column block: the blocks one XCD runs at a time share both the
  // A rows of a few m-tiles and the weights of a few column blocks in its L2
  int tile, nb;
  tile_of_block<kMxSuperM>(b, nnb, tile, nb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;

  __shared__ __attribute__((aligned(16))) uint8_t Sh[2][BM * QP];
  __shared__ __attribute__((aligned(16))) uint8_t Sl[2][BM * QP];
  __shared__ __attribute__((aligned(16))) uint8_t Ss[2][BM * 4];
  // MXFP4: the chunk's 4 E8M0 bytes of each of the block's 256 weight rows,
  // staged with the A chunk (one dword load per thread instead of one byte
  // load per lane and subtile)
  __shared__ uint32_t Bs[2][FMT == MOE_W_MXFP4 ? 256 : 1];
  // FP8: the chunk's fp32 block scales of the block's two 128-row weight
  // blocks (gate and up rows, or the two halves of 256 down rows)
  __shared__ float Fs[2][2];
  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (tid < 64) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) {
        dbg_segment(ti.seg0, ti.rows, a.A);
        s_ti = ti;
      }
    }
  }
  __syncthreads();
  if (!s_valid) return;
  // the tile is the same for the whole block: keep it in scalar registers
  const int e = __builtin_amdgcn_readfirstlane(s_ti.e);
  const int seg0 = __builtin_amdgcn_readfirstlane(s_ti.seg0);
  const int rows = __builtin_amdgcn_readfirstlane(s_ti.rows);
  const uint8_t* rec = record_of(a, e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);
  // rows past the tile read its first row: valid memory, outputs discarded
  if (tid < BM) {
    const int rr = tid < rows ? tid : 0;
    src_row[tid] = GATED ? dbg_clamp(a.sorted_idx[seg0 + rr], a.A, kDbgSorted) / a.k : seg0 + rr;
  }
  const int ncol0 = nb * NCOLB + wave * (NH * 16);
  // 32-bit byte offsets from the (scalar) weight and scale bases: a weight
  // matrix has fewer than 2^32 bytes
  uint32_t boff[NSUB];
#pragma unroll
  for (int j = 0; j < NSUB; ++j) {
    int row;
    if constexpr (GATED)
      row = (j < NH) ? ncol0 + j * 16 + l16 : a.I + ncol0 + (j - NH) * 16 + l16;
    else
      row = ncol0 + j * 16 + l16;
    // (the scales come through LDS: Bs, Fs)
    boff[j] = FMT == MOE_W_MXFP4 ? (uint32_t)row * (uint32_t)(K / 2) + g * 16
                                 : (uint32_t)row * (uint32_t)K + g * 16;
  }
  // the weight row whose scales thread tid stages: block-local row tid =
  // (wave tid/64, subtile (tid/16)%4, lane row tid%16)
  uint32_t bso = 0;
  if constexpr (FMT == MOE_W_MXFP4) {
    const int sw = tid >> 6, sj = (tid >> 4) & 3, sl = tid & 15;
    const int c0 = nb * NCOLB + sw * (NH * 16);
    int row;
    if constexpr (GATED)
      row = (sj < NH) ? c0 + sj * 16 + sl : a.I + c0 + (sj - NH) * 16 + sl;
    else
      row = c0 + sj * 16 + sl;
    bso = (uint32_t)row * (uint32_t)(K / 32);
  }
  f32x4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();

  // A chunk: BM rows x (128 hi + 128 lo bytes), two 16-byte pieces of each
  // per thread, plus one scale dword per row (threads 0..BM-1).  Named
  // registers (an array here was kept in scratch memory).  32-bit offsets:
  // the split operands have fewer than 2^32 bytes (checked by the caller).
  uint4 h0, h1, l0, l1;
  uint32_t sv = 0, bsv = 0;
  float fsv = 0.0f;
  int fsrow = 0;  // FP8: the 128-row block whose scale thread tid < 2 stages
  if constexpr (FMT == MOE_W_FP8_B128)
    fsrow = GATED ? (tid == 0 ? nb : a.I / 128 + nb) : nb * 2 + (tid & 1);
  const int KS = K / 32;
  const int ar0 = tid >> 3, ar1 = (tid + NT) >> 3, acol = (tid & 7) * 16;
  const uint32_t ao0 = (uint32_t)src_row[ar0] * (uint32_t)K + acol;
  const uint32_t ao1 = (uint32_t)src_row[ar1] * (uint32_t)K + acol;
  const uint32_t aos = (uint32_t)src_row[tid < BM ? tid : 0] * (uint32_t)KS;
  auto a_issue = [&](int c) {
    const uint32_t cc = (uint32_t)(c * KC);
    h0 = *reinterpret_cast<const uint4*>(a.aq_hi + (ao0 + cc));
    l0 = *reinterpret_cast<const uint4*>(a.aq_lo + (ao0 + cc));
    h1 = *reinterpret_cast<const uint4*>(a.aq_hi + (ao1 + cc));
    l1 = *reinterpret_cast<const uint4*>(a.aq_lo + (ao1 + cc));
    if (tid < BM) sv = *reinterpret_cast<const uint32_t*>(a.aq_sc + (aos + (uint32_t)(c * 4)));
    if constexpr (FMT == MOE_W_MXFP4)
      bsv = *reinterpret_cast<const uint32_t*>(sc + (bso + (uint32_t)(c * 4)));
    if constexpr (FMT == MOE_W_FP8_B128)
      if (tid < 2) fsv = reinterpret_cast<const float*>(sc)[(size_t)fsrow * (K / 128) + c];
  };
  auto a_store = [&](int buf) {
    const int p0 = ar0 * QP + ((acol >> 4) ^ a_swz(ar0)) * 16;
    const int p1 = ar1 * QP + ((acol >> 4) ^ a_swz(ar1)) * 16;
    *reinterpret_cast<uint4*>(&Sh[buf][p0]) = h0;
    *reinterpret_cast<uint4*>(&Sl[buf][p0]) = l0;
    *reinterpret_cast<uint4*>(&Sh[buf][p1]) = h1;
    *reinterpret_cast<uint4*>(&Sl[buf][p1]) = l1;
    if (tid < BM) *reinterpret_cast<uint32_t*>(&Ss[buf][tid * 4]) = sv;
    if constexpr (FMT == MOE_W_MXFP4) Bs[buf][tid] = bsv;
    if constexpr (FMT == MOE_W_FP8_B128)
      if (tid < 2) Fs[buf][tid] = fsv;
  };
  auto b_issue = [&](int c, QRaw<FMT> (&r)[NSUB]) {
#pragma unroll
    for (int j = 0; j < NSUB; ++j) {
      if constexpr (FMT == MOE_W_MXFP4) {
        r[j].q[0] = *reinterpret_cast<const uint4*>(w + (boff[j] + (uint32_t)(c * (KC / 2))));
      } else {
        const uint8_t* p = w + (boff[j] + (uint32_t)(c * KC));
        r[j].q[0] = *reinterpret_cast<const uint4*>(p);
        r[j].q[1] = *reinterpret_cast<const uint4*>(p + 64);
      }
    }
  };
  // one m-subtile's A fragments at a time (hi, lo: 16 registers), the next
  // subtile's read from LDS while these are used, against the chunk's 4 raw
  // B subtiles; accumulators pinned after each step
  auto compute = [&](int buf, const QRaw<FMT> (&r)[NSUB]) {
    auto frag = [&](int i, i32x8& h, i32x8& l, int& sa) {
      const int rw = i * 16 + l16, sw = a_swz(rw);
      const int o0 = rw * QP + ((2 * g) ^ sw) * 16, o1 = rw * QP + ((2 * g + 1) ^ sw) * 16;
      const i32x4 h0 = *reinterpret_cast<const i32x4*>(&Sh[buf][o0]);
      const i32x4 h1 = *reinterpret_cast<const i32x4*>(&Sh[buf][o1]);
      const i32x4 l0 = *reinterpret_cast<const i32x4*>(&Sl[buf][o0]);
      const i32x4 l1 = *reinterpret_cast<const i32x4*>(&Sl[buf][o1]);
      h = i32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      l = i32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      sa = Ss[buf][rw * 4 + g];
    };
    i32x8 ah, al;
    int sa;
    frag(0, ah, al, sa);
    float fb0 = 0.0f, fb1 = 0.0f;  // FP8: the chunk's two block scales
    if constexpr (FMT == MOE_W_FP8_B128) {
      fb0 = Fs[buf][0];
      fb1 = Fs[buf][1];
    }
    int sbv[NSUB];  // MXFP4: this lane's scale byte of each subtile
    if constexpr (FMT == MOE_W_MXFP4) {
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
        sbv[j] = reinterpret_cast<const uint8_t*>(Bs[buf])[(wave * 64 + j * 16 + l16) * 4 + g];
    }
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      i32x8 nh, nl;
      int ns = 0;
      if (i + 1 < MSUB) frag(i + 1, nh, nl, ns);
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        if constexpr (FMT == MOE_W_MXFP4) {
          const i32x4 bq = {(int)r[j].q[0].x, (int)r[j].q[0].y, (int)r[j].q[0].z, (int)r[j].q[0].w};
          acc[i][j] = mfma_mx(ah, bq, sa, sbv[j], acc[i][j]);
          acc[i][j] = mfma_mx(al, bq, sa, sbv[j], acc[i][j]);
          pin_a(acc[i][j]);
        } else {
          const i32x8 bq = {(int)r[j].q[0].x, (int)r[j].q[0].y, (int)r[j].q[0].z, (int)r[j].q[0].w,
                            (int)r[j].q[1].x, (int)r[j].q[1].y, (int)r[j].q[1].z, (int)r[j].q[1].w};
          f32x4 t = mfma_f8(ah, bq, sa, f32x4{0.f, 0.f, 0.f, 0.f});
          t = mfma_f8(al, bq, sa, t);
          // subtile j's 128-row block: gate / up, or the half of the down rows
          const float bs = (GATED ? j < NH : wave < 2) ? fb0 : fb1;
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[i][j][u] = fmaf(bs, t[u], acc[i][j][u]);
          pin(acc[i][j]);  // the block-scale FMA reads it as a VALU operand
        }
      }
      if (i + 1 < MSUB) {
        ah = nh;
        al = nl;
        sa = ns;
      }
    }
  };

  // Chunk c is computed from LDS buffer c % 2 and register buffer rx / ry
  // while the loads of chunk c+1 are in flight; after the compute its A share
  // goes to the other LDS buffer; one barrier per chunk.  K/128 is even; the
  // last prefetch re-reads the last chunk (valid memory, never used).
  QRaw<FMT> rx[NSUB], ry[NSUB];
  a_issue(0);
  b_issue(0, rx);
  a_store(0);
  __syncthreads();
  for (int c = 0; c < nch; c += 2) {
    a_issue(c + 1);
    b_issue(c + 1, ry);
    compute(0, rx);
    a_store(1);
    __syncthreads();
    const int c2 = c + 2 < nch ? c + 2 : nch - 1;
    a_issue(c2);
    b_issue(c2, rx);
    compute(1, ry);
    a_store(0);
    __syncthreads();
  }

  if constexpr (GATED) {
    // h goes out split for the down GEMM: the wave's 32 columns are one block
    static_assert(NH == 2, "one 32-column block of h per wave");
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = i * 16 + g * 4 + r;
        float hv[NH];
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float gv = acc[i][j][r], uv = acc[i][j + NH][r];
          hv[j] = gv / (1.0f + expf(-gv)) * uv;
        }
        const size_t row = (size_t)(seg0 + (m < rows ? m : 0));
        h32_split_store(hv[0], hv[1], m < rows, l16, ncol0, a.hq_hi + row * a.I,
                        a.hq_lo + row * a.I, a.hq_sc + row * (a.I / 32));
      }
  } else {
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = i * 16 + g * 4 + r;
          if (m < rows)
            a.y_perm[(size_t)(seg0 + m) * a.H + ncol0 + j * 16 + l16] = f32_to_bf16_rne(acc[i][j][r]);
        }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void ffn_gateup_mx_kernel(FfnArgs a) {
  ffn_mx_pipe_body<FMT, true>(a);
}
template <int FMT>
__global__ __launch_bounds__(256) void ffn_down_mx_kernel(FfnArgs a) {
  ffn_mx_pipe_body<FMT, false>(a);
}

// ---------------------------------------------------------------------------
// MXFP4 prefill over an LDS-DMA pipeline: a 128-row x 256-weight-row tile on
// 8 waves (2 row halves x 4 column quarters, 64 x 64 outputs per wave).
// Every operand byte goes from global memory straight into LDS
// (global_load_lds_dwordx4: lane l of one instruction writes 16 bytes at
// base + 16 l), two K chunks deep, so no registers hold loads in flight.
// Waits are explicit: at chunk c a wave waits for its own copies of chunk c
// (vmcnt) and for its LDS reads of chunk c-1 (lgkmcnt), then one barrier
// makes all copies visible and frees chunk c-1's stage for chunk c+1.
// ---------------------------------------------------------------------------
// m-tiles per super-tile of the copy-pipeline kernels: MXFP4 4 (large prefill
// FFN 9.87 -> 9.81 ms against 8; 16, 32 and 64 within 4 % and slower), NVFP4 8
// (4 and 2 measured 1 % slower)
constexpr int kDmaSuperM = 4;
constexpr int kNvSuperM = 8;
template <int BM, int BN>
struct MxDmaStage {
  uint8_t ah[BM * 128];  // A hi [row][128 B]: 16-byte unit u stored at u ^ a_swz(row)
  uint8_t al[BM * 128];  // A lo, same layout
  uint8_t b[BN * 64];        // weights [row][64 B]: unit u stored at u ^ b_swz(row)
  // scales, the chunk's 4 E8M0 bytes per row, ordered so that a lane's four
  // subtiles of a 64-row group are one 16-byte read: A row (half h,
  // subtile i, l) at h*64 + 4l + i, weight row (group q, subtile j, l) at
  // q*64 + 4l + j
  __attribute__((aligned(16))) uint32_t as[BM];
  __attribute__((aligned(16))) uint32_t bs[BN];
};

template <bool GATED, int MB, int WAVES, int BN>
__device__ __forceinline__ void ffn_mx_dma_body(const FfnArgs& a, MxDmaStage<MB * 64, BN>& s0,
                                                MxDmaStage<MB * 64, BN>& s1) {
  static_assert(BN == 256 || BN == 512, "256 or 512 weight rows per block");
  constexpr int BM = MB * 64, WN = WAVES / MB;  // MB row groups of 64 x WN column groups
  constexpr int NSUB = BN / 16 / WN;        // 16-row weight subtiles per wave
  constexpr int NQ = NSUB / 4;              // 64-row weight groups per wave
  constexpr int MSUB = 4, NH = GATED ? 2 : 4;
  constexpr int NCOLB = GATED ? BN / 2 : BN;  // output columns per block
  constexpr int CPA = BM / 8 / WAVES;         // 1 KB copies of A hi (and lo) per wave
  constexpr int CPB = BN / 16 / WAVES;        // 1 KB copies of weights per wave
  constexpr int NBS = BN / 64;                // 256 B copies of weight scales
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I, nch = K / KC, KS = K / 32;
  const int nnb = N_out / NCOLB;
  const int b = (int)blockIdx.x;
  int tile, nb;
  tile_of_block<kDmaSuperM>(b, nnb, tile, nb);
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave / WN, nw = wave % WN;

  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (tid < 64) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) {
        dbg_segment(ti.seg0, ti.rows, a.A);
        s_ti = ti;
      }
    }
  }
  __syncthreads();
  if (!s_valid) return;
  const int e = __builtin_amdgcn_readfirstlane(s_ti.e);
  const int seg0 = __builtin_amdgcn_readfirstlane(s_ti.seg0);
  const int rows = __builtin_amdgcn_readfirstlane(s_ti.rows);
  const uint8_t* rec = record_of(a, e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);
  // rows past the tile read its first row: valid memory, outputs discarded
  if (tid < BM) {
    const int rr = tid < rows ? tid : 0;
    src_row[tid] = GATED ? dbg_clamp(a.sorted_idx[seg0 + rr], a.A, kDbgSorted) / a.k : seg0 + rr;
  }
  __syncthreads();
  // weight row of block-local row br = (group br/64, subtile (br/16)%4,
  // br%16); a gated group is 32 gate rows then the matching 32 up rows
  auto wrow = [&](int br) {
    const int q = br >> 6, j = (br >> 4) & 3, l = br & 15;
    if constexpr (GATED) {
      const int c0 = nb * NCOLB + q * (NH * 16);
      return j < NH ? c0 + j * 16 + l : a.I + c0 + (j - NH) * 16 + l;
    } else {
      return nb * NCOLB + br;
    }
  };
  // This wave's copies per chunk: A hi and lo units of rows 8n..8n+7 for
  // n = CPA*wave + q, weights of rows 16n..16n+15 for n = CPB*wave + q (16 B
  // per lane each), one dword per lane of weight scales (groups wave,
  // wave + 8, ...) and, on waves 0 and 1, of A scales (half = wave).  32-bit
  // offsets (the caller checks the sizes).
  constexpr int NSB = (NBS + WAVES - 1) / WAVES;  // weight-scale copies per wave
  uint32_t ao[CPA], wo[CPB], sob[NSB], soa = 0;
#pragma unroll
  for (int q = 0; q < CPA; ++q) {
    const int ar = (wave * CPA + q) * 8 + (lane >> 3);
    ao[q] = (uint32_t)src_row[ar] * (uint32_t)K + (uint32_t)(((lane & 7) ^ a_swz(ar)) * 16);
  }
#pragma unroll
  for (int q = 0; q < CPB; ++q) {
    const int br = (wave * CPB + q) * 16 + (lane >> 2);
    wo[q] = (uint32_t)wrow(br) * (uint32_t)(K / 2) + (uint32_t)(((lane & 3) ^ b_swz(br)) * 16);
  }
#pragma unroll
  for (int q = 0; q < NSB; ++q) {
    const int grp64 = wave + q * WAVES;
    sob[q] = grp64 < NBS ? (uint32_t)wrow(grp64 * 64 + (lane & 3) * 16 + (lane >> 2)) * (uint32_t)KS : 0u;
  }
  if (wave < MB) soa = (uint32_t)src_row[wave * 64 + (lane & 3) * 16 + (lane >> 2)] * (uint32_t)KS;
  auto issue = [&](int c, MxDmaStage<BM, BN>& S) {
    const uint32_t ka = (uint32_t)(c * KC), kb = (uint32_t)(c * (KC / 2)), ks = (uint32_t)(c * 4);
#pragma unroll
    for (int q = 0; q < CPA; ++q) {
      const int n = wave * CPA + q;
      dma16(a.aq_hi, ao[q] + ka, S.ah + n * 1024);
      dma16(a.aq_lo, ao[q] + ka, S.al + n * 1024);
    }
#pragma unroll
    for (int q = 0; q < CPB; ++q) dma16(w, wo[q] + kb, S.b + (wave * CPB + q) * 1024);
#pragma unroll
    for (int q = 0; q < NSB; ++q)
      if (wave + q * WAVES < NBS) dma4(sc, sob[q] + ks, S.bs + (wave + q * WAVES) * 64);
    if (wave < MB) dma4(a.aq_sc, soa + ks, S.as + wave * 64);
  };

  f32x4 acc[MSUB][NSUB];
#pragma unroll
  for (int i = 0; i < MSUB; ++i)
#pragma unroll
    for (int j = 0; j < NSUB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the wave's weight subtiles, then its 4 row subtiles (the next one's A
  // fragments read while the current one's MFMAs run)
  auto compute = [&](const MxDmaStage<BM, BN>& S) {
    i32x4 bq[NSUB];
    int sb[NSUB];
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int grp64 = nw * NQ + qq;
      const uint4 bsv = *reinterpret_cast<const uint4*>(&S.bs[grp64 * 64 + l16 * 4]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = qq * 4 + jj, br = grp64 * 64 + jj * 16 + l16;
        bq[j] = *reinterpret_cast<const i32x4*>(S.b + br * 64 + ((g ^ b_swz(br)) * 16));
        const uint32_t d = jj == 0 ? bsv.x : jj == 1 ? bsv.y : jj == 2 ? bsv.z : bsv.w;
        sb[j] = (int)((d >> (8 * g)) & 0xffu);
      }
    }
    const uint4 asv = *reinterpret_cast<const uint4*>(&S.as[mh * 64 + l16 * 4]);
    auto frag = [&](int i, i32x8& h, i32x8& l, int& sa) {
      const int r = mh * 64 + i * 16 + l16, sw = a_swz(r);
      const uint8_t* ph = S.ah + r * 128;
      const uint8_t* pl = S.al + r * 128;
      const i32x4 h0 = *reinterpret_cast<const i32x4*>(ph + (((2 * g) ^ sw) * 16));
      const i32x4 h1 = *reinterpret_cast<const i32x4*>(ph + (((2 * g + 1) ^ sw) * 16));
      const i32x4 l0 = *reinterpret_cast<const i32x4*>(pl + (((2 * g) ^ sw) * 16));
      const i32x4 l1 = *reinterpret_cast<const i32x4*>(pl + (((2 * g + 1) ^ sw) * 16));
      h = i32x8{h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      l = i32x8{l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
      const uint32_t d = i == 0 ? asv.x : i == 1 ? asv.y : i == 2 ? asv.z : asv.w;
      sa = (int)((d >> (8 * g)) & 0xffu);
    };
    i32x8 ah, al;
    int sa;
    frag(0, ah, al, sa);
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      i32x8 nh, nl;
      int ns = 0;
      if (i + 1 < MSUB) frag(i + 1, nh, nl, ns);
#pragma unroll
      for (int j = 0; j < NSUB; ++j) {
        acc[i][j] = mfma_mx(ah, bq[j], sa, sb[j], acc[i][j]);
        acc[i][j] = mfma_mx(al, bq[j], sa, sb[j], acc[i][j]);
        if constexpr (NSUB > 4) pin_a(acc[i][j]);  // accumulators in AGPRs
      }
      if (i + 1 < MSUB) {
        ah = nh;
        al = nl;
        sa = ns;
      }
    }
  };

  // K/128 >= 2 (even).  Two stages, separate LDS objects, each step naming
  // its own: chunk c+1 is copied while chunk c is computed.
  auto step = [&](int c, const MxDmaStage<BM, BN>& cur, MxDmaStage<BM, BN>& nxt) {
    MOE_DMA_SYNC(0);
    if (c + 1 < nch) issue(c + 1, nxt);
    compute(cur);
  };
  issue(0, s0);
  for (int c = 0; c < nch; c += 2) {
    step(c, s0, s1);
    step(c + 1, s1, s0);
  }

  const int m_base = mh * 64;
  if constexpr (GATED) {
    // h goes out split for the down GEMM: group qq's 32 columns are one block
    static_assert(NH == 2, "one 32-column block of h per weight group");
#pragma unroll
    for (int qq = 0; qq < NQ; ++qq) {
      const int c0 = nb * NCOLB + (nw * NQ + qq) * (NH * 16);
#pragma unroll
      for (int i = 0; i < MSUB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m_base + i * 16 + g * 4 + r;
          float hv[NH];
#pragma unroll
          for (int jj = 0; jj < NH; ++jj) {
            const float gv = acc[i][qq * 4 + jj][r], uv = acc[i][qq * 4 + NH + jj][r];
            hv[jj] = gv / (1.0f + expf(-gv)) * uv;
          }
          const size_t row = (size_t)(seg0 + (m < rows ? m : 0));
          h32_split_store(hv[0], hv[1], m < rows, l16, c0, a.hq_hi + row * a.I,
                          a.hq_lo + row * a.I, a.hq_sc + row * (a.I / 32));
        }
    }
  } else {
    const int ncol0 = nb * NCOLB + nw * (NSUB * 16);
#pragma unroll
    for (int i = 0; i < MSUB; ++i)
#pragma unroll
      for (int j = 0; j < NSUB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m_base + i * 16 + g * 4 + r;
          if (m < rows)
            a.y_perm[(size_t)(seg0 + m) * a.H + ncol0 + j * 16 + l16] = f32_to_bf16_rne(acc[i][j][r]);
        }
  }
}

// 128 rows x 512 weight rows on 8 waves, one block per CU (the 7168 x 2048
// layer's gate/up kernel measured 7.1 ms, against 8.0 ms for 128 x 256 over
// three stages and 8.6 ms for 64 x 256 on 4 waves, two blocks per CU)
constexpr int kDmaMB = 2, kDmaWaves = 8, kDmaBN = 512;
constexpr int kDmaBM = kDmaMB * 64;
__global__ __launch_bounds__(kDmaWaves * 64) void ffn_gateup_mxd_kernel(FfnArgs a) {
  __shared__ MxDmaStage<kDmaBM, kDmaBN> s0, s1;
  ffn_mx_dma_body<true, kDmaMB, kDmaWaves, kDmaBN>(a, s0, s1);
}
__global__ __launch_bounds__(kDmaWaves * 64) void ffn_down_mxd_kernel(FfnArgs a) {
  __shared__ MxDmaStage<kDmaBM, kDmaBN> s0, s1;
  ffn_mx_dma_body<false, kDmaMB, kDmaWaves, kDmaBN>(a, s0, s1);
}

// ---------------------------------------------------------------------------
// NVFP4 prefill over the LDS-DMA pipeline: bf16 activations and E2M1 codes
// with their E4M3 block scales copied straight into LDS (two stages), the
// codes decoded to bf16 per lane right before the 32x32x16 bf16 MFMAs (that
// shape runs at twice the rate of 16x16x32 here: 2.5 against 1.3 PFLOP/s
// measured).  WAVES waves as MB row groups of 64 rows x WAVES/MB column
// groups over BN weight rows; a wave owns 2 x NB output blocks of 32 x 32.
//   32x32x16 operands (checked on the device): lane l holds row (A) or
//   column (B) l % 32 and 8 consecutive K at 8*(l/32) of the step's 16; result
//   value v of lane l is C[8*(v/4) + 4*(l/32) + v%4][l % 32].  Within a chunk
//   the K order is permuted the same way for A and B: step s, lane half h,
//   element e is K = 64h + 8s + e, so lane half h reads only the chunk's
//   half h of the activation row (one 16-byte unit per step) and of the
//   weight codes (32 bytes), and 4 of the row's 8 scale bytes.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void pin_a16(f32x16& acc) { asm volatile("" : "+a"(acc)); }

template <int BM, int BN>
struct NvDmaStage {
  // activation rows, bf16: the chunk's first and second 64 K values (128 B
  // each), 16-byte unit u stored at u ^ a_swz(row)
  uint8_t a0[BM * 128];
  uint8_t a1[BM * 128];
  uint8_t b[BN * 64];                    // E2M1 codes [row][64 B], unit u at u ^ b_swz(row)
  __attribute__((aligned(16))) uint2 bs[BN];  // the chunk's 8 E4M3 scale bytes per row
};

template <bool GATED, int MB, int WAVES, int BN>
__device__ __forceinline__ void ffn_nv_dma_body(const FfnArgs& a, NvDmaStage<MB * 64, BN>& s0,
                                                NvDmaStage<MB * 64, BN>& s1) {
  static_assert(MB == 1 || MB == 2, "64 or 128 rows per block");
  constexpr int BM = MB * 64, NWG = WAVES / MB;  // column groups
  constexpr int WR = BN / NWG;                   // weight rows per wave
  constexpr int NB = WR / 32;                    // 32-column blocks per wave
  constexpr int NCOLB = GATED ? BN / 2 : BN;     // output columns per block
  constexpr int CPA = BM / 8 / WAVES;            // 1 KB copies per activation half per wave
  constexpr int CPB = BN / 16 / WAVES;           // 1 KB copies of codes per wave
  constexpr int CPS = BN / 32 / WAVES;           // 256 B copies of scales per wave
  static_assert(CPA >= 1 && CPB >= 1 && CPS >= 1 && NB % 2 == 0, "block shape");
  using Stage = NvDmaStage<BM, BN>;
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I, nch = K / KC;
  const int nnb = N_out / NCOLB;
  const int b = (int)blockIdx.x;
  int tile, nb;
  tile_of_block<kNvSuperM>(b, nnb, tile, nb);
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mh = wave / NWG, nw = wave % NWG;

  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (tid < 64) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) {
        dbg_segment(ti.seg0, ti.rows, a.A);
        s_ti = ti;
      }
    }
  }
  __syncthreads();
  if (!s_valid) return;
  const int e = __builtin_amdgcn_readfirstlane(s_ti.e);
  const int seg0 = __builtin_amdgcn_readfirstlane(s_ti.seg0);
  const int rows = __builtin_amdgcn_readfirstlane(s_ti.rows);
  const uint8_t* rec = record_of(a, e);
  const uint8_t* w = rec + (GATED ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (GATED ? a.off_w13s : a.off_w2s);
  const uint8_t* asrc = reinterpret_cast<const uint8_t*>(GATED ? a.x : a.hbuf);
  // the record's fp32 tensor scales (gate, up, down), read once up front
  const float* tsp = reinterpret_cast<const float*>(rec + a.off_ts);
  const float ts0 = tsp[GATED ? 0 : 2], ts1 = GATED ? tsp[1] : 1.0f;
  // rows past the tile read its first row: valid memory, outputs discarded
  if (tid < BM) {
    const int rr = tid < rows ? tid : 0;
    src_row[tid] = GATED ? dbg_clamp(a.sorted_idx[seg0 + rr], a.A, kDbgSorted) / a.k : seg0 + rr;
  }
  __syncthreads();
  // weight row of block-local row br = (column group br/WR, 32-row block
  // (br/32) % NB, row br%32); a gated group's first NB/2 blocks are gate rows,
  // the rest the matching up rows
  auto wrow = [&](int br) {
    if constexpr (GATED) {
      const int q = br / WR, n = (br >> 5) % NB, j = br & 31;
      const int col = nb * NCOLB + q * (WR / 2) + (n % (NB / 2)) * 32 + j;
      return n < NB / 2 ? col : a.I + col;
    } else {
      return nb * NCOLB + br;
    }
  };
  // 32-bit byte offsets (the caller checks the sizes)
  uint32_t ao[CPA], wo[CPB], so[CPS];
#pragma unroll
  for (int q = 0; q < CPA; ++q) {
    const int ar = (wave * CPA + q) * 8 + (lane >> 3);
    ao[q] = (uint32_t)src_row[ar] * (uint32_t)(K * 2) + (uint32_t)(((lane & 7) ^ a_swz(ar)) * 16);
  }
#pragma unroll
  for (int q = 0; q < CPB; ++q) {
    const int br = (wave * CPB + q) * 16 + (lane >> 2);
    wo[q] = (uint32_t)wrow(br) * (uint32_t)(K / 2) + (uint32_t)(((lane & 3) ^ b_swz(br)) * 16);
  }
#pragma unroll
  for (int q = 0; q < CPS; ++q) {
    const int br = (wave * CPS + q) * 32 + (lane >> 1);
    so[q] = (uint32_t)wrow(br) * (uint32_t)(K / 16) + (uint32_t)((lane & 1) * 4);
  }
  auto issue = [&](int c, Stage& S) {
    const uint32_t ka = (uint32_t)(c * KC * 2), kb = (uint32_t)(c * (KC / 2)), ks = (uint32_t)(c * 8);
#pragma unroll
    for (int q = 0; q < CPA; ++q) {
      const int n = wave * CPA + q;
      dma16(asrc, ao[q] + ka, S.a0 + n * 1024);
      dma16(asrc, ao[q] + ka + 128, S.a1 + n * 1024);
    }
#pragma unroll
    for (int q = 0; q < CPB; ++q) dma16(w, wo[q] + kb, S.b + (wave * CPB + q) * 1024);
#pragma unroll
    for (int q = 0; q < CPS; ++q) dma4(sc, so[q] + ks, &S.bs[(wave * CPS + q) * 32]);
  };

  f32x16 acc[2][NB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  auto compute = [&](const Stage& S) {
    const uint8_t* ap = h ? S.a1 : S.a0;
    uint4 code[NB][2];
    float scl[NB][4];  // the lane's 4 block scales (K blocks 4h .. 4h+3) per column block
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int br = nw * WR + n * 32 + l32;
      const uint8_t* pb = S.b + br * 64;
      code[n][0] = *reinterpret_cast<const uint4*>(pb + (((2 * h) ^ b_swz(br)) * 16));
      code[n][1] = *reinterpret_cast<const uint4*>(pb + (((2 * h + 1) ^ b_swz(br)) * 16));
      const uint2 sv = S.bs[br];
      const int s4 = (int)(h ? sv.y : sv.x);
      scl[n][0] = __builtin_amdgcn_cvt_f32_fp8(s4, 0);
      scl[n][1] = __builtin_amdgcn_cvt_f32_fp8(s4, 1);
      scl[n][2] = __builtin_amdgcn_cvt_f32_fp8(s4, 2);
      scl[n][3] = __builtin_amdgcn_cvt_f32_fp8(s4, 3);
    }
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      bf16x8 af[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int r = mh * 64 + mb * 32 + l32;
        af[mb] = *reinterpret_cast<const bf16x8*>(ap + r * 128 + ((st ^ a_swz(r)) * 16));
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const uint4 q = code[n][st >> 2];
        const uint32_t d = (st & 3) == 0 ? q.x : (st & 3) == 1 ? q.y : (st & 3) == 2 ? q.z : q.w;
        const bf16x8 bv = fp4x8_to_bf16_mul(d, scl[n][st >> 1]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          acc[mb][n] = mfma32(af[mb], bv, acc[mb][n]);
          pin_a16(acc[mb][n]);
        }
      }
    }
  };

  // K/128 >= 2 (even): two stages, chunk c+1 copied while chunk c is computed
  auto step = [&](int c, const Stage& cur, Stage& nxt) {
    MOE_DMA_SYNC(0);
    if (c + 1 < nch) issue(c + 1, nxt);
    compute(cur);
  };
  issue(0, s0);
  for (int c = 0; c < nch; c += 2) {
    step(c, s0, s1);
    step(c + 1, s1, s0);
  }

  // lane (l32, h), value v: row 8*(v/4) + 4h + v%4 of the 32-row block
  if constexpr (GATED) {
    const float tsg = ts0, tsu = ts1;
#pragma unroll
    for (int n = 0; n < NB / 2; ++n) {
      const int col = nb * NCOLB + nw * (WR / 2) + n * 32 + l32;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mh * 64 + mb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (m < rows) {
            const float gv = acc[mb][n][v] * tsg, uv = acc[mb][n + NB / 2][v] * tsu;
            const float hv = gv / (1.0f + expf(-gv)) * uv;
            a.hbuf[(size_t)(seg0 + m) * a.I + col] = f32_to_bf16_rne(hv);
          }
        }
    }
  } else {
    const float tsd = ts0;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int col = nb * NCOLB + nw * WR + n * 32 + l32;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = mh * 64 + mb * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
          if (m < rows)
            a.y_perm[(size_t)(seg0 + m) * a.H + col] = f32_to_bf16_rne(acc[mb][n][v] * tsd);
        }
    }
  }
}

// 64 rows x 256 weight rows on 4 waves: 68 KB of LDS, two blocks per CU
// (measured 433 us for the 4096-token NVFP4 layer, against 463 us for 64 x 512
// and 519 us for 128 x 512 on 8 waves, one block per CU)
constexpr int kNvMB = 1, kNvWaves = 4, kNvBN = 256;
__global__ __launch_bounds__(kNvWaves * 64) void ffn_gateup_nvd_kernel(FfnArgs a) {
  __shared__ NvDmaStage<kNvMB * 64, kNvBN> s0, s1;
  ffn_nv_dma_body<true, kNvMB, kNvWaves, kNvBN>(a, s0, s1);
}
__global__ __launch_bounds__(kNvWaves * 64) void ffn_down_nvd_kernel(FfnArgs a) {
  __shared__ NvDmaStage<kNvMB * 64, kNvBN> s0, s1;
  ffn_nv_dma_body<false, kNvMB, kNvWaves, kNvBN>(a, s0, s1);
}

// bf16 rows [R][K] -> E4M3 hi / lo (A order) and E8M0 scales per 32 along K;
// workgroup b converts rows [8b, 8b + 8).
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src, int R,
                                                         int K, uint8_t* hi, uint8_t* lo,
                                                         uint8_t* sc) {
  const int r0 = blockIdx.x * 8, n = min(8, R - r0);
  if (n <= 0) return;
  prep_a_mx<256>(src + (size_t)r0 * K, n, K, K, hi + (size_t)r0 * K, lo + (size_t)r0 * K,
                 sc + (size_t)r0 * (K / 32));
}

// Decode one expert record to fp32 with the same decoders as the GEMMs.
template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ rec, FfnArgs a,
                                                      float* __restrict__ w13,
                                                      float* __restrict__ w2) {
  const int rows13 = 2 * a.I, K13 = a.H, K2 = a.I;
  const long n13 = (long)rows13 * (K13 / 32), n2 = (long)a.H * (K2 / 32);
  for (long u = blockIdx.x * 256L + threadIdx.x; u < n13 + n2; u += (long)gridDim.x * 256) {
    const bool first = u < n13;
    const long v = first ? u : u - n13;
    const int K = first ? K13 : K2;
    const int row = (int)(v / (K / 32)), k0 = (int)(v % (K / 32)) * 32;
    BRaw<FMT> raw;
    load_b_raw<FMT>(rec + (first ? a.off_w13 : a.off_w2), rec + (first ? a.off_w13s : a.off_w2s),
                    row, K, k0, raw);
    bf16x8 b[4];
    decode_b<FMT>(raw, b);
    const float bs = block_scale<FMT>(raw);
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
  a.aq_hi = a.aq_lo = a.aq_sc = nullptr;
}

template <int MSUB, int MH, typename K1, typename K2>
static void launch_pipe(const FfnArgs& a, K1 k1, K2 k2, hipStream_t s) {
  // whole super-tiles: the grid is then a multiple of 8 as well
  const int64_t mt = grid_m_tiles(max_tiles_for(a.A, a.E, MSUB * 16 * MH), kSuperM);
  k1<<<(unsigned)(mt * (a.I / 128)), 256 * MH, 0, s>>>(a);
  k2<<<(unsigned)(mt * (a.H / 256)), 256 * MH, 0, s>>>(a);
}

// The pipelined prefill kernels need K/128 even for both GEMMs and the
// column blocks to divide I (128) and H (256).
static bool pipe_ok(const FfnArgs& a) { return a.H % 256 == 0 && a.I % 256 == 0; }

static int64_t al256(int64_t n) { return (n + 255) / 256 * 256; }

// Workspace of one moe_expert_ffn call: h (bf16 [A][I]); or, on the
// block-scaled prefill path (which never forms bf16 h), the split A operands
// of both GEMMs from the same start: h as hi [A][I], lo [A][I], scales
// [A][I/32], then x as hi [T][H], lo, scales.  The size covers both.
struct FfnWs {
  int64_t h, hq_hi, hq_lo, hq_sc, xq_hi, xq_lo, xq_sc, total;
};
static bool quantized_prefill_fmt(int fmt) { return fmt == MOE_W_MXFP4 || fmt == MOE_W_FP8_B128; }
static FfnWs ffn_ws(int fmt, int64_t T, int64_t k, int H, int I) {
  FfnWs w{};
  const int64_t A = T * k;
  w.h = 0;
  int64_t end = al256(A * I * 2);
  if (quantized_prefill_fmt(fmt)) {
    int64_t p = 0;
    w.hq_hi = p; p += al256(A * I);
    w.hq_lo = p; p += al256(A * I);
    w.hq_sc = p; p += al256(A * I / 32);
    w.xq_hi = p; p += al256(T * H);
    w.xq_lo = p; p += al256(T * H);
    w.xq_sc = p; p += al256(T * H / 32);
    end = end > p ? end : p;
  }
  w.total = end + 256;
  return w;
}

template <int FMT>
static void launch_ffn(const FfnArgs& a, bool decode, hipStream_t s) {
  if constexpr (FMT == MOE_W_MXFP4 || FMT == MOE_W_FP8_B128) {
    const int T = a.A / a.k;
    // the kernels address the split operands with 32-bit offsets
    const bool fits = (int64_t)T * a.H < (1ll << 32) && (int64_t)a.A * a.I < (1ll << 32);
    if (!decode && pipe_ok(a) && fits) {
      // split x once; gate/up, whose epilogue writes h split; down
      const FfnWs L = ffn_ws(FMT, T, a.k, a.H, a.I);
      uint8_t* ws = reinterpret_cast<uint8_t*>(a.hbuf);
      FfnArgs g = a;
      g.aq_hi = ws + L.xq_hi; g.aq_lo = ws + L.xq_lo; g.aq_sc = ws + L.xq_sc;
      g.hq_hi = ws + L.hq_hi; g.hq_lo = ws + L.hq_lo; g.hq_sc = ws + L.hq_sc;  // gate/up writes h split
      FfnArgs d = a;
      d.aq_hi = ws + L.hq_hi; d.aq_lo = ws + L.hq_lo; d.aq_sc = ws + L.hq_sc;
      quant_rows_kernel<<<(unsigned)((T + 7) / 8), 256, 0, s>>>(
          a.x, T, a.H, ws + L.xq_hi, ws + L.xq_lo, ws + L.xq_sc);
      // (FP8 on a 128 x 256 copy-pipeline tile measured 0.91 ms against 0.86 ms on
      // these 64-row kernels for its skewed 2048-token batch: LDS-bound)
      if (FMT == MOE_W_MXFP4 && a.I % (kDmaBN / 2) == 0 && a.H % kDmaBN == 0) {
        // 128-row tiles on the LDS-DMA pipeline
        const int64_t mt =
            grid_m_tiles(max_tiles_for(a.A, a.E, kDmaBM), kDmaSuperM);
        ffn_gateup_mxd_kernel<<<(unsigned)(mt * (a.I / (kDmaBN / 2))), kDmaWaves * 64, 0, s>>>(g);
        ffn_down_mxd_kernel<<<(unsigned)(mt * (a.H / kDmaBN)), kDmaWaves * 64, 0, s>>>(d);
      } else {
        const int64_t mt = grid_m_tiles(max_tiles_for(a.A, a.E, 64), kMxSuperM);
        ffn_gateup_mx_kernel<FMT><<<(unsigned)(mt * (a.I / 128)), 256, 0, s>>>(g);
        ffn_down_mx_kernel<FMT><<<(unsigned)(mt * (a.H / 256)), 256, 0, s>>>(d);
      }
      return;
    }
  }
  if (decode) {
    const int64_t mt = max_tiles_for(a.A, a.E, 16);
    ffn_gateup_decode_kernel<FMT><<<(unsigned)(mt * (a.I / kGuCols)), 256, 0, s>>>(a);
    ffn_down_decode_kernel<FMT><<<(unsigned)(mt * (a.H / kDnCols)), 256, 0, s>>>(a);
  } else if (pipe_ok(a)) {
    if constexpr (FMT == MOE_W_NVFP4) {
      // the activations are read as bytes with 32-bit offsets
      const bool fits = (int64_t)(a.A / a.k) * a.H * 2 < (1ll << 32) &&
                        (int64_t)a.A * a.I * 2 < (1ll << 32);
      if (fits && a.I % (kNvBN / 2) == 0 && a.H % kNvBN == 0) {
        const int64_t mt =
            grid_m_tiles(max_tiles_for(a.A, a.E, kNvMB * 64), kNvSuperM);
        ffn_gateup_nvd_kernel<<<(unsigned)(mt * (a.I / (kNvBN / 2))), kNvWaves * 64, 0, s>>>(a);
        ffn_down_nvd_kernel<<<(unsigned)(mt * (a.H / kNvBN)), kNvWaves * 64, 0, s>>>(a);
        return;
      }
    }
    // 64 rows per wave (more needs too many registers for two waves per SIMD);
    // a 128-row tile over 8 waves (MH = 2) measured slower than 64-row tiles
    launch_pipe<4, 1>(a, ffn_gateup_pipe_kernel<FMT, 4, 1>, ffn_down_pipe_kernel<FMT, 4, 1>, s);
  } else {
    const int64_t mt = max_tiles_for(a.A, a.E, kPreMSUB * 16);
    ffn_gateup_tile_kernel<FMT><<<(unsigned)(mt * (a.I / 128)), 256, 0, s>>>(a);
    ffn_down_tile_kernel<FMT><<<(unsigned)(mt * (a.H / 128)), 256, 0, s>>>(a);
  }
}

#ifdef MOE_DEBUG
uint32_t dbg_take_ffn() { return dbg_take_unit(); }
#endif

}  // namespace moe

using namespace moe;


extern "C" size_t moe_expert_ffn_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W || T < 0 || k < 1 || W->E < 1) return 0;
  return (size_t)ffn_ws(W->fmt, T, k, W->H, W->I).total;
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

  // few rows per expert -> bandwidth-bound split-K kernels
  const bool decode = (variant == 1 || (variant == 0 && A <= 2 * (int64_t)W->E)) &&
                      W->I % kGuCols == 0 && W->H % kDnCols == 0;
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  switch (W->fmt) {
    case MOE_W_BF16: launch_ffn<MOE_W_BF16>(a, decode, s); break;
    case MOE_W_MXFP4: launch_ffn<MOE_W_MXFP4>(a, decode, s); break;
    case MOE_W_NVFP4: launch_ffn<MOE_W_NVFP4>(a, decode, s); break;
    default: launch_ffn<MOE_W_FP8_B128>(a, decode, s); break;
  }
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
