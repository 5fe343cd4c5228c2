// Per-expert SwiGLU FFN over the permuted rows (grouped GEMM on the bf16 MFMA
// V_MFMA_F32_16X16X32_BF16): one launch for gate/up with the SiLU*mul
// epilogue, one for down.
//
// Work unit = (m-tile of one expert's rows, block of output columns).  Each
// workgroup finds its (expert, first row) from `counts` itself (a wave-wide
// prefix sum of per-expert tile counts), so no extra launch or host sync is
// needed and the whole call can be captured into a graph.
//
// Operands.  A = activations: bf16 rows gathered by token (gate/up) or the
// contiguous h rows (down).  B = expert weights, read from HBM into registers
// in their stored format and decoded there to bf16 (every MXFP4 value, NVFP4
// E2M1 x E4M3 product and E4M3 value is exact in bf16); FP8 block scales and
// NVFP4 tensor scales multiply fp32 partial sums.
//
// K mapping.  For a 128-wide K chunk, lane group g = lane/16 owns the 32
// consecutive K values [32g, 32g+32) of its row; MFMA step s consumes values
// [32g+8s, 32g+8s+8).  A and B use the same mapping, so each output is the
// full dot product whatever the instruction's internal K order.
//
// Two kernel families:
//  * decode (few rows per expert): m-tile = 16 rows; the 4 waves of a
//    workgroup split K (chunks w, w+4, ...), each wave issues the loads of
//    up to 4 chunks before consuming any (16 KB in flight per wave), and the
//    4 partial sums are added in wave order through LDS (deterministic).
//    Bandwidth-bound: each touched expert's weights are read once.
//  * prefill (many rows): m-tile = 64 rows staged in LDS, each wave owns
//    16 x 4 output columns over the full K.
#include "ffn_common.h"

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
  if (l16 < ti.rows) tok = GATED ? a.sorted_idx[ti.seg0 + l16] : ti.seg0 + l16;
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
      if (ok) s_ti = ti;
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
// even (the last prefetch re-reads the last chunk).  Blocks are numbered so
// that consecutive logical blocks (the column blocks of one tile, which read
// the same A rows) land on one XCD: hardware block b runs on XCD b % 8.
// ----------------------------------------------------------------------------
template <int FMT, bool GATED, int MSUB, int MH>
__device__ __forceinline__ void ffn_pipe_body(const FfnArgs& a) {
  // MH row groups of MSUB*16 rows; 4*MH waves: wave = (row group, column quarter)
  constexpr int NT = 256 * MH, WM = MSUB * 16, BM = WM * MH, NSUB = 4, NH = GATED ? 2 : 4;
  constexpr int NCOLB = GATED ? 128 : 256;  // output columns per block
  const int N_out = GATED ? a.I : a.H;
  const int K = GATED ? a.H : a.I, nch = K / KC;
  const int nnb = N_out / NCOLB;
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  const int lid = (b & 7) * (G >> 3) + (b >> 3);  // G is a multiple of 8
  const int tile = lid / nnb, nb = lid - tile * nnb;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = (tid >> 6) & 3, mh = tid >> 8;  // column quarter, row group

  __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * A_PITCH];
  __shared__ int src_row[BM];
  __shared__ TileInfo s_ti;
  __shared__ int s_valid;
  if (tid < 64) {
    TileInfo ti;
    const bool ok = find_tile<BM>(a.counts, a.offsets, a.E, tile, lane, ti);
    if (lane == 0) {
      s_valid = ok;
      if (ok) s_ti = ti;
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
    src_row[r] = GATED ? a.sorted_idx[seg0 + rr] / a.k : seg0 + rr;
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
  };
  auto a_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MSUB; ++i) {
      const int q = tid + NT * i, r = q >> 4, col = (q & 15) * 8;
      *reinterpret_cast<uint4*>(&As[buf][r * A_PITCH + col]) = av[i];
    }
  };
  auto b_issue = [&](int c, BRaw<FMT> (&r)[NSUB]) {
#pragma unroll
    for (int j = 0; j < NSUB; ++j) load_b_raw<FMT>(w, sc, brow[j], K, c * KC + g * 32, r[j]);
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
      decode_b<FMT>(r[j], bv);
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
}

template <int MSUB, int MH, typename K1, typename K2>
static void launch_pipe(const FfnArgs& a, K1 k1, K2 k2, hipStream_t s) {
  const int64_t mt = max_tiles_for(a.A, a.E, MSUB * 16 * MH);
  auto pad8 = [](int64_t n) { return (unsigned)((n + 7) / 8 * 8); };
  k1<<<pad8(mt * (a.I / 128)), 256 * MH, 0, s>>>(a);
  k2<<<pad8(mt * (a.H / 256)), 256 * MH, 0, s>>>(a);
}

// The pipelined prefill kernels need K/128 even for both GEMMs and the
// column blocks to divide I (128) and H (256).
static bool pipe_ok(const FfnArgs& a) { return a.H % 256 == 0 && a.I % 256 == 0; }

template <int FMT>
static void launch_ffn(const FfnArgs& a, bool decode, hipStream_t s) {
  if (decode) {
    const int64_t mt = max_tiles_for(a.A, a.E, 16);
    ffn_gateup_decode_kernel<FMT><<<(unsigned)(mt * (a.I / kGuCols)), 256, 0, s>>>(a);
    ffn_down_decode_kernel<FMT><<<(unsigned)(mt * (a.H / kDnCols)), 256, 0, s>>>(a);
  } else if (pipe_ok(a)) {
    // 64 rows per wave (more needs too many registers for two waves per SIMD);
    // a 128-row tile over 8 waves (MH = 2) measured slower than 64-row tiles
    launch_pipe<4, 1>(a, ffn_gateup_pipe_kernel<FMT, 4, 1>, ffn_down_pipe_kernel<FMT, 4, 1>, s);
  } else {
    const int64_t mt = max_tiles_for(a.A, a.E, kPreMSUB * 16);
    ffn_gateup_tile_kernel<FMT><<<(unsigned)(mt * (a.I / 128)), 256, 0, s>>>(a);
    ffn_down_tile_kernel<FMT><<<(unsigned)(mt * (a.H / 128)), 256, 0, s>>>(a);
  }
}

}  // namespace moe

using namespace moe;

static size_t ws_h_bytes(int64_t A, int I) { return (size_t)((A * I * 2 + 255) / 256 * 256); }

extern "C" size_t moe_expert_ffn_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W || T < 0 || k < 1 || W->E < 1) return 0;
  return ws_h_bytes((int64_t)T * k, W->I) + 256;
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
