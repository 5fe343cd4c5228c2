// The MoE layer for decode-sized batches (moe_forward_decode).  Kernel
// boundaries are the only waits between workgroups.  Three forms:
//
//  * one weight stream (MXFP4, T <= 16, T*k*(I/128) a multiple of 256): two
//    launches, dec_fused_tok_kernel (a workgroup per (token, slot, 128 h
//    columns) routes its token, computes that h slice and its share of the
//    down projection as fp32 partials) and dec_fused_combine_kernel;
//  * token-major (T <= 16, H <= 2048): two launches, dec_gateup_tok_kernel
//    (routing inside) and dec_down_tok_kernel (combine folded in);
//  * tile-major (larger T), four launches:
//  1. route + permute: one workgroup (route_permute_small_kernel).
//  2. gate/up: a persistent grid sized by occupancy.  Each workgroup stages x,
//     sorted_idx and the 16-row tile list in LDS in one round trip, then takes
//     units u = blockIdx.x, +gridDim.x, ... (unit = one tile x 32 h-columns;
//     the 4 waves split K), two at a time with both units' weights in flight
//     before either is computed; SiLU(gate)*up is rounded to bf16 into h.
//  3. down: the same unit scheme over (tile x 64 output columns), h rows
//     read with the weights; y_perm is rounded to bf16.
//  4. combine: moe_combine's kernel (one workgroup per token).  Finishing
//     the combine inside the down kernel needs a device-scope release per
//     unit (an L2 write-back on this chip), which costs far more than a
//     launch.
//
// Arithmetic per element: fp32 MFMA accumulation, K partials summed in wave
// order, bf16 rounding of h and y_perm, combine in top-k order in fp32.
#include "ffn_common.h"
#include "route_common.h"

namespace moe {

constexpr int kDT = 64, kDA = 256, kDTiles = 256;
constexpr int kTokMaxT = 16, kTokMaxH = 2048;  // token-major path: T <= 16, H <= 2048

struct DecArgs {
  FfnArgs f;
  const float* logits;
  int T, renorm;
  int* ids;
  float* wts;
  int* counts;
  int* offsets;
  int* sorted;
  int* inv;
  const uint16_t* y_shared;
  uint16_t* y;
  float* part;  // fused path: per-(token, slot, h-slice) down partials [T*k][I/128][H]
};

// ----------------------------------------------------------------------------
// tile table of a workgroup: 16-row tiles of every expert with rows, ascending
// ----------------------------------------------------------------------------
struct TileTable {
  int cnt[kMaxE];
  int off[kMaxE];
  int tb[kMaxE];
  int tile_e[kDTiles];
  int tile_m0[kDTiles];
  int tile_slot[kDTiles];  // record index of the tile's expert (slot table applied)
  int wave_tot[16];
};

// Per-thread registers of the tile-table inputs (entries e = tid + i*NT).
template <int NT>
struct TileRegs {
  int c[kMaxE / NT], o[kMaxE / NT], s[kMaxE / NT];
};

// Issues the reads of counts, offsets and the slot table; nothing waits here,
// so the caller can put other loads in the same round trip.
template <int NT>
__device__ __forceinline__ void tiles_load(const FfnArgs& a, TileRegs<NT>& r) {
#pragma unroll
  for (int i = 0; i < kMaxE / NT; ++i) {
    const int e = threadIdx.x + i * NT;
    r.c[i] = 0;
    r.o[i] = 0;
    r.s[i] = e;
    if (e < a.E) {
      r.c[i] = a.counts[e];
      r.o[i] = a.offsets[e];
      dbg_segment(r.o[i], r.c[i], a.A);
    }
  }
  if (a.slot_of) {
#pragma unroll
    for (int i = 0; i < kMaxE / NT; ++i) {
      const int e = threadIdx.x + i * NT;
      if (e < a.E) r.s[i] = dbg_clamp(a.slot_of[e], a.E, kDbgSlot);
    }
  }
}

// All NT threads: builds the table from what tiles_load read; returns the
// number of tiles.  Starts and ends with a barrier.
template <int NT>
__device__ __forceinline__ int tiles_build(const FfnArgs& a, const TileRegs<NT>& r, TileTable& L) {
  const int E = a.E;
#pragma unroll
  for (int i = 0; i < kMaxE / NT; ++i) {
    const int e = threadIdx.x + i * NT;
    if (e < E) {
      L.cnt[e] = r.c[i];
      L.off[e] = r.o[i];
      L.tb[e] = (r.c[i] + 15) / 16;
    }
  }
  __syncthreads();
  const int n = block_exclusive_scan<NT>(L.tb, E, L.wave_tot);
#pragma unroll
  for (int i = 0; i < kMaxE / NT; ++i) {
    const int e = threadIdx.x + i * NT;
    if (e < E) {
      const int first = L.tb[e], m = (r.c[i] + 15) / 16;
      for (int t = 0; t < m; ++t) {
        L.tile_e[first + t] = e;
        L.tile_m0[first + t] = t * 16;
        L.tile_slot[first + t] = r.s[i];
      }
    }
  }
  __syncthreads();
  return n;
}

__device__ __forceinline__ const uint8_t* tile_record(const FfnArgs& a, const TileTable& L,
                                                      int tile) {
  return a.base + (size_t)L.tile_slot[tile] * a.stride;
}

// Rows of bf16 from global to LDS by all NT threads: batch q0 of B uint4 per
// thread.  stage_load issues the loads, stage_store writes what arrived, so
// other loads can be issued between the two.  row_elems % 8 == 0.
template <int NT, int B>
__device__ __forceinline__ void stage_load(uint4 (&v)[B], const uint16_t* src, int src_pitch,
                                           int nrows, int row_elems, int q0) {
  const int c8 = row_elems / 8, n = nrows * c8;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int q = q0 + b * NT + (int)threadIdx.x;
    v[b] = uint4{0u, 0u, 0u, 0u};  // defined on every path: keeps v in registers
    if (q < n) {
      const int r = q / c8, c = (q - r * c8) * 8;
      v[b] = *reinterpret_cast<const uint4*>(src + (size_t)r * src_pitch + c);
    }
  }
}

template <int NT, int B>
__device__ __forceinline__ void stage_store(const uint4 (&v)[B], uint16_t* dst, int dst_pitch,
                                            int nrows, int row_elems, int q0) {
  const int c8 = row_elems / 8, n = nrows * c8;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const int q = q0 + b * NT + (int)threadIdx.x;
    if (q < n) {
      const int r = q / c8, c = (q - r * c8) * 8;
      *reinterpret_cast<uint4*>(dst + (size_t)r * dst_pitch + c) = v[b];
    }
  }
}

// ----------------------------------------------------------------------------
// expert units: gate/up (MODE_GU) and down (MODE_DN)
//
// A unit is one 16-row tile times four 16-column subtiles of the weight
// matrix: gate/up takes 16 gate + 16 up columns twice (32 h-columns), down
// takes 64 output columns.  The 4 waves split K: wave w owns the contiguous
// 128-wide chunks [w*CPW, w*CPW + CPW) (K = 512 * CPW).  CPW is a
// compile-time count, so a load and its use are never guarded by separate
// runtime branches (which would make the compiler wait for loads still needed
// later).  With MXFP4 and four chunks per wave a lane's scale bytes of a
// weight row (4 chunks x 4 lane groups) come in one 16-byte load.
// ----------------------------------------------------------------------------
constexpr int MODE_GU = 0, MODE_DN = 1;

template <int FMT, int CPW, int MODE>
struct UnitRaw {
  static constexpr bool S4 = FMT == MOE_W_MXFP4 && CPW == 4;  // scales as one uint4 per subtile
  BRaw<FMT> w[CPW][4];                   // [chunk slot][subtile]
  uint4 a[MODE == MODE_DN ? CPW : 1][4];  // down: h row chunk of this lane
  uint4 s4[S4 ? 4 : 1];
};

struct UnitPos {
  int tile, cb, e, rows, seg0;
};

__device__ __forceinline__ UnitPos unit_pos(const TileTable& L, int unit, int n_cb) {
  UnitPos q;
  q.tile = unit / n_cb;
  q.cb = unit - q.tile * n_cb;
  q.e = L.tile_e[q.tile];
  const int m0 = L.tile_m0[q.tile];
  q.rows = min(16, L.cnt[q.e] - m0);
  q.seg0 = L.off[q.e] + m0;
  return q;
}

// Loads of chunk slot j (K chunk wave*CPW + j) of a unit.
template <int FMT, int CPW, int MODE>
__device__ __forceinline__ void unit_issue_chunk(const FfnArgs& a, const TileTable& L,
                                                 const int* sidx, int unit, int n_cb, int j,
                                                 UnitRaw<FMT, CPW, MODE>& R) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const UnitPos q = unit_pos(L, unit, n_cb);
  const uint8_t* rec = tile_record(a, L, q.tile);
  const int c = wave * CPW + j;
  if constexpr (MODE == MODE_DN) {
    // h rows (stored by assignment; sidx maps sorted position -> assignment)
    // first: waiting for them never waits for the weights issued after.
    // Lanes past the tile's rows read its first row (discarded at use).
    const uint16_t* arow = a.hbuf + (size_t)sidx[q.seg0 + (l16 < q.rows ? l16 : 0)] * a.I;
    const uint4* src = reinterpret_cast<const uint4*>(arow + c * KC + g * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) R.a[j][i] = src[i];
  }
  const int K = MODE == MODE_GU ? a.H : a.I;
  const uint8_t* w = rec + (MODE == MODE_GU ? a.off_w13 : a.off_w2);
  const uint8_t* sc = rec + (MODE == MODE_GU ? a.off_w13s : a.off_w2s);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = MODE == MODE_GU ? (s < 2 ? 0 : a.I) + q.cb * 32 + (s & 1) * 16 + l16
                                    : q.cb * 64 + s * 16 + l16;
    if constexpr (UnitRaw<FMT, CPW, MODE>::S4) {
      R.w[j][s].q[0] = *reinterpret_cast<const uint4*>(w + (((size_t)row * K + c * KC + g * 32) >> 1));
      if (j == 0)  // bytes [16*wave, 16*wave + 16) of the row's scales
        R.s4[s] = *reinterpret_cast<const uint4*>(sc + (size_t)row * (K / 32) + wave * 16);
    } else {
      load_b_raw<FMT>(w, sc, row, K, c * KC + g * 32, R.w[j][s]);
    }
  }
}

template <int FMT, int CPW, int MODE>
__device__ __forceinline__ void unit_issue(const FfnArgs& a, const TileTable& L, const int* sidx,
                                           int unit, int n_cb, UnitRaw<FMT, CPW, MODE>& R) {
#pragma unroll
  for (int j = 0; j < CPW; ++j) unit_issue_chunk<FMT, CPW, MODE>(a, L, sidx, unit, n_cb, j, R);
}

struct NoIssue {
  __device__ __forceinline__ void operator()(int) const {}
};

// x rows come from LDS (xs, pitch xp) for gate/up; sidx holds sorted_idx.
// pre(j) runs before chunk slot j is computed (it issues the next unit's
// loads slot by slot, so computing starts as soon as this unit's data is in).
template <int FMT, int CPW, int MODE, typename Pre = NoIssue>
__device__ __forceinline__ void unit_finish(const FfnArgs& a, const TileTable& L, const int* sidx,
                                            const uint16_t* xs, int xp, f32x4 (&red)[4][4][64],
                                            int unit, int n_cb, const UnitRaw<FMT, CPW, MODE>& R,
                                            Pre pre = Pre()) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const UnitPos q = unit_pos(L, unit, n_cb);
  const bool live = l16 < q.rows;
  const uint16_t* xrow = nullptr;
  if constexpr (MODE == MODE_GU) xrow = xs + (sidx[q.seg0 + (live ? l16 : 0)] / a.k) * xp;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    pre(u);
    const int c = wave * CPW + u;
    bf16x8 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v;
      if constexpr (MODE == MODE_GU)
        v = *reinterpret_cast<const uint4*>(xrow + c * KC + g * 32 + i * 8);
      else
        v = R.a[u][i];
      av[i] = live ? bits_to_bf16x8(v.x, v.y, v.z, v.w) : bits_to_bf16x8(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 b[4];
      if constexpr (UnitRaw<FMT, CPW, MODE>::S4) {
        BRaw<FMT> r = R.w[u][j];
        const uint4 sv = R.s4[j];
        const uint32_t d = u == 0 ? sv.x : u == 1 ? sv.y : u == 2 ? sv.z : sv.w;
        r.s = (d >> (8 * g)) & 0xffu;
        decode_b<FMT>(r, b);
      } else {
        decode_b<FMT>(R.w[u][j], b);
      }
      if constexpr (FMT == MOE_W_FP8_B128) {
        f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) t = mfma16(av[i], b[i], t);
        const float bs = block_scale<FMT>(R.w[u][j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(bs, t[r], acc[j][r]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j] = mfma16(av[i], b[i], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  // K partials summed in wave order (fixed order: deterministic)
  if constexpr (MODE == MODE_GU) {
    if (wave < 2) {
      f32x4 gs = red[0][wave][lane], us = red[0][2 + wave][lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4 gw = red[w][wave][lane], uw = red[w][2 + wave][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gs[r] += gw[r];
          us[r] += uw[r];
        }
      }
      float tsg = 1.0f, tsu = 1.0f;
      if constexpr (FMT == MOE_W_NVFP4) {
        const float* ts = reinterpret_cast<const float*>(tile_record(a, L, q.tile) + a.off_ts);
        tsg = ts[0];
        tsu = ts[1];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = g * 4 + r;
        if (m < q.rows) {
          const float gv = gs[r] * tsg, uv = us[r] * tsu;
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          a.hbuf[(size_t)sidx[q.seg0 + m] * a.I + q.cb * 32 + wave * 16 + l16] =
              f32_to_bf16_rne(hv);
        }
      }
    }
  } else {
    f32x4 ys = red[0][wave][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 yw = red[w][wave][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) ys[r] += yw[r];
    }
    float tsd = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4)
      tsd = reinterpret_cast<const float*>(tile_record(a, L, q.tile) + a.off_ts)[2];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = g * 4 + r;
      if (m < q.rows)
        a.y_perm[(size_t)(q.seg0 + m) * a.H + q.cb * 64 + wave * 16 + l16] =
            f32_to_bf16_rne(ys[r] * tsd);
    }
  }
  __syncthreads();  // red is rewritten by the next unit
}

// Units go in pairs: the second unit's loads are issued chunk slot by chunk
// slot while the first is computed.  Nothing stays in flight across
// iterations, so no register holding a pending load is ever copied (a copy
// would wait for the load).
template <int FMT, int CPW>
__global__ __launch_bounds__(256) void dec_gateup_kernel(DecArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][H + 8]
  __shared__ TileTable L;
  __shared__ f32x4 red[4][4][64];
  __shared__ int sidx[kDA];
  const FfnArgs& a = p.f;
  const int xp = a.H + 8, tid = threadIdx.x, T = p.T;
  // one round trip: x rows, sorted_idx, counts/offsets/slot table
  uint4 xv[8];
  stage_load<256, 8>(xv, a.x, a.H, T, a.H, 0);
  const int sid = tid < a.A ? dbg_clamp(a.sorted_idx[tid], a.A, kDbgSorted) : 0;
  TileRegs<256> tr;
  tiles_load<256>(a, tr);
  stage_store<256, 8>(xv, xs, xp, T, a.H, 0);
  for (int q0 = 256 * 8; q0 < T * (a.H / 8); q0 += 256 * 8) {  // x beyond 32 KB
    stage_load<256, 8>(xv, a.x, a.H, T, a.H, q0);
    stage_store<256, 8>(xv, xs, xp, T, a.H, q0);
  }
  if (tid < a.A) sidx[tid] = sid;
  const int n_tiles = tiles_build<256>(a, tr, L);  // its barriers publish xs and sidx
  const int n_cb = a.I / 32, U = n_tiles * n_cb, G = (int)gridDim.x;
  UnitRaw<FMT, CPW, MODE_GU> ra, rb;
  for (int u = blockIdx.x; u < U; u += 2 * G) {
    unit_issue<FMT, CPW, MODE_GU>(a, L, sidx, u, n_cb, ra);
    if (u + G < U) {
      unit_finish<FMT, CPW, MODE_GU>(a, L, sidx, xs, xp, red, u, n_cb, ra, [&](int j) {
        unit_issue_chunk<FMT, CPW, MODE_GU>(a, L, sidx, u + G, n_cb, j, rb);
      });
      unit_finish<FMT, CPW, MODE_GU>(a, L, sidx, xs, xp, red, u + G, n_cb, rb);
    } else {
      unit_finish<FMT, CPW, MODE_GU>(a, L, sidx, xs, xp, red, u, n_cb, ra);
    }
  }
}

template <int FMT, int CPW>
__global__ __launch_bounds__(256) void dec_down_kernel(FfnArgs a) {
  __shared__ TileTable L;
  __shared__ f32x4 red[4][4][64];
  __shared__ int sidx[kDA];
  const int tid = threadIdx.x;
  const int sid = tid < a.A ? dbg_clamp(a.sorted_idx[tid], a.A, kDbgSorted) : 0;
  TileRegs<256> tr;
  tiles_load<256>(a, tr);
  if (tid < a.A) sidx[tid] = sid;
  const int n_tiles = tiles_build<256>(a, tr, L);
  const int n_cb = a.H / 64, U = n_tiles * n_cb, G = (int)gridDim.x;
  UnitRaw<FMT, CPW, MODE_DN> ra, rb;
  for (int u = blockIdx.x; u < U; u += 2 * G) {
    unit_issue<FMT, CPW, MODE_DN>(a, L, sidx, u, n_cb, ra);
    if (u + G < U) {
      unit_finish<FMT, CPW, MODE_DN>(a, L, nullptr, nullptr, 0, red, u, n_cb, ra, [&](int j) {
        unit_issue_chunk<FMT, CPW, MODE_DN>(a, L, sidx, u + G, n_cb, j, rb);
      });
      unit_finish<FMT, CPW, MODE_DN>(a, L, nullptr, nullptr, 0, red, u + G, n_cb, rb);
    } else {
      unit_finish<FMT, CPW, MODE_DN>(a, L, nullptr, nullptr, 0, red, u, n_cb, ra);
    }
  }
}

// ----------------------------------------------------------------------------
// token-major gate/up (small T): the grid is a multiple of T and workgroup b
// serves token t = b % T only, so it routes that one token itself (wave 0:
// one round trip for the logits row, then the top-k) and needs nothing from
// any other workgroup.  Its units u = b, b + G, ... are (t, expert slot j,
// 32 h-columns cb) with u = t + T*(j + k*cb); an expert's weights are read
// once per token that picked it.  The token's x row is row 0 of the MFMA A
// operand (the other 15 rows are zero); wave w takes the contiguous K chunks
// [w*CPW, w*CPW + CPW) and the 4 partial sums are added in wave order.  With
// MXFP4 and four chunks per wave a lane's 16 scale bytes of a weight row
// (4 chunks x 4 lane groups) come in one load, not one byte per chunk.  h is
// stored by assignment (t*k + j).  Workgroup t (< T) also writes the token's
// ids and weights.
// ----------------------------------------------------------------------------
template <int FMT, int CPW>
struct TokRaw {
  static constexpr bool S4 = FMT == MOE_W_MXFP4 && CPW == 4;  // scales as one uint4 per subtile
  BRaw<FMT> w[CPW][4];
  uint4 s4[S4 ? 4 : 1];
};

__device__ __forceinline__ void tok_unit(int u, int T, int k, int& j, int& cb) {
  const int r = u / T;
  j = r % k;
  cb = r / k;
}

template <int FMT, int CPW>
__device__ __forceinline__ void tok_issue_chunk(const FfnArgs& a, const int* eslot, int T, int u,
                                                int c_slot, TokRaw<FMT, CPW>& R) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int j, cb;
  tok_unit(u, T, a.k, j, cb);
  const uint8_t* rec = a.base + (size_t)eslot[j] * a.stride;
  const int c = wave * CPW + c_slot;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int row = (s < 2 ? 0 : a.I) + cb * 32 + (s & 1) * 16 + l16;
    if constexpr (TokRaw<FMT, CPW>::S4) {
      R.w[c_slot][s].q[0] = *reinterpret_cast<const uint4*>(
          rec + a.off_w13 + (((size_t)row * a.H + c * KC + g * 32) >> 1));
      if (c_slot == 0)  // bytes [16*wave, 16*wave + 16) of the row's scales
        R.s4[s] = *reinterpret_cast<const uint4*>(rec + a.off_w13s + (size_t)row * (a.H / 32) +
                                                  wave * 16);
    } else {
      load_b_raw<FMT>(rec + a.off_w13, rec + a.off_w13s, row, a.H, c * KC + g * 32,
                      R.w[c_slot][s]);
    }
  }
}

// MXFP4 takes the block-scaled MFMA: x as E4M3 hi + lo (mh, ml, ms: A order,
// E8M0 per 32) against the packed weights and their scale bytes, no decode.
template <int FMT, int CPW, typename Pre = NoIssue>
__device__ __forceinline__ void tok_finish(const FfnArgs& a, const int* eslot, const uint16_t* xs,
                                           const uint8_t* mh, const uint8_t* ml, const uint8_t* ms,
                                           const uint8_t* mz, f32x4 (&red)[4][4][64], int T, int t,
                                           int u,
                                           const TokRaw<FMT, CPW>& R, Pre pre = Pre()) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  f32x4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int cs = 0; cs < CPW; ++cs) {
    pre(cs);
    const int c = wave * CPW + cs;
    if constexpr (FMT == MOE_W_MXFP4) {
      // row 0 is the token; lanes of rows 1..15 read a zero block (scale 1)
      const int off = l16 == 0 ? c * KC + g * 32 : -1;
      const i32x8 ah = *reinterpret_cast<const i32x8*>(off < 0 ? mz : mh + off);
      const i32x8 al = *reinterpret_cast<const i32x8*>(off < 0 ? mz : ml + off);
      const int sa = off < 0 ? 127 : ms[c * 4 + g];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 q = R.w[cs][s].q[0];
        const i32x4 b = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
        int sb;
        if constexpr (TokRaw<FMT, CPW>::S4) {
          const uint32_t d = cs == 0 ? R.s4[s].x : cs == 1 ? R.s4[s].y : cs == 2 ? R.s4[s].z : R.s4[s].w;
          sb = (int)((d >> (8 * g)) & 0xffu);
        } else {
          sb = (int)R.w[cs][s].s;
        }
        acc[s] = mfma_mx(ah, b, sa, sb, acc[s]);
        acc[s] = mfma_mx(al, b, sa, sb, acc[s]);
        pin(acc[s]);
      }
      continue;
    }
    bf16x8 av[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 v = *reinterpret_cast<const uint4*>(xs + c * KC + g * 32 + q * 8);
      av[q] = l16 == 0 ? bits_to_bf16x8(v.x, v.y, v.z, v.w) : bits_to_bf16x8(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 b[4];
      decode_b<FMT>(R.w[cs][s], b);
      if constexpr (FMT == MOE_W_FP8_B128) {
        f32x4 tt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) tt = mfma16(av[q], b[q], tt);
        const float bs = block_scale<FMT>(R.w[cs][s]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(bs, tt[r], acc[s][r]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[s] = mfma16(av[q], b[q], acc[s]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) red[wave][s][lane] = acc[s];
  __syncthreads();
  if (wave < 2 && g == 0) {  // row 0: lanes 0..15, element 0
    float gs = red[0][wave][lane][0], us = red[0][2 + wave][lane][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      gs += red[w][wave][lane][0];
      us += red[w][2 + wave][lane][0];
    }
    int j, cb;
    tok_unit(u, T, a.k, j, cb);
    float tsg = 1.0f, tsu = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4) {
      const float* ts =
          reinterpret_cast<const float*>(a.base + (size_t)eslot[j] * a.stride + a.off_ts);
      tsg = ts[0];
      tsu = ts[1];
    }
    const float gv = gs * tsg, uv = us * tsu;
    const float hv = gv / (1.0f + expf(-gv)) * uv;
    a.hbuf[(size_t)(t * a.k + j) * a.I + cb * 32 + wave * 16 + l16] = f32_to_bf16_rne(hv);
  }
  __syncthreads();  // red is rewritten by the next unit
}

template <int FMT, int CPW, int VPL>
__global__ __launch_bounds__(256) void dec_gateup_tok_kernel(DecArgs p) {
  constexpr bool MX = FMT == MOE_W_MXFP4;
  __shared__ __attribute__((aligned(16))) uint16_t xs[MX ? 8 : kTokMaxH];
  __shared__ __attribute__((aligned(32))) uint8_t mx[MX ? 2 * kTokMaxH + kTokMaxH / 32 + 32 : 64];
  __shared__ f32x4 red[4][4][64];
  __shared__ int eslot[kMaxK];
  const FfnArgs& a = p.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = p.T, k = a.k, E = a.E, t = blockIdx.x % T;
  uint8_t *mh = mx, *ml = mx + kTokMaxH, *ms = mx + 2 * kTokMaxH;
  uint8_t* mz = ms + kTokMaxH / 32;  // 32 zero bytes: A rows 1..15
  if (tid < 8) reinterpret_cast<uint32_t*>(mz)[tid] = 0u;
  // one round trip: (wave 0) the token's logits row and its x row
  float lv[VPL];
  if (wave == 0) route_load<VPL>(p.logits + (size_t)t * E, E, lane, lv);
  if constexpr (MX) {
    // waves 1..3 split the x row while wave 0 routes
    if (wave > 0) prep_a_mx<192>(a.x + (size_t)t * a.H, 1, a.H, a.H, mh, ml, ms, tid - 64);
  } else {
    uint4 xv = uint4{0u, 0u, 0u, 0u};
    if (tid < a.H / 8) xv = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H)[tid];
    if (tid < a.H / 8) reinterpret_cast<uint4*>(xs)[tid] = xv;
  }
  // Wave 0 runs only the rounds that this workgroup's units need (their
  // assignment slots j <= jneed) before the weight loads start; workgroup
  // t < T, which also writes the token's ids and weights, finishes the other
  // rounds and the softmax while its first loads are in flight.
  const int U = T * k * (a.I / 32), G = (int)gridDim.x, b = (int)blockIdx.x;
  int jneed = 0;
  for (int u = b; u < U; u += G) jneed = max(jneed, (u / T) % k);
  TopK<VPL> st;
  if (wave == 0) {
    topk_begin<VPL>(lv, E, lane, st);
    for (int r = 0; r <= jneed; ++r) topk_round<VPL>(st, r, lane);
    if (lane <= jneed) eslot[lane] = a.slot_of ? dbg_clamp(a.slot_of[st.id_r], a.E, kDbgSlot) : st.id_r;
  }
  __syncthreads();
  TokRaw<FMT, CPW> ra, rb;
  for (int u = b; u < U; u += 2 * G) {
#pragma unroll
    for (int cs = 0; cs < CPW; ++cs) tok_issue_chunk<FMT, CPW>(a, eslot, T, u, cs, ra);
    if (b < T && u == b && wave == 0) {  // b == t
      for (int r = jneed + 1; r < k; ++r) topk_round<VPL>(st, r, lane);
      const float w = topk_weight<VPL>(st, lv, E, k, p.renorm, lane);
      if (lane < k) {
        p.ids[t * k + lane] = st.id_r;
        p.wts[t * k + lane] = w;
      }
    }
    if (u + G < U) {
      tok_finish<FMT, CPW>(a, eslot, xs, mh, ml, ms, mz, red, T, t, u, ra,
                           [&](int cs) { tok_issue_chunk<FMT, CPW>(a, eslot, T, u + G, cs, rb); });
      tok_finish<FMT, CPW>(a, eslot, xs, mh, ml, ms, mz, red, T, t, u + G, rb);
    } else {
      tok_finish<FMT, CPW>(a, eslot, xs, mh, ml, ms, mz, red, T, t, u, ra);
    }
  }
}

// The permutation outputs of a token-major call (counts, offsets, sorted_idx,
// inv_idx) from the routing ids, by one workgroup: stable rank inside each
// wave's 64 assignments from per-bit ballot match masks, earlier waves through
// per-wave histograms, then an exclusive scan of the counts.  Same results as
// route_permute_small_kernel.
__device__ __forceinline__ void permute_block(const DecArgs& p, int* lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.f.E, A = p.f.A;
  int* whist = lds;             // [4][E]
  int* hist = lds + 4 * E;      // [E]
  int* wave_tot = hist + kMaxE;  // [16]
  for (int i = tid; i < 4 * E; i += 256) whist[i] = 0;
  const bool live = tid < A;
  const int e = live ? p.ids[tid] : -1;
  __syncthreads();
  uint64_t m = __ballot(live);
#pragma unroll
  for (int b = 0; b < 10; ++b) {  // E <= 1024: 10 id bits
    const uint64_t on = __ballot(live && ((e >> b) & 1));
    m &= ((e >> b) & 1) ? on : ~on;
  }
  if (!live) m = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = __popcll(m & below);
  if (live && rank == 0) whist[wave * E + e] = __popcll(m);
  __syncthreads();
  for (int i = tid; i < E; i += 256) {
    const int c = whist[i] + whist[E + i] + whist[2 * E + i] + whist[3 * E + i];
    hist[i] = c;
    p.counts[i] = c;
  }
  if (live)
    for (int w = 0; w < wave; ++w) rank += whist[w * E + e];
  __syncthreads();
  const int total = block_exclusive_scan<256>(hist, E, wave_tot);
  for (int i = tid; i < E; i += 256) p.offsets[i] = hist[i];
  if (tid == 0) p.offsets[E] = total;
  if (live) {
    const int pos = hist[e] + rank;
    p.sorted[pos] = tid;
    p.inv[tid] = pos;
  }
}

// ----------------------------------------------------------------------------
// token-major down + combine (small T): workgroup (t, cb) computes y[t] for
// output columns [32*cb, 32*cb + 32).  Wave w takes the token's experts
// j = w, w+4, ... (NJ of them; past k it repeats the last expert and the
// result is unused, so no load is guarded by a branch), all of K, in groups
// of 4 chunks of 128.  The expert's h row is row 0 of the MFMA A operand (the
// other 15 rows are zero).  Each expert's output is rounded to bf16 (the
// y_perm value), then the workgroup sums them in top-k order in fp32 with the
// routing weights, adds the shared expert and rounds once.
// ----------------------------------------------------------------------------
constexpr int kTokCols = 32;

template <int FMT, int NJ>
__global__ __launch_bounds__(256) void dec_down_tok_kernel(DecArgs p) {
  extern __shared__ __attribute__((aligned(32))) uint16_t hs[];  // [k][I + 8]
  __shared__ float yp[kMaxK][kTokCols];
  __shared__ float ew[kMaxK];
  const FfnArgs& a = p.f;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int k = a.k, I = a.I, H = a.H, hp = I + 8;
  const int n_cb = H / kTokCols, t = blockIdx.x / n_cb, cb = blockIdx.x - t * n_cb;
  if (t == p.T) {  // the one extra workgroup: permutation outputs
    permute_block(p, reinterpret_cast<int*>(hs));
    return;
  }
  constexpr bool MX = FMT == MOE_W_MXFP4;
  uint8_t* mh = reinterpret_cast<uint8_t*>(hs);  // MXFP4: hi [k][I] | lo [k][I] | scales [k][I/32]
  uint8_t* ml = mh + (size_t)k * I;
  uint8_t* ms = ml + (size_t)k * I;
  uint8_t* mz = ms + (size_t)k * (I / 32);  // 32 zero bytes: A rows 1..15
  if (MX && tid < 8) reinterpret_cast<uint32_t*>(mz)[tid] = 0u;
  // One round trip for the token's k h rows (stored by assignment; the first
  // round of them in registers), its ids and weights.  Each wave reads the
  // ids of its own experts and issues their first weight loads before the h
  // rows are converted and staged, so the weight stream starts one round trip
  // after launch; the h loads, issued first, complete first.
  const uint16_t* hsrc = a.hbuf + (size_t)t * k * I;
  const int nh = k * (I / 8);
  uint4 hv[8];
  if constexpr (MX)
    prep_a_mx_load<256>(hsrc, k, I, I, 0, tid, *reinterpret_cast<uint4(*)[4]>(hv));
  else
    stage_load<256, 8>(hv, hsrc, I, k, I, 0);
  float w_v = 0.0f;
  if (tid < k) w_v = p.wts[t * k + tid];
  const uint8_t* rec[NJ];
  int jj[NJ];
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    jj[i] = min(wave + 4 * i, k - 1);
    const int id = __builtin_amdgcn_readfirstlane(p.ids[t * k + jj[i]]);
    const int slot = a.slot_of ? __builtin_amdgcn_readfirstlane(dbg_clamp(a.slot_of[id], a.E, kDbgSlot)) : id;
    rec[i] = a.base + (size_t)slot * a.stride;
  }
  const int nchunks = I / KC;
  BRaw<FMT> raw[NJ][2][4];
  // MXFP4: a lane's scale bytes of the 4 chunks (4 lane groups each) are 16
  // consecutive bytes of the row's scales, loaded at once
  uint4 s4[MX ? NJ : 1][2];
  auto issue = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NJ; ++i)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int row = cb * kTokCols + sub * 16 + l16;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (MX)
            raw[i][sub][u].q[0] = *reinterpret_cast<const uint4*>(
                rec[i] + a.off_w2 + (((size_t)row * I + (c0 + u) * KC + g * 32) >> 1));
          else
            load_b_raw<FMT>(rec[i] + a.off_w2, rec[i] + a.off_w2s, row, I, (c0 + u) * KC + g * 32,
                            raw[i][sub][u]);
        }
        if constexpr (MX)
          s4[i][sub] = *reinterpret_cast<const uint4*>(rec[i] + a.off_w2s + (size_t)row * (I / 32) +
                                                       c0 * 4);
      }
  };
  issue(0);
  if constexpr (MX) {
    prep_a_mx_store<256>(*reinterpret_cast<const uint4(*)[4]>(hv), k, I, 0, tid, mh, ml, ms);
    for (int i0 = 256 * 4; i0 < nh; i0 += 256 * 4) {  // k*I > 8192 only
      uint4 v[4];
      prep_a_mx_load<256>(hsrc, k, I, I, i0, tid, v);
      prep_a_mx_store<256>(v, k, I, i0, tid, mh, ml, ms);
    }
  } else {
    stage_store<256, 8>(hv, hs, hp, k, I, 0);
    for (int q0 = 256 * 8; q0 < nh; q0 += 256 * 8) {
      stage_load<256, 8>(hv, hsrc, I, k, I, q0);
      stage_store<256, 8>(hv, hs, hp, k, I, q0);
    }
  }
  if (tid < k) ew[tid] = w_v;
  __syncthreads();
  f32x4 acc[NJ][2];
#pragma unroll
  for (int i = 0; i < NJ; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0;;) {
#pragma unroll
    for (int i = 0; i < NJ; ++i) {
      if constexpr (MX) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u;
          // row 0 is the expert's h row; lanes of rows 1..15 read a zero block
          const int off = l16 == 0 ? jj[i] * I + c * KC + g * 32 : -1;
          const i32x8 ah = *reinterpret_cast<const i32x8*>(off < 0 ? mz : mh + off);
          const i32x8 al = *reinterpret_cast<const i32x8*>(off < 0 ? mz : ml + off);
          const int sa = off < 0 ? 127 : ms[jj[i] * (I / 32) + c * 4 + g];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const uint4 q = raw[i][sub][u].q[0];
            const i32x4 b = {(int)q.x, (int)q.y, (int)q.z, (int)q.w};
            const uint4 sv = s4[i][sub];
            const uint32_t d = u == 0 ? sv.x : u == 1 ? sv.y : u == 2 ? sv.z : sv.w;
            const int sb = (int)((d >> (8 * g)) & 0xffu);
            acc[i][sub] = mfma_mx(ah, b, sa, sb, acc[i][sub]);
            acc[i][sub] = mfma_mx(al, b, sa, sb, acc[i][sub]);
            pin(acc[i][sub]);
          }
        }
        continue;
      }
      const uint16_t* hrow = hs + jj[i] * hp;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        bf16x8 av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = *reinterpret_cast<const uint4*>(hrow + (c0 + u) * KC + g * 32 + q * 8);
          av[q] = l16 == 0 ? bits_to_bf16x8(v.x, v.y, v.z, v.w) : bits_to_bf16x8(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          bf16x8 b[4];
          decode_b<FMT>(raw[i][sub][u], b);
          if constexpr (FMT == MOE_W_FP8_B128) {
            f32x4 tt = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) tt = mfma16(av[q], b[q], tt);
            const float bs = block_scale<FMT>(raw[i][sub][u]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][sub][r] = fmaf(bs, tt[r], acc[i][sub][r]);
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][sub] = mfma16(av[q], b[q], acc[i][sub]);
          }
        }
      }
    }
    c0 += 4;
    if (c0 >= nchunks) break;
    issue(c0);
  }
  // row 0 of each expert's 16x16 result sits in lanes 0..15, element 0
#pragma unroll
  for (int i = 0; i < NJ; ++i) {
    const int j = wave + 4 * i;
    if (j < k && g == 0) {
      float tsd = 1.0f;
      if constexpr (FMT == MOE_W_NVFP4) tsd = reinterpret_cast<const float*>(rec[i] + a.off_ts)[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
        yp[j][sub * 16 + l16] = bf16_to_f32(f32_to_bf16_rne(acc[i][sub][0] * tsd));
    }
  }
  __syncthreads();
  if (tid < kTokCols) {
    const int col = cb * kTokCols + tid;
    float y = 0.0f;
    for (int j = 0; j < k; ++j) y = fmaf(ew[j], yp[j][tid], y);
    if (p.y_shared) y += bf16_to_f32(p.y_shared[(size_t)t * H + col]);
    p.y[(size_t)t * H + col] = f32_to_bf16_rne(y);
  }
}

// ----------------------------------------------------------------------------
// fused token-major layer (MXFP4 weights, small T).  Workgroup u (16 waves)
// serves unit (t, j, q), u = t + T*(j + k*q): token t, its expert slot j and
// the 128 h-columns [128q, 128q + 128).  It routes token t itself (wave 0,
// rounds 0..j), computes those h-columns in full and then their share of the
// down projection for every output column:
//   gate/up: wave w owns h-columns 128q + 8w .. + 8; the MFMA's 16 B columns
//            are their 8 gate rows (lanes 0..7) and 8 up rows (lanes 8..15),
//            all of K (H/128 chunks); the token's x row is A row 0;
//   h:       SiLU(gate)*up, rounded to bf16, split into E4M3 hi + lo with an
//            E8M0 scale per 32 (one K chunk of the down projection);
//   down:    wave w owns output rows [w*H/16, (w+1)*H/16), K = the slice;
//            fp32 partial outputs go to part[(t*k + j)*(I/128) + q][H].
// The slice's down weights are loaded while the second half of the gate/up
// chunks is computed, so the workgroup's loads form one stream; the layer
// is one weight stream over the whole chip instead of two launches' worth.
// Workgroup 0 also routes all T tokens (one wave each) and writes ids,
// weights, counts, offsets, sorted_idx and inv_idx while its loads fly.
// dec_fused_combine_kernel then sums each expert's partials (q ascending),
// rounds to bf16 (the y_perm value) and combines in top-k order.
// ----------------------------------------------------------------------------
constexpr int kFuWaves = 16, kFuSlice = 128, kFuMinUnits = 256;

// NC = H/128 gate/up chunks per wave, NS = H/256 down subtiles per wave.
template <int NC, int VPL>
__global__ __launch_bounds__(1024) void dec_fused_tok_kernel(DecArgs p) {
  static_assert(NC % 4 == 0, "H is a multiple of 512");
  constexpr int NS = NC / 2, NSV = NC / 4;
  const FfnArgs& a = p.f;
  __shared__ __attribute__((aligned(32))) uint8_t mx[2 * kTokMaxH + kTokMaxH / 32 + 32];
  __shared__ __attribute__((aligned(32))) uint8_t hx[2 * kFuSlice + 32];
  __shared__ __attribute__((aligned(16))) uint16_t hb[kFuSlice];
  __shared__ float gu[kFuWaves][16];
  __shared__ int eslot[kMaxK];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = p.T, k = a.k, E = a.E, H = a.H, I = a.I, Q = I / kFuSlice;
  const int u = (int)blockIdx.x, t = u % T, r_ = u / T, j = r_ % k, q = r_ / k;
  uint8_t *mh = mx, *ml = mx + kTokMaxH, *ms = mx + 2 * kTokMaxH;
  uint8_t* mz = ms + kTokMaxH / 32;  // 32 zero bytes: A rows 1..15
  uint8_t *hh = hx, *hl = hx + kFuSlice, *hs = hx + 2 * kFuSlice;  // h slice: hi, lo, 4 scales
  if (tid < 8) reinterpret_cast<uint32_t*>(mz)[tid] = 0u;
  // one round trip: (wave 0) the token's logits row; waves 1..15 split its x row
  // Workgroup 0 also routes every token (wave w: token w) and writes the
  // routing and permutation outputs while its weight loads are in flight; its
  // waves < T load their logits rows now, with the rest of the prologue.
  const bool writer = u == 0;
  float lv[VPL];
  if (wave == 0 || (writer && wave < T))
    route_load<VPL>(p.logits + (size_t)(wave == 0 ? t : wave) * E, E, lane, lv);
  if (wave > 0)
    prep_a_mx<(kFuWaves - 1) * 64>(a.x + (size_t)t * H, 1, H, H, mh, ml, ms, tid - 64);
  TopK<VPL> st;
  if (wave == 0) {
    topk_begin<VPL>(lv, E, lane, st);
    for (int r = 0; r <= j; ++r) topk_round<VPL>(st, r, lane);
    if (lane == j) eslot[0] = a.slot_of ? dbg_clamp(a.slot_of[st.id_r], a.E, kDbgSlot) : st.id_r;
  }
  __syncthreads();
  const uint8_t* rec = a.base + (size_t)eslot[0] * a.stride;
  // gate/up loads: chunk c of B column l16, and the row's H/32 scale bytes
  const int hcol = q * kFuSlice + wave * 8 + (l16 & 7);
  const int wrow = (l16 < 8 ? 0 : I) + hcol;
  const uint8_t* wp = rec + a.off_w13 + (size_t)wrow * (H / 2) + g * 16;
  const uint8_t* sp = rec + a.off_w13s + (size_t)wrow * (H / 32);
  // scales first: loads complete in issue order, and chunk 0 needs its scale
  uint4 w[NC];
  uint4 sv[NSV];
#pragma unroll
  for (int i = 0; i < NSV; ++i) sv[i] = *reinterpret_cast<const uint4*>(sp + 16 * i);
#pragma unroll
  for (int c = 0; c < NC; ++c) w[c] = *reinterpret_cast<const uint4*>(wp + c * (KC / 2));
  if (writer) {
    __shared__ int pid[kDA];
    if (wave < T) {  // wave 0 has token 0's rounds 0..j (j = 0) done
      if (wave > 0) {
        topk_begin<VPL>(lv, E, lane, st);
        topk_round<VPL>(st, 0, lane);
      }
      for (int r = 1; r < k; ++r) topk_round<VPL>(st, r, lane);
      const float wv = topk_weight<VPL>(st, lv, E, k, p.renorm, lane);
      if (lane < k) {
        p.ids[wave * k + lane] = st.id_r;
        p.wts[wave * k + lane] = wv;
        pid[wave * k + lane] = st.id_r;
      }
    }
    __syncthreads();
    // stable counting sort by expert, brute force over the A <= 256 ids
    const int A = T * k;
    for (int e = tid; e < E; e += 1024) {
      int cnt = 0, below = 0;
      for (int i = 0; i < A; ++i) {
        const int v = pid[i];
        cnt += v == e;
        below += v < e;
      }
      p.counts[e] = cnt;
      p.offsets[e] = below;
    }
    if (tid == 0) p.offsets[E] = A;
    if (tid < A) {
      const int e = pid[tid];
      int pos = 0;
      for (int i = 0; i < A; ++i) {
        const int v = pid[i];
        pos += v < e || (v == e && i < tid);
      }
      p.sorted[pos] = tid;
      p.inv[tid] = pos;
    }
  }
  uint4 w2[NS];
  uint32_t s2[NS];
  const int drow0 = wave * (H / kFuWaves) + l16;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c == NC / 2) {  // the slice's down weights, behind the first half of the chunks
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int row = drow0 + s * 16;
        w2[s] = *reinterpret_cast<const uint4*>(rec + a.off_w2 + (size_t)row * (I / 2) +
                                                q * (kFuSlice / 2) + g * 16);
        s2[s] = *reinterpret_cast<const uint32_t*>(rec + a.off_w2s + (size_t)row * (I / 32) +
                                                   q * 4);
      }
    }
    // A row 0 is the token; lanes of rows 1..15 read a zero block (scale 1)
    const int off = l16 == 0 ? c * KC + g * 32 : -1;
    const i32x8 ah = *reinterpret_cast<const i32x8*>(off < 0 ? mz : mh + off);
    const i32x8 al = *reinterpret_cast<const i32x8*>(off < 0 ? mz : ml + off);
    const int sa = off < 0 ? 127 : ms[c * 4 + g];
    const uint4 sq = sv[c / 4];
    const uint32_t d = (c & 3) == 0 ? sq.x : (c & 3) == 1 ? sq.y : (c & 3) == 2 ? sq.z : sq.w;
    const int sb = (int)((d >> (8 * g)) & 0xffu);
    const i32x4 bq = {(int)w[c].x, (int)w[c].y, (int)w[c].z, (int)w[c].w};
    acc = mfma_mx(ah, bq, sa, sb, acc);
    acc = mfma_mx(al, bq, sa, sb, acc);
    pin(acc);
  }
  // row 0 of the 16x16 result: lanes 0..15, element 0 (gate in 0..7, up in 8..15)
  if (g == 0) gu[wave][l16] = acc[0];
  __syncthreads();
  if (tid < kFuSlice) {
    const float gv = gu[tid >> 3][tid & 7], uv = gu[tid >> 3][8 + (tid & 7)];
    hb[tid] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
  }
  __syncthreads();
  if (wave == 0) {  // the h slice as one A row of the down MFMA (16 pieces of 8)
    uint4 v[4] = {};
    if (lane < kFuSlice / 8) v[0] = reinterpret_cast<const uint4*>(hb)[lane];
    prep_a_mx_store<64>(v, 1, kFuSlice, 0, lane, hh, hl, hs);
  }
  __syncthreads();
  const int offh = l16 == 0 ? g * 32 : -1;
  const i32x8 dh = *reinterpret_cast<const i32x8*>(offh < 0 ? mz : hh + offh);
  const i32x8 dl = *reinterpret_cast<const i32x8*>(offh < 0 ? mz : hl + offh);
  const int sd = offh < 0 ? 127 : hs[g];
  float* out = p.part + ((size_t)(t * k + j) * Q + q) * H;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const i32x4 bq = {(int)w2[s].x, (int)w2[s].y, (int)w2[s].z, (int)w2[s].w};
    const int sb = (int)((s2[s] >> (8 * g)) & 0xffu);
    f32x4 y4 = f32x4{0.f, 0.f, 0.f, 0.f};
    y4 = mfma_mx(dh, bq, sd, sb, y4);
    y4 = mfma_mx(dl, bq, sd, sb, y4);
    pin(y4);  // keeps the MFMAs (and their operands) out of the g == 0 branch: every lane feeds them
    if (g == 0) out[drow0 + s * 16] = y4[0];
  }
}

// y[t] = bf16( sum_j w_tj * bf16( sum_q part[t, j, q] ) (+ y_shared[t]) ), sums
// in q then j order.  Workgroup (t, 64 columns): thread (j, column pair) sums
// one expert's partials for two columns (all its loads in one round trip),
// then 64 threads combine the experts in top-k order.
constexpr int kFuCols = 64;

__global__ __launch_bounds__(256) void dec_fused_combine_kernel(DecArgs p) {
  const int k = p.f.k, H = p.f.H, Q = p.f.I / kFuSlice, n_cb = H / kFuCols;
  __shared__ float ew[kMaxK];
  __shared__ float yp[kMaxK][kFuCols];
  const int tid = threadIdx.x, t = blockIdx.x / n_cb;
  const int c0 = (blockIdx.x - t * n_cb) * kFuCols, pr = tid & 31;
  // the routing weight is loaded with the partials (one round trip), stored after
  const float wv = tid < k ? p.wts[t * k + tid] : 0.0f;
  for (int jj = tid >> 5; jj < k; jj += 8) {
    const float* src = p.part + (size_t)(t * k + jj) * Q * H + c0 + 2 * pr;
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll 4
    for (int qq = 0; qq < Q; ++qq) {
      const float2 v = *reinterpret_cast<const float2*>(src + (size_t)qq * H);
      s0 += v.x;
      s1 += v.y;
    }
    yp[jj][2 * pr] = bf16_to_f32(f32_to_bf16_rne(s0));
    yp[jj][2 * pr + 1] = bf16_to_f32(f32_to_bf16_rne(s1));
  }
  if (tid < k) ew[tid] = wv;
  __syncthreads();
  if (tid < kFuCols) {
    const int c = c0 + tid;
    float y = 0.0f;
    for (int jj = 0; jj < k; ++jj) y = fmaf(ew[jj], yp[jj][tid], y);
    if (p.y_shared) y += bf16_to_f32(p.y_shared[(size_t)t * H + c]);
    p.y[(size_t)t * H + c] = f32_to_bf16_rne(y);
  }
}

static int g_cus = 0;

// Raise a kernel's dynamic-LDS limit once (the largest request so far is kept).
template <typename K>
static bool lds_ok(K kern, size_t dyn_bytes, size_t& granted) {
  if (dyn_bytes <= granted) return true;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_bytes) != hipSuccess)
    return false;
  granted = dyn_bytes;
  return true;
}

template <int FMT, int CPW>
static int launch_gateup(const DecArgs& p, hipStream_t s) {
  const size_t x_lds = (size_t)p.T * (p.f.H + 8) * 2;
  static size_t granted = 0, occ_for = 0;
  static int per_cu = 0;
  auto k = dec_gateup_kernel<FMT, CPW>;
  if (!lds_ok(k, x_lds, granted)) return set_error(MOE_ERR_HIP, "moe_forward_decode: LDS attribute");
  if (occ_for != x_lds) {  // persistent grid: as many workgroups as fit on the device at once
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), 256,
                                                     x_lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    occ_for = x_lds;
  }
  k<<<per_cu * g_cus, 256, x_lds, s>>>(p);
  return MOE_OK;
}

template <int FMT, int CPW, int VPL>
static int launch_gateup_tok(const DecArgs& p, hipStream_t s) {
  static int per_cu = 0;
  auto k = dec_gateup_tok_kernel<FMT, CPW, VPL>;
  if (!per_cu &&
      (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), 256,
                                                    0) != hipSuccess || per_cu < 1))
    per_cu = 1;
  // a multiple of T, so that every workgroup serves one token
  const int G = p.T * ((per_cu * g_cus) / p.T > 0 ? (per_cu * g_cus) / p.T : 1);
  k<<<G, 256, 0, s>>>(p);
  return MOE_OK;
}

template <int FMT, int CPW>
static int launch_down(const DecArgs& p, hipStream_t s) {
  static int per_cu = 0;
  auto k = dec_down_kernel<FMT, CPW>;
  if (!per_cu &&
      (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k), 256,
                                                    0) != hipSuccess || per_cu < 1))
    per_cu = 1;
  k<<<per_cu * g_cus, 256, 0, s>>>(p.f);
  return MOE_OK;
}

// One workgroup per (token, 32 columns) plus one for the permutation outputs.
template <int FMT, int NJ>
static int launch_down_tok(const DecArgs& p, hipStream_t s) {
  const size_t h_lds = FMT == MOE_W_MXFP4 ? (size_t)p.f.k * (2 * p.f.I + p.f.I / 32) + 32
                                           : (size_t)p.f.k * (p.f.I + 8) * 2;
  const size_t perm_lds = ((size_t)5 * p.f.E + kMaxE + 16) * 4;
  const size_t lds = h_lds > perm_lds ? h_lds : perm_lds;
  static size_t granted = 0;
  auto k = dec_down_tok_kernel<FMT, NJ>;
  if (!lds_ok(k, lds, granted)) return set_error(MOE_ERR_HIP, "moe_forward_decode: LDS attribute");
  k<<<p.T * (p.f.H / kTokCols) + 1, 256, lds, s>>>(p);
  return MOE_OK;
}

// Small batches (T <= 16, H <= 2048) take the token-major path: two launches,
// no permutation on the critical path (few experts are shared by its tokens).
static bool token_major(int T, int H) { return T <= kTokMaxT && H <= kTokMaxH; }

template <int FMT, int CPW>
static int launch_gateup_tok_vpl(const DecArgs& p, hipStream_t s) {
  return p.f.E <= 256 ? launch_gateup_tok<FMT, CPW, 4>(p, s) : launch_gateup_tok<FMT, CPW, 16>(p, s);
}

// The fused path: MXFP4 weights, E <= 256 (routing state in few registers),
// token-major shapes whose units fill the chip's compute units (256 on
// MI355X, one unit each) in whole rounds: a partial last round would cost a
// whole round.
static bool fused_path(int fmt, int E, int T, int k, int H, int I) {
  const int U = T * k * (I / kFuSlice);
  return fmt == MOE_W_MXFP4 && E <= 256 && token_major(T, H) && I % kFuSlice == 0 &&
         H % 512 == 0 && U >= kFuMinUnits && U % kFuMinUnits == 0;
}

template <int NC>
static int launch_fused_nc(const DecArgs& p, hipStream_t s) {
  const int U = p.T * p.f.k * (p.f.I / kFuSlice);
  dec_fused_tok_kernel<NC, 4><<<U, 1024, 0, s>>>(p);  // E <= 256: 4 logits per lane
  return MOE_OK;
}

static int launch_fused(const DecArgs& p, hipStream_t s) {
  int st;
  switch (p.f.H / 128) {
    case 4: st = launch_fused_nc<4>(p, s); break;
    case 8: st = launch_fused_nc<8>(p, s); break;
    case 12: st = launch_fused_nc<12>(p, s); break;
    default: st = launch_fused_nc<16>(p, s); break;
  }
  if (st) return st;
  dec_fused_combine_kernel<<<p.T * (p.f.H / kFuCols), 256, 0, s>>>(p);
  return check_launch("moe_forward_decode");
}

// K chunks per wave: H / 512 for gate/up, I / 512 for the tile-major down
template <int FMT>
static int launch_decode(DecArgs& p, hipStream_t s) {
  int st;
  if (fused_path(FMT, p.f.E, p.T, p.f.k, p.f.H, p.f.I)) return launch_fused(p, s);
  if (token_major(p.T, p.f.H)) {
    switch (p.f.H / 512) {
      case 1: st = launch_gateup_tok_vpl<FMT, 1>(p, s); break;
      case 2: st = launch_gateup_tok_vpl<FMT, 2>(p, s); break;
      case 3: st = launch_gateup_tok_vpl<FMT, 3>(p, s); break;
      default: st = launch_gateup_tok_vpl<FMT, 4>(p, s); break;
    }
    if (st) return st;
    switch ((p.f.k + 3) / 4) {
      case 1: st = launch_down_tok<FMT, 1>(p, s); break;
      case 2: st = launch_down_tok<FMT, 2>(p, s); break;
      case 3: st = launch_down_tok<FMT, 3>(p, s); break;
      default: st = launch_down_tok<FMT, 4>(p, s); break;
    }
    if (st) return st;
    return check_launch("moe_forward_decode");
  }
  const int rp = moe_route_permute(p.logits, p.T, p.f.E, p.f.k, p.renorm, p.ids, p.wts, p.counts,
                                   p.offsets, p.sorted, p.inv, nullptr, 0,
                                   reinterpret_cast<moe_stream_t>(s));
  if (rp) return rp;
  switch (p.f.H / 512) {
    case 1: st = launch_gateup<FMT, 1>(p, s); break;
    case 2: st = launch_gateup<FMT, 2>(p, s); break;
    case 3: st = launch_gateup<FMT, 3>(p, s); break;
    default: st = launch_gateup<FMT, 4>(p, s); break;
  }
  if (st) return st;
  switch (p.f.I / 512) {
    case 1: st = launch_down<FMT, 1>(p, s); break;
    case 2: st = launch_down<FMT, 2>(p, s); break;
    case 3: st = launch_down<FMT, 3>(p, s); break;
    default: st = launch_down<FMT, 4>(p, s); break;
  }
  if (st) return st;
  if ((st = check_launch("moe_forward_decode"))) return st;
  return moe_combine(p.f.y_perm, p.inv, p.wts, p.T, p.f.k, p.f.H, p.y_shared, p.y,
                     reinterpret_cast<moe_stream_t>(s));
}

#ifdef MOE_DEBUG
uint32_t dbg_take_decode() { return dbg_take_unit(); }
#endif

}  // namespace moe

using namespace moe;

static size_t dec_align(size_t v) { return (v + 255) / 256 * 256; }

// Workspace: h [A][I] bf16 | y_perm [A][H] bf16 (| fused path: down partials
// [A][I/128][H] fp32).
static size_t dec_ws_bytes(int fmt, int E, int H, int I, int T, int k) {
  const size_t A = (size_t)T * k;
  size_t n = dec_align(A * I * 2) + dec_align(A * H * 2);
  if (fused_path(fmt, E, T, k, H, I)) n += dec_align(A * (I / kFuSlice) * H * 4);
  return n;
}

// Enough for every batch of at most T tokens: the partials exist only for the
// batch sizes that take the one-stream path (some T' <= 16), so the size is
// the largest over T' <= T.
extern "C" size_t moe_forward_decode_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W || T < 0 || k < 1) return 0;
  size_t n = dec_ws_bytes(W->fmt, W->E, W->H, W->I, T, k);
  for (int t2 = 1; t2 <= T && t2 <= kTokMaxT; ++t2) {
    const size_t m = dec_ws_bytes(W->fmt, W->E, W->H, W->I, t2, k);
    n = m > n ? m : n;
  }
  return n;
}

extern "C" int moe_forward_decode(const moe_experts* W, const int32_t* slot_of_expert,
                                  const float* logits, const uint16_t* x, int32_t T, int32_t k,
                                  int32_t renorm, int32_t* topk_ids, float* topk_w,
                                  int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                                  int32_t* inv_idx, const uint16_t* y_shared, uint16_t* y,
                                  void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (!W) return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode: W is NULL");
  Layout Lo;
  if (W->E < 1 || W->E > kMaxE || !layout_of(W->fmt, W->H, W->I, &Lo))
    return set_error(MOE_ERR_UNSUPPORTED, "moe_forward_decode: fmt=%d E=%d H=%d I=%d", W->fmt,
                     W->E, W->H, W->I);
  if (!W->base || !aligned16(W->base) || W->stride < Lo.stride || W->stride % 256)
    return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode: base/stride");
  if (T < 0 || k < 1 || k > W->E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode: need T>=0, 1<=k<=min(E,%d)", kMaxK);
  if (!moe_forward_decode_supported(W->H, W->I, T, k))
    return set_error(MOE_ERR_UNSUPPORTED,
                     "moe_forward_decode: T=%d k=%d H=%d I=%d outside the decode limits", T, k,
                     W->H, W->I);
  if (T == 0) return MOE_OK;
  const void* ptrs[] = {logits, x, topk_ids, topk_w, counts, offsets, sorted_idx, inv_idx, y, ws};
  for (const void* q : ptrs)
    if (!q || !aligned16(q)) return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode: pointer");
  if ((y_shared && !aligned16(y_shared)) || (slot_of_expert && !aligned16(slot_of_expert)))
    return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode: pointer");
  if (ws_bytes < moe_forward_decode_workspace(W, T, k))
    return set_error(MOE_ERR_WORKSPACE, "moe_forward_decode: workspace %zu too small", ws_bytes);
  if (!g_cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return set_error(MOE_ERR_HIP, "moe_forward_decode: device query failed");
    g_cus = n;
  }
  DecArgs p;
  FfnArgs& f = p.f;
  f.E = W->E; f.H = W->H; f.I = W->I; f.k = k; f.A = T * k;
  f.base = static_cast<const uint8_t*>(W->base);
  f.stride = W->stride;
  f.slot_of = slot_of_expert;
  f.off_w13 = Lo.w13; f.off_w13s = Lo.w13s < 0 ? 0 : Lo.w13s;
  f.off_w2 = Lo.w2; f.off_w2s = Lo.w2s < 0 ? 0 : Lo.w2s;
  f.off_ts = Lo.ts < 0 ? 0 : Lo.ts;
  f.x = x;
  f.counts = counts; f.offsets = offsets; f.sorted_idx = sorted_idx;
  const size_t A = (size_t)T * k;
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  f.hbuf = reinterpret_cast<uint16_t*>(wsb);
  f.y_perm = reinterpret_cast<uint16_t*>(wsb + dec_align(A * W->I * 2));
  p.part = fused_path(W->fmt, W->E, T, k, W->H, W->I)
               ? reinterpret_cast<float*>(wsb + dec_align(A * W->I * 2) + dec_align(A * W->H * 2))
               : nullptr;
  p.logits = logits;
  p.T = T;
  p.renorm = renorm;
  p.ids = topk_ids; p.wts = topk_w; p.counts = counts; p.offsets = offsets;
  p.sorted = sorted_idx; p.inv = inv_idx;
  p.y_shared = y_shared;
  p.y = y;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  switch (W->fmt) {
    case MOE_W_BF16: return launch_decode<MOE_W_BF16>(p, s);
    case MOE_W_MXFP4: return launch_decode<MOE_W_MXFP4>(p, s);
    case MOE_W_NVFP4: return launch_decode<MOE_W_NVFP4>(p, s);
    default: return launch_decode<MOE_W_FP8_B128>(p, s);
  }
}

extern "C" int moe_forward_decode_supported(int32_t H, int32_t I, int32_t T, int32_t k) {
  // routing in one workgroup; the units hold K/512 chunks of 128 per wave
  // (H and I in {512, 1024, 1536, 2048}); gate/up keeps the batch's x in LDS
  if (T < 0 || k < 1 || T > kDT || T * k > kDA) return 0;
  if (H % 512 || I % 512 || H > 2048 || I > 2048 || H < 512 || I < 512) return 0;
  const size_t gu_lds = (size_t)T * (H + 8) * 2 + sizeof(TileTable) + sizeof(f32x4) * 4 * 4 * 64 +
                        sizeof(int) * kDA;
  return gu_lds <= 160 * 1024;  // the token-major down's h rows (k <= 16) always fit
}

// ---------------------------------------------------------------------------
// moe_forward_decode_noalloc: the same layer call with its scratch (h, y_perm
// and the one-stream path's fp32 partials) in a fixed array of device memory
// that every GPU holds for the life of the process, for callers that cannot
// allocate (graph capture, tight serving loops).  The array's host-side name
// is only a stand-in: its device address is looked up once per device with
// hipGetSymbolAddress and that pointer is what the kernels receive.
// ---------------------------------------------------------------------------
#include <mutex>

static constexpr size_t kNoAllocScratchBytes = 8u << 20;
static constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
static std::mutex g_scratch_mu;
static void* g_scratch_dev[kNoAllocMaxDevices] = {};

static int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices)
    return set_error(MOE_ERR_HIP, "moe_forward_decode_noalloc: no current device (or index >= %d)",
                     kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return set_error(MOE_ERR_HIP, "moe_forward_decode_noalloc: hipGetSymbolAddress: %s",
                       hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

extern "C" size_t moe_forward_decode_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

extern "C" int moe_forward_decode_noalloc(const moe_experts* W, const int32_t* slot_of_expert,
                                          const float* logits, const uint16_t* x, int32_t T,
                                          int32_t k, int32_t renorm, int32_t* topk_ids,
                                          float* topk_w, int32_t* counts, int32_t* offsets,
                                          int32_t* sorted_idx, int32_t* inv_idx,
                                          const uint16_t* y_shared, uint16_t* y,
                                          moe_stream_t stream) {
  if (!W) return set_error(MOE_ERR_INVALID_ARG, "moe_forward_decode_noalloc: W is NULL");
  const size_t need = moe_forward_decode_workspace(W, T, k);
  if (need > kNoAllocScratchBytes)
    return set_error(MOE_ERR_WORKSPACE,
                     "moe_forward_decode_noalloc: T=%d k=%d H=%d I=%d needs %zu bytes of scratch; "
                     "the static scratch holds %zu (use moe_forward_decode with a workspace)",
                     T, k, W->H, W->I, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  const int st = scratch_of_current_device(&ws);
  if (st) return st;
  return moe_forward_decode(W, slot_of_expert, logits, x, T, k, renorm, topk_ids, topk_w, counts,
                            offsets, sorted_idx, inv_idx, y_shared, y, ws, kNoAllocScratchBytes,
                            stream);
}
