// The MoE layer for decode-sized batches in three launches.  Kernel
// boundaries are the only synchronisation between workgroups.
//
//  1. route + permute: one workgroup (route_permute_small_kernel).
//  2. gate/up: a persistent grid sized by occupancy.  Each workgroup builds the
//     16-row tile list in LDS from counts/offsets (one round trip) and then
//     takes units u = blockIdx.x, +gridDim.x, ... (unit = one tile x 32
//     h-columns, K split over the 4 waves).  The weight loads of the next unit
//     are issued before the current unit is computed (two register buffers,
//     alternated without copies), so HBM requests never stop; the few
//     activation rows of a unit come from L2 while its weights are decoded.
//  3. down + combine: workgroup b owns output columns [b*NCOL, b*NCOL+NCOL) of
//     y for every token.  Its waves first issue the W2 loads of that column
//     slice for all their tiles, then stage every h row in LDS (overlapping
//     the weight fetch), compute y_perm of the slice into LDS and finish with
//     the weighted combine of the slice.  No data crosses workgroups inside a
//     launch.
//
// Per-element arithmetic (K split, MFMA order, bf16 rounding of h and y_perm,
// combine order) is that of the decode kernels of moe_expert_ffn and of
// moe_combine, so the results are bit-identical to the separate calls.
#include "ffn_common.h"
#include "route_common.h"

namespace moe {

constexpr int kDT = 64, kDA = 256, kDTiles = 256;
constexpr int kDGuCols = 32;  // gate/up unit: 16 + 16 h-columns (2 gate + 2 up subtiles)

struct DecArgs {
  FfnArgs f;
  const float* logits;
  int T, renorm, h_pitch;
  int* ids;
  float* wts;
  int* counts;
  int* offsets;
  int* sorted;
  int* inv;
  const uint16_t* y_shared;
  uint16_t* y;
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
    }
  }
  if (a.slot_of) {
#pragma unroll
    for (int i = 0; i < kMaxE / NT; ++i) {
      const int e = threadIdx.x + i * NT;
      if (e < a.E) r.s[i] = a.slot_of[e];
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
// gate/up
// ----------------------------------------------------------------------------
// CPW = K chunks of 128 per wave (H = 512 * CPW): a compile-time count, so a
// load and its use are never guarded by separate runtime branches (which
// would make the compiler wait for loads still needed later).
template <int FMT, int CPW>
struct GuRaw {
  BRaw<FMT> r[CPW][4];  // [chunk slot][subtile]
};

template <int FMT, int CPW>
__device__ __forceinline__ void gu_issue(const FfnArgs& a, const TileTable& L, int unit, int n_gu,
                                         GuRaw<FMT, CPW>& R) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int tile = unit / n_gu, cb = unit - tile * n_gu;
  const uint8_t* rec = tile_record(a, L, tile);
  const uint8_t* w = rec + a.off_w13;
  const uint8_t* sc = rec + a.off_w13s;
  const int n0 = cb * kDGuCols;
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = wave + 4 * u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_b_raw<FMT>(w, sc, (j < 2 ? n0 : a.I + n0) + (j & 1) * 16 + l16, a.H, c * KC + g * 32,
                      R.r[u][j]);
  }
}

// x rows come from LDS (xs, pitch xp); sidx holds sorted_idx.  The only global
// loads of a unit are its weights, so waiting for them never waits for the
// next unit's weights, which were issued later.
template <int FMT, int CPW>
__device__ __forceinline__ void gu_finish(const FfnArgs& a, const TileTable& L, const int* sidx,
                                          const uint16_t* xs, int xp, f32x4 (&red)[4][4][64],
                                          int unit, int n_gu, const GuRaw<FMT, CPW>& R) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar branches
  const int tile = unit / n_gu, cb = unit - tile * n_gu;
  const int e = L.tile_e[tile], m0 = L.tile_m0[tile];
  const int rows = min(16, L.cnt[e] - m0), seg0 = L.off[e] + m0;
  const int n0 = cb * kDGuCols;
  const uint16_t* arow = l16 < rows ? xs + (sidx[seg0 + l16] / a.k) * xp : nullptr;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = wave + 4 * u;
    {
      bf16x8 av[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        av[q] = arow ? *reinterpret_cast<const bf16x8*>(arow + c * KC + g * 32 + q * 8)
                     : bits_to_bf16x8(0u, 0u, 0u, 0u);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 b[4];
        decode_b<FMT>(R.r[u][j], b);
        if constexpr (FMT == MOE_W_FP8_B128) {
          f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; ++q) t = mfma16(av[q], b[q], t);
          const float bs = block_scale<FMT>(R.r[u][j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[j][r] = fmaf(bs, t[r], acc[j][r]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[j] = mfma16(av[q], b[q], acc[j]);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  if (wave < 2) {
    f32x4 gs = red[0][wave][lane], us = red[0][2 + wave][lane];
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const f32x4 gq = red[q][wave][lane], uq = red[q][2 + wave][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        gs[r] += gq[r];
        us[r] += uq[r];
      }
    }
    float tsg = 1.0f, tsu = 1.0f;
    if constexpr (FMT == MOE_W_NVFP4) {
      const float* ts = reinterpret_cast<const float*>(tile_record(a, L, tile) + a.off_ts);
      tsg = ts[0];
      tsu = ts[1];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = g * 4 + r;
      if (m < rows) {
        const float gv = gs[r] * tsg, uv = us[r] * tsu;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        a.hbuf[(size_t)(seg0 + m) * a.I + n0 + wave * 16 + l16] = f32_to_bf16_rne(hv);
      }
    }
  }
  __syncthreads();  // red is rewritten by the next unit
}

template <int FMT, int CPW>
__global__ __launch_bounds__(256) void dec_gateup_kernel(FfnArgs a, int T) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];  // [T][H + 8]
  __shared__ TileTable L;
  __shared__ f32x4 red[4][4][64];
  __shared__ int sidx[kDA];
  const int xp = a.H + 8, tid = threadIdx.x;
  // one round trip: x rows, sorted_idx, counts/offsets/slot table
  uint4 xv[8];
  stage_load<256, 8>(xv, a.x, a.H, T, a.H, 0);
  const int sid = tid < a.A ? a.sorted_idx[tid] : 0;
  TileRegs<256> tr;
  tiles_load<256>(a, tr);
  stage_store<256, 8>(xv, xs, xp, T, a.H, 0);
  for (int q0 = 256 * 8; q0 < T * (a.H / 8); q0 += 256 * 8) {  // x beyond 32 KB
    stage_load<256, 8>(xv, a.x, a.H, T, a.H, q0);
    stage_store<256, 8>(xv, xs, xp, T, a.H, q0);
  }
  if (tid < a.A) sidx[tid] = sid;
  const int n_tiles = tiles_build<256>(a, tr, L);  // its barriers publish xs and sidx
  const int n_gu = a.I / kDGuCols, U1 = n_tiles * n_gu, G = (int)gridDim.x;
  // Units go in pairs: both pairs' weights are issued before the first is
  // computed.  Nothing stays in flight across iterations, so no register
  // holding a pending load is ever copied (a copy would wait for the load).
  GuRaw<FMT, CPW> ra, rb;
  for (int u = blockIdx.x; u < U1; u += 2 * G) {
    gu_issue<FMT, CPW>(a, L, u, n_gu, ra);
    if (u + G < U1) {
      gu_issue<FMT, CPW>(a, L, u + G, n_gu, rb);
      gu_finish<FMT, CPW>(a, L, sidx, xs, xp, red, u, n_gu, ra);
      gu_finish<FMT, CPW>(a, L, sidx, xs, xp, red, u + G, n_gu, rb);
    } else {
      gu_finish<FMT, CPW>(a, L, sidx, xs, xp, red, u, n_gu, ra);
    }
  }
}

// ----------------------------------------------------------------------------
// down + combine, one column slice of y per workgroup (8 waves)
// ----------------------------------------------------------------------------
struct K2Extra {
  int inv[kDA];
  float w[kDA];
};

constexpr int kK2Threads = 512, kK2Waves = kK2Threads / 64;
// tiles of one wave whose weight loads are in flight together (register budget)
template <int FMT>
constexpr int k2_tiles() {
  return FMT == MOE_W_BF16 ? 2 : FMT == MOE_W_FP8_B128 ? 4 : 8;
}

template <int FMT, int NCOL, int MT>
__device__ __forceinline__ void k2_issue(const FfnArgs& a, const TileTable& L, int n_tiles, int t0,
                                         int c0, int n0, BRaw<FMT> (&raw)[MT][4]) {
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int nchunks = a.I / KC;
#pragma unroll
  for (int s = 0; s < MT; ++s) {
    const int tile = t0 + kK2Waves * s;
    if (tile < n_tiles) {
      const uint8_t* rec = tile_record(a, L, tile);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (c0 + u < nchunks) {
          if (l16 < NCOL)
            load_b_raw<FMT>(rec + a.off_w2, rec + a.off_w2s, n0 + l16, a.I, (c0 + u) * KC + g * 32,
                            raw[s][u]);
          else
            raw[s][u] = BRaw<FMT>{};
        }
      }
    }
  }
}

template <int FMT, int NCOL>
__global__ __launch_bounds__(kK2Threads) void dec_down_combine_kernel(DecArgs p) {
  constexpr int MT = k2_tiles<FMT>();
  extern __shared__ __attribute__((aligned(16))) uint16_t dyn[];
  __shared__ TileTable L;
  __shared__ K2Extra X;
  const FfnArgs& a = p.f;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int T = p.T, k = a.k, A = T * k, I = a.I, H = a.H;
  uint16_t* hs = dyn;                          // [A][h_pitch]
  uint16_t* yp = dyn + (size_t)A * p.h_pitch;  // [A][NCOL]

  // inv/weights and the tile table in one round trip
  int inv_v = 0;
  float w_v = 0.0f;
  if (tid < A) {
    inv_v = p.inv[tid];
    w_v = p.wts[tid];
  }
  TileRegs<kK2Threads> tr;
  tiles_load<kK2Threads>(a, tr);
  if (tid < A) {
    X.inv[tid] = inv_v;
    X.w[tid] = w_v;
  }
  const int n_tiles = tiles_build<kK2Threads>(a, tr, L);
  const int n0 = blockIdx.x * NCOL, nchunks = I / KC;
  // the first weight group of every wave goes out before the h rows are
  // staged; the staging then waits for both, which arrive together
  BRaw<FMT> raw[MT][4];
  k2_issue<FMT, NCOL, MT>(a, L, n_tiles, wave, 0, n0, raw);
  for (int q0 = 0; q0 < A * (I / 8); q0 += kK2Threads * 8) {
    uint4 v[8];
    stage_load<kK2Threads, 8>(v, a.hbuf, I, A, I, q0);
    stage_store<kK2Threads, 8>(v, hs, p.h_pitch, A, I, q0);
  }
  __syncthreads();

  bool first = true;
  for (int t0 = wave; t0 < n_tiles; t0 += kK2Waves * MT) {
    f32x4 acc[MT];
#pragma unroll
    for (int s = 0; s < MT; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nchunks; c0 += 4) {
      if (!first) k2_issue<FMT, NCOL, MT>(a, L, n_tiles, t0, c0, n0, raw);
      first = false;
#pragma unroll
      for (int s = 0; s < MT; ++s) {
        const int tile = t0 + kK2Waves * s;
        if (tile < n_tiles) {
          const int e = L.tile_e[tile], m0 = L.tile_m0[tile];
          const int rows = min(16, L.cnt[e] - m0), seg0 = L.off[e] + m0;
          const uint16_t* arow = l16 < rows ? hs + (seg0 + l16) * p.h_pitch : nullptr;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int c = c0 + u;
            if (c < nchunks) {
              bf16x8 av[4], b[4];
#pragma unroll
              for (int q = 0; q < 4; ++q)
                av[q] = arow ? *reinterpret_cast<const bf16x8*>(arow + c * KC + g * 32 + q * 8)
                             : bits_to_bf16x8(0u, 0u, 0u, 0u);
              decode_b<FMT>(raw[s][u], b);
              if constexpr (FMT == MOE_W_FP8_B128) {
                f32x4 t = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int q = 0; q < 4; ++q) t = mfma16(av[q], b[q], t);
                const float bs = block_scale<FMT>(raw[s][u]);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(bs, t[r], acc[s][r]);
              } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[s] = mfma16(av[q], b[q], acc[s]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int s = 0; s < MT; ++s) {
      const int tile = t0 + kK2Waves * s;
      if (tile < n_tiles && l16 < NCOL) {
        const int e = L.tile_e[tile], m0 = L.tile_m0[tile];
        const int rows = min(16, L.cnt[e] - m0), seg0 = L.off[e] + m0;
        float tsd = 1.0f;
        if constexpr (FMT == MOE_W_NVFP4)
          tsd = reinterpret_cast<const float*>(tile_record(a, L, tile) + a.off_ts)[2];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = g * 4 + r;
          if (m < rows) yp[(seg0 + m) * NCOL + l16] = f32_to_bf16_rne(acc[s][r] * tsd);
        }
      }
    }
  }
  __syncthreads();
  // combine of this column slice: fp32 sum in j order, one bf16 rounding
  for (int i = tid; i < T * NCOL; i += kK2Threads) {
    const int t = i / NCOL, c = i - t * NCOL;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j)
      acc = fmaf(X.w[t * k + j], bf16_to_f32(yp[X.inv[t * k + j] * NCOL + c]), acc);
    if (p.y_shared) acc += bf16_to_f32(p.y_shared[(size_t)t * H + n0 + c]);
    p.y[(size_t)t * H + n0 + c] = f32_to_bf16_rne(acc);
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
  auto k1 = dec_gateup_kernel<FMT, CPW>;
  if (!lds_ok(k1, x_lds, granted))
    return set_error(MOE_ERR_HIP, "moe_forward_decode: LDS attribute");
  if (occ_for != x_lds) {  // persistent grid: as many workgroups as fit on the device at once
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(k1),
                                                     256, x_lds) != hipSuccess || per_cu < 1)
      per_cu = 1;
    occ_for = x_lds;
  }
  k1<<<per_cu * g_cus, 256, x_lds, s>>>(p.f, p.T);
  return MOE_OK;
}

template <int FMT>
static int launch_decode(DecArgs& p, hipStream_t s) {
  const int A = p.T * p.f.k;
  const int ncol = (p.f.H / 16 >= g_cus) ? 16 : 8;
  const size_t h_lds = (size_t)A * p.h_pitch * 2 + (size_t)A * ncol * 2;
  static size_t g2a = 0, g2b = 0;
  int st;
  switch (p.f.H / 512) {
    case 1: st = launch_gateup<FMT, 1>(p, s); break;
    case 2: st = launch_gateup<FMT, 2>(p, s); break;
    case 3: st = launch_gateup<FMT, 3>(p, s); break;
    default: st = launch_gateup<FMT, 4>(p, s); break;
  }
  if (st) return st;
  if (ncol == 16) {
    auto k2 = dec_down_combine_kernel<FMT, 16>;
    if (!lds_ok(k2, h_lds, g2a)) return set_error(MOE_ERR_HIP, "moe_forward_decode: LDS attribute");
    k2<<<p.f.H / 16, kK2Threads, h_lds, s>>>(p);
  } else {
    auto k2 = dec_down_combine_kernel<FMT, 8>;
    if (!lds_ok(k2, h_lds, g2b)) return set_error(MOE_ERR_HIP, "moe_forward_decode: LDS attribute");
    k2<<<p.f.H / 8, kK2Threads, h_lds, s>>>(p);
  }
  return check_launch("moe_forward_decode");
}

}  // namespace moe

using namespace moe;

static size_t dec_align(size_t v) { return (v + 255) / 256 * 256; }

extern "C" size_t moe_forward_decode_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W || T < 0 || k < 1) return 0;
  return dec_align((size_t)T * k * W->I * 2) + 256;
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
  f.hbuf = static_cast<uint16_t*>(ws);
  f.y_perm = nullptr;
  p.logits = logits;
  p.T = T;
  p.renorm = renorm;
  p.h_pitch = W->I + 8;
  p.ids = topk_ids; p.wts = topk_w; p.counts = counts; p.offsets = offsets;
  p.sorted = sorted_idx; p.inv = inv_idx;
  p.y_shared = y_shared;
  p.y = y;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int st = moe_route_permute(logits, T, W->E, k, renorm, topk_ids, topk_w, counts, offsets,
                             sorted_idx, inv_idx, nullptr, 0, stream);
  if (st) return st;
  switch (W->fmt) {
    case MOE_W_BF16: return launch_decode<MOE_W_BF16>(p, s);
    case MOE_W_MXFP4: return launch_decode<MOE_W_MXFP4>(p, s);
    case MOE_W_NVFP4: return launch_decode<MOE_W_NVFP4>(p, s);
    default: return launch_decode<MOE_W_FP8_B128>(p, s);
  }
}

extern "C" int moe_forward_decode_supported(int32_t H, int32_t I, int32_t T, int32_t k) {
  // routing in one workgroup; gate/up units hold H/512 chunks of 128 per wave
  // (H in {512, 1024, 1536, 2048}) and keep the batch's x rows in LDS;
  // down+combine keeps all h rows in LDS
  if (T < 0 || k < 1 || T > kDT || T * k > kDA) return 0;
  if (H % 512 || I % 128 || H > 2048 || I > 16384 || H < 512 || I < 128) return 0;
  const size_t lds_max = 160 * 1024;
  const size_t gu_lds = (size_t)T * (H + 8) * 2 + sizeof(TileTable) + sizeof(f32x4) * 4 * 4 * 64 +
                        sizeof(int) * kDA;
  const size_t dn_lds = (size_t)T * k * (I + 8) * 2 + (size_t)T * k * 16 * 2 + sizeof(TileTable) +
                        sizeof(K2Extra);
  return gu_lds <= lds_max && dn_lds <= lds_max;
}
