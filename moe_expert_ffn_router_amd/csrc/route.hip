// Router: top-k experts per token with renormalised softmax weights.
//
// One wavefront per token.  Lane l holds logits l, l+64, ... of its token as
// order-preserving 32-bit keys (-0.0 mapped to +0.0) packed with their
// complemented expert index.  Each of the k rounds takes the lane-local and
// then the DPP wave maximum of the packed values, which is the largest key
// and, among equal keys, the lowest index.  The owner clears the winner; lane
// j < k keeps round j's winner and finally computes exp(l_j - l_0) / sum over
// the k selected.
//
// Decode-sized batches (T <= 64, T*k <= 256) also have a fused kernel that
// routes and permutes in one workgroup (one launch instead of two).
#include "route_common.h"

namespace moe {

template <int VPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                    int k, int renorm, int* __restrict__ ids,
                                                    float* __restrict__ wts) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int id;
  float w;
  route_token<VPL>(logits + (size_t)t * E, E, k, renorm, lane, id, w);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    wts[(size_t)t * k + lane] = w;
  }
}

constexpr int kSmallA = 256;
constexpr int kSmallT = 64;

// Route + permute for T <= 64, T*k <= 256 in one workgroup of 16 waves.
// Stable rank of assignment a among equal experts: within its wave, the lanes
// holding the same expert are found with one ballot per expert-id bit (their
// AND is the match mask) and counted below the lane; earlier waves contribute
// through per-wave histograms (the lowest lane of each match group adds the
// group's size), summed in wave order.  No atomics: deterministic.
constexpr int kSmallW = kSmallA / 64;

template <int VPL>
__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int renorm, int* __restrict__ ids,
    float* __restrict__ wts, int* __restrict__ counts, int* __restrict__ offsets,
    int* __restrict__ sorted_idx, int* __restrict__ inv_idx) {
  __shared__ int sid[kSmallA];
  __shared__ int whist[kSmallW][kMaxE];
  __shared__ int hist[kMaxE];
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int A = T * k;
  for (int i = tid; i < kSmallW * E; i += 1024) whist[i / E][i % E] = 0;
  for (int t = wave; t < T; t += 16) {
    int id;
    float w;
    route_token<VPL>(logits + (size_t)t * E, E, k, renorm, lane, id, w);
    if (lane < k) {
      ids[t * k + lane] = id;
      wts[t * k + lane] = w;
      sid[t * k + lane] = id;
    }
  }
  __syncthreads();
  int e = 0, rank = 0;
  if (wave < kSmallW) {  // waves 0..3 own assignments 64*wave + lane
    const bool live = tid < A;
    e = live ? sid[tid] : -1;
    uint64_t m = __ballot(live);
#pragma unroll
    for (int b = 0; b < 10; ++b) {  // E <= 1024: 10 id bits
      const uint64_t on = __ballot(live && ((e >> b) & 1));
      m &= ((e >> b) & 1) ? on : ~on;
    }
    if (!live) m = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    rank = __popcll(m & below);
    if (live && rank == 0) whist[wave][e] = __popcll(m);
  }
  __syncthreads();
  for (int i = tid; i < E; i += 1024) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kSmallW; ++w) c += whist[w][i];
    hist[i] = c;
    counts[i] = c;
  }
  if (tid < A)
    for (int w = 0; w < wave; ++w) rank += whist[w][e];
  __syncthreads();
  const int total = block_exclusive_scan_1024(hist, E, wave_tot);
  if (tid < E) offsets[tid] = hist[tid];
  if (tid == 0) offsets[E] = total;
  if (tid < A) {
    const int p = hist[e] + rank;
    sorted_idx[p] = tid;
    inv_idx[tid] = p;
  }
}

static int route_launch(const float* logits, int T, int E, int k, int renorm, int* ids, float* w,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  switch (vpl_of(E)) {
    case 1: route_kernel<1><<<grid, block, 0, s>>>(logits, T, E, k, renorm, ids, w); break;
    case 2: route_kernel<2><<<grid, block, 0, s>>>(logits, T, E, k, renorm, ids, w); break;
    case 4: route_kernel<4><<<grid, block, 0, s>>>(logits, T, E, k, renorm, ids, w); break;
    case 8: route_kernel<8><<<grid, block, 0, s>>>(logits, T, E, k, renorm, ids, w); break;
    default: route_kernel<16><<<grid, block, 0, s>>>(logits, T, E, k, renorm, ids, w); break;
  }
  return check_launch("moe_route");
}

static int check_route_args(const char* who, const float* logits, int T, int E, int k,
                            const int* ids, const float* w) {
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "%s: need T>=0, 1<=E<=%d, 1<=k<=min(E,%d) "
                     "(T=%d E=%d k=%d)", who, kMaxE, kMaxK, T, E, k);
  if (T == 0) return MOE_OK;
  if (!logits || !ids || !w) return set_error(MOE_ERR_INVALID_ARG, "%s: null pointer", who);
  if (!aligned16(logits) || !aligned16(ids) || !aligned16(w))
    return set_error(MOE_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", who);
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                         int32_t* topk_ids, float* topk_w, moe_stream_t stream) {
  int st = check_route_args("moe_route", logits, T, E, k, topk_ids, topk_w);
  if (st || T == 0) return st;
  return route_launch(logits, T, E, k, renorm, topk_ids, topk_w,
                      reinterpret_cast<hipStream_t>(stream));
}

extern "C" int moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k,
                                 int32_t renorm, int32_t* topk_ids, float* topk_w,
                                 int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                                 int32_t* inv_idx, void* ws, size_t ws_bytes,
                                 moe_stream_t stream) {
  int st = check_route_args("moe_route_permute", logits, T, E, k, topk_ids, topk_w);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (T > 0 && T <= kSmallT && T * k <= kSmallA) {
    if (!counts || !offsets || !sorted_idx || !inv_idx || !aligned16(counts) ||
        !aligned16(offsets) || !aligned16(sorted_idx) || !aligned16(inv_idx))
      return set_error(MOE_ERR_INVALID_ARG, "moe_route_permute: permutation outputs");
    switch (vpl_of(E)) {
#define MOE_RP(V)                                                                         \
  case V:                                                                                 \
    route_permute_small_kernel<V><<<1, 1024, 0, s>>>(logits, T, E, k, renorm, topk_ids,   \
                                                     topk_w, counts, offsets, sorted_idx, \
                                                     inv_idx);                            \
    break;
      MOE_RP(1) MOE_RP(2) MOE_RP(4) MOE_RP(8) MOE_RP(16)
#undef MOE_RP
    }
    return check_launch("moe_route_permute");
  }
  if (T > 0) {
    st = route_launch(logits, T, E, k, renorm, topk_ids, topk_w, s);
    if (st) return st;
  }
  return moe_permute(topk_ids, T, k, E, counts, offsets, sorted_idx, inv_idx, ws, ws_bytes,
                     stream);
}
