// Token -> expert permutation: a stable counting sort of the flat assignment
// index a = t*k + j by expert id, with no order-dependent atomics.
//
// The A assignments are cut into chunks (one workgroup of 4 waves each): A <=
// 1024 is one chunk of up to 16 segments of 64, larger A chunks of 256 (one
// segment per wave, so that a prefill batch spreads over many workgroups).  Inside a segment, one wave sorts the
// 64 keys (expert << 6 | lane) with a bitonic network over lane shuffles,
// which gives every element its rank among equal experts in lower lanes and
// every group its size.  Per-(segment, expert) sizes are prefix-summed in
// LDS, per-(chunk, expert) sizes across chunks in a tiny scan kernel, and
// per-expert totals into offsets.  Position of a = offsets[e] + (earlier
// chunks' e-count) + (earlier segments' e-count) + rank.
//
// A <= 1024 runs as one fused workgroup (one launch, used by decode batches);
// larger A runs histogram -> scan -> scatter over chunks of 256.
#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kBlockChunk = 256;  // assignments per workgroup of the multi-block path

template <int CH>
struct ChunkLds {
  static constexpr int kSegs = CH / 64;
  uint16_t segcnt[kSegs][kMaxE];  // per-segment counts, then exclusive prefix
  int rank[CH];                   // rank inside its segment, by chunk position
  int key[CH];                    // expert of each chunk position (E = invalid)
};

// Sort-based stable ranks of one 64-wide segment.  `key` is the expert id of
// this lane's element (E for lanes past the end of the input).
template <int CH>
__device__ __forceinline__ void segment_ranks(int key, int lane, int seg, int E, ChunkLds<CH>& L) {
  uint32_t v = ((uint32_t)key << 6) | (uint32_t)lane;
#pragma unroll
  for (int kk = 2; kk <= 64; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      const uint32_t o = __shfl_xor(v, j, 64);
      const bool up = (lane & kk) == 0;
      const bool lower = (lane & j) == 0;
      const uint32_t mn = o < v ? o : v, mx = o < v ? v : o;
      v = (lower == up) ? mn : mx;
    }
  }
  const int sk = (int)(v >> 6);
  const int orig = (int)(v & 63u);
  const int prev = __shfl_up(sk, 1, 64);
  const bool head = (lane == 0) || (prev != sk);
  int start = head ? lane : 0;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(start, d, 64);
    if (lane >= d) start = o > start ? o : start;
  }
  const int rank = lane - start;
  const int nxt = __shfl_down(sk, 1, 64);
  const bool tail = (lane == 63) || (nxt != sk);
  L.rank[seg * 64 + orig] = rank;
  if (tail && sk < E) L.segcnt[seg][sk] = (uint16_t)(rank + 1);
}

// Ranks of one chunk: fills L.key, L.rank and L.segcnt (as exclusive
// per-expert prefix over segments); returns per-expert chunk totals through
// `total` (one expert per thread, strided).  Ends with a barrier.
template <int CH>
__device__ void chunk_ranks(const int* __restrict__ ids, int A, int E, int chunk, ChunkLds<CH>& L,
                            int* __restrict__ total_out /* LDS or null */) {
  constexpr int kSegs = ChunkLds<CH>::kSegs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kSegs * E; i += kPermThreads) L.segcnt[i / E][i % E] = 0;
  __syncthreads();
  for (int seg = wave; seg < kSegs; seg += kPermThreads / 64) {
    const int pos = seg * 64 + lane;
    const int a = chunk * CH + pos;
    int key = (a < A) ? ids[a] : E;
    key = (key >= 0 && key < E) ? key : E;  // out-of-range ids are never scattered
    L.key[pos] = key;
    segment_ranks(key, lane, seg, E, L);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) {
    int run = 0;
#pragma unroll
    for (int s = 0; s < kSegs; ++s) {
      const int c = L.segcnt[s][e];
      L.segcnt[s][e] = (uint16_t)run;
      run += c;
    }
    if (total_out) total_out[e] = run;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kPermThreads) void permute_fused_kernel(
    const int* __restrict__ ids, int A, int E, int* __restrict__ counts, int* __restrict__ offsets,
    int* __restrict__ sorted_idx, int* __restrict__ inv_idx) {
  __shared__ ChunkLds<kChunk> L;
  __shared__ int tot[kMaxE];
  __shared__ int wave_tot[4];
  chunk_ranks<kChunk>(ids, A, E, 0, L, tot);
  for (int e = threadIdx.x; e < E; e += kPermThreads) counts[e] = tot[e];
  __syncthreads();
  const int total = block_exclusive_scan_256(tot, E, wave_tot);
  for (int e = threadIdx.x; e < E; e += kPermThreads) offsets[e] = tot[e];
  if (threadIdx.x == 0) offsets[E] = total;
  for (int pos = threadIdx.x; pos < A; pos += kPermThreads) {
    const int e = L.key[pos];
    if (e >= E) continue;
    const int p = tot[e] + L.segcnt[pos >> 6][e] + L.rank[pos];
    sorted_idx[p] = pos;
    inv_idx[pos] = p;
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_hist_kernel(const int* __restrict__ ids,
                                                                   int A, int E,
                                                                   int* __restrict__ blkcnt) {
  __shared__ int h[kMaxE];
  for (int e = threadIdx.x; e < E; e += kPermThreads) h[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kBlockChunk;
  for (int i = threadIdx.x; i < kBlockChunk; i += kPermThreads) {
    const int a = base + i;
    if (a < A) {
      const int e = ids[a];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);  // integer counts: order-independent
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPermThreads) blkcnt[(size_t)blockIdx.x * E + e] = h[e];
}

// One workgroup of 1024 threads: per expert, exclusive prefix of the chunk
// counts across chunks (in place) and the totals; then offsets = exclusive scan
// of the totals.  Thread (part, e) = (tid / E, tid % E) takes the part-th of P
// contiguous chunk ranges of expert e: it sums its range first (32 loads in
// flight), the parts' sums meet in LDS, then it reads the range again and
// overwrites it with running prefixes.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void permute_scan_kernel(int nblk, int E,
                                                                   int* __restrict__ blkcnt,
                                                                   int* __restrict__ counts,
                                                                   int* __restrict__ offsets) {
  __shared__ int part_sum[kScanThreads];
  __shared__ int tot[kMaxE];
  __shared__ int wave_tot[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int P = max(1, min(16, kScanThreads / E));  // parts per expert, P * E <= 1024
  const int part = tid / E, e = tid - part * E;
  const bool active = part < P;
  const int b_lo = active ? (int)((int64_t)part * nblk / P) : 0;
  const int b_hi = active ? (int)((int64_t)(part + 1) * nblk / P) : 0;
  int sum = 0;
  for (int b0 = b_lo; b0 < b_hi; b0 += 32) {
    int c[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = b0 + i < b_hi ? blkcnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += c[i];
  }
  part_sum[tid] = sum;
  __syncthreads();
  int run = 0;
  for (int q = 0; q < part && active; ++q) run += part_sum[q * E + e];
  if (active && part == P - 1) {
    tot[e] = run + sum;
    counts[e] = run + sum;
  }
  for (int b0 = b_lo; b0 < b_hi; b0 += 32) {
    int c[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = b0 + i < b_hi ? blkcnt[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (b0 + i < b_hi) {
        blkcnt[(size_t)(b0 + i) * E + e] = run;
        run += c[i];
      }
  }
  __syncthreads();
  const int total = block_exclusive_scan<kScanThreads>(tot, E, wave_tot);
  for (int x = tid; x < E; x += kScanThreads) offsets[x] = tot[x];
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(
    const int* __restrict__ ids, int A, int E, const int* __restrict__ blkbase,
    const int* __restrict__ offsets, int* __restrict__ sorted_idx, int* __restrict__ inv_idx) {
  __shared__ ChunkLds<kBlockChunk> L;
  __shared__ int base[kMaxE];
  for (int e = threadIdx.x; e < E; e += kPermThreads)
    base[e] = offsets[e] + blkbase[(size_t)blockIdx.x * E + e];
  chunk_ranks<kBlockChunk>(ids, A, E, blockIdx.x, L, nullptr);
  const int c0 = blockIdx.x * kBlockChunk;
  for (int pos = threadIdx.x; pos < kBlockChunk; pos += kPermThreads) {
    const int e = L.key[pos];
    if (e >= E) continue;
    const int a = c0 + pos;
    const int p = base[e] + L.segcnt[pos >> 6][e] + L.rank[pos];
    sorted_idx[p] = a;
    inv_idx[a] = p;
  }
}

}  // namespace moe

extern "C" size_t moe_permute_workspace(int32_t T, int32_t k, int32_t E) {
  if (T <= 0 || k <= 0 || E <= 0) return 256;
  const int64_t A = (int64_t)T * k;
  const int64_t nblk = (A + moe::kBlockChunk - 1) / moe::kBlockChunk;
  return (size_t)(((nblk * E * 4) + 255) / 256 * 256);
}

extern "C" int moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E,
                           int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                           int32_t* inv_idx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  using namespace moe;
  if (T < 0 || E < 1 || E > kMaxE || k < 1 || k > E || k > kMaxK)
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: need T>=0, 1<=E<=%d, 1<=k<=min(E,%d)",
                     kMaxE, kMaxK);
  const int64_t A64 = (int64_t)T * k;
  if (A64 > (1 << 30)) return set_error(MOE_ERR_UNSUPPORTED, "moe_permute: T*k too large");
  const int A = (int)A64;
  if (!counts || !offsets) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  if (A > 0 && (!topk_ids || !sorted_idx || !inv_idx))
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: null pointer");
  if (!aligned16(counts) || !aligned16(offsets) || (A > 0 && (!aligned16(topk_ids) ||
      !aligned16(sorted_idx) || !aligned16(inv_idx))))
    return set_error(MOE_ERR_INVALID_ARG, "moe_permute: pointers must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (A <= kChunk) {
    permute_fused_kernel<<<1, kPermThreads, 0, s>>>(topk_ids, A, E, counts, offsets, sorted_idx,
                                                    inv_idx);
    return check_launch("moe_permute(fused)");
  }
  const int nblk = (A + kBlockChunk - 1) / kBlockChunk;
  const size_t need = moe_permute_workspace(T, k, E);
  if (!ws || ws_bytes < need)
    return set_error(MOE_ERR_WORKSPACE, "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
  if (!aligned16(ws)) return set_error(MOE_ERR_INVALID_ARG, "moe_permute: ws misaligned");
  int* blk = static_cast<int*>(ws);
  permute_hist_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, A, E, blk);
  permute_scan_kernel<<<1, kScanThreads, 0, s>>>(nblk, E, blk, counts, offsets);
  permute_scatter_kernel<<<nblk, kPermThreads, 0, s>>>(topk_ids, A, E, blk, offsets, sorted_idx,
                                                      inv_idx);
  return check_launch("moe_permute");
}
