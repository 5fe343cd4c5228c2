/*
 * moe_layer.h — C ABI of the MI355X (gfx950) MoE-layer forward library.
 *
 * One Mixture-of-Experts layer forward as used by an edge MoE serving engine
 * (FreeToken pages: supported-models guide, sections "MoE strategies",
 * "expert bank & LRU slot cache", "minimum cache constraint", "how
 * quantizations land"; README feature list; fork README, production
 * configuration): route each token to k experts, group the (token, slot)
 * assignments by expert, run each expert's SwiGLU FFN over its rows with
 * weights stored as BF16 / MXFP4 / NVFP4 / FP8, and combine the k outputs of
 * every token with its routing weights.  Experts are addressed through a slot
 * table into a fixed HBM pool that an LRU policy refills from a pinned host
 * bank.
 *
 * Conventions shared by every call
 *  - All pointers are owned by the caller.  "device" pointers are HIP device
 *    memory (or host memory mapped for the device), "host" pointers ordinary
 *    host memory.  No call allocates device memory; scratch space is passed
 *    in as `ws` after sizing it with the matching *_workspace query.
 *  - Calls enqueue work on the given stream and return without waiting, so
 *    route / permute / expert_ffn / combine can be captured into a HIP graph.
 *  - Every call validates its arguments before enqueueing anything and
 *    returns a moe_status; nothing aborts or throws across the ABI.  On an
 *    error, moe_last_error() returns a message for the calling thread.
 *  - Device pointers must be 16-byte aligned.  Results are deterministic:
 *    there are no floating-point atomics, so repeated calls on the same
 *    inputs give identical bits.
 *  - bf16 tensors are passed as uint16_t bit patterns; fp32 as float.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t; NULL = null stream */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad size, null pointer, misalignment, bad id      */
  MOE_ERR_UNSUPPORTED = 2, /* shape or format outside the supported set         */
  MOE_ERR_HIP = 3,         /* a HIP runtime call or kernel launch failed        */
  MOE_ERR_CAPACITY = 4,    /* cache: more distinct experts needed than slots    */
  MOE_ERR_WORKSPACE = 5    /* ws too small (see the *_workspace queries)         */
} moe_status;

/* Expert weight storage formats (README "Broad MoE & ecosystem support";
 * guide "CPU layer split" lists bf16, nvfp4, mxfp4 and fp8 experts). */
typedef enum {
  MOE_W_BF16 = 0,     /* plain bf16                                             */
  MOE_W_MXFP4 = 1,    /* E2M1 codes, one E8M0 scale per 32 along K              */
  MOE_W_NVFP4 = 2,    /* E2M1 codes, one E4M3 scale per 16 along K, and one
                         fp32 scale per (expert, projection)                    */
  MOE_W_FP8_B128 = 3  /* E4M3 codes, one fp32 scale per 128 x 128 block         */
} moe_wfmt;

/* Byte offsets of the sections inside one expert record; -1 = absent.
 *
 * One expert = one record; sections start at 256-byte aligned offsets in the
 * order w13, w13_scale, w2, w2_scale, tensor_scale, and the record stride is
 * the payload rounded up to 256.  All matrices are row-major with K (the
 * reduction index) contiguous:
 *   w13  [2I][H]  rows 0..I-1 = gate projection, rows I..2I-1 = up projection
 *   w2   [H][I]   down projection
 *   E2M1 codes: two per byte, element 2i in the low nibble, 2i+1 in the high
 *   MXFP4 scales [rows][K/32] E8M0;  NVFP4 scales [rows][K/16] E4M3 (>= 0)
 *   NVFP4 tensor_scale fp32[3] = (gate, up, down)
 *   FP8 scales fp32 [rows/128][K/128]                                         */
typedef struct {
  int64_t w13, w13_scale, w2, w2_scale, tensor_scale;
  int64_t payload_bytes; /* bytes that carry data (sum of section sizes)      */
  int64_t stride;        /* record size in memory (payload rounded to 256)    */
} moe_expert_layout;

/* Fill *out for format fmt and sizes H (hidden), I (expert intermediate).
 * Supported: H and I multiples of 128, 128 <= H, I <= 16384.               */
int moe_expert_layout_query(int32_t fmt, int32_t H, int32_t I, moe_expert_layout* out);

/* One layer's experts.  Record of expert e is at
 *   base + (slot_of_expert ? slot_of_expert[e] : e) * stride                 */
typedef struct {
  int32_t fmt;        /* moe_wfmt                                             */
  int32_t E;          /* experts in the layer, 1..1024                        */
  int32_t H, I;       /* hidden size, expert intermediate size                */
  const void* base;   /* device: E records, or the S records of a slot pool   */
  int64_t stride;     /* bytes between records, == moe_expert_layout.stride   */
} moe_experts;

/* ---------------------------------------------------------------------------
 * moe_route — router top-k with renormalised weights.
 * The pages state that each token activates a few experts of the layer
 * (guide, "MoE strategies") and give no router formula; this computes, per
 * token t, the k experts with the largest logits (ties -> lower index wins,
 * -0.0 == +0.0), in that order, and the softmax over those k logits
 * (renorm = 1) or the full-softmax probabilities of those k (renorm = 0).
 *   logits   device fp32 [T][E] row-major
 *   topk_ids device int32 [T][k] (out)     topk_w device fp32 [T][k] (out)
 * 1 <= k <= min(E, 16), 1 <= E <= 1024, T >= 0 (T = 0 is a no-op).
 * NaN logits give unspecified (but in-range) ids.                           */
int moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
              int32_t* topk_ids, float* topk_w, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_permute — group the A = T*k assignments a = t*k + j by expert
 * (stable counting sort; the fork README's per-layer prefill MoE kernel works
 * on per-expert row blocks):
 *   counts[e]     = #{a : topk_ids[a] == e}               device int32 [E]
 *   offsets[e]    = sum of counts[0..e-1], offsets[E] = A   device int32 [E+1]
 *   sorted_idx[p] = assignments in expert order, ascending a in each expert
 *                                                           device int32 [A]
 *   inv_idx[a]    = p with sorted_idx[p] == a                device int32 [A]
 * Ids must lie in [0, E) (an id outside gives unspecified output but no
 * out-of-bounds access).  ws: device, >= moe_permute_workspace(T, k, E).    */
size_t moe_permute_workspace(int32_t T, int32_t k, int32_t E);
int moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* counts,
                int32_t* offsets, int32_t* sorted_idx, int32_t* inv_idx, void* ws,
                size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_route_permute — moe_route followed by moe_permute, same arguments and
 * results as the two calls.  For decode-sized batches (T <= 64, T*k <= 256)
 * both steps run in one workgroup (one launch); otherwise it issues the two
 * calls' kernels.  ws as for moe_permute (unused on the one-launch path).    */
int moe_route_permute(const float* logits, int32_t T, int32_t E, int32_t k, int32_t renorm,
                      int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_idx, int32_t* inv_idx, void* ws, size_t ws_bytes,
                      moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_expert_ffn — per-expert SwiGLU FFN over the permuted rows.
 * For every expert e with rows p in [offsets[e], offsets[e+1]):
 *   x_p      = x[sorted_idx[p] / k]                       (bf16 row, H)
 *   h_p      = SiLU(x_p W_gate[e]^T) * (x_p W_up[e]^T)    (I values)
 *   y_perm_p = h_p W_down[e]^T                            (H values, bf16)
 * with SiLU(z) = z / (1 + e^-z), fp32 accumulation, weights used exactly:
 * MXFP4 and FP8 weights feed the block-scaled MFMA as stored (prefill) or
 * decoded to bf16 (decode variants); NVFP4 and BF16 are decoded to bf16 (the
 * NVFP4 block part is exact in bf16); FP8 block scales and NVFP4 tensor
 * scales are applied to fp32 partial sums.  For the block-scaled MFMA the
 * bf16 activations (x, then h) are split into E4M3 hi + lo with one E8M0
 * scale per 32; hi + lo differs from the bf16 value by at most 2^-10 times
 * the block scale, i.e. at most 2^-17 of the block's largest magnitude.  The activation
 * is not named on the pages; SwiGLU is the plainest reading for the MoE
 * families the guide lists.
 *   slot_of_expert  device int32 [E] or NULL (identity); only entries of
 *                   experts with counts[e] > 0 are read and must lie in
 *                   [0, pool slots)
 *   x               device bf16 [T][H]
 *   counts, offsets, sorted_idx   from moe_permute
 *   y_perm          device bf16 [T*k][H] (out, permuted order)
 *   variant         0 = choose by size, 1 = small-batch (decode) kernels,
 *                   2 = tiled (prefill) kernels; all give the same result up
 *                   to fp32 summation order
 * ws: device, >= moe_expert_ffn_workspace(W, T, k): h bf16 [T*k][I], or,
 *     on the MXFP4 / FP8 prefill path, the split activations of both GEMMs
 *     in the same space (that path never forms bf16 h).                     */
size_t moe_expert_ffn_workspace(const moe_experts* W, int32_t T, int32_t k);
int moe_expert_ffn(const moe_experts* W, const int32_t* slot_of_expert, const uint16_t* x,
                   int32_t T, int32_t k, const int32_t* counts, const int32_t* offsets,
                   const int32_t* sorted_idx, uint16_t* y_perm, int32_t variant, void* ws,
                   size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_combine — weighted sum of each token's k expert outputs.  The pages
 * say a token activates a few experts of its layer (guide, "MoE strategies";
 * feature article, its activated-experts passage) and print no formula for
 * how their outputs merge; the plainest reading, taken here, is the
 * routing-weighted sum of the activated experts' outputs:
 *   y[t] = sum_{j<k} topk_w[t][j] * y_perm[inv_idx[t*k+j]]  (+ y_shared[t])
 * summed in j order in fp32, rounded once to bf16 (nearest-even).
 *   y_perm device bf16 [T*k][H]; inv_idx device int32 [T*k];
 *   topk_w device fp32 [T][k]; y_shared device bf16 [T][H] or NULL (the
 *   always-on shared expert, weight 1.0); y device bf16 [T][H] (out).
 * H a multiple of 8.                                                        */
int moe_combine(const uint16_t* y_perm, const int32_t* inv_idx, const float* topk_w, int32_t T,
                int32_t k, int32_t H, const uint16_t* y_shared, uint16_t* y,
                moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_decode — the whole layer for decode-sized batches in one call.
 * T <= 16 (H <= 2048): two launches, token-major — gate/up workgroups route
 * their own token (one wave, from the logits) and store h by assignment; the
 * down workgroups fold in the combine, and one extra workgroup writes the
 * permutation outputs.  With MXFP4 weights, E <= 256 and T*k*(I/128) a
 * multiple of 256 (whole rounds of one workgroup per compute unit) the first
 * launch does the whole expert FFN instead: a workgroup per (token, expert
 * slot, 128 h-columns) computes those h-columns and their share of the down
 * projection for every output column (fp32 partials in the workspace); the
 * second sums the partials and combines.  16 < T <= 64: four launches — route + permute in one
 * workgroup, gate/up and down as persistent grids over 16-row expert tiles,
 * combine.  Writes every output
 * of moe_route_permute + moe_expert_ffn + moe_combine: topk_ids / topk_w
 * [T][k], counts [E], offsets [E+1], sorted_idx / inv_idx [T*k] (identical
 * to moe_route_permute), y [T][H] (y_shared [T][H] nullable, added with
 * weight 1); y agrees with the separate calls within the parity tolerance
 * (the FFN kernels split K their own way; fixed order, so repeat calls give
 * the same bits).  The pages' "graph-compatible execution" (README feature
 * list; fork production configuration, --cuda-graph-max-bs) is served with
 * two (or four) graph nodes per layer.  Shapes outside
 * moe_forward_decode_supported(H, I, T, k) return MOE_ERR_UNSUPPORTED (use
 * the separate calls): T <= 64, T*k <= 256, H and I in {512, 1024, 1536,
 * 2048}, T*(H+8)*2 bytes of x fitting in LDS beside the tile table.
 *   ws: device, >= moe_forward_decode_workspace(W, T, k) bytes (holds h,
 *   y_perm and the partials; contents on entry are ignored; the size for T
 *   also serves every smaller batch).                                       */
int moe_forward_decode_supported(int32_t H, int32_t I, int32_t T, int32_t k);
size_t moe_forward_decode_workspace(const moe_experts* W, int32_t T, int32_t k);
int moe_forward_decode(const moe_experts* W, const int32_t* slot_of_expert, const float* logits,
                       const uint16_t* x, int32_t T, int32_t k, int32_t renorm, int32_t* topk_ids,
                       float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted_idx,
                       int32_t* inv_idx, const uint16_t* y_shared, uint16_t* y, void* ws,
                       size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_forward_decode_noalloc — for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): moe_forward_decode with the same arguments and results but no
 * workspace argument.  Its scratch (h, y_perm and the one-stream path's fp32
 * partials) lives in a fixed array of moe_forward_decode_noalloc_max_scratch()
 * = 8 MiB of device memory that each GPU the library runs on holds until the
 * process ends; its device address is looked up on the first call on each
 * device (hipGetSymbolAddress; nothing is allocated by this library).  A call
 * whose moe_forward_decode_workspace(W, T, k) exceeds that size returns
 * MOE_ERR_WORKSPACE before enqueueing anything.  Every call on one GPU shares
 * that GPU's array (its contents on entry are ignored, nothing needs
 * clearing): calls that overlap on one GPU (other streams, or other threads)
 * race and give undefined results; serialise them.                        */
size_t moe_forward_decode_noalloc_max_scratch(void);
int moe_forward_decode_noalloc(const moe_experts* W, const int32_t* slot_of_expert,
                               const float* logits, const uint16_t* x, int32_t T, int32_t k,
                               int32_t renorm, int32_t* topk_ids, float* topk_w, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_idx, int32_t* inv_idx,
                               const uint16_t* y_shared, uint16_t* y, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_dequant_expert — decode one expert record to fp32 with the same device
 * decoders the FFN kernels use (for checking every code on the device).
 *   w13 device fp32 [2I][H] (out), w2 device fp32 [H][I] (out); the NVFP4
 *   tensor scales are applied, the FP8 block scales too (one fp32 product).  */
int moe_dequant_expert(const moe_experts* W, int32_t expert, float* w13, float* w2,
                       moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * moe_shared_ffn — the always-on shared expert (the large-prefill workload's
 * "plus 1 always-on shared expert", added to every token's output with
 * weight 1 by moe_combine / moe_forward_decode through y_shared): the dense
 * SwiGLU FFN of every token row with one BF16 expert record (W->base points
 * at it; W->fmt BF16, W->H, W->I its sizes), no routing or permutation.
 *   x:  device bf16 [T][H];  y: device bf16 [T][H] (out)
 *   gate/up and down are dense bf16 GEMMs on the bf16 MFMA with fp32
 *   accumulation (this library's kernels); h = bf16(SiLU(gate) * up) is formed
 *   from the fp32 accumulators of the gate/up product.
 *   ws: device, >= moe_shared_ffn_workspace(W, T) bytes (h, bf16 [T][I]);
 *   enqueued on `stream`; allocates nothing.
 * Other formats return MOE_ERR_UNSUPPORTED (moe_expert_ffn with E = 1, k = 1
 * computes the same for any format). */
size_t moe_shared_ffn_workspace(const moe_experts* W, int32_t T);
int moe_shared_ffn(const moe_experts* W, const uint16_t* x, int32_t T, uint16_t* y, void* ws,
                   size_t ws_bytes, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * Expert-slot cache (guide, "expert bank & LRU slot cache", "MoE strategies"
 * offload, "minimum cache constraint").  A fixed pool of S slots in HBM,
 * shared by all layers, holds expert records; the slot table maps
 * (layer, expert) to a slot.  The handle owns host metadata only.
 *
 * Policy (deterministic LRU; the pages give only "LRU" and "most recent active
 * step" per (layer, expert)):
 *   needed  = experts with counts[e] > 0, ascending
 *   |needed| > S            -> MOE_ERR_CAPACITY, state unchanged
 *   misses  = needed not resident, ascending; each takes the lowest empty
 *             slot, else the slot whose owner is not needed now with the
 *             smallest (last-active step, slot index)
 *   every needed slot's last-active step := the step clock; clock += 1
 *
 * moe_cache_create
 *   pool_dev        device, S * slot_bytes bytes (slot s at s * slot_bytes)
 *   bank_host       host memory allocated pinned (hipHostMalloc / torch
 *                   pin_memory), n_layers * E records of slot_bytes, record of
 *                   (layer, e) at (layer * E + e) * slot_bytes
 *   slot_table_dev  device int32 [n_layers][E]; the cache writes the slot of
 *                   every expert it makes resident (other entries untouched)
 *   The cache starts empty.  1 <= S, slot_bytes > 0 and a multiple of 256.  */
typedef struct moe_cache* moe_cache_t;

int moe_cache_create(moe_cache_t* out, int32_t n_layers, int32_t E, int32_t S,
                     int64_t slot_bytes, void* pool_dev, const void* bank_host,
                     int32_t* slot_table_dev);
void moe_cache_destroy(moe_cache_t cache);

/* expert_cache_lookup — run the policy for one (layer-)step.
 *   counts_host  host int32 [E] (the caller's copy of moe_permute's counts)
 *   miss_expert, miss_slot   host int32 [E] (out): the fills to make, in order
 *   n_miss, n_hit            host (out)
 *   slot_row_host            host int32 [E] (out, may be NULL): the layer's
 *                            slot table row after this step (-1 = not resident)
 * On MOE_ERR_CAPACITY nothing changes.  Host-only; touches no device memory. */
int expert_cache_lookup(moe_cache_t cache, int32_t layer, const int32_t* counts_host,
                        int32_t* miss_expert, int32_t* miss_slot, int32_t* n_miss,
                        int32_t* n_hit, int32_t* slot_row_host);

/* expert_cache_row — the current slot of every expert of `layer` (host int32
 * [E] out; -1 = not resident), as the policy state stands now (other layers'
 * lookups may have evicted some since this layer's last lookup).  Host-only;
 * changes nothing. */
int expert_cache_row(moe_cache_t cache, int32_t layer, int32_t* slot_row_host);

/* expert_cache_fill — make the lookup's misses resident and publish the slot
 * table row for `layer`:
 *   1. `side` waits for all work already enqueued on `compute` (so a victim
 *      slot is never overwritten while an earlier FFN still reads it);
 *   2. one hipMemcpyAsync host->device per miss, bank -> pool slot, on `side`;
 *   3. the layer's slot-table row is copied host->device on `side`;
 *   4. `compute` waits for `side`.
 * Work enqueued on `compute` afterwards sees the filled slots.  miss arrays
 * as returned by expert_cache_lookup for the same layer.                     */
int expert_cache_fill(moe_cache_t cache, int32_t layer, const int32_t* miss_expert,
                      const int32_t* miss_slot, int32_t n_miss, moe_stream_t side,
                      moe_stream_t compute);

/* expert_cache_fill_groups — the fills of one lookup as groups that expert
 * FFN work can run behind (FlashML-org / FreeToken README feature list,
 * "full-layer double-buffered prefill streaming"; the article on FreeToken's
 * design, its section on full-layer double-buffered prefill streaming: copy
 * the next block's weights while the current block computes):
 *   1. the layer's slot-table row is copied host->device on `compute` (hit
 *      entries are unchanged; a miss entry names a slot whose bytes land with
 *      its group);
 *   2. `side` waits for all work already enqueued on `compute` (no victim slot
 *      is overwritten while an earlier FFN still reads it);
 *   3. the misses, in lookup order, are split into n_groups consecutive groups
 *      of equal size (to within one); group g's copies are issued on `side`
 *      and its end is recorded in the handle's event g.
 * `compute` is NOT made to wait: work on `compute` that reads only hit experts
 * may run at once; work that reads group g's experts must come after
 * expert_cache_wait_group(g).  n_groups in [1, min(16, n_miss)], or 0 when
 * n_miss is 0.  Miss arrays as returned by expert_cache_lookup for the same
 * layer.  Errors leave the copies already enqueued in place.              */
int expert_cache_fill_groups(moe_cache_t cache, int32_t layer, const int32_t* miss_expert,
                             const int32_t* miss_slot, int32_t n_miss, int32_t n_groups,
                             moe_stream_t side, moe_stream_t compute);

/* expert_cache_wait_group — make `compute` wait for group `group` (0..15) of
 * the latest expert_cache_fill_groups call (a group index past that call's
 * n_groups names an older, already recorded group). */
int expert_cache_wait_group(moe_cache_t cache, int32_t group, moe_stream_t compute);

/* expert_cache_plan — the policy for one (layer-)step that may need more
 * distinct experts than the pool holds (README feature list, "full-layer
 * double-buffered prefill streaming"; feature article, its two-buffer
 * mechanism: one buffer computed on while the next is filled).  The pages give
 * no rule; read here as: if the step's experts fit (|needed| <= S) they form
 * one wave, otherwise waves of at most floor(S/2) experts (at least one),
 * resident experts first, then the others, each ascending.  Each wave is one
 * lookup (the policy above, one clock tick).  Under that policy a wave never
 * evicts an expert the wave before it reads (S >= 2), so the next wave's
 * copies can overlap the current wave's FFN.  Never refuses for capacity.
 *   counts_host     host int32 [E]
 *   wave_of_expert  host int32 [E] (out, may be NULL): wave of each needed
 *                   expert, -1 for the others
 *   fill_expert, fill_slot  host int32 [E] (out, may be NULL): all fills, wave
 *                   by wave, each wave's in lookup order
 *   wave_fill_end   host int32 [E] (out, may be NULL): wave w's fills are
 *                   [wave_fill_end[w-1], wave_fill_end[w]) (0 for w = 0)
 *   n_waves, n_hit  host (out; n_hit may be NULL)
 * Host-only; touches no device memory. */
int expert_cache_plan(moe_cache_t cache, int32_t layer, const int32_t* counts_host,
                      int32_t* wave_of_expert, int32_t* fill_expert, int32_t* fill_slot,
                      int32_t* wave_fill_end, int32_t* n_waves, int32_t* n_hit);

/* moe_expert_ffn_streamed — moe_expert_ffn for one (layer-)step through the
 * cache's pool, with the fills streamed under the computation (README feature
 * list, "full-layer double-buffered prefill streaming"; guide, "MoE
 * strategies" offload):
 *   the step is planned as in expert_cache_plan; for each wave, the layer's
 *   slot-table row is published on `compute`, the wave's misses are copied
 *   host->device on `side` in min(n_groups, misses) groups of equal size (to
 *   within one), the expert FFN runs on `compute` over the wave's hit experts
 *   at once and over each group's experts once that group has landed.  Wave
 *   w's copies wait only for the FFN work of wave w-2 (and everything enqueued
 *   on `compute` before the call): two staging sets.  y_perm rows of every
 *   needed expert are written exactly as by one moe_expert_ffn call (same
 *   tiles; bit-identical).
 *   pool_W          the cache's pool as experts: E = the cache's E, base = its
 *                   pool, stride = its slot_bytes
 *   x, T, k, offsets, sorted_idx, y_perm   as for moe_expert_ffn (device)
 *   counts_host     host int32 [E]: the caller's copy of moe_permute's counts
 *   n_groups        1..16
 *   ws              device, >= moe_expert_ffn_streamed_workspace(pool_W, T, k)
 *   fill_expert, fill_slot, wave_fill_end, n_waves, n_hit   as for
 *                   expert_cache_plan (host out, each may be NULL)
 * Returns without waiting; the slot-table row for `layer` on the device is the
 * one after the last wave once `compute` reaches the end of the call's work.
 * Allocates nothing (the handle's pinned per-wave records are reused; the host
 * blocks only when a record's previous copy is still pending). */
size_t moe_expert_ffn_streamed_workspace(const moe_experts* pool_W, int32_t T, int32_t k);
int moe_expert_ffn_streamed(moe_cache_t cache, int32_t layer, const moe_experts* pool_W,
                            const uint16_t* x, int32_t T, int32_t k, const int32_t* counts_host,
                            const int32_t* offsets, const int32_t* sorted_idx, uint16_t* y_perm,
                            int32_t n_groups, void* ws, size_t ws_bytes, moe_stream_t side,
                            moe_stream_t compute, int32_t* fill_expert, int32_t* fill_slot,
                            int32_t* wave_fill_end, int32_t* n_waves, int32_t* n_hit);

/* moe_cache_resize — change the pool to new_S slots at run time, without
 * reloading the experts that stay resident (FlashML-org / FreeToken README
 * feature list, elastic VRAM: the expert cache and the KV cache re-split while
 * the engine runs; guide, "expert bank & LRU slot cache": the LRU keeps each
 * (layer, expert)'s last active step).  The pages give no rule for what a
 * smaller pool keeps; read here as LRU order:
 *   kept   = the min(new_S, resident count) residents with the latest
 *            last-active step (ties: lower slot); the others are dropped
 *   placed = kept residents in ascending old-slot order into slots 0, 1, ...
 *   last-active steps and the step clock are unchanged.
 *   new_pool_dev  device, new_S * slot_bytes bytes: the pool from now on; or
 *                 NULL to keep the current pool, which must then hold
 *                 new_S * slot_bytes bytes (the caller's allocation)
 *   move_from, move_to  host int32 [min(S, new_S)] (out, may be NULL): old and
 *                 new slot of every kept resident, in placement order
 *   n_moves       host (out, may be NULL): number of kept residents
 * Device side (handles created with pool, bank and table): `compute` waits
 * for every fill already issued on `side`; kept records are copied device to
 * device on `compute` (in place, only those whose slot changes; the ascending
 * packing never overwrites a record before it has moved); every layer's
 * slot-table row is rewritten; the call returns once `compute` has drained
 * (host-synchronous, not for graph capture), so the old pool may be freed on
 * return.  Host-only handles update the metadata alone (new_pool_dev NULL).
 * Experts descriptors built over the old pool must be rebuilt over the new. */
int moe_cache_resize(moe_cache_t cache, int32_t new_S, void* new_pool_dev, int32_t* move_from,
                     int32_t* move_to, int32_t* n_moves, moe_stream_t side,
                     moe_stream_t compute);

/* ---------------------------------------------------------------------------
 * CPU execution of experts (guide, "MoE strategies": the cpu strategy computes
 * missed experts on the CPU from host memory; hybrid splits one step's misses
 * between fetching over PCIe and CPU execution, both at once; "CPU layer
 * split": the CPU executor serves bf16, nvfp4 and mxfp4 experts — this one
 * also serves fp8).  A pool of host threads owned by the handle. */
typedef struct moe_cpu_pool* moe_cpu_pool_t;
int moe_cpu_pool_create(moe_cpu_pool_t* out, int32_t threads); /* threads incl. the caller's */
void moe_cpu_pool_destroy(moe_cpu_pool_t pool);

/* moe_cpu_expert_ffn — the expert FFN of moe_expert_ffn on the CPU, for the
 * listed experts only, all operands in host memory:
 *   W          experts whose base is HOST memory (e.g. one layer of the pinned
 *              bank: record of expert e at base + e * stride)
 *   experts    host int32 [n_experts] (each once, in [0, E))
 *   x          host bf16 [T][H];  offsets host int32 [E+1];  sorted_idx host
 *              int32 [T*k] (as from moe_permute)
 *   y_perm     host bf16 [T*k][H]: rows [offsets[e], offsets[e+1]) of every
 *              listed expert are written, others untouched
 * Weights decode exactly to fp32; products accumulate in fp32 (fixed order);
 * h = bf16(SiLU(gate) * up) and y are rounded to bf16 as on the GPU path.
 * Results do not depend on the thread count.  Synchronous; host only. */
int moe_cpu_expert_ffn(moe_cpu_pool_t pool, const moe_experts* W, const int32_t* experts,
                       int32_t n_experts, const uint16_t* x, int32_t T, int32_t k,
                       const int32_t* offsets, const int32_t* sorted_idx, uint16_t* y_perm);

/* moe_bench_bw — calibrate this machine (guide, "use ft bench bw to calibrate";
 * "hybrid's automatic decision"): the fetch path's rate (pinned host -> device
 * copies of n_records expert records of bank_W into pool_dev on `stream`) and
 * the CPU executor's rate (each of those records as an expert with one token
 * row), both in record payload bytes per second.  hybrid_recommended is set
 * when the CPU rate is at least `threshold` times the copy rate (the pages'
 * default threshold is 2.0); fetch_fraction = h2d / (h2d + cpu) is the share
 * of a step's misses to fetch so that fetching and CPU execution take equal
 * time (the q* split).  Synchronous; pool_dev holds n_records records. */
typedef struct {
  double h2d_bytes_per_s, cpu_bytes_per_s, threshold, fetch_fraction;
  int32_t hybrid_recommended;
} moe_bw_profile;
int moe_bench_bw(moe_cpu_pool_t pool, const moe_experts* bank_W, void* pool_dev,
                 int32_t n_records, moe_stream_t stream, double threshold, moe_bw_profile* out);

/* expert_cache_plan_hybrid — the policy of one hybrid step (guide, "MoE
 * strategies": hybrid fetches part of a step's misses over PCIe and computes
 * the rest on the CPU, overlapped; "expert bank & LRU slot cache": each
 * (layer, expert)'s most recent active step lets the per-layer fetch cap take
 * the most active misses first).  The pages fix no rule; read here as:
 *   misses   = needed experts not resident, ordered by their last active
 *              step, latest first (never active last; ties lower expert first)
 *   n_fetch  = ceil(fetch_fraction * |misses|), at most max_fetch when
 *              max_fetch >= 0 (fetch_fraction 1 = offload, 0 = cpu strategy)
 *   the first n_fetch misses are fetched: with the hits they form the GPU step
 *   (planned as expert_cache_plan); the other misses run on the CPU and take
 *   no slot; their last active step is the step's clock (a step with no GPU
 *   expert still advances the clock).
 *   cpu_expert  host int32 [E] (out, may be NULL): the CPU experts, ascending
 *   n_cpu       host (out);  other outputs as for expert_cache_plan
 * Host-only; touches no device memory. */
int expert_cache_plan_hybrid(moe_cache_t cache, int32_t layer, const int32_t* counts_host,
                             double fetch_fraction, int32_t max_fetch, int32_t* cpu_expert,
                             int32_t* n_cpu, int32_t* fill_expert, int32_t* fill_slot,
                             int32_t* wave_fill_end, int32_t* n_waves, int32_t* n_hit);

/* moe_expert_ffn_hybrid — one hybrid step of the expert FFN: the policy of
 * expert_cache_plan_hybrid; the GPU step runs as in moe_expert_ffn_streamed
 * (grouped fills on `side`, the FFN behind them on `compute`), and while it
 * runs the calling thread computes the CPU experts with moe_cpu_expert_ffn
 * from the cache's bank (x, offsets and sorted_idx are first copied down into
 * host_stage on `compute`), then copies their y_perm rows up on `compute`.
 * Returns once the CPU share is done and its rows' copies are enqueued;
 * `compute` then holds every y_perm row of the step.
 *   cpu_pool       moe_cpu_pool_create handle
 *   host_stage     PINNED host memory, >= moe_expert_ffn_hybrid_host_bytes
 *                  (x, offsets, sorted_idx and the CPU rows); reused by the
 *                  next call once its copies are done (the call waits)
 *   fetch_fraction, max_fetch   as for expert_cache_plan_hybrid
 *   the other arguments and outputs as for moe_expert_ffn_streamed, plus
 *   cpu_expert / n_cpu (host out) as for expert_cache_plan_hybrid.
 * CPU experts' y_perm rows are the CPU executor's (fp32 accumulation in
 * another order: equal to the GPU's within the parity tolerance, not
 * bit-identical).  Allocates no device memory. */
size_t moe_expert_ffn_hybrid_host_bytes(const moe_experts* pool_W, int32_t T, int32_t k);
int moe_expert_ffn_hybrid(moe_cache_t cache, int32_t layer, const moe_experts* pool_W,
                          moe_cpu_pool_t cpu_pool, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* counts_host, const int32_t* offsets,
                          const int32_t* sorted_idx, uint16_t* y_perm, double fetch_fraction,
                          int32_t max_fetch, int32_t n_groups, void* ws, size_t ws_bytes,
                          void* host_stage, size_t host_bytes, moe_stream_t side,
                          moe_stream_t compute, int32_t* cpu_expert, int32_t* n_cpu,
                          int32_t* fill_expert, int32_t* fill_slot, int32_t* wave_fill_end,
                          int32_t* n_waves, int32_t* n_hit);

/* Counters since creation: steps, hits, misses, bytes copied host->device. */
int moe_cache_stats(moe_cache_t cache, int64_t* steps, int64_t* hits, int64_t* misses,
                    int64_t* bytes_filled);

/* ---------------------------------------------------------------------------
 * Diagnostics. */
const char* moe_status_str(int status);
const char* moe_last_error(void); /* thread-local; "" when none */
int moe_version(void);            /* ABI version, currently 1 */

/* Bounds-checked builds (the library compiled with -DMOE_DEBUG; a separate
 * build, see the package's build script).  There, every index a kernel takes
 * from a caller's array is range-checked before use: slot-table entries
 * against [0, E) of the moe_experts they address (the struct carries no
 * pool size, so with a pool of S < E slots an entry in [S, E) passes),
 * sorted_idx values against T*k, each expert's row segment (offsets[e],
 * counts[e]) against [0, T*k), inv_idx values in moe_combine against T*k.
 * An out-of-range value is replaced by an in-range one (the kernel stays
 * inside its buffers; its results are then meaningless) and sets a flag:
 *   1 = slot, 2 = sorted index, 4 = row segment, 8 = inverse index
 *   (0x80000000: the flags could not be read).
 * moe_debug_take writes the flags raised since the previous call into *flags
 * and clears them; it synchronizes the device.  Release builds compile the
 * checks away and return MOE_ERR_UNSUPPORTED with *flags = 0.  For callers
 * that want their own inputs checked (the pages' engine states no such
 * interface). */
int moe_debug_take(uint32_t* flags);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
