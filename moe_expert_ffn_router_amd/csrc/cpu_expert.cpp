// Host (CPU) expert executor and the host-memory / PCIe bandwidth calibration
// (FreeToken guide, "MoE strategies": the cpu strategy computes a missed
// expert on the CPU from host memory instead of fetching it; hybrid splits a
// step's misses between fetching and CPU execution, run at the same time;
// "use ft bench bw to calibrate": the split comes from the measured host-
// memory and PCIe bandwidths of the real kernels).
//
// The executor reads expert records straight from the (pinned) host bank.
// Weights are decoded one row at a time into fp32 (exact for every format)
// and multiplied with fp32 activation rows; h = SiLU(g) * u is rounded to
// bf16 before the down projection and y to bf16 (the GPU path rounds at the
// same two places).  Work is split over a persistent thread pool by weight
// rows: each gate/up row produces one h column for every token row, each down
// row one output column; no floating-point result depends on the thread
// count (every dot product is one thread's, summed in a fixed order).
#include <math.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <new>
#include <thread>
#include <vector>

#include "moe_internal.h"

namespace {

// ---------------------------------------------------------------------------
// format decode (from the bit fields; the same definitions as the device's)
// ---------------------------------------------------------------------------
float e2m1_f(uint32_t c) {
  const uint32_t s = (c >> 3) & 1u, e = (c >> 1) & 3u, m = c & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
  return s ? -mag : mag;
}
float e4m3_f(uint32_t b) {
  const uint32_t s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  float mag;
  if (e == 0) mag = ldexpf((float)m, -9);
  else if (e == 15 && m == 7) mag = NAN;
  else mag = ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
  return s ? -mag : mag;
}
float e8m0_f(uint32_t b) { return b == 255 ? NAN : ldexpf(1.0f, (int)b - 127); }
float bf16_f(uint16_t v) {
  uint32_t u = (uint32_t)v << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}
uint16_t f_bf16(float f) {  // round to nearest even, NaN kept quiet
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

struct Tables {
  float e2m1[16], e4m3[256], e8m0[256], pair[256][2];
  Tables() {
    for (int i = 0; i < 16; ++i) e2m1[i] = e2m1_f(i);
    for (int i = 0; i < 256; ++i) {
      e4m3[i] = e4m3_f(i);
      e8m0[i] = e8m0_f(i);
      pair[i][0] = e2m1[i & 15];
      pair[i][1] = e2m1[i >> 4];
    }
  }
};
const Tables& tables() {
  static const Tables t;
  return t;
}

// Row n (K values) of a weight matrix -> fp32 out[K].
//   fmt BF16: w = bf16 [N][K]; MXFP4: codes [N][K/2] + E8M0 [N][K/32];
//   NVFP4: codes + E4M3 [N][K/16] times ts; FP8: E4M3 [N][K] + fp32 [N/128][K/128]
__attribute__((target("avx2,fma"))) void decode_row(int fmt, const uint8_t* w, const uint8_t* sc,
                                                     float ts, int n, int K, float* out) {
  const Tables& T = tables();
  switch (fmt) {
    case MOE_W_BF16: {
      const uint16_t* r = reinterpret_cast<const uint16_t*>(w) + (size_t)n * K;
      for (int i = 0; i < K; ++i) out[i] = bf16_f(r[i]);
      break;
    }
    case MOE_W_MXFP4: {
      const uint8_t* r = w + (size_t)n * (K / 2);
      const uint8_t* s = sc + (size_t)n * (K / 32);
      for (int b = 0; b < K / 32; ++b) {
        const float f = T.e8m0[s[b]];
        for (int i = 0; i < 16; ++i) {
          const uint8_t v = r[b * 16 + i];
          out[b * 32 + 2 * i] = T.pair[v][0] * f;
          out[b * 32 + 2 * i + 1] = T.pair[v][1] * f;
        }
      }
      break;
    }
    case MOE_W_NVFP4: {
      const uint8_t* r = w + (size_t)n * (K / 2);
      const uint8_t* s = sc + (size_t)n * (K / 16);
      for (int b = 0; b < K / 16; ++b) {
        const float f = T.e4m3[s[b]];  // code * block scale is exact; tensor scale once
        for (int i = 0; i < 8; ++i) {
          const uint8_t v = r[b * 8 + i];
          out[b * 16 + 2 * i] = (T.pair[v][0] * f) * ts;
          out[b * 16 + 2 * i + 1] = (T.pair[v][1] * f) * ts;
        }
      }
      break;
    }
    default: {  // FP8, 128 x 128 blocks
      const uint8_t* r = w + (size_t)n * K;
      const float* s = reinterpret_cast<const float*>(sc) + (size_t)(n / 128) * (K / 128);
      for (int b = 0; b < K / 128; ++b) {
        const float f = s[b];
        for (int i = 0; i < 128; ++i) out[b * 128 + i] = T.e4m3[r[b * 128 + i]] * f;
      }
      break;
    }
  }
}

__attribute__((target("avx2,fma"))) float dot(const float* a, const float* b, int K) {
  // 8 independent partial sums, combined in a fixed order
  float p[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int i = 0;
  for (; i + 8 <= K; i += 8)
    for (int j = 0; j < 8; ++j) p[j] = fmaf(a[i + j], b[i + j], p[j]);
  for (; i < K; ++i) p[0] = fmaf(a[i], b[i], p[0]);
  return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

// ---------------------------------------------------------------------------
// persistent thread pool: run(n_tasks, fn) calls fn(task) for every task on the
// pool's threads and the caller's, and returns once every pool thread has
// finished this round (so no thread still reads the round's function or
// counters when the next round sets them)
// ---------------------------------------------------------------------------
struct Pool {
  std::vector<std::thread> th;
  std::mutex mu;
  std::condition_variable cv, done_cv;
  std::function<void(int)> fn;
  int n_tasks = 0;
  std::atomic<int> next{0};
  int finished = 0;  // pool threads done with the current round
  uint64_t gen = 0;
  bool stop = false;

  explicit Pool(int n) {
    for (int i = 0; i < n; ++i) th.emplace_back([this] { loop(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu);
      stop = true;
    }
    cv.notify_all();
    for (auto& t : th) t.join();
  }
  void work() {
    for (int t; (t = next.fetch_add(1)) < n_tasks;) fn(t);
  }
  void loop() {
    uint64_t seen = 0;
    for (;;) {
      {
        std::unique_lock<std::mutex> lk(mu);
        cv.wait(lk, [&] { return stop || gen != seen; });
        if (stop) return;
        seen = gen;
      }
      work();
      {
        std::lock_guard<std::mutex> lk(mu);
        if (++finished == (int)th.size()) done_cv.notify_all();
      }
    }
  }
  void run(int tasks, std::function<void(int)> f) {
    {
      std::lock_guard<std::mutex> lk(mu);
      fn = std::move(f);
      n_tasks = tasks;
      next.store(0);
      finished = 0;
      ++gen;
    }
    cv.notify_all();
    work();
    std::unique_lock<std::mutex> lk(mu);
    done_cv.wait(lk, [&] { return finished == (int)th.size(); });
  }
};

}  // namespace

struct moe_cpu_pool {
  Pool pool;
  int threads;
  explicit moe_cpu_pool(int n) : pool(n - 1), threads(n) {}
};

using moe::set_error;

extern "C" int moe_cpu_pool_create(moe_cpu_pool_t* out, int32_t threads) {
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "moe_cpu_pool_create: out is NULL");
  *out = nullptr;
  if (threads < 1 || threads > 1024)
    return set_error(MOE_ERR_INVALID_ARG, "moe_cpu_pool_create: threads %d not in [1, 1024]",
                     threads);
  if (!__builtin_cpu_supports("avx2") || !__builtin_cpu_supports("fma"))
    return set_error(MOE_ERR_UNSUPPORTED, "moe_cpu_pool_create: the CPU executor needs AVX2 and FMA");
  moe_cpu_pool* p = new (std::nothrow) moe_cpu_pool(threads);
  if (!p) return set_error(MOE_ERR_INVALID_ARG, "moe_cpu_pool_create: out of host memory");
  *out = p;
  return MOE_OK;
}

extern "C" void moe_cpu_pool_destroy(moe_cpu_pool_t p) { delete p; }

extern "C" int moe_cpu_expert_ffn(moe_cpu_pool_t pool, const moe_experts* W,
                                  const int32_t* experts, int32_t n_experts, const uint16_t* x,
                                  int32_t T, int32_t k, const int32_t* offsets,
                                  const int32_t* sorted_idx, uint16_t* y_perm) {
  const char* who = "moe_cpu_expert_ffn";
  if (!pool || !W) return set_error(MOE_ERR_INVALID_ARG, "%s: null pool or W", who);
  moe::Layout Lo;
  if (W->E < 1 || !moe::layout_of(W->fmt, W->H, W->I, &Lo))
    return set_error(MOE_ERR_UNSUPPORTED, "%s: fmt=%d H=%d I=%d", who, W->fmt, W->H, W->I);
  if (!W->base || W->stride < Lo.stride || n_experts < 0 || T < 0 || k < 1 ||
      (n_experts > 0 && (!experts || !x || !offsets || !sorted_idx || !y_perm)))
    return set_error(MOE_ERR_INVALID_ARG, "%s: bad argument", who);
  const int H = W->H, I = W->I, A = T * k;
  for (int i = 0; i < n_experts; ++i) {
    const int e = experts[i];
    if (e < 0 || e >= W->E || offsets[e] < 0 || offsets[e + 1] < offsets[e] || offsets[e + 1] > A)
      return set_error(MOE_ERR_INVALID_ARG, "%s: expert %d or its offsets out of range", who, e);
    for (int p = offsets[e]; p < offsets[e + 1]; ++p)
      if (sorted_idx[p] < 0 || sorted_idx[p] >= A)
        return set_error(MOE_ERR_INVALID_ARG, "%s: sorted_idx[%d] out of range", who, p);
  }
  Pool& P = pool->pool;
  constexpr int kRowsPerTask = 16;
  std::vector<float> xs, hs;  // activation rows and h rows of one expert, fp32
  for (int i = 0; i < n_experts; ++i) {
    const int e = experts[i];
    const int p0 = offsets[e], R = offsets[e + 1] - p0;
    if (R == 0) continue;
    const uint8_t* rec = static_cast<const uint8_t*>(W->base) + (size_t)e * W->stride;
    const float* ts = Lo.ts >= 0 ? reinterpret_cast<const float*>(rec + Lo.ts) : nullptr;
    xs.resize((size_t)R * H);
    hs.resize((size_t)R * I);
    for (int r = 0; r < R; ++r) {
      const uint16_t* src = x + (size_t)(sorted_idx[p0 + r] / k) * H;
      for (int c = 0; c < H; ++c) xs[(size_t)r * H + c] = bf16_f(src[c]);
    }
    // gate/up: task = kRowsPerTask h columns (their gate and up rows)
    const uint8_t* w13 = rec + Lo.w13;
    const uint8_t* s13 = Lo.w13s >= 0 ? rec + Lo.w13s : nullptr;
    P.run((I + kRowsPerTask - 1) / kRowsPerTask, [&](int t) {
      std::vector<float> g(H), u(H);
      for (int c = t * kRowsPerTask; c < (t + 1) * kRowsPerTask && c < I; ++c) {
        decode_row(W->fmt, w13, s13, ts ? ts[0] : 1.0f, c, H, g.data());
        decode_row(W->fmt, w13, s13, ts ? ts[1] : 1.0f, I + c, H, u.data());
        for (int r = 0; r < R; ++r) {
          const float gv = dot(xs.data() + (size_t)r * H, g.data(), H);
          const float uv = dot(xs.data() + (size_t)r * H, u.data(), H);
          hs[(size_t)r * I + c] = bf16_f(f_bf16(gv / (1.0f + expf(-gv)) * uv));
        }
      }
    });
    // down: task = kRowsPerTask output columns
    const uint8_t* w2 = rec + Lo.w2;
    const uint8_t* s2 = Lo.w2s >= 0 ? rec + Lo.w2s : nullptr;
    P.run((H + kRowsPerTask - 1) / kRowsPerTask, [&](int t) {
      std::vector<float> d(I);
      for (int c = t * kRowsPerTask; c < (t + 1) * kRowsPerTask && c < H; ++c) {
        decode_row(W->fmt, w2, s2, ts ? ts[2] : 1.0f, c, I, d.data());
        for (int r = 0; r < R; ++r)
          y_perm[(size_t)(p0 + r) * H + c] = f_bf16(dot(hs.data() + (size_t)r * I, d.data(), I));
      }
    });
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Calibration: the pinned host -> device copy rate of expert records (the
// fetch path) and the CPU executor's rate on one-row experts (its weight
// stream), both in expert-record bytes per second.
// ---------------------------------------------------------------------------
extern "C" int moe_bench_bw(moe_cpu_pool_t pool, const moe_experts* bank_W, void* pool_dev,
                            int32_t n_records, moe_stream_t stream, double threshold,
                            moe_bw_profile* out) {
  const char* who = "moe_bench_bw";
  if (!pool || !bank_W || !pool_dev || !out || n_records < 1 || n_records > bank_W->E)
    return set_error(MOE_ERR_INVALID_ARG, "%s: bad argument", who);
  moe::Layout Lo;
  if (!moe::layout_of(bank_W->fmt, bank_W->H, bank_W->I, &Lo) || bank_W->stride < Lo.stride)
    return set_error(MOE_ERR_UNSUPPORTED, "%s: fmt=%d H=%d I=%d", who, bank_W->fmt, bank_W->H,
                     bank_W->I);
  const size_t rb = (size_t)bank_W->stride;
  const uint8_t* bank = static_cast<const uint8_t*>(bank_W->base);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // fetch path: n_records record copies on `stream`, timed with events
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
    return set_error(MOE_ERR_HIP, "%s: hipEventCreate failed", who);
  hipError_t err = hipMemcpyAsync(pool_dev, bank, rb, hipMemcpyHostToDevice, s);  // warm
  if (err == hipSuccess) err = hipEventRecord(e0, s);
  for (int i = 0; err == hipSuccess && i < n_records; ++i)
    err = hipMemcpyAsync(static_cast<uint8_t*>(pool_dev) + (size_t)i * rb, bank + (size_t)i * rb,
                         rb, hipMemcpyHostToDevice, s);
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err == hipSuccess) err = hipEventSynchronize(e1);
  float ms = 0.f;
  if (err == hipSuccess) err = hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", who, hipGetErrorString(err));
  const double h2d = (double)n_records * rb / (ms * 1e-3);
  // CPU path: each record as an expert with one token row
  const int H = bank_W->H;
  std::vector<uint16_t> x((size_t)H, 0x3f80);  // 1.0
  std::vector<uint16_t> y((size_t)H);
  std::vector<int32_t> ids(n_records), offs(bank_W->E + 1, 0), sidx(1, 0);
  for (int i = 0; i < n_records; ++i) ids[i] = i;
  double best = 0.0;
  for (int rep = 0; rep < 3; ++rep) {
    const auto t0 = std::chrono::steady_clock::now();
    for (int i = 0; i < n_records; ++i) {
      for (int e = 0; e <= bank_W->E; ++e) offs[e] = e > i ? 1 : 0;
      const int st = moe_cpu_expert_ffn(pool, bank_W, ids.data() + i, 1, x.data(), 1, 1,
                                        offs.data(), sidx.data(), y.data());
      if (st) return st;
    }
    const double sec = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
    const double rate = (double)n_records * Lo.payload / sec;
    best = rate > best ? rate : best;
  }
  out->h2d_bytes_per_s = h2d * (double)Lo.payload / (double)rb;  // record payload per second
  out->cpu_bytes_per_s = best;
  out->threshold = threshold;
  out->hybrid_recommended = best >= threshold * out->h2d_bytes_per_s ? 1 : 0;
  out->fetch_fraction = out->h2d_bytes_per_s / (out->h2d_bytes_per_s + best);
  return MOE_OK;
}
