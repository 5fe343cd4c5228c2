// The always-on shared expert: a dense SwiGLU FFN over every token, with no
// routing or permutation, so its two products are plain bf16 GEMMs and go to
// hipBLASLt (fp32 accumulation); the SiLU(gate)*up step between them is the
// one kernel of this file.
//   gate/up:  G[T][2I] fp32 = x[T][H] * W13^T    (W13 [2I][H]: gate rows, then up rows)
//   h:        h[T][I] = bf16( SiLU(G[:, i]) * G[:, I + i] )
//   down:     y[T][H] = bf16( h * W2^T )          (W2 [H][I])
// In hipBLASLt's column-major terms each product is D = op(A) * B with A the
// weight matrix (stored K-major, so op = transpose) and B the activations.
#include <hipblaslt/hipblaslt.h>

#include <mutex>

#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void swiglu_rows_kernel(const float* __restrict__ g, int T, int I,
                                                          uint16_t* __restrict__ h) {
  const size_t n = (size_t)T * I;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t t = i / I, c = i - t * I;
    const float gv = g[t * 2 * I + c], uv = g[t * 2 * I + I + c];
    h[i] = f32_to_bf16_rne(gv / (1.0f + expf(-gv)) * uv);
  }
}

namespace {

constexpr size_t kLtWorkspace = 64u << 20;  // hipBLASLt's own scratch inside the caller's workspace
constexpr int kMaxDevices = 64;

std::mutex g_mu;
hipblasLtHandle_t g_handle[kMaxDevices] = {};

hipblasLtHandle_t handle_for_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS)
    g_handle[dev] = nullptr;
  return g_handle[dev];
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// D[n_out][T] (column-major, ld n_out) = op_T(Wt: K x n_out, ld K) * X (K x T, ld K)
int lt_gemm(hipblasLtHandle_t h, const void* w, const void* x, void* d, hipDataType d_type,
            int n_out, int T, int K, void* lt_ws, hipStream_t s, const char* what) {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  int st = MOE_OK;
  const hipblasOperation_t opT = HIPBLAS_OP_T, opN = HIPBLAS_OP_N;
  const uint64_t wsb = kLtWorkspace;
  const float alpha = 1.0f, beta = 0.0f;
  hipblasLtMatmulHeuristicResult_t res{};
  int n_res = 0;
  if (hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opT, sizeof(opT)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opN, sizeof(opN)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, K, n_out, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, K, T, K) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&ld, d_type, n_out, T, n_out) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                            sizeof(wsb)) != HIPBLAS_STATUS_SUCCESS) {
    st = set_error(MOE_ERR_HIP, "%s: hipBLASLt descriptor set-up failed", what);
  } else if (hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, 1, &res, &n_res) !=
                 HIPBLAS_STATUS_SUCCESS ||
             n_res < 1) {
    st = set_error(MOE_ERR_UNSUPPORTED, "%s: hipBLASLt has no algorithm for %d x %d x %d", what,
                   n_out, T, K);
  } else if (hipblasLtMatmul(h, desc, &alpha, w, la, x, lb, &beta, d, ld, d, ld, &res.algo, lt_ws,
                             kLtWorkspace, s) != HIPBLAS_STATUS_SUCCESS) {
    st = set_error(MOE_ERR_HIP, "%s: hipblasLtMatmul failed", what);
  }
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (desc) hipblasLtMatmulDescDestroy(desc);
  return st;
}

}  // namespace
}  // namespace moe

using namespace moe;

// Workspace: G fp32 [T][2I] | h bf16 [T][I] | hipBLASLt scratch (64 MiB).
extern "C" size_t moe_shared_ffn_workspace(const moe_experts* W, int32_t T) {
  if (!W || T < 0) return 0;
  return align256((size_t)T * 2 * W->I * 4) + align256((size_t)T * W->I * 2) + kLtWorkspace;
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
  hipblasLtHandle_t h = handle_for_device();
  if (!h) return set_error(MOE_ERR_HIP, "moe_shared_ffn: hipblasLtCreate failed");
  const int H = W->H, I = W->I;
  const uint8_t* rec = static_cast<const uint8_t*>(W->base);  // expert 0
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* g = reinterpret_cast<float*>(wsb);
  uint16_t* hb = reinterpret_cast<uint16_t*>(wsb + align256((size_t)T * 2 * I * 4));
  void* lt_ws = wsb + align256((size_t)T * 2 * I * 4) + align256((size_t)T * I * 2);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int st = lt_gemm(h, rec + Lo.w13, x, g, HIP_R_32F, 2 * I, T, H, lt_ws, s, "moe_shared_ffn gate/up");
  if (st) return st;
  const size_t n = (size_t)T * I;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  swiglu_rows_kernel<<<grid, 256, 0, s>>>(g, T, I, hb);
  if ((st = check_launch("moe_shared_ffn"))) return st;
  return lt_gemm(h, rec + Lo.w2, hb, y, HIP_R_16BF, H, T, I, lt_ws, s, "moe_shared_ffn down");
}
