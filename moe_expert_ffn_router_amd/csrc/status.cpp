// Status strings, the thread-local error message, and the expert record layout.
#include <stdarg.h>
#include <stdio.h>

#include "moe_internal.h"

namespace moe {

static thread_local char g_last_error[512] = {0};

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return MOE_OK;
}

static int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool layout_of(int fmt, int H, int I, Layout* o) {
  if (H < 128 || I < 128 || H > 16384 || I > 16384 || H % 128 || I % 128) return false;
  const int64_t h = H, i = I;
  int64_t sz[5] = {-1, -1, -1, -1, -1};  // w13, w13s, w2, w2s, ts
  switch (fmt) {
    case MOE_W_BF16: sz[0] = 2 * i * h * 2; sz[2] = h * i * 2; break;
    case MOE_W_MXFP4: sz[0] = i * h; sz[1] = 2 * i * h / 32; sz[2] = h * i / 2; sz[3] = h * i / 32; break;
    case MOE_W_NVFP4:
      sz[0] = i * h; sz[1] = 2 * i * h / 16; sz[2] = h * i / 2; sz[3] = h * i / 16; sz[4] = 12;
      break;
    case MOE_W_FP8_B128:
      sz[0] = 2 * i * h; sz[1] = (2 * i / 128) * (h / 128) * 4; sz[2] = h * i;
      sz[3] = (h / 128) * (i / 128) * 4;
      break;
    default: return false;
  }
  int64_t off[5], pos = 0, payload = 0;
  for (int s = 0; s < 5; ++s) {
    if (sz[s] < 0) { off[s] = -1; continue; }
    pos = round_up(pos, 256);
    off[s] = pos;
    pos += sz[s];
    payload += sz[s];
  }
  o->w13 = off[0]; o->w13s = off[1]; o->w2 = off[2]; o->w2s = off[3]; o->ts = off[4];
  o->payload = payload;
  o->stride = round_up(pos, 256);
  return true;
}

}  // namespace moe

extern "C" {

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    case MOE_ERR_CAPACITY: return "MOE_ERR_CAPACITY";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return moe::g_last_error; }

int moe_version(void) { return 1; }

int moe_debug_take(uint32_t* flags) {
  if (!flags) return moe::set_error(MOE_ERR_INVALID_ARG, "moe_debug_take: flags is NULL");
#ifdef MOE_DEBUG
  *flags = moe::dbg_take_ffn() | moe::dbg_take_decode() | moe::dbg_take_combine();
  return MOE_OK;
#else
  *flags = 0;
  return moe::set_error(MOE_ERR_UNSUPPORTED,
                        "moe_debug_take: release build (the bounds checks need -DMOE_DEBUG)");
#endif
}

int moe_expert_layout_query(int32_t fmt, int32_t H, int32_t I, moe_expert_layout* out) {
  moe::g_last_error[0] = 0;
  if (!out) return moe::set_error(MOE_ERR_INVALID_ARG, "moe_expert_layout_query: out is NULL");
  moe::Layout L;
  if (!moe::layout_of(fmt, H, I, &L))
    return moe::set_error(MOE_ERR_UNSUPPORTED,
                          "moe_expert_layout_query: fmt=%d H=%d I=%d unsupported (H, I multiples "
                          "of 128 in [128, 16384])", fmt, H, I);
  out->w13 = L.w13; out->w13_scale = L.w13s; out->w2 = L.w2; out->w2_scale = L.w2s;
  out->tensor_scale = L.ts; out->payload_bytes = L.payload; out->stride = L.stride;
  return MOE_OK;
}

}  // extern "C"
