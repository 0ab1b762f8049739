// C ABI of libattn (declared in include/attn.h): argument validation and kernel dispatch.
// Every check below runs on the host before the first HIP call, so invalid calls enqueue nothing.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn.h"
#include "launch.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 40;  // far above any device memory
constexpr int64_t kMaxGrid = 0x7fffffff;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Checks B, H, T >= 1 and that B*H*T*d elements stay addressable; returns the element count.
int check_shape(int B, int H, int T, int d, int64_t* n) {
  if (B < 1 || H < 1 || T < 1) return ATTN_ERR_SHAPE;
  const int64_t bh = (int64_t)B * H;
  if (bh > 0x7fffffff) return ATTN_ERR_SHAPE;
  const int64_t rows = bh * T;
  if (rows > kMaxElems / 256) return ATTN_ERR_SHAPE;
  *n = rows * d;
  return ATTN_OK;
}

int elem_bytes(int dtype) { return dtype == ATTN_BF16 ? 2 : 4; }

}  // namespace

extern "C" {

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "B, H and T must be >= 1 and the tensor must fit in memory";
    case ATTN_ERR_HEAD_DIM: return "head dim not supported for this entry point and dtype";
    case ATTN_ERR_DTYPE: return "unknown dtype (expected ATTN_BF16 or ATTN_F32)";
    case ATTN_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case ATTN_ERR_WINDOW: return "causal must be 0 or 1; window must be >= -1 and -1 when causal == 0";
    case ATTN_ERR_ALIAS: return "an output overlaps an input it must not overlap";
    case ATTN_ERR_ARG: return "argument out of range";
    case ATTN_ERR_HIP: return "HIP launch failed";
    default: return "unknown attn status code";
  }
}

int attn_version(void) { return 100; }

int attn_sssl_windows(int T, int n_layer, const char* pattern, int* windows) {
  if (pattern == nullptr || windows == nullptr) return ATTN_ERR_NULL;
  if (T < 1) return ATTN_ERR_SHAPE;
  if (n_layer < 1) return ATTN_ERR_ARG;
  const size_t len = strnlen(pattern, 4096);
  if (len == 0 || len == 4096) return ATTN_ERR_ARG;
  for (size_t i = 0; i < len; ++i) {
    const char c = pattern[i];
    if (c != 'S' && c != 's' && c != 'L' && c != 'l') return ATTN_ERR_ARG;
  }
  // Layer l takes pattern[l % len]; 'L' is the full length, 'S' half of it; the last layer is
  // always full ("Подробный технический разбор реализации Autoresearch", habr.com, train.py
  // listing, GPT._compute_window_sizes).
  for (int l = 0; l < n_layer; ++l) {
    const char c = pattern[l % len];
    windows[l] = (c == 'L' || c == 'l') ? T : T / 2;
  }
  windows[n_layer - 1] = T;
  return ATTN_OK;
}

int attn_rope_table(float* cos_tab, float* sin_tab, int T, int d, double base, void* stream) {
  if (cos_tab == nullptr || sin_tab == nullptr) return ATTN_ERR_NULL;
  if (T < 1) return ATTN_ERR_SHAPE;
  if (d < 2 || d > 256 || (d & 1)) return ATTN_ERR_HEAD_DIM;
  if (!(base > 1.0) || !isfinite(base)) return ATTN_ERR_ARG;
  if (!aligned16(cos_tab) || !aligned16(sin_tab)) return ATTN_ERR_ALIGN;
  const int64_t bytes = (int64_t)T * (d / 2) * 4;
  if (overlap(cos_tab, bytes, sin_tab, bytes)) return ATTN_ERR_ALIAS;
  if (((int64_t)T * (d / 2) + 255) / 256 > kMaxGrid) return ATTN_ERR_SHAPE;
  hipError_t e = attn::launch_rope_table(cos_tab, sin_tab, T, d, base, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out, const float* cos_tab,
                     const float* sin_tab, int B, int H, int T, int d, float eps, int dtype,
                     void* stream) {
  // q and q_out are both given or both NULL (then only k is processed).
  if (!k || !k_out || !cos_tab || !sin_tab || (q == nullptr) != (q_out == nullptr))
    return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  int64_t n = 0;
  if (int rc = check_shape(B, H, T, d, &n)) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ATTN_ERR_ARG;
  if (2 * (int64_t)B * H > 0x7fffffff) return ATTN_ERR_SHAPE;  // q's and k's heads, as int
  if ((q && !aligned16(q)) || !aligned16(k) || (q_out && !aligned16(q_out)) || !aligned16(k_out) ||
      !aligned16(cos_tab) || !aligned16(sin_tab))
    return ATTN_ERR_ALIGN;
  const int64_t bytes = n * elem_bytes(dtype);
  if (k_out != k && overlap(k_out, bytes, k, bytes)) return ATTN_ERR_ALIAS;
  if (q != nullptr) {
    if (q_out != q && overlap(q_out, bytes, q, bytes)) return ATTN_ERR_ALIAS;
    if (overlap(q_out, bytes, k, bytes) || overlap(k_out, bytes, q, bytes) ||
        overlap(q_out, bytes, k_out, bytes))
      return ATTN_ERR_ALIAS;
  }
  hipError_t e = attn::launch_qknorm_rope(q, k, q_out, k_out, cos_tab, sin_tab, B, H, T, d, eps,
                                          dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
             int T, int d, int window, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (dtype == ATTN_BF16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype == ATTN_F32 && d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  int64_t n = 0;
  if (int rc = check_shape(B, H, T, d, &n)) return rc;
  if (causal != 0 && causal != 1) return ATTN_ERR_WINDOW;
  if (window < -1 || (causal == 0 && window != -1)) return ATTN_ERR_WINDOW;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  const int64_t bytes = n * elem_bytes(dtype);
  if (overlap(out, bytes, q, bytes) || overlap(out, bytes, k, bytes) ||
      overlap(out, bytes, v, bytes))
    return ATTN_ERR_ALIAS;
  const int64_t bh = (int64_t)B * H;
  if (lse != nullptr) {
    const int64_t lbytes = bh * T * 4;
    if (overlap(lse, lbytes, q, bytes) || overlap(lse, lbytes, k, bytes) ||
        overlap(lse, lbytes, v, bytes) || overlap(lse, lbytes, out, bytes))
      return ATTN_ERR_ALIAS;
  }
  // One head's [T][d] slab (plus a query block of padding rows) must stay below 2^31 bytes: the
  // bf16 kernel addresses it through 32-bit buffer offsets.
  if (dtype == ATTN_BF16 && ((int64_t)T + 128) * d * 2 >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
  const int64_t tiles = (dtype == ATTN_BF16) ? (T + 127) / 128 : (T + 63) / 64;
  if (bh * tiles > kMaxGrid) return ATTN_ERR_SHAPE;
  hipError_t e;
  if (dtype == ATTN_BF16)
    e = attn::launch_attn_fwd_bf16(q, k, v, out, lse, B, H, T, d, window, causal,
                                   (hipStream_t)stream);
  else
    e = attn::launch_attn_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)out,
                                  lse, B, H, T, d, window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

namespace {

// Checks shared by attn_fwd_qnorm and attn_fwd_qknorm (k here is the tensor the attention
// kernel reads as keys).
int check_qnorm_args(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                     int T, int d, float eps, int window, int causal, int dtype, int64_t* n) {
  if (!q || !k || !v || !out || !cos_tab || !sin_tab) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (int rc = check_shape(B, H, T, d, n)) return rc;
  if (causal != 0 && causal != 1) return ATTN_ERR_WINDOW;
  if (window < -1 || (causal == 0 && window != -1)) return ATTN_ERR_WINDOW;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ATTN_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(cos_tab) ||
      !aligned16(sin_tab))
    return ATTN_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  const int64_t bytes = *n * 2;
  if (overlap(out, bytes, q, bytes) || overlap(out, bytes, k, bytes) ||
      overlap(out, bytes, v, bytes))
    return ATTN_ERR_ALIAS;
  const int64_t bh = (int64_t)B * H;
  if (lse != nullptr) {
    const int64_t lbytes = bh * T * 4;
    if (overlap(lse, lbytes, q, bytes) || overlap(lse, lbytes, k, bytes) ||
        overlap(lse, lbytes, v, bytes) || overlap(lse, lbytes, out, bytes))
      return ATTN_ERR_ALIAS;
  }
  // 32-bit buffer offsets: one head's slab plus a query block, and the rotation tables.
  if (((int64_t)T + 128) * d * 2 >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
  if (bh * ((T + 127) / 128) > kMaxGrid) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

int attn_fwd_qnorm(const void* q, const void* k, const void* v, void* out, float* lse,
                   const float* cos_tab, const float* sin_tab, int B, int H, int T, int d,
                   float eps, int window, int causal, int dtype, void* stream) {
  int64_t n = 0;
  if (int rc = check_qnorm_args(q, k, v, out, lse, cos_tab, sin_tab, B, H, T, d, eps, window,
                                causal, dtype, &n))
    return rc;
  const hipError_t e = attn::launch_attn_fwd_bf16_qknorm(q, k, v, out, lse, cos_tab, sin_tab, eps,
                                                         B, H, T, d, window, causal,
                                                         (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* k_work, void* out,
                    float* lse, const float* cos_tab, const float* sin_tab, int B, int H, int T,
                    int d, float eps, int window, int causal, int dtype, void* stream) {
  if (!k_work) return ATTN_ERR_NULL;
  int64_t n = 0;
  if (int rc = check_qnorm_args(q, k_work, v, out, lse, cos_tab, sin_tab, B, H, T, d, eps,
                                window, causal, dtype, &n))
    return rc;
  if (!k) return ATTN_ERR_NULL;
  if (!aligned16(k)) return ATTN_ERR_ALIGN;
  if (2 * (int64_t)B * H > 0x7fffffff) return ATTN_ERR_SHAPE;
  const int64_t bytes = n * 2;
  if (k_work != k && overlap(k_work, bytes, k, bytes)) return ATTN_ERR_ALIAS;
  if (overlap(k_work, bytes, q, bytes) || overlap(k_work, bytes, v, bytes) ||
      overlap(out, bytes, k, bytes))
    return ATTN_ERR_ALIAS;
  if (lse != nullptr && overlap(lse, (int64_t)B * H * T * 4, k, bytes)) return ATTN_ERR_ALIAS;
  hipError_t e = attn::launch_qknorm_rope(nullptr, k, nullptr, k_work, cos_tab, sin_tab, B, H, T,
                                          d, eps, ATTN_BF16, (hipStream_t)stream);
  if (e == hipSuccess)
    e = attn::launch_attn_fwd_bf16_qknorm(q, k_work, v, out, lse, cos_tab, sin_tab, eps, B, H, T,
                                          d, window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
