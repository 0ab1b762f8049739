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
constexpr int64_t kMaxItems = kMaxGrid;  // work items (workgroups) of one attention launch

static_assert(attn::kDecodeScratchBytes == ATTN_DECODE_SCRATCH_BYTES,
              "the header states the decode scratch size");

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Validates one call's shape: B, H, H_kv, T >= 1, H_kv divides H, a known layout, and element
// counts that stay addressable. Fills dm and the element counts of q (and out) and of k (and v).
int check_dims(int B, int H, int H_kv, int T, int d, int layout, attn::Dims* dm, int64_t* n_q,
               int64_t* n_kv) {
  if (B < 1 || H < 1 || H_kv < 1 || T < 1) return ATTN_ERR_SHAPE;
  if (H % H_kv != 0) return ATTN_ERR_SHAPE;
  if (layout != ATTN_LAYOUT_BHTD && layout != ATTN_LAYOUT_BTHD) return ATTN_ERR_ARG;
  const int64_t bh = (int64_t)B * H;
  if (bh > 0x7fffffff) return ATTN_ERR_SHAPE;
  const int64_t rows = bh * T;
  if (rows > kMaxElems / 256) return ATTN_ERR_SHAPE;
  // Row strides of the [B][T][H][d] order (H * d elements) stay below 2^24, so that the offsets
  // of a block of up to 128 rows fit an int.
  if ((int64_t)H * d >= (int64_t(1) << 24)) return ATTN_ERR_SHAPE;
  *n_q = rows * d;
  *n_kv = (int64_t)B * H_kv * T * d;
  *dm = attn::Dims{B, H, H_kv, T, d, layout};
  return ATTN_OK;
}

// Bytes between consecutive rows (tokens) of one head of q and of k.
int64_t q_row_bytes(const attn::Dims& dm, int eb) {
  return (int64_t)(dm.layout == ATTN_LAYOUT_BTHD ? dm.H * dm.d : dm.d) * eb;
}
int64_t kv_row_bytes(const attn::Dims& dm, int eb) {
  return (int64_t)(dm.layout == ATTN_LAYOUT_BTHD ? dm.H_kv * dm.d : dm.d) * eb;
}

// The bf16 attention kernels address one head's rows (plus a query block of padding rows)
// through 32-bit buffer offsets: (T + 128) row strides must stay below 2^31 bytes.
bool slab_fits(const attn::Dims& dm) {
  const int64_t rs = q_row_bytes(dm, 2) > kv_row_bytes(dm, 2) ? q_row_bytes(dm, 2)
                                                               : kv_row_bytes(dm, 2);
  return ((int64_t)dm.T + 128) * rs < (int64_t(1) << 31);
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
    case ATTN_ERR_SCRATCH:
      return "the call needs more scratch than the library's fixed device array holds";
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

int attn_qknorm_rope_ex(const void* q, const void* k, void* q_out, void* k_out,
                        const float* cos_tab, const float* sin_tab, int B, int H, int H_kv, int T,
                        int d, int layout, float eps, int dtype, void* stream) {
  // q and q_out are both given or both NULL (then only k is processed).
  if (!k || !k_out || !cos_tab || !sin_tab || (q == nullptr) != (q_out == nullptr))
    return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H, H_kv, T, d, layout, &dm, &n_q, &n_kv)) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ATTN_ERR_ARG;
  if (2 * (int64_t)B * H > 0x7fffffff) return ATTN_ERR_SHAPE;  // q's and k's heads, as int
  if ((q && !aligned16(q)) || !aligned16(k) || (q_out && !aligned16(q_out)) || !aligned16(k_out) ||
      !aligned16(cos_tab) || !aligned16(sin_tab))
    return ATTN_ERR_ALIGN;
  const int64_t qb = n_q * elem_bytes(dtype), kb = n_kv * elem_bytes(dtype);
  if (k_out != k && overlap(k_out, kb, k, kb)) return ATTN_ERR_ALIAS;
  if (q != nullptr) {
    if (q_out != q && overlap(q_out, qb, q, qb)) return ATTN_ERR_ALIAS;
    if (overlap(q_out, qb, k, kb) || overlap(k_out, kb, q, qb) || overlap(q_out, qb, k_out, kb))
      return ATTN_ERR_ALIAS;
  }
  hipError_t e = attn::launch_qknorm_rope(q, k, q_out, k_out, cos_tab, sin_tab, dm, eps, dtype,
                                          (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out, const float* cos_tab,
                     const float* sin_tab, int B, int H, int T, int d, float eps, int dtype,
                     void* stream) {
  return attn_qknorm_rope_ex(q, k, q_out, k_out, cos_tab, sin_tab, B, H, H, T, d,
                             ATTN_LAYOUT_BHTD, eps, dtype, stream);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                int H_kv, int T, int d, int layout, int window, int causal, int dtype,
                void* stream) {
  if (!q || !k || !v || !out) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (dtype == ATTN_BF16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype == ATTN_F32 && d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H, H_kv, T, d, layout, &dm, &n_q, &n_kv)) return rc;
  if (causal != 0 && causal != 1) return ATTN_ERR_WINDOW;
  if (window < -1 || (causal == 0 && window != -1)) return ATTN_ERR_WINDOW;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return ATTN_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  const int64_t qb = n_q * elem_bytes(dtype), kb = n_kv * elem_bytes(dtype);
  if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb))
    return ATTN_ERR_ALIAS;
  const int64_t bh = (int64_t)B * H;
  if (lse != nullptr) {
    const int64_t lbytes = bh * T * 4;
    if (overlap(lse, lbytes, q, qb) || overlap(lse, lbytes, k, kb) ||
        overlap(lse, lbytes, v, kb) || overlap(lse, lbytes, out, qb))
      return ATTN_ERR_ALIAS;
  }
  if (dtype == ATTN_BF16 && !slab_fits(dm)) return ATTN_ERR_SHAPE;
  const int64_t tiles = (dtype == ATTN_BF16) ? (T + 127) / 128 : (T + 63) / 64;
  if (bh * tiles > kMaxItems) return ATTN_ERR_SHAPE;
  hipError_t e;
  if (dtype == ATTN_BF16)
    e = attn::launch_attn_fwd_bf16(q, k, v, out, lse, dm, window, causal, (hipStream_t)stream);
  else
    e = attn::launch_attn_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)out,
                                  lse, dm, window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
             int T, int d, int window, int causal, int dtype, void* stream) {
  return attn_fwd_ex(q, k, v, out, lse, B, H, H, T, d, ATTN_LAYOUT_BHTD, window, causal, dtype,
                     stream);
}

namespace {

// Checks shared by attn_fwd_qnorm_ex and attn_fwd_qknorm_ex (k here is the tensor the attention
// kernel reads as keys).
int check_qnorm_args(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                     int H_kv, int T, int d, int layout, float eps, int window, int causal,
                     int dtype, attn::Dims* dm, int64_t* n_q, int64_t* n_kv) {
  if (!q || !k || !v || !out || !cos_tab || !sin_tab) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (int rc = check_dims(B, H, H_kv, T, d, layout, dm, n_q, n_kv)) return rc;
  if (causal != 0 && causal != 1) return ATTN_ERR_WINDOW;
  if (window < -1 || (causal == 0 && window != -1)) return ATTN_ERR_WINDOW;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ATTN_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(cos_tab) ||
      !aligned16(sin_tab))
    return ATTN_ERR_ALIGN;
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_ALIGN;
  const int64_t qb = *n_q * 2, kb = *n_kv * 2;
  if (overlap(out, qb, q, qb) || overlap(out, qb, k, kb) || overlap(out, qb, v, kb))
    return ATTN_ERR_ALIAS;
  const int64_t bh = (int64_t)B * H;
  if (lse != nullptr) {
    const int64_t lbytes = bh * T * 4;
    if (overlap(lse, lbytes, q, qb) || overlap(lse, lbytes, k, kb) ||
        overlap(lse, lbytes, v, kb) || overlap(lse, lbytes, out, qb))
      return ATTN_ERR_ALIAS;
  }
  if (!slab_fits(*dm)) return ATTN_ERR_SHAPE;
  if (bh * ((T + 127) / 128) > kMaxItems) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

int attn_fwd_qnorm_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                      const float* cos_tab, const float* sin_tab, int B, int H, int H_kv, int T,
                      int d, int layout, float eps, int window, int causal, int dtype,
                      void* stream) {
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_qnorm_args(q, k, v, out, lse, cos_tab, sin_tab, B, H, H_kv, T, d, layout,
                                eps, window, causal, dtype, &dm, &n_q, &n_kv))
    return rc;
  const hipError_t e = attn::launch_attn_fwd_bf16_qknorm(q, k, v, out, lse, cos_tab, sin_tab, eps,
                                                         dm, window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_qnorm(const void* q, const void* k, const void* v, void* out, float* lse,
                   const float* cos_tab, const float* sin_tab, int B, int H, int T, int d,
                   float eps, int window, int causal, int dtype, void* stream) {
  return attn_fwd_qnorm_ex(q, k, v, out, lse, cos_tab, sin_tab, B, H, H, T, d, ATTN_LAYOUT_BHTD,
                           eps, window, causal, dtype, stream);
}

int attn_fwd_qknorm_ex(const void* q, const void* k, const void* v, void* k_work, void* out,
                       float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                       int H_kv, int T, int d, int layout, float eps, int window, int causal,
                       int dtype, void* stream) {
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (!k_work) {
    // k normalised and rotated inside the attention kernel, not written (d <= 64)
    if (int rc = check_qnorm_args(q, k, v, out, lse, cos_tab, sin_tab, B, H, H_kv, T, d, layout,
                                  eps, window, causal, dtype, &dm, &n_q, &n_kv))
      return rc;
    if (d > 64) return ATTN_ERR_NULL;
    const hipError_t e = attn::launch_attn_fwd_bf16_qknorm_kin(
        q, k, v, out, lse, cos_tab, sin_tab, eps, dm, window, causal, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  if (int rc = check_qnorm_args(q, k_work, v, out, lse, cos_tab, sin_tab, B, H, H_kv, T, d,
                                layout, eps, window, causal, dtype, &dm, &n_q, &n_kv))
    return rc;
  if (!k) return ATTN_ERR_NULL;
  if (!aligned16(k)) return ATTN_ERR_ALIGN;
  if (2 * (int64_t)B * H > 0x7fffffff) return ATTN_ERR_SHAPE;
  const int64_t qb = n_q * 2, kb = n_kv * 2;
  if (k_work != k && overlap(k_work, kb, k, kb)) return ATTN_ERR_ALIAS;
  if (overlap(k_work, kb, q, qb) || overlap(k_work, kb, v, kb) || overlap(out, qb, k, kb))
    return ATTN_ERR_ALIAS;
  if (lse != nullptr && overlap(lse, (int64_t)B * H * T * 4, k, kb)) return ATTN_ERR_ALIAS;
  hipError_t e = attn::launch_qknorm_rope(nullptr, k, nullptr, k_work, cos_tab, sin_tab, dm, eps,
                                          ATTN_BF16, (hipStream_t)stream);
  if (e == hipSuccess)
    e = attn::launch_attn_fwd_bf16_qknorm(q, k_work, v, out, lse, cos_tab, sin_tab, eps, dm,
                                          window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* k_work, void* out,
                    float* lse, const float* cos_tab, const float* sin_tab, int B, int H, int T,
                    int d, float eps, int window, int causal, int dtype, void* stream) {
  return attn_fwd_qknorm_ex(q, k, v, k_work, out, lse, cos_tab, sin_tab, B, H, H, T, d,
                            ATTN_LAYOUT_BHTD, eps, window, causal, dtype, stream);
}

// ---------------------------------------------------------------------------------------------
// Value-embedding gate.
// ---------------------------------------------------------------------------------------------

namespace {

// Shape, dtype and alignment checks of a gate call on [B][H_kv][T][d] rows (layout as given);
// gb = bytes of the gate logits (one element per row).
int check_gate_dims(const void* v, const void* ve, const void* z, int B, int H_kv, int T, int d,
                    int layout, int dtype, attn::Dims* dm, int64_t* vb, int64_t* gb) {
  if (!v || !ve || !z) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H_kv, H_kv, T, d, layout, dm, &n_q, &n_kv)) return rc;
  if (!aligned16(v) || !aligned16(ve) ||
      (reinterpret_cast<uintptr_t>(z) & (uintptr_t)(elem_bytes(dtype) - 1)))
    return ATTN_ERR_ALIGN;
  *vb = n_kv * elem_bytes(dtype);
  *gb = (int64_t)B * H_kv * T * elem_bytes(dtype);
  return ATTN_OK;
}

}  // namespace

int attn_value_gate_ex(const void* v, const void* ve, const void* gate_logits, void* v_out, int B,
                       int H_kv, int T, int d, int layout, int dtype, void* stream) {
  if (!v_out) return ATTN_ERR_NULL;
  attn::Dims dm;
  int64_t vb = 0, gb = 0;
  if (int rc = check_gate_dims(v, ve, gate_logits, B, H_kv, T, d, layout, dtype, &dm, &vb, &gb))
    return rc;
  if (!aligned16(v_out)) return ATTN_ERR_ALIGN;
  if (v_out != v && overlap(v_out, vb, v, vb)) return ATTN_ERR_ALIAS;
  if (overlap(v_out, vb, ve, vb) || overlap(v_out, vb, gate_logits, gb)) return ATTN_ERR_ALIAS;
  attn::GateArgs vg;
  vg.v = v;
  vg.ve = ve;
  vg.z = gate_logits;
  vg.v_out = v_out;
  const hipError_t e = attn::launch_qknorm_rope(nullptr, nullptr, nullptr, nullptr, nullptr,
                                                nullptr, dm, 0.0f, dtype, (hipStream_t)stream, vg);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_qknorm_ve_ex(const void* q, const void* k, const void* v, const void* ve,
                          const void* gate_logits, void* k_work, void* v_work, void* out,
                          float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                          int H_kv, int T, int d, int layout, float eps, int window, int causal,
                          int dtype, void* stream) {
  if (!k_work || !v_work) return ATTN_ERR_NULL;
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_qnorm_args(q, k_work, v_work, out, lse, cos_tab, sin_tab, B, H, H_kv, T, d,
                                layout, eps, window, causal, dtype, &dm, &n_q, &n_kv))
    return rc;
  attn::Dims dg;
  int64_t vb = 0, gb = 0;
  if (int rc = check_gate_dims(v, ve, gate_logits, B, H_kv, T, d, layout, dtype, &dg, &vb, &gb))
    return rc;
  if (!k) return ATTN_ERR_NULL;
  if (!aligned16(k)) return ATTN_ERR_ALIGN;
  if (2 * (int64_t)B * H + 2 > 0x7fffffff) return ATTN_ERR_SHAPE;  // rows of k and v, as int
  const int64_t qb = n_q * 2, kb = n_kv * 2;
  // k_work may be k and v_work may be v (in place); nothing else written overlaps anything read.
  if (k_work != k && overlap(k_work, kb, k, kb)) return ATTN_ERR_ALIAS;
  if (v_work != v && overlap(v_work, kb, v, kb)) return ATTN_ERR_ALIAS;
  if (overlap(k_work, kb, q, qb) || overlap(k_work, kb, v, kb) || overlap(k_work, kb, ve, kb) ||
      overlap(k_work, kb, gate_logits, gb) || overlap(k_work, kb, v_work, kb))
    return ATTN_ERR_ALIAS;
  if (overlap(v_work, kb, q, qb) || overlap(v_work, kb, k, kb) || overlap(v_work, kb, ve, kb) ||
      overlap(v_work, kb, gate_logits, gb))
    return ATTN_ERR_ALIAS;
  if (overlap(out, qb, k, kb) || overlap(out, qb, v, kb) || overlap(out, qb, ve, kb) ||
      overlap(out, qb, gate_logits, gb))
    return ATTN_ERR_ALIAS;
  if (lse != nullptr) {
    const int64_t lbytes = (int64_t)B * H * T * 4;
    if (overlap(lse, lbytes, k, kb) || overlap(lse, lbytes, v, kb) ||
        overlap(lse, lbytes, ve, kb) || overlap(lse, lbytes, gate_logits, gb))
      return ATTN_ERR_ALIAS;
  }
  attn::GateArgs vg;
  vg.v = v;
  vg.ve = ve;
  vg.z = gate_logits;
  vg.v_out = v_work;
  hipError_t e = attn::launch_qknorm_rope(nullptr, k, nullptr, k_work, cos_tab, sin_tab, dm, eps,
                                          ATTN_BF16, (hipStream_t)stream, vg);
  if (e == hipSuccess)
    e = attn::launch_attn_fwd_bf16_qknorm(q, k_work, v_work, out, lse, cos_tab, sin_tab, eps, dm,
                                          window, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_value_gate_bwd_ex(const void* ve, const void* gate_logits, const void* dv, void* dve,
                           void* dgate_logits, int B, int H_kv, int T, int d, int layout,
                           int dtype, void* stream) {
  if (!dve || !dgate_logits) return ATTN_ERR_NULL;
  attn::Dims dm;
  int64_t vb = 0, gb = 0;
  // dv takes v's place in the shape checks
  if (int rc = check_gate_dims(dv, ve, gate_logits, B, H_kv, T, d, layout, dtype, &dm, &vb, &gb))
    return rc;
  if (!aligned16(dve) ||
      (reinterpret_cast<uintptr_t>(dgate_logits) & (uintptr_t)(elem_bytes(dtype) - 1)))
    return ATTN_ERR_ALIGN;
  if (dve != dv && overlap(dve, vb, dv, vb)) return ATTN_ERR_ALIAS;
  if (overlap(dve, vb, ve, vb) || overlap(dve, vb, gate_logits, gb) ||
      overlap(dgate_logits, gb, ve, vb) || overlap(dgate_logits, gb, gate_logits, gb) ||
      overlap(dgate_logits, gb, dv, vb) || overlap(dgate_logits, gb, dve, vb))
    return ATTN_ERR_ALIAS;
  const hipError_t e = attn::launch_value_gate_bwd(ve, gate_logits, dv, dve, dgate_logits, dm,
                                                   dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// ---------------------------------------------------------------------------------------------
// Backward pass.
// ---------------------------------------------------------------------------------------------

int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H,
                int H_kv, int T, int d, int layout, int window, int causal, int dtype,
                void* stream) {
  if (!q || !k || !v || !out || !dout || !lse || !delta || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (dtype == ATTN_BF16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype == ATTN_F32 && d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H, H_kv, T, d, layout, &dm, &n_q, &n_kv)) return rc;
  if (causal != 0 && causal != 1) return ATTN_ERR_WINDOW;
  if (window < -1 || (causal == 0 && window != -1)) return ATTN_ERR_WINDOW;
  const void* tens[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* t : tens)
    if (!aligned16(t)) return ATTN_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
    return ATTN_ERR_ALIGN;
  const int64_t eb = elem_bytes(dtype);
  const int64_t qb = n_q * eb, kb = n_kv * eb, lb = (int64_t)B * H * T * 4;
  // Outputs (dq, dk, dv, delta) overlap no input and no other output.
  const void* in_p[] = {q, k, v, out, dout, lse};
  const int64_t in_n[] = {qb, kb, kb, qb, qb, lb};
  const void* out_p[] = {dq, dk, dv, delta};
  const int64_t out_n[] = {qb, kb, kb, lb};
  for (int o = 0; o < 4; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(out_p[o], out_n[o], in_p[i], in_n[i])) return ATTN_ERR_ALIAS;
    for (int o2 = o + 1; o2 < 4; ++o2)
      if (overlap(out_p[o], out_n[o], out_p[o2], out_n[o2])) return ATTN_ERR_ALIAS;
  }
  if (dtype == ATTN_BF16 && !slab_fits(dm)) return ATTN_ERR_SHAPE;
  const int64_t bh = (int64_t)B * H;
  if (bh * ((T + 127) / 128) > kMaxItems) return ATTN_ERR_SHAPE;
  if (dtype == ATTN_F32 && bh * T * (d / 16) > kMaxGrid) return ATTN_ERR_SHAPE;
  const hipError_t e = attn::launch_attn_bwd(q, k, v, out, dout, lse, delta, dq, dk, dv, dm,
                                             window, causal, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int T,
             int d, int window, int causal, int dtype, void* stream) {
  return attn_bwd_ex(q, k, v, out, dout, lse, delta, dq, dk, dv, B, H, H, T, d, ATTN_LAYOUT_BHTD,
                     window, causal, dtype, stream);
}

int attn_qknorm_rope_bwd_ex(const void* q, const void* k, const void* dq_in, const void* dk_in,
                            void* dq_out, void* dk_out, const float* cos_tab,
                            const float* sin_tab, int B, int H, int H_kv, int T, int d,
                            int layout, float eps, int dtype, void* stream) {
  // q, dq_in and dq_out are all given or all NULL (then only k's rows are processed).
  const bool has_q = q != nullptr;
  if (!k || !dk_in || !dk_out || !cos_tab || !sin_tab || (dq_in != nullptr) != has_q ||
      (dq_out != nullptr) != has_q)
    return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  attn::Dims dm;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H, H_kv, T, d, layout, &dm, &n_q, &n_kv)) return rc;
  if (!(eps >= 0.0f) || !isfinite(eps)) return ATTN_ERR_ARG;
  if (2 * (int64_t)B * H > 0x7fffffff) return ATTN_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(dk_in) || !aligned16(dk_out) || !aligned16(cos_tab) ||
      !aligned16(sin_tab) || (has_q && (!aligned16(q) || !aligned16(dq_in) || !aligned16(dq_out))))
    return ATTN_ERR_ALIGN;
  const int64_t eb = elem_bytes(dtype), qb = n_q * eb, kb = n_kv * eb;
  // Each output may be its own gradient input (in place) and overlaps nothing else.
  if (dk_out != dk_in && overlap(dk_out, kb, dk_in, kb)) return ATTN_ERR_ALIAS;
  if (overlap(dk_out, kb, k, kb)) return ATTN_ERR_ALIAS;
  if (has_q) {
    if (dq_out != dq_in && overlap(dq_out, qb, dq_in, qb)) return ATTN_ERR_ALIAS;
    if (overlap(dq_out, qb, q, qb) || overlap(dq_out, qb, k, kb) || overlap(dq_out, qb, dk_in, kb) ||
        overlap(dq_out, qb, dk_out, kb) || overlap(dk_out, kb, q, qb) ||
        overlap(dk_out, kb, dq_in, qb))
      return ATTN_ERR_ALIAS;
  }
  const hipError_t e = attn::launch_qknorm_rope_bwd(q, k, dq_in, dk_in, dq_out, dk_out, cos_tab,
                                                    sin_tab, dm, eps, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_qknorm_rope_bwd(const void* q, const void* k, const void* dq_in, const void* dk_in,
                         void* dq_out, void* dk_out, const float* cos_tab, const float* sin_tab,
                         int B, int H, int T, int d, float eps, int dtype, void* stream) {
  return attn_qknorm_rope_bwd_ex(q, k, dq_in, dk_in, dq_out, dk_out, cos_tab, sin_tab, B, H, H, T,
                                 d, ATTN_LAYOUT_BHTD, eps, dtype, stream);
}

// ---------------------------------------------------------------------------------------------
// Decode.
// ---------------------------------------------------------------------------------------------

long long attn_decode_workspace_bytes(int B, int H, int S, int d, int window) {
  if (B < 1 || H < 1 || S < 1 || d < 1 || d > 256 || window < -1) return -1;
  return (long long)attn::decode_workspace_bytes(B, H, S, d, window);
}

}  // extern "C"

namespace {

// Checks of one decode call shared by attn_decode_ex and attn_decode_noalloc_ex. workspace is the
// caller's buffer (ws_bytes long) or, for the allocation-free call, nullptr (nothing to check).
int check_decode(const void* q, const void* k_cache, const void* v_cache, const int* lengths,
                 const void* out, const float* lse, const void* workspace, long long ws_bytes,
                 int B, int H, int H_kv, int S, int d, int layout, int window, int dtype,
                 attn::Dims* dm, int64_t* need) {
  if (!q || !k_cache || !v_cache || !out) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (dtype == ATTN_BF16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (dtype == ATTN_F32 && d != 16 && d != 32 && d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  int64_t n_q = 0, n_kv = 0;
  if (int rc = check_dims(B, H, H_kv, S, d, layout, dm, &n_q, &n_kv)) return rc;
  if (window < -1) return ATTN_ERR_WINDOW;
  const void* vec[] = {q, k_cache, v_cache, out, workspace};
  for (const void* t : vec)
    if (t && !aligned16(t)) return ATTN_ERR_ALIGN;
  if ((lengths && (reinterpret_cast<uintptr_t>(lengths) & 3u)) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return ATTN_ERR_ALIGN;
  *need = attn::decode_workspace_bytes(B, H, S, d, window);
  if (workspace && ws_bytes < *need) return ATTN_ERR_ARG;
  const int64_t eb = elem_bytes(dtype);
  const int64_t qb = (int64_t)B * H * d * eb, kb = n_kv * eb;
  // Written: out, lse, workspace; none overlaps another buffer.
  const void* bufs[] = {q, k_cache, v_cache, lengths, out, lse, workspace};
  const int64_t len[] = {qb, kb, kb, (int64_t)B * 4, qb, (int64_t)B * H * 4, *need};
  for (int w = 4; w < 7; ++w) {
    if (!bufs[w]) continue;
    for (int o = 0; o < 7; ++o)
      if (o != w && bufs[o] && overlap(bufs[w], len[w], bufs[o], len[o])) return ATTN_ERR_ALIAS;
  }
  if ((int64_t)B * H_kv * attn::decode_splits(B, H, S, d, window) > kMaxGrid)
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int* lengths,
                   void* out, float* lse, void* workspace, long long workspace_bytes, int B,
                   int H, int H_kv, int S, int d, int layout, int window, int dtype,
                   void* stream) {
  if (!workspace) return ATTN_ERR_NULL;
  attn::Dims dm;
  int64_t need = 0;
  if (int rc = check_decode(q, k_cache, v_cache, lengths, out, lse, workspace, workspace_bytes, B,
                            H, H_kv, S, d, layout, window, dtype, &dm, &need))
    return rc;
  const hipError_t e = attn::launch_attn_decode(q, k_cache, v_cache, lengths, out, lse, workspace,
                                                dm, window, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode_noalloc_ex(const void* q, const void* k_cache, const void* v_cache,
                           const int* lengths, void* out, float* lse, int B, int H, int H_kv,
                           int S, int d, int layout, int window, int dtype, void* stream) {
  attn::Dims dm;
  int64_t need = 0;
  if (int rc = check_decode(q, k_cache, v_cache, lengths, out, lse, nullptr, 0, B, H, H_kv, S, d,
                            layout, window, dtype, &dm, &need))
    return rc;
  if (need > attn::kDecodeScratchBytes) return ATTN_ERR_SCRATCH;
  // The partial kernel writes every split slot the merge then reads, so the scratch needs no
  // clearing between calls.
  void* ws = nullptr;
  if (attn::decode_scratch(&ws) != hipSuccess) return ATTN_ERR_HIP;
  const hipError_t e = attn::launch_attn_decode(q, k_cache, v_cache, lengths, out, lse, ws, dm,
                                                window, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* lengths,
                void* out, float* lse, void* workspace, long long workspace_bytes, int B, int H,
                int S, int d, int window, int dtype, void* stream) {
  return attn_decode_ex(q, k_cache, v_cache, lengths, out, lse, workspace, workspace_bytes, B, H,
                        H, S, d, ATTN_LAYOUT_BHTD, window, dtype, stream);
}

}  // extern "C"
