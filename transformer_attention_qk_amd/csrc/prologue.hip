// RoPE tables and the fused QK-RMSNorm + RoPE prologue.
//
// Operations from "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея
// Карпаты" (habr.com, article 1010198), train.py listing: `norm` (weightless RMSNorm over the
// head dim), `apply_rotary_emb` (half-split rotation) and `GPT._precompute_rotary_embeddings`
// (theta = t * base^(-2j/d)). Normalising before rotating gives the same result as the listing's
// rotate-then-normalise order, because the rotation keeps each row's sum of squares.
//
// The prologue is bound by HBM: it reads and writes every element of q and k once (8*d bytes per
// token per head in bf16). Each row of d elements is handled by a group of L lanes; a lane holds E
// elements of the first half and the E matching elements of the second half, so the rotation is
// lane-local and only the sum of squares crosses lanes (xor shuffles inside the group).
#include "common.hpp"
#include "launch.hpp"

namespace attn {

__global__ __launch_bounds__(256) void rope_table_kernel(float* __restrict__ cos_tab,
                                                         float* __restrict__ sin_tab, int T,
                                                         int half, int d, double base) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)T * half) return;
  const int t = (int)(idx / half);
  const int j = (int)(idx % half);
  const double inv_freq = 1.0 / pow(base, (2.0 * j) / (double)d);
  const double theta = (double)t * inv_freq;
  cos_tab[idx] = (float)cos(theta);
  sin_tab[idx] = (float)sin(theta);
}

hipError_t launch_rope_table(float* cos_tab, float* sin_tab, int T, int d, double base,
                             hipStream_t stream) {
  const int half = d / 2;
  const int64_t n = (int64_t)T * half;
  const unsigned grid = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, stream, cos_tab, sin_tab, T, half,
                     d, base);
  return hipGetLastError();
}

template <typename Elem, int E>
struct Vec;
template <>
struct Vec<bf16, 8> {
  static __device__ __forceinline__ void load(const bf16* p, float* x) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo_to_f32(w[i]);
      x[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  }
  static __device__ __forceinline__ void store(bf16* p, const float* x) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    *reinterpret_cast<u32x4*>(p) = w;
  }
};
template <>
struct Vec<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* x) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = w[i];
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    f32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = x[i];
    *reinterpret_cast<f32x4*>(p) = w;
  }
};

// Elements per lane per half: 16-byte accesses for both dtypes.
template <typename Elem>
constexpr int kE = (sizeof(Elem) == 2) ? 8 : 4;

// Rows [0, q_rows) are rows of q, rows [q_rows, q_rows + rows) rows of k (q_rows = 0: k only).
template <typename Elem, int D>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    const Elem* __restrict__ q, const Elem* __restrict__ k, Elem* q_out, Elem* k_out,
    const float* __restrict__ cos_tab, const float* __restrict__ sin_tab, int64_t q_rows,
    int64_t rows, int T, float eps) {
  constexpr int E = kE<Elem>;
  constexpr int HALF = D / 2;
  static_assert(HALF % E == 0, "half head dim must be a multiple of the lane vector");
  constexpr int L = HALF / E;  // lanes per row (1, 2, 4, 8 or 16)
  constexpr int ROWS_PER_BLOCK = 256 / L;
  const int64_t row = (int64_t)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / L;
  const int sub = threadIdx.x % L;
  // Every lane of a row group shares `row`, so a group is either fully active or fully inactive
  // and the xor shuffles below never read a lane of another row.
  if (row >= q_rows + rows) return;
  const bool is_q = row < q_rows;
  const int64_t r = is_q ? row : row - q_rows;
  const Elem* src = (is_q ? q : k) + r * D;
  Elem* dst = (is_q ? q_out : k_out) + r * D;
  const int t = (int)(r % T);
  const int j0 = sub * E;

  float x1[E], x2[E];
  Vec<Elem, E>::load(src + j0, x1);
  Vec<Elem, E>::load(src + HALF + j0, x2);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) ss = fmaf(x1[i], x1[i], fmaf(x2[i], x2[i], ss));
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);

  float c[E], s[E];
  const float* ct = cos_tab + (int64_t)t * HALF + j0;
  const float* st = sin_tab + (int64_t)t * HALF + j0;
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    Vec<float, 4>::load(ct + i, c + i);
    Vec<float, 4>::load(st + i, s + i);
  }
  float y1[E], y2[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const float a = x1[i] * rinv;
    const float b = x2[i] * rinv;
    y1[i] = fmaf(a, c[i], b * s[i]);
    y2[i] = fmaf(b, c[i], -(a * s[i]));
  }
  Vec<Elem, E>::store(dst + j0, y1);
  Vec<Elem, E>::store(dst + HALF + j0, y2);
}

template <typename Elem, int D>
static hipError_t launch_qknorm_rope_t(const void* q, const void* k, void* q_out, void* k_out,
                                       const float* cos_tab, const float* sin_tab, int B, int H,
                                       int T, float eps, hipStream_t stream) {
  constexpr int L = (D / 2) / kE<Elem>;
  constexpr int ROWS_PER_BLOCK = 256 / L;
  const int64_t rows = (int64_t)B * H * T;
  const int64_t q_rows = (q != nullptr) ? rows : 0;
  const int64_t grid = (q_rows + rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  hipLaunchKernelGGL((qknorm_rope_kernel<Elem, D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const Elem*)q, (const Elem*)k, (Elem*)q_out, (Elem*)k_out, cos_tab, sin_tab,
                     q_rows, rows, T, eps);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, int B, int H, int T,
                              int d, float eps, int dtype, hipStream_t stream) {
#define ATTN_QKN_CASE(ELEM, DD)                                                              \
  if (d == DD)                                                                               \
    return launch_qknorm_rope_t<ELEM, DD>(q, k, q_out, k_out, cos_tab, sin_tab, B, H, T, eps, \
                                          stream);
  if (dtype == 0) {
    ATTN_QKN_CASE(bf16, 16)
    ATTN_QKN_CASE(bf16, 32)
    ATTN_QKN_CASE(bf16, 64)
    ATTN_QKN_CASE(bf16, 128)
  } else {
    ATTN_QKN_CASE(float, 16)
    ATTN_QKN_CASE(float, 32)
    ATTN_QKN_CASE(float, 64)
    ATTN_QKN_CASE(float, 128)
  }
#undef ATTN_QKN_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
