// RoPE tables and the fused QK-RMSNorm + RoPE prologue.
//
// Operations from "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея
// Карпаты" (habr.com, article 1010198), train.py listing: `norm` (weightless RMSNorm over the
// head dim), `apply_rotary_emb` (half-split rotation) and `GPT._precompute_rotary_embeddings`
// (theta = t * base^(-2j/d)). Normalising before rotating gives the same result as the listing's
// rotate-then-normalise order, because the rotation keeps each row's sum of squares.
//
// The prologue is bound by HBM: it reads and writes every element of q and k once (8*d bytes per
// token per head in bf16). Each row of d elements is handled by a group of lanes, one 16-byte
// chunk per lane, so every load and store of a wave covers whole rows; the rotation partners swap
// chunks and the sum of squares crosses the group by xor shuffles. The rotation factors of a
// position are loaded once for several heads.
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

// Rows are grouped by position: a block handles TPB positions t of R heads, where the heads are
// q's B*H heads (when q is given) followed by k's B*H_kv heads; a head's rows start at
// b * stride.b + h * stride.h and are stride.t elements apart (either storage order). A row is handled by L = d / E lanes, lane i
// holding the row's i-th 16-byte chunk, so a wave's loads and stores cover whole rows. The
// element j < d/2 and its rotation partner j + d/2 sit in lanes i and i ^ (L/2), which swap
// their chunks with one xor shuffle per 32-bit word; the sum of squares crosses the L lanes by
// xor shuffles too. A row group loads the rotation factors of its position once for its R rows.
template <typename Elem, int D, int R>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    const Elem* __restrict__ q, const Elem* __restrict__ k, Elem* q_out, Elem* k_out,
    const float* __restrict__ cos_tab, const float* __restrict__ sin_tab, Strides sq, Strides sk,
    int H, int H_kv, int heads_q, int heads, int T, int t_blocks, float eps) {
  constexpr int E = kE<Elem>;
  constexpr int HALF = D / 2;
  constexpr int L = D / E;      // lanes per row (2 .. 32)
  constexpr int TPB = 256 / L;  // positions per block
  const int tb = (int)(blockIdx.x % (unsigned)t_blocks);
  const int h0 = (int)(blockIdx.x / (unsigned)t_blocks) * R;
  const int t = tb * TPB + (int)threadIdx.x / L;
  const int sub = (int)threadIdx.x % L;
  // All L lanes of a row group share t, so a group is either fully active or fully inactive and
  // the xor shuffles below never read a lane of another row.
  if (t >= T) return;
  const bool first = sub < L / 2;
  const int j0 = (sub % (L / 2)) * E;  // frequency of the chunk's first element
  const int total = heads_q + heads;

  float c[E], s[E];
  const float* ct = cos_tab + (int64_t)t * HALF + j0;
  const float* st = sin_tab + (int64_t)t * HALF + j0;
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    Vec<float, 4>::load(ct + i, c + i);
    Vec<float, 4>::load(st + i, s + i);
  }
  // Element offset of row t of head h (block-uniform apart from t).
  auto row = [&](int h) -> int64_t {
    if (h < heads_q) return (int64_t)(h / H) * sq.b + (int64_t)(h % H) * sq.h + (int64_t)t * sq.t;
    const int hk = h - heads_q;
    return (int64_t)(hk / H_kv) * sk.b + (int64_t)(hk % H_kv) * sk.h + (int64_t)t * sk.t;
  };
  u32x4 raw[R];
  int64_t off[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = h0 + r;  // block-uniform
    if (h < total) {
      off[r] = row(h) + sub * E;
      raw[r] = *reinterpret_cast<const u32x4*>((h < heads_q ? q : k) + off[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = h0 + r;
    if (h >= total) break;
    u32x4 part;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) part[wd] = (uint32_t)__shfl_xor((int)raw[r][wd], L / 2);
    float x[E], xp[E];
    Vec<Elem, E>::load(reinterpret_cast<const Elem*>(&raw[r]), x);
    Vec<Elem, E>::load(reinterpret_cast<const Elem*>(&part), xp);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
    for (int o = L / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
    float y[E];
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const float a = x[i] * rinv, b = xp[i] * rinv;
      // first half: x_j cos + x_{j+h} sin; second half: -x_j sin + x_{j+h} cos
      y[i] = first ? fmaf(a, c[i], b * s[i]) : fmaf(a, c[i], -(b * s[i]));
    }
    Vec<Elem, E>::store((h < heads_q ? q_out : k_out) + off[r], y);
  }
}

template <typename Elem, int D>
static hipError_t launch_qknorm_rope_t(const void* q, const void* k, void* q_out, void* k_out,
                                       const float* cos_tab, const float* sin_tab, const Dims& dm,
                                       float eps, hipStream_t stream) {
  constexpr int R = 2;  // rows per lane
  constexpr int L = D / kE<Elem>;
  constexpr int TPB = 256 / L;
  const int T = dm.T;
  const Geometry geo = make_geometry(dm);
  const int heads = dm.B * dm.H_kv;
  const int heads_q = (q != nullptr) ? dm.B * dm.H : 0;
  const int t_blocks = (T + TPB - 1) / TPB;
  const int64_t grid = (int64_t)t_blocks * ((heads_q + heads + R - 1) / R);
  hipLaunchKernelGGL((qknorm_rope_kernel<Elem, D, R>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const Elem*)q, (const Elem*)k, (Elem*)q_out, (Elem*)k_out, cos_tab, sin_tab,
                     geo.q, geo.kv, dm.H, dm.H_kv, heads_q, heads, T, t_blocks, eps);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, const Dims& dm,
                              float eps, int dtype, hipStream_t stream) {
  const int d = dm.d;
#define ATTN_QKN_CASE(ELEM, DD) \
  if (d == DD) return launch_qknorm_rope_t<ELEM, DD>(q, k, q_out, k_out, cos_tab, sin_tab, dm, eps, stream);
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
