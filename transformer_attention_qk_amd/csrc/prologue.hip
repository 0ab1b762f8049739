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
//
// VG: the launch also applies the value-embedding gate ("Подробный технический разбор реализации
// Autoresearch", train.py listing, `CausalSelfAttention.forward`: v + 2 sigmoid(gate logit) ve,
// one gate per token and kv head) to the B*H_kv rows of v, which follow the other rows from head
// index v_start (a multiple of R, so no block mixes the two kinds of row). v, ve and v_out share
// k's strides; the gate logits z sit at b * sz.b + h * sz.h + t * sz.t.
template <typename Elem, int D, int R, bool VG>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    const Elem* __restrict__ q, const Elem* __restrict__ k, Elem* q_out, Elem* k_out,
    const float* __restrict__ cos_tab, const float* __restrict__ sin_tab, Strides sq, Strides sk,
    FastDiv H, FastDiv H_kv, int heads_q, int heads, int T, FastDiv t_blocks, float eps,
    const Elem* v, const Elem* ve, const Elem* zg, Elem* v_out, Strides sz, int v_start) {
  constexpr int E = kE<Elem>;
  constexpr int HALF = D / 2;
  constexpr int L = D / E;      // lanes per row (2 .. 32)
  constexpr int TPB = 256 / L;  // positions per block
  const int hb = (int)t_blocks.div(blockIdx.x);
  const int tb = (int)blockIdx.x - hb * (int)t_blocks.d;
  const int h0 = hb * R;
  const int t_loc = (int)threadIdx.x / L;
  const int t0 = tb * TPB;
  // Positions past T (in the last block of positions) redo row T - 1 and store nothing. All L
  // lanes of a row group share t, so the xor shuffles below never mix rows.
  const bool valid = t0 + t_loc < T;
  const int t = valid ? t0 + t_loc : T - 1;
  const int r_loc = t - t0;  // row of t within the block
  const int sub = (int)threadIdx.x % L;
  const bool first = sub < L / 2;
  const int j0 = (sub % (L / 2)) * E;  // frequency of the chunk's first element
  const int total = heads_q + heads;
  if constexpr (VG) {
    if (h0 >= v_start) {  // block-uniform: rows of v
      const int lane_v = r_loc * sk.t + sub * E;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int hv = h0 + r - v_start;
        if (hv >= heads) break;
        const uint32_t b = H_kv.div((uint32_t)hv), hk = (uint32_t)hv - b * H_kv.d;
        const int64_t base = (int64_t)b * sk.b + (int64_t)hk * sk.h + (int64_t)t0 * sk.t;
        const float z = (float)zg[(int64_t)b * sz.b + (int64_t)hk * sz.h + (int64_t)t * sz.t];
        float x[E], e[E], y[E];
        Vec<Elem, E>::load(v + base + lane_v, x);
        Vec<Elem, E>::load(ve + base + lane_v, e);
        // 2 sigmoid(z) in (0, 2): 0 for z -> -inf (exp overflows to inf), 2 for z -> +inf
        const float g = 2.0f / (1.0f + expf(-z));
#pragma unroll
        for (int i = 0; i < E; ++i) y[i] = fmaf(g, e[i], x[i]);
        if (valid) Vec<Elem, E>::store(v_out + base + lane_v, y);
      }
      return;
    }
  }

  // A row's element offset splits into a block-uniform part (head h at position t0) and this
  // lane's part, which stays below 2^31 (TPB row strides; the host bounds H * d).
  auto head_base = [&](int h) -> int64_t {
    if (h < heads_q) {
      const uint32_t b = H.div((uint32_t)h);
      return (int64_t)b * sq.b + (int64_t)(h - b * H.d) * sq.h + (int64_t)t0 * sq.t;
    }
    const uint32_t hk = (uint32_t)(h - heads_q), b = H_kv.div(hk);
    return (int64_t)b * sk.b + (int64_t)(hk - b * H_kv.d) * sk.h + (int64_t)t0 * sk.t;
  };
  const int lane_q = r_loc * sq.t + sub * E, lane_k = r_loc * sk.t + sub * E;
  u32x4 raw[R];
  int64_t base[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int h = h0 + r;  // block-uniform
    if (h < total) {
      base[r] = head_base(h);
      const Elem* src = (h < heads_q) ? q + base[r] + lane_q : k + base[r] + lane_k;
      raw[r] = *reinterpret_cast<const u32x4*>(src);
    }
  }
  // The rotation factors of position t, loaded after the rows so those go out first.
  float c[E], s[E];
  const float* ct = cos_tab + (int64_t)t * HALF + j0;
  const float* st = sin_tab + (int64_t)t * HALF + j0;
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    Vec<float, 4>::load(ct + i, c + i);
    Vec<float, 4>::load(st + i, s + i);
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
    if (valid)
      Vec<Elem, E>::store((h < heads_q) ? q_out + base[r] + lane_q : k_out + base[r] + lane_k, y);
  }
}

// Backward of the prologue for the same rows: given the raw row x and the gradient dy of
// y = RoPE(RMSNorm(x)), dx = r (g - xh mean(g xh)) with r = (mean(x^2) + eps)^(-1/2), xh = r x
// and g the rotation of dy by the opposite angles (g_j = dy_j cos + dy_{j+h} (-sin) in the first
// half, g_{j+h} = dy_j sin + dy_{j+h} cos in the second): the chain rule of `norm` and
// `apply_rotary_emb`. Same row grouping as the forward; dx may be dy itself (each lane reads its
// chunks of the row, and the partner's through a shuffle, before any lane of the row stores).
template <typename Elem, int D>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(
    const Elem* __restrict__ q, const Elem* __restrict__ k, const Elem* dq_in, const Elem* dk_in,
    Elem* dq_out, Elem* dk_out, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, Strides sq, Strides sk, FastDiv H, FastDiv H_kv,
    int heads_q, int heads, int T, FastDiv t_blocks, float eps) {
  constexpr int E = kE<Elem>;
  constexpr int HALF = D / 2;
  constexpr int L = D / E;
  constexpr int TPB = 256 / L;
  const int h = (int)t_blocks.div(blockIdx.x);  // block-uniform
  const int tb = (int)blockIdx.x - h * (int)t_blocks.d;
  const int t_loc = (int)threadIdx.x / L;
  const int t0 = tb * TPB;
  const bool valid = t0 + t_loc < T;
  const int t = valid ? t0 + t_loc : T - 1;
  const int r_loc = t - t0;
  const int sub = (int)threadIdx.x % L;
  const bool first = sub < L / 2;
  const int j0 = (sub % (L / 2)) * E;
  int64_t base;
  int lane_off;
  if (h < heads_q) {
    const uint32_t b = H.div((uint32_t)h);
    base = (int64_t)b * sq.b + (int64_t)(h - b * H.d) * sq.h + (int64_t)t0 * sq.t;
    lane_off = r_loc * sq.t + sub * E;
  } else {
    const uint32_t hk = (uint32_t)(h - heads_q), b = H_kv.div(hk);
    base = (int64_t)b * sk.b + (int64_t)(hk - b * H_kv.d) * sk.h + (int64_t)t0 * sk.t;
    lane_off = r_loc * sk.t + sub * E;
  }
  const bool isq = h < heads_q;
  const int64_t off = base + lane_off;
  const u32x4 xraw = *reinterpret_cast<const u32x4*>((isq ? q : k) + off);
  const u32x4 graw = *reinterpret_cast<const u32x4*>((isq ? dq_in : dk_in) + off);
  float c[E], s[E];
  const float* ct = cos_tab + (int64_t)t * HALF + j0;
  const float* st = sin_tab + (int64_t)t * HALF + j0;
#pragma unroll
  for (int i = 0; i < E; i += 4) {
    Vec<float, 4>::load(ct + i, c + i);
    Vec<float, 4>::load(st + i, s + i);
  }
  u32x4 gpart;
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) gpart[wd] = (uint32_t)__shfl_xor((int)graw[wd], L / 2);
  float x[E], dy[E], dyp[E];
  Vec<Elem, E>::load(reinterpret_cast<const Elem*>(&xraw), x);
  Vec<Elem, E>::load(reinterpret_cast<const Elem*>(&graw), dy);
  Vec<Elem, E>::load(reinterpret_cast<const Elem*>(&gpart), dyp);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) ss = fmaf(x[i], x[i], ss);
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
  const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + eps);
  float g[E], xh[E], gx = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    // first half: dy_j cos - dy_{j+h} sin; second half: dy_j sin + dy_{j+h} cos (own = dy of
    // this lane's element, partner = the other half's)
    g[i] = first ? fmaf(dy[i], c[i], -(dyp[i] * s[i])) : fmaf(dy[i], c[i], dyp[i] * s[i]);
    xh[i] = x[i] * rinv;
    gx = fmaf(g[i], xh[i], gx);
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) gx += __shfl_xor(gx, o);
  const float mgx = gx * (1.0f / D);
  float dx[E];
#pragma unroll
  for (int i = 0; i < E; ++i) dx[i] = rinv * fmaf(-xh[i], mgx, g[i]);
  if (valid) Vec<Elem, E>::store((isq ? dq_out : dk_out) + off, dx);
}

template <typename Elem, int D>
static hipError_t launch_qknorm_rope_bwd_t(const void* q, const void* k, const void* dq_in,
                                           const void* dk_in, void* dq_out, void* dk_out,
                                           const float* cos_tab, const float* sin_tab,
                                           const Dims& dm, float eps, hipStream_t stream) {
  constexpr int L = D / kE<Elem>;
  constexpr int TPB = 256 / L;
  const int T = dm.T;
  const Geometry geo = make_geometry(dm);
  const int heads = dm.B * dm.H_kv;
  const int heads_q = (q != nullptr) ? dm.B * dm.H : 0;
  const int t_blocks = (T + TPB - 1) / TPB;
  const int64_t grid = (int64_t)t_blocks * (heads_q + heads);
  hipLaunchKernelGGL((qknorm_rope_bwd_kernel<Elem, D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const Elem*)q, (const Elem*)k, (const Elem*)dq_in, (const Elem*)dk_in,
                     (Elem*)dq_out, (Elem*)dk_out, cos_tab, sin_tab, geo.q, geo.kv,
                     make_fastdiv((uint32_t)dm.H), make_fastdiv((uint32_t)dm.H_kv), heads_q,
                     heads, T, make_fastdiv((uint32_t)t_blocks), eps);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope_bwd(const void* q, const void* k, const void* dq_in,
                                  const void* dk_in, void* dq_out, void* dk_out,
                                  const float* cos_tab, const float* sin_tab, const Dims& dm,
                                  float eps, int dtype, hipStream_t stream) {
  const int d = dm.d;
#define ATTN_QKNB_CASE(ELEM, DD)                                                                \
  if (d == DD)                                                                                  \
    return launch_qknorm_rope_bwd_t<ELEM, DD>(q, k, dq_in, dk_in, dq_out, dk_out, cos_tab,      \
                                              sin_tab, dm, eps, stream);
  if (dtype == 0) {
    ATTN_QKNB_CASE(bf16, 16)
    ATTN_QKNB_CASE(bf16, 32)
    ATTN_QKNB_CASE(bf16, 64)
    ATTN_QKNB_CASE(bf16, 128)
  } else {
    ATTN_QKNB_CASE(float, 16)
    ATTN_QKNB_CASE(float, 32)
    ATTN_QKNB_CASE(float, 64)
    ATTN_QKNB_CASE(float, 128)
  }
#undef ATTN_QKNB_CASE
  return hipErrorInvalidValue;
}

// Backward of the value-embedding gate for the B*H_kv rows of v: with g = 2 sigmoid(z) and dv the
// gradient of the gated rows, dve = g dv and dz = g (1 - g/2) sum_j ve_j dv_j (the derivative of
// 2 sigmoid is 2 sigmoid (1 - sigmoid)); the gradient of v itself is dv unchanged. Same row
// grouping as the prologue: L lanes per row, the row sum crossing them by xor shuffles; lane 0 of
// a row writes dz. dve may be dv itself (each lane reads its chunk before writing it).
template <typename Elem, int D>
__global__ __launch_bounds__(256) void value_gate_bwd_kernel(
    const Elem* __restrict__ ve, const Elem* __restrict__ zg, const Elem* dv, Elem* dve,
    Elem* __restrict__ dz, Strides sk, Strides sz, FastDiv H_kv, int T, FastDiv t_blocks) {
  constexpr int E = kE<Elem>;
  constexpr int L = D / E;
  constexpr int TPB = 256 / L;
  const int h = (int)t_blocks.div(blockIdx.x);  // block-uniform: kv head row b * H_kv + hk
  const int tb = (int)blockIdx.x - h * (int)t_blocks.d;
  const int t_loc = (int)threadIdx.x / L;
  const int t0 = tb * TPB;
  const bool valid = t0 + t_loc < T;
  const int t = valid ? t0 + t_loc : T - 1;
  const int sub = (int)threadIdx.x % L;
  const uint32_t b = H_kv.div((uint32_t)h), hk = (uint32_t)h - b * H_kv.d;
  const int64_t off = (int64_t)b * sk.b + (int64_t)hk * sk.h + (int64_t)t * sk.t + sub * E;
  const int64_t zoff = (int64_t)b * sz.b + (int64_t)hk * sz.h + (int64_t)t * sz.t;
  const float z = (float)zg[zoff];
  float e[E], g_in[E], out[E];
  Vec<Elem, E>::load(ve + off, e);
  Vec<Elem, E>::load(dv + off, g_in);
  const float g = 2.0f / (1.0f + expf(-z));
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    dot = fmaf(e[i], g_in[i], dot);
    out[i] = g * g_in[i];
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o);
  if (valid) {
    Vec<Elem, E>::store(dve + off, out);
    if (sub == 0) dz[zoff] = (Elem)(g * (1.0f - 0.5f * g) * dot);
  }
}

template <typename Elem, int D>
static hipError_t launch_value_gate_bwd_t(const void* ve, const void* z, const void* dv, void* dve,
                                          void* dz, const Dims& dm, hipStream_t stream) {
  constexpr int L = D / kE<Elem>;
  constexpr int TPB = 256 / L;
  const int T = dm.T;
  const Geometry geo = make_geometry(dm);
  const int t_blocks = (T + TPB - 1) / TPB;
  const int64_t grid = (int64_t)t_blocks * dm.B * dm.H_kv;
  const Strides sz = (dm.layout == 0) ? Strides{(int64_t)dm.H_kv * T, T, 1}
                                      : Strides{(int64_t)T * dm.H_kv, 1, dm.H_kv};
  hipLaunchKernelGGL((value_gate_bwd_kernel<Elem, D>), dim3((unsigned)grid), dim3(256), 0, stream,
                     (const Elem*)ve, (const Elem*)z, (const Elem*)dv, (Elem*)dve, (Elem*)dz,
                     geo.kv, sz, make_fastdiv((uint32_t)dm.H_kv), T,
                     make_fastdiv((uint32_t)t_blocks));
  return hipGetLastError();
}

hipError_t launch_value_gate_bwd(const void* ve, const void* z, const void* dv, void* dve,
                                 void* dz, const Dims& dm, int dtype, hipStream_t stream) {
  const int d = dm.d;
#define ATTN_VGB_CASE(ELEM, DD) \
  if (d == DD) return launch_value_gate_bwd_t<ELEM, DD>(ve, z, dv, dve, dz, dm, stream);
  if (dtype == 0) {
    ATTN_VGB_CASE(bf16, 16)
    ATTN_VGB_CASE(bf16, 32)
    ATTN_VGB_CASE(bf16, 64)
    ATTN_VGB_CASE(bf16, 128)
  } else {
    ATTN_VGB_CASE(float, 16)
    ATTN_VGB_CASE(float, 32)
    ATTN_VGB_CASE(float, 64)
    ATTN_VGB_CASE(float, 128)
  }
#undef ATTN_VGB_CASE
  return hipErrorInvalidValue;
}

template <typename Elem, int D, bool VG>
static hipError_t launch_qknorm_rope_t(const void* q, const void* k, void* q_out, void* k_out,
                                       const float* cos_tab, const float* sin_tab, const Dims& dm,
                                       float eps, const GateArgs& vg, hipStream_t stream) {
  constexpr int R = 2;  // rows per lane
  constexpr int L = D / kE<Elem>;
  constexpr int TPB = 256 / L;
  const int T = dm.T;
  const Geometry geo = make_geometry(dm);
  const int heads = dm.B * dm.H_kv;
  const int heads_q = (q != nullptr) ? dm.B * dm.H : 0;
  // Rows: q's (if any), k's (if any), then, with the gate, v's from a multiple of R.
  if (k == nullptr && (q != nullptr || !VG)) return hipErrorInvalidValue;
  const int qk_rows = heads_q + ((k != nullptr) ? heads : 0);
  const int v_start = VG ? (qk_rows + R - 1) / R * R : qk_rows;
  const int rows = VG ? v_start + heads : qk_rows;
  const int t_blocks = (T + TPB - 1) / TPB;
  const int64_t grid = (int64_t)t_blocks * ((rows + R - 1) / R);
  // gate logits: [B][H_kv][T] beside [B][H_kv][T][d] tensors, [B][T][H_kv] beside [B][T][H_kv][d]
  const Strides sz = (dm.layout == 0) ? Strides{(int64_t)dm.H_kv * T, T, 1}
                                      : Strides{(int64_t)T * dm.H_kv, 1, dm.H_kv};
  hipLaunchKernelGGL((qknorm_rope_kernel<Elem, D, R, VG>), dim3((unsigned)grid), dim3(256), 0,
                     stream, (const Elem*)q, (const Elem*)k, (Elem*)q_out, (Elem*)k_out, cos_tab,
                     sin_tab, geo.q, geo.kv, make_fastdiv((uint32_t)dm.H),
                     make_fastdiv((uint32_t)dm.H_kv), heads_q, heads, T,
                     make_fastdiv((uint32_t)t_blocks), eps, (const Elem*)vg.v, (const Elem*)vg.ve,
                     (const Elem*)vg.z, (Elem*)vg.v_out, sz, v_start);
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, const Dims& dm,
                              float eps, int dtype, hipStream_t stream, const GateArgs& vg) {
  const int d = dm.d;
  const bool gate = vg.v != nullptr;
#define ATTN_QKN_CASE(ELEM, DD)                                                                 \
  if (d == DD)                                                                                  \
    return gate ? launch_qknorm_rope_t<ELEM, DD, true>(q, k, q_out, k_out, cos_tab, sin_tab, dm, \
                                                       eps, vg, stream)                          \
                : launch_qknorm_rope_t<ELEM, DD, false>(q, k, q_out, k_out, cos_tab, sin_tab,    \
                                                        dm, eps, vg, stream);
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
