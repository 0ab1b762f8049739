// fp32 attention forward: every step in fp32 (dot products, online softmax, P v).
//
// Computes out_i = sum_{j in A(i)} softmax_j(q_i . k_j / sqrt(d)) v_j and lse_i, as defined in
// "Projeção em um Subespaço de Consulta" (unhomeschool.com), sections "O que a Atenção Calcula",
// "Escalonamento por sqrt(d_k)" and "A Máscara Causal", with the (W, 0) window of the attention
// call in the train.py listing of "Подробный технический разбор реализации Autoresearch"
// (habr.com, article 1010198), `CausalSelfAttention.forward`.
//
// This path serves fp32 inputs (small shapes, tight tolerances); the bf16 MFMA kernel is the
// throughput path. One 64-lane workgroup owns 64 consecutive queries of one head, one query per
// lane; key/value tiles of 32 rows are staged in LDS and read as broadcasts. The softmax runs in
// the base-2 domain with log2(e)/sqrt(d) folded into one scale, with the running-maximum
// rescaling of a one-pass softmax.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace attn {

template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                          const float* __restrict__ K,
                                                          const float* __restrict__ V,
                                                          float* __restrict__ O,
                                                          float* __restrict__ LSE, Geometry geo,
                                                          int BH, int T, int window, int causal,
                                                          float scale_log2, int nqb) {
  constexpr int BN = 32;
  __shared__ float ks[BN * D];
  __shared__ float vs[BN * D];
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);  // heaviest query blocks first
  const int bh = (int)(blockIdx.x % BH);
  const int64_t hoff = geo.q_head(bh), kvoff = geo.kv_head(bh);
  const int qs = geo.q.t, ks_ = geo.kv.t;  // row strides in elements
  const int q0 = qb * 64;
  const int i = q0 + (int)threadIdx.x;

  float qr[D];
#pragma unroll
  for (int c = 0; c < D; ++c) qr[c] = (i < T) ? Q[hoff + (int64_t)i * qs + c] : 0.f;
  float o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;

  int lo = 0, hi = T;
  if (causal) {
    hi = min(T, q0 + 64);
    if (window >= 0) lo = max(0, q0 - window);
  }
  for (int kt = lo; kt < hi; kt += BN) {
    __syncthreads();
    for (int e = threadIdx.x; e < BN * D; e += 64) {
      const int j = kt + e / D;
      const bool in = j < T;
      ks[e] = in ? K[kvoff + (int64_t)j * ks_ + e % D] : 0.f;
      vs[e] = in ? V[kvoff + (int64_t)j * ks_ + e % D] : 0.f;
    }
    __syncthreads();
    const int jn = min(BN, hi - kt);
    for (int jj = 0; jj < jn; ++jj) {
      const int j = kt + jj;
      const bool vis = !causal || (j <= i && (window < 0 || i - j <= window));
      if (!vis) continue;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) s = fmaf(qr[c], ks[jj * D + c], s);
      s *= scale_log2;
      if (s > m) {
        const float a = exp2f(m - s);
        l *= a;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] *= a;
        m = s;
      }
      const float p = exp2f(s - m);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = fmaf(p, vs[jj * D + c], o[c]);
    }
  }
  if (i < T) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) O[hoff + (int64_t)i * qs + c] = o[c] * inv;
    if (LSE) LSE[(int64_t)bh * T + i] = (m + log2f(l)) * kLn2;
  }
}

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                               float* lse, const Dims& dm, int window, int causal,
                               hipStream_t stream) {
  const int BH = dm.B * dm.H, T = dm.T, d = dm.d;
  const Geometry geo = make_geometry(dm);
  const int nqb = (T + 63) / 64;
  const unsigned grid = (unsigned)((int64_t)BH * nqb);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
#define ATTN_F32_CASE(DD)                                                                       \
  if (d == DD) {                                                                                \
    hipLaunchKernelGGL(attn_fwd_f32_kernel<DD>, dim3(grid), dim3(64), 0, stream, q, k, v, out, \
                       lse, geo, BH, T, window, causal, scale_log2, nqb);                      \
    return hipGetLastError();                                                                   \
  }
  ATTN_F32_CASE(16)
  ATTN_F32_CASE(32)
  ATTN_F32_CASE(64)
  ATTN_F32_CASE(128)
#undef ATTN_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
