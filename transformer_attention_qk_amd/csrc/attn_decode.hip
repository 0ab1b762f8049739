// Decode: one new query per (batch, head) against the cached keys and values (generation appends
// one token at a time and runs the same forward, "A Máscara Causal" on "Projeção em um Subespaço
// de Consulta", unhomeschool.com; "O Que um Modelo de Linguagem Prevê": autoregressive
// generation). The newest token (position n - 1 of a batch entry with n cached tokens, its own
// key and value included) attends to keys max(0, n - 1 - window) .. n - 1:
//   out = sum_j softmax_j(q . k_j / sqrt(d)) v_j,   lse = ln sum_j exp(q . k_j / sqrt(d)).
//
// A single query row is a matrix-vector product, bound by reading the cache (4 d bytes per key
// in bf16), so the work is split over the keys: one workgroup per (batch, kv head, chunk of 128
// keys) stages its chunk of K and V in LDS with coalesced 16-byte loads, then for every query
// head of the group forms the chunk's scores (fp32), its maximum m, weights exp2(s - m) and
// their sum l, and the weighted sum of the V rows, written unnormalised with m and l to the
// caller's workspace. A merge kernel combines the chunks of each (batch, head):
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  out = sum_c o_c 2^(m_c - M) / L,
//   lse = (M + log2 L) ln 2.
// The weights stay fp32 (no bf16 rounding), every sum is fp32, out is rounded once.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kDecodeChunk = 128;  // keys per workgroup
constexpr int kDecodeHeads = 4;    // query heads per pass over a staged chunk

template <typename Elem, int D>
struct DecCfg {
  static constexpr int CK = kDecodeChunk;
  static constexpr int HB = kDecodeHeads;
  static constexpr int E = 16 / (int)sizeof(Elem);          // elements per 16-byte chunk
  static constexpr int CHR = D / E;                          // 16-byte chunks per row
  static constexpr int ROWB = D * (int)sizeof(Elem) + 16;    // padded LDS row (bank spread)
  static constexpr int V_BYTES = CK * ROWB;
  static_assert(CK <= 128, "two threads per key: a chunk holds at most 128 keys");
  static constexpr int RED = 4 * HB * D * 4;  // per-wave partial sums of the outputs
  static constexpr int LDS = V_BYTES + HB * D * 4 + HB * CK * 4 + 2 * HB * 4 + RED;
};

template <typename Elem>
__device__ __forceinline__ float elem_f32(Elem x) { return (float)x; }

// The 16 bytes of w as fp32 values (8 bf16 or 4 fp32), converted exactly.
template <typename Elem>
__device__ __forceinline__ void chunk_f32(u32x4 w, float (&x)[16 / sizeof(Elem)]) {
  if constexpr (sizeof(Elem) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = bf16lo_to_f32(w[i]);
      x[2 * i + 1] = bf16hi_to_f32(w[i]);
    }
  } else {
    const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = f[i];
  }
}

template <typename Elem, int D>
__global__ __launch_bounds__(256, 2) void attn_decode_partial(
    const Elem* __restrict__ Qv, const Elem* __restrict__ K, const Elem* __restrict__ V,
    const int* __restrict__ lengths, float* __restrict__ ws, Geometry geo, int H_kv, int S,
    int window, int n_split, int64_t parts, float scale_log2) {
  using C = DecCfg<Elem, D>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  char* vs = smem;
  float* qs = reinterpret_cast<float*>(smem + C::V_BYTES);        // [HB][D]
  float* ss = qs + C::HB * D;                                     // [HB][CK]
  float* ms = ss + C::HB * C::CK;                                 // [HB]
  float* ls = ms + C::HB;                                         // [HB]
  float* red = ls + C::HB;                                        // [4 waves][HB][D]
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = (int)blockIdx.x % n_split;
  const int bg = (int)blockIdx.x / n_split;
  const int b = bg / H_kv, g = bg - b * H_kv;
  const int H = (int)geo.H.d, G = (int)geo.group.d;
  int n = (lengths != nullptr) ? lengths[b] : S;
  n = min(max(n, 1), S);
  const int lo = (window >= 0) ? max(0, n - 1 - window) : 0;
  const int c0 = lo + split * C::CK;
  const int cnt = min(n, c0 + C::CK) - c0;  // keys of this chunk (block-uniform; may be <= 0)
  // Workspace: unnormalised outputs [B][H][n_split][D], then m and l [B][H][n_split].
  float* ws_o = ws;
  float* ws_m = ws + parts * D;
  float* ws_l = ws_m + parts;

  if (cnt <= 0) {  // an empty chunk (short entry): weight 0 in the merge
    for (int idx = tid; idx < G * D; idx += 256) {
      const int hh = idx / D, e = idx - hh * D;
      const int64_t part = ((int64_t)b * H + g * G + hh) * n_split + split;
      ws_o[part * D + e] = 0.f;
      if (e == 0) {
        ws_m[part] = -INFINITY;
        ws_l[part] = 0.f;
      }
    }
    return;
  }

  // Threads 2 j and 2 j + 1 hold the two halves of key j's row in registers (the reads of a wave
  // cover 32 consecutive rows); the V rows are staged in LDS. Every load is issued before the
  // first store, so their latencies overlap.
  const int64_t kvoff = (int64_t)b * geo.kv.b + (int64_t)g * geo.kv.h;
  const int kj = tid >> 1, half = tid & 1;
  const bool live = kj < cnt;
  u32x4 kr[C::CHR / 2];
  if (live) {
    const Elem* krow = K + kvoff + (int64_t)(c0 + kj) * geo.kv.t + half * (D / 2);
#pragma unroll
    for (int c = 0; c < C::CHR / 2; ++c) kr[c] = *reinterpret_cast<const u32x4*>(krow + c * C::E);
  }
  {
    constexpr int LPT = (C::CK * C::CHR + 255) / 256;
    u32x4 xv[LPT];
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int p = u * 256 + tid;
      const int r = p / C::CHR, c = p - r * C::CHR;
      if (r < cnt)
        xv[u] = *reinterpret_cast<const u32x4*>(V + kvoff + (int64_t)(c0 + r) * geo.kv.t + c * C::E);
    }
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
      const int p = u * 256 + tid;
      const int r = p / C::CHR, c = p - r * C::CHR;
      if (r < cnt) *reinterpret_cast<u32x4*>(vs + r * C::ROWB + 16 * c) = xv[u];
    }
  }
  if (!live) {
#pragma unroll
    for (int c = 0; c < C::CHR / 2; ++c) kr[c] = u32x4{0u, 0u, 0u, 0u};
  }

  for (int hb0 = 0; hb0 < G; hb0 += C::HB) {
    const int nh = min(C::HB, G - hb0);
    __syncthreads();  // the chunk is staged; the previous pass is done with qs, ss
    for (int idx = tid; idx < nh * D; idx += 256) {
      const int hh = idx / D, e = idx - hh * D;
      qs[hh * D + e] = elem_f32(Qv[((int64_t)b * H + g * G + hb0 + hh) * D + e]);
    }
    __syncthreads();
    // Scores: threads 2 j and 2 j + 1 take the two halves of key j's dot product with each head.
    for (int hh = 0; hh < nh; ++hh) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < C::CHR / 2; ++c) {
        float y[C::E];
        chunk_f32<Elem>(kr[c], y);
#pragma unroll
        for (int e = 0; e < C::E; ++e)
          acc = fmaf(qs[hh * D + half * (D / 2) + c * C::E + e], y[e], acc);
      }
      acc += __shfl_xor(acc, 1);
      if (half == 0 && kj < C::CK) ss[hh * C::CK + kj] = live ? acc * scale_log2 : -INFINITY;
    }
    __syncthreads();
    // Per head: maximum, weights, their sum (one wave per head).
    for (int hh = wave; hh < nh; hh += 4) {
      float m = -INFINITY;
      for (int j = lane; j < C::CK; j += 64) m = fmaxf(m, ss[hh * C::CK + j]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      float l = 0.f;
      for (int j = lane; j < C::CK; j += 64) {
        const float p = (j < cnt) ? __builtin_amdgcn_exp2f(ss[hh * C::CK + j] - m) : 0.f;
        ss[hh * C::CK + j] = p;
        l += p;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
      if (lane == 0) {
        ms[hh] = m;
        ls[hh] = l;
      }
    }
    __syncthreads();
    // Weighted sum of the V rows: thread t takes the 16-byte chunk c = t % CHR of the rows of
    // key group kg = t / CHR (keys kg, kg + NKG, ...); the key groups of a wave meet through xor
    // shuffles, the four waves' sums in LDS.
    {
      constexpr int NKG = 256 / C::CHR;
      const int c = tid % C::CHR, kg = tid / C::CHR;
      float acc[C::HB][C::E];
#pragma unroll
      for (int hh = 0; hh < C::HB; ++hh)
#pragma unroll
        for (int e = 0; e < C::E; ++e) acc[hh][e] = 0.f;
#pragma unroll 4
      for (int j = kg; j < cnt; j += NKG) {
        float y[C::E];
        chunk_f32<Elem>(*reinterpret_cast<const u32x4*>(vs + j * C::ROWB + 16 * c), y);
#pragma unroll
        for (int hh = 0; hh < C::HB; ++hh) {
          const float pj = (hh < nh) ? ss[hh * C::CK + j] : 0.f;
#pragma unroll
          for (int e = 0; e < C::E; ++e) acc[hh][e] = fmaf(pj, y[e], acc[hh][e]);
        }
      }
#pragma unroll
      for (int o = C::CHR; o < 64; o <<= 1)
#pragma unroll
        for (int hh = 0; hh < C::HB; ++hh)
#pragma unroll
          for (int e = 0; e < C::E; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], o);
      if (lane < C::CHR) {
#pragma unroll
        for (int hh = 0; hh < C::HB; ++hh)
#pragma unroll
          for (int e = 0; e < C::E; ++e) red[(wave * C::HB + hh) * D + c * C::E + e] = acc[hh][e];
      }
      __syncthreads();
      for (int idx = tid; idx < nh * D; idx += 256) {
        const int hh = idx / D, ee = idx - hh * D;
        const float o = red[(0 * C::HB + hh) * D + ee] + red[(1 * C::HB + hh) * D + ee] +
                        red[(2 * C::HB + hh) * D + ee] + red[(3 * C::HB + hh) * D + ee];
        const int64_t part = ((int64_t)b * H + g * G + hb0 + hh) * n_split + split;
        ws_o[part * D + ee] = o;
        if (ee == 0) {
          ws_m[part] = ms[hh];
          ws_l[part] = ls[hh];
        }
      }
    }
  }
}

template <typename Elem, int D>
__global__ __launch_bounds__(128) void attn_decode_merge(const float* __restrict__ ws,
                                                         Elem* __restrict__ out,
                                                         float* __restrict__ lse, int n_split,
                                                         int64_t parts) {
  __shared__ float red[2][2];
  const int bh = (int)blockIdx.x, tid = (int)threadIdx.x, nt = (int)blockDim.x;
  const float* ws_m = ws + parts * D + (int64_t)bh * n_split;
  const float* ws_l = ws + parts * D + parts + (int64_t)bh * n_split;
  const float* ws_o = ws + (int64_t)bh * n_split * D;
  // M = max_c m_c and L = sum_c l_c 2^(m_c - M) over the chunks (empty chunks: l = 0), reduced
  // over the block (at most two waves).
  auto block_reduce = [&](float x, bool is_max) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float y = __shfl_xor(x, o);
      x = is_max ? fmaxf(x, y) : x + y;
    }
    if ((tid & 63) == 0) red[is_max][tid >> 6] = x;
    __syncthreads();
    const int nw = (nt + 63) / 64;
    float r = red[is_max][0];
    for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, red[is_max][w]) : r + red[is_max][w];
    return r;
  };
  float m = -INFINITY;
  for (int c = tid; c < n_split; c += nt) m = fmaxf(m, ws_m[c]);
  const float M = block_reduce(m, true);
  float l = 0.f;
  for (int c = tid; c < n_split; c += nt)
    l += (ws_l[c] > 0.f) ? ws_l[c] * __builtin_amdgcn_exp2f(ws_m[c] - M) : 0.f;
  const float L = block_reduce(l, false);
  const float inv = 1.0f / L;
  for (int e = tid; e < D; e += nt) {
    float o = 0.f;
#pragma unroll 4
    for (int c = 0; c < n_split; ++c) {
      const float w = (ws_l[c] > 0.f) ? __builtin_amdgcn_exp2f(ws_m[c] - M) : 0.f;
      o = fmaf(ws_o[(int64_t)c * D + e], w, o);
    }
    out[(int64_t)bh * D + e] = (Elem)(o * inv);
  }
  if (tid == 0 && lse != nullptr) lse[bh] = (M + __log2f(L)) * kLn2;
}

int decode_splits(int S, int window) {
  const int keys = (window >= 0 && window + 1 < S) ? window + 1 : S;
  return (keys + kDecodeChunk - 1) / kDecodeChunk;
}

int64_t decode_workspace_bytes(int B, int H, int S, int d, int window) {
  return (int64_t)B * H * decode_splits(S, window) * (d + 2) * 4;
}

template <typename Elem, int D>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const int* lengths,
                                  void* out, float* lse, void* ws, const Dims& dm, int window,
                                  hipStream_t stream) {
  const int n_split = decode_splits(dm.T, window);
  const int64_t parts = (int64_t)dm.B * dm.H * n_split;
  const Geometry geo = make_geometry(dm);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL((attn_decode_partial<Elem, D>), dim3((unsigned)(dm.B * dm.H_kv * n_split)),
                     dim3(256), 0, stream, (const Elem*)q, (const Elem*)k, (const Elem*)v, lengths,
                     (float*)ws, geo, dm.H_kv, dm.T, window, n_split, parts, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_merge<Elem, D>), dim3((unsigned)(dm.B * dm.H)),
                     dim3(D < 128 ? D : 128), 0, stream, (const float*)ws, (Elem*)out, lse,
                     n_split, parts);
  return hipGetLastError();
}

hipError_t launch_attn_decode(const void* q, const void* k, const void* v, const int* lengths,
                              void* out, float* lse, void* ws, const Dims& dm, int window,
                              int dtype, hipStream_t stream) {
#define ATTN_DEC_CASE(ELEM, DD) \
  if (dm.d == DD) return launch_decode_t<ELEM, DD>(q, k, v, lengths, out, lse, ws, dm, window, stream);
  if (dtype == 0) {
    ATTN_DEC_CASE(bf16, 32)
    ATTN_DEC_CASE(bf16, 64)
    ATTN_DEC_CASE(bf16, 128)
  } else {
    ATTN_DEC_CASE(float, 16)
    ATTN_DEC_CASE(float, 32)
    ATTN_DEC_CASE(float, 64)
    ATTN_DEC_CASE(float, 128)
  }
#undef ATTN_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
