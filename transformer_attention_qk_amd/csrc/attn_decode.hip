// Decode: one new query per (batch, head) against the cached keys and values (generation appends
// one token at a time and runs the same forward, "A Máscara Causal" on "Projeção em um Subespaço
// de Consulta", unhomeschool.com; "O Que um Modelo de Linguagem Prevê": autoregressive
// generation). The newest token (position n - 1 of a batch entry with n cached tokens, its own
// key and value included) attends to keys max(0, n - 1 - window) .. n - 1:
//   out = sum_j softmax_j(q . k_j / sqrt(d)) v_j,   lse = ln sum_j exp(q . k_j / sqrt(d)).
//
// A single query row is a matrix-vector product, bound by reading the cache (4 d bytes per key
// in bf16), so the work is split over the keys, and what keeps the reads near the HBM rate is how
// many bytes each wave has in flight. A workgroup takes (batch, kv head, split of the keys); each
// of its four waves loads its own 4096 / d rows of K and of V straight into registers (16 KB in
// bf16, every load issued before the first use) and, for every query head of the group (GQA: the
// cache is read once for the whole group), forms the scores (fp32), their maximum m, the weights
// exp2(s - m), their sum l and the weighted sum of the V rows with shuffles inside the wave only.
// The four waves' (m, l, o) meet in LDS, one barrier per query head. With one split per
// (batch, kv head) (many heads, short caches) the workgroup writes out and lse itself; otherwise
// it writes its split's o, unnormalised, with m and l to the caller's workspace, and a merge
// kernel combines the splits of each (batch, head):
//   M = max_c m_c,  L = sum_c l_c 2^(m_c - M),  out = sum_c o_c 2^(m_c - M) / L,
//   lse = (M + log2 L) ln 2.
// The weights stay fp32 (no bf16 rounding), every sum is fp32, out is rounded once.
#include <math.h>

#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace attn {

constexpr int kDecodeWaves = 4;  // waves per workgroup, each with its own rows

// Keys per wave and batch: 4096 / d rows of K and of V, i.e. 8 (bf16) or 16 (fp32) 16-byte
// loads per lane and tensor. A split of the keys is one workgroup's four waves: one batch each
// while that gives at most kDecodeTargetGroups workgroups, else fewer splits with several batches
// per wave (long caches), which keeps the merge short.
constexpr int decode_wave_keys(int d) { return d >= 4096 ? 1 : 4096 / d; }
constexpr int decode_split_keys(int d) { return kDecodeWaves * decode_wave_keys(d); }
constexpr int kDecodeTargetGroups = 2048;
// One split per (batch, kv head) instead, written out without a merge, when those workgroups give
// at least kDecodeSingleWaves waves and each wave takes at most kDecodeSingleBatches batches.
constexpr int kDecodeSingleWaves = 256;
constexpr int kDecodeSingleBatches = 4;

template <typename Elem, int D>
struct DecCfg {
  static constexpr int E = 16 / (int)sizeof(Elem);  // elements per 16-byte chunk
  static constexpr int CHR = D / E;                  // lanes per row: one chunk each
  static constexpr int RPL = 64 / CHR;               // rows covered by one load of a wave
  static constexpr int KW = decode_wave_keys(D);     // rows per wave
  static constexpr int NL = KW / RPL;                // loads per lane and tensor
  static_assert(CHR >= 1 && CHR <= 64 && 64 % CHR == 0, "a row must span a power of two lanes");
  static_assert(NL >= 1 && NL * RPL == KW, "rows per wave must be whole loads");
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

// FINAL: one split per (batch, kv head) (n_split = 1); the workgroup writes out and lse itself
// and the workspace is not touched.
template <typename Elem, int D, bool FINAL, int NW = kDecodeWaves>
__global__ __launch_bounds__(64 * NW) void attn_decode_partial(
    const Elem* __restrict__ Qv, const Elem* __restrict__ K, const Elem* __restrict__ V,
    const int* __restrict__ lengths, float* __restrict__ ws, Elem* __restrict__ out,
    float* __restrict__ lse, Geometry geo, int H_kv, int S, int window, int n_split,
    int64_t parts, float scale_log2) {
  using C = DecCfg<Elem, D>;
  // Per query head (two heads alternate, so one barrier per head suffices): each wave's
  // unnormalised o[D], then its m and l.
  __shared__ float red[2][NW][D + 2];
  const int tid = (int)threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = (int)blockIdx.x % n_split;
  const int bg = (int)blockIdx.x / n_split;
  const int b = bg / H_kv, g = bg - b * H_kv;
  const int H = (int)geo.H.d, G = (int)geo.group.d;
  int n = (lengths != nullptr) ? lengths[b] : S;
  n = min(max(n, 1), S);
  const int lo = (window >= 0) ? max(0, n - 1 - window) : 0;
  // The entry's keys [lo, n) in n_split equal splits, each in four equal parts, one per wave;
  // a wave takes its part in batches of KW rows. Parts past n are empty.
  const int per_split = (n - lo + n_split - 1) / n_split;
  const int s0 = lo + split * per_split;
  const int s1 = min(n, s0 + per_split);
  const int per_wave = (per_split + NW - 1) / NW;
  const int w0 = s0 + wave * per_wave;
  const int cnt = min(s1, w0 + per_wave) - w0;  // rows of this wave (wave-uniform; may be <= 0)
  // Workspace: unnormalised outputs [B][H][n_split][D], then m and l [B][H][n_split].
  float* ws_o = ws;
  float* ws_m = ws + parts * D;
  float* ws_l = ws_m + parts;

  // Lane l holds chunk c = l % CHR of rows rl + RPL u (u < NL) of a batch, so the reads of one
  // load cover RPL consecutive rows.
  const int64_t kvoff = (int64_t)b * geo.kv.b + (int64_t)g * geo.kv.h;
  const int rl = lane / C::CHR, c = lane % C::CHR;
  u32x4 kr[C::NL], vr[C::NL];
  auto load_batch = [&](int r0) {
#pragma unroll
    for (int u = 0; u < C::NL; ++u) {
      const int r = r0 + u * C::RPL + rl;
      kr[u] = u32x4{0u, 0u, 0u, 0u};
      vr[u] = u32x4{0u, 0u, 0u, 0u};
      if (r < cnt) {
        const int64_t off = kvoff + (int64_t)(w0 + r) * geo.kv.t + c * C::E;
        kr[u] = *reinterpret_cast<const u32x4*>(K + off);
        vr[u] = *reinterpret_cast<const u32x4*>(V + off);
      }
    }
  };
  load_batch(0);  // before the query is read, so the cache reads go out first

  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    float qv[C::E];
    chunk_f32<Elem>(*reinterpret_cast<const u32x4*>(Qv + ((int64_t)b * H + h) * D + c * C::E), qv);
    // Running maximum m (base-2 units), sum l and this lane's chunk of the weighted V sum over the
    // wave's batches (one-pass softmax; the first batch sets m).
    float m = -INFINITY, l = 0.f, acc[C::E];
#pragma unroll
    for (int e = 0; e < C::E; ++e) acc[e] = 0.f;
    for (int r0 = 0; r0 < cnt; r0 += C::KW) {
      // The registers hold the first batch for the first head, and for every head when the
      // part is one batch.
      if (r0 > 0 || (hh > 0 && cnt > C::KW)) load_batch(r0);
      // Scores: this lane's part of each row's dot product, summed over the row's CHR lanes;
      // rows past the part are -inf.
      float sc[C::NL];
      float mb = -INFINITY;
#pragma unroll
      for (int u = 0; u < C::NL; ++u) {
        float y[C::E];
        chunk_f32<Elem>(kr[u], y);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < C::E; ++e) a = fmaf(qv[e], y[e], a);
#pragma unroll
        for (int o = 1; o < C::CHR; o <<= 1) a += __shfl_xor(a, o);
        sc[u] = (r0 + u * C::RPL + rl < cnt) ? a * scale_log2 : -INFINITY;
        mb = fmaxf(mb, sc[u]);
      }
      // The lanes of a row share its score, so the wave's reductions cross the row groups only.
#pragma unroll
      for (int o = C::CHR; o < 64; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
      const float mn = fmaxf(m, mb);              // finite: the batch has a row
      const float f = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first batch
      float lb = 0.f;
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] *= f;
#pragma unroll
      for (int u = 0; u < C::NL; ++u) {
        const float p = __builtin_amdgcn_exp2f(sc[u] - mn);  // 0 for rows past the part
        lb += p;
        float y[C::E];
        chunk_f32<Elem>(vr[u], y);
#pragma unroll
        for (int e = 0; e < C::E; ++e) acc[e] = fmaf(p, y[e], acc[e]);
      }
      l = fmaf(l, f, lb);
      m = mn;
    }
    // Sums over the row groups (acc and l are per lane until here; m is already the wave's).
#pragma unroll
    for (int o = C::CHR; o < 64; o <<= 1) {
      l += __shfl_xor(l, o);
#pragma unroll
      for (int e = 0; e < C::E; ++e) acc[e] += __shfl_xor(acc[e], o);
    }
    float* rw = red[hh & 1][wave];
    if (rl == 0) {
#pragma unroll
      for (int e = 0; e < C::E; ++e) rw[c * C::E + e] = acc[e];
    }
    if (lane == 0) {
      rw[D] = m;
      rw[D + 1] = l;
    }
    __syncthreads();
    // The split's (m, l, o) from its waves' (empty parts: l = 0, weight 0).
    if (tid < D) {
      float (*rp)[D + 2] = red[hh & 1];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (rp[w][D + 1] > 0.f) M = fmaxf(M, rp[w][D]);
      float L = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float lw = rp[w][D + 1];
        if (lw > 0.f) {
          const float fw = __builtin_amdgcn_exp2f(rp[w][D] - M);
          L = fmaf(lw, fw, L);
          o = fmaf(rp[w][tid], fw, o);
        }
      }
      if constexpr (FINAL) {  // L > 0: the entry has a key, and it is in this split
        out[((int64_t)b * H + h) * D + tid] = (Elem)(o * (1.0f / L));
        if (tid == 0 && lse != nullptr) lse[(int64_t)b * H + h] = (M + __log2f(L)) * kLn2;
      } else {
        const int64_t part = ((int64_t)b * H + h) * n_split + split;
        ws_o[part * D + tid] = o;
        if (tid == 0) {
          ws_m[part] = M;
          ws_l[part] = L;
        }
      }
    }
  }
}

// One block of 256 threads per (batch, head): thread (e, cg) folds output element e over the
// splits c = cg, cg + NG, ... (NG = 256 / D) in one pass with a running maximum, then the NG
// partial results meet in LDS.
template <typename Elem, int D>
__global__ __launch_bounds__(256) void attn_decode_merge(const float* __restrict__ ws,
                                                         Elem* __restrict__ out,
                                                         float* __restrict__ lse, int n_split,
                                                         int64_t parts) {
  constexpr int NG = 256 / D;
  __shared__ float sm[3][NG][D];
  const int bh = (int)blockIdx.x, tid = (int)threadIdx.x;
  const int e = tid % D, cg = tid / D;
  const float* ws_m = ws + parts * D + (int64_t)bh * n_split;
  const float* ws_l = ws_m + parts;
  const float* ws_o = ws + (int64_t)bh * n_split * D;
  // Empty splits (l = 0, m = -inf, o = 0) get weight 0.
  float M = -INFINITY, L = 0.f, o = 0.f;
#pragma unroll 8
  for (int c = cg; c < n_split; c += NG) {
    const float lc = ws_l[c], mc = ws_m[c], oc = ws_o[(int64_t)c * D + e];
    if (lc > 0.f) {
      const float mn = fmaxf(M, mc);
      const float f = __builtin_amdgcn_exp2f(M - mn), w = __builtin_amdgcn_exp2f(mc - mn);
      L = fmaf(L, f, lc * w);
      o = fmaf(o, f, oc * w);
      M = mn;
    }
  }
  sm[0][cg][e] = M;
  sm[1][cg][e] = L;
  sm[2][cg][e] = o;
  __syncthreads();
  if (cg == 0) {
    float Mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < NG; ++i)
      if (sm[1][i][e] > 0.f) Mt = fmaxf(Mt, sm[0][i][e]);
    float Lt = 0.f, ot = 0.f;
#pragma unroll
    for (int i = 0; i < NG; ++i) {
      if (sm[1][i][e] > 0.f) {
        const float w = __builtin_amdgcn_exp2f(sm[0][i][e] - Mt);
        Lt = fmaf(sm[1][i][e], w, Lt);
        ot = fmaf(sm[2][i][e], w, ot);
      }
    }
    out[(int64_t)bh * D + e] = (Elem)(ot * (1.0f / Lt));
    if (e == 0 && lse != nullptr) lse[bh] = (Mt + __log2f(Lt)) * kLn2;
  }
}

// Scratch of the allocation-free decode entry point: the split partials live in this fixed
// device array (one copy per GPU, held until the process ends) instead of a caller workspace.
// Host code never passes the array's name to a kernel: it is a host-side stand-in there. The
// device address comes from hipGetSymbolAddress, once per device, and is kept below.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);  // racing threads store the same address
  }
  *ptr = p;
  return hipSuccess;
}

// Compute units of the current device (cached per device; threads that race on the first query
// store the same value).
static int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  if (slot && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

int decode_splits(int B, int H, int S, int d, int window) {
  const int keys = (window >= 0 && window + 1 < S) ? window + 1 : S;
  const int64_t by_keys = (keys + decode_split_keys(d) - 1) / decode_split_keys(d);
  const int64_t heads = (int64_t)B * H;
  const int64_t cap = (kDecodeTargetGroups + heads - 1) / heads;
  return (int)(by_keys < cap ? by_keys : cap);
}

int64_t decode_workspace_bytes(int B, int H, int S, int d, int window) {
  return (int64_t)B * H * decode_splits(B, H, S, d, window) * (d + 2) * 4;
}

template <typename Elem, int D>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const int* lengths,
                                  void* out, float* lse, void* ws, const Dims& dm, int window,
                                  hipStream_t stream) {
  const Geometry geo = make_geometry(dm);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  // One split per (batch, kv head), with no merge launch, when those workgroups alone give
  // kDecodeSingleWaves waves and no wave takes more than kDecodeSingleBatches batches.
  const int keys = (window >= 0 && window + 1 < dm.T) ? window + 1 : dm.T;
  if ((int64_t)dm.B * dm.H_kv * kDecodeWaves >= kDecodeSingleWaves &&
      keys <= kDecodeSingleBatches * decode_split_keys(D)) {
    // bf16 with more than four batches and at most one workgroup per compute unit: eight waves
    // instead of four (each with at most two batches), twice the loads in flight for the same
    // workgroups. An eight-wave workgroup takes a whole compute unit's registers, so with more
    // workgroups than compute units four waves keep them all resident at once. (Sixteen waves
    // would cap the registers at 128 per lane, below what a wave's batch takes: it spills.)
    const int batches = (keys + decode_wave_keys(D) - 1) / decode_wave_keys(D);
    const dim3 grid((unsigned)(dm.B * dm.H_kv));
#define ATTN_DEC_SINGLE(NWV)                                                                     \
  hipLaunchKernelGGL((attn_decode_partial<Elem, D, true, NWV>), grid, dim3(64 * NWV), 0, stream, \
                     (const Elem*)q, (const Elem*)k, (const Elem*)v, lengths, (float*)ws,        \
                     (Elem*)out, lse, geo, dm.H_kv, dm.T, window, 1, (int64_t)dm.B * dm.H,       \
                     scale_log2)
    bool eight = false;
    if constexpr (sizeof(Elem) == 2) {
      eight = batches > 4 && (int64_t)dm.B * dm.H_kv <= device_cus();
      if (eight) ATTN_DEC_SINGLE(8);
    }
    if (!eight) ATTN_DEC_SINGLE(4);
#undef ATTN_DEC_SINGLE
    return hipGetLastError();
  }
  const int n_split = decode_splits(dm.B, dm.H, dm.T, D, window);
  const int64_t parts = (int64_t)dm.B * dm.H * n_split;
  hipLaunchKernelGGL((attn_decode_partial<Elem, D, false>),
                     dim3((unsigned)(dm.B * dm.H_kv * n_split)), dim3(256), 0, stream,
                     (const Elem*)q, (const Elem*)k, (const Elem*)v, lengths, (float*)ws,
                     (Elem*)out, lse, geo, dm.H_kv, dm.T, window, n_split, parts, scale_log2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_merge<Elem, D>), dim3((unsigned)(dm.B * dm.H)), dim3(256), 0,
                     stream, (const float*)ws, (Elem*)out, lse, n_split, parts);
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
