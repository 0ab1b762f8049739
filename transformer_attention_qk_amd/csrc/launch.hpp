// Internal launchers (host side). Arguments have been validated by the C ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.hpp"

namespace attn {

// Shape of one call: q and out are [B, H, T, d], k and v [B, H_kv, T, d] (H_kv divides H), all
// stored as [B][H][T][d] (layout 0) or [B][T][H][d] (layout 1).
struct Dims {
  int B, H, H_kv, T, d, layout;
};

// Where the rows of one (batch, head) live: element offset b * b + h * h + t * t of a [B, H, T, d]
// tensor stored as [B][H][T][d] or as [B][T][H][d]; q and out share one, k and v another (k and
// v have H / group heads: grouped-query attention maps q head h to kv head h / group).
struct Strides {
  int64_t b, h;
  int t;
};
struct Geometry {
  Strides q, kv;
  FastDiv H, group;  // query heads, and query heads per kv head
  __host__ __device__ __forceinline__ int64_t q_head(int bh) const {
    const uint32_t b = H.div((uint32_t)bh), h = (uint32_t)bh - b * H.d;
    return (int64_t)b * q.b + (int64_t)h * q.h;
  }
  __host__ __device__ __forceinline__ int64_t kv_head(int bh) const {
    const uint32_t b = H.div((uint32_t)bh), h = (uint32_t)bh - b * H.d;
    return (int64_t)b * kv.b + (int64_t)group.div(h) * kv.h;
  }
};

inline Geometry make_geometry(const Dims& dm) {
  Geometry g;
  const int64_t d = dm.d;
  if (dm.layout == 0) {  // [B][H][T][d]
    g.q = Strides{(int64_t)dm.H * dm.T * d, (int64_t)dm.T * d, (int)d};
    g.kv = Strides{(int64_t)dm.H_kv * dm.T * d, (int64_t)dm.T * d, (int)d};
  } else {  // [B][T][H][d]
    g.q = Strides{(int64_t)dm.T * dm.H * d, d, (int)(dm.H * d)};
    g.kv = Strides{(int64_t)dm.T * dm.H_kv * d, d, (int)(dm.H_kv * d)};
  }
  g.H = make_fastdiv((uint32_t)dm.H);
  g.group = make_fastdiv((uint32_t)(dm.H / dm.H_kv));
  return g;
}


// Heads per group of the head-grouped work order (see the kernels): all heads when the tiles
// they stream (bytes_per_head each) fit in the last-level cache together, else 32, so that the
// workgroups resident at once work on few heads and share their tiles through an XCD's L2.
inline int group_heads(int n_heads, int64_t bytes_per_head) {
  constexpr int64_t kCacheBudget = int64_t(128) << 20;  // half of MI355X's 256 MB Infinity Cache
  return ((int64_t)n_heads * bytes_per_head <= kCacheBudget) ? n_heads : 32;
}

hipError_t launch_rope_table(float* cos_tab, float* sin_tab, int T, int d, double base,
                             hipStream_t stream);

// Value-embedding gate rows of a prologue launch: v_out = v + 2 sigmoid(z) ve (v == nullptr: none).
struct GateArgs {
  const void *v = nullptr, *ve = nullptr, *z = nullptr;
  void* v_out = nullptr;
};

// dtype: 0 = bf16, 1 = f32. d in {16, 32, 64, 128}. q == nullptr: no q rows (q_out unused);
// k == nullptr: no k rows (then vg must name v rows).
hipError_t launch_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, const Dims& dm,
                              float eps, int dtype, hipStream_t stream,
                              const GateArgs& vg = GateArgs{});

// Backward of the gate: dve = g dv, dz = g (1 - g/2) sum_j ve_j dv_j with g = 2 sigmoid(z).
hipError_t launch_value_gate_bwd(const void* ve, const void* z, const void* dv, void* dve,
                                 void* dz, const Dims& dm, int dtype, hipStream_t stream);

// bf16 attention on MFMA. d in {32, 64, 128}.
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                const Dims& dm, int window, int causal, hipStream_t stream);

// bf16 attention on MFMA whose Q rows are RMS-normalised and rotated inside the kernel (k must
// already be normalised and rotated). d in {32, 64, 128}.
hipError_t launch_attn_fwd_bf16_qknorm(const void* q, const void* k, const void* v, void* out,
                                       float* lse, const float* cos_tab, const float* sin_tab,
                                       float eps, const Dims& dm, int window, int causal,
                                       hipStream_t stream);

// The same with raw k: each K tile is RMS-normalised and rotated inside the kernel, in LDS, and
// the normalised k is not written. d in {32, 64}.
hipError_t launch_attn_fwd_bf16_qknorm_kin(const void* q, const void* k, const void* v, void* out,
                                           float* lse, const float* cos_tab,
                                           const float* sin_tab, float eps, const Dims& dm,
                                           int window, int causal, hipStream_t stream);

// fp32 attention. d in {16, 32, 64, 128}.
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                               float* lse, const Dims& dm, int window, int causal,
                               hipStream_t stream);

// Backward of the QK-norm + RoPE prologue: dq_out, dk_out from the raw rows q, k and the
// gradients dq_in, dk_in of the prologue's outputs (outputs may equal the inputs' gradients).
// q == nullptr: k rows only.
hipError_t launch_qknorm_rope_bwd(const void* q, const void* k, const void* dq_in,
                                  const void* dk_in, void* dq_out, void* dk_out,
                                  const float* cos_tab, const float* sin_tab, const Dims& dm,
                                  float eps, int dtype, hipStream_t stream);

// Attention backward: delta (fp32 [B][H][T]) = rowsum(dout * out), then dq, dk, dv.
// bf16: d in {32, 64, 128}; f32: d in {16, 32, 64, 128}.
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, float* delta, void* dq, void* dk,
                           void* dv, const Dims& dm, int window, int causal, int dtype,
                           hipStream_t stream);

// Decode: one query per (batch, head) against a cache of dm.T slots (lengths: device int32 [B]
// or nullptr for all dm.T). ws: decode_workspace_bytes(...) bytes of device memory.
int decode_splits(int B, int H, int S, int d, int window);
int64_t decode_workspace_bytes(int B, int H, int S, int d, int window);
hipError_t launch_attn_decode(const void* q, const void* k, const void* v, const int* lengths,
                              void* out, float* lse, void* ws, const Dims& dm, int window,
                              int dtype, hipStream_t stream);

// Decode scratch for callers that cannot allocate: a static device array of
// kDecodeScratchBytes per GPU. decode_scratch returns its device address on the current device.
constexpr int64_t kDecodeScratchBytes = int64_t(8) << 20;
hipError_t decode_scratch(void** ptr);

}  // namespace attn
