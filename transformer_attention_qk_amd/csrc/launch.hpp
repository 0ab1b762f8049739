// Internal launchers (host side). Arguments have been validated by the C ABI layer in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

hipError_t launch_rope_table(float* cos_tab, float* sin_tab, int T, int d, double base,
                             hipStream_t stream);

// dtype: 0 = bf16, 1 = f32. d in {16, 32, 64, 128}. q == nullptr: k rows only (q_out unused).
hipError_t launch_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                              const float* cos_tab, const float* sin_tab, int B, int H, int T,
                              int d, float eps, int dtype, hipStream_t stream);

// bf16 attention on MFMA. d in {32, 64, 128}.
hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int d, int window, int causal,
                                hipStream_t stream);

// bf16 attention on MFMA whose Q rows are RMS-normalised and rotated inside the kernel (k must
// already be normalised and rotated). d in {32, 64, 128}.
hipError_t launch_attn_fwd_bf16_qknorm(const void* q, const void* k, const void* v, void* out,
                                       float* lse, const float* cos_tab, const float* sin_tab,
                                       float eps, int B, int H, int T, int d, int window,
                                       int causal, hipStream_t stream);

// fp32 attention. d in {16, 32, 64, 128}.
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                               float* lse, int B, int H, int T, int d, int window, int causal,
                               hipStream_t stream);

}  // namespace attn
