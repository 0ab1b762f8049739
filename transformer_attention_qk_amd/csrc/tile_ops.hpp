// LDS tile layout, buffer-resource loads and lane exchanges shared by the MFMA attention kernels
// (forward and backward) of libattn.
#pragma once

#include "common.hpp"

namespace attn {

// Physical 16-byte chunk of logical chunk c in LDS row r of a K tile: quarter-wave K reads
// touch 16 consecutive rows at one logical chunk, which this spreads over all 64 banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;
  else if constexpr (D == 64) return (r >> 1) & 7;
  else return r & 15;
}
// Same for a V tile: half-wave transposing reads touch 4 consecutive rows x 64 bytes.
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 32) return 0;
  else if constexpr (D == 64) return ((r >> 1) & 1) << 2;
  else return (r & 3) << 2;
}

// Same for the staged rows of rotation factors (d/2 fp32 per row, CPR = d/8 chunks): a half-wave
// reads one logical chunk of 16 consecutive rows, RPL of which share a 256-byte LDS line, so the
// chunk is rotated by the row's line index to put the 16 reads on distinct banks.
template <int D>
__device__ __forceinline__ int swz_rope(int r) {
  constexpr int CPR = D / 8;
  constexpr int RPL = (256 / (CPR * 16)) > 0 ? 256 / (CPR * 16) : 1;
  return (r / RPL) % CPR;
}

typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

// Word 3 of a raw (unswizzled, stride 0) buffer resource on gfx9-family GPUs: 32-bit data format.
constexpr int kBufferWord3 = 0x00020000;
// Offset past any head slab (slabs are < 2^31 bytes): such buffer loads return zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), (short)0, bytes, kBufferWord3);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Direct global -> LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane L's bytes
// land at LDS address lds_base + 16 L (lds_base is wave-uniform, through M0), its source is the
// buffer offset voff (out of range reads zero). Written in assembly because the compiler, which
// cannot tell which LDS bytes such a load writes, drains every outstanding one before each
// barrier; the kernel waits for them itself with s_waitcnt vmcnt. The instruction returns no
// registers, so nothing in flight can be overwritten.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Raw buffer resource (stride 0) over [base, base + bytes), as four scalar words.
__device__ __forceinline__ u32x4 head_rsrc_words(const bf16* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)bytes);
  r[3] = (uint32_t)kBufferWord3;
  return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Lanes l and l + 32 hold the same query row. v_permlane32_swap exchanges the upper half of one
// register with the lower half of another; applied to two copies of x, each lane ends up holding
// its own value in one result and its partner's in the other, so the max (or sum) of the two
// results is the pair's max (or sum) in every lane.
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

__device__ __forceinline__ u32x2 ds_read_tr16_b64(const char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4_ptr)((__attribute__((address_space(3))) char*)(p)));
  return __builtin_bit_cast(u32x2, v);
}

// Sum of the two bf16 halves of w, added to acc in fp32 (v_dot2_f32_bf16 with (1, 1)).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

// Mask of a launch, fixed at compile time so the per-element test is exactly what is needed.
enum MaskMode { kNonCausal = 0, kCausal = 1, kCausalWindow = 2 };

}  // namespace attn
