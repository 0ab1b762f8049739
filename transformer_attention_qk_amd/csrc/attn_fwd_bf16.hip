// bf16 attention forward on gfx950 MFMA: causal / sliding-window flash attention with LSE.
//
// What it computes: out_i = sum_{j in A(i)} softmax_j(q_i . k_j / sqrt(d)) v_j and
// lse_i = ln sum_{j in A(i)} exp(q_i . k_j / sqrt(d)), where A(i) is the causal set j <= i cut
// to i - j <= window when window >= 0 ("Projeção em um Subespaço de Consulta", unhomeschool.com:
// "O que a Atenção Calcula", "Escalonamento por sqrt(d_k)", "A Máscara Causal"; the (W, 0)
// window of the attention call in `CausalSelfAttention.forward`, train.py listing of
// "Подробный технический разбор реализации Autoresearch", habr.com, article 1010198). The pages
// describe the attention kernel they call only as a one-pass kernel with sub-quadratic memory;
// the tiling and the one-pass (running maximum) softmax below are this library's design.
//
// Layout of the work:
//   - A workgroup of 4 waves owns BM = 128 consecutive queries of one (batch, head); wave w owns
//     queries [32w, 32w + 32) of that block. Workgroups are launched heaviest query block first
//     (the last blocks of a causal head see the most keys).
//   - Key/value tiles of BN = 64 rows flow HBM -> registers -> LDS through 2-slot LDS rings with
//     one barrier per tile: V one tile ahead, K two tiles ahead when the loop is pipelined
//     (below), else one.
//   - S^T = K Q^T per 32-key block with v_mfma_f32_32x32x16_bf16: A = K from LDS (16 bytes per
//     lane), B = Q^T kept in registers for the whole workgroup. In the accumulator each lane owns
//     one query (lane % 32) and 16 keys, so row maxima and sums are lane-local plus one exchange
//     between lanes l and l + 32.
//   - O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T accumulator (rounded to
//     bf16), A = V^T read from the row-major V tile with ds_read_b64_tr_b16, which transposes
//     4x16 blocks of 16-bit values between lanes. The key order inside each 16-key MFMA step
//     follows the S^T accumulator's register order on both operands.
//   - Software pipeline inside each wave (d <= 64): the iteration for tile t issues the scores
//     of tile t+1 on the matrix cores while the vector ALUs exponentiate tile t, then issues
//     P(t) V(t) while the vector ALUs mask and reduce the scores of tile t+1. Unmasked tiles
//     (the bulk) run this as one straight-line block with an explicit MFMA / VALU interleave.
//   - Row sums of the weights are taken with v_dot2_f32_bf16 on the bf16-rounded weights, i.e.
//     on exactly the values the P V product uses.
//   - LDS rows are XOR-swizzled in 16-byte chunks so that the K reads (16 rows x 16 bytes per
//     quarter-wave) and the transposing V reads (4 rows x 64 bytes per half-wave) hit distinct
//     banks.
//   - Tiles the mask hides completely are never loaded; 32-key blocks a wave cannot see are
//     skipped by that wave; the elementwise mask is applied only on blocks that straddle the
//     diagonal, the window edge or the end of the sequence.
//   - Global loads are buffer loads whose range is the head's [T][d] slab: rows past T read as
//     zero without a branch, and prefetches past the last tile are sent out of range, so every
//     load and LDS store is unconditional and no prefetch is waited on before it is consumed.
//   - The running maximum is raised lazily: only when a tile's maximum exceeds it by more than
//     kRescaleSlack (base-2 units) are the accumulators rescaled. Until then the weights
//     exp2(s - m) stay below 2^kRescaleSlack, which fp32 sums and bf16 weights hold exactly as
//     well as weights below 1.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace attn {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;             // queries per workgroup
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LPT = BN * CH / 256;  // 16-byte chunks per thread per K or V tile
  // Software-pipelined loop (two score accumulators live at once) fed by direct global -> LDS
  // loads for d <= 64; at d = 128 that does not fit the registers of two waves per SIMD, and the
  // matrix work per tile (twice that of d = 64 for the same softmax work) leaves the vector ALUs
  // less to hide anyway.
  static constexpr bool PIPE = D <= 64;
  // Pipelined: a ring of NSTAGE (K tile, V tile) stages filled PREFETCH tiles ahead.
  // Otherwise: K ring (2 tiles), then V ring (2 tiles), staged through registers.
  static constexpr int NSTAGE = 4;
  static constexpr int PREFETCH = NSTAGE - 1;
  static constexpr int LDS_BYTES = PIPE ? NSTAGE * 2 * TILE_BYTES : 4 * TILE_BYTES;
  static constexpr int DMA_PER_TILE = 2 * LPT;  // direct loads per thread per (K, V) tile pair
  static_assert(LPT >= 1, "tile too small for 256 threads");
};

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

typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

constexpr float kRescaleSlack = 8.0f;
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

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedDSRead = 0x100;
// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt and lgkmcnt left unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

template <int D, int MODE>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int T, int window_arg,
    float scale_log2, int nqt) {
  using C = FwdCfg<D>;
  constexpr bool causal = MODE != kNonCausal;
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int qt = nqt - 1 - (int)(blockIdx.x / BH);  // heaviest query block first
  const int bh = (int)(blockIdx.x % BH);
  const int64_t hoff = (int64_t)bh * T * D;
  const int q0 = qt * C::BM;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + l32;  // the query this lane owns in S^T and O^T

  const int slab = T * C::ROW_BYTES;  // bytes of one head's [T][d] slab (< 2^31, checked)
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q + hoff, slab);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + hoff, slab);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + hoff, slab);

  // Keys any query of the workgroup sees: [kv_lo, kv_hi). Keys some query of this wave sees:
  // [w_lo, w_hi); keys every query of the wave sees (no mask needed): [f_lo, f_hi).
  int kv_lo = 0, kv_hi = T, w_lo = 0, w_hi = T, f_lo = 0, f_hi = T;
  if constexpr (causal) {
    kv_hi = min(T, q0 + C::BM);
    w_hi = min(T, qw0 + 32);
    f_hi = min(T, qw0 + 1);
    if constexpr (MODE == kCausalWindow) {
      kv_lo = max(0, q0 - window);
      w_lo = max(0, qw0 - window);
      f_lo = qw0 + 31 - window;
    }
  }
  const int t_begin = kv_lo / C::BN;
  const int t_end = (kv_hi + C::BN - 1) / C::BN;
  auto active = [&](int t, int kb) {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 < w_hi) && (b0 + 32 > w_lo);
  };
  auto full = [&](int t, int kb) {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 >= f_lo) && (b0 + 32 <= f_hi);
  };
  auto fast = [&](int t) { return full(t, 0) && full(t, 1); };

  // Q^T fragments (B operand): lane holds Q[qi][16 s + 8 hi .. +8); rows past T read as zero.
  bf16x8 qf[C::KSTEPS];
  auto load_q = [&]() {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(qi * C::ROW_BYTES + 32 * s + 16 * hi)));
  };

  // ---- global -> register staging, LDS stores ---------------------------------------------
  auto gload = [&](__amdgpu_buffer_rsrc_t r, int t, bool needed, u32x4(&st)[C::LPT]) {
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const uint32_t off =
          needed ? (uint32_t)((t * C::BN + e / C::CH) * C::ROW_BYTES + 16 * (e % C::CH)) : kOutOfRange;
      st[u] = buffer_load16(r, off);
    }
  };
  auto lstore_k = [&](int slot, const u32x4(&st)[C::LPT]) {
    char* base = smem + slot * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH, c = e % C::CH;
      *reinterpret_cast<u32x4*>(base + r * C::ROW_BYTES + 16 * (c ^ swz_k<D>(r))) = st[u];
    }
  };
  auto lstore_v = [&](int slot, const u32x4(&st)[C::LPT]) {
    char* base = smem + (2 + slot) * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH, c = e % C::CH;
      *reinterpret_cast<u32x4*>(base + r * C::ROW_BYTES + 16 * (c ^ swz_v<D>(r))) = st[u];
    }
  };

  // Lane-constant parts of the LDS read addresses.
  // K (A operand of S^T): row 32 kb + l32, logical chunk 2 s + hi.
  const int k_row_off = l32 * C::ROW_BYTES;
  const int k_swz = swz_k<D>(l32);
  // V (A operand of O^T via the transposing read): lane (4a + b) of each 16-lane group addresses
  // row k0 + a, columns 32 db + 16 g1 + 4 b .. +4, where g1 = (lane / 16) % 2.
  const int v_a = (lane & 15) >> 2;
  const int v_b = lane & 3;
  const int v_g1 = (lane >> 4) & 1;
  const int v_swz = swz_v<D>(v_a);  // row = (multiple of 4) + v_a, so the swizzle is lane-constant

  // ---- stages of a tile ---------------------------------------------------------------------
  // Scores of tile t (K from ring slot `slot`) for the blocks this wave sees.
  auto scores = [&](int slot, int t, f32x16(&sa)[2], auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const char* kb_base = smem + slot * C::TILE_BYTES;
    const bool a0 = FAST || active(t, 0), a1 = FAST || active(t, 1);
    if (a0) sa[0] = f32x16{};
    if (a1) sa[1] = f32x16{};
    auto step = [&](int s, int kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_base + 32 * kb * C::ROW_BYTES +
                                                        k_row_off + 16 * ((2 * s + hi) ^ k_swz));
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sa[kb], 0, 0, 0);
    };
    if constexpr (C::PIPE) {
      // the two accumulation chains interleaved
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        if (a0) step(s, 0);
        if (a1) step(s, 1);
      }
    } else {
      // one block after the other keeps fewer K fragments in flight (register budget at d=128)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!(kb == 0 ? a0 : a1)) continue;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) step(s, kb);
      }
    }
  };

  // Mask the scores of tile t and return their row maximum (raw, pair-reduced).
  auto mask_max = [&](int t, f32x16(&sa)[2], auto fast_tag) -> float {
    constexpr bool FAST = decltype(fast_tag)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!FAST) {
        if (!active(t, kb)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sa[kb][r] = -INFINITY;
          continue;
        }
        if (!full(t, kb)) {
          // Register r holds key b0 + c_r with c_r = 8 (r / 4) + r % 4. With dq = qi - b0, the
          // key is visible iff 0 <= dq - c_r (causal) and dq - c_r <= window (one unsigned
          // compare covers both), and b0 + c_r < T where the block runs past the sequence end.
          const int b0 = t * C::BN + 32 * kb + 4 * hi;
          const int dq = qi - b0;
          const bool tail = t * C::BN + 32 * kb + 32 > T;  // wave-uniform
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 8 * (r >> 2) + (r & 3);
            bool vis = true;
            if constexpr (MODE == kCausal) vis = dq >= c;
            if constexpr (MODE == kCausalWindow) vis = (unsigned)(dq - c) <= (unsigned)window;
            if (tail) vis = vis & (b0 + c < T);
            sa[kb][r] = vis ? sa[kb][r] : -INFINITY;
          }
        }
      }
    }
    // Tree reduction over the 32 values of the lane, then across the lane pair.
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m8[i] = fmaxf(fmaxf(sa[i >> 2][4 * (i & 3)], sa[i >> 2][4 * (i & 3) + 1]),
                    fmaxf(sa[i >> 2][4 * (i & 3) + 2], sa[i >> 2][4 * (i & 3) + 3]));
    const float m2a = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
    const float m2b = fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7]));
    return pair_max(fmaxf(m2a, m2b));
  };

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;           // running maximum of the scaled scores, base-2 units
  float l_run0 = 0.f, l_run1 = 0.f;  // this lane's part of the running sum (two chains)

  // Lazy running-maximum update with a tile's row maximum (raw scores).
  auto decide = [&](float mx) {
    const float m_tile = mx * scale_log2;
    if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      m_run = m_new;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  };

  // P = exp2(s * scale - m), rounded to bf16 in the B-operand order of the P V product; the row
  // sums add the rounded values.
  auto exps = [&](const f32x16(&sa)[2], bf16x8(&pf)[2][2]) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sa[kb][8 * tt + 2 * e], scale_log2, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sa[kb][8 * tt + 2 * e + 1], scale_log2, -m_use));
          w[e] = pack_bf16x2(p0, p1);
          if (e & 1)
            l_run1 = add_bf16_pair(w[e], l_run1);
          else
            l_run0 = add_bf16_pair(w[e], l_run0);
        }
        pf[kb][tt] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  // O^T += V^T P^T for tile t (V from ring slot `slot`).
  auto pv = [&](int slot, int t, const bf16x8(&pf)[2][2], auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const char* vb = smem + (2 + slot) * C::TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!FAST) {
        if (!active(t, kb)) continue;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          u32x2 part[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int row = 32 * kb + 16 * tt + 8 * u + 4 * hi + v_a;
            const int c = 4 * db + 2 * v_g1 + (v_b >> 1);
            part[u] = ds_read_tr16_b64(vb + row * C::ROW_BYTES + 16 * (c ^ v_swz) + 8 * (v_b & 1));
          }
          const u32x4 a4{part[0][0], part[0][1], part[1][0], part[1][1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                              pf[kb][tt], oacc[db], 0, 0, 0);
        }
      }
    }
  };

  if constexpr (C::PIPE) {
    // Stage st holds a K tile then a V tile; tile t lives in stage (t - t0) % NSTAGE.
    const u32x4 rk_w = head_rsrc_words(K + hoff, slab);
    const u32x4 rv_w = head_rsrc_words(V + hoff, slab);
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
    // Issue the direct loads of tile t (out of range when not needed) into stage st. Wave w
    // fills 1 KiB runs (w * LPT + u) of each tile; lane L of a run writes chunk p = run * 64 + L,
    // i.e. row p / CH at physical chunk p % CH, so it loads the logical chunk that the row's
    // swizzle puts there.
    auto dma_tile = [&](int t, bool needed, int st) {
      const uint32_t kb_ = lds0 + st * 2 * C::TILE_BYTES;
      const uint32_t vb_ = kb_ + C::TILE_BYTES;
#pragma unroll
      for (int u = 0; u < C::LPT; ++u) {
        const int run = wave * C::LPT + u;
        const int p = run * 64 + lane;
        const int r = p / C::CH, pc = p % C::CH;
        const uint32_t row_off = (uint32_t)((t * C::BN + r) * C::ROW_BYTES);
        dma16(rk_w, kb_ + run * 1024, needed ? row_off + 16 * (pc ^ swz_k<D>(r)) : kOutOfRange);
        dma16(rv_w, vb_ + run * 1024, needed ? row_off + 16 * (pc ^ swz_v<D>(r)) : kOutOfRange);
      }
    };
    auto kslot = [&](int t) { return 2 * ((t - t_begin) % C::NSTAGE); };      // K ring slot
    auto vslot = [&](int t) { return 2 * ((t - t_begin) % C::NSTAGE) - 1; };  // V, as pv() adds 2

    // ---- prologue: tiles t0, t0+1 and the Q fragments, then tile t0+2 in flight -----------
    // The wait for Q is a compiler-visible s_waitcnt vmcnt(0) issued before tile t0+2: the
    // compiler then knows Q is in registers and puts no wait of its own inside the loop (such a
    // wait would also stall on the tiles in flight).
    dma_tile(t_begin, true, 0);
    dma_tile(t_begin + 1, t_begin + 1 < t_end, 1);
    load_q();
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
#pragma unroll
    for (int j = 2; j < C::PREFETCH; ++j) dma_tile(t_begin + j, t_begin + j < t_end, j);
    f32x16 sacc[2][2];  // masked scores of the current tile and (being computed) of the next
    {
      float mx;
      if (fast(t_begin)) {
        scores(kslot(t_begin), t_begin, sacc[0], std::true_type{});
        mx = mask_max(t_begin, sacc[0], std::true_type{});
      } else {
        scores(kslot(t_begin), t_begin, sacc[0], std::false_type{});
        mx = mask_max(t_begin, sacc[0], std::false_type{});
      }
      decide(mx);
    }

    // ---- main loop -----------------------------------------------------------------------
    // Iteration t: load tile t + PREFETCH into the stage tile t - 1 used (all reads of it ended
    // before the previous barrier); scores of t+1 alongside the exponentials of t; P(t) V(t)
    // alongside the mask and maximum of t+1; running-maximum update for t+1; wait until tile
    // t+2 has landed; barrier.
    auto body = [&](int t, f32x16(&cur)[2], f32x16(&nxt)[2]) {
      const bool has_next = t + 1 < t_end;
      dma_tile(t + C::PREFETCH, t + C::PREFETCH < t_end, (t - t_begin + C::PREFETCH) % C::NSTAGE);
      bf16x8 pf[2][2];
      float mx = -INFINITY;
      if (has_next && fast(t) && fast(t + 1)) {
        scores(kslot(t + 1), t + 1, nxt, std::true_type{});
        exps(cur, pf);
        pv(vslot(t), t, pf, std::true_type{});
        mx = mask_max(t + 1, nxt, std::true_type{});
        // Phase A: the K fragment reads of t+1 go out first, then the score MFMAs of t+1
        // alternate with the exponentials of t.
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2 * C::KSTEPS, 0);
#pragma unroll
        for (int j = 0; j < 2 * C::KSTEPS; ++j) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedVALU, 96 / (2 * C::KSTEPS), 0);
        }
        // Phase B: the P V MFMAs of t, each with its V reads issued two MFMAs ahead, alternate
        // with the mask and maximum of t+1.
        __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 4, 0);
#pragma unroll
        for (int j = 0; j < 4 * C::DB; ++j) {
          __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
          if (j + 2 < 4 * C::DB) __builtin_amdgcn_sched_group_barrier(kSchedDSRead, 2, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedVALU, 3, 0);
        }
      } else {
        if (has_next) scores(kslot(t + 1), t + 1, nxt, std::false_type{});
        if (active(t, 0) || active(t, 1)) {
          exps(cur, pf);
          pv(vslot(t), t, pf, std::false_type{});
        }
        if (has_next) mx = mask_max(t + 1, nxt, std::false_type{});
      }
      if (has_next) decide(mx);
      wait_vmcnt<(C::PREFETCH - 2) * C::DMA_PER_TILE>();  // tile t + 2 has landed
      __syncthreads();
    };
    int t = t_begin;
    for (; t + 1 < t_end; t += 2) {
      body(t, sacc[0], sacc[1]);
      body(t + 1, sacc[1], sacc[0]);
    }
    if (t < t_end) body(t, sacc[0], sacc[1]);
  } else {
    // ---- unpipelined: K and V one tile ahead; scores, softmax and P V of a tile in its own
    // iteration --------------------------------------------------------------------------------
    load_q();
    {
      u32x4 k0[C::LPT], v0[C::LPT];
      gload(rk, t_begin, true, k0);
      gload(rv, t_begin, true, v0);
      lstore_k(0, k0);
      lstore_v(0, v0);
    }
    __syncthreads();
    u32x4 kst[C::LPT], vst[C::LPT];
    for (int t = t_begin; t < t_end; ++t) {
      const int i = t - t_begin;
      gload(rk, t + 1, t + 1 < t_end, kst);
      gload(rv, t + 1, t + 1 < t_end, vst);
      if (active(t, 0) || active(t, 1)) {
        f32x16 sa[2];
        bf16x8 pf[2][2];
        scores(i & 1, t, sa, std::false_type{});
        decide(mask_max(t, sa, std::false_type{}));
        exps(sa, pf);
        pv(i & 1, t, pf, std::false_type{});
      }
      lstore_k((i + 1) & 1, kst);
      lstore_v((i + 1) & 1, vst);
      __syncthreads();
    }
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 ------------------------------------
  const float l_tot = pair_sum(l_run0 + l_run1);
  if (qi < T) {
    const float inv = 1.0f / l_tot;
    bf16* orow = O + hoff + (int64_t)qi * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g + 4 * hi) = w;
      }
    }
    if (hi == 0 && LSE != nullptr) LSE[(int64_t)bh * T + qi] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, int MODE>
static hipError_t launch_bf16_t(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int window, hipStream_t stream) {
  const int BH = B * H;
  const int nqt = (T + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const unsigned grid = (unsigned)((int64_t)BH * nqt);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, MODE>), dim3(grid), dim3(256), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)out, lse, BH, T, window,
                     scale_log2, nqt);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bf16_d(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int window, int causal, hipStream_t stream) {
  // A window of T - 1 or more hides nothing: run it as plain causal.
  if (!causal) return launch_bf16_t<D, kNonCausal>(q, k, v, out, lse, B, H, T, -1, stream);
  if (window < 0 || window >= T - 1) return launch_bf16_t<D, kCausal>(q, k, v, out, lse, B, H, T, -1, stream);
  return launch_bf16_t<D, kCausalWindow>(q, k, v, out, lse, B, H, T, window, stream);
}

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int d, int window, int causal,
                                hipStream_t stream) {
  if (d == 32) return launch_bf16_d<32>(q, k, v, out, lse, B, H, T, window, causal, stream);
  if (d == 64) return launch_bf16_d<64>(q, k, v, out, lse, B, H, T, window, causal, stream);
  if (d == 128) return launch_bf16_d<128>(q, k, v, out, lse, B, H, T, window, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
