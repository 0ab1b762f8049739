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
//   - Work items are (batch*head, block of BM = 128 queries). A workgroup of 4 waves owns one
//     item at a time; wave w owns queries [32w, 32w + 32) of the block.
//   - The grid is persistent: as many workgroups as the GPU holds at once, each walking its own
//     list of items. Items are ranked heaviest first (the last query blocks of a causal head see
//     the most keys) and dealt out in a snake order (rank k*P + g on even passes, k*P + P-1-g on
//     odd ones), which pairs heavy with light items per workgroup.
//   - Key/value tiles of BN = 64 rows flow HBM -> registers -> LDS through a 2-slot LDS ring,
//     one tile ahead, with one barrier per tile. The prefetch runs straight across item
//     boundaries: while the last tile of an item is consumed, the first tile of the workgroup's
//     next item is already in flight, so a workgroup never waits on a cold start after its first
//     item. The next item's Q block is fetched during the current item's first tile into the
//     other half of a double-buffered LDS Q area (d <= 64; at d = 128 the items are long and Q
//     is read straight from global memory at item start).
//   - S^T = K Q^T per 32-key block with v_mfma_f32_32x32x16_bf16: A = K from LDS (16 bytes per
//     lane), B = Q^T kept in registers for the whole workgroup. In the accumulator each lane owns
//     one query (lane % 32) and 16 keys, so row maxima and sums are lane-local plus one exchange
//     between lanes l and l + 32.
//   - O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T accumulator (rounded to
//     bf16), A = V^T read from the row-major V tile with ds_read_b64_tr_b16, which transposes
//     4x16 blocks of 16-bit values between lanes. The key order inside each 16-key MFMA step
//     follows the S^T accumulator's register order on both operands.
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
  static constexpr int BM = 128;             // queries per work item
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LPT = BN * CH / 256;  // 16-byte chunks per thread per K or V tile
  static constexpr bool QLDS = D <= 64;      // next item's Q staged through LDS
  static constexpr int Q_BYTES = BM * ROW_BYTES;
  static constexpr int QPT = BM * CH / 256;  // 16-byte chunks per thread per Q block
  // K ring (2 tiles), V ring (2 tiles), then the Q double buffer.
  static constexpr int KV_BYTES = 4 * TILE_BYTES;
  static constexpr int LDS_BYTES = KV_BYTES + (QLDS ? 2 * Q_BYTES : 0);
  static_assert(LPT >= 1 && QPT >= 1, "tile too small for 256 threads");
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
  const int P = (int)gridDim.x;
  const int g = (int)blockIdx.x;
  const int n_items = BH * nqt;
  const int slab = T * C::ROW_BYTES;  // bytes of one head's [T][d] slab (< 2^31, checked)

  // Item list of this workgroup: heaviest-first ranks dealt out in snake order.
  auto rank_of = [&](int k) { return k * P + ((k & 1) ? (P - 1 - g) : g); };
  auto decode = [&](int rank, int& bh, int& q0, int& tb, int& te) {
    const int qt = nqt - 1 - rank / BH;
    bh = rank % BH;
    q0 = qt * C::BM;
    int lo = 0, up = T;
    if constexpr (causal) {
      up = min(T, q0 + C::BM);
      if constexpr (MODE == kCausalWindow) lo = max(0, q0 - window);
    }
    tb = lo / C::BN;
    te = (up + C::BN - 1) / C::BN;
  };

  // Per-item, per-wave key ranges: keys some query of the wave sees are [w_lo, w_hi); keys every
  // query of the wave sees (no mask needed) are [f_lo, f_hi).
  int qw0 = 0, qi = 0, w_lo = 0, w_hi = T, f_lo = 0, f_hi = T;
  auto setup_wave = [&](int q0) {
    qw0 = q0 + 32 * wave;
    qi = qw0 + l32;  // the query this lane owns in S^T and O^T
    w_lo = 0;
    w_hi = T;
    f_lo = 0;
    f_hi = T;
    if constexpr (causal) {
      w_hi = min(T, qw0 + 32);
      f_hi = min(T, qw0 + 1);
      if constexpr (MODE == kCausalWindow) {
        w_lo = max(0, qw0 - window);
        f_lo = qw0 + 31 - window;
      }
    }
  };
  auto active = [&](int t, int kb) {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 < w_hi) && (b0 + 32 > w_lo);
  };
  auto full = [&](int t, int kb) {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 >= f_lo) && (b0 + 32 <= f_hi);
  };

  // ---- global -> register staging -------------------------------------------------------
  u32x4 kst[C::LPT], vst[C::LPT], qst[C::QPT];
  auto gload_kv = [&](int bh, int t, bool needed) {
    const int64_t hoff = (int64_t)bh * T * D;
    const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + hoff, slab);
    const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + hoff, slab);
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const uint32_t off =
          needed ? (uint32_t)((t * C::BN + e / C::CH) * C::ROW_BYTES + 16 * (e % C::CH)) : kOutOfRange;
      kst[u] = buffer_load16(rk, off);
      vst[u] = buffer_load16(rv, off);
    }
  };
  auto gload_q = [&](int bh, int q0) {
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q + (int64_t)bh * T * D, slab);
#pragma unroll
    for (int u = 0; u < C::QPT; ++u) {
      const int e = tid + 256 * u;
      qst[u] = buffer_load16(rq, (uint32_t)((q0 + e / C::CH) * C::ROW_BYTES + 16 * (e % C::CH)));
    }
  };
  // ---- LDS stores (16-byte chunks, XOR-swizzled rows) ------------------------------------
  auto lstore_kv = [&](int slot) {
    char* kb_ = smem + slot * C::TILE_BYTES;
    char* vb_ = smem + (2 + slot) * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH, c = e % C::CH;
      *reinterpret_cast<u32x4*>(kb_ + r * C::ROW_BYTES + 16 * (c ^ swz_k<D>(r))) = kst[u];
      *reinterpret_cast<u32x4*>(vb_ + r * C::ROW_BYTES + 16 * (c ^ swz_v<D>(r))) = vst[u];
    }
  };
  auto lstore_q = [&](int buf) {
    char* qb = smem + C::KV_BYTES + buf * C::Q_BYTES;
#pragma unroll
    for (int u = 0; u < C::QPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH, c = e % C::CH;
      *reinterpret_cast<u32x4*>(qb + r * C::ROW_BYTES + 16 * (c ^ swz_k<D>(r))) = qst[u];
    }
  };

  // Lane-constant parts of the LDS read addresses.
  // K (A operand of S^T): row 32 kb + l32, logical chunk 2 s + hi. The Q block uses the same
  // layout, wave w reading rows 32 w + l32 (the swizzle of those rows equals that of l32).
  const int k_row_off = l32 * C::ROW_BYTES;
  const int k_swz = swz_k<D>(l32);
  // V (A operand of O^T via the transposing read): lane (4a + b) of each 16-lane group addresses
  // row k0 + a, columns 32 db + 16 g1 + 4 b .. +4, where g1 = (lane / 16) % 2.
  const int v_a = (lane & 15) >> 2;
  const int v_b = lane & 3;
  const int v_g1 = (lane >> 4) & 1;
  const int v_swz = swz_v<D>(v_a);  // row = (multiple of 4) + v_a, so the swizzle is lane-constant

  // Q^T fragments (B operand of S^T): lane holds Q[qi][16 s + 8 hi .. +8).
  bf16x8 qf[C::KSTEPS];
  auto q_from_global = [&](int bh) {
    const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q + (int64_t)bh * T * D, slab);
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(qi * C::ROW_BYTES + 32 * s + 16 * hi)));
  };
  auto q_from_lds = [&](int buf) {
    const char* qb = smem + C::KV_BYTES + buf * C::Q_BYTES + 32 * wave * C::ROW_BYTES + k_row_off;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      qf[s] = *reinterpret_cast<const bf16x8*>(qb + 16 * ((2 * s + hi) ^ k_swz));
  };

  // ---- per-item accumulators --------------------------------------------------------------
  f32x16 oacc[C::DB];
  float m_run, l_run0, l_run1;  // running max (base-2 units) and this lane's two partial sums
  auto reset = [&]() {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
    m_run = -INFINITY;
    l_run0 = 0.f;
    l_run1 = 0.f;
  };

  // ---- one tile: S^T = K Q^T, mask, softmax, O^T += V^T P^T -------------------------------
  // FAST: both 32-key blocks visible to every query of the wave. The tile is then one
  // straight-line block with the two score chains interleaved, which lets the compiler hide LDS
  // and MFMA latencies behind each other. Otherwise each block is skipped or masked as needed.
  auto compute_tile = [&](int slot, int t, auto fast_tag) {
    constexpr bool FAST = decltype(fast_tag)::value;
    const bool a0 = FAST || active(t, 0), a1 = FAST || active(t, 1);
    const char* kbuf = smem + slot * C::TILE_BYTES;
    const char* vbuf = smem + (2 + slot) * C::TILE_BYTES;
    f32x16 sa[2];
    if constexpr (FAST) {
      sa[0] = f32x16{};
      sa[1] = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf + 32 * kb * C::ROW_BYTES +
                                                            k_row_off + 16 * ((2 * s + hi) ^ k_swz));
          sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sa[kb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!(kb == 0 ? a0 : a1)) continue;
        bf16x8 a[C::KSTEPS];
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s)
          a[s] = *reinterpret_cast<const bf16x8*>(kbuf + 32 * kb * C::ROW_BYTES + k_row_off +
                                                  16 * ((2 * s + hi) ^ k_swz));
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], qf[s], acc, 0, 0, 0);
        sa[kb] = acc;
      }
    }

    // Mask, then the tile's row maximum (raw scores; the scale is positive).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!FAST) {
        if (!(kb == 0 ? a0 : a1)) {
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
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sa[kb][r], sa[kb][r + 1]));
    }
    mx = pair_max(mx);
    const float m_tile = mx * scale_log2;
    // Raise the running maximum only when the tile exceeds it by more than the slack (always
    // on a row's first visible tile, since m_run starts at -inf).
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
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

    // P = exp2(s * scale - m), rounded to bf16 in the B-operand order of the P V product; the
    // row sums add the rounded values.
    bf16x8 pf[2][2];
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

    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (!FAST) {
        if (!(kb == 0 ? a0 : a1)) continue;
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
            part[u] = ds_read_tr16_b64(vbuf + row * C::ROW_BYTES + 16 * (c ^ v_swz) + 8 * (v_b & 1));
          }
          const u32x4 a4{part[0][0], part[0][1], part[1][0], part[1][1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                              pf[kb][tt], oacc[db], 0, 0, 0);
        }
      }
    }
  };
  auto tile = [&](int slot, int t) {
    // At d = 128 the straight-line form needs more registers than two waves per SIMD have.
    if (D <= 64 && full(t, 0) && full(t, 1))
      compute_tile(slot, t, std::true_type{});
    else if (active(t, 0) || active(t, 1))
      compute_tile(slot, t, std::false_type{});
  };

  // ---- epilogue of an item: O = O^T / l, LSE = (m + log2 l) ln 2 -------------------------
  auto epilogue = [&](int bh) {
    const float l_tot = pair_sum(l_run0 + l_run1);
    if (qi < T) {
      const float inv = 1.0f / l_tot;
      bf16* orow = O + (int64_t)bh * T * D + (int64_t)qi * D;
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          u32x2 w;
          w[0] = pack_bf16x2(oacc[db][4 * gg] * inv, oacc[db][4 * gg + 1] * inv);
          w[1] = pack_bf16x2(oacc[db][4 * gg + 2] * inv, oacc[db][4 * gg + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * gg + 4 * hi) = w;
        }
      }
      if (hi == 0 && LSE != nullptr) LSE[(int64_t)bh * T + qi] = (m_run + __log2f(l_tot)) * kLn2;
    }
  };

  // ---- the item stream ---------------------------------------------------------------------
  int k = 0;
  int bh, q0, tb, te;
  decode(rank_of(0), bh, q0, tb, te);  // g < P <= n_items
  setup_wave(q0);
  q_from_global(bh);
  gload_kv(bh, tb, true);
  lstore_kv(0);
  reset();
  __syncthreads();

  // The workgroup's next item, if any.
  int rank_n = rank_of(1);
  bool more = rank_n < n_items;
  int nbh = 0, nq0 = 0, ntb = 0, nte = 0;
  if (more) decode(rank_n, nbh, nq0, ntb, nte);

  int t = tb, slot = 0;
  while (true) {
    const bool last = (t + 1 == te);
    // Prefetch the next tile of the stream (it may belong to the next item).
    if (!last)
      gload_kv(bh, t + 1, true);
    else
      gload_kv(nbh, ntb, more);
    // During an item's first tile, fetch the next item's Q block.
    const bool qpref = C::QLDS && more && (t == tb);
    if (qpref) gload_q(nbh, nq0);

    tile(slot, t);
    if (last) epilogue(bh);

    lstore_kv(slot ^ 1);
    if (qpref) lstore_q((k + 1) & 1);
    __syncthreads();

    if (last) {
      if (!more) break;
      ++k;
      bh = nbh;
      q0 = nq0;
      tb = ntb;
      te = nte;
      t = tb;
      setup_wave(q0);
      if constexpr (C::QLDS)
        q_from_lds(k & 1);
      else
        q_from_global(bh);
      reset();
      rank_n = rank_of(k + 1);
      more = rank_n < n_items;
      if (more) decode(rank_n, nbh, nq0, ntb, nte);
    } else {
      ++t;
    }
    slot ^= 1;
  }
}

template <int D, int MODE>
static hipError_t launch_bf16_t(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int window, hipStream_t stream) {
  // Workgroups the GPU holds at once, queried once per instantiation (a cache of a device
  // property).
  static int resident = 0;
  if (resident == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_fwd_bf16_kernel<D, MODE>, 256, 0);
    if (e != hipSuccess) return e;
    resident = cus * (per_cu > 0 ? per_cu : 1);
  }
  const int BH = B * H;
  const int nqt = (T + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const int64_t n_items = (int64_t)BH * nqt;
  const unsigned grid = (unsigned)(n_items < resident ? n_items : resident);
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
