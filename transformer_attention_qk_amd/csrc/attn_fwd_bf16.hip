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
// Work split: items are (batch*head, block of BM = 128 queries); a workgroup of 4 waves owns one
// item at a time, wave w owning queries [32w, 32w + 32) of the block. Per wave:
//   - S^T = K Q^T per 32-key block with v_mfma_f32_32x32x16_bf16: A = K from LDS (16 bytes per
//     lane), B = Q^T kept in registers for the whole item. In the accumulator each lane owns one
//     query (lane % 32) and 16 keys, so row maxima and sums are lane-local plus one exchange
//     between lanes l and l + 32.
//   - O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T accumulator (rounded to
//     bf16), A = V^T read from the row-major V tile with ds_read_b64_tr_b16, which transposes
//     4x16 blocks of 16-bit values between lanes. The key order inside each 16-key MFMA step
//     follows the S^T accumulator's register order on both operands.
//   - Row sums of the weights are taken with v_dot2_f32_bf16 on the bf16-rounded weights, i.e.
//     on exactly the values the P V product uses.
//   - The running maximum is raised lazily: only when a tile's maximum exceeds it by more than
//     kRescaleSlack (base-2 units) are the accumulators rescaled. Until then the weights
//     exp2(s - m) stay below 2^kRescaleSlack, which fp32 sums and bf16 weights hold exactly as
//     well as weights below 1.
//   - 32-key blocks a wave cannot see are skipped; the elementwise mask (a compile-time mode) is
//     applied only on blocks that straddle the diagonal, the window edge or the sequence end.
// LDS rows are XOR-swizzled in 16-byte chunks so that the K reads (16 rows x 16 bytes per
// quarter-wave) and the transposing V reads (4 rows x 64 bytes per half-wave) hit distinct banks.
//
// Two kernels:
//   - attn_fwd_bf16_stream (d <= 64): a persistent grid. Each workgroup walks a list of items
//     ranked heaviest first (the last query blocks of a causal head see the most keys) and dealt
//     out in snake order, and streams the K/V tiles of all its items through a 4-stage LDS ring
//     with direct global -> LDS loads (buffer_load ... lds) three tiles ahead, across item
//     boundaries. The next item's Q block arrives by the same route during the current item's
//     last tile. Inside an item each wave runs a software pipeline: the scores of tile t+1 go to
//     the matrix cores while the vector ALUs exponentiate tile t, then P(t) V(t) while the
//     vector ALUs mask and reduce the scores of tile t+1.
//   - attn_fwd_bf16_tile (d = 128): one workgroup per item, K/V staged through registers one
//     tile ahead. The pipelined form needs more registers than two waves per SIMD have at
//     d = 128, where the matrix work per tile doubles while the softmax work stays the same.
// Global loads are buffer loads whose range is the head's [T][d] slab: rows past T read as zero
// without a branch, and loads of tiles that do not exist are sent out of range, so every load is
// unconditional.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "common.hpp"
#include "launch.hpp"
#include "tile_ops.hpp"

namespace attn {

template <int D>
struct FwdCfg {
  static constexpr int BM = 128;             // queries per item
  static constexpr int BN = 64;              // keys per tile
  static constexpr int KSTEPS = D / 16;      // MFMA k-steps of S^T = K Q^T
  static constexpr int DB = D / 32;          // 32-row blocks of O^T
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int LPT = BN * CH / 256;  // 16-byte chunks per thread per K or V tile
  static_assert(LPT >= 1, "tile too small for 256 threads");
  // Streaming kernel: ring of NSTAGE (K tile, V tile) stages filled PREFETCH tiles ahead, then
  // one Q block.
  static constexpr int NSTAGE = 4;
  static constexpr int PREFETCH = NSTAGE - 1;
  static constexpr int Q_BYTES = BM * ROW_BYTES;
  static constexpr int STREAM_LDS = NSTAGE * 2 * TILE_BYTES + Q_BYTES;
  static constexpr int DMA_PER_TILE = 2 * LPT;             // direct loads per thread per stage
  static constexpr int DMA_PER_Q = Q_BYTES / (1024 * 4);   // direct loads per thread per Q block
  // Rotation factors staged for an item transition of the QKN streaming kernel: table rows
  // (cos, then sin, d/2 floats each) of the 8 bases q0 + 16 m and of the 16 offsets e < 16,
  // each table's part padded to whole 1 KiB runs; they fit in the K half of a ring stage.
  static constexpr int ROPE_ROWS = 8 + 16;
  static constexpr int ROPE_PART = (ROPE_ROWS * D * 2 + 1023) / 1024 * 1024;  // bytes per table
  static constexpr int ROPE_RUNS = 2 * ROPE_PART / 1024;
  static_assert(2 * ROPE_PART <= TILE_BYTES, "staged rotation factors must fit in a K tile");
  // Tile kernel: K ring (2 tiles), then V ring (2 tiles).
  static constexpr int TILE_LDS = 4 * TILE_BYTES;
};

// Headroom of the lazy running maximum (base-2 units).
constexpr float kRescaleSlack = 8.0f;

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0) with expcnt and lgkmcnt left unconstrained.
constexpr int kWaitVmcnt0 = 0x0F70;

// Per-wave state and stages of one item (block of 128 queries of one head).
//
// QKN = true: the Q rows arrive raw and are RMS-normalised, rotated and scaled by log2(e)/sqrt(d)
// here (fp32, one rounding to bf16), and K rows arrive normalised and rotated. Each such row has
// Euclidean norm at most sqrt(d), so a score q.k/sqrt(d) lies in [-sqrt(d), sqrt(d)] and
// exp2 of a score in base-2 units lies in [2^-(sqrt(d) log2 e), 2^(sqrt(d) log2 e)]
// (2^-16.4 .. 2^16.4 at d = 128): the softmax needs no running maximum, no rescaling and no
// subtraction, and its weights and sums stay far inside the bf16 and fp32 ranges. The row sum of
// T such weights stays finite for any T below 2^100.
template <int D, int MODE, bool QKN>
struct WaveTile {
  using C = FwdCfg<D>;
  static constexpr bool causal = MODE != kNonCausal;
  int T, window, lane, l32, hi, wave;
  int q_rs;  // bytes between consecutive q (and out) rows
  float scale_log2;
  // lane-constant LDS addressing. K (A operand of S^T): row 32 kb + l32, logical chunk
  // 2 s + hi. V (A operand of O^T via the transposing read): lane (4a + b) of each 16-lane group
  // addresses row k0 + a, columns 32 db + 16 g1 + 4 b .. +4, g1 = (lane / 16) % 2.
  int k_row_off, k_swz, v_a, v_b, v_g1, v_swz;
  // item: this wave's queries, the keys some of them see [w_lo, w_hi), the keys all of them see
  // [f_lo, f_hi)
  int qw0, qi, w_lo, w_hi, f_lo, f_hi;
  bf16x8 qf[C::KSTEPS];  // Q^T fragments (B operand): Q[qi][16 s + 8 hi .. +8)
  f32x16 oacc[C::DB];
  float m_run, l_run0, l_run1;  // running max (base-2 units) and this lane's two partial sums

  __device__ __forceinline__ void init(int T_, int window_, float scale_log2_, int tid, int q_rs_) {
    T = T_;
    q_rs = q_rs_;
    window = window_;
    scale_log2 = scale_log2_;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    lane = tid & 63;
    l32 = lane & 31;
    hi = lane >> 5;
    k_row_off = l32 * C::ROW_BYTES;
    k_swz = swz_k<D>(l32);
    v_a = (lane & 15) >> 2;
    v_b = lane & 3;
    v_g1 = (lane >> 4) & 1;
    v_swz = swz_v<D>(v_a);  // row = (multiple of 4) + v_a, so the swizzle is lane-constant
  }
  __device__ __forceinline__ void set_item(int q0) {
    qw0 = q0 + 32 * wave;
    qi = qw0 + l32;
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
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
    m_run = QKN ? 0.f : -INFINITY;
    l_run0 = 0.f;
    l_run1 = 0.f;
  }
  __device__ __forceinline__ bool active(int t, int kb) const {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 < w_hi) && (b0 + 32 > w_lo);
  }
  __device__ __forceinline__ bool full(int t, int kb) const {
    const int b0 = t * C::BN + 32 * kb;
    return (b0 >= f_lo) && (b0 + 32 <= f_hi);
  }
  // (bitwise operators: the operands are cheap scalar tests, evaluated without branches)
  __device__ __forceinline__ bool fast(int t) const { return (int)full(t, 0) & (int)full(t, 1); }
  __device__ __forceinline__ bool any(int t) const { return (int)active(t, 0) | (int)active(t, 1); }
  // Both blocks of tile t computed for this wave (some keys may still be masked).
  __device__ __forceinline__ bool act2(int t) const { return active(t, 0) & active(t, 1); }

  // Rotation factors of the lane's Q row at the frequencies it holds (QKN only): cos and sin at
  // columns 16 s + 8 hi .. +8 for s < KSTEPS/2, as 16-byte loads.
  struct Rope {
    f32x4 c[C::KSTEPS / 2][2], s[C::KSTEPS / 2][2];
  };
  // The lane index, recomputed where it is used (the item transitions) instead of keeping the
  // values derived from it live through the tile loop.
  __device__ __forceinline__ int lane_now() const {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  }
  __device__ __forceinline__ int q_row(int q0) const { return q0 + 32 * wave + (lane_now() & 31); }
  __device__ __forceinline__ void load_rope(int q0, const float* cos_tab, const float* sin_tab,
                                            Rope& r) const {
    if constexpr (QKN) {
      // Buffer loads with one 32-bit offset register: the tables' T * d/2 floats are far below
      // 2^31 bytes (T * d < 2^30 is checked before launch).
      constexpr int HALF = D / 2;
      const int tab_bytes = T * HALF * 4;
      const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(cos_tab), (short)0, tab_bytes, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(sin_tab), (short)0, tab_bytes, kBufferWord3);
      const uint32_t off = (uint32_t)(min(q_row(q0), T - 1) * HALF + 8 * (lane_now() >> 5)) * 4;
#pragma unroll
      for (int s = 0; s < C::KSTEPS / 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          r.c[s][h] = __builtin_bit_cast(f32x4, buffer_load16(rc, off + 64 * s + 16 * h));
          r.s[s][h] = __builtin_bit_cast(f32x4, buffer_load16(rs, off + 64 * s + 16 * h));
        }
    }
  }
  // The same factors from the rows staged in LDS at rope_lds (layout above): the row's position
  // q0 + 32 wave + l splits into the base q0 + 16 m, m = 2 wave + l / 16, and the offset
  // e = l % 16, and the angle-addition formulas
  //   cos((b + e) w) = cos(b w) cos(e w) - sin(b w) sin(e w)
  //   sin((b + e) w) = sin(b w) cos(e w) + cos(b w) sin(e w)
  // give the factors in fp32 from the two table rows.
  __device__ __forceinline__ void rope_from_lds(const char* rope_lds, Rope& r) const {
    if constexpr (QKN) {
      constexpr int RB = D * 2;  // bytes of one staged row (d/2 floats)
      const int ln = lane_now();
      const int l = ln & 31, col = 32 * (ln >> 5);  // byte offset of column 8 hi
      // Rows are stored with their 16-byte chunks rotated by swz_rope (see the staging loads).
      const int rb = 2 * wave + (l >> 4), rl = 8 + (l & 15);
      const char* cb = rope_lds + rb * RB;
      const char* cl = rope_lds + rl * RB;
      const int sb = swz_rope<D>(rb), sl = swz_rope<D>(rl), c0 = col / 16;
#pragma unroll
      for (int s = 0; s < C::KSTEPS / 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = c0 + 4 * s + h;  // logical chunk of columns 16 s + 8 hi + 4 h .. +4
          const int ob = 16 * (c ^ sb), ol = 16 * (c ^ sl);
          const f32x4 c_b = *reinterpret_cast<const f32x4*>(cb + ob);
          const f32x4 s_b = *reinterpret_cast<const f32x4*>(cb + C::ROPE_PART + ob);
          const f32x4 c_l = *reinterpret_cast<const f32x4*>(cl + ol);
          const f32x4 s_l = *reinterpret_cast<const f32x4*>(cl + C::ROPE_PART + ol);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            r.c[s][h][e] = fmaf(c_b[e], c_l[e], -(s_b[e] * s_l[e]));
            r.s[s][h][e] = fmaf(s_b[e], c_l[e], c_b[e] * s_l[e]);
          }
        }
    }
  }
  // This lane's raw Q values xf[s] = Q[row][16 s + 8 hi .. +8) of the item at q0, from global
  // memory (rows past T read as zero) or from the Q block staged in LDS with the K layout (wave
  // w reads rows 32 w + l32, whose swizzle equals that of l32).
  __device__ __forceinline__ void load_q_global(__amdgpu_buffer_rsrc_t rq, int q0,
                                                bf16x8 (&xf)[C::KSTEPS]) const {
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      xf[s] = __builtin_bit_cast(
          bf16x8, buffer_load16(rq, (uint32_t)(q_row(q0) * q_rs + 32 * s + 16 * hi)));
  }
  __device__ __forceinline__ void load_q_lds(const char* qbuf, bf16x8 (&xf)[C::KSTEPS]) const {
    const int ln = lane_now();
    const int r = ln & 31, h = ln >> 5, sw = swz_k<D>(r);
    const char* qb = qbuf + (32 * wave + r) * C::ROW_BYTES;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
      xf[s] = *reinterpret_cast<const bf16x8*>(qb + 16 * ((2 * s + h) ^ sw));
  }
  // qf (the Q^T fragments, B operand of the scores) of the item at q0 from the raw values. With
  // QKN the row is normalised (weightless RMSNorm over the head dim; the other half of the row
  // sits in lane l ^ 32), rotated by the half-split rotation at its position (column j < d/2
  // pairs with column j + d/2, which is in xf[s + KSTEPS/2] of the same lane) and scaled by
  // log2(e)/sqrt(d), in fp32; rows past T become zero.
  __device__ __forceinline__ void set_q(const bf16x8 (&xf)[C::KSTEPS], const Rope& rope, int q0,
                                        float eps) {
    if constexpr (!QKN) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) qf[s] = xf[s];
    } else {
      float x[C::KSTEPS][8];
      float ss = 0.f;
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        const u32x4 w = __builtin_bit_cast(u32x4, xf[s]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[s][2 * e] = bf16lo_to_f32(w[e]);
          x[s][2 * e + 1] = bf16hi_to_f32(w[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[s][e], x[s][e], ss);
      }
      ss = pair_sum(ss);
      // v_rsq_f32 (about 1 ulp) is ample here: the row is rounded to bf16 right after.
      const float rinv = (q_row(q0) < T)
                             ? (kLog2e * (1.0f / sqrtf((float)D))) *
                                   __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps)
                             : 0.f;
#pragma unroll
      for (int s = 0; s < C::KSTEPS / 2; ++s) {
        u32x4 w1, w2;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          float y1[2], y2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float c = rope.c[s][(e + u) >> 2][(e + u) & 3];
            const float sn = rope.s[s][(e + u) >> 2][(e + u) & 3];
            const float a = x[s][e + u] * rinv;
            const float b = x[s + C::KSTEPS / 2][e + u] * rinv;
            y1[u] = fmaf(a, c, b * sn);
            y2[u] = fmaf(b, c, -(a * sn));
          }
          w1[e / 2] = pack_bf16x2(y1[0], y1[1]);
          w2[e / 2] = pack_bf16x2(y2[0], y2[1]);
        }
        qf[s] = __builtin_bit_cast(bf16x8, w1);
        qf[s + C::KSTEPS / 2] = __builtin_bit_cast(bf16x8, w2);
      }
    }
  }

  // Scores of tile t (K tile at kbuf) for the blocks this wave sees. INTERLEAVE runs the two
  // accumulation chains side by side (more independent work, more K fragments in flight).
  template <bool FAST, bool INTERLEAVE>
  __device__ __forceinline__ void scores(const char* kbuf, int t, f32x16 (&sa)[2]) {
    const bool a0 = FAST || active(t, 0), a1 = FAST || active(t, 1);
    // Both accumulators are defined on every path, so no earlier value stays live through here.
    sa[0] = f32x16{};
    sa[1] = f32x16{};
    auto step = [&](int s, int kb) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kbuf + 32 * kb * C::ROW_BYTES + k_row_off +
                                                        16 * ((2 * s + hi) ^ k_swz));
      sa[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sa[kb], 0, 0, 0);
    };
    if constexpr (INTERLEAVE) {
#pragma unroll
      for (int s = 0; s < C::KSTEPS; ++s) {
        if (a0) step(s, 0);
        if (a1) step(s, 1);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!(kb == 0 ? a0 : a1)) continue;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) step(s, kb);
      }
    }
  }

  // Mask the scores of tile t and return their row maximum (raw, pair-reduced; with QKN only the
  // mask is applied and 0 is returned).
  template <bool FAST>
  __device__ __forceinline__ float mask_max(int t, f32x16 (&sa)[2]) {
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
          // key is visible iff c_r <= dq (causal), c_r >= dq - window (window) and
          // c_r <= T - 1 - b0 (sequence end): one upper and one lower limit per lane. The block
          // needs the upper test only if it reaches past the wave's first query or the sequence
          // end, and the lower one only if it starts before the wave's last query's window; a
          // window of 32 or more keys never needs both in one block, so each register takes one
          // compare there.
          const int bb = t * C::BN + 32 * kb;  // the block's first key (wave-uniform)
          const bool need_hi = (causal && bb + 31 > qw0) || (bb + 32 > T);
          const bool need_lo = (MODE == kCausalWindow) && (bb < qw0 + 31 - window);
          const int b0 = bb + 4 * hi;
          const int dq = qi - b0;
          int hi_c = causal ? dq : 0x7fffffff;
          if (bb + 32 > T) hi_c = min(hi_c, T - 1 - b0);
          int lo_c = dq - window;
          // Opaque to the optimiser: otherwise it hoists the 16-32 per-register lane masks of a
          // loop-invariant edge out of the loops and spills them.
          asm volatile("" : "+v"(hi_c), "+v"(lo_c));
          if (need_hi && need_lo) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 8 * (r >> 2) + (r & 3);
              sa[kb][r] = ((c <= hi_c) & (c >= lo_c)) ? sa[kb][r] : -INFINITY;
            }
          } else if (need_hi) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 8 * (r >> 2) + (r & 3);
              sa[kb][r] = (c <= hi_c) ? sa[kb][r] : -INFINITY;
            }
          } else {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int c = 8 * (r >> 2) + (r & 3);
              sa[kb][r] = (c >= lo_c) ? sa[kb][r] : -INFINITY;
            }
          }
        }
      }
    }
    if constexpr (QKN) return 0.f;
    // Tree reduction over the 32 values of the lane, then across the lane pair.
    float m8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      m8[i] = fmaxf(fmaxf(sa[i >> 2][4 * (i & 3)], sa[i >> 2][4 * (i & 3) + 1]),
                    fmaxf(sa[i >> 2][4 * (i & 3) + 2], sa[i >> 2][4 * (i & 3) + 3]));
    const float m2a = fmaxf(fmaxf(m8[0], m8[1]), fmaxf(m8[2], m8[3]));
    const float m2b = fmaxf(fmaxf(m8[4], m8[5]), fmaxf(m8[6], m8[7]));
    return pair_max(fmaxf(m2a, m2b));
  }

  // Lazy running-maximum update with a tile's row maximum (raw scores); nothing with QKN. Only
  // the rows whose maximum grew by more than the slack move it (the others keep m_run, so their
  // factor is exactly 1): a row's arithmetic depends on its own scores alone, never on whether
  // another row of the wave triggered a rescale.
  __device__ __forceinline__ void decide(float mx) {
    if constexpr (QKN) return;
    const float m_tile = mx * scale_log2;
    const bool need = m_tile > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? m_tile : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
      m_run = m_new;
      l_run0 *= alpha;
      l_run1 *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
  }

  // P = exp2(s * scale - m) (with QKN: exp2(s), the scores being in base-2 units already),
  // rounded to bf16 in the B-operand order of the P V product; the row sums add the rounded
  // values.
  __device__ __forceinline__ void exps(const f32x16 (&sa)[2], bf16x8 (&pf)[2][2]) {
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p0, p1;
          if constexpr (QKN) {
            p0 = __builtin_amdgcn_exp2f(sa[kb][8 * tt + 2 * e]);
            p1 = __builtin_amdgcn_exp2f(sa[kb][8 * tt + 2 * e + 1]);
          } else {
            p0 = __builtin_amdgcn_exp2f(fmaf(sa[kb][8 * tt + 2 * e], scale_log2, -m_use));
            p1 = __builtin_amdgcn_exp2f(fmaf(sa[kb][8 * tt + 2 * e + 1], scale_log2, -m_use));
          }
          w[e] = pack_bf16x2(p0, p1);
          if (e & 1)
            l_run1 = add_bf16_pair(w[e], l_run1);
          else
            l_run0 = add_bf16_pair(w[e], l_run0);
        }
        pf[kb][tt] = __builtin_bit_cast(bf16x8, w);
      }
    }
  }

  // O^T += V^T P^T for tile t (V tile at vbuf).
  template <bool FAST>
  __device__ __forceinline__ void pv(const char* vbuf, int t, const bf16x8 (&pf)[2][2]) {
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
            part[u] = ds_read_tr16_b64(vbuf + row * C::ROW_BYTES + 16 * (c ^ v_swz) + 8 * (v_b & 1));
          }
          const u32x4 a4{part[0][0], part[0][1], part[1][0], part[1][1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                              pf[kb][tt], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // One pipelined step with a next tile: the scores of both 32-key blocks of tile t+1 (K tile at
  // kbuf) go to the matrix cores while the vector ALUs exponentiate tile t's scores (cur), then
  // P(t) V(t) (V tile at vbuf). The compiler places each LDS read near its product and
  // interleaves the exponentials with the products.
  __device__ __forceinline__ void step_pipelined(const char* kbuf, const char* vbuf,
                                                 const f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    bf16x8 kf[2][C::KSTEPS];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[kb][s] = *reinterpret_cast<const bf16x8*>(kbuf + 32 * kb * C::ROW_BYTES + k_row_off +
                                                     16 * ((2 * s + hi) ^ k_swz));
    u32x2 vp[2][2][C::DB][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int row = 32 * kb + 16 * tt + 8 * u + 4 * hi + v_a;
            const int c = 4 * db + 2 * v_g1 + (v_b >> 1);
            vp[kb][tt][db][u] =
                ds_read_tr16_b64(vbuf + row * C::ROW_BYTES + 16 * (c ^ v_swz) + 8 * (v_b & 1));
          }
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        nxt[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kb][s], qf[s],
                                                          s == 0 ? f32x16{} : nxt[kb], 0, 0, 0);
    bf16x8 pf[2][2];
    exps(cur, pf);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const u32x4 a4{vp[kb][tt][db][0][0], vp[kb][tt][db][0][1], vp[kb][tt][db][1][0],
                         vp[kb][tt][db][1][1]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a4),
                                                              pf[kb][tt], oacc[db], 0, 0, 0);
        }
  }

  // Unpipelined tile: scores, mask and maximum, update, exponentials, P V.
  __device__ __forceinline__ void whole_tile(const char* kbuf, const char* vbuf, int t) {
    f32x16 sa[2];
    bf16x8 pf[2][2];
    scores<false, false>(kbuf, t, sa);
    decide(mask_max<false>(t, sa));
    exps(sa, pf);
    pv<false>(vbuf, t, pf);
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 for this wave's queries of head offset hoff.
  // Lane l and l + 32 hold the two 8-byte halves of each 16-byte chunk (columns 32 db + 8 g ..
  // +8) of row qi; one v_permlane32_swap per word gathers chunk 2m into lane l and chunk 2m + 1
  // into lane l + 32, so each store writes 16 bytes per lane, 32 contiguous bytes per row.
  __device__ __forceinline__ void store(bf16* O, float* LSE, int64_t hoff, int64_t lse_off) {
    const float l_tot = pair_sum(l_run0 + l_run1);
    const float inv = 1.0f / l_tot;
    u32x4 ch[C::DB][2];
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        uint32_t x[2], y[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int g0 = 2 * m, g1 = 2 * m + 1;
          x[k] = pack_bf16x2(oacc[db][4 * g0 + 2 * k] * inv, oacc[db][4 * g0 + 2 * k + 1] * inv);
          y[k] = pack_bf16x2(oacc[db][4 * g1 + 2 * k] * inv, oacc[db][4 * g1 + 2 * k + 1] * inv);
          // lanes < 32 get (own x, partner's x), lanes >= 32 (partner's y, own y)
          const auto sw = __builtin_amdgcn_permlane32_swap(x[k], y[k], false, false);
          x[k] = sw[0];
          y[k] = sw[1];
        }
        ch[db][m] = u32x4{x[0], x[1], y[0], y[1]};
      }
    }
    if (qi < T) {
      bf16* orow = O + hoff + (int64_t)qi * (q_rs / 2);
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int m = 0; m < 2; ++m)
          *reinterpret_cast<u32x4*>(orow + 32 * db + 16 * m + 8 * hi) = ch[db][m];
      if (hi == 0 && LSE != nullptr) LSE[lse_off + qi] = (m_run + __log2f(l_tot)) * kLn2;
    }
  }
};

// Key range [lo, up) of an item's query block and its tile range [tb, te).
template <int D, int MODE>
__host__ __device__ __forceinline__ void item_tiles(int q0, int T, int window, int& tb, int& te) {
  using C = FwdCfg<D>;
  int lo = 0, up = T;
  if constexpr (MODE != kNonCausal) {
    up = min(T, q0 + C::BM);
    if constexpr (MODE == kCausalWindow) lo = max(0, q0 - window);
  }
  tb = lo / C::BN;
  te = (up + C::BN - 1) / C::BN;
}

// Head-grouped item order of the streaming kernel (rounds = 0: the snake order). Round k gives
// the workgroups of class c = g mod 8 the heads c + 8 (k per_round + j), j < per_round, all of
// their nqt query blocks at once: workgroup i = g / 8 of the class takes head j = i / nqt and the
// query block q(k nqt + i mod nqt) (rank order: 0 is the heaviest, the last block of the head),
// byte e of the table, four to a word so that the kernel reads it with scalar loads (a vector
// load would count among the tile loads the kernel waits for).
constexpr int kOrderBytes = 256;
struct ItemOrder {
  int rounds;
  int nqt;
  int per_round;
  unsigned q4[kOrderBytes / 4];
};

// ---------------------------------------------------------------------------------------------
// Streaming kernel (d <= 64): persistent grid, direct-to-LDS K/V stream, pipelined tiles.
//
// KN (with QKN): K arrives raw, and each stream tile's 64 rows are RMS-normalised and rotated in
// LDS, in place, once the tile has landed and before any wave reads it (the layer in one launch:
// no separate k pass, no normalised k written). A tile is normalised by every item that streams
// it. The rotation angles are formed in the kernel: the lane's frequencies w_j (radians per
// position) come from row 1 of the rotation tables as atan2(sin w_j, cos w_j), and the angle of
// position t is t w_j reduced to one turn in fp32 before v_sin_f32 / v_cos_f32, so the rotated
// rows differ from the k pass's (fp64 table) by the fp32 error of t w_j (below 2e-4 rad for
// t < 2^13). At d = 64 a tile that follows the previous one (64 positions on, the common case
// inside an item) instead advances each lane's cos and sin by the rotation of 64 w_j, four fp32
// operations per frequency in place of a sine and a cosine; each step adds a few ulps, and the
// direct form restarts the run wherever the stream jumps (a new item). The row's RMS uses
// v_rsq_f32 (about 1 ulp) where the k pass divides by a square root.
// ---------------------------------------------------------------------------------------------
template <int D, int MODE, bool QKN, bool KN>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_stream(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, float eps, Geometry geo, FastDiv fd_bh, int T,
    int window_arg, float scale_log2, int nqt, const ItemOrder ord) {
  using C = FwdCfg<D>;
  static_assert(!KN || QKN, "keys are normalised in the kernel only beside q");
  const int BH = (int)fd_bh.d;  // heads B * H; items are (head, query block) pairs
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  __shared__ __attribute__((aligned(16))) char smem[C::STREAM_LDS];
  const int tid = threadIdx.x;
  const int q_rs = geo.q.t * 2, kv_rs = geo.kv.t * 2;  // row strides in bytes
  WaveTile<D, MODE, QKN> w;
  w.init(T, window, scale_log2, tid, q_rs);
  const int P = (int)gridDim.x;
  const int g = (int)blockIdx.x;
  const int n_items = BH * nqt;
  // bytes spanned by one head's T rows (< 2^31, checked); rows past T read as zero
  const int q_slab = T * q_rs, kv_slab = T * kv_rs;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  const char* qbuf = smem + C::NSTAGE * 2 * C::TILE_BYTES;

  // (KN) Each wave normalises rows 16 w .. 16 w + 15 of a K tile -- the rows its own direct
  // loads brought in, so its own s_waitcnt covers them and the barrier that follows (the one
  // that publishes the landed tile) publishes the normalised rows too -- four lanes per row; lane
  // quarter p = lane % 4 holds chunk p of the row (columns 8 p .. 8 p + 7) and, at d = 64, chunk
  // p + 4 (their rotation partners, d/2 further); at d = 32 the partner chunk p ^ 2 sits in lane
  // p ^ 2. kfr[i]: turns per position of the lane's frequency index 8 (p % (CH / 2)) + i.
  constexpr int KCH = C::CH;  // 16-byte chunks per row
  // kcs, ksn: cos and sin of the lane's row angles for the tile normalised last (first key at
  // key_t0, wave-uniform); kc64, ks64: cos and sin of 64 w, the step to the next tile of a run.
  // (d = 64 only: at d = 32 the 32 extra registers would cost the third workgroup per compute
  // unit, so every tile forms its angles afresh.)
  constexpr bool KINC = D >= 64;
  float kfr[8], kcs[8], ksn[8], kc64[8], ks64[8];
  int key_t0 = -2 * C::BN;
  if constexpr (KN) {
    static_assert(C::LPT * 64 / C::CH == 16, "a wave's direct loads of a K tile are its 16 rows");
    const int p = w.lane & 3;
    const int j0 = 8 * (p % (KCH / 2));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float c1 = T > 1 ? cos_tab[D / 2 + j0 + i] : 1.f;
      const float s1 = T > 1 ? sin_tab[D / 2 + j0 + i] : 0.f;
      kfr[i] = atan2f(s1, c1) * 0.15915494309189535f;  // 1 / (2 pi)
      float turns = (float)C::BN * kfr[i];
      turns -= rintf(turns);
      kc64[i] = __builtin_amdgcn_cosf(turns);
      ks64[i] = __builtin_amdgcn_sinf(turns);
      kcs[i] = 1.f;
      ksn[i] = 0.f;
    }
    // formed before the first direct load is issued, so their wait waits for nothing else
    asm volatile("" : "+v"(kfr[0]), "+v"(kfr[1]), "+v"(kfr[2]), "+v"(kfr[3]), "+v"(kfr[4]),
                 "+v"(kfr[5]), "+v"(kfr[6]), "+v"(kfr[7]) : : "memory");
  }
  // RMSNorm (weightless, eps) and the half-split rotation of the raw K tile in stage st, whose
  // first key is at position t0: y_j = x_j cos + x_{j+d/2} sin, y_{j+d/2} = x_{j+d/2} cos - x_j sin
  // with x = the row over its RMS, in fp32 with one rounding to bf16 (the k pass's arithmetic).
  // Rows past T stay as loaded (zero).
  auto norm_k_tile = [&](unsigned st, int t0) {
    const int ln = w.lane;
    const int r = 16 * w.wave + (ln >> 2), p = ln & 3;
    const int sw = swz_k<D>(r);
    char* row = smem + st * (2 * C::TILE_BYTES) + r * C::ROW_BYTES;
    if (KINC && t0 == key_t0 + C::BN) {
      // the next tile of a run of consecutive tiles: the angles advance by 64 w
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float c = kcs[i], sv = ksn[i];
        kcs[i] = fmaf(c, kc64[i], -(sv * ks64[i]));
        ksn[i] = fmaf(sv, kc64[i], c * ks64[i]);
      }
    } else {
      const float tpos = (float)(t0 + r);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // v_sin_f32 / v_cos_f32 take the angle in turns; reduced to [-1/2, 1/2] first
        float turns = tpos * kfr[i];
        turns -= rintf(turns);
        kcs[i] = __builtin_amdgcn_cosf(turns);
        ksn[i] = __builtin_amdgcn_sinf(turns);
      }
    }
    key_t0 = t0;
    const float(&cs)[8] = kcs;
    const float(&sn)[8] = ksn;
    // sums over the row's four lanes (lanes 4 m .. 4 m + 3, a DPP quad)
    auto quad_sum = [](float x) {
      x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1,
                                                                0xF, 0xF, false));  // lane ^ 1
      x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E,
                                                                0xF, 0xF, false));  // lane ^ 2
      return x;
    };
    if constexpr (KCH == 8) {  // d = 64: both halves of the pair in this lane
      u32x4* pa = reinterpret_cast<u32x4*>(row + 16 * (p ^ sw));
      u32x4* pb = reinterpret_cast<u32x4*>(row + 16 * ((p + 4) ^ sw));
      const u32x4 wa = *pa, wb = *pb;
      float a[8], b[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = bf16lo_to_f32(wa[e]);
        a[2 * e + 1] = bf16hi_to_f32(wa[e]);
        b[2 * e] = bf16lo_to_f32(wb[e]);
        b[2 * e + 1] = bf16hi_to_f32(wb[e]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(a[i], a[i], fmaf(b[i], b[i], ss));
      ss = quad_sum(ss);
      // v_rsq_f32 (about 1 ulp) is ample: the row is rounded to bf16 right after
      const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
      u32x4 ya, yb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y1[2], y2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * e + u;
          const float xa = a[i] * rinv, xb = b[i] * rinv;
          y1[u] = fmaf(xa, cs[i], xb * sn[i]);
          y2[u] = fmaf(xb, cs[i], -(xa * sn[i]));
        }
        ya[e] = pack_bf16x2(y1[0], y1[1]);
        yb[e] = pack_bf16x2(y2[0], y2[1]);
      }
      if (t0 + r < T) {
        *pa = ya;
        *pb = yb;
      }
    } else {  // d = 32: the partner chunk is in lane ^ 2
      static_assert(KCH == 4, "K normalisation in the kernel covers d = 32 and d = 64");
      u32x4* pa = reinterpret_cast<u32x4*>(row + 16 * (p ^ sw));
      const u32x4 wa = *pa;
      u32x4 wb;
#pragma unroll
      for (int e = 0; e < 4; ++e)  // lane ^ 2 (DPP quad permutation 2, 3, 0, 1)
        wb[e] = (uint32_t)__builtin_amdgcn_mov_dpp((int)wa[e], 0x4E, 0xF, 0xF, false);
      float a[8], b[8];
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = bf16lo_to_f32(wa[e]);
        a[2 * e + 1] = bf16hi_to_f32(wa[e]);
        b[2 * e] = bf16lo_to_f32(wb[e]);
        b[2 * e + 1] = bf16hi_to_f32(wb[e]);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss = fmaf(a[i], a[i], ss);
      ss = quad_sum(ss);
      const float rinv = __builtin_amdgcn_rsqf(ss * (1.0f / D) + eps);
      const bool first = p < 2;
      u32x4 ya;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * e + u;
          const float xa = a[i] * rinv, xb = b[i] * rinv;
          y[u] = first ? fmaf(xa, cs[i], xb * sn[i]) : fmaf(xa, cs[i], -(xb * sn[i]));
        }
        ya[e] = pack_bf16x2(y[0], y[1]);
      }
      if (t0 + r < T) *pa = ya;
    }
  };

  // Items of this workgroup, as ranks r = qb * BH + bh in heaviest-first order (qb counts query
  // blocks from the head's last one). Workgroup g runs on XCD g mod 8 (round-robin dispatch).
  // Head-grouped order (ord.rounds > 0): the query blocks of a head all run in the same round on
  // one XCD, so each K/V tile is read from its L2 by all of them at nearly the same time, and the
  // per-round permutations of the blocks (chosen by the launcher) even out the workgroups' loads.
  // Snake order otherwise: rank r sits at position r mod P of its round; when P is a multiple of
  // 8 the odd rounds reverse the order within each class of workgroups g = c mod 8, so a head's
  // query blocks still share an XCD when BH is a multiple of 8, but in different rounds.
  const int g_rev = ((P & 7) == 0) ? ((((P >> 3) - 1 - (g >> 3)) << 3) + (g & 7)) : (P - 1 - g);
  auto rank_of = [&](int k) {
    if (ord.rounds > 0) {
      if (k >= ord.rounds) return n_items;
      const int i = g >> 3;
      const int j = i / ord.nqt, s = i - j * ord.nqt;
      const int e = k * ord.nqt + s;
      const int q = (int)((ord.q4[e >> 2] >> (8 * (e & 3))) & 0xffu);
      return q * BH + (g & 7) + 8 * (k * ord.per_round + j);
    }
    return k * P + ((k & 1) ? g_rev : g);
  };
  auto decode = [&](int rank, int& bh, int& q0, int& tb, int& te) {
    const int qb = (int)fd_bh.div((uint32_t)rank);
    bh = rank - qb * BH;
    q0 = (nqt - 1 - qb) * C::BM;
    item_tiles<D, MODE>(q0, T, window, tb, te);
  };

  // Offsets of this lane's 16-byte chunks inside a K and a V tile: lane L of run
  // (wave * LPT + u) fills chunk p = run * 64 + L of the tile, i.e. row p / CH at physical chunk
  // p % CH, so it loads the logical chunk the row's swizzle puts there.
  uint32_t kofs[C::LPT], vofs[C::LPT];
#pragma unroll
  for (int u = 0; u < C::LPT; ++u) {
    const unsigned p = (unsigned)((w.wave * C::LPT + u) * 64 + w.lane);
    const unsigned r = p / C::CH, pc = p % C::CH;
    kofs[u] = r * kv_rs + 16 * (pc ^ swz_k<D>((int)r));
    vofs[u] = r * kv_rs + 16 * (pc ^ swz_v<D>((int)r));
  }
  // Direct loads of the Q block of an item into the Q buffer (K layout).
  auto dma_q = [&](int bh, int q0) {
    const u32x4 rq = head_rsrc_words(Q + geo.q_head(bh), q_slab);
    const uint32_t qb_ = lds0 + C::NSTAGE * 2 * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::DMA_PER_Q; ++u) {
      const unsigned run = (unsigned)(w.wave * C::DMA_PER_Q + u);
      const unsigned p = run * 64 + (unsigned)w.lane;
      const unsigned r = p / C::CH, pc = p % C::CH;
      dma16(rq, qb_ + run * 1024, ((unsigned)q0 + r) * q_rs + 16 * (pc ^ swz_k<D>((int)r)));
    }
  };

  // (QKN) Direct loads of the rotation-factor rows of the item at q0 into the K half of stage st
  // (run r of the ROPE_RUNS: table r / (runs per table), 1 KiB run within it; chunks past the
  // staged rows are sent out of range). Rows past T are clamped to T - 1.
  auto dma_rope = [&](int q0, unsigned st) {
    constexpr int RPP = C::ROPE_PART / 1024;     // runs per table
    constexpr int CPR = D / 8;                   // 16-byte chunks per staged row
    const u32x4 rc = head_rsrc_words((const bf16*)cos_tab, T * D * 2);
    const u32x4 rs = head_rsrc_words((const bf16*)sin_tab, T * D * 2);
    const uint32_t base = lds0 + st * (2 * C::TILE_BYTES);
    for (int r = w.wave; r < C::ROPE_RUNS; r += 4) {  // wave-uniform
      const int part = r / RPP, run = r % RPP;
      const int p = run * 64 + w.lane;
      // staged row row_i, physical chunk col holds logical chunk col ^ swz_rope(row_i)
      const int row_i = p / CPR, col = p % CPR;
      const int row = row_i < 8 ? min(q0 + 16 * row_i, T - 1) : min(row_i - 8, T - 1);
      const uint32_t off = row_i < C::ROPE_ROWS
                               ? (uint32_t)(row * (D * 2) + 16 * (col ^ swz_rope<D>(row_i)))
                               : kOutOfRange;
      dma16(part ? rs : rc, base + part * C::ROPE_PART + run * 1024, off);
    }
  };

  // The K/V stream: one tile per step, across items. The cursor holds the next tile to issue
  // (pt of [pt, pte) of the item of rank index pk), that head's K and V buffer resources and the
  // stage the tile goes to. Once the items run out, out-of-range loads keep the count per step
  // (and so the waits) the same.
  int pk = 0, pt = 0, pte = 0;
  bool pvalid = true;
  // (KN) first key positions of the two most recently issued tiles (-1: no tile)
  int kpos_prev = -1, kpos_cur = -1;
  u32x4 prk, prv;
  unsigned st_issue = 0;
  auto seek = [&](int rank) {
    int bh_, q0_;
    decode(rank, bh_, q0_, pt, pte);
    const int64_t hoff = geo.kv_head(bh_);
    prk = head_rsrc_words(K + hoff, kv_slab);
    prv = head_rsrc_words(V + hoff, kv_slab);
  };
  seek(rank_of(0));  // g < P <= n_items
  auto issue_next = [&]() {
    const uint32_t kb_ = lds0 + st_issue * (2 * C::TILE_BYTES) + w.wave * (C::LPT * 1024);
    const uint32_t vb_ = kb_ + C::TILE_BYTES;
    const uint32_t base = pvalid ? (uint32_t)(pt * C::BN * kv_rs) : kOutOfRange;
    if constexpr (KN) {
      kpos_prev = kpos_cur;
      kpos_cur = pvalid ? pt * C::BN : -1;
    }
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      dma16(prk, kb_ + u * 1024, base + kofs[u]);
      dma16(prv, vb_ + u * 1024, base + vofs[u]);
    }
    st_issue = (st_issue + 1) & (C::NSTAGE - 1);
    if (pvalid && ++pt >= pte) {
      const int r = rank_of(++pk);
      pvalid = r < n_items;
      if (pvalid) seek(r);
    }
  };

  // Workgroup prologue: the first item's rotation rows (QKN; into the K half of the last stage,
  // which the stream reaches only in the first tile step) and its Q block, then tiles 0 and 1 of
  // the stream, all by direct loads. Only the rows, the Q block and tile 0 are waited for here;
  // tile 1 lands while the first item's first scores are formed (it is waited for after them),
  // and tile 2 goes out once the Q fragments are formed.
  int k = 0, bh, q0, tb, te;
  decode(rank_of(0), bh, q0, tb, te);
  w.set_item(q0);
  if constexpr (QKN) dma_rope(q0, C::NSTAGE - 1);
  dma_q(bh, q0);
  issue_next();
  issue_next();
  wait_vmcnt<C::DMA_PER_TILE>();
  // (KN) the wave's rows of tile 0, in place, before the barrier publishes them
  if constexpr (KN) norm_k_tile(0, kpos_prev);
  __syncthreads();
  typename WaveTile<D, MODE, QKN>::Rope rope;
  {
    w.rope_from_lds(smem + (C::NSTAGE - 1) * (2 * C::TILE_BYTES), rope);
    bf16x8 xf[C::KSTEPS];
    w.load_q_lds(qbuf, xf);
    w.set_q(xf, rope, q0, eps);
  }
  // Every wave has read its Q rows and rotation rows before any wave loads into the Q buffer (the
  // first item's last step) or into that stage (the first tile step).
  __syncthreads();
  issue_next();
  unsigned st_comp = 0;  // stage of the tile being consumed

  while (true) {
    // Item prologue: scores, mask and maximum of its first tile.
    f32x16 sacc[2][2];
    {
      const char* kb0 = smem + st_comp * (2 * C::TILE_BYTES);
      float mx;
      if (w.fast(tb)) {
        w.template scores<true, true>(kb0, tb, sacc[0]);
        mx = w.template mask_max<true>(tb, sacc[0]);
      } else {
        w.template scores<false, true>(kb0, tb, sacc[0]);
        mx = w.template mask_max<false>(tb, sacc[0]);
      }
      w.decide(mx);
    }
    if (k == 0) {
      // The workgroup's first item: tile 1 of the stream, issued in the workgroup prologue, has
      // landed (tile 2 may still be in flight) before any wave reads it.
      wait_vmcnt<C::DMA_PER_TILE>();
      if constexpr (KN) {
        if (kpos_prev >= 0) norm_k_tile(1, kpos_prev);
      }
      __syncthreads();
    }
    const int rank_n = rank_of(k + 1);
    const bool more = rank_n < n_items;
    int nbh = 0, nq0 = 0, ntb = 0, nte = 0;
    if (more) decode(rank_n, nbh, nq0, ntb, nte);

    // Tile t: the next stream tile is issued into the stage tile t-1 used (all reads of it ended
    // before the previous barrier); scores of t+1 alongside the exponentials of t; P(t) V(t)
    // alongside the mask and maximum of t+1; running-maximum update; wait until the stream tile
    // two ahead has landed; barrier. The item's last tile also fetches the next item's Q block,
    // issued before the stream tile so the same wait covers it.
    // HAS_NEXT: t + 1 < te, fixed at compile time so that the last tile of an item has its own
    // code, where the registers of the rotation factors are free.
    auto body = [&](auto has_next_c, int t, f32x16(&cur)[2], f32x16(&nxt)[2]) {
      constexpr bool has_next = decltype(has_next_c)::value;
      if (!has_next && more) {
        dma_q(nbh, nq0);
        if constexpr (QKN) {
          // The K half of this stage is free once tile t's keys are consumed: in the previous
          // step, or in this item's prologue when t is its only tile (then after a barrier).
          if (te - tb == 1) __syncthreads();
          dma_rope(nq0, st_comp);
        }
      }
      issue_next();
      const char* kn = smem + ((st_comp + 1) & (C::NSTAGE - 1)) * (2 * C::TILE_BYTES);
      const char* vc = smem + st_comp * (2 * C::TILE_BYTES) + C::TILE_BYTES;
      bf16x8 pf[2][2];
      float mx = -INFINITY;
      // Every step with a next tile runs the same software pipeline: the scores of both blocks
      // of tile t+1 are computed (a block this wave does not see costs its MFMAs, which keeps one
      // code path and the accumulators in fixed registers) and then masked unless the tile is
      // fully visible; tile t's blocks that the wave does not see hold -inf scores (zero
      // weights), so its exponentials and P V need no guards.
      if constexpr (has_next) {
        // d = 64: the score products of t+1 and the P V products of t in one scheduling region;
        // d = 32, where the step has half the products for the same exponentials, measures
        // faster with the three parts in sequence.
        if constexpr (D >= 64) {
          w.step_pipelined(kn, vc, cur, nxt);
        } else {
          w.template scores<true, true>(kn, t + 1, nxt);
          w.exps(cur, pf);
          w.template pv<true>(vc, t, pf);
        }
        if (w.fast(t + 1))
          mx = w.template mask_max<true>(t + 1, nxt);
        else
          mx = w.template mask_max<false>(t + 1, nxt);
      } else {
        if (w.any(t)) {
          w.exps(cur, pf);
          w.template pv<false>(vc, t, pf);
        }
      }
      if (has_next) w.decide(mx);
      wait_vmcnt<(C::PREFETCH - 2) * C::DMA_PER_TILE>();  // the tile two stages ahead has landed
      if constexpr (KN) {
        // (KN) the wave's rows of that tile (issued one step before this step's), in place,
        // before the barrier publishes them
        if (kpos_prev >= 0) norm_k_tile((st_comp + 2) & (C::NSTAGE - 1), kpos_prev);
      }
      __syncthreads();
      st_comp = (st_comp + 1) & (C::NSTAGE - 1);
    };
    const std::true_type more_tiles;
    const std::false_type last_tile;
    int t = tb;
    for (; t + 2 < te; t += 2) {
      body(more_tiles, t, sacc[0], sacc[1]);
      body(more_tiles, t + 1, sacc[1], sacc[0]);
    }
    if (t + 1 < te) {
      body(more_tiles, t, sacc[0], sacc[1]);
      sacc[0][0] = sacc[1][0];
      sacc[0][1] = sacc[1][1];
      ++t;
    }
    // One instance of the last step (two would invite the compiler to hoist their common loads
    // above the branch, into code where those registers are taken).
    body(last_tile, t, sacc[0], sacc[1]);

    // Item epilogue, after the barrier so the stores do not sit between a stream tile's loads
    // and the wait for them. The next item's Q fragments are formed first: no store is then in
    // flight between the rotation factors' loads and their use.
    if (!more) {
      w.store(O, LSE, geo.q_head(bh), (int64_t)bh * T);
      // The stream's last loads (out of range, writing zeros) land before the workgroup's LDS
      // is released.
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      break;
    }
    {
      // (QKN) the new rows' rotation factors were staged in the K half of the last tile's stage
      // during the last step.
      w.rope_from_lds(smem + ((st_comp + C::NSTAGE - 1) & (C::NSTAGE - 1)) * (2 * C::TILE_BYTES),
                      rope);
      bf16x8 xf[C::KSTEPS];
      w.load_q_lds(qbuf, xf);
      w.set_q(xf, rope, nq0, eps);
    }
    w.store(O, LSE, geo.q_head(bh), (int64_t)bh * T);
    ++k;
    bh = nbh;
    q0 = nq0;
    tb = ntb;
    te = nte;
    w.set_item(q0);
    // Every wave has read its Q rows and rotation factors before any wave issues loads into the
    // Q buffer (the new item's last step) or into that stage (its first step).
    if (QKN || te - tb == 1) __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// Tile kernel (d = 128): one workgroup per item, K/V staged through registers one tile ahead.
// ---------------------------------------------------------------------------------------------
template <int D, int MODE, bool QKN>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_tile(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, const float* __restrict__ cos_tab,
    const float* __restrict__ sin_tab, float eps, Geometry geo, int BH, int T, int window_arg,
    float scale_log2, int nqt, int group_heads) {
  using C = FwdCfg<D>;
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  __shared__ __attribute__((aligned(16))) char smem[C::TILE_LDS];
  const int tid = threadIdx.x;
  const int q_rs = geo.q.t * 2, kv_rs = geo.kv.t * 2;  // row strides in bytes
  WaveTile<D, MODE, QKN> w;
  w.init(T, window, scale_log2, tid, q_rs);
  // Item order: heads in groups of kGroup; within a group the query blocks go heaviest first,
  // each block index for all the group's heads in turn. Workgroup i runs on XCD i % 8
  // (round-robin dispatch), so with groups of 32 a head's blocks all land on one XCD, and the
  // workgroups resident at once cover few heads, whose K/V tiles are then read from that XCD's
  // L2 rather than from HBM; when all heads' K/V fit in the caches together the group is every
  // head (plain heaviest-first order).
  const int kGroup = group_heads;
  const int i = (int)blockIdx.x;
  const int g = i / (kGroup * nqt);
  const int gsize = min(kGroup, BH - g * kGroup);
  const int r = i - g * kGroup * nqt;
  const int bh = g * kGroup + r % gsize;
  const int q0 = (nqt - 1 - r / gsize) * C::BM;
  const int64_t hoff = geo.q_head(bh), kvoff = geo.kv_head(bh);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + kvoff, T * kv_rs);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + kvoff, T * kv_rs);
  int tb, te;
  item_tiles<D, MODE>(q0, T, window, tb, te);
  auto gload = [&](__amdgpu_buffer_rsrc_t r, int t, bool needed, u32x4(&st)[C::LPT]) {
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const uint32_t off =
          needed ? (uint32_t)((t * C::BN + e / C::CH) * kv_rs + 16 * (e % C::CH)) : kOutOfRange;
      st[u] = buffer_load16(r, off);
    }
  };
  auto lstore = [&](int slot, const u32x4(&ks)[C::LPT], const u32x4(&vs)[C::LPT]) {
    char* kb_ = smem + slot * C::TILE_BYTES;
    char* vb_ = smem + (2 + slot) * C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH, c = e % C::CH;
      *reinterpret_cast<u32x4*>(kb_ + r * C::ROW_BYTES + 16 * (c ^ swz_k<D>(r))) = ks[u];
      *reinterpret_cast<u32x4*>(vb_ + r * C::ROW_BYTES + 16 * (c ^ swz_v<D>(r))) = vs[u];
    }
  };

  // The item's Q rows, their rotation factors and its first K/V tile are all requested before
  // the q norm waits for the first two, so the tile's latency overlaps theirs.
  w.set_item(q0);
  u32x4 kst[C::LPT], vst[C::LPT];
  {
    bf16x8 xf[C::KSTEPS];
    typename WaveTile<D, MODE, QKN>::Rope rope;
    w.load_q_global(head_rsrc(Q + hoff, T * q_rs), q0, xf);
    w.load_rope(q0, cos_tab, sin_tab, rope);
    gload(rk, tb, true, kst);
    gload(rv, tb, true, vst);
    w.set_q(xf, rope, q0, eps);
  }

  lstore(0, kst, vst);
  __syncthreads();
  for (int t = tb; t < te; ++t) {
    const int i = t - tb;
    gload(rk, t + 1, t + 1 < te, kst);
    gload(rv, t + 1, t + 1 < te, vst);
    if (w.any(t)) w.whole_tile(smem + (i & 1) * C::TILE_BYTES, smem + (2 + (i & 1)) * C::TILE_BYTES, t);
    lstore((i + 1) & 1, kst, vst);
    __syncthreads();
  }
  w.store(O, LSE, hoff, (int64_t)bh * T);
}

// Workgroups of one kernel instantiation that the current device holds at once. Each
// instantiation (Kern is a distinct function, so Tag is a distinct type) keeps its own per-device
// cache; threads that race on the first query store the same value, through relaxed atomics.
template <typename Tag, typename Kern>
static hipError_t resident_workgroups(Kern kern, int* out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool slot = dev >= 0 && dev < kMaxDevices;
  if (slot) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, 0);
  if (e != hipSuccess) return e;
  const int n = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  if (slot) cached[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return hipSuccess;
}

// A permutation perm (slot -> block) with base[s] + c[perm[s]] <= cap for every slot s, if one
// exists (bipartite matching by augmenting paths; n is at most a few dozen).
static bool match_under(const std::vector<int>& base, const std::vector<int>& c, int cap,
                        std::vector<int>& perm) {
  const int n = (int)c.size();
  std::vector<int> owner(n, -1);  // owner[q]: slot holding block q
  std::vector<char> seen;
  std::function<bool(int)> aug = [&](int s) {
    for (int q = 0; q < n; ++q) {
      if (base[s] + c[q] > cap || seen[q]) continue;
      seen[q] = 1;
      if (owner[q] < 0 || aug(owner[q])) {
        owner[q] = s;
        return true;
      }
    }
    return false;
  };
  for (int s = 0; s < n; ++s) {
    seen.assign(n, 0);
    if (!aug(s)) return false;
  }
  perm.assign(n, 0);
  for (int q = 0; q < n; ++q) perm[owner[q]] = q;
  return true;
}

// Per-round permutations sig[k] of the n query blocks over the n workgroups of a head's group
// (block costs c, in tiles plus one for the transition, in rank order), so that the workgroups'
// summed costs stay close to their mean. Rounds alternate the identity and the reverse (which
// pairs heavy with light blocks); an odd count of three or more starts with the best triple
// (sig 1 over every permutation when n <= 8, sig 2 by bottleneck matching); single swaps within
// a round that lower the largest sum finish it. Returns the largest sum.
static int balance_rounds(const std::vector<int>& c, int R, std::vector<std::vector<int>>& sig) {
  const int n = (int)c.size();
  sig.assign(R, std::vector<int>(n));
  for (int k = 0; k < R; ++k)
    for (int q = 0; q < n; ++q) sig[k][q] = (k % 2 == 0) ? q : n - 1 - q;
  if (R % 2 == 1 && R >= 3 && n >= 2 && n <= 8) {
    // rounds 0..2: identity, the best sig 1, then sig 2 by bottleneck matching; the rest pairs
    const int cmin = *std::min_element(c.begin(), c.end());
    const int cmax = *std::max_element(c.begin(), c.end());
    int csum = 0;
    for (int x : c) csum += x;
    int best = 3 * cmax + 1;
    std::vector<int> s1(n), base(n), p2, best1, best2;
    for (int q = 0; q < n; ++q) s1[q] = q;
    do {
      int bmax = 0;
      for (int q = 0; q < n; ++q) {
        base[q] = c[q] + c[s1[q]];
        bmax = std::max(bmax, base[q]);
      }
      const int lb = std::max(bmax + cmin, (3 * csum + n - 1) / n);
      for (int cap = lb; cap < best; ++cap) {
        if (match_under(base, c, cap, p2)) {
          best = cap;
          best1 = s1;
          best2 = p2;
          break;
        }
      }
    } while (std::next_permutation(s1.begin(), s1.end()));
    if (!best1.empty()) {
      sig[1] = best1;
      sig[2] = best2;
      for (int k = 3; k < R; ++k)
        for (int q = 0; q < n; ++q) sig[k][q] = (k % 2 == 1) ? n - 1 - q : q;
    }
  }
  std::vector<int> load(n, 0);
  for (int k = 0; k < R; ++k)
    for (int q = 0; q < n; ++q) load[q] += c[sig[k][q]];
  for (int it = 0; it < 64 * n * R; ++it) {
    const int sm = (int)(std::max_element(load.begin(), load.end()) - load.begin());
    int bk = -1, bs = -1, bnew = load[sm];
    for (int k = 0; k < R; ++k)
      for (int s2 = 0; s2 < n; ++s2) {
        if (s2 == sm) continue;
        const int a = sig[k][sm], b = sig[k][s2];
        const int m2 = std::max(load[sm] - c[a] + c[b], load[s2] - c[b] + c[a]);
        if (m2 < bnew) {
          bnew = m2;
          bk = k;
          bs = s2;
        }
      }
    if (bk < 0) break;
    const int a = sig[bk][sm], b = sig[bk][bs];
    load[sm] += c[b] - c[a];
    load[bs] += c[a] - c[b];
    sig[bk][sm] = b;
    sig[bk][bs] = a;
  }
  return *std::max_element(load.begin(), load.end());
}

// The head-grouped order for a launch of P workgroups, or rounds = 0 (the snake order) when the
// shape does not divide into whole rounds, the table does not fit, or the best permutations found
// leave a workgroup more than 8 % above the mean. Permutations are kept per (costs, rounds).
// ATTN_ITEM_ORDER=snake in the environment (read at each launch) keeps the snake order, for
// comparing the two; outputs are bitwise the same either way.
template <int D, int MODE>
static ItemOrder item_order(int P, int BH, int T, int window, int nqt) {
  ItemOrder ord{};
  const char* env = std::getenv("ATTN_ITEM_ORDER");
  if (env != nullptr && std::strcmp(env, "snake") == 0) return ord;
  if (P % 8 != 0 || BH % 8 != 0 || nqt < 1 || nqt > 255) return ord;
  const int J = P / 8, hpc = BH / 8;
  if (J % nqt != 0) return ord;
  const int per_round = J / nqt;
  if (hpc % per_round != 0) return ord;
  const int R = hpc / per_round;
  if ((int64_t)R * nqt > kOrderBytes) return ord;
  std::vector<int> c(nqt);
  int64_t total = 0;
  for (int q = 0; q < nqt; ++q) {
    int tb = 0, te = 0;
    item_tiles<D, MODE>((nqt - 1 - q) * FwdCfg<D>::BM, T, window, tb, te);
    c[q] = te - tb + 1;
    total += c[q];
  }
  static std::mutex mu;
  static std::map<std::pair<std::vector<int>, int>, std::pair<int, std::vector<std::vector<int>>>>
      cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(c, R);
  auto it = cache.find(key);
  if (it == cache.end()) {
    std::vector<std::vector<int>> sig;
    const int mx = balance_rounds(c, R, sig);
    it = cache.emplace(key, std::make_pair(mx, std::move(sig))).first;
  }
  const int mx = it->second.first;
  if ((int64_t)mx * nqt * 100 > (int64_t)108 * R * total) return ord;  // above 1.08 x the mean
  ord.rounds = R;
  ord.nqt = nqt;
  ord.per_round = per_round;
  for (int k = 0; k < R; ++k)
    for (int q = 0; q < nqt; ++q) {
      const int e = k * nqt + q;
      ord.q4[e >> 2] |= (unsigned)it->second.second[k][q] << (8 * (e & 3));
    }
  return ord;
}

// Launch arguments shared by the entry points.
struct Bf16Args {
  const void *q, *k, *v;
  void* out;
  float* lse;
  const float *cos_tab, *sin_tab;
  float eps;
  int B, H, T, window;
  Geometry geo;
};

template <int D, int MODE, bool QKN, bool KN = false>
static hipError_t launch_bf16_t(const Bf16Args& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const int nqt = (a.T + FwdCfg<D>::BM - 1) / FwdCfg<D>::BM;
  const int64_t n_items = (int64_t)BH * nqt;
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  if constexpr (D <= 64) {
    int resident = 0;
    struct Tag {};
    hipError_t e = resident_workgroups<Tag>(attn_fwd_bf16_stream<D, MODE, QKN, KN>, &resident);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(n_items < resident ? n_items : resident);
    const ItemOrder ord = item_order<D, MODE>((int)grid, BH, a.T, a.window, nqt);
    hipLaunchKernelGGL((attn_fwd_bf16_stream<D, MODE, QKN, KN>), dim3(grid), dim3(256), 0, stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.out, a.lse,
                       a.cos_tab, a.sin_tab, a.eps, a.geo, make_fastdiv((uint32_t)BH), a.T,
                       a.window, scale_log2, nqt, ord);
  } else {
    static_assert(!KN, "keys are normalised in the kernel only by the streaming kernel (d <= 64)");
    hipLaunchKernelGGL((attn_fwd_bf16_tile<D, MODE, QKN>), dim3((unsigned)n_items), dim3(256), 0,
                       stream, (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, (bf16*)a.out,
                       a.lse, a.cos_tab, a.sin_tab, a.eps, a.geo, BH, a.T, a.window, scale_log2, nqt,
                       group_heads(BH, (int64_t)a.T * D * 2 * 2));
  }
  return hipGetLastError();
}

template <int D, bool QKN, bool KN = false>
static hipError_t launch_bf16_d(Bf16Args a, int causal, hipStream_t stream) {
  // A window of T - 1 or more hides nothing: run it as plain causal.
  if (!causal) {
    a.window = -1;
    return launch_bf16_t<D, kNonCausal, QKN, KN>(a, stream);
  }
  if (a.window < 0 || a.window >= a.T - 1) {
    a.window = -1;
    return launch_bf16_t<D, kCausal, QKN, KN>(a, stream);
  }
  return launch_bf16_t<D, kCausalWindow, QKN, KN>(a, stream);
}

template <bool QKN>
static hipError_t launch_bf16(const Bf16Args& a, int d, int causal, hipStream_t stream) {
  if (d == 32) return launch_bf16_d<32, QKN>(a, causal, stream);
  if (d == 64) return launch_bf16_d<64, QKN>(a, causal, stream);
  if (d == 128) return launch_bf16_d<128, QKN>(a, causal, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                const Dims& dm, int window, int causal, hipStream_t stream) {
  const Bf16Args a{q, k, v, out, lse, nullptr, nullptr, 0.f, dm.B, dm.H, dm.T, window,
                   make_geometry(dm)};
  return launch_bf16<false>(a, dm.d, causal, stream);
}

hipError_t launch_attn_fwd_bf16_qknorm(const void* q, const void* k, const void* v, void* out,
                                       float* lse, const float* cos_tab, const float* sin_tab,
                                       float eps, const Dims& dm, int window, int causal,
                                       hipStream_t stream) {
  const Bf16Args a{q, k, v, out, lse, cos_tab, sin_tab, eps, dm.B, dm.H, dm.T, window,
                   make_geometry(dm)};
  return launch_bf16<true>(a, dm.d, causal, stream);
}

hipError_t launch_attn_fwd_bf16_qknorm_kin(const void* q, const void* k, const void* v, void* out,
                                           float* lse, const float* cos_tab,
                                           const float* sin_tab, float eps, const Dims& dm,
                                           int window, int causal, hipStream_t stream) {
  const Bf16Args a{q, k, v, out, lse, cos_tab, sin_tab, eps, dm.B, dm.H, dm.T, window,
                   make_geometry(dm)};
  if (dm.d == 32) return launch_bf16_d<32, true, true>(a, causal, stream);
  if (dm.d == 64) return launch_bf16_d<64, true, true>(a, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
