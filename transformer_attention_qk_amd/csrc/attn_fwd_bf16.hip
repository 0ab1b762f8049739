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
//     queries [32w, 32w + 32) of that block. Workgroups are launched heaviest query block first.
//   - Key/value tiles of BN = 64 rows are copied HBM -> registers -> LDS, double-buffered: the
//     loads of tile t+1 are issued before tile t is consumed, so one barrier per tile suffices.
//   - S^T = K Q^T per 32-key block with v_mfma_f32_32x32x16_bf16: A = K from LDS (16 bytes per
//     lane), B = Q^T kept in registers for the whole workgroup. In the accumulator each lane owns
//     one query (lane % 32) and 16 keys, so row maxima and sums are lane-local plus one exchange
//     between lanes l and l + 32.
//   - O^T += V^T P^T with the same MFMA: B = P^T straight from the S^T accumulator (rounded to
//     bf16), A = V^T read from the row-major V tile with ds_read_b64_tr_b16, which transposes
//     4x16 blocks of 16-bit values between lanes. The key order inside each 16-key MFMA step
//     follows the S^T accumulator's register order on both operands.
//   - LDS rows are XOR-swizzled in 16-byte chunks so that the K reads (16 rows x 16 bytes per
//     quarter-wave) and the transposing V reads (4 rows x 64 bytes per half-wave) hit distinct
//     banks.
//   - Tiles the mask hides completely are never loaded; 32-key blocks a wave cannot see are
//     skipped by that wave; the elementwise mask is applied only on blocks that straddle the
//     diagonal, the window edge or the end of the sequence.
//   - Global loads are buffer loads whose range is the head's [T][d] slab: rows past T read as
//     zero without a branch, and the prefetch of the tile after the last one is sent out of
//     range, so every load and LDS store is unconditional and the compiler never has to wait
//     on a prefetch before it is consumed.
//   - The running maximum is raised lazily: only when a tile's maximum exceeds it by more than
//     kRescaleSlack (base-2 units) are the accumulators rescaled. Until then the weights
//     exp2(s - m) stay below 2^kRescaleSlack, which fp32 sums and bf16 weights hold exactly as
//     well as weights below 1.
#include <math.h>

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
  static constexpr int LPT = BN * CH / 256;  // 16-byte chunks per thread per tile
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile then V tile
  static_assert(LPT >= 1, "tile too small for 256 threads");
};

// Physical 16-byte chunk of logical chunk c in LDS row r of the K tile: quarter-wave K reads
// touch 16 consecutive rows at one logical chunk, which this spreads over all 64 banks.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 32) return (r >> 2) & 3;
  else if constexpr (D == 64) return (r >> 1) & 7;
  else return r & 15;
}
// Same for the V tile: half-wave transposing reads touch 4 consecutive rows x 64 bytes.
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

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    bf16* __restrict__ O, float* __restrict__ LSE, int BH, int T, int window, int causal,
    float scale_log2, int nqt) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE_BYTES];

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

  // Q^T fragments (B operand): lane holds Q[qi][16 s + 8 hi .. +8); rows past T read as zero.
  bf16x8 qf[C::KSTEPS];
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, (uint32_t)(qi * C::ROW_BYTES + 32 * s + 16 * hi)));

  // Keys any query of this workgroup can see, and those of this wave.
  int kv_lo = 0, kv_hi = T, w_lo = 0, w_hi = T;
  if (causal) {
    kv_hi = min(T, q0 + C::BM);
    w_hi = min(T, qw0 + 32);
    if (window >= 0) {
      kv_lo = max(0, q0 - window);
      w_lo = max(0, qw0 - window);
    }
  }
  const int t_begin = kv_lo / C::BN;
  const int t_end = (kv_hi + C::BN - 1) / C::BN;

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running maximum of the scaled scores, base-2 units
  float l_run = 0.f;        // this lane's part of the running sum (its 16 keys per block)

  // Global -> register staging of one K and one V tile (rows past T read as zero; a tile that
  // is not needed is sent out of range and costs no memory traffic).
  u32x4 kst[C::LPT], vst[C::LPT];
  auto gload = [&](int t, bool needed) {
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const uint32_t off = needed ? (uint32_t)((t * C::BN + e / C::CH) * C::ROW_BYTES + 16 * (e % C::CH))
                                  : kOutOfRange;
      kst[u] = buffer_load16(rk, off);
      vst[u] = buffer_load16(rv, off);
    }
  };
  auto lstore = [&](int buf) {
    char* kb_ = smem + buf * C::STAGE_BYTES;
    char* vb_ = kb_ + C::TILE_BYTES;
#pragma unroll
    for (int u = 0; u < C::LPT; ++u) {
      const int e = tid + 256 * u;
      const int r = e / C::CH;
      const int c = e % C::CH;
      *reinterpret_cast<u32x4*>(kb_ + r * C::ROW_BYTES + 16 * (c ^ swz_k<D>(r))) = kst[u];
      *reinterpret_cast<u32x4*>(vb_ + r * C::ROW_BYTES + 16 * (c ^ swz_v<D>(r))) = vst[u];
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

  gload(t_begin, true);
  lstore(0);
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    gload(t + 1, t + 1 < t_end);
    const char* kbuf = smem + buf * C::STAGE_BYTES;
    const char* vbuf = kbuf + C::TILE_BYTES;
    const int kt0 = t * C::BN;

    bool active[2], full[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int b0 = kt0 + 32 * kb;
      active[kb] = (b0 < w_hi) && (b0 + 32 > w_lo);
      bool f = (b0 + 32 <= T);
      if (causal) f = f && (b0 + 31 <= qw0) && (window < 0 || qw0 + 31 - b0 <= window);
      full[kb] = f;
    }

    if (active[0] || active[1]) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!active[kb]) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              kbuf + 32 * kb * C::ROW_BYTES + k_row_off + 16 * ((2 * s + hi) ^ k_swz));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }

      // Mask, then the tile's row maximum (raw scores; the scale is positive).
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!active[kb]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = -INFINITY;
          continue;
        }
        if (!full[kb]) {
          const int b0 = kt0 + 32 * kb + 4 * hi;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = b0 + 8 * (r >> 2) + (r & 3);
            bool vis = key < T;
            if (causal) vis = vis && key <= qi && (window < 0 || qi - key <= window);
            if (!vis) sacc[kb][r] = -INFINITY;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      }
      mx = pair_max(mx);
      const float m_tile = mx * scale_log2;
      // Raise the running maximum only when the tile exceeds it by more than the slack (always
      // on a row's first visible tile, since m_run starts at -inf).
      if (__builtin_amdgcn_ballot_w64(m_tile > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = __builtin_amdgcn_exp2f(m_run - ((m_new == -INFINITY) ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;

      // P = exp2(s * scale - m), rounded to bf16 in the B-operand order of the P V product.
      bf16x8 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * tt + 2 * e], scale_log2, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb][8 * tt + 2 * e + 1], scale_log2, -m_use));
            l_run += p0 + p1;
            w[e] = pack_bf16x2(p0, p1);
          }
          pf[kb][tt] = __builtin_bit_cast(bf16x8, w);
        }
      }

      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (!active[kb]) continue;
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

    lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
  const float l_tot = pair_sum(l_run);
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

hipError_t launch_attn_fwd_bf16(const void* q, const void* k, const void* v, void* out, float* lse,
                                int B, int H, int T, int d, int window, int causal,
                                hipStream_t stream) {
  const int BH = B * H;
  const int nqt = (T + 127) / 128;
  const unsigned grid = (unsigned)((int64_t)BH * nqt);
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
#define ATTN_BF16_CASE(DD)                                                                   \
  if (d == DD) {                                                                             \
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<DD>, dim3(grid), dim3(256), 0, stream,          \
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)out, lse, BH, T, \
                       window, causal, scale_log2, nqt);                                     \
    return hipGetLastError();                                                                \
  }
  ATTN_BF16_CASE(32)
  ATTN_BF16_CASE(64)
  ATTN_BF16_CASE(128)
#undef ATTN_BF16_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
