// Backward pass of the causal / sliding-window attention on gfx950.
//
// The gradients are those of the forward definition (the exact derivatives of
// out_i = sum_{j in A(i)} softmax_j(c q_i . k_j) v_j with c = 1/sqrt(d); the attention of
// "Projeção em um Subespaço de Consulta", unhomeschool.com, "O que a Atenção Calcula", used in
// the training step of the train.py listing of "Подробный технический разбор реализации
// Autoresearch", habr.com, article 1010198, whose `loss.backward()` differentiates it). With
// P_ij = exp(c q_i . k_j - lse_i) recomputed from the forward's LSE:
//   dV_j = sum_i P_ij dO_i            dP_ij = dO_i . v_j
//   D_i  = dO_i . O_i  (= sum_j P_ij dP_ij)          dS_ij = P_ij (dP_ij - D_i)
//   dQ_i = c sum_j dS_ij k_j          dK_j = c sum_i dS_ij q_i
// Grouped-query heads: a kv head's dK, dV sum over the query heads of its group.
//
// Kernels per bf16 call, in launch order:
//   - attn_bwd_dq_bf16: one workgroup per (batch * head, block of 128 queries), wave w owning
//     queries [32 w, 32 w + 32): the forward's layout (S^T = K Q^T, lane = query), with
//     dP^T = V dO^T beside it and dQ^T += K^T dS^T. It also forms D_i = dO_i . O_i in fp32 for
//     its rows (their dO is in registers already, so D_i costs one read of the row's O) and
//     writes it for the next kernel. The fp32 path runs attn_bwd_delta (one pass over out and
//     dout) for D instead.
//   - attn_bwd_dkdv_bf16: one workgroup per (batch, kv head, block of 128 keys), wave w owning
//     keys [32 w, 32 w + 32). The wave keeps its K and V rows in registers (B operands) and
//     walks the query tiles that see its keys (all query heads of the group), staged in LDS:
//     S = Q K^T and dP = dO V^T with v_mfma_f32_32x32x16_bf16 (A = Q, dO rows from LDS); in the
//     accumulators each lane owns one key and 16 queries, so P and dS are formed in place and
//     feed dV^T += dO^T P and dK^T += Q^T dS as B operands, with A = dO^T, Q^T read from the
//     same tiles by transposing LDS reads (ds_read_b64_tr_b16).
// Computing dQ in its own kernel recomputes S and dP once more instead of accumulating dQ across
// key blocks with atomics: no scratch memory and no ordering nondeterminism.
// P and dS are rounded to bf16 (nearest even) for the matrix products; every accumulation is
// fp32; dQ, dK, dV are rounded to bf16 once at the end.
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tile_ops.hpp"

namespace attn {

template <int D>
struct BwdCfg {
  static constexpr int KS = D / 16;          // 16-wide MFMA k-steps over d
  static constexpr int DB = D / 32;          // 32-row blocks of d in the transposed products
  static constexpr int CH = D / 8;           // 16-byte chunks per row
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int TR = 64;              // rows per staged tile
  static constexpr int TILE_BYTES = TR * ROW_BYTES;
  static constexpr int LPT = TR * CH / 256;  // 16-byte chunks per thread per tile
  static_assert(LPT >= 1, "tile too small for 256 threads");
};

// Rows of a staged tile are XOR-swizzled in 16-byte chunks by swz_v, which depends on the row
// only through row % 4, so the transposing reads (rows 4 apart share a swizzle) stay
// lane-constant.
template <int D>
__device__ __forceinline__ int tile_chunk(int row, int c) {
  return c ^ swz_v<D>(row);
}

// 16 bytes at logical chunk c of tile row `row`.
template <int D>
__device__ __forceinline__ bf16x8 tile_row16(const char* tile, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + row * BwdCfg<D>::ROW_BYTES +
                                          16 * tile_chunk<D>(row, c));
}

// A operand of a product whose contraction runs over the 16 tile rows r0 .. r0 + 15 and whose
// output rows are the tile's columns 32 db .. 32 db + 31. The rows follow the register order of
// a 32x32 accumulator: k-slot j of lane half h is row r0 + 8 (j / 4) + 4 h + j % 4, the order in
// which an accumulator's registers 8 t .. 8 t + 7 (packed to bf16) hold their rows.
template <int D>
__device__ __forceinline__ bf16x8 tile_tr16(const char* tile, int r0, int db, int lane) {
  const int hi = lane >> 5, va = (lane & 15) >> 2, vb = lane & 3, vg1 = (lane >> 4) & 1;
  u32x2 part[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int row = r0 + 8 * u + 4 * hi + va;
    const int c = 4 * db + 2 * vg1 + (vb >> 1);
    part[u] = ds_read_tr16_b64(tile + row * BwdCfg<D>::ROW_BYTES + 16 * tile_chunk<D>(row, c) +
                               8 * (vb & 1));
  }
  const u32x4 a4{part[0][0], part[0][1], part[1][0], part[1][1]};
  return __builtin_bit_cast(bf16x8, a4);
}

// Cooperative staging of tile rows row0 .. row0 + 63 of one head (buffer range = the head's T
// rows, so rows past T read as zero) into a swizzled LDS tile, in two halves so that the loads of
// the next tile are in flight while the current one is used: load_tile into registers, then
// store_tile into the LDS buffer that no wave reads any more.
template <int D>
__device__ __forceinline__ void load_tile(u32x4 (&x)[BwdCfg<D>::LPT], __amdgpu_buffer_rsrc_t r,
                                          int row0, int rs, int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int u = 0; u < C::LPT; ++u) {
    const int p = u * 256 + tid;
    x[u] = buffer_load16(r, (uint32_t)((row0 + p / C::CH) * rs + 16 * (p % C::CH)));
  }
}
template <int D>
__device__ __forceinline__ void store_tile(char* tile, const u32x4 (&x)[BwdCfg<D>::LPT], int tid) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int u = 0; u < C::LPT; ++u) {
    const int p = u * 256 + tid;
    const int row = p / C::CH, c = p % C::CH;
    *reinterpret_cast<u32x4*>(tile + row * C::ROW_BYTES + 16 * tile_chunk<D>(row, c)) = x[u];
  }
}

// Workgroup i of a grid of n_heads * n_blocks: heads in groups of kGroup, and within a group
// block rank 0 for every head of the group, then rank 1, and so on.
__device__ __forceinline__ void group_order(int i, int n_heads, int n_blocks, int kGroup,
                                            int& head, int& rank) {
  const int g = i / (kGroup * n_blocks);
  const int gsize = min(kGroup, n_heads - g * kGroup);
  const int r = i - g * kGroup * n_blocks;
  head = g * kGroup + r % gsize;
  rank = r / gsize;
}

// Register r of a 32x32 accumulator holds row 8 (r / 4) + 4 (lane / 32) + r % 4.
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// Visibility of key j to query i under the launch's mask (R4, R5), with both inside [0, T).
template <int MODE>
__device__ __forceinline__ bool visible_qk(int i, int j, int T, int window) {
  bool v = (i < T) & (j < T);
  if constexpr (MODE != kNonCausal) v = v & (j <= i);
  if constexpr (MODE == kCausalWindow) v = v & (i - j <= window);
  return v;
}
// Some pair of queries [qa, qa + 32) and keys [ka, ka + 32) is visible.
template <int MODE>
__device__ __forceinline__ bool block_any(int qa, int ka, int T, int window) {
  bool v = (qa < T) & (ka < T);
  if constexpr (MODE != kNonCausal) v = v & (qa + 31 >= ka);
  if constexpr (MODE == kCausalWindow) v = v & (qa - (ka + 31) <= window);
  return v;
}
// Every pair is visible.
template <int MODE>
__device__ __forceinline__ bool block_all(int qa, int ka, int T, int window) {
  bool v = (qa + 32 <= T) & (ka + 32 <= T);
  if constexpr (MODE != kNonCausal) v = v & (qa >= ka + 31);
  if constexpr (MODE == kCausalWindow) v = v & (qa + 31 - ka <= window);
  return v;
}

// ---------------------------------------------------------------------------------------------
// D_i = dO_i . O_i (fp32), one row per group of L = d / E lanes (16-byte chunks).
// ---------------------------------------------------------------------------------------------
template <typename Elem, int D>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const Elem* __restrict__ O,
                                                             const Elem* __restrict__ dO,
                                                             float* __restrict__ delta,
                                                             Geometry geo, FastDiv fT,
                                                             int n_rows) {
  constexpr int E = 16 / (int)sizeof(Elem);
  constexpr int L = D / E;
  constexpr int RPB = 256 / L;
  const int n = (int)blockIdx.x * RPB + (int)threadIdx.x / L;
  const int sub = (int)threadIdx.x % L;
  const bool valid = n < n_rows;
  const int nn = valid ? n : n_rows - 1;  // the group redoes the last row and stores nothing
  const int bh = (int)fT.div((uint32_t)nn), t = nn - bh * (int)fT.d;
  const int64_t off = geo.q_head(bh) + (int64_t)t * geo.q.t + sub * E;
  const u32x4 a = *reinterpret_cast<const u32x4*>(O + off);
  const u32x4 b = *reinterpret_cast<const u32x4*>(dO + off);
  float acc = 0.f;
  if constexpr (sizeof(Elem) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(bf16lo_to_f32(a[w]), bf16lo_to_f32(b[w]), acc);
      acc = fmaf(bf16hi_to_f32(a[w]), bf16hi_to_f32(b[w]), acc);
    }
  } else {
    // (whole-vector casts: a cast of a subscripted vector element is not reliable here)
    const f32x4 af = __builtin_bit_cast(f32x4, a), bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(af[w], bf[w], acc);
  }
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if (valid && sub == 0) delta[nn] = acc;
}

// ---------------------------------------------------------------------------------------------
// dK, dV (bf16 MFMA).
// ---------------------------------------------------------------------------------------------
// Two workgroups per CU (two waves per SIMD): a wave's chain of loads, MFMAs and exponentials
// leaves the SIMD idle between its own instructions, and the second wave fills those gaps.
// PASS selects the outputs: kBothPasses computes dK and dV together (d <= 64); at d = 128 the two
// accumulator sets do not fit two waves' registers, so one launch computes dV (S and P only) and
// a second dK (S, dP and dS): S is computed twice, a quarter more MFMA work for twice the waves.
constexpr int kBothPasses = 2, kPassDV = 0, kPassDK = 1;
template <int D, int MODE, int PASS>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_bf16(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    bf16* __restrict__ dK, bf16* __restrict__ dV, Geometry geo, int H_kv, int T, int window_arg,
    float scale_log2, float scale, int nkb, int group_heads) {
  using C = BwdCfg<D>;
  // Two buffers, each: Q tile, dO tile, then LSE (base 2) and D of its 64 queries.
  constexpr int NBUF = 2;
  constexpr int BUF = 2 * C::TILE_BYTES + 2 * C::TR * 4;
  __shared__ __attribute__((aligned(16))) char smem[NBUF * BUF];
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  const int tid = (int)threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Item order: kv heads in groups of `group_heads`; within a group the key blocks go heaviest
  // first (with a causal mask the first blocks see the most queries), each block index for all
  // of the group's heads in turn. Workgroup i runs on XCD i % 8, so with groups of 32 a head's
  // blocks share one XCD's L2 and the workgroups resident at once read the query tiles of few
  // heads; when every head's tiles fit in the caches at once the group is all heads (plain
  // heaviest-first order).
  const int BG = (int)gridDim.x / nkb;
  int kblk, bg;  // bg = b * H_kv + g
  group_order((int)blockIdx.x, BG, nkb, group_heads, bg, kblk);
  const int b = bg / H_kv, g = bg - b * H_kv;
  const int group = (int)geo.group.d, H = (int)geo.H.d;
  const int k0 = kblk * 128, kw0 = k0 + 32 * wave;
  const int q_rs = geo.q.t * 2, kv_rs = geo.kv.t * 2;
  const int64_t kvoff = (int64_t)b * geo.kv.b + (int64_t)g * geo.kv.h;

  // This wave's K and V rows as B operands: lane l holds row kw0 + l % 32, elements
  // 16 s + 8 (l / 32) .. + 8.
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + kvoff, T * kv_rs);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + kvoff, T * kv_rs);
  constexpr bool DO_DV = PASS != kPassDK, DO_DK = PASS != kPassDV;
  bf16x8 kf[C::KS], vf[C::KS];  // vf: only where dP is needed (dK)
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const uint32_t off = (uint32_t)((kw0 + l32) * kv_rs + 32 * s + 16 * hi);
    kf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rk, off));
    if constexpr (DO_DK) vf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rv, off));
  }
  f32x16 dka[C::DB], dva[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
    dka[db] = f32x16{};
    dva[db] = f32x16{};
  }

  // Queries that see a key of [k0, k0 + 128).
  int q_lo = 0, q_hi = T;
  if constexpr (MODE != kNonCausal) q_lo = k0;
  if constexpr (MODE == kCausalWindow) q_hi = min(T, k0 + 128 + window);
  const int key = kw0 + l32;

  // The query tiles: for each query head of the group, tiles qt0, qt0 + 64, ... below q_hi.
  const int qt0 = q_lo / C::TR * C::TR;
  const int n_qt = (q_hi - qt0 + C::TR - 1) / C::TR;  // >= 1: q_lo = k0 < T and q_hi > k0
  const int n_tiles = group * n_qt;
  auto tile_of = [&](int i, int& bh, int& qt, int64_t& qoff) {
    const int hg = i / n_qt;
    const int h = g * group + hg;
    bh = b * H + h;
    qt = qt0 + (i - hg * n_qt) * C::TR;
    qoff = (int64_t)b * geo.q.b + (int64_t)h * geo.q.h;
  };
  u32x4 xq[C::LPT], xdo[C::LPT];
  float xl = 0.f, xd = 0.f;
  auto fetch = [&](int i) {
    int bh, qt;
    int64_t qoff;
    tile_of(i, bh, qt, qoff);
    load_tile<D>(xq, head_rsrc(Q + qoff, T * q_rs), qt, q_rs, tid);
    load_tile<D>(xdo, head_rsrc(dO + qoff, T * q_rs), qt, q_rs, tid);
    if (tid < C::TR) {
      const int qi = qt + tid;
      xl = (qi < T) ? LSE[(int64_t)bh * T + qi] * kLog2e : 0.f;
      xd = (qi < T) ? Delta[(int64_t)bh * T + qi] : 0.f;
    }
  };
  auto put = [&](int buf) {
    char* base = smem + buf * BUF;
    store_tile<D>(base, xq, tid);
    store_tile<D>(base + C::TILE_BYTES, xdo, tid);
    if (tid < C::TR) {
      float* ls = reinterpret_cast<float*>(base + 2 * C::TILE_BYTES);
      ls[tid] = xl;
      ls[C::TR + tid] = xd;
    }
  };
  // Scores S = Q K^T and dP = dO V^T of the tile in buffer `buf`, both 32-query halves (four
  // independent MFMA chains).
  auto scores2 = [&](int buf, f32x16(&sa)[2], f32x16(&dp)[2], int s0, int s1) {
    const char* qtile = smem + buf * BUF;
    const char* dotile = qtile + C::TILE_BYTES;
#pragma unroll
    for (int sub = s0; sub < s1; ++sub) {
      sa[sub] = f32x16{};
      dp[sub] = f32x16{};
    }
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
#pragma unroll
      for (int sub = s0; sub < s1; ++sub) {
        sa[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tile_row16<D>(qtile, 32 * sub + l32, 2 * s + hi), kf[s], sa[sub], 0, 0, 0);
        if constexpr (DO_DK)
          dp[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tile_row16<D>(dotile, 32 * sub + l32, 2 * s + hi), vf[s], dp[sub], 0, 0, 0);
      }
    }
  };
  // P and dS of the tile at query qt in buffer `buf` from its scores, then dV^T += dO^T P and
  // dK^T += Q^T dS. A half this wave does not see is masked to zero weights.
  auto grads = [&](int buf, int qt, const f32x16(&sa)[2], const f32x16(&dp)[2], int s0,
                   int s1) {
    const char* qtile = smem + buf * BUF;
    const char* dotile = qtile + C::TILE_BYTES;
    const float* lse_s = reinterpret_cast<const float*>(qtile + 2 * C::TILE_BYTES);
    const float* del_s = lse_s + C::TR;
#pragma unroll
    for (int sub = s0; sub < s1; ++sub) {
      const int qs = qt + 32 * sub;
      // Register r: query qs + acc_row(r); lane: key kw0 + l32.
      const bool all = block_all<MODE>(qs, kw0, T, window);
      float p[16], ds[16];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + 32 * sub + 8 * gq + 4 * hi);
        f32x4 d4 = f32x4{};
        if constexpr (DO_DK) d4 = *reinterpret_cast<const f32x4*>(del_s + 32 * sub + 8 * gq + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * gq + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(sa[sub][r], scale_log2, -l4[e]));
          if (!all) pr = visible_qk<MODE>(qs + acc_row(r, hi), key, T, window) ? pr : 0.f;
          p[r] = pr;
          if constexpr (DO_DK) ds[r] = pr * (dp[sub][r] - d4[e]);
        }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 pw, dw;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (DO_DV) pw[e] = pack_bf16x2(p[8 * tt + 2 * e], p[8 * tt + 2 * e + 1]);
          if constexpr (DO_DK) dw[e] = pack_bf16x2(ds[8 * tt + 2 * e], ds[8 * tt + 2 * e + 1]);
        }
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, dw);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          if constexpr (DO_DV)
            dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tile_tr16<D>(dotile, 32 * sub + 16 * tt, db, lane), pb, dva[db], 0, 0, 0);
          if constexpr (DO_DK)
            dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                tile_tr16<D>(qtile, 32 * sub + 16 * tt, db, lane), dsb, dka[db], 0, 0, 0);
        }
      }
    }
  };
  auto qt_of = [&](int i) { return qt0 + (i - (i / n_qt) * n_qt) * C::TR; };
  // A tile neither half of which this wave sees is skipped (wave-uniform).
  auto seen = [&](int i) {
    const int qt = qt_of(i);
    return (int)block_any<MODE>(qt, kw0, T, window) | (int)block_any<MODE>(qt + 32, kw0, T, window);
  };

  fetch(0);
  put(0);
  __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    // Tile i + 1's loads fly while tile i is used; they land in the other buffer, whose last
    // readers (tile i - 1) passed the barrier that ended the previous step.
    if (i + 1 < n_tiles) fetch(i + 1);
    if (seen(i)) {
      f32x16 sa[2], dp[2];
      if constexpr (PASS == kPassDK) {
        // one 32-query half at a time: the registers of a second half's S and dP are not there
        scores2(i & 1, sa, dp, 0, 1);
        grads(i & 1, qt_of(i), sa, dp, 0, 1);
        scores2(i & 1, sa, dp, 1, 2);
        grads(i & 1, qt_of(i), sa, dp, 1, 2);
      } else {
        scores2(i & 1, sa, dp, 0, 2);
        grads(i & 1, qt_of(i), sa, dp, 0, 2);
      }
    }
    if (i + 1 < n_tiles) put((i + 1) & 1);
    __syncthreads();
  }

  // Lane l holds key kw0 + l % 32; register r of block db holds d = 32 db + acc_row(r).
  if (key < T) {
    bf16* krow = dK + kvoff + (int64_t)key * geo.kv.t;
    bf16* vrow = dV + kvoff + (int64_t)key * geo.kv.t;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 wk, wv;
        wk[0] = pack_bf16x2(dka[db][4 * gq] * scale, dka[db][4 * gq + 1] * scale);
        wk[1] = pack_bf16x2(dka[db][4 * gq + 2] * scale, dka[db][4 * gq + 3] * scale);
        wv[0] = pack_bf16x2(dva[db][4 * gq], dva[db][4 * gq + 1]);
        wv[1] = pack_bf16x2(dva[db][4 * gq + 2], dva[db][4 * gq + 3]);
        if constexpr (DO_DK) *reinterpret_cast<u32x2*>(krow + 32 * db + 8 * gq + 4 * hi) = wk;
        if constexpr (DO_DV) *reinterpret_cast<u32x2*>(vrow + 32 * db + 8 * gq + 4 * hi) = wv;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// dQ (bf16 MFMA).
// ---------------------------------------------------------------------------------------------
template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_bwd_dq_bf16(
    const bf16* __restrict__ Q, const bf16* __restrict__ K, const bf16* __restrict__ V,
    const bf16* __restrict__ O, const bf16* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ Delta, bf16* __restrict__ dQ, Geometry geo, int BH, int T,
    int window_arg, float scale_log2, float scale, int nqb, int group_heads) {
  using C = BwdCfg<D>;
  // Two buffers, each: K tile, V tile.
  constexpr int BUF = 2 * C::TILE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  const int tid = (int)threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Same order as the dK/dV kernel, heaviest (last) query blocks first.
  int qr, bh;
  group_order((int)blockIdx.x, BH, nqb, group_heads, bh, qr);
  const int qb = nqb - 1 - qr;
  const int q0 = qb * 128, qw0 = q0 + 32 * wave, qi = qw0 + l32;
  const int q_rs = geo.q.t * 2, kv_rs = geo.kv.t * 2;
  const int64_t qoff = geo.q_head(bh), kvoff = geo.kv_head(bh);

  // Q^T and dO^T fragments (B operands): lane l holds row qi, elements 16 s + 8 (l / 32) .. + 8.
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(Q + qoff, T * q_rs);
  const __amdgpu_buffer_rsrc_t rdo = head_rsrc(dO + qoff, T * q_rs);
  bf16x8 qf[C::KS], dof[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const uint32_t off = (uint32_t)(qi * q_rs + 32 * s + 16 * hi);
    qf[s] = __builtin_bit_cast(bf16x8, buffer_load16(rq, off));
    dof[s] = __builtin_bit_cast(bf16x8, buffer_load16(rdo, off));
  }
  const float lse2 = (qi < T) ? LSE[(int64_t)bh * T + qi] * kLog2e : 0.f;
  // D_i = dO_i . O_i (fp32) from the lane's half of the row and its partner's (lane ^ 32), with
  // O read in dO's pattern; written for the dK/dV kernel, which runs after this one. Rows past T
  // read as zero and are not written.
  float dlt;
  {
    const __amdgpu_buffer_rsrc_t ro = head_rsrc(O + qoff, T * q_rs);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 ow = buffer_load16(ro, (uint32_t)(qi * q_rs + 32 * s + 16 * hi));
      const u32x4 dw = __builtin_bit_cast(u32x4, dof[s]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(bf16lo_to_f32(dw[e]), bf16lo_to_f32(ow[e]), part);
        part = fmaf(bf16hi_to_f32(dw[e]), bf16hi_to_f32(ow[e]), part);
      }
    }
    dlt = part + __shfl_xor(part, 32);
    if (qi < T && hi == 0) Delta[(int64_t)bh * T + qi] = dlt;
  }
  f32x16 dqa[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dqa[db] = f32x16{};

  int k_lo = 0, k_hi = T;
  if constexpr (MODE != kNonCausal) k_hi = min(T, q0 + 128);
  if constexpr (MODE == kCausalWindow) k_lo = max(0, q0 - window);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(K + kvoff, T * kv_rs);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(V + kvoff, T * kv_rs);

  const int kt0 = k_lo / C::TR * C::TR;
  const int n_tiles = (k_hi - kt0 + C::TR - 1) / C::TR;  // >= 1 for a block holding a query < T
  u32x4 xk[C::LPT], xv[C::LPT];
  auto put = [&](int buf) {
    store_tile<D>(smem + buf * BUF, xk, tid);
    store_tile<D>(smem + buf * BUF + C::TILE_BYTES, xv, tid);
  };
  if (n_tiles > 0) {
    load_tile<D>(xk, rk, kt0, kv_rs, tid);
    load_tile<D>(xv, rv, kt0, kv_rs, tid);
    put(0);
  }
  __syncthreads();
  for (int i = 0; i < n_tiles; ++i) {
    const int kt = kt0 + i * C::TR;
    if (i + 1 < n_tiles) {  // next tile in flight while this one is used (see the dK/dV kernel)
      load_tile<D>(xk, rk, kt + C::TR, kv_rs, tid);
      load_tile<D>(xv, rv, kt + C::TR, kv_rs, tid);
    }
    const char* ktile = smem + (i & 1) * BUF;
    const char* vtile = ktile + C::TILE_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ks = kt + 32 * kb;
      if (!block_any<MODE>(qw0, ks, T, window)) continue;  // wave-uniform
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tile_row16<D>(ktile, 32 * kb + l32, 2 * s + hi), qf[s], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tile_row16<D>(vtile, 32 * kb + l32, 2 * s + hi), dof[s], dpacc, 0, 0, 0);
      }
      // Register r: key ks + acc_row(r); lane: query qi.
      const bool all = block_all<MODE>(qw0, ks, T, window);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pr = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -lse2));
        if (!all) pr = visible_qk<MODE>(qi, ks + acc_row(r, hi), T, window) ? pr : 0.f;
        ds[r] = pr * (dpacc[r] - dlt);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        u32x4 dw;
#pragma unroll
        for (int e = 0; e < 4; ++e) dw[e] = pack_bf16x2(ds[8 * tt + 2 * e], ds[8 * tt + 2 * e + 1]);
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, dw);
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              tile_tr16<D>(ktile, 32 * kb + 16 * tt, db, lane), dsb, dqa[db], 0, 0, 0);
      }
    }
    if (i + 1 < n_tiles) put((i + 1) & 1);
    __syncthreads();
  }

  if (qi < T) {
    bf16* row = dQ + qoff + (int64_t)qi * geo.q.t;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 w;
        w[0] = pack_bf16x2(dqa[db][4 * gq] * scale, dqa[db][4 * gq + 1] * scale);
        w[1] = pack_bf16x2(dqa[db][4 * gq + 2] * scale, dqa[db][4 * gq + 3] * scale);
        *reinterpret_cast<u32x2*>(row + 32 * db + 8 * gq + 4 * hi) = w;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// fp32 path: every step in fp32. One thread per (row, 16-element chunk of d); each thread
// recomputes the scores of its row with every key (or query) it pairs with.
// ---------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ float dot_rows(const float* __restrict__ a, const float* __restrict__ b) {
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(a + c);
    const f32x4 y = *reinterpret_cast<const f32x4*>(b + c);
    acc = fmaf(x[0], y[0], acc);
    acc = fmaf(x[1], y[1], acc);
    acc = fmaf(x[2], y[2], acc);
    acc = fmaf(x[3], y[3], acc);
  }
  return acc;
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dQ, Geometry geo, int T, int window_arg, float scale, int n_threads) {
  constexpr int NC = D / 16;
  const int n = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (n >= n_threads) return;
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  const int c = n % NC, row = n / NC;
  const int bh = row / T, i = row % T;
  const float* q = Q + geo.q_head(bh) + (int64_t)i * geo.q.t;
  const float* dor = dO + geo.q_head(bh) + (int64_t)i * geo.q.t;
  const int64_t kvoff = geo.kv_head(bh);
  const float lse = LSE[(int64_t)bh * T + i], dlt = Delta[(int64_t)bh * T + i];
  float acc[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.f;
  int lo = 0, hi = T;
  if constexpr (MODE != kNonCausal) hi = i + 1;
  if constexpr (MODE == kCausalWindow) lo = max(0, i - window);
  for (int j = lo; j < hi; ++j) {
    const float* kr = K + kvoff + (int64_t)j * geo.kv.t;
    const float* vr = V + kvoff + (int64_t)j * geo.kv.t;
    const float p = expf(scale * dot_rows<D>(q, kr) - lse);
    const float ds = p * (dot_rows<D>(dor, vr) - dlt);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = fmaf(ds, kr[16 * c + e], acc[e]);
  }
  float* out = dQ + geo.q_head(bh) + (int64_t)i * geo.q.t + 16 * c;
#pragma unroll
  for (int e = 0; e < 16; ++e) out[e] = scale * acc[e];
}

template <int D, int MODE>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dK, float* __restrict__ dV, Geometry geo, int H_kv, int T, int window_arg,
    float scale, int n_threads) {
  constexpr int NC = D / 16;
  const int n = (int)blockIdx.x * 256 + (int)threadIdx.x;
  if (n >= n_threads) return;
  const int window = (MODE == kCausalWindow) ? window_arg : -1;
  const int c = n % NC, row = n / NC;
  const int bg = row / T, j = row % T;
  const int b = bg / H_kv, g = bg % H_kv;
  const int group = (int)geo.group.d, H = (int)geo.H.d;
  const int64_t kvoff = (int64_t)b * geo.kv.b + (int64_t)g * geo.kv.h;
  const float* kr = K + kvoff + (int64_t)j * geo.kv.t;
  const float* vr = V + kvoff + (int64_t)j * geo.kv.t;
  float ak[16], av[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) ak[e] = av[e] = 0.f;
  int lo = 0, hi = T;
  if constexpr (MODE != kNonCausal) lo = j;
  if constexpr (MODE == kCausalWindow) hi = min(T, j + window + 1);
  for (int hg = 0; hg < group; ++hg) {
    const int h = g * group + hg, bh = b * H + h;
    const int64_t qoff = (int64_t)b * geo.q.b + (int64_t)h * geo.q.h;
    for (int i = lo; i < hi; ++i) {
      const float* q = Q + qoff + (int64_t)i * geo.q.t;
      const float* dor = dO + qoff + (int64_t)i * geo.q.t;
      const float p = expf(scale * dot_rows<D>(q, kr) - LSE[(int64_t)bh * T + i]);
      const float ds = p * (dot_rows<D>(dor, vr) - Delta[(int64_t)bh * T + i]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        av[e] = fmaf(p, dor[16 * c + e], av[e]);
        ak[e] = fmaf(ds, q[16 * c + e], ak[e]);
      }
    }
  }
  float* ko = dK + kvoff + (int64_t)j * geo.kv.t + 16 * c;
  float* vo = dV + kvoff + (int64_t)j * geo.kv.t + 16 * c;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    ko[e] = scale * ak[e];
    vo[e] = av[e];
  }
}

// ---------------------------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------------------------
template <typename Elem, int D>
static hipError_t launch_delta_t(const void* out, const void* dout, float* delta, const Dims& dm,
                                 hipStream_t stream) {
  constexpr int L = D / (16 / (int)sizeof(Elem));
  constexpr int RPB = 256 / L;
  const int n_rows = dm.B * dm.H * dm.T;
  const unsigned grid = (unsigned)((n_rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((attn_bwd_delta_kernel<Elem, D>), dim3(grid), dim3(256), 0, stream,
                     (const Elem*)out, (const Elem*)dout, delta, make_geometry(dm),
                     make_fastdiv((uint32_t)dm.T), n_rows);
  return hipGetLastError();
}

// dQ first: its kernel also forms delta, which the dK/dV kernel reads.
template <int D, int MODE>
static hipError_t launch_bwd_bf16_t(const void* q, const void* k, const void* v, const void* out,
                                    const void* dout, const float* lse, float* delta, void* dq,
                                    void* dk, void* dv, const Dims& dm, int window,
                                    hipStream_t stream) {
  const Geometry geo = make_geometry(dm);
  const float scale = (float)(1.0 / sqrt((double)D));
  const float scale_log2 = (float)(1.4426950408889634 / sqrt((double)D));
  const int nkb = (dm.T + 127) / 128;
  const int gh = group_heads(dm.B * dm.H_kv, (int64_t)dm.T * D * 2 * 2);
  auto dkdv = [&](auto pass_c) {
    constexpr int PASS = decltype(pass_c)::value;
    hipLaunchKernelGGL((attn_bwd_dkdv_bf16<D, MODE, PASS>),
                       dim3((unsigned)(dm.B * dm.H_kv * nkb)), dim3(256), 0, stream,
                       (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse,
                       delta, (bf16*)dk, (bf16*)dv, geo, dm.H_kv, dm.T, window, scale_log2, scale,
                       nkb, gh);
    return hipGetLastError();
  };
  const int BH = dm.B * dm.H;
  hipLaunchKernelGGL((attn_bwd_dq_bf16<D, MODE>), dim3((unsigned)(BH * nkb)), dim3(256), 0,
                     stream, (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)out,
                     (const bf16*)dout, lse, delta, (bf16*)dq, geo, BH, dm.T, window, scale_log2,
                     scale, nkb, group_heads(BH, (int64_t)dm.T * D * 2 * 2));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D <= 64) {
    e = dkdv(std::integral_constant<int, kBothPasses>{});
  } else {
    e = dkdv(std::integral_constant<int, kPassDV>{});
    if (e == hipSuccess) e = dkdv(std::integral_constant<int, kPassDK>{});
  }
  return e;
}

template <int D, int MODE>
static hipError_t launch_bwd_f32_t(const void* q, const void* k, const void* v, const void* dout,
                                   const float* lse, const float* delta, void* dq, void* dk,
                                   void* dv, const Dims& dm, int window, hipStream_t stream) {
  const Geometry geo = make_geometry(dm);
  const float scale = (float)(1.0 / sqrt((double)D));
  // Thread counts fit in int (checked by the entry point); the grids are formed in 64 bits so
  // that rounding up to whole workgroups cannot overflow.
  const int nq = dm.B * dm.H * dm.T * (D / 16), nk = dm.B * dm.H_kv * dm.T * (D / 16);
  const int64_t gq = ((int64_t)nq + 255) / 256, gk = ((int64_t)nk + 255) / 256;
  hipLaunchKernelGGL((attn_bwd_dq_f32<D, MODE>), dim3((unsigned)gq), dim3(256), 0,
                     stream, (const float*)q, (const float*)k, (const float*)v,
                     (const float*)dout, lse, delta, (float*)dq, geo, dm.T, window, scale, nq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_f32<D, MODE>), dim3((unsigned)gk), dim3(256),
                     0, stream, (const float*)q, (const float*)k, (const float*)v,
                     (const float*)dout, lse, delta, (float*)dk, (float*)dv, geo, dm.H_kv, dm.T,
                     window, scale, nk);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, float* delta, void* dq,
                               void* dk, void* dv, const Dims& dm, int window, int causal,
                               int dtype, hipStream_t stream) {
  if constexpr (D < 32) {
    if (dtype == 0) return hipErrorInvalidValue;  // bf16 needs d >= 32 (32-wide MFMA tiles)
  }
  // bf16: the dQ kernel forms delta itself; fp32: the delta kernel runs first.
  if (dtype != 0) {
    const hipError_t e = launch_delta_t<float, D>(out, dout, delta, dm, stream);
    if (e != hipSuccess) return e;
  }
  // A window of T - 1 or more hides nothing: run it as plain causal (as the forward does).
  const int mode = !causal ? kNonCausal
                           : ((window >= 0 && window < dm.T - 1) ? kCausalWindow : kCausal);
#define ATTN_BWD_CASE(M)                                                                        \
  if (mode == M) {                                                                              \
    if constexpr (D >= 32) {                                                                    \
      if (dtype == 0)                                                                           \
        return launch_bwd_bf16_t<D, M>(q, k, v, out, dout, lse, delta, dq, dk, dv, dm, window,  \
                                       stream);                                                 \
    }                                                                                           \
    return launch_bwd_f32_t<D, M>(q, k, v, dout, lse, delta, dq, dk, dv, dm, window, stream);   \
  }
  ATTN_BWD_CASE(kNonCausal)
  ATTN_BWD_CASE(kCausal)
  ATTN_BWD_CASE(kCausalWindow)
#undef ATTN_BWD_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, float* delta, void* dq, void* dk,
                           void* dv, const Dims& dm, int window, int causal, int dtype,
                           hipStream_t stream) {
  switch (dm.d) {
    case 32: return launch_bwd_d<32>(q, k, v, out, dout, lse, delta, dq, dk, dv, dm, window, causal, dtype, stream);
    case 64: return launch_bwd_d<64>(q, k, v, out, dout, lse, delta, dq, dk, dv, dm, window, causal, dtype, stream);
    case 128: return launch_bwd_d<128>(q, k, v, out, dout, lse, delta, dq, dk, dv, dm, window, causal, dtype, stream);
    default: break;
  }
  if (dtype == 1 && dm.d == 16)
    return launch_bwd_d<16>(q, k, v, out, dout, lse, delta, dq, dk, dv, dm, window, causal, dtype, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
