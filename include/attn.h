/*
 * attn.h — C ABI of libattn.so: QK-RMSNorm + RoPE + causal / sliding-window attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (page title, then the part of the page):
 *   [HABR] "Подробный технический разбор реализации Autoresearch, ИИ-исследователя Андрея
 *          Карпаты" (habr.com, article 1010198), its train.py listing: `norm`,
 *          `apply_rotary_emb`, `GPT._precompute_rotary_embeddings`,
 *          `GPT._compute_window_sizes`, `CausalSelfAttention.forward`.
 *   [GEOM] "Projeção em um Subespaço de Consulta" (unhomeschool.com, geometry_of_andrea),
 *          sections "O que a Atenção Calcula", "A Máscara Causal", "Escalonamento por sqrt(d_k)".
 *
 * Conventions for every entry point:
 *   - Tensors are dense and contiguous. The entry points without a suffix take row-major
 *     [B][H][T][d] (batch, head, token, channel) tensors whose k and v have as many heads as q.
 *     Their _ex variants add H_kv and layout: q and out are [B, H, T, d], k and v [B, H_kv, T, d]
 *     with H_kv dividing H (grouped-query attention: q head h attends with kv head
 *     h / (H / H_kv)), all stored in the order that layout names (attn_layout). lse is always
 *     [B][H][T]. The call without a suffix equals its _ex variant with H_kv = H and
 *     ATTN_LAYOUT_BHTD.
 *   - Pointers named as device pointers must point to device memory of the current HIP device;
 *     the caller allocates and frees all of them. The library allocates no memory, keeps no
 *     mutable global state beyond a per-device cache of how many workgroups the GPU holds at
 *     once, never synchronises the host, and is safe to call from several threads (the calls
 *     are ordered only by the stream the caller passes).
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream. Work is only
 *     enqueued: results are ready once that stream has been synchronised.
 *   - Every entry point validates its arguments before making any HIP call and returns one of the
 *     ATTN_* codes below; on an error no work is enqueued. A kernel fault is not reported by the
 *     call that launched it but by the caller's next synchronisation of the stream.
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage order of q, k, v and out in the _ex entry points. */
typedef enum attn_layout {
  ATTN_LAYOUT_BHTD = 0, /* [B][H][T][d]: each head's rows are contiguous */
  ATTN_LAYOUT_BTHD = 1  /* [B][T][H][d]: the order the projections produce in [HABR]
                           `CausalSelfAttention.forward` (q, k, v viewed as (B, T, heads, d)
                           before the attention call); row stride H * d (H_kv * d for k, v) */
} attn_layout;

/* Element type of q, k, v and out (the prologue and attention compute in fp32 internally). */
typedef enum attn_dtype {
  ATTN_BF16 = 0, /* bfloat16; matrix products on bf16 MFMA with fp32 accumulation */
  ATTN_F32 = 1   /* float32; all arithmetic in fp32 */
} attn_dtype;

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* B, H, H_kv or T < 1, H_kv not dividing H, or a tensor too large */
  ATTN_ERR_HEAD_DIM = 3,    /* head dim d not supported for this entry point and dtype */
  ATTN_ERR_DTYPE = 4,       /* dtype is not an attn_dtype value */
  ATTN_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_WINDOW = 6,      /* causal is not 0/1, or causal == 0 with window >= 0 */
  ATTN_ERR_ALIAS = 7,       /* out or lse overlaps an input it must not overlap */
  ATTN_ERR_ARG = 8,         /* another argument is out of range (eps, base, pattern, n_layer,
                               layout) */
  ATTN_ERR_HIP = 9,         /* the HIP runtime refused the launch */
  ATTN_ERR_SCRATCH = 10     /* an allocation-free call needs more scratch than the library's
                               fixed device array (ATTN_DECODE_SCRATCH_BYTES) holds */
};

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_strerror(int code);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int attn_version(void);

/*
 * Per-layer attention windows of a layer pattern such as "SSSL" ([HABR]
 * `GPT._compute_window_sizes`): layer l uses pattern[l % len(pattern)]; 'L' is T (full causal)
 * and 'S' is T / 2 (integer division); the last layer is always 'L'. Letters are
 * case-insensitive.
 *   T          sequence length, >= 1
 *   n_layer    number of layers, >= 1
 *   pattern    NUL-terminated, non-empty, only 'S'/'L' (either case)
 *   windows    HOST pointer to n_layer ints, written on success
 * Host-only: makes no HIP call.
 */
int attn_sssl_windows(int T, int n_layer, const char* pattern, int* windows);

/*
 * RoPE tables ([HABR] `GPT._precompute_rotary_embeddings`): for t < T and j < d/2,
 * theta = t * base^(-2j/d), cos_tab[t][j] = cos(theta), sin_tab[t][j] = sin(theta).
 * The angles and their cosines and sines are computed in fp64 on the device and rounded to fp32.
 *   cos_tab, sin_tab   DEVICE pointers to fp32 [T][d/2], written
 *   T >= 1; d even with 2 <= d <= 256; base > 1
 */
int attn_rope_table(float* cos_tab, float* sin_tab, int T, int d, double base, void* stream);

/*
 * QK-norm then RoPE on q and k ([HABR] `norm`, `apply_rotary_emb` and their use in
 * `CausalSelfAttention.forward`). For every row x (one token of one head) of q and of k:
 *   r = 1 / sqrt(mean_j x_j^2 + eps), x <- r * x                       (weightless RMSNorm)
 *   with h = d/2 and position t (the row's token index):
 *   y_j     =  x_j * cos[t][j] + x_{j+h} * sin[t][j]
 *   y_{j+h} = -x_j * sin[t][j] + x_{j+h} * cos[t][j]                   (half-split rotation)
 * The rotation preserves the row's sum of squares, so normalising before or after it gives the
 * same result. Arithmetic is fp32; bf16 outputs are rounded to nearest even.
 *   q, k            DEVICE [B][H][T][d] of dtype, read
 *   q_out, k_out    DEVICE [B][H][T][d] of dtype, written; q_out may equal q and k_out may equal
 *                   k (in place); any other overlap is ATTN_ERR_ALIAS
 *   q and q_out may both be NULL: then only k is processed (one of them NULL is ATTN_ERR_NULL)
 *   cos_tab, sin_tab DEVICE fp32 [T][d/2] from attn_rope_table (only rows t < T are read)
 *   d in {16, 32, 64, 128}; eps >= 0 and finite
 */
int attn_qknorm_rope(const void* q, const void* k, void* q_out, void* k_out,
                     const float* cos_tab, const float* sin_tab,
                     int B, int H, int T, int d, float eps, int dtype, void* stream);

/*
 * Attention forward ([GEOM] "O que a Atenção Calcula", "Escalonamento por sqrt(d_k)",
 * "A Máscara Causal"; window as in [HABR] `CausalSelfAttention.forward`, which calls the
 * attention kernel with window_size = (W, 0)):
 *   s_ij   = q_i . k_j / sqrt(d)
 *   A(i)   = { j : j <= i and (window < 0 or i - j <= window) }   if causal == 1
 *            { all j < T }                                        if causal == 0
 *   lse_i  = ln sum_{j in A(i)} exp(s_ij)                         (natural log, fp32)
 *   out_i  = sum_{j in A(i)} exp(s_ij - lse_i) v_j
 * A(i) is never empty. window >= T - 1 is the same as window = -1 (full causal).
 *   q, k, v   DEVICE [B][H][T][d] of dtype, read
 *   out       DEVICE [B][H][T][d] of dtype, written; must not overlap q, k, v or lse
 *   lse       DEVICE fp32 [B][H][T], written; may be NULL (then not written)
 *   window    -1 = unlimited, >= 0 = causal band width (keys i-window .. i)
 *   causal    1 = causal mask, 0 = every key visible (requires window == -1)
 *   d         dtype ATTN_BF16: {32, 64, 128}; ATTN_F32: {16, 32, 64, 128}
 * bf16: q k^T and P v run on bf16 MFMA with fp32 accumulation; the softmax is fp32 and the
 * probabilities are rounded to bf16 (nearest even) before the P v product; out is rounded to
 * nearest even. f32: every step in fp32.
 * Results do not depend on the order in which the kernels take (head, query block) items: the
 * environment variable ATTN_ITEM_ORDER=snake (read at each call) replaces the bf16 d <= 64
 * kernels' head-grouped order with the snake order, for comparison, with bitwise the same
 * outputs.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
             int B, int H, int T, int d, int window, int causal, int dtype, void* stream);

/*
 * Attention forward whose kernel applies QK-norm and RoPE to q itself as it loads each block of
 * q rows (the normalised q is never written to memory); k must already be normalised and
 * rotated (attn_qknorm_rope with q = NULL, or the k_work of attn_fwd_qknorm), e.g. a layer's
 * cached keys. Result: attn_fwd(RoPE(RMSNorm(q)), k, v) with lse and out as in attn_fwd.
 * The softmax runs without a running maximum: a normalised, rotated q row has Euclidean norm
 * <= sqrt(d), so every score q.k/sqrt(d) lies within |k_j| of 0, and exp of it stays far inside
 * the fp32 and bf16 ranges for every row of k with Euclidean norm <= 2 sqrt(d) (normalised rows
 * have norm <= sqrt(d)). Rows of k beyond that bound are outside this entry point's contract.
 *   q                DEVICE [B][H][T][d] bf16, read (before norm and rotation)
 *   k                DEVICE [B][H][T][d] bf16, read (after norm and rotation)
 *   v, out, lse      as in attn_fwd; out must not overlap q, k or v
 *   cos_tab, sin_tab DEVICE fp32 [T][d/2] from attn_rope_table
 *   eps              >= 0 and finite, as in attn_qknorm_rope
 *   window, causal   as in attn_fwd
 *   d in {32, 64, 128}; dtype must be ATTN_BF16 (else ATTN_ERR_DTYPE)
 * Rounding differs from attn_qknorm_rope + attn_fwd in one place: q's normalised, rotated row is
 * multiplied by log2(e)/sqrt(d) in fp32 before its one rounding to bf16.
 */
int attn_fwd_qnorm(const void* q, const void* k, const void* v, void* out, float* lse,
                   const float* cos_tab, const float* sin_tab, int B, int H, int T, int d,
                   float eps, int window, int causal, int dtype, void* stream);

/*
 * One attention layer of [HABR] `CausalSelfAttention.forward` after the projections: QK-norm
 * and RoPE on q and k, then attention, i.e. the result of attn_qknorm_rope followed by attn_fwd.
 * It runs as attn_qknorm_rope(NULL, k, NULL, k_work, ...) followed by
 * attn_fwd_qnorm(q, k_work, v, ...): the normalised q is never written to memory. Both
 * normalised rows have Euclidean norm <= sqrt(d), so every score q.k/sqrt(d) lies in
 * [-sqrt(d), sqrt(d)] and the softmax runs without a running maximum or rescaling.
 *   q, k, v          DEVICE [B][H][T][d] bf16, read (q and k before norm and rotation)
 *   k_work           DEVICE [B][H][T][d] bf16, written with RoPE(RMSNorm(k)) (the caller may
 *                    keep it, e.g. as the layer's keys); may equal k (normalised in place);
 *                    any other overlap with q, k, v, out or lse is ATTN_ERR_ALIAS.
 *                    NULL (d in {32, 64} only, else ATTN_ERR_NULL): the layer runs as one
 *                    launch that RMS-normalises and rotates each key tile in on-chip memory as
 *                    it streams in, and the normalised k is written nowhere
 *   out, lse         as in attn_fwd; out must not overlap q, k, v or k_work
 *   cos_tab, sin_tab DEVICE fp32 [T][d/2] from attn_rope_table
 *   eps              >= 0 and finite, as in attn_qknorm_rope
 *   window, causal   as in attn_fwd
 *   d in {32, 64, 128}; dtype must be ATTN_BF16 (else ATTN_ERR_DTYPE)
 * Rounding differs from attn_qknorm_rope + attn_fwd in one place: q's normalised, rotated row is
 * multiplied by log2(e)/sqrt(d) in fp32 before its one rounding to bf16. With k_work NULL the
 * keys' rotation angles are also formed in the kernel in fp32 (t times the frequency that row 1
 * of the tables gives, reduced to one turn; at d = 64 consecutive key tiles advance the previous
 * tile's cos and sin by the rotation of 64 positions), which moves a rotated key by up to about
 * 2e-4 of its norm against the table's angles for T below 8192, and a key row's RMS uses the
 * hardware reciprocal square root (about 1 ulp) before the row's one rounding to bf16.
 */
int attn_fwd_qknorm(const void* q, const void* k, const void* v, void* k_work, void* out,
                    float* lse, const float* cos_tab, const float* sin_tab, int B, int H, int T,
                    int d, float eps, int window, int causal, int dtype, void* stream);

/*
 * Grouped-query and [B][T][H][d] variants of the four entry points above ([HABR] `GPTConfig`
 * and `CausalSelfAttention`: n_kv_head key/value heads, n_kv_head dividing n_head, each shared
 * by a group of n_head / n_kv_head query heads; q, k, v viewed in the (B, T, heads, d) order of
 * the projections before the attention call). Arguments, rules and
 * results are those of the entry point without the suffix, with these differences:
 *   H_kv     heads of k, v (and k_out, k_work); H_kv >= 1 and H % H_kv == 0, else
 *            ATTN_ERR_SHAPE. q, out and q_out have H heads; lse is [B][H][T].
 *   layout   an attn_layout value (else ATTN_ERR_ARG); every tensor argument except lse, cos_tab
 *            and sin_tab is stored in that order.
 * Query head h of batch b attends with kv head h / (H / H_kv) of batch b. The attn_qknorm_rope_ex
 * prologue normalises and rotates the B*H rows of q and the B*H_kv rows of k per position.
 * The bf16 attention kernels address one head's rows through 32-bit byte offsets: for
 * ATTN_BF16, (T + 128) * (largest row stride in bytes) must be below 2^31, else ATTN_ERR_SHAPE
 * (row stride: d * 2 for ATTN_LAYOUT_BHTD, H * d * 2 for q and H_kv * d * 2 for k, v in
 * ATTN_LAYOUT_BTHD). Every entry point also needs H * d < 2^24, else ATTN_ERR_SHAPE.
 */
int attn_qknorm_rope_ex(const void* q, const void* k, void* q_out, void* k_out,
                        const float* cos_tab, const float* sin_tab, int B, int H, int H_kv, int T,
                        int d, int layout, float eps, int dtype, void* stream);
int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, float* lse, int B, int H,
                int H_kv, int T, int d, int layout, int window, int causal, int dtype,
                void* stream);
int attn_fwd_qnorm_ex(const void* q, const void* k, const void* v, void* out, float* lse,
                      const float* cos_tab, const float* sin_tab, int B, int H, int H_kv, int T,
                      int d, int layout, float eps, int window, int causal, int dtype,
                      void* stream);
int attn_fwd_qknorm_ex(const void* q, const void* k, const void* v, void* k_work, void* out,
                       float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                       int H_kv, int T, int d, int layout, float eps, int window, int causal,
                       int dtype, void* stream);

/*
 * Value-embedding gate ([HABR] `CausalSelfAttention.forward`, the value-residual step of layers
 * that have a value embedding): every row of v gets its embedding row added with a gate,
 *   v'[b][h][t][:] = v[b][h][t][:] + 2 sigmoid(z[b][h][t]) * ve[b][h][t][:]
 * one gate per (batch, kv head, token), in (0, 2), 1 at z = 0. z is the output of the listing's
 * `ve_gate` linear layer (a projection, outside this library), the gate logits.
 *   v, ve        DEVICE, [B][H_kv][T][d] (ATTN_LAYOUT_BHTD) or [B][T][H_kv][d] (ATTN_LAYOUT_BTHD),
 *                16-byte aligned, dtype elements (read)
 *   gate_logits  DEVICE, dtype elements, [B][H_kv][T] beside ATTN_LAYOUT_BHTD tensors and
 *                [B][T][H_kv] beside ATTN_LAYOUT_BTHD ones (read)
 *   v_out        DEVICE, v's shape (written); may be v itself (in place); any other overlap with
 *                v, ve or gate_logits is ATTN_ERR_ALIAS
 *   d in {16, 32, 64, 128}; dtype ATTN_BF16 or ATTN_F32
 * Arithmetic is fp32 (one rounding of each output for bf16). HBM-bound: reads v, ve and the
 * logits, writes v_out.
 */
int attn_value_gate_ex(const void* v, const void* ve, const void* gate_logits, void* v_out, int B,
                       int H_kv, int T, int d, int layout, int dtype, void* stream);

/*
 * attn_fwd_qknorm_ex for a layer with a value embedding: the k-only QK-norm + RoPE kernel also
 * writes v_work = the gated v (attn_value_gate_ex's rows, in the same launch), then the attention
 * kernel reads q, k_work and v_work. Arguments as in attn_fwd_qknorm_ex and attn_value_gate_ex;
 * v_work (written, v's shape) may be v itself. k_work and v_work overlap nothing else that the call
 * reads or writes, and out and lse overlap none of the inputs (ATTN_ERR_ALIAS). bf16 only.
 */
int attn_fwd_qknorm_ve_ex(const void* q, const void* k, const void* v, const void* ve,
                          const void* gate_logits, void* k_work, void* v_work, void* out,
                          float* lse, const float* cos_tab, const float* sin_tab, int B, int H,
                          int H_kv, int T, int d, int layout, float eps, int window, int causal,
                          int dtype, void* stream);

/*
 * Backward pass of attn_fwd / attn_fwd_ex: the gradients of sum(dout * out) with respect to q, k
 * and v ([HABR] the training step's `loss.backward()` through `CausalSelfAttention.forward`; the
 * gradients are the exact derivatives of the attn_fwd definition). With c = 1/sqrt(d) and
 * P_ij = exp(c q_i . k_j - lse_i) on the visible set A(i) (0 elsewhere):
 *   delta_i = dout_i . out_i
 *   dv_j = sum_i P_ij dout_i
 *   dS_ij = P_ij (dout_i . v_j - delta_i)
 *   dq_i = c sum_j dS_ij k_j,    dk_j = c sum_i dS_ij q_i
 * With H_kv < H a kv head's dk, dv sum over the query heads of its group.
 *   q, k, v, out, lse   what attn_fwd(_ex) was given and returned (lse is required here)
 *   dout                DEVICE, q's shape and dtype: the gradient of out
 *   delta               DEVICE fp32 [B][H][T], written (a by-product the caller allocates)
 *   dq                  DEVICE, q's shape and dtype, written
 *   dk, dv              DEVICE, k's shape and dtype, written
 *   window, causal, B, H, H_kv, T, d, layout, dtype   as in attn_fwd_ex (attn_bwd: H_kv = H,
 *                       ATTN_LAYOUT_BHTD)
 * No output (dq, dk, dv, delta) may overlap an input or another output (ATTN_ERR_ALIAS).
 * bf16: S, dP and the four products run on bf16 MFMA with fp32 accumulation; P and dS are
 * recomputed in fp32 and rounded to bf16 (nearest even) for the products; dq, dk, dv are rounded
 * to bf16 once. f32: every step in fp32. Deterministic: no atomics, fixed summation order.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int T,
             int d, int window, int causal, int dtype, void* stream);
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H,
                int H_kv, int T, int d, int layout, int window, int causal, int dtype,
                void* stream);

/*
 * Backward of attn_qknorm_rope(_ex) ([HABR] `norm` and `apply_rotary_emb`): for each raw row x
 * with r = 1/sqrt(mean_j x_j^2 + eps) and x^ = r x, given dy (the gradient of the normalised,
 * rotated row), g = the rotation of dy by the opposite angle
 *   g_j = dy_j cos[t][j] - dy_{j+h} sin[t][j],   g_{j+h} = dy_j sin[t][j] + dy_{j+h} cos[t][j]
 * and dx = r (g - x^ mean_j(g_j x^_j)).
 *   q, k            DEVICE, the raw rows the forward prologue was given (read)
 *   dq_in, dk_in    DEVICE, gradients of the prologue's outputs (read)
 *   dq_out, dk_out  DEVICE, gradients of q and k (written); dq_out may equal dq_in and dk_out
 *                   dk_in (in place); any other overlap is ATTN_ERR_ALIAS
 *   q, dq_in and dq_out may all be NULL: then only k's rows are processed (some but not all of
 *   them NULL is ATTN_ERR_NULL)
 *   cos_tab, sin_tab, eps, d, dtype and the shape arguments as in attn_qknorm_rope(_ex)
 * Arithmetic is fp32; bf16 outputs are rounded to nearest even.
 */
int attn_qknorm_rope_bwd(const void* q, const void* k, const void* dq_in, const void* dk_in,
                         void* dq_out, void* dk_out, const float* cos_tab, const float* sin_tab,
                         int B, int H, int T, int d, float eps, int dtype, void* stream);
int attn_qknorm_rope_bwd_ex(const void* q, const void* k, const void* dq_in, const void* dk_in,
                            void* dq_out, void* dk_out, const float* cos_tab,
                            const float* sin_tab, int B, int H, int H_kv, int T, int d,
                            int layout, float eps, int dtype, void* stream);

/*
 * Backward of attn_value_gate_ex: given dv (the gradient of the gated rows v'), with
 * g = 2 sigmoid(z),
 *   dve = g * dv,   dgate_logits = g (1 - g / 2) * sum_j ve_j dv_j   (one per row)
 * and the gradient of v is dv itself (not written). ve, gate_logits, shapes, layout and dtype as
 * in attn_value_gate_ex; dv is v's shape (read); dve (written, v's shape) may be dv itself;
 * dgate_logits (written, gate_logits' shape) overlaps nothing else (ATTN_ERR_ALIAS). Arithmetic
 * is fp32; bf16 outputs are rounded to nearest even.
 */
int attn_value_gate_bwd_ex(const void* ve, const void* gate_logits, const void* dv, void* dve,
                           void* dgate_logits, int B, int H_kv, int T, int d, int layout,
                           int dtype, void* stream);

/*
 * Decode: one generation step ([GEOM] "A Máscara Causal": inference runs the same masked forward
 * as training; generation appends one token at a time). For every (batch b, head h) the newest
 * token's query q[b][h] (already normalised and rotated, like the rows attn_fwd takes) attends
 * to the cached keys and values of its batch entry, n_b = lengths[b] tokens with its own key and
 * value at position n_b - 1: keys j with max(0, n_b - 1 - window) <= j < n_b (window = -1: all
 * n_b), i.e. the last row of attn_fwd over the prefix:
 *   out[b][h] = sum_j softmax_j(q . k_j / sqrt(d)) v_j,   lse[b][h] = ln sum_j exp(q . k_j / sqrt(d))
 *   q, out           DEVICE [B][H][d] of dtype (read / written)
 *   k_cache, v_cache DEVICE [B][H_kv][S][d] (ATTN_LAYOUT_BHTD) or [B][S][H_kv][d]
 *                    (ATTN_LAYOUT_BTHD) of dtype, S = the cache's capacity; slots past n_b unread
 *   lengths          DEVICE int32 [B]: n_b, clamped to [1, S] on the device; NULL: every n_b = S
 *   lse              DEVICE fp32 [B][H], written; may be NULL
 *   workspace        DEVICE scratch of at least attn_decode_workspace_bytes(B, H, S, d, window)
 *                    bytes (16-byte aligned), owned by the caller; its contents may be
 *                    overwritten (shapes with one key split per head leave it untouched) and
 *                    calls that share one workspace must be ordered on one stream
 *   window           -1 or >= 0 (else ATTN_ERR_WINDOW)
 *   d, dtype         ATTN_BF16: {32, 64, 128}; ATTN_F32: {16, 32, 64, 128}
 * Scores, weights and sums are fp32 for both dtypes (the weights are not rounded); out is
 * rounded once. No written buffer may overlap another argument's buffer (ATTN_ERR_ALIAS); a
 * workspace below the required size is ATTN_ERR_ARG. attn_decode is attn_decode_ex with
 * H_kv = H and ATTN_LAYOUT_BHTD.
 * attn_decode_workspace_bytes returns the size, or -1 for B, H, S < 1, d outside [1, 256] or
 * window < -1; it is host-only.
 */
long long attn_decode_workspace_bytes(int B, int H, int S, int d, int window);
int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* lengths,
                void* out, float* lse, void* workspace, long long workspace_bytes, int B, int H,
                int S, int d, int window, int dtype, void* stream);
int attn_decode_ex(const void* q, const void* k_cache, const void* v_cache, const int* lengths,
                   void* out, float* lse, void* workspace, long long workspace_bytes, int B,
                   int H, int H_kv, int S, int d, int layout, int window, int dtype, void* stream);

/*
 * attn_decode_ex for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * results, with the split partials in a fixed device array of ATTN_DECODE_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends, instead of a caller workspace.
 * It calls no hipMalloc, hipFree or allocating routine. Arguments, errors and results are those
 * of attn_decode_ex without workspace / workspace_bytes; a shape whose
 * attn_decode_workspace_bytes exceeds ATTN_DECODE_SCRATCH_BYTES is ATTN_ERR_SCRATCH (nothing is
 * enqueued). Every call on a GPU shares that GPU's array: calls that may overlap on one GPU
 * (different streams, or threads without ordering) race and must be serialised by the caller,
 * e.g. by issuing them on one stream. Nothing needs clearing between calls: each call writes
 * every slot it later reads. The first call on a device looks up the array's address
 * (hipGetSymbolAddress) and keeps it.
 */
#define ATTN_DECODE_SCRATCH_BYTES (8LL << 20)
int attn_decode_noalloc_ex(const void* q, const void* k_cache, const void* v_cache,
                           const int* lengths, void* out, float* lse, int B, int H, int H_kv,
                           int S, int d, int layout, int window, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
