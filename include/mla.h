/*
 * mla.h -- C ABI of the MI355X (gfx950) multi-head latent attention library.
 *
 * The library computes one attention layer of multi-head latent attention (MLA):
 * keys and values are jointly compressed into a low-rank latent c = W_DKV x, and only
 * that latent (plus, for the decoupled form, one rotary key k_R shared by all heads)
 * is cached.  Three families are supported, each as defined on one of the pages:
 *
 *   MLA_ROPE_DECOUPLED_INTERLEAVED -- bird-of-paradise/deepseek-mla ``src/mla.py``,
 *       ``MultiHeadLatentAttention.forward``: query latent c_Q = W_DQ x,
 *       q_C = W_UQ c_Q, q_R = RoPE(W_QR c_Q); cached c = W_DKV x and
 *       k_R = RoPE(W_KR x); keys [W_UK c ; k_R], values W_UV c;
 *       scale 1/sqrt(d_nope + d_rope).  RoPE pairs (2j, 2j+1) (``apply_rotary_emb``).
 *   MLA_ROPE_FULL_HALFSPLIT -- frankenstein-transformer ``latent/mla_attn``,
 *       ``MLAAttention.forward``: q = RoPE(W_Q x), k = RoPE(W_UK c), v = W_UV c,
 *       scale 1/sqrt(d_nope).  RoPE pairs (j, j + d/2) (``_apply_rope``).
 *   MLA_ROPE_NONE with n_latent_heads = L > 1 -- frankenstein-transformer
 *       ``latent/mlra_attn``, ``MLRAAttention.forward``: the latent is L disjoint
 *       blocks; query head h reads block g = h / (n_heads / L) through its own
 *       block up-projections; q = W_Q x; no RoPE; scale 1/sqrt(d_nope).
 *
 * Every row computes causal softmax attention (query at position p sees keys at
 * positions <= p), then y = W_O [o_1; ...; o_H].
 *
 * Citations below name a page by tag and a section of it by function or class:
 *   [MLA page]  frankenstein-transformer docs, ``latent/mla_attn``
 *   [MLRA page] frankenstein-transformer docs, ``latent/mlra_attn``
 *   [DSV2 page] bird-of-paradise/deepseek-mla, ``src/mla.py``
 * Every entry point's comment names its source passage, or says that it is the library's own.
 *
 * Conventions for every entry point:
 *   - Weights are row-major [out_features][in_features] (torch.nn.Linear layout) in
 *     the element type of dims->dtype.  MLRA up-projections w_uk / w_uv are L dense
 *     blocks [n_heads*d_nope/L][r_kv/L] stored back to back.
 *   - Activations x are row-major in dims->dtype; outputs y are float32.
 *   - All pointers named *_dev or pointing at tensors are device pointers (hipMalloc
 *     or torch CUDA tensors).  The caller owns every buffer; the library never
 *     allocates, frees or keeps a pointer after returning.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     stream-ordered and asynchronous: no host synchronisation happens inside.
 *   - Host-visible argument errors are reported before anything is launched; a
 *     failed launch returns MLA_ERR_HIP.  Device-side lengths (start_pos_dev,
 *     ctx_len_dev) are trusted to respect the host bounds passed beside them.
 *   - Work on one workspace must not overlap in time (two streams using the same
 *     workspace race).  Inputs, outputs, caches and workspaces must not alias.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad enum */
  MLA_ERR_SHAPE = 2,         /* dimension rules of the pages violated (odd RoPE dim, L not dividing r_kv or n_heads) */
  MLA_ERR_CAPACITY = 3,      /* batch or positions exceed the cache's max_batch / max_seq */
  MLA_ERR_UNSUPPORTED = 4,   /* valid MLA, but outside what the kernels implement (listed per entry point) */
  MLA_ERR_WORKSPACE = 5,     /* workspace pointer missing or smaller than mla_workspace_bytes() */
  MLA_ERR_HIP = 6            /* a HIP runtime call or kernel launch failed */
} mla_status;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype;

typedef enum {
  MLA_ROPE_NONE = 0,
  MLA_ROPE_DECOUPLED_INTERLEAVED = 1,
  MLA_ROPE_FULL_HALFSPLIT = 2
} mla_rope_mode;

typedef enum {
  MLA_OP_CACHE_APPEND = 0,
  MLA_OP_PREFILL = 1,
  MLA_OP_DECODE = 2,
  MLA_OP_DECODE_ATTENTION = 3,
  MLA_OP_PREFILL_ATTENTION = 4,
  MLA_OP_PREFILL_CHUNK = 5
} mla_op;

/* Layer dimensions.
 *   d_model        input / output width
 *   n_heads        H, query heads
 *   d_nope         per-head query/key width of the decompressed part (head_dim)
 *   d_v            per-head value width; must equal d_nope (all pages use one head_dim)
 *   d_rope         decoupled rotary width (DECOUPLED only; 0 otherwise); even
 *   r_kv           latent rank (total over all latent heads)
 *   r_q            query latent rank; 0 = queries straight from x through w_q
 *                  (and, for DECOUPLED, q_R through w_qr applied to x)
 *   n_latent_heads L (1 = MLA); L > 1 requires MLA_ROPE_NONE, L | r_kv and L | n_heads
 *   rope_mode      mla_rope_mode
 *   dtype          mla_dtype of x, weights and cache
 *   rope_base      RoPE base (the pages default to 10000)
 *   softmax_scale  <= 0 selects the family default given above
 */
typedef struct {
  int32_t d_model, n_heads, d_nope, d_v, d_rope, r_kv, r_q, n_latent_heads;
  int32_t rope_mode, dtype;
  float rope_base, softmax_scale;
} mla_dims;

/* Projection weights; a family leaves the matrices it does not use NULL.
 *   w_dq [r_q][d_model]            w_uq [H*d_nope][r_q]        w_qr [H*d_rope][r_q or d_model]
 *   w_q  [H*d_nope][d_model]       w_dkv [r_kv][d_model]       w_kr [d_rope][d_model]
 *   w_uk, w_uv [H*d_nope][r_kv] (MLRA: [L][H*d_nope/L][r_kv/L])  w_o [d_model][H*d_v]   */
typedef struct {
  const void *w_dq, *w_uq, *w_qr, *w_q, *w_dkv, *w_kr, *w_uk, *w_uv, *w_o;
} mla_weights;

/* The latent cache (the only inference state; the DSV2 page's cache_kv / cache_rk).
 *   ckv [max_batch][max_seq][r_kv]   latent rows, dtype of dims
 *   kr  [max_batch][max_seq][d_rope] rotary keys, stored AFTER rotation at their
 *       absolute position (NULL when d_rope == 0)
 * Row t of sequence b holds token position t. */
typedef struct {
  void *ckv, *kr;
  int32_t max_batch, max_seq;
} mla_cache;

/* Human-readable name of a status code (static storage).
 * Source: the library's own (the pages define no error codes). */
const char* mla_status_str(mla_status s);

/* Checks dims against the pages' rules and the kernels' limits.
 * Source: the pages' constructor checks -- [MLA page] ``MLAAttention.__init__`` and
 * [MLRA page] ``MLRAAttention.__init__`` (their ValueErrors: the latent-head count L must
 * divide the latent rank and the heads), and the even-width assertion of [DSV2 page]
 * ``apply_rotary_emb`` (a rotary width must be even).  The kernel limits are the library's own.
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_SHAPE or MLA_ERR_UNSUPPORTED.
 * Kernel limits: d_nope <= 256 (FULL_HALFSPLIT: d_nope divides 128), d_rope <= 64,
 * r_kv / L <= 512, n_heads / L <= 128 * 64.  Host only; no GPU needed. */
mla_status mla_validate(const mla_dims* dims);

/* Source: the library's own (caller-owned scratch; the pages allocate inside forward).
 * Bytes of device workspace entry point `op` needs for `batch` sequences of
 * `seq_or_max_ctx` tokens (prefill: S; decode: the largest ctx_len; chunked prefill:
 * start_pos + T).  Returns 0 for invalid arguments and for ops that need none
 * (MLA_OP_CACHE_APPEND).  Host only. */
size_t mla_workspace_bytes(const mla_dims* dims, int op, int32_t batch, int32_t seq_or_max_ctx);

/* Fused down-projection + RoPE + cache write ([DSV2 page] ``forward`` cached path:
 * the current latent and rotary key are written at rows start_pos .. start_pos+T-1).
 *   x              [B][T][d_model], tokens of sequence b at positions start_pos_dev[b]+t
 *   start_pos_dev  int32 [B] device array; max_start >= every entry (host bound)
 *   cache          rows start_pos[b] .. start_pos[b]+T-1 of sequence b are overwritten
 *                  with c = W_DKV x and k_R = RoPE(W_KR x, position); nothing else changes.
 * Errors: CAPACITY if B > max_batch or max_start + T > max_seq. */
mla_status mla_cache_append(const mla_dims* dims, const mla_weights* w, const void* x,
                            int32_t B, int32_t T, const int32_t* start_pos_dev, int32_t max_start,
                            const mla_cache* cache, void* stream);

/* Causal prefill of B sequences of S tokens at positions 0..S-1.
 * Source: [MLA page] ``MLAAttention.forward``, [MLRA page] ``MLRAAttention.forward`` and
 * [DSV2 page] ``MultiHeadLatentAttention.forward`` without a cache (start_pos 0), per
 * family as listed at the top of this file: explicit K/V up-projection from the latent, flash-style causal
 * attention on bf16 MFMA (fp32 MFMA for MLA_DTYPE_F32), then W_O.
 *   x      [B][S][d_model]
 *   cache  optional (NULL allowed): rows 0..S-1 of each sequence are written
 *   y      [B][S][d_model] float32, fully overwritten
 * Errors: CAPACITY if a cache is given and B > max_batch or S > max_seq. */
mla_status mla_prefill(const mla_dims* dims, const mla_weights* w, const void* x,
                       int32_t B, int32_t S, const mla_cache* cache, float* y,
                       void* workspace, size_t ws_bytes, void* stream);

/* One decode step: one new token per sequence, absorbed form.
 * Source: [DSV2 page] ``MultiHeadLatentAttention.forward``, cached path with start_pos:
 * the new token's latent and rotary key are written at its row, and its query attends to
 * every cached row up to and including its own (MLRA family: [MLRA page]
 * ``MLRAAttention.forward`` restricted to the last row).  The absorption of W_UK into the
 * query and of W_UV after the weighted latent sum is associativity of those products.
 * The new token of sequence b sits at position ctx_len_dev[b]: its latent and rotary key
 * are appended at that row, then it attends over rows 0..ctx_len[b] (ctx_len[b]+1 keys,
 * itself included) with W_UK folded into the query and W_UV applied to the
 * attention-weighted latent sum.  The caller advances ctx_len; the library never does.
 *   x            [B][d_model]
 *   ctx_len_dev  int32 [B] device array, 0 <= ctx_len[b] <= max_ctx
 *   y            [B][d_model] float32
 * Errors: CAPACITY if B > max_batch or max_ctx + 1 > max_seq;
 *         UNSUPPORTED for MLA_ROPE_FULL_HALFSPLIT (RoPE on the decompressed key does not
 *         commute with the absorption). */
mla_status mla_decode(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B,
                      const int32_t* ctx_len_dev, int32_t max_ctx, const mla_cache* cache,
                      float* y, void* workspace, size_t ws_bytes, void* stream);

/* The attention core of one decode step over the latent cache (split-context kernel
 * plus log-sum-exp combine), for absorbed queries that the caller already formed.
 * Source: the score q . k_j and softmax-weighted value sum of [DSV2 page]
 * ``MultiHeadLatentAttention.forward`` (scores of the decompressed and rotary parts added,
 * scaled by 1/sqrt(d_nope + d_rope)), rewritten over the cached latent rows by
 * associativity: q_C . (W_UK c_j) = (W_UK^T q_C) . c_j.
 * Head h (latent block g = h / (H/L), width rb = r_kv/L) computes
 *   s_j = scale * (q_lat[b][h] . ckv[b][j][g*rb : (g+1)*rb] + q_rope[b][h] . kr[b][j]),
 *   z[b][h] = sum_j softmax_j(s) ckv[b][j][g*rb : (g+1)*rb],   j = 0 .. ctx_len[b]
 * where scale is dims->softmax_scale or the family default.
 *   q_lat   [B][H][rb]      dtype of dims (unscaled W_UK,h^T q_C,h)
 *   q_rope  [B][H][d_rope]  dtype of dims (rotated; NULL when d_rope == 0)
 *   z       [B][H][rb]      dtype of dims, fully overwritten
 * The cache rows 0..ctx_len[b] must already hold the latents (this call writes nothing
 * to the cache).  Errors as mla_decode. */
mla_status mla_decode_attention(const mla_dims* dims, const void* q_lat, const void* q_rope,
                                int32_t B, const int32_t* ctx_len_dev, int32_t max_ctx,
                                const mla_cache* cache, void* z,
                                void* workspace, size_t ws_bytes, void* stream);

/* mla_decode_attention for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace argument.  Source: the
 * library's own.  The split partials live in a fixed device array inside the library, one
 * per GPU, of mla_decode_attention_noalloc_max_bytes() bytes (96 MiB), held from the first
 * call on that GPU until the process ends.  Arguments, results and errors as
 * mla_decode_attention, plus MLA_ERR_WORKSPACE (before any launch) when the shapes need more
 * than that: mla_workspace_bytes(dims, MLA_OP_DECODE_ATTENTION, B, max_ctx) must not exceed it.
 * Every call on one GPU shares that array: calls on one GPU that overlap in time (other
 * streams, other threads) race; calls on different GPUs do not.  The call makes no
 * allocation (no hipMalloc / hipFree). */
mla_status mla_decode_attention_noalloc(const mla_dims* dims, const void* q_lat, const void* q_rope,
                                        int32_t B, const int32_t* ctx_len_dev, int32_t max_ctx,
                                        const mla_cache* cache, void* z, void* stream);

/* Source: the library's own.  Size in bytes of mla_decode_attention_noalloc's per-GPU array. */
size_t mla_decode_attention_noalloc_max_bytes(void);

/* The attention core of prefill: explicit K/V up-projection of the cached latent rows
 * 0..S-1 ([DSV2 page] ``forward``: UK_proj / UV_proj of C_KV) and flash-style causal
 * attention over them.
 *   q       [B][S][H][d_nope + d_rope] dtype of dims: per head the decompressed query
 *           followed by its rotated decoupled part (FULL_HALFSPLIT: the rotated query)
 *   cache   rows 0..S-1 hold the latent (and rotated k_R)
 *   w       uses w_uk and w_uv only
 *   o       [B][S][H][d_v] dtype of dims, fully overwritten (softmax-weighted values)
 * Errors: CAPACITY if B > max_batch or S > max_seq. */
mla_status mla_prefill_attention(const mla_dims* dims, const mla_weights* w, const void* q,
                                 int32_t B, int32_t S, const mla_cache* cache, void* o,
                                 void* workspace, size_t ws_bytes, void* stream);

/* Continued (chunked) prefill: T new tokens per sequence at positions start_pos ..
 * start_pos+T-1 over a cache whose rows 0..start_pos-1 already hold the earlier tokens'
 * latents ([DSV2 page] ``forward`` with start_pos > 0: the new latents and rotary keys are
 * written at rows start_pos.., the keys and values of rows 0..start_pos+T-1 are
 * up-projected, and new token i attends to the keys at positions <= start_pos + i).
 * start_pos = 0 gives mla_prefill with a cache.
 *   x          [B][T][d_model]
 *   start_pos  host int32, the same for every sequence (the page's start_pos)
 *   cache      rows start_pos .. start_pos+T-1 of each sequence are written; rows
 *              0..start_pos-1 are read and must hold the earlier tokens
 *   y          [B][T][d_model] float32, fully overwritten
 * Workspace: mla_workspace_bytes(dims, MLA_OP_PREFILL_CHUNK, B, start_pos + T).
 * Errors: CAPACITY if B > max_batch or start_pos + T > max_seq. */
mla_status mla_prefill_chunk(const mla_dims* dims, const mla_weights* w, const void* x,
                             int32_t B, int32_t T, int32_t start_pos, const mla_cache* cache,
                             float* y, void* workspace, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Training: the layer as a trainable module with dropout on the attention weights
 * ([DSV2 page] ``MultiHeadLatentAttention.__init__`` / ``forward``: dropout after the
 * softmax, before the product with the values; [MLA page] ``MLAAttention``: the same).
 * Family: MLA_ROPE_DECOUPLED_INTERLEAVED with a query latent (r_q > 0), one latent head.
 * Dropout draws: SplitMix64 (Steele, Lea, Flood, OOPSLA 2014); the weight of query i on key
 * j in head h of sequence b is kept when bits 16 (j % 4) .. 16 (j % 4) + 15 of the
 * generator's output n + 1 from state seed, n = (b * n_heads + h) * 2^38 + i * 2^18 + j / 4,
 * are >= floor(p * 2^16); a kept weight is scaled by 1 / (1 - p).  The same (seed, p) must be
 * passed to the forward and the backward.  B * n_heads <= 2^24 and S <= 2^20 (else
 * MLA_ERR_SHAPE).
 * ------------------------------------------------------------------------------------- */

/* Gradients of sum(dy * y) with respect to x and the weights (float32, shapes as the inputs /
 * mla_weights; every array fully overwritten).  The family's unused matrices have none. */
typedef struct {
  float *dx, *dw_dq, *dw_uq, *dw_qr, *dw_dkv, *dw_kr, *dw_uk, *dw_uv, *dw_o;
} mla_grads;

/* Source: the library's own.  Bytes of the state mla_train_forward keeps for the backward
 * (query latent, queries, latent, rotary keys, keys, values, attention outputs, per-row
 * log-sum-exp) for B sequences of S tokens; 0 for unsupported dims.  Host only. */
size_t mla_train_saved_bytes(const mla_dims* dims, int32_t B, int32_t S);

/* Source: the library's own.  Workspace bytes of mla_train_backward.  Host only. */
size_t mla_train_workspace_bytes(const mla_dims* dims, int32_t B, int32_t S);

/* Causal forward with dropout p in [0, 1) on the attention weights.
 * Source: [DSV2 page] ``MultiHeadLatentAttention.forward`` (training mode, no cache).
 *   x [B][S][d_model]; y [B][S][d_model] float32 (overwritten); saved: caller-owned device
 *   buffer of mla_train_saved_bytes, filled for mla_train_backward.  p = 0 gives mla_prefill's
 *   result (up to rounding).
 * Errors: UNSUPPORTED outside the family above, INVALID_ARG for p outside [0, 1) or missing
 * pointers, WORKSPACE if saved_bytes is too small, HIP for a failed launch. */
mla_status mla_train_forward(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B, int32_t S,
                             float dropout_p, uint64_t seed, float* y, void* saved, size_t saved_bytes,
                             void* stream);

/* Backward of mla_train_forward: the chain rule through the output projection, the dropped-
 * out softmax attention (per-row log-sum-exp and dropout mask recomputed), the rotations
 * (by the negative angle; the rotary key's gradient summed over heads) and the projections.
 * Source: [DSV2 page] ``MultiHeadLatentAttention.forward`` differentiated.
 *   dy [B][S][d_model] float32; saved: as filled by mla_train_forward with the same x, w, p,
 *   seed; g: gradient arrays (float32, fully overwritten).
 * Errors as mla_train_forward; WORKSPACE if ws_bytes < mla_train_workspace_bytes. */
mla_status mla_train_backward(const mla_dims* dims, const mla_weights* w, const void* x, int32_t B, int32_t S,
                              float dropout_p, uint64_t seed, const float* dy, const void* saved,
                              size_t saved_bytes, const mla_grads* g, void* workspace, size_t ws_bytes,
                              void* stream);

/* ---------------------------------------------------------------------------------------
 * Compressed convolutional attention (CCA) and its grouped-query form (CCGQA): a related
 * latent method in which queries, keys and values are down-projected into a compressed
 * latent and attention runs entirely inside it ([CCA page] frankenstein-transformer docs,
 * ``latent/cca_attn``).  CCA is the case n_kv_heads == n_heads.
 * ------------------------------------------------------------------------------------- */

/* Layer dimensions ([CCA page] ``CCAAttention.__init__`` / ``CCGQAAttention.__init__``).
 *   d_model          E, input / output width
 *   n_heads          Hq, query heads
 *   n_kv_heads       Hkv, key / value heads (divides Hq; = Hq for CCA)
 *   head_dim         d_h, latent width per head (even: RoPE in the latent)
 *   num_conv_layers  0, 1 (the depth-wise sequence convolution) or 2 (then the head-grouped one)
 *   conv_kernel_seq  kernel of the sequence convolution; conv_kernel_ch of the grouped one
 *   qk_mean          1: add the pre-convolution q-k mean to q and k
 *   value_shift      1: the first half of the value channels from the current token, the
 *                    second half from the previous token (Hkv even)
 *   dtype            mla_dtype of x, weights and the attention operands
 *   rope_base        RoPE base (10000 on the page) */
typedef struct {
  int32_t d_model, n_heads, n_kv_heads, head_dim;
  int32_t num_conv_layers, conv_kernel_seq, conv_kernel_ch;
  int32_t qk_mean, value_shift, dtype;
  float rope_base;
} mla_cca_dims;

/* Weights, row-major [out][in] in the element type of dims (device pointers).
 *   w_qk      [(Hq + Hkv) d_h][E]     packed q / k down-projection
 *   w_v       [Hkv d_h][E]            value projection; with value_shift the current-token
 *                                     projection's Hkv d_h / 2 rows, then the previous-token one's
 *   w_o       [E][Hq d_h]             output up-projection
 *   conv_seq  [(Hq + Hkv) d_h][k_seq] depth-wise convolution filters (used if num_conv_layers >= 1)
 *   conv_ch   [(Hq + Hkv) d_h][d_h][k_ch] head-grouped convolution filters (if num_conv_layers == 2)
 *   key_temperature  beta (host value): the normalised keys are scaled by exp(beta) */
typedef struct {
  const void *w_qk, *w_v, *w_o, *conv_seq, *conv_ch;
  float key_temperature;
} mla_cca_weights;

/* Checks CCA dims.  Source: the ValueErrors of [CCA page] ``CCAAttention.__init__`` and
 * ``CCGQAAttention.__init__`` (E divisible by the heads, Hkv dividing Hq, an even d_h, 0-2
 * convolution layers, an even Hkv for value shift); kernel limits (the library's own):
 * d_h <= 128 (<= 64 for MLA_DTYPE_F32), kernels 1..8.
 * Returns MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_SHAPE or MLA_ERR_UNSUPPORTED.  Host only. */
mla_status mla_cca_validate(const mla_cca_dims* dims);

/* Source: the library's own.  Workspace bytes mla_cca_prefill needs for B sequences of S
 * tokens (0 for invalid arguments).  Host only. */
size_t mla_cca_workspace_bytes(const mla_cca_dims* dims, int32_t B, int32_t S);

/* Causal forward of B sequences of S tokens at positions 0..S-1.
 * Source: [CCA page] ``CCAAttention.forward`` (n_kv_heads == n_heads) and
 * ``CCGQAAttention.forward`` (query head h attends with key / value head h / (Hq / Hkv)), in
 * decoder mode without dropout: packed down-projection, ``_apply_causal_convs``, q-k-mean,
 * value shift, QK L2-norm with key temperature, half-split RoPE, causal softmax attention
 * with scale d_h^-1/2, output up-projection.
 *   x  [B][S][E]          y  [B][S][E] float32, fully overwritten
 * Errors: as the validation, INVALID_ARG for missing pointers, WORKSPACE if ws_bytes is below
 * mla_cca_workspace_bytes(dims, B, S), HIP for a failed launch. */
mla_status mla_cca_prefill(const mla_cca_dims* dims, const mla_cca_weights* w, const void* x,
                           int32_t B, int32_t S, float* y, void* workspace, size_t ws_bytes,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
