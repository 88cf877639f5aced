/*
 * lvsa.h -- C ABI of liblvsa.so: block-sparse softmax attention for video
 * diffusion transformers on AMD Instinct MI355X (gfx950), with the two mask
 * builders it runs on (LVSA and Draft Attention) and a dense baseline.
 *
 * Sources (cited by page title and section):
 *   [LVSA]  "LVSA: Training-Free Sparse Attention for Long Video Diffusion"
 *           (gist.science explainer), technical summary §1 "Problem
 *           statement", §2 "Methodology" (core mechanism, complexity).
 *   [DRAFT] "科学家提出视频扩散模型加速方法，在H100实现一倍以上端到端加速"
 *           (163.com article on Draft Attention): [t,h,w] reshape, average
 *           pooling into a draft map, sparse mask, pool_h*pool_w = block_size,
 *           reorder into contiguous blocks.
 *
 * Conventions shared by every call
 *   - Tensors Q, K, V, O are [heads, n, d], row-major, contiguous, batch 1.
 *     Tokens are frame-major over the [t, h, w] grid: n = (t*H + y)*W + x.
 *   - d is 64 or 128. dtype LVSA_BF16 (bfloat16 bits) or LVSA_F32.
 *     O is always fp32. For attention, n*d must be below 2^30 (one head of
 *     bf16 K or V stays under 2 GiB).
 *   - Every pointer argument is a device pointer (memory the caller
 *     allocated with hipMalloc or a framework allocator) unless marked
 *     "host". Device pointers must be 16-byte aligned. The caller owns every
 *     buffer, including workspaces; the library keeps no device memory and
 *     no pointers between calls.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).
 *     All device work is enqueued asynchronously on it; outputs are valid
 *     once the stream has been synchronised.
 *   - Return value: LVSA_OK (0) or a negative lvsa_status. Arguments are
 *     validated on the host before anything is launched; on error nothing
 *     is launched and lvsa_last_error() describes the failure. No C++
 *     exception crosses this boundary. Calls are thread-safe (the error text
 *     is thread-local).
 *   - Device-side index data (kv_idx, kv_cnt, block_valid) cannot be checked
 *     on the host: kernels clamp kv_cnt to max_kv, skip list entries outside
 *     [0, number of KV blocks) and clamp block_valid to [0, block size], so a
 *     bad list never causes an out-of-bounds access.
 */
#ifndef LVSA_H
#define LVSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LVSA_OK = 0,
  LVSA_EINVAL = -1,      /* an argument is invalid (shape, pointer, parameter) */
  LVSA_ERANGE = -2,      /* an output capacity is too small */
  LVSA_EDEVICE = -3,     /* no usable GPU, or a HIP launch/runtime error */
  LVSA_ENOMEM = -4,      /* workspace too small */
  LVSA_EUNSUPPORTED = -5 /* valid request outside what the kernels implement */
} lvsa_status;

typedef enum { LVSA_F32 = 0, LVSA_BF16 = 1 } lvsa_dtype;

/* Draft pooling of Q and K: the mean (the article's choice) or the maximum
 * (the variant it compares against). */
typedef enum { LVSA_POOL_MEAN = 0, LVSA_POOL_MAX = 1 } lvsa_pool;

/* Text of the calling thread's last failure ("" if none). Host pointer owned
 * by the library, valid until the thread's next call. */
const char* lvsa_last_error(void);

/* Library version string (host pointer, static). */
const char* lvsa_version(void);

/* ------------------------------------------------------------------------
 * LVSA frame mask  [LVSA §2 "Core mechanism"]
 *
 * Query frame t (0 <= t < T) attends to A(t) = G_s ∪ W(t):
 *   G_s  = { f in [0,T) : f ≡ step (mod T_per) }   rotating global anchors;
 *          over T_per consecutive steps every frame is an anchor exactly once.
 *   W(t) = the first k frames in the order of the key (|f - t|, f): a window
 *          centred on t, the earlier frame first on ties, shifted inward at the
 *          ends. k starts at `window` and grows one frame at a time while
 *          |A(t)| < min(C, T) and k < T (the expanding window keeps |A(t)| at
 *          the budget C). If the anchors plus the base window already exceed C
 *          the set is kept whole.
 * ------------------------------------------------------------------------ */

/* Host-only. Exact max over t of |A(t)| for these parameters (>= 1), or a
 * negative lvsa_status. Use it as `cap` for lvsa_mask. Requires T >= 1,
 * C >= 1, window >= 1, T_per >= 1, step >= 0. */
int lvsa_mask_capacity(int T, int C, int window, int T_per, int step);

/* Writes kv_idx [T, cap] int32 (frames of A(t) ascending, then -1 padding)
 * and kv_cnt [T] int32 (= |A(t)|). Both are device buffers owned by the
 * caller. LVSA_ERANGE if cap < lvsa_mask_capacity(...). The mask is the same
 * for every head and layer of one denoising step. */
int lvsa_mask(int T, int C, int window, int T_per, int step, int32_t* kv_idx, int32_t* kv_cnt, int cap,
              void* stream);

/* ------------------------------------------------------------------------
 * Draft Attention mask builder and reorder  [DRAFT]
 *
 * Grid [T, H, grid_w] tokens; tiles of pool_h x pool_w tokens (block size
 * bs = pool_h*pool_w). The grid is padded at the bottom/right to multiples of
 * the tile: Hp = ceil(H/pool_h)*pool_h, Wp likewise; nb = T*(Hp/pool_h)*(Wp/pool_w)
 * blocks in raster order (t, hb, wb); N_pad = nb*bs.
 *   perm[p]        (p < N_pad)  original token at reordered slot p, -1 for a pad;
 *                  within a block the valid tokens come first, in (hi, wi) order.
 *   inv_perm[n]    (n < T*H*grid_w)  reordered slot of token n.
 *   block_valid[b] number of valid tokens of block b (they are its first slots).
 * Pooling: for each head, block and channel c, acc = +0.0f, then acc += x for
 *   each valid token in slot order (each add rounded to fp32), mean = acc/count
 *   (one IEEE fp32 division). Applied to Q and to K. With LVSA_POOL_MAX the
 *   pooled value is the largest x over the valid tokens, plus +0.0f (so a
 *   zero result is +0); Q and K must then be finite.
 * Draft map: s[h,i,j] = fold over c = 0..d-1 of acc = fl(acc + fl(q̄[i,c]*k̄[j,c]))
 *   starting from +0.0f, no fused multiply-add (the unscaled logit: softmax and
 *   1/sqrt(d) do not change a row's ranking).
 * Top-k: each row keeps k = clamp(floor((1 - sparsity)*nb + 0.5), 1, nb) blocks,
 *   larger score first, lower block index first on a tie, -0 equal to +0,
 *   stored in ascending block order. Scores must be finite.
 * ------------------------------------------------------------------------ */

/* Host-only. Grid facts: *nb, *n_pad, *block_size, *k (for this sparsity).
 * Any output pointer may be NULL. Returns LVSA_OK or LVSA_EINVAL. */
int draft_grid_info(int T, int H, int grid_w, int pool_h, int pool_w, double sparsity, int* nb, int* n_pad,
                    int* block_size, int* k);

/* Host-only. Bytes of device workspace draft_mask_and_perm needs:
 * pooled Q̄ and K̄, each [heads, nb, d] fp32, at byte offsets 0 and
 * heads*nb*d*4, then K̄ transposed, [heads, d, nb] fp32, at byte offset
 * 2*heads*nb*d*4. Returns 0 for invalid arguments. */
size_t draft_workspace_bytes(int heads, int T, int H, int grid_w, int d, int pool_h, int pool_w);

/* Full Draft mask builder on Q, K (and the reorder of Q, K, V).
 *   q, k, v     [heads, T*H*grid_w, d] of dtype dt (v may be NULL when v_perm is NULL)
 *   pool_mode   LVSA_POOL_MEAN or LVSA_POOL_MAX (LVSA_EINVAL otherwise)
 *   kv_idx      out [heads, nb, k] int32 (k from draft_grid_info)
 *   kv_cnt      out [heads, nb] int32 (= k)
 *   perm        out [N_pad] int32; inv_perm out [T*H*grid_w] int32; block_valid out [nb] int32
 *   q_perm, k_perm, v_perm  out [heads, N_pad, d] of dtype dt: the reordered
 *               tensors, pads zero. All three NULL to skip the reorder.
 *   workspace   device buffer of ws_bytes >= draft_workspace_bytes(...);
 *               holds Q̄, K̄ and K̄ᵀ on return (layout above).
 * Requires block size <= 1024 and nb <= 4096. */
int draft_mask_and_perm(const void* q, const void* k, const void* v, int dt, int heads, int T, int H, int grid_w,
                        int d, int pool_h, int pool_w, double sparsity, int pool_mode, int32_t* kv_idx, int32_t* kv_cnt,
                        int32_t* perm, int32_t* inv_perm, int32_t* block_valid, void* q_perm, void* k_perm,
                        void* v_perm, void* workspace, size_t ws_bytes, void* stream);

/* draft_mask_and_perm for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and outputs without the workspace, which
 * comes from a device array the library holds, one copy per GPU, reserved
 * when the library is loaded and kept until the process ends. The call makes
 * no hipMalloc, hipFree or other allocation; the caller still passes every
 * input and output buffer.
 *   Limit: 3*heads*nb*d*4 bytes (pooled Q̄, K̄ and K̄ᵀ) must fit in
 *   LVSA_NOALLOC_SCRATCH_BYTES, i.e. heads*nb*d <= 4194304 (the
 *   HunyuanVideo-shaped 24 heads x 990 blocks x 128 channels needs
 *   3041280); larger requests return LVSA_ENOMEM before anything runs.
 *   Every call on one GPU uses that GPU's one array, and each call writes
 *   all of the part it reads, so nothing is carried from the previous call;
 *   calls that overlap in time on the same GPU (other streams, other host
 *   threads) race on it and must be serialised by the caller. */
#define LVSA_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
int draft_mask_and_perm_noalloc(const void* q, const void* k, const void* v, int dt, int heads, int T, int H,
                                int grid_w, int d, int pool_h, int pool_w, double sparsity, int pool_mode,
                                int32_t* kv_idx, int32_t* kv_cnt, int32_t* perm, int32_t* inv_perm,
                                int32_t* block_valid, void* q_perm, void* k_perm, void* v_perm, void* stream);

/* The draft map itself, materialised: scores [heads, nb_q, nb_k] fp32 from
 * q̄ [heads, nb_q, d] and k̄ [heads, nb_k, d] fp32, same fixed arithmetic as
 * above. For inspection and testing; draft_mask_and_perm never stores it. */
int draft_scores(const float* qbar, const float* kbar, int heads, int nb_q, int nb_k, int d, float* scores,
                 void* stream);

/* Row gather: dst[h, i, :] = src[h, dst_to_src[i], :], or zeros where
 * dst_to_src[i] < 0 or >= n_src. src [heads, n_src, d], dst [heads, n_dst, d],
 * element type dt (bf16 or fp32); the map is [n_dst] int32. With
 * dst_to_src = inv_perm it scatters a reordered O back to token order; with
 * perm it builds a reordered tensor. src and dst must not overlap; d*esize
 * must be a multiple of 16 bytes; one head of src or dst must hold fewer
 * than 2^31 16-byte chunks (LVSA_EINVAL otherwise). */
int token_permute(const void* src, void* dst, int dt, int heads, int n_src, int n_dst, int d,
                  const int32_t* dst_to_src, void* stream);

/* ------------------------------------------------------------------------
 * Attention  [LVSA §1 "Problem statement" (dense), §2 "Complexity"
 * (frame-block-sparse); DRAFT (block-sparse on the reordered tokens)]
 *
 * Query row i of head h belongs to query block qb = i / block_q. Its keys
 * are the valid rows of the KV blocks kv_idx[hm][qb][0 .. kv_cnt[hm][qb]-1],
 * hm = (mask_heads > 1 ? h : 0): block b holds rows
 * [b*block_k, b*block_k + valid(b)) ∩ [0, n), valid(b) = block_valid[b] if
 * block_valid is non-NULL, else block_k. With block_valid, query rows at a
 * slot >= block_valid[qb] are pads: their output rows are 0 (requires
 * block_q == block_k). A query with no keys gets output 0.
 *   O[h,i,:] = sum_j exp(s_ij - m_i) V[h,j,:] / sum_j exp(s_ij - m_i),
 *   s_ij = scale * <Q[h,i,:], K[h,j,:]>, m_i = max_j s_ij   (not causal).
 * scale must be finite and > 0 (LVSA_EINVAL otherwise): keys outside the
 * set enter the kernels as scores of -infinity before the scale is applied.
 * Inputs whose fp32 dot products overflow (|<q, k>| above ~3.4e38) are
 * outside the domain: their rows come out NaN.
 * bf16: QKᵀ and PV on bf16 MFMA with fp32 accumulation; probabilities are
 * rounded to bf16 for the PV product and the row sum uses those same rounded
 * values. fp32: fp32 arithmetic throughout. O is fp32 [heads, n, d].
 *
 * LVSA:  block_q = block_k = P (tokens per frame), mask_heads = 1, kv_idx =
 *        the lvsa_mask output (cap = max_kv), block_valid = NULL.
 * Draft: block_q = block_k = pool_h*pool_w on q_perm/k_perm/v_perm,
 *        mask_heads = heads, block_valid from draft_mask_and_perm; then
 *        token_permute(O_perm -> O, inv_perm).
 * A call may enqueue more than one kernel on `stream` (bf16, d = 128,
 * blocks that end in a tile of 1-32 rows, such as 1560-row frames, and
 * lists of up to 128 entries: the rows of the full 128-row tiles, then the
 * short tails of four blocks per workgroup); O is complete once the stream
 * has run past the call.
 * ------------------------------------------------------------------------ */
int block_sparse_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int n, int d,
                          int block_q, int block_k, const int32_t* kv_idx, const int32_t* kv_cnt, int max_kv,
                          int mask_heads, const int32_t* block_valid, float scale, void* stream);

/* Draft attention without the reorder  [DRAFT: blocks of the block-sparse
 * kernel are the pool_h x pool_w tiles of the draft map; the reorder only
 * makes each block contiguous]
 *
 * Same result as reordering Q, K, V (draft_mask_and_perm), running
 * block_sparse_attn_fwd with block_q = block_k = pool_h*pool_w and
 * block_valid, and scattering O back with token_permute, but on the raster
 * layout: q, k, v [heads, T*H*grid_w, d] bf16 and o [heads, T*H*grid_w, d]
 * fp32 in token order. Block b is tile (t, hb, wb) in raster order (as in
 * draft_grid_info); its keys are the valid tokens of the tile, taken in
 * (hi, wi) order; kv_idx [heads, nb, max_kv] and kv_cnt [heads, nb] are the
 * per-head lists of draft_mask_and_perm (entries outside [0, nb) skipped).
 * Every output row is written. Requires dt = LVSA_BF16, d = 128,
 * pool_h*pool_w a multiple of 64 and pool_w dividing 64 (LVSA_EUNSUPPORTED
 * otherwise); n*d < 2^30. */
int draft_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int T, int H,
                   int grid_w, int d, int pool_h, int pool_w, const int32_t* kv_idx, const int32_t* kv_cnt,
                   int max_kv, float scale, void* stream);

/* Dense baseline: every query attends to all n keys. Same arithmetic and
 * layout as block_sparse_attn_fwd. */
int dense_attn_fwd(const void* q, const void* k, const void* v, float* o, int dt, int heads, int n, int d,
                   float scale, void* stream);

/* ------------------------------------------------------------------------
 * FP8 (OCP E4M3) variant  [DRAFT: the article names quantization as the
 * step after its sparse mask; it fixes no format, so the choices below are
 * this library's]
 *
 * Format: E4M3 "fn" bytes (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, largest finite 448, no infinity; 0x7F/0xFF are NaN and
 * never produced). One dequantization factor per (tensor, head).
 * ------------------------------------------------------------------------ */

/* Per-head quantization of src [heads, n, d] (dt bf16 or fp32, finite
 * values): scale[h] = fl32(max|src[h]| / 448) (1 when the head is all
 * zeros), code = the E4M3 value nearest fl32(x / scale[h]) after clamping
 * the quotient to [-448, 448], ties to the even mantissa; the value a code
 * stands for is decode(code) * scale[h].
 * transpose = 0: dst [heads, n, d], ld must be 0.
 * transpose = 1: dst [heads, d, ld], dst[h, c, i] = code of src[h, i, c];
 *   ld (row pitch in bytes) a multiple of 16 and >= n; bytes n .. ld-1 of a
 *   row are set to 0. This is the layout the attention takes V in.
 * scales: device float[heads], written. d is 64 or 128; n*d < 2^30,
 * d*ld < 2^31, heads <= 65535. src, dst 16-byte aligned; scales 4-byte
 * aligned. */
int quantize_fp8_e4m3(const void* src, int dt, int heads, int n, int d, int transpose, int ld, uint8_t* dst,
                      float* scales, void* stream);

/* Block-sparse attention on E4M3 operands: q8, k8 [heads, n, 128] codes,
 * vt8 [heads, 128, ldv] codes of Vᵀ (quantize_fp8_e4m3 with transpose = 1;
 * every byte of a row, padding included, must be a finite code, which the
 * quantizer guarantees), q_scale, k_scale, v_scale device float[heads].
 * Same key lists, block_valid, pad rows and output layout as
 * block_sparse_attn_fwd (Draft: q8/k8/vt8 quantized from the reordered
 * tensors), on the values q = q_scale[h] * decode(q8) (likewise k, v):
 *   s_ij = scale * <q_i, k_j> (exact products, fp32 sums, on the FP8
 *   matrix cores), probabilities exp(s_ij - m) in fp32 with m a score of
 *   the row that lags its running maximum (moved to the maximum whenever a
 *   tile's probabilities could exceed 2^8, so every one is <= 2^8), the
 *   probabilities rounded to E4M3 (nearest even) for the PV product, the row
 *   sum over the unrounded fp32 values, O fp32 [heads, n, 128].
 * Requires d = 128, n a multiple of 4, block_k >= 64 and a multiple of 4
 * (LVSA_EUNSUPPORTED otherwise); ldv a multiple of 16, >= n (LVSA_EINVAL);
 * n*128 < 2^30. */
int block_sparse_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv,
                              const float* q_scale, const float* k_scale, const float* v_scale, float* o, int heads,
                              int n, int d, int block_q, int block_k, const int32_t* kv_idx, const int32_t* kv_cnt,
                              int max_kv, int mask_heads, const int32_t* block_valid, float scale, void* stream);

/* FP8 Draft attention on the raster layout  [DRAFT, as draft_attn_fwd]:
 * draft_attn_fwd's blocks, lists and output on E4M3 operands (q8, k8
 * [heads, T*H*grid_w, 128], vt8 [heads, 128, ldv], per-head scales), with
 * block_sparse_attn_fwd_fp8's arithmetic. Requires d = 128,
 * pool_h*pool_w a multiple of 64, pool_w in {4, 8, 16, 32, 64} and grid_w a
 * multiple of 4 (LVSA_EUNSUPPORTED otherwise). */
int draft_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv, const float* q_scale,
                       const float* k_scale, const float* v_scale, float* o, int heads, int T, int H, int grid_w,
                       int d, int pool_h, int pool_w, const int32_t* kv_idx, const int32_t* kv_cnt, int max_kv,
                       float scale, void* stream);

/* Dense FP8 attention: every query attends to all n keys; arithmetic and
 * layouts as block_sparse_attn_fwd_fp8 (d = 128, n a multiple of 4). */
int dense_attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* vt8, int ldv, const float* q_scale,
                       const float* k_scale, const float* v_scale, float* o, int heads, int n, int d, float scale,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LVSA_H */
