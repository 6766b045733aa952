/*
 * tplayer.h -- C ABI of the tensor-parallel decoder-layer shard library
 * (libtplayer.so, HIP kernels for MI355X / gfx950).
 *
 * Each entry point computes one step of ONE tensor-parallel rank's share of a
 * Megatron-style pre-norm decoder layer.  Sources (web pages):
 *   P1 "Tensor Parallel：当一张 GPU 放不下一个大模型" (mini vLLM series)
 *   P2 "张量并行（Tensor Parallelism）推理部署实战：从 Megatron-LM 切分原理到
 *       vLLM 多卡配置与性能调优"
 *   P3 "Tensor Parallel 深入解析：多加 GPU，推理为什么可能更慢"
 *
 * Common rules for every call:
 *   - Tensor arguments are DEVICE pointers owned by the caller (the library
 *     never allocates, frees or keeps them).  Matrices are row-major and
 *     contiguous unless strides are given.  Strides are in elements.
 *   - Weights use the nn.Linear layout [out_features, in_features]: the
 *     input dimension is contiguous, i.e. the stored array is W^T of the
 *     mathematical Y = X W (P2 sections 1.1 / 1.2 sketches; P3 "两张卡如何共同
 *     算出一层" notes that the stored form may be the transpose).
 *   - There is no rank argument: a call acts on the shard it is given.  Host
 *     code slices shards (contiguous blocks in rank order).
 *   - `stream` is a hipStream_t (NULL: the default stream).  Calls enqueue
 *     work and return without synchronising.  Arguments are validated on the
 *     host before anything is enqueued; a non-TP_OK status means nothing was
 *     launched, except TP_ERR_HIP, which reports a failed launch (see
 *     tp_last_error()).
 *   - dtype: TP_BF16 = bfloat16 storage, TP_F32 = float32 storage.
 *     Accumulation is always float32.  bf16 results are rounded to nearest
 *     even.
 *   - Fast vector paths need 16-byte aligned base pointers and row lengths
 *     that are multiples of 16 bytes; other inputs take a slower element path
 *     (same arithmetic; sums may be ordered differently, so results can differ
 *     in the last float32 bits).  For given sizes, alignment and dtype a call
 *     always takes the same path and gives the same bits.
 */
#ifndef TPLAYER_H
#define TPLAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = 1,         /* a required pointer is NULL                        */
  TP_ERR_SHAPE = 2,        /* non-positive or inconsistent sizes, Hq % Hkv != 0  */
  TP_ERR_DTYPE = 3,        /* dtype / activation enum out of range or unsupported */
  TP_ERR_ALIGN = 4,        /* pointer alignment below the element size          */
  TP_ERR_WORKSPACE = 5,    /* workspace missing or smaller than required        */
  TP_ERR_HIP = 6,          /* a HIP runtime call failed (tp_last_error has text) */
  TP_ERR_UNSUPPORTED = 7   /* valid request outside what the kernels implement  */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum { TP_ACT_NONE = 0, TP_ACT_SWIGLU = 1, TP_ACT_GELU = 2 } tp_act;

/*
 * Column-parallel linear on one rank (P1 "Column Parallel Linear：按输出维度切";
 * P2 1.1; P3 "两张卡如何共同算出一层").  Every rank holds the full input and a
 * block of output features; the result is that rank's output slice and needs
 * no exchange:
 *     y[m, n] = sum_k x[m, k] * w[n, k]        (Y_r = X W_r)
 *   x : [M, K]  dtype dt      (the replicated full input)
 *   w : [N, K]  dtype dt      (the rank's output-feature block, N = N_full / R)
 *   y : [M, N]  dtype dt
 * M <= 64 takes the weight-streaming path (decode); larger M the MFMA tile path.
 */
tp_status tp_column_linear(const void* x, const void* w, void* y,
                           int64_t M, int64_t K, int64_t N,
                           tp_dtype dt, void* stream);

/*
 * Row-parallel linear on one rank (P1 "Row Parallel Linear：按输入维度切";
 * P2 1.2).  Input and weight are split along the input dimension; the result
 * is this rank's float32 PARTIAL of the full output, which must be summed over
 * ranks (tp_reduce_partials) -- never concatenated:
 *     partial[m, n] = sum_k x[m, k] * w[n, k]  (Y_r = X_r W_r)
 *   x       : [M, K]  dtype dt   (the rank's input slice, K = K_full / R)
 *   w       : [N, K]  dtype dt   (the rank's input-feature block)
 *   partial : [M, N]  float32
 */
tp_status tp_row_linear_partial(const void* x, const void* w, float* partial,
                                int64_t M, int64_t K, int64_t N,
                                tp_dtype dt, void* stream);

/*
 * Rank-local activation on the intermediate slice (P1 "MLP 里的 tensor
 * parallel": activation(gate_i) * up_i needs no exchange; P2 section 二:
 * GELU between fc1 and fc2).
 *     TP_ACT_SWIGLU: h = g * sigmoid(g) * u
 *     TP_ACT_GELU:   h = 0.5 * g * (1 + erf(g / sqrt(2)))    (u unused)
 *     TP_ACT_NONE:   h = g                                   (u unused)
 *   gate : element (m, i) at gate[m * ld + i]   dtype dt
 *   up   : element (m, i) at up[m * ld + i]     dtype dt (SWIGLU only; else may be NULL)
 *   h    : [M, I] contiguous                    dtype dt
 * A fused gate|up projection output [M, 2I] is passed as gate = base,
 * up = base + I, ld = 2I.
 */
tp_status tp_swiglu_local(const void* gate, const void* up, void* h,
                          int64_t M, int64_t I, int64_t ld,
                          tp_act act, tp_dtype dt, void* stream);

/*
 * Column-parallel linear with the rank-local activation fused into its
 * epilogue (P1 "MLP 里的 tensor parallel": gate_i and up_i are both local to
 * rank i, so activation(gate_i) * up_i needs no exchange; P2 section 二: GELU
 * directly after the column-parallel fc1).  The activation is applied to the
 * float32 sums of the projection, so the gate and up products are never
 * rounded and the [M, 2I] gate|up intermediate never reaches memory; only h
 * is rounded to bf16.  (tp_column_linear followed by tp_swiglu_local stores
 * g and u as bf16 first, so the two routes agree to bf16 rounding of g and u,
 * not bit for bit.)
 *     TP_ACT_SWIGLU: h[m, i] = act(x . w[i, :], x . w[I + i, :])   w: [2I, K]
 *                    (gate rows, then the matching up rows)
 *     TP_ACT_GELU:   h[m, i] = gelu(x . w[i, :])                    w: [I, K]
 *     TP_ACT_NONE:   same as tp_column_linear (N = I)
 *   x : [M, K], h : [M, I] contiguous.  dt must be TP_BF16 for SWIGLU/GELU;
 *   K % 8 == 0 and 16-byte aligned x and w (TP_ERR_UNSUPPORTED otherwise).
 */
tp_status tp_column_linear_act(const void* x, const void* w, void* h,
                               int64_t M, int64_t K, int64_t I,
                               tp_act act, tp_dtype dt, void* stream);

/*
 * Attention over the rank's local heads (P1 "Attention 里的 tensor parallel":
 * each rank attends only over its own heads and keeps their KV; P2 2.1).
 * Grouped KV heads (P3 "权重变小，不代表所有显存都按比例变小"): local q head h
 * reads local KV head h / (Hq / Hkv).
 *     o[b,s,h,:] = softmax_t(scale * q[b,s,h,:] . k[b,t,h/G,:]) v[b,t,h/G,:]
 * Causal masking is aligned to the end of the key span: query row s sits at
 * position s + Skv - Sq and sees keys t <= that position.  Decode is Sq = 1.
 *   q : element (b,s,h,d) at q[b*qs[0] + s*qs[1] + h*qs[2] + d]
 *   k, v : element (b,t,j,d) at k[b*kvs[0] + t*kvs[1] + j*kvs[2] + d] (same strides)
 *   o : element (b,s,h,d) at o[b*os[0] + s*os[1] + h*os[2] + d]
 *   dt must be TP_BF16; D must be 128 (TP_ERR_UNSUPPORTED otherwise).
 *   Decode (Sq = 1) with G = Hq/Hkv <= 32 takes a split-key path: one pass
 *   writes per-chunk partials into the workspace and a second pass combines
 *   them; it needs ((Skv-1) * kvs[1] + D) * 2 < 2^31 (TP_ERR_UNSUPPORTED
 *   otherwise).  Other shapes (prefill, or G > 32) need no workspace.
 *   workspace: device scratch of at least tp_local_attention_workspace(...)
 *   bytes (may be NULL when that is 0), owned by the caller, used only during
 *   the call's execution on `stream`; calls that overlap in time must not
 *   share one workspace.
 */
tp_status tp_local_attention(const void* q, const int64_t qs[3],
                             const void* k, const void* v, const int64_t kvs[3],
                             void* o, const int64_t os[3],
                             int64_t B, int64_t Sq, int64_t Skv,
                             int64_t Hq, int64_t Hkv, int64_t D,
                             int causal, float scale, tp_dtype dt,
                             void* workspace, size_t workspace_bytes, void* stream);

size_t tp_local_attention_workspace(int64_t B, int64_t Sq, int64_t Skv,
                                    int64_t Hq, int64_t Hkv, int64_t D);

/*
 * Append the current decode token's k and v to the rank's local KV cache at
 * key position `pos` (P1 "Tensor parallel 对 KV cache 的影响": each rank keeps
 * the cache of its own heads only).
 *   k_new, v_new : element (b,j,d) at k_new[b*new_stride + j*D + d]
 *   k_cache, v_cache : element (b,t,j,d) at k_cache[b*cs[0] + t*cs[1] + j*cs[2] + d],
 *                      t < T (the cache's key capacity)
 *   0 <= pos < T (TP_ERR_SHAPE otherwise).  dt must be TP_BF16.
 */
tp_status tp_kv_append(const void* k_new, const void* v_new, int64_t new_stride,
                       void* k_cache, void* v_cache, const int64_t cs[3],
                       int64_t B, int64_t Hkv, int64_t D, int64_t T, int64_t pos,
                       tp_dtype dt, void* stream);

/*
 * One decode step's cache append and local attention in one launch (the same
 * P1 section: each rank appends its own heads' k/v and attends over its own
 * heads; P3 GQA section for the q -> KV head map): equal, bit for bit, to
 *     tp_kv_append(k_new, v_new, new_stride, k_cache, v_cache, cs, B, Hkv, D, T, pos)
 *     tp_local_attention(q, k_cache, v_cache, Sq = 1, Skv = pos + 1)
 * on the same stream.
 *   q : element (b,h,d) at q[b*qs[0] + h*qs[1] + d]                bf16
 *   k_new, v_new : element (b,j,d) at k_new[b*new_stride + j*D + d] bf16
 *   k_cache, v_cache : element (b,t,j,d) at k_cache[b*cs[0] + t*cs[1] + j*cs[2] + d]
 *   o : element (b,h,d) at o[b*os[0] + h*os[1] + d]                bf16
 *   0 <= pos < T, new_stride >= Hkv*D (TP_ERR_SHAPE otherwise).  dt must be
 *   TP_BF16, D = 128, G = Hq/Hkv <= 32, (pos*cs[1] + D)*2 < 2^31
 *   (TP_ERR_UNSUPPORTED otherwise).  Strides and new_stride multiples of 8
 *   elements (os: of 4), q, k_new, v_new and the caches 16-byte aligned, o
 *   8-byte aligned (TP_ERR_ALIGN otherwise).
 *   workspace: as for tp_local_attention, of at least
 *   tp_local_attention_workspace(B, 1, pos + 1, Hq, Hkv, D) bytes.
 */
tp_status tp_decode_attention_append(const void* q, const int64_t qs[2],
                                     const void* k_new, const void* v_new, int64_t new_stride,
                                     void* k_cache, void* v_cache, const int64_t cs[3],
                                     int64_t T, int64_t pos, void* o, const int64_t os[2],
                                     int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                     float scale, tp_dtype dt,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_decode_attention_append without the workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The chunk partials go to a buffer
 * the library owns: a static device array of 8,486,400 bytes on each GPU the
 * call runs on, kept until the process ends.  That size covers every call this
 * entry point accepts (a key span is split only for at most 255 (sequence, KV
 * head) pairs); a request needing more returns TP_ERR_WORKSPACE.  The call
 * allocates nothing, and needs no clearing between calls (every partial it
 * reads was written earlier in the same call).
 * All calls on one GPU share that buffer: calls that overlap in time on one
 * GPU (e.g. on two streams) race and give undefined results; serialise them.
 * Results equal tp_decode_attention_append's bit for bit.  Every other
 * argument, limit and error as tp_decode_attention_append; TP_ERR_HIP if the
 * buffer's device address cannot be obtained.
 */
tp_status tp_decode_attention_append_noalloc(const void* q, const int64_t qs[2],
                                             const void* k_new, const void* v_new,
                                             int64_t new_stride, void* k_cache, void* v_cache,
                                             const int64_t cs[3], int64_t T, int64_t pos, void* o,
                                             const int64_t os[2], int64_t B, int64_t Hq,
                                             int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                             void* stream);

/*
 * The arithmetic of the all-reduce after a row-parallel linear (P1 "Row
 * Parallel Linear": the partial outputs are summed; P2 section 二
 * all_reduce(output); P3: partials must be summed, not concatenated),
 * emulated on one GPU as an in-HBM sum of every rank's partial:
 *     y[m, n] = sum_{r=0}^{R-1} partials[r][m, n] (+ residual[m, n])
 * summed in float32 in rank order 0..R-1, the residual added last, then
 * rounded once to out_dt.
 *   partials : host array of R device pointers to [M, N] float32 buffers
 *   residual : [M, N] in res_dt, or NULL (res_dt is then ignored).  A
 *              residual stream kept in float32 is passed with res_dt = TP_F32
 *              while y is bf16, and the other way round.
 *   y        : [M, N] out_dt.  y may be the residual buffer itself when
 *              res_dt == out_dt; any other overlap of the two is TP_ERR_SHAPE.
 *   1 <= R <= 16
 */
tp_status tp_reduce_partials(const float* const* partials, int64_t R,
                             const void* residual, tp_dtype res_dt, void* y,
                             int64_t M, int64_t N, tp_dtype out_dt, void* stream);

/*
 * The all-reduce's arithmetic followed by the next sub-block's pre-norm, in
 * one pass (P2 section 二 all_reduce(output) + the residual; the RMSNorm is
 * the standard pre-norm of a decoder layer, not on the source pages):
 *     y  = sum_{r=0}^{R-1} partials[r] (+ residual)     (as tp_reduce_partials,
 *                                                       stored as y_dt)
 *     yn = y * rsqrt(mean_n y^2 + eps) * gamma          (as tp_rmsnorm on the
 *                                                       stored y)
 * Both outputs equal the two unfused calls bit for bit.  In a pre-norm layer
 * y is the residual stream h (kept in float32 with y_dt = TP_F32, it is never
 * rounded) and yn the normalised input of the next column-parallel GEMM.
 *   partials : host array of R device pointers to [M, N] float32 buffers
 *   residual : [M, N] in res_dt, or NULL;  y : [M, N] in y_dt (may be the
 *   residual buffer itself when res_dt == y_dt; other overlaps TP_ERR_SHAPE);
 *   gamma : [N] dt;  yn : [M, N] dt;  1 <= R <= 16
 */
tp_status tp_reduce_partials_rmsnorm(const float* const* partials, int64_t R,
                                     const void* residual, tp_dtype res_dt,
                                     void* y, tp_dtype y_dt, const void* gamma, void* yn,
                                     int64_t M, int64_t N, float eps, tp_dtype dt, void* stream);

/*
 * Replicated pre-norm RMSNorm (every rank normalises the full hidden row):
 *     y[m, :] = x[m, :] * rsqrt(mean_n x[m, n]^2 + eps) * gamma[:]
 * in float32 arithmetic.  x : [M, N] in x_dt (a float32 residual stream may
 * feed a bf16 normalisation); gamma : [N] and y : [M, N] in dt.
 * Not on the source pages (a standard pre-norm layer's normalisation).
 */
tp_status tp_rmsnorm(const void* x, tp_dtype x_dt, const void* gamma, void* y,
                     int64_t M, int64_t N, float eps, tp_dtype dt, void* stream);

/*
 * Decode attention over the rank's local heads with a paged KV cache (P1
 * "Tensor parallel 对 KV cache 的影响": every rank keeps a KV pool holding only
 * its own heads; the block table is the same on all ranks because blocks are
 * allotted along the token axis; each rank reads the same logical blocks'
 * physical blocks, its heads only).  One query token per sequence:
 *     o[b,h,:] = softmax_t(scale * q[b,h,:] . K_b[t,h/G,:]) V_b[t,h/G,:],  t < L_b
 * where L_b = context_lens[b] and key t of sequence b is slot t % block_size
 * of physical block block_table[b * table_stride + t / block_size]:
 *   q : element (b,h,d) at q[b*qs[0] + h*qs[1] + d]          bf16
 *   k_pool, v_pool : element (blk,slot,j,d) at pool[blk*ps[0] + slot*ps[1] + j*ps[2] + d]
 *   o : element (b,h,d) at o[b*os[0] + h*os[1] + d]          bf16
 *   block_table : int32 [B, table_stride] device; context_lens : int32 [B] device
 *   1 <= context_lens[b] <= max_context_len (values outside are clamped into
 *   that range); table entries outside [0, num_blocks) read as zero K/V.
 *   table_stride >= ceil(max_context_len / block_size) (TP_ERR_SHAPE).
 *   dt must be TP_BF16, D = 128, block_size a multiple of 16, G = Hq/Hkv <= 32
 *   (TP_ERR_UNSUPPORTED otherwise).
 *   workspace: device scratch of tp_paged_attention_workspace(...) bytes (NULL
 *   when 0), caller-owned, used only during the call; overlapping calls must
 *   not share one.
 */
tp_status tp_paged_attention_decode(const void* q, const int64_t qs[2], const void* k_pool,
                                    const void* v_pool, const int64_t ps[3], int64_t num_blocks,
                                    const int32_t* block_table, int64_t table_stride,
                                    const int32_t* context_lens, int64_t max_context_len,
                                    int64_t block_size, void* o, const int64_t os[2], int64_t B,
                                    int64_t Hq, int64_t Hkv, int64_t D, float scale, tp_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream);

size_t tp_paged_attention_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_context_len,
                                    int64_t block_size);

/*
 * Store the current decode token's k and v of every sequence b in its paged
 * slot, position context_lens[b] - 1 (the same P1 section: the rank's pool
 * holds only its heads):
 *   k_new, v_new : element (b,j,d) at k_new[b*new_stride + j*D + d]   bf16
 *   pools, block_table, context_lens as in tp_paged_attention_decode.
 * Sequences whose position or table entry is out of range are skipped.
 */
tp_status tp_paged_kv_append(const void* k_new, const void* v_new, int64_t new_stride, void* k_pool,
                             void* v_pool, const int64_t ps[3], int64_t num_blocks,
                             const int32_t* block_table, int64_t table_stride,
                             const int32_t* context_lens, int64_t B, int64_t Hkv, int64_t D,
                             int64_t block_size, tp_dtype dt, void* stream);

/*
 * The paged cache's append and decode attention in one launch (the same P1
 * section): equal, bit for bit, to tp_paged_kv_append(...) followed by
 * tp_paged_attention_decode(...) with the same arguments, provided no slot
 * written by the append is read by another sequence of the call or through a
 * second table entry (no block shared with a sequence that reads that slot,
 * no block listed twice up to a sequence's length).
 *   k_new, v_new : element (b,j,d) at k_new[b*new_stride + j*D + d]   bf16,
 *   16-byte aligned, new_stride >= Hkv*D and a multiple of 8.
 *   Every other argument, limit and error as tp_paged_attention_decode.
 */
tp_status tp_paged_decode_attention_append(const void* q, const int64_t qs[2], const void* k_new,
                                           const void* v_new, int64_t new_stride, void* k_pool,
                                           void* v_pool, const int64_t ps[3], int64_t num_blocks,
                                           const int32_t* block_table, int64_t table_stride,
                                           const int32_t* context_lens, int64_t max_context_len,
                                           int64_t block_size, void* o, const int64_t os[2],
                                           int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                           float scale, tp_dtype dt, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * Greedy token choice of a vocab-parallel lm_head (P1 "lm_head 怎么处理": the
 * lm_head is split by vocab rows, column-parallel; under greedy decoding each
 * rank takes the largest logit of its vocab block and an all-gather /
 * all-reduce of those pairs finds the global one).
 *
 * Local step, per token row m of the rank's logits:
 *     (max_val[m], max_idx[m]) = max over j of (logits[m, j], vocab_offset + j)
 * under the order: NaN counts as -inf; a larger value wins; equal values go to
 * the lower vocab id (max_val is -inf when the row holds no number).
 *   logits  : [M, V_r] float32 device, contiguous (e.g. the rank's fp32 logits
 *             from tp_row_linear_partial(h, W_vocab_r, ...))
 *   max_val : [M] float32 device;  max_idx : [M] int64 device (global vocab ids)
 *   vocab_offset: first vocab id of the rank's block (r * V / R for contiguous
 *   blocks).  M, V_r <= 2^31 - 1 (TP_ERR_UNSUPPORTED otherwise).
 */
tp_status tp_vocab_argmax_local(const float* logits, int64_t M, int64_t V_r, int64_t vocab_offset,
                                float* max_val, int64_t* max_idx, void* stream);

/*
 * The exchange's arithmetic on one GPU: combine the R ranks' local pairs in
 * rank order with the same order as above (ties -> lowest vocab id), giving
 * the argmax over the full vocab.
 *   vals : host array of R device pointers to [M] float32
 *   idxs : host array of R device pointers to [M] int64
 *   out_val : [M] float32, out_idx : [M] int64 (device);  1 <= R <= 64
 */
tp_status tp_vocab_argmax_reduce(const float* const* vals, const int64_t* const* idxs, int64_t R,
                                 int64_t M, float* out_val, int64_t* out_idx, void* stream);

/* Static text for a status code. */
const char* tp_status_string(tp_status s);

/* Text of the last TP_ERR_HIP failure on the calling thread ("" if none). */
const char* tp_last_error(void);

/* Library version string. */
const char* tp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TPLAYER_H */
