/*
 * mqa_qkv.h -- C ABI of the fused QKV projection + grouped-query attention
 * library for AMD Instinct MI355X (gfx950).
 *
 * The operations are the hot path of one attention layer:
 *   1. qkv_proj          one GEMM  qkv = x . W_qkv  replacing the separate
 *                        q/k/v projections ("Optimize LlamaAttention by fusing
 *                        QKV projections", transformers PR #40092, the diff of
 *                        LlamaAttention.forward);
 *      qkv_proj_append   the same GEMM for a decode step, also writing the
 *                        new token's K and V rows into the KV caches;
 *      qkv_proj_rope, qkv_proj_append_rope  the same with the rotary
 *                        position embedding of Q and K in the epilogue;
 *   2. the split into Q, K, V is not a call: Q, K and V are strided views of
 *      the packed qkv rows (same diff: query columns first, then key, then
 *      value; within a block the column is head*d + c).  The attention calls
 *      take a token stride, so no copy is ever made;
 *   3. gqa_attn_prefill  exact softmax(scale . Q K^T) V with H_q query heads
 *                        sharing H_kv KV heads ("MHA -> GQA" blog, section 3.2;
 *                        FlashAttention-3 page, the recap of tiling with
 *                        softmax rescaling being exact);
 *      gqa_attn_prefill_varlen  the same over a packed variable-length batch;
 *      gqa_attn_prefill_fp8     the same with the scores computed from e4m3
 *                        Q and K after an incoherent (random-sign Hadamard)
 *                        map (FlashAttention-3 page, FP8 section);
 *   4. gqa_attn_decode   one new query per sequence against a contiguous KV
 *                        cache with per-sequence lengths ("MHA -> GQA" blog,
 *                        section 3.1), split over the keys with an exact
 *                        partial-softmax combine (FlashAttention-3 page, HN
 *                        thread: the softmax is split and recombined);
 *      gqa_attn_decode_paged  the same over a paged KV cache.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller; outputs are
 *     fully overwritten (never accumulated), in the style of an op that
 *     mutates a caller-allocated `out` ("custom op overhead" gist).
 *   - The library never allocates device memory and never synchronises;
 *     calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream) and reentrant.  The one exception to "caller-owned scratch" is
 *     gqa_attn_decode_noalloc, which uses a static per-GPU buffer.
 *   - Arguments are validated on the host before any HIP call.  A rejected
 *     call launches nothing and returns MQKV_ERR_INVALID (malformed) or
 *     MQKV_ERR_UNSUPPORTED (well-formed but not implemented); a failed launch
 *     returns MQKV_ERR_HIP.  mqkv_last_error() gives the thread-local detail.
 *   - Device-side lengths are clamped to their buffers (decode: seq_lens to
 *     [0, L_max]), so no device value leads outside them.
 *   - dtypes: MQKV_BF16 (bf16 storage, fp32 accumulation, round-to-nearest-
 *     even outputs) or MQKV_F32 (fp32 throughout).
 *   - bf16 prefill multiplies P by V on fp16 matrix cores; each 64-key tile
 *     of V is converted as V * 2^-s with a power-of-two exponent s of its own
 *     (s = 0 when the tile lies inside fp16's range) and the accumulator
 *     follows with exact power-of-two rescales, so every finite bf16 V,
 *     however large or small, gives a finite result.  Values at least 2^-29
 *     of their tile's largest |v| convert exactly; smaller ones are rounded
 *     with an absolute error of at most max(2^-39 * that largest |v|, 2^-25)
 *     (a tile's largest |v| includes keys a causal row does not see).  bf16
 *     decode multiplies on bf16 matrix cores, where every finite bf16 V is an
 *     exact operand, with P carried as the sum of two bf16 parts (about 16
 *     bits).
 *   - Alignment: every data pointer 16-byte aligned; element strides multiples
 *     of 8 (bf16) or 4 (fp32) elements.
 */
#ifndef MQA_QKV_H
#define MQA_QKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mqkv_status {
  MQKV_OK = 0,
  MQKV_ERR_INVALID = 1,      /* malformed arguments; nothing launched            */
  MQKV_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. d not 64/128)    */
  MQKV_ERR_HIP = 3           /* a HIP runtime call or launch failed              */
} mqkv_status;

typedef enum mqkv_dtype { MQKV_F32 = 0, MQKV_BF16 = 1 } mqkv_dtype;

/*
 * Fused QKV projection (PR #40092, LlamaAttention.forward diff).
 *
 *   qkv[m, n] = sum_k x[m, k] * w_qkv[k, n] (+ bias[n]),   N = (H_q + 2*H_kv) * d
 *
 * x      [M, hidden]  row-major, dtype `dtype`
 * w_qkv  [hidden, N]  row-major (the x . W orientation; a torch nn.Linear
 *                     weight is its transpose), columns [Q | K | V], head-major
 * bias   [N] or NULL
 * qkv    [M, N]       row-major output
 * workspace, workspace_bytes: optional device scratch (NULL/0 allowed).  With
 *   at least qkv_proj_workspace_bytes(...) bytes, small-M (<= 128 rows) bf16
 *   calls split the hidden dimension over more workgroups and reduce the fp32
 *   partials in a second kernel (fixed order, deterministic); otherwise a
 *   single-pass kernel runs.  The result is within rounding either way.
 * Requires hidden >= 1 and hidden a multiple of 8 (bf16) / 4 (fp32), d in {64, 128},
 * H_q % H_kv == 0.  M == 0 is a no-op.
 */
size_t qkv_proj_workspace_bytes(int64_t M, int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d,
                                mqkv_dtype dtype);

mqkv_status qkv_proj(const void* x, const void* w_qkv, const void* bias, void* qkv,
                     int64_t M, int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d,
                     mqkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-step projection with the KV-cache append fused into its epilogue.
 *
 * The GEMM of qkv_proj with M = B rows, row b being sequence b's new token.
 * The same kernels also write the K and V column blocks of row b into the
 * caches, at that token's position:
 *
 *   k_cache[b, seq_lens[b]-1, g, c] = qkv[b, H_q*d + g*d + c]
 *   v_cache[b, seq_lens[b]-1, g, c] = qkv[b, (H_q+H_kv)*d + g*d + c]
 *
 * so gqa_attn_decode can follow directly with the same seq_lens: the new token
 * is the last attended key, the cache convention of gqa_attn_decode (decode
 * against a cache, "MHA -> GQA" blog, section 3.1).  Both copies of the values
 * are bit-identical.  Nothing else of the caches is touched.  A row b whose
 * seq_lens[b] lies outside [1, L_max] is projected but not appended.
 *
 * k_cache, v_cache [B, L_max, H_kv, d] contiguous, dtype `dtype`, 16-byte aligned
 * seq_lens         [B] device int32: the lengths including the new token
 * x, w_qkv, bias, qkv, workspace (qkv_proj_workspace_bytes(B, ...)) and their
 * requirements are those of qkv_proj; additionally L_max >= 1.  B == 0 is a
 * no-op.  The call allocates and synchronises nothing, so a whole decode step
 * (this call, then gqa_attn_decode) can be captured and replayed as one HIP
 * graph, the launch-overhead remedy the "custom op overhead" gist measures
 * (its eager vs full-graph timing table).
 */
mqkv_status qkv_proj_append(const void* x, const void* w_qkv, const void* bias, void* qkv,
                            void* k_cache, void* v_cache, const int32_t* seq_lens,
                            int32_t B, int64_t hidden, int32_t H_q, int32_t H_kv, int32_t d,
                            int32_t L_max, mqkv_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * qkv_proj with the rotary position embedding of the Q and K heads fused into
 * its epilogue (the positional step the "custom op overhead" gist's forward
 * applies to q and k right after the split; the FlashAttention-3 news page,
 * FP8 section, counts rotary among the memory-bound steps ahead of attention
 * that are best fused).  The pages do not define the rotation; this is
 * RoFormer's: for row m at position p = positions[m], plane i of every Q and
 * K head, its components (2i, 2i+1) at columns c0 + 2i and c0 + 2i + 1 of a
 * head starting at column c0, turns counter-clockwise by
 *
 *   a = fp32(fp32(p) * inv_freq[i])              (one fp32 rounding)
 *   y[2i]   = x[2i] cos a - x[2i+1] sin a
 *   y[2i+1] = x[2i] sin a + x[2i+1] cos a
 *
 * where x is the projection with its bias, in fp32 before the output rounding.
 * V columns are as in qkv_proj.  sin and cos are evaluated on the device to a
 * few fp32 ulps for |a| < 2^22.  Checkpoints that pair components (c, c + d/2)
 * instead use this call after permuting each Q and K head's columns of W (and
 * bias) so that c -> 2c and c + d/2 -> 2c + 1; attention scores are unchanged
 * by such a permutation of Q and K alike.
 *
 * positions [M] device int32 (any values; converted to fp32 exactly for
 *           |p| < 2^24), 4-byte aligned
 * inv_freq  [d/2] device fp32 rotation frequencies theta_i (usually
 *           base^(-2i/d)), 4-byte aligned
 * Other arguments, requirements and errors are those of qkv_proj;
 * MQKV_ERR_INVALID if positions or inv_freq is NULL or misaligned.
 */
mqkv_status qkv_proj_rope(const void* x, const void* w_qkv, const void* bias, void* qkv,
                          const int32_t* positions, const float* inv_freq, int64_t M, int64_t hidden,
                          int32_t H_q, int32_t H_kv, int32_t d, mqkv_dtype dtype, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * qkv_proj_append with the rotary embedding of qkv_proj_rope: row b is rotated
 * at the position of its own cache slot, p = seq_lens[b] - 1 (clamped to
 * [0, L_max - 1] for rows that are not appended), so a decode step reproduces
 * the prefill row at that position.  The appended K is the rotated K (the same
 * bits as qkv's K columns); V is not rotated.  Arguments as qkv_proj_append,
 * plus inv_freq as in qkv_proj_rope (MQKV_ERR_INVALID if NULL or misaligned).
 */
mqkv_status qkv_proj_append_rope(const void* x, const void* w_qkv, const void* bias, void* qkv,
                                 void* k_cache, void* v_cache, const int32_t* seq_lens,
                                 const float* inv_freq, int32_t B, int64_t hidden, int32_t H_q,
                                 int32_t H_kv, int32_t d, int32_t L_max, mqkv_dtype dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Grouped-query attention over a whole sequence (prefill).
 *
 *   q(b,i,h,c) = q[(b*L_q  + i)*q_tok_stride  + h*d + c]
 *   k(b,j,g,c) = k[(b*L_kv + j)*kv_tok_stride + g*d + c]   (v likewise)
 *   query head h reads KV head g = h / (H_q / H_kv)  (contiguous groups)
 *   O(b,i,h,:) = sum_j softmax_j(scale * q(b,i,h,:) . k(b,j,g,:)) v(b,j,g,:)
 *   causal: key j is visible to query i iff j <= i + (L_kv - L_q)
 *           (bottom-right alignment; requires L_q <= L_kv)
 *
 * With q = qkv, k = qkv + H_q*d, v = qkv + (H_q+H_kv)*d and both strides = N,
 * this consumes qkv_proj's output in place.
 * o    [B, L_q, H_q, d] contiguous, dtype o_dtype (bf16 or fp32 for bf16 inputs;
 *      fp32 for fp32 inputs)
 * lse  [B, H_q, L_q] fp32 natural-log normaliser ln sum_j exp(scale q.k_j), or NULL
 * workspace: device scratch, 16-byte aligned, at least
 *   gqa_attn_prefill_workspace_bytes(B, L_kv, H_kv, d, in_dtype) bytes (0 for
 *   fp32 inputs, where NULL is allowed).  bf16 calls first write V there once
 *   more, as fp16 key-major tiles ready to be copied into LDS; its contents are
 *   dead after the call.  Calls that share a workspace must not overlap.
 * scale must be finite and >= 0.  B == 0 or L_q == 0 is a no-op; L_kv >= 1.
 */
size_t gqa_attn_prefill_workspace_bytes(int32_t B, int32_t L_kv, int32_t H_kv, int32_t d,
                                        mqkv_dtype in_dtype);

mqkv_status gqa_attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                             int32_t B, int32_t L_q, int32_t L_kv, int32_t H_q, int32_t H_kv,
                             int32_t d, int64_t q_tok_stride, int64_t kv_tok_stride,
                             int32_t causal, float scale, mqkv_dtype in_dtype,
                             mqkv_dtype o_dtype, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Prefill over a packed batch of variable-length sequences (bf16).
 *
 * The variable-length layout the FlashAttention-3 page lists among its further
 * optimisations (its closing section).  Sequence b owns the packed tokens
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q and o, and
 * [cu_seqlens_kv[b], cu_seqlens_kv[b+1]) of k and v; it is attended exactly as
 * gqa_attn_prefill attends one sequence (same head mapping and bottom-right
 * causal alignment per sequence):
 *
 *   q(t,h,c) = q[t*q_tok_stride + h*d + c]     t in [0, total_q)
 *   k(t,g,c) = k[t*kv_tok_stride + g*d + c]    t in [0, total_kv)   (v likewise)
 *
 * cu_seqlens_q, cu_seqlens_kv  [B+1] device int32, non-decreasing, from 0 to
 *                 total_q / total_kv; no sequence longer than max_L_q / max_L_kv.
 *                 Device values are clamped to those bounds, so they never lead
 *                 outside the buffers.
 * o    [total_q, H_q, d] contiguous, dtype o_dtype (bf16 or fp32)
 * lse  [H_q, total_q] fp32 natural-log normalisers, or NULL
 * workspace: at least gqa_attn_prefill_workspace_bytes(B, max_L_kv, H_kv, d,
 *   MQKV_BF16) bytes (the V images).  With at least
 *   gqa_attn_prefill_varlen_workspace_bytes(B, max_L_kv, total_q, H_q, H_kv, d)
 *   bytes (nonzero for B <= 1024) and lengths that differ (total_q !=
 *   B*max_L_q or total_kv != B*max_L_kv) the call also plans a schedule
 *   there: every row block of the batch (a sequence's query block of one KV
 *   head group) is listed by the key tiles it runs, most first, and
 *   persistent workgroups, one per resident slot of the GPU, take the list in
 *   that order, each claiming its next block with one atomic increment of a
 *   counter in the workspace (the FlashAttention-3 page's closing section
 *   lists persistent kernels and variable-length batches among its further
 *   optimisations).  Otherwise the grid has one workgroup per row block of a
 *   max_L_q sequence, sequence by sequence, the heaviest blocks of each
 *   sequence first.  Either way each row is computed alike (d = 128:
 *   bit-identical results; d = 64 small batches may split a block's keys
 *   between two waves on the grid path, which rounds differently).  With
 *   malformed cu_seqlens (decreasing, or lengths summing past total_q) rows
 *   may be left unwritten; no access leaves the buffers.
 * A query row that sees no key (a sequence with no keys, or L_q > L_kv under
 * the causal mask) gets O = 0 and LSE = -inf.  Each sequence's result is
 * bit-identical to a gqa_attn_prefill call on that sequence alone.
 * fp32 inputs return MQKV_ERR_UNSUPPORTED.  B == 0, max_L_q == 0 or
 * total_q == 0 is a no-op; max_L_kv >= 1, total_kv >= 1.
 */
size_t gqa_attn_prefill_varlen_workspace_bytes(int32_t B, int32_t max_L_kv, int32_t total_q, int32_t H_q,
                                               int32_t H_kv, int32_t d);

mqkv_status gqa_attn_prefill_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                    int32_t B, int32_t max_L_q, int32_t max_L_kv, int32_t total_q,
                                    int32_t total_kv, int32_t H_q, int32_t H_kv, int32_t d,
                                    int64_t q_tok_stride, int64_t kv_tok_stride, int32_t causal,
                                    float scale, mqkv_dtype in_dtype, mqkv_dtype o_dtype,
                                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill with FP8 scores and incoherent processing (bf16 inputs, d = 128).
 *
 * The FlashAttention-3 page, FP8 section: outlier features of Q and K inflate
 * the e4m3 quantisation error; multiplying both by one random orthogonal
 * matrix (a Hadamard transform with random signs) leaves Q K^T unchanged and
 * spreads the outliers before the cast.  The call computes
 *
 *   q' = q . diag(signs) . H / sqrt(d),  k' likewise  (H: Sylvester Hadamard;
 *        signs == NULL: q' = q, k' = k, plain FP8 attention)
 *   q8 = e4m3(q' / s_q)   one fp32 scale per query row: s_q = max|q'| / 448
 *   k8 = e4m3(k' / s_k)   one fp32 scale per 64-key tile of each KV head:
 *                         s_k = max |k'| over the tile / 448
 *   S  = scale * (q8 . k8) * s_q * s_k   on the fp8 matrix cores, fp32 sums
 *   O  = softmax(S) V     V and P as in gqa_attn_prefill (V unquantised)
 *
 * e4m3 is the OCP e4m3fn encoding (max 448, no infinities), rounded to nearest
 * even after saturating to +-448.  Layout, GQA mapping, causal alignment, o,
 * lse, strides and alignment are those of gqa_attn_prefill with
 * in_dtype = MQKV_BF16.
 * signs  [d] device fp32 (the random signs, +-1), or NULL; 16-byte aligned.
 *        Other values are used as given (a diagonal scaling then makes the map
 *        non-orthogonal and changes the result).
 * workspace: gqa_attn_prefill_fp8_workspace_bytes(B, L_q, L_kv, H_q, H_kv, d)
 *   bytes, 16-byte aligned: the V tiles of gqa_attn_prefill and the e4m3 K
 *   tiles with their scales, both written by one pre-pass over K and V; Q is
 *   mapped and quantised inside the attention kernel.  Dead after the call.
 * d != 128 returns MQKV_ERR_UNSUPPORTED (the workspace size is then 0).
 */
size_t gqa_attn_prefill_fp8_workspace_bytes(int32_t B, int32_t L_q, int32_t L_kv, int32_t H_q,
                                            int32_t H_kv, int32_t d);

mqkv_status gqa_attn_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const float* signs, int32_t B, int32_t L_q, int32_t L_kv,
                                 int32_t H_q, int32_t H_kv, int32_t d, int64_t q_tok_stride,
                                 int64_t kv_tok_stride, int32_t causal, float scale,
                                 mqkv_dtype o_dtype, void* workspace, size_t workspace_bytes,
                                 void* stream);

/*
 * Bytes of device workspace gqa_attn_decode needs for these sizes: fp32
 * partial outputs and softmax statistics of every work unit.  kv_split: keys
 * per split, 0 = the library's choice.  Returns 0 for arguments
 * gqa_attn_decode would reject.
 */
size_t gqa_attn_decode_workspace_bytes(int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                                       int32_t L_max, int32_t kv_split);

/*
 * One decode step of grouped-query attention over a contiguous KV cache.
 *
 *   q(b,h,c)       = q[b*q_tok_stride + h*d + c]          (e.g. a view of qkv rows)
 *   k_cache, v_cache [B, L_max, H_kv, d] contiguous
 *   seq_lens [B] device int32, clamped to [0, L_max]: sequence b attends to
 *   keys [0, seq_lens[b]) (the new token's K/V are already in the cache).  A
 *   sequence with no keys gets O = 0 and LSE = -inf
 *   o   [B, H_q, d] contiguous (o_dtype), lse [B, H_q] fp32 or NULL
 *
 * The keys of every (sequence, KV head) are cut into work units: splits of
 * kv_split keys (a multiple of 32 in [32, 65536]), or with kv_split = 0 the
 * library's choice -- for large caches an equal share of all attended keys per
 * resident workgroup, crossing sequence boundaries, so that ragged lengths
 * stay balanced.  Each unit writes a partial (max, sum, output) triple to
 * `workspace` and a second kernel combines them exactly (softmax rescaling).
 * For short caches with kv_split = 0 the library may instead merge each
 * segment's partials inside one workgroup and leave the workspace unused; the
 * result is the same to within rounding.
 * workspace: >= gqa_attn_decode_workspace_bytes(...) bytes, 16-byte aligned;
 *   no initial contents needed; calls that overlap must not share one.
 */
mqkv_status gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* seq_lens, void* o, float* lse, int32_t B,
                            int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                            int64_t q_tok_stride, float scale, int32_t kv_split,
                            void* workspace, size_t workspace_bytes, mqkv_dtype in_dtype,
                            mqkv_dtype o_dtype, void* stream);

/*
 * gqa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).
 *
 * Arguments, results and errors are those of gqa_attn_decode.  The split
 * partials go to a static device buffer of MQKV_DECODE_NOALLOC_SCRATCH_BYTES
 * per GPU, held until the process ends; the call allocates and frees nothing.
 * Sizes whose partials need more than that (gqa_attn_decode's workspace for
 * this dtype) return MQKV_ERR_UNSUPPORTED, with nothing launched.  The buffer
 * needs no initial contents.  Every call on one GPU uses the same buffer:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be serialised by the caller.  The first call on a device looks up the
 * buffer's device address (the library's only mutable host state, guarded by
 * a lock).
 */
#define MQKV_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)

mqkv_status gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* seq_lens, void* o, float* lse, int32_t B,
                                    int32_t H_q, int32_t H_kv, int32_t d, int32_t L_max,
                                    int64_t q_tok_stride, float scale, int32_t kv_split,
                                    mqkv_dtype in_dtype, mqkv_dtype o_dtype, void* stream);

/*
 * Decode over a paged KV cache (bf16).
 *
 * The same operation as gqa_attn_decode, with the cache in fixed-size pages
 * (the PagedAttention layout that the "MHA -> GQA" blog, section 3.2, names as
 * non-contiguous storage).  Key j of sequence b is row j % page_size of page
 * block_table[b * pages_per_seq + j / page_size]:
 *
 *   k(b, j, g, c) = k_pages[((page * page_size) + j % page_size) * H_kv * d + g*d + c]
 *
 * (v likewise).  The MFMA path is kept: each 16-key block of a page is read
 * straight into the matrix operands, so the cache needs no gather copy.
 *
 * k_pages, v_pages [num_pages, page_size, H_kv, d] contiguous bf16
 * block_table      [B, pages_per_seq] device int32 page ids.  Only the entries
 *                  covering keys [0, seq_lens[b]) are read.  A page id outside
 *                  [0, num_pages) is never dereferenced: its keys read as
 *                  zero vectors.
 * seq_lens         [B] device int32, clamped to [0, pages_per_seq * page_size];
 *                  a sequence with no keys gets O = 0 and LSE = -inf
 * page_size        a positive multiple of 16
 * Everything else, the workspace (gqa_attn_decode_workspace_bytes with
 * L_max = pages_per_seq * page_size), the split and the results are those of
 * gqa_attn_decode: a paged cache holding the same rows as a contiguous one
 * gives bit-identical outputs.  fp32 inputs return MQKV_ERR_UNSUPPORTED.
 */
mqkv_status gqa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o,
                                  float* lse, int32_t B, int32_t H_q, int32_t H_kv, int32_t d,
                                  int32_t page_size, int32_t pages_per_seq, int32_t num_pages,
                                  int64_t q_tok_stride, float scale, int32_t kv_split,
                                  void* workspace, size_t workspace_bytes, mqkv_dtype in_dtype,
                                  mqkv_dtype o_dtype, void* stream);

/* Static description of a status code. */
const char* mqkv_status_string(mqkv_status s);

/* Thread-local detail of the last non-OK status returned on this thread ("" if none). */
const char* mqkv_last_error(void);

/* ABI version of this header (major*100 + minor). */
int32_t mqkv_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MQA_QKV_H */
