/*
 * pagedkv.h — C ABI of libpagedkv.so: paged KV-cache write and block-table
 * attention decode for AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Every pointer is a DEVICE pointer (memory on the current HIP device) unless it is
 *    marked [host].  Tensors are dense, row-major and contiguous in the shapes given.
 *  - The caller owns every buffer: caches, tables, queries, outputs and workspace.
 *    The write, copy and attention calls allocate nothing, keep no state besides a
 *    thread-local error string, never synchronise, and enqueue work only on `stream`
 *    (a hipStream_t; NULL is the default stream); each returns once its work is
 *    enqueued, so any of them may be recorded into a captured graph (pkv_graph_*).
 *    The exceptions, all marked below: the host block manager (pkv_bm_*), which owns
 *    host memory between its create and destroy, and pkv_graph_end, which instantiates
 *    an executable graph.
 *  - Arguments are checked on the host before anything is enqueued.  A non-zero
 *    return is one of the PKV_ERR_* codes; nothing was enqueued then, and
 *    pkv_last_error() describes the problem.  PKV_ERR_HIP reports a launch failure.
 *  - Every argument is required: no size, count or scale has a default (the pages
 *    warn that a misnamed attention argument silently falls back to scale 1.0 or one
 *    head: "KVCache Optimization Skill", Appendix A, parameter-name table).
 *  - Device-side preconditions that the host cannot check without reading device
 *    memory are listed per call.  The kernels clamp every index they derive from
 *    device data into its buffer, so a violated precondition gives unspecified
 *    values, never an out-of-bounds access.
 *
 * Cache layout ("KVCache Optimization Skill", Layer 3, 3.1; ai6s.net KVCache article,
 * section 4.1, ND branch; hotelren.com "Paged KV Cache and Packed Sequence", 2.1):
 *     cache[num_blocks][block_size][num_kv_heads][head_dim]
 * The flat row index of (physical block P, offset o) is the slot P * block_size + o;
 * logical position p of sequence b lives in slot
 *     block_table[b][p / block_size] * block_size + p % block_size.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef PKV_API
#define PKV_API __attribute__((visibility("default")))
#endif

/* Return codes. */
enum {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,         /* a required pointer is NULL */
    PKV_ERR_SHAPE = -2,        /* a size or count is negative or inconsistent */
    PKV_ERR_DTYPE = -3,        /* unknown dtype code */
    PKV_ERR_UNSUPPORTED = -4,  /* a valid combination this library does not implement */
    PKV_ERR_ALIGN = -5,        /* a pointer is not 16-byte aligned */
    PKV_ERR_SCALE = -6,        /* softmax_scale is NaN, infinite or <= 0 */
    PKV_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required */
    PKV_ERR_HIP = -8           /* the HIP runtime reported an error at launch */
};

/* Element types of caches, queries and outputs. */
enum { PKV_F32 = 0, PKV_BF16 = 1 };

/* Library version (major * 100 + minor). */
PKV_API int pkv_version(void);

/* Text describing the last non-OK status returned on the calling thread. */
PKV_API const char* pkv_last_error(void);

/*
 * slot_mapping for one step: sequence b already holds lens_before[b] tokens and appends
 * n_b = cu_new[b+1] - cu_new[b] tokens, packed in order.  Token t of sequence b is at
 * logical position lens_before[b] + (t - cu_new[b]) and gets
 *     slot_mapping[t] = block_table[b][pos / block_size] * block_size + pos % block_size.
 * ("KVCache Optimization Skill", Layer 3, 3.1 mapping formula and 3.3 slot_mapping
 * construction, of which the sequential form b * max_seq_len + pos is the special case
 * of the identity table; "Paged KV Cache and Packed Sequence", 2.2, index snippet.)
 *
 *   slot_mapping  [num_tokens] int64, written
 *   block_table   [batch][max_blocks_per_seq] int32
 *   lens_before   [batch] int32
 *   cu_new        [batch + 1] int32, cu_new[0] = 0, non-decreasing, cu_new[batch] = num_tokens
 *   block_size    power of two in [1, 256]
 * Device preconditions: each position's logical block < max_blocks_per_seq (else the
 * slot is written as -1, which pkv_kv_cache_write skips).
 */
PKV_API int pkv_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                     const int32_t* lens_before, const int32_t* cu_new,
                     int32_t batch, int64_t num_tokens, int32_t max_blocks_per_seq,
                     int32_t block_size, void* stream);

/*
 * Cache write by slot_mapping: for each token t,
 *     k_cache.view(num_blocks * block_size, num_kv_heads, head_dim_k)[slot_mapping[t]] = k_new[t]
 *     v_cache.view(num_blocks * block_size, num_kv_heads, head_dim_v)[slot_mapping[t]] = v_new[t]
 * A byte copy with no conversion ("KVCache Optimization Skill", Mode 2 step 3 and the
 * division of labour after 3.3: slot_mapping drives writes, block_table drives reads;
 * ai6s.net article, 4.2, cache write loop).
 *
 *   k_new [num_tokens][num_kv_heads][head_dim_k], v_new [num_tokens][num_kv_heads][head_dim_v]
 *   k_cache [num_blocks][block_size][num_kv_heads][head_dim_k], v_cache likewise with head_dim_v
 *   slot_mapping [num_tokens] int64
 * For the MLA latent cache pass (kv_nope, k_rope, cache_nope, cache_rope) with
 * num_kv_heads = 1, head_dim_k = 512, head_dim_v = 64: the two caches share slots.
 * num_tokens = 0 enqueues nothing.
 * Device preconditions: slots in [0, num_blocks * block_size) and distinct within one
 * call (a slot outside the range is skipped; duplicated slots leave either row).
 */
PKV_API int pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim_k, int32_t head_dim_v, int32_t block_size,
                       int64_t num_blocks, int32_t dtype, void* stream);

/*
 * slot_mapping and the cache write in one launch (the two calls above, fused): token i
 * of sequence b (packed row t = cu_new[b] + i) is written to slot
 * block_table[b][pos / block_size] * block_size + pos % block_size, pos = lens_before[b] + i,
 * and that slot is stored in slot_mapping_out[t] when slot_mapping_out is not NULL (so
 * later layers of the same step can call pkv_kv_cache_write with it).
 *   max_new_tokens [host] >= every n_b = cu_new[b+1] - cu_new[b]; batch <= 65535.
 * Other arguments and preconditions as for pkv_slot_mapping and pkv_kv_cache_write.
 */
PKV_API int pkv_kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* lens_before,
                        const int32_t* cu_new, int64_t* slot_mapping_out, int32_t batch,
                        int64_t num_tokens, int32_t max_new_tokens, int32_t max_blocks_per_seq,
                        int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                        int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream);

/*
 * INT8 KV cache.  The pages name the knobs of a quantized cache (antiquant_scale,
 * dequant_scale_key/value: "KVCache Optimization Skill", Layer 3 notes; the ai6s.net article
 * on low-precision caches) but not the scheme.  The one taken: symmetric int8 codes with one
 * fp32 scale per (token, kv head) row,
 *   s = max|x| / 127,  q = round_half_even(x / s) clamped to [-127, 127]  (IEEE fp32 divisions;
 *   a zero row has s = 0 and zero codes),  x ~ q * s.
 * Caches: codes k_cache, v_cache [num_blocks][block_size][num_kv_heads][head_dim] int8 and
 * scales k_scale, v_scale [num_blocks][num_kv_heads][block_size] fp32: the scale of slot
 * (block P, offset o) and kv head h is at (P * num_kv_heads + h) * block_size + o, so a
 * block's scales of one head are adjacent (the decode reads a run of tokens' scales at once).
 *
 * pkv_kv_cache_write_int8: quantize k_new, v_new [num_tokens][num_kv_heads][head_dim]
 * (dtype f32 or bf16) row by row and store codes and scales at slot_mapping[t] (int64;
 * slots outside the pool are skipped).  head_dim 64 or 128; all arrays 16-byte aligned;
 * K and V arrays distinct.
 */
PKV_API int pkv_kv_cache_write_int8(const void* k_new, const void* v_new, void* k_cache,
                            void* v_cache, float* k_scale, float* v_scale,
                            const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int64_t num_blocks,
                            int32_t dtype, void* stream);

/*
 * Decode over the INT8 caches: as pkv_paged_attn_decode_ex without the new-token write (write
 * it first with pkv_kv_cache_write_int8), with bf16 q and out, head_dim 64 or 128, and 1..16
 * query heads per kv head; with 5..16 of them block_size must be at least 1024 / head_dim
 * (8 or 16) and batch at most 1024, else PKV_ERR_UNSUPPORTED.  score = scale * s_k * (q . q_k),
 * out = sum softmax * s_v * q_v, accumulated in fp32.  window, stages and workspace as for
 * pkv_paged_attn_decode_ex (pkv_decode_workspace_size bytes suffice).
 */
PKV_API int pkv_paged_attn_decode_int8(void* out, float* lse_out, const void* q, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* seq_lens_kv,
                               int32_t batch, int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int64_t num_blocks, float softmax_scale,
                               int32_t window, int32_t stages, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * The INT8 decode step with the quantizing write folded into the pass: for each sequence b, the step's bf16 rows k_new[b], v_new[b] [batch][Hkv][head_dim]
 * are quantized exactly as pkv_kv_cache_write_int8 does (the same codes and scales, bit for
 * bit), stored at logical position seq_lens_kv[b] - 1 (its slot in slot_mapping_out [batch],
 * or -1 for a row longer than max_seq_len_kv, which writes nothing), and attended to with
 * the other seq_lens_kv[b] - 1 cached tokens.  Equal to slot_mapping + pkv_kv_cache_write_int8
 * + pkv_paged_attn_decode_int8, in one pass ("KVCache Optimization Skill", 3.6: write by
 * slot_mapping, then attention reads kv_len + 1 tokens; Layer 3 notes on the quantized cache).
 * Any of 1..16 query heads per kv head (with 5..16 the range that holds a sequence's last
 * key writes it before reading it back).  Other arguments, stages, workspace and
 * preconditions as for pkv_paged_attn_decode_int8.
 */
PKV_API int pkv_paged_attn_decode_int8_append(void* out, float* lse_out, const void* q,
                                      const void* k_new, const void* v_new, void* k_cache,
                                      void* v_cache, float* k_scale, float* v_scale,
                                      const int32_t* block_table, const int32_t* seq_lens_kv,
                                      int64_t* slot_mapping_out, int32_t batch,
                                      int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks, float softmax_scale,
                                      int32_t window, int32_t stages, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * INT8 MLA latent cache: the 512-wide nope row and the 64-wide rope row of each token are
 * quantized separately by the scheme above (one fp32 scale each per token):
 *   nope_codes [num_blocks][block_size][512] int8, rope_codes [num_blocks][block_size][64]
 *   int8, nope_scale and rope_scale [num_blocks][block_size] fp32 (one kv head: slot order).
 * pkv_kv_cache_write_int8_mla: quantize kv_nope [num_tokens][512] and k_rope
 * [num_tokens][64] (f32 or bf16) into them at slot_mapping (slots outside the pool are
 * skipped); all arrays 16-byte aligned.
 * pkv_paged_attn_decode_mla_int8: the MLA-absorbed decode of pkv_paged_attn_decode over
 * these caches: score = scale * (s_nope * (q . codes_nope) + s_rope * (q_rope . codes_rope)),
 * out = sum softmax * s_nope * codes_nope; bf16 q, q_rope and out; block_size >= 4 (a power
 * of two); num_q_heads, workspace (pkv_decode_workspace_size with 1 kv head and head_dim_v
 * 512), stages and preconditions as for the MLA form of pkv_paged_attn_decode /
 * pkv_paged_attn_decode_split / _combine (stages 1, 2, 3).
 */
PKV_API int pkv_kv_cache_write_int8_mla(const void* kv_nope, const void* k_rope, void* nope_codes,
                                        void* rope_codes, float* nope_scale, float* rope_scale,
                                        const int64_t* slot_mapping, int64_t num_tokens,
                                        int32_t block_size, int64_t num_blocks, int32_t dtype,
                                        void* stream);
PKV_API int pkv_paged_attn_decode_mla_int8(void* out, float* lse_out, const void* q, const void* q_rope,
                                           const void* nope_codes, const void* rope_codes,
                                           const float* nope_scale, const float* rope_scale,
                                           const int32_t* block_table, const int32_t* seq_lens_kv,
                                           int32_t batch, int32_t max_blocks_per_seq,
                                           int32_t max_seq_len_kv, int32_t num_q_heads,
                                           int32_t block_size, int64_t num_blocks,
                                           float softmax_scale, int32_t stages, void* workspace,
                                           size_t workspace_bytes, void* stream);

/*
 * The MLA-absorbed decode step over the INT8 latent cache with the quantizing write folded
 * into the pass: for each sequence b the step's bf16 latent rows nope_new[b] [batch][512] and
 * rope_new[b] [batch][64] are quantized exactly as pkv_kv_cache_write_int8_mla does (the same
 * codes and scales, bit for bit), stored at logical position seq_lens_kv[b] - 1 (its slot in
 * slot_mapping_out [batch], or -1 for a row longer than max_seq_len_kv, which writes nothing),
 * and attended to with the other seq_lens_kv[b] - 1 cached tokens.  Equal to slot_mapping +
 * pkv_kv_cache_write_int8_mla + pkv_paged_attn_decode_mla_int8, in one pass ("KVCache
 * Optimization Skill", 3.6: write by slot_mapping, then attention reads kv_len + 1 tokens;
 * Mode 3, the compressed latent cache).  The caches and scales are written; the nope and rope
 * arrays must be distinct.  Other arguments, stages, workspace and preconditions as for
 * pkv_paged_attn_decode_mla_int8.
 */
PKV_API int pkv_paged_attn_decode_mla_int8_append(void* out, float* lse_out, const void* q,
                                          const void* q_rope, const void* nope_new,
                                          const void* rope_new, void* nope_codes, void* rope_codes,
                                          float* nope_scale, float* rope_scale,
                                          const int32_t* block_table, const int32_t* seq_lens_kv,
                                          int64_t* slot_mapping_out, int32_t batch,
                                          int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                          int32_t num_q_heads, int32_t block_size,
                                          int64_t num_blocks, float softmax_scale, int32_t stages,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The MLA latent row normalised, rotated and written in one launch: the fused writer the
 * pages place in front of the MLA cache (npu_kv_rmsnorm_rope_cache, keyed by slot_mapping;
 * "KVCache Optimization Skill", Mode 3 and its cache-write fusion note), which they name
 * without defining.  Readings taken: for token t with kv[t] = [c | k_pe],
 *   cache_nope[slot_t] = c / sqrt(mean(c^2) + eps) * gamma                 (RMSNorm)
 *   cache_rope[slot_t] = [x1 cos - x2 sin | x2 cos + x1 sin]                (rotary, half-split)
 * with x1 = k_pe[:Dr/2], x2 = k_pe[Dr/2:], cos = cos[t], sin = sin[t] (the caller's angles for
 * the token's position).  fp32 arithmetic, one rounding to the cache dtype.
 *   kv [num_tokens][head_dim_nope + head_dim_rope], gamma [head_dim_nope], both in dtype
 *   cos, sin [num_tokens][head_dim_rope / 2] fp32
 *   cache_nope [num_blocks][block_size][1][head_dim_nope], cache_rope [...][1][head_dim_rope]
 *   slot_mapping [num_tokens] int64 (as for pkv_kv_cache_write; slots outside the pool are
 *   skipped)
 * Supported: f32 or bf16; head_dim_nope a multiple of 16 bytes' worth of elements, at most
 * 1024 (bf16) / 512 (f32); head_dim_rope a multiple of 32 bytes' worth, at most 256 / 128.
 * All arrays 16-byte aligned.
 */
PKV_API int pkv_kv_rmsnorm_rope_cache(const void* kv, const void* gamma, const float* cos,
                              const float* sin, void* cache_nope, void* cache_rope,
                              const int64_t* slot_mapping, int64_t num_tokens,
                              int32_t head_dim_nope, int32_t head_dim_rope, int32_t block_size,
                              int64_t num_blocks, float eps, int32_t dtype, void* stream);

/*
 * Bytes of workspace pkv_paged_attn_decode needs for these sizes (0 if none).  The
 * workspace holds split-KV partial results; its contents need no initialisation, and
 * calls that may run at the same time need separate workspaces.
 */
PKV_API size_t pkv_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim_v, int32_t max_seq_len_kv);

/*
 * Paged-attention decode: one query row per sequence and head attends to all
 * seq_lens_kv[b] cached tokens of its sequence, read through block_table
 * ("KVCache Optimization Skill", Mode 2 step 4, 3.6 data flow — the decode reads
 * kv_len + 1 tokens, the token just written included — and Appendix E, decode uses no
 * mask; Mode 3 for MLA; "Paged KV Cache and Packed Sequence", 3.3 and 4.2).
 *
 *   out [batch][num_q_heads][head_dim_v], same dtype as q, written
 *   lse_out [batch][num_q_heads] fp32 natural-log sum-exp of the scaled scores, or NULL
 *   q [batch][num_q_heads][head_dim_qk]
 *   q_rope [batch][num_q_heads][head_dim_rope] or NULL
 *   k_cache [num_blocks][block_size][num_kv_heads][head_dim_qk]
 *   v_cache [num_blocks][block_size][num_kv_heads][head_dim_v]  (MLA: the same pointer
 *           as k_cache — value = cache_nope)
 *   k_rope_cache [num_blocks][block_size][num_kv_heads][head_dim_rope] or NULL; given
 *           exactly when q_rope is (skill page, Mode 3 constraints)
 *   block_table [batch][max_blocks_per_seq] int32; seq_lens_kv [batch] int32 (= L'_b)
 *   max_seq_len_kv [host] an upper bound of seq_lens_kv, <= max_blocks_per_seq * block_size
 *   softmax_scale [host] > 0 (e.g. 1/sqrt(head_dim); MLA 1/sqrt(512 + 64))
 *   workspace: at least pkv_decode_workspace_size(...) bytes, 16-byte aligned (may be
 *           NULL when that size is 0)
 * score(h, p) = softmax_scale * (q[h] . K_p + q_rope[h] . Krope_p) with K/V of kv head
 * h / (num_q_heads / num_kv_heads); out[h] = sum_p softmax(score)_p * V_p.
 * Supported: MHA/GQA with head_dim_qk = head_dim_v in {64, 128}, 1 <= q heads per kv
 * head <= 16, f32 or bf16; MLA with num_kv_heads = 1, head_dim_qk = head_dim_v = 512,
 * head_dim_rope = 64, bf16, num_q_heads a multiple of 16.  block_size a power of two in
 * [1, 256].  Accumulation is fp32; out is rounded once to its dtype.
 * Device preconditions: 0 <= seq_lens_kv[b] <= max_seq_len_kv; block_table entries for
 * the logical blocks in use lie in [0, num_blocks); entries past them are never read.
 * Padding rows: seq_lens_kv[b] = 0 marks a row with no sequence (a batch kept at a fixed
 * size, as a captured step needs): its out is 0 and its lse -inf, and no block_table
 * entry of it is read.  The same holds for every decode entry point below; the append
 * forms also write no cache row for it and report slot -1 in slot_mapping_out[b].
 */
PKV_API int pkv_paged_attn_decode(void* out, float* lse_out, const void* q, const void* q_rope,
                          const void* k_cache, const void* v_cache, const void* k_rope_cache,
                          const int32_t* block_table, const int32_t* seq_lens_kv,
                          int32_t batch, int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                          int32_t head_dim_v, int32_t head_dim_rope, int32_t block_size,
                          int64_t num_blocks, float softmax_scale, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two launches pkv_paged_attn_decode makes, exposed separately (same arguments, same
 * checks) so a caller can time or schedule them on their own.  _split runs the split-KV
 * pass: rows of sequences that fit one split are finished in `out`/`lse_out`, the others
 * leave partial softmax states (max, sum, unnormalised output per split) in `workspace`.
 * _combine then merges those states (out = sum_s e^(m_s - M) o_s / sum_s e^(m_s - M) l_s,
 * lse = M + log of that sum, M = max_s m_s) and enqueues nothing when no row was split.
 * Calling _split then _combine on one stream equals pkv_paged_attn_decode, bit for bit.
 */
PKV_API int pkv_paged_attn_decode_split(void* out, float* lse_out, const void* q, const void* q_rope,
                                const void* k_cache, const void* v_cache,
                                const void* k_rope_cache, const int32_t* block_table,
                                const int32_t* seq_lens_kv, int32_t batch,
                                int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                                int32_t head_dim_v, int32_t head_dim_rope, int32_t block_size,
                                int64_t num_blocks, float softmax_scale, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream);
PKV_API int pkv_paged_attn_decode_combine(void* out, float* lse_out, const void* q, const void* q_rope,
                                  const void* k_cache, const void* v_cache,
                                  const void* k_rope_cache, const int32_t* block_table,
                                  const int32_t* seq_lens_kv, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim_qk, int32_t head_dim_v,
                                  int32_t head_dim_rope, int32_t block_size, int64_t num_blocks,
                                  float softmax_scale, int32_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * One decode step of one layer with the cache write folded into the attention pass:
 * for each sequence b, the new K/V row of this step (k_new[b], v_new[b]) is stored at
 * logical position seq_lens_kv[b] - 1, and query b attends to all seq_lens_kv[b] tokens,
 * that one included.  Equal to pkv_kv_cache_append (one token per sequence,
 * lens_before = seq_lens_kv - 1) followed by pkv_paged_attn_decode, in one pass over the
 * cache: the new token's K/V are taken from k_new/v_new instead of being read back
 * ("KVCache Optimization Skill", 3.6: write by slot_mapping, then attention reads
 * kv_len + 1 tokens).
 *   k_new, v_new [batch][num_kv_heads][head_dim], 16-byte aligned
 *   slot_mapping_out [batch] int64 or NULL: the slot written for each sequence
 *   stages: 1 = the split pass only (writes, single-split rows, partial states),
 *           2 = the combine pass only, 3 = both.  1 then 2 on one stream equals 3.
 * MHA/GQA only (no rope); other arguments, workspace and preconditions as for
 * pkv_paged_attn_decode (with head_dim_qk = head_dim_v = head_dim).
 */
PKV_API int pkv_paged_attn_decode_append(void* out, float* lse_out, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens_kv,
                                 int64_t* slot_mapping_out, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float softmax_scale,
                                 int32_t dtype, int32_t stages, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * The MLA-absorbed decode step with the cache write folded into the pass: for each
 * sequence b, the step's latent row (nope_new[b] [512], rope_new[b] [64], bf16) is the key
 * and value at position seq_lens_kv[b] - 1, read from those rows, and stored at its slot of
 * cache_nope / cache_rope (reported in slot_mapping_out [batch], or -1 for a row longer than
 * max_seq_len_kv, which writes nothing).  Equal to pkv_kv_cache_append of the two rows
 * followed by pkv_paged_attn_decode with q_rope ("KVCache Optimization Skill", Mode 3 and
 * 3.6: write by slot_mapping, then attention reads kv_len + 1 tokens).
 *   q_nope [batch][num_q_heads][512], q_rope [batch][num_q_heads][64], out like q_nope;
 *   cache_nope [nb][bs][1][512], cache_rope [nb][bs][1][64]; stages and workspace as for
 *   pkv_paged_attn_decode_append (pkv_decode_workspace_size(batch, Hq, 1, 512, max) bytes).
 */
PKV_API int pkv_paged_attn_decode_mla_append(void* out, float* lse_out, const void* q_nope,
                                     const void* q_rope, const void* nope_new,
                                     const void* rope_new, void* cache_nope, void* cache_rope,
                                     const int32_t* block_table, const int32_t* seq_lens_kv,
                                     int64_t* slot_mapping_out, int32_t batch,
                                     int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                     int32_t num_q_heads, int32_t block_size, int64_t num_blocks,
                                     float softmax_scale, int32_t stages, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * Packed varlen attention over the paged cache: sequence b owns query rows
 * [cu_seqlens_q[b], cu_seqlens_q[b+1]) of the packed stream (n_b rows) and
 * seq_lens_kv[b] = L'_b cached tokens, its own new rows included (they were written
 * with pkv_kv_cache_write first).  With causal != 0, row i of sequence b sees keys
 * p <= L'_b - n_b + i (bottom-right causal, the query's own token included); with
 * causal = 0 it sees all L'_b keys.  Queries of different sequences never see each
 * other ("Paged KV Cache and Packed Sequence", 3.1-3.3 and 4.1; "KVCache Optimization
 * Skill", Appendix C, sparse_mode 3, and Appendix E).
 *
 *   out [total_q][num_q_heads][head_dim], q [total_q][num_q_heads][head_dim]
 *   lse_out [total_q][num_q_heads] fp32 or NULL
 *   cu_seqlens_q [batch + 1] int32 (cu_seqlens_q[0] = 0); seq_lens_kv [batch] int32
 *   max_seqlen_q [host] >= every n_b
 * Supported: head_dim in {64, 128}, 1 <= q heads per kv head <= 16, bf16;
 * block_size a power of two in [1, 256].
 * Device preconditions: n_b <= seq_lens_kv[b]; table entries as for decode.
 */
PKV_API int pkv_paged_attn_varlen(void* out, float* lse_out, const void* q,
                          const int32_t* cu_seqlens_q, const int32_t* seq_lens_kv,
                          const void* k_cache, const void* v_cache, const int32_t* block_table,
                          int32_t batch, int64_t total_q, int32_t max_seqlen_q,
                          int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int64_t num_blocks,
                          float softmax_scale, int32_t causal, int32_t dtype, void* stream);

/*
 * Sliding-window (band) forms.  The band is sparse_mode 4 with pre_tokens ("KVCache
 * Optimization Skill", Appendix C: sliding-window models), read as: a query row sees only
 * the `window` most recent of the keys it would otherwise see, its own position included,
 * i.e. positions [hi - window + 1, hi] with hi its last visible position (pre_tokens =
 * window - 1; the LLM-serving page's "keep only the latest N tokens" is window = N).
 * window = 0 keeps every key (the forms above); window < 0 is PKV_ERR_SHAPE.
 *
 * pkv_paged_attn_decode_ex: MHA/GQA decode (no rope) with the window; with k_new and v_new
 * given it is pkv_paged_attn_decode_append (the new row of each sequence is written at
 * position seq_lens_kv[b] - 1 and read from k_new/v_new), with both NULL a plain decode
 * over the cache (slot_mapping_out then unused).  stages as for decode_append; workspace:
 * pkv_decode_workspace_size(...) bytes suffice for any window.  Other arguments, support
 * and preconditions as for pkv_paged_attn_decode_append / pkv_paged_attn_decode.
 * MTP decode (next_n + 1 query tokens per sequence, causal): pkv_paged_attn_decode_mtp
 * below, or pkv_paged_attn_varlen(_ex) with n_b = next_n + 1 (skill page, Appendix E).
 */
PKV_API int pkv_paged_attn_decode_ex(void* out, float* lse_out, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens_kv,
                             int64_t* slot_mapping_out, int32_t batch, int32_t max_blocks_per_seq,
                             int32_t max_seq_len_kv, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float softmax_scale, int32_t dtype, int32_t window, int32_t stages,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): pkv_paged_attn_decode_append (both
 * passes, stages = 3) with no workspace argument.  The split pass keeps its partial states
 * in a fixed array inside the library, PKV_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, which
 * each GPU the library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc, no allocating library routine); the caller still owns q, the new rows, the
 * caches, the table, the lengths, out, lse_out and slot_mapping_out.
 *   - A batch whose partial states exceed the array (pkv_decode_workspace_size(...) above
 *     PKV_NOALLOC_SCRATCH_BYTES; the Llama-7B decode layer with 32 sequences of up to 2K
 *     tokens needs about 4.3 MB) returns PKV_ERR_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on a GPU (two
 *     streams, two host threads) race and give undefined results; calls ordered on one
 *     stream are safe.  Nothing in the array needs clearing between calls.
 *   - The stream must belong to the current device (its copy of the array is looked up once,
 *     on the first call on that device).
 * Arguments, support, preconditions and results as for pkv_paged_attn_decode_append.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
PKV_API int pkv_paged_attn_decode_append_noalloc(void* out, float* lse_out, const void* q,
                                         const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens_kv, int64_t* slot_mapping_out,
                                         int32_t batch, int32_t max_blocks_per_seq,
                                         int32_t max_seq_len_kv, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int64_t num_blocks,
                                         float softmax_scale, int32_t dtype, void* stream);

/*
 * Multi-token decode (MTP: next_n + 1 = num_q_tokens query tokens per sequence, causal;
 * "KVCache Optimization Skill", Appendix E, sparse_mode 3 with next_n): sequence b's rows
 * are q[b * num_q_tokens + i], i < num_q_tokens, the last num_q_tokens of its
 * seq_lens_kv[b] cached tokens (written beforehand with pkv_kv_cache_write).  Row i sees
 * keys p <= seq_lens_kv[b] - num_q_tokens + i (and, with window > 0, the `window` most
 * recent of those).  The same result as pkv_paged_attn_varlen_ex with
 * cu_seqlens_q[b] = b * num_q_tokens and causal = 1, computed like a decode: each K/V row is
 * read once per kv head for all the sequence's query tokens and heads.
 *   q, out [batch * num_q_tokens][num_q_heads][head_dim]; lse_out [batch * num_q_tokens][num_q_heads]
 *   workspace: pkv_decode_mtp_workspace_size(...) bytes, 16-byte aligned
 *   stages: 1 = the range pass, 2 = the combine pass, 3 = both (1 then 2 equals 3).
 * Supported: bf16, head_dim 64 or 128, num_q_tokens * (num_q_heads / num_kv_heads) <= 16,
 * block_size >= 4 (head_dim 128) / 8 (head_dim 64), batch <= 1024; other shapes return
 * PKV_ERR_UNSUPPORTED (pkv_paged_attn_varlen_ex covers them).  Device preconditions:
 * num_q_tokens <= seq_lens_kv[b] <= max_seq_len_kv, or seq_lens_kv[b] = 0 (padding: the
 * sequence's rows are 0 with lse -inf); table entries as for pkv_paged_attn_decode.
 */
PKV_API size_t pkv_decode_mtp_workspace_size(int32_t batch, int32_t num_q_tokens,
                                             int32_t num_q_heads, int32_t num_kv_heads,
                                             int32_t head_dim_v, int32_t max_seq_len_kv);
PKV_API int pkv_paged_attn_decode_mtp(void* out, float* lse_out, const void* q,
                                      const void* k_cache, const void* v_cache,
                                      const int32_t* block_table, const int32_t* seq_lens_kv,
                                      int32_t batch, int32_t num_q_tokens,
                                      int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      float softmax_scale, int32_t dtype, int32_t window,
                                      int32_t stages, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * MTP decode with the step's cache write folded into the pass ("KVCache Optimization
 * Skill", 3.6 and Appendix E): sequence b's num_q_tokens new K/V rows
 * k_new/v_new[b * num_q_tokens + i] are stored at positions seq_lens_kv[b] - num_q_tokens + i
 * (the query tokens' own positions) and read from k_new/v_new by the attention, which is
 * pkv_paged_attn_decode_mtp over the cache after those writes; for valid inputs, equal bit
 * for bit to pkv_kv_cache_append (lens_before = seq_lens_kv - num_q_tokens) followed by
 * pkv_paged_attn_decode_mtp, in one attention launch.  The slot of row b * num_q_tokens + i
 * goes to slot_mapping_out[b * num_q_tokens + i] when it is not NULL; a sequence longer
 * than max_seq_len_kv writes nothing (slots -1), as for pkv_paged_attn_decode_append.
 *   k_new, v_new [batch * num_q_tokens][num_kv_heads][head_dim], 16-byte aligned
 * stages (1 the range pass with the writes, 2 the combine, 3 both), workspace, support and
 * other preconditions as for pkv_paged_attn_decode_mtp.
 */
PKV_API int pkv_paged_attn_decode_mtp_append(void* out, float* lse_out, const void* q, const void* k_new,
                                     const void* v_new, void* k_cache, void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens_kv,
                                     int32_t batch, int32_t num_q_tokens, int32_t max_blocks_per_seq,
                                     int32_t max_seq_len_kv, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, float softmax_scale, int32_t dtype,
                                     int32_t window, int32_t stages, void* workspace,
                                     size_t workspace_bytes, int64_t* slot_mapping_out, void* stream);

/* pkv_paged_attn_varlen with the window (causal or not: hi = the row's last visible key). */
PKV_API int pkv_paged_attn_varlen_ex(void* out, float* lse_out, const void* q,
                             const int32_t* cu_seqlens_q, const int32_t* seq_lens_kv,
                             const void* k_cache, const void* v_cache, const int32_t* block_table,
                             int32_t batch, int64_t total_q, int32_t max_seqlen_q,
                             int32_t max_blocks_per_seq, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float softmax_scale, int32_t causal, int32_t window, int32_t dtype,
                             void* stream);

/*
 * One packed chunk with its cache write folded into the attention pass ("KVCache
 * Optimization Skill", 3.6: the step's K/V are written by slot, then attention reads the
 * cached tokens and the new ones; "Paged KV Cache and Packed Sequence", 4.1).  Sequence b's
 * n_b new rows k_new/v_new[cu_seqlens_q[b] + i] are stored at logical position
 * pos = seq_lens_kv[b] - n_b + i, slot block_table[b][pos / block_size] * block_size +
 * pos % block_size (the slot rule of pkv_kv_cache_append with lens_before = seq_lens_kv -
 * n_b: -1 for pos < 0 or pos >= max_blocks_per_seq * block_size, nothing written for a slot
 * outside [0, num_blocks * block_size)); the slot goes to slot_mapping_out[cu_seqlens_q[b] + i]
 * when slot_mapping_out is not NULL.  The attention is pkv_paged_attn_varlen_ex over the
 * cache after those writes, the new keys read from k_new/v_new instead of back from the
 * cache.  For valid inputs the result equals pkv_kv_cache_append followed by
 * pkv_paged_attn_varlen_ex bit for bit (out, lse, both caches, slots), in one launch.
 *   k_new, v_new [total_q][num_kv_heads][head_dim], q's dtype, 16-byte aligned, distinct
 *           from the caches
 *   slot_mapping_out [total_q] int64 or NULL
 * Other arguments, support and preconditions as for pkv_paged_attn_varlen_ex; the written
 * slots must not be read as cached keys by any row of the call (distinct positions in
 * blocks no other sequence reads, as copy on write ensures).
 */
PKV_API int pkv_paged_attn_varlen_append(void* out, float* lse_out, const void* q, const void* k_new,
                                 const void* v_new, const int32_t* cu_seqlens_q,
                                 const int32_t* seq_lens_kv, void* k_cache, void* v_cache,
                                 const int32_t* block_table, int32_t batch, int64_t total_q,
                                 int32_t max_seqlen_q, int32_t max_blocks_per_seq,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float softmax_scale,
                                 int32_t causal, int32_t window, int32_t dtype,
                                 int64_t* slot_mapping_out, void* stream);

/*
 * ---------------------------------------------------------------- block management
 * Host block manager of one cache pool ("Paged KV Cache and Packed Sequence", 2.1-2.2,
 * 5.2 and 5.3).  [host] only: no call touches the GPU.  A manager owns num_blocks
 * physical blocks of block_size slots, a free list, a reference count per block, and per
 * sequence (a caller-chosen int64 id) its length and logical -> physical block list.
 *  - Blocks are taken from the end of the free list (the block freed last is reused
 *    first) and only when a token crosses into a new logical block.
 *  - pkv_bm_fork gives `child` the blocks of `parent` and raises each block's count
 *    (prefix sharing: beam search, parallel sampling).
 *  - pkv_bm_free lowers the counts of all of a sequence's blocks, then returns the
 *    blocks whose count reached 0 to the free list in the sequence's block order.
 *  - Copy on write: when pkv_bm_append must write into a partly filled last block that
 *    another sequence shares, it takes a fresh block in its place and reports the pair
 *    (shared block, fresh block) in copy_out; the caller copies that block's rows
 *    (pkv_kv_cache_copy_blocks, once per cache array) before writing the new rows.
 * Calls return PKV_OK or a PKV_ERR_* code and then change nothing: PKV_ERR_SHAPE for an
 * unknown or duplicate id, or a sequence longer than max_blocks_per_seq blocks;
 * PKV_ERR_WORKSPACE when the free list cannot cover an append (the cache is full).
 * A manager is not thread safe; calls on one manager must not overlap.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* New manager with every block free; NULL (and pkv_last_error) on invalid sizes. */
PKV_API pkv_block_manager* pkv_bm_create(int64_t num_blocks, int32_t block_size,
                                         int32_t max_blocks_per_seq);
/* Frees the manager and all it holds (NULL is a no-op). */
PKV_API void pkv_bm_destroy(pkv_block_manager* bm);
/* Blocks on the free list (-1 for NULL). */
PKV_API int64_t pkv_bm_num_free(const pkv_block_manager* bm);
/* Registers an empty sequence (ids are >= 0; negative ids mark padding rows below). */
PKV_API int pkv_bm_add(pkv_block_manager* bm, int64_t seq);
/* Registers `child` (a new id >= 0) sharing every block of `parent` (same length). */
PKV_API int pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
/*
 * Extends `seq` by num_tokens >= 0 tokens.  slots_out [host] [num_tokens] int64 or NULL:
 * the slot of each new token (block * block_size + offset), in order, ready for
 * pkv_kv_cache_write.  copy_out [host] [2] int64 and num_copies [host]: *num_copies is
 * set to 0 or 1, and to 1 with copy_out = {source block, destination block} when a shared
 * last block was copied on write; both may be NULL only when no copy is needed (else
 * PKV_ERR_NULL and nothing changes).
 */
PKV_API int pkv_bm_append(pkv_block_manager* bm, int64_t seq, int32_t num_tokens,
                          int64_t* slots_out, int64_t* copy_out, int32_t* num_copies);
/*
 * The host side of one decode step for a fixed-size batch: row i appends one token to
 * sequence seqs[i] (as pkv_bm_append, rows in order), or is a padding row when seqs[i] < 0.
 * Then row i of table [n][max_blocks_per_seq] int32 and seq_lens [n] int32 (or NULL) get
 * the sequence's blocks and new length (padding rows: pad_block everywhere, length 0),
 * ready for pkv_upload and pkv_paged_attn_decode_ex with k_new/v_new.  slots_out [n] int64
 * or NULL gets each row's new slot (-1 for padding rows).  copies_out [n][2] int64 gets the
 * copy-on-write pairs of the step, *num_copies of them, to run (pkv_kv_cache_copy_blocks)
 * before the decode writes.  All [host].  Everything is checked first: on an error (an id
 * unknown or listed twice, a sequence over max_blocks_per_seq, too few free blocks)
 * nothing changes.
 */
PKV_API int pkv_bm_decode_step(pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                               int64_t* slots_out, int64_t* copies_out, int32_t* num_copies,
                               int32_t* table, int32_t* seq_lens, int32_t pad_block);
/* Releases `seq` (counts first, then blocks at count 0 back to the free list). */
PKV_API int pkv_bm_free(pkv_block_manager* bm, int64_t seq);
/* [host] *len = tokens of `seq`. */
PKV_API int pkv_bm_length(const pkv_block_manager* bm, int64_t seq, int64_t* len);
/* [host] *count = sequences holding physical block `block` (0 when free). */
PKV_API int pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block, int32_t* count);
/*
 * [host] Batch view for one step: row i of table [n][max_blocks_per_seq] int32 gets the
 * blocks of seqs[i] followed by pad_block in every unused entry; seq_lens [n] int32 (or
 * NULL) gets their lengths.  The two arrays are what the decode calls take as
 * block_table and seq_lens_kv once copied to the device (pkv_upload).
 */
PKV_API int pkv_bm_table(const pkv_block_manager* bm, const int64_t* seqs, int32_t n,
                         int32_t* table, int32_t* seq_lens, int32_t pad_block);

/*
 * Measurement aid (not part of the decode path): reads `bytes` bytes from the device buffer
 * `src` with 16-byte non-temporal loads, `grid` workgroups of 256 threads striding over it,
 * and writes (almost never) one word to `sink`.  Its bandwidth is the practical HBM read
 * ceiling the HBM-bound kernels are compared with, next to the 8 TB/s vendor figure; "Paged
 * KV Cache and Packed Sequence", 5.4, times memory movement beside the kernel the same way.
 *   src 16-byte aligned, bytes a positive multiple of 16, sink [1] uint32, grid in [1, 65536].
 */
PKV_API int pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t grid,
                            void* stream);

/*
 * Measurement aid (not part of the decode path): the read floor of a paged decode's own
 * access pattern.  Reads, with no arithmetic, the bytes a decode over the same arguments
 * reads: rows p in [0, min(seq_lens[b], max_seq_len_kv)) of sequence b from both caches,
 * row = block_table[b][p / block_size] * block_size + p % block_size ("Paged KV Cache and
 * Packed Sequence", 2.2), one workgroup per (slice of slice_bytes of a row, sequence, split
 * of split_tokens rows), and writes (almost never) one word to `sink`.  With slice_bytes =
 * one head's row and split_tokens = the decode's split it is the decode's own pattern.
 *   k_cache, v_cache [num_blocks][block_size][row_bytes] (16-byte aligned), block_table
 *   [batch][max_blocks_per_seq] int32, seq_lens [batch] int32, sink [1] uint32, all device.
 *   row_bytes a multiple of slice_bytes, slice_bytes a positive multiple of 16, block_size
 *   a power of two in [1, 256], split_tokens in [1, 1024], max_seq_len_kv in
 *   [0, max_blocks_per_seq * block_size]; lengths are clamped to it and table entries to
 *   [0, num_blocks).  batch 0 or max_seq_len_kv 0: PKV_OK, nothing enqueued.
 */
PKV_API int pkv_gather_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                            int32_t max_seq_len_kv, int32_t block_size, int64_t num_blocks,
                            int32_t row_bytes, int32_t slice_bytes, int32_t split_tokens,
                            uint32_t* sink, void* stream);

/*
 * Copies whole blocks inside one cache array: for i < num_pairs, block pairs[2i] of
 * pool [num_blocks][block_bytes] is copied to block pairs[2i+1] (the copy-on-write pairs
 * of pkv_bm_append; call once per cache array: K, V, and the scale arrays of an INT8
 * cache).  pairs [num_pairs][2] int64 on the device; a pair naming a block outside
 * [0, num_blocks), or the same block twice, is skipped.  block_bytes a positive multiple
 * of 4 and pool 4-byte aligned (16 for the fast path).  Precondition: no destination
 * block is the source or destination of another pair.
 */
PKV_API int pkv_kv_cache_copy_blocks(void* pool, int64_t block_bytes, int64_t num_blocks,
                                     const int64_t* pairs, int32_t num_pairs, void* stream);

/*
 * ---------------------------------------------------------------- captured steps
 * A decode step (uploads of the host-built tables, the cache write, the attention) can be
 * recorded once and replayed on `stream`, so a step costs one launch instead of several
 * ("Paged KV Cache and Packed Sequence", 5.3: the block table stays a host-built tensor
 * whose new contents are copied in before each replay).  Host arguments (sizes, pointers,
 * max_seq_len_kv) are fixed at capture; device data (tables, lengths, inputs) is read at
 * each replay.  Keep the batch fixed with padding rows (seq_lens_kv = 0).
 */
/* Copies `bytes` from host memory to the device on `stream`.  In a captured step the copy
 * reads src_host at each replay; src_host must then be pinned (hipHostMalloc) and must not
 * be rewritten until that replay has run (double-buffer it). */
PKV_API int pkv_upload(void* dst, const void* src_host, size_t bytes, void* stream);
/* Starts recording the work enqueued on `stream` by this thread (a created stream, not
 * NULL) into a graph; nothing runs until the graph is launched. */
PKV_API int pkv_graph_begin(void* stream);
/* Ends the recording and instantiates it: *graph_out is an executable graph handle. */
PKV_API int pkv_graph_end(void* stream, void** graph_out);
/* Replays a graph on `stream` (asynchronous, like the calls it recorded). */
PKV_API int pkv_graph_launch(void* graph, void* stream);
/* Destroys a graph handle (NULL is a no-op); no replay of it may still be pending. */
PKV_API int pkv_graph_destroy(void* graph);

/*
 * Step runner: a recorded decode step replayed with double-buffered host-built inputs (the
 * table and lengths: "Paged KV Cache and Packed Sequence", 5.3, the host filling the next
 * step's table while this step runs).  The caller owns two device buffers and two pinned
 * host buffers (hipHostMalloc) of `bytes` each (a multiple of 4, all 16-byte aligned), and
 * records graph j (reading device buffer j) between pkv_runner_capture_begin(r, j, s) and
 * pkv_runner_capture_end(r, s) on a created stream s; capture_begin records, as the
 * graph's first node, a copy kernel of host buffer j into device buffer j.  Then per step:
 *   h = pkv_runner_host_buffer(r)   [host] blocks until the replay that last read this
 *                                   buffer has run (two steps back), returns it to fill;
 *   pkv_runner_launch(r, stream)    replays the matching graph on `stream` (any stream, NULL
 *                                   included): the copy, then the recorded step.
 * The runner owns two events and the two graphs; it allocates no device memory and uses
 * no stream of its own.  pkv_runner_destroy waits for its pending work first.
 */
typedef struct pkv_step_runner pkv_step_runner;
/* NULL (and pkv_last_error) on NULL or repeated buffers, bytes = 0 or a HIP error. */
PKV_API pkv_step_runner* pkv_runner_create(void* dev0, void* dev1, const void* host0,
                                           const void* host1, size_t bytes);
PKV_API int pkv_runner_destroy(pkv_step_runner* r);
/* Starts recording graph j (0 or 1) on `stream`; PKV_ERR_SHAPE if j is recorded already or
 * another capture of this runner is open. */
PKV_API int pkv_runner_capture_begin(pkv_step_runner* r, int32_t j, void* stream);
PKV_API int pkv_runner_capture_end(pkv_step_runner* r, void* stream);
/* The executable graph j (for pkv_graph_launch without an upload), or NULL. */
PKV_API void* pkv_runner_graph(pkv_step_runner* r, int32_t j);
/* [host] The host buffer the next pkv_runner_launch copies in, once free; NULL on error. */
PKV_API void* pkv_runner_host_buffer(pkv_step_runner* r);
/* Enqueues the next step (copy + recorded step, one graph replay) as described above;
 * PKV_ERR_SHAPE if its graph was not recorded. */
PKV_API int pkv_runner_launch(pkv_step_runner* r, void* stream);
/* The copy the runner records: `bytes` (a multiple of 4) from pinned host memory src_host
 * (hipHostMalloc; read through its device view) to device memory dst, both 16-byte
 * aligned, by a kernel on `stream` (so that a graph records it as a kernel node, and it
 * needs no copy engine).  PKV_ERR_HIP if src_host has no device view (not pinned). */
PKV_API int pkv_upload_kernel(void* dst, const void* src_host, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
