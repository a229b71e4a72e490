/*
 * pkv_oracle.c — plain fp64 CPU oracle for paged-attention decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the bench's CPU-baseline leg use it.
 * It shares no code, header or constant with the HIP library.
 *
 * It computes, slowly and directly, what the pages define:
 *   - the logical -> physical address map ("KVCache Optimization Skill", Layer 3,
 *     3.1 "Physical Memory Layout and Logical Mapping"; the hotelren.com source note
 *     "Paged KV Cache and Packed Sequence", section 2.2, index snippet);
 *   - the slot_mapping write of new K/V rows (same skill page, Mode 2 step 3 and
 *     3.3 "slot_mapping Construction"; the ai6s.net article, section 4.2, cache
 *     write loop);
 *   - softmax attention of each query row over the K/V of its own sequence, read
 *     in logical order through block_table (skill page Mode 2 step 4 and Mode 3
 *     "MLA compressed cache"; source note sections 3.2-3.3 and 4.3).
 * Every floating-point value is widened exactly to double; all arithmetic is fp64.
 *
 * Readings where the pages leave a step open (listed in the design notes):
 *   - new-token position is 0-based: token j of sequence b sits at pos = L_b + j;
 *   - causal visibility includes the query's own position and is bottom-right
 *     aligned: row i of a chunk of n rows in a sequence of total length L' sees
 *     positions p <= L' - n + i;
 *   - GQA: q head h reads kv head h / (Hq / Hkv);
 *   - a row with no visible key outputs 0 and lse = -inf.
 *
 * Parity of every function here is pinned by tests against printed examples,
 * closed forms and brute force; none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_TABLE (-2)   /* logical block past max_blocks_per_seq or bad physical id */
#define ORC_ERR_SLOT (-3)    /* slot out of range */
#define ORC_ERR_DUP (-4)     /* two tokens write the same slot */
#define ORC_ERR_LEN (-5)     /* bad lengths (cu_q decreasing, n_b > L'_b, ...) */
#define ORC_ERR_MEM (-6)

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2   /* values already widened (e.g. int8 codes times their scale) */

int orc_version(void) { return 1; }

/* Threads an OpenMP region of the oracle will use (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* One element of a stored tensor, widened exactly to double. */
static double load_elem(const void* base, int64_t idx, int dtype) {
    if (dtype == ORC_F32) {
        return (double)((const float*)base)[idx];
    } else if (dtype == ORC_F64) {
        return ((const double*)base)[idx];
    } else {
        /* bf16 is the top half of an fp32: put the 16 bits back on top. */
        uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
}

/*
 * Physical slot of logical position `pos` of sequence b (skill page 3.1 mapping
 * formula; source-note 2.2 snippet):
 *     logical block = pos / block_size, offset = pos % block_size,
 *     physical block = block_table[b, logical block],
 *     slot = physical block * block_size + offset.
 * Returns -1 if the table cannot serve the position.
 */
int64_t orc_slot_of(const int32_t* block_table, int32_t max_blocks_per_seq,
                    int32_t b, int64_t pos, int32_t block_size, int64_t num_blocks) {
    if (pos < 0 || block_size <= 0) return -1;
    int64_t logical_block = pos / block_size;
    int64_t offset = pos % block_size;
    if (logical_block >= max_blocks_per_seq) return -1;
    int64_t physical = block_table[(int64_t)b * max_blocks_per_seq + logical_block];
    if (physical < 0 || physical >= num_blocks) return -1;
    return physical * block_size + offset;
}

/*
 * slot_mapping for a step that appends n_b = cu_new[b+1] - cu_new[b] tokens to
 * sequence b, which already holds L_b = lens_before[b] tokens.  Token t (packed
 * order) of sequence b is at position L_b + (t - cu_new[b]).  The slots of one step
 * must be distinct (two tokens may not share a cache row).
 */
int orc_slot_mapping(const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                     const int32_t* lens_before, const int32_t* cu_new,
                     int32_t block_size, int64_t num_blocks, int64_t* slots_out) {
    if (batch < 0 || block_size <= 0 || num_blocks < 0) return ORC_ERR_ARG;
    if (batch > 0 && cu_new[0] != 0) return ORC_ERR_LEN;
    for (int32_t b = 0; b < batch; ++b) {
        if (cu_new[b + 1] < cu_new[b] || lens_before[b] < 0) return ORC_ERR_LEN;
        for (int32_t t = cu_new[b]; t < cu_new[b + 1]; ++t) {
            int64_t pos = (int64_t)lens_before[b] + (t - cu_new[b]);
            int64_t s = orc_slot_of(block_table, max_blocks_per_seq, b, pos, block_size,
                                    num_blocks);
            if (s < 0) return ORC_ERR_TABLE;
            slots_out[t] = s;
        }
    }
    int64_t T = batch > 0 ? cu_new[batch] : 0;
    int64_t total_slots = num_blocks * (int64_t)block_size;
    uint8_t* seen = (uint8_t*)calloc((size_t)(total_slots > 0 ? total_slots : 1), 1);
    if (!seen) return ORC_ERR_MEM;
    int rc = ORC_OK;
    for (int64_t t = 0; t < T; ++t) {
        if (seen[slots_out[t]]) { rc = ORC_ERR_DUP; break; }
        seen[slots_out[t]] = 1;
    }
    free(seen);
    return rc;
}

/*
 * Cache write: row t of `rows` (row_bytes bytes) is copied to row slots[t] of the
 * cache viewed as [num_slots, row_bytes].  A plain byte copy: no conversion.
 * (Skill page Mode 2 step 3; ai6s.net article 4.2 write loop.)
 */
int orc_kv_write(uint8_t* cache, int64_t num_slots, int64_t row_bytes, const uint8_t* rows,
                 const int64_t* slots, int64_t num_tokens) {
    if (num_slots < 0 || row_bytes <= 0 || num_tokens < 0) return ORC_ERR_ARG;
    uint8_t* seen = (uint8_t*)calloc((size_t)(num_slots > 0 ? num_slots : 1), 1);
    if (!seen) return ORC_ERR_MEM;
    for (int64_t t = 0; t < num_tokens; ++t) {
        if (slots[t] < 0 || slots[t] >= num_slots) { free(seen); return ORC_ERR_SLOT; }
        if (seen[slots[t]]) { free(seen); return ORC_ERR_DUP; }
        seen[slots[t]] = 1;
    }
    free(seen);
    for (int64_t t = 0; t < num_tokens; ++t)
        memcpy(cache + slots[t] * row_bytes, rows + t * row_bytes, (size_t)row_bytes);
    return ORC_OK;
}

/*
 * The ATB form of the same write (ai6s.net article, section 4.2): for request i with
 * seqlen[i] new tokens whose end position in the cache is token_offset[i], token j
 * goes to cache row token_offset[i] - seqlen[i] + j of that request's contiguous
 * region; new rows are packed request after request.  `cache` is viewed as
 * [batch, max_seq_len, row_bytes].  Kept as an independent formulation of the write.
 */
int orc_kv_write_contiguous(uint8_t* cache, int32_t batch, int64_t max_seq_len,
                            int64_t row_bytes, const uint8_t* newkv,
                            const int32_t* seqlen, const int32_t* token_offset) {
    int64_t prefix = 0;
    for (int32_t i = 0; i < batch; ++i) {
        for (int32_t j = 0; j < seqlen[i]; ++j) {
            int64_t row = (int64_t)token_offset[i] - seqlen[i] + j;
            if (row < 0 || row >= max_seq_len) return ORC_ERR_SLOT;
            memcpy(cache + ((int64_t)i * max_seq_len + row) * row_bytes,
                   newkv + (prefix + j) * row_bytes, (size_t)row_bytes);
        }
        prefix += seqlen[i];
    }
    return ORC_OK;
}

/*
 * Paged attention.
 *   q        [T, Hq, Dqk]       (T = cu_q[batch]; decode: cu_q = 0,1,...,B)
 *   q_rope   [T, Hq, Dr] or NULL (MLA: the rope part of the query)
 *   k_cache  [nb, bs, Hkv, Dqk]; v_cache [nb, bs, Hkv, Dv] (MLA passes the same
 *            cache_nope for both, so Dv = Dqk there)
 *   k_rope   [nb, bs, Hkv, Dr] or NULL, present iff q_rope is
 *   seq_lens_kv[b] = L'_b, the number of cached tokens of sequence b after the write.
 * Row i of sequence b (n_b = cu_q[b+1]-cu_q[b] rows) sees positions p in [lo, hi] with
 *   hi = L'_b - 1             if causal == 0   (decode, sparse_mode 0)
 *   hi = L'_b - n_b + i       if causal != 0   (bottom-right causal, self included)
 *   lo = max(0, hi - window + 1) if window > 0 (band / sliding window: the `window` most
 *        recent positions up to hi, the row's own included), else lo = 0.
 * score_p = scale * (q . K_p + q_rope . Krope_p); out = sum_p softmax_p * V_p;
 * lse = max + log(sum exp(score - max)).  Empty rows: out 0, lse -inf.
 * `touched` (nb*bs bytes, or NULL) marks every cache row read.
 */
int orc_paged_attention(const void* q, const void* q_rope, int32_t dtype,
                        const void* k_cache, const void* v_cache, const void* k_rope,
                        const int32_t* block_table, int32_t batch, int32_t max_blocks_per_seq,
                        const int32_t* cu_q, const int32_t* seq_lens_kv,
                        int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim_qk, int32_t head_dim_v, int32_t head_dim_rope,
                        int32_t block_size, int64_t num_blocks, double scale, int32_t causal,
                        int32_t window, double* out, double* lse, uint8_t* touched,
                        int32_t num_threads) {
    if (batch < 0 || num_q_heads <= 0 || num_kv_heads <= 0) return ORC_ERR_ARG;
    if (num_q_heads % num_kv_heads != 0) return ORC_ERR_ARG;
    if ((q_rope == NULL) != (k_rope == NULL)) return ORC_ERR_ARG;
    if (dtype != ORC_F32 && dtype != ORC_BF16 && dtype != ORC_F64) return ORC_ERR_ARG;
    if (batch > 0 && cu_q[0] != 0) return ORC_ERR_LEN;
    for (int32_t b = 0; b < batch; ++b) {
        int32_t n = cu_q[b + 1] - cu_q[b];
        if (n < 0 || seq_lens_kv[b] < 0 || n > seq_lens_kv[b]) return ORC_ERR_LEN;
    }
    const int32_t group = num_q_heads / num_kv_heads;
    const int32_t Dr = q_rope ? head_dim_rope : 0;
    const int64_t T = batch > 0 ? cu_q[batch] : 0;
    int32_t max_len = 0;
    for (int32_t b = 0; b < batch; ++b)
        if (seq_lens_kv[b] > max_len) max_len = seq_lens_kv[b];

    /* Every table entry that serves a visible position must be a real block. */
    for (int32_t b = 0; b < batch; ++b)
        for (int64_t p = 0; p < seq_lens_kv[b]; ++p)
            if (orc_slot_of(block_table, max_blocks_per_seq, b, p, block_size, num_blocks) < 0)
                return ORC_ERR_TABLE;

    const int64_t rows = T * num_q_heads;
#ifdef _OPENMP
    if (num_threads > 0) omp_set_num_threads(num_threads);
#endif
    int failed = 0;
#pragma omp parallel
    {
        double* score = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)(head_dim_v > 0 ? head_dim_v : 1));
        if (!score || !acc) {
#pragma omp atomic write
            failed = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < rows; ++r) {
            if (!score || !acc) continue;
            const int64_t t = r / num_q_heads;
            const int32_t h = (int32_t)(r % num_q_heads);
            const int32_t g = h / group;
            int32_t b = 0;                     /* the sequence that owns packed row t */
            while (!(t >= cu_q[b] && t < cu_q[b + 1])) ++b;
            const int64_t i = t - cu_q[b];
            const int64_t n = cu_q[b + 1] - cu_q[b];
            const int64_t visible = causal ? (seq_lens_kv[b] - n + i + 1) : seq_lens_kv[b];
            int64_t lo = 0;                    /* first visible position */
            if (window > 0 && visible - window > 0) lo = visible - window;

            double m = -INFINITY;
            for (int64_t p = lo; p < visible; ++p) {
                int64_t slot = orc_slot_of(block_table, max_blocks_per_seq, b, p,
                                           block_size, num_blocks);
                double s = 0.0;
                for (int32_t d = 0; d < head_dim_qk; ++d)
                    s += load_elem(q, (t * num_q_heads + h) * head_dim_qk + d, dtype) *
                         load_elem(k_cache, (slot * num_kv_heads + g) * head_dim_qk + d, dtype);
                for (int32_t d = 0; d < Dr; ++d)
                    s += load_elem(q_rope, (t * num_q_heads + h) * Dr + d, dtype) *
                         load_elem(k_rope, (slot * num_kv_heads + g) * Dr + d, dtype);
                score[p] = scale * s;
                if (score[p] > m) m = score[p];
                if (touched) {
#pragma omp atomic write
                    touched[slot] = 1;
                }
            }
            double z = 0.0;
            for (int32_t d = 0; d < head_dim_v; ++d) acc[d] = 0.0;
            for (int64_t p = lo; p < visible; ++p) {
                int64_t slot = orc_slot_of(block_table, max_blocks_per_seq, b, p,
                                           block_size, num_blocks);
                double w = exp(score[p] - m);
                z += w;
                for (int32_t d = 0; d < head_dim_v; ++d)
                    acc[d] += w * load_elem(v_cache, (slot * num_kv_heads + g) * head_dim_v + d,
                                            dtype);
            }
            for (int32_t d = 0; d < head_dim_v; ++d)
                out[r * head_dim_v + d] = visible > 0 ? acc[d] / z : 0.0;
            if (lse) lse[r] = visible > 0 ? m + log(z) : -INFINITY;
        }
        free(score);
        free(acc);
    }
    return failed ? ORC_ERR_MEM : ORC_OK;
}

/*
 * Merge of partial softmax states (the second pass of a split-KV decode).  State s
 * of row r carries the max m_s, the sum l_s = sum exp(score - m_s) and the
 * unnormalised o_s = sum exp(score - m_s) V over its own key range.  With
 * M = max_s m_s:  l = sum_s e^(m_s - M) l_s,  out = sum_s e^(m_s - M) o_s / l,
 * lse = M + log l.  States with l_s = 0 (empty ranges) contribute nothing.
 * Layout: m, l [S, rows]; o [S, rows, D]; out [rows, D]; lse [rows].
 */
int orc_merge_states(const double* m, const double* l, const double* o, int32_t num_states,
                     int64_t rows, int32_t dim, double* out, double* lse) {
    for (int64_t r = 0; r < rows; ++r) {
        double M = -INFINITY;
        for (int32_t s = 0; s < num_states; ++s)
            if (l[s * rows + r] > 0.0 && m[s * rows + r] > M) M = m[s * rows + r];
        double z = 0.0;
        for (int32_t d = 0; d < dim; ++d) out[r * dim + d] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        for (int32_t s = 0; s < num_states; ++s) {
            if (!(l[s * rows + r] > 0.0)) continue;
            double w = exp(m[s * rows + r] - M);
            z += w * l[s * rows + r];
            for (int32_t d = 0; d < dim; ++d)
                out[r * dim + d] += w * o[(s * rows + r) * dim + d];
        }
        for (int32_t d = 0; d < dim; ++d) out[r * dim + d] /= z;
        lse[r] = M + log(z);
    }
    return ORC_OK;
}
