// Host-side declarations shared by the C-ABI front end (api.hip) and the kernel files.
// Each launcher enqueues on the given stream and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Sets the calling thread's pkv_last_error() text; returns code.
int set_error_v(int code, const char* fmt, va_list ap);

// ------------------------------------------------------------------ slot_mapping + write
struct SlotParams {
    int64_t* slots;
    const int32_t* table;
    const int32_t* lens_before;
    const int32_t* cu_new;
    int64_t num_tokens;
    int32_t batch;
    int32_t mbs;
    int32_t bs_log2;
};
hipError_t launch_slot_mapping(const SlotParams& p, hipStream_t s);

struct WriteParams {
    const uint8_t* src[2];   // k_new, v_new
    uint8_t* dst[2];         // k_cache, v_cache
    int64_t row_bytes[2];
    const int64_t* slots;
    int64_t num_tokens;
    int64_t num_slots;       // num_blocks * block_size
};
hipError_t launch_kv_write(const WriteParams& p, hipStream_t s);

// slot_mapping and write in one launch: workgroup (b, i, K-or-V) appends new token i of
// sequence b.
struct AppendParams {
    const uint8_t* src[2];
    uint8_t* dst[2];
    int64_t row_bytes[2];
    const int32_t* table;
    const int32_t* lens_before;
    const int32_t* cu_new;
    int64_t* slots_out;      // may be null
    int64_t num_tokens;
    int64_t num_slots;
    int32_t batch, max_new, mbs, bs_log2;
};
hipError_t launch_kv_append(const AppendParams& p, hipStream_t s);

// Block copies inside one pool (copy on write of a shared block): pair i copies block
// pairs[2i] to block pairs[2i+1]; pairs naming a block outside the pool, or the same block
// twice, are skipped.
struct CopyBlocksParams {
    uint8_t* pool;
    const int64_t* pairs;
    int64_t block_bytes;
    int64_t num_blocks;
    int32_t num_pairs;
};
hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s);
// The decode's K/V reads without arithmetic: one workgroup per (slice of slice_bytes of a
// row, sequence, split of split_tokens rows); lengths clamped to [0, len_cap], table entries
// to [0, num_blocks).  split_tokens in [1, 1024], slice_bytes a multiple of 16 dividing
// row_bytes, len_cap <= mbs * 2^bs_log2.
struct GatherReadParams {
    const uint8_t* k;
    const uint8_t* v;
    const int32_t* table;      // [batch][mbs]
    const int32_t* seq_lens;   // [batch]
    uint32_t* sink;
    int64_t num_blocks;
    int32_t batch, mbs, bs_log2, len_cap, row_bytes, slice_bytes, split_tokens;
};
hipError_t launch_gather_read(const GatherReadParams& p, hipStream_t s);
// bytes (a multiple of 4; both ends 16-byte aligned) from pinned host memory, addressed by
// its device view (hipHostGetDevicePointer), into dst, by a kernel (so that a graph can
// record it as a kernel node).
hipError_t launch_host_copy(void* dst, const void* src_dev_view, int64_t bytes, hipStream_t s);

// Quantizing write of the INT8 cache: per (token, kv head) row, s = max|x| / 127 and
// q = round_half_even(x / s) into the int8 caches and the fp32 scale arrays.
struct QuantWriteParams {
    const void* k_new;       // [T][Hkv][D] in the input dtype
    const void* v_new;
    int8_t* k_cache;         // [nb * bs][Hkv][D]
    int8_t* v_cache;
    float* k_scale;          // [nb][Hkv][bs]: a block's scales of one head are contiguous
    float* v_scale;
    const int64_t* slots;
    int64_t num_tokens, num_slots;
    int32_t hkv;
    int32_t bs_log2;
    int32_t which_base;      // 0: blockIdx.y picks K (0) or V (1); 1: the launch writes V only
};
hipError_t launch_kv_write_int8(const QuantWriteParams& p, int in_dtype, int head_dim, hipStream_t s);
// The MLA latent cache: k_new/k_cache/k_scale are the 512-wide nope rows, v_new/v_cache/
// v_scale the 64-wide rope rows (one kv head), each quantized with its own scale.
hipError_t launch_kv_write_int8_mla(const QuantWriteParams& p, int in_dtype, hipStream_t s);

// RMSNorm + RoPE + write of the MLA latent row (one wave per token).
struct NormRopeParams {
    const void* kv;          // [T][dn + dr]
    const void* gamma;       // [dn]
    const float* cos;        // [T][dr / 2]
    const float* sin;
    void* cache_nope;        // [nb * bs][dn]
    void* cache_rope;        // [nb * bs][dr]
    const int64_t* slots;
    int64_t num_tokens, num_slots;
    int32_t dn, dr;
    float eps;
};
hipError_t launch_norm_rope_write(const NormRopeParams& p, int dtype, hipStream_t s);

// ------------------------------------------------------------------ decode (MHA / GQA)
// Split-KV plan: sequence b's tokens are cut into ceil(L'_b / split_tokens) chunks; one
// workgroup handles (kv head, sequence, chunk).  Partial states go to the workspace and
// a second kernel merges them.  The plan depends on host-known sizes only, so results
// do not depend on where blocks sit.
// Workspace layout (each part 256-byte aligned):
//   [o fp32 B*Hq*max_splits*Dv][(m, l) fp32 B*Hq*max_splits*2]
// With 4..16 query heads per kv head the bf16 path may instead run the range-streaming
// kernel (gqa_stream_supported): `parts` workgroups per kv head, each leaving at most two
// partial states; its workspace is laid out from offset 0 as
//   [o fp32 Hkv*parts*2*G*Dv][(m, l) fp32 Hkv*parts*2*G*2][tile prefix int32 B+1]
// and ws_bytes covers both layouts.
struct DecodePlan {
    int32_t split_tokens;
    int32_t max_splits;
    size_t ws_bytes;
    size_t ws_o_offset;
    size_t ws_ml_offset;
    int32_t parts;
    size_t st_o_offset, st_ml_offset, st_pre_offset;
};
// qn > 0: the multi-token decode, which always runs the range-streaming kernel with qn
// query tokens per sequence; 0: decode (that kernel only for bf16 with 4..16 heads per kv head).
DecodePlan plan_decode(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim_v, int32_t max_seq_len_kv, bool byte_rows = false,
                       int32_t qn = 0);

struct DecodeParams {
    void* out;
    float* lse;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    const int32_t* table;
    const int32_t* seq_lens;
    float* ws_o;             // [B][Hq][max_splits][D]
    float* ws_ml;            // [B][Hq][max_splits][2]
    int32_t batch, mbs, hq, hkv, group;
    int32_t bs_log2;
    int32_t split_tokens, max_splits;
    int32_t len_cap;         // min(max_seq_len_kv, mbs * block_size)
    int64_t num_blocks;
    float scale_log2;        // softmax_scale * log2(e)
    // Append mode (decode step that also writes this step's token): the token at
    // position seq_lens[b] - 1 is read from k_new/v_new rows [B][Hkv][D] instead of the
    // cache, and the workgroup whose split holds it writes its head slice to the cache.
    const void* k_new;       // null: plain decode
    const void* v_new;
    void* k_cache_w;         // writable views of the caches (append mode)
    void* v_cache_w;
    int64_t* slots_out;      // [B] or null
    // Range-streaming kernel (parts > 0): workgroups per kv head, and the tile prefix
    // [B + 1] it leaves for its combine; ws_o / ws_ml then hold its partial states.
    int32_t parts;
    int32_t* tile_prefix;
    // INT8 caches (launch_decode_int8): one fp32 scale per (slot, kv head) row, else null;
    // in append mode (k_new set, 1..4 query heads per kv head) the writable views of the
    // code caches (k_cache_w / v_cache_w) and of the scales below take the new token.
    const float* k_scale;
    const float* v_scale;
    float* k_scale_w;
    float* v_scale_w;
    // Sliding window (band): > 0 keeps the `window` most recent keys of each sequence
    // (window_start below); 0 keeps all of them.  Splits and tiles then start at the
    // window start rounded down to a multiple of 32 keys.
    int32_t window;
    // Query tokens per sequence (range-streaming kernel only; 1 for decode): q, out and lse
    // rows are [B * qn][Hq]; token i of sequence b sees keys below seq_lens[b] - qn + 1 + i.
    int32_t qn;
};
// dtype: 0 f32, 1 bf16; head_dim 64 or 128.  bf16 with 4..16 query heads per kv head runs
// on the matrix cores (launch_gqa_decode: the range-streaming kernel when p.parts > 0,
// else the per-split one), everything else on the vector ALU.
hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, hipStream_t s);
bool gqa_mfma_supported(int dtype, int group);
// Head dim, block size and batch the range-streaming kernel takes (any column count <= 16).
bool gqa_stream_shape_supported(int head_dim, int bs_log2, int batch);
bool gqa_stream_supported(int dtype, int group, int head_dim, int bs_log2, int batch);
// Ranges per kv head: 2 workgroups per CU, or 4 in the compact layout (bf16 when the planned
// length is at least kStreamCompactMinKeys: the merge of twice the ranges pays off only on
// long contexts), or 5 over INT8 codes (5..16 query heads per kv head).
int gqa_stream_parts(int num_kv_heads, bool compact, bool int8);
constexpr int32_t kStreamCompactMinKeys = 4096;
hipError_t launch_gqa_decode(const DecodeParams& p, int head_dim, hipStream_t s);
hipError_t launch_gqa_stream_combine(const DecodeParams& p, int head_dim, hipStream_t s);
// The range-streaming kernel over INT8 codes (p.parts > 0, p.k_scale / p.v_scale set,
// blocks of at least 1024 / head_dim keys); its combine is launch_gqa_stream_combine.
hipError_t launch_gqa_decode_int8(const DecodeParams& p, int head_dim, hipStream_t s);
// Decode over the INT8 caches (p.k_scale / p.v_scale set): bf16 queries and output.
// 1..4 query heads per kv head: split-KV with the generic combine; p.parts > 0 (5..16):
// launch_gqa_decode_int8.
hipError_t launch_decode_int8(const DecodeParams& p, int head_dim, hipStream_t s);
// Kv heads per workgroup of the INT8 split-KV decode: with one query head per kv head and
// an even number of kv heads, a pair of adjacent heads, whose rows of a token are one
// contiguous piece; else 1.  The plan sizes the splits for it.
int int8_head_group(int32_t group, int32_t num_kv_heads);

// Merge of split partials (second launch of a split decode).
struct CombineParams {
    void* out;
    float* lse;
    const float* ws_o;
    const float* ws_ml;
    const int32_t* seq_lens;
    int32_t batch, hq, dim, split_tokens, max_splits, len_cap;
    int32_t window;          // as DecodeParams::window (the splits start where the pass put them)
};
hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t s);

// ------------------------------------------------------------------ MFMA attention
// One core for the two dense-contraction paths: the MLA-absorbed decode (rows = query
// heads of one token, key = nope || rope, value = nope) and the packed varlen causal
// chunk (rows = (query token, query head) pairs of one kv head).  Rows are grouped 32 per
// wave, 4 waves per workgroup; the workgroup walks a key range in 32-key tiles.
struct MfmaParams {
    void* out;               // [rows][Dv] in q's dtype (decode: [B][Hq][Dv]; varlen: [T][Hq][Dv])
    float* lse;              // [rows] or null
    const void* q;           // [.., Hq, Dqk main part]
    const void* q_rope;      // MLA: [B][Hq][Dr]; else null
    const void* k_cache;     // [nb][bs][Hkv][Dk]
    const void* v_cache;     // varlen: [nb][bs][Hkv][Dv]; MLA: unused (value = nope part of K)
    const void* k_rope;      // MLA: [nb][bs][1][Dr]
    const int32_t* table;
    const int32_t* seq_lens;  // L'_b
    const int32_t* cu_q;      // varlen: [B+1]
    float* ws_o;             // MLA splits: [B][Hq][max_splits][Dv]
    float* ws_ml;            // [B][Hq][max_splits][2]
    int32_t batch, mbs, hq, hkv, group;
    int32_t bs_log2;
    int32_t split_tokens, max_splits;   // MLA
    int32_t len_cap;
    int32_t q_blocks;        // varlen: query blocks per sequence in the grid
    int32_t causal;
    int32_t window;          // varlen: > 0 keeps each row's `window` most recent visible keys
    int64_t num_blocks;
    float scale_log2;
    // MLA over the INT8 cache (else null): k_cache / k_rope hold int8 codes, these their
    // fp32 scales [nb][1][bs] (nope, rope).
    const float* k_scale;
    const float* r_scale;
    // MLA append (else null): the step's bf16 latent rows nope [B][512] and rope [B][64],
    // attended at position seq_lens[b] - 1 and written there through the writable views
    // (INT8: quantized, codes into k_cache_w / rope_w and scales into the scale views).
    const void* k_new;
    const void* rope_new;
    void* k_cache_w;
    void* rope_w;
    // Varlen append (else null): the step's new K/V rows [T][Hkv][D] (v_new), attended at
    // positions seq_lens[b] - n_b + i and written there through k_cache_w / v_cache_w.
    const void* v_new;
    void* v_cache_w;
    float* k_scale_w;
    float* r_scale_w;
    int64_t* slots_out;      // [B] or null
};
// MLA decode: Dqk = 512 + Dr 64, Dv = 512, bf16 queries over the bf16 or the INT8 latent
// cache; one workgroup per (sequence, split, group of 128 heads).  Returns the launch status.
DecodePlan plan_mla(int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t max_seq_len_kv);
int32_t mla_head_groups(int32_t num_q_heads);
hipError_t launch_mla_decode(const MfmaParams& p, hipStream_t s);
// Varlen chunk: head_dim 64 or 128, bf16.
hipError_t launch_varlen(const MfmaParams& p, int head_dim, hipStream_t s);
int32_t varlen_tokens_per_block(int32_t group);

}  // namespace pkv
