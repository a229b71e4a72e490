// C-ABI front end of libpagedkv.so: host-side argument checks, then one or two kernel
// launches on the caller's stream.  No allocation, no synchronisation, no state except
// the thread-local text of the last error.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/pagedkv.h"
#include "pkv_internal.h"

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace pkv {
int set_error_v(int code, const char* fmt, va_list ap) {
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    return code;
}
}  // namespace pkv

namespace {

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    pkv::set_error_v(code, fmt, ap);
    va_end(ap);
    return code;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return PKV_OK;
    return fail(PKV_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool pow2_in(int32_t v, int32_t lo, int32_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

int log2i(int32_t v) {
    int r = 0;
    while ((1 << r) < v) ++r;
    return r;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_last_error(void) { return g_err; }

int pkv_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                     const int32_t* lens_before, const int32_t* cu_new, int32_t batch,
                     int64_t num_tokens, int32_t max_blocks_per_seq, int32_t block_size,
                     void* stream) {
    if (batch < 0 || num_tokens < 0) return fail(PKV_ERR_SHAPE, "slot_mapping: negative batch or num_tokens");
    if (max_blocks_per_seq <= 0) return fail(PKV_ERR_SHAPE, "slot_mapping: max_blocks_per_seq must be > 0");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "slot_mapping: block_size %d is not a power of two in [1, 256]", block_size);
    if (batch == 0 || num_tokens == 0) return PKV_OK;
    if (!slot_mapping || !block_table || !lens_before || !cu_new)
        return fail(PKV_ERR_NULL, "slot_mapping: NULL pointer argument");
    pkv::SlotParams p{slot_mapping, block_table, lens_before, cu_new, num_tokens, batch,
                      max_blocks_per_seq, log2i(block_size)};
    return hip_status(pkv::launch_slot_mapping(p, (hipStream_t)stream), "slot_mapping launch");
}

int pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                       const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                       int32_t head_dim_k, int32_t head_dim_v, int32_t block_size,
                       int64_t num_blocks, int32_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "kv_cache_write: unknown dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || head_dim_k <= 0 || head_dim_v <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "kv_cache_write: sizes must be positive (num_tokens >= 0)");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write: block_size %d is not a power of two in [1, 256]", block_size);
    if (num_tokens > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "kv_cache_write: num_tokens too large");
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !slot_mapping)
        return fail(PKV_ERR_NULL, "kv_cache_write: NULL pointer argument");
    if (k_cache == v_cache) return fail(PKV_ERR_SHAPE, "kv_cache_write: k_cache and v_cache must differ");
    const int eb = elem_bytes(dtype);
    pkv::WriteParams p{};
    p.src[0] = static_cast<const uint8_t*>(k_new);
    p.src[1] = static_cast<const uint8_t*>(v_new);
    p.dst[0] = static_cast<uint8_t*>(k_cache);
    p.dst[1] = static_cast<uint8_t*>(v_cache);
    p.row_bytes[0] = (int64_t)num_kv_heads * head_dim_k * eb;
    p.row_bytes[1] = (int64_t)num_kv_heads * head_dim_v * eb;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    for (int i = 0; i < 2; ++i) {
        if ((reinterpret_cast<uintptr_t>(p.src[i]) | reinterpret_cast<uintptr_t>(p.dst[i])) % eb)
            return fail(PKV_ERR_ALIGN, "kv_cache_write: pointers must be aligned to the element size");
    }
    return hip_status(pkv::launch_kv_write(p, (hipStream_t)stream), "kv_cache_write launch");
}

int pkv_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t grid, void* stream) {
    if (!src || !sink) return fail(PKV_ERR_NULL, "stream_read: NULL src or sink");
    if (!aligned16(src) || reinterpret_cast<uintptr_t>(sink) % 4)
        return fail(PKV_ERR_ALIGN, "stream_read: src must be 16-byte and sink 4-byte aligned");
    if (bytes <= 0 || bytes % 16) return fail(PKV_ERR_SHAPE, "stream_read: bytes must be a positive multiple of 16");
    if (grid < 1 || grid > 65536) return fail(PKV_ERR_SHAPE, "stream_read: grid must be in [1, 65536]");
    return hip_status(pkv::launch_stream_read(src, bytes, sink, grid, (hipStream_t)stream), "stream_read launch");
}

int pkv_gather_read(const void* k_cache, const void* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                    int32_t max_seq_len_kv, int32_t block_size, int64_t num_blocks,
                    int32_t row_bytes, int32_t slice_bytes, int32_t split_tokens,
                    uint32_t* sink, void* stream) {
    if (batch < 0 || max_blocks_per_seq < 1 || num_blocks < 1)
        return fail(PKV_ERR_SHAPE, "gather_read: batch >= 0, max_blocks_per_seq >= 1, num_blocks >= 1");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "gather_read: block_size must be a power of two in [1, 256]");
    if (slice_bytes < 16 || slice_bytes % 16 || row_bytes < slice_bytes || row_bytes % slice_bytes)
        return fail(PKV_ERR_SHAPE, "gather_read: slice_bytes a positive multiple of 16 dividing row_bytes");
    if (split_tokens < 1 || split_tokens > 1024)
        return fail(PKV_ERR_SHAPE, "gather_read: split_tokens must be in [1, 1024]");
    if (max_seq_len_kv < 0 || (int64_t)max_seq_len_kv > (int64_t)max_blocks_per_seq * block_size)
        return fail(PKV_ERR_SHAPE, "gather_read: max_seq_len_kv must be in [0, max_blocks_per_seq * block_size]");
    if (num_blocks > INT64_MAX / ((int64_t)block_size * row_bytes))
        return fail(PKV_ERR_SHAPE, "gather_read: cache size overflows");
    if (batch == 0 || max_seq_len_kv == 0) return PKV_OK;
    if (!k_cache || !v_cache || !block_table || !seq_lens || !sink)
        return fail(PKV_ERR_NULL, "gather_read: NULL pointer argument");
    if (!aligned16(k_cache) || !aligned16(v_cache) || reinterpret_cast<uintptr_t>(sink) % 4)
        return fail(PKV_ERR_ALIGN, "gather_read: caches must be 16-byte and sink 4-byte aligned");
    pkv::GatherReadParams p{};
    p.k = static_cast<const uint8_t*>(k_cache);
    p.v = static_cast<const uint8_t*>(v_cache);
    p.table = block_table;
    p.seq_lens = seq_lens;
    p.sink = sink;
    p.num_blocks = num_blocks;
    p.batch = batch;
    p.mbs = max_blocks_per_seq;
    p.bs_log2 = log2i(block_size);
    p.len_cap = max_seq_len_kv;
    p.row_bytes = row_bytes;
    p.slice_bytes = slice_bytes;
    p.split_tokens = split_tokens;
    return hip_status(pkv::launch_gather_read(p, (hipStream_t)stream), "gather_read launch");
}

int pkv_kv_cache_copy_blocks(void* pool, int64_t block_bytes, int64_t num_blocks,
                             const int64_t* pairs, int32_t num_pairs, void* stream) {
    if (num_pairs < 0 || block_bytes <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "kv_cache_copy_blocks: sizes must be positive (num_pairs >= 0)");
    if (block_bytes % 4) return fail(PKV_ERR_ALIGN, "kv_cache_copy_blocks: block_bytes must be a multiple of 4");
    if (num_blocks > INT64_MAX / block_bytes) return fail(PKV_ERR_SHAPE, "kv_cache_copy_blocks: pool size overflows");
    if (num_pairs == 0) return PKV_OK;
    if (!pool || !pairs) return fail(PKV_ERR_NULL, "kv_cache_copy_blocks: NULL pointer argument");
    if (reinterpret_cast<uintptr_t>(pool) % 4) return fail(PKV_ERR_ALIGN, "kv_cache_copy_blocks: pool must be 4-byte aligned");
    pkv::CopyBlocksParams p{};
    p.pool = static_cast<uint8_t*>(pool);
    p.pairs = pairs;
    p.block_bytes = block_bytes;
    p.num_blocks = num_blocks;
    p.num_pairs = num_pairs;
    return hip_status(pkv::launch_copy_blocks(p, (hipStream_t)stream), "kv_cache_copy_blocks launch");
}

int pkv_upload(void* dst, const void* src_host, size_t bytes, void* stream) {
    if (bytes == 0) return PKV_OK;
    if (!dst || !src_host) return fail(PKV_ERR_NULL, "upload: NULL pointer argument");
    return hip_status(hipMemcpyAsync(dst, src_host, bytes, hipMemcpyHostToDevice, (hipStream_t)stream),
                      "upload");
}

int pkv_graph_begin(void* stream) {
    if (!stream) return fail(PKV_ERR_NULL, "graph_begin: capture needs a created stream, not the NULL stream");
    return hip_status(hipStreamBeginCapture((hipStream_t)stream, hipStreamCaptureModeThreadLocal),
                      "graph_begin");
}

int pkv_graph_end(void* stream, void** graph_out) {
    if (!stream || !graph_out) return fail(PKV_ERR_NULL, "graph_end: NULL stream or graph_out");
    *graph_out = nullptr;
    hipGraph_t g = nullptr;
    int rc = hip_status(hipStreamEndCapture((hipStream_t)stream, &g), "graph_end: end capture");
    if (rc != PKV_OK) return rc;
    hipGraphExec_t exec = nullptr;
    rc = hip_status(hipGraphInstantiate(&exec, g, nullptr, nullptr, 0), "graph_end: instantiate");
    (void)hipGraphDestroy(g);
    if (rc == PKV_OK) *graph_out = exec;
    return rc;
}

int pkv_graph_launch(void* graph, void* stream) {
    if (!graph) return fail(PKV_ERR_NULL, "graph_launch: NULL graph");
    return hip_status(hipGraphLaunch((hipGraphExec_t)graph, (hipStream_t)stream), "graph_launch");
}

int pkv_graph_destroy(void* graph) {
    if (!graph) return PKV_OK;
    return hip_status(hipGraphExecDestroy((hipGraphExec_t)graph), "graph_destroy");
}

int pkv_kv_cache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int32_t* block_table, const int32_t* lens_before,
                        const int32_t* cu_new, int64_t* slot_mapping_out, int32_t batch,
                        int64_t num_tokens, int32_t max_new_tokens, int32_t max_blocks_per_seq,
                        int32_t num_kv_heads, int32_t head_dim_k, int32_t head_dim_v,
                        int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "kv_cache_append: unknown dtype %d", dtype);
    if (batch < 0 || num_tokens < 0 || max_new_tokens < 0 || num_kv_heads <= 0 || head_dim_k <= 0 ||
        head_dim_v <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
        return fail(PKV_ERR_SHAPE, "kv_cache_append: sizes must be positive (batch, num_tokens, max_new_tokens >= 0)");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: block_size %d is not a power of two in [1, 256]", block_size);
    if (num_tokens > 0x7fffffffLL || batch > 65535)
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_append: at most 65535 sequences and 2^31 - 1 tokens");
    if (batch == 0 || num_tokens == 0 || max_new_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !block_table || !lens_before || !cu_new)
        return fail(PKV_ERR_NULL, "kv_cache_append: NULL pointer argument");
    if (k_cache == v_cache) return fail(PKV_ERR_SHAPE, "kv_cache_append: k_cache and v_cache must differ");
    const int eb = elem_bytes(dtype);
    pkv::AppendParams p{};
    p.src[0] = static_cast<const uint8_t*>(k_new);
    p.src[1] = static_cast<const uint8_t*>(v_new);
    p.dst[0] = static_cast<uint8_t*>(k_cache);
    p.dst[1] = static_cast<uint8_t*>(v_cache);
    p.row_bytes[0] = (int64_t)num_kv_heads * head_dim_k * eb;
    p.row_bytes[1] = (int64_t)num_kv_heads * head_dim_v * eb;
    for (int i = 0; i < 2; ++i) {
        if ((reinterpret_cast<uintptr_t>(p.src[i]) | reinterpret_cast<uintptr_t>(p.dst[i])) % eb)
            return fail(PKV_ERR_ALIGN, "kv_cache_append: pointers must be aligned to the element size");
    }
    p.table = block_table;
    p.lens_before = lens_before;
    p.cu_new = cu_new;
    p.slots_out = slot_mapping_out;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.batch = batch;
    p.max_new = max_new_tokens;
    p.mbs = max_blocks_per_seq;
    p.bs_log2 = log2i(block_size);
    return hip_status(pkv::launch_kv_append(p, (hipStream_t)stream), "kv_cache_append launch");
}

int pkv_kv_rmsnorm_rope_cache(const void* kv, const void* gamma, const float* cos, const float* sin,
                              void* cache_nope, void* cache_rope, const int64_t* slot_mapping,
                              int64_t num_tokens, int32_t head_dim_nope, int32_t head_dim_rope,
                              int32_t block_size, int64_t num_blocks, float eps, int32_t dtype,
                              void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_ERR_DTYPE, "kv_rmsnorm_rope_cache: unknown dtype %d", dtype);
    if (num_tokens < 0 || head_dim_nope <= 0 || head_dim_rope <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "kv_rmsnorm_rope_cache: head dims and num_blocks must be positive");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "kv_rmsnorm_rope_cache: block_size %d is not a power of two in [1, 256]",
                    block_size);
    const int per16 = 16 / elem_bytes(dtype);
    if (head_dim_nope % per16 || head_dim_nope / per16 > 128 || head_dim_rope % (2 * per16) ||
        head_dim_rope / 2 / per16 > 64)
        return fail(PKV_ERR_UNSUPPORTED,
                    "kv_rmsnorm_rope_cache: head_dim_nope must be a multiple of %d up to %d and head_dim_rope "
                    "a multiple of %d up to %d",
                    per16, 128 * per16, 2 * per16, 128 * per16);
    if (!isfinite(eps) || eps < 0.0f) return fail(PKV_ERR_SHAPE, "kv_rmsnorm_rope_cache: eps must be finite and >= 0");
    if (num_tokens > 0x7fffffffLL * 4) return fail(PKV_ERR_UNSUPPORTED, "kv_rmsnorm_rope_cache: too many tokens");
    if (num_tokens == 0) return PKV_OK;
    if (!kv || !gamma || !cos || !sin || !cache_nope || !cache_rope || !slot_mapping)
        return fail(PKV_ERR_NULL, "kv_rmsnorm_rope_cache: NULL pointer argument");
    if (!aligned16(kv) || !aligned16(gamma) || !aligned16(cos) || !aligned16(sin) || !aligned16(cache_nope) ||
        !aligned16(cache_rope))
        return fail(PKV_ERR_ALIGN, "kv_rmsnorm_rope_cache: kv, gamma, cos, sin and caches must be 16-byte aligned");
    if (cache_nope == cache_rope)
        return fail(PKV_ERR_SHAPE, "kv_rmsnorm_rope_cache: cache_nope and cache_rope must differ");
    pkv::NormRopeParams p{};
    p.kv = kv;
    p.gamma = gamma;
    p.cos = cos;
    p.sin = sin;
    p.cache_nope = cache_nope;
    p.cache_rope = cache_rope;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.dn = head_dim_nope;
    p.dr = head_dim_rope;
    p.eps = eps;
    return hip_status(pkv::launch_norm_rope_write(p, dtype, (hipStream_t)stream), "kv_rmsnorm_rope_cache launch");
}

size_t pkv_decode_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim_v, int32_t max_seq_len_kv) {
    if (batch <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim_v <= 0 ||
        max_seq_len_kv <= 0 || num_q_heads % num_kv_heads)
        return 0;
    if (num_kv_heads == 1 && head_dim_v == 512)   // the MLA-absorbed shape
        return pkv::plan_mla(batch, num_q_heads, head_dim_v, max_seq_len_kv).ws_bytes;
    // the larger of the bf16 and INT8 plans (INT8 runs more ranges per kv head)
    const size_t a = pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim_v, max_seq_len_kv).ws_bytes;
    const size_t b = pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim_v, max_seq_len_kv, true).ws_bytes;
    return a > b ? a : b;
}

}  // extern "C"

namespace {

// Host-side checks shared by the decode entry points; fills the kernel parameters.
int prepare_decode(pkv::DecodeParams& p, pkv::DecodePlan& plan, void* out, float* lse_out,
                   const void* q, const void* q_rope, const void* k_cache, const void* v_cache,
                   const void* k_rope_cache, const int32_t* block_table,
                   const int32_t* seq_lens_kv, int32_t batch, int32_t max_blocks_per_seq,
                   int32_t max_seq_len_kv, int32_t num_q_heads, int32_t num_kv_heads,
                   int32_t head_dim_qk, int32_t head_dim_v, int32_t head_dim_rope,
                   int32_t block_size, int64_t num_blocks, float softmax_scale, int32_t dtype,
                   void* workspace, size_t workspace_bytes, bool* nothing_to_do,
                   int32_t window = 0, bool allow_stream = true, bool byte_rows = false,
                   int32_t qn = 0) {
    *nothing_to_do = false;
    if (window < 0) return fail(PKV_ERR_SHAPE, "decode: window must be >= 0 (0: no window)");
    if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "decode: unknown dtype %d", dtype);
    if (batch < 0) return fail(PKV_ERR_SHAPE, "decode: negative batch");
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return fail(PKV_ERR_SHAPE, "decode: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
    if (head_dim_qk <= 0 || head_dim_v <= 0 || head_dim_rope < 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "decode: head dims, max_blocks_per_seq and num_blocks must be positive");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "decode: block_size %d is not a power of two in [1, 256]", block_size);
    if ((int64_t)max_seq_len_kv > (int64_t)max_blocks_per_seq * block_size || max_seq_len_kv <= 0)
        return fail(PKV_ERR_SHAPE, "decode: max_seq_len_kv %d must be in [1, max_blocks_per_seq * block_size]",
                    max_seq_len_kv);
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.0f))
        return fail(PKV_ERR_SCALE, "decode: softmax_scale must be finite and > 0");
    if ((q_rope == nullptr) != (k_rope_cache == nullptr))
        return fail(PKV_ERR_NULL, "decode: q_rope and k_rope_cache must be given together or not at all");
    const bool mla = q_rope != nullptr;
    if (!mla && head_dim_rope != 0)
        return fail(PKV_ERR_SHAPE, "decode: head_dim_rope must be 0 without rope inputs");
    if (mla) {
        return fail(PKV_ERR_UNSUPPORTED, "decode: internal: MLA arguments reached the MHA path");
    }
    const int group = num_q_heads / num_kv_heads;
    if (head_dim_qk != head_dim_v || (head_dim_qk != 64 && head_dim_qk != 128))
        return fail(PKV_ERR_UNSUPPORTED, "decode: head_dim %d/%d not supported (64 or 128, equal)",
                    head_dim_qk, head_dim_v);
    if (group > 16)
        return fail(PKV_ERR_UNSUPPORTED, "decode: %d query heads per kv head (max 16)", group);
    if (batch == 0) {
        *nothing_to_do = true;
        return PKV_OK;
    }
    if (!out || !q || !k_cache || !v_cache || !block_table || !seq_lens_kv)
        return fail(PKV_ERR_NULL, "decode: NULL pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_ERR_ALIGN, "decode: out, q and caches must be 16-byte aligned");
    // With a window a sequence's splits cover at most window + 31 keys (they start at the
    // window start rounded down to 32): plan for that length.
    const int32_t plan_len = window > 0 && window < max_seq_len_kv - 31 ? window + 31 : max_seq_len_kv;
    plan = pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim_v, plan_len, byte_rows, qn);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
        return fail(PKV_ERR_WORKSPACE, "decode: workspace needs %zu bytes (16-byte aligned), got %zu",
                    plan.ws_bytes, workspace ? workspace_bytes : (size_t)0);
    if ((int64_t)num_kv_heads * batch * plan.max_splits > 0x7fffffffLL)
        return fail(PKV_ERR_SHAPE, "decode: grid too large");

    p = pkv::DecodeParams{};
    p.out = out;
    p.lse = lse_out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.table = block_table;
    p.seq_lens = seq_lens_kv;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    p.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_o_offset) : nullptr;
    p.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_ml_offset) : nullptr;
    p.batch = batch;
    p.mbs = max_blocks_per_seq;
    p.hq = num_q_heads;
    p.hkv = num_kv_heads;
    p.group = group;
    p.bs_log2 = log2i(block_size);
    p.split_tokens = plan.split_tokens;
    p.max_splits = plan.max_splits;
    p.len_cap = max_seq_len_kv;
    p.num_blocks = num_blocks;
    p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
    p.window = window;
    p.qn = qn > 0 ? qn : 1;
    if (qn > 0 || (allow_stream && pkv::gqa_stream_supported(dtype, group, head_dim_v, p.bs_log2, batch))) {
        p.parts = plan.parts;
        p.ws_o = reinterpret_cast<float*>(ws + plan.st_o_offset);
        p.ws_ml = reinterpret_cast<float*>(ws + plan.st_ml_offset);
        p.tile_prefix = reinterpret_cast<int32_t*>(ws + plan.st_pre_offset);
    }
    return PKV_OK;
}

// Whether the split pass can leave partial states: several splits per sequence, or
// several ranges per kv head for the range-streaming kernel.
bool needs_combine(const pkv::DecodeParams& p, const pkv::DecodePlan& plan) {
    return p.parts > 0 ? p.parts > 1 : plan.max_splits > 1;
}

int launch_combine_for(const pkv::DecodeParams& p, int32_t head_dim_v, int32_t dtype,
                       hipStream_t s) {
    if (p.parts > 0) return hip_status(pkv::launch_gqa_stream_combine(p, head_dim_v, s), "decode combine launch");
    pkv::CombineParams c{};
    c.out = p.out;
    c.lse = p.lse;
    c.ws_o = p.ws_o;
    c.ws_ml = p.ws_ml;
    c.seq_lens = p.seq_lens;
    c.batch = p.batch;
    c.hq = p.hq;
    c.dim = head_dim_v;
    c.split_tokens = p.split_tokens;
    c.max_splits = p.max_splits;
    c.len_cap = p.len_cap;
    c.window = p.window;
    return hip_status(pkv::launch_combine(c, dtype, s), "decode combine launch");
}

}  // namespace

namespace {

// MLA-absorbed decode: checks and launch (split pass, then combine when stages ask).
int run_mla_decode(void* out, float* lse_out, const void* q, const void* q_rope,
                   const void* k_cache, const void* v_cache, const void* k_rope_cache,
                   const int32_t* block_table, const int32_t* seq_lens_kv, int32_t batch,
                   int32_t max_blocks_per_seq, int32_t max_seq_len_kv, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim_qk, int32_t head_dim_v,
                   int32_t head_dim_rope, int32_t block_size, int64_t num_blocks,
                   float softmax_scale, int32_t dtype, void* workspace, size_t workspace_bytes,
                   int stages, hipStream_t s, const float* nope_scale = nullptr,
                   const float* rope_scale = nullptr, const void* nope_new = nullptr,
                   const void* rope_new = nullptr, int64_t* slots_out = nullptr) {
    if (num_kv_heads != 1 || head_dim_qk != 512 || head_dim_v != 512 || head_dim_rope != 64)
        return fail(PKV_ERR_UNSUPPORTED,
                    "decode (MLA): needs 1 kv head, head_dim_qk = head_dim_v = 512, head_dim_rope = 64");
    if (dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "decode (MLA): bf16 only");
    if (v_cache != k_cache)
        return fail(PKV_ERR_UNSUPPORTED, "decode (MLA): v_cache must be k_cache (value = cache_nope)");
    if (batch == 0) return PKV_OK;
    if (!out || !q || !k_cache || !block_table || !seq_lens_kv)
        return fail(PKV_ERR_NULL, "decode: NULL pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(q_rope) || !aligned16(k_cache) ||
        !aligned16(k_rope_cache))
        return fail(PKV_ERR_ALIGN, "decode: out, q, q_rope and caches must be 16-byte aligned");
    const pkv::DecodePlan plan = pkv::plan_mla(batch, num_q_heads, head_dim_v, max_seq_len_kv);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace)))
        return fail(PKV_ERR_WORKSPACE, "decode: workspace needs %zu bytes (16-byte aligned), got %zu",
                    plan.ws_bytes, workspace ? workspace_bytes : (size_t)0);
    const int64_t hgs = pkv::mla_head_groups(num_q_heads);
    if (hgs * ((int64_t)batch * plan.max_splits + 7) > 0x7fffffffLL)
        return fail(PKV_ERR_SHAPE, "decode: grid too large");
    pkv::MfmaParams p{};
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    p.out = out;
    p.lse = lse_out;
    p.q = q;
    p.q_rope = q_rope;
    p.k_cache = k_cache;
    p.v_cache = nullptr;
    p.k_rope = k_rope_cache;
    p.table = block_table;
    p.seq_lens = seq_lens_kv;
    p.ws_o = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_o_offset) : nullptr;
    p.ws_ml = plan.ws_bytes ? reinterpret_cast<float*>(ws + plan.ws_ml_offset) : nullptr;
    p.batch = batch;
    p.mbs = max_blocks_per_seq;
    p.hq = num_q_heads;
    p.hkv = 1;
    p.group = num_q_heads;
    p.bs_log2 = log2i(block_size);
    p.split_tokens = plan.split_tokens;
    p.max_splits = plan.max_splits;
    p.len_cap = max_seq_len_kv;
    p.num_blocks = num_blocks;
    p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
    p.k_scale = nope_scale;
    p.r_scale = rope_scale;
    if (nope_new) {   // append: the new latent rows are attended and written in the pass
        p.k_new = nope_new;
        p.rope_new = rope_new;
        p.k_cache_w = const_cast<void*>(k_cache);
        p.rope_w = const_cast<void*>(k_rope_cache);
        p.k_scale_w = const_cast<float*>(nope_scale);   // INT8: the scales it writes
        p.r_scale_w = const_cast<float*>(rope_scale);
        p.slots_out = slots_out;
    }
    int rc = PKV_OK;
    if (stages & 1) {
        rc = hip_status(pkv::launch_mla_decode(p, s), "decode (MLA) launch");
        if (rc != PKV_OK) return rc;
    }
    if ((stages & 2) && plan.max_splits > 1) {
        pkv::CombineParams c{};
        c.out = out;
        c.lse = lse_out;
        c.ws_o = p.ws_o;
        c.ws_ml = p.ws_ml;
        c.seq_lens = seq_lens_kv;
        c.batch = batch;
        c.hq = num_q_heads;
        c.dim = head_dim_v;
        c.split_tokens = plan.split_tokens;
        c.max_splits = plan.max_splits;
        c.len_cap = max_seq_len_kv;
        rc = hip_status(pkv::launch_combine(c, dtype, s), "decode (MLA) combine launch");
    }
    return rc;
}

// Checks common to every decode entry before the MHA/MLA split.  Returns PKV_OK and sets
// *mla when the rope inputs select the MLA path.
int check_decode_common(const void* q_rope, const void* k_rope_cache, int32_t dtype, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                        int32_t head_dim_v, int32_t head_dim_rope, int32_t max_blocks_per_seq,
                        int32_t max_seq_len_kv, int32_t block_size, int64_t num_blocks,
                        float softmax_scale, bool* mla) {
    *mla = false;
    if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "decode: unknown dtype %d", dtype);
    if (batch < 0) return fail(PKV_ERR_SHAPE, "decode: negative batch");
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return fail(PKV_ERR_SHAPE, "decode: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
    if (head_dim_qk <= 0 || head_dim_v <= 0 || head_dim_rope < 0 || max_blocks_per_seq <= 0 ||
        num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "decode: head dims, max_blocks_per_seq and num_blocks must be positive");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "decode: block_size %d is not a power of two in [1, 256]", block_size);
    if ((int64_t)max_seq_len_kv > (int64_t)max_blocks_per_seq * block_size || max_seq_len_kv <= 0)
        return fail(PKV_ERR_SHAPE, "decode: max_seq_len_kv %d must be in [1, max_blocks_per_seq * block_size]",
                    max_seq_len_kv);
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.0f))
        return fail(PKV_ERR_SCALE, "decode: softmax_scale must be finite and > 0");
    if ((q_rope == nullptr) != (k_rope_cache == nullptr))
        return fail(PKV_ERR_NULL, "decode: q_rope and k_rope_cache must be given together or not at all");
    *mla = q_rope != nullptr;
    if (!*mla && head_dim_rope != 0)
        return fail(PKV_ERR_SHAPE, "decode: head_dim_rope must be 0 without rope inputs");
    return PKV_OK;
}

}  // namespace

extern "C" {

#define PKV_DECODE_ARGS                                                                    \
    out, lse_out, q, q_rope, k_cache, v_cache, k_rope_cache, block_table, seq_lens_kv, batch, \
        max_blocks_per_seq, max_seq_len_kv, num_q_heads, num_kv_heads, head_dim_qk,           \
        head_dim_v, head_dim_rope, block_size, num_blocks, softmax_scale, dtype, workspace,   \
        workspace_bytes

int pkv_paged_attn_decode(void* out, float* lse_out, const void* q, const void* q_rope,
                          const void* k_cache, const void* v_cache, const void* k_rope_cache,
                          const int32_t* block_table, const int32_t* seq_lens_kv,
                          int32_t batch, int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                          int32_t head_dim_v, int32_t head_dim_rope, int32_t block_size,
                          int64_t num_blocks, float softmax_scale, int32_t dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    bool mla = false;
    int rc = check_decode_common(q_rope, k_rope_cache, dtype, batch, num_q_heads, num_kv_heads,
                                 head_dim_qk, head_dim_v, head_dim_rope, max_blocks_per_seq,
                                 max_seq_len_kv, block_size, num_blocks, softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    if (mla) return run_mla_decode(PKV_DECODE_ARGS, 3, (hipStream_t)stream);
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    rc = prepare_decode(p, plan, PKV_DECODE_ARGS, &idle);
    if (rc != PKV_OK || idle) return rc;
    hipStream_t s = (hipStream_t)stream;
    rc = hip_status(pkv::launch_decode(p, dtype, head_dim_qk, s), "decode split launch");
    if (rc != PKV_OK || !needs_combine(p, plan)) return rc;
    return launch_combine_for(p, head_dim_v, dtype, s);
}

int pkv_paged_attn_decode_split(void* out, float* lse_out, const void* q, const void* q_rope,
                                const void* k_cache, const void* v_cache,
                                const void* k_rope_cache, const int32_t* block_table,
                                const int32_t* seq_lens_kv, int32_t batch,
                                int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim_qk,
                                int32_t head_dim_v, int32_t head_dim_rope, int32_t block_size,
                                int64_t num_blocks, float softmax_scale, int32_t dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
    bool mla = false;
    int rc = check_decode_common(q_rope, k_rope_cache, dtype, batch, num_q_heads, num_kv_heads,
                                 head_dim_qk, head_dim_v, head_dim_rope, max_blocks_per_seq,
                                 max_seq_len_kv, block_size, num_blocks, softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    if (mla) return run_mla_decode(PKV_DECODE_ARGS, 1, (hipStream_t)stream);
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    rc = prepare_decode(p, plan, PKV_DECODE_ARGS, &idle);
    if (rc != PKV_OK || idle) return rc;
    return hip_status(pkv::launch_decode(p, dtype, head_dim_qk, (hipStream_t)stream),
                      "decode split launch");
}

int pkv_paged_attn_decode_combine(void* out, float* lse_out, const void* q, const void* q_rope,
                                  const void* k_cache, const void* v_cache,
                                  const void* k_rope_cache, const int32_t* block_table,
                                  const int32_t* seq_lens_kv, int32_t batch,
                                  int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                  int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim_qk, int32_t head_dim_v,
                                  int32_t head_dim_rope, int32_t block_size, int64_t num_blocks,
                                  float softmax_scale, int32_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    bool mla = false;
    int rc = check_decode_common(q_rope, k_rope_cache, dtype, batch, num_q_heads, num_kv_heads,
                                 head_dim_qk, head_dim_v, head_dim_rope, max_blocks_per_seq,
                                 max_seq_len_kv, block_size, num_blocks, softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    if (mla) return run_mla_decode(PKV_DECODE_ARGS, 2, (hipStream_t)stream);
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    rc = prepare_decode(p, plan, PKV_DECODE_ARGS, &idle);
    if (rc != PKV_OK || idle || !needs_combine(p, plan)) return rc;
    return launch_combine_for(p, head_dim_v, dtype, (hipStream_t)stream);
}

int pkv_paged_attn_decode_mla_append(void* out, float* lse_out, const void* q_nope,
                                     const void* q_rope, const void* nope_new,
                                     const void* rope_new, void* cache_nope, void* cache_rope,
                                     const int32_t* block_table, const int32_t* seq_lens_kv,
                                     int64_t* slot_mapping_out, int32_t batch,
                                     int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                     int32_t num_q_heads, int32_t block_size, int64_t num_blocks,
                                     float softmax_scale, int32_t stages, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "decode_mla_append: stages must be 1, 2 or 3");
    if (!nope_new || !rope_new) return fail(PKV_ERR_NULL, "decode_mla_append: NULL new rows");
    if (!q_rope || !cache_rope) return fail(PKV_ERR_NULL, "decode_mla_append: NULL q_rope or cache_rope");
    if (!aligned16(nope_new) || !aligned16(rope_new))
        return fail(PKV_ERR_ALIGN, "decode_mla_append: the new rows must be 16-byte aligned");
    if (cache_nope == cache_rope) return fail(PKV_ERR_SHAPE, "decode_mla_append: the two caches must differ");
    bool mla = false;
    int rc = check_decode_common(q_rope, cache_rope, PKV_BF16, batch, num_q_heads, 1, 512, 512, 64,
                                 max_blocks_per_seq, max_seq_len_kv, block_size, num_blocks,
                                 softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    return run_mla_decode(out, lse_out, q_nope, q_rope, cache_nope, cache_nope, cache_rope, block_table,
                          seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads, 1,
                          512, 512, 64, block_size, num_blocks, softmax_scale, PKV_BF16, workspace,
                          workspace_bytes, stages, (hipStream_t)stream, nullptr, nullptr, nope_new,
                          rope_new, slot_mapping_out);
}

#undef PKV_DECODE_ARGS

}  // extern "C"

namespace {

// MHA/GQA decode with an optional sliding window and an optional new token per sequence
// (k_new/v_new given: written at position seq_lens_kv[b] - 1 in the same pass).
int run_decode_mha(void* out, float* lse_out, const void* q, const void* k_new, const void* v_new,
                   void* k_cache, void* v_cache, const int32_t* block_table,
                   const int32_t* seq_lens_kv, int64_t* slot_mapping_out, int32_t batch,
                   int32_t max_blocks_per_seq, int32_t max_seq_len_kv, int32_t num_q_heads,
                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                   float softmax_scale, int32_t dtype, int32_t window, int32_t stages,
                   void* workspace, size_t workspace_bytes, hipStream_t s, const char* who) {
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "%s: stages must be 1, 2 or 3", who);
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    int rc = prepare_decode(p, plan, out, lse_out, q, nullptr, k_cache, v_cache, nullptr,
                            block_table, seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv,
                            num_q_heads, num_kv_heads, head_dim, head_dim, 0, block_size,
                            num_blocks, softmax_scale, dtype, workspace, workspace_bytes, &idle,
                            window);
    if (rc != PKV_OK || idle) return rc;
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "%s: k_new and v_new must be given together or not at all", who);
    if (k_new) {
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PKV_ERR_ALIGN, "%s: k_new and v_new must be 16-byte aligned", who);
        if (k_cache == v_cache) return fail(PKV_ERR_SHAPE, "%s: k_cache and v_cache must differ", who);
        p.k_new = k_new;
        p.v_new = v_new;
        p.k_cache_w = k_cache;
        p.v_cache_w = v_cache;
        p.slots_out = slot_mapping_out;
    }
    if (stages & 1) {
        rc = hip_status(pkv::launch_decode(p, dtype, head_dim, s), "decode split launch");
        if (rc != PKV_OK) return rc;
    }
    if ((stages & 2) && needs_combine(p, plan)) return launch_combine_for(p, head_dim, dtype, s);
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode_append(void* out, float* lse_out, const void* q, const void* k_new,
                                 const void* v_new, void* k_cache, void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens_kv,
                                 int64_t* slot_mapping_out, int32_t batch,
                                 int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float softmax_scale,
                                 int32_t dtype, int32_t stages, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    if (!k_new || !v_new) return fail(PKV_ERR_NULL, "decode_append: NULL k_new or v_new");
    return run_decode_mha(out, lse_out, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                          slot_mapping_out, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, dtype, 0,
                          stages, workspace, workspace_bytes, (hipStream_t)stream, "decode_append");
}

int pkv_paged_attn_decode_ex(void* out, float* lse_out, const void* q, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens_kv,
                             int64_t* slot_mapping_out, int32_t batch, int32_t max_blocks_per_seq,
                             int32_t max_seq_len_kv, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                             float softmax_scale, int32_t dtype, int32_t window, int32_t stages,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return run_decode_mha(out, lse_out, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                          slot_mapping_out, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, dtype,
                          window, stages, workspace, workspace_bytes, (hipStream_t)stream,
                          "decode_ex");
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free decode step
// The split pass's partial states of pkv_paged_attn_decode_append_noalloc live in this
// fixed array instead of a caller workspace: one copy per GPU the library runs on, held
// until the process ends, shared by every call on that GPU (calls that overlap on one GPU
// race).  Nothing in it has to start at zero: the split pass writes every partial state
// and tile prefix the combine reads, in each call.
static __device__ __align__(256) uint8_t scratch[PKV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's copy of `scratch`, looked up once per device with
// that device current.  In host code the array's name only identifies the symbol; it is
// never a device address.
int scratch_on_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "decode_append_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(PKV_ERR_UNSUPPORTED, "decode_append_noalloc: device %d (at most %d devices)", dev,
                    kMaxDevices);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "decode_append_noalloc: hipGetSymbolAddress(scratch)");
        if (!p) return fail(PKV_ERR_HIP, "decode_append_noalloc: no device address for the scratch array");
        g_scratch_ptr[dev].store(p, std::memory_order_release);   // the same value from any racer
    }
    *ptr = p;
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode_append_noalloc(void* out, float* lse_out, const void* q,
                                         const void* k_new, const void* v_new, void* k_cache,
                                         void* v_cache, const int32_t* block_table,
                                         const int32_t* seq_lens_kv, int64_t* slot_mapping_out,
                                         int32_t batch, int32_t max_blocks_per_seq,
                                         int32_t max_seq_len_kv, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t block_size, int64_t num_blocks,
                                         float softmax_scale, int32_t dtype, void* stream) {
    if (!k_new || !v_new) return fail(PKV_ERR_NULL, "decode_append_noalloc: NULL k_new or v_new");
    void* ws = nullptr;
    int rc = scratch_on_current_device(&ws);
    if (rc != PKV_OK) return rc;
    rc = run_decode_mha(out, lse_out, q, k_new, v_new, k_cache, v_cache, block_table, seq_lens_kv,
                        slot_mapping_out, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads,
                        num_kv_heads, head_dim, block_size, num_blocks, softmax_scale, dtype, 0, 3,
                        ws, (size_t)PKV_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream,
                        "decode_append_noalloc");
    if (rc == PKV_ERR_WORKSPACE) {   // every other argument was accepted before this check
        const size_t need = pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len_kv).ws_bytes;
        return fail(PKV_ERR_WORKSPACE,
                    "decode_append_noalloc: this batch needs %zu bytes of partial states; the fixed "
                    "scratch holds %zu (use pkv_paged_attn_decode_append with a workspace, or fewer "
                    "sequences, heads or a smaller max_seq_len_kv)",
                    need, (size_t)PKV_NOALLOC_SCRATCH_BYTES);
    }
    return rc;
}

size_t pkv_decode_mtp_workspace_size(int32_t batch, int32_t num_q_tokens, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim_v, int32_t max_seq_len_kv) {
    if (batch <= 0 || num_q_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
        head_dim_v <= 0 || max_seq_len_kv <= 0 || num_q_heads % num_kv_heads)
        return 0;
    return pkv::plan_decode(batch, num_q_heads, num_kv_heads, head_dim_v, max_seq_len_kv, false,
                            num_q_tokens).ws_bytes;
}

// pkv_paged_attn_decode_mtp, and with k_new / v_new given its append form.
static int mtp_impl(void* out, float* lse_out, const void* q, const void* k_cache,
                    const void* v_cache, const int32_t* block_table,
                    const int32_t* seq_lens_kv, int32_t batch, int32_t num_q_tokens,
                    int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int64_t num_blocks, float softmax_scale,
                    int32_t dtype, int32_t window, int32_t stages, void* workspace,
                    size_t workspace_bytes, const void* k_new, const void* v_new,
                    int64_t* slot_mapping_out, void* stream) {
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "decode_mtp: stages must be 1, 2 or 3");
    if (num_q_tokens < 1) return fail(PKV_ERR_SHAPE, "decode_mtp: num_q_tokens must be >= 1");
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return fail(PKV_ERR_SHAPE, "decode_mtp: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
    if (dtype != PKV_BF16 && dtype != PKV_F32) return fail(PKV_ERR_DTYPE, "decode_mtp: unknown dtype %d", dtype);
    const int64_t cols = (int64_t)num_q_tokens * (num_q_heads / num_kv_heads);
    if (dtype != PKV_BF16 || cols > 16)
        return fail(PKV_ERR_UNSUPPORTED, "decode_mtp: bf16 with num_q_tokens * (query heads per kv head) <= 16 "
                    "(got %lld); pkv_paged_attn_varlen_ex covers the rest", (long long)cols);
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "decode_mtp: block_size %d is not a power of two in [1, 256]", block_size);
    if (!pkv::gqa_stream_shape_supported(head_dim, log2i(block_size), batch))
        return fail(PKV_ERR_UNSUPPORTED, "decode_mtp: head_dim %d, block_size %d, batch %d not supported "
                    "(head_dim 64/128, block_size >= 1024 / (2 head_dim), batch <= 1024); "
                    "pkv_paged_attn_varlen_ex covers the rest", head_dim, block_size, batch);
    if ((int64_t)batch * num_q_tokens > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "decode_mtp: too many rows");
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    int rc = prepare_decode(p, plan, out, lse_out, q, nullptr, k_cache, v_cache, nullptr, block_table,
                            seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads,
                            num_kv_heads, head_dim, head_dim, 0, block_size, num_blocks, softmax_scale,
                            dtype, workspace, workspace_bytes, &idle, window, true, false, num_q_tokens);
    if (rc != PKV_OK || idle) return rc;
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "decode_mtp_append: k_new and v_new must both be given");
    if (k_new) {
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PKV_ERR_ALIGN, "decode_mtp_append: k_new and v_new must be 16-byte aligned");
        if (k_cache == v_cache) return fail(PKV_ERR_SHAPE, "decode_mtp_append: k_cache and v_cache must differ");
        p.k_new = k_new;
        p.v_new = v_new;
        p.k_cache_w = const_cast<void*>(k_cache);
        p.v_cache_w = const_cast<void*>(v_cache);
        p.slots_out = slot_mapping_out;
    }
    hipStream_t s = (hipStream_t)stream;
    if (stages & 1) {
        rc = hip_status(pkv::launch_gqa_decode(p, head_dim, s), "decode_mtp launch");
        if (rc != PKV_OK) return rc;
    }
    if ((stages & 2) && needs_combine(p, plan)) return launch_combine_for(p, head_dim, dtype, s);
    return PKV_OK;
}

int pkv_paged_attn_decode_mtp(void* out, float* lse_out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens_kv, int32_t batch, int32_t num_q_tokens,
                              int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, float softmax_scale,
                              int32_t dtype, int32_t window, int32_t stages, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return mtp_impl(out, lse_out, q, k_cache, v_cache, block_table, seq_lens_kv, batch, num_q_tokens,
                    max_blocks_per_seq, max_seq_len_kv, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, softmax_scale, dtype, window, stages, workspace, workspace_bytes, nullptr,
                    nullptr, nullptr, stream);
}

int pkv_paged_attn_decode_mtp_append(void* out, float* lse_out, const void* q, const void* k_new,
                                     const void* v_new, void* k_cache, void* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens_kv,
                                     int32_t batch, int32_t num_q_tokens, int32_t max_blocks_per_seq,
                                     int32_t max_seq_len_kv, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int64_t num_blocks, float softmax_scale, int32_t dtype,
                                     int32_t window, int32_t stages, void* workspace,
                                     size_t workspace_bytes, int64_t* slot_mapping_out, void* stream) {
    if (batch > 0 && (!k_new || !v_new)) return fail(PKV_ERR_NULL, "decode_mtp_append: NULL pointer argument");
    return mtp_impl(out, lse_out, q, k_cache, v_cache, block_table, seq_lens_kv, batch, num_q_tokens,
                    max_blocks_per_seq, max_seq_len_kv, num_q_heads, num_kv_heads, head_dim, block_size,
                    num_blocks, softmax_scale, dtype, window, stages, workspace, workspace_bytes, k_new,
                    v_new, slot_mapping_out, stream);
}

int pkv_kv_cache_write_int8_mla(const void* kv_nope, const void* k_rope, void* nope_codes,
                                void* rope_codes, float* nope_scale, float* rope_scale,
                                const int64_t* slot_mapping, int64_t num_tokens, int32_t block_size,
                                int64_t num_blocks, int32_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_ERR_DTYPE, "kv_cache_write_int8_mla: unknown input dtype %d", dtype);
    if (num_tokens < 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "kv_cache_write_int8_mla: num_blocks must be positive (num_tokens >= 0)");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write_int8_mla: block_size %d is not a power of two in [1, 256]",
                    block_size);
    if (num_tokens > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "kv_cache_write_int8_mla: too many tokens");
    if (num_tokens == 0) return PKV_OK;
    if (!kv_nope || !k_rope || !nope_codes || !rope_codes || !nope_scale || !rope_scale || !slot_mapping)
        return fail(PKV_ERR_NULL, "kv_cache_write_int8_mla: NULL pointer argument");
    if (!aligned16(kv_nope) || !aligned16(k_rope) || !aligned16(nope_codes) || !aligned16(rope_codes) ||
        !aligned16(nope_scale) || !aligned16(rope_scale))
        return fail(PKV_ERR_ALIGN, "kv_cache_write_int8_mla: all arrays must be 16-byte aligned");
    if (nope_codes == rope_codes || nope_scale == rope_scale)
        return fail(PKV_ERR_SHAPE, "kv_cache_write_int8_mla: nope and rope arrays must differ");
    pkv::QuantWriteParams p{};
    p.k_new = kv_nope;
    p.v_new = k_rope;
    p.k_cache = static_cast<int8_t*>(nope_codes);
    p.v_cache = static_cast<int8_t*>(rope_codes);
    p.k_scale = nope_scale;
    p.v_scale = rope_scale;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.hkv = 1;
    p.bs_log2 = log2i(block_size);
    return hip_status(pkv::launch_kv_write_int8_mla(p, dtype, (hipStream_t)stream),
                      "kv_cache_write_int8_mla launch");
}

int pkv_paged_attn_decode_mla_int8(void* out, float* lse_out, const void* q, const void* q_rope,
                                   const void* nope_codes, const void* rope_codes,
                                   const float* nope_scale, const float* rope_scale,
                                   const int32_t* block_table, const int32_t* seq_lens_kv, int32_t batch,
                                   int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                                   int32_t num_q_heads, int32_t block_size, int64_t num_blocks,
                                   float softmax_scale, int32_t stages, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "decode_mla_int8: stages must be 1, 2 or 3");
    if (!q_rope || !rope_codes) return fail(PKV_ERR_NULL, "decode_mla_int8: q_rope and rope_codes are required");
    bool mla = false;
    int rc = check_decode_common(q_rope, rope_codes, PKV_BF16, batch, num_q_heads, 1, 512, 512, 64,
                                 max_blocks_per_seq, max_seq_len_kv, block_size, num_blocks,
                                 softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    if (block_size < 4)
        return fail(PKV_ERR_UNSUPPORTED, "decode_mla_int8: block_size %d (needs >= 4: a 4-key group's scales are one load)",
                    block_size);
    if (batch == 0) return PKV_OK;
    if (!nope_scale || !rope_scale) return fail(PKV_ERR_NULL, "decode_mla_int8: NULL scale array");
    if (!aligned16(nope_scale) || !aligned16(rope_scale))
        return fail(PKV_ERR_ALIGN, "decode_mla_int8: scale arrays must be 16-byte aligned");
    return run_mla_decode(out, lse_out, q, q_rope, nope_codes, nope_codes, rope_codes, block_table,
                          seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads, 1, 512,
                          512, 64, block_size, num_blocks, softmax_scale, PKV_BF16, workspace,
                          workspace_bytes, stages, (hipStream_t)stream, nope_scale, rope_scale);
}

int pkv_paged_attn_decode_mla_int8_append(void* out, float* lse_out, const void* q, const void* q_rope,
                                          const void* nope_new, const void* rope_new,
                                          void* nope_codes, void* rope_codes, float* nope_scale,
                                          float* rope_scale, const int32_t* block_table,
                                          const int32_t* seq_lens_kv, int64_t* slot_mapping_out,
                                          int32_t batch, int32_t max_blocks_per_seq,
                                          int32_t max_seq_len_kv, int32_t num_q_heads,
                                          int32_t block_size, int64_t num_blocks, float softmax_scale,
                                          int32_t stages, void* workspace, size_t workspace_bytes,
                                          void* stream) {
    const char* who = "decode_mla_int8_append";
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "%s: stages must be 1, 2 or 3", who);
    if (!q_rope || !rope_codes) return fail(PKV_ERR_NULL, "%s: q_rope and rope_codes are required", who);
    bool mla = false;
    int rc = check_decode_common(q_rope, rope_codes, PKV_BF16, batch, num_q_heads, 1, 512, 512, 64,
                                 max_blocks_per_seq, max_seq_len_kv, block_size, num_blocks,
                                 softmax_scale, &mla);
    if (rc != PKV_OK) return rc;
    if (block_size < 4)
        return fail(PKV_ERR_UNSUPPORTED, "%s: block_size %d (needs >= 4: a 4-key group's scales are one load)",
                    who, block_size);
    if (batch == 0) return PKV_OK;
    if (!nope_new || !rope_new) return fail(PKV_ERR_NULL, "%s: NULL new rows", who);
    if (!nope_scale || !rope_scale) return fail(PKV_ERR_NULL, "%s: NULL scale array", who);
    if (!aligned16(nope_scale) || !aligned16(rope_scale) || !aligned16(nope_new) || !aligned16(rope_new))
        return fail(PKV_ERR_ALIGN, "%s: scale arrays and new rows must be 16-byte aligned", who);
    if (nope_codes == rope_codes || nope_scale == rope_scale)
        return fail(PKV_ERR_SHAPE, "%s: the nope and rope arrays must differ", who);
    return run_mla_decode(out, lse_out, q, q_rope, nope_codes, nope_codes, rope_codes, block_table,
                          seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads, 1, 512,
                          512, 64, block_size, num_blocks, softmax_scale, PKV_BF16, workspace,
                          workspace_bytes, stages, (hipStream_t)stream, nope_scale, rope_scale,
                          nope_new, rope_new, slot_mapping_out);
}

int pkv_kv_cache_write_int8(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                            float* k_scale, float* v_scale, const int64_t* slot_mapping,
                            int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int64_t num_blocks, int32_t dtype, void* stream) {
    if (dtype != PKV_F32 && dtype != PKV_BF16)
        return fail(PKV_ERR_DTYPE, "kv_cache_write_int8: unknown input dtype %d", dtype);
    if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0)
        return fail(PKV_ERR_SHAPE, "kv_cache_write_int8: num_kv_heads and num_blocks must be positive");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write_int8: head_dim %d not supported (64 or 128)", head_dim);
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write_int8: block_size %d is not a power of two in [1, 256]",
                    block_size);
    if (num_tokens * num_kv_heads > 0x7fffffffLL * 16)
        return fail(PKV_ERR_UNSUPPORTED, "kv_cache_write_int8: too many rows");
    if (num_tokens == 0) return PKV_OK;
    if (!k_new || !v_new || !k_cache || !v_cache || !k_scale || !v_scale || !slot_mapping)
        return fail(PKV_ERR_NULL, "kv_cache_write_int8: NULL pointer argument");
    if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(k_scale) || !aligned16(v_scale))
        return fail(PKV_ERR_ALIGN, "kv_cache_write_int8: arrays must be 16-byte aligned");
    if (k_cache == v_cache || k_scale == v_scale)
        return fail(PKV_ERR_SHAPE, "kv_cache_write_int8: K and V need their own codes and scales");
    pkv::QuantWriteParams p{};
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache = static_cast<int8_t*>(k_cache);
    p.v_cache = static_cast<int8_t*>(v_cache);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    p.slots = slot_mapping;
    p.num_tokens = num_tokens;
    p.num_slots = num_blocks * block_size;
    p.hkv = num_kv_heads;
    p.bs_log2 = log2i(block_size);
    return hip_status(pkv::launch_kv_write_int8(p, dtype, head_dim, (hipStream_t)stream),
                      "kv_cache_write_int8 launch");
}

}  // extern "C"

namespace {

// Decode over the INT8 caches; with k_new / v_new (bf16, 1..4 query heads per kv head) the
// step's token is quantized, written and attended in the same pass.
int run_decode_int8(void* out, float* lse_out, const void* q, const void* k_new, const void* v_new,
                    void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                    const int32_t* block_table, const int32_t* seq_lens_kv, int64_t* slot_mapping_out,
                    int32_t batch, int32_t max_blocks_per_seq, int32_t max_seq_len_kv,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                    int64_t num_blocks, float softmax_scale, int32_t window, int32_t stages,
                    void* workspace, size_t workspace_bytes, void* stream, const char* who) {
    if (stages < 1 || stages > 3) return fail(PKV_ERR_SHAPE, "%s: stages must be 1, 2 or 3", who);
    // 1..4 query heads per kv head: the split kernel; 5..16: the range-streaming kernel, whose
    // code loads need blocks of at least 1024 / head_dim keys.
    const int group = num_kv_heads > 0 && num_q_heads % num_kv_heads == 0 ? num_q_heads / num_kv_heads : 0;
    const bool ranges = group > 4;
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "%s: k_new and v_new must be given together or not at all", who);
    if (ranges && (group > 16 || (head_dim != 64 && head_dim != 128) || block_size <= 0 ||
                   (block_size & (block_size - 1)) || block_size < 1024 / head_dim ||
                   !pkv::gqa_stream_supported(PKV_BF16, group, head_dim, log2i(block_size), batch)))
        return fail(PKV_ERR_UNSUPPORTED,
                    "%s: %d query heads per kv head needs at most 16, head_dim 64 or 128, "
                    "block_size >= %d and batch <= 1024 (got head_dim %d, block_size %d, batch %d)",
                    who, group, head_dim == 64 ? 16 : 8, head_dim, block_size, batch);
    pkv::DecodeParams p;
    pkv::DecodePlan plan{};
    bool idle = false;
    // The codes are one byte per element; the host checks run on the bf16 query shape.
    int rc = prepare_decode(p, plan, out, lse_out, q, nullptr, k_cache, v_cache, nullptr, block_table,
                            seq_lens_kv, batch, max_blocks_per_seq, max_seq_len_kv, num_q_heads,
                            num_kv_heads, head_dim, head_dim, 0, block_size, num_blocks, softmax_scale,
                            PKV_BF16, workspace, workspace_bytes, &idle, window, ranges, true);
    if (rc != PKV_OK || idle) return rc;
    if (ranges != (p.parts > 0)) return fail(PKV_ERR_UNSUPPORTED, "%s: no kernel for this shape", who);
    if (!k_scale || !v_scale) return fail(PKV_ERR_NULL, "%s: NULL scale array", who);
    if (!aligned16(k_scale) || !aligned16(v_scale))
        return fail(PKV_ERR_ALIGN, "%s: scale arrays must be 16-byte aligned", who);
    p.k_scale = k_scale;
    p.v_scale = v_scale;
    if (k_new) {
        if (!aligned16(k_new) || !aligned16(v_new))
            return fail(PKV_ERR_ALIGN, "%s: k_new and v_new must be 16-byte aligned", who);
        if (k_cache == v_cache || k_scale == v_scale)
            return fail(PKV_ERR_SHAPE, "%s: the K and V caches (and their scales) must differ", who);
        p.k_new = k_new;
        p.v_new = v_new;
        p.k_cache_w = k_cache;
        p.v_cache_w = v_cache;
        p.k_scale_w = k_scale;
        p.v_scale_w = v_scale;
        p.slots_out = slot_mapping_out;
    }
    hipStream_t s = (hipStream_t)stream;
    if (stages & 1) {
        rc = hip_status(pkv::launch_decode_int8(p, head_dim, s), "decode_int8 split launch");
        if (rc != PKV_OK) return rc;
    }
    if ((stages & 2) && needs_combine(p, plan)) return launch_combine_for(p, head_dim, PKV_BF16, s);
    return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_attn_decode_int8(void* out, float* lse_out, const void* q, const void* k_cache,
                               const void* v_cache, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, const int32_t* seq_lens_kv, int32_t batch,
                               int32_t max_blocks_per_seq, int32_t max_seq_len_kv, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, float softmax_scale, int32_t window, int32_t stages,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return run_decode_int8(out, lse_out, q, nullptr, nullptr, const_cast<void*>(k_cache),
                           const_cast<void*>(v_cache), const_cast<float*>(k_scale),
                           const_cast<float*>(v_scale), block_table, seq_lens_kv, nullptr, batch,
                           max_blocks_per_seq, max_seq_len_kv, num_q_heads, num_kv_heads, head_dim,
                           block_size, num_blocks, softmax_scale, window, stages, workspace,
                           workspace_bytes, stream, "decode_int8");
}

int pkv_paged_attn_decode_int8_append(void* out, float* lse_out, const void* q, const void* k_new,
                                      const void* v_new, void* k_cache, void* v_cache, float* k_scale,
                                      float* v_scale, const int32_t* block_table,
                                      const int32_t* seq_lens_kv, int64_t* slot_mapping_out,
                                      int32_t batch, int32_t max_blocks_per_seq,
                                      int32_t max_seq_len_kv, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                      int64_t num_blocks, float softmax_scale, int32_t window,
                                      int32_t stages, void* workspace, size_t workspace_bytes,
                                      void* stream) {
    if (!k_new || !v_new) return fail(PKV_ERR_NULL, "decode_int8_append: NULL k_new or v_new");
    return run_decode_int8(out, lse_out, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                           block_table, seq_lens_kv, slot_mapping_out, batch, max_blocks_per_seq,
                           max_seq_len_kv, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                           softmax_scale, window, stages, workspace, workspace_bytes, stream,
                           "decode_int8_append");
}

int pkv_paged_attn_varlen(void* out, float* lse_out, const void* q, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens_kv, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, int32_t batch, int64_t total_q,
                          int32_t max_seqlen_q, int32_t max_blocks_per_seq, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                          int64_t num_blocks, float softmax_scale, int32_t causal, int32_t dtype,
                          void* stream) {
    return pkv_paged_attn_varlen_ex(out, lse_out, q, cu_seqlens_q, seq_lens_kv, k_cache, v_cache,
                                    block_table, batch, total_q, max_seqlen_q, max_blocks_per_seq,
                                    num_q_heads, num_kv_heads, head_dim, block_size, num_blocks,
                                    softmax_scale, causal, 0, dtype, stream);
}

}  // extern "C"

namespace {

// pkv_paged_attn_varlen_ex, and with k_new / v_new given its append form.
int varlen_impl(void* out, float* lse_out, const void* q, const int32_t* cu_seqlens_q,
                const int32_t* seq_lens_kv, const void* k_cache, const void* v_cache,
                const int32_t* block_table, int32_t batch, int64_t total_q,
                int32_t max_seqlen_q, int32_t max_blocks_per_seq, int32_t num_q_heads,
                int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int64_t num_blocks, float softmax_scale, int32_t causal, int32_t window,
                int32_t dtype, const void* k_new, const void* v_new, int64_t* slot_mapping_out,
                void* stream) {
    if (window < 0) return fail(PKV_ERR_SHAPE, "varlen: window must be >= 0 (0: no window)");
    if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_DTYPE, "varlen: unknown dtype %d", dtype);
    if (batch < 0 || total_q < 0 || max_seqlen_q < 0)
        return fail(PKV_ERR_SHAPE, "varlen: negative batch, total_q or max_seqlen_q");
    if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads)
        return fail(PKV_ERR_SHAPE, "varlen: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    num_q_heads, num_kv_heads);
    if (max_blocks_per_seq <= 0 || num_blocks <= 0 || head_dim <= 0)
        return fail(PKV_ERR_SHAPE, "varlen: head_dim, max_blocks_per_seq and num_blocks must be positive");
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.0f))
        return fail(PKV_ERR_SCALE, "varlen: softmax_scale must be finite and > 0");
    if (!pow2_in(block_size, 1, 256))
        return fail(PKV_ERR_UNSUPPORTED, "varlen: block_size %d is not a power of two in [1, 256]", block_size);
    if (dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "varlen: bf16 only");
    if (head_dim != 64 && head_dim != 128)
        return fail(PKV_ERR_UNSUPPORTED, "varlen: head_dim %d not supported (64 or 128)", head_dim);
    const int group = num_q_heads / num_kv_heads;
    if (group > 16) return fail(PKV_ERR_UNSUPPORTED, "varlen: %d query heads per kv head (max 16)", group);
    if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return PKV_OK;
    if (!out || !q || !cu_seqlens_q || !seq_lens_kv || !k_cache || !v_cache || !block_table)
        return fail(PKV_ERR_NULL, "varlen: NULL pointer argument");
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
        return fail(PKV_ERR_ALIGN, "varlen: out, q and caches must be 16-byte aligned");
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(PKV_ERR_NULL, "varlen_append: k_new and v_new must both be given");
    if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(PKV_ERR_ALIGN, "varlen_append: k_new and v_new must be 16-byte aligned");
    if (k_new && (k_new == k_cache || v_new == v_cache || k_new == v_cache || v_new == k_cache))
        return fail(PKV_ERR_SHAPE, "varlen_append: the new rows must not be the caches");
    const int tpb = pkv::varlen_tokens_per_block(group);
    const int64_t qblocks = (max_seqlen_q + tpb - 1) / tpb;
    if ((int64_t)num_kv_heads * qblocks * batch > 0x7fffffffLL)
        return fail(PKV_ERR_SHAPE, "varlen: grid too large");
    pkv::MfmaParams p{};
    p.out = out;
    p.lse = lse_out;
    p.q = q;
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.table = block_table;
    p.seq_lens = seq_lens_kv;
    p.cu_q = cu_seqlens_q;
    p.batch = batch;
    p.mbs = max_blocks_per_seq;
    p.hq = num_q_heads;
    p.hkv = num_kv_heads;
    p.group = group;
    p.bs_log2 = log2i(block_size);
    p.len_cap = (int32_t)((int64_t)max_blocks_per_seq * block_size > 0x7fffffffLL
                              ? 0x7fffffff : (int64_t)max_blocks_per_seq * block_size);
    p.q_blocks = (int32_t)qblocks;
    p.causal = causal ? 1 : 0;
    p.window = window;
    p.num_blocks = num_blocks;
    p.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
    p.k_new = k_new;
    p.v_new = v_new;
    p.k_cache_w = const_cast<void*>(k_cache);
    p.v_cache_w = const_cast<void*>(v_cache);
    p.slots_out = slot_mapping_out;
    return hip_status(pkv::launch_varlen(p, head_dim, (hipStream_t)stream), "varlen launch");
}

}  // namespace

extern "C" {

int pkv_paged_attn_varlen_ex(void* out, float* lse_out, const void* q, const int32_t* cu_seqlens_q,
                             const int32_t* seq_lens_kv, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, int32_t batch, int64_t total_q,
                             int32_t max_seqlen_q, int32_t max_blocks_per_seq, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int64_t num_blocks, float softmax_scale, int32_t causal, int32_t window,
                             int32_t dtype, void* stream) {
    return varlen_impl(out, lse_out, q, cu_seqlens_q, seq_lens_kv, k_cache, v_cache, block_table, batch,
                       total_q, max_seqlen_q, max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, softmax_scale, causal, window, dtype, nullptr, nullptr,
                       nullptr, stream);
}

int pkv_paged_attn_varlen_append(void* out, float* lse_out, const void* q, const void* k_new,
                                 const void* v_new, const int32_t* cu_seqlens_q,
                                 const int32_t* seq_lens_kv, void* k_cache, void* v_cache,
                                 const int32_t* block_table, int32_t batch, int64_t total_q,
                                 int32_t max_seqlen_q, int32_t max_blocks_per_seq,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float softmax_scale,
                                 int32_t causal, int32_t window, int32_t dtype,
                                 int64_t* slot_mapping_out, void* stream) {
    if (batch > 0 && total_q > 0 && max_seqlen_q > 0 && (!k_new || !v_new))
        return fail(PKV_ERR_NULL, "varlen_append: NULL pointer argument");
    return varlen_impl(out, lse_out, q, cu_seqlens_q, seq_lens_kv, k_cache, v_cache, block_table, batch,
                       total_q, max_seqlen_q, max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim,
                       block_size, num_blocks, softmax_scale, causal, window, dtype, k_new, v_new,
                       slot_mapping_out, stream);
}

}  // extern "C"
