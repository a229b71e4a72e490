// MHA/GQA decode over the paged cache with MFMA for gfx950, used for 4..16 query heads per
// kv head ("KVCache Optimization Skill", 3.4-3.6 and Mode 1; "Paged KV Cache and Packed
// Sequence", 2.2-2.3).  With G query heads on one kv head, every K/V row serves G dot
// products and G weighted sums: on the vector ALU that is G times the work per byte of
// the MHA case and the VALU, not HBM, sets the pace; on the matrix cores it is a few
// percent of the time the bytes take.
//
// Per tile of 32 keys of one kv head (both kernels below), one wave computes, with the G
// heads as the 16 columns of v_mfma_f32_16x16x32_bf16 (columns past G hold zero queries
// and are not stored):
//  * S^T (16 keys x 16 heads, two per tile) = K . Q^T, K rows from LDS, Q^T in registers;
//  * lane (g, n) holds 4 keys of head n in each half: the head's max and sum take two
//    lane-swap steps, and P^T (bf16) is the B operand of O^T += V^T . P^T with k-slot
//    8 g + 4 h + r standing for key 16 h + 4 g + r;
//  * V^T comes from the row-major V tile with ds_read_b64_tr_b16; K and V rows are
//    unpadded with their 16-byte chunks XOR-swizzled by row.
// The K/V rows reach LDS by direct loads (global_load_lds_dwordx4), several tiles ahead,
// each wave through its own LDS stages (one wave both loads and consumes: no barrier).
//
// gqa_stream_kernel (blocks of at least 4 rows per wave load, up to 1024 sequences): a
// fixed number of workgroups per kv head, all resident at once; the tiles of all
// sequences, laid end to end, are cut into equal contiguous ranges, one per workgroup.
// A workgroup streams its range without a break at sequence boundaries (the next
// sequence's query rows travel with its first tile), finishes in place every sequence
// that lies wholly inside its range, and leaves (m, l, o) for the at most two that cross
// its ends; gqa_stream_combine_kernel merges those.  Equal ranges keep every compute unit
// busy to the end, and the per-workgroup start-up happens once, not once per split.
//
// gqa_decode_kernel (all other shapes): one workgroup per (sequence, split of
// split_tokens keys, kv head), longest sequences first, block-table entries staged in LDS
// by chunks; splits of one sequence are merged by the generic combine kernel.
//
// Append mode reads this step's token from the new rows, and the workgroup whose range
// holds it writes the kv head's slice to the cache.
//
// Multi-token decode (MTP, "KVCache Optimization Skill", Appendix E: next_n + 1 query tokens
// per sequence, causal): the range kernel takes qn query tokens per sequence, the product
// columns standing for (token, head) pairs, qn * G <= 16.  Column (i, h) sees keys up to
// L - qn + i (bottom-right causal, its own token included), so only a sequence's last tile
// is masked differently per column; every K/V row is still read once per kv head.
#include "mfma_common.h"

namespace pkv {

namespace {

using namespace mfma;

template <int D>
struct GqaCfg {
    static constexpr int kRowBytes = 2 * D;             // one K or V row of one head
    static constexpr int kRowChunks = kRowBytes / 16;
    static constexpr int kRowShift = D == 128 ? 0 : 1;  // rows per 256-byte line: 1 or 2
    static constexpr int kHalf = kKeys * kRowBytes;     // K (or V) part of a stage
    static constexpr int kStage = 2 * kHalf;
    static constexpr int kDmaHalf = kHalf / 1024;       // wave loads per half tile
    static constexpr int kDma = 2 * kDmaHalf;           // wave loads per tile
    static constexpr int kRpi = 1024 / kRowBytes;       // rows per wave load: 4 or 8
    static constexpr int kSteps = D / 32;               // S^T k-steps
    static constexpr int kDTiles = D / 16;              // 16-row tiles of O^T
    static_assert(2 * kDma < 64, "vmcnt range");
};

// ------------------------------------------------------------------ per-tile math
// Scores of the tile in `stage`: full tiles keep the raw S^T entries; a tile that is not
// wholly inside the key range [k_lo, k_end) scales them and sets keys outside it to -inf.
// Entry (h, r) of lane (g, n) is key kb + 16 h + 4 g + r.  Returns the head's max over the
// tile (scaled, log2 units).
template <int D>
__device__ __forceinline__ float tile_scores(const uint8_t* stage, const bf16x8_t* qf, int n, int g,
                                             bool full, int kb, int k_lo, int k_end, float scale_log2,
                                             float* sv, const float* kscale = nullptr) {
    using C = GqaCfg<D>;
    f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int r = 16 * h + n;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
            const uint8_t* src = stage + r * C::kRowBytes + swz<C::kRowChunks, C::kRowShift>(r, 4 * s + g) * 16;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(src));
            sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[h], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * C::kSteps, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * C::kSteps, 0);
    if (kscale) {   // INT8 codes: the dot products times each key's K scale
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(kscale + 4 * g);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(kscale + 16 + 4 * g);
        sacc[0] *= s0;
        sacc[1] *= s1;
    }
    float tmax;
    if (full) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][e & 3];
        tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        tmax *= scale_log2;
    } else {
        tmax = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = kb + 16 * (e >> 2) + 4 * g + (e & 3);
            sv[e] = (key >= k_lo && key < k_end) ? sacc[e >> 2][e & 3] * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, sv[e]);
        }
    }
    return max_xor32(max_xor16(tmax));
}

// P^T of the tile against the running max, then O^T += V^T . P^T (V half of `stage`).
template <int D>
__device__ __forceinline__ void tile_pv(const uint8_t* stage, RowState& st, bool full, const float* sv,
                                        float scale_log2, int n, int g, f32x4* oacc,
                                        const float* vscale = nullptr) {
    using C = GqaCfg<D>;
    // INT8 codes: each key's V scale goes into its weight for the value sum (P' = p s_v; the
    // masked keys' stale scales never reach it), while l sums the fp32 p.
    float vs[8];
    if (vscale) {
        const f32x4 s0 = *reinterpret_cast<const f32x4*>(vscale + 4 * g);
        const f32x4 s1 = *reinterpret_cast<const f32x4*>(vscale + 16 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) { vs[e] = s0[e]; vs[4 + e] = s1[e]; }
    }
    u32x4 pw;
    if (full) {
        const float mneg = -st.m;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float e0 = fast_exp2(__builtin_fmaf(sv[e], scale_log2, mneg));
            const float e1 = fast_exp2(__builtin_fmaf(sv[e + 1], scale_log2, mneg));
            st.l += e0 + e1;
            pw[e >> 1] = vscale ? pack_bf16(e0 * vs[e], e1 * vs[e + 1]) : pack_bf16(e0, e1);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float e0 = sv[e] == -INFINITY ? 0.0f : fast_exp2(sv[e] - st.m);
            const float e1 = sv[e + 1] == -INFINITY ? 0.0f : fast_exp2(sv[e + 1] - st.m);
            st.l += e0 + e1;
            pw[e >> 1] = vscale ? pack_bf16(sv[e] == -INFINITY ? 0.0f : e0 * vs[e],
                                            sv[e + 1] == -INFINITY ? 0.0f : e1 * vs[e + 1])
                                : pack_bf16(e0, e1);
        }
    }
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
    const uint8_t* vt = stage + C::kHalf;
    // Lane (g, n) reads rows 16 h + 4 g + n / 4, value columns 16 dt + 4 (n % 4) .. + 3.
    const int r0 = 4 * g + (n >> 2), r1 = 16 + r0;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
        const int c = 2 * dt + ((n & 3) >> 1);
        const uint8_t* a0 = vt + r0 * C::kRowBytes + swz<C::kRowChunks, C::kRowShift>(r0, c) * 16 + 8 * (n & 1);
        const uint8_t* a1 = vt + r1 * C::kRowBytes + swz<C::kRowChunks, C::kRowShift>(r1, c) * 16 + 8 * (n & 1);
        // Assemble the operand from whole dwords: extracting the 16-bit elements one by
        // one made the compiler keep only the first dword of each read.
        const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(a0));
        const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(a1));
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * C::kDTiles, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::kDTiles, 0);
}

// Rescale for a tile whose max grew past the slack (or the first finite one).
template <int D>
__device__ __forceinline__ void rescale(RowState& st, float tmax, f32x4* oacc) {
    using C = GqaCfg<D>;
    const bool grow = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
    const float mnew = grow ? tmax : st.m;
    const float alpha = !grow ? 1.0f : (st.m == -INFINITY ? 0.0f : fast_exp2(st.m - mnew));
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) oacc[dt] *= alpha;
    st.m = mnew;
}

__device__ __forceinline__ bool must_rescale(const RowState& st, float tmax) {
    return tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
}

// Final output of one (sequence, kv head): the G rows in bf16 and their lse.
template <int D>
__device__ __forceinline__ void store_final(const DecodeParams& p, int64_t row, int g, float m, float l_tot,
                                            const f32x4* oacc) {
    using C = GqaCfg<D>;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + row * D + 4 * g;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) {
        const uint32_t w0 = bf16_bits(oacc[dt][0] * inv) | ((uint32_t)bf16_bits(oacc[dt][1] * inv) << 16);
        const uint32_t w1 = bf16_bits(oacc[dt][2] * inv) | ((uint32_t)bf16_bits(oacc[dt][3] * inv) << 16);
        *reinterpret_cast<uint2*>(out + 16 * dt) = make_uint2(w0, w1);
    }
    if (p.lse && g == 0) p.lse[row] = l_tot > 0.0f ? (m + __log2f(l_tot)) * kLn2f : -INFINITY;
}

// No visible key: output 0, lse -inf.
template <int D>
__device__ __forceinline__ void store_empty(const DecodeParams& p, int64_t row, int g) {
    using C = GqaCfg<D>;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + row * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) *reinterpret_cast<uint2*>(out + 16 * dt) = make_uint2(0u, 0u);
    if (p.lse && g == 0) p.lse[row] = -INFINITY;
}

// The kv head's slices of sequence b's qn new K and V rows (rows b qn + i of k_new / v_new,
// positions L - qn + i) to their slots (append mode), by the first 2 kRowChunks lanes.
// A row longer than the length bound (a broken precondition) appends nothing: its slots are
// reported as -1 (the lookups of the new keys, from `new_key` on, then never match either).
template <int D>
__device__ __forceinline__ void append_row(const DecodeParams& p, int b, int kvh, int L, int lane, int qn = 1) {
    using C = GqaCfg<D>;
    if (uniform_load(p.seq_lens + b) > p.len_cap) {
        if (p.slots_out && kvh == 0 && lane < qn) p.slots_out[(int64_t)b * qn + lane] = -1;
        return;
    }
    if (lane >= 2 * C::kRowChunks) return;
    const int32_t* trow = p.table + (int64_t)b * p.mbs;
    const int which = lane / C::kRowChunks;
    const int64_t off = (int64_t)(lane % C::kRowChunks) * 16;
    for (int i = 0; i < qn; ++i) {
        const int pos = L - qn + i;
        int64_t slot = -1;
        if (pos >= 0) {
            const int32_t phys = min(max(trow[pos >> p.bs_log2], 0), (int32_t)(p.num_blocks - 1));
            slot = ((int64_t)phys << p.bs_log2) | (pos & ((1 << p.bs_log2) - 1));
            const int64_t new_off = (((int64_t)b * qn + i) * p.hkv + kvh) * D * 2;
            const uint8_t* src = reinterpret_cast<const uint8_t*>(which ? p.v_new : p.k_new) + new_off;
            uint8_t* dst = reinterpret_cast<uint8_t*>(which ? p.v_cache_w : p.k_cache_w) +
                           slot * (int64_t)p.hkv * D * 2 + (int64_t)kvh * D * 2;
            st16(dst + off, ld16(src + off));
        }
        if (p.slots_out && kvh == 0 && lane == 0) p.slots_out[(int64_t)b * qn + i] = slot;
    }
}

// INT8 form: the kv head's slices of the new bf16 K and V rows quantized as the writer does
// (s = max|x| / 127, q = round_half_even(x / s), the same fp32 operations, so the same codes
// and scale bit for bit) and stored at the slot with their scales; two values per lane.
// The caller waits for the stores before any load of that key.
template <int D>
__device__ __forceinline__ void append_row_i8(const DecodeParams& p, int b, int kvh, int L, int lane) {
    if (uniform_load(p.seq_lens + b) > p.len_cap) {
        if (p.slots_out && kvh == 0 && lane == 0) p.slots_out[b] = -1;
        return;
    }
    const int32_t* trow = p.table + (int64_t)b * p.mbs;
    const int32_t phys = min(max(trow[(L - 1) >> p.bs_log2], 0), (int32_t)(p.num_blocks - 1));
    const int off_in_block = (L - 1) & ((1 << p.bs_log2) - 1);
    const int64_t slot = ((int64_t)phys << p.bs_log2) | off_in_block;
    const int64_t sc_idx = (((int64_t)phys * p.hkv + kvh) << p.bs_log2) | off_in_block;
    const int64_t src_off = (((int64_t)b * p.hkv + kvh) * D + 2 * (lane % (D / 2))) * 2;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint32_t pair = *reinterpret_cast<const uint32_t*>(
            reinterpret_cast<const uint8_t*>(which ? p.v_new : p.k_new) + src_off);
        const float x0 = bf16_lo(pair), x1 = bf16_hi(pair);
        float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
        for (int sft = 1; sft < D / 2; sft <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sft, 64));
        const float sc = __fdiv_rn(amax, 127.0f);
        uint32_t w = 0u;
        if (sc > 0.0f) {
            const float q0 = fminf(fmaxf(rintf(__fdiv_rn(x0, sc)), -127.0f), 127.0f);
            const float q1 = fminf(fmaxf(rintf(__fdiv_rn(x1, sc)), -127.0f), 127.0f);
            w = ((uint32_t)(int)q0 & 0xffu) | (((uint32_t)(int)q1 & 0xffu) << 8);
        }
        if (lane < D / 2) {
            uint8_t* dst = reinterpret_cast<uint8_t*>(which ? p.v_cache_w : p.k_cache_w) +
                           slot * (int64_t)p.hkv * D + (int64_t)kvh * D + 2 * lane;
            *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
            if (lane == 0) (which ? p.v_scale_w : p.k_scale_w)[sc_idx] = sc;
        }
    }
    if (p.slots_out && kvh == 0 && lane == 0) p.slots_out[b] = slot;
}

// ================================================================== range-streaming kernel
constexpr int kStreamStages = 3;       // LDS stages: two tiles in flight while one is used
constexpr int kStreamCompactStages = 2;   // compact layout: one tile in flight while one is used
constexpr int kStreamMaxBatch = 1024;  // sequences whose tile prefix fits LDS
constexpr int kStreamWgs = 512;        // workgroups per launch (all kv heads): 2 per CU
constexpr int kStreamWgsCompact = 1024;  // compact layout: 4 per CU, one wave on every SIMD
// INT8: the wave's instructions (the code conversion above all), not the memory, set the
// pace, so time falls with the waves per CU: a bf16 buffer of one half tile (K, then V)
// leaves room for 5 workgroups per CU.
constexpr int kStreamWgsI8 = 1280;

// LDS of the range kernel.  Default layout (bf16): kStreamStages tile stages, a ring of query
// rows per stage, the tile prefix and the lengths.  Compact layout (under 40 KiB, for four
// workgroups per CU; INT8 always, bf16 on long contexts): two stages (INT8: of codes as
// loaded, K rows of D bytes, V rows, then 1 KiB whose first 256 bytes are the tile's 32 K
// and 32 V scales, plus a bf16 half tile the wave converts the K codes, then the V codes
// into: under 32 KiB, five workgroups per CU) and the tile prefix; the query rows stay in
// registers and the lengths are read from memory.
template <int D, bool I8 = false, bool COMPACT = I8>
struct StreamCfg {
    using C = GqaCfg<D>;
    static constexpr int kCodeHalf = kKeys * D;                       // K (or V) codes of a tile
    static constexpr int kCodeStage = 2 * kCodeHalf + 1024;
    static constexpr int kCodeRpi = 1024 / D;                         // code rows per wave load: 8 or 16
    static constexpr int kCodeDmaHalf = kKeys / kCodeRpi;             // wave loads per half: 4 or 2
    static constexpr int kDma = I8 ? 2 * kCodeDmaHalf + 1 : C::kDma;  // wave loads per tile
    static constexpr bool kCompact = COMPACT;                     // Q in registers, no lengths
    static_assert(COMPACT || !I8, "INT8 runs in the compact layout");
    static constexpr int kStages = kCompact ? kStreamCompactStages : kStreamStages;
    static constexpr int kPerCu = (I8 ? kStreamWgsI8 : kCompact ? kStreamWgsCompact : kStreamWgs) / 256;
    static constexpr int kStagesBytes = I8 ? kStages * kCodeStage + C::kHalf : kStages * C::kStage;
    static constexpr int kBufOff = kStages * kCodeStage;              // INT8: the bf16 tile
    static constexpr int kQSlot = kCompact ? 0 : 16 * C::kRowBytes;   // one segment's query rows
    static constexpr int kQOff = kStagesBytes;
    static constexpr int kPreOff = kQOff + kStages * kQSlot;          // [batch + 1] first tile
    static constexpr int kLenOff = kPreOff + (kStreamMaxBatch + 1) * 4 + 12;  // [batch] lengths
    static constexpr int kSmem = kLenOff + (kCompact ? 0 : kStreamMaxBatch * 4);
    static_assert(kSmem <= 160 * 1024 / kPerCu, "the workgroups of a CU share its LDS");
    static_assert(2 * kDma < 64, "vmcnt range");
};

// Start of range w of P over T tiles, and the range that holds tile x.
__device__ __forceinline__ int range_start(int w, int T, int P) { return (int)((int64_t)w * T / P); }
__device__ __forceinline__ int range_of(int x, int T, int P) { return (int)(((int64_t)(x + 1) * P - 1) / T); }

// Position in the end-to-end tile order: sequence b holds tiles [pre, end) and has
// length L; its visible keys start at ks (a sliding window moves it up) and its tiles at
// ksa = ks rounded down to a tile; seg counts the sequences with tiles entered so far.
struct Cursor {
    int b, pre, end, L, ks, ksa, seg;
    int ks_last;                      // first key the last query token sees (>= ks)
    int new_key;                      // append mode: first key read from the new rows (L - qn), else INT_MAX
};

// Append mode: the first key of sequence b that comes from the new rows, L - qn (qn new
// rows per sequence: 1 for decode), unless the row is longer than the length bound; INT_MAX
// (no key) otherwise and outside append mode.
template <bool APPEND>
__device__ __forceinline__ int new_key_of(const DecodeParams& p, int b, int L, int qn = 1) {
    if (!APPEND) return INT_MAX;
    return uniform_load(p.seq_lens + b) <= p.len_cap ? L - qn : INT_MAX;
}

template <int D, bool APPEND, bool I8 = false, bool COMPACT = I8>
__global__ __launch_bounds__(64) void gqa_stream_kernel(DecodeParams p) {
    using C = GqaCfg<D>;
    using S = StreamCfg<D, I8, COMPACT>;
    constexpr int kStg = S::kStages;
    __shared__ __attribute__((aligned(16))) uint8_t smem[S::kSmem];
    int32_t* s_pre = reinterpret_cast<int32_t*>(smem + S::kPreOff);
    int32_t* s_len = S::kCompact ? nullptr : reinterpret_cast<int32_t*>(smem + S::kLenOff);
    // Visible length of sequence b: per lane, and (b uniform) in SGPRs.
    auto lane_len = [&](int b) { return S::kCompact ? min(p.seq_lens[b], p.len_cap) : s_len[b]; };
    auto uni_len = [&](int b) {
        return S::kCompact ? min(uniform_load(p.seq_lens + b), p.len_cap)
                           : __builtin_amdgcn_readfirstlane(s_len[b]);
    };

    const int lane = threadIdx.x;
    const int n = lane & 15;          // head column of this lane; A-operand row
    const int g = lane >> 4;          // k-slot group
    const int kvh = blockIdx.x % p.hkv;
    const int w = blockIdx.x / p.hkv;
    const int P = p.parts;
    const int G = p.group;
    const int qn = max(p.qn, 1);      // query tokens per sequence (1: decode)
    const int NC = qn * G;            // columns in use: (token, head) pairs
    const bool valid = n < NC;
    const int tok = valid ? n / G : 0;
    const int hcol = n - tok * G;
    const int back = qn - 1 - tok;    // this column sees keys below L - back
    auto out_row = [&](int b) { return ((int64_t)b * qn + tok) * p.hq + kvh * G + hcol; };

    // Tiles of every sequence and their prefix over the batch (the same in every
    // workgroup; workgroup 0 also leaves it for the combine).  Tiles start at the first
    // key the first query token sees.
    int total = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
        const int b = c0 + lane;
        const int L = b < p.batch ? min(p.seq_lens[b], p.len_cap) : 0;
        const int nt = L > 0 ? (L - window_start32(L - qn + 1, p.window) + kKeys - 1) / kKeys : 0;
        int v = nt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (b < p.batch) {
            s_pre[b] = total + v - nt;
            if constexpr (!S::kCompact) s_len[b] = L;
            if (blockIdx.x == 0) p.tile_prefix[b] = total + v - nt;
        }
        total += __shfl(v, 63, 64);
    }
    const int T = __builtin_amdgcn_readfirstlane(total);
    if (lane == 0) {
        s_pre[p.batch] = T;
        if (blockIdx.x == 0) p.tile_prefix[p.batch] = T;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int x0 = T > 0 ? range_start(w, T, P) : 0;
    const int x1 = T > 0 ? range_start(w + 1, T, P) : 0;
    const int ntw = x1 - x0;

    // Sequences with no key (range 0 of each kv head): output 0, lse -inf.  Append mode:
    // the range that holds a sequence's last tile writes its new rows.
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
        const int b = c0 + lane;
        bool empty = false, mine = false;
        if (b < p.batch) {
            const int e = s_pre[b + 1];
            empty = lane_len(b) <= 0;
            mine = e > s_pre[b] && e - 1 >= x0 && e - 1 < x1;
            if (APPEND && empty && p.slots_out && w == 0 && kvh == 0)
                for (int i = 0; i < qn; ++i) p.slots_out[(int64_t)b * qn + i] = -1;
        }
        uint64_t em = w == 0 ? __ballot(empty) : 0ull;
        while (em) {
            const int bb = c0 + __builtin_ctzll(em);
            em &= em - 1;
            if (valid) store_empty<D>(p, out_row(bb), g);
        }
        if (APPEND) {
            uint64_t mm = __ballot(mine);
            while (mm) {
                const int bb = c0 + __builtin_ctzll(mm);
                mm &= mm - 1;
                if constexpr (I8) append_row_i8<D>(p, bb, kvh, uni_len(bb), lane);
                else append_row<D>(p, bb, kvh, uni_len(bb), lane, qn);
            }
        }
    }
    // INT8: the new codes are read back from the cache by this range's last tile of the
    // sequence (bf16 reads the new rows instead), so the stores complete first.
    if constexpr (APPEND && I8) __threadfence_block();
    if (ntw <= 0) return;

    // The sequence that holds tile x0 (the first with tiles past x0).
    int b0 = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
        const int b = c0 + lane;
        const uint64_t m = __ballot(b < p.batch && s_pre[b + 1] > x0);
        if (m) {
            b0 = c0 + __builtin_ctzll(m);
            break;
        }
    }
    b0 = __builtin_amdgcn_readfirstlane(b0);
    auto cursor_at = [&](int b) {
        Cursor c;
        c.b = b;
        c.pre = __builtin_amdgcn_readfirstlane(s_pre[b]);
        c.end = __builtin_amdgcn_readfirstlane(s_pre[b + 1]);
        c.L = uni_len(b);
        c.ks = window_start(c.L - qn + 1, p.window);
        c.ks_last = window_start(c.L, p.window);
        c.ksa = c.ks & ~(kKeys - 1);
        c.seg = 0;
        c.new_key = new_key_of<APPEND>(p, b, c.L, qn);
        return c;
    };
    // Move c to the sequence that holds tile x (x never moves back).
    auto advance = [&](Cursor& c, int x) {
        if (x < c.end) return;
        do {
            ++c.b;
            c.pre = c.end;
            c.end = __builtin_amdgcn_readfirstlane(s_pre[c.b + 1]);
        } while (x >= c.end);
        c.L = uni_len(c.b);
        c.ks = window_start(c.L - qn + 1, p.window);
        c.ks_last = window_start(c.L, p.window);
        c.ksa = c.ks & ~(kKeys - 1);
        c.new_key = new_key_of<APPEND>(p, c.b, c.L, qn);
        ++c.seg;
    };

    // Per-lane part of the loads: wave load j of a half fills LDS slots 64 j .. 64 j + 63
    // of the K (V) tile: slot q is row q / kRowChunks, physical chunk q % kRowChunks,
    // which holds logical chunk swz(row, physical chunk) of that row.
    const uint32_t row_bytes = (uint32_t)(p.hkv * D * 2);            // one cache slot
    const int lrow = lane / C::kRowChunks;                           // row within a wave load
    uint32_t lchunk[C::kDmaHalf];
#pragma unroll
    for (int j = 0; j < C::kDmaHalf; ++j)
        lchunk[j] = (uint32_t)swz<C::kRowChunks, C::kRowShift>(j * C::kRpi + lrow, lane % C::kRowChunks) * 16u;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_cache) + kvh * D * 2;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_cache) + kvh * D * 2;
    // INT8: code rows of D bytes (this kv head's slice of a slot of hkv D bytes), 16 bytes
    // per lane, kept in the order loaded (the conversion applies the swizzle).
    const uint32_t crow_bytes = (uint32_t)(p.hkv * D);
    const int crow = lane / (D / 16);
    const uint32_t cchunk = (uint32_t)(lane % (D / 16)) * 16u;
    const uint32_t cvoff = (uint32_t)crow * crow_bytes + cchunk;
    const uint8_t* kcodes = reinterpret_cast<const uint8_t*>(p.k_cache) + kvh * D;
    const uint8_t* vcodes = reinterpret_cast<const uint8_t*>(p.v_cache) + kvh * D;
    const int bs_mask = (1 << p.bs_log2) - 1;
    const int32_t last_block = (int32_t)(p.num_blocks - 1);
    uint8_t* const qring = smem + S::kQOff;
    // Compact layout: the query fragments of the segment whose first tile was issued last.  With two
    // stages that tile is issued one tile ahead, and the consume side takes the fragments
    // at the segment's start, before it issues the next tile.
    static_assert(!S::kCompact || kStg == 2, "one query register set");
    u32x4 qnext[C::kSteps];
    const int nq = (NC * C::kRowBytes + 1023) / 1024;
    const uint8_t* const qbase = reinterpret_cast<const uint8_t*>(p.q);

    // Issue side.  The block-table entries of a tile (one per wave load; every wave load
    // lies in one block) are read through the scalar cache one tile before its loads.
    Cursor ic = cursor_at(b0);
    int32_t pe[C::kDmaHalf];          // entries of the pending tile
    int32_t pe_last = 0;              // entry of the block of the sequence's last key
    auto prep = [&](int u) {          // entries of local tile u
        advance(ic, x0 + u);
        const int kb = ic.ksa + (x0 + u - ic.pre) * kKeys;
        const int32_t* trow = p.table + (int64_t)ic.b * p.mbs;
        const int last_idx = (ic.L - 1) >> p.bs_log2;
        if (p.bs_log2 >= 5) {         // the tile lies in one block: one entry
            const int32_t e = uniform_load(trow + min(kb >> p.bs_log2, last_idx));
#pragma unroll
            for (int j = 0; j < C::kDmaHalf; ++j) pe[j] = e;
        } else {
#pragma unroll
            for (int j = 0; j < C::kDmaHalf; ++j) pe[j] = uniform_load(trow + min((kb + j * C::kRpi) >> p.bs_log2, last_idx));
        }
        pe_last = uniform_load(trow + last_idx);
    };
    auto issue = [&](int u) {         // loads of local tile u (prep(u) done)
        const int x = x0 + u;
        const int kb = ic.ksa + (x - ic.pre) * kKeys;
        uint8_t* stage = smem + (u % kStg) * (I8 ? S::kCodeStage : C::kStage);
        if ((x == ic.pre || u == 0) && S::kCompact) {   // first tile of a segment: its query rows first
            // into register set seg % kStg (lane (g, n): column n's 16-byte pieces g, 4 + g,
            // ...; columns past NC re-read the last one)
            const int c = min(n, NC - 1);
            const int ct = c / G;
            const int64_t qrow = ((int64_t)ic.b * qn + ct) * p.hq + kvh * G + (c - ct * G);
            const uint8_t* src = qbase + qrow * C::kRowBytes + 16 * g;
#pragma unroll
            for (int s = 0; s < C::kSteps; ++s) qnext[s] = ld16(src + 64 * s);
        } else if (x == ic.pre || u == 0) {
            // LDS row c of the slot is column c: query token c / G, head c % G of the kv
            // head (bytes past the NC rows re-read the last row).
            uint8_t* qdst = qring + (ic.seg % kStg) * S::kQSlot;
            for (int j = 0; j < nq; ++j) {
                const int byte = j * 1024 + 16 * lane;
                const int c = min(byte / C::kRowBytes, NC - 1);
                const int ct = c / G;
                const int64_t qrow = ((int64_t)ic.b * qn + ct) * p.hq + kvh * G + (c - ct * G);
                lds_dma16(qbase + qrow * C::kRowBytes + (byte & (C::kRowBytes - 1)), qdst + j * 1024);
            }
        }
        if constexpr (I8) {
            // Codes: wave load j of a half takes rows j kCodeRpi .. (one block: blocks hold
            // at least kCodeRpi keys; its entry is pe[2 j]).  Then one load of the scales:
            // lanes 0-7 the K scales of keys 4 i .. 4 i + 3, lanes 8-15 the V scales (a run
            // of 4 in the [block][kv head][offset] layout), the others re-read lane 0's.
            const int L = ic.L;
            const bool whole = x + 1 < ic.end;
            if (whole && p.bs_log2 >= 5) {
                // Blocks of at least 32 keys: the tile (keys from a multiple of 32) lies in
                // one block, so one row base serves every wave load and the 32 scales are
                // one run of the block's.
                const uint32_t blk = (uint32_t)min(max(pe[0], 0), last_block);
                const uint64_t row0 = ((uint64_t)blk << p.bs_log2) | (uint32_t)(kb & bs_mask);
                const uint8_t* kc = kcodes + row0 * crow_bytes;
                const uint8_t* vc = vcodes + row0 * crow_bytes;
#pragma unroll
                for (int j = 0; j < S::kCodeDmaHalf; ++j) {
                    const uint64_t off = (uint64_t)(j * S::kCodeRpi) * crow_bytes;
                    lds_dma16_s(kc + off, cvoff, stage + j * 1024);
                    lds_dma16_s(vc + off, cvoff, stage + S::kCodeHalf + j * 1024);
                }
                const int gi = lane < 16 ? (lane & 7) : 0;
                const int64_t sidx = ((((int64_t)blk * p.hkv + kvh) << p.bs_log2) | (kb & bs_mask)) + 4 * gi;
                const float* sc = (lane >= 8 && lane < 16) ? p.v_scale : p.k_scale;
                lds_dma16(sc + sidx, stage + 2 * S::kCodeHalf);
                return;
            }
            const int64_t last_slot = ((int64_t)min(max(pe_last, 0), last_block) << p.bs_log2) | ((L - 1) & bs_mask);
#pragma unroll
            for (int j = 0; j < S::kCodeDmaHalf; ++j) {
                const uint32_t blk = (uint32_t)min(max(pe[2 * j], 0), last_block);
                const int key0 = kb + j * S::kCodeRpi;
                if (whole) {
                    const uint64_t off = (uint64_t)(((uint64_t)blk << p.bs_log2) | (uint32_t)(key0 & bs_mask)) * crow_bytes;
                    lds_dma16_s(kcodes + off, cvoff, stage + j * 1024);
                    lds_dma16_s(vcodes + off, cvoff, stage + S::kCodeHalf + j * 1024);
                } else {              // rows past the end re-read the last key
                    const int key = key0 + crow;
                    const int64_t slot = key < L ? (((int64_t)blk << p.bs_log2) | (key & bs_mask)) : last_slot;
                    lds_dma16(kcodes + slot * crow_bytes + cchunk, stage + j * 1024);
                    lds_dma16(vcodes + slot * crow_bytes + cchunk, stage + S::kCodeHalf + j * 1024);
                }
            }
            {
                const int gi = lane < 16 ? (lane & 7) : 0;      // 4-key group of this lane
                // its block's entry pe[4 gi / kRpi], by a tree of selects on the index bits
                // (a chain of equality selects becomes a scratch-memory lookup)
                const int e_idx = (4 * gi) / C::kRpi;
                int32_t tv[C::kDmaHalf];
#pragma unroll
                for (int jj = 0; jj < C::kDmaHalf; ++jj) tv[jj] = pe[jj];
#pragma unroll
                for (int lv = 1; lv < C::kDmaHalf; lv <<= 1)
#pragma unroll
                    for (int jj = 0; jj + lv < C::kDmaHalf; jj += 2 * lv) tv[jj] = (e_idx & lv) ? tv[jj + lv] : tv[jj];
                const int32_t e = tv[0];
                const int key = kb + 4 * gi;
                const int64_t slot = key < L ? (((int64_t)min(max(e, 0), last_block) << p.bs_log2) | (key & bs_mask))
                                             : ((int64_t)min(max(pe_last, 0), last_block) << p.bs_log2) | (((L - 1) & ~3) & bs_mask);
                const int64_t sidx = (((slot >> p.bs_log2) * p.hkv + kvh) << p.bs_log2) | (slot & bs_mask);
                const float* sc = (lane >= 8 && lane < 16) ? p.v_scale : p.k_scale;
                lds_dma16(sc + sidx, stage + 2 * S::kCodeHalf);
            }
            return;
        }
        // full tile with no new key: SGPR base per wave load, constant lane offsets
        if (x + 1 < ic.end && !(APPEND && kb + kKeys > ic.new_key)) {
#pragma unroll
            for (int j = 0; j < C::kDmaHalf; ++j) {
                const uint32_t blk = (uint32_t)min(max(pe[j], 0), last_block);
                const uint64_t off = (uint64_t)(((uint64_t)blk << p.bs_log2) | (uint32_t)((kb + j * C::kRpi) & bs_mask)) * row_bytes;
                const uint32_t voff = (uint32_t)lrow * row_bytes + lchunk[j];
                lds_dma16_s(kbase + off, voff, stage + j * 1024);
                lds_dma16_s(vbase + off, voff, stage + C::kHalf + j * 1024);
            }
        } else {                      // last tile (or one with new keys): rows past the end re-read the last key
            const int L = ic.L;
            const int64_t last_slot = ((int64_t)min(max(pe_last, 0), last_block) << p.bs_log2) | ((L - 1) & bs_mask);
#pragma unroll
            for (int j = 0; j < C::kDmaHalf; ++j) {
                const int key = kb + j * C::kRpi + lrow;
                const int64_t slot = key < L ? (((int64_t)min(max(pe[j], 0), last_block) << p.bs_log2) | (key & bs_mask))
                                             : last_slot;
                const uint8_t* ks = kbase + slot * row_bytes + lchunk[j];
                const uint8_t* vs = vbase + slot * row_bytes + lchunk[j];
                if (APPEND && key >= ic.new_key) {   // new row b qn + (key - new_key), the last for keys past the end
                    const int64_t new_off = (((int64_t)ic.b * qn + (min(key, L - 1) - ic.new_key)) * p.hkv + kvh) * D * 2;
                    ks = reinterpret_cast<const uint8_t*>(p.k_new) + new_off + lchunk[j];
                    vs = reinterpret_cast<const uint8_t*>(p.v_new) + new_off + lchunk[j];
                }
                lds_dma16(ks, stage + j * 1024);
                lds_dma16(vs, stage + C::kHalf + j * 1024);
            }
        }
    };
    auto feed = [&](int u) {
        if (u >= ntw) return;
        issue(u);
        if (u + 1 < ntw) prep(u + 1);
    };
    prep(0);
#pragma unroll
    for (int u = 0; u < kStg - 1; ++u) feed(u);

    // INT8: the codes of tile t (this wave's own loads) into the bf16 tile, logical 16-byte
    // chunk c of row r at physical chunk swz(r, c) as the products read it; LDS accesses of
    // one wave complete in order, so the previous tile's reads of it are done first.
    // The bf16 tile the products read, and (INT8) the tile's K and V scales.
    auto tile_of = [&](int t) -> const uint8_t* {
        return I8 ? smem + S::kBufOff : smem + (t % kStg) * C::kStage;
    };
    // The tile whose V half the value product reads: INT8 converts V into the same buffer
    // as K, so its "stage" starts one half before the buffer (only its V half is read).
    auto vtile_of = [&](int t) -> const uint8_t* {
        return I8 ? smem + S::kBufOff - C::kHalf : smem + (t % kStg) * C::kStage;
    };
    auto kscale_of = [&](int t) -> const float* {
        return I8 ? reinterpret_cast<const float*>(smem + (t % kStg) * S::kCodeStage + 2 * S::kCodeHalf) : nullptr;
    };
    auto vscale_of = [&](int t) -> const float* {
        return I8 ? reinterpret_cast<const float*>(smem + (t % kStg) * S::kCodeStage + 2 * S::kCodeHalf) + kKeys
                  : nullptr;
    };
    // Half h (0: K, 1: V) of tile t's codes into the bf16 half-tile buffer; the V half
    // overwrites K after the scores have read it (same wave, LDS in order).
    auto convert = [&](int t, int h) {
        const uint8_t* cs = smem + (t % kStg) * S::kCodeStage + h * S::kCodeHalf;
        uint8_t* bf = smem + S::kBufOff;
        constexpr int kUnits = kKeys * D / 16 / 64;       // 16-code units per lane and half
        // All reads first: a store to the bf16 tile may alias a later read as far as the
        // compiler knows, so interleaved it would wait out each read's latency.
        u32x4 raw[kUnits];
#pragma unroll
        for (int i = 0; i < kUnits; ++i) raw[i] = *reinterpret_cast<const u32x4*>(cs + (lane + 64 * i) * 16);
#pragma unroll
        for (int i = 0; i < kUnits; ++i) {
            const int ui = lane + 64 * i;
            const int r = ui / (D / 16);
            const int u16 = ui % (D / 16);
            u32x4 lo, hi;
            codes_to_bf16(raw[i], lo, hi);
            uint8_t* row = bf + r * C::kRowBytes;
            *reinterpret_cast<u32x4*>(row + swz<C::kRowChunks, C::kRowShift>(r, 2 * u16) * 16) = lo;
            *reinterpret_cast<u32x4*>(row + swz<C::kRowChunks, C::kRowShift>(r, 2 * u16 + 1) * 16) = hi;
        }
    };

    // Consume side: one segment (the part of a sequence inside the range) at a time.
    Cursor cc = cursor_at(b0);
    int t = 0;
    while (t < ntw) {
        advance(cc, x0 + t);
        const int tend = min(cc.end, x1) - x0;         // local end of the segment
        const bool whole = cc.pre >= x0 && cc.end <= x1;
        const int slot = t == 0 ? 0 : 1;               // partial state: first or last segment
        wait_tile<S::kDma>(min(ntw - 1 - t, kStg - 2));
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        // This segment's query rows (Q^T fragments: k-step s covers dims 32 s .. 32 s + 31;
        // lane (g, n) holds 8 of them of head n, zero for columns past G).
        bf16x8_t qf[C::kSteps];
        if constexpr (S::kCompact) {
#pragma unroll
            for (int s = 0; s < C::kSteps; ++s)
                qf[s] = __builtin_bit_cast(bf16x8_t, valid ? qnext[s] : u32x4{0u, 0u, 0u, 0u});
        } else {
            const uint8_t* qs = qring + (cc.seg % kStg) * S::kQSlot + n * C::kRowBytes;
#pragma unroll
            for (int s = 0; s < C::kSteps; ++s) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(qs + (4 * s + g) * 16);
                qf[s] = __builtin_bit_cast(bf16x8_t, valid ? v : u32x4{0u, 0u, 0u, 0u});
            }
        }
        RowState st;
        f32x4 oacc[C::kDTiles];
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float sv[8];
        float tmax = 0.0f;
        bool full = false;
        // Tiles of the segment; a tile that raises some head's max by more than the slack
        // leaves the inner loop to rescale, so that inside it the accumulators are only
        // touched by products.
        while (t < tend) {
            for (; t < tend; ++t) {
                wait_tile<S::kDma>(min(ntw - 1 - t, kStg - 2));
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                feed(t + kStg - 1);
                if constexpr (I8) convert(t, 0);
                const int kb = cc.ksa + (x0 + t - cc.pre) * kKeys;
                // every column sees the whole tile: past the last token's window start and
                // before the first token's end
                full = kb >= cc.ks_last && kb + kKeys <= cc.L - (qn - 1);
                tmax = tile_scores<D>(tile_of(t), qf, n, g, full, kb,
                                      window_start(cc.L - back, p.window), cc.L - back,
                                      p.scale_log2, sv, kscale_of(t));
                if (__any(must_rescale(st, tmax))) break;
                if constexpr (I8) convert(t, 1);
                tile_pv<D>(vtile_of(t), st, full, sv, p.scale_log2, n, g, oacc, vscale_of(t));
            }
            if (t >= tend) break;
            rescale<D>(st, tmax, oacc);
            if constexpr (I8) convert(t, 1);
            tile_pv<D>(vtile_of(t), st, full, sv, p.scale_log2, n, g, oacc, vscale_of(t));
            ++t;
        }
        float l_tot = st.l + __shfl_xor(st.l, 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        if (valid) {
            if (whole) {
                store_final<D>(p, out_row(cc.b), g, st.m, l_tot, oacc);
            } else {
                const int64_t ps = ((int64_t)(kvh * P + w) * 2 + slot) * NC + n;
                float* o = p.ws_o + ps * D + 4 * g;
#pragma unroll
                for (int dt = 0; dt < C::kDTiles; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[dt];
                if (g == 0) {
                    p.ws_ml[ps * 2] = st.m;
                    p.ws_ml[ps * 2 + 1] = l_tot;
                }
            }
        }
    }
}

// Merge of the partial states of sequences that cross range ends: workgroup (b, kv head),
// parts from the non-empty ranges first .. last of that kv head (part of the first range:
// its last segment unless the sequence starts exactly at the range start; ranges are
// empty when there are fewer tiles than ranges).  The (m, l) of all parts are staged in
// LDS with one round of loads, then every o element is read once.
template <int D, int MAXP>
__global__ __launch_bounds__(256) void gqa_stream_combine_kernel(DecodeParams p) {
    __shared__ float s_w[16][MAXP];   // m, then the weight e^(m - M)
    __shared__ float s_l[16][MAXP];
    __shared__ float s_inv[16];
    const int b = blockIdx.x / p.hkv;
    const int kvh = blockIdx.x % p.hkv;
    const int T = p.tile_prefix[p.batch];
    const int pre = p.tile_prefix[b];
    const int end = p.tile_prefix[b + 1];
    if (end <= pre) return;
    const int P = p.parts;
    const int wf = range_of(pre, T, P);
    const int wl = range_of(end - 1, T, P);
    if (wf == wl) return;
    const int G = p.group;
    const int qn = max(p.qn, 1);
    const int NC = qn * G;            // columns: (query token, head) pairs
    const int np = wl - wf + 1;
    const int first_slot = range_start(wf, T, P) == pre ? 0 : 1;
    auto part = [&](int j, int n) {   // partial index of part j (range wf + j), column n
        return ((int64_t)(kvh * P + wf + j) * 2 + (j == 0 ? first_slot : 0)) * NC + n;
    };
    auto row_of = [&](int n) {        // output row of column n
        const int t = n / G;
        return ((int64_t)b * qn + t) * p.hq + kvh * G + (n - t * G);
    };
    for (int i = threadIdx.x; i < np * NC; i += blockDim.x) {
        const int j = i / NC, n = i % NC;
        const bool empty = range_start(wf + j, T, P) == range_start(wf + j + 1, T, P);
        const int64_t ps = part(j, n);
        s_w[n][j] = empty ? -INFINITY : p.ws_ml[ps * 2];
        s_l[n][j] = empty ? 0.0f : p.ws_ml[ps * 2 + 1];
    }
    __syncthreads();
    if (threadIdx.x < NC) {
        const int n = threadIdx.x;
        float M = -INFINITY;
        for (int j = 0; j < np; ++j) M = fmaxf(M, s_w[n][j]);
        float lsum = 0.0f;
        for (int j = 0; j < np; ++j) {
            const float f = s_w[n][j] == -INFINITY ? 0.0f : fast_exp2(s_w[n][j] - M);
            s_w[n][j] = f;
            lsum = fmaf(f, s_l[n][j], lsum);
        }
        s_inv[n] = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        const int64_t row = row_of(n);
        if (p.lse) p.lse[row] = lsum > 0.0f ? (M + __log2f(lsum)) * kLn2f : -INFINITY;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NC * (D / 4); i += blockDim.x) {
        const int n = i / (D / 4);
        const int d = (i % (D / 4)) * 4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int j = 0; j < np; ++j) {
            const float f = s_w[n][j];
            if (f == 0.0f) continue;
            const f32x4 o = *reinterpret_cast<const f32x4*>(p.ws_o + part(j, n) * D + d);
            acc += f * o;
        }
        const float inv = s_inv[n];
        const int64_t row = row_of(n);
        const uint32_t w0 = bf16_bits(acc[0] * inv) | ((uint32_t)bf16_bits(acc[1] * inv) << 16);
        const uint32_t w1 = bf16_bits(acc[2] * inv) | ((uint32_t)bf16_bits(acc[3] * inv) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.out) + row * D + d) = make_uint2(w0, w1);
    }
}

// ================================================================== per-split kernel
template <int D>
struct ItemCfg {
    using C = GqaCfg<D>;
    static constexpr int kSmem = kStages * C::kStage + 2 * kTabEntries * 4;
};

template <int D, bool APPEND>
__global__ __launch_bounds__(64) void gqa_decode_kernel(DecodeParams p) {
    using C = GqaCfg<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[ItemCfg<D>::kSmem];

    const int lane = threadIdx.x;
    const int n = lane & 15;          // head column of this lane; A-operand row
    const int g = lane >> 4;          // k-slot group

    // Work items (sequence, split), the longest sequences first; the kv head varies
    // fastest.  A sequence with no key is one item (it writes zeros).
    const int kvh = blockIdx.x % p.hkv;
    int b, split;
    {
        auto nsplits = [&](int, int len) {
            return len > 0 ? (len - window_start32(len, p.window) + p.split_tokens - 1) / p.split_tokens : 1;
        };
        if (!find_item<64>(blockIdx.x / p.hkv, p.batch, p.seq_lens, p.len_cap, nsplits,
                           reinterpret_cast<int32_t*>(smem + kStages * C::kStage), b, split))
            return;
        b = __builtin_amdgcn_readfirstlane(b);          // the same in every lane
        split = __builtin_amdgcn_readfirstlane(split);
    }
    const int G = p.group;
    const int L = min(p.seq_lens[b], p.len_cap);
    const bool valid = n < G;
    const int64_t row = (int64_t)b * p.hq + kvh * G + min(n, G - 1);
    if (L <= 0) {   // a padding row: output 0, lse -inf, nothing written
        if (valid) store_empty<D>(p, row, g);
        if (APPEND && p.slots_out && kvh == 0 && split == 0 && threadIdx.x == 0) p.slots_out[b] = -1;
        return;
    }
    const int ks = window_start(L, p.window);                         // first visible key
    const int ksa = ks & ~(kKeys - 1);
    const int k_begin = ksa + split * p.split_tokens;
    if (k_begin >= L) return;
    const int k_end = min(L, k_begin + p.split_tokens);
    const int ntiles = (k_end - k_begin + kKeys - 1) / kKeys;
    const int bs_mask = (1 << p.bs_log2) - 1;
    const int32_t* trow = p.table + (int64_t)b * p.mbs;
    const uint32_t row_bytes = (uint32_t)(p.hkv * D * 2);            // one cache slot
    const int64_t new_off = ((int64_t)b * p.hkv + kvh) * D * 2;      // this head's new rows

    const int new_key = new_key_of<APPEND>(p, b, L);                  // INT_MAX: none
    if (APPEND && L - 1 >= k_begin && L - 1 < k_end) append_row<D>(p, b, kvh, L, lane);

    // Q^T fragments: k-step s covers dims 32 s .. 32 s + 31; this lane holds 8 of them of
    // head n (zero for columns past G).
    bf16x8_t qf[C::kSteps];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
        const u32x4 v = ld16(reinterpret_cast<const uint8_t*>(p.q) + (row * D + 32 * s + 8 * g) * 2);
        qf[s] = __builtin_bit_cast(bf16x8_t, valid ? v : u32x4{0u, 0u, 0u, 0u});
    }

    TableChunks<64> tab;
    tab.lds = reinterpret_cast<int32_t*>(smem + kStages * C::kStage);
    tab.row = trow;
    tab.k_begin = k_begin;
    tab.k_end = k_end;
    tab.bs_log2 = p.bs_log2;
    tab.tid = lane;
    tab.last_block = (int32_t)(p.num_blocks - 1);
    int32_t treg[TableChunks<64>::kRegs];
    tab.load(0, treg);
    tab.store(0, treg);
    // Q and the first chunk must be resident before the loop: otherwise the wait for
    // them, placed inside the loop, would also wait for the tile loads issued there.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

    int lrow[C::kDmaHalf];
    uint32_t lchunk[C::kDmaHalf];
#pragma unroll
    for (int j = 0; j < C::kDmaHalf; ++j) {
        const int q = j * 64 + lane;
        lrow[j] = q / C::kRowChunks;
        lchunk[j] = (uint32_t)swz<C::kRowChunks, C::kRowShift>(lrow[j], q % C::kRowChunks) * 16u;
    }
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_cache) + kvh * D * 2;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_cache) + kvh * D * 2;
    // Full tiles inside one block (blocks of >= 32 keys) that do not hold this step's token:
    // one scalar read of the block table (one tile ahead), then an SGPR base per half.
    const bool fast_rows = p.bs_log2 >= 5;
    auto fast_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        return fast_rows && kb + kKeys <= k_end && !(APPEND && kb + kKeys > new_key);
    };
    auto entry_of = [&](int u) { return uniform_load(trow + ((k_begin + u * kKeys) >> p.bs_log2)); };
    int32_t next_entry = fast_tile(0) ? entry_of(0) : 0;
    auto issue_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        const int chunk = u / kChunkTiles;
        uint8_t* stage = smem + (u % kStages) * C::kStage;
        const int32_t entry = next_entry;
        if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
        if (fast_tile(u)) {
            const uint32_t blk = (uint32_t)min(max(entry, 0), tab.last_block);
            const uint64_t slot0 = ((uint64_t)blk << p.bs_log2) | (uint32_t)(kb & bs_mask);
#pragma unroll
            for (int j = 0; j < C::kDmaHalf; ++j) {
                const uint32_t voff = (uint32_t)lrow[j] * row_bytes + lchunk[j];
                lds_dma16_s(kbase + slot0 * row_bytes, voff, stage + j * 1024);
                lds_dma16_s(vbase + slot0 * row_bytes, voff, stage + C::kHalf + j * 1024);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < C::kDmaHalf; ++j) {
            const int key = min(kb + lrow[j], k_end - 1);
            const uint64_t slot = ((uint64_t)tab.block_of(key, chunk) << p.bs_log2) | (uint32_t)(key & bs_mask);
            const uint8_t* ks = kbase + slot * row_bytes + lchunk[j];
            const uint8_t* vs = vbase + slot * row_bytes + lchunk[j];
            if (APPEND && key == new_key) {
                ks = reinterpret_cast<const uint8_t*>(p.k_new) + new_off + lchunk[j];
                vs = reinterpret_cast<const uint8_t*>(p.v_new) + new_off + lchunk[j];
            }
            lds_dma16(ks, stage + j * 1024);
            lds_dma16(vs, stage + C::kHalf + j * 1024);
        }
    };

    RowState st;
    f32x4 oacc[C::kDTiles];
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Table chunks and the loads of tile u (issued kStages - 1 tiles ahead).  The reads of
    // the stage a load overwrites were consumed by earlier products, so they are done.
    auto feed = [&](int u) {
        if (u >= ntiles) return;
        const int c = u / kChunkTiles;
        if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load(c + 1, treg);
        if (u % kChunkTiles == kChunkTiles / 2 && tab.exists(c + 1)) tab.store(c + 1, treg);
        issue_tile(u);
    };
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u) feed(u);

    // Tile t: wait for its loads (this wave's own), issue tile t + 3, scores, then P and
    // O.  A tile that raises some head's max by more than the slack leaves the loop to
    // rescale O^T, so that inside the loop the accumulators are only touched by products.
    int t = 0;
    float sv[8];
    float tmax = 0.0f;
    bool full = false;
    while (t < ntiles) {
        for (; t < ntiles; ++t) {
            wait_tile<C::kDma>(min(ntiles - 1 - t, kStages - 2));
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            feed(t + kStages - 1);
            const int kb = k_begin + t * kKeys;
            full = kb >= ks && kb + kKeys <= k_end;
            tmax = tile_scores<D>(smem + (t % kStages) * C::kStage, qf, n, g, full, kb, ks, k_end, p.scale_log2,
                                  sv);
            if (__any(must_rescale(st, tmax))) break;
            tile_pv<D>(smem + (t % kStages) * C::kStage, st, full, sv, p.scale_log2, n, g, oacc);
        }
        if (t >= ntiles) break;
        rescale<D>(st, tmax, oacc);
        tile_pv<D>(smem + (t % kStages) * C::kStage, st, full, sv, p.scale_log2, n, g, oacc);
        ++t;
    }

    // ---------------------------------------------------------------- epilogue
    float l_tot = st.l + __shfl_xor(st.l, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!valid) return;
    const int nsplit = (L - ksa + p.split_tokens - 1) / p.split_tokens;
    if (nsplit == 1) {
        store_final<D>(p, row, g, st.m, l_tot, oacc);
    } else {
        const int64_t ps = row * p.max_splits + split;
        float* o = p.ws_o + ps * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[dt];
        if (g == 0) {
            p.ws_ml[ps * 2] = st.m;
            p.ws_ml[ps * 2 + 1] = l_tot;
        }
    }
}

}  // namespace

bool gqa_mfma_supported(int dtype, int group) { return dtype == 1 && group >= 4 && group <= 16; }

bool gqa_stream_supported(int dtype, int group, int head_dim, int bs_log2, int batch) {
    const int rpi_log2 = head_dim == 128 ? 2 : 3;    // every wave load within one block
    return gqa_mfma_supported(dtype, group) && bs_log2 >= rpi_log2 && batch <= kStreamMaxBatch;
}

bool gqa_stream_shape_supported(int head_dim, int bs_log2, int batch) {
    const int rpi_log2 = head_dim == 128 ? 2 : 3;
    return (head_dim == 64 || head_dim == 128) && bs_log2 >= rpi_log2 && batch <= kStreamMaxBatch;
}

int gqa_stream_parts(int num_kv_heads, bool compact, bool int8) {
    const int wgs = int8 ? kStreamWgsI8 : compact ? kStreamWgsCompact : kStreamWgs;
    // at most kStreamWgsCompact parts per kv head (the combine's bound)
    return num_kv_heads >= wgs ? 1 : min(wgs / num_kv_heads, kStreamWgsCompact);
}

hipError_t launch_gqa_decode_int8(const DecodeParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.hkv * p.parts));
    if (p.k_new) {
        if (head_dim == 64) hipLaunchKernelGGL((gqa_stream_kernel<64, true, true>), grid, dim3(64), 0, s, p);
        else hipLaunchKernelGGL((gqa_stream_kernel<128, true, true>), grid, dim3(64), 0, s, p);
    } else {
        if (head_dim == 64) hipLaunchKernelGGL((gqa_stream_kernel<64, false, true>), grid, dim3(64), 0, s, p);
        else hipLaunchKernelGGL((gqa_stream_kernel<128, false, true>), grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_gqa_decode(const DecodeParams& p, int head_dim, hipStream_t s) {
    if (p.parts > 0) {
        const dim3 grid((unsigned)((int64_t)p.hkv * p.parts));
        // the plan chose the compact layout when it planned more than kStreamWgs ranges
        const bool compact = (int64_t)p.hkv * p.parts > kStreamWgs;
        if (head_dim == 64) {
            if (compact) {
                if (p.k_new) hipLaunchKernelGGL((gqa_stream_kernel<64, true, false, true>), grid, dim3(64), 0, s, p);
                else hipLaunchKernelGGL((gqa_stream_kernel<64, false, false, true>), grid, dim3(64), 0, s, p);
            } else {
                if (p.k_new) hipLaunchKernelGGL((gqa_stream_kernel<64, true>), grid, dim3(64), 0, s, p);
                else hipLaunchKernelGGL((gqa_stream_kernel<64, false>), grid, dim3(64), 0, s, p);
            }
        } else {
            if (compact) {
                if (p.k_new) hipLaunchKernelGGL((gqa_stream_kernel<128, true, false, true>), grid, dim3(64), 0, s, p);
                else hipLaunchKernelGGL((gqa_stream_kernel<128, false, false, true>), grid, dim3(64), 0, s, p);
            } else {
                if (p.k_new) hipLaunchKernelGGL((gqa_stream_kernel<128, true>), grid, dim3(64), 0, s, p);
                else hipLaunchKernelGGL((gqa_stream_kernel<128, false>), grid, dim3(64), 0, s, p);
            }
        }
        return hipGetLastError();
    }
    const dim3 grid((unsigned)((int64_t)p.hkv * p.batch * p.max_splits));
    if (head_dim == 64) {
        if (p.k_new) hipLaunchKernelGGL((gqa_decode_kernel<64, true>), grid, dim3(64), 0, s, p);
        else hipLaunchKernelGGL((gqa_decode_kernel<64, false>), grid, dim3(64), 0, s, p);
    } else {
        if (p.k_new) hipLaunchKernelGGL((gqa_decode_kernel<128, true>), grid, dim3(64), 0, s, p);
        else hipLaunchKernelGGL((gqa_decode_kernel<128, false>), grid, dim3(64), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_gqa_stream_combine(const DecodeParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.batch * p.hkv));
    // at most kStreamWgs (compact layout: kStreamWgsCompact) parts per kv head
    if (p.parts <= kStreamWgs) {
        if (head_dim == 64) hipLaunchKernelGGL((gqa_stream_combine_kernel<64, kStreamWgs>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gqa_stream_combine_kernel<128, kStreamWgs>), grid, dim3(256), 0, s, p);
    } else {
        if (head_dim == 64) hipLaunchKernelGGL((gqa_stream_combine_kernel<64, kStreamWgsCompact>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((gqa_stream_combine_kernel<128, kStreamWgsCompact>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace pkv
