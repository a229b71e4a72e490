// Paged-attention decode for MHA/GQA on gfx950 ("KVCache Optimization Skill", Mode 2
// step 4 and 3.6; "Paged KV Cache and Packed Sequence", 3.3 and 4.2: the kernel walks
// each sequence's physical blocks through block_table).
//
// Decode reads every cached K/V byte once and does about one flop per byte, so the
// kernel is bound by HBM bandwidth.  Design:
//  * one workgroup (4 wave64s) per (kv head, sequence, split of split_tokens tokens), or
//    per pair of adjacent kv heads when each has one query head (MHA): the pair's rows of
//    a token are one contiguous piece of the cache row; the kv head (pair) varies fastest
//    in blockIdx, so workgroups in flight together read neighbouring head slices of the
//    same physical blocks;
//  * each workgroup computes all G = Hq / Hkv query heads of its kv head, so a K/V row
//    is read from HBM once however many query heads share it (GQA);
//  * a token's K (or V) row of one head is D * elem bytes, loaded as 16-byte
//    non-temporal vectors by LPT = D * elem / 16 lanes (2 LPT for a head pair); a wave
//    covers TPW = 64 / LPT tokens per load (half as many for a pair) and issues all K and
//    V loads of a 32-token step (16 for a pair) before using any;
//  * block-table entries of the next step are fetched one step ahead, one entry per
//    lane, and handed to the lanes that need them with a cross-lane shuffle, so address
//    translation never waits on memory; any power-of-two block size works;
//  * rows of the wave keep their own online-softmax state (max, sum, output), merged
//    across rows with shuffles and across waves in LDS at the end;
//  * tokens past the sequence length are never loaded (masked by selection), so stale
//    or NaN rows in a block's tail cannot leak into the sum.
// A second kernel merges the splits of each (sequence, head) with the log-sum-exp rule.
// (Merging in the same launch, by the last workgroup to arrive, needs a device-scope
// release/acquire per workgroup; on gfx950 that write-back of the L2 made the decode
// about ten times slower than the extra launch.)
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kWaves = 4;
constexpr int kStepTokens = 32;   // tokens a wave loads per step

template <typename T> struct ElemBytes;
template <> struct ElemBytes<float> { static constexpr int v = 4; };
template <> struct ElemBytes<bf16_t> { static constexpr int v = 2; };

// HP adjacent kv heads share a workgroup (HP = 2 only with one query head per kv head): a
// token's HP head rows are contiguous in the cache, so a load covers HP * D * elem bytes of
// it; steps shrink to kStepTokens / HP tokens to keep the loads in flight per lane the same.
template <typename T, int D, int HP>
struct Shape {
    static constexpr int kEpl = 16 / ElemBytes<T>::v;  // elements per lane per load
    static constexpr int kLpt = D / kEpl;              // lanes per head row
    static constexpr int kLpr = kLpt * HP;             // lanes per token (HP head rows)
    static constexpr int kTpw = kWave / kLpr;          // tokens per wave load
    static constexpr int kStep = kStepTokens / HP;     // tokens per step
    static constexpr int kNj = kStep / kTpw;           // loads per step (each of K, V)
    static_assert(kLpr >= 1 && kLpr <= 64 && kTpw * kLpr == kWave && kNj >= 1, "bad shape");
};

// q . k over the lane's EPL elements (fp32 accumulate).
template <typename T>
__device__ __forceinline__ float lane_dot(const u32x4& q, const u32x4& k);
template <>
__device__ __forceinline__ float lane_dot<bf16_t>(const u32x4& q, const u32x4& k) {
    float a = dot2_bf16(q[0], k[0], 0.0f);
    a = dot2_bf16(q[1], k[1], a);
    a = dot2_bf16(q[2], k[2], a);
    return dot2_bf16(q[3], k[3], a);
}
template <>
__device__ __forceinline__ float lane_dot<float>(const u32x4& q, const u32x4& k) {
    float a = __uint_as_float(q[0]) * __uint_as_float(k[0]);
    a = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), a);
    a = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), a);
    return fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), a);
}

// Widen a 16-byte vector to EPL floats.
template <typename T>
__device__ __forceinline__ void widen(const u32x4& v, float* f);
template <>
__device__ __forceinline__ void widen<bf16_t>(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[2 * i] = bf16_lo(v[i]); f[2 * i + 1] = bf16_hi(v[i]); }
}
template <>
__device__ __forceinline__ void widen<float>(const u32x4& v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<bf16_t>(void* out, int64_t idx, float v) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16(v);
}
template <>
__device__ __forceinline__ void store_out<float>(void* out, int64_t idx, float v) {
    reinterpret_cast<float*>(out)[idx] = v;
}

template <typename T, int D, int GP, bool APPEND, int HP>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    static_assert(HP == 1 || GP == 1, "head pairs only with one query head per kv head");
    using S = Shape<T, D, HP>;
    constexpr int EPL = S::kEpl, LPT = S::kLpt, LPR = S::kLpr, TPW = S::kTpw, NJ = S::kNj;
    constexpr int STEP = S::kStep;
    constexpr int EB = ElemBytes<T>::v;
    __shared__ float sm_m[kWaves][GP * HP];
    __shared__ float sm_l[kWaves][GP * HP];
    __shared__ float sm_o[kWaves][GP * HP][D];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int row = lane / LPR;
    const int hs = (lane / LPT) % HP;   // which head of the workgroup's HP
    const int col = lane % LPT;

    int id = blockIdx.x;
    const int kvp = id % (p.hkv / HP);
    const int kvh = kvp * HP + hs;
    id /= p.hkv / HP;
    const int b = id % p.batch;
    const int split = id / p.batch;
    const int L = min(p.seq_lens[b], p.len_cap);
    // Keys [ks, L) are visible (a sliding window moves ks up); the splits start at ks
    // rounded down to a step, and the keys below ks in the first one are not loaded.
    const int ks = window_start(L, p.window);
    const int ksa = ks & ~(kStepTokens - 1);
    const int t0 = ksa + split * p.split_tokens;
    if (L <= 0) {   // no visible key (a padding row): output 0, lse -inf, nothing written
        if (split == 0) {
            if (APPEND && p.slots_out && kvp == 0 && threadIdx.x == 0) p.slots_out[b] = -1;
            for (int i = threadIdx.x; i < HP * p.group * D; i += blockDim.x) {
                const int h = kvp * HP * p.group + i / D;
                store_out<T>(p.out, ((int64_t)b * p.hq + h) * D + i % D, 0.0f);
                if (p.lse && i % D == 0) p.lse[(int64_t)b * p.hq + h] = -INFINITY;
            }
        }
        return;
    }
    if (t0 >= L) return;
    const int t1 = min(L, t0 + p.split_tokens);
    const int nsplit = (L - ksa + p.split_tokens - 1) / p.split_tokens;
    const int per_wave = p.split_tokens / kWaves;
    const int w0 = t0 + wave * per_wave;
    const int w1 = min(t1, w0 + per_wave);
    const int bs_mask = (1 << p.bs_log2) - 1;
    const int32_t last_block = (int32_t)(p.num_blocks - 1);
    const int32_t* trow = p.table + (int64_t)b * p.mbs;

    // Append mode: this step's token sits at L - 1; its K/V come from the new rows.  A row
    // longer than the length bound (a broken precondition) appends nothing: its slot is
    // reported as -1 and it attends to its first len_cap cached keys, as without append.
    const bool app = APPEND && p.seq_lens[b] <= p.len_cap;
    const int pos_new = app ? L - 1 : -1;
    const int64_t new_off = ((int64_t)b * p.hkv + kvh) * D * EB;
    if (APPEND && !app && split == 0 && p.slots_out && kvp == 0 && threadIdx.x == 0)
        p.slots_out[b] = -1;
    if (app && pos_new >= t0 && pos_new < t1) {
        int32_t phys = trow[pos_new >> p.bs_log2];
        phys = min(max(phys, 0), last_block);
        const int64_t slot = ((int64_t)phys << p.bs_log2) | (pos_new & bs_mask);
        // the HP head rows of the workgroup are contiguous in both the new rows and the cache
        const int64_t src0 = ((int64_t)b * p.hkv + kvp * HP) * D * EB;
        const int64_t dst = (slot * p.hkv + kvp * HP) * D * EB;
        constexpr int kChunks = HP * D * EB / 16;
        const int i = threadIdx.x;
        if (i < 2 * kChunks) {
            const int which = i / kChunks;
            const int64_t off = (int64_t)(i % kChunks) * 16;
            const uint8_t* src = reinterpret_cast<const uint8_t*>(which ? p.v_new : p.k_new) + src0;
            uint8_t* dstp = reinterpret_cast<uint8_t*>(which ? p.v_cache_w : p.k_cache_w) + dst;
            st16(dstp + off, ld16(src + off));
        }
        if (p.slots_out && kvp == 0 && threadIdx.x == 0) p.slots_out[b] = slot;
    }

    // Queries of the group (padded heads repeat the last real one and are not stored).
    u32x4 qv[GP];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const int h = kvh * p.group + min(g, p.group - 1);
        const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) +
                            (((int64_t)b * p.hq + h) * D + col * EPL) * EB;
        qv[g] = ld16(qp);
    }
    float m[GP], l[GP], o[GP][EPL];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
    }

    const int64_t slot_stride = (int64_t)p.hkv * D * EB;      // bytes per cache row
    const int64_t head_off = ((int64_t)kvh * D + col * EPL) * EB;
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_cache) + head_off;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_cache) + head_off;
    const uint8_t* knew =
        APPEND ? reinterpret_cast<const uint8_t*>(p.k_new) + new_off + col * EPL * EB : nullptr;
    const uint8_t* vnew =
        APPEND ? reinterpret_cast<const uint8_t*>(p.v_new) + new_off + col * EPL * EB : nullptr;

    // Table entries of the blocks a step touches: lane i holds entry (first block + i).
    // Steps start at multiples of 32 tokens, so a step spans at most 32 blocks.
    auto load_table = [&](int base) -> int32_t {
        const int blk0 = base >> p.bs_log2;
        const int nblk = ((min(base + STEP, w1) - 1) >> p.bs_log2) - blk0 + 1;
        return (base < w1 && lane < nblk) ? trow[blk0 + lane] : 0;
    };

    int32_t tbl = load_table(w0);
    for (int base = w0; base < w1; base += STEP) {
        const int32_t tbl_next = load_table(base + STEP);
        const int blk0 = base >> p.bs_log2;
        u32x4 kr[NJ], vr[NJ];
        bool valid[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int tok = base + j * TPW + row;
            valid[j] = tok >= ks && tok < w1;
            int32_t phys = __shfl(tbl, (tok >> p.bs_log2) - blk0, 64);
            phys = min(max(phys, 0), last_block);
            const int64_t slot = ((int64_t)phys << p.bs_log2) | (tok & bs_mask);
            kr[j] = u32x4{0u, 0u, 0u, 0u};
            vr[j] = u32x4{0u, 0u, 0u, 0u};
            if (valid[j]) {
                const uint8_t* kp = kbase + slot * slot_stride;
                const uint8_t* vp = vbase + slot * slot_stride;
                if (APPEND && tok == pos_new) {
                    kp = knew;
                    vp = vnew;
                }
                kr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp));
                vr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp));
            }
        }
        float vf[NJ][EPL];
#pragma unroll
        for (int j = 0; j < NJ; ++j) widen<T>(vr[j], vf[j]);

#pragma unroll
        for (int g = 0; g < GP; ++g) {
            if (g >= p.group) break;
            float s[NJ];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float dotp = group_sum<LPT>(lane_dot<T>(qv[g], kr[j]));
                s[j] = valid[j] ? dotp * p.scale_log2 : -INFINITY;
                mx = fmaxf(mx, s[j]);
            }
            const float mnew = fmaxf(m[g], mx);
            if (mnew != -INFINITY) {
                const float alpha = fast_exp2(m[g] - mnew);
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) o[g][e] *= alpha;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float pj = fast_exp2(s[j] - mnew);
                    l[g] += pj;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pj, vf[j][e], o[g][e]);
                }
                m[g] = mnew;
            }
        }
        tbl = tbl_next;
    }

    // Merge the rows of this wave, then the waves of the workgroup.
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        if (g >= p.group) break;
        const float mw = cross_row_max<LPR>(m[g]);
        const float f = (m[g] == -INFINITY) ? 0.0f : fast_exp2(m[g] - mw);
        const float lw = cross_row_sum<LPR>(l[g] * f);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = cross_row_sum<LPR>(o[g][e] * f);
        if (row == 0) {
            const int gi = g * HP + hs;
#pragma unroll
            for (int e = 0; e < EPL; ++e) sm_o[wave][gi][col * EPL + e] = o[g][e];
            if (col == 0) {
                sm_m[wave][gi] = mw;
                sm_l[wave][gi] = lw;
            }
        }
    }
    __syncthreads();

    for (int i = threadIdx.x; i < HP * p.group * D; i += blockDim.x) {
        const int gi = i / D;   // g * HP + head of the pair
        const int d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][gi]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (sm_m[w][gi] == -INFINITY) ? 0.0f : fast_exp2(sm_m[w][gi] - M);
            acc = fmaf(f, sm_o[w][gi][d], acc);
            lsum = fmaf(f, sm_l[w][gi], lsum);
        }
        const int h = (kvp * HP + gi % HP) * p.group + gi / HP;
        const int64_t bh = (int64_t)b * p.hq + h;
        if (nsplit == 1) {
            store_out<T>(p.out, bh * D + d, acc / lsum);
            if (p.lse && d == 0) p.lse[bh] = (M + __log2f(lsum)) * kLn2;
        } else {
            const int64_t ps = bh * p.max_splits + split;
            p.ws_o[ps * D + d] = acc;
            if (d == 0) {
                p.ws_ml[ps * 2] = M;
                p.ws_ml[ps * 2 + 1] = lsum;
            }
        }
    }
}

// Four output values of one row: bf16 (one 8-byte store) or fp32 (one 16-byte store).
__device__ __forceinline__ void store_out4(bf16_t* out, int64_t idx, float a, float b, float c, float d) {
    const uint32_t w0 = f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
    const uint32_t w1 = f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
    *reinterpret_cast<uint2*>(out + idx) = make_uint2(w0, w1);
}
__device__ __forceinline__ void store_out4(float* out, int64_t idx, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(out + idx) = make_float4(a, b, c, d);
}

// dim / 4 threads per (sequence, query head) row, 256 / (dim / 4) rows per workgroup.  Each
// thread folds the row's split (m, l) pairs itself (the same few values for the whole row:
// one cache line, no barrier) and merges its four value columns, the split partials read
// with 16-byte loads.
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    const int tpr = p.dim / 4;
    const int64_t bh = (int64_t)blockIdx.x * (blockDim.x / tpr) + threadIdx.x / tpr;
    if (bh >= (int64_t)p.batch * p.hq) return;
    const int d = 4 * (threadIdx.x % tpr);
    const int b = (int)(bh / p.hq);
    const int L = min(p.seq_lens[b], p.len_cap);
    const int ns = L > 0 ? (L - window_start32(L, p.window) + p.split_tokens - 1) / p.split_tokens : 0;
    if (ns <= 1) return;   // the split kernel wrote this row directly
    const float* ml = p.ws_ml + bh * p.max_splits * 2;
    const float* o = p.ws_o + bh * p.max_splits * p.dim + d;
    // One pass, the running max rescaling what is merged so far: a split's (m, l) and its
    // values are read together, with no wait for the other splits' maxima first.  (Every
    // split here has at least one key; a max of -inf would still weigh 0, not NaN.)
    float M = -INFINITY;
    float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float lsum = 0.0f;
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
        const float ms = ml[2 * s], ls = ml[2 * s + 1];
        const float4 v = *reinterpret_cast<const float4*>(o + (int64_t)s * p.dim);
        const float mn = fmaxf(M, ms);
        const float a = M == -INFINITY ? 0.0f : fast_exp2(M - mn);
        const float w = ms == -INFINITY ? 0.0f : fast_exp2(ms - mn);
        M = mn;
        lsum = fmaf(w, ls, lsum * a);
        acc.x = fmaf(w, v.x, acc.x * a);
        acc.y = fmaf(w, v.y, acc.y * a);
        acc.z = fmaf(w, v.z, acc.z * a);
        acc.w = fmaf(w, v.w, acc.w * a);
    }
    const float inv = 1.0f / lsum;
    store_out4(reinterpret_cast<T*>(p.out), bh * p.dim + d, acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (p.lse && d == 0) p.lse[bh] = (M + __log2f(lsum)) * kLn2;
}

template <typename T, int D, bool APPEND>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t s) {
    const int G = p.group;
    const int gp = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : G <= 8 ? 8 : 16;
    // One query head per kv head and an even number of kv heads: two adjacent heads per
    // workgroup (512-byte bf16 row pieces; the same bytes read ~4 % faster than in 256-byte
    // pieces on the Llama-7B-shaped decode).
    const bool pairs = gp == 1 && p.hkv % 2 == 0 && Shape<T, D, 2>::kLpr <= kWave;
    const dim3 grid((unsigned)((int64_t)(pairs ? p.hkv / 2 : p.hkv) * p.batch * p.max_splits));
    if (pairs) {
        hipLaunchKernelGGL((decode_split_kernel<T, D, 1, APPEND, 2>), grid, dim3(256), 0, s, p);
        return hipGetLastError();
    }
    switch (gp) {
        case 1: hipLaunchKernelGGL((decode_split_kernel<T, D, 1, APPEND, 1>), grid, dim3(256), 0, s, p); break;
        case 2: hipLaunchKernelGGL((decode_split_kernel<T, D, 2, APPEND, 1>), grid, dim3(256), 0, s, p); break;
        case 4: hipLaunchKernelGGL((decode_split_kernel<T, D, 4, APPEND, 1>), grid, dim3(256), 0, s, p); break;
        case 8: hipLaunchKernelGGL((decode_split_kernel<T, D, 8, APPEND, 1>), grid, dim3(256), 0, s, p); break;
        default: hipLaunchKernelGGL((decode_split_kernel<T, D, 16, APPEND, 1>), grid, dim3(256), 0, s, p); break;
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeParams& p, hipStream_t s) {
    return p.k_new ? launch_decode_t<T, D, true>(p, s) : launch_decode_t<T, D, false>(p, s);
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

DecodePlan plan_decode(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim_v, int32_t max_seq_len_kv, bool byte_rows, int32_t qn) {
    DecodePlan pl{};
    const int G = num_q_heads / num_kv_heads;
    // Larger groups carry more partial state per split: use longer splits for them.  Over
    // one-byte INT8 rows: 256 keys when a workgroup reads a pair of kv heads' contiguous rows
    // (one query head per kv head), else twice the bf16 split (the same bytes per workgroup).
    int split = G <= 2 ? 256 : G <= 4 ? 512 : 1024;
    if (byte_rows) split = int8_head_group(G, num_kv_heads) > 1 ? 256 : split * 2;
    const int64_t pairs = (int64_t)batch * num_kv_heads;
    auto nsplits = [&](int sp) { return (int64_t)(max_seq_len_kv + sp - 1) / sp; };
    // Keep at least ~4 workgroups per compute unit in flight on long sequences.
    while (split > kWaves * kStepTokens && pairs * nsplits(split) < 1024) split /= 2;
    pl.split_tokens = split;
    pl.max_splits = (int32_t)(max_seq_len_kv > 0 ? nsplits(split) : 1);
    if (pl.max_splits > 1) {
        const size_t rows = (size_t)batch * num_q_heads * pl.max_splits;
        pl.ws_o_offset = 0;
        pl.ws_ml_offset = align256(rows * head_dim_v * sizeof(float));
        pl.ws_bytes = pl.ws_ml_offset + rows * 2 * sizeof(float);
    }
    if (gqa_mfma_supported(1, G) || qn > 0) {   // the range-streaming layout, if that kernel runs
        const bool compact = byte_rows ? G > 4 : max_seq_len_kv >= kStreamCompactMinKeys;
        pl.parts = gqa_stream_parts(num_kv_heads, compact, byte_rows);
        const size_t parts = (size_t)num_kv_heads * pl.parts * 2 * G * (qn > 0 ? qn : 1);
        pl.st_o_offset = 0;
        pl.st_ml_offset = align256(parts * head_dim_v * sizeof(float));
        pl.st_pre_offset = align256(pl.st_ml_offset + parts * 2 * sizeof(float));
        const size_t st_bytes = pl.st_pre_offset + ((size_t)batch + 1) * sizeof(int32_t);
        if (st_bytes > pl.ws_bytes) pl.ws_bytes = st_bytes;
    }
    return pl;
}

hipError_t launch_decode(const DecodeParams& p, int dtype, int head_dim, hipStream_t s) {
    if (gqa_mfma_supported(dtype, p.group)) return launch_gqa_decode(p, head_dim, s);
    if (dtype == 1) {
        return head_dim == 64 ? launch_decode_d<bf16_t, 64>(p, s) : launch_decode_d<bf16_t, 128>(p, s);
    }
    return head_dim == 64 ? launch_decode_d<float, 64>(p, s) : launch_decode_d<float, 128>(p, s);
}

hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t s) {
    // four value columns per thread; the head dims (64, 128, 512) divide 1024, so whole rows
    // fill a workgroup of 256 threads
    if (p.dim % 4 || 1024 % p.dim) return hipErrorInvalidValue;
    const int rows_per_wg = 1024 / p.dim;
    const int64_t rows = (int64_t)p.batch * p.hq;
    const dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
    if (dtype == 1) hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
