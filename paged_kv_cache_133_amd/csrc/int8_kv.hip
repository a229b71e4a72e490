// INT8 KV cache: the quantizing write and the decode that reads it.  The pages name the
// knobs of a quantized cache (antiquant_scale, dequant_scale_key/value: "KVCache
// Optimization Skill", Layer 3 notes; the ai6s.net article on low-precision caches) but
// not the scheme.  The one taken: symmetric int8 codes with one fp32 scale per (token, kv
// head) row, s = max|x| / 127 and q = round_half_even(x / s) (IEEE fp32 divisions; a zero
// row has s = 0 and zero codes).  The caches hold the codes [nb][bs][Hkv][D] int8 and the
// scales [nb][Hkv][bs] fp32 (a block's scales of one head side by side), one pair for K
// and one for V.
//
// Decode is bound by HBM bytes, and int8 rows are half the bf16 bytes (plus 4 bytes of
// scale per row): the same split-KV schedule as decode_split_kernel on the vector ALU.
//  * a token's row of one head is D bytes, 16 codes per lane and 16-byte load: D / 16
//    lanes per row, 64 / (D / 16) tokens per wave load;
//  * K codes go to bf16 pairs (exact for |q| <= 127) for v_dot2_f32_bf16 against the bf16
//    query; the row's K scale multiplies the finished dot product;
//  * V codes are widened once per token and shared by the group's heads; the row's V scale
//    is folded into the softmax weight: o += (p s_v) q_v, l += p;
//  * each row of lanes takes NJ consecutive tokens of a step, so with blocks of at least NJ
//    tokens their K (V) scales are NJ adjacent floats of one block and head: one load per
//    row, issued with the code loads (scales laid out per (token, head) cost a sixth of
//    the kernel's time: every token's scale was a separate access);
//  * with one query head per kv head a workgroup takes a pair of adjacent kv heads, whose
//    rows of a token are one contiguous piece, over splits of 256 keys; otherwise splits
//    are twice as long as for bf16 rows, for the same bytes per workgroup.
// Keys below the window start are not loaded; the new token is written beforehand by the
// quantizing write (the attention reads the same codes later steps will).
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

constexpr float kLn2i8 = 0.69314718055994530942f;
constexpr int kWavesI8 = 4;
constexpr int kStepTokensI8 = 32;

// Signed byte k of a dword as float.
__device__ __forceinline__ float sbyte(uint32_t w, int k) { return (float)(int)(int8_t)(w >> (8 * k)); }
// Two floats as a bf16 pair (exact for the codes, |q| <= 127).
__device__ __forceinline__ uint32_t pack_bf16_pair(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// ------------------------------------------------------------------ quantizing write
// One group of D / 8 lanes per (token, kv head) row: 8 values per lane.  blockIdx.y picks K
// or V.  Rows whose slot lies outside the pool are skipped.
template <typename T, int D>
__global__ __launch_bounds__(256) void kv_write_int8_kernel(QuantWriteParams p) {
    constexpr int kLpr = D / 8;                       // lanes per row
    constexpr int kRpw = 64 / kLpr;                   // rows per wave
    const int which = p.which_base + blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kRpw + lane / kLpr;
    const int c = lane % kLpr;
    const int64_t rows = p.num_tokens * p.hkv;
    const bool live = row < rows;
    const int64_t t = live ? row / p.hkv : 0;
    const int h = live ? (int)(row % p.hkv) : 0;
    const int64_t slot = live ? p.slots[t] : -1;
    float x[8];
    float amax = 0.0f;
    if (live) {
        const uint8_t* src = reinterpret_cast<const uint8_t*>(which ? p.v_new : p.k_new) +
                             (row * D + c * 8) * (int64_t)sizeof(T);
        if constexpr (sizeof(T) == 2) {
            const u32x4 v = ld16(src);
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(v[i]); x[2 * i + 1] = bf16_hi(v[i]); }
        } else {
            const u32x4 a = ld16(src), b = ld16(src + 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) { x[i] = __uint_as_float(a[i]); x[4 + i] = __uint_as_float(b[i]); }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
    }
#pragma unroll
    for (int s = 1; s < kLpr; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s, 64));
    if (!live || slot < 0 || slot >= p.num_slots) return;
    const int64_t sc_idx = (((slot >> p.bs_log2) * p.hkv + h) << p.bs_log2) | (slot & ((1 << p.bs_log2) - 1));
    const float sc = __fdiv_rn(amax, 127.0f);
    uint32_t w[2] = {0u, 0u};
    if (sc > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float qf = fminf(fmaxf(rintf(__fdiv_rn(x[i], sc)), -127.0f), 127.0f);
            w[i >> 2] |= ((uint32_t)(int)qf & 0xffu) << (8 * (i & 3));
        }
    }
    uint8_t* dst = reinterpret_cast<uint8_t*>(which ? p.v_cache : p.k_cache) + (slot * p.hkv + h) * D + c * 8;
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    if (c == 0) (which ? p.v_scale : p.k_scale)[sc_idx] = sc;
}

// ------------------------------------------------------------------ int8 decode
// Register budget: one query head per kv head fits 128 VGPRs (4 waves per SIMD, 77 -> 74 us
// on the Llama-7B INT8 step); four fit 256 without accumulation registers (2 waves).
// APPEND (the write folded into the pass, as in decode_split_kernel): the token at
// seq_lens[b] - 1 comes from the bf16 rows k_new / v_new [B][Hkv][D]; the wave whose keys
// hold it quantizes it as the writer does (the same operations, so the same codes and scale
// bit for bit) and stores the codes and scales at its slot (reported in slots_out) before
// its loop, which then reads it back like any cached token.  A row longer than the length
// bound writes nothing (slot -1) and attends to its first len_cap cached keys.
// HP adjacent kv heads per workgroup (HP > 1 only with one query head per kv head): a
// token's HP head rows are one contiguous piece of HP * D bytes, read by HP * D / 16 lanes;
// each row of lanes still takes NJ consecutive tokens, so a step is kStepTokensI8 / HP
// tokens and the loads in flight per lane stay the same.
template <int D, int GP, bool APPEND, int HP>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(GP == 1 ? 4 : 2)))
void decode_int8_kernel(DecodeParams p) {
    static_assert(HP == 1 || GP == 1, "head groups only with one query head per kv head");
    constexpr int EPL = 16;                           // codes per lane per load
    constexpr int LPT = D / EPL;                      // lanes per head row
    constexpr int LPR = LPT * HP;                     // lanes per token (HP head rows)
    constexpr int NJ = kStepTokensI8 / (64 / LPT);    // loads per step (each of K, V)
    constexpr int STEP = kStepTokensI8 / HP;          // tokens per step
    static_assert(NJ == 2 || NJ == 4, "a row of lanes takes 2 or 4 tokens per step");
    static_assert(LPR <= 64 && (64 / LPR) * NJ == STEP, "bad head grouping");
    __shared__ float sm_m[kWavesI8][GP * HP];
    __shared__ float sm_l[kWavesI8][GP * HP];
    __shared__ float sm_o[kWavesI8][GP * HP][D];

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
    const int ks = window_start(L, p.window);
    const int ksa = ks & ~(kStepTokensI8 - 1);
    // The sequence's nsplit splits (the count the merge uses) share its steps evenly, in whole
    // steps per wave, unless that could leave the last split empty.
    int split_keys = p.split_tokens;
    {
        const int steps = (L - ksa + kStepTokensI8 - 1) / kStepTokensI8;
        const int ns = max((L - ksa + p.split_tokens - 1) / p.split_tokens, 1);
        const int per_wave_steps = ((steps + ns - 1) / ns + kWavesI8 - 1) / kWavesI8;
        const int even = per_wave_steps * kWavesI8 * kStepTokensI8;
        if (even > 0 && (int64_t)(ns - 1) * even < L - ksa) split_keys = even;
    }
    const int t0 = ksa + split * split_keys;
    const bool app = APPEND && p.seq_lens[b] <= p.len_cap;
    const int pos_new = app ? L - 1 : -1;
    if (APPEND && !app && split == 0 && p.slots_out && kvp == 0 && threadIdx.x == 0)
        p.slots_out[b] = -1;
    if (L <= 0) {   // no visible key: output 0, lse -inf
        if (split == 0) {
            for (int i = threadIdx.x; i < HP * p.group * D; i += blockDim.x) {
                const int h = kvp * HP * p.group + i / D;
                reinterpret_cast<uint16_t*>(p.out)[((int64_t)b * p.hq + h) * D + i % D] = 0;
                if (p.lse && i % D == 0) p.lse[(int64_t)b * p.hq + h] = -INFINITY;
            }
        }
        return;
    }
    if (t0 >= L) return;
    const int t1 = min(L, t0 + split_keys);
    const int nsplit = (L - ksa + p.split_tokens - 1) / p.split_tokens;
    const int per_wave = split_keys / kWavesI8;
    const int w0 = t0 + wave * per_wave;
    const int w1 = min(t1, w0 + per_wave);
    const int bs_mask = (1 << p.bs_log2) - 1;
    const int32_t last_block = (int32_t)(p.num_blocks - 1);
    const int32_t* trow = p.table + (int64_t)b * p.mbs;

    // Queries of the group (bf16; padded heads repeat the last real one, not stored): the
    // lane's 16 elements as 8 bf16 pairs.
    uint32_t qv[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        const int h = kvh * p.group + min(g, p.group - 1);
        const uint8_t* qp = reinterpret_cast<const uint8_t*>(p.q) + (((int64_t)b * p.hq + h) * D + col * EPL) * 2;
        const u32x4 a = ld16(qp), c = ld16(qp + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) { qv[g][i] = a[i]; qv[g][4 + i] = c[i]; }
    }
    float m[GP], l[GP], o[GP][EPL];
#pragma unroll
    for (int g = 0; g < GP; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = 0.0f;
    }

    const int64_t slot_stride = (int64_t)p.hkv * D;               // bytes per cache row
    const int64_t head_off = (int64_t)kvh * D + col * EPL;
    // Append: the wave whose keys hold the new token quantizes its K and V rows (two values
    // per lane; the HP heads' rows one after another), stores the codes and scales at its
    // slot and waits for those stores; its loop then reads the token back like any cached
    // one.  No other wave touches that token.
    if (APPEND && pos_new >= w0 && pos_new < w1) {
        const int32_t phys = min(max(trow[pos_new >> p.bs_log2], 0), last_block);
        const int64_t slot = ((int64_t)phys << p.bs_log2) | (pos_new & bs_mask);
#pragma unroll
        for (int hh = 0; hh < HP; ++hh) {
        const int kvw = kvp * HP + hh;   // the head whose row is written
        const int64_t sc_idx = (((int64_t)phys * p.hkv + kvw) << p.bs_log2) | (pos_new & bs_mask);
        const int64_t src_off = (((int64_t)b * p.hkv + kvw) * D + 2 * (lane % (D / 2))) * 2;
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
                               slot * slot_stride + (int64_t)kvw * D + 2 * lane;
                *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w;
                if (lane == 0) (which ? p.v_scale_w : p.k_scale_w)[sc_idx] = sc;
            }
        }
        }
        if (p.slots_out && kvp == 0 && lane == 0) p.slots_out[b] = slot;
        __threadfence_block();   // the stores complete before this wave's loads of the token
    }
    const uint8_t* kbase = reinterpret_cast<const uint8_t*>(p.k_cache) + head_off;
    const uint8_t* vbase = reinterpret_cast<const uint8_t*>(p.v_cache) + head_off;

    // Table entries of the blocks a step touches: lane i holds entry (first block + i).
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
        float ksc[NJ], vsc[NJ];
        bool valid[NJ];
        int64_t sbase[NJ];            // scale index of each token: ((block, head), offset)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int tok = base + row * NJ + j;
            valid[j] = tok >= ks && tok < w1;
            int32_t phys = __shfl(tbl, (tok >> p.bs_log2) - blk0, 64);
            phys = min(max(phys, 0), last_block);
            const int64_t slot = ((int64_t)phys << p.bs_log2) | (tok & bs_mask);
            sbase[j] = (((int64_t)phys * p.hkv + kvh) << p.bs_log2) | (tok & bs_mask);
            kr[j] = u32x4{0u, 0u, 0u, 0u};
            vr[j] = u32x4{0u, 0u, 0u, 0u};
            if (valid[j]) {
                kr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + slot * slot_stride));
                vr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + slot * slot_stride));
            }
        }
        // The row's NJ consecutive K and V scales: one aligned load each when a block holds
        // at least NJ tokens (the row's first token is a multiple of NJ), else per token.
        // Tokens outside [ks, w1) get scale 0 (their rows are zero and their weights 0).
        if ((1 << p.bs_log2) >= NJ) {
            if constexpr (NJ == 4) {
                const f32x4 a = *reinterpret_cast<const f32x4*>(p.k_scale + sbase[0]);
                const f32x4 c = *reinterpret_cast<const f32x4*>(p.v_scale + sbase[0]);
#pragma unroll
                for (int j = 0; j < NJ; ++j) { ksc[j] = a[j]; vsc[j] = c[j]; }
            } else {
                const float2 a = *reinterpret_cast<const float2*>(p.k_scale + sbase[0]);
                const float2 c = *reinterpret_cast<const float2*>(p.v_scale + sbase[0]);
                ksc[0] = a.x; ksc[1] = a.y;
                vsc[0] = c.x; vsc[1] = c.y;
            }
        } else {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                ksc[j] = p.k_scale[sbase[j]];
                vsc[j] = p.v_scale[sbase[j]];
            }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            ksc[j] = valid[j] ? ksc[j] : 0.0f;
            vsc[j] = valid[j] ? vsc[j] : 0.0f;
        }
        // K codes as bf16 pairs; V codes widened once for all heads of the group.
        uint32_t kb[NJ][8];
        float vf[NJ][EPL];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kb[j][2 * i] = pack_bf16_pair(sbyte(kr[j][i], 0), sbyte(kr[j][i], 1));
                kb[j][2 * i + 1] = pack_bf16_pair(sbyte(kr[j][i], 2), sbyte(kr[j][i], 3));
#pragma unroll
                for (int k = 0; k < 4; ++k) vf[j][4 * i + k] = sbyte(vr[j][i], k);
            }
        }

#pragma unroll
        for (int g = 0; g < GP; ++g) {
            if (g >= p.group) break;
            float s[NJ];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                float a = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) a = dot2_bf16(qv[g][i], kb[j][i], a);
                const float dotp = group_sum<LPT>(a) * ksc[j];
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
                    const float pv = pj * vsc[j];
#pragma unroll
                    for (int e = 0; e < EPL; ++e) o[g][e] = fmaf(pv, vf[j][e], o[g][e]);
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
        const int gi = i / D;   // g * HP + head of the group
        const int d = i % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWavesI8; ++w) M = fmaxf(M, sm_m[w][gi]);
        float acc = 0.0f, lsum = 0.0f;
#pragma unroll
        for (int w = 0; w < kWavesI8; ++w) {
            const float f = (sm_m[w][gi] == -INFINITY) ? 0.0f : fast_exp2(sm_m[w][gi] - M);
            acc = fmaf(f, sm_o[w][gi][d], acc);
            lsum = fmaf(f, sm_l[w][gi], lsum);
        }
        const int h = (kvp * HP + gi % HP) * p.group + gi / HP;
        const int64_t bh = (int64_t)b * p.hq + h;
        if (nsplit == 1) {
            reinterpret_cast<uint16_t*>(p.out)[bh * D + d] = f32_to_bf16(acc / lsum);
            if (p.lse && d == 0) p.lse[bh] = (M + __log2f(lsum)) * kLn2i8;
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

}  // namespace

int int8_head_group(int32_t group, int32_t num_kv_heads) {
    // Pairs: on the Llama-7B INT8 step 72.3 -> 69.6 us with 256-key splits (groups of 4
    // with 8-token steps: 76; pairs over 128 or 512 keys: 73.8, 71.3).
    return group == 1 && num_kv_heads % 2 == 0 ? 2 : 1;
}

hipError_t launch_kv_write_int8(const QuantWriteParams& p, int in_dtype, int head_dim, hipStream_t s) {
    const int rpw = 64 / (head_dim / 8);
    const int64_t rows = p.num_tokens * p.hkv;
    const dim3 grid((unsigned)((rows + 4 * rpw - 1) / (4 * rpw)), 2);
    if (in_dtype == 1) {
        if (head_dim == 64) hipLaunchKernelGGL((kv_write_int8_kernel<bf16_t, 64>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((kv_write_int8_kernel<bf16_t, 128>), grid, dim3(256), 0, s, p);
    } else {
        if (head_dim == 64) hipLaunchKernelGGL((kv_write_int8_kernel<float, 64>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((kv_write_int8_kernel<float, 128>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

hipError_t launch_kv_write_int8_mla(const QuantWriteParams& p, int in_dtype, hipStream_t s) {
    QuantWriteParams q = p;
    const int64_t rows = p.num_tokens;                                  // one kv head
    const dim3 gn((unsigned)((rows + 3) / 4), 1);                       // 512 wide: one row per wave
    const dim3 gr((unsigned)((rows + 31) / 32), 1);                     // 64 wide: eight per wave
    q.which_base = 0;
    if (in_dtype == 1) hipLaunchKernelGGL((kv_write_int8_kernel<bf16_t, 512>), gn, dim3(256), 0, s, q);
    else hipLaunchKernelGGL((kv_write_int8_kernel<float, 512>), gn, dim3(256), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    q.which_base = 1;
    if (in_dtype == 1) hipLaunchKernelGGL((kv_write_int8_kernel<bf16_t, 64>), gr, dim3(256), 0, s, q);
    else hipLaunchKernelGGL((kv_write_int8_kernel<float, 64>), gr, dim3(256), 0, s, q);
    return hipGetLastError();
}

template <int D, bool APPEND>
void launch_decode_int8_d(const DecodeParams& p, dim3 grid, hipStream_t s) {
    const int gp = p.group <= 1 ? 1 : (p.group <= 2 ? 2 : 4);
    const int hp = int8_head_group(p.group, p.hkv);
    if (hp == 2) hipLaunchKernelGGL((decode_int8_kernel<D, 1, APPEND, 2>), grid, dim3(256), 0, s, p);
    else if (gp == 1) hipLaunchKernelGGL((decode_int8_kernel<D, 1, APPEND, 1>), grid, dim3(256), 0, s, p);
    else if (gp == 2) hipLaunchKernelGGL((decode_int8_kernel<D, 2, APPEND, 1>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((decode_int8_kernel<D, 4, APPEND, 1>), grid, dim3(256), 0, s, p);
}

hipError_t launch_decode_int8(const DecodeParams& p, int head_dim, hipStream_t s) {
    if (p.parts > 0) return launch_gqa_decode_int8(p, head_dim, s);
    const int hp = int8_head_group(p.group, p.hkv);
    const dim3 grid((unsigned)((int64_t)(p.hkv / hp) * p.batch * p.max_splits));
    const bool append = p.k_new != nullptr;
    if (head_dim == 64) {
        if (append) launch_decode_int8_d<64, true>(p, grid, s);
        else launch_decode_int8_d<64, false>(p, grid, s);
    } else {
        if (append) launch_decode_int8_d<128, true>(p, grid, s);
        else launch_decode_int8_d<128, false>(p, grid, s);
    }
    return hipGetLastError();
}

}  // namespace pkv
