// MLA-absorbed decode over the paged INT8 cache with MFMA for gfx950 ("KVCache
// Optimization Skill", Mode 3: key = cache_nope || cache_rope, value = cache_nope, rope
// passed separately; the cache holds int8 codes with one fp32 scale per token for nope and
// one for rope).  The bf16 cache runs mla_wide_kernel.
//
// A workgroup of four waves owns 64 heads (16 per wave) of one (sequence, split) and walks
// its keys in tiles of 32, each wave over the whole 576-wide contraction, with
// v_mfma_f32_16x16x32_bf16 over bf16 copies of the codes (exact: |q| <= 127).  The two
// head groups of 128 heads are launched onto the same XCD so that the second read of a tile
// comes from its L2.
//  * the codes of a tile (512 + 64 bytes per key) and its keys' scales reach LDS by direct
//    loads two tiles ahead; each wave converts the eight keys it loaded into one of two
//    bf16 buffers (32 nope rows of 1024 bytes padded to 1056, then 32 rope rows of 128
//    bytes with their chunks XOR-swizzled by row) before the tile's barrier;
//  * S^T (16 keys x 16 heads, two per tile) = K . Q^T: K rows from the buffer as the A
//    operand, Q^T of the wave's 16 heads in the accumulation registers as B (72); the nope
//    and rope sums are kept apart and weighed per key with the two scales;
//  * lane (g, n) (g = lane / 16) holds 8 keys of head n: the head's max and sum take two
//    cross-lane steps, and P'^T = bf16(p s_nope) (the nope scale folded into the value
//    weight; l sums the fp32 p) is the B operand of the next product with k-slot
//    8 g + 4 h + r standing for accumulator entry r of key half h;
//  * O^T (512 x 16 heads, 128 registers) += V^T . P'^T, the A operand built by two
//    ds_read_b64_tr_b16 per product from the nope part of the same buffer rows;
//  * the online-softmax rescale is lane-local and applied only when a head's max grows by
//    more than 2^8 (P <= 256 in between).  Full tiles skip the masking.
#include "mfma_common.h"

namespace pkv {

namespace {

using namespace mfma;

struct MlaCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kHeads = kWaves * 16;              // query heads per workgroup
    // bf16 stage: 32 nope rows of 1024 bytes padded to 1056, then 32 rope rows of 128
    // bytes with their chunks XOR-swizzled by row.
    // The 32-byte padding was measured on gfx950 to serve both the 16-byte K reads and the
    // 8-byte transposing V reads of the products without bank conflicts (a probe of the two
    // read patterns: 191 and 161 B/clk per CU, against 112 and 112 with 16-byte padding).
    static constexpr int kNopeRow = 1024 + 32;
    static constexpr int kRopeBase = kKeys * kNopeRow;
    static constexpr int kStage = kRopeBase + kKeys * 128;
    static constexpr int kSteps = 576 / 32;                 // S^T k-steps (16 nope, 2 rope)
    static constexpr int kDTiles = 512 / 16;                // 16-row tiles of O^T
    static_assert(kKeys * 128 == kWaves * 1024, "one rope load per wave");
};

// LDS row (within a 16-key half) of the key behind accumulator row 4 g + r: the four keys
// of one transposing read (r = 0..3) sit two LDS rows apart.
__device__ __forceinline__ int mla_row(int g, int r) { return (g & 2) * 4 + (g & 1) + 2 * r; }
// Physical 16-byte chunk of rope chunk c in rope row r.
__device__ __forceinline__ int rope_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// LDS of the INT8 form: three stages of codes as loaded (32 nope rows of 512 bytes, then per
// wave 1 KiB: its 8 rope rows of 64 bytes, the 8 nope scales, the 8 rope scales, padding),
// two bf16 buffers (a bf16 stage plus the tile's 32 nope and 32 rope scales), the table.
struct MlaI8Cfg {
    static constexpr int kCodeStages = 3;
    static constexpr int kNopeCodes = kKeys * 512;
    static constexpr int kAux = 1024;
    static constexpr int kCodeStage = kNopeCodes + MlaCfg::kWaves * kAux;
    static constexpr int kBuf = MlaCfg::kStage + 2 * kKeys * 4;
    static constexpr int kBufOff = kCodeStages * kCodeStage;
    static constexpr int kTabOff = kBufOff + 2 * kBuf;
    static constexpr int kSmem = kTabOff + 2 * kTabEntries * 4;
    static constexpr int kDma = 5;                          // wave loads per tile: 4 nope + 1 rope and scales
    static_assert(kSmem <= 160 * 1024, "LDS");
    static_assert(kBuf % 16 == 0, "buffer alignment");
};

// Code k of a dword as float.
__device__ __forceinline__ float code_of(uint32_t w, int k) { return (float)(int)(int8_t)(w >> (8 * k)); }
// 16 codes as 16 bf16 (exact), codes 0-7 in lo, 8-15 in hi.
__device__ __forceinline__ void codes_to_bf16(u32x4 v, u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t a = pack_bf16(code_of(v[i], 0), code_of(v[i], 1));
        const uint32_t b = pack_bf16(code_of(v[i], 2), code_of(v[i], 3));
        if (i < 2) { lo[2 * i] = a; lo[2 * i + 1] = b; }
        else { hi[2 * i - 4] = a; hi[2 * i - 3] = b; }
    }
}

__global__ __launch_bounds__(MlaCfg::kThreads) void mla_int8_kernel(MfmaParams p) {
    using C = MlaCfg;
    using I = MlaI8Cfg;
    constexpr int kTabOff = I::kTabOff;
    __shared__ __attribute__((aligned(16))) uint8_t smem[I::kSmem];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 15;          // head of this lane inside the wave; A-operand row
    const int g = lane >> 4;          // k-slot group

    // Workgroups are dealt to the 8 XCDs round-robin; the head groups of one work unit
    // take ids that differ by a multiple of 8 and follow each other on one XCD.  Units
    // (sequence, split) are numbered without gaps, the longest sequences first.
    const int hgs = (p.hq + C::kHeads - 1) / C::kHeads;
    const int id = blockIdx.x;
    const int hg = (id >> 3) % hgs;
    const int unit = ((id >> 3) / hgs) * 8 + (id & 7);
    int b, split;
    {
        auto nsplits = [&](int, int len) { return len > 0 ? (len + p.split_tokens - 1) / p.split_tokens : 1; };
        if (!find_item<C::kThreads>(unit, p.batch, p.seq_lens, p.len_cap, nsplits,
                                    reinterpret_cast<int32_t*>(smem + kTabOff), b, split))
            return;
        b = __builtin_amdgcn_readfirstlane(b);          // the same in every lane
        split = __builtin_amdgcn_readfirstlane(split);
    }
    if (split >= p.max_splits) return;
    const int L = min(p.seq_lens[b], p.len_cap);
    if (L <= 0) {   // no visible key: output 0, lse -inf (one unit per such sequence)
        const int h0 = hg * C::kHeads + wid * 16 + (lane & 15);
        if (h0 < p.hq) {
            uint16_t* o0 = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)b * p.hq + h0) * 512 + 4 * (lane >> 4);
            for (int dt = 0; dt < 32; ++dt) *reinterpret_cast<uint2*>(o0 + 16 * dt) = make_uint2(0u, 0u);
            if (p.lse && lane < 16) p.lse[(int64_t)b * p.hq + h0] = -INFINITY;
        }
        return;
    }
    // The sequence's ns = ceil(L / split_tokens) splits (the count the merge uses) share its
    // tiles evenly, so that its units are of one size for the longest-first order; if an
    // even share could leave the last split empty they keep split_tokens keys each.
    int split_keys = p.split_tokens;
    {
        const int tiles = (L + kKeys - 1) / kKeys;
        const int ns = (L + p.split_tokens - 1) / p.split_tokens;
        const int even = (tiles + ns - 1) / ns;
        if ((int64_t)(ns - 1) * even < tiles) split_keys = even * kKeys;
    }
    const int k_begin = split * split_keys;
    if (k_begin >= L) return;
    const int k_end = min(L, k_begin + split_keys);
    const int ntiles = (k_end - k_begin + kKeys - 1) / kKeys;
    const int head = hg * C::kHeads + wid * 16 + n;
    const bool valid = head < p.hq;
    const int64_t row = (int64_t)b * p.hq + min(head, p.hq - 1);

    // Q^T fragments: k-step s covers dims 32 s .. 32 s + 31; this lane holds 8 of them.
    bf16x8_t qf[C::kSteps];
    {
        const uint8_t* qn = reinterpret_cast<const uint8_t*>(p.q) + row * 512 * 2;
        const uint8_t* qr = reinterpret_cast<const uint8_t*>(p.q_rope) + row * 64 * 2;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
            const int dim = 32 * s + 8 * g;
            qf[s] = __builtin_bit_cast(bf16x8_t, ld16(dim < 512 ? qn + dim * 2 : qr + (dim - 512) * 2));
            // Keep Q^T in the accumulation registers (the products read their B operand
            // from there directly), leaving the VGPRs to O^T and the operands in flight.
            asm volatile("" : "+a"(qf[s]));
        }
    }

    TableChunks<C::kThreads> tab;
    tab.lds = reinterpret_cast<int32_t*>(smem + kTabOff);
    tab.row = p.table + (int64_t)b * p.mbs;
    tab.k_begin = k_begin;
    tab.k_end = k_end;
    tab.bs_log2 = p.bs_log2;
    tab.tid = tid;
    tab.last_block = (int32_t)(p.num_blocks - 1);
    int32_t treg[TableChunks<C::kThreads>::kRegs];
    tab.load(0, treg);
    tab.store(0, treg);
    // Q and the first chunk must be resident before the loop: otherwise the wait for
    // them, placed inside the loop, would also wait for the tile loads issued there.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_sync();

    // Loads of one tile: wave w fills nope rows 8 w .. 8 w + 7 (one load per row, lane =
    // 16-byte chunk; the row's slot is the same for the whole wave) and rope rows
    // 8 w .. 8 w + 7 (one load, lane = row 8 w + lane / 8, physical chunk lane % 8).
    const int bs_mask = (1 << p.bs_log2) - 1;
    // Full tiles with blocks of at least 8 keys: the wave's 8 rows are consecutive slots of
    // one block, found with one scalar read of the block table; every load then uses that
    // row base in SGPRs and a constant offset per lane.
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);
    const bool fast_rows = p.bs_log2 >= 3;
    // The table entry of the next tile is read one tile ahead, off the critical path.
    auto fast_tile = [&](int u) {
        return fast_rows && k_begin + (u + 1) * kKeys <= k_end;
    };
    auto entry_of = [&](int u) { return uniform_load(tab.row + ((k_begin + u * kKeys + 8 * wid_u) >> p.bs_log2)); };
    int32_t next_entry = fast_tile(0) ? entry_of(0) : 0;
    auto issue_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        const int chunk = u / kChunkTiles;
        // Wave w loads the codes of keys 8 w .. 8 w + 7: their nope rows (4 loads of two
        // rows) and one load whose lanes 0-31 take the 8 rope rows, 32-33 the 8 nope
        // scales, 34-35 the 8 rope scales (scales are in slot order per block, and a
        // group of 4 keys lies in one block), the others re-read lane 32's bytes.
        uint8_t* cs = smem + (u % I::kCodeStages) * I::kCodeStage;
        uint8_t* aux = cs + I::kNopeCodes + wid_u * I::kAux;
        const uint8_t* ncodes = reinterpret_cast<const uint8_t*>(p.k_cache);
        const uint8_t* rcodes = reinterpret_cast<const uint8_t*>(p.k_rope);
        const uint8_t* nsc = reinterpret_cast<const uint8_t*>(p.k_scale);
        const uint8_t* rsc = reinterpret_cast<const uint8_t*>(p.r_scale);
        const int32_t entry = next_entry;
        if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
        const int q = lane >= 32 && lane < 36 ? lane - 32 : 0;
        if (fast_tile(u)) {
            const int key0 = kb + 8 * wid_u;
            const int32_t blk = min(max(entry, 0), tab.last_block);
            const uint64_t slot0 = ((uint64_t)(uint32_t)blk << p.bs_log2) | (uint32_t)(key0 & bs_mask);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                lds_dma16_s(ncodes + slot0 * 512u + j * 1024, (uint32_t)lane * 16u, cs + (8 * wid_u) * 512 + j * 1024);
            const uint8_t* src = lane < 32 ? rcodes + slot0 * 64u + lane * 16
                                           : ((q & 2) ? rsc : nsc) + slot0 * 4u + (q & 1) * 16;
            lds_dma16(src, aux);
            return;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = min(kb + 8 * wid + 2 * j + (lane >> 5), k_end - 1);
            const uint64_t slot = ((uint64_t)tab.block_of(key, chunk) << p.bs_log2) | (uint32_t)(key & bs_mask);
            lds_dma16(ncodes + slot * 512u + (lane & 31) * 16, cs + (8 * wid_u + 2 * j) * 512);
        }
        // keys past the range: their rope row and scales come from the last key (its
        // 4-key group for the scales); their weights are 0
        const int key = lane < 32 ? min(kb + 8 * wid + (lane >> 2), k_end - 1)
                                  : min(kb + 8 * wid + 4 * (q & 1), (k_end - 1) & ~3);
        const uint64_t slot = ((uint64_t)tab.block_of(key, chunk) << p.bs_log2) | (uint32_t)(key & bs_mask);
        lds_dma16(lane < 32 ? rcodes + slot * 64u + (lane & 3) * 16 : ((q & 2) ? rsc : nsc) + slot * 4u, aux);
    };

    // S^T reads: A-operand row n of key half h is LDS row 16 h + mla_row(n / 4, n % 4);
    // k-step s < 16 reads nope chunk 4 s + g, k-step 16 + i rope chunk 4 i + g.
    const int krow = mla_row(n >> 2, n & 3);
    int k_off[2], rope_off[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 16 * h + krow;
        k_off[h] = r * C::kNopeRow + 16 * g;
#pragma unroll
        for (int i = 0; i < 2; ++i) rope_off[h][i] = C::kRopeBase + r * 128 + rope_chunk(r, 4 * i + g) * 16;
    }
    // O^T reads: lane (g, n) reads LDS rows 16 h + mla_row(g, n / 4), value columns
    // 16 dt + 4 (n % 4) .. + 3.
    int v_off[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) v_off[h] = (16 * h + mla_row(g, n >> 2)) * C::kNopeRow + 8 * (n & 3);

    // INT8: this wave's keys of tile t, codes -> bf16 buffer t & 1 (it reads only what it
    // loaded itself, so its own load counter is the only wait), scales beside them.
    auto convert = [&](int t) {
        const uint8_t* cs = smem + (t % I::kCodeStages) * I::kCodeStage;
        uint8_t* bf = smem + I::kBufOff + (t & 1) * I::kBuf;
        // All reads first: a store to the bf16 buffer may alias a later read as far as the
        // compiler knows, so interleaved it would wait out each read's latency.
        const uint8_t* aux = cs + I::kNopeCodes + wid_u * I::kAux;
        u32x4 raw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ci = lane + 64 * i;
            raw[i] = *reinterpret_cast<const u32x4*>(cs + (8 * wid_u + (ci >> 5)) * 512 + (ci & 31) * 16);
        }
        const u32x4 rraw = *reinterpret_cast<const u32x4*>(aux + (lane & 31) * 16);
        const float sc_in = *reinterpret_cast<const float*>(aux + 512 + ((lane - 32) & 15) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {          // nope: 8 rows x 32 chunks of 16 codes
            const int ci = lane + 64 * i;
            const int r = 8 * wid_u + (ci >> 5);
            const int c16 = ci & 31;
            u32x4 lo, hi;
            codes_to_bf16(raw[i], lo, hi);
            *reinterpret_cast<u32x4*>(bf + r * C::kNopeRow + c16 * 32) = lo;
            *reinterpret_cast<u32x4*>(bf + r * C::kNopeRow + c16 * 32 + 16) = hi;
        }
        if (lane < 32) {                       // rope: row 8 w + lane / 4, dims 16 (lane % 4) ..
            const int r = 8 * wid_u + (lane >> 2);
            const int c4 = lane & 3;
            u32x4 lo, hi;
            codes_to_bf16(rraw, lo, hi);
            *reinterpret_cast<u32x4*>(bf + C::kRopeBase + r * 128 + rope_chunk(r, 2 * c4) * 16) = lo;
            *reinterpret_cast<u32x4*>(bf + C::kRopeBase + r * 128 + rope_chunk(r, 2 * c4 + 1) * 16) = hi;
        } else if (lane < 48) {                // scales: 8 nope, then 8 rope
            const int qq = lane - 32;
            *reinterpret_cast<float*>(bf + C::kStage + ((qq >> 3) * kKeys + 8 * wid_u + (qq & 7)) * 4) = sc_in;
        }
    };

    RowState st;
    f32x4 oacc[C::kDTiles];
#pragma unroll
    for (int dt = 0; dt < C::kDTiles; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Scores of tile t: full tiles keep the raw S^T entries; the last tile of a range scales
    // them and sets keys past the range (and all keys of heads past num_q_heads) to -inf.
    // Entry (h, r) of lane (g, n) is key 16 h + mla_row(g, r) of the tile.  Returns the
    // head's max over the tile (scaled, log2 units).
    auto scores = [&](int t, bool full, float* sv, float* sn) -> float {
        const uint8_t* stage = smem + I::kBufOff + (t & 1) * I::kBuf;
        f32x4 sacc[2], racc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            sacc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
            racc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < C::kSteps; ++s) {
                const uint8_t* src = s < 16 ? stage + k_off[h] + 64 * s : stage + rope_off[h][s - 16];
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(src));
                if (s >= 16) racc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], racc[h], 0, 0, 0);
                else sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[s], sacc[h], 0, 0, 0);
            }
        }
        // Keep six K reads in flight ahead of the products (left alone, the compiler
        // issues each read just before its product and waits out the LDS latency).
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
        for (int i = 0; i < 2 * C::kSteps - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
        // per key: s_nope * (q_nope . codes) + s_rope * (q_rope . codes)
        const float* scn = reinterpret_cast<const float*>(stage + C::kStage);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = 16 * (e >> 2) + mla_row(g, e & 3);
            sn[e] = scn[key];
            sacc[e >> 2][e & 3] = sn[e] * sacc[e >> 2][e & 3] + scn[kKeys + key] * racc[e >> 2][e & 3];
        }
        float tmax;
        if (full) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][e & 3];
            tmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            tmax *= p.scale_log2;
        } else {
            const int kb = k_begin + t * kKeys;
            tmax = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int key = kb + 16 * (e >> 2) + mla_row(g, e & 3);
                sv[e] = (valid && key < k_end) ? sacc[e >> 2][e & 3] * p.scale_log2 : -INFINITY;
                if (sv[e] == -INFINITY) sn[e] = 0.0f;   // no stale scale reaches P'
                tmax = fmaxf(tmax, sv[e]);
            }
        }
        return max_xor32(max_xor16(tmax));
    };

    // P^T of tile t against the running max (k-slot 8 g + 4 h + r is entry (h, r); l adds
    // the fp32 weights, the products take them rounded), then O^T += V^T . P^T.
    auto probs_pv = [&](int t, bool full, const float* sv, const float* sn) {
        u32x4 pw;
        if (full) {
            const float mneg = -st.m;
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float e0 = fast_exp2(__builtin_fmaf(sv[e], p.scale_log2, mneg));
                const float e1 = fast_exp2(__builtin_fmaf(sv[e + 1], p.scale_log2, mneg));
                st.l += e0 + e1;
                pw[e >> 1] = pack_bf16(e0 * sn[e], e1 * sn[e + 1]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float e0 = sv[e] == -INFINITY ? 0.0f : fast_exp2(sv[e] - st.m);
                const float e1 = sv[e + 1] == -INFINITY ? 0.0f : fast_exp2(sv[e + 1] - st.m);
                st.l += e0 + e1;
                pw[e >> 1] = pack_bf16(e0 * sn[e], e1 * sn[e + 1]);
            }
        }
        const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw);
        const uint8_t* stage = smem + I::kBufOff + (t & 1) * I::kBuf;
        const uint8_t* v0 = stage + v_off[0];
        const uint8_t* v1 = stage + v_off[1];
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) {
            // Assemble the operand from whole dwords: extracting the 16-bit elements one
            // by one made the compiler keep only the first dword of each read.
            const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(v0 + 32 * dt));
            const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(v1 + 32 * dt));
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, oacc[dt], 0, 0, 0);
        }
        // Twelve transposing reads (six products) in flight ahead of the products.
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 12, 0);
#pragma unroll
        for (int i = 0; i < C::kDTiles - 6; ++i) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
    };

    // Table chunks and the loads of tile u (issued kAhead tiles ahead).
    auto feed = [&](int u) {
        if (u >= ntiles) return;
        const int c = u / kChunkTiles;
        if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load(c + 1, treg);
        if (u % kChunkTiles == kChunkTiles / 2 && tab.exists(c + 1)) tab.store(c + 1, treg);
        issue_tile(u);
    };
    constexpr int kAhead = I::kCodeStages - 1;   // tiles issued ahead
#pragma unroll
    for (int u = 0; u < kAhead; ++u) feed(u);

    // Tile t: wait for this wave's codes, convert them, barrier (buffer t & 1 complete, the
    // code stage of tile t - 1 free, staged table entries visible), issue tile t + 2,
    // scores, then P and O.  A tile that raises some head's max by more than the
    // slack leaves the loop to rescale O^T, so that inside the loop the accumulators are
    // only touched by the products.
    int t = 0;
    float sv[8], sn[8];
    float tmax = 0.0f;
    bool full = false;
    while (t < ntiles) {
        for (; t < ntiles; ++t) {
            // This wave's codes of tile t (tile t + 1 may stay in flight), into bf16; the
            // barrier publishes buffer t & 1 and frees the code stage of tile t - 1
            // (converted) and buffer (t + 1) & 1 (read by tile t - 1) for reuse.
            wait_tile<I::kDma>(min(ntiles - 1 - t, 1));
            convert(t);
            block_sync();
            feed(t + kAhead);
            full = k_begin + (t + 1) * kKeys <= k_end;
            tmax = scores(t, full, sv, sn);
            const bool grow = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
            if (__any(grow)) break;
            probs_pv(t, full, sv, sn);
        }
        if (t >= ntiles) break;
        {
            const bool grow = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
            const float mnew = grow ? tmax : st.m;
            const float alpha = !grow ? 1.0f : (st.m == -INFINITY ? 0.0f : fast_exp2(st.m - mnew));
            st.l *= alpha;
#pragma unroll
            for (int dt = 0; dt < C::kDTiles; ++dt) oacc[dt] *= alpha;
            st.m = mnew;
        }
        probs_pv(t, full, sv, sn);
        ++t;
    }

    // ---------------------------------------------------------------- epilogue
    float l_tot = st.l + __shfl_xor(st.l, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (!valid) return;
    const int nsplit = (L + p.split_tokens - 1) / p.split_tokens;
    if (nsplit == 1) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + row * 512 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) {
            const uint32_t w0 = bf16_bits(oacc[dt][0] * inv) | ((uint32_t)bf16_bits(oacc[dt][1] * inv) << 16);
            const uint32_t w1 = bf16_bits(oacc[dt][2] * inv) | ((uint32_t)bf16_bits(oacc[dt][3] * inv) << 16);
            *reinterpret_cast<uint2*>(out + 16 * dt) = make_uint2(w0, w1);
        }
        if (p.lse && g == 0) p.lse[row] = l_tot > 0.0f ? (st.m + __log2f(l_tot)) * kLn2f : -INFINITY;
    } else {
        const int64_t ps = row * p.max_splits + split;
        float* o = p.ws_o + ps * 512 + 4 * g;
#pragma unroll
        for (int dt = 0; dt < C::kDTiles; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt) = oacc[dt];
        if (g == 0) {
            p.ws_ml[ps * 2] = st.m;
            p.ws_ml[ps * 2 + 1] = l_tot;
        }
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

int32_t mla_head_groups(int32_t num_q_heads) {
    return (num_q_heads + MlaCfg::kHeads - 1) / MlaCfg::kHeads;
}

DecodePlan plan_mla(int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t max_seq_len_kv) {
    DecodePlan pl{};
    const int64_t hgs = mla_head_groups(num_q_heads);
    auto nsplits = [&](int sp) { return (int64_t)(max_seq_len_kv + sp - 1) / sp; };
    // A split's partial state is Hq x Dv fp32 (256 KiB at 128 x 512): long splits keep that
    // traffic small; shorten them only while the grid would leave compute units idle.  With
    // one workgroup per CU the time also depends on how the units pack onto the CUs: on 64
    // sequences of 2K-8K keys (splits of a sequence evenly sized) a sweep measured 1536 best
    // (163.3 us; 1024: 177.8, 1280: 197.6, 2048: 190.2).
    int split = 1536;
    while (split > 256 && batch * hgs * nsplits(split) < 512) split /= 2;
    pl.split_tokens = split;
    pl.max_splits = (int32_t)(max_seq_len_kv > 0 ? nsplits(split) : 1);
    if (pl.max_splits <= 1) return pl;
    const size_t rows = (size_t)batch * num_q_heads * pl.max_splits;
    pl.ws_o_offset = 0;
    pl.ws_ml_offset = align256(rows * head_dim_v * sizeof(float));
    pl.ws_bytes = pl.ws_ml_offset + rows * 2 * sizeof(float);
    return pl;
}

hipError_t launch_mla_decode(const MfmaParams& p, hipStream_t s) {
    if (!p.k_scale) return launch_mla_wide(p, s);   // bf16: one workgroup for 128 heads
    // ids: (unit / 8, head group, unit % 8) with units = batch * max_splits rounded up to 8
    const int64_t hgs = mla_head_groups(p.hq);
    const int64_t units = ((int64_t)p.batch * p.max_splits + 7) / 8 * 8;
    const dim3 grid((unsigned)(hgs * units));
    hipLaunchKernelGGL(mla_int8_kernel, grid, dim3(MlaCfg::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
