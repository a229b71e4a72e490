// MLA-absorbed decode over the paged bf16 cache, one workgroup per (sequence, split) for
// all 128 query heads ("KVCache Optimization Skill", Mode 3: key = cache_nope ||
// cache_rope, value = cache_nope, one latent head shared by every query head): each K/V
// tile goes from HBM into LDS once and serves every head.
//
// Four waves, one per SIMD, 32 heads each, v_mfma_f32_32x32x16_bf16 for both products:
//  * S^T (32 keys x 32 heads) = K . Q^T over the 576-wide contraction (36 k-steps): K rows
//    from LDS as the A operand, Q^T of the wave's heads resident in VGPRs (144) as B.
//    The accumulator (lane l: head l % 32, keys 8 q + 4 (l / 32) + r) is already the B
//    operand P^T of the value product once the keys of k-step ks are numbered
//    16 ks + 8 (e / 4) + 4 (l / 32) + e % 4 for element e, so P needs no data movement;
//  * O^T (512 value columns x 32 heads: 16 tiles, all 256 AGPRs) += V^T . P^T, the A
//    operand by two transposing LDS reads (four keys at one value column per lane each).
// Each wave runs one tile apart: S^T(t + 1) is computed while the exponentials of P^T(t)
// are formed, then P . V of tile t.  The value products are inline assembly with their
// accumulators in AGPRs (built with MFMA results in VGPRs, the compiler would put O^T
// there too); it does not know them as MFMAs, so the cycles an MFMA result needs before
// anything else reads it (the rare rescale, the epilogue) and the wait states after a
// VALU write of an operand are spelled out.
//
// LDS stage: 32 nope rows of 1024 bytes padded to 1040, key k in row
// (k & 16) | 4 (k & 3) | ((k >> 2) & 3), so that the 16 lanes of a K read hit 16 different
// bank groups and the four rows of a transposing read (keys 4 h + a, a = 0..3, of a
// 16-key group) sit 16 banks apart; then 32 rope rows of 128 bytes (key k in row k), their
// 16-byte chunks XOR-swizzled by row.  Four stages, the tile pipeline of mfma_common.h.
#include "mfma_common.h"

namespace pkv {

namespace {

using namespace mfma;

struct WideCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kHeads = kWaves * 32;              // query heads per workgroup
    static constexpr int kNopeRow = 1024 + 16;
    static constexpr int kRopeBase = kKeys * kNopeRow;
    static constexpr int kStage = kRopeBase + kKeys * 128;
    static constexpr int kTabOff = kStages * kStage;
    static constexpr int kSmem = kTabOff + 2 * kTabEntries * 4;
    static constexpr int kDma = 9;                          // wave loads per tile: 8 nope rows + 8 rope rows
    static constexpr int kKRing = 4;                        // K operands in flight ahead of their product
    static constexpr int kVRing = 4;                        // V operands in flight ahead of their product
    static_assert(kSmem <= 160 * 1024, "LDS");
    static_assert(kKeys == 32 && kStages == 4, "tile of 32 keys, four stages");
    static_assert(3 * kThreads + 24 <= 2 * kTabEntries, "work-order scratch fits the table area");
};

// LDS nope row of key k of a tile.
__device__ __forceinline__ int wide_row(int k) { return (k & 16) | ((k & 3) << 2) | ((k >> 2) & 3); }
// Physical 16-byte chunk of rope chunk c in rope row r (an involution).
__device__ __forceinline__ int wide_rope_chunk(int r, int c) { return c ^ ((r >> 1) & 7); }

// Every AGPR times alpha (per lane), three instructions each: O^T holds all 256 AGPRs, so
// they are named directly, and the statement takes all of O^T as operands (no other value
// can sit in an AGPR there).  Its operands %16 (a VGPR scratch) and %17 (alpha).
#define PKV_RS1(n) "v_accvgpr_read_b32 %16, a" n "\n\tv_mul_f32 %16, %16, %17\n\tv_accvgpr_write_b32 a" n ", %16\n\t"
#define PKV_RS10(d) PKV_RS1(d "0") PKV_RS1(d "1") PKV_RS1(d "2") PKV_RS1(d "3") PKV_RS1(d "4") \
                    PKV_RS1(d "5") PKV_RS1(d "6") PKV_RS1(d "7") PKV_RS1(d "8") PKV_RS1(d "9")
#define PKV_RS_ALL                                                                                   \
    PKV_RS1("0") PKV_RS1("1") PKV_RS1("2") PKV_RS1("3") PKV_RS1("4") PKV_RS1("5") PKV_RS1("6")         \
    PKV_RS1("7") PKV_RS1("8") PKV_RS1("9") PKV_RS10("1") PKV_RS10("2") PKV_RS10("3") PKV_RS10("4")     \
    PKV_RS10("5") PKV_RS10("6") PKV_RS10("7") PKV_RS10("8") PKV_RS10("9") PKV_RS10("10")              \
    PKV_RS10("11") PKV_RS10("12") PKV_RS10("13") PKV_RS10("14") PKV_RS10("15") PKV_RS10("16")         \
    PKV_RS10("17") PKV_RS10("18") PKV_RS10("19") PKV_RS10("20") PKV_RS10("21") PKV_RS10("22")         \
    PKV_RS10("23") PKV_RS10("24") PKV_RS1("250") PKV_RS1("251") PKV_RS1("252") PKV_RS1("253")         \
    PKV_RS1("254") PKV_RS1("255")

// Cycles for an MFMA result written by inline assembly to be readable by anything else.
__device__ __forceinline__ void wait_mfma_result() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// APPEND: the key at seq_lens[b] - 1 is the step's new latent row, read from p.k_new /
// p.rope_new instead of the cache; the split that holds it also stores it at its slot
// (reported in slots_out).  A row longer than the length bound writes nothing (slot -1)
// and attends to its first len_cap cached keys.
template <bool APPEND>
__global__ __launch_bounds__(WideCfg::kThreads) void mla_wide_kernel(MfmaParams p) {
    using C = WideCfg;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;        // head of this lane inside the wave
    const int h = lane >> 5;          // k-slot half

    // Workgroups are dealt to the 8 XCDs round-robin; the head groups of one work unit
    // (more than 128 heads) take ids that differ by a multiple of 8.  Units (sequence,
    // split) are numbered without gaps, the longest sequences first.
    const int hgs = (p.hq + C::kHeads - 1) / C::kHeads;
    const int id = blockIdx.x;
    const int hg = (id >> 3) % hgs;
    const int unit = ((id >> 3) / hgs) * 8 + (id & 7);
    int b, split;
    {
        auto nsplits = [&](int, int len) { return len > 0 ? (len + p.split_tokens - 1) / p.split_tokens : 1; };
        if (!find_item<C::kThreads>(unit, p.batch, p.seq_lens, p.len_cap, nsplits,
                                    reinterpret_cast<int32_t*>(smem + C::kTabOff), b, split))
            return;
        b = __builtin_amdgcn_readfirstlane(b);
        split = __builtin_amdgcn_readfirstlane(split);
    }
    if (split >= p.max_splits) return;
    const int L = min(p.seq_lens[b], p.len_cap);
    const int head = hg * C::kHeads + wid * 32 + l32;
    const bool valid = head < p.hq;
    const int64_t row = (int64_t)b * p.hq + min(head, p.hq - 1);
    if (L <= 0) {   // no visible key: output 0, lse -inf (one unit per such sequence)
        if (valid) {
            uint16_t* o0 = reinterpret_cast<uint16_t*>(p.out) + row * 512 + 256 * h;
            for (int c = 0; c < 32; ++c) *reinterpret_cast<uint4*>(o0 + 8 * c) = make_uint4(0u, 0u, 0u, 0u);
            if (p.lse && h == 0) p.lse[row] = -INFINITY;
        }
        return;
    }
    // The sequence's ns splits share its tiles evenly, unless an even share could leave the
    // last split empty.
    int split_keys = p.split_tokens;
    {
        const int tiles = (L + kKeys - 1) / kKeys;
        const int ns = (L + p.split_tokens - 1) / p.split_tokens;
        const int even = (tiles + ns - 1) / ns;
        if ((int64_t)(ns - 1) * even < tiles) split_keys = even * kKeys;
    }
    const int k_begin = split * split_keys;
    const bool app = APPEND && p.seq_lens[b] <= p.len_cap;
    const int new_key = app ? L - 1 : INT_MAX;
    if (APPEND && !app && split == 0 && hg == 0 && p.slots_out && tid == 0) p.slots_out[b] = -1;
    if (k_begin >= L) return;
    const int k_end = min(L, k_begin + split_keys);
    const int ntiles = (k_end - k_begin + kKeys - 1) / kKeys;
    if (APPEND && hg == 0 && new_key >= k_begin && new_key < k_end && wid < 2) {
        const int32_t phys = min(max(p.table[(int64_t)b * p.mbs + (new_key >> p.bs_log2)], 0),
                                 (int32_t)(p.num_blocks - 1));
        const int64_t slot = ((int64_t)phys << p.bs_log2) | (new_key & ((1 << p.bs_log2) - 1));
        if (wid == 0) {
            st16(reinterpret_cast<uint8_t*>(p.k_cache_w) + slot * 1024 + lane * 16,
                 ld16(reinterpret_cast<const uint8_t*>(p.k_new) + (int64_t)b * 1024 + lane * 16));
            if (p.slots_out && lane == 0) p.slots_out[b] = slot;
        } else if (lane < 8) {
            st16(reinterpret_cast<uint8_t*>(p.rope_w) + slot * 128 + lane * 16,
                 ld16(reinterpret_cast<const uint8_t*>(p.rope_new) + (int64_t)b * 128 + lane * 16));
        }
    }

    // Q^T fragments: k-step s covers dims 16 s .. 16 s + 15, this lane 8 of them.  Loaded
    // before the first wait so that no wait for them lands inside the tile loop.
    bf16x8_t qf[36];
    {
        const uint8_t* qn = reinterpret_cast<const uint8_t*>(p.q) + row * 512 * 2;
        const uint8_t* qr = reinterpret_cast<const uint8_t*>(p.q_rope) + row * 64 * 2;
#pragma unroll
        for (int s = 0; s < 36; ++s) {
            const int dim = 16 * s + 8 * h;
            qf[s] = __builtin_bit_cast(bf16x8_t, ld16(dim < 512 ? qn + dim * 2 : qr + (dim - 512) * 2));
        }
    }

    TableChunks<C::kThreads> tab;
    tab.lds = reinterpret_cast<int32_t*>(smem + C::kTabOff);
    tab.row = p.table + (int64_t)b * p.mbs;
    tab.k_begin = k_begin;
    tab.k_end = k_end;
    tab.bs_log2 = p.bs_log2;
    tab.tid = tid;
    tab.last_block = (int32_t)(p.num_blocks - 1);
    int32_t treg[TableChunks<C::kThreads>::kRegs];
    tab.load(0, treg);
    tab.store(0, treg);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_sync();

    // Loads of one tile: wave w fills the nope rows of keys 8 w .. 8 w + 7 (one load per
    // row, lane = 16-byte chunk) and their rope rows (one load: lane = row 8 w + lane / 8,
    // physical chunk lane % 8).
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);
    const int bs_mask = (1 << p.bs_log2) - 1;
    const uint8_t* nope_g = reinterpret_cast<const uint8_t*>(p.k_cache);
    const uint8_t* rope_g = reinterpret_cast<const uint8_t*>(p.k_rope);
    const int rope_r = 8 * wid_u + (lane >> 3);
    const int rope_c = wide_rope_chunk(rope_r, lane & 7);
    const uint32_t rope_voff = (uint32_t)((lane >> 3) * 128 + rope_c * 16);
    // Full tiles with blocks of at least 8 keys: the wave's 8 keys are consecutive slots of
    // one block, found with one scalar read of the block table (one tile ahead).
    const bool fast_rows = p.bs_log2 >= 3;
    auto fast_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        return fast_rows && kb + kKeys <= k_end && !(APPEND && new_key >= kb && new_key < kb + kKeys);
    };
    auto entry_of = [&](int u) { return uniform_load(tab.row + ((k_begin + u * kKeys + 8 * wid_u) >> p.bs_log2)); };
    int32_t next_entry = fast_tile(0) ? entry_of(0) : 0;
    auto issue_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        const int chunk = u / kChunkTiles;
        uint8_t* stage = smem + (u % kStages) * C::kStage;
        const int32_t entry = next_entry;
        if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
        if (fast_tile(u)) {
            const int key0 = kb + 8 * wid_u;
            const int32_t blk = min(max(entry, 0), tab.last_block);
            const uint64_t slot0 = ((uint64_t)(uint32_t)blk << p.bs_log2) | (uint32_t)(key0 & bs_mask);
            const uint8_t* nb = nope_g + slot0 * 1024u;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                lds_dma16_s(nb + j * 1024, (uint32_t)lane * 16u, stage + wide_row(8 * wid_u + j) * C::kNopeRow);
            lds_dma16_s(rope_g + slot0 * 128u, rope_voff, stage + C::kRopeBase + wid_u * 1024);
            return;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = min(kb + 8 * wid_u + j, k_end - 1);
            const uint32_t blk = __builtin_amdgcn_readfirstlane(tab.block_of(key, chunk));
            const uint8_t* src = nope_g + (((uint64_t)blk << p.bs_log2) | (uint32_t)(key & bs_mask)) * 1024u + lane * 16;
            if (APPEND && key == new_key)
                src = reinterpret_cast<const uint8_t*>(p.k_new) + (int64_t)b * 1024 + lane * 16;
            lds_dma16(src, stage + wide_row(8 * wid_u + j) * C::kNopeRow);
        }
        const int key = min(kb + rope_r, k_end - 1);
        const uint32_t blk = tab.block_of(key, chunk);
        const uint8_t* src = rope_g + (((uint64_t)blk << p.bs_log2) | (uint32_t)(key & bs_mask)) * 128u + rope_c * 16;
        if (APPEND && key == new_key)
            src = reinterpret_cast<const uint8_t*>(p.rope_new) + (int64_t)b * 128 + rope_c * 16;
        lds_dma16(src, stage + C::kRopeBase + wid_u * 1024);
    };
    // Table chunks and the loads of tile u.
    auto feed = [&](int u) {
        if (u >= ntiles) return;
        const int c = u / kChunkTiles;
        if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load(c + 1, treg);
        if (u % kChunkTiles == kChunkTiles / 2 && tab.exists(c + 1)) tab.store(c + 1, treg);
        issue_tile(u);
    };

    // Per-lane LDS offsets inside a stage.  K read of k-step s < 32: nope row of key l % 32,
    // bytes 32 s + 16 h; rope k-step 32 + i: rope chunk 2 i + h of that key.  Transposing
    // read of V (k-step ks, read rd, value tile ct): lane (G = lane / 16, a = lane / 4 % 4,
    // j = lane % 4) addresses key 16 ks + 8 rd + 4 h + a (nope row 16 ks + 2 rd + 4 a + h),
    // columns 32 ct + 16 (G % 2) + 4 j .. + 3.
    const int k_off = wide_row(l32) * C::kNopeRow + 16 * h;
    int r_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r_off[i] = C::kRopeBase + l32 * 128 + wide_rope_chunk(l32, 2 * i + h) * 16;
    const int v_off = (4 * ((lane >> 2) & 3) + h) * C::kNopeRow + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    auto k_operand = [&](const uint8_t* stage, int s) -> bf16x8_t {
        const uint8_t* src = s < 32 ? stage + k_off + 32 * s : stage + r_off[s - 32];
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(src));
    };
    auto v_operand = [&](const uint8_t* stage, int m) -> bf16x8_t {   // m = 16 ks + ct
        const int ks = m >> 4, ct = m & 15;
        const uint8_t* base = stage + v_off + (16 * ks) * C::kNopeRow + 64 * ct;
        const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(base));
        const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(base + 2 * C::kNopeRow));
        return __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
    };

    RowState st;
    f32x16 oacc[16];
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16{};

    // Prologue: tiles 0..2 issued, tile 0 in LDS, S^T(0).
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u) feed(u);
    wait_tile<C::kDma>(min(ntiles - 1, kStages - 2));
    block_sync();
    f32x16 s_cur;
    {
        const uint8_t* stage = smem;
        s_cur = f32x16{};
#pragma unroll
        for (int s = 0; s < 36; ++s)
            s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(stage, s), qf[s], s_cur, 0, 0, 0);
    }

    for (int t = 0; t < ntiles; ++t) {
        // Row max of tile t (scaled, log2 units): full tiles keep the raw entries; the last
        // tile of a range scales them and sets keys past the range (and all keys of heads
        // past num_q_heads) to -inf.  Entry i of a lane is key 8 (i / 4) + 4 h + i % 4.
        const int kb = k_begin + t * kKeys;
        const bool full = kb + kKeys <= k_end;
        float tmax;
        if (full) {
            tmax = s_cur[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, s_cur[i]);
            tmax *= p.scale_log2;
        } else {
            tmax = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb + 8 * (i >> 2) + 4 * h + (i & 3);
                s_cur[i] = (valid && key < k_end) ? s_cur[i] * p.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, s_cur[i]);
            }
        }
        tmax = max_xor32(tmax);
        const bool grow = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
        if (__any(grow)) {
            const float mnew = grow ? tmax : st.m;
            const float alpha = !grow ? 1.0f : (st.m == -INFINITY ? 0.0f : fast_exp2(st.m - mnew));
            st.l *= alpha;
            // O^T is still 0 in lanes that have seen no key yet: only a grown finite max
            // needs the products scaled (rare after the first tile).
            if (__any(grow && st.m != -INFINITY)) {
                wait_mfma_result();
                float tmp;
                asm volatile(PKV_RS_ALL "s_nop 4"
                             : "+a"(oacc[0]), "+a"(oacc[1]), "+a"(oacc[2]), "+a"(oacc[3]),
                               "+a"(oacc[4]), "+a"(oacc[5]), "+a"(oacc[6]), "+a"(oacc[7]),
                               "+a"(oacc[8]), "+a"(oacc[9]), "+a"(oacc[10]), "+a"(oacc[11]),
                               "+a"(oacc[12]), "+a"(oacc[13]), "+a"(oacc[14]), "+a"(oacc[15]),
                               "=&v"(tmp)
                             : "v"(alpha));
            }
            st.m = mnew;
        }
        // Tile t + 3 goes into the stage of tile t - 1 once the barrier has freed it; the
        // loads of a fast tile are spread over the value products below (one per product),
        // others are issued here at once.
        const int u = t + kStages - 1;
        bool spread = false;
        uint64_t slot_u = 0;
        if (t + 1 < ntiles) {
            wait_tile<C::kDma>(min(ntiles - 2 - t, kStages - 3));
            block_sync();
            if (u < ntiles) {
                const int c = u / kChunkTiles;
                if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load(c + 1, treg);
                if (u % kChunkTiles == kChunkTiles / 2 && tab.exists(c + 1)) tab.store(c + 1, treg);
                if (fast_tile(u)) {
                    const int32_t entry = next_entry;
                    if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
                    const int32_t blk = min(max(entry, 0), tab.last_block);
                    slot_u = ((uint64_t)(uint32_t)blk << p.bs_log2) | (uint32_t)((k_begin + u * kKeys + 8 * wid_u) & bs_mask);
                    spread = true;
                } else {
                    issue_tile(u);
                }
            }
        }
        uint8_t* ustage = smem + (u % kStages) * C::kStage;
        // S^T(t + 1) (on a stage no load writes any more when t + 1 = ntiles: a throw-away
        // result that keeps this region straight-line), interleaved step by step with the
        // exponentials of P^T(t); each step a scheduling region of its own.
        const uint8_t* kst = smem + ((t + 1) % kStages) * C::kStage;
        const float sc = full ? p.scale_log2 : 1.0f;
        const float mneg = st.m == -INFINITY ? 0.0f : -st.m;
        bf16x8_t kring[C::kKRing];
#pragma unroll
        for (int s = 0; s < C::kKRing; ++s) kring[s] = k_operand(kst, s);
        __builtin_amdgcn_sched_barrier(0);
        // two accumulation chains (even and odd k-steps), so that consecutive products do
        // not wait for each other's result
        f32x16 s_ev = f32x16{}, s_od = f32x16{};
        u32x4 pw[2];
#pragma unroll
        for (int s = 0; s < 36; ++s) {
            const bf16x8_t ka = kring[s % C::kKRing];
            if (s + C::kKRing < 36) kring[s % C::kKRing] = k_operand(kst, s + C::kKRing);
            if (s & 1) s_od = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s_od, 0, 0, 0);
            else s_ev = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s_ev, 0, 0, 0);
            if (s < 8) {   // exponential pair s of P^T(t)
                const int i = 2 * s;
                const float e0 = fast_exp2(__builtin_fmaf(s_cur[i], sc, mneg));
                const float e1 = fast_exp2(__builtin_fmaf(s_cur[i + 1], sc, mneg));
                st.l += e0 + e1;
                pw[i >> 3][(i & 7) >> 1] = pack_bf16(e0, e1);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // O^T += V^T . P^T(t): 32 products, the transposing reads kVRing products ahead.
        const uint8_t* vst = smem + (t % kStages) * C::kStage;
        bf16x8_t vring[C::kVRing];
#pragma unroll
        for (int m = 0; m < C::kVRing; ++m) vring[m] = v_operand(vst, m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const bf16x8_t va = vring[m % C::kVRing];
            if (m + C::kVRing < 32) vring[m % C::kVRing] = v_operand(vst, m + C::kVRing);
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw[m >> 4]);
            // s_nop 2: its operands may have just been written by VALU instructions
            asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(oacc[m & 15]) : "v"(va), "v"(pb));
            if (spread && m < 8)
                lds_dma16_s(nope_g + (slot_u + m) * 1024u, (uint32_t)lane * 16u,
                            ustage + wide_row(8 * wid_u + m) * C::kNopeRow);
            if (spread && m == 8)
                lds_dma16_s(rope_g + slot_u * 128u, rope_voff, ustage + C::kRopeBase + wid_u * 1024);
            __builtin_amdgcn_sched_barrier(0);
        }
        s_cur = s_ev + s_od;
    }

    // ---------------------------------------------------------------- epilogue
    wait_mfma_result();   // the last value products, before O^T is read
    float l_tot = st.l + __shfl_xor(st.l, 32, 64);   // the two key halves of each head
    const int nsplit = (L + p.split_tokens - 1) / p.split_tokens;
    if (valid) {
        // Accumulator entry i of tile ct: value column 32 ct + 8 (i / 4) + 4 h + i % 4.  One
        // store path for both cases (the normalized bf16 row, or the split's fp32 partial
        // state), one tile at a time: with two separate paths, or left free, the compiler
        // moves every AGPR into VGPRs first and spills.
        const bool single = nsplit == 1;
        const float inv = single ? (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) : 1.0f;
        const int64_t ps = row * p.max_splits + split;
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + row * 512 + 4 * h;
        float* ow = p.ws_o + (single ? 0 : ps * 512) + 4 * h;
#pragma unroll
        for (int ct = 0; ct < 16; ++ct) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 x = f32x4{oacc[ct][4 * q], oacc[ct][4 * q + 1], oacc[ct][4 * q + 2], oacc[ct][4 * q + 3]} * inv;
                if (single) {
                    const uint32_t w0 = bf16_bits(x[0]) | ((uint32_t)bf16_bits(x[1]) << 16);
                    const uint32_t w1 = bf16_bits(x[2]) | ((uint32_t)bf16_bits(x[3]) << 16);
                    *reinterpret_cast<uint2*>(out + 32 * ct + 8 * q) = make_uint2(w0, w1);
                } else {
                    *reinterpret_cast<f32x4*>(ow + 32 * ct + 8 * q) = x;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (h == 0) {
            if (single) {
                if (p.lse) p.lse[row] = l_tot > 0.0f ? (st.m + __log2f(l_tot)) * kLn2f : -INFINITY;
            } else {
                p.ws_ml[ps * 2] = st.m;
                p.ws_ml[ps * 2 + 1] = l_tot;
            }
        }
    }
}

}  // namespace

int32_t mla_wide_head_groups(int32_t num_q_heads) {
    return (num_q_heads + WideCfg::kHeads - 1) / WideCfg::kHeads;
}

hipError_t launch_mla_wide(const MfmaParams& p, hipStream_t s) {
    // ids: (unit / 8, head group, unit % 8) with units = batch * max_splits rounded up to 8
    const int64_t hgs = mla_wide_head_groups(p.hq);
    const int64_t units = ((int64_t)p.batch * p.max_splits + 7) / 8 * 8;
    const dim3 grid((unsigned)(hgs * units));
    if (p.k_new) hipLaunchKernelGGL((mla_wide_kernel<true>), grid, dim3(WideCfg::kThreads), 0, s, p);
    else hipLaunchKernelGGL((mla_wide_kernel<false>), grid, dim3(WideCfg::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
