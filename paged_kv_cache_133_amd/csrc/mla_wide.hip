// MLA-absorbed decode over the paged cache, one workgroup per (sequence, split) for all
// 128 query heads ("KVCache Optimization Skill", Mode 3: key = cache_nope || cache_rope,
// value = cache_nope, one latent head shared by every query head): each K/V tile goes
// from HBM into LDS once and serves every head.
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
// bf16 stage of a tile: 32 nope rows of 1024 bytes padded to 1040, key k in row
// (k & 16) | 4 (k & 3) | ((k >> 2) & 3), so that the 16 lanes of a K read hit 16 different
// bank groups and the four rows of a transposing read (keys 4 h + a, a = 0..3, of a
// 16-key group) sit 16 banks apart; then 32 rope rows of 128 bytes (key k in row k), their
// 16-byte chunks XOR-swizzled by row.
//  * bf16 cache: four stages, filled straight from HBM (the tile pipeline of mfma_common.h);
//  * INT8 cache (codes with one fp32 scale per key for the nope part and one for the rope
//    part): the codes reach one of two code stages by direct loads three tiles ahead; each
//    wave converts the keys it loaded itself into one of three bf16 stages (the codes
//    exactly, the scales beside them) one tile ahead, just before the tile's one barrier,
//    which publishes them.  A key's score weighs the nope and rope sums by
//    their own scales, s = s_nope (q . nope) + s_rope (q . rope), in one accumulator: the
//    nope products, times s_nope / s_rope', then the rope products added, times s_rope'
//    (s_rope' = s_rope, raised to s_nope 2^-60 and to 2^-126 where it is smaller: the ratio
//    stays finite, and the rope term moves by at most 2^-60 of the nope scale); the nope
//    scale goes into the value weight (P' = bf16(p s_nope)) while l adds p.
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

// INT8 LDS: two code stages (32 nope rows of 512 codes, then per wave 1 KiB: its 8 rope
// rows of 64 codes, its 8 nope and 8 rope scales), three bf16 stages each followed by three
// per-key factors of the tile (s_nope, s_nope / s_rope', s_rope'), the table.
struct WideI8Cfg {
    static constexpr int kCodeStages = 2;
    static constexpr int kNopeCodes = kKeys * 512;
    static constexpr int kAux = 1024;
    static constexpr int kCodeStage = kNopeCodes + WideCfg::kWaves * kAux;
    static constexpr int kBufs = 3;
    static constexpr int kBuf = WideCfg::kStage + 3 * kKeys * 4;
    static constexpr int kBufOff = kCodeStages * kCodeStage;
    static constexpr int kTabOff = kBufOff + kBufs * kBuf;
    static constexpr int kSmem = kTabOff + 2 * kTabEntries * 4;
    static constexpr int kDma = 5;                          // wave loads per tile: 4 nope + 1 rope and scales
    static_assert(kSmem <= 160 * 1024, "LDS");
    static_assert(kBuf % 16 == 0 && kCodeStage % 16 == 0, "alignment");
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

// One latent row quantized as the INT8 writer does it: s = max|x| / 127, q = round half to
// even of x / s clamped to [-127, 127] (fp32 divisions; a zero row has s = 0 and zero codes).
// G lanes hold 8 bf16 values each (src: 16 bytes); lanes that `store` write their 8 codes at
// dst and lane 0 the scale.  The max is exact in any order, so the codes and the scale equal
// the writer's bit for bit.
template <int G>
__device__ __forceinline__ void quant_row8(const uint8_t* src, uint8_t* dst, float* scale, int lane,
                                           bool store) {
    const u32x4 v = ld16(src);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(v[i]); x[2 * i + 1] = bf16_hi(v[i]); }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int sft = 1; sft < G; sft <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sft, 64));
    const float sc = __fdiv_rn(amax, 127.0f);
    uint32_t w[2] = {0u, 0u};
    if (sc > 0.0f) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float qf = fminf(fmaxf(rintf(__fdiv_rn(x[i], sc)), -127.0f), 127.0f);
            w[i >> 2] |= ((uint32_t)(int)qf & 0xffu) << (8 * (i & 3));
        }
    }
    if (store) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
        if (lane == 0) *scale = sc;
    }
}

// Cycles for an MFMA result written by inline assembly to be readable by anything else.
__device__ __forceinline__ void wait_mfma_result() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// APPEND: the key at seq_lens[b] - 1 is the step's new latent row.  bf16: read from
// p.k_new / p.rope_new instead of the cache; the split that holds it also stores it at its
// slot (reported in slots_out).  INT8: every workgroup of the split that holds it quantizes
// the row as the writer does (the same codes and scales, bit for bit; the workgroups of
// other head groups store the same bytes) and stores it before its first load, which then
// reads it back like any cached key.  A row longer than the length bound writes nothing
// (slot -1) and attends to its first len_cap cached keys.
// I8: p.k_cache / p.k_rope hold int8 codes, p.k_scale / p.r_scale their scales [nb][bs].
template <bool APPEND, bool I8>
__global__ __launch_bounds__(WideCfg::kThreads) void mla_wide_kernel(MfmaParams p) {
    using C = WideCfg;
    using W8 = WideI8Cfg;
    constexpr int kTabOff = I8 ? W8::kTabOff : C::kTabOff;
    __shared__ __attribute__((aligned(16))) uint8_t smem[I8 ? W8::kSmem : C::kSmem];

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
                                    reinterpret_cast<int32_t*>(smem + kTabOff), b, split))
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
    if (APPEND && I8 && new_key >= k_begin && new_key < k_end && wid < 2) {
        const int32_t phys = min(max(p.table[(int64_t)b * p.mbs + (new_key >> p.bs_log2)], 0),
                                 (int32_t)(p.num_blocks - 1));
        const int64_t slot = ((int64_t)phys << p.bs_log2) | (new_key & ((1 << p.bs_log2) - 1));
        if (wid == 0) {        // nope: 8 values per lane
            quant_row8<64>(reinterpret_cast<const uint8_t*>(p.k_new) + (int64_t)b * 1024 + lane * 16,
                           reinterpret_cast<uint8_t*>(p.k_cache_w) + slot * 512 + lane * 8,
                           p.k_scale_w + slot, lane, true);
            if (hg == 0 && p.slots_out && lane == 0) p.slots_out[b] = slot;
        } else {               // rope: lanes 0-7, 8 values each
            const int l8 = lane & 7;
            quant_row8<8>(reinterpret_cast<const uint8_t*>(p.rope_new) + (int64_t)b * 128 + l8 * 16,
                          reinterpret_cast<uint8_t*>(p.rope_w) + slot * 64 + l8 * 8,
                          p.r_scale_w + slot, l8, lane < 8);
        }
        // the stores complete before the loads below (the wait and barrier after the first
        // table chunk's load cover them)
    }
    if (APPEND && !I8 && hg == 0 && new_key >= k_begin && new_key < k_end && wid < 2) {
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
    tab.lds = reinterpret_cast<int32_t*>(smem + kTabOff);
    tab.row = p.table + (int64_t)b * p.mbs;
    tab.k_begin = k_begin;
    tab.k_end = k_end;
    tab.bs_log2 = p.bs_log2;
    tab.tid = tid;
    tab.last_block = (int32_t)(p.num_blocks - 1);
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);
    tab.load_lds(0, wid_u);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_sync();

    // The bf16 stage of tile t (what the products read).  INT8: the offset (t % 3 stages)
    // is put in a scalar register explicitly; left to itself the compiler spent vector
    // registers on it and spilled.
    auto stage_of = [&](int t) -> uint8_t* {
        if constexpr (I8) return smem + __builtin_amdgcn_readfirstlane(W8::kBufOff + (t % W8::kBufs) * W8::kBuf);
        else return smem + (t % kStages) * C::kStage;
    };
    auto code_stage = [&](int u) -> uint8_t* {
        return smem + __builtin_amdgcn_readfirstlane((u % W8::kCodeStages) * W8::kCodeStage);
    };

    // Loads of one tile.  bf16: wave w fills the nope rows of keys 8 w .. 8 w + 7 (one load
    // per row, lane = 16-byte chunk) and their rope rows (one load: lane = row 8 w + lane / 8,
    // physical chunk lane % 8).  INT8: wave w loads the codes of keys 8 w .. 8 w + 7 into
    // code stage u % 2: their nope rows (4 loads of two rows) and one load whose lanes 0-31
    // take the 8 rope rows, 32-33 the 8 nope scales and 34-35 the 8 rope scales (a block's
    // scales are in slot order, and an aligned group of 4 keys lies in one block); the
    // other lanes re-read lane 32's bytes.
    const int bs_mask = (1 << p.bs_log2) - 1;
    const uint8_t* nope_g = reinterpret_cast<const uint8_t*>(p.k_cache);
    const uint8_t* rope_g = reinterpret_cast<const uint8_t*>(p.k_rope);
    const uint8_t* nsc_g = reinterpret_cast<const uint8_t*>(p.k_scale);
    const uint8_t* rsc_g = reinterpret_cast<const uint8_t*>(p.r_scale);
    const int rope_r = 8 * wid_u + (lane >> 3);
    const int rope_c = wide_rope_chunk(rope_r, lane & 7);
    const uint32_t rope_voff = (uint32_t)((lane >> 3) * 128 + rope_c * 16);
    // Full tiles with blocks of at least 8 keys: the wave's 8 keys are consecutive slots of
    // one block, found with one scalar read of the block table (one tile ahead).
    const bool fast_rows = p.bs_log2 >= 3;
    auto fast_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        return fast_rows && kb + kKeys <= k_end && !(APPEND && !I8 && new_key >= kb && new_key < kb + kKeys);
    };
    auto entry_of = [&](int u) { return uniform_load(tab.row + ((k_begin + u * kKeys + 8 * wid_u) >> p.bs_log2)); };
    int32_t next_entry = fast_tile(0) ? entry_of(0) : 0;
    // INT8, fast tile: load j (< 4: nope rows 8 w + 2 j and 8 w + 2 j + 1; 4: rope rows and
    // scales) from the wave's first slot.
    auto code_load = [&](int u, uint64_t slot0, int j) {
        uint8_t* cs = code_stage(u);
        if (j < 4) {
            lds_dma16_s(nope_g + slot0 * 512u + j * 1024, (uint32_t)lane * 16u, cs + (8 * wid_u + 2 * j) * 512);
        } else {
            const int ln = opaque(lane), q = ln >= 32 && ln < 36 ? ln - 32 : 0;
            const uint8_t* src = ln < 32 ? rope_g + (slot0 * 64u + (uint32_t)(ln * 16))
                                         : ((q & 2) ? rsc_g : nsc_g) + (slot0 * 4u + (uint32_t)((q & 1) * 16));
            lds_dma16(src, cs + W8::kNopeCodes + wid_u * W8::kAux);
        }
    };
    auto issue_tile = [&](int u) {
        const int kb = k_begin + u * kKeys;
        const int chunk = u / kChunkTiles;
        const int32_t entry = next_entry;
        if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
        if (fast_tile(u)) {
            const int key0 = kb + 8 * wid_u;
            const int32_t blk = min(max(entry, 0), tab.last_block);
            const uint64_t slot0 = ((uint64_t)(uint32_t)blk << p.bs_log2) | (uint32_t)(key0 & bs_mask);
            if constexpr (I8) {
#pragma unroll
                for (int j = 0; j < 5; ++j) code_load(u, slot0, j);
            } else {
                uint8_t* stage = stage_of(u);
                const uint8_t* nb = nope_g + slot0 * 1024u;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    lds_dma16_s(nb + j * 1024, (uint32_t)lane * 16u, stage + wide_row(8 * wid_u + j) * C::kNopeRow);
                lds_dma16_s(rope_g + slot0 * 128u, rope_voff, stage + C::kRopeBase + wid_u * 1024);
            }
            return;
        }
        const int ln = opaque(lane);   // per-lane addresses are computed here, not hoisted
        if constexpr (I8) {
            // keys past the range: their rows and scales come from the last key (its 4-key
            // group for the scales); the conversion gives them scale 0
            uint8_t* cs = code_stage(u);
            const int q = ln >= 32 && ln < 36 ? ln - 32 : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = min(kb + 8 * wid_u + 2 * j + (ln >> 5), k_end - 1);
                const uint64_t slot = ((uint64_t)tab.block_of(key, chunk) << p.bs_log2) | (uint32_t)(key & bs_mask);
                lds_dma16(nope_g + (slot * 512u + (uint32_t)((ln & 31) * 16)), cs + (8 * wid_u + 2 * j) * 512);
            }
            const int key = ln < 32 ? min(kb + 8 * wid_u + (ln >> 2), k_end - 1)
                                    : min(kb + 8 * wid_u + 4 * (q & 1), (k_end - 1) & ~3);
            const uint64_t slot = ((uint64_t)tab.block_of(key, chunk) << p.bs_log2) | (uint32_t)(key & bs_mask);
            lds_dma16(ln < 32 ? rope_g + (slot * 64u + (uint32_t)((ln & 3) * 16)) : ((q & 2) ? rsc_g : nsc_g) + slot * 4u,
                      cs + W8::kNopeCodes + wid_u * W8::kAux);
        } else {
            uint8_t* stage = stage_of(u);
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
        }
    };
    // The next table chunk (as the loads of a chunk's first tile are issued; it is used 32
    // tiles later) and the loads of tile u.
    auto next_chunk = [&](int u) {
        const int c = u / kChunkTiles;
        if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load_lds(c + 1, wid_u);
    };
    auto feed = [&](int u) {
        if (u >= ntiles) return;
        next_chunk(u);
        issue_tile(u);
    };

    // INT8 conversion of this wave's keys of tile u (code stage u % 2 -> bf16 stage u % 3),
    // in ten pieces of one LDS read and one write: piece j < 8 is the nope row of key
    // 8 w + j (lane = 8 codes), 8 the rope rows (lane = row 8 w + lane / 8, 8 codes), 9 the
    // factors of the 8 keys (lanes 0-7; keys past the range get s_nope = 0, so that no
    // stale scale reaches a weight, and a finite score).  The wave reads only what it
    // loaded itself, so its own load counter is the only wait.
    auto conv_read = [&](int u, int j) -> u32x2 {
        const uint8_t* cs = code_stage(u);
        const uint8_t* aux = cs + W8::kNopeCodes + wid_u * W8::kAux;
        if (j < 8) return *reinterpret_cast<const u32x2*>(cs + (8 * wid_u + j) * 512 + lane * 8);
        const int ln = opaque(lane);   // (pieces 8 and 9: addresses computed here, not hoisted)
        if (j == 8) return *reinterpret_cast<const u32x2*>(aux + ln * 8);
        const uint32_t* sc = reinterpret_cast<const uint32_t*>(aux + 512) + (ln & 7);
        return u32x2{sc[0], sc[8]};
    };
    // wide_row(8 w + j) = wide_row(8 w) + 4 (j % 4) + j / 4 (disjoint bit fields)
    const int conv_nope = wide_row(8 * wid_u) * C::kNopeRow + lane * 16;
    auto conv_write = [&](int u, int j, u32x2 c) {
        uint8_t* bf = stage_of(u);
        if (j < 8) {
            *reinterpret_cast<u32x4*>(bf + conv_nope + (4 * (j & 3) + (j >> 2)) * C::kNopeRow) = codes8_to_bf16(c[0], c[1]);
        } else if (j == 8) {
            const int ln = opaque(lane);
            const int r = 8 * wid_u + (ln >> 3);
            *reinterpret_cast<u32x4*>(bf + C::kRopeBase + r * 128 + wide_rope_chunk(r, ln & 7) * 16) =
                codes8_to_bf16(c[0], c[1]);
        } else if (lane < 8) {
            const int key = 8 * wid_u + opaque(lane);
            const bool in = k_begin + u * kKeys + key < k_end;
            const float sn = in ? __uint_as_float(c[0]) : 0.0f;
            const float srp = fmaxf(fmaxf(in ? __uint_as_float(c[1]) : 0.0f, sn * 0x1p-60f), 0x1p-126f);
            float* f = reinterpret_cast<float*>(bf + C::kStage) + key;
            f[0] = sn;
            f[kKeys] = sn / srp;
            f[2 * kKeys] = srp;
        }
    };

    // All reads first: a store to the bf16 stage may alias a later read as far as the
    // compiler knows, so interleaved, every read would wait out the one before it.
    auto convert = [&](int u) {
        u32x2 c[10];
#pragma unroll
        for (int j = 0; j < 10; ++j) c[j] = conv_read(u, j);
#pragma unroll
        for (int j = 0; j < 10; ++j) conv_write(u, j, c[j]);
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
    // INT8: factor n (0: s_nope, 1: s_nope / s_rope', 2: s_rope') of this lane's keys
    // 8 q + 4 h .. + 3.
    auto scales4 = [&](const uint8_t* stage, int n, int q) -> f32x4 {
        return *reinterpret_cast<const f32x4*>(stage + C::kStage + (n * kKeys + 8 * q + 4 * h) * 4);
    };

    RowState st;
    f32x16 oacc[16];
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) oacc[ct] = f32x16{};

    // Prologue.  bf16: tiles 0..2 issued, tile 0 in LDS.  INT8: tiles 0..2 issued, tile 0
    // converted (tile 2 into its code stage once read).  Then S^T(0).
    if constexpr (I8) {
        feed(0);
        feed(1);
        if (ntiles > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(W8::kDma));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        convert(0);
        feed(2);
    } else {
#pragma unroll
        for (int u = 0; u < kStages - 1; ++u) feed(u);
        wait_tile<C::kDma>(min(ntiles - 1, kStages - 2));
    }
    block_sync();
    f32x16 s_cur;
    {
        const uint8_t* stage = stage_of(0);
        s_cur = f32x16{};
#pragma unroll
        for (int s = 0; s < (I8 ? 32 : 36); ++s)
            s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(stage, s), qf[s], s_cur, 0, 0, 0);
        if constexpr (I8) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 r = scales4(stage, 1, q);
#pragma unroll
                for (int e = 0; e < 4; ++e) s_cur[4 * q + e] *= r[e];
            }
#pragma unroll
            for (int s = 32; s < 36; ++s)
                s_cur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(stage, s), qf[s], s_cur, 0, 0, 0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 r = scales4(stage, 2, q);
#pragma unroll
                for (int e = 0; e < 4; ++e) s_cur[4 * q + e] *= r[e];
            }
        }
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
        // Tile t + 3 goes into the stage of tile t - 1 (INT8: the code stage of tile t + 1,
        // converted just before) once the barrier has freed it; the loads of a fast tile are
        // spread over the products below (one per product), others are issued here at once.
        // INT8: this wave converts its keys of tile t + 1 into bf16 stage (t + 1) % 3 here,
        // where no operand reads compete for LDS (among the products, the conversion's
        // stores cost three times as much), and the barrier publishes it; the wait lets the
        // codes of tile t + 2, and a table chunk issued after them, stay in flight.
        const int u = t + 3;
        bool spread = false;
        uint64_t slot_u = 0;
        if (t + 1 < ntiles) {
            if constexpr (I8) {
                const int v = t + 2;
                if (v >= ntiles) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
                else if (v % kChunkTiles == 0 && tab.exists(v / kChunkTiles + 1))
                    __builtin_amdgcn_s_waitcnt(waitcnt_vm(W8::kDma + 4));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(W8::kDma));
                convert(t + 1);
            } else {
                wait_tile<C::kDma>(min(ntiles - 2 - t, kStages - 3));
            }
            block_sync();
            if (u < ntiles) {
                if constexpr (!I8) next_chunk(u);
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
        // S^T(t + 1) (on a stage no load writes any more when t + 1 = ntiles: a throw-away
        // result that keeps this region straight-line), interleaved step by step with the
        // exponentials of P^T(t); each step a scheduling region of its own.
        const uint8_t* kst = stage_of(t + 1);
        const uint8_t* vst = stage_of(t);
        const float sc = full ? p.scale_log2 : 1.0f;
        const float mneg = st.m == -INFINITY ? 0.0f : -st.m;
        bf16x8_t kring[C::kKRing];
#pragma unroll
        for (int s = 0; s < C::kKRing; ++s) kring[s] = k_operand(kst, s);
        f32x4 vsc;   // INT8: the nope scales of tile t (the value weights) of 4 keys
        if constexpr (I8) vsc = scales4(vst, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        // bf16: two accumulation chains (even and odd k-steps), so that consecutive products
        // do not wait for each other's result.  INT8: the 32 nope k-steps in one chain here;
        // its rope k-steps follow among the value products.
        constexpr int kSteps = I8 ? 32 : 36;
        f32x16 s_ev = f32x16{}, s_od = f32x16{};
        u32x4 pw[2];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            const bf16x8_t ka = kring[s % C::kKRing];
            if (s + C::kKRing < kSteps) kring[s % C::kKRing] = k_operand(kst, s + C::kKRing);
            if (!I8 && (s & 1)) s_od = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s_od, 0, 0, 0);
            else s_ev = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], s_ev, 0, 0, 0);
            if (s < 8) {   // exponential pair s of P^T(t)
                const int i = 2 * s;
                const float e0 = fast_exp2(__builtin_fmaf(s_cur[i], sc, mneg));
                const float e1 = fast_exp2(__builtin_fmaf(s_cur[i + 1], sc, mneg));
                st.l += e0 + e1;
                if constexpr (I8) {
                    pw[i >> 3][(i & 7) >> 1] = pack_bf16(e0 * vsc[i & 3], e1 * vsc[(i & 3) + 1]);
                    if (s % 2 == 1 && s < 7) vsc = scales4(vst, 0, s / 2 + 1);
                } else {
                    pw[i >> 3][(i & 7) >> 1] = pack_bf16(e0, e1);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // O^T += V^T . P^T(t): 32 products, the transposing reads kVRing products ahead.
        // INT8, among them: the scores of tile t + 1 completed (products 0-14: the nope sums
        // times s_nope / s_rope', the four rope products, times s_rope').
        bf16x8_t vring[C::kVRing];
#pragma unroll
        for (int m = 0; m < C::kVRing; ++m) vring[m] = v_operand(vst, m);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 ksc[2];
        bf16x8_t rk[2];
#pragma unroll
        for (int m = 0; m < 32; ++m) {
            const bf16x8_t va = vring[m % C::kVRing];
            if (m + C::kVRing < 32) vring[m % C::kVRing] = v_operand(vst, m + C::kVRing);
            const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw[m >> 4]);
            // s_nop 2: its operands may have just been written by VALU instructions
            asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(oacc[m & 15]) : "v"(va), "v"(pb));
            if constexpr (I8) {
                if (m < 16) {
                    // the nope sums times s_nope / s_rope' (products 1-2), the rope products
                    // (3, 5, 7, 9), times s_rope' (12, 14); factors of 8 keys, two operands
                    // in flight
                    if (m == 1 || m == 2 || m == 12 || m == 14) {
                        const int i0 = m == 1 || m == 12 ? 0 : 8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) s_ev[i0 + e] *= ksc[e >> 2][e & 3];
                    }
                    if (m == 0 || m == 1 || m == 10 || m == 12) {
                        const int n = m < 10 ? 1 : 2, q = m == 0 || m == 10 ? 0 : 2;
                        ksc[0] = scales4(kst, n, q);
                        ksc[1] = scales4(kst, n, q + 1);
                    }
                    if (m >= 3 && m <= 9 && (m & 1))
                        s_ev = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rk[((m - 3) >> 1) & 1], qf[32 + ((m - 3) >> 1)], s_ev, 0, 0, 0);
                    if (m == 1 || m == 2 || m == 3 || m == 5) {
                        const int i = m <= 2 ? m - 1 : (m - 3) / 2 + 2;   // rope k-step 32 + i
                        rk[i & 1] = k_operand(kst, 32 + i);
                    }
                }
                // the codes of tile t + 3 (products 16-20), then a table chunk (21)
                if (spread && m >= 16 && m < 21) code_load(u, slot_u, m - 16);
                if (m == 21 && u < ntiles) next_chunk(u);
            } else {
                uint8_t* ustage = stage_of(u);
                if (spread && m < 8)
                    lds_dma16_s(nope_g + (slot_u + m) * 1024u, (uint32_t)lane * 16u,
                                ustage + wide_row(8 * wid_u + m) * C::kNopeRow);
                if (spread && m == 8)
                    lds_dma16_s(rope_g + slot_u * 128u, rope_voff, ustage + C::kRopeBase + wid_u * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (I8) s_cur = s_ev;
        else s_cur = s_ev + s_od;
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

int32_t mla_head_groups(int32_t num_q_heads) {
    return (num_q_heads + WideCfg::kHeads - 1) / WideCfg::kHeads;
}

DecodePlan plan_mla(int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t max_seq_len_kv) {
    DecodePlan pl{};
    const int64_t groups64 = (num_q_heads + 63) / 64;   // the scale the threshold below was set at
    auto nsplits = [&](int sp) { return (int64_t)(max_seq_len_kv + sp - 1) / sp; };
    // A split's partial state is Hq x Dv fp32 (256 KiB at 128 x 512): long splits keep that
    // traffic small; shorten them only while the grid would leave compute units idle.  With
    // one workgroup per CU the time also depends on how the units pack onto the CUs: on 64
    // sequences of 2K-8K keys (splits of a sequence evenly sized) a sweep of the bf16 kernel
    // measured 1536 best (131 us; 512: 165, 768: 151, 1024: 159, 2048: 146).
    int split = 1536;
    while (split > 256 && batch * groups64 * nsplits(split) < 512) split /= 2;
    pl.split_tokens = split;
    pl.max_splits = (int32_t)(max_seq_len_kv > 0 ? nsplits(split) : 1);
    if (pl.max_splits <= 1) return pl;
    const size_t rows = (size_t)batch * num_q_heads * pl.max_splits;
    pl.ws_o_offset = 0;
    pl.ws_ml_offset = (rows * head_dim_v * sizeof(float) + 255) & ~(size_t)255;
    pl.ws_bytes = pl.ws_ml_offset + rows * 2 * sizeof(float);
    return pl;
}

hipError_t launch_mla_decode(const MfmaParams& p, hipStream_t s) {
    // ids: (unit / 8, head group, unit % 8) with units = batch * max_splits rounded up to 8
    const int64_t hgs = mla_head_groups(p.hq);
    const int64_t units = ((int64_t)p.batch * p.max_splits + 7) / 8 * 8;
    const dim3 grid((unsigned)(hgs * units));
    if (p.k_scale && p.k_new) hipLaunchKernelGGL((mla_wide_kernel<true, true>), grid, dim3(WideCfg::kThreads), 0, s, p);
    else if (p.k_scale) hipLaunchKernelGGL((mla_wide_kernel<false, true>), grid, dim3(WideCfg::kThreads), 0, s, p);
    else if (p.k_new) hipLaunchKernelGGL((mla_wide_kernel<true, false>), grid, dim3(WideCfg::kThreads), 0, s, p);
    else hipLaunchKernelGGL((mla_wide_kernel<false, false>), grid, dim3(WideCfg::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
