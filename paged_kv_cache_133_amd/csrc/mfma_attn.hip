// MFMA attention over the paged cache for gfx950: the MLA-absorbed decode ("KVCache
// Optimization Skill", Mode 3: key = cache_nope || cache_rope, value = cache_nope,
// rope passed separately) and the packed varlen causal chunk ("Paged KV Cache and
// Packed Sequence", 3.1-3.3 and 4.1; skill page Appendix C/E, sparse_mode 3).
//
// Both are dense contractions: 128 query heads share one latent head (MLA), G query
// heads and up to thousands of query tokens share each kv head (varlen).  The layout:
//  * a workgroup owns groups of 32 query rows and walks one key range in tiles of 32
//    keys; each tile's K (and V) rows are gathered through the block table into LDS once
//    and read by all waves (two LDS buffers: the next tile's global loads are in flight
//    while the current tile is computed).  Varlen: four row groups, one wave each.  MLA:
//    two row groups (64 heads) of four waves; each wave does a quarter of the 576-wide
//    Q.K contraction (the four partial S are summed through LDS in a fixed order, so all
//    four waves hold bitwise the same S) and a quarter of the 512 output columns.  The two
//    head groups of one (sequence, split) are launched onto the same XCD so that the
//    second read of a K/V tile can come from that XCD's L2;
//  * S^T = K . Q^T with v_mfma_f32_32x32x16_bf16: K rows come from LDS as the A operand,
//    Q^T sits in registers as the B operand for the whole key range;
//  * in the S^T accumulator each lane holds 16 keys of one query row, so the row max and
//    sum need one cross-lane step, and P^T (bf16) is already in the B-operand layout of
//    the next product once keys are numbered the way the accumulator holds them.  Tiles
//    that every row of the workgroup sees whole skip the masking;
//  * O^T += V^T . P^T: the A operand (four consecutive keys at one value column per lane
//    and read) comes straight from the row-major V tile with ds_read_b64_tr_b16;
//  * O^T keeps one query row per lane as well, so the online-softmax rescale is
//    lane-local; it is applied only when a row's max grows by more than 2^8 (P <= 256 in
//    between), which after the first tiles almost never happens.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kSlotRing = 4;      // tiles whose slots are kept in LDS (current + 3 ahead)
constexpr float kLn2f = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;   // log2 units a row max may grow before rescaling
// s_waitcnt operand (gfx9 encoding) that waits for all vector-memory loads only:
// vmcnt = 0, expcnt = 7 and lgkmcnt = 15 (no wait on those).
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;   // bf16 pair (1, 1)

// MODE 0: MLA decode (K row = 512 nope + 64 rope, V = the nope part of the same row).
// MODE 1: varlen (K and V rows of one kv head, DQK = DV = D).
template <int MODE, int D>
struct MCfg {
    static constexpr int kGroups = MODE == 0 ? 2 : 4;      // row groups of 32 query rows
    static constexpr int kSplitD = MODE == 0 ? 4 : 1;      // waves per row group
    static constexpr int kRows = kGroups * 32;             // query rows per workgroup
    static constexpr int kWaves = kGroups * kSplitD;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kDqk = MODE == 0 ? 576 : D;
    static constexpr int kDv = MODE == 0 ? 512 : D;
    static constexpr int kKMain = MODE == 0 ? 512 : D;     // dims read from k_cache
    // LDS rows: MLA pads each 1152-byte row by 16 bytes; varlen rows are unpadded and
    // their 16-byte chunks are XOR-swizzled by row (see swz()), which keeps both the
    // 16-row column reads of K and the 4-row transposing reads of V free of bank conflicts.
    static constexpr bool kSwizzle = MODE != 0;
    static constexpr int kRowK = kDqk * 2 + (kSwizzle ? 0 : 16);   // LDS bytes per K row
    static constexpr int kRowV = MODE == 0 ? kRowK : kDv * 2;
    static constexpr int kRowChunks = kDqk * 2 / 16;                // 16-byte chunks per row
    static constexpr int kRowShift = kDqk * 2 >= 256 ? 0 : (kDqk * 2 == 128 ? 1 : 2);
    static constexpr int kKeys = 32;                        // keys per tile
    static constexpr int kTileK = kKeys * kRowK;
    static constexpr int kTileV = MODE == 0 ? 0 : kKeys * kRowV;
    static constexpr int kBuf = kTileK + kTileV;
    static constexpr int kChunkK = kDqk * 2 / 16;          // 16-byte chunks per key (K)
    static constexpr int kChunkV = MODE == 0 ? 0 : kDv * 2 / 16;
    static constexpr int kChunks = kChunkK + kChunkV;
    static constexpr int kTileChunks = kKeys * kChunks;
    static constexpr int kPerThread = (kTileChunks + kThreads - 1) / kThreads;
    static constexpr int kSteps = kDqk / 16 / kSplitD;     // k-steps of S^T per wave
    static constexpr int kMTiles = kDv / 32 / kSplitD;     // 32-row tiles of O^T per wave
    static constexpr int kSx = kSplitD > 1 ? kWaves * 16 * 64 * 4 : 0;   // S exchange bytes
    static constexpr int kSlotBytes = kSlotRing * kKeys * 4;
    static constexpr int kSmem = 2 * kBuf + kSx + kSlotBytes;
    static_assert(kSteps * 16 * kSplitD == kDqk && kMTiles * 32 * kSplitD == kDv, "split");
};

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Physical 16-byte chunk of logical chunk c in LDS row r (varlen tiles).  Rows sharing a
// 256-byte bank line (x = r >> shift) get distinct XOR patterns: 16 consecutive rows land
// on 16 different chunks, and any 4 consecutive rows map a chunk pair {2i, 2i+1} to 8
// different chunks.
template <int CPR, int SHIFT>
__device__ __forceinline__ int swz(int r, int c) {
    const int x = r >> SHIFT;
    return c ^ ((2 * (x & (CPR / 2 - 1))) ^ ((x / (CPR / 2)) & 1));
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint8_t* lds_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds_addr));
}

struct RowInfo {
    const uint8_t* q;        // start of the row's query (main part)
    const uint8_t* q_rope;   // MLA rope part
    int64_t out_row;         // output row index (row-major [rows][Dv])
    int vis;                 // last visible key position (inclusive)
    bool valid;
};

template <int MODE, int D>
__global__ __launch_bounds__((MCfg<MODE, D>::kThreads)) void mfma_attn_kernel(MfmaParams p) {
    using C = MCfg<MODE, D>;
    constexpr int kThreads = C::kThreads;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int wave = wid / C::kSplitD;      // row group
    const int dh = wid % C::kSplitD;        // half of the contraction / output columns
    const int lane = tid & 63;
    const int lrow = lane & 31;        // query row of this lane inside the wave
    const int lhalf = lane >> 5;       // which half of the k-slots / keys

    // ---------------------------------------------------------------- work item
    int b, kvh = 0, split = 0, k_begin, k_end;
    RowInfo ri;
    int nrows_any;
    int L;
    if constexpr (MODE == 0) {
        // Workgroups are dealt to the 8 XCDs round-robin; the head groups of one work unit
        // take ids that differ by a multiple of 8 and follow each other on one XCD.
        const int hgs = (p.hq + C::kRows - 1) / C::kRows;
        const int id = blockIdx.x;
        const int xcd = id & 7;
        const int slot = id >> 3;
        const int hg = slot % hgs;
        const int unit = (slot / hgs) * 8 + xcd;
        b = unit % p.batch;
        split = unit / p.batch;
        if (split >= p.max_splits) return;
        L = min(p.seq_lens[b], p.len_cap);
        k_begin = split * p.split_tokens;
        if (k_begin >= L) return;
        k_end = min(L, k_begin + p.split_tokens);
        const int h = hg * C::kRows + wave * 32 + lrow;
        ri.valid = h < p.hq;
        const int hc = min(h, p.hq - 1);
        ri.q = reinterpret_cast<const uint8_t*>(p.q) + ((int64_t)b * p.hq + hc) * 512 * 2;
        ri.q_rope = reinterpret_cast<const uint8_t*>(p.q_rope) + ((int64_t)b * p.hq + hc) * 64 * 2;
        ri.out_row = (int64_t)b * p.hq + hc;
        ri.vis = L - 1;
        nrows_any = 1;
    } else {
        int id = blockIdx.x;
        kvh = id % p.hkv;
        id /= p.hkv;
        const int qb = id % p.q_blocks;
        b = id / p.q_blocks;
        const int G = p.group;
        const int tw = 32 / G;                         // query tokens per row group
        const int tpb = C::kGroups * tw;               // query tokens per workgroup
        const int q0 = p.cu_q[b];
        const int n = p.cu_q[b + 1] - q0;
        L = min(p.seq_lens[b], p.len_cap);
        const int i_first = qb * tpb;
        if (i_first >= n || n <= 0 || L <= 0) return;
        const int i_last = min(n, i_first + tpb) - 1;
        const int i = i_first + wave * tw + lrow / G;
        const int g = lrow % G;
        ri.valid = (lrow < tw * G) && (i < n);
        const int ic = ri.valid ? i : i_first;
        const int hq = kvh * G + (ri.valid ? g : 0);
        ri.q = reinterpret_cast<const uint8_t*>(p.q) + ((int64_t)(q0 + ic) * p.hq + hq) * D * 2;
        ri.q_rope = nullptr;
        ri.out_row = (int64_t)(q0 + ic) * p.hq + hq;
        ri.vis = p.causal ? (L - n + ic) : (L - 1);
        k_begin = 0;
        k_end = p.causal ? min(L, L - n + i_last + 1) : L;
        nrows_any = 1;
    }
    (void)nrows_any;
    const int ntiles = (k_end - k_begin + C::kKeys - 1) / C::kKeys;
    // Keys below full_end are visible to every row of the workgroup.
    int full_end = k_end;
    if constexpr (MODE == 1) {
        if (p.causal) {
            const int n = p.cu_q[b + 1] - p.cu_q[b];
            const int tpb = C::kGroups * (32 / p.group);
            full_end = min(k_end, L - n + (int)(blockIdx.x / p.hkv % p.q_blocks) * tpb + 1);
        }
    }

    // ---------------------------------------------------------------- Q^T fragments
    bf16x8_t qf[C::kSteps];
#pragma unroll
    for (int s = 0; s < C::kSteps; ++s) {
        const int dim = 16 * (s + dh * C::kSteps) + 8 * lhalf;
        const uint8_t* src;
        if (MODE == 0 && dim >= 512) src = ri.q_rope + (dim - 512) * 2;
        else src = ri.q + dim * 2;
        qf[s] = __builtin_bit_cast(bf16x8_t, ld16(src));
    }
    // Q must be resident before the loop: otherwise the wait for it, placed inside the
    // loop, also waits for the K/V loads issued there and serialises the pipeline.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---------------------------------------------------------------- tile pipeline
    // Slots of tile u (one per key, -1 past the range) are looked up two tiles ahead into
    // an LDS ring; the K/V rows of tile u are loaded into registers one tile ahead and
    // stored to one of two LDS buffers just before tile u is used.
    const int32_t* trow = p.table + (int64_t)b * p.mbs;
    const int bs_mask = (1 << p.bs_log2) - 1;
    const int32_t last_block = (int32_t)(p.num_blocks - 1);
    int32_t* ring = reinterpret_cast<int32_t*>(smem + 2 * C::kBuf + C::kSx);

    // The table entry of a key of tile u is fetched early and turned into a slot only
    // where it is stored (slot_of), so that its load overlaps the tile being computed.
    // Every lane loads an in-range entry (keys past the range are clamped to the last
    // one); threads < kKeys then publish the slot of key tid of tile u, -1 past the range.
    auto table_entry = [&](int u) -> int32_t {
        const int key = min(k_begin + u * C::kKeys + (tid & (C::kKeys - 1)), k_end - 1);
        return trow[key >> p.bs_log2];
    };
    auto slot_of = [&](int u, int32_t raw) -> int32_t {
        const int key = k_begin + u * C::kKeys + tid;
        if (tid >= C::kKeys || u >= ntiles || key >= k_end) return -1;
        const int32_t phys = min(max(raw, 0), last_block);
        return (phys << p.bs_log2) | (key & bs_mask);
    };

    // Chunk i of this thread (16 bytes) is the same piece of every tile: it lies at
    // src_base[i] + slot * src_stride[i] and lands at LDS offset dst_off[i] of a buffer.
    // Chunks past the tile (the last i, when the tile does not divide evenly) repeat a
    // chunk of the tile and are not stored.
    const uint8_t* src_base[C::kPerThread];
    uint32_t src_stride[C::kPerThread];
    int key_of[C::kPerThread];
    int dst_off[C::kPerThread];
#pragma unroll
    for (int i = 0; i < C::kPerThread; ++i) {
        const int c = (tid + kThreads * i) % C::kTileChunks;
        const int j = c / C::kChunks;
        const int part = c % C::kChunks;
        key_of[i] = j;
        if (part < C::kKMain * 2 / 16) {
            src_base[i] = reinterpret_cast<const uint8_t*>(p.k_cache) + kvh * C::kKMain * 2 + part * 16;
            src_stride[i] = (uint32_t)(p.hkv * C::kKMain * 2);
        } else if (MODE == 0) {
            src_base[i] = reinterpret_cast<const uint8_t*>(p.k_rope) + (part - C::kKMain * 2 / 16) * 16;
            src_stride[i] = (uint32_t)((C::kDqk - C::kKMain) * 2);
        } else {
            src_base[i] = reinterpret_cast<const uint8_t*>(p.v_cache) + kvh * C::kDv * 2 + (part - C::kChunkK) * 16;
            src_stride[i] = (uint32_t)(p.hkv * C::kDv * 2);
        }
        if constexpr (C::kSwizzle) {
            dst_off[i] = part < C::kChunkK
                             ? j * C::kRowK + swz<C::kRowChunks, C::kRowShift>(j, part) * 16
                             : C::kTileK + j * C::kRowV +
                                   swz<C::kRowChunks, C::kRowShift>(j, part - C::kChunkK) * 16;
        } else {
            dst_off[i] = part < C::kChunkK ? j * C::kRowK + part * 16
                                           : C::kTileK + j * C::kRowV + (part - C::kChunkK) * 16;
        }
    }
    // Every lane issues all of its loads: keys past the range read slot 0 (always
    // allocated) and are zeroed when stored, by the bits of 'live'.  Loads under a branch
    // would make every later wait a wait for all outstanding loads.
    auto load_tile = [&](int u, u32x4* st, uint32_t& live) {
        const int32_t* slots = ring + (u % kSlotRing) * C::kKeys;
        int32_t sv[C::kPerThread];
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) sv[i] = slots[key_of[i]];
        live = 0;
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) {
            live |= (sv[i] >= 0 ? 1u : 0u) << i;
            const uint64_t off = (uint64_t)(uint32_t)max(sv[i], 0) * src_stride[i];
            st[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src_base[i] + off));
        }
    };
    auto store_tile = [&](uint8_t* buf, const u32x4* st, uint32_t live) {
#pragma unroll
        for (int i = 0; i < C::kPerThread; ++i) {
            if (tid + kThreads * i >= C::kTileChunks) break;
            const u32x4 z{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(buf + dst_off[i]) = ((live >> i) & 1u) ? st[i] : z;
        }
    };

    // ---------------------------------------------------------------- running state
    float m_run = -INFINITY;      // per row (log2 units), equal in lanes l and l ^ 32
    float l_run = 0.0f;           // this lane's partial sum (its half of each 32-key block)
    f32x16 oacc[C::kMTiles];
#pragma unroll
    for (int mt = 0; mt < C::kMTiles; ++mt) oacc[mt] = f32x16{};

    // One tile: S^T, softmax update, P^T, O^T += V^T P^T.
    auto compute_tile = [&](int t) {
        const int kb = k_begin + t * C::kKeys;
        const uint8_t* buf = smem + (t & 1) * C::kBuf;
        f32x16 sacc = f32x16{};
        const uint8_t* kread = buf + lrow * C::kRowK;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
            const int chunk = 2 * (s + dh * C::kSteps) + lhalf;     // 16 dims = 2 chunks
            int pos;
            if constexpr (C::kSwizzle) pos = swz<C::kRowChunks, C::kRowShift>(lrow, chunk) * 16;
            else pos = chunk * 16;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(kread + pos));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
        if constexpr (C::kSplitD > 1) {
            // Sum the partial S of the row group's waves, always in the order of their
            // contraction parts, so that every wave of the group gets the same bits.
            f32x4* sx = reinterpret_cast<f32x4*>(smem + 2 * C::kBuf);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                sx[(wid * 4 + q) * 64 + lane] = f32x4{sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
            __syncthreads();
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 tot = sx[((wave * C::kSplitD) * 4 + q) * 64 + lane];
#pragma unroll
                for (int o = 1; o < C::kSplitD; ++o) tot += sx[((wave * C::kSplitD + o) * 4 + q) * 64 + lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[4 * q + e] = tot[e];
            }
        }

        // Raise the running max of each row if this tile's max exceeds it by more than the
        // slack (tmax in scaled log2 units, -inf if the row sees no key of the tile).
        auto update_max = [&](float tmax) {
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const bool grow = tmax > m_run + kRescaleSlack || (m_run == -INFINITY && tmax != -INFINITY);
            if (__any(grow)) {
                const float mnew = grow ? tmax : m_run;
                const float alpha = (m_run == -INFINITY) ? 0.0f : fast_exp2(m_run - mnew);
                l_run *= alpha;
#pragma unroll
                for (int mt = 0; mt < C::kMTiles; ++mt) oacc[mt] *= alpha;
                m_run = mnew;
            }
        };

        // P^T in the B-operand layout: k-slot j of k-step ks is accumulator entry 8 ks + j.
        // The row sum adds the rounded weights, so numerator and denominator agree.
        u32x4 pw[2];
        if (kb + C::kKeys <= full_end) {
            // Every row sees every key of the tile: no masking, scores stay finite.
            float tmax = sacc[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sacc[r]);
            update_max(tmax * p.scale_log2);
            const float mneg = -m_run;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float e0 = fast_exp2(__builtin_fmaf(sacc[r], p.scale_log2, mneg));
                const float e1 = fast_exp2(__builtin_fmaf(sacc[r + 1], p.scale_log2, mneg));
                const uint32_t w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)e0, (__bf16)e1});
                l_run = dot2_bf16(w, kOnesBf16x2, l_run);
                pw[r >> 3][(r & 7) >> 1] = w;
            }
        } else {
            // Boundary tile: keys past the range or past a row's last visible position
            // get weight 0; a row with nothing visible so far keeps m = -inf.
            float sv[16];
            float tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb + 8 * (r >> 2) + 4 * lhalf + (r & 3);
                const bool ok = ri.valid && key < k_end && key <= ri.vis;
                sv[r] = ok ? sacc[r] * p.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, sv[r]);
            }
            update_max(tmax);
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const float e0 = sv[r] == -INFINITY ? 0.0f : fast_exp2(sv[r] - m_run);
                const float e1 = sv[r + 1] == -INFINITY ? 0.0f : fast_exp2(sv[r + 1] - m_run);
                const uint32_t w = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)e0, (__bf16)e1});
                l_run = dot2_bf16(w, kOnesBf16x2, l_run);
                pw[r >> 3][(r & 7) >> 1] = w;
            }
        }

        // O^T += V^T . P^T; V^T comes from the row-major V tile by transposing reads
        const uint8_t* vbuf = buf + (MODE == 0 ? 0 : C::kTileK);
        const int grp = lane >> 4;
        const int kk = lane & 15;
#pragma unroll
        for (int mt = 0; mt < C::kMTiles; ++mt) {
            const int d0 = 32 * (mt + dh * C::kMTiles) + 16 * (grp & 1) + 4 * (kk & 3);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int t0 = 16 * ks + 4 * (grp >> 1) + (kk >> 2);
                int plo, phi;
                if constexpr (C::kSwizzle) {
                    constexpr int kVChunks = C::kDv * 2 / 16;
                    constexpr int kVShift = C::kDv * 2 >= 256 ? 0 : (C::kDv * 2 == 128 ? 1 : 2);
                    const int cv = (d0 * 2) >> 4, w = (d0 * 2) & 15;
                    plo = swz<kVChunks, kVShift>(t0, cv) * 16 + w;
                    phi = swz<kVChunks, kVShift>(t0 + 8, cv) * 16 + w;
                } else {
                    plo = phi = d0 * 2;
                }
                // Assemble the operand from whole dwords: extracting the 16-bit elements
                // one by one made the compiler keep only the first dword of each read.
                const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(vbuf + t0 * C::kRowV + plo));
                const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(vbuf + (t0 + 8) * C::kRowV + phi));
                const bf16x8_t a = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    a, __builtin_bit_cast(bf16x8_t, pw[ks]), oacc[mt], 0, 0, 0);
            }
        }
    };

    u32x4 st[C::kPerThread];
    uint32_t lv = 0;
    if (ntiles > 0) {
        for (int u = 0; u < 2; ++u) {
            const int32_t sl = slot_of(u, table_entry(u));
            if (tid < C::kKeys) ring[u * C::kKeys + tid] = sl;
        }
        __syncthreads();
        load_tile(0, st, lv);
        store_tile(smem, st, lv);
        __syncthreads();
    }
    // Iteration t: look up tile t+2, load tile t+1, compute tile t, publish the slots,
    // store tile t+1, barrier.
    for (int t = 0; t < ntiles; ++t) {
        const int32_t raw = table_entry(t + 2);
        if (t + 1 < ntiles) load_tile(t + 1, st, lv);
        compute_tile(t);
        const int32_t sl = slot_of(t + 2, raw);
        if (tid < C::kKeys) ring[((t + 2) % kSlotRing) * C::kKeys + tid] = sl;
        if (t + 1 < ntiles) store_tile(smem + ((t + 1) & 1) * C::kBuf, st, lv);
        __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);   // the two key halves of each block
    if (!ri.valid) return;
    bool final_out = true;
    int64_t ps = 0;
    if constexpr (MODE == 0) {
        const int nsplit = (L + p.split_tokens - 1) / p.split_tokens;
        final_out = nsplit == 1;
        ps = ri.out_row * p.max_splits + split;
    }
    if (final_out) {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + ri.out_row * C::kDv;
#pragma unroll
        for (int mt = 0; mt < C::kMTiles; ++mt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d = 32 * (mt + dh * C::kMTiles) + 8 * a + 4 * lhalf;
                const uint32_t w0 = bf16_bits(oacc[mt][4 * a] * inv) |
                                    ((uint32_t)bf16_bits(oacc[mt][4 * a + 1] * inv) << 16);
                const uint32_t w1 = bf16_bits(oacc[mt][4 * a + 2] * inv) |
                                    ((uint32_t)bf16_bits(oacc[mt][4 * a + 3] * inv) << 16);
                *reinterpret_cast<uint2*>(out + d) = make_uint2(w0, w1);
            }
        }
        if (p.lse && lhalf == 0 && dh == 0)
            p.lse[ri.out_row] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2f : -INFINITY;
    } else {
        float* o = p.ws_o + ps * C::kDv;
#pragma unroll
        for (int mt = 0; mt < C::kMTiles; ++mt) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int d = 32 * (mt + dh * C::kMTiles) + 8 * a + 4 * lhalf;
                *reinterpret_cast<f32x4*>(o + d) =
                    f32x4{oacc[mt][4 * a], oacc[mt][4 * a + 1], oacc[mt][4 * a + 2], oacc[mt][4 * a + 3]};
            }
        }
        if (lhalf == 0 && dh == 0) {
            p.ws_ml[ps * 2] = m_run;
            p.ws_ml[ps * 2 + 1] = l_tot;
        }
    }
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

int32_t mla_head_groups(int32_t num_q_heads) {
    return (num_q_heads + MCfg<0, 512>::kRows - 1) / MCfg<0, 512>::kRows;
}

DecodePlan plan_mla(int32_t batch, int32_t num_q_heads, int32_t head_dim_v, int32_t max_seq_len_kv) {
    DecodePlan pl{};
    const int64_t hgs = mla_head_groups(num_q_heads);
    auto nsplits = [&](int sp) { return (int64_t)(max_seq_len_kv + sp - 1) / sp; };
    // A split's partial state is Hq x Dv fp32 (256 KiB at 128 x 512): long splits keep that
    // traffic small; shorten them only while the grid would leave compute units idle.
    int split = 1024;
    while (split > 256 && batch * hgs * nsplits(split) < 1024) split /= 2;
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
    // ids: (unit / 8, head group, unit % 8) with units = batch * max_splits rounded up to 8
    const int64_t hgs = mla_head_groups(p.hq);
    const int64_t units = ((int64_t)p.batch * p.max_splits + 7) / 8 * 8;
    const dim3 grid((unsigned)(hgs * units));
    hipLaunchKernelGGL((mfma_attn_kernel<0, 512>), grid, dim3(MCfg<0, 512>::kThreads), 0, s, p);
    return hipGetLastError();
}

int32_t varlen_tokens_per_block(int32_t group) { return MCfg<1, 128>::kGroups * (32 / group); }

hipError_t launch_varlen(const MfmaParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.hkv * p.q_blocks * p.batch));
    if (head_dim == 64) hipLaunchKernelGGL((mfma_attn_kernel<1, 64>), grid, dim3(MCfg<1, 64>::kThreads), 0, s, p);
    else hipLaunchKernelGGL((mfma_attn_kernel<1, 128>), grid, dim3(MCfg<1, 128>::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
