// Packed varlen causal chunk over the paged cache with MFMA for gfx950 ("Paged KV Cache
// and Packed Sequence", 3.1-3.3 and 4.1; skill page Appendix C/E, sparse_mode 3): G query
// heads and up to thousands of query tokens share each kv head.
//
// Four waves of 32 query rows (tokens x heads of one kv head) walk the key range in tiles
// of 32 keys (the tile pipeline of mfma_common.h) with v_mfma_f32_32x32x16_bf16; K and V
// rows are unpadded in LDS with their 16-byte chunks XOR-swizzled by row:
//  * S^T = K . Q^T: K rows from LDS as the A operand, Q^T in registers as the B operand;
//  * in the S^T accumulator each lane holds 16 keys of one query row, so the row max and
//    sum need one cross-lane step, and P^T (bf16) is already in the B-operand layout of
//    the next product once keys are numbered the way the accumulator holds them;
//  * O^T += V^T . P^T: the A operand (four consecutive keys at one value column per lane
//    and read) comes straight from the row-major V tile with ds_read_b64_tr_b16;
//  * O^T keeps one query row per lane, so the online-softmax rescale is lane-local; it is
//    applied only when a row's max grows by more than 2^8 (P <= 256 in between), which
//    after the first tiles almost never happens.  Tiles that every row of the workgroup
//    sees whole skip the masking.
// Append mode (the chunk's cache write folded into the pass, "KVCache Optimization Skill",
// 3.6: write by slot, then attend over the cached tokens and the new ones): the n_b new
// K/V rows of sequence b sit at positions seq_lens[b] - n_b + i; every workgroup reads
// keys from there on out of the new rows themselves (their packed rows have the cache
// slot's row layout), and the workgroup of a query block stores its tokens' rows of its
// kv head at their slots, which no workgroup of the launch reads back.
#include "mfma_common.h"

namespace pkv {

namespace {

using namespace mfma;

// ================================================================== varlen chunk
template <int D>
struct VarCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = kWaves * 64;
    static constexpr int kRows = kWaves * 32;               // query rows per workgroup
    static constexpr int kRowBytes = 2 * D;                 // one K or V row
    static constexpr int kRowChunks = kRowBytes / 16;
    static constexpr int kRowShift = D == 128 ? 0 : 1;      // rows per 256-byte line: 1 or 2
    static constexpr int kHalf = kKeys * kRowBytes;         // K (or V) part of a stage
    static constexpr int kStage = 2 * kHalf;
    static constexpr int kDma = kStage / 1024 / kWaves;     // wave loads per tile
    static constexpr int kSteps = D / 16;
    static constexpr int kMTiles = D / 32;
    static constexpr int kSmem = kStages * kStage + 2 * kTabEntries * 4;
    static_assert(kDma * 1024 * kWaves == kStage, "tile");
};

template <int D, bool APPEND>
__device__ __forceinline__ void varlen_body(const MfmaParams& p) {
    using C = VarCfg<D>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::kSmem];

    const int tid = threadIdx.x;
    const int wid = tid >> 6;
    const int lane = tid & 63;
    const int lrow = lane & 31;        // query row of this lane inside the wave
    const int lhalf = lane >> 5;       // which half of the k-slots / keys

    const int G = p.group;
    const int tw = 32 / G;                         // query tokens per wave
    const int tpb = C::kWaves * tw;                // query tokens per workgroup
    // Work items (sequence, query block), the longest sequences first and, within one,
    // the last query blocks (most keys) first; the kv head varies fastest.
    const int kvh = blockIdx.x % p.hkv;
    int b, qb;
    {
        int j;
        // (append mode: a sequence with new rows but no visible key still stores its slots)
        auto qblocks = [&](int s, int len) {
            const int n = p.cu_q[s + 1] - p.cu_q[s];
            return (n > 0 && (APPEND || len > 0)) ? (n + tpb - 1) / tpb : 0;
        };
        if (!find_item<C::kThreads>(blockIdx.x / p.hkv, p.batch, p.seq_lens, p.len_cap, qblocks,
                                    reinterpret_cast<int32_t*>(smem + kStages * C::kStage), b, j))
            return;
        b = __builtin_amdgcn_readfirstlane(b);          // the same in every lane
        qb = __builtin_amdgcn_readfirstlane(qblocks(b, min(p.seq_lens[b], p.len_cap)) - 1 - j);
    }
    const int q0 = p.cu_q[b];
    const int nq = p.cu_q[b + 1] - q0;
    const int L = min(p.seq_lens[b], p.len_cap);
    const int i_first = qb * tpb;
    if (i_first >= nq || nq <= 0) return;
    const uint32_t row_bytes = (uint32_t)(p.hkv * D * 2);             // one cache slot
    // Append mode: new keys start at new_start (seq_lens[b] - n_b, before the length bound);
    // this workgroup stores the rows of its tokens for its kv head (slot rule of
    // pkv_kv_cache_append: no slot past the table's capacity, none outside the pool).
    // The first kWrDefer 16-byte pieces of each thread go by direct loads into the last
    // tile stage (free until the loop issues its first load there) and are stored once
    // the query rows are in, so that their latency hides under the query loads; any
    // further pieces (fewer than four query heads per kv head: more tokens per
    // workgroup) are copied at once.
    const int new_start = APPEND ? p.seq_lens[b] - nq : INT_MAX;
    constexpr int kWrDefer = C::kStage / 16 / C::kThreads;
    constexpr int kRowChunks = D * 2 / 16;
    constexpr int kRowsPerPass = C::kThreads / kRowChunks;
    uint8_t* const wr_buf = smem + (kStages - 1) * C::kStage;
    int32_t wr_entry[kWrDefer];       // staged piece d: its block-table entry (read now, used later)
    const int wr_rows = APPEND ? 2 * min(nq - i_first, tpb) : 0;
    const int bs_mask_w = (1 << p.bs_log2) - 1;
    // Piece k of this thread: row r = tid / kRowChunks + k kRowsPerPass (K of token
    // i_first + r / 2 if r is even, else V), 16 bytes at chunk tid % kRowChunks.
    auto piece_pos = [&](int r) { return (int64_t)new_start + i_first + (r >> 1); };
    auto piece_off = [&]() { return (int64_t)kvh * D * 2 + (tid % kRowChunks) * 16; };
    auto piece_src = [&](int r) {
        return reinterpret_cast<const uint8_t*>((r & 1) ? p.v_new : p.k_new) + (int64_t)(q0 + i_first + (r >> 1)) * row_bytes + piece_off();
    };
    // The slot of a piece (the rule of pkv_kv_cache_append) from its table entry; the
    // kv head 0 workgroup reports it for K pieces of chunk 0, and stores outside the pool
    // are skipped.
    auto piece_store = [&](int r, int32_t entry, const u32x4& val) {
        const int64_t pos = piece_pos(r);
        const int64_t slot = (pos >= 0 && pos < p.len_cap) ? (((int64_t)entry << p.bs_log2) | (pos & bs_mask_w)) : -1;
        if ((r & 1) == 0 && kvh == 0 && tid % kRowChunks == 0 && p.slots_out) p.slots_out[q0 + i_first + (r >> 1)] = slot;
        if (slot < 0 || slot >= (p.num_blocks << p.bs_log2)) return;
        st16(reinterpret_cast<uint8_t*>((r & 1) ? p.v_cache_w : p.k_cache_w) + slot * row_bytes + piece_off(), val);
    };
    auto piece_entry = [&](int r) -> int32_t {
        const int64_t pos = piece_pos(r);
        return (pos >= 0 && pos < p.len_cap) ? p.table[(int64_t)b * p.mbs + (pos >> p.bs_log2)] : 0;
    };
    if constexpr (APPEND) {
#pragma unroll
        for (int d = 0; d < kWrDefer; ++d) {
            const int r = tid / kRowChunks + d * kRowsPerPass;
            wr_entry[d] = 0;
            if (r < wr_rows) {
                lds_dma16(piece_src(r), wr_buf + (d * C::kThreads + (tid & ~63)) * 16);
                wr_entry[d] = piece_entry(r);
            }
        }
        for (int r = tid / kRowChunks + kWrDefer * kRowsPerPass; r < wr_rows; r += kRowsPerPass)
            piece_store(r, piece_entry(r), ld16(piece_src(r)));
    }
    // The staged pieces to their slots (after a wait for the direct loads and a barrier).
    auto store_staged = [&]() {
        if constexpr (APPEND) {
#pragma unroll
            for (int d = 0; d < kWrDefer; ++d) {
                const int r = tid / kRowChunks + d * kRowsPerPass;
                if (r < wr_rows)
                    piece_store(r, wr_entry[d], *reinterpret_cast<const u32x4*>(wr_buf + (d * C::kThreads + tid) * 16));
            }
        }
    };
    if (L <= 0) {
        if constexpr (APPEND) {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            block_sync();
            store_staged();
        }
        return;
    }
    const int i_last = min(nq, i_first + tpb) - 1;
    const int i = i_first + wid * tw + lrow / G;
    const bool valid = (lrow < tw * G) && (i < nq);
    const int ic = valid ? i : i_first;
    const int hq = kvh * G + (valid ? lrow % G : 0);
    const int64_t out_row = (int64_t)(q0 + ic) * p.hq + hq;
    const int vis = p.causal ? (L - nq + ic) : (L - 1);
    const int k_end = p.causal ? min(L, L - nq + i_last + 1) : L;
    // keys below full_end are visible to every row of the workgroup
    const int full_end = p.causal ? min(k_end, L - nq + i_first + 1) : k_end;
    // Sliding window: a row sees keys [vis - window + 1, vis]; the workgroup's tiles start
    // at its first row's lower bound rounded down to a tile, and keys from full_lo on are
    // above every row's lower bound.
    const int lo_row = p.window > 0 ? vis - p.window + 1 : 0;
    const int kstart = p.window > 0 ? max(0, (p.causal ? L - nq + i_first : L - 1) - p.window + 1) & ~(kKeys - 1) : 0;
    const int full_lo = p.window > 0 ? (p.causal ? L - nq + i_last : L - 1) - p.window + 1 : 0;
    const int ntiles = (k_end - kstart + kKeys - 1) / kKeys;

    bf16x8_t qf[C::kSteps];
    {
        const uint8_t* qrow = reinterpret_cast<const uint8_t*>(p.q) + out_row * D * 2;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s)
            qf[s] = __builtin_bit_cast(bf16x8_t, ld16(qrow + (16 * s + 8 * lhalf) * 2));
    }

    TableChunks<C::kThreads> tab;
    tab.lds = reinterpret_cast<int32_t*>(smem + kStages * C::kStage);
    tab.row = p.table + (int64_t)b * p.mbs;
    tab.k_begin = kstart;
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
    store_staged();

    // Loads of one tile: wave load J = wid * kDma + j fills LDS slots 64 J .. 64 J + 63
    // of the stage; the first half of the stage is the K tile, the second the V tile.
    // Slot q of a half is row q / kRowChunks, physical chunk q % kRowChunks, which holds
    // logical chunk swz(row, physical chunk) of that row.
    const int bs_mask = (1 << p.bs_log2) - 1;
    const uint32_t block_bytes = row_bytes << p.bs_log2;
    const bool v_part = wid >= C::kWaves / 2;                         // uniform per wave
    const uint8_t* cache = reinterpret_cast<const uint8_t*>(v_part ? p.v_cache : p.k_cache) + kvh * D * 2;
    // Full tiles with blocks of at least 16 keys: the wave's 16 rows are consecutive slots
    // of one block, found with one scalar read of the block table; every load then uses
    // that row base in SGPRs and a constant offset per lane.
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);
    const bool fast_rows = p.bs_log2 >= 4;
    const uint8_t* cache_u = reinterpret_cast<const uint8_t*>(wid_u >= C::kWaves / 2 ? p.v_cache : p.k_cache) + kvh * D * 2;
    // append mode: this kv head's slice of the new rows of the wave's half (K or V)
    const uint8_t* new_u = reinterpret_cast<const uint8_t*>(wid_u >= C::kWaves / 2 ? p.v_new : p.k_new) + kvh * D * 2;
    uint32_t fast_voff[C::kDma];
#pragma unroll
    for (int j = 0; j < C::kDma; ++j) {
        const int q = (wid * C::kDma + j) * 64 + lane - (v_part ? C::kHalf / 16 : 0);
        const int r = q / C::kRowChunks;
        fast_voff[j] = (uint32_t)(r - 16 * (wid & 1)) * row_bytes +
                       (uint32_t)swz<C::kRowChunks, C::kRowShift>(r, q % C::kRowChunks) * 16u;
    }
    // The table entry of the next tile is read one tile ahead, off the critical path.
    // Append mode: a full tile of new keys is 32 consecutive new rows (one base, the same
    // lane offsets); a tile with both kinds of key takes the per-row path.
    auto fast_tile = [&](int u) {
        return fast_rows && kstart + (u + 1) * kKeys <= k_end && !(APPEND && kstart + (u + 1) * kKeys > new_start);
    };
    auto new_tile = [&](int u) {
        return APPEND && kstart + u * kKeys >= new_start && kstart + (u + 1) * kKeys <= k_end;
    };
    auto entry_of = [&](int u) { return uniform_load(tab.row + ((kstart + u * kKeys + 16 * (wid_u & 1)) >> p.bs_log2)); };
    int32_t next_entry = fast_tile(0) ? entry_of(0) : 0;
    auto issue_tile = [&](int u) {
        const int kb = kstart + u * kKeys;
        const int chunk = u / kChunkTiles;
        uint8_t* stage = smem + (u % kStages) * C::kStage;
        const int32_t entry = next_entry;
        if (u + 1 < ntiles && fast_tile(u + 1)) next_entry = entry_of(u + 1);
        if (fast_tile(u)) {
            const int key0 = kb + 16 * (wid_u & 1);
            const int32_t blk = min(max(entry, 0), tab.last_block);
            const uint64_t slot0 = ((uint64_t)(uint32_t)blk << p.bs_log2) | (uint32_t)(key0 & bs_mask);
            const uint8_t* sb = cache_u + slot0 * row_bytes;
#pragma unroll
            for (int j = 0; j < C::kDma; ++j) lds_dma16_s(sb, fast_voff[j], stage + (wid_u * C::kDma + j) * 1024);
            return;
        }
        if (new_tile(u)) {
            const int key0 = kb + 16 * (wid_u & 1);
            const uint8_t* sb = new_u + (int64_t)(q0 + key0 - new_start) * row_bytes;
#pragma unroll
            for (int j = 0; j < C::kDma; ++j) lds_dma16_s(sb, fast_voff[j], stage + (wid_u * C::kDma + j) * 1024);
            return;
        }
#pragma unroll
        for (int j = 0; j < C::kDma; ++j) {
            const int J = wid * C::kDma + j;
            const int q = J * 64 + lane - (v_part ? C::kHalf / 16 : 0);
            const int r = q / C::kRowChunks;
            const int c = swz<C::kRowChunks, C::kRowShift>(r, q % C::kRowChunks);
            const int key = min(kb + r, k_end - 1);
            const uint32_t blk = tab.block_of(key, chunk);
            const uint8_t* src = cache + ((uint64_t)blk * block_bytes +
                                          (uint32_t)(key & bs_mask) * row_bytes + (uint32_t)c * 16u);
            if (APPEND && key >= new_start)
                src = reinterpret_cast<const uint8_t*>(v_part ? p.v_new : p.k_new) + kvh * D * 2 +
                      (int64_t)(q0 + key - new_start) * row_bytes + c * 16;
            lds_dma16(src, stage + J * 1024);
        }
    };

    RowState st;
    f32x16 oacc[C::kMTiles];
#pragma unroll
    for (int mt = 0; mt < C::kMTiles; ++mt) oacc[mt] = f32x16{};

    // S^T of tile t (its K reads and products; the caller places the scheduling hints).
    auto mma_scores = [&](int t) -> f32x16 {
        const uint8_t* stage = smem + (t % kStages) * C::kStage;
        f32x16 sacc = f32x16{};
        const uint8_t* krow = stage + lrow * C::kRowBytes;
#pragma unroll
        for (int s = 0; s < C::kSteps; ++s) {
            const int pos = swz<C::kRowChunks, C::kRowShift>(lrow, 2 * s + lhalf) * 16;
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(krow + pos));
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc, 0, 0, 0);
        }
        return sacc;
    };
    // The row's max over tile t (scaled, log2 units).  Full tiles keep the raw S^T entries;
    // boundary tiles scale them and set keys past the range or past a row's last visible
    // position to -inf.  Entry r of a lane is key 8 (r / 4) + 4 lhalf + r % 4 of the tile.
    auto row_max = [&](int t, bool full, const f32x16& sacc, float* sv) -> float {
        float tmax;
        if (full) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = sacc[r];
            tmax = sv[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, sv[r]);
            tmax *= p.scale_log2;
        } else {
            const int kb = kstart + t * kKeys;
            tmax = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb + 8 * (r >> 2) + 4 * lhalf + (r & 3);
                const bool ok = valid && key >= lo_row && key < k_end && key <= vis;
                sv[r] = ok ? sacc[r] * p.scale_log2 : -INFINITY;
                tmax = fmaxf(tmax, sv[r]);
            }
        }
        return max_xor32(tmax);
    };

    // O^T += V^T . P^T of one tile (the V^T operands read by transposing LDS reads).
    auto mma_values = [&](bf16x8_t (*va)[2], const u32x4* pw) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mt = 0; mt < C::kMTiles; ++mt)
                oacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    va[mt][ks], __builtin_bit_cast(bf16x8_t, pw[ks]), oacc[mt], 0, 0, 0);
    };

    // Table chunks and the loads of tile u (issued kStages - 1 tiles ahead).
    auto feed = [&](int u) {
        if (u >= ntiles) return;
        const int c = u / kChunkTiles;
        if (u % kChunkTiles == 0 && tab.exists(c + 1)) tab.load(c + 1, treg);
        if (u % kChunkTiles == kChunkTiles / 2 && tab.exists(c + 1)) tab.store(c + 1, treg);
        issue_tile(u);
    };
#pragma unroll
    for (int u = 0; u < kStages - 1; ++u) feed(u);

    // Software pipeline, one tile apart: iteration t takes the max of S^T(t) (computed in
    // iteration t - 1) and rescales O^T if some row's max grew past the slack; then, after
    // the barrier that makes tile t + 1 visible and frees the stage of tile t - 1 (tile
    // t + 3 is issued into it), the products of S^T(t + 1) are interleaved with the
    // exponentials of P^T(t), and O^T += V^T . P^T(t) follows.  The last iteration
    // computes a throw-away S^T on a stage nobody writes any more, which keeps that region
    // one straight-line block for the scheduler.
    wait_tile<C::kDma>(min(ntiles - 1, kStages - 2));
    block_sync();
    f32x16 s_cur = mma_scores(0);
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, C::kSteps, 0);
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, C::kSteps, 0);
    for (int t = 0; t < ntiles; ++t) {
        const bool full = kstart + t * kKeys >= full_lo && kstart + t * kKeys + kKeys <= full_end;
        float sv[16];
        const float tmax = row_max(t, full, s_cur, sv);
        const bool grow = tmax > st.m + kRescaleSlack || (st.m == -INFINITY && tmax != -INFINITY);
        if (__any(grow)) {
            const float mnew = grow ? tmax : st.m;
            const float alpha = !grow ? 1.0f : (st.m == -INFINITY ? 0.0f : fast_exp2(st.m - mnew));
            st.l *= alpha;
#pragma unroll
            for (int mt = 0; mt < C::kMTiles; ++mt) oacc[mt] *= alpha;
            st.m = mnew;
        }
        if (t + 1 < ntiles) {
            wait_tile<C::kDma>(min(ntiles - 2 - t, kStages - 3));
            block_sync();
            feed(t + kStages - 1);
        }
        // S^T(t + 1) interleaved with the exponentials of P^T(t) and the V reads of tile t,
        // step by step (each step a scheduling region of its own, so that the compiler
        // cannot gather the products at one end): step i issues product i of S^T(t + 1)
        // (if any), exponential pair i of P^T(t) and the transposing reads of V^T operand i.  The
        // K reads of all steps go first.  Then the P . V products.
        const uint8_t* kst = smem + ((t + 1) % kStages) * C::kStage + lrow * C::kRowBytes;
        bf16x8_t ka[C::kSteps];
#pragma unroll
        for (int i = 0; i < C::kSteps; ++i)
            ka[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                        kst + swz<C::kRowChunks, C::kRowShift>(lrow, 2 * i + lhalf) * 16));
        __builtin_amdgcn_sched_barrier(0);
        const float sc = full ? p.scale_log2 : 1.0f;
        const float mneg = st.m == -INFINITY ? 0.0f : -st.m;
        const uint8_t* vbuf = smem + (t % kStages) * C::kStage + C::kHalf;
        const int grp = lane >> 4;
        const int kk = lane & 15;
        f32x16 s_next = f32x16{};
        u32x4 pw[2];
        bf16x8_t va[C::kMTiles][2];
        constexpr int kPipeSteps = C::kSteps > 8 ? C::kSteps : 8;   // >= 8 exponential pairs
        static_assert(2 * C::kMTiles <= kPipeSteps, "steps cover the V operands");
#pragma unroll
        for (int i = 0; i < kPipeSteps; ++i) {
            if (i < C::kSteps)
                s_next = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[i], s_next, 0, 0, 0);
            if (i < 8) {
                const int r = 2 * i;
                const float e0 = fast_exp2(__builtin_fmaf(sv[r], sc, mneg));
                const float e1 = fast_exp2(__builtin_fmaf(sv[r + 1], sc, mneg));
                st.l += e0 + e1;
                pw[r >> 3][(r & 7) >> 1] = pack_bf16(e0, e1);
            }
            if (i < 2 * C::kMTiles) {
                const int mt = i >> 1, ks = i & 1;
                const int d0 = 32 * mt + 16 * (grp & 1) + 4 * (kk & 3);
                const int cv = (d0 * 2) >> 4, w = (d0 * 2) & 15;
                const int t0 = 16 * ks + 4 * (grp >> 1) + (kk >> 2);
                const int plo = swz<C::kRowChunks, C::kRowShift>(t0, cv) * 16 + w;
                const int phi = swz<C::kRowChunks, C::kRowShift>(t0 + 8, cv) * 16 + w;
                const u32x2 lo = __builtin_bit_cast(u32x2, lds_read_tr(vbuf + t0 * C::kRowBytes + plo));
                const u32x2 hi = __builtin_bit_cast(u32x2, lds_read_tr(vbuf + (t0 + 8) * C::kRowBytes + phi));
                va[mt][ks] = __builtin_bit_cast(bf16x8_t, u32x4{lo[0], lo[1], hi[0], hi[1]});
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        mma_values(va, pw);
        s_cur = s_next;
    }

    // ---------------------------------------------------------------- epilogue
    const float l_tot = st.l + __shfl_xor(st.l, 32, 64);   // the two key halves of each block
    if (!valid) return;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + out_row * D;
#pragma unroll
    for (int mt = 0; mt < C::kMTiles; ++mt) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d = 32 * mt + 8 * a + 4 * lhalf;
            const uint32_t w0 = bf16_bits(oacc[mt][4 * a] * inv) | ((uint32_t)bf16_bits(oacc[mt][4 * a + 1] * inv) << 16);
            const uint32_t w1 = bf16_bits(oacc[mt][4 * a + 2] * inv) | ((uint32_t)bf16_bits(oacc[mt][4 * a + 3] * inv) << 16);
            *reinterpret_cast<uint2*>(out + d) = make_uint2(w0, w1);
        }
    }
    if (p.lse && lhalf == 0) p.lse[out_row] = l_tot > 0.0f ? (st.m + __log2f(l_tot)) * kLn2f : -INFINITY;
}

// The plain pass, and the append pass held to two waves per SIMD (its writes' registers
// would otherwise take it past 256 and halve the waves per SIMD).
template <int D>
__global__ __launch_bounds__(VarCfg<D>::kThreads) void varlen_kernel(MfmaParams p) {
    varlen_body<D, false>(p);
}
template <int D>
__global__ __launch_bounds__(VarCfg<D>::kThreads, 2) void varlen_append_kernel(MfmaParams p) {
    varlen_body<D, true>(p);
}

}  // namespace

int32_t varlen_tokens_per_block(int32_t group) { return VarCfg<128>::kWaves * (32 / group); }

hipError_t launch_varlen(const MfmaParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.hkv * p.q_blocks * p.batch));
    if (p.k_new) {
        if (head_dim == 64) hipLaunchKernelGGL(varlen_append_kernel<64>, grid, dim3(VarCfg<64>::kThreads), 0, s, p);
        else hipLaunchKernelGGL(varlen_append_kernel<128>, grid, dim3(VarCfg<128>::kThreads), 0, s, p);
    } else {
        if (head_dim == 64) hipLaunchKernelGGL(varlen_kernel<64>, grid, dim3(VarCfg<64>::kThreads), 0, s, p);
        else hipLaunchKernelGGL(varlen_kernel<128>, grid, dim3(VarCfg<128>::kThreads), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace pkv
