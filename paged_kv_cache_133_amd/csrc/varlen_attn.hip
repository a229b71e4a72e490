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

template <int D>
__global__ __launch_bounds__(VarCfg<D>::kThreads) void varlen_kernel(MfmaParams p) {
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
        auto qblocks = [&](int s, int len) {
            const int n = p.cu_q[s + 1] - p.cu_q[s];
            return (n > 0 && len > 0) ? (n + tpb - 1) / tpb : 0;
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
    if (i_first >= nq || nq <= 0 || L <= 0) return;
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

    // Loads of one tile: wave load J = wid * kDma + j fills LDS slots 64 J .. 64 J + 63
    // of the stage; the first half of the stage is the K tile, the second the V tile.
    // Slot q of a half is row q / kRowChunks, physical chunk q % kRowChunks, which holds
    // logical chunk swz(row, physical chunk) of that row.
    const int bs_mask = (1 << p.bs_log2) - 1;
    const uint32_t row_bytes = (uint32_t)(p.hkv * D * 2);             // one cache slot
    const uint32_t block_bytes = row_bytes << p.bs_log2;
    const bool v_part = wid >= C::kWaves / 2;                         // uniform per wave
    const uint8_t* cache = reinterpret_cast<const uint8_t*>(v_part ? p.v_cache : p.k_cache) + kvh * D * 2;
    // Full tiles with blocks of at least 16 keys: the wave's 16 rows are consecutive slots
    // of one block, found with one scalar read of the block table; every load then uses
    // that row base in SGPRs and a constant offset per lane.
    const int wid_u = __builtin_amdgcn_readfirstlane(wid);
    const bool fast_rows = p.bs_log2 >= 4;
    const uint8_t* cache_u = reinterpret_cast<const uint8_t*>(wid_u >= C::kWaves / 2 ? p.v_cache : p.k_cache) + kvh * D * 2;
    uint32_t fast_voff[C::kDma];
#pragma unroll
    for (int j = 0; j < C::kDma; ++j) {
        const int q = (wid * C::kDma + j) * 64 + lane - (v_part ? C::kHalf / 16 : 0);
        const int r = q / C::kRowChunks;
        fast_voff[j] = (uint32_t)(r - 16 * (wid & 1)) * row_bytes +
                       (uint32_t)swz<C::kRowChunks, C::kRowShift>(r, q % C::kRowChunks) * 16u;
    }
    // The table entry of the next tile is read one tile ahead, off the critical path.
    auto fast_tile = [&](int u) { return fast_rows && kstart + (u + 1) * kKeys <= k_end; };
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

}  // namespace

int32_t varlen_tokens_per_block(int32_t group) { return VarCfg<128>::kWaves * (32 / group); }

hipError_t launch_varlen(const MfmaParams& p, int head_dim, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)p.hkv * p.q_blocks * p.batch));
    if (head_dim == 64) hipLaunchKernelGGL(varlen_kernel<64>, grid, dim3(VarCfg<64>::kThreads), 0, s, p);
    else hipLaunchKernelGGL(varlen_kernel<128>, grid, dim3(VarCfg<128>::kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
