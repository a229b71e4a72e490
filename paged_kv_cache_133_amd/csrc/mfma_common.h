// Device pieces shared by the MFMA attention kernels for gfx950 (MLA-absorbed decode
// and packed varlen chunk): vector types, the explicit wait and barrier of the tile
// pipeline, loads from global memory straight into LDS, transposing LDS reads, the
// block-table chunks staged in LDS, and the chunk swizzle of unpadded LDS rows.
//
// Tile pipeline.  The K/V rows of a tile of 32 keys go from global memory straight into
// LDS (global_load_lds_dwordx4: each lane names its own 16-byte source, the destination
// is 16 bytes per lane after a wave-uniform base), into one of four LDS stages, three
// tiles ahead of the tile being computed: no registers hold data in flight, so the loads
// of three tiles overlap the math.  Their completion is waited for explicitly (the
// vector-memory counter, per wave) followed by one workgroup barrier per tile.  The
// block-table entries of the next 1024 keys are staged in LDS 512 keys before they are
// needed, so no load of the table sits in the in-order counter between the K/V loads.
// Keys past the range are read from the range's last key (a real, finite row) and get
// weight 0.
#pragma once

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace mfma {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2f = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;           // log2 units a row max may grow before rescaling
constexpr int kKeys = 32;                       // keys per tile
constexpr int kStages = 4;                      // LDS stages of the tile pipeline
constexpr int kChunkTiles = 32;                 // tiles per staged chunk of the block table
constexpr int kChunkKeys = kChunkTiles * kKeys;
constexpr int kTabEntries = kChunkKeys + 16;    // entries per chunk buffer (>= 1024 + 1)

// s_waitcnt immediate (gfx9 layout): vmcnt in bits 3:0 and 15:14, expcnt in 6:4,
// lgkmcnt in 11:8; expcnt and lgkmcnt at their maxima do not wait.
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x402;             // VALU and transcendental
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Wait for this wave's loads into LDS of tile t, with n in {0, 1, 2} later tiles (each
// of at least PER loads) allowed to stay in flight.
template <int PER>
__device__ __forceinline__ void wait_tile(int n) {
    static_assert(kStages == 4, "waits cover up to two later tiles");
    if (n >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PER));
    else if (n == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(PER));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Workgroup barrier after this wave's LDS writes have completed.  No memory fence: a
// fence would also wait for the loads still in flight into LDS.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 16 bytes per lane from src into LDS at lds_base + 16 * lane (lds_base wave-uniform, in
// M0).  Written as inline asm on purpose: the compiler then does not know that LDS is
// written here and does not make every later LDS read wait for all of these loads (it
// cannot tell the stages of one LDS array apart); the kernels wait for them explicitly.
// s_nop: an SALU write of M0 needs one wait state before a load that writes LDS.
__device__ __forceinline__ void lds_dma16(const void* src, uint8_t* lds_base) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_base;
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(m0) : "memory");
}

// x, opaque to the compiler: per-lane values derived from it inside a loop are computed
// there, where they are needed, instead of being hoisted out and held in registers (or
// spilled) across the whole loop.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// 4 bytes per lane from src into LDS at lds_base + 4 * lane, as lds_dma16.
__device__ __forceinline__ void lds_dma4(const void* src, uint8_t* lds_base) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_base;
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" :: "v"(src), "{m0}"(m0) : "memory");
}

// The same with a wave-uniform 64-bit base in SGPRs and a 32-bit offset per lane (the
// saddr form), for loads whose addresses differ from lane to lane only by constants.
// s_nop 4: an SGPR or M0 written by a VALU instruction needs five wait states before a
// vector-memory instruction reads it.
__device__ __forceinline__ void lds_dma16_s(const uint8_t* sbase, uint32_t voff, uint8_t* lds_base) {
    const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds_base;
    // The base is the same in every lane; reading it from the first lane puts it in SGPRs
    // also where the compiler cannot prove that (it is then a no-op where it can).
    const uint64_t a = reinterpret_cast<uintptr_t>(sbase);
    const uint64_t sa = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sa), "{m0}"(m0) : "memory");
}

// Read of a wave-uniform int32 through the scalar data cache (a load from the constant
// address space; p must be the same in every lane).
__device__ __forceinline__ int32_t uniform_load(const int32_t* p) {
    const uint64_t a = reinterpret_cast<uintptr_t>(p);
    const uint64_t sa = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) << 32);
    return *reinterpret_cast<const __attribute__((address_space(4))) int32_t*>(sa);
}

// max(x, x of lane ^ 32) and max(x, x of lane ^ 16) with the gfx950 lane-swap
// instructions (fmax of the two swapped copies), instead of LDS-routed shuffles.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ s16x4 lds_read_tr(const uint8_t* lds_addr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(lds_addr));
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)a, (__bf16)b});
}

// 8 int8 codes (two dwords) as 8 bf16 (exact: |code| <= 127).  (A byte-permute form, fp32
// 2^23 + (c + 128) minus 2^23 + 128, takes more instructions and measured slower.)
__device__ __forceinline__ u32x4 codes8_to_bf16(uint32_t x, uint32_t y) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t v = i ? y : x;
        const float c0 = (float)(int)(int8_t)(v), c1 = (float)(int)(int8_t)(v >> 8);
        const float c2 = (float)(int)(int8_t)(v >> 16), c3 = (float)(int)(int8_t)(v >> 24);
        r[2 * i] = pack_bf16(c0, c1);
        r[2 * i + 1] = pack_bf16(c2, c3);
    }
    return r;
}
// 16 int8 codes as 16 bf16, codes 0-7 in lo, 8-15 in hi.
__device__ __forceinline__ void codes_to_bf16(u32x4 v, u32x4& lo, u32x4& hi) {
    lo = codes8_to_bf16(v[0], v[1]);
    hi = codes8_to_bf16(v[2], v[3]);
}

// ------------------------------------------------------------------ block-table chunks
// Chunk c holds the entries of keys [k_begin + 1024 c, k_begin + 1024 (c + 1)) in LDS
// buffer c & 1.  Entries are loaded into registers when the chunk before it starts to
// be used and stored 16 tiles later; the barrier of every tile publishes them.
template <int NT>
struct TableChunks {
    static constexpr int kRegs = (kChunkKeys + 1 + NT - 1) / NT;
    int32_t* lds;            // [2][kTabEntries]
    const int32_t* row;      // this sequence's block-table row
    int k_begin, k_end, bs_log2, tid;
    int32_t last_block;

    __device__ int first_entry(int c) const { return (k_begin + c * kChunkKeys) >> bs_log2; }
    __device__ bool exists(int c) const { return k_begin + c * kChunkKeys < k_end; }
    __device__ void load(int c, int32_t* regs) const {
        const int e0 = first_entry(c);
        const int e1 = (min(k_end, k_begin + (c + 1) * kChunkKeys) - 1) >> bs_log2;
#pragma unroll
        for (int j = 0; j < kRegs; ++j) regs[j] = row[min(e0 + tid + j * NT, e1)];
    }
    __device__ void store(int c, const int32_t* regs) const {
        int32_t* dst = lds + (c & 1) * kTabEntries;
#pragma unroll
        for (int j = 0; j < kRegs; ++j)
            if (tid + j * NT < kTabEntries) dst[tid + j * NT] = min(max(regs[j], 0), last_block);
    }
    // Chunk c's entries straight into LDS buffer c & 1, without registers: four loads of 64
    // entries per wave of a 4-wave workgroup (a range starts on a tile, so a chunk spans at
    // most 1024 entries); entries past the chunk's last repeat it.  Completion is waited for
    // with the wave's load counter like the tile loads, and published by the barriers
    // before the chunk is used.
    __device__ void load_lds(int c, int wave) const {
        static_assert(NT == 256 && 16 * 64 <= kTabEntries, "four waves, 1024 entries");
        const int e0 = first_entry(c);
        const int e1 = (min(k_end, k_begin + (c + 1) * kChunkKeys) - 1) >> bs_log2;
        uint8_t* dst = reinterpret_cast<uint8_t*>(lds + (c & 1) * kTabEntries);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int blk = 4 * j + wave;
            lds_dma4(row + min(e0 + 64 * blk + (int)(threadIdx.x & 63), e1), dst + blk * 256);
        }
    }
    // Physical block of key (all keys of one tile lie in one chunk), clamped into the pool.
    __device__ uint32_t block_of(int key, int chunk) const {
        return (uint32_t)min(max(lds[(chunk & 1) * kTabEntries + (key >> bs_log2) - first_entry(chunk)], 0), last_block);
    }
};

// ------------------------------------------------------------------ work order
// Work item `item` of a launch in which sequence b contributes count(b, L_b) items.  Up
// to NT sequences are taken longest first (ties: lower index first), so that the longest
// work starts first and the live items are numbered without gaps (and so spread evenly
// over the XCDs); more sequences than that are taken in index order.  Sets seq and j
// (the item's index within its sequence); false if item is past the last item.  All NT
// threads of the workgroup must call it; lds needs 3 NT + 24 ints and is free afterwards.
template <int NT, typename Count>
__device__ bool find_item(int item, int batch, const int32_t* seq_lens, int len_cap, Count count,
                          int32_t* lds, int& seq, int& j) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    int32_t* s_len = lds;                 // [NT] lengths of the chunk's sequences
    int32_t* s_cnt = lds + NT;            // [NT] item counts by position in the order
    int32_t* s_seq = lds + 2 * NT;        // [NT] sequence at each position
    int32_t* s_wave = lds + 3 * NT;       // [NT / 64] per-wave sums
    int32_t* s_res = lds + 3 * NT + 16;   // found, sequence, index
    const bool ranked = batch <= NT;
    if (tid == 0) s_res[0] = 0;
    int base = 0;                         // items of the chunks before
    for (int c0 = 0; c0 < batch; c0 += NT) {
        const int bb = c0 + tid;
        int len = 0, cnt = 0;
        if (bb < batch) {
            len = min(seq_lens[bb], len_cap);
            cnt = count(bb, len);
        }
        int pos = tid;
        if (ranked) {
            s_len[tid] = bb < batch ? len : -1;
            __syncthreads();
            if (bb < batch) {
                pos = 0;
                for (int o = 0; o < batch; ++o) {
                    const int lo = s_len[o];
                    pos += (lo > len) || (lo == len && o < tid);
                }
            }
        }
        s_cnt[pos] = bb < batch ? cnt : 0;
        s_seq[pos] = bb;
        __syncthreads();
        int v = s_cnt[tid];
        const int own = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int u = __shfl_up(v, d, 64);
            if (lane >= d) v += u;
        }
        if (lane == 63) s_wave[wid] = v;
        __syncthreads();
        int incl = base + v;
        for (int w = 0; w < wid; ++w) incl += s_wave[w];
        if (item >= incl - own && item < incl) {
            s_res[0] = 1;
            s_res[1] = s_seq[tid];
            s_res[2] = item - (incl - own);
        }
        for (int w = 0; w < NT / 64; ++w) base += s_wave[w];
        __syncthreads();
        if (s_res[0]) break;
    }
    const bool found = s_res[0] != 0;
    seq = s_res[1];
    j = s_res[2];
    __syncthreads();
    return found;
}

// ------------------------------------------------------------------ online softmax state
struct RowState {
    float m = -INFINITY;     // running max (log2 units), equal in every lane of the row
    float l = 0.0f;          // this lane's part of the running sum
};

// Physical 16-byte chunk of logical chunk c in LDS row r (an involution).  Rows sharing
// a 256-byte bank line (x = r >> SHIFT) get distinct XOR patterns: 16 consecutive rows
// land on 16 different chunks, and any 4 consecutive rows map a chunk pair {2i, 2i+1}
// to 8 different chunks.
template <int CPR, int SHIFT>
__device__ __forceinline__ int swz(int r, int c) {
    const int x = r >> SHIFT;
    return c ^ ((2 * (x & (CPR / 2 - 1))) ^ ((x / (CPR / 2)) & 1));
}

}  // namespace mfma
}  // namespace pkv
