// slot_mapping and the cache write ("KVCache Optimization Skill", Layer 3, 3.1 and 3.3;
// "Paged KV Cache and Packed Sequence", 2.2; ai6s.net KVCache article, 4.2).
//
// Both are tiny next to the attention read: the write moves 2 x T rows (8 KiB each for
// a 32-head, 128-dim bf16 layer).  The copy uses 16-byte vector loads/stores, one
// workgroup per (token, K-or-V) row, so rows of both caches are written in one launch.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

// One workgroup per sequence; threads walk that sequence's new tokens.
__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotParams p) {
    const int b = blockIdx.x;
    // cu_new comes from device memory: clamp it into [0, num_tokens]
    const int32_t first = max(p.cu_new[b], 0);
    const int32_t last = (int32_t)min((int64_t)p.cu_new[b + 1], p.num_tokens);
    const int64_t before = p.lens_before[b];
    const int32_t bs_mask = (1 << p.bs_log2) - 1;
    for (int32_t t = first + (int32_t)threadIdx.x; t < last; t += blockDim.x) {
        const int64_t pos = before + (t - first);
        const int64_t logical = pos >> p.bs_log2;
        int64_t slot = -1;
        if (logical >= 0 && logical < p.mbs) {
            const int64_t phys = p.table[(int64_t)b * p.mbs + logical];
            slot = (phys << p.bs_log2) | (pos & bs_mask);
        }
        p.slots[t] = slot;
    }
}

}  // namespace

hipError_t launch_slot_mapping(const SlotParams& p, hipStream_t s) {
    hipLaunchKernelGGL(slot_mapping_kernel, dim3(p.batch), dim3(256), 0, s, p);
    return hipGetLastError();
}

namespace {

// blockIdx.x = token, blockIdx.y = 0 (K) / 1 (V).  VEC = bytes per access (16 when the
// row size and both base pointers allow it, else 4 or 2).
template <int VEC>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteParams p) {
    const int64_t t = blockIdx.x;
    const int which = blockIdx.y;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) return;   // outside the pool: skipped
    const int64_t rb = p.row_bytes[which];
    const uint8_t* src = p.src[which] + t * rb;
    uint8_t* dst = p.dst[which] + slot * rb;
    for (int64_t off = (int64_t)threadIdx.x * VEC; off < rb; off += (int64_t)blockDim.x * VEC) {
        if constexpr (VEC == 16) {
            st16(dst + off, ld16(src + off));
        } else if constexpr (VEC == 4) {
            *reinterpret_cast<uint32_t*>(dst + off) = *reinterpret_cast<const uint32_t*>(src + off);
        } else {
            *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(src + off);
        }
    }
}

}  // namespace

hipError_t launch_kv_write(const WriteParams& p, hipStream_t s) {
    auto aligned = [&](int v) {
        for (int i = 0; i < 2; ++i) {
            if (p.row_bytes[i] % v) return false;
            if (reinterpret_cast<uintptr_t>(p.src[i]) % v) return false;
            if (reinterpret_cast<uintptr_t>(p.dst[i]) % v) return false;
        }
        return true;
    };
    const int64_t widest = p.row_bytes[0] > p.row_bytes[1] ? p.row_bytes[0] : p.row_bytes[1];
    int threads = 256;
    dim3 grid((unsigned)p.num_tokens, 2);
    if (aligned(16)) {
        while (threads > 64 && (int64_t)(threads / 2) * 16 >= widest) threads /= 2;
        hipLaunchKernelGGL(kv_write_kernel<16>, grid, dim3(threads), 0, s, p);
    } else if (aligned(4)) {
        hipLaunchKernelGGL(kv_write_kernel<4>, grid, dim3(threads), 0, s, p);
    } else {
        hipLaunchKernelGGL(kv_write_kernel<2>, grid, dim3(threads), 0, s, p);
    }
    return hipGetLastError();
}

namespace {

// blockIdx = (new-token index i within its sequence, sequence b, K or V).
template <int VEC>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
    const int i = blockIdx.x;
    const int b = blockIdx.y;
    const int which = blockIdx.z;
    const int64_t first = max(p.cu_new[b], 0);
    const int64_t last = min((int64_t)p.cu_new[b + 1], p.num_tokens);
    const int64_t t = first + i;
    if (t >= last) return;
    const int64_t pos = (int64_t)p.lens_before[b] + i;
    const int64_t logical = pos >> p.bs_log2;
    int64_t slot = -1;
    if (pos >= 0 && logical < p.mbs) {
        const int64_t phys = p.table[(int64_t)b * p.mbs + logical];
        slot = (phys << p.bs_log2) | (pos & ((1 << p.bs_log2) - 1));
    }
    if (which == 0 && threadIdx.x == 0 && p.slots_out) p.slots_out[t] = slot;
    if (slot < 0 || slot >= p.num_slots) return;
    const int64_t rb = p.row_bytes[which];
    const uint8_t* src = p.src[which] + t * rb;
    uint8_t* dst = p.dst[which] + slot * rb;
    for (int64_t off = (int64_t)threadIdx.x * VEC; off < rb; off += (int64_t)blockDim.x * VEC) {
        if constexpr (VEC == 16) {
            st16(dst + off, ld16(src + off));
        } else if constexpr (VEC == 4) {
            *reinterpret_cast<uint32_t*>(dst + off) = *reinterpret_cast<const uint32_t*>(src + off);
        } else {
            *reinterpret_cast<uint16_t*>(dst + off) = *reinterpret_cast<const uint16_t*>(src + off);
        }
    }
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, hipStream_t s) {
    auto aligned = [&](int v) {
        for (int i = 0; i < 2; ++i) {
            if (p.row_bytes[i] % v) return false;
            if (reinterpret_cast<uintptr_t>(p.src[i]) % v) return false;
            if (reinterpret_cast<uintptr_t>(p.dst[i]) % v) return false;
        }
        return true;
    };
    const int64_t widest = p.row_bytes[0] > p.row_bytes[1] ? p.row_bytes[0] : p.row_bytes[1];
    int threads = 256;
    const dim3 grid((unsigned)p.max_new, (unsigned)p.batch, 2);
    if (aligned(16)) {
        while (threads > 64 && (int64_t)(threads / 2) * 16 >= widest) threads /= 2;
        hipLaunchKernelGGL(kv_append_kernel<16>, grid, dim3(threads), 0, s, p);
    } else if (aligned(4)) {
        hipLaunchKernelGGL(kv_append_kernel<4>, grid, dim3(threads), 0, s, p);
    } else {
        hipLaunchKernelGGL(kv_append_kernel<2>, grid, dim3(threads), 0, s, p);
    }
    return hipGetLastError();
}

namespace {

// blockIdx.x = pair, blockIdx.y strides over the block's bytes.
template <int VEC>
__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksParams p) {
    const int64_t src = p.pairs[2 * (int64_t)blockIdx.x];
    const int64_t dst = p.pairs[2 * (int64_t)blockIdx.x + 1];
    if (src < 0 || src >= p.num_blocks || dst < 0 || dst >= p.num_blocks || src == dst) return;
    const uint8_t* s = p.pool + src * p.block_bytes;
    uint8_t* d = p.pool + dst * p.block_bytes;
    const int64_t step = (int64_t)gridDim.y * blockDim.x * VEC;
    for (int64_t off = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * VEC; off < p.block_bytes; off += step) {
        if constexpr (VEC == 16) {
            st16(d + off, ld16(s + off));
        } else {
            *reinterpret_cast<uint32_t*>(d + off) = *reinterpret_cast<const uint32_t*>(s + off);
        }
    }
}

// Measurement aid: the practical HBM read ceiling the HBM-bound kernels are compared with.
// Grid-stride 16-byte non-temporal loads over n16 vectors; the XOR of every word is stored
// only if it equals a constant, so the loads cannot be dropped and (almost) nothing is
// written.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                          uint32_t* sink) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Measurement aid: the read floor of a paged decode's own access pattern.  Workgroup
// (slice, sequence, split) reads rows [split * split_tokens, +split_tokens) of both caches,
// clamped to the sequence's length, through the block table (row = entry * bs + offset),
// slice_bytes of each row; the split's table entries are staged in LDS first.  Eight
// 16-byte loads of each cache per thread are in flight between uses, as in the decode.
constexpr int kGatherEntries = 1040;   // table entries of one split: split_tokens / bs + 2
__global__ __launch_bounds__(256) void gather_read_kernel(GatherReadParams p) {
    constexpr int U = 8;
    __shared__ int32_t tab[kGatherEntries];
    const int nslices = p.row_bytes / p.slice_bytes;
    const int id = blockIdx.x;
    const int slice = id % nslices;
    const int b = (id / nslices) % p.batch;
    const int split = id / (nslices * p.batch);
    const int L = min(max(p.seq_lens[b], 0), p.len_cap);
    const int t0 = split * p.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(L, t0 + p.split_tokens);
    const int blk0 = t0 >> p.bs_log2;
    const int nblk = ((t1 - 1) >> p.bs_log2) - blk0 + 1;
    const int32_t last = (int32_t)(p.num_blocks - 1);
    for (int i = threadIdx.x; i < nblk; i += blockDim.x)
        tab[i] = min(max(p.table[(int64_t)b * p.mbs + blk0 + i], 0), last);
    __syncthreads();
    const int chunks = p.slice_bytes / 16;
    const int n = (t1 - t0) * chunks;
    const int64_t col = (int64_t)slice * p.slice_bytes;
    const int bs_mask = (1 << p.bs_log2) - 1;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int e = threadIdx.x; e < n; e += (int)blockDim.x * U) {
        u32x4 kr[U], vr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int eu = min(e + (int)blockDim.x * u, n - 1);
            const int tok = t0 + eu / chunks;
            const int64_t row = ((int64_t)tab[(tok >> p.bs_log2) - blk0] << p.bs_log2) | (tok & bs_mask);
            const int64_t off = row * p.row_bytes + col + (int64_t)(eu % chunks) * 16;
            kr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.k + off));
            vr[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v + off));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= kr[u] ^ vr[u];
    }
    if (acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u) p.sink[0] = acc.z;
}

// Copy of n4 int32 words from pinned host memory (its device view) into device memory: one
// 16-byte word per thread where the two ends allow it, 4-byte words for the tail.
__global__ __launch_bounds__(256) void host_copy_kernel(const uint32_t* __restrict__ src,
                                                        uint32_t* __restrict__ dst, int64_t n4) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n16 = n4 / 4;
    if (i < n16) {
        reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
    } else if (i < n16 + (n4 & 3)) {
        const int64_t k = 4 * n16 + (i - n16);
        dst[k] = src[k];
    }
}

}  // namespace

hipError_t launch_host_copy(void* dst, const void* src_dev_view, int64_t bytes, hipStream_t s) {
    const int64_t n4 = bytes / 4;
    const int64_t threads = n4 / 4 + (n4 & 3);
    const unsigned grid = (unsigned)((threads + 255) / 256);
    hipLaunchKernelGGL(host_copy_kernel, dim3(grid), dim3(256), 0, s,
                       static_cast<const uint32_t*>(src_dev_view), static_cast<uint32_t*>(dst), n4);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                       static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_gather_read(const GatherReadParams& p, hipStream_t s) {
    const int64_t nsplit = ((int64_t)p.len_cap + p.split_tokens - 1) / p.split_tokens;
    const int64_t grid = (int64_t)(p.row_bytes / p.slice_bytes) * p.batch * nsplit;
    if (grid <= 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gather_read_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t s) {
    const bool v16 = p.block_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(p.pool) % 16 == 0;
    const int64_t per_wg = 256LL * (v16 ? 16 : 4);
    const int64_t chunks = (p.block_bytes + per_wg - 1) / per_wg;
    const dim3 grid((unsigned)p.num_pairs, (unsigned)(chunks < 16 ? chunks : 16));
    if (v16) hipLaunchKernelGGL(copy_blocks_kernel<16>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(copy_blocks_kernel<4>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
