// RMSNorm + RoPE + cache write of the MLA latent row in one launch: the fused writer the
// pages use in front of the MLA cache (npu_kv_rmsnorm_rope_cache, keyed by slot_mapping;
// "KVCache Optimization Skill", Mode 3 and its cache-write fusion note).  The pages name
// it without defining it; the readings taken are the oracle's: RMSNorm with gamma and eps
// over the nope part, rotary embedding in the half-split form over the rope part with the
// token's cosines and sines.
//
// One wave per token: the nope part is read once in 16-byte chunks (one or two per lane),
// its mean square reduced across the wave, scaled and stored to cache_nope[slot]; the
// lanes holding rope chunk i also read chunk i + Dr/2, rotate the pairs and store both to
// cache_rope[slot].  Like the plain write, a slot outside the pool is skipped.  The step
// moves a few bytes per token: it is bound by launch latency, not by HBM.
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

namespace {

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kPer16 = 4;
    static __device__ __forceinline__ void widen(const u32x4& v, float* x) {
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(v[i]);
    }
    static __device__ __forceinline__ u32x4 narrow(const float* x) {
        return u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
    }
};
template <> struct Elem<bf16_t> {
    static constexpr int kPer16 = 8;
    static __device__ __forceinline__ void widen(const u32x4& v, float* x) {
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = bf16_lo(v[i]);
            x[2 * i + 1] = bf16_hi(v[i]);
        }
    }
    static __device__ __forceinline__ u32x4 narrow(const float* x) {
        u32x4 v;
        for (int i = 0; i < 4; ++i)
            v[i] = (uint32_t)f32_to_bf16(x[2 * i]) | ((uint32_t)f32_to_bf16(x[2 * i + 1]) << 16);
        return v;
    }
};

template <typename T>
__global__ __launch_bounds__(256) void norm_rope_write_kernel(NormRopeParams p) {
    constexpr int E = Elem<T>::kPer16;
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= p.num_tokens) return;
    const int64_t slot = p.slots[t];
    if (slot < 0 || slot >= p.num_slots) return;    // outside the pool: skipped
    const int dn = p.dn, dr = p.dr, half = p.dr / 2;
    const uint8_t* row = reinterpret_cast<const uint8_t*>(p.kv) + t * (int64_t)(dn + dr) * sizeof(T);

    // RMSNorm of the nope part: chunks lane and lane + 64 (dn <= 128 chunks).
    const int nc = dn / E;
    float x[2][E];
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = lane + 64 * k;
        if (c < nc) {
            Elem<T>::widen(ld16(row + (int64_t)c * 16), x[k]);
#pragma unroll
            for (int i = 0; i < E; ++i) ss = fmaf(x[k][i], x[k][i], ss);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float inv = 1.0f / sqrtf(ss / (float)dn + p.eps);
    uint8_t* nope = reinterpret_cast<uint8_t*>(p.cache_nope) + slot * (int64_t)dn * sizeof(T);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int c = lane + 64 * k;
        if (c < nc) {
            float g[E], y[E];
            Elem<T>::widen(ld16(reinterpret_cast<const uint8_t*>(p.gamma) + (int64_t)c * 16), g);
#pragma unroll
            for (int i = 0; i < E; ++i) y[i] = x[k][i] * inv * g[i];
            st16(nope + (int64_t)c * 16, Elem<T>::narrow(y));
        }
    }

    // RoPE of the rope part: lane l < half / E turns pairs (l E + i, half + l E + i).
    if (lane < half / E) {
        const int e0 = lane * E;
        float x1[E], x2[E], cs[E], sn[E], o1[E], o2[E];
        Elem<T>::widen(ld16(row + (int64_t)(dn + e0) * sizeof(T)), x1);
        Elem<T>::widen(ld16(row + (int64_t)(dn + half + e0) * sizeof(T)), x2);
        const float* cp = p.cos + t * half + e0;
        const float* sp = p.sin + t * half + e0;
#pragma unroll
        for (int i = 0; i < E; i += 4) {
            const u32x4 cv = ld16(cp + i), sv = ld16(sp + i);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                cs[i + j] = __uint_as_float(cv[j]);
                sn[i + j] = __uint_as_float(sv[j]);
            }
        }
#pragma unroll
        for (int i = 0; i < E; ++i) {
            o1[i] = fmaf(x1[i], cs[i], -x2[i] * sn[i]);
            o2[i] = fmaf(x2[i], cs[i], x1[i] * sn[i]);
        }
        uint8_t* rope = reinterpret_cast<uint8_t*>(p.cache_rope) + slot * (int64_t)dr * sizeof(T);
        st16(rope + (int64_t)e0 * sizeof(T), Elem<T>::narrow(o1));
        st16(rope + (int64_t)(half + e0) * sizeof(T), Elem<T>::narrow(o2));
    }
}

}  // namespace

hipError_t launch_norm_rope_write(const NormRopeParams& p, int dtype, hipStream_t s) {
    const dim3 grid((unsigned)((p.num_tokens + 3) / 4));
    if (dtype == 1) hipLaunchKernelGGL(norm_rope_write_kernel<bf16_t>, grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL(norm_rope_write_kernel<float>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace pkv
