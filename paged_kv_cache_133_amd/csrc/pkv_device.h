// Device-side helpers shared by the gfx950 kernels: 16-byte vector types, bf16
// widening, wavefront reductions with DPP, and the fp32 exp2 the softmax uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace pkv {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct bf16_t { uint16_t bits; };  // storage tag for bf16 tensors

// Widen the low / high bf16 of a packed pair to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 2-term bf16 dot product accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// DPP lane moves inside a 16-lane row (bound_ctrl: lanes read 0 if the source is off).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kRowMirror = 0x140;     // lane i <-> 15-i within each 16 lanes

// Sum over aligned groups of N lanes (N = 1, 2, 4, 8, 16, 32, 64); every lane of the
// group receives the group sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<kQuadXor1>(v);
    if constexpr (N >= 4) v += dpp<kQuadXor2>(v);
    if constexpr (N >= 8) v += dpp<kRowHalfMirror>(v);
    if constexpr (N >= 16) v += dpp<kRowMirror>(v);
    if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Reduce across lanes that differ only in bits >= log2(STRIDE) (the "rows" of STRIDE
// lanes each); every lane receives the result for its column.
template <int STRIDE>
__device__ __forceinline__ float cross_row_max(float v) {
#pragma unroll
    for (int s = STRIDE; s < kWave; s <<= 1) v = fmaxf(v, __shfl_xor(v, s, 64));
    return v;
}
template <int STRIDE>
__device__ __forceinline__ float cross_row_sum(float v) {
#pragma unroll
    for (int s = STRIDE; s < kWave; s <<= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// 2^x in fp32 (v_exp_f32).  Arguments here are <= 0 or -inf; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// First key a decode query at position L - 1 sees under a sliding window of `window` keys
// (the band of "KVCache Optimization Skill", Appendix C, sparse_mode 4; window <= 0: none).
__device__ __forceinline__ int window_start(int L, int window) { return window > 0 ? max(0, L - window) : 0; }
// The same rounded down to a multiple of 32 keys: where a sequence's splits and tiles begin.
__device__ __forceinline__ int window_start32(int L, int window) { return window_start(L, window) & ~31; }

// 16-byte global load / store.
__device__ __forceinline__ u32x4 ld16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace pkv
