// Device helpers shared by the attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// 2^x on the hardware transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a row of 16 lanes (gfx9 encodings).
enum : int {
    kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
    kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
    kDppHalfMirror = 0x141, // lane i <-> 7-i inside each group of 8
    kDppMirror = 0x140,     // lane i <-> 15-i inside each row of 16
};

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum over each aligned group of G consecutive lanes (G in {1,2,4,8,16}); every
// lane of the group gets the group sum. Butterfly over DPP moves, which the
// compiler folds into the adds (v_add_f32_dpp).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    if constexpr (G >= 2) x += dpp<kDppXor1>(x);
    if constexpr (G >= 4) x += dpp<kDppXor2>(x);
    if constexpr (G >= 8) x += dpp<kDppHalfMirror>(x);
    if constexpr (G >= 16) x += dpp<kDppMirror>(x);
    return x;
}

// group_sum over N independent values, stage by stage: each DPP move reads a
// register written N instructions earlier, so no wait states are needed
// between a write and the DPP read of it.
template <int G, int N>
__device__ __forceinline__ void group_sum_n(float (&x)[N]) {
    static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
    if constexpr (G >= 2) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] += dpp<kDppXor1>(x[i]);
    }
    if constexpr (G >= 4) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] += dpp<kDppXor2>(x[i]);
    }
    if constexpr (G >= 8) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] += dpp<kDppHalfMirror>(x[i]);
    }
    if constexpr (G >= 16) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] += dpp<kDppMirror>(x[i]);
    }
}

__device__ __forceinline__ float4 operator*(float4 a, float s) {
    return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

// acc + <a, b> as a chain of four FMAs into the running sum
__device__ __forceinline__ float fma4(float acc, float4 a, float4 b) {
    acc = __builtin_fmaf(a.x, b.x, acc);
    acc = __builtin_fmaf(a.y, b.y, acc);
    acc = __builtin_fmaf(a.z, b.z, acc);
    return __builtin_fmaf(a.w, b.w, acc);
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }

// Streaming load (read once): nontemporal hint, so the line is not kept
// in the caches at the expense of data that is reused.
__device__ __forceinline__ float4 ld4_stream(const float *p) {
    typedef float v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}

// Rotate-half rotary embedding (a rotation by angle theta_i of the pair
// (x_i, x_{i+d/2}), i < d/2) of one element x whose pair partner is xp, or of
// four componentwise: a first-half element becomes x c - xp s, a second-half
// element xp s + x c, with c, s the cosine and sine of its pair's angle.
__device__ __forceinline__ float rope_half1(float x, float xp, float c, float s, bool lo) {
    return lo ? x * c - xp * s : xp * s + x * c;
}
__device__ __forceinline__ float4 rope_half(float4 x, float4 xp, float4 c, float4 s, bool lo) {
    return make_float4(rope_half1(x.x, xp.x, c.x, s.x, lo), rope_half1(x.y, xp.y, c.y, s.y, lo),
                       rope_half1(x.z, xp.z, c.z, s.z, lo), rope_half1(x.w, xp.w, c.w, s.w, lo));
}

}  // namespace attn
