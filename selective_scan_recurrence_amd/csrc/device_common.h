// Device helpers shared by the kernel files: element loads/stores for the io
// dtypes and the fast transcendental forms the kernels use.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.44269504088896340736f;

// io element types: f32 is stored as float, bf16 as its 16 raw bits.
using bf16_t = uint16_t;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// f32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ bf16_t bf16_rne(float v) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(v));
}

__device__ __forceinline__ void store_io(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_io(bf16_t* p, float v) { *p = bf16_rne(v); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// SiLU(c) = c / (1 + e^-c), with the hardware reciprocal.
__device__ __forceinline__ float silu(float c) {
    return c * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-c * kLog2e));
}

constexpr float kLn2 = 0.69314718055994530942f;

// softplus with the threshold-20 branch of "mambazip mamba1/model.rs"
// (softplus): v above 20, else log(1 + e^v), on the transcendental unit.
// With w = e^v (v_exp_f32) and u = 1 + w rounded, log(1 + w) is taken as
// log(u) * w / (u - 1), which cancels the rounding error of u (Goldberg,
// "What Every Computer Scientist Should Know About Floating-Point
// Arithmetic", Theorem 4); when u rounds to 1 the result is w itself.  The
// error is a few ulp of the result for every v.
__device__ __forceinline__ float softplus(float v) {
    if (v > 20.0f) return v;
    const float w = __builtin_amdgcn_exp2f(v * kLog2e);
    const float u = 1.0f + w;
    return u == 1.0f ? w : __builtin_amdgcn_logf(u) * kLn2 * (w * __builtin_amdgcn_rcpf(u - 1.0f));
}

// logistic(v) = 1 / (1 + e^-v), the derivative of softplus, with the hardware
// exponential and reciprocal.
__device__ __forceinline__ float sigmoid(float v) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
}

// Token range of sequence i: [t0, t0 + len) of the token axis.  Without
// spans (cu null) every sequence has L tokens at i*L.  With spans, one that
// is negative, reversed, past T or longer than L is taken as empty and
// reported through bad.
struct SeqSpan {
    int64_t t0;
    int len;
    bool bad;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int i, int L, int64_t T) {
    if (!cu) return SeqSpan{(int64_t)i * L, L, false};
    const int a = cu[i], b = cu[i + 1];
    const bool bad = a < 0 || b < a || (int64_t)b > T || b - a > L;
    return SeqSpan{bad ? 0 : (int64_t)a, bad ? 0 : b - a, bad};
}

// DPP quad permute: lane q of each group of four lanes reads lane P<q>.
template <int P0, int P1, int P2, int P3>
__device__ __forceinline__ float quad_perm(float v) {
    constexpr int ctrl = P0 | (P1 << 2) | (P2 << 4) | (P3 << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl,
                                                                 0xF, 0xF, true));
}
template <int K>
__device__ __forceinline__ float quad_bcast(float v) { return quad_perm<K, K, K, K>(v); }
// lane q reads lane (q - R) mod 4
template <int R>
__device__ __forceinline__ float quad_rot(float v) {
    return quad_perm<(4 - R) & 3, (5 - R) & 3, (6 - R) & 3, (7 - R) & 3>(v);
}
// lane q reads lane q ^ 1 / q ^ 2
__device__ __forceinline__ float quad_xor1(float v) { return quad_perm<1, 0, 3, 2>(v); }
__device__ __forceinline__ float quad_xor2(float v) { return quad_perm<2, 3, 0, 1>(v); }

}  // namespace ssm
