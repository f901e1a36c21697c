// device.h -- gfx950 building blocks of the librattn kernels (MFMA fragments,
// aligned vector loads).  Internal header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// K consecutive elements of one row, loaded with the widest aligned loads.
template <typename T, int K>
struct Row {
    T e[K];
};

template <typename T, int K>
__device__ inline Row<T, K> load_row(const T *p) {
    Row<T, K> r;
    constexpr int B = K * (int)sizeof(T);
    constexpr int A = B < 16 ? B : 16;
    __builtin_memcpy(&r, __builtin_assume_aligned(p, A), B);
    return r;
}

template <typename T, int K>
__device__ inline Row<T, K> zero_row() {
    Row<T, K> r;
#pragma unroll
    for (int i = 0; i < K; ++i) r.e[i] = T(0.0f);
    return r;
}

// An MFMA operand fragment: the 8 consecutive k-values one lane supplies to a
// 16x16 output tile over a 32-long contraction.  bf16: one v_mfma_f32_16x16x32_bf16;
// fp32: eight v_mfma_f32_16x16x4_f32 (one per slot).  In both, lane l supplies
// row/column l%16 and k-slots 8*(l/16)..8*(l/16)+7, and the 16x16 fp32 result
// leaves rows 4*(l/16)+i (i = 0..3) of column l%16 in lane l.
template <typename T>
struct Ops;

template <>
struct Ops<bf16> {
    struct frag {
        bf16x8 v;
    };
    static __device__ inline frag load8(const bf16 *p) {
        frag f;
        __builtin_memcpy(&f, __builtin_assume_aligned(p, 16), 16);
        return f;
    }
    static __device__ inline frag zero() {
        frag f;
        f.v = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        return f;
    }
    static __device__ inline void set(frag &f, int i, float x) { f.v[i] = (bf16)x; }
    static __device__ inline void set_raw(frag &f, int i, bf16 x) { f.v[i] = x; }
    static __device__ inline f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
    }
    static constexpr bool kSplitU = true;  // U is fed as bf16 hi + lo halves
};

template <>
struct Ops<float> {
    struct frag {
        float e[8];
    };
    static __device__ inline frag load8(const float *p) {
        frag f;
        __builtin_memcpy(&f, __builtin_assume_aligned(p, 16), 32);
        return f;
    }
    static __device__ inline frag zero() {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f.e[i] = 0.0f;
        return f;
    }
    static __device__ inline void set(frag &f, int i, float x) { f.e[i] = x; }
    static __device__ inline void set_raw(frag &f, int i, float x) { f.e[i] = x; }
    static __device__ inline f32x4 mma(const frag &a, const frag &b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[i], b.e[i], c, 0, 0, 0);
        return c;
    }
    static constexpr bool kSplitU = false;
};

__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace rattn
