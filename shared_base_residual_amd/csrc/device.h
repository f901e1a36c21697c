// device.h -- gfx950 building blocks of the librattn kernels (MFMA fragments,
// aligned vector loads).  Internal header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace rattn {

// Raises kernel fn's dynamic-LDS limit to `lds` bytes on the current device.
// The attribute call is costly on the launch path, so each (kernel, device)
// remembers the largest limit set so far (Slot: one static table per kernel).
template <typename Slot>
inline hipError_t ensure_lds(const void *fn, int lds) {
    static std::atomic<int> set[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (set[dev].load(std::memory_order_relaxed) >= lds) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e == hipSuccess) {
        int cur = set[dev].load(std::memory_order_relaxed);
        while (cur < lds && !set[dev].compare_exchange_weak(cur, lds)) {
        }
    }
    return e;
}

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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
    // Half fragment: 4 k-values per lane over a 16-long contraction (lane l
    // supplies k-slots 4*(l/16)..4*(l/16)+3), one v_mfma_f32_16x16x16_bf16.
    struct frag4 {
        bf16x4 v;
    };
    static __device__ inline void set4(frag4 &f, int i, float x) { f.v[i] = (bf16)x; }
    static __device__ inline void set4_raw(frag4 &f, int i, bf16 x) { f.v[i] = x; }
    static __device__ inline f32x4 mma16(const frag4 &a, const frag4 &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a.v, b.v, c, 0, 0, 0);
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
    struct frag4 {
        float e[4];
    };
    static __device__ inline void set4(frag4 &f, int i, float x) { f.e[i] = x; }
    static __device__ inline void set4_raw(frag4 &f, int i, float x) { f.e[i] = x; }
    static __device__ inline f32x4 mma16(const frag4 &a, const frag4 &b, f32x4 c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.e[i], b.e[i], c, 0, 0, 0);
        return c;
    }
    static constexpr bool kSplitU = false;
};

__device__ inline float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- int8 keys -------------------------------------------------------------
//
// Base keys stored as excess-128 int8 codes (byte u = code + 128) enter the
// score product as fp16 values 1024 + u = 1152 + code, which are exact: a byte
// permute builds {0x64, u_1, 0x64, u_0} for each pair of codes, and 0x64uu is
// the fp16 number 1024 + uu.  The query rows meet them in an fp16 MFMA; the
// constant 1152 * sum(q) per query row is taken off by starting the score
// accumulator at minus that value.
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));

// Four floats to fp16 (round to nearest even).
__device__ inline f16x4 to_f16x4(f32x4 x) { return __builtin_convertvector(x, f16x4); }

__device__ inline f16x8 codes_to_f16(uint32_t w0, uint32_t w1) {
    constexpr uint32_t kHi = 0x64646464u;  // v_perm_b32 selectors 4..7 take bytes of the first operand
    u32x4 r;
    r[0] = __builtin_amdgcn_perm(kHi, w0, 0x04010400u);  // {0x64, w0.b1, 0x64, w0.b0}
    r[1] = __builtin_amdgcn_perm(kHi, w0, 0x04030402u);  // {0x64, w0.b3, 0x64, w0.b2}
    r[2] = __builtin_amdgcn_perm(kHi, w1, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(kHi, w1, 0x04030402u);
    return __builtin_bit_cast(f16x8, r);
}

__device__ inline f32x4 mma_f16(const f16x8 &a, const f16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Four floats to bf16 (round to nearest even).
__device__ inline bf16x4 to_bf16x4(float a, float b, float c, float d) {
    const bf16x2 x = __builtin_convertvector(f32x2{a, b}, bf16x2);
    const bf16x2 y = __builtin_convertvector(f32x2{c, d}, bf16x2);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane p supplies the address of 4 consecutive 16-bit elements x_p[0..3];
// lane 4a + b receives {x_{4i+a}[b] : i = 0..3}.  With lane 4i + a pointing at
// row i, columns c + 4a of a row-major tile, lane 4a + b gets column c + 4a + b
// of rows 0..3: a 4-long column segment, as an MFMA operand wants it.
__device__ inline bf16x4 lds_tr4(const void *p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(__attribute__((address_space(3))) char *)p);
    return __builtin_bit_cast(bf16x4, v);
}

// ---- staging through LDS ---------------------------------------------------
//
// Tiles are copied from global memory into LDS with gfx950's direct loads
// (global_load_lds_dwordx4): one instruction moves 16 bytes per lane, lane l
// landing at LDS byte (base + 16 l), with no registers in between.  Rows of a
// tile are stored as 16-byte chunks, permuted within the row by an XOR with
// bits of the row index so that the MFMA operand reads (16 rows at one column,
// or one row across 16 lanes) touch distinct banks.

// Physical chunk of logical chunk c in row `row` of a region whose rows hold
// `cpa` (a power of two) chunks.  An involution: it also maps physical to logical.
__device__ inline int swz(int row, int c, int cpa, int lg) {
    return cpa >= 16 ? (c ^ (row & 15)) : (c ^ ((row >> (4 - lg)) & (cpa - 1)));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ inline uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

// One direct load: 16 bytes from gsrc (per lane) to LDS byte lds_base + 16*lane.
// lds_base must be wave-uniform: it is an M0 input operand ("{m0}"), so the
// compiler itself writes M0 and knows it is live here.  Written as inline
// assembly so that the compiler does not treat every later LDS read as
// dependent on it (it would wait for all outstanding loads before each read);
// completion is awaited explicitly with wait_vmcnt before the stage is read.
// One wait state (s_nop 0) between the M0 write and the load, which the
// compiler cannot see inside the statement.
__device__ inline void dma16(const void *gsrc, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "{m0}"(lds_base) : "memory");
}

// The same with a wave-uniform 64-bit base (SGPR pair) and a per-lane 32-bit
// byte offset (the instruction's saddr form).
__device__ inline void dma16s(const void *sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}

// One direct load of 4 bytes per lane: gsrc (per lane) to LDS byte lds_base + 4*lane.
__device__ inline void dma4(const void *gsrc, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gsrc), "{m0}"(lds_base) : "memory");
}

// Streaming variants (nontemporal bit): for data read exactly once, such as
// the base and private key/value rows.  On gfx950 the direct loads sustain
// about 7.3 TB/s with the bit against 5.9 TB/s without it (a one-workgroup-
// per-CU ring over 1 GiB); data that other workgroups re-read through L2 (the
// low-rank rows) keeps the default policy.
__device__ inline void dma16s_nt(const void *sbase, uint32_t voff, uint32_t lds_base) {
    lds_base = __builtin_amdgcn_readfirstlane(lds_base);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_base)
                 : "memory");
}

// A pointer that is the same in every lane, moved to scalar registers.
template <typename P>
__device__ inline P *uniform_ptr(P *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (P *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Requests every 64-byte line of the kernel's parameter block (a struct P
// passed by value, at the start of the kernel argument segment) at once and
// waits for them together.  The compiler reads parameter fields lazily, with a
// wait after each batch; without this, each batch that touches a new line is a
// separate round trip to memory at the start of every workgroup.
template <typename P>
__device__ __attribute__((always_inline)) inline void touch_params() {
    constexpr int kLines = (int)((sizeof(P) + 63) / 64);
    typedef const __attribute__((address_space(4))) uint32_t kword;
    kword *ka = (kword *)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kLines; ++i) acc ^= ka[16 * i];
    asm volatile("" ::"s"(acc));
}

// s_waitcnt vmcnt(n) (n clamped to the 6-bit field), leaving the other counters.
// The immediate must be a constant, hence the table.
__device__ inline void wait_vmcnt(int n) {
#define RATTN_VM(N) \
    case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (((N) >> 4) << 14) | (7 << 4) | (15 << 8)); break;
    switch (n < 63 ? (n > 0 ? n : 0) : 63) {
        RATTN_VM(0) RATTN_VM(1) RATTN_VM(2) RATTN_VM(3) RATTN_VM(4) RATTN_VM(5) RATTN_VM(6) RATTN_VM(7)
        RATTN_VM(8) RATTN_VM(9) RATTN_VM(10) RATTN_VM(11) RATTN_VM(12) RATTN_VM(13) RATTN_VM(14) RATTN_VM(15)
        RATTN_VM(16) RATTN_VM(17) RATTN_VM(18) RATTN_VM(19) RATTN_VM(20) RATTN_VM(21) RATTN_VM(22) RATTN_VM(23)
        RATTN_VM(24) RATTN_VM(25) RATTN_VM(26) RATTN_VM(27) RATTN_VM(28) RATTN_VM(29) RATTN_VM(30) RATTN_VM(31)
        RATTN_VM(32) RATTN_VM(33) RATTN_VM(34) RATTN_VM(35) RATTN_VM(36) RATTN_VM(37) RATTN_VM(38) RATTN_VM(39)
        RATTN_VM(40) RATTN_VM(41) RATTN_VM(42) RATTN_VM(43) RATTN_VM(44) RATTN_VM(45) RATTN_VM(46) RATTN_VM(47)
        RATTN_VM(48) RATTN_VM(49) RATTN_VM(50) RATTN_VM(51) RATTN_VM(52) RATTN_VM(53) RATTN_VM(54) RATTN_VM(55)
        RATTN_VM(56) RATTN_VM(57) RATTN_VM(58) RATTN_VM(59) RATTN_VM(60) RATTN_VM(61) RATTN_VM(62)
        default: __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (15 << 8)); break;
    }
#undef RATTN_VM
}

// Workgroup barrier for the staging ring: waits for this wave's own LDS reads
// (lgkmcnt(0)), then s_barrier.  No vmcnt(0): direct loads of later stages stay
// in flight (their completion is awaited explicitly with wait_vmcnt).  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ inline void ring_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Maxima of values that are never NaN (scores: finite or -inf), as v_max_f32 /
// v_max3_f32 written out.  fmaxf would first quiet each operand (IEEE mode), a
// v_max_f32 of the operand with itself, on the softmax's critical path.
__device__ inline float amax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ inline float amax3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Maximum over the four lanes l, l^16, l^32, l^48 (the lanes that hold one
// query row's scores), with gfx950's cross-lane swaps on the VALU instead of
// two LDS round trips.  permlane32_swap(x, x) leaves (x[l mod 32], x[l mod 32 + 32])
// in the two results; permlane16_swap does the same for 16-lane rows 0<->1 and 2<->3.
__device__ inline float row_max4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = amax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return amax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the four lanes l, l^16, l^32, l^48 (one query row's lanes), with
// the gfx950 lane swaps.
__device__ inline float row_sum4(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over the lanes l' of the wave with l' = l (mod g), g a power of two in
// 1..32, every such lane receiving it; all steps on the VALU: DPP rotations by 8
// and 4 within 16-lane rows (after the first, the values repeat with period 8,
// so a rotation adds the same partner as an xor would), quad permutes for 2 and
// 1, and the gfx950 lane swaps across rows (16) and halves (32).  No LDS round
// trip, unlike __shfl_xor.
template <int CTRL>
__device__ inline float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ inline float lane_group_sum(float x, int g) {
    if (g <= 8) x += dpp_mov<0x128>(x);  // row_ror:8
    if (g <= 4) x += dpp_mov<0x124>(x);  // row_ror:4
    if (g <= 2) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
    if (g <= 1) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
    if (g <= 16) {
        const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    }
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ inline float lane_max64(float x) {
    x = fmaxf(x, dpp_mov<0x128>(x));
    x = fmaxf(x, dpp_mov<0x124>(x));
    x = fmaxf(x, dpp_mov<0x4E>(x));
    x = fmaxf(x, dpp_mov<0xB1>(x));
    return row_max4(x);
}

}  // namespace rattn
