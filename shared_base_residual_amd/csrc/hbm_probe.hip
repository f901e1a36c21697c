// hbm_probe.hip -- achievable HBM read bandwidth of this GPU (gfx950), for the
// benchmark's roofline figures.  Not part of librattn: a separate small
// library (libhbm_probe.so) that bench.py loads to report the read rate a
// streaming kernel reaches beside the 8 TB/s specification.
//
// Two readers of one contiguous buffer, each touching every byte once:
//   * vector loads: every thread streams 16-byte nontemporal loads
//     (global_load_dwordx4 nt) over a grid-strided range, eight in flight,
//     and folds them into one word per workgroup (so that nothing is elided);
//   * direct loads into LDS: each workgroup streams a contiguous slice through
//     a four-stage LDS ring with global_load_lds_dwordx4 (nontemporal), the
//     load form the attention kernels use.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_vec(const u32x4 *__restrict__ src, int64_t n16, uint32_t *sink) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    // one word per workgroup (lane 0 of each wave XORs in; order does not matter)
    if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

// Direct loads: workgroup b streams bytes [b * per, (b + 1) * per) of the
// buffer (per a multiple of 4 KiB x waves) through a ring of 4 stages of
// `waves` KiB each; every wave loads 1 KiB per stage and waits for its own
// loads three stages later.  The LDS contents are never read: the loads' only
// effect is the traffic, which is what is measured.
__global__ __launch_bounds__(512) void probe_lds(const char *__restrict__ src, int64_t per, uint32_t *sink) {
    extern __shared__ __attribute__((aligned(16))) char ring[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const char *base = src + (int64_t)blockIdx.x * per + (int64_t)wave * 1024 + 16 * lane;
    const int64_t step = (int64_t)nw * 1024;
    const int64_t n = per / step;
    for (int64_t s = 0; s < n; ++s) {
        const uint32_t lds = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)ring +
                             (uint32_t)(((s & 3) * nw + wave) * 1024);
        const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(base + s * step), "{m0}"(m0) : "memory");
        if (s >= 3) __builtin_amdgcn_s_waitcnt((3 & 15) | ((3 >> 4) << 14) | (7 << 4) | (15 << 8));  // vmcnt(3)
    }
    __builtin_amdgcn_s_waitcnt((0) | (0 << 14) | (7 << 4) | (15 << 8));  // vmcnt(0)
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = reinterpret_cast<const uint32_t *>(ring)[0];
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) of device memory at `buf` once with the
// vector-load reader: `blocks` workgroups of 256 threads.  `sink` holds at
// least `blocks` words (written, not cleared).  Returns a hipError_t.
int hbm_probe_vec(const void *buf, int64_t bytes, void *sink, int blocks, void *stream) {
    if (!buf || !sink || bytes % 16 || blocks < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_vec, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4 *)buf, bytes / 16, (uint32_t *)sink);
    return (int)hipGetLastError();
}

// The same with the direct-load reader: `blocks` workgroups of `waves` waves
// (1..8), each over bytes / blocks contiguous bytes, which must be a multiple
// of waves KiB.  Uses 4 * waves KiB of LDS per workgroup.
int hbm_probe_lds(const void *buf, int64_t bytes, void *sink, int blocks, int waves, void *stream) {
    if (!buf || !sink || blocks < 1 || waves < 1 || waves > 8) return (int)hipErrorInvalidValue;
    const int64_t per = bytes / blocks;
    if (per * blocks != bytes || per % ((int64_t)waves * 1024)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_lds, dim3(blocks), dim3(64 * waves), 4 * waves * 1024, (hipStream_t)stream,
                       (const char *)buf, per, (uint32_t *)sink);
    return (int)hipGetLastError();
}

}  // extern "C"
