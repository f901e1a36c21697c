// quant.hip -- base keys to int8 codes with one scale per tensor (gfx950).
//
// PolyKV (section 2B, asymmetric compression) stores the shared pool's keys
// as int8 with per-tensor linear quantisation, written once and read by every
// agent.  Here: amax = max |K| over the n given elements, scale s = amax / 127
// (an fp64 division rounded once to fp32; s = 1 when amax = 0), and each code
// is round-half-to-even(K / s) in fp64, clamped to [-127, 127] and stored as
// the byte code + 128 (excess-128), the form the attention kernels read.
// Four small launches on one stream: clear the maximum, reduce it, form the
// scale, write the codes.  The reduction is an atomic maximum over the
// non-negative floats' bit patterns, so the result does not depend on order.
#include "device.h"

namespace rattn {

__global__ __launch_bounds__(64) void quant_clear(uint32_t *slot) {
    if (threadIdx.x == 0) slot[0] = 0u;
}

template <typename T>
__global__ __launch_bounds__(256) void quant_amax(const T *__restrict__ k, int64_t n, uint32_t *slot) {
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        m = fmaxf(m, fabsf((float)k[i]));
    m = lane_max64(m);
    if ((threadIdx.x & 63) == 0) atomicMax(slot, __float_as_uint(m));  // m >= 0: bits order as values
}

__global__ __launch_bounds__(64) void quant_scale(uint32_t *slot) {
    if (threadIdx.x == 0) {
        const float amax = __uint_as_float(slot[0]);
        const float s = amax > 0.0f ? (float)((double)amax / 127.0) : 1.0f;
        slot[0] = __float_as_uint(s);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void quant_codes(const T *__restrict__ k, int64_t n, const float *scale,
                                                   uint8_t *__restrict__ codes) {
    const double s = (double)scale[0];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        double x = __builtin_rint((double)(float)k[i] / s);
        x = x < -127.0 ? -127.0 : (x > 127.0 ? 127.0 : x);
        codes[i] = (uint8_t)((int)x + 128);
    }
}

template <typename T>
static hipError_t quantize_t(const void *k, int64_t n, void *codes, float *scale, hipStream_t st) {
    uint32_t *slot = reinterpret_cast<uint32_t *>(scale);
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(quant_clear, dim3(1), dim3(64), 0, st, slot);
    hipLaunchKernelGGL((quant_amax<T>), dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const T *>(k), n, slot);
    hipLaunchKernelGGL(quant_scale, dim3(1), dim3(64), 0, st, slot);
    hipLaunchKernelGGL((quant_codes<T>), dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const T *>(k), n,
                       static_cast<const float *>(scale), static_cast<uint8_t *>(codes));
    return hipGetLastError();
}

hipError_t launch_quantize(const void *k, int64_t n, int bf16_in, void *codes, float *scale, hipStream_t st) {
    return bf16_in ? quantize_t<bf16>(k, n, codes, scale, st) : quantize_t<float>(k, n, codes, scale, st);
}

}  // namespace rattn
