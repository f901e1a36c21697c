// values3.hip -- base values to 3-bit codes after a Walsh-Hadamard rotation
// (gfx950).
//
// PolyKV (section 2B, TurboQuant MSE) rotates every value vector with a fast
// Walsh-Hadamard transform, so that its coordinates approach a standard
// normal, and maps each coordinate to one of eight Lloyd-Max centroids for
// N(0, 1).  Here, per vector v of d elements (one wave per vector):
//   z = H_d v (Sylvester order, entries +-1) by butterflies in fp64: lane l
//     holds coordinates l (and l + 64 for d = 128); strides below 64 pair
//     lanes l and l ^ h, stride 64 pairs a lane's two coordinates.  The
//     stages commute and every sum of +-1 multiples of bf16 values is exact
//     in fp64, so z does not depend on the order;
//   ||v||^2 summed over the wave in fp64, ||v|| = sqrt (correctly rounded);
//   u_j = z_j / ||v|| (0 for a zero vector); code_j = #{k : u_j >= b_k} over
//     the seven inner boundaries of the quantiser (host-derived, fp64);
//   bit plane p of the codes = the wave's ballot of bit p (coordinate j at
//     bit j of the 64-bit word of its half), stored as three planes of d / 8
//     bytes; scale = fp32(||v|| / d).
#include "device.h"

namespace rattn {

struct ValuesCodebook {
    double b[7];  // inner boundaries, ascending
};

template <typename T, int D>
__global__ __launch_bounds__(256) void values3_encode(const T *__restrict__ v, int64_t n, ValuesCodebook cb,
                                                      uint8_t *__restrict__ codes, float *__restrict__ scale) {
    constexpr int NS = D / 64;  // coordinates per lane
    const int lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    for (int64_t i = w0; i < n; i += nw) {
        double z[NS];
        double ss = 0.0;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            z[s] = (double)(float)v[i * D + 64 * s + lane];
            ss += z[s] * z[s];
        }
        // ||v||^2 over the wave (every lane ends with the sum)
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) ss += __shfl_xor(ss, h);
        // z = H_d v: stride 64 within the lane, then strides 32 .. 1 across lanes
        if constexpr (NS == 2) {
            const double a = z[0], b = z[1];
            z[0] = a + b;
            z[1] = a - b;
        }
#pragma unroll
        for (int h = 32; h >= 1; h >>= 1) {
            const bool hi = (lane & h) != 0;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const double o = __shfl_xor(z[s], h);
                z[s] = hi ? o - z[s] : z[s] + o;
            }
        }
        const double nrm = __builtin_sqrt(ss);
        uint64_t planes[3][NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const double u = nrm > 0.0 ? z[s] / nrm : 0.0;
            int c = 0;
#pragma unroll
            for (int k = 0; k < 7; ++k) c += u >= cb.b[k] ? 1 : 0;
#pragma unroll
            for (int p = 0; p < 3; ++p) planes[p][s] = __builtin_amdgcn_ballot_w64(((c >> p) & 1) != 0);
        }
        // lanes 0 .. 3 NS - 1 store one 64-bit word each: plane k / NS, half k % NS
        if (lane < 3 * NS) {
            uint64_t word = 0;
#pragma unroll
            for (int k = 0; k < 3 * NS; ++k)
                if (lane == k) word = planes[k / NS][k % NS];
            *reinterpret_cast<uint64_t *>(codes + i * (3 * D / 8) + 8 * lane) = word;
        }
        if (lane == 0) scale[i] = (float)(nrm / (double)D);
    }
}

template <typename T, int D>
static hipError_t encode_t(const void *v, int64_t n, const ValuesCodebook &cb, void *codes, float *scale,
                           hipStream_t st) {
    int64_t blocks = (n + 3) / 4;  // four waves (vectors) per workgroup
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL((values3_encode<T, D>), dim3((unsigned)blocks), dim3(256), 0, st, static_cast<const T *>(v),
                       n, cb, static_cast<uint8_t *>(codes), scale);
    return hipGetLastError();
}

hipError_t launch_values3_encode(const void *v, int64_t n, int D, int bf16_in, const double *boundaries, void *codes,
                                 float *scale, hipStream_t st) {
    ValuesCodebook cb;
    for (int k = 0; k < 7; ++k) cb.b[k] = boundaries[k];
    if (D == 128)
        return bf16_in ? encode_t<bf16, 128>(v, n, cb, codes, scale, st) : encode_t<float, 128>(v, n, cb, codes, scale, st);
    return bf16_in ? encode_t<bf16, 64>(v, n, cb, codes, scale, st) : encode_t<float, 64>(v, n, cb, codes, scale, st);
}

}  // namespace rattn
