// gather.hip -- logical base cache from a paged pool (gfx950).
//
// Logical base token j of KV head k lives in slot j % page of physical page
// table[j / page] (the page table plays the part of the bCache block pointers
// of the ForkKV Guide's DualRadixTree lookup).  Pure data movement: 16-byte
// vector copies, byte-exact.  Also the optional debug check of a table: a
// count of its entries outside the pool, reading nothing but the table.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (KV head, logical page); row bytes are a multiple of 16.
__global__ __launch_bounds__(256) void gather_base_kernel(const u32x4 *__restrict__ pool,
                                                          const int32_t *__restrict__ table,
                                                          u32x4 *__restrict__ dst, int64_t L, int HK, int ps,
                                                          int row_vec) {
    const int64_t n_pages = (L + ps - 1) / ps;
    const int64_t b = blockIdx.x;
    const int k = (int)(b % HK);
    const int64_t lp = b / HK;
    if (lp >= n_pages) return;
    const int64_t phys = table[lp];
    const int64_t j0 = lp * ps;
    const int rows = (int)(L - j0 < ps ? L - j0 : ps);
    const u32x4 *src = pool + ((phys * HK + k) * ps) * row_vec;
    u32x4 *d = dst + ((int64_t)k * L + j0) * row_vec;
    for (int i = threadIdx.x; i < rows * row_vec; i += blockDim.x) d[i] = src[i];
}

hipError_t launch_gather(const void *pool, const int32_t *table, void *dst, int64_t L, int HK, int ps,
                         int row_bytes, hipStream_t st) {
    const int64_t n_pages = (L + ps - 1) / ps;
    if (n_pages == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_base_kernel, dim3((unsigned)(n_pages * HK)), dim3(256), 0, st,
                       static_cast<const u32x4 *>(pool), table, static_cast<u32x4 *>(dst), L, HK, ps,
                       row_bytes / 16);
    return hipGetLastError();
}

// The debug check of a table: one workgroup counts the entries outside
// [0, n_phys) (a grid-stride walk, then a workgroup sum through LDS) and
// writes the count.  The table alone is read; no entry is followed.
__global__ __launch_bounds__(1024) void check_table_kernel(const int32_t *__restrict__ table, int64_t n,
                                                           int64_t n_phys, int32_t *bad) {
    __shared__ int s_cnt[16];
    int c = 0;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int64_t e = table[i];
        c += (e < 0 || e >= n_phys) ? 1 : 0;
    }
    for (int h = 32; h >= 1; h >>= 1) c += __shfl_xor(c, h);
    if ((threadIdx.x & 63) == 0) s_cnt[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += s_cnt[w];
        bad[0] = t;
    }
}

hipError_t launch_check_table(const int32_t *table, int64_t n, int64_t n_phys, int32_t *bad, hipStream_t st) {
    hipLaunchKernelGGL(check_table_kernel, dim3(1), dim3(1024), 0, st, table, n, n_phys, bad);
    return hipGetLastError();
}

}  // namespace rattn
