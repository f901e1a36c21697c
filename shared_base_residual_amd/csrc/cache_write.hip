// cache_write.hip -- the cache-write path upstream of the attention kernels
// (gfx950): the rank-r projection that fills the low-rank caches, and the
// append of new base key/value rows into a paged pool with copy-on-write.
//
// Low-rank projection (ForkKV Guide, "Mathematical Decomposition of LoRA KV
// Activations": the residual cache may hold the factored X A; DualRadixTree
// Case B: on a base hit with an adapter miss only this projection runs;
// LRAgent, "Schemi di Condivisione": BaseShared recomputes each agent's LR
// cache X A_i on an agent switch, BaseLRShared shares A and so one LR cache):
//     Lk[n][pos0 + t] = X[t] A_k,n      Lv[n][pos0 + t] = X[t] A_v,n
// for T new tokens.  A streaming contraction: each byte of X is read once from
// HBM, while every set's A (small, L2-resident) is staged through LDS and
// reused by all the tokens of a workgroup, so the kernel is bound by the read
// of X.  With one X for all sets (the shared context's layer input), one read
// of X serves every agent's columns, as one base tile serves every agent in
// the attention kernels.
//
// MFMA form: out^T = A^T X^T over 16 columns x 16 tokens per tile
// (v_mfma_f32_16x16x32_bf16): the A operand is 16 rows of A^T (one per output
// column, k contiguous) read from LDS, the B operand 16 token rows of X read
// straight from global memory (16 bytes per lane), so each lane ends with four
// consecutive columns of one token, stored as one 8-byte bf16 write.
#include "device.h"
#include "internal.h"

namespace rattn {

constexpr int kLrWaves = 4;           // waves per workgroup
constexpr int kLrTokWave = 32;        // tokens per wave (two 16-token MFMA blocks)
constexpr int kLrTok = kLrWaves * kLrTokWave;  // tokens per workgroup
constexpr int kLrCols = 128;          // output columns per workgroup (8 tiles of 16)
constexpr int kLrKc = 128;            // d_in per LDS chunk (256 bytes per A^T row)

// LDS: two chunks of kLrCols A^T rows of kLrKc bf16 (16 chunks of 16 bytes per
// row, chunk q of row c stored at chunk q ^ (c & 15), so that 16 lanes reading
// one logical chunk of 16 rows touch distinct banks).
__global__ __launch_bounds__(64 * kLrWaves) void lr_project_kernel(LrParams p) {
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, j4 = lane >> 4;
    const int64_t tb = blockIdx.x;
    const int cb = blockIdx.y;  // column block
    // column block -> (X set, first global column, columns in the block)
    const int cpb = p.cols_per_xset;  // columns one X set feeds (all sets' 2r when X is shared)
    const int blocks_per_x = (cpb + kLrCols - 1) / kLrCols;
    const int xs = cb / blocks_per_x;
    const int c0 = xs * cpb + (cb - xs * blocks_per_x) * kLrCols;
    const int ncol = cpb - (c0 - xs * cpb) < kLrCols ? cpb - (c0 - xs * cpb) : kLrCols;
    const int nct = (ncol + 15) >> 4;  // 16-column tiles in use (wave-uniform)
    const bf16 *x = static_cast<const bf16 *>(p.x) + (int64_t)xs * p.T * p.d_in;

    // A^T row of global column c: set n = c / 2r, k or v by (c / r) % 2, row c % r
    auto a_row = [&](int c) -> const bf16 * {
        const int n = c / (2 * p.r), rem = c - n * 2 * p.r;
        const int kv = rem >= p.r, j = rem - kv * p.r;
        const int na = p.shared_a ? 0 : n;
        return static_cast<const bf16 *>(kv ? p.av : p.ak) + ((int64_t)na * p.r + j) * p.d_in;
    };

    // ---- this wave's share of each A^T chunk fill: kLrCols rows x 16 chunks =
    // 2048 chunks, 32 direct loads of 64 chunks; wave w issues loads w, w + 4, ...
    // Load i covers rows 4i .. 4i + 3; lane l writes LDS chunk 64 i + l (row
    // 4i + l / 16, physical chunk l % 16) from logical chunk (l % 16) ^ (row & 15).
    constexpr int kLoads = kLrCols * 16 / 64;
    constexpr int kLoadsPerWave = kLoads / kLrWaves;
    uint32_t a_goff[kLoadsPerWave];  // byte offset within the chunk's k range
    const bf16 *a_src[kLoadsPerWave];
#pragma unroll
    for (int u = 0; u < kLoadsPerWave; ++u) {
        const int i = wave + kLrWaves * u;
        const int row = 4 * i + (lane >> 4);
        const int phys = lane & 15, logical = phys ^ (row & 15);
        const int c = c0 + (row < ncol ? row : ncol - 1);  // rows past the block repeat a valid one
        a_src[u] = a_row(c);
        a_goff[u] = (uint32_t)(16 * logical);
    }
    const uint32_t lds0 = lds_addr(smem);
    auto fill = [&](int chunk, int buf) {
        const int64_t kofs = (int64_t)chunk * kLrKc;
#pragma unroll
        for (int u = 0; u < kLoadsPerWave; ++u) {
            const int i = wave + kLrWaves * u;
            const char *g = reinterpret_cast<const char *>(a_src[u] + kofs) + a_goff[u];
            dma16(g, lds0 + (uint32_t)(buf * kLrCols * 256 + 1024 * i));
        }
    };

    // ---- this wave's token rows (B operand), clamped to the last token
    const int64_t tw = tb * kLrTok + wave * kLrTokWave;
    const bf16 *xr[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        int64_t t = tw + 16 * b + n16;
        t = t < p.T ? t : p.T - 1;
        xr[b] = x + t * p.d_in + 8 * j4;
    }

    f32x4 acc[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[b][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = p.d_in / kLrKc;
    // X operands of a chunk: 4 contraction steps of 32 x 2 token blocks
    Ops<bf16>::frag xf[2][4], xn[2][4];
    auto load_x = [&](Ops<bf16>::frag (&dst)[2][4], int chunk) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) dst[b][s] = Ops<bf16>::load8(xr[b] + chunk * kLrKc + 32 * s);
    };
    fill(0, 0);
    load_x(xf, 0);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int buf = ch & 1;
        // the next chunk's A^T rows and X rows are requested before this chunk's products
        if (ch + 1 < nchunks) {
            fill(ch + 1, buf ^ 1);
            load_x(xn, ch + 1);
            wait_vmcnt(kLoadsPerWave + 8);  // this chunk's fill (and X) landed; the next one's in flight
        } else {
            wait_vmcnt(0);
        }
        __syncthreads();  // every wave's share of this chunk's A^T rows is in LDS
        const char *st = smem + buf * kLrCols * 256;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                if (jj < nct) {
                    const int row = 16 * jj + n16;
                    const int phys = (4 * s + j4) ^ (row & 15);
                    Ops<bf16>::frag af = Ops<bf16>::load8(
                        reinterpret_cast<const bf16 *>(st + row * 256 + 16 * phys));
#pragma unroll
                    for (int b = 0; b < 2; ++b) acc[b][jj] = Ops<bf16>::mma(af, xf[b][s], acc[b][jj]);
                }
            }
        }
        __syncthreads();  // everyone is done with this buffer before it is refilled
        if (ch + 1 < nchunks) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) xf[b][s] = xn[b][s];
        }
    }

    // ---- store: lane (n16, j4) holds columns c0 + 16 jj + 4 j4 + i of token tw + 16 b + n16
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t t = tw + 16 * b + n16;
        if (t >= p.T) continue;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int cl = 16 * jj + 4 * j4;
            if (jj >= nct || cl >= ncol) continue;
            const int c = c0 + cl;
            const int n = c / (2 * p.r), rem = c - n * 2 * p.r;
            const int kv = rem >= p.r, j = rem - kv * p.r;
            bf16 *dst = static_cast<bf16 *>(kv ? p.lv : p.lk) + ((int64_t)n * p.cache_len + p.pos0 + t) * p.r + j;
            const bf16x4 v = to_bf16x4(acc[b][jj][0], acc[b][jj][1], acc[b][jj][2], acc[b][jj][3]);
            __builtin_memcpy(__builtin_assume_aligned(dst, 8), &v, 8);
        }
    }
}

hipError_t launch_lr_project(const LrParams &p, hipStream_t st) {
    if (p.T == 0) return hipSuccess;
    const int64_t tblocks = (p.T + kLrTok - 1) / kLrTok;
    const int blocks_per_x = (p.cols_per_xset + kLrCols - 1) / kLrCols;
    const size_t lds = 2 * kLrCols * 256;
    struct Slot {};
    const hipError_t e = ensure_lds<Slot>(reinterpret_cast<const void *>(lr_project_kernel), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(lr_project_kernel, dim3((unsigned)tblocks, (unsigned)(p.n_xsets * blocks_per_x)),
                       dim3(64 * kLrWaves), lds, st, p);
    return hipGetLastError();
}

// ------------------------------------------------------------ paged append --
//
// Appends T new rows per KV head at logical positions cur_len .. cur_len+T-1
// of a sequence whose (already updated) block table is `table`, into both
// pools; and, when the plan copied a shared page (copy-on-write: the first
// write to a shared page goes to a private copy), fills rows 0 .. off-1
// (off = cur_len % page) of every head of the copy from the shared original.
// The two parts touch disjoint rows, so one launch does both.  Pure data
// movement in 16-byte vectors: the result is byte-exact.
__global__ __launch_bounds__(256) void append_kv_kernel(AppendParams p) {
    const int64_t rv = p.row_vec;
    const int64_t n_copy = (int64_t)p.HK * p.off * rv;
    const int64_t n_all = n_copy + (int64_t)p.HK * p.T * rv;
    const u32x4 *kn = static_cast<const u32x4 *>(p.k_new), *vn = static_cast<const u32x4 *>(p.v_new);
    u32x4 *pk = static_cast<u32x4 *>(p.pool_k), *pv = static_cast<u32x4 *>(p.pool_v);
    for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < n_all; v += (int64_t)gridDim.x * blockDim.x) {
        if (v < n_copy) {
            const int64_t row = v / rv, c = v - row * rv;
            const int64_t h = row / p.off, slot = row - h * p.off;
            const int64_t src = (((int64_t)p.cow_src * p.HK + h) * p.ps + slot) * rv + c;
            const int64_t dst = (((int64_t)p.cow_dst * p.HK + h) * p.ps + slot) * rv + c;
            pk[dst] = pk[src];
            pv[dst] = pv[src];
        } else {
            const int64_t w = v - n_copy;
            const int64_t row = w / rv, c = w - row * rv;
            const int64_t h = row / p.T, t = row - h * p.T;
            const int64_t pos = p.cur_len + t;
            const int64_t lp = pos / p.ps, slot = pos - lp * p.ps;
            const int64_t page = p.table[lp];
            const int64_t dst = ((page * p.HK + h) * p.ps + slot) * rv + c;
            pk[dst] = kn[(h * p.T + t) * rv + c];
            pv[dst] = vn[(h * p.T + t) * rv + c];
        }
    }
}

hipError_t launch_append_kv(const AppendParams &p, hipStream_t st) {
    const int64_t n_all = ((int64_t)p.HK * p.off + (int64_t)p.HK * p.T) * p.row_vec;
    if (n_all == 0) return hipSuccess;
    int64_t blocks = (n_all + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace rattn
