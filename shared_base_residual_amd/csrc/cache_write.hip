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
// column, k contiguous), the B operand 16 token rows of X, both read from LDS,
// so each lane ends with four consecutive columns of one token, stored as one
// 8-byte bf16 write.  Both operands stream through a four-stage LDS ring of
// 64-wide slices of the contraction (direct loads, three slices in flight):
// with 128 tokens per workgroup the A^T rows are as many bytes as the X rows,
// and the loop is bound by how many loads are in flight, not by the products.
#include "device.h"
#include "internal.h"

namespace rattn {

constexpr int kLrWaves = 4;           // waves per workgroup
constexpr int kLrTokWave = 32;        // tokens per wave (two 16-token MFMA blocks)
constexpr int kLrTok = kLrWaves * kLrTokWave;  // tokens per workgroup
constexpr int kLrCols = 128;          // output columns per workgroup (8 tiles of 16)
constexpr int kLrKc = 64;             // d_in per stage (128 bytes per row: 8 chunks of 16)
constexpr int kLrStages = 4;
constexpr int kLrRegion = 128 * kLrKc * 2;     // bytes of one region (A^T rows or X rows) of a stage
constexpr int kLrStage = 2 * kLrRegion;        // A^T region, then X region

// Row x of a region holds chunk q (16 bytes) at physical chunk q ^ ((x >> 1) & 7):
// the 16 rows an MFMA operand read touches (row pairs share a 256-byte bank
// line) land on distinct banks.
__device__ inline int lr_phys(int row, int q) { return q ^ ((row >> 1) & 7); }

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

    // ---- this wave's loads of a stage: each region is 128 rows x 8 chunks =
    // 16 direct loads of 64 chunks; wave w issues loads w, w + 4, w + 8, w + 12
    // of both.  Load i covers rows 8i .. 8i + 7; lane l writes physical chunk
    // l % 8 of row 8i + l / 8, read from that row's logical chunk.
    constexpr int kPer = 16 / kLrWaves;  // loads per region per wave
    const bf16 *a_src[kPer], *x_src[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int i = wave + kLrWaves * u;
        const int row = 8 * i + (lane >> 3);
        const int logical = lr_phys(row, lane & 7);  // the swizzle is its own inverse
        a_src[u] = a_row(c0 + (row < ncol ? row : ncol - 1)) + 8 * logical;  // rows past the block repeat a valid one
        int64_t t = tb * kLrTok + row;
        t = t < p.T ? t : p.T - 1;  // tokens past the end repeat the last one
        x_src[u] = x + t * p.d_in + 8 * logical;
    }
    const uint32_t lds0 = lds_addr(smem);
    auto fill = [&](int chunk, int stage) {
        const int64_t kofs = (int64_t)chunk * kLrKc;
        const uint32_t sb = lds0 + (uint32_t)(stage * kLrStage);
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int i = wave + kLrWaves * u;
            dma16(a_src[u] + kofs, sb + (uint32_t)(1024 * i));
            dma16(x_src[u] + kofs, sb + (uint32_t)(kLrRegion + 1024 * i));
        }
    };
    constexpr int kFpw = 2 * kPer;  // loads per wave per stage

    f32x4 acc[2][8];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[b][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nchunks = p.d_in / kLrKc;
    for (int i = 0; i < kLrStages - 1 && i < nchunks; ++i) fill(i, i);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int later = (nchunks - 1 - ch) < (kLrStages - 2) ? (nchunks - 1 - ch) : (kLrStages - 2);
        wait_vmcnt(later * kFpw);  // this wave's loads of slice ch have landed
        ring_barrier();            // ... everyone's, and everyone is done with slice ch - 1
        if (ch + kLrStages - 1 < nchunks) fill(ch + kLrStages - 1, (ch + kLrStages - 1) % kLrStages);
        const char *st = smem + (size_t)(ch % kLrStages) * kLrStage;
#pragma unroll
        for (int s = 0; s < kLrKc / 32; ++s) {
            Ops<bf16>::frag xf[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int row = kLrTokWave * wave + 16 * b + n16;
                xf[b] = Ops<bf16>::load8(
                    reinterpret_cast<const bf16 *>(st + kLrRegion + row * 128 + 16 * lr_phys(row, 4 * s + j4)));
            }
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                if (jj < nct) {
                    const int row = 16 * jj + n16;
                    const Ops<bf16>::frag af =
                        Ops<bf16>::load8(reinterpret_cast<const bf16 *>(st + row * 128 + 16 * lr_phys(row, 4 * s + j4)));
#pragma unroll
                    for (int b = 0; b < 2; ++b) acc[b][jj] = Ops<bf16>::mma(af, xf[b], acc[b][jj]);
                }
            }
        }
    }

    // ---- store: lane (n16, j4) holds columns c0 + 16 jj + 4 j4 + i of token tw + 16 b + n16
    const int64_t tw = tb * kLrTok + wave * kLrTokWave;
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
    const size_t lds = (size_t)kLrStages * kLrStage;
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
