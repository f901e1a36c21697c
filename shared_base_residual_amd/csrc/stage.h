// stage.h -- the LDS staging ring shared by the librattn kernels (gfx950):
// stage geometry, where a work item's tokens come from, the direct-load fill
// of one stage, and lane offsets of the MFMA operand reads.  Internal header.
#pragma once
#include "device.h"
#include "internal.h"

namespace rattn {

// ------------------------------------------------------------- geometry --

// Layout of one LDS stage, in 16-byte chunks: K rows, V rows, Lk rows, Lv rows.
struct Geo {
    int T;                    // tokens per stage
    int nst;                  // stages in the ring
    int cpr_kv, lg_kv;        // chunks per K (or V) row, its log2
    int cpr_lr, cpa_lr, lg_lr;  // valid / allocated (power of two) chunks per Lk row
    int ofs_v, ofs_lk, ofs_lv;  // region offsets (chunks)
    int chunks;               // chunks per stage
    int stage_bytes;          // stride between stages
};

__device__ inline int ilog2(int x) { return 31 - __builtin_clz(x); }

// Where the tokens of a work item come from.
template <typename T>
struct Src {
    const T *kb, *vb;         // contiguous: this head's rows; paged: pool + this head's offset
    int64_t page_stride;      // paged: elements per physical page (0: contiguous)
    int ps;                   // page size (paged)
    int pg0;                  // first logical page of the split
    const int *pages;         // LDS copy of the split's page-table entries (paged)
    const T *lk, *lv;         // low-rank rows: first agent of the workgroup (or the shared one)
    int64_t lr_agent_stride;  // elements between agents' low-rank caches
    int r;                    // rank
    int lr_es_shift;          // log2(r * sizeof(T) / 16): chunks per agent row
    int tlast;                // last valid token of the item
};

template <typename T, int D>
__device__ inline const T *kv_row(const Src<T> &s, const T *base, int tok) {
    if (s.page_stride) {
        const int64_t pg = s.pages[tok / s.ps - s.pg0];
        return base + pg * s.page_stride + (int64_t)(tok % s.ps) * D;
    }
    return base + (int64_t)tok * D;
}

// ------------------------------------------------------------ stage fill --
//
// A stage holds four regions of the tile: K rows, V rows, Lk rows, Lv rows (the
// last two only with a residual).  The tile's rows are cut into 16-row groups;
// wave w fills group w % G (G = T / 16) of the regions r with
// (r * G + w % G) % nw == w (nw waves), so every wave fills a fixed part: one
// page lookup and one uniform base per region and tile, and lane offsets that
// depend on the lane only (the swizzle repeats every 16 rows).  Each direct load
// moves 64 chunks of 16 bytes; a region row of cpa chunks gives 16 * cpa chunks
// per group, ceil(16 * cpa / 64) loads (the last one partial when 16 * cpa < 64).
// Lane offsets are 32-bit: the low-rank rows one workgroup reads span less than
// 2^31 bytes (checked on the host).

constexpr int kMaxKvLoads = 8;   // direct loads per group of a K (or V) region (fp32, d = 128)

struct FillPlan {
    int G, g;                 // groups per tile, this wave's group
    bool rK, rV, rL, rLv;     // regions this wave fills
    int n_kv, n_lr;           // loads per group of a K/V region, of an Lk/Lv region
    int fpw;                  // loads this wave issues per stage
    uint32_t kv_off[kMaxKvLoads];  // lane byte offset from the group's first K/V row
    int kv_row[kMaxKvLoads];       // lane's row within the group (for clamping)
    uint32_t lr_stride;            // bytes between agents' low-rank caches
    bool kv_nt;                    // K/V rows are read by this workgroup only: stream them
};

template <typename T, int D>
__device__ __attribute__((always_inline)) inline void make_fill_plan(FillPlan &f, const Geo &g, const Src<T> &s,
                                                                     bool resid, int wave, int lane, int nw = 4) {
    constexpr int ES = (int)sizeof(T);
    // (group, region) pairs pi = region * G + group go round-robin to the waves:
    // wave w fills the pairs with pi % nw == w (nw a multiple of G)
    f.G = g.T >> 4;
    f.g = wave % f.G;
    auto mine = [&](int region) { return (region * f.G + f.g) % nw == wave; };
    f.rK = mine(0);
    f.rV = mine(1);
    f.rL = resid && mine(2);
    f.rLv = resid && mine(3);
    f.n_kv = (16 * g.cpr_kv) >> 6;
    f.n_lr = resid ? ((16 * g.cpa_lr + 63) >> 6) : 0;
    f.fpw = (f.rK ? f.n_kv : 0) + (f.rV ? f.n_kv : 0) + (f.rL ? f.n_lr : 0) + (f.rLv ? f.n_lr : 0);
#pragma unroll
    for (int i = 0; i < kMaxKvLoads; ++i) {
        const int q = 64 * i + lane;
        const int row = q >> g.lg_kv;
        const int c = swz(row, q & (g.cpr_kv - 1), g.cpr_kv, g.lg_kv);
        f.kv_row[i] = row;
        f.kv_off[i] = (uint32_t)(row * D * ES + 16 * c);
    }
    f.lr_stride = (uint32_t)(s.lr_agent_stride * ES);
    f.kv_nt = false;
}

// Lane byte offset of low-rank load i of a group (agent, row and chunk), and the
// lane's row within the group.  Computed per load: a workgroup issues few.
template <typename T>
__device__ inline uint32_t lr_lane_off(const FillPlan &f, const Geo &g, const Src<T> &s, int i, int lane, int *row_out) {
    constexpr int ES = (int)sizeof(T);
    const int q = 64 * i + lane;
    const int row = q >> g.lg_lr;
    int c = swz(row, q & (g.cpa_lr - 1), g.cpa_lr, g.lg_lr);
    c = c < g.cpr_lr ? c : 0;  // allocated-only chunk: any valid data (never read)
    const int agent = c >> s.lr_es_shift;
    const int cin = c - (agent << s.lr_es_shift);
    *row_out = row < 16 ? row : 15;
    return (uint32_t)(row * s.r * ES + 16 * cin) + (uint32_t)agent * f.lr_stride;
}

// Issues this wave's loads of the tile starting at token t0 into `stage`.
// clamp: rows past the item's last token read that token instead (the tail
// tile); otherwise every row is valid and a uniform base per region serves.
// Always the same number of loads per wave (f.fpw), which the ring's waits count.
template <typename T, int D>
__device__ __attribute__((always_inline)) inline void fill_stage(const FillPlan &f, const Geo &g, const Src<T> &s, int t0, char *stage, bool clamp,
                                  int lane) {
    constexpr int ES = (int)sizeof(T);
    const int tg0 = t0 + 16 * f.g;  // the group's first token
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(stage));
    if (!clamp) {
        if (f.rK || f.rV) {
            const char *kb = uniform_ptr(reinterpret_cast<const char *>(kv_row<T, D>(s, s.kb, tg0)));
            const char *vb = uniform_ptr(reinterpret_cast<const char *>(kv_row<T, D>(s, s.vb, tg0)));
            const uint32_t lk0 = lds0 + 16 * (16 * f.g * g.cpr_kv), lv0 = lds0 + 16 * (g.ofs_v + 16 * f.g * g.cpr_kv);
            if (f.kv_nt) {
#pragma unroll
                for (int i = 0; i < kMaxKvLoads; ++i)
                    if (i < f.n_kv && f.rK) dma16s_nt(kb, f.kv_off[i], lk0 + 1024 * i);
#pragma unroll
                for (int i = 0; i < kMaxKvLoads; ++i)
                    if (i < f.n_kv && f.rV) dma16s_nt(vb, f.kv_off[i], lv0 + 1024 * i);
            } else {
#pragma unroll
                for (int i = 0; i < kMaxKvLoads; ++i)
                    if (i < f.n_kv && f.rK) dma16s(kb, f.kv_off[i], lk0 + 1024 * i);
#pragma unroll
                for (int i = 0; i < kMaxKvLoads; ++i)
                    if (i < f.n_kv && f.rV) dma16s(vb, f.kv_off[i], lv0 + 1024 * i);
            }
        }
        if (f.rL || f.rLv) {
            const char *lk = uniform_ptr(reinterpret_cast<const char *>(s.lk + (int64_t)tg0 * s.r));
            const char *lv = uniform_ptr(reinterpret_cast<const char *>(s.lv + (int64_t)tg0 * s.r));
            const int nchunk = 16 * g.cpa_lr;  // chunks of one group of a low-rank region
            for (int i = 0; i < f.n_lr; ++i) {
                if (64 * i + lane < nchunk) {
                    int row;
                    const uint32_t off = lr_lane_off(f, g, s, i, lane, &row);
                    if (f.rL) dma16s(lk, off, lds0 + 16 * (g.ofs_lk + 16 * f.g * g.cpa_lr) + 1024 * i);
                    if (f.rLv) dma16s(lv, off, lds0 + 16 * (g.ofs_lv + 16 * f.g * g.cpa_lr) + 1024 * i);
                }
            }
        }
        return;
    }
    // tail tile: per-lane rows, clamped to the item's last token
#pragma unroll
    for (int i = 0; i < kMaxKvLoads; ++i) {
        if (i < f.n_kv && (f.rK || f.rV)) {
            int tok = tg0 + f.kv_row[i];
            tok = tok < s.tlast ? tok : s.tlast;
            const uint32_t rowoff = f.kv_off[i] - (uint32_t)(f.kv_row[i] * D * ES);  // chunk part
            // (the tail tile: the default policy serves)
            if (f.rK)
                dma16(reinterpret_cast<const char *>(kv_row<T, D>(s, s.kb, tok)) + rowoff,
                      lds0 + 16 * (16 * f.g * g.cpr_kv) + 1024 * i);
            if (f.rV)
                dma16(reinterpret_cast<const char *>(kv_row<T, D>(s, s.vb, tok)) + rowoff,
                      lds0 + 16 * (g.ofs_v + 16 * f.g * g.cpr_kv) + 1024 * i);
        }
    }
    // (the loads are issued K then V per i here; the count per wave is the same)
    const int nchunk = 16 * g.cpa_lr;
    for (int i = 0; i < f.n_lr; ++i) {
        if ((f.rL || f.rLv) && 64 * i + lane < nchunk) {
            int row;
            const uint32_t off = lr_lane_off(f, g, s, i, lane, &row);
            int tok = tg0 + row;
            tok = tok < s.tlast ? tok : s.tlast;
            const uint32_t rel = off - (uint32_t)(row * s.r * ES);  // agent and chunk part
            if (f.rL)
                dma16(reinterpret_cast<const char *>(s.lk + (int64_t)tok * s.r) + rel,
                      lds0 + 16 * (g.ofs_lk + 16 * f.g * g.cpa_lr) + 1024 * i);
            if (f.rLv)
                dma16(reinterpret_cast<const char *>(s.lv + (int64_t)tok * s.r) + rel,
                      lds0 + 16 * (g.ofs_lv + 16 * f.g * g.cpa_lr) + 1024 * i);
        }
    }
}

// Byte offsets (within a stage) of the LDS operands a lane reads in a 16-token
// step, for the step's first row at 0; a step at row0 adds row0 * row bytes.
// All rows a lane touches are row0 + x with x < 16, and row0 is a multiple of
// 16, so the swizzle depends on x only.
template <typename T, int D, int CPAD>
struct ReadOfs {
    static constexpr int ES = (int)sizeof(T);
    static constexpr int FC = 8 * ES / 16;                                  // chunks per 8-element fragment
    static constexpr int VB = (D / 16) * ES, VC = VB >= 16 ? VB / 16 : 1;  // a value-row segment
    static constexpr int CPL = CPAD > 0 ? CPAD / 16 : 1;
    static constexpr int LB = CPL * ES, LC = LB >= 16 ? LB / 16 : 1;        // a low-rank value segment
    static constexpr int CSx = CPAD > 0 ? CPAD / 32 : 1;
    uint32_t k[D / 32][FC];
    uint32_t v[4][VC];
    uint32_t lk[CSx][FC];
    uint32_t lv[4][LC];
};

// Offset of element col of row x in a swizzled region starting at chunk rbase.
__device__ inline uint32_t elem_ofs(int rbase, int x, int col_byte, int cpa, int lg) {
    return (uint32_t)(16 * (rbase + (x << lg) + swz(x, col_byte >> 4, cpa, lg)) + (col_byte & 15));
}

template <typename T, int K, int NC>
__device__ inline Row<T, K> lds_get(const char *base, const uint32_t (&ofs)[NC]) {
    Row<T, K> out;
    constexpr int B = K * (int)sizeof(T);
    if constexpr (B >= 16) {
#pragma unroll
        for (int c = 0; c < B / 16; ++c)
            __builtin_memcpy(reinterpret_cast<char *>(&out) + 16 * c, __builtin_assume_aligned(base + ofs[c], 16), 16);
    } else {
        __builtin_memcpy(&out, __builtin_assume_aligned(base + ofs[0], B), B);
    }
    return out;
}

}  // namespace rattn
