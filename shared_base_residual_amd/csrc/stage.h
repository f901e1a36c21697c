// stage.h -- the LDS staging ring shared by the librattn kernels (gfx950):
// stage geometry, where a work item's tokens come from, the direct-load fill
// of one stage, and lane offsets of the MFMA operand reads.  Internal header.
#pragma once
#include "device.h"
#include "internal.h"

namespace rattn {

// ------------------------------------------------------------- geometry --

// Layout of one LDS stage, in 16-byte chunks: K rows, V rows, Lk rows, Lv rows.
// K and V rows are token-major.  The low-rank regions are agent-major within
// each 16-token group: group gg holds, for each agent a of the workgroup, that
// agent's 16 rows (r elements each) back to back -- the same bytes as one
// contiguous piece of the agent's cache, so each direct load reads contiguous
// memory.
struct Geo {
    int T;                    // tokens per stage
    int nst;                  // stages in the ring
    int cpr_kv, lg_kv;        // chunks per V row (and K row with unquantised keys), its log2
    int cpr_k, lg_k;          // chunks per K row (fewer with int8 keys), its log2
    int cpa_lr, lg_lr;        // chunks per low-rank row of one agent (r * sizeof(T) / 16), its log2
    int na_lr;                // agents in the low-rank regions
    int lr_grp;               // chunks of one 16-token group of a low-rank region (16 * na_lr * cpa_lr)
    int H;                    // KV heads staged: K regions 0..H-1 (T rows of cpr_k chunks each),
                              // then V regions (T rows of cpr_kv), then Lk, Lv
    int ofs_v, ofs_lk, ofs_lv;  // region offsets (chunks): V of head 0, Lk, Lv
    int ofs_vq;               // 3-bit values: codes and scales, 64 chunks per (head, 16-token group)
    int chunks;               // chunks per stage
    int stage_bytes;          // stride between stages
};

__device__ inline int ilog2(int x) { return 31 - __builtin_clz(x); }
// n / d for small non-negative n and d >= 1 (wave counts, a dozen or so), by counting.
__device__ inline int small_div(int n, int d) {
    int q = 0;
    for (int x = d; x <= n; x += d) ++q;
    return q;
}

// Where the tokens of a work item come from.
template <typename T>
struct Src {
    const T *kb, *vb;         // contiguous: the first head's rows; paged: pool + that head's offset
    int64_t head_stride;      // V (and unquantised K): elements from one staged head to the next
    int64_t page_stride;      // V (and unquantised K), paged: elements per physical page (0: contiguous)
    int64_t k_head_stride;    // the same for K, in elements of T (int8 keys: two codes per element)
    int64_t k_page_stride;
    FastDiv fps;              // page size (paged)
    int pg0;                  // first logical page of the split
    const int *pages;         // LDS copy of the split's page-table entries (paged)
    const T *lk, *lv;         // low-rank rows: first agent of the workgroup (or the shared one)
    int64_t lr_agent_stride;  // elements between agents' low-rank caches
    int r;                    // rank
    int tlast;                // last valid token of the item
    const uint8_t *vq;        // 3-bit values: the codes of the first staged head (48 bytes per token)
    const float *vs;          // and its scales (one per token)
    int64_t vq_hs;            // tokens per head (the stride of both, in vectors)
};

// Row `tok` of a K or V region source: RE elements of T per row, page_stride
// elements per physical page (0: contiguous).
template <typename T, int RE>
__device__ inline const T *kv_row(const Src<T> &s, const T *base, int tok, int64_t page_stride) {
    if (page_stride) {
        const int lp = fdiv(tok, s.fps);
        const int64_t pg = s.pages[lp - s.pg0];
        return base + pg * page_stride + (int64_t)(tok - lp * s.fps.d) * RE;
    }
    return base + (int64_t)tok * RE;
}

// ------------------------------------------------------------ stage fill --
//
// A stage holds the regions of one tile: the K rows of each staged head, the V
// rows of each, and with a residual the Lk and Lv rows.  The tile's rows are cut
// into 16-row groups (G = T / 16).  The (region, group) pairs pi = region * G +
// group go round-robin to the nw filling waves: wave w fills the pairs with
// pi % nw == w, each with one page lookup and one uniform base per tile and lane
// offsets that depend on the lane only (the swizzle repeats every 16 rows).  Each
// direct load moves 64 chunks of 16 bytes: a K/V group of 16 rows of cpr_kv chunks
// takes 16 * cpr_kv / 64 loads, a low-rank group ceil(lr_grp / 64) (the last one
// partial when lr_grp is not a multiple of 64).  Lane offsets are 32-bit: the
// low-rank rows one workgroup reads span less than 2^31 bytes (checked on the host).

constexpr int kMaxKvLoads = 8;   // direct loads per group of a K (or V) region (fp32, d = 128)

struct FillPlan {
    int G, lgG;               // groups per tile (a power of two), its log2
    int npairs;               // (region, group) pairs per tile
    int pbeg, pend, pstep;    // the pairs this wave fills: pbeg, pbeg + pstep, ... < pend
    int n_kv, n_lr;           // loads per group of a V (and unquantised K) region, of an Lk/Lv region
    int n_k;                  // loads per group of a K region
    int fpw;                  // loads this wave issues per stage
    uint32_t lr_stride;       // bytes between agents' low-rank caches
    bool kv_nt;               // K/V rows are read by this workgroup only: stream them
    bool vq3;                 // V pairs stage 3-bit codes and scales (two loads each)
    uint32_t kv_off[kMaxKvLoads];  // lane byte offset of V (or K) load i from the group's first row
                                   // (only the first d * sizeof(T) / 64 are set and used)
    uint32_t k_off[kMaxKvLoads];   // the same for K rows of KRE elements
};

// Lane byte offset of K/V load i of a group from the group's first row, and the
// lane's row within the group.  Recomputed per load (a few integer operations)
// rather than kept in registers.
// cpr, lg: chunks per row of the region and its log2; rowb: bytes per row.
__device__ inline uint32_t kv_lane_off(int cpr, int lg, int rowb, int i, int lane, int *row_out) {
    const int q = 64 * i + lane;
    const int row = q >> lg;
    const int c = swz(row, q & (cpr - 1), cpr, lg);
    *row_out = row;
    return (uint32_t)(row * rowb + 16 * c);
}

// wave: index among the nw filling waves (a wave with wave >= nw fills nothing).
// lr_own: with a residual and nw >= 2, the last filling wave fills every
// low-rank pair and the others share the K/V pairs, so that low-rank rows
// (mostly L2 hits) do not queue behind HBM reads in one wave's load order.
// KRE: elements of T per K row (D, or D / 2 for int8 keys: two codes per element).
template <typename T, int D, int KRE = D>
__device__ __attribute__((always_inline)) inline void make_fill_plan(FillPlan &f, const Geo &g, const Src<T> &s,
                                                                     bool resid, int wave, int lane, int nw,
                                                                     bool lr_own = false, bool vq3 = false) {
    constexpr int ES = (int)sizeof(T);
    f.G = g.T >> 4;
    f.lgG = ilog2(f.G);
    const int nkv = 2 * g.H * f.G;
    f.npairs = nkv + (resid ? 2 * f.G : 0);
    if (wave >= nw) {
        f.pbeg = f.pend = 0;
        f.pstep = 1;
    } else if (lr_own && resid && nw >= 2) {
        if (wave == nw - 1) {
            f.pbeg = nkv;
            f.pend = f.npairs;
            f.pstep = 1;
        } else {
            f.pbeg = wave;
            f.pend = nkv;
            f.pstep = nw - 1;
        }
    } else {
        f.pbeg = wave;
        f.pend = f.npairs;
        f.pstep = nw;
    }
    f.n_kv = (16 * g.cpr_kv) >> 6;
    f.n_k = (16 * g.cpr_k) >> 6;
    f.n_lr = resid ? ((g.lr_grp + 63) >> 6) : 0;
    f.fpw = 0;
    f.vq3 = vq3;
    const int nk_pairs = g.H * f.G;  // K pairs come first, then V
    const int n_v = vq3 ? 2 : f.n_kv;
    for (int pi = f.pbeg; pi < f.pend; pi += f.pstep) f.fpw += pi < nk_pairs ? f.n_k : pi < nkv ? n_v : f.n_lr;
    f.lr_stride = (uint32_t)(s.lr_agent_stride * ES);
    f.kv_nt = false;
    constexpr int NKV = D * ES / 64;  // loads per V group: 16 rows of d elements
    constexpr int NK = KRE * ES / 64;  // loads per K group
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
        int row;
        f.kv_off[i] = kv_lane_off(g.cpr_kv, g.lg_kv, D * ES, i, lane, &row);
    }
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        int row;
        f.k_off[i] = kv_lane_off(g.cpr_k, g.lg_k, KRE * ES, i, lane, &row);
    }
}

// Lane byte offset of low-rank load i of a group (agent, row and chunk, from
// the first agent's row of the group's first token), and the lane's row within
// the group.  Chunk q of the group region is chunk q % cpa of row
// (q / cpa) % 16 of agent q / (16 cpa).  Computed per load: a workgroup issues few.
__device__ inline uint32_t lr_lane_off(uint32_t lr_stride, const Geo &g, int i, int lane, int *row_out) {
    const int q = 64 * i + lane;
    const int a = q >> (4 + g.lg_lr);
    const int qa = q & ((16 << g.lg_lr) - 1);
    const int x = qa >> g.lg_lr;
    const int c = swz(x, qa & (g.cpa_lr - 1), g.cpa_lr, g.lg_lr);
    *row_out = x;
    return (uint32_t)(16 * ((x << g.lg_lr) + c)) + (uint32_t)a * lr_stride;
}

// LDS byte offset of byte cb of agent a's row x in a low-rank region whose
// group starts at chunk rbase (the same swizzle as the fill).
__device__ inline uint32_t lr_ofs(const Geo &g, int rbase, int a, int x, int cb) {
    return (uint32_t)(16 * (rbase + ((16 * a + x) << g.lg_lr) + swz(x, cb >> 4, g.cpa_lr, g.lg_lr)) + (cb & 15));
}

// Issues this wave's loads of the tile starting at token t0 into `stage`.
// clamp: rows past the item's last token read that token instead (the tail
// tile); otherwise every row is valid and a uniform base per pair serves.
// Always the same number of loads per wave (f.fpw), which the ring's waits count.
// One K or V group of 16 rows of RE elements: N direct loads at lane offsets off[].
template <typename T, int RE>
__device__ __attribute__((always_inline)) inline void fill_kv_group(const FillPlan &f, const Src<T> &s,
                                                                    const T *base, int64_t page_stride,
                                                                    const uint32_t *off, int lg, int tg0,
                                                                    uint32_t dst, bool clamp, int lane) {
    constexpr int ES = (int)sizeof(T);
    constexpr int N = RE * ES / 64;
    if (!clamp) {
        const char *b = uniform_ptr(reinterpret_cast<const char *>(kv_row<T, RE>(s, base, tg0, page_stride)));
        if (f.kv_nt) {
#pragma unroll
            for (int i = 0; i < N; ++i) dma16s_nt(b, off[i], dst + 1024 * i);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) dma16s(b, off[i], dst + 1024 * i);
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int row = (64 * i + lane) >> lg;
            int tok = tg0 + row;
            tok = tok < s.tlast ? tok : s.tlast;
            const uint32_t rowoff = off[i] - (uint32_t)(row * RE * ES);  // chunk part
            dma16(reinterpret_cast<const char *>(kv_row<T, RE>(s, base, tok, page_stride)) + rowoff, dst + 1024 * i);
        }
    }
}

// One 16-token group of 3-bit values of one head: lanes 0..47 load the 768
// bytes of codes (16 bytes each, token tg0 + lane / 3), lanes 0..15 the 16
// scales (4 bytes each) into bytes 768..831 of the group's 1 KiB region.
// Tokens past the item's last read that token instead.  Two direct loads.
template <typename T>
__device__ __attribute__((always_inline)) inline void fill_vq_group(const Src<T> &s, int head, int tg0,
                                                                    uint32_t dst, int lane) {
    const uint8_t *codes = s.vq + (int64_t)head * s.vq_hs * 48;
    const float *scales = s.vs + (int64_t)head * s.vq_hs;
    if (lane < 48) {
        int tok = tg0 + lane / 3;
        tok = tok < s.tlast ? tok : s.tlast;
        dma16(codes + (int64_t)tok * 48 + 16 * (lane % 3), dst);
    }
    if (lane < 16) {
        int tok = tg0 + lane;
        tok = tok < s.tlast ? tok : s.tlast;
        dma4(scales + tok, dst + 768);
    }
}

template <typename T, int D, int KRE = D>
__device__ __attribute__((always_inline)) inline void fill_stage(const FillPlan &f, const Geo &g, const Src<T> &s,
                                                                 int t0, char *stage, bool clamp, int lane) {
    constexpr int ES = (int)sizeof(T);
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(stage));
    const int nkv = 2 * g.H * f.G;  // K pairs (regions 0 .. H-1), then V pairs, come first
    for (int pi = f.pbeg; pi < f.pend; pi += f.pstep) {
        const int gg = pi & (f.G - 1);
        const int tg0 = t0 + 16 * gg;  // the group's first token
        if (pi < nkv) {
            const int region = pi >> f.lgG;
            if (region >= g.H && f.vq3) {  // 3-bit codes and scales of head region - H
                fill_vq_group<T>(s, region - g.H, tg0, lds0 + 16 * (g.ofs_vq + ((region - g.H) * f.G + gg) * 64),
                                 lane);
            } else if (region >= g.H) {  // V rows of head region - H
                const T *base = s.vb + (int64_t)(region - g.H) * s.head_stride;
                const uint32_t dst = lds0 + 16 * (g.ofs_v + ((region - g.H) * g.T + 16 * gg) * g.cpr_kv);
                fill_kv_group<T, D>(f, s, base, s.page_stride, f.kv_off, g.lg_kv, tg0, dst, clamp, lane);
            } else {  // K rows of head region
                const T *base = s.kb + (int64_t)region * s.k_head_stride;
                const uint32_t dst = lds0 + 16 * ((region * g.T + 16 * gg) * g.cpr_k);
                fill_kv_group<T, KRE>(f, s, base, s.k_page_stride, f.k_off, g.lg_k, tg0, dst, clamp, lane);
            }
        } else {
            // Lk (first) or Lv rows of every agent of the workgroup
            const bool isv = pi >= nkv + f.G;
            const T *lbase = isv ? s.lv : s.lk;
            const uint32_t dst = lds0 + 16 * ((isv ? g.ofs_lv : g.ofs_lk) + gg * g.lr_grp);
            const char *b = uniform_ptr(reinterpret_cast<const char *>(lbase + (int64_t)tg0 * s.r));
            for (int i = 0; i < f.n_lr; ++i) {
                if (64 * i + lane < g.lr_grp) {
                    int row;
                    const uint32_t off = lr_lane_off(f.lr_stride, g, i, lane, &row);
                    if (!clamp) {
                        dma16s(b, off, dst + 1024 * i);
                    } else {
                        int tok = tg0 + row;
                        tok = tok < s.tlast ? tok : s.tlast;
                        const uint32_t rel = off - (uint32_t)(row * s.r * ES);  // agent and chunk part
                        dma16(reinterpret_cast<const char *>(lbase + (int64_t)tok * s.r) + rel, dst + 1024 * i);
                    }
                }
            }
        }
    }
}

// The same fill for one staged head when every filling wave owns a single
// 16-row group (nw a multiple of G): wave w fills group w % G of the regions r
// with (r * G + w % G) % nw == w.  Fewer instructions per tile than the
// general walk over pairs, for kernels whose filling waves also compute.
struct GroupFill {
    int g;                    // this wave's group
    bool rK, rV, rL, rLv;     // regions it fills
    int n_lr;                 // loads per group of an Lk/Lv region
    int fpw;                  // loads per stage
    uint32_t lr_stride;       // bytes between agents' low-rank caches
    uint32_t kv_off[kMaxKvLoads];  // as in FillPlan
};

template <typename T, int D>
__device__ __attribute__((always_inline)) inline void make_group_fill(GroupFill &f, const Geo &g, const Src<T> &s,
                                                                       bool resid, int wave, int lane, int nw) {
    constexpr int ES = (int)sizeof(T);
    constexpr int NKV = D * ES / 64;
    const int G = g.T >> 4;
    f.g = wave % G;
    auto mine = [&](int region) { return (region * G + f.g) % nw == wave; };
    f.rK = mine(0);
    f.rV = mine(1);
    f.rL = resid && mine(2);
    f.rLv = resid && mine(3);
    f.n_lr = resid ? ((g.lr_grp + 63) >> 6) : 0;
    f.fpw = (f.rK ? NKV : 0) + (f.rV ? NKV : 0) + (f.rL ? f.n_lr : 0) + (f.rLv ? f.n_lr : 0);
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
        int row;
        f.kv_off[i] = kv_lane_off(g.cpr_kv, g.lg_kv, D * ES, i, lane, &row);
    }
    f.lr_stride = (uint32_t)(s.lr_agent_stride * ES);
}

template <typename T, int D>
__device__ __attribute__((always_inline)) inline void fill_group(const GroupFill &f, const Geo &g, const Src<T> &s,
                                                                  int t0, char *stage, bool clamp, int lane) {
    constexpr int ES = (int)sizeof(T);
    constexpr int NKV = D * ES / 64;
    const int tg0 = t0 + 16 * f.g;  // the group's first token
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(stage));
    const uint32_t lk0 = lds0 + 16 * (16 * f.g * g.cpr_kv), lv0 = lds0 + 16 * (g.ofs_v + 16 * f.g * g.cpr_kv);
    const uint32_t ll0 = lds0 + 16 * (g.ofs_lk + f.g * g.lr_grp), lw0 = lds0 + 16 * (g.ofs_lv + f.g * g.lr_grp);
    if (!clamp) {
        if (f.rK || f.rV) {
            const char *kb = uniform_ptr(reinterpret_cast<const char *>(kv_row<T, D>(s, s.kb, tg0, s.page_stride)));
            const char *vb = uniform_ptr(reinterpret_cast<const char *>(kv_row<T, D>(s, s.vb, tg0, s.page_stride)));
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                if (f.rK) dma16s(kb, f.kv_off[i], lk0 + 1024 * i);
#pragma unroll
            for (int i = 0; i < NKV; ++i)
                if (f.rV) dma16s(vb, f.kv_off[i], lv0 + 1024 * i);
        }
        if (f.rL || f.rLv) {
            const char *lk = uniform_ptr(reinterpret_cast<const char *>(s.lk + (int64_t)tg0 * s.r));
            const char *lv = uniform_ptr(reinterpret_cast<const char *>(s.lv + (int64_t)tg0 * s.r));
            for (int i = 0; i < f.n_lr; ++i) {
                if (64 * i + lane < g.lr_grp) {
                    int row;
                    const uint32_t off = lr_lane_off(f.lr_stride, g, i, lane, &row);
                    if (f.rL) dma16s(lk, off, ll0 + 1024 * i);
                    if (f.rLv) dma16s(lv, off, lw0 + 1024 * i);
                }
            }
        }
        return;
    }
    // tail tile: per-lane rows, clamped to the item's last token
#pragma unroll
    for (int i = 0; i < NKV; ++i) {
        if (f.rK || f.rV) {
            const int row = (64 * i + lane) >> g.lg_kv;
            int tok = tg0 + row;
            tok = tok < s.tlast ? tok : s.tlast;
            const uint32_t rowoff = f.kv_off[i] - (uint32_t)(row * D * ES);  // chunk part
            if (f.rK)
                dma16(reinterpret_cast<const char *>(kv_row<T, D>(s, s.kb, tok, s.page_stride)) + rowoff, lk0 + 1024 * i);
            if (f.rV)
                dma16(reinterpret_cast<const char *>(kv_row<T, D>(s, s.vb, tok, s.page_stride)) + rowoff, lv0 + 1024 * i);
        }
    }
    for (int i = 0; i < f.n_lr; ++i) {
        if ((f.rL || f.rLv) && 64 * i + lane < g.lr_grp) {
            int row;
            const uint32_t off = lr_lane_off(f.lr_stride, g, i, lane, &row);
            int tok = tg0 + row;
            tok = tok < s.tlast ? tok : s.tlast;
            const uint32_t rel = off - (uint32_t)(row * s.r * ES);  // agent and chunk part
            if (f.rL) dma16(reinterpret_cast<const char *>(s.lk + (int64_t)tok * s.r) + rel, ll0 + 1024 * i);
            if (f.rLv) dma16(reinterpret_cast<const char *>(s.lv + (int64_t)tok * s.r) + rel, lw0 + 1024 * i);
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
