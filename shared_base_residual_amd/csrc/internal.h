// internal.h -- work decomposition shared by the host dispatcher and the HIP
// kernels of librattn.  Not installed; the public interface is include/rattn.h.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define RATTN_HD __host__ __device__ inline
#else
#define RATTN_HD inline
#endif

namespace rattn {

// Division of a non-negative int n < 2^31 by a divisor d >= 1 fixed at plan
// time, as one multiply and shift: with l = ceil(log2 d) and
// m = floor(2^(32+l) / d) + 1, floor(n * m / 2^(32+l)) = floor(n / d), because
// the excess n * (m - 2^(32+l)/d) / 2^(32+l) is below n / 2^(32+l) < 2^(-1-l)
// <= 1 / (2d) (the round-up method of Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994).  m < 2^33, so n * m fits in
// 64 bits.  Kernels take these instead of runtime divisions, which cost a long
// dependent instruction sequence each at the start of every workgroup.
struct FastDiv {
    uint64_t m;
    int sh;  // 32 + l
    int d;
};

// Host side; a divisor below 1 (an empty dimension) is taken as 1.
inline FastDiv make_fastdiv(int d) {
    FastDiv f;
    if (d < 1) d = 1;
    int l = 0;
    while ((1ll << l) < (long long)d) ++l;
    f.d = d;
    f.sh = 32 + l;  // <= 63
    f.m = ((uint64_t)1 << f.sh) / (uint64_t)d + 1;
    return f;
}

RATTN_HD int fdiv(int n, const FastDiv &f) { return (int)(((uint64_t)(uint32_t)n * f.m) >> f.sh); }

// Largest padded residual width (agents sharing a row block times r) a decode
// row block is given when r allows; bounds the split kernel's registers
// (bf16 / fp32 inputs).  r = 128 still runs, with 128 columns.
constexpr int kMaxResidCols = 64;
constexpr int kMaxResidColsF32 = 32;
constexpr int kMaxResidColsHard = 128;
// Split-kernel instantiations whose registers fit without spilling to scratch:
// eight compute waves run the twelve-wave kernel (168 registers a lane), which
// holds up to 32 residual columns (64 at d = 64) for bf16 inputs, and none at
// d = 128 (64 at d = 64) for fp32; the eight-wave kernel (256 registers) holds
// every width except fp32 at d = 128 with 128 columns.  The planner keeps to
// these and the launcher instantiates nothing else.
RATTN_HD constexpr bool split_wide_ok(bool bf16, int D, int cpad) {
    return bf16 ? cpad <= (D == 64 ? 64 : 32) : cpad <= (D == 64 ? 64 : 0);
}
RATTN_HD constexpr bool split_ok(bool bf16, int D, int cpad) { return bf16 || D == 64 || cpad <= 64; }
// Context tokens per split are a multiple of this (4 waves x 32-token chunks),
// which also keeps every 16-token MFMA tile inside one 16-aligned page.
constexpr int kSplitQuantum = 128;

// Query rows of one KV head are ordered (agent, query token, head-in-group):
// row = agent * rpa + t * g + hh, rpa = q_len * g rows per agent.  The rows are
// cut into MFMA row blocks of at most 16 rows.  When an agent has <= 16 rows, a
// block holds `apb` whole agents; otherwise an agent spans `bpa` blocks.
struct RowBlock {
    int a0;  // first agent
    int na;  // agents in the block
    int f;   // first row within the agent (rpa > 16 only)
    int nr;  // valid rows (<= 16)
};

RATTN_HD RowBlock prefix_block(int b, int n_agents, int rpa, int apb, int bpa) {
    RowBlock rb;
    if (rpa <= 16) {
        rb.a0 = b * apb;
        rb.na = n_agents - rb.a0 < apb ? n_agents - rb.a0 : apb;
        rb.f = 0;
        rb.nr = rb.na * rpa;
    } else {
        rb.a0 = b / bpa;
        rb.na = 1;
        rb.f = 16 * (b % bpa);
        rb.nr = rpa - rb.f < 16 ? rpa - rb.f : 16;
    }
    return rb;
}

// The same with the divisions by bpa and rpa as FastDiv.
RATTN_HD RowBlock prefix_block(int b, int n_agents, int rpa, int apb, const FastDiv &bpa) {
    RowBlock rb;
    if (rpa <= 16) {
        rb.a0 = b * apb;
        rb.na = n_agents - rb.a0 < apb ? n_agents - rb.a0 : apb;
        rb.f = 0;
        rb.nr = rb.na * rpa;
    } else {
        rb.a0 = fdiv(b, bpa);
        rb.na = 1;
        rb.f = 16 * (b - rb.a0 * bpa.d);
        rb.nr = rpa - rb.f < 16 ? rpa - rb.f : 16;
    }
    return rb;
}

// Agent and row-within-agent of row m (< nr) of a block.
RATTN_HD void block_row(const RowBlock &rb, int m, const FastDiv &rpa, int *agent, int *ria) {
    if (rpa.d <= 16) {
        const int a = fdiv(m, rpa);
        *agent = rb.a0 + a;
        *ria = m - a * rpa.d;
    } else {
        *agent = rb.a0;
        *ria = rb.f + m;
    }
}

// Splits per query row the merge handles (weights staged in LDS).
constexpr int kMaxSlots = 512;

// Online softmax: the reference max of a row is raised only when a score
// exceeds it by more than this (log2 units), so weights stay below 2^4 and most
// steps skip the rescale of the accumulators (a step rescales when any of its
// rows' max grows, which for a fresh row max is nearly every early step).  The
// bf16 kernels add a row's weights into its sum as rounded to bf16, exactly as
// the P V product sees them, so a row dominated by one key still normalises to
// that key's value.
constexpr float kRescaleSlack = 4.0f;

struct DecodeParams {
    const void *q, *kb, *vb;
    const int32_t *table;
    const void *lk, *lv, *bk, *bv, *kp, *vp;
    float *out, *lse;
    float *p_ml;      // [H_kv, N*rpa, n_slots, 2]  running max (log2 units), sum of weights l
    void *p_o;        // [H_kv, N*rpa, n_slots, d]  P V_base (+ private P V): fp32 unnormalised (fp32
                      // path); fp16 divided by l (bf16 path: half the bytes, every value within |V|)
    void *p_w;        // [H_kv, N*rpa, n_slots, r]  P Lv, in the same form as p_o
    int64_t L, S;     // < 2^30 (validated on the host)
    int N, QL, HQ, HK, g, r, lr_shift, rpa, apb, bpa, ps, shared_lr;
    int causal;       // private token j is visible to query token t only if j <= t
    float c;          // softmax scale * log2(e) (times the key scale with int8 keys)
    int kq8;          // base keys are excess-128 int8 codes with one scale (no private tokens then)
    float u_scale;    // int8 keys: 1 / key scale, applied to U so that the correction adds to code scores
    int n_blocks, n_rg, n_ps;
    int H, n_hg;      // KV heads per prefix item (sharing its low-rank tile), head groups
    int bpg;          // 16-row blocks per prefix row group (1, 2 or 4)
    int masked;       // per-agent caches, several agents per block, U and W r columns wide
    int tok_ps;
    int pb, n_prg, n_pv;
    int tok_pv;
    int n_slots, n_prefix_items, n_items, per_xcd;
    // Workgroup i runs on XCD i % 8, as its (i / 8)-th workgroup there.  Each XCD
    // takes a contiguous share of the prefix items (pre_per of them), then a
    // share of the private items (pv_per).
    int pre_per, pv_per;
    int nw;           // compute waves per workgroup (4 or 8)
    int np;           // load waves per workgroup: they issue every direct load of the
                      // ring and wait for it, so no compute wave stalls on issue
    int lr_own;       // the last load wave fills only the low-rank regions
    // LDS staging ring: tokens per stage, stages, bytes per stage (prefix items
    // and private items), and where the split's page-table copy lives.
    int T_pre, nst_pre, stage_bytes_pre;
    int T_pv, nst_pv, stage_bytes_pv;
    int table_lds_off;
    // the same divisors for one multiply each (see FastDiv)
    FastDiv fd_hg, fd_rg, fd_hk, fd_pv, fd_prg, fd_rpa, fd_bpa, fd_g, fd_ps;
    FastDiv fd_hq, fd_ql;  // query heads, query tokens (the merge's row index)
    // Base values as 3-bit codes after a Walsh-Hadamard rotation (with int8 keys):
    // vb then holds [H_kv, L, 3 d / 8] bytes of codes and vs the [H_kv, L] scales.
    // The split kernel stages the codes and scales and its load waves decode them
    // to bf16 (scale times centroid) in the stage's value region, so the partial
    // O is in the rotated coordinates; the merge applies H_d once per row.
    const float *vs;
    int vq3;
    int vbuf_off;   // LDS byte offset of the two decoded value buffers (after the ring)
    float vq_c[8];  // centroids, ascending
};

// Size of the static device buffer that rattn_decode_noalloc keeps its split
// partials in (one per GPU, held until the process ends).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;

// Dynamic LDS a split or prefill workgroup may use: all of gfx950's 160 KiB per
// workgroup (neither kernel declares static LDS).
constexpr int kLdsMax = 160 * 1024;
// Page-table entries of one split copied into LDS.
constexpr int kMaxPagesPerSplit = 2048;

}  // namespace rattn

namespace rattn {

// Chunked prefill: one workgroup of eight waves per (KV head, agent, block of
// query rows of that agent), no split of the context.  A wave owns one or two
// 16-row MFMA blocks: two where the accumulators of both fit in registers, one
// for the wide residual widths (d = 128 with 64 or more residual columns, d = 64
// with 128), whose two-block form would spill to scratch.
constexpr int kPrefillWaves = 8;
RATTN_HD constexpr int prefill_blocks_per_wave(int D, int cpad) {
    return (D == 128 ? cpad >= 64 : cpad >= 128) ? 1 : 2;
}
RATTN_HD constexpr int prefill_rows(int D, int cpad) { return 16 * kPrefillWaves * prefill_blocks_per_wave(D, cpad); }

struct PrefillParams {
    const void *q, *kb, *vb;
    const int32_t *table;
    const void *lk, *lv, *bk, *bv, *kp, *vp;
    float *out, *lse;
    int64_t L, S;     // prefix tokens, chunk tokens (= q_len)
    int N, QL, HQ, HK, g, r, lr_shift, ps, shared_lr;
    float c;          // softmax scale * log2(e)
    int rpa;          // query rows per agent per KV head (q_len * g)
    int n_qb;         // row blocks per (agent, KV head)
    int n_items, per_xcd;
    int T;            // keys per LDS stage (128, else 64 when the page table leaves no room)
    int nst_pre, stage_bytes_pre, nst_ch, stage_bytes_ch;
    int table_lds_off;
    FastDiv fd_ps;    // page size
};

}  // namespace rattn

namespace rattn {

// Low-rank cache projection of T new tokens (rattn_lr_project).  Output
// column c of the workgroup grid belongs to set n = c / 2r, to Lk when
// (c / r) % 2 == 0 and to Lv otherwise, component j = c % r.
struct LrParams {
    const void *x;        // [n_xsets, T, d_in]
    const void *ak, *av;  // A^T of keys and values: [shared_a ? 1 : n_sets, r, d_in]
    void *lk, *lv;        // [n_sets, cache_len, r]
    int64_t T, pos0, cache_len;
    int d_in, r, shared_a;
    int n_xsets;          // 1 (one X for every set) or n_sets
    int cols_per_xset;    // output columns one X set feeds: 2r per set it feeds
};

// Paged append of T new rows per KV head (rattn_append_kv); 16-byte vectors.
struct AppendParams {
    void *pool_k, *pool_v;        // [n_phys, H_kv, page, d]
    const int32_t *table;         // the sequence's block table, already updated
    const void *k_new, *v_new;    // [H_kv, T, d]
    int64_t cur_len, T;
    int HK, ps, row_vec;          // row_vec: 16-byte vectors per row (d * element size / 16)
    int off;                      // rows copied from cow_src to cow_dst (cur_len % page, 0 without a copy)
    int cow_src, cow_dst;
};

}  // namespace rattn

namespace rattn {

// Decode with the residual keys rebuilt per token in registers (and rotated by
// position when a frequency vector is given): one workgroup per (split, KV
// head, group of agents), of eight waves (four with the rotation at ranks
// above 16, whose state takes the registers of a second wave per SIMD).  Each agent of the group
// takes tg = waves / agents waves (at most the steps of a stage), which share
// out the 16-token steps of every stage and write separate partials.
constexpr int recon_waves(bool rope, int r) { return rope && r > 16 ? 4 : 8; }
constexpr int kReconTMax = 64;  // tokens per LDS stage (64, or 32 when three such stages do not fit)

struct ReconParams {
    const void *q, *kb, *vb, *lk, *lv, *bk;
    const float *theta;  // [d / 2] rotation frequencies (radians per position), or null
    float *p_ml;         // the bf16 decode workspace layout: max/sum, P V_base / l and P Lv / l as fp16
    void *p_o, *p_w;
    int64_t L;
    int N, QL, HQ, HK, g, rpa, r, shared_lr;
    float c;             // softmax scale * log2(e)
    int n_ag;            // agent groups
    int apg;             // agents per group (<= kReconMaxAgents)
    int tg;              // waves (token groups) per agent; partial slot = split * tg + token group
    int T;               // tokens per LDS stage (a multiple of 16 tg)
    int n_splits, tok_split, n_slots;
    int n_items, per_xcd;
    int nst, stage_bytes;
};

}  // namespace rattn

