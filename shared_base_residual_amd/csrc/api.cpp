// api.cpp -- C ABI of librattn: host-side validation, work decomposition and
// dispatch.  Every check runs before the first HIP call, so argument errors
// return a status without touching the device.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "rattn.h"
#include "internal.h"

namespace rattn {
hipError_t launch_decode(int bf16_in, const DecodeParams &dp, int D, int cpad, size_t lds, unsigned stages,
                         hipStream_t st);
hipError_t launch_gather(const void *pool, const int32_t *table, void *dst, int64_t L, int HK, int ps,
                         int row_bytes, hipStream_t st);
hipError_t launch_prefill(const PrefillParams &pp, int D, int cpad, size_t lds, hipStream_t st);
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_lr_project(const LrParams &p, hipStream_t st);
hipError_t launch_append_kv(const AppendParams &p, hipStream_t st);
hipError_t launch_quantize(const void *k, int64_t n, int bf16_in, void *codes, float *scale, hipStream_t st);
hipError_t launch_recon(const ReconParams &p, hipStream_t st);
hipError_t launch_check_table(const int32_t *table, int64_t n, int64_t n_phys, int32_t *bad, hipStream_t st);
hipError_t launch_values3_encode(const void *v, int64_t n, int D, int bf16_in, const double *boundaries, void *codes,
                                 float *scale, hipStream_t st);
}  // namespace rattn

static_assert(rattn::kNoAllocScratchBytes == RATTN_NOALLOC_SCRATCH_BYTES, "static scratch size in the header");

namespace {

thread_local int g_last_hip = 0;

#ifndef RATTN_TARGET_ITEMS
#define RATTN_TARGET_ITEMS 256
#endif
constexpr int kTargetItems = RATTN_TARGET_ITEMS;  // split-kernel workgroups aimed for
#ifndef RATTN_LR_OWN
#define RATTN_LR_OWN 0
#endif

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t roundup(int64_t a, int64_t b) { return cdiv(a, b) * b; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// The 8-level minimum-MSE (Lloyd-Max) quantiser of N(0, 1) behind the 3-bit
// values (PolyKV, section 2B): the fixed point of Lloyd's two conditions, each
// centroid the N(0, 1) mean of its cell, (pdf(a) - pdf(b)) / (cdf(b) - cdf(a))
// over [a, b), and each inner boundary the midpoint of its two centroids.
// Iterated on the non-negative half from 0.5, 1.5, 2.5, 3.5 and mirrored, so
// the middle boundary is exactly 0.
struct ValuesCodebook {
    double c[8], b[7];
};

const ValuesCodebook &values_codebook() {
    static const ValuesCodebook cb = [] {
        const double inv_sqrt2pi = 0.39894228040143267794, inv_sqrt2 = 0.70710678118654752440;
        auto pdf = [&](double x) { return isinf(x) ? 0.0 : inv_sqrt2pi * exp(-0.5 * x * x); };
        auto cdf = [&](double x) { return isinf(x) ? 1.0 : 0.5 * (1.0 + erf(x * inv_sqrt2)); };
        double c[4] = {0.5, 1.5, 2.5, 3.5};
        for (int it = 0; it < 10000; ++it) {
            const double e[5] = {0.0, 0.5 * (c[0] + c[1]), 0.5 * (c[1] + c[2]), 0.5 * (c[2] + c[3]), INFINITY};
            double n[4], dmax = 0.0;
            for (int i = 0; i < 4; ++i) {
                n[i] = (pdf(e[i]) - pdf(e[i + 1])) / (cdf(e[i + 1]) - cdf(e[i]));
                dmax = fmax(dmax, fabs(n[i] - c[i]));
            }
            for (int i = 0; i < 4; ++i) c[i] = n[i];
            if (dmax <= 1e-16) break;
        }
        ValuesCodebook k;
        for (int i = 0; i < 4; ++i) {
            k.c[4 + i] = c[i];
            k.c[3 - i] = -c[i];
        }
        k.b[3] = 0.0;
        for (int i = 0; i < 3; ++i) {
            k.b[4 + i] = 0.5 * (c[i] + c[i + 1]);
            k.b[2 - i] = -k.b[4 + i];
        }
        return k;
    }();
    return cb;
}

int pow2ceil(int x) {
    int v = 1;
    while (v < x) v <<= 1;
    return v;
}

size_t esize(int dtype) { return dtype == RATTN_BF16 ? 2 : 4; }

int check_desc(const rattn_desc *d, int op) {
    if (!d) return RATTN_E_NULL;
    if (d->n_agents < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->rank < 0 ||
        d->q_len < 1 || d->prefix_len < 0 || d->priv_len < 0 || d->page_size < 0 || d->n_phys_pages < 0)
        return RATTN_E_SHAPE;
    if (d->n_q_heads % d->n_kv_heads) return RATTN_E_SHAPE;
    if (d->prefix_len + d->priv_len < 1) return RATTN_E_SHAPE;
    if (d->dtype != RATTN_F32 && d->dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    if (d->shared_lr != 0 && d->shared_lr != 1) return RATTN_E_SHAPE;
    if (d->head_dim != 64 && d->head_dim != 128) return RATTN_E_UNSUPPORTED;
    const int r = d->rank;
    if (!(r == 0 || r == 8 || r == 16 || r == 32 || r == 64 || r == 128)) return RATTN_E_UNSUPPORTED;
    if (d->page_size > 0) {
        if (d->page_size % 16) return RATTN_E_UNSUPPORTED;
        if (d->prefix_len > 0 && d->n_phys_pages < 1) return RATTN_E_SHAPE;
    }
    if (op == RATTN_OP_PREFILL && d->q_len != d->priv_len) return RATTN_E_SHAPE;
    if (op != RATTN_OP_DECODE && op != RATTN_OP_PREFILL && op != RATTN_OP_RECONSTRUCT) return RATTN_E_SHAPE;
    if (op == RATTN_OP_RECONSTRUCT) {
        // rebuilt residual keys: bf16, d = 128, rank 16 or 32, a contiguous base
        // cache, no private tokens, at most 16 query rows per agent and KV head
        if (d->dtype != RATTN_BF16 || d->head_dim != 128 || (d->rank != 16 && d->rank != 32) ||
            d->page_size != 0 || d->priv_len != 0 || d->prefix_len < 1 ||
            (int64_t)d->q_len * (d->n_q_heads / d->n_kv_heads) > 16 || d->k_format != RATTN_KEYS_DTYPE ||
            d->v_format != RATTN_VALUES_DTYPE)
            return RATTN_E_UNSUPPORTED;
    }
    if (d->k_format != RATTN_KEYS_DTYPE && d->k_format != RATTN_KEYS_INT8) return RATTN_E_SHAPE;
    if (d->k_format == RATTN_KEYS_INT8) {
        if (!(d->k_scale > 0.f && d->k_scale <= 3.0e38f)) return RATTN_E_SHAPE;
        // int8 base keys: bf16 decode over a shared prefix, d = 128, no private tokens
        if (d->dtype != RATTN_BF16 || d->head_dim != 128 || d->priv_len != 0 || d->prefix_len < 1 ||
            op != RATTN_OP_DECODE)
            return RATTN_E_UNSUPPORTED;
    }
    if (d->v_format != RATTN_VALUES_DTYPE && d->v_format != RATTN_VALUES_FWHT3) return RATTN_E_SHAPE;
    if (d->v_format == RATTN_VALUES_FWHT3) {
        // 3-bit values: with int8 keys (so bf16 decode, d = 128, no private tokens), contiguous cache
        if (d->k_format != RATTN_KEYS_INT8 || d->page_size != 0 || op != RATTN_OP_DECODE)
            return RATTN_E_UNSUPPORTED;
    }
    // Index arithmetic inside the kernels uses 32-bit row and item counts.
    const int64_t rows = (int64_t)d->n_agents * d->q_len * d->n_q_heads;
    if (rows > (1ll << 28) || d->prefix_len > (1ll << 30) || d->priv_len > (1ll << 30))
        return RATTN_E_UNSUPPORTED;
    return RATTN_OK;
}

struct Plan {
    rattn::DecodeParams dp;
    int cpad;
    size_t lds;
    size_t off_ml, off_o, off_w, total;
};

int make_plan(const rattn_desc *d, int op, Plan *pl) {
    rattn::DecodeParams &p = pl->dp;
    p = rattn::DecodeParams{};
    const int N = d->n_agents, HK = d->n_kv_heads, g = d->n_q_heads / d->n_kv_heads, r = d->rank;
    const int D = d->head_dim;
    const int64_t L = d->prefix_len, S = d->priv_len;
    const int rpa = d->q_len * g;
    const bool resid = r > 0 && L > 0;
    p.L = L;
    p.S = S;
    p.N = N;
    p.QL = d->q_len;
    p.HQ = d->n_q_heads;
    p.HK = HK;
    p.g = g;
    p.r = r;
    p.lr_shift = 0;
    while (r > 0 && (1 << p.lr_shift) < r) ++p.lr_shift;
    p.rpa = rpa;
    p.ps = d->page_size;
    p.shared_lr = d->shared_lr;
    p.causal = op == RATTN_OP_PREFILL;
    p.lr_own = RATTN_LR_OWN;
    const float scale = d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)D);
    p.c = scale * 1.44269504088896340736f;
    p.kq8 = d->k_format == RATTN_KEYS_INT8;
    p.vq3 = d->v_format == RATTN_VALUES_FWHT3;
    for (int k = 0; k < 8; ++k) p.vq_c[k] = p.vq3 ? (float)values_codebook().c[k] : 0.0f;
    p.u_scale = 1.0f;
    if (p.kq8) {  // scores in code units: the exponent's scale takes the key scale, U its inverse
        p.c = (float)((double)scale * 1.44269504088896340736 * (double)d->k_scale);
        p.u_scale = (float)(1.0 / (double)d->k_scale);
    }

    // The decomposition: the masked mode first where it applies, else (or when
    // its ring does not fit) block-diagonal residual columns.
    auto plan_rows = [&](bool mask_ok) -> int {
        // Row blocks over the prefix.  bf16 per-agent caches of rank >= 32 put as many
        // agents in a block as its 16 rows hold (the masked mode: U and W stay r
        // columns wide); otherwise the agents of a block are bounded by the residual
        // columns their block-diagonal U and W take.
        const bool can_mask = mask_ok && resid && !d->shared_lr && d->dtype == RATTN_BF16 && r >= 32;
        if (rpa <= 16) {
            int apb = 16 / rpa;
            if (resid && !d->shared_lr && !can_mask) {
                const int cap = d->dtype == RATTN_BF16 ? rattn::kMaxResidCols : rattn::kMaxResidColsF32;
                const int by_cols = cap / r;
                if (by_cols < apb) apb = by_cols;
            }
            if (apb > N) apb = N;
            if (apb < 1) apb = 1;
            p.apb = apb;
            p.bpa = 1;
            p.n_blocks = (int)cdiv(N, apb);
            p.pb = 1;
        } else {
            p.apb = 1;
            p.bpa = (int)cdiv(rpa, 16);
            p.n_blocks = N * p.bpa;
            p.pb = p.bpa;
        }
        p.n_prg = (int)cdiv(p.pb, 4);
        p.masked = can_mask && rpa <= 16 && p.apb > 1;
        int cols = 0;
        if (resid) cols = d->shared_lr || p.masked ? r : (rpa <= 16 ? p.apb * r : r);
        pl->cpad = resid ? (pow2ceil(cols) < 32 ? 32 : pow2ceil(cols)) : 0;
        if (pl->cpad > rattn::kMaxResidColsHard) return RATTN_E_UNSUPPORTED;
        if (!rattn::split_ok(d->dtype == RATTN_BF16, D, pl->cpad)) return RATTN_E_UNSUPPORTED;

        const int es = (int)esize(d->dtype);
        const int kv_row = D * es;                   // bytes of one value row (and key row, unquantised)
        const int k_row = p.kq8 ? D : kv_row;         // bytes of one key row (int8: one per element)
        // 3-bit values: a stage holds, per 16-token group and head, 1 KiB for the
        // codes and scales (two loads) instead of value rows, which are decoded into
        // two buffers of H T rows after the ring; HBM holds 3 d / 8 + 4 bytes per
        // value vector
        const int vq_row = p.vq3 ? 64 : 0;
        const int v_hbm = p.vq3 ? 3 * D / 8 + 4 : kv_row;
        // Row groups of bpg blocks: the agents of a group, and the low-rank bytes per
        // token a stage holds for them (or for the shared cache).
        int ag_max = 1, nb_min = 4, nb_max = 1, lr_row = 0;
        auto group_stats = [&](int bpg) -> int {
            p.bpg = bpg;
            p.n_rg = (int)cdiv(p.n_blocks, bpg);
            ag_max = 1;
            nb_min = bpg;
            nb_max = 1;
            for (int rg = 0; L > 0 && rg < p.n_rg; ++rg) {
                const int b0 = bpg * rg;
                const int nb = p.n_blocks - b0 < bpg ? p.n_blocks - b0 : bpg;
                const rattn::RowBlock x0 = rattn::prefix_block(b0, N, rpa, p.apb, p.bpa);
                const rattn::RowBlock x1 = rattn::prefix_block(b0 + nb - 1, N, rpa, p.apb, p.bpa);
                const int na = x1.a0 + x1.na - x0.a0;
                if (na > ag_max) ag_max = na;
                if (nb < nb_min) nb_min = nb;
                if (nb > nb_max) nb_max = nb;
            }
            // the stage fill addresses one workgroup's low-rank rows with 32-bit offsets
            if (resid && (int64_t)(d->shared_lr ? 1 : ag_max) * L * r * es >= (1ll << 31)) return RATTN_E_UNSUPPORTED;
            lr_row = resid ? (d->shared_lr ? 1 : ag_max) * r * es : 0;
            return RATTN_OK;
        };

        // Context splits for H KV heads per prefix item.
        auto plan_splits = [&](int H) -> int {
            p.H = H;
            p.n_hg = HK / H;
            p.n_ps = 0;
            p.n_pv = 0;
            if (L > 0) {
                const int64_t base = (int64_t)p.n_hg * p.n_rg;
                int64_t n = cdiv(kTargetItems, base);
                const int64_t nmax = cdiv(L, rattn::kSplitQuantum);
                if (n > nmax) n = nmax;
                if (n < 1) n = 1;
                // n splits of a 128-multiple length; trailing splits may be empty, which
                // keeps the split count (and the workspace) non-decreasing in L.
                p.tok_ps = (int)roundup(cdiv(L, n), rattn::kSplitQuantum);
                p.n_ps = (int)n;
            }
            if (S > 0) {
                const int64_t base = (int64_t)N * HK * p.n_prg;
                int64_t n = cdiv(kTargetItems, base);
                const int64_t nmax = cdiv(S, rattn::kSplitQuantum);
                if (n > nmax) n = nmax;
                if (n < 1) n = 1;
                p.tok_pv = (int)roundup(cdiv(S, n), rattn::kSplitQuantum);
                p.n_pv = (int)n;
            }
            p.n_slots = p.n_ps + p.n_pv;
            if (p.n_slots > rattn::kMaxSlots) return RATTN_E_UNSUPPORTED;
            const int64_t n_pre = (int64_t)p.n_ps * p.n_rg * p.n_hg;
            const int64_t n_all = n_pre + (int64_t)N * p.n_prg * p.n_pv * HK;
            if (n_all > (1ll << 30)) return RATTN_E_UNSUPPORTED;
            p.n_prefix_items = (int)n_pre;
            p.n_items = (int)n_all;
            p.pre_per = (int)cdiv(n_pre, 8);
            p.pv_per = (int)cdiv(n_all - n_pre, 8);
            p.per_xcd = p.pre_per + p.pv_per;
            if (d->page_size > 0 && L > 0 && cdiv(p.tok_ps, d->page_size) + 1 > rattn::kMaxPagesPerSplit)
                return RATTN_E_UNSUPPORTED;
            return RATTN_OK;
        };

        // Loads the busiest of np load waves issues per stage (the fill plan's
        // round-robin of (region, group) pairs over 2H K/V regions and, with a
        // residual, the Lk and Lv regions); a wave may have at most 63 loads
        // outstanding, and a ring keeps nst - 1 stages in flight.
        auto max_fpw = [&](int T, int H, int lr_row_bytes, int np) {
            const int G = T / 16, nkv = 2 * H * G, npairs = nkv + (lr_row_bytes ? 2 * G : 0);
            const int n_kv = (16 * (kv_row / 16)) / 64, n_lr = (16 * (lr_row_bytes / 16) + 63) / 64;
            const int n_k = (16 * (k_row / 16)) / 64;  // K pairs (the first H G) take n_k loads
            const bool own = p.lr_own && lr_row_bytes && np >= 2;  // as make_fill_plan
            int mx = 0;
            for (int w = 0; w < np; ++w) {
                int f = 0;
                const int b = own ? (w == np - 1 ? nkv : w) : w, e = own && w < np - 1 ? nkv : npairs;
                const int st = own ? (w == np - 1 ? 1 : np - 1) : np;
                for (int pi = b; pi < e; pi += st) f += pi < H * G ? n_k : pi < nkv ? (p.vq3 ? 2 : n_kv) : n_lr;
                if (f > mx) mx = f;
            }
            return mx;
        };
        auto fit_vmcnt = [&](int T, int H, int lr_row_bytes, int *nst) {
            // Two load waves (three when the low-rank rows have their own), four
            // when a tile takes 40 or more loads: on gfx950 a wave's direct loads
            // are back-pressured at issue, so large tiles stream faster from more
            // waves.  More if the outstanding-load limit needs them, then fewer stages.
            const int G = T / 16;
            const int tile_loads = H * G * ((p.vq3 ? 2 : (16 * (kv_row / 16)) / 64) + (16 * (k_row / 16)) / 64) +
                                   (lr_row_bytes ? 2 * G * ((16 * (lr_row_bytes / 16) + 63) / 64) : 0);
            // (int8 keys: four, whose tiles take fewer loads than the rule counts on)
            const int np0 = (tile_loads >= 40 || p.kq8) && p.nw + 4 <= 12 ? 4 : (p.lr_own ? 3 : 2);
            for (int np = np0; np <= 4; np += 1) {
                const int f = max_fpw(T, H, lr_row_bytes, np);
                if (f * (*nst - 1) <= 63) {
                    if (np > p.np) p.np = np;
                    return true;
                }
            }
            const int f = max_fpw(T, H, lr_row_bytes, 4);
            p.np = 4;
            while (*nst > (p.vq3 ? 3 : 2) && f * (*nst - 1) > 63) --*nst;
            return f * (*nst - 1) <= 63;
        };

        // LDS staging ring.  A stage holds T tokens of keys and values of the item's
        // heads and, for prefix items with a residual, the low-rank rows (Lk and Lv)
        // of every agent the workgroup serves (agent-major within each 16-token
        // group).  T must give every wave whole 16-token steps: a row group of nblk
        // blocks of H heads runs nw / (H nblk) waves per row tile.  min_nst: stages
        // the prefix ring needs.
        auto plan_lds = [&](int nw, int min_nst) -> bool {
            p.nw = nw;
            p.np = p.lr_own ? 3 : 2;
            // the split's page-table entries sit after the ring
            const int table_bytes = d->page_size > 0 && L > 0 ? (int)(cdiv(p.tok_ps, d->page_size) + 1) * 4 + 16 : 0;
            auto pick = [&](int tg_max, int H, int lr_row_bytes, int need, int *T, int *nst, int *stage) {
                for (int t = 128; t >= 16; t /= 2) {
                    if (t % (16 * tg_max) || t > 16 * nw) continue;  // the fill gives each 16-row group one wave
                    const int sb = t * (H * (k_row + (p.vq3 ? vq_row : kv_row)) + 2 * lr_row_bytes);
                    const int vbuf = p.vq3 ? 2 * H * t * kv_row : 0;  // the decoded value buffers
                    const int n = (rattn::kLdsMax - table_bytes - vbuf) / sb;
                    // (3-bit values keep nst - 2 tiles in flight: at least three stages)
                    if (n >= 3 || (!p.vq3 && t == 16 * tg_max && n >= need)) {
                        *T = t;
                        const int cap = p.vq3 ? 6 : 4;  // (small 3-bit stages: more of them in flight)
                        *nst = n < cap ? n : cap;
                        *stage = sb;
                        return true;
                    }
                }
                return false;
            };
            int lds_ring = 0;
            if (L > 0) {
                if (p.H * nb_max > nw) return false;
                const int tg_max = nw / (p.H * nb_min);
                if (!pick(tg_max, p.H, lr_row, min_nst, &p.T_pre, &p.nst_pre, &p.stage_bytes_pre)) return false;
                if (!fit_vmcnt(p.T_pre, p.H, lr_row, &p.nst_pre)) return false;
                lds_ring = p.nst_pre * p.stage_bytes_pre;
                p.vbuf_off = lds_ring;
                if (p.vq3) lds_ring += 2 * p.H * p.T_pre * kv_row;
            }
            if (S > 0) {
                int tg_max = 1;
                for (int g0 = 0; g0 < p.pb; g0 += 4) {
                    const int nb = p.pb - g0 < 4 ? p.pb - g0 : 4;
                    if (nw / nb > tg_max) tg_max = nw / nb;
                }
                if (!pick(tg_max, 1, 0, 2, &p.T_pv, &p.nst_pv, &p.stage_bytes_pv)) return false;
                if (!fit_vmcnt(p.T_pv, 1, 0, &p.nst_pv)) return false;
                const int b = p.nst_pv * p.stage_bytes_pv;
                if (b > lds_ring) lds_ring = b;
            }
            // After the ring, the token-group merge (one slot of per-lane state per
            // wave) reuses the same memory.
            const int cpl = pl->cpad > 0 ? pl->cpad / 16 : 1;
            const int per_lane = 4 * (D / 16) + 4 * cpl;
            int lds = lds_ring;
            const int lds_merge = nw * (64 * per_lane + 32) * (int)sizeof(float);
            if (lds_merge > lds) lds = lds_merge;
            // The split's page-table entries.
            p.table_lds_off = (lds + 15) & ~15;
            if (d->page_size > 0 && L > 0) lds = p.table_lds_off + (int)(cdiv(p.tok_ps, d->page_size) + 1) * 4;
            if (lds > rattn::kLdsMax) return false;
            pl->lds = (size_t)lds;
            return true;
        };

        // Several KV heads per prefix item share its staged low-rank rows (read once
        // instead of once per head): the most heads whose row tiles fit eight waves
        // and whose ring still keeps two or more tiles in flight.  Eight waves (two
        // per SIMD) when an item has two or more row tiles, else four.
        // Among the row-group sizes (4, 2 or 1 blocks) and head counts that plan,
        // the one that reads the fewest bytes per context token into the
        // workgroups: each row group reads the K/V of every head, each (head group,
        // row group) its agents' low-rank rows.
        bool planned = false;
        int64_t best_cost = -1;
        rattn::DecodeParams best;
        size_t best_lds = 0;
        for (int bpg = 4; bpg >= 1; bpg /= 2) {
            if (bpg > 1 && bpg > p.n_blocks && bpg != 4) continue;
            const int gs = group_stats(bpg);
            if (gs != RATTN_OK) return gs;
            for (int H = 8; H >= 1; H /= 2) {
                if (HK % H || (H > 1 && !resid)) continue;
                const int st = plan_splits(H);
                if (st != RATTN_OK) return st;
                const int tiles_min = L > 0 ? H * nb_min : (p.pb < 4 ? p.pb : 4);
                const int need = H > 1 ? 3 : 2;
                // Eight compute waves run the twelve-wave kernel (168 registers a
                // lane), whose wider residual variants would spill to scratch.
                const bool wide = rattn::split_wide_ok(d->dtype == RATTN_BF16, D, pl->cpad);
                const bool ok = (tiles_min >= 2 && wide && plan_lds(8, need)) || plan_lds(4, need);
                if (!ok) continue;
                // Preference: a prefix tile of 32 or more tokens (the per-tile
                // synchronisation is a large share of a tile's time), then the
                // fewest bytes staged per context token, then more heads per item.
                const int64_t bytes = (int64_t)p.n_rg * HK * (k_row + v_hbm) + (int64_t)p.n_hg * p.n_rg * 2 * lr_row;
                const int64_t cost = (L > 0 && p.T_pre < 32 ? (int64_t)1 << 40 : 0) + bytes * 16 + (8 - p.H);
                if (best_cost < 0 || cost < best_cost) {
                    best_cost = cost;
                    best = p;
                    best_lds = pl->lds;
                }
                planned = true;
            }
            if (planned && (L == 0 || !resid)) break;  // nothing to trade
        }
        if (!planned) return RATTN_E_UNSUPPORTED;
        p = best;
        pl->lds = best_lds;
        return RATTN_OK;
    };
    int pst = plan_rows(true);
    if (pst != RATTN_OK) pst = plan_rows(false);
    if (pst != RATTN_OK) return pst;
    p.fd_hg = rattn::make_fastdiv(p.n_hg);
    p.fd_rg = rattn::make_fastdiv(p.n_rg);
    p.fd_hk = rattn::make_fastdiv(p.HK);
    p.fd_pv = rattn::make_fastdiv(p.n_pv);
    p.fd_prg = rattn::make_fastdiv(p.n_prg);
    p.fd_rpa = rattn::make_fastdiv(p.rpa);
    p.fd_bpa = rattn::make_fastdiv(p.bpa);
    p.fd_g = rattn::make_fastdiv(p.g);
    p.fd_ps = rattn::make_fastdiv(p.ps);
    p.fd_hq = rattn::make_fastdiv(p.HQ);
    p.fd_ql = rattn::make_fastdiv(p.QL);

    // Workspace: the (max, sum), O and W partials of every (KV head, row, split).
    const int64_t rows_kv = (int64_t)HK * N * rpa;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    // partial O and W: fp16 (divided by the row's weight sum) on the bf16 path, fp32 otherwise
    const size_t pes = d->dtype == RATTN_BF16 ? 2 : sizeof(float);
    pl->off_ml = take((size_t)rows_kv * p.n_slots * 2 * sizeof(float));
    pl->off_o = take((size_t)rows_kv * p.n_slots * D * pes);
    pl->off_w = take(resid ? (size_t)rows_kv * p.n_slots * r * pes : 0);
    pl->total = off;
    return RATTN_OK;
}

// ---- chunked prefill through its own kernel (bf16; a paged prefix whose
// table fits in LDS).  Other prefill calls run on the split kernel with the
// causal mask.
struct PrefillPlan {
    rattn::PrefillParams pp;
    int cpad;
    size_t lds;
};

bool prefill_direct(const rattn_desc *d) {
    if (d->dtype != RATTN_BF16) return false;
    if (d->page_size > 0 && d->prefix_len > 0 &&
        (d->prefix_len - 1) / d->page_size + 1 > rattn::kMaxPagesPerSplit)
        return false;
    return true;
}

int make_prefill_plan(const rattn_desc *d, PrefillPlan *pl) {
    rattn::PrefillParams &p = pl->pp;
    p = rattn::PrefillParams{};
    const int N = d->n_agents, HK = d->n_kv_heads, g = d->n_q_heads / d->n_kv_heads, r = d->rank;
    const int D = d->head_dim;
    const int64_t L = d->prefix_len, S = d->priv_len;
    const bool resid = r > 0 && L > 0;
    p.L = L;
    p.S = S;
    p.N = N;
    p.QL = d->q_len;
    p.HQ = d->n_q_heads;
    p.HK = HK;
    p.g = g;
    p.r = resid ? r : 0;
    p.lr_shift = 0;
    while (r > 0 && (1 << p.lr_shift) < r) ++p.lr_shift;
    p.ps = d->page_size;
    p.fd_ps = rattn::make_fastdiv(p.ps);
    p.shared_lr = d->shared_lr;
    const float scale = d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)D);
    p.c = scale * 1.44269504088896340736f;
    p.rpa = d->q_len * g;
    pl->cpad = resid ? (pow2ceil(r) < 32 ? 32 : pow2ceil(r)) : 0;
    p.n_qb = (int)cdiv(p.rpa, rattn::prefill_rows(D, pl->cpad));
    const int64_t items = (int64_t)HK * N * p.n_qb;
    if (items > (1ll << 30)) return RATTN_E_UNSUPPORTED;
    p.n_items = (int)items;
    p.per_xcd = (int)cdiv(items, 8);

    // LDS rings: prefix tiles (keys, values and the low-rank rows), chunk tiles
    // (keys and values); T keys per stage, two to eight stages, the split's
    // page-table entries after them.  128-key stages halve the ring's
    // synchronisation per key against 64-key ones; 64 when 128 leaves no room.
    const int es = (int)esize(d->dtype);
    const int kv_chunks = D * es / 16;
    const int lr_chunks = resid ? pow2ceil(r * es / 16) : 0;
    const int table_bytes = d->page_size > 0 && L > 0 ? (int)((L - 1) / d->page_size + 1) * 4 : 0;
    auto plan_tile = [&](int T) -> bool {
        p.T = T;
        p.stage_bytes_pre = T * 16 * (2 * kv_chunks + 2 * lr_chunks);
        p.stage_bytes_ch = T * 16 * (2 * kv_chunks);
        const int room = rattn::kLdsMax - table_bytes;
        p.nst_pre = room / p.stage_bytes_pre < 8 ? room / p.stage_bytes_pre : 8;
        p.nst_ch = room / p.stage_bytes_ch < 8 ? room / p.stage_bytes_ch : 8;
        if (p.nst_pre < 2 || p.nst_ch < 2) return false;
        int ring = p.nst_pre * p.stage_bytes_pre;
        if (p.nst_ch * p.stage_bytes_ch > ring) ring = p.nst_ch * p.stage_bytes_ch;
        p.table_lds_off = ring;
        pl->lds = (size_t)(ring + table_bytes);
        return true;
    };
    if (!plan_tile(128) && !plan_tile(64) && !plan_tile(32)) return RATTN_E_UNSUPPORTED;
    return RATTN_OK;
}

// ---- decode with rebuilt residual keys (rattn_decode_reconstruct): its split
// kernel writes the decode workspace layout, whose merge launch finishes it.
struct ReconPlan {
    rattn::ReconParams rp;
    rattn::DecodeParams dp;  // for the merge
    size_t off_ml, off_o, off_w, total;
};

int make_recon_plan(const rattn_desc *d, bool rope, ReconPlan *pl) {
    rattn::ReconParams &p = pl->rp;
    p = rattn::ReconParams{};
    const int N = d->n_agents, HK = d->n_kv_heads, g = d->n_q_heads / d->n_kv_heads, r = d->rank;
    const int D = d->head_dim;
    const int64_t L = d->prefix_len;
    p.L = L;
    p.N = N;
    p.QL = d->q_len;
    p.HQ = d->n_q_heads;
    p.HK = HK;
    p.g = g;
    p.rpa = d->q_len * g;
    p.r = r;
    p.shared_lr = d->shared_lr;
    const float scale = d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)D);
    p.c = scale * 1.44269504088896340736f;
    // agents in balanced groups of at most one per wave; each agent's rows take
    // waves / agents waves, at most one per 16-token step of a stage
    const int waves = rattn::recon_waves(rope, r);
    const int n_groups = (int)cdiv(N, waves);
    p.apg = (int)cdiv(N, n_groups);
    p.n_ag = (int)cdiv(N, p.apg);
    const int na_lr = d->shared_lr ? 1 : p.apg;
    if ((int64_t)na_lr * L * r * 2 >= (1ll << 31)) return RATTN_E_UNSUPPORTED;  // 32-bit fill offsets
    auto stage_of = [&](int t) { return t * (2 * D * 2 + 2 * na_lr * r * 2); };
    const int room = rattn::kLdsMax;
    p.T = rattn::kReconTMax;
    if (room / stage_of(p.T) < 3) p.T /= 2;
    p.stage_bytes = stage_of(p.T);
    const int nst = room / p.stage_bytes;
    p.nst = nst < 4 ? nst : 4;
    if (p.nst < 2) return RATTN_E_UNSUPPORTED;
    p.tg = waves / p.apg;
    if (p.tg > p.T / 16) p.tg = p.T / 16;
    if (p.tg == 3) p.tg = 2;  // a power of two, dividing the steps of a stage
    const int64_t base = (int64_t)HK * p.n_ag;
    int64_t n = cdiv(kTargetItems, base);
    const int64_t nmax = cdiv(L, p.T);
    if (n > nmax) n = nmax;
    if (n > rattn::kMaxSlots / p.tg) n = rattn::kMaxSlots / p.tg;
    if (n < 1) n = 1;
    p.tok_split = (int)roundup(cdiv(L, n), p.T);
    p.n_splits = (int)cdiv(L, p.tok_split);
    p.n_slots = p.n_splits * p.tg;
    if (p.n_slots > rattn::kMaxSlots) return RATTN_E_UNSUPPORTED;
    const int64_t items = (int64_t)p.n_splits * base;
    if (items > (1ll << 30)) return RATTN_E_UNSUPPORTED;
    p.n_items = (int)items;
    p.per_xcd = (int)cdiv(items, 8);

    // the merge: every field combine_kernel reads
    rattn::DecodeParams &q = pl->dp;
    q = rattn::DecodeParams{};
    q.L = L;
    q.N = N;
    q.QL = d->q_len;
    q.HQ = d->n_q_heads;
    q.HK = HK;
    q.g = g;
    q.r = r;
    q.rpa = p.rpa;
    q.n_ps = p.n_slots;  // every slot carries W
    q.n_slots = p.n_slots;
    q.fd_hq = rattn::make_fastdiv(q.HQ);
    q.fd_ql = rattn::make_fastdiv(q.QL);
    q.fd_g = rattn::make_fastdiv(g);
    const int64_t rows_kv = (int64_t)HK * N * p.rpa;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += (bytes + 255) & ~(size_t)255;
        return o;
    };
    pl->off_ml = take((size_t)rows_kv * p.n_slots * 2 * sizeof(float));
    pl->off_o = take((size_t)rows_kv * p.n_slots * D * 2);  // fp16, divided by l
    pl->off_w = take((size_t)rows_kv * p.n_slots * r * 2);
    pl->total = off;
    return RATTN_OK;
}

int check_args(const rattn_desc *d, const rattn_args *a) {
    if (!a) return RATTN_E_NULL;
    const bool paged = d->page_size > 0;
    const bool pre = d->prefix_len > 0;
    const bool resid = d->rank > 0 && pre;
    if (!a->q || !a->out) return RATTN_E_NULL;
    if (pre && (!a->k_base || !a->v_base)) return RATTN_E_NULL;
    if (paged && pre && !a->block_table) return RATTN_E_NULL;
    if (!paged && a->block_table) return RATTN_E_NULL;
    if (resid && (!a->lk || !a->lv || !a->bk || !a->bv)) return RATTN_E_NULL;
    if (d->priv_len > 0 && (!a->k_priv || !a->v_priv)) return RATTN_E_NULL;
    const void *ptrs[] = {a->q, a->k_base, a->v_base, a->lk, a->lv, a->bk, a->bv, a->k_priv, a->v_priv, a->out};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return RATTN_E_ALIGN;
    if (a->lse && !aligned(a->lse, 4)) return RATTN_E_ALIGN;
    if (a->block_table && !aligned(a->block_table, 4)) return RATTN_E_ALIGN;
    if (d->v_format == RATTN_VALUES_FWHT3) {
        if (pre && !a->v_scale) return RATTN_E_NULL;
        if (a->v_scale && !aligned(a->v_scale, 16)) return RATTN_E_ALIGN;
    } else if (a->v_scale) {
        return RATTN_E_NULL;
    }
    return RATTN_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return RATTN_OK;
    g_last_hip = (int)e;
    return RATTN_E_HIP;
}

int run_attention(const rattn_desc *d, const rattn_args *a, void *ws, size_t ws_bytes, void *stream, int op,
                  unsigned stages) {
    if (stages == 0 || (stages & ~(unsigned)RATTN_STAGE_ALL)) return RATTN_E_SHAPE;
    int st = check_desc(d, op);
    if (st) return st;
    st = check_args(d, a);
    if (st) return st;
    if (op == RATTN_OP_PREFILL && prefill_direct(d)) {
        PrefillPlan pp;
        st = make_prefill_plan(d, &pp);
        if (st) return st;
        rattn::PrefillParams &q = pp.pp;
        q.q = a->q;
        q.kb = a->k_base;
        q.vb = a->v_base;
        q.table = a->block_table;
        q.lk = a->lk;
        q.lv = a->lv;
        q.bk = a->bk;
        q.bv = a->bv;
        q.kp = a->k_priv;
        q.vp = a->v_priv;
        q.out = a->out;
        q.lse = a->lse;
        if (!(stages & RATTN_STAGE_SPLIT)) return RATTN_OK;  // no merge pass on this path
        return hip_status(rattn::launch_prefill(q, d->head_dim, pp.cpad, pp.lds, static_cast<hipStream_t>(stream)));
    }
    Plan pl;
    st = make_plan(d, op, &pl);
    if (st) return st;
    if (!ws) return RATTN_E_WORKSPACE;
    if (ws_bytes < pl.total) return RATTN_E_WORKSPACE;
    if (!aligned(ws, 256)) return RATTN_E_ALIGN;

    char *w = static_cast<char *>(ws);
    rattn::DecodeParams &p = pl.dp;
    p.q = a->q;
    p.kb = a->k_base;
    p.vb = a->v_base;
    p.table = a->block_table;
    p.lk = a->lk;
    p.lv = a->lv;
    p.bk = a->bk;
    p.bv = a->bv;
    p.kp = a->k_priv;
    p.vp = a->v_priv;
    p.out = a->out;
    p.lse = a->lse;
    p.vs = a->v_scale;
    p.p_ml = reinterpret_cast<float *>(w + pl.off_ml);
    p.p_o = w + pl.off_o;
    p.p_w = w + pl.off_w;
    if (!(d->rank > 0 && d->prefix_len > 0)) p.r = 0;  // no residual without a prefix
    return hip_status(rattn::launch_decode(d->dtype == RATTN_BF16, p, d->head_dim, pl.cpad, pl.lds, stages,
                                           static_cast<hipStream_t>(stream)));
}

void fill_plan_info(const Plan &pl, rattn_plan_info *info) {
    *info = rattn_plan_info{};
    info->n_prefix_splits = pl.dp.n_ps;
    info->prefix_split_len = pl.dp.tok_ps;
    info->n_priv_splits = pl.dp.n_pv;
    info->priv_split_len = pl.dp.tok_pv;
    info->row_blocks = pl.dp.n_blocks;
    info->agents_per_block = pl.dp.apb;
    info->resid_cols = pl.cpad;
    info->work_items = pl.dp.n_items;
    info->heads_per_item = pl.dp.H;
    info->waves = pl.dp.nw + pl.dp.np;
    info->masked = pl.dp.masked;
    info->blocks_per_group = pl.dp.bpg;
    info->path = 0;
    info->rows_per_item = 0;
}

}  // namespace

extern "C" {

int rattn_version(void) { return RATTN_VERSION; }

int rattn_last_hip_error(void) { return g_last_hip; }

const char *rattn_status_str(int s) {
    switch (s) {
        case RATTN_OK: return "ok";
        case RATTN_E_NULL: return "null or forbidden pointer";
        case RATTN_E_SHAPE: return "inconsistent shape";
        case RATTN_E_UNSUPPORTED: return "unsupported configuration";
        case RATTN_E_WORKSPACE: return "workspace missing or too small";
        case RATTN_E_ALIGN: return "misaligned pointer";
        case RATTN_E_HIP: return "HIP runtime error";
        case RATTN_E_SCRATCH: return "call needs more than the static scratch buffer holds";
        case RATTN_E_POOL: return "page pool: not enough free pages";
        default: return "unknown status";
    }
}

int rattn_workspace_bytes(const rattn_desc *desc, int op, size_t *bytes) {
    if (!bytes) return RATTN_E_NULL;
    int st = check_desc(desc, op);
    if (st) return st;
    if (op == RATTN_OP_PREFILL && prefill_direct(desc)) {
        PrefillPlan pp;
        st = make_prefill_plan(desc, &pp);
        if (st) return st;
        *bytes = 0;  // the prefill kernel needs no workspace
        return RATTN_OK;
    }
    if (op == RATTN_OP_RECONSTRUCT) {
        // enough for the call with or without a rotation (their plans differ)
        ReconPlan rp, rp2;
        st = make_recon_plan(desc, false, &rp);
        if (st) return st;
        st = make_recon_plan(desc, true, &rp2);
        if (st) return st;
        *bytes = rp.total > rp2.total ? rp.total : rp2.total;
        return RATTN_OK;
    }
    Plan pl;
    st = make_plan(desc, op, &pl);
    if (st) return st;
    *bytes = pl.total;
    return RATTN_OK;
}

int rattn_decode_plan(const rattn_desc *desc, rattn_plan_info *info) {
    if (!info) return RATTN_E_NULL;
    int st = check_desc(desc, RATTN_OP_DECODE);
    if (st) return st;
    Plan pl;
    st = make_plan(desc, RATTN_OP_DECODE, &pl);
    if (st) return st;
    fill_plan_info(pl, info);
    return RATTN_OK;
}

int rattn_prefill_plan(const rattn_desc *desc, rattn_plan_info *info) {
    if (!info) return RATTN_E_NULL;
    int st = check_desc(desc, RATTN_OP_PREFILL);
    if (st) return st;
    if (prefill_direct(desc)) {
        PrefillPlan pp;
        st = make_prefill_plan(desc, &pp);
        if (st) return st;
        *info = rattn_plan_info{};
        info->n_prefix_splits = desc->prefix_len > 0 ? 1 : 0;
        info->prefix_split_len = desc->prefix_len;
        info->row_blocks = (int)((pp.pp.rpa + 15) / 16);
        info->agents_per_block = 1;
        info->resid_cols = pp.cpad;
        info->work_items = pp.pp.n_items;
        info->heads_per_item = 1;
        info->waves = rattn::kPrefillWaves;
        info->blocks_per_group = rattn::prefill_blocks_per_wave(desc->head_dim, pp.cpad) * rattn::kPrefillWaves;
        info->path = 1;
        info->rows_per_item = rattn::prefill_rows(desc->head_dim, pp.cpad);
        return RATTN_OK;
    }
    Plan pl;
    st = make_plan(desc, RATTN_OP_PREFILL, &pl);
    if (st) return st;
    fill_plan_info(pl, info);
    return RATTN_OK;
}

int rattn_decode(const rattn_desc *desc, const rattn_args *args, void *workspace, size_t workspace_bytes,
                 void *stream) {
    return run_attention(desc, args, workspace, workspace_bytes, stream, RATTN_OP_DECODE, RATTN_STAGE_ALL);
}

int rattn_prefill_chunk(const rattn_desc *desc, const rattn_args *args, void *workspace,
                        size_t workspace_bytes, void *stream) {
    return run_attention(desc, args, workspace, workspace_bytes, stream, RATTN_OP_PREFILL, RATTN_STAGE_ALL);
}

int rattn_decode_noalloc(const rattn_desc *desc, const rattn_args *args, void *stream) {
    int st = check_desc(desc, RATTN_OP_DECODE);
    if (st) return st;
    st = check_args(desc, args);
    if (st) return st;
    Plan pl;
    st = make_plan(desc, RATTN_OP_DECODE, &pl);
    if (st) return st;
    if (pl.total > rattn::kNoAllocScratchBytes) return RATTN_E_SCRATCH;
    void *ws = nullptr;
    st = hip_status(rattn::noalloc_scratch(&ws));
    if (st) return st;
    return run_attention(desc, args, ws, rattn::kNoAllocScratchBytes, stream, RATTN_OP_DECODE, RATTN_STAGE_ALL);
}

int rattn_lr_project(const rattn_lr_desc *d, const void *x, const void *ak_t, const void *av_t, void *lk, void *lv,
                     void *stream) {
    if (!d) return RATTN_E_NULL;
    if (d->n_sets < 1 || d->d_in < 1 || d->rank < 1 || d->n_tokens < 0 || d->pos0 < 0 || d->cache_len < 0 ||
        (d->shared_x != 0 && d->shared_x != 1) || (d->shared_a != 0 && d->shared_a != 1))
        return RATTN_E_SHAPE;
    if (d->pos0 + d->n_tokens > d->cache_len) return RATTN_E_SHAPE;
    if (d->shared_x && d->shared_a && d->n_sets != 1) return RATTN_E_SHAPE;
    if (d->dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    const int r = d->rank;
    if (!(r == 8 || r == 16 || r == 32 || r == 64 || r == 128) || d->d_in % 128) return RATTN_E_UNSUPPORTED;
    // index arithmetic: columns and workgroup counts in 32 bits
    if ((int64_t)d->n_sets * 2 * r > (1ll << 24) || d->n_tokens > (1ll << 40)) return RATTN_E_UNSUPPORTED;
    if (d->n_tokens == 0) return RATTN_OK;
    if (!x || !ak_t || !av_t || !lk || !lv) return RATTN_E_NULL;
    const void *ptrs[] = {x, ak_t, av_t, lk, lv};
    for (const void *p : ptrs)
        if (!aligned(p, 16)) return RATTN_E_ALIGN;
    rattn::LrParams p{};
    p.x = x;
    p.ak = ak_t;
    p.av = av_t;
    p.lk = lk;
    p.lv = lv;
    p.T = d->n_tokens;
    p.pos0 = d->pos0;
    p.cache_len = d->cache_len;
    p.d_in = d->d_in;
    p.r = r;
    p.shared_a = d->shared_a;
    p.n_xsets = d->shared_x ? 1 : d->n_sets;
    p.cols_per_xset = d->shared_x ? d->n_sets * 2 * r : 2 * r;
    return hip_status(rattn::launch_lr_project(p, static_cast<hipStream_t>(stream)));
}

int rattn_append_kv(const rattn_desc *d, void *pool_k, void *pool_v, const int32_t *table, int64_t cur_len,
                    int64_t n_new, const void *k_new, const void *v_new, int32_t cow_src, int32_t cow_dst,
                    void *stream) {
    if (!d) return RATTN_E_NULL;
    if (d->n_kv_heads < 1 || d->head_dim < 1 || d->page_size < 1 || d->n_phys_pages < 1 || cur_len < 0 ||
        n_new < 0)
        return RATTN_E_SHAPE;
    if (d->dtype != RATTN_F32 && d->dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    if (d->page_size % 16 || (d->head_dim * esize(d->dtype)) % 16) return RATTN_E_UNSUPPORTED;
    if ((cow_src < 0) != (cow_dst < 0)) return RATTN_E_SHAPE;
    if (cow_src >= 0 && (cow_src >= d->n_phys_pages || cow_dst >= d->n_phys_pages || cow_src == cow_dst))
        return RATTN_E_SHAPE;
    if (cow_src >= 0 && cur_len % d->page_size == 0) return RATTN_E_SHAPE;  // nothing to keep from the original
    if (d->n_phys_pages > INT32_MAX || (cur_len + n_new) / d->page_size > INT32_MAX) return RATTN_E_UNSUPPORTED;
    const int64_t rows = (int64_t)d->n_kv_heads * (n_new + d->page_size);
    if (rows > (1ll << 40)) return RATTN_E_UNSUPPORTED;
    if (n_new == 0 && cow_src < 0) return RATTN_OK;
    if (!pool_k || !pool_v || (n_new > 0 && (!table || !k_new || !v_new))) return RATTN_E_NULL;
    const void *ptrs[] = {pool_k, pool_v, k_new, v_new};
    for (const void *p : ptrs)
        if (p && !aligned(p, 16)) return RATTN_E_ALIGN;
    if (table && !aligned(table, 4)) return RATTN_E_ALIGN;
    rattn::AppendParams p{};
    p.pool_k = pool_k;
    p.pool_v = pool_v;
    p.table = table;
    p.k_new = k_new;
    p.v_new = v_new;
    p.cur_len = cur_len;
    p.T = n_new;
    p.HK = d->n_kv_heads;
    p.ps = d->page_size;
    p.row_vec = (int)(d->head_dim * esize(d->dtype) / 16);
    p.off = cow_src >= 0 ? (int)(cur_len % d->page_size) : 0;
    p.cow_src = cow_src;
    p.cow_dst = cow_dst;
    return hip_status(rattn::launch_append_kv(p, static_cast<hipStream_t>(stream)));
}

int rattn_quantize_keys(const void *k, int64_t n, int32_t dtype, void *codes, float *scale, void *stream) {
    if (n < 1) return RATTN_E_SHAPE;
    if (dtype != RATTN_F32 && dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    if (!k || !codes || !scale) return RATTN_E_NULL;
    if (!aligned(k, esize(dtype)) || !aligned(scale, 4)) return RATTN_E_ALIGN;
    return hip_status(rattn::launch_quantize(k, n, dtype == RATTN_BF16, codes, scale, static_cast<hipStream_t>(stream)));
}

int rattn_quantize_values(const void *v, int64_t n, int32_t head_dim, int32_t dtype, void *codes, float *scale,
                          void *stream) {
    if (n < 1) return RATTN_E_SHAPE;
    if (head_dim != 64 && head_dim != 128) return RATTN_E_UNSUPPORTED;
    if (dtype != RATTN_F32 && dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    if (!v || !codes || !scale) return RATTN_E_NULL;
    if (!aligned(v, esize(dtype)) || !aligned(codes, 8) || !aligned(scale, 4)) return RATTN_E_ALIGN;
    return hip_status(rattn::launch_values3_encode(v, n, head_dim, dtype == RATTN_BF16, values_codebook().b, codes,
                                                   scale, static_cast<hipStream_t>(stream)));
}

int rattn_values_codebook(double *centroids, double *boundaries) {
    if (!centroids || !boundaries) return RATTN_E_NULL;
    const ValuesCodebook &cb = values_codebook();
    for (int k = 0; k < 8; ++k) centroids[k] = cb.c[k];
    for (int k = 0; k < 7; ++k) boundaries[k] = cb.b[k];
    return RATTN_OK;
}

int rattn_decode_reconstruct(const rattn_desc *desc, const rattn_args *args, const float *rope_theta,
                             void *workspace, size_t workspace_bytes, void *stream) {
    int st = check_desc(desc, RATTN_OP_RECONSTRUCT);
    if (st) return st;
    st = check_args(desc, args);
    if (st) return st;
    ReconPlan pl;
    st = make_recon_plan(desc, rope_theta != nullptr, &pl);
    if (st) return st;
    if (!workspace) return RATTN_E_WORKSPACE;
    if (workspace_bytes < pl.total) return RATTN_E_WORKSPACE;
    if (!aligned(workspace, 256)) return RATTN_E_ALIGN;
    if (rope_theta && !aligned(rope_theta, 4)) return RATTN_E_ALIGN;
    char *w = static_cast<char *>(workspace);
    rattn::ReconParams &p = pl.rp;
    p.q = args->q;
    p.kb = args->k_base;
    p.vb = args->v_base;
    p.lk = args->lk;
    p.lv = args->lv;
    p.bk = args->bk;
    p.theta = rope_theta;
    p.p_ml = reinterpret_cast<float *>(w + pl.off_ml);
    p.p_o = w + pl.off_o;
    p.p_w = w + pl.off_w;
    rattn::DecodeParams &q = pl.dp;
    q.p_ml = p.p_ml;
    q.p_o = p.p_o;
    q.p_w = p.p_w;
    q.bv = args->bv;
    q.out = args->out;
    q.lse = args->lse;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    st = hip_status(rattn::launch_recon(p, s));
    if (st) return st;
    return hip_status(rattn::launch_decode(1, q, desc->head_dim, 0, 0, RATTN_STAGE_COMBINE, s));
}

int rattn_attention_stages(const rattn_desc *desc, int op, const rattn_args *args, void *workspace,
                           size_t workspace_bytes, void *stream, unsigned stages) {
    if (op != RATTN_OP_DECODE && op != RATTN_OP_PREFILL) return RATTN_E_SHAPE;
    return run_attention(desc, args, workspace, workspace_bytes, stream, op, stages);
}

int rattn_gather_base(const rattn_desc *d, const void *pool, const int32_t *block_table, void *dst,
                      void *stream) {
    if (!d) return RATTN_E_NULL;
    if (d->n_kv_heads < 1 || d->head_dim < 1 || d->prefix_len < 0 || d->page_size < 0 || d->n_phys_pages < 0)
        return RATTN_E_SHAPE;
    if (d->dtype != RATTN_F32 && d->dtype != RATTN_BF16) return RATTN_E_UNSUPPORTED;
    if (d->page_size == 0 || d->page_size % 16) return RATTN_E_UNSUPPORTED;
    if ((d->head_dim * esize(d->dtype)) % 16) return RATTN_E_UNSUPPORTED;
    if (d->prefix_len == 0) return RATTN_OK;
    if (d->n_phys_pages < 1) return RATTN_E_SHAPE;
    if (!pool || !block_table || !dst) return RATTN_E_NULL;
    if (!aligned(pool, 16) || !aligned(dst, 16) || !aligned(block_table, 4)) return RATTN_E_ALIGN;
    return hip_status(rattn::launch_gather(pool, block_table, dst, d->prefix_len, d->n_kv_heads, d->page_size,
                                           (int)(d->head_dim * esize(d->dtype)), static_cast<hipStream_t>(stream)));
}

int rattn_check_block_table(const rattn_desc *d, const int32_t *block_table, int32_t *bad_count, void *stream) {
    if (!d || !bad_count) return RATTN_E_NULL;
    if (d->prefix_len < 0 || d->page_size < 0 || d->n_phys_pages < 0) return RATTN_E_SHAPE;
    if (d->page_size == 0 || d->page_size % 16) return RATTN_E_UNSUPPORTED;
    if (!aligned(bad_count, 4)) return RATTN_E_ALIGN;
    const int64_t n = cdiv(d->prefix_len, d->page_size);
    if (n > 0 && !block_table) return RATTN_E_NULL;
    if (block_table && !aligned(block_table, 4)) return RATTN_E_ALIGN;
    return hip_status(rattn::launch_check_table(block_table, n, d->n_phys_pages, bad_count,
                                                static_cast<hipStream_t>(stream)));
}

}  // extern "C"
