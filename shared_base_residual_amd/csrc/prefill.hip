// prefill.hip -- chunked-prefill kernel of librattn (gfx950).
//
// Agent a appends a chunk of C tokens with private keys and values; chunk query
// t attends the shared prefix (base keys/values plus the rank-r residual) and
// chunk tokens 0..t.  The residual algebra is the decode kernel's (ForkKV Guide,
// "Fused ResidualAttention"; LRAgent, "Flash-LoRA-Attention"):
//   score  s = scale * (q . K_base[j] + (q Bk_a^T) . Lk[j])
//   output o = sum_j p_j V[j] + (sum_j p_j Lv[j]) Bv_a
// With BaseLRShared (LRAgent, "Schemi di Condivisione": the down-projection A is
// shared) Lk and Lv are one cache for every agent, so the score correction is
// one dense rank-r MFMA contraction per key tile, like the base product.
//
// This is MFMA-bound work (thousands of query rows per KV head), so a workgroup
// takes 256 query rows of one (KV head, agent) and streams the whole context
// once: the prefix, then the chunk with the causal mask, through the same LDS
// ring as the decode kernel (direct global->LDS loads, several tiles in
// flight).  Each of the eight waves (two per SIMD, so one wave's MFMAs overlap
// the other's softmax) owns 32 rows (two 16-row MFMA blocks); every tile
// fetched into LDS feeds all 256 rows.  With wide residuals (d = 128 and 64 or
// more residual columns, d = 64 and 128) a wave owns one block and a workgroup
// 128 rows, so that the accumulators stay in registers.  Workgroups of one KV
// head run on one XCD (workgroup i runs on XCD i % 8), where they share its
// tiles through that XCD's L2.
//
// Per 32 keys and wave: S^T = K Q^T (keys as the A operand, query rows as B),
// + Lk U^T (U = q Bk_a^T as bf16 hi + lo halves), online softmax in the log2
// domain with the scale folded into the exponent (exp2(s * scale*log2(e) - m)),
// O^T += V^T P^T and W^T += Lv^T P^T with P straight from the score registers.
// At the end O^T += Bv^T W^T (W as hi + lo halves), so Bv
// is applied once per row, and o = O / l is written.  No split-K, no workspace.
#include "device.h"
#include "internal.h"
#include "stage.h"

namespace rattn {

template <typename T, int D, int CPAD>
__global__ __launch_bounds__(512) void prefill_kernel(PrefillParams p) {
    touch_params<PrefillParams>();
    using O = Ops<T>;
    using frag = typename O::frag;
    constexpr int KS = D / 32;
    constexpr int VPL = D / 16;
    constexpr int CS = CPAD / 32;
    constexpr int CSx = CS > 0 ? CS : 1;
    constexpr int CPL = CPAD / 16;
    constexpr int CPLx = CPL > 0 ? CPL : 1;
    constexpr int ES = (int)sizeof(T);
    constexpr int NCB = prefill_blocks_per_wave(D, CPAD);  // 16-row blocks per wave
    constexpr int NW = kPrefillWaves;
    constexpr int ROWS = prefill_rows(D, CPAD);  // query rows per workgroup

    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15;
    const int j4 = lane >> 4;

    const int bid = blockIdx.x;
    const int li = (bid & 7) * p.per_xcd + (bid >> 3);
    if (li >= p.n_items) return;
    // items: KV head slowest, so that consecutive items (one XCD) share a head
    const int per_head = p.N * p.n_qb;
    const int k = li / per_head;
    const int rest = li - k * per_head;
    const int a = rest / p.n_qb;
    const int qb = rest - a * p.n_qb;
    const int R0 = qb * ROWS + wave * (NCB * 16);  // this wave's first row within (a, k)

    const bool resid = CPAD > 0 && p.r > 0 && p.L > 0;
    const float cl2 = p.c;

    // ---- this lane's query row in each block, and the query rows as B operands
    const T *qp = static_cast<const T *>(p.q);
    bool vm[NCB];
    int tq[NCB];
    int64_t qrow[NCB];
    frag qB[NCB][KS];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const int ria = R0 + 16 * cb + n16;
        vm[cb] = ria < p.rpa;
        const int rr = vm[cb] ? ria : 0;
        tq[cb] = rr / p.g;
        const int hh = rr - tq[cb] * p.g;
        qrow[cb] = ((int64_t)a * p.QL + tq[cb]) * p.HQ + (int64_t)k * p.g + hh;
#pragma unroll
        for (int s = 0; s < KS; ++s)
            qB[cb][s] = vm[cb] ? O::load8(qp + qrow[cb] * D + 32 * s + 8 * j4) : O::zero();
    }
    // last chunk token any row of the workgroup may see
    int rmax = qb * ROWS + ROWS - 1;
    rmax = rmax < p.rpa - 1 ? rmax : p.rpa - 1;
    const int t_hi = rmax / p.g + 1;  // chunk keys [0, t_hi)

    // ---- U = q Bk_a^T as the B operand of the rank-r score
    // correction (bf16 hi + lo halves).  U^T = Bk Q^T with MFMA; A-operand row
    // rho of output tile 2s+h is residual column 32s + 8(rho/4) + 4h + rho%4, so
    // each lane's results land in its own B-operand slots.  The Bk rows are the
    // same for both blocks.
    frag uH[NCB][CSx], uL[NCB][CSx];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int s = 0; s < CSx; ++s) {
            uH[cb][s] = O::zero();
            uL[cb][s] = O::zero();
        }
    if constexpr (CPAD > 0) {
        if (resid) {
            const T *bk = static_cast<const T *>(p.bk) + (int64_t)a * p.r * p.HK * D + (int64_t)k * D + 8 * j4;
            const int64_t ldb = (int64_t)p.HK * D;
#pragma unroll
            for (int s = 0; s < CSx; ++s) {
                frag bkf[2][KS];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    int crow = 32 * s + 8 * (n16 >> 2) + 4 * h + (n16 & 3);
                    crow = crow < p.r ? crow : 0;
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) bkf[h][s2] = O::load8(bk + crow * ldb + 32 * s2);
                }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    float uv[8];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s2 = 0; s2 < KS; ++s2) acc = O::mma(bkf[h][s2], qB[cb][s2], acc);
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int c = 32 * s + 8 * j4 + 4 * h + i;
                            uv[4 * h + i] = (vm[cb] && c < p.r) ? acc[i] : 0.0f;
                        }
                    }
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        O::set(uH[cb][s], i, uv[i]);
                        const float hi = (float)(bf16)uv[i];
                        O::set(uL[cb][s], i, uv[i] - hi);
                    }
                }
            }
        }
    }
    wait_vmcnt(0);  // every register load has landed: nothing pending inside the rings

    // l: each row's weight sum, in every element (a ones-row product, below)
    f32x4 o[NCB][VPL], w[NCB][CPLx], l[NCB];
    float m[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) o[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < CPLx; ++i) w[cb][i] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[cb] = -1.0e30f;
        l[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    int *s_pages = reinterpret_cast<int *>(smem + p.table_lds_off);
    const int kv_rowb = D * ES;

    // ---- one phase: the prefix (with residual) or the chunk (causal)
    for (int phase = 0; phase < 2; ++phase) {
        const bool pre = phase == 0;
        const int t0 = 0;
        const int t1 = pre ? (int)p.L : t_hi;
        if (t1 <= 0) continue;
        const bool res = pre && resid;
        Geo g;
        g.T = p.T;
        g.nst = pre ? p.nst_pre : p.nst_ch;
        g.stage_bytes = pre ? p.stage_bytes_pre : p.stage_bytes_ch;
        g.cpr_kv = D * ES / 16;
        g.lg_kv = ilog2(g.cpr_kv);
        g.cpr_k = g.cpr_kv;
        g.lg_k = g.lg_kv;
        if (res) {
            g.cpa_lr = p.r * ES / 16;
            g.lg_lr = ilog2(g.cpa_lr);
            g.na_lr = 1;  // one agent's (or the shared) low-rank rows
        } else {
            g.cpa_lr = 1;
            g.lg_lr = 0;
            g.na_lr = 0;
        }
        g.lr_grp = 16 * g.na_lr * g.cpa_lr;
        g.H = 1;
        g.ofs_v = g.T * g.cpr_kv;
        g.ofs_lk = 2 * g.T * g.cpr_kv;
        g.ofs_lv = g.ofs_lk + (res ? g.T * g.cpa_lr : 0);
        g.chunks = g.ofs_lv + (res ? g.T * g.cpa_lr : 0);

        Src<T> src;
        src.tlast = t1 - 1;
        src.r = p.r > 0 ? p.r : 1;
        src.lk = src.lv = nullptr;
        src.lr_agent_stride = 0;
        src.head_stride = 0;
        src.page_stride = 0;
        src.k_head_stride = 0;
        src.k_page_stride = 0;
        src.fps = p.fd_ps;
        src.pg0 = 0;
        src.pages = s_pages;
        if (pre) {
            src.kb = static_cast<const T *>(p.kb);
            src.vb = static_cast<const T *>(p.vb);
            if (p.ps > 0) {
                src.page_stride = (int64_t)p.HK * p.ps * D;
                src.kb += (int64_t)k * p.ps * D;
                src.vb += (int64_t)k * p.ps * D;
                const int npg = fdiv(t1 - 1, p.fd_ps) + 1;
                for (int i = threadIdx.x; i < npg; i += 64 * NW) s_pages[i] = p.table[i];
                __syncthreads();
            } else {
                src.kb += (int64_t)k * p.L * D;
                src.vb += (int64_t)k * p.L * D;
            }
            src.k_page_stride = src.page_stride;
            src.k_head_stride = src.head_stride;
            if (res) {
                const int64_t a_lr = p.shared_lr ? 0 : a;
                src.lk = static_cast<const T *>(p.lk) + a_lr * p.L * p.r;
                src.lv = static_cast<const T *>(p.lv) + a_lr * p.L * p.r;
                src.lr_agent_stride = p.L * p.r;
            }
        } else {
            const int64_t seg = ((int64_t)a * p.HK + k) * p.S * D;
            src.kb = static_cast<const T *>(p.kp) + seg;
            src.vb = static_cast<const T *>(p.vp) + seg;
        }

        GroupFill fp;
        make_group_fill<T, D>(fp, g, src, res, wave, lane, NW);
        ReadOfs<T, D, CPAD> ro;
        {
            using RO = ReadOfs<T, D, CPAD>;
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int c = 0; c < RO::FC; ++c)
                    ro.k[s][c] = elem_ofs(0, n16, (32 * s + 8 * j4) * ES + 16 * c, g.cpr_kv, g.lg_kv);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < RO::VC; ++c)
                    ro.v[i][c] = elem_ofs(g.ofs_v, 4 * j4 + i, VPL * n16 * ES + 16 * c, g.cpr_kv, g.lg_kv);
#pragma unroll
            for (int s = 0; s < RO::CSx; ++s) {
                int col = 32 * s + 8 * j4;
                col = col < p.r ? col : 0;  // padding column: U is zero there
#pragma unroll
                for (int c = 0; c < RO::FC; ++c)
                    ro.lk[s][c] = res ? elem_ofs(g.ofs_lk, n16, col * ES + 16 * c, g.cpa_lr, g.lg_lr) : 0u;
            }
            int colv = RO::CPL * n16;
            colv = colv < p.r ? colv : 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c = 0; c < RO::LC; ++c)
                    ro.lv[i][c] = res ? elem_ofs(g.ofs_lv, 4 * j4 + i, colv * ES + 16 * c, g.cpa_lr, g.lg_lr) : 0u;
        }
        // transposed value reads: for d-tile jj, lane 4i + a of group j4 points at
        // key row 4*j4 + i, columns 16*jj + 4a (the other 16 keys: +16 rows)
        uint32_t vtr[VPL];
#pragma unroll
        for (int jj = 0; jj < VPL; ++jj)
            vtr[jj] = elem_ofs(g.ofs_v, 4 * j4 + (n16 >> 2), 2 * (16 * jj + 4 * (n16 & 3)), g.cpr_kv, g.lg_kv);
        // the same for the Lv rows: residual column tile jj, columns 16*jj + 4a
        // (padding columns c >= r read column 0; their W is dropped at the end)
        uint32_t wtr[CPLx];
#pragma unroll
        for (int jj = 0; jj < CPLx; ++jj) {
            int col = 16 * jj + 4 * (n16 & 3);
            col = col < p.r ? col : 0;
            wtr[jj] = res ? elem_ofs(g.ofs_lv, 4 * j4 + (n16 >> 2), 2 * col, g.cpa_lr, g.lg_lr) : 0u;
        }
        const int lr_rowb = 16 * g.cpa_lr;
        const int n_tiles = (t1 - t0 + g.T - 1) / g.T;
        const int fpw = fp.fpw;
        // contiguous caches with one 16-token group per wave: every wave fills
        // all regions of its group, straight from per-wave source rows
        const bool own = p.ps == 0 && (g.T >> 4) == NW;
        auto fill = [&](int tile, int stage) {
            const int tt = t0 + tile * g.T;
            char *sp = smem + (size_t)stage * g.stage_bytes;
            if (own && tt + g.T - 1 <= src.tlast) {
                constexpr int NKV = D * ES / 64;
                const int tg0 = tt + 16 * wave;
                const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(sp));
                const char *kb = uniform_ptr(reinterpret_cast<const char *>(src.kb + (int64_t)tg0 * D));
                const char *vb = uniform_ptr(reinterpret_cast<const char *>(src.vb + (int64_t)tg0 * D));
                const uint32_t lk0 = lds0 + 16 * (16 * wave * g.cpr_kv), lv0 = lds0 + 16 * (g.ofs_v + 16 * wave * g.cpr_kv);
#pragma unroll
                for (int i = 0; i < NKV; ++i) dma16s(kb, fp.kv_off[i], lk0 + 1024 * i);
#pragma unroll
                for (int i = 0; i < NKV; ++i) dma16s(vb, fp.kv_off[i], lv0 + 1024 * i);
                if (res) {
                    const char *lk = uniform_ptr(reinterpret_cast<const char *>(src.lk + (int64_t)tg0 * src.r));
                    const char *lv = uniform_ptr(reinterpret_cast<const char *>(src.lv + (int64_t)tg0 * src.r));
                    const uint32_t ll0 = lds0 + 16 * (g.ofs_lk + wave * g.lr_grp), lw0 = lds0 + 16 * (g.ofs_lv + wave * g.lr_grp);
                    for (int i = 0; i < fp.n_lr; ++i) {
                        if (64 * i + lane < g.lr_grp) {
                            int row;
                            const uint32_t off = lr_lane_off(fp.lr_stride, g, i, lane, &row);
                            dma16s(lk, off, ll0 + 1024 * i);
                            dma16s(lv, off, lw0 + 1024 * i);
                        }
                    }
                }
                return;
            }
            fill_group<T, D>(fp, g, src, tt, sp, tt + g.T - 1 > src.tlast, lane);
        };
        for (int i = 0; i < g.nst - 1 && i < n_tiles; ++i) fill(i, i);

        for (int it = 0; it < n_tiles; ++it) {
            const int later = (n_tiles - 1 - it) < (g.nst - 2) ? (n_tiles - 1 - it) : (g.nst - 2);
            wait_vmcnt(later * fpw);
            ring_barrier();
            const char *st = smem + (size_t)(it % g.nst) * g.stage_bytes;
            const int tt = t0 + it * g.T;
            const bool masked = !pre || tt + g.T > t1;

            // 32 keys at a time: two 16-key halves per step
            for (int sub = 0; sub < g.T / 32; ++sub) {
                const char *stk = st + 32 * sub * kv_rowb;
                const char *stl = st + 32 * sub * lr_rowb;
                const int tk = tt + 32 * sub;
                // raw scores (unscaled) of the two 16-key halves for the row blocks
                f32x4 sc[NCB][2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    frag kf[KS];
#pragma unroll
                    for (int s = 0; s < KS; ++s) {
                        const Row<T, 8> kr = lds_get<T, 8>(stk + 16 * h * kv_rowb, ro.k[s]);
                        __builtin_memcpy(&kf[s], &kr, sizeof(frag));
                    }
                    frag lkf[CSx];
                    if constexpr (CPAD > 0) {
                        if (res) {
#pragma unroll
                            for (int s = 0; s < CS; ++s) {
                                const Row<T, 8> lr = lds_get<T, 8>(stl + 16 * h * lr_rowb, ro.lk[s]);
                                __builtin_memcpy(&lkf[s], &lr, sizeof(frag));
                            }
                        }
                    }
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < KS; ++s) acc = O::mma(kf[s], qB[cb][s], acc);
                        if constexpr (CPAD > 0) {
                            if (res) {
#pragma unroll
                                for (int s = 0; s < CS; ++s) {
                                    acc = O::mma(lkf[s], uH[cb][s], acc);
                                    acc = O::mma(lkf[s], uL[cb][s], acc);
                                }
                            }
                        }
                        sc[cb][h] = acc;
                    }
                }
                // this wave's share of the refill (stage of tile it - 1, free since the
                // barrier), issued behind the score products of the first or second
                // 32-key step (odd waves the second): the direct loads of all eight
                // waves at one point would queue at the CU's address unit and stall
                // every wave, and later steps leave the two-stage ring too little
                // time to land them
                if (sub == (wave & 1 & (g.T / 32 - 1)) && it + g.nst - 1 < n_tiles)
                    fill(it + g.nst - 1, (it + g.nst - 1) % g.nst);
                if (masked) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int key = tk + 16 * h + 4 * j4 + i;
                                if (key >= t1 || (!pre && key > tq[cb])) sc[cb][h][i] = -__builtin_inff();
                            }
                }

                // online softmax per block (log2 domain); P as the B operand over 32 keys:
                // slots 0..3 = keys 4*j4+i of the first half, 4..7 = the second half.
                // A row's maximum passes the slack iff one of its four lanes' maxima
                // does (the scale is positive and rounding keeps the order), so the
                // cross-lane maxima are formed only on the steps where some lane's
                // passes.  (Scores are finite or -inf, never NaN.)
                float lmx[NCB];
                bool lane_grow = false;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    lmx[cb] = amax3(amax3(sc[cb][0][0], sc[cb][0][1], sc[cb][0][2]),
                                    amax3(sc[cb][0][3], sc[cb][1][0], sc[cb][1][1]), amax(sc[cb][1][2], sc[cb][1][3]));
                    lane_grow = lane_grow || lmx[cb] * cl2 > m[cb] + kRescaleSlack;
                }
                if (__builtin_amdgcn_ballot_w64(lane_grow)) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const float mx = row_max4(lmx[cb]) * cl2;  // scaled (log2 units); -inf stays -inf
                        const bool grow = mx > m[cb] + kRescaleSlack;
                        const float m_new = grow ? mx : m[cb];
                        const float alpha = fexp2(m[cb] - m_new);
                        m[cb] = m_new;
#pragma unroll
                        for (int i = 0; i < VPL; ++i) o[cb][i] *= alpha;
#pragma unroll
                        for (int i = 0; i < CPLx; ++i) w[cb][i] *= alpha;
                        l[cb] *= alpha;
                    }
                }
                frag pB[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    float e[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) e[i] = fexp2(__builtin_fmaf(sc[cb][i >> 2][i & 3], cl2, -m[cb]));
                    pB[cb].v = __builtin_shufflevector(to_bf16x4(e[0], e[1], e[2], e[3]), to_bf16x4(e[4], e[5], e[6], e[7]),
                                                       0, 1, 2, 3, 4, 5, 6, 7);
                }
                // row sums on the matrix unit: a ones operand against P^T adds each
                // row's weights exactly as the P V product takes them (bf16)
                {
                    frag ones;
                    ones.v = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) l[cb] = O::mma(ones, pB[cb], l[cb]);
                }

                // O^T += V^T P^T (tile jj holds d = 16*jj + m in row m), shared V
                // operand read transposed from LDS: slots 0..3 = keys 4*j4+i of the
                // first half, 4..7 = the second half, like P
                // (every V read issued before the first product: the scores are dead
                // by now, so their registers hold the operands and the LDS latency
                // is paid once per step)
                frag vA[VPL];
#pragma unroll
                for (int jj = 0; jj < VPL; ++jj) {
                    const bf16x4 v0 = lds_tr4(stk + vtr[jj]);
                    const bf16x4 v1 = lds_tr4(stk + 16 * kv_rowb + vtr[jj]);
                    vA[jj].v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
                for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) o[cb][jj] = O::mma(vA[jj], pB[cb], o[cb][jj]);
                // W^T += Lv^T P^T (tile jj holds c = 16*jj + m in row m), Lv read
                // transposed like V
                if constexpr (CPAD > 0) {
                    if (res) {
#pragma unroll
                        for (int jj = 0; jj < CPL; ++jj) {
                            const bf16x4 w0 = lds_tr4(stl + wtr[jj]);
                            const bf16x4 w1 = lds_tr4(stl + 16 * lr_rowb + wtr[jj]);
                            frag wA;
                            wA.v = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                            for (int cb = 0; cb < NCB; ++cb) w[cb][jj] = O::mma(wA, pB[cb], w[cb][jj]);
                        }
                    }
                }
            }
        }
        // the ring is drained (the last iteration waited for every load); every wave
        // must be done reading before the next phase refills the stages
        __syncthreads();
    }

    // ---- epilogue: O^T += Bv^T W^T, o = O / l, written with lse
    // Bv as the A operand of O^T += Bv^T W^T: for d-tile jj and contraction step
    // s, lane (n16, j4) supplies Bv[kappa][16*jj + n16] for the 8 residual
    // columns kappa = 16*(2s + i/4) + 4*j4 + i%4 (i < 8), the columns whose W
    // this lane holds (W^T tiles 2s and 2s + 1).
    constexpr int NBS = CPL / 2 > 0 ? CPL / 2 : 1;  // contraction steps of 8 columns per lane group
    // one contraction step's Bv operands at a time (all of them at once would
    // hold NBS * d / 16 fragments in registers)
    if constexpr (CPAD > 0) {
        if (resid) {
            const T *bv = static_cast<const T *>(p.bv) + (int64_t)a * p.r * p.HK * D + (int64_t)k * D + n16;
            const int64_t ldb = (int64_t)p.HK * D;
#pragma unroll
            for (int s = 0; s < NBS; ++s) {
                frag bvf[VPL];
#pragma unroll
                for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        int kap = 16 * (2 * s + (i >> 2)) + 4 * j4 + (i & 3);
                        kap = kap < p.r ? kap : 0;
                        O::set_raw(bvf[jj], i, bv[kap * ldb + 16 * jj]);
                    }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    // B operand: this lane's W (row n16, columns 16*(2s + i/4) + 4*j4 + i%4), hi + lo
                    frag wH, wL;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const int jt = 2 * s + (i >> 2);  // W^T tile
                        // padding columns (c >= r) hold P Lv of a stand-in column: drop them
                        const bool real = jt < CPLx && 16 * jt + 4 * j4 + (i & 3) < p.r;
                        const float x = real ? w[cb][jt < CPLx ? jt : 0][i & 3] : 0.0f;
                        const float hi = (float)(bf16)x;
                        O::set(wH, i, x);
                        O::set(wL, i, x - hi);
                    }
#pragma unroll
                    for (int jj = 0; jj < VPL; ++jj) {
                        o[cb][jj] = O::mma(bvf[jj], wH, o[cb][jj]);
                        o[cb][jj] = O::mma(bvf[jj], wL, o[cb][jj]);
                    }
                }
            }
        }
    }
    const float LN2 = 0.69314718055994530942f;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        const float lr = l[cb][0];  // the whole row's sum
        if (vm[cb]) {
            const float inv = 1.0f / lr;
            // tile jj, element i of this lane: d = 16*jj + 4*j4 + i
            float *po = p.out + qrow[cb] * D + 4 * j4;
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) *reinterpret_cast<f32x4 *>(po + 16 * jj) = o[cb][jj] * inv;
            if (j4 == 0 && p.lse) p.lse[qrow[cb]] = (m[cb] + __builtin_log2f(lr)) * LN2;
        }
    }
}

template <typename T, int D, int CP>
struct PrefillSlot {};

template <typename T, int D, int CP>
static hipError_t launch_prefill_one(const PrefillParams &pp, size_t lds, hipStream_t st) {
    auto *fn = prefill_kernel<T, D, CP>;
    const hipError_t e = ensure_lds<PrefillSlot<T, D, CP>>(reinterpret_cast<const void *>(fn), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(8 * pp.per_xcd), dim3(64 * kPrefillWaves), lds, st, pp);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams &pp, int D, int cpad, size_t lds, hipStream_t st) {
    if (D == 128) {
        switch (cpad) {
            case 0: return launch_prefill_one<bf16, 128, 0>(pp, lds, st);
            case 32: return launch_prefill_one<bf16, 128, 32>(pp, lds, st);
            case 64: return launch_prefill_one<bf16, 128, 64>(pp, lds, st);
            default: return launch_prefill_one<bf16, 128, 128>(pp, lds, st);
        }
    }
    switch (cpad) {
        case 0: return launch_prefill_one<bf16, 64, 0>(pp, lds, st);
        case 32: return launch_prefill_one<bf16, 64, 32>(pp, lds, st);
        case 64: return launch_prefill_one<bf16, 64, 64>(pp, lds, st);
        default: return launch_prefill_one<bf16, 64, 128>(pp, lds, st);
    }
}

}  // namespace rattn
