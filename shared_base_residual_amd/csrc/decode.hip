// decode.hip -- decode kernel of librattn (gfx950).
//
// Fused residual attention for N agents that share one base KV cache
// (ForkKV Guide, "Fused ResidualAttention"; LRAgent, "Flash-LoRA-Attention"):
//   score  s = scale * (q . K_base[j] + (q Bk_a^T) . Lk_a[j])
//   output o = sum_j p_j V_base[j] + (sum_j p_j Lv_a[j]) Bv_a
// One launch.  Each workgroup takes one (KV head, row group, context split):
//   * it computes U = scale*log2(e) * q Bk_a^T for its query rows with MFMA;
//   * it streams the base K/V tiles once for all agents' query rows (one MFMA
//     contraction over the rows of every agent), adds the rank-r score
//     correction with a second MFMA over the agents' Lk rows, runs an online
//     softmax in the log2 domain and accumulates P V_base and P Lv.  Private
//     tokens are extra work items with per-agent keys and no residual;
//   * it writes its partial state (max, sum, O, W) to the workspace and takes a
//     ticket on a per-(KV head, agent) counter; the workgroup that completes an
//     agent merges that agent's rows: a log-sum-exp merge over the splits with
//     wavefront shuffles, then o = (sum w O + (sum w W) Bv_a^(k)) / sum w l, so
//     Bv is applied once per row, not per token.  It resets the counter to zero.
//
// Layout of the streaming loop (S^T formulation): the MFMA A operand is the key
// tile (rows = 16 tokens), the B operand the query rows (columns = 16 query
// rows), so the scores arrive with one query row per lane column and the
// softmax statistics of a row live in the lanes that own it.  The value product
// is O^T = V^T P^T, so P feeds the B operand straight from the score registers.
// Every lane reads 16 contiguous bytes per key row and d/16 contiguous elements
// per value row; the value tile needs no transpose through LDS.
//
// Loads never branch: token indices beyond the split are clamped to its last
// token (finite data) and those scores are masked to -inf, so their weights are
// exactly zero.  Chunks are software-pipelined two deep.
#include "device.h"
#include "internal.h"

namespace rattn {

template <typename T, int D, int CPAD>
struct Chunk {
    static constexpr int KS = D / 32;
    static constexpr int VPL = D / 16;
    static constexpr int CS = CPAD > 0 ? CPAD / 32 : 1;
    static constexpr int CPL = CPAD > 0 ? CPAD / 16 : 1;
    typename Ops<T>::frag k[2][KS];
    Row<T, VPL> v[8];
    typename Ops<T>::frag lk[2][CS];
    Row<T, CPL> lv[8];
};

// Per-lane, loop-invariant state of one work item's token stream.
template <typename T, int D, int CPAD>
struct Stream {
    const T *kb, *vb;       // contiguous segment base, or paged pool
    const int32_t *table;   // NULL: contiguous
    int64_t page_stride;    // elements per physical page (all heads)
    int64_t head_off;       // elements to this head inside a page
    int ps;
    int tlast;              // last valid token of the item
    int tlast16;            // its 16-aligned tile start
    const T *lk[Chunk<T, D, CPAD>::CS];  // this lane's low-rank column pointers (token 0)
    const T *lv;
    int r;
    bool resid;

    // First row of the 16-token tile starting at t16 (clamped into the item).
    __device__ inline int tile_row0(int t16) const { return t16 < tlast16 ? t16 : tlast16; }
    __device__ inline const T *tile_ptr(const T *base, int t16c) const {
        if (table) {
            const int64_t pg = table[t16c / ps];
            return base + pg * page_stride + head_off + (int64_t)(t16c % ps) * D;
        }
        return base + (int64_t)t16c * D;
    }
};

template <typename T, int D, int CPAD>
__device__ inline void load_chunk(Chunk<T, D, CPAD> &ch, const Stream<T, D, CPAD> &st, int tc, int n16,
                                  int j4) {
    using O = Ops<T>;
    constexpr int KS = Chunk<T, D, CPAD>::KS, VPL = Chunk<T, D, CPAD>::VPL, CS = Chunk<T, D, CPAD>::CS,
                  CPL = Chunk<T, D, CPAD>::CPL;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int t16 = tc + 16 * c;
        const int t16c = st.tile_row0(t16);
        const T *kt = st.tile_ptr(st.kb, t16c);
        const T *vt = st.tile_ptr(st.vb, t16c);
        int tk = t16 + n16;
        tk = tk < st.tlast ? tk : st.tlast;
        const T *krow = kt + (tk - t16c) * D + 8 * j4;
#pragma unroll
        for (int s = 0; s < KS; ++s) ch.k[c][s] = O::load8(krow + 32 * s);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int tv = t16 + 4 * j4 + i;
            tv = tv < st.tlast ? tv : st.tlast;
            ch.v[4 * c + i] = load_row<T, VPL>(vt + (tv - t16c) * D + VPL * n16);
        }
        if (CPAD > 0 && st.resid) {
#pragma unroll
            for (int s = 0; s < CS; ++s) ch.lk[c][s] = O::load8(st.lk[s] + (int64_t)tk * st.r);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                int tv = t16 + 4 * j4 + i;
                tv = tv < st.tlast ? tv : st.tlast;
                ch.lv[4 * c + i] = load_row<T, CPL>(st.lv + (int64_t)tv * st.r);
            }
        }
    }
}

template <typename T, int D, int CPAD>
struct Acc {
    f32x4 o[D / 16];
    f32x4 w[CPAD > 0 ? CPAD / 16 : 1];
    float m, l;
};

// One 32-token chunk: scores, online softmax, value and low-rank value products.
template <typename T, int D, int CPAD>
__device__ inline void compute_chunk(Acc<T, D, CPAD> &acc, const Chunk<T, D, CPAD> &ch,
                                     const typename Ops<T>::frag *qB, const typename Ops<T>::frag *uH,
                                     const typename Ops<T>::frag *uL, float cl2, bool resid, int tc,
                                     int t1, bool causal, int tq, int j4) {
    using O = Ops<T>;
    using frag = typename O::frag;
    constexpr int KS = Chunk<T, D, CPAD>::KS, VPL = Chunk<T, D, CPAD>::VPL, CS = CPAD / 32,
                  CPL = CPAD / 16;
    f32x4 sc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) a = O::mma(ch.k[c][s], qB[s], a);
        a *= cl2;
        if (CPAD > 0 && resid) {
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                a = O::mma(ch.lk[c][s], uH[s], a);
                if constexpr (O::kSplitU) a = O::mma(ch.lk[c][s], uL[s], a);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = tc + 16 * c + 4 * j4 + i;
            if (t >= t1 || (causal && t > tq)) a[i] = -__builtin_inff();
        }
        sc[c] = a;
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(acc.m, mx);
    const float alpha = fexp2(acc.m - m_new);
    acc.m = m_new;
    frag pB;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float e = fexp2(sc[i >> 2][i & 3] - m_new);
        psum += e;
        O::set(pB, i, e);
    }
    acc.l = acc.l * alpha + psum;
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc.o[i] *= alpha;
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj) {
        frag vA;
#pragma unroll
        for (int i = 0; i < 8; ++i) O::set_raw(vA, i, ch.v[i].e[jj]);
        acc.o[jj] = O::mma(vA, pB, acc.o[jj]);
    }
    if (CPAD > 0 && resid) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) acc.w[i] *= alpha;
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) {
            frag wA;
#pragma unroll
            for (int i = 0; i < 8; ++i) O::set_raw(wA, i, ch.lv[i].e[jj]);
            acc.w[jj] = O::mma(wA, pB, acc.w[jj]);
        }
    }
}

// ------------------------------------------------------------------- merge --

// Expected completion tickets of (KV head, agent a): one per prefix item whose
// row group holds some of a's rows, one per private item of a.
__device__ inline unsigned expected_tickets(const DecodeParams &p, int a) {
    unsigned e = 0;
    if (p.n_ps > 0) {
        int nrg = 1;
        if (p.rpa > 16) nrg = (a * p.bpa + p.bpa - 1) / 4 - (a * p.bpa) / 4 + 1;
        e += (unsigned)(p.n_ps * nrg);
    }
    if (p.n_pv > 0) e += (unsigned)(p.n_pv * p.n_prg);
    return e;
}

// One wavefront merges the splits of one query row and writes out/lse.
// wbuf: n_slots floats of LDS for the weights, wr: r floats for the merged W.
template <typename T, int D>
__device__ inline void merge_row(const DecodeParams &p, int k, int a, int ria, float *wbuf, float *wr, int lane) {
    constexpr int DPL = D / 64;
    const int t = ria / p.g, hh = ria % p.g;
    const int64_t R = ((int64_t)a * p.QL + t) * p.HQ + (int64_t)k * p.g + hh;
    const int64_t rec0 = ((int64_t)k * p.N * p.rpa + (int64_t)a * p.rpa + ria) * p.n_slots;
    const int ns = p.n_slots, r = p.r;

    float mx = -3.0e38f;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, p.p_ml[(rec0 + s) * 2]);
    mx = wave_max(mx);
    float lsum = 0.0f;
    for (int s = lane; s < ns; s += 64) {
        const float2 ml = *reinterpret_cast<const float2 *>(p.p_ml + (rec0 + s) * 2);
        const float w = fexp2(ml.x - mx);
        wbuf[s] = w;
        lsum += w * ml.y;
    }
    lsum = wave_sum(lsum);
    __builtin_amdgcn_wave_barrier();

    float o[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
    const float *po = p.p_o + rec0 * D + DPL * lane;
    for (int s0 = 0; s0 < ns; s0 += 16) {
        float v[16][DPL], wv[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int s = s0 + u;
            const int sc = s < ns ? s : ns - 1;
            wv[u] = s < ns ? wbuf[sc] : 0.0f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) v[u][e] = po[(int64_t)sc * D + e];
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[e] += wv[u] * v[u][e];
    }
    if (r > 0 && p.n_ps > 0) {
        for (int j = lane; j < r; j += 64) {
            float wj = 0.0f;
            const float *pw = p.p_w + rec0 * r + j;
            for (int s0 = 0; s0 < p.n_ps; s0 += 16) {
                float v[16], wv[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const int s = s0 + u;
                    const int sc = s < p.n_ps ? s : p.n_ps - 1;
                    wv[u] = s < p.n_ps ? wbuf[sc] : 0.0f;
                    v[u] = pw[(int64_t)sc * r];
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) wj += wv[u] * v[u];
            }
            wr[j] = wj;
        }
        __builtin_amdgcn_wave_barrier();
        const T *bv = static_cast<const T *>(p.bv) + (int64_t)a * r * p.HK * D + (int64_t)k * D + DPL * lane;
        for (int j0 = 0; j0 < r; j0 += 8) {
            float bvv[8][DPL];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < DPL; ++e) bvv[u][e] = (float)bv[(int64_t)(j0 + u) * p.HK * D + e];
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < DPL; ++e) o[e] += wr[j0 + u] * bvv[u][e];
        }
    }
    const float inv = 1.0f / lsum;
#pragma unroll
    for (int e = 0; e < DPL; ++e) p.out[R * D + DPL * lane + e] = o[e] * inv;
    if (lane == 0 && p.lse) p.lse[R] = (mx + __builtin_log2f(lsum)) * 0.69314718055994530942f;
    __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------ split kernel --

template <typename T, int D, int CPAD>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    using O = Ops<T>;
    using frag = typename O::frag;
    constexpr int KS = D / 32;
    constexpr int VPL = D / 16;
    constexpr int CS = CPAD / 32;
    constexpr int CSx = CS > 0 ? CS : 1;
    constexpr int CPLx = CPAD > 0 ? CPAD / 16 : 1;

    extern __shared__ float smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int n16 = lane & 15;
    const int j4 = lane >> 4;

    // Workgroup i is dispatched to XCD i % 8.  Items are numbered KV-head fastest
    // and laid out so that the KV heads of one (split, row group) run back to back
    // on one XCD, where they share the low-rank rows through that XCD's L2.
    const int bid = blockIdx.x;
    const int li = (bid & 7) * p.per_xcd + (bid >> 3);
    if (li >= p.n_items) return;

    int k, slot, nblk, blk0, agent_p = 0;
    int t0, t1;
    bool prefix;
    if (li < p.n_prefix_items) {
        k = li % p.HK;
        const int rest = li / p.HK;
        const int rg = rest % p.n_rg;
        const int s = rest / p.n_rg;
        blk0 = rg * 4;
        nblk = p.n_blocks - blk0 < 4 ? p.n_blocks - blk0 : 4;
        t0 = s * p.tok_ps;
        t1 = t0 + p.tok_ps < p.L ? t0 + p.tok_ps : (int)p.L;
        slot = s;
        prefix = true;
    } else {
        const int l2 = li - p.n_prefix_items;
        k = l2 % p.HK;
        int rest = l2 / p.HK;
        const int s = rest % p.n_pv;
        rest /= p.n_pv;
        const int prg = rest % p.n_prg;
        agent_p = rest / p.n_prg;
        blk0 = prg * 4;
        nblk = p.pb - blk0 < 4 ? p.pb - blk0 : 4;
        t0 = s * p.tok_pv;
        t1 = t0 + p.tok_pv < p.S ? t0 + p.tok_pv : (int)p.S;
        slot = p.n_ps + s;
        prefix = false;
    }
    const bool resid = prefix && (CPAD > 0) && p.r > 0;
    const bool causal = !prefix && p.causal;
    const int TG = 4 / nblk;  // waves sharing one row block (token groups)
    const int rbi = wave / TG;
    const int tg = wave % TG;
    const bool active = rbi < nblk && t0 < t1;

    // Row block of this wave.
    RowBlock blk;
    if (prefix) {
        blk = prefix_block(blk0 + rbi, p.N, p.rpa, p.apb, p.bpa);
    } else {
        blk.a0 = agent_p;
        blk.na = 1;
        blk.f = p.rpa <= 16 ? 0 : 16 * (blk0 + rbi);
        blk.nr = p.rpa - blk.f < 16 ? p.rpa - blk.f : 16;
    }
    // Query row owned by this lane's column.
    const bool vm = rbi < nblk && n16 < blk.nr;
    int agent_m = 0, ria = 0;
    if (vm) block_row(blk, n16, p.rpa, &agent_m, &ria);
    const int tq = ria / p.g, hh = ria % p.g;
    const int64_t qrow = ((int64_t)agent_m * p.QL + tq) * p.HQ + (int64_t)k * p.g + hh;
    const int64_t grow = (int64_t)agent_m * p.rpa + ria;
    const float cl2 = p.c;

    const T *qp = static_cast<const T *>(p.q);
    const int cvalid = resid ? (p.shared_lr ? p.r : blk.na * p.r) : 0;

    // Query rows as the B operand of S^T = K Q^T.
    frag qB[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qB[s] = vm ? O::load8(qp + qrow * D + 32 * s + 8 * j4) : O::zero();

    // Token stream of this item.
    Stream<T, D, CPAD> st;
    st.r = p.r;
    st.resid = resid;
    st.tlast = t1 - 1;
    st.tlast16 = st.tlast & ~15;
    if (prefix) {
        st.kb = static_cast<const T *>(p.kb);
        st.vb = static_cast<const T *>(p.vb);
        if (p.ps > 0) {
            st.table = p.table;
            st.ps = p.ps;
            st.page_stride = (int64_t)p.HK * p.ps * D;
            st.head_off = (int64_t)k * p.ps * D;
        } else {
            st.table = nullptr;
            st.ps = 16;
            st.page_stride = 0;
            st.head_off = 0;
            st.kb += (int64_t)k * p.L * D;
            st.vb += (int64_t)k * p.L * D;
        }
    } else {
        const int64_t seg = ((int64_t)agent_p * p.HK + k) * p.S * D;
        st.kb = static_cast<const T *>(p.kp) + seg;
        st.vb = static_cast<const T *>(p.vp) + seg;
        st.table = nullptr;
        st.ps = 16;
        st.page_stride = 0;
        st.head_off = 0;
    }
    {
        const T *lk = static_cast<const T *>(p.lk);
        const T *lv = static_cast<const T *>(p.lv);
#pragma unroll
        for (int s = 0; s < CSx; ++s) {
            const int cc = 32 * s + 8 * j4;
            int lr = 0, col = 0;
            if (resid && cc < cvalid) {
                lr = p.shared_lr ? 0 : blk.a0 + (cc >> p.lr_shift);
                col = cc & (p.r - 1);
            } else if (resid) {
                lr = p.shared_lr ? 0 : blk.a0;  // padding column: any finite data (U is zero there)
            }
            st.lk[s] = lk + (int64_t)lr * p.L * p.r + col;
        }
        const int cl = CPLx * n16;
        int lr = 0, col = 0;
        if (resid && cl < cvalid) {
            lr = p.shared_lr ? 0 : blk.a0 + (cl >> p.lr_shift);
            col = cl & (p.r - 1);
        } else if (resid) {
            lr = p.shared_lr ? 0 : blk.a0;
        }
        st.lv = lv + (int64_t)lr * p.L * p.r + col;
    }

    // First chunk's loads go out before U is computed.
    Chunk<T, D, CPAD> ca, cb;
    const int step = 32 * TG;
    int tc = t0 + 32 * tg;
    if (active) load_chunk(ca, st, tc, n16, j4);

    // U = scale*log2(e) * q Bk^T as the B operand of the rank-r score correction,
    // block-diagonal over the agents of the block (bf16 carries hi + lo halves).
    // Computed as U^T = Bk Q^T with MFMA; A-operand row rho of output tile 2s+h
    // is residual column 32s + 8(rho/4) + 4h + rho%4, so that each lane's
    // results land in its own B-operand slots.
    frag uH[CSx], uL[CSx];
#pragma unroll
    for (int s = 0; s < CSx; ++s) {
        uH[s] = O::zero();
        uL[s] = O::zero();
    }
    if (CPAD > 0 && resid && active) {
        const T *bk = static_cast<const T *>(p.bk);
        const int64_t ldb = (int64_t)p.HK * D;
        const int rmask = p.r - 1;
        const int na_loop = p.shared_lr ? blk.na : 1;
#pragma unroll
        for (int s = 0; s < CSx; ++s) {
            float uv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) uv[i] = 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int crow = 32 * s + 8 * (n16 >> 2) + 4 * h + (n16 & 3);  // A-operand row
                for (int ai = 0; ai < na_loop; ++ai) {
                    int arow, colr;
                    if (p.shared_lr) {
                        arow = blk.a0 + ai;
                        colr = crow < p.r ? crow : 0;
                    } else {
                        const bool okc = crow < cvalid;
                        arow = blk.a0 + (okc ? (crow >> p.lr_shift) : 0);
                        colr = okc ? (crow & rmask) : 0;
                    }
                    const T *brow = bk + ((int64_t)arow * p.r + colr) * ldb + (int64_t)k * D + 8 * j4;
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) a = O::mma(O::load8(brow + 32 * s2), qB[s2], a);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 32 * s + 8 * j4 + 4 * h + i;  // column this lane received
                        bool keep = vm && c < cvalid;
                        if (p.shared_lr)
                            keep = keep && agent_m == blk.a0 + ai;
                        else
                            keep = keep && blk.a0 + (c >> p.lr_shift) == agent_m;
                        if (keep) uv[4 * h + i] += a[i] * cl2;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                O::set(uH[s], i, uv[i]);
                if constexpr (O::kSplitU) {
                    const float hi = (float)(bf16)uv[i];
                    O::set(uL[s], i, uv[i] - hi);
                }
            }
        }
    }

    Acc<T, D, CPAD> acc;
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CPLx; ++i) acc.w[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m = -1.0e30f;
    acc.l = 0.0f;

    if (active) {
        for (; tc < t1; tc += 2 * step) {
            load_chunk(cb, st, tc + step, n16, j4);
            compute_chunk(acc, ca, qB, uH, uL, cl2, resid, tc, t1, causal, tq, j4);
            if (tc + step >= t1) break;
            load_chunk(ca, st, tc + 2 * step, n16, j4);
            compute_chunk(acc, cb, qB, uH, uL, cl2, resid, tc + step, t1, causal, tq, j4);
        }
    }
    float m_run = acc.m, l_run = acc.l;
    // Sum of weights over the four lanes that share this query row.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // ---- merge the token groups of a row block (same lane layout in every wave)
    constexpr int PER_LANE = 4 * VPL + 4 * CPLx;
    // Waves 1..3 publish their state (wave 0 always has tg == 0): three slots.
    if (TG > 1) {
        float *sm = smem + (size_t)(wave - 1) * (64 * PER_LANE + 32);
        if (tg > 0) {
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm[(4 * jj + i) * 64 + lane] = acc.o[jj][i];
#pragma unroll
            for (int jj = 0; jj < CPLx; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) sm[(4 * VPL + 4 * jj + i) * 64 + lane] = acc.w[jj][i];
            if (j4 == 0) {
                sm[64 * PER_LANE + n16] = m_run;
                sm[64 * PER_LANE + 16 + n16] = l_run;
            }
        }
        __syncthreads();
        if (tg == 0) {
            float mt = m_run;
            for (int w = 1; w < TG; ++w)
                mt = fmaxf(mt, smem[(size_t)(wave + w - 1) * (64 * PER_LANE + 32) + 64 * PER_LANE + n16]);
            const float s0 = fexp2(m_run - mt);
            l_run *= s0;
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) acc.o[jj] *= s0;
#pragma unroll
            for (int jj = 0; jj < CPLx; ++jj) acc.w[jj] *= s0;
            for (int w = 1; w < TG; ++w) {
                const float *sw = smem + (size_t)(wave + w - 1) * (64 * PER_LANE + 32);
                const float sf = fexp2(sw[64 * PER_LANE + n16] - mt);
                l_run += sf * sw[64 * PER_LANE + 16 + n16];
#pragma unroll
                for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc.o[jj][i] += sf * sw[(4 * jj + i) * 64 + lane];
#pragma unroll
                for (int jj = 0; jj < CPLx; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc.w[jj][i] += sf * sw[(4 * VPL + 4 * jj + i) * 64 + lane];
            }
            m_run = mt;
        }
    }

    // ---- write this split's partial state of every valid row
    if (tg == 0 && vm) {
        const int64_t rec = ((int64_t)k * p.N * p.rpa + grow) * p.n_slots + slot;
        float ov[4 * VPL];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) ov[VPL * i + jj] = acc.o[jj][i];
        float *po = p.p_o + rec * D + 4 * VPL * j4;
#pragma unroll
        for (int c = 0; c < VPL; ++c)
            *reinterpret_cast<f32x4 *>(po + 4 * c) = f32x4{ov[4 * c], ov[4 * c + 1], ov[4 * c + 2], ov[4 * c + 3]};
        if (resid) {
            const int arel = agent_m - blk.a0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < CPLx; ++jj) {
                    const int c = CPLx * (4 * j4 + i) + jj;
                    if (c < cvalid && (p.shared_lr || (c >> p.lr_shift) == arel))
                        p.p_w[rec * p.r + (c & (p.r - 1))] = acc.w[jj][i];
                }
        }
        if (j4 == 0) {
            p.p_ml[rec * 2] = m_run;
            p.p_ml[rec * 2 + 1] = l_run;
        }
    }

    // ---- completion tickets; the workgroup that completes an agent merges it
    __shared__ int s_last[64];
    __shared__ int s_nlast;
    __threadfence();  // release this thread's partial stores (device scope)
    __syncthreads();
    if (threadIdx.x == 0) {
        int a_lo, a_hi;
        if (prefix) {
            const RowBlock b0 = prefix_block(blk0, p.N, p.rpa, p.apb, p.bpa);
            const RowBlock b1 = prefix_block(blk0 + nblk - 1, p.N, p.rpa, p.apb, p.bpa);
            a_lo = b0.a0;
            a_hi = b1.a0 + b1.na - 1;
        } else {
            a_lo = a_hi = agent_p;
        }
        int nl = 0;
        for (int a = a_lo; a <= a_hi; ++a) {
            const unsigned old = atomicAdd(p.cnt + (int64_t)k * p.N + a, 1u);
            if (old + 1 == expected_tickets(p, a)) s_last[nl++] = a;
        }
        s_nlast = nl;
    }
    __syncthreads();
    const int nl = s_nlast;
    if (nl > 0) {
        __threadfence();  // acquire: every item's partials of these agents are visible
        float *wbuf = smem + (size_t)wave * (kMaxSlots + 128);
        float *wr = wbuf + kMaxSlots;
        for (int i = 0; i < nl; ++i) {
            const int a = s_last[i];
            for (int ria = wave; ria < p.rpa; ria += 4) merge_row<T, D>(p, k, a, ria, wbuf, wr, lane);
        }
        // Ready for the next call.  An atomic at device scope, like the tickets: a
        // plain store could stay in this XCD's L2 while the next call's tickets
        // are counted at the device-wide coherence point.
        if (threadIdx.x == 0)
            for (int i = 0; i < nl; ++i) atomicExch(p.cnt + (int64_t)k * p.N + s_last[i], 0u);
    }
}

// ---------------------------------------------------------------- launchers --

template <typename T>
static hipError_t launch_decode_t(const DecodeParams &dp, int D, int cpad, size_t lds, hipStream_t st) {
    const dim3 grid(8 * dp.per_xcd);
#define RATTN_SPLIT(DD, CP) \
    hipLaunchKernelGGL((decode_split_kernel<T, DD, CP>), grid, dim3(256), lds, st, dp)
    if (D == 128) {
        switch (cpad) {
            case 0: RATTN_SPLIT(128, 0); break;
            case 32: RATTN_SPLIT(128, 32); break;
            case 64: RATTN_SPLIT(128, 64); break;
            default: RATTN_SPLIT(128, 128); break;
        }
    } else {
        switch (cpad) {
            case 0: RATTN_SPLIT(64, 0); break;
            case 32: RATTN_SPLIT(64, 32); break;
            case 64: RATTN_SPLIT(64, 64); break;
            default: RATTN_SPLIT(64, 128); break;
        }
    }
#undef RATTN_SPLIT
    return hipGetLastError();
}

hipError_t launch_decode(int bf16_in, const DecodeParams &dp, int D, int cpad, size_t lds, hipStream_t st) {
    if (bf16_in) return launch_decode_t<bf16>(dp, D, cpad, lds, st);
    return launch_decode_t<float>(dp, D, cpad, lds, st);
}

}  // namespace rattn
