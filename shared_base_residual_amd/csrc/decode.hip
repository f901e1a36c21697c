// decode.hip -- decode kernels of librattn (gfx950).
//
// Fused residual attention for N agents that share one base KV cache
// (ForkKV Guide, "Fused ResidualAttention"; LRAgent, "Flash-LoRA-Attention"):
//   score  s = scale * (q . K_base[j] + (q Bk_a^T) . Lk_a[j])
//   output o = sum_j p_j V_base[j] + (sum_j p_j Lv_a[j]) Bv_a
// Three launches on the caller's stream:
//   1. u_prologue   U = scale*log2(e) * q Bk_a^(k)^T, fp32, one row per query row;
//   2. decode_split per (KV head, row group, context split): streams the base
//      K/V tiles once for all agents' query rows (one MFMA contraction over the
//      rows of every agent), adds the rank-r score correction with a second MFMA
//      over the agents' Lk rows, runs an online softmax in the log2 domain, and
//      accumulates P V_base and P Lv; private tokens are extra work items with
//      per-agent keys and no residual.  Partials (max, sum, O, W) go to the
//      workspace;
//   3. combine per query row: log-sum-exp merge of the splits (wave shuffles),
//      then o = (sum w O + (sum w W) Bv_a^(k)) / sum w l: Bv is applied once per
//      row, not per token.
//
// Layout inside decode_split (S^T formulation): the MFMA A operand is the key
// tile (rows = 16 tokens), the B operand the query rows (columns = 16 query
// rows), so the scores arrive with one query row per lane column and the
// softmax statistics of a row live in the lanes that own it.  The value product
// is O^T = V^T P^T, so P feeds the B operand straight from the score registers.
// Every lane reads 16 contiguous bytes per key row and 16*(d/16)/8 contiguous
// bytes per value row; the value tile needs no transpose through LDS.
#include "device.h"
#include "internal.h"

namespace rattn {

// ---------------------------------------------------------------- prologue --

template <typename T>
__global__ __launch_bounds__(256) void u_prologue_kernel(UParams p, int D) {
    const int blk = blockIdx.x;  // (a, t, k)
    const int k = blk % p.HK;
    const int at = blk / p.HK;   // a * QL + t
    const int a = at / p.QL;
    const T *q = static_cast<const T *>(p.q);
    const T *bk = static_cast<const T *>(p.bk);
    const int64_t ldb = (int64_t)p.HK * D;
    for (int idx = threadIdx.x; idx < p.g * p.r; idx += blockDim.x) {
        const int hh = idx / p.r, j = idx % p.r;
        const int h = k * p.g + hh;
        const T *qr = q + ((int64_t)at * p.HQ + h) * D;
        const T *br = bk + ((int64_t)a * p.r + j) * ldb + (int64_t)k * D;
        float acc = 0.0f;
        for (int dd = 0; dd < D; ++dd) acc += (float)qr[dd] * (float)br[dd];
        p.u[((int64_t)at * p.HQ + h) * p.r + j] = acc * p.c;
    }
}

// ------------------------------------------------------------ split kernel --

template <typename T, int D, int CPAD>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
    using O = Ops<T>;
    using frag = typename O::frag;
    constexpr int KS = D / 32;     // contraction steps over the head dimension
    constexpr int VPL = D / 16;    // value columns per lane per token = O^T tiles
    constexpr int CS = CPAD / 32;  // contraction steps over residual columns
    constexpr int CPL = CPAD / 16; // residual columns per lane per token = W^T tiles
    constexpr int CPLx = CPL > 0 ? CPL : 1;
    constexpr int CSx = CS > 0 ? CS : 1;

    extern __shared__ float smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n16 = lane & 15;
    const int j4 = lane >> 4;

    // Workgroup i is dispatched to XCD i % 8.  Items are numbered KV-head fastest
    // and laid out so that the KV heads of one (split, row group) run back to back
    // on one XCD, where they share the low-rank rows through that XCD's L2.
    const int bid = blockIdx.x;
    const int li = (bid & 7) * p.per_xcd + (bid >> 3);
    if (li >= p.n_items) return;

    int k, slot, nblk, blk0, agent_p = 0;
    int64_t t0, t1;
    bool prefix;
    if (li < p.n_prefix_items) {
        k = li % p.HK;
        const int rest = li / p.HK;
        const int rg = rest % p.n_rg;
        const int s = rest / p.n_rg;
        blk0 = rg * 4;
        nblk = p.n_blocks - blk0 < 4 ? p.n_blocks - blk0 : 4;
        t0 = (int64_t)s * p.tok_ps;
        t1 = t0 + p.tok_ps < p.L ? t0 + p.tok_ps : p.L;
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
        t0 = (int64_t)s * p.tok_pv;
        t1 = t0 + p.tok_pv < p.S ? t0 + p.tok_pv : p.S;
        slot = p.n_ps + s;
        prefix = false;
    }
    const bool resid = prefix && (CPAD > 0) && p.r > 0;
    const bool causal = !prefix && p.causal;
    const bool paged = prefix && p.ps > 0;
    const int TG = 4 / nblk;  // waves sharing one row block (token groups)
    const int rbi = wave / TG;
    const int tg = wave % TG;
    const bool active = rbi < nblk;

    // Row block of this wave.
    RowBlock blk;
    if (prefix) {
        blk = prefix_block(blk0 + rbi, p.N, p.rpa, p.apb, p.bpa);
    } else {
        blk.a0 = agent_p;
        blk.na = 1;
        blk.f = 16 * (blk0 + rbi);
        blk.nr = p.rpa - blk.f < 16 ? p.rpa - blk.f : 16;
        if (p.rpa <= 16) blk.f = 0;
    }
    // Query row owned by this lane's column.
    const bool vm = active && n16 < blk.nr;
    int agent_m = 0, ria = 0;
    if (vm) block_row(blk, n16, p.rpa, &agent_m, &ria);
    const int tq = ria / p.g, hh = ria % p.g;
    const int64_t qrow = ((int64_t)agent_m * p.QL + tq) * p.HQ + (int64_t)k * p.g + hh;
    const int64_t grow = (int64_t)agent_m * p.rpa + ria;

    const T *qp = static_cast<const T *>(p.q);
    const T *kb = static_cast<const T *>(prefix ? p.kb : p.kp);
    const T *vb = static_cast<const T *>(prefix ? p.vb : p.vp);
    const T *lk = static_cast<const T *>(p.lk);
    const T *lv = static_cast<const T *>(p.lv);
    // Offset of the (contiguous) segment this item streams.
    const int64_t seg = prefix ? (int64_t)k * p.L * D : ((int64_t)agent_p * p.HK + k) * p.S * D;
    const int cvalid = resid ? (p.shared_lr ? p.r : blk.na * p.r) : 0;

    // Query rows as the B operand of S^T = K Q^T.
    frag qB[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qB[s] = vm ? O::load8(qp + qrow * D + 32 * s + 8 * j4) : O::zero();

    // U (block-diagonal over the agents of the block) as the B operand of the
    // rank-r score correction; bf16 carries it as hi + lo halves.
    frag uH[CSx], uL[CSx];
#pragma unroll
    for (int s = 0; s < CSx; ++s) {
        uH[s] = O::zero();
        uL[s] = O::zero();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int c = 32 * s + 8 * j4 + i;
            float v = 0.0f;
            if (resid && vm && c < cvalid) {
                if (p.shared_lr)
                    v = p.u[qrow * p.r + c];
                else if (blk.a0 + c / p.r == agent_m)
                    v = p.u[qrow * p.r + (c % p.r)];
            }
            O::set(uH[s], i, v);
            if constexpr (O::kSplitU) {
                const float hi = (float)(bf16)v;
                O::set(uL[s], i, v - hi);
            }
        }
    }

    f32x4 accO[VPL];
    f32x4 accW[CPLx];
#pragma unroll
    for (int i = 0; i < VPL; ++i) accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CPLx; ++i) accW[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -1.0e30f, l_run = 0.0f;

    // Pointer to token t16 (16-aligned) of the streamed segment; tokens
    // t16..t16+15 are contiguous rows of d elements.
    auto tile = [&](const T *base, int64_t t16) -> const T * {
        if (paged) {
            const int64_t pg = p.table[t16 / p.ps];
            return base + ((pg * p.HK + k) * p.ps + (t16 % p.ps)) * D;
        }
        return base + seg + t16 * D;
    };

    if (active) {
        for (int64_t tc = t0 + 32 * tg; tc < t1; tc += 32 * TG) {
            // ---- loads of this 32-token chunk
            frag kA[2][KS];
            frag lkA[2][CSx];
            Row<T, VPL> vR[8];
            Row<T, CPLx> lvR[8];
            const T *kt[2], *vt[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int64_t t16 = tc + 16 * c;
                kt[c] = t16 < t1 ? tile(kb, t16) : kb;
                vt[c] = t16 < t1 ? tile(vb, t16) : vb;
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int64_t t = tc + 16 * c + n16;
                const bool ok = t < t1;
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    kA[c][s] = ok ? O::load8(kt[c] + n16 * D + 32 * s + 8 * j4) : O::zero();
#pragma unroll
                for (int s = 0; s < CSx; ++s) {
                    const int cc = 32 * s + 8 * j4;
                    lkA[c][s] = O::zero();
                    if (resid && ok && cc < cvalid) {
                        const int64_t lr = p.shared_lr ? 0 : blk.a0 + cc / p.r;
                        lkA[c][s] = O::load8(lk + (lr * p.L + t) * p.r + (cc % p.r));
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int tl = 16 * (i >> 2) + 4 * j4 + (i & 3);
                const int64_t t = tc + tl;
                const bool ok = t < t1;
                vR[i] = ok ? load_row<T, VPL>(vt[i >> 2] + (4 * j4 + (i & 3)) * D + VPL * n16)
                           : zero_row<T, VPL>();
                lvR[i] = zero_row<T, CPLx>();
                const int cl = CPLx * n16;
                if (resid && ok && cl < cvalid) {
                    const int64_t lr = p.shared_lr ? 0 : blk.a0 + cl / p.r;
                    lvR[i] = load_row<T, CPLx>(lv + (lr * p.L + t) * p.r + (cl % p.r));
                }
            }

            // ---- scores S^T (rows = tokens, columns = query rows), log2 domain
            f32x4 sc[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s) acc = O::mma(kA[c][s], qB[s], acc);
                acc *= p.c;
                if (resid) {
#pragma unroll
                    for (int s = 0; s < CS; ++s) {
                        acc = O::mma(lkA[c][s], uH[s], acc);
                        if constexpr (O::kSplitU) acc = O::mma(lkA[c][s], uL[s], acc);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t t = tc + 16 * c + 4 * j4 + i;
                    if (t >= t1 || (causal && t > tq)) acc[i] = -__builtin_inff();
                }
                sc[c] = acc;
            }

            // ---- online softmax for this lane's query row
            float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                             fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = fexp2(m_run - m_new);
            m_run = m_new;
            frag pB;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e = fexp2(sc[i >> 2][i & 3] - m_new);
                psum += e;
                O::set(pB, i, e);
            }
            l_run = l_run * alpha + psum;
#pragma unroll
            for (int i = 0; i < VPL; ++i) accO[i] *= alpha;
            if (resid) {
#pragma unroll
                for (int i = 0; i < CPLx; ++i) accW[i] *= alpha;
            }

            // ---- O^T += V^T P^T and W^T += Lv^T P^T
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) {
                frag vA;
#pragma unroll
                for (int i = 0; i < 8; ++i) O::set_raw(vA, i, vR[i].e[jj]);
                accO[jj] = O::mma(vA, pB, accO[jj]);
            }
            if (resid) {
#pragma unroll
                for (int jj = 0; jj < CPL; ++jj) {
                    frag wA;
#pragma unroll
                    for (int i = 0; i < 8; ++i) O::set_raw(wA, i, lvR[i].e[jj]);
                    accW[jj] = O::mma(wA, pB, accW[jj]);
                }
            }
        }
    }
    // Sum of weights over the four lanes that share this query row.
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);

    // ---- merge the token groups of a row block (same lane layout in every wave)
    constexpr int PER_LANE = 4 * VPL + 4 * CPLx;
    // Waves 1..3 publish their state (wave 0 always has tg == 0): three slots.
    if (TG > 1) {
        float *st = smem + (size_t)(wave - 1) * (64 * PER_LANE + 32);
        if (tg > 0) {
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[(4 * jj + i) * 64 + lane] = accO[jj][i];
#pragma unroll
            for (int jj = 0; jj < CPLx; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) st[(4 * VPL + 4 * jj + i) * 64 + lane] = accW[jj][i];
            if (j4 == 0) {
                st[64 * PER_LANE + n16] = m_run;
                st[64 * PER_LANE + 16 + n16] = l_run;
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
            for (int jj = 0; jj < VPL; ++jj) accO[jj] *= s0;
#pragma unroll
            for (int jj = 0; jj < CPLx; ++jj) accW[jj] *= s0;
            for (int w = 1; w < TG; ++w) {
                const float *sw = smem + (size_t)(wave + w - 1) * (64 * PER_LANE + 32);
                const float sf = fexp2(sw[64 * PER_LANE + n16] - mt);
                l_run += sf * sw[64 * PER_LANE + 16 + n16];
#pragma unroll
                for (int jj = 0; jj < VPL; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accO[jj][i] += sf * sw[(4 * jj + i) * 64 + lane];
#pragma unroll
                for (int jj = 0; jj < CPLx; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) accW[jj][i] += sf * sw[(4 * VPL + 4 * jj + i) * 64 + lane];
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
            for (int jj = 0; jj < VPL; ++jj) ov[VPL * i + jj] = accO[jj][i];
        float *po = p.p_o + rec * D + 4 * VPL * j4;
#pragma unroll
        for (int c = 0; c < VPL; ++c)
            *reinterpret_cast<f32x4 *>(po + 4 * c) = f32x4{ov[4 * c], ov[4 * c + 1], ov[4 * c + 2], ov[4 * c + 3]};
        if (resid) {
            const int arel = agent_m - blk.a0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < CPL; ++jj) {
                    const int c = CPLx * (4 * j4 + i) + jj;
                    if (c < cvalid && (p.shared_lr || c / p.r == arel)) p.p_w[rec * p.r + (c % p.r)] = accW[jj][i];
                }
        }
        if (j4 == 0) {
            p.p_ml[rec * 2] = m_run;
            p.p_ml[rec * 2 + 1] = l_run;
        }
    }
}

// ----------------------------------------------------------------- combine --

template <typename T, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
    __shared__ float s_w[1024];
    __shared__ float s_o[256];
    __shared__ float s_wr[256];
    __shared__ float s_ml[2];
    const int R = blockIdx.x;  // (a * QL + t) * HQ + h
    const int h = R % p.HQ;
    const int at = R / p.HQ;
    const int a = at / p.QL, t = at % p.QL;
    const int k = h / p.g, hh = h % p.g;
    const int64_t grow = (int64_t)a * p.rpa + (int64_t)t * p.g + hh;
    const int64_t rec0 = ((int64_t)k * p.N * p.rpa + grow) * p.n_slots;
    const int tid = threadIdx.x, lane = tid & 63;
    const int ns = p.n_slots;

    // Wave 0: maximum over the splits and the merged weight sum (wave shuffles).
    if (tid < 64) {
        float mx = -3.0e38f;
        for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, p.p_ml[(rec0 + s) * 2]);
        mx = wave_max(mx);
        float l = 0.0f;
        for (int s = lane; s < ns; s += 64) {
            const float w = fexp2(p.p_ml[(rec0 + s) * 2] - mx);
            if (s < 1024) s_w[s] = w;
            l += w * p.p_ml[(rec0 + s) * 2 + 1];
        }
        l = wave_sum(l);
        if (lane == 0) {
            s_ml[0] = mx;
            s_ml[1] = l;
        }
    }
    __syncthreads();
    const float mx = s_ml[0], lsum = s_ml[1];
    constexpr int NG = 256 / D;  // slot groups
    const int sg = tid / D, dd = tid % D;
    float acc = 0.0f;
    for (int s = sg; s < ns; s += NG) {
        const float w = s < 1024 ? s_w[s] : fexp2(p.p_ml[(rec0 + s) * 2] - mx);
        acc += w * p.p_o[(rec0 + s) * D + dd];
    }
    s_o[tid] = acc;
    // Residual value columns, prefix splits only.
    if (p.r > 0) {
        const int gr = 256 / p.r;  // r divides 256
        const int sgw = tid / p.r, jw = tid % p.r;
        float aw = 0.0f;
        if (sgw < gr)
            for (int s = sgw; s < p.n_ps; s += gr) {
                const float w = s < 1024 ? s_w[s] : fexp2(p.p_ml[(rec0 + s) * 2] - mx);
                aw += w * p.p_w[(rec0 + s) * p.r + jw];
            }
        s_wr[tid] = aw;
    }
    __syncthreads();
    if (tid < D) {
        float o = 0.0f;
        for (int g2 = 0; g2 < NG; ++g2) o += s_o[g2 * D + tid];
        if (p.r > 0) {
            const int gr = 256 / p.r;
            const T *bv = static_cast<const T *>(p.bv) + (int64_t)a * p.r * p.HK * D + (int64_t)k * D + tid;
            for (int j = 0; j < p.r; ++j) {
                float wj = 0.0f;
                for (int g2 = 0; g2 < gr; ++g2) wj += s_wr[g2 * p.r + j];
                o += wj * (float)bv[(int64_t)j * p.HK * D];
            }
        }
        p.out[(int64_t)R * D + tid] = o / lsum;
    }
    if (tid == 0 && p.lse) p.lse[R] = (mx + __builtin_log2f(lsum)) * 0.69314718055994530942f;
}

// ---------------------------------------------------------------- launchers --

template <typename T>
static hipError_t launch_decode_t(const DecodeParams &dp, const CombineParams &cp, const UParams &up, int D,
                                  int cpad, size_t lds, hipStream_t st) {
    if (dp.r > 0 && dp.L > 0) {
        hipLaunchKernelGGL(u_prologue_kernel<T>, dim3(dp.N * dp.QL * dp.HK), dim3(256), 0, st, up, D);
    }
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
        hipLaunchKernelGGL((combine_kernel<T, 128>), dim3(dp.N * dp.QL * dp.HQ), dim3(256), 0, st, cp);
    } else {
        switch (cpad) {
            case 0: RATTN_SPLIT(64, 0); break;
            case 32: RATTN_SPLIT(64, 32); break;
            case 64: RATTN_SPLIT(64, 64); break;
            default: RATTN_SPLIT(64, 128); break;
        }
        hipLaunchKernelGGL((combine_kernel<T, 64>), dim3(dp.N * dp.QL * dp.HQ), dim3(256), 0, st, cp);
    }
#undef RATTN_SPLIT
    return hipGetLastError();
}

hipError_t launch_decode(int bf16_in, const DecodeParams &dp, const CombineParams &cp, const UParams &up, int D,
                         int cpad, size_t lds, hipStream_t st) {
    if (bf16_in) return launch_decode_t<bf16>(dp, cp, up, D, cpad, lds, st);
    return launch_decode_t<float>(dp, cp, up, D, cpad, lds, st);
}

}  // namespace rattn
