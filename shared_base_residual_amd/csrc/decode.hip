// decode.hip -- split-K attention kernel of librattn (gfx950).
//
// Fused residual attention for N agents that share one base KV cache
// (ForkKV Guide, "Fused ResidualAttention"; LRAgent, "Flash-LoRA-Attention"):
//   score  s = scale * (q . K_base[j] + (q Bk_a^T) . Lk_a[j])
//   output o = sum_j p_j V_base[j] + (sum_j p_j Lv_a[j]) Bv_a
// Two launches.  The split kernel: each workgroup takes one (group of KV heads,
// row group, context split) and runs compute waves and load waves:
//   * the load waves stream the split's tokens in tiles of T tokens through a
//     ring of LDS stages with direct global->LDS loads (several tiles in
//     flight) and wait for them; a stage holds the tile's base keys and values
//     of the item's heads and the low-rank rows (Lk, Lv) of every agent the
//     workgroup serves, each read from HBM once and shared by all compute waves;
//   * each compute wave forms U = q Bk_a^T for its rows with MFMA, then owns one
//     16-row MFMA row block (query rows of one or more agents) of one head and a
//     share of each tile's tokens: one MFMA contraction scores the base keys
//     against all agents' rows, a second adds the rank-r correction over the
//     agents' Lk rows; online softmax in the log2 domain; P V_base and P Lv
//     accumulate in registers.  Private tokens (decode suffix, causal prefill
//     chunk) are extra work items with per-agent keys and no residual;
//   * the partial state (max, sum, O, W) of every row goes to the workspace.
// Variants: int8 base keys (PolyKV, section 2B; codes scored on fp16 MFMAs
// against fp16 query rows) and, with them, 3-bit Walsh-Hadamard-rotated values
// (the compute waves decode each tile's codes into a double buffer of bf16 rows,
// and the merge undoes the rotation).
// The merge kernel: one workgroup per query row combines the splits with a
// log-sum-exp merge (lane reductions, one LDS pass) and applies Bv once per
// row: o = (sum w O + (sum w W) Bv_a^(k)) / sum w l (LRAgent: B is applied once
// per query block, not per token).
//
// Operand layout (S^T formulation): the MFMA A operand is the key tile (rows =
// 16 tokens), the B operand the query rows (columns = 16 query rows), so the
// scores arrive with one query row per lane column and the softmax statistics
// of a row live in the lanes that own it.  The value product is O^T = V^T P^T
// over 16-token steps (v_mfma_f32_16x16x16_bf16), so P feeds the B operand
// straight from the score registers, and V^T comes from gfx950's transposing
// LDS read.
//
// Loads never branch on the data: token indices beyond the split are clamped
// to its last token (finite data) and those scores are masked to -inf, so
// their weights are exactly zero.
#include <mutex>

#include "device.h"
#include "internal.h"
#include "stage.h"

namespace rattn {

template <typename T, int D, int CPAD>
struct Acc {
    f32x4 o[D / 16];
    f32x4 w[CPAD > 0 ? CPAD / 16 : 1];
    float m, l;  // l: this lane's share of the row's weight sum (fp32 step)
    f32x4 ls;    // bf16 step: the row's weight sum in every element (a ones-row product)
};

// Reads K consecutive elements whose chunks sit at base + ofs[c].
// One 16-token step of one wave: scores for its row block, online softmax,
// value and low-rank value products.  kvb / lrb: the stage plus row0 times the
// K/V and low-rank row bytes; t: token of the step's first row; `masked`:
// some token of the step may lie past t1 or (causal) past the row's position.
template <typename T, int D, int CPAD>
__device__ inline void step16(Acc<T, D, CPAD> &acc, const ReadOfs<T, D, CPAD> &ro, const char *kvb, const char *lrb,
                              int t, bool masked, const typename Ops<T>::frag *qB, const typename Ops<T>::frag *uH,
                              const typename Ops<T>::frag *uL, float cl2, bool resid, int t1, bool causal, int tq,
                              int j4) {
    using O = Ops<T>;
    using frag = typename O::frag;
    using frag4 = typename O::frag4;
    constexpr int KS = D / 32, VPL = D / 16;
    constexpr int CS = CPAD / 32, CPL = CPAD / 16;

    // S^T = K Q^T for 16 tokens x 16 query rows
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const Row<T, 8> kr = lds_get<T, 8>(kvb, ro.k[s]);
        frag kf;
        __builtin_memcpy(&kf, &kr, sizeof(kf));
        a = O::mma(kf, qB[s], a);
    }
    a *= cl2;
    if (CS > 0 && resid) {
#pragma unroll
        for (int s = 0; s < CS; ++s) {
            const Row<T, 8> lr = lds_get<T, 8>(lrb, ro.lk[s]);
            frag lf;
            __builtin_memcpy(&lf, &lr, sizeof(lf));
            a = O::mma(lf, uH[s], a);
            if constexpr (O::kSplitU) a = O::mma(lf, uL[s], a);
        }
    }
    if (masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = t + 4 * j4 + i;
            if (tt >= t1 || (causal && tt > tq)) a[i] = -__builtin_inff();
        }
    }

    // online softmax (log2 domain); the four lanes of a row are j4 = 0..3.
    // The O and W accumulators are rescaled only on the steps where some row's
    // reference max grows (a branch uniform over the wave); on the others
    // alpha is exactly 1.
    // The cross-lane maximum is formed only on the steps where some lane's own
    // maximum passes the slack (a row's does iff one of its lanes' does).
    const float lmx = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
    float alpha = 1.0f;
    if (__builtin_amdgcn_ballot_w64(lmx > acc.m + kRescaleSlack)) {
        float mx = fmaxf(lmx, __shfl_xor(lmx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool grow = mx > acc.m + kRescaleSlack;
        const float m_new = grow ? mx : acc.m;
        alpha = fexp2(acc.m - m_new);
        acc.m = m_new;
#pragma unroll
        for (int i = 0; i < VPL; ++i) acc.o[i] *= alpha;
        if constexpr (CPAD > 0) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc.w[i] *= alpha;
        }
    }
    frag4 pB;
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float e = fexp2(a[i] - acc.m);
        psum += e;
        O::set4(pB, i, e);
    }
    acc.l = acc.l * alpha + psum;

    // O^T += V^T P^T: output tile jj holds d = VPL*m + jj in row m
    Row<T, VPL> vr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = lds_get<T, VPL>(kvb, ro.v[i]);
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj) {
        frag4 vA;
#pragma unroll
        for (int i = 0; i < 4; ++i) O::set4_raw(vA, i, vr[i].e[jj]);
        acc.o[jj] = O::mma16(vA, pB, acc.o[jj]);
    }
    // W^T += Lv^T P^T over the block's residual columns
    if constexpr (CPAD > 0) {
        if (resid) {
            Row<T, CPL> lr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) lr[i] = lds_get<T, CPL>(lrb, ro.lv[i]);
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                frag4 wA;
#pragma unroll
                for (int i = 0; i < 4; ++i) O::set4_raw(wA, i, lr[i].e[jj]);
                acc.w[jj] = O::mma16(wA, pB, acc.w[jj]);
            }
        }
    }
}

// The bf16 step: the same contraction with every LDS operand read issued before
// the first MFMA that needs it, raw (unscaled) scores with the scale folded into
// the exponent, a VALU cross-lane maximum, and the value operands (V and Lv)
// read with gfx950's transposing LDS read, so that output tile jj holds
// d = 16*jj + m in row m (lane (n16, j4) holds d = 16*jj + 4*j4 + i).
// vtr / wtr: lane offsets of the transposed V and Lv reads; U (uH, uL) is
// unscaled.
// MASKED: the tile's rows belong to na agents with separate rank-CPAD caches;
// the score correction runs per agent (that agent's Lk rows against every row's
// U) and is added only in the lanes of that agent's rows, and W accumulates per
// agent with P kept only in those lanes, so W (and U) hold CPAD columns whatever
// the number of agents.
// arow: the agent (0 .. na-1 within the tile) of this lane's row, -1 if none;
// ast: LDS bytes from one agent's low-rank rows to the next.
// KQ8: the keys are excess-128 int8 codes (kb: the K rows, vb: the V rows of
// the step; without KQ8 both are kvb) met by the fp16 query rows qH; kinit
// starts each row's score at minus 1152 times the sum of its fp16 query
// (so the product gives q . code), and U arrives divided by the key scale.
template <int D, int CPAD, bool MASKED, bool KQ8 = false>
__device__ inline void step16_bf16(Acc<bf16, D, CPAD> &acc, const ReadOfs<bf16, D, CPAD> &ro, const uint32_t *vtr,
                                   const uint32_t *wtr, const char *kvb, const char *lrb, int t, bool masked,
                                   const Ops<bf16>::frag *qB, const Ops<bf16>::frag *uH, const Ops<bf16>::frag *uL,
                                   float cl2, bool resid, int t1, bool causal, int tq, int j4, int na, int arow,
                                   int ast, const char *vb = nullptr, const f16x8 *qH = nullptr,
                                   float kinit = 0.0f) {
    using O = Ops<bf16>;
    using frag = O::frag;
    using frag4 = O::frag4;
    constexpr int KS = D / 32, VPL = D / 16;
    constexpr int CS = CPAD / 32, CPL = CPAD / 16;
    constexpr int CSx = CS > 0 ? CS : 1;
    if constexpr (!KQ8) vb = kvb;

    frag kf[KS], lf[CSx];
    f16x8 kh[KQ8 ? KS : 1];
    if constexpr (KQ8) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint32_t w[2];
            __builtin_memcpy(w, __builtin_assume_aligned(kvb + ro.k[s][0], 8), 8);
            kh[s] = codes_to_f16(w[0], w[1]);
        }
    } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            const Row<bf16, 8> kr = lds_get<bf16, 8>(kvb, ro.k[s]);
            __builtin_memcpy(&kf[s], &kr, sizeof(frag));
        }
    }
    if (CS > 0 && resid) {
#pragma unroll
        for (int s = 0; s < CS; ++s) {
            const Row<bf16, 8> lr = lds_get<bf16, 8>(lrb, ro.lk[s]);
            __builtin_memcpy(&lf[s], &lr, sizeof(frag));
        }
    }
    // S^T = K Q^T + Lk U^T, raw, in two independent accumulator chains (even
    // and odd contraction steps, U hi and U lo) so that consecutive MFMAs do not
    // wait for each other's results; summed once at the end
    f32x4 a = {kinit, kinit, kinit, kinit}, a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        if constexpr (KQ8) {
            if (s & 1)
                a2 = mma_f16(kh[s], qH[s], a2);
            else
                a = mma_f16(kh[s], qH[s], a);
        } else {
            if (s & 1)
                a2 = O::mma(kf[s], qB[s], a2);
            else
                a = O::mma(kf[s], qB[s], a);
        }
    }
    if (CS > 0 && resid) {
        if constexpr (MASKED) {
            // agent ag's Lk rows against every row's U, kept (times 1.0, else 0.0:
            // the products are finite) only in the lanes of agent ag's rows
            for (int ag = 0; ag < na; ++ag) {
                if (ag > 0) {
#pragma unroll
                    for (int s = 0; s < CS; ++s) {
                        const Row<bf16, 8> lr = lds_get<bf16, 8>(lrb + ag * ast, ro.lk[s]);
                        __builtin_memcpy(&lf[s], &lr, sizeof(frag));
                    }
                }
                f32x4 t = {0.f, 0.f, 0.f, 0.f}, t2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < CS; ++s) {
                    t = O::mma(lf[s], uH[s], t);
                    t2 = O::mma(lf[s], uL[s], t2);
                }
                const float keep = arow == ag ? 1.0f : 0.0f;
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = __builtin_fmaf(t[i] + t2[i], keep, a[i]);
            }
        } else {
#pragma unroll
            for (int s = 0; s < CS; ++s) {
                a = O::mma(lf[s], uH[s], a);
                a2 = O::mma(lf[s], uL[s], a2);
            }
        }
    }
    a += a2;
    // value operands: issued now, consumed after the softmax
    bf16x4 va[VPL];
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj) va[jj] = lds_tr4(vb + vtr[jj]);
    bf16x4 wa[CPL > 0 ? CPL : 1];
    if constexpr (CPL > 0) {
        if (resid) {
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) wa[jj] = lds_tr4(lrb + wtr[jj]);
        }
    }
    if (masked) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tt = t + 4 * j4 + i;
            if (tt >= t1 || (causal && tt > tq)) a[i] = -__builtin_inff();
        }
    }

    // online softmax (log2 domain, running max in scaled units).  A row's
    // maximum passes the slack iff one of its four lanes' maxima does (the
    // scale is positive and rounding keeps the order), so the cross-lane
    // maximum is formed only on the steps where some lane's passes.
    const float lmx = amax3(a[0], a[1], amax(a[2], a[3]));  // scores are finite or -inf
    if (__builtin_amdgcn_ballot_w64(lmx * cl2 > acc.m + kRescaleSlack)) {
        const float mx = row_max4(lmx) * cl2;  // -inf stays -inf
        const bool grow = mx > acc.m + kRescaleSlack;
        const float m_new = grow ? mx : acc.m;
        const float alpha = fexp2(acc.m - m_new);
        acc.m = m_new;
#pragma unroll
        for (int i = 0; i < VPL; ++i) acc.o[i] *= alpha;
        if constexpr (CPAD > 0) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc.w[i] *= alpha;
        }
        acc.ls *= alpha;
    }
    f32x4 ev;
#pragma unroll
    for (int i = 0; i < 4; ++i) ev[i] = fexp2(__builtin_fmaf(a[i], cl2, -acc.m));
    frag4 pB;
    pB.v = to_bf16x4(ev[0], ev[1], ev[2], ev[3]);
    // row sums on the matrix unit: a ones operand against P^T adds each row's
    // weights exactly as the P V product takes them (bf16), over all 16 tokens
    {
        frag4 ones;
        ones.v = bf16x4{(bf16)1.0f, (bf16)1.0f, (bf16)1.0f, (bf16)1.0f};
        acc.ls = O::mma16(ones, pB, acc.ls);
    }

    // O^T += V^T P^T and W^T += Lv^T P^T
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj) {
        frag4 vA;
        vA.v = va[jj];
        acc.o[jj] = O::mma16(vA, pB, acc.o[jj]);
    }
    if constexpr (CPL > 0) {
        if (resid) {
            if constexpr (MASKED) {
                // Two agents per product: the contraction runs over (agent,
                // token) pairs, slots 0-3 of a lane agent ag's four tokens and
                // slots 4-7 agent ag + 1's same four tokens, each agent's weights
                // kept only in its own rows' lanes.  One 16x16x32 product takes
                // the passes of one 16x16x16 product on this chip.
                // An odd last agent pairs with itself, its second half weighted 0
                // (arow never equals na).
                const bf16x4 z4 = bf16x4{};
                for (int ag = 0; ag < na; ag += 2) {
                    const int agb = ag + 1 < na ? ag + 1 : ag;
                    if (ag > 0) {
#pragma unroll
                        for (int jj = 0; jj < CPL; ++jj) wa[jj] = lds_tr4(lrb + ag * ast + wtr[jj]);
                    }
                    bf16x4 wb[CPL];
#pragma unroll
                    for (int jj = 0; jj < CPL; ++jj) wb[jj] = lds_tr4(lrb + agb * ast + wtr[jj]);
                    frag pp;
                    pp.v = __builtin_shufflevector(arow == ag ? pB.v : z4, arow == ag + 1 ? pB.v : z4, 0, 1, 2, 3,
                                                   4, 5, 6, 7);
#pragma unroll
                    for (int jj = 0; jj < CPL; ++jj) {
                        frag wA;
                        wA.v = __builtin_shufflevector(wa[jj], wb[jj], 0, 1, 2, 3, 4, 5, 6, 7);
                        acc.w[jj] = O::mma(wA, pp, acc.w[jj]);
                    }
                }
            } else {
#pragma unroll
                for (int jj = 0; jj < CPL; ++jj) {
                    frag4 wA;
                    wA.v = wa[jj];
                    acc.w[jj] = O::mma16(wA, pB, acc.w[jj]);
                }
            }
        }
    }
}

// 3-bit values (PolyKV, section 2B): the value codes of a stage become bf16
// value rows in `vrows` (laid out like a stage's value region), scale times
// centroid in the rotated coordinates; the compute waves then read them like
// any value rows, and the merge undoes the rotation.  Work units: chunk m of
// value group q (q = head * G + 16-token group, m = 0..3), one 16-byte chunk of
// 8 coordinates per lane; lane (x, c4) = (lane / 4, lane % 4) takes token x of
// the group, coordinates 32 c4 + 8 m .. + 7 (bits 8 m .. 8 m + 7 of the three
// 32-bit plane words of coordinates 32 c4 ..).  Codes become byte selectors
// (v_perm_b32) into the low and high bytes of the token's eight scaled centroids.
__device__ inline uint32_t spread4(uint32_t x) {  // bit i of x (i < 4) to bit 0 of byte i
    return (x * 0x00204081u) & 0x01010101u;
}

// Units u0 .. u1 - 1 (u = 4 q + m) of the stage at `stage`.
__device__ inline void decode_values3(const Geo &g, int G, int u0, int u1, const char *stage, char *vrows, int lane,
                                      const float *cent) {
    const int x = lane >> 2, c4 = lane & 3;
    uint32_t w0 = 0, w1 = 0, w2 = 0, tl0 = 0, tl1 = 0, th0 = 0, th1 = 0;
    char *row = vrows;
    for (int u = u0; u < u1; ++u) {
        const int q = u >> 2, m = u & 3;
        if (m == 0 || u == u0) {  // a new group: its plane words, scale and centroid table
            const char *vq = stage + 16 * (g.ofs_vq + q * 64);
            w0 = *reinterpret_cast<const uint32_t *>(vq + 48 * x + 4 * c4);
            w1 = *reinterpret_cast<const uint32_t *>(vq + 48 * x + 16 + 4 * c4);
            w2 = *reinterpret_cast<const uint32_t *>(vq + 48 * x + 32 + 4 * c4);
            const float sg = *reinterpret_cast<const float *>(vq + 768 + 4 * x);
            // The token's scaled centroids as bf16, entries 0..7.  The codebook is
            // symmetric (c_k = -c_{7-k}), so entries 4..7 are two packed conversions
            // and entries 0..3 the same values reversed with the sign bit flipped.
            const uint32_t e45 =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{sg * cent[4], sg * cent[5]}, bf16x2));
            const uint32_t e67 =
                __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{sg * cent[6], sg * cent[7]}, bf16x2));
            const uint32_t e01 = __builtin_amdgcn_perm(e67, e67, 0x01000302u) ^ 0x80008000u;  // (-e7, -e6)
            const uint32_t e23 = __builtin_amdgcn_perm(e45, e45, 0x01000302u) ^ 0x80008000u;  // (-e5, -e4)
            // low and high bytes of entries 0..3 and 4..7: the byte tables of v_perm_b32
            tl0 = __builtin_amdgcn_perm(e23, e01, 0x06040200u);
            tl1 = __builtin_amdgcn_perm(e67, e45, 0x06040200u);
            th0 = __builtin_amdgcn_perm(e23, e01, 0x07050301u);
            th1 = __builtin_amdgcn_perm(e67, e45, 0x07050301u);
            const int h = q / G, gg = q - h * G;
            row = vrows + 16 * ((h * g.T + 16 * gg + x) * g.cpr_kv);
        }
        u32x4 out;
#pragma unroll
        for (int hq = 0; hq < 2; ++hq) {  // coordinates 8 m + 4 hq .. + 3 of the lane's 32
            const int b = 8 * m + 4 * hq;
            const uint32_t sel = spread4(__builtin_amdgcn_ubfe(w0, b, 4)) |
                                 (spread4(__builtin_amdgcn_ubfe(w1, b, 4)) << 1) |
                                 (spread4(__builtin_amdgcn_ubfe(w2, b, 4)) << 2);  // byte i: code of b + i
            const uint32_t lo = __builtin_amdgcn_perm(tl1, tl0, sel), hi = __builtin_amdgcn_perm(th1, th0, sel);
            out[2 * hq] = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // coordinate pairs (0, 1), (2, 3)
            out[2 * hq + 1] = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
        }
        *reinterpret_cast<u32x4 *>(row + 16 * swz(x, 4 * c4 + m, g.cpr_kv, g.lg_kv)) = out;
    }
}

// ------------------------------------------------------------ split kernel --

// MAXW: most waves a workgroup of this instantiation runs (compute + load
// waves): 8 leaves each wave up to 256 VGPRs, 12 up to 168.
// MASKED (bf16, per-agent caches of rank CPAD >= 32 with several agents per
// 16-row block): U and W hold CPAD columns and the rank-r products run per agent
// of the block (see step16_bf16).
// KQ8 (bf16 only): base keys are excess-128 int8 codes with one scale; only
// prefix items exist then (no private tokens).
template <typename T, int D, int CPAD, bool MASKED, int MAXW, bool KQ8 = false, bool VQ3 = false>
__global__ __launch_bounds__(64 * MAXW) void decode_split_kernel(DecodeParams p) {
    using O = Ops<T>;
    using frag = typename O::frag;
    static_assert(!KQ8 || sizeof(T) == 2, "int8 keys with bf16 queries and values only");
    static_assert(!VQ3 || KQ8, "3-bit values come with int8 keys");
    constexpr int KS = D / 32;
    constexpr int VPL = D / 16;
    constexpr int CS = CPAD / 32;
    constexpr int CSx = CS > 0 ? CS : 1;
    constexpr int CPLx = CPAD > 0 ? CPAD / 16 : 1;
    constexpr int ES = (int)sizeof(T);
    constexpr int KRE = KQ8 ? D / 2 : D;  // elements of T per staged K row (int8: two codes each)

    extern __shared__ __attribute__((aligned(16))) char smem[];
    touch_params<DecodeParams>();

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int n16 = lane & 15;
    const int j4 = lane >> 4;

    // Workgroup i is dispatched to XCD i % 8.  Each XCD takes an equal share of
    // the prefix items first, then an equal share of the private items.  Prefix
    // items are numbered KV-head fastest, so the KV heads of one (split, row
    // group) run back to back on one XCD, where they share the low-rank rows
    // through that XCD's L2.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, pos = bid >> 3;
    int li;
    if (pos < p.pre_per) {
        li = xcd * p.pre_per + pos;
        if (li >= p.n_prefix_items) return;
    } else {
        const int iv = xcd * p.pv_per + (pos - p.pre_per);
        if (iv >= p.n_items - p.n_prefix_items) return;
        li = p.n_prefix_items + iv;
    }

    int k0, nh, slot, nblk, blk0, agent_p = 0;
    int t0, t1;
    bool prefix;
    if (li < p.n_prefix_items) {
        // prefix item: H KV heads starting at k0 (head groups fastest), one row group, one split
        const int rest = fdiv(li, p.fd_hg);
        const int hg = li - rest * p.n_hg;
        k0 = hg * p.H;
        nh = p.H;
        const int s = fdiv(rest, p.fd_rg);
        const int rg = rest - s * p.n_rg;
        blk0 = rg * p.bpg;
        nblk = p.n_blocks - blk0 < p.bpg ? p.n_blocks - blk0 : p.bpg;
        t0 = s * p.tok_ps;
        t1 = t0 + p.tok_ps < p.L ? t0 + p.tok_ps : (int)p.L;
        slot = s;
        prefix = true;
    } else {
        const int l2 = li - p.n_prefix_items;
        int rest = fdiv(l2, p.fd_hk);
        k0 = l2 - rest * p.HK;
        nh = 1;
        const int r2 = fdiv(rest, p.fd_pv);
        const int s = rest - r2 * p.n_pv;
        agent_p = fdiv(r2, p.fd_prg);
        const int prg = r2 - agent_p * p.n_prg;
        blk0 = prg * 4;
        nblk = p.pb - blk0 < 4 ? p.pb - blk0 : 4;
        t0 = s * p.tok_pv;
        t1 = t0 + p.tok_pv < p.S ? t0 + p.tok_pv : (int)p.S;
        slot = p.n_ps + s;
        prefix = false;
    }
    if (t1 < t0) t1 = t0;  // an empty trailing split
    const bool resid = prefix && (CPAD > 0) && p.r > 0;
    const bool causal = !prefix && p.causal;
    // Agents the workgroup serves.
    int a_lo, a_hi;
    if (prefix) {
        const RowBlock b0 = prefix_block(blk0, p.N, p.rpa, p.apb, p.fd_bpa);
        const RowBlock b1 = prefix_block(blk0 + nblk - 1, p.N, p.rpa, p.apb, p.fd_bpa);
        a_lo = b0.a0;
        a_hi = b1.a0 + b1.na - 1;
    } else {
        a_lo = a_hi = agent_p;
    }

    // ---- stage geometry and token source of this item
    Geo g;
    g.T = prefix ? p.T_pre : p.T_pv;
    g.nst = prefix ? p.nst_pre : p.nst_pv;
    g.stage_bytes = prefix ? p.stage_bytes_pre : p.stage_bytes_pv;
    g.cpr_kv = D * ES / 16;
    g.lg_kv = ilog2(g.cpr_kv);
    g.cpr_k = KRE * ES / 16;
    g.lg_k = ilog2(g.cpr_k);
    if (resid) {
        g.cpa_lr = p.r * ES / 16;
        g.lg_lr = ilog2(g.cpa_lr);
        g.na_lr = p.shared_lr ? 1 : a_hi - a_lo + 1;
    } else {
        g.cpa_lr = 1;
        g.lg_lr = 0;
        g.na_lr = 0;
    }
    g.lr_grp = 16 * g.na_lr * g.cpa_lr;
    g.H = nh;
    g.ofs_v = nh * g.T * g.cpr_k;
    // 3-bit values: a stage holds no value rows (they are decoded into a double
    // buffer after the ring, vbuf_off), but their codes and scales at its end
    g.ofs_lk = g.ofs_v + (VQ3 ? 0 : nh * g.T * g.cpr_kv);
    g.ofs_lv = g.ofs_lk + (resid ? (g.T >> 4) * g.lr_grp : 0);
    g.chunks = g.ofs_lv + (resid ? (g.T >> 4) * g.lr_grp : 0);
    g.ofs_vq = g.chunks;
    if constexpr (VQ3) g.chunks += nh * (g.T >> 4) * 64;
    const int vbuf_bytes = VQ3 ? nh * g.T * g.cpr_kv * 16 : 0;  // one decoded buffer

    int *s_pages = reinterpret_cast<int *>(smem + p.table_lds_off);
    Src<T> src;
    src.tlast = t1 > t0 ? t1 - 1 : t0;
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
    src.vq = nullptr;
    src.vs = nullptr;
    src.vq_hs = 0;
    if constexpr (VQ3) {  // prefix items of a contiguous base cache only (the planner's limits)
        src.vq = static_cast<const uint8_t *>(p.vb) + (int64_t)k0 * p.L * 48;
        src.vs = p.vs + (int64_t)k0 * p.L;
        src.vq_hs = p.L;
    }
    if (prefix) {
        src.kb = static_cast<const T *>(p.kb);
        src.vb = static_cast<const T *>(p.vb);
        if (p.ps > 0) {
            src.page_stride = (int64_t)p.HK * p.ps * D;
            src.k_page_stride = (int64_t)p.HK * p.ps * KRE;
            src.kb += (int64_t)k0 * p.ps * KRE;
            src.vb += (int64_t)k0 * p.ps * D;
            src.head_stride = (int64_t)p.ps * D;
            src.k_head_stride = (int64_t)p.ps * KRE;
            src.pg0 = fdiv(t0, p.fd_ps);
        } else {
            src.kb += (int64_t)k0 * p.L * KRE;
            src.vb += (int64_t)k0 * p.L * D;
            src.head_stride = p.L * D;
            src.k_head_stride = p.L * KRE;
        }
        if (resid) {
            const int64_t a_lr = p.shared_lr ? 0 : a_lo;
            src.lk = static_cast<const T *>(p.lk) + a_lr * p.L * p.r;
            src.lv = static_cast<const T *>(p.lv) + a_lr * p.L * p.r;
            src.lr_agent_stride = p.L * p.r;
        }
    } else {
        const int64_t seg = ((int64_t)agent_p * p.HK + k0) * p.S * D;  // one head per private item
        src.kb = static_cast<const T *>(p.kp) + seg;
        src.vb = static_cast<const T *>(p.vp) + seg;
    }
    if constexpr (KQ8) {
        if (!prefix) return;  // never planned: int8 keys come without private tokens
    }
    if (src.page_stride && t1 > t0) {
        // the split's page-table entries, read once into LDS
        const int npg = fdiv(t1 - 1, p.fd_ps) - src.pg0 + 1;
        for (int i = threadIdx.x; i < npg; i += blockDim.x) s_pages[i] = p.table[src.pg0 + i];
        __syncthreads();
    }

    // The fill plan of this wave.
    const bool compute_wave = wave < p.nw;  // the others only load
    FillPlan fp;
    make_fill_plan<T, D, KRE>(fp, g, src, resid, compute_wave ? p.np : wave - p.nw, lane, p.np, p.lr_own != 0, VQ3);
    // keys and values that no other workgroup reads are streamed past the caches
    fp.kv_nt = prefix ? p.n_rg == 1 : p.n_prg == 1;
    const int n_tiles = (t1 - t0 + g.T - 1) >> ilog2(g.T);  // T is a power of two
    const int fpw = fp.fpw;
    auto fill = [&](int tile, int stage) {
        const int tt = t0 + tile * g.T;
        fill_stage<T, D, KRE>(fp, g, src, tt, smem + (size_t)stage * g.stage_bytes, tt + g.T - 1 > src.tlast, lane);
    };
    // ---- the load waves start the ring (tiles 0 .. nst-2) at once, before the
    // compute waves set up their rows, load the queries and form U
    if (fpw)
        for (int i = 0; i < g.nst - 1 && i < n_tiles; ++i) fill(i, i);
    // Row tiles: nblk row blocks of each of the nh heads; TG waves share a tile
    // (token groups).
    const int TG = small_div(p.nw, nh * nblk);
    const int rbi = small_div(wave, TG);
    const int tg = wave - rbi * TG;
    const int hw = rbi < nh * nblk ? small_div(rbi, nblk) : 0;  // this wave's head within the item
    const int bw = rbi < nh * nblk ? rbi - hw * nblk : 0;         // and its row block
    const int k = k0 + hw;                            // this wave's KV head

    // Row block of this wave.
    RowBlock blk;
    if (prefix) {
        blk = prefix_block(blk0 + bw, p.N, p.rpa, p.apb, p.fd_bpa);
    } else {
        blk.a0 = agent_p;
        blk.na = 1;
        blk.f = p.rpa <= 16 ? 0 : 16 * (blk0 + bw);
        blk.nr = p.rpa - blk.f < 16 ? p.rpa - blk.f : 16;
    }
    const bool wave_on = compute_wave && rbi < nh * nblk;
    // Query row owned by this lane's column.
    const bool vm = wave_on && n16 < blk.nr;
    int agent_m = 0, ria = 0;
    if (vm) block_row(blk, n16, p.fd_rpa, &agent_m, &ria);
    const int arow_m = agent_m - blk.a0;  // the row's agent within the block
    const int tq = fdiv(ria, p.fd_g), hh = ria - tq * p.g;
    const int64_t qrow = ((int64_t)agent_m * p.QL + tq) * p.HQ + (int64_t)k * p.g + hh;
    const int64_t grow = (int64_t)agent_m * p.rpa + ria;
    const float cl2 = p.c;
    const int cvalid = resid ? (p.shared_lr ? p.r : blk.na * p.r) : 0;
    const int lr_col0 = resid && !p.shared_lr ? (blk.a0 - a_lo) * p.r : 0;  // block's first column in the tile

    // Query rows as the B operand of S^T = K Q^T.
    const T *qp = static_cast<const T *>(p.q);
    frag qB[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qB[s] = O::zero();
    if (wave_on) {
#pragma unroll
        for (int s = 0; s < KS; ++s)
            if (vm) qB[s] = O::load8(qp + qrow * D + 32 * s + 8 * j4);
    }

    // ---- lane offsets of this wave's LDS reads: its head's K and V regions
    // of the stage (chunks)
    const int kreg = hw * g.T * g.cpr_k, vreg = g.ofs_v + hw * g.T * g.cpr_kv;
    ReadOfs<T, D, CPAD> ro;
    {
        using RO = ReadOfs<T, D, CPAD>;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int c = 0; c < RO::FC; ++c)
                ro.k[s][c] = KQ8 ? elem_ofs(kreg, n16, 32 * s + 8 * j4, g.cpr_k, g.lg_k)  // 8 code bytes
                                 : elem_ofs(kreg, n16, (32 * s + 8 * j4) * ES + 16 * c, g.cpr_k, g.lg_k);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < RO::VC; ++c)
                ro.v[i][c] = elem_ofs(vreg, 4 * j4 + i, VPL * n16 * ES + 16 * c, g.cpr_kv, g.lg_kv);
#pragma unroll
        for (int s = 0; s < RO::CSx; ++s) {
            int col = 32 * s + 8 * j4;
            col = lr_col0 + (col < cvalid ? col : 0);  // padding column: U is zero there
#pragma unroll
            for (int c = 0; c < RO::FC; ++c)
                ro.lk[s][c] = resid ? lr_ofs(g, g.ofs_lk, col >> p.lr_shift, n16, (col & (p.r - 1)) * ES + 16 * c) : 0u;
        }
        int colv = RO::CPL * n16;
        colv = lr_col0 + (colv < cvalid ? colv : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < RO::LC; ++c)
                ro.lv[i][c] =
                    resid ? lr_ofs(g, g.ofs_lv, colv >> p.lr_shift, 4 * j4 + i, (colv & (p.r - 1)) * ES + 16 * c) : 0u;
    }
    const int kv_rowb = D * ES, lr_rowb = 16 * g.na_lr * g.cpa_lr;  // a step at row0 starts row0 * these bytes in
    const int k_rowb = KRE * ES;                                       // (K rows: k_rowb)
    // bf16 step: transposed value reads.  For d-tile jj, lane (4i + a, j4) points at
    // row 4*j4 + i, columns 16*jj + 4a (residual columns of the block; padding
    // columns read column 0 of the block, their W is dropped at the store).
    uint32_t vtr[VPL], wtr[CPLx];
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj)
        vtr[jj] = elem_ofs(vreg, 4 * j4 + (n16 >> 2), ES * (16 * jj + 4 * (n16 & 3)), g.cpr_kv, g.lg_kv);
#pragma unroll
    for (int jj = 0; jj < CPLx; ++jj) {
        int col = 16 * jj + 4 * (n16 & 3);
        col = lr_col0 + (col < cvalid ? col : 0);
        wtr[jj] = resid ? lr_ofs(g, g.ofs_lv, col >> p.lr_shift, 4 * j4 + (n16 >> 2), (col & (p.r - 1)) * ES) : 0u;
    }

    // U = scale*log2(e) * q Bk^T as the B operand of the rank-r score correction,
    // block-diagonal over the agents of the block (bf16 carries hi + lo halves).
    // Computed as U^T = Bk Q^T with MFMA; A-operand row rho of output tile 2s+h
    // is residual column 32s + 8(rho/4) + 4h + rho%4, so that each lane's
    // results land in its own B-operand slots.
    frag uH[CSx], uL[CSx];
    constexpr bool kBf16 = sizeof(T) == 2;
    // the bf16 step folds the scale into the exponent; with int8 keys the
    // exponent's scale includes the key scale, so U is divided by it
    const float uscale = KQ8 ? p.u_scale : kBf16 ? 1.0f : cl2;
#pragma unroll
    for (int s = 0; s < CSx; ++s) {
        uH[s] = O::zero();
        uL[s] = O::zero();
    }
    if (MASKED && resid && wave_on && n_tiles > 0) {
        // Per-agent caches, one agent at a time: U^T = Bk_a Q^T for every row of
        // the block, kept in the lanes of agent a's rows (the columns are that
        // agent's own, so every lane ends with its own agent's U).
        const T *bk = static_cast<const T *>(p.bk);
        const int64_t ldb = (int64_t)p.HK * D;
        float uv[CSx][8];
#pragma unroll
        for (int s = 0; s < CSx; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) uv[s][i] = 0.0f;
        // two agents' Bk rows in flight: the next agent's loads overlap this one's MFMAs
        auto load_bk = [&](frag (&bkf)[CSx][2][KS], int ag) {
#pragma unroll
            for (int s = 0; s < CSx; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int crow = 32 * s + 8 * (n16 >> 2) + 4 * h + (n16 & 3);  // A-operand row (< CPAD = r)
                    const T *brow = bk + ((int64_t)(blk.a0 + ag) * p.r + crow) * ldb + (int64_t)k * D + 8 * j4;
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) bkf[s][h][s2] = O::load8(brow + 32 * s2);
                }
        };
        auto use_bk = [&](const frag (&bkf)[CSx][2][KS], int ag) {
            const bool keep = vm && arow_m == ag;
#pragma unroll
            for (int s = 0; s < CSx; ++s)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int s2 = 0; s2 < KS; ++s2) a = O::mma(bkf[s][h][s2], qB[s2], a);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (keep) uv[s][4 * h + i] = a[i] * uscale;
                }
        };
        if constexpr (CSx <= 2) {
            frag bk0[CSx][2][KS], bk1[CSx][2][KS];
            load_bk(bk0, 0);
            for (int ag = 0; ag < blk.na; ag += 2) {
                if (ag + 1 < blk.na) load_bk(bk1, ag + 1);
                use_bk(bk0, ag);
                if (ag + 2 < blk.na) load_bk(bk0, ag + 2);
                if (ag + 1 < blk.na) use_bk(bk1, ag + 1);
            }
        } else {  // rank 128: one agent at a time (registers)
            frag bk0[CSx][2][KS];
            for (int ag = 0; ag < blk.na; ++ag) {
                load_bk(bk0, ag);
                use_bk(bk0, ag);
            }
        }
#pragma unroll
        for (int s = 0; s < CSx; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                O::set(uH[s], i, uv[s][i]);
                if constexpr (O::kSplitU) {
                    const float hi = (float)(bf16)uv[s][i];
                    O::set(uL[s], i, uv[s][i] - hi);
                }
            }
    }
    if (!MASKED && CPAD > 0 && resid && wave_on && n_tiles > 0 && !p.shared_lr) {
        // Per-agent caches: one Bk row per A-operand row; every load is issued
        // before the first MFMA (one memory round trip).
        const T *bk = static_cast<const T *>(p.bk);
        const int64_t ldb = (int64_t)p.HK * D;
        const int rmask = p.r - 1;
        frag bkf[CSx][2][KS];
#pragma unroll
        for (int s = 0; s < CSx; ++s)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int crow = 32 * s + 8 * (n16 >> 2) + 4 * h + (n16 & 3);  // A-operand row
                const bool okc = crow < cvalid;
                const int arow = blk.a0 + (okc ? (crow >> p.lr_shift) : 0);
                const int colr = okc ? (crow & rmask) : 0;
                const T *brow = bk + ((int64_t)arow * p.r + colr) * ldb + (int64_t)k * D + 8 * j4;
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) bkf[s][h][s2] = O::load8(brow + 32 * s2);
            }
#pragma unroll
        for (int s = 0; s < CSx; ++s) {
            float uv[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s2 = 0; s2 < KS; ++s2) a = O::mma(bkf[s][h][s2], qB[s2], a);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 32 * s + 8 * j4 + 4 * h + i;  // column this lane received
                    const bool keep = vm && c < cvalid && blk.a0 + (c >> p.lr_shift) == agent_m;
                    uv[4 * h + i] = keep ? a[i] * uscale : 0.0f;
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
    if (CPAD > 0 && resid && wave_on && n_tiles > 0 && p.shared_lr) {
        // One cache for all agents: each agent of the block has its own Bk.
        const T *bk = static_cast<const T *>(p.bk);
        const int64_t ldb = (int64_t)p.HK * D;
        const int rmask = p.r - 1;
        const int na_loop = blk.na;
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
                        if (keep) uv[4 * h + i] += a[i] * uscale;
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

    // int8 keys: the query rows as fp16 (exact for bf16 values of normal range)
    // and each row's score offset, minus 1152 times the sum of those values
    f16x8 qH[KQ8 ? KS : 1];
    float kinit = 0.0f;
    if constexpr (KQ8) {
        if (compute_wave) wait_vmcnt(0);
        float qs = 0.0f;
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const f16 h = (f16)(float)qB[s].v[i];
                qH[s][i] = h;
                qs += (float)h;
            }
        kinit = -1152.0f * row_sum4(qs);
    }

    // Every register load (q, Bk) of a compute wave has landed, so the compiler
    // has nothing pending inside the ring loop and adds no waits of its own there.
    if (compute_wave) wait_vmcnt(0);

    Acc<T, D, CPAD> acc;
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc.o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CPLx; ++i) acc.w[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    acc.m = -1.0e30f;
    acc.l = 0.0f;
    acc.ls = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- the ring.  Load waves: wait for their loads of tile i, meet the others
    // at the ring barrier (everyone is done with tile i-1), refill that stage.
    // Compute waves: meet at the barrier (tile i has landed), compute it.  Each
    // role runs a loop of its own with the same barriers, so neither carries the
    // other's state through its loop.
    const int spw = g.T / (16 * TG);  // 16-token steps per wave per tile
    // 3-bit values: each compute wave decodes its share of the value groups of a
    // tile into buffer (tile % 2): tile 0 after a first barrier, tile i + 1 after
    // computing tile i (that buffer's last reader, tile i - 1, finished before
    // barrier i).  The load waves only load: their loop is bound by the issue of
    // the direct loads, so decoding there lengthens every tile.
    auto decode_share = [&](int j) {
        if constexpr (VQ3) {
            const int G = g.T >> 4, U = 4 * nh * G;
            decode_values3(g, G, wave * U / p.nw, (wave + 1) * U / p.nw, smem + (size_t)(j % g.nst) * g.stage_bytes,
                           smem + p.vbuf_off + (j & 1) * vbuf_bytes, lane, p.vq_c);
        }
    };
    if (!compute_wave) {
        if constexpr (VQ3) {
            // tile i + 1 is decoded after barrier i, so it must have landed by then:
            // this wave waits one tile ahead, and the ring keeps nst - 2 tiles in flight
            int issued = n_tiles < g.nst - 1 ? n_tiles : g.nst - 1;  // tiles 0 .. issued - 1
            auto wait_landed = [&](int j) {  // this wave's loads of tiles 0 .. j have landed
                const int after = issued - 1 - j;
                wait_vmcnt(after > 0 ? after * fpw : 0);
            };
            wait_landed(n_tiles > 1 ? 1 : 0);
            ring_barrier();  // tiles 0 and 1 have landed
            for (int i = 0; i < n_tiles; ++i) {
                ring_barrier();
                if (i + g.nst - 1 < n_tiles) {
                    if (fpw) fill(i + g.nst - 1, (i + g.nst - 1) % g.nst);
                    ++issued;
                }
                if (i + 2 < n_tiles) wait_landed(i + 2);
            }
        } else {
            for (int i = 0; i < n_tiles; ++i) {
                const int later = (n_tiles - 1 - i) < (g.nst - 2) ? (n_tiles - 1 - i) : (g.nst - 2);
                wait_vmcnt(later * fpw);  // this wave's loads of tile i have landed
                ring_barrier();
                if (fpw && i + g.nst - 1 < n_tiles) fill(i + g.nst - 1, (i + g.nst - 1) % g.nst);
            }
        }
    } else {
        if constexpr (VQ3) {
            ring_barrier();  // tiles 0 and 1 have landed
            if (n_tiles > 0) decode_share(0);
        }
        for (int i = 0; i < n_tiles; ++i) {
            ring_barrier();
            if (wave_on) {
                const char *st = smem + (size_t)(i % g.nst) * g.stage_bytes;
                const int tt = t0 + i * g.T;
                const bool masked = causal || tt + g.T > t1;
                for (int u = 0; u < spw; ++u) {
                    const int row0 = 16 * (tg * spw + u);
                    if constexpr (KQ8) {
                        // K rows (int8) and V rows have different pitches: two stage bases
                        const int ko = __builtin_amdgcn_readfirstlane((int)(st - smem) + row0 * k_rowb);
                        // (3-bit values: the decoded buffer i % 2, laid out like a stage's value
                        // region, whose offset the read offsets include)
                        const int vo = __builtin_amdgcn_readfirstlane(
                            VQ3 ? p.vbuf_off + (i & 1) * vbuf_bytes - 16 * g.ofs_v + row0 * kv_rowb
                                : (int)(st - smem) + row0 * kv_rowb);
                        const int lo = __builtin_amdgcn_readfirstlane((int)(st - smem) + row0 * lr_rowb);
                        step16_bf16<D, CPAD, MASKED, true>(acc, ro, vtr, wtr, smem + ko, smem + lo, tt + row0, masked,
                                                           qB, uH, uL, cl2, resid, t1, causal, tq, j4, blk.na,
                                                           vm ? arow_m : -1, 256 * g.cpa_lr, smem + vo, qH, kinit);
                    } else if constexpr (kBf16) {
                        // the step's stage offsets as opaque wave-uniform values: one add per
                        // operand read, rather than per-read offsets advanced every step
                        const int ko = __builtin_amdgcn_readfirstlane((int)(st - smem) + row0 * kv_rowb);
                        const int lo = __builtin_amdgcn_readfirstlane((int)(st - smem) + row0 * lr_rowb);
                        step16_bf16<D, CPAD, MASKED>(acc, ro, vtr, wtr, smem + ko, smem + lo,
                                                     tt + row0, masked, qB, uH, uL, cl2, resid, t1, causal, tq, j4,
                                                     blk.na, vm ? arow_m : -1, 256 * g.cpa_lr);
                    }
                    else
                        step16<T, D, CPAD>(acc, ro, st + row0 * kv_rowb, st + row0 * lr_rowb, tt + row0, masked, qB, uH,
                                           uL, cl2, resid, t1, causal, tq, j4);
                }
            }
            if constexpr (VQ3) {
                if (i + 1 < n_tiles) decode_share(i + 1);
            }
        }
    }
    float m_run = acc.m, l_run;
    if constexpr (kBf16) {
        l_run = acc.ls[0];  // already the whole row's sum
    } else {
        // sum of weights over the four lanes that share this query row
        l_run = acc.l;
        l_run += __shfl_xor(l_run, 16);
        l_run += __shfl_xor(l_run, 32);
    }

    // ---- merge the token groups of a row block (same lane layout in every wave);
    // the stages are free now (every load was awaited in the last iteration).
    __syncthreads();
    float *smf = reinterpret_cast<float *>(smem);
    constexpr int PER_LANE = 4 * VPL + 4 * CPLx;
    if (TG > 1) {
        // waves with tg > 0 publish their state: one slot per wave
        float *sm = smf + (size_t)wave * (64 * PER_LANE + 32);
        if (compute_wave && tg > 0) {
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
        if (compute_wave && tg == 0) {
            float mt = m_run;
            for (int w = 1; w < TG; ++w)
                mt = fmaxf(mt, smf[(size_t)(wave + w) * (64 * PER_LANE + 32) + 64 * PER_LANE + n16]);
            const float s0 = fexp2(m_run - mt);
            l_run *= s0;
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) acc.o[jj] *= s0;
#pragma unroll
            for (int jj = 0; jj < CPLx; ++jj) acc.w[jj] *= s0;
            for (int w = 1; w < TG; ++w) {
                const float *sw = smf + (size_t)(wave + w) * (64 * PER_LANE + 32);
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
    if (kBf16 && tg == 0 && vm) {
        // natural order: tile jj, element i of this lane is d (or c) = 16*jj + 4*j4 + i;
        // O and W divided by the row's weight sum, as fp16 (a row without a visible
        // token, l = 0, stores zeros and gets weight 0 in the merge)
        const int64_t rec = ((int64_t)k * p.N * p.rpa + grow) * p.n_slots + slot;
        const float inv_l = l_run > 0.0f ? 1.0f / l_run : 0.0f;
        f16 *po = static_cast<f16 *>(p.p_o) + rec * D + 4 * j4;
        f16 *pw = static_cast<f16 *>(p.p_w) + rec * p.r;
#pragma unroll
        for (int jj = 0; jj < VPL; ++jj) *reinterpret_cast<f16x4 *>(po + 16 * jj) = to_f16x4(acc.o[jj] * inv_l);
        if (resid) {
            const int arel = agent_m - blk.a0;
            if constexpr (MASKED) {
                // every column is this row's own agent's (element stores: measured
                // faster here than the vector form below, through the schedule of the
                // whole kernel rather than the stores themselves)
#pragma unroll
                for (int jj = 0; jj < CPLx; ++jj)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 16 * jj + 4 * j4 + i;
                        if (c < cvalid) pw[c & (p.r - 1)] = (f16)(acc.w[jj][i] * inv_l);
                    }
            } else {
                // the lane's four columns c0 .. c0 + 3 of tile jj belong to one agent (r >= 8)
#pragma unroll
                for (int jj = 0; jj < CPLx; ++jj) {
                    const int c0 = 16 * jj + 4 * j4;
                    if (c0 < cvalid && (p.shared_lr || (c0 >> p.lr_shift) == arel))
                        *reinterpret_cast<f16x4 *>(pw + (c0 & (p.r - 1))) = to_f16x4(acc.w[jj] * inv_l);
                }
            }
        }
        if (j4 == 0) *reinterpret_cast<float2 *>(p.p_ml + rec * 2) = float2{m_run, l_run};
    }
    if (!kBf16 && tg == 0 && vm) {
        const int64_t rec = ((int64_t)k * p.N * p.rpa + grow) * p.n_slots + slot;
        float ov[4 * VPL];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) ov[VPL * i + jj] = acc.o[jj][i];
        float *po = static_cast<float *>(p.p_o) + rec * D + 4 * VPL * j4;
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
                        static_cast<float *>(p.p_w)[rec * p.r + (c & (p.r - 1))] = acc.w[jj][i];
                }
        }
        if (j4 == 0) *reinterpret_cast<float2 *>(p.p_ml + rec * 2) = float2{m_run, l_run};
    }
}


// ---------------------------------------------------------------- combine --

// One workgroup (512 threads) per query row R = (a * q_len + t) * H_q + h: a
// log-sum-exp merge of the row's split partials, then o += (sum w W) Bv_a^(k)
// (Bv applied once per row), o /= sum w l.  The partial O rows of one query row
// are contiguous ([n_slots][d] floats) and are read as float4 by all threads;
// thread t always lands on column group t % (d/4), so it accumulates one float4
// and the threads of a column group are summed through LDS at the end.  The
// first batch of O, W and Bv loads is issued before the weight pass, so the
// row costs about two memory round trips.
constexpr int kCombineThreads = 512;
static_assert(kMaxSlots <= kCombineThreads, "the merge gives each slot one thread");
constexpr int kCombineBatch = 8;  // float4 loads of O per thread per batch

template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(DecodeParams p) {
    constexpr int NT = kCombineThreads, NWV = NT / 64, D4 = D / 4, B = kCombineBatch;
    __shared__ float s_w[kMaxSlots];
    __shared__ f32x4 s_o[NT];
    __shared__ float s_red[2 * NWV];
    __shared__ f32x4 s_wp[NWV * 32];  // per-wave W column-group sums
    __shared__ float s_wt[128];       // merged W (r <= 128)
    __shared__ float s_wbv[NWV * D];  // per-wave (W Bv) column sums
    __shared__ float s_fw[D];         // 3-bit values: the merged O before the inverse rotation
    touch_params<DecodeParams>();
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int R = blockIdx.x;  // (agent, query token, query head), < 2^31
    const int at = fdiv(R, p.fd_hq), h = R - at * p.HQ;
    const int a = fdiv(at, p.fd_ql), t = at - a * p.QL;
    const int k = fdiv(h, p.fd_g), ria = t * p.g + (h - k * p.g);
    const int64_t rec0 = ((int64_t)k * p.N * p.rpa + (int64_t)a * p.rpa + ria) * p.n_slots;
    const int ns = p.n_slots, nps = p.n_ps, r = p.r;
    const bool wres = r > 0 && nps > 0;
    const int R4 = wres ? r / 4 : 1;  // 2 .. 32, divides NT

    // this thread's slot statistics (one slot per thread: n_slots <= kMaxSlots = NT),
    // loaded first: the weight pass waits for it alone
    const float2 ml = tid < ns ? *reinterpret_cast<const float2 *>(p.p_ml + (rec0 + tid) * 2) : float2{-3.0e38f, 0.0f};
    // Partial O and W, read four elements at a time (q = slot * D/4 + column group):
    // fp16 divided by the slot's weight sum on the bf16 path (so slot s enters with
    // weight w_s l_s), fp32 unnormalised otherwise (weight w_s).
    constexpr bool kHalf = sizeof(T) == 2;
    constexpr int PE = kHalf ? 2 : 4;
    auto load4 = [](const char *b, int q) -> f32x4 {
        if constexpr (kHalf)
            return __builtin_convertvector(*reinterpret_cast<const f16x4 *>(b + 8 * (int64_t)q), f32x4);
        else
            return *reinterpret_cast<const f32x4 *>(b + 16 * (int64_t)q);
    };
    // first batch of O, W and Bv, issued now
    const char *po = static_cast<const char *>(p.p_o) + rec0 * D * PE;
    const int nq = ns * D4;
    f32x4 ob[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const int q = tid + u * NT;
        ob[u] = q < nq ? load4(po, q) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const char *pw = static_cast<const char *>(p.p_w) + rec0 * (wres ? r : 0) * PE;
    const int nqw = wres ? nps * R4 : 0;
    f32x4 wb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + u * NT;
        wb[u] = q < nqw ? load4(pw, q) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Bv rows: thread t takes columns 8 (t % CPR) .. + 7 of rows j = t / CPR + RPR u
    // (CPR = D / 8 threads per row, RPR = NT / CPR rows per round), every row of
    // Bv_a^(k) in one batch of 16-byte loads
    constexpr int CPR = D / 8, RPR = NT / CPR, NU = kMaxResidColsHard / RPR;
    const T *bv = static_cast<const T *>(p.bv) + (int64_t)a * r * p.HK * D + (int64_t)k * D + 8 * (tid % CPR);
    const int64_t ldb = (int64_t)p.HK * D;
    Row<T, 8> bvr[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int j = tid / CPR + RPR * u;
        bvr[u] = (wres && j < r) ? load_row<T, 8>(bv + (int64_t)j * ldb) : zero_row<T, 8>();
    }

    // weights of the slots: w_s = exp2(m_s - M), L = sum w_s l_s
    float M, Lsum;
    const float *sw;  // w of slot s at sw[s]
    if (ns <= 64) {
        // every wave forms all of them from the first 64 slots' statistics
        // (lane = slot), into a block of its own: no workgroup barrier
        const float2 m1 = lane < ns ? (wv == 0 ? ml : *reinterpret_cast<const float2 *>(p.p_ml + (rec0 + lane) * 2))
                                    : float2{-3.0e38f, 0.0f};
        M = lane_max64(m1.x);
        const float w1 = lane < ns ? fexp2(m1.x - M) : 0.0f;
        Lsum = lane_group_sum(w1 * m1.y, 1);
        s_w[wv * 64 + lane] = kHalf ? w1 * m1.y : w1;
        __builtin_amdgcn_wave_barrier();
        sw = s_w + wv * 64;
    } else {
        const float mloc = lane_max64(ml.x);
        if (lane == 0) s_red[wv] = mloc;
        __syncthreads();
        M = s_red[0];
#pragma unroll
        for (int i = 1; i < NWV; ++i) M = fmaxf(M, s_red[i]);
        const float w = tid < ns ? fexp2(ml.x - M) : 0.0f;
        s_w[tid] = kHalf ? w * ml.y : w;
        const float lloc = lane_group_sum(w * ml.y, 1);
        if (lane == 0) s_red[NWV + wv] = lloc;
        __syncthreads();
        Lsum = 0.0f;
#pragma unroll
        for (int i = 0; i < NWV; ++i) Lsum += s_red[NWV + i];
        sw = s_w;
    }

    // O = sum_s w_s O_s
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < B; ++u) {
        const int q = tid + u * NT;
        if (q < nq) acc += sw[q / D4] * ob[u];
    }
    for (int q0 = B * NT; q0 < nq; q0 += B * NT) {
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int q = q0 + tid + u * NT;
            ob[u] = q < nq ? load4(po, q) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const int q = q0 + tid + u * NT;
            if (q < nq) acc += sw[q / D4] * ob[u];
        }
    }
    // W = sum over prefix slots of w_s W_s.  Thread t holds column group t % (r/4):
    // reduce over the lanes of a wave that share it (xor shuffles), then over
    // the waves through LDS, in a fixed order.
    f32x4 wacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int q = tid + u * NT;
        if (q < nqw) wacc += sw[q / R4] * wb[u];
    }
    for (int q = tid + 2 * NT; q < nqw; q += NT) wacc += sw[q / R4] * load4(pw, q);
    if (wres) {
#pragma unroll
        for (int e = 0; e < 4; ++e) wacc[e] = lane_group_sum(wacc[e], R4);
        if (lane < R4) s_wp[wv * R4 + lane] = wacc;
    }
    // O: column group t % (d/4); lanes l and l ^ 32 share it (d/4 = 32) or
    // l, l ^ 16, l ^ 32, l ^ 48 (d/4 = 16)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = lane_group_sum(acc[e], D4);
    if (lane < D4) s_o[wv * D4 + lane] = acc;
    __syncthreads();
    if (wres && tid < r) {
        float x = 0.0f;
#pragma unroll
        for (int i = 0; i < NWV; ++i) x += s_wp[i * R4 + (tid >> 2)][tid & 3];
        s_wt[tid] = x;
    }
    __syncthreads();
    // (W Bv) over this thread's rows j of Bv, for its 8 columns; summed over the
    // lanes of a wave that share the columns (xor shuffles), then over the waves
    float wbv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wbv[i] = 0.0f;
    if (wres) {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int j = tid / CPR + RPR * u;
            if (j < r) {
                const float wj = s_wt[j];
#pragma unroll
                for (int i = 0; i < 8; ++i) wbv[i] += wj * (float)bvr[u].e[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) wbv[i] = lane_group_sum(wbv[i], CPR);
    }
    if (lane < CPR)
#pragma unroll
        for (int i = 0; i < 8; ++i) s_wbv[wv * D + 8 * lane + i] = wbv[i];
    __syncthreads();

    // o[d] for d = tid (< D)
    float o = 0.0f;
    if (tid < D) {
        const int c4 = tid >> 2, e = tid & 3;
#pragma unroll
        for (int i = 0; i < NWV; ++i) o += s_o[i * D4 + c4][e];
    }
    if (p.vq3) {
        // 3-bit values were decoded in the rotated coordinates: o <- H_d o (Sylvester
        // order, entries +-1), the stride-64 butterfly through LDS, strides 32 .. 1
        // between lanes (pair j, j ^ h: the lower index takes a + b, the upper a - b)
        if (tid < D) s_fw[tid] = o;
        __syncthreads();
        if (tid < D) {
            if constexpr (D == 128) {
                const float lo = s_fw[tid & 63], hi = s_fw[(tid & 63) | 64];
                o = tid < 64 ? lo + hi : lo - hi;
            }
#pragma unroll
            for (int hh = 32; hh >= 1; hh >>= 1) {
                const float u = __shfl_xor(o, hh);
                o = (lane & hh) ? u - o : o + u;
            }
        }
    }
    if (tid < D) {
        if (wres)
#pragma unroll
            for (int i = 0; i < NWV; ++i) o += s_wbv[i * D + tid];
        p.out[(int64_t)R * D + tid] = o / Lsum;  // R * D reaches 2^35 within the row limit
        if (tid == 0 && p.lse) p.lse[R] = (M + __builtin_log2f(Lsum)) * 0.69314718055994530942f;
    }
}

// ---------------------------------------------------------------- launchers --

template <typename T, int D, int CP, bool M, int W, bool Q, bool V>
struct SplitSlot {};

template <typename T, int D, int CP, bool M, int W, bool Q = false, bool V = false>
static hipError_t launch_split_w(const DecodeParams &dp, size_t lds, hipStream_t st) {
    auto *fn = decode_split_kernel<T, D, CP, M, W, Q, V>;
    const hipError_t e = ensure_lds<SplitSlot<T, D, CP, M, W, Q, V>>(reinterpret_cast<const void *>(fn), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(8 * dp.per_xcd), dim3(64 * (dp.nw + dp.np)), lds, st, dp);
    return hipGetLastError();
}

// Only the instantiations that fit in registers (split_ok, split_wide_ok) exist;
// the planner never asks for another.
template <typename T, int D, int CP, bool M, bool Q = false, bool V = false>
static hipError_t launch_split(const DecodeParams &dp, size_t lds, hipStream_t st) {
    constexpr bool kBf = sizeof(T) == 2;
    if constexpr (!split_ok(kBf, D, CP) || (Q && (!kBf || D != 128))) {
        return hipErrorInvalidValue;
    } else {
        if (dp.nw + dp.np <= 8) return launch_split_w<T, D, CP, M, 8, Q, V>(dp, lds, st);
        if constexpr (split_wide_ok(kBf, D, CP))
            return launch_split_w<T, D, CP, M, 12, Q, V>(dp, lds, st);
        else
            return hipErrorInvalidValue;
    }
}

template <typename T>
static hipError_t launch_split_t(const DecodeParams &dp, int D, int cpad, size_t lds, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        if (dp.kq8 && dp.vq3) {  // int8 keys and 3-bit values: d = 128 only
            if (D != 128) return hipErrorInvalidValue;
            if (dp.masked) {
                switch (cpad) {
                    case 32: return launch_split<T, 128, 32, true, true, true>(dp, lds, st);
                    case 64: return launch_split<T, 128, 64, true, true, true>(dp, lds, st);
                    default: return launch_split<T, 128, 128, true, true, true>(dp, lds, st);
                }
            }
            switch (cpad) {
                case 0: return launch_split<T, 128, 0, false, true, true>(dp, lds, st);
                case 32: return launch_split<T, 128, 32, false, true, true>(dp, lds, st);
                case 64: return launch_split<T, 128, 64, false, true, true>(dp, lds, st);
                default: return launch_split<T, 128, 128, false, true, true>(dp, lds, st);
            }
        }
        if (dp.kq8) {  // int8 base keys: d = 128 only
            if (D != 128) return hipErrorInvalidValue;
            if (dp.masked) {
                switch (cpad) {
                    case 32: return launch_split<T, 128, 32, true, true>(dp, lds, st);
                    case 64: return launch_split<T, 128, 64, true, true>(dp, lds, st);
                    default: return launch_split<T, 128, 128, true, true>(dp, lds, st);
                }
            }
            switch (cpad) {
                case 0: return launch_split<T, 128, 0, false, true>(dp, lds, st);
                case 32: return launch_split<T, 128, 32, false, true>(dp, lds, st);
                case 64: return launch_split<T, 128, 64, false, true>(dp, lds, st);
                default: return launch_split<T, 128, 128, false, true>(dp, lds, st);
            }
        }
        if (dp.masked) {  // per-agent caches of rank cpad >= 32, several agents per block
            if (D == 128) {
                switch (cpad) {
                    case 32: return launch_split<T, 128, 32, true>(dp, lds, st);
                    case 64: return launch_split<T, 128, 64, true>(dp, lds, st);
                    default: return launch_split<T, 128, 128, true>(dp, lds, st);
                }
            }
            switch (cpad) {
                case 32: return launch_split<T, 64, 32, true>(dp, lds, st);
                case 64: return launch_split<T, 64, 64, true>(dp, lds, st);
                default: return launch_split<T, 64, 128, true>(dp, lds, st);
            }
        }
    }
    if (D == 128) {
        switch (cpad) {
            case 0: return launch_split<T, 128, 0, false>(dp, lds, st);
            case 32: return launch_split<T, 128, 32, false>(dp, lds, st);
            case 64: return launch_split<T, 128, 64, false>(dp, lds, st);
            default: return launch_split<T, 128, 128, false>(dp, lds, st);
        }
    }
    switch (cpad) {
        case 0: return launch_split<T, 64, 0, false>(dp, lds, st);
        case 32: return launch_split<T, 64, 32, false>(dp, lds, st);
        case 64: return launch_split<T, 64, 64, false>(dp, lds, st);
        default: return launch_split<T, 64, 128, false>(dp, lds, st);
    }
}

template <typename T>
static hipError_t launch_combine_t(const DecodeParams &dp, int D, hipStream_t st) {
    const int64_t rows = (int64_t)dp.N * dp.QL * dp.HQ;
    const dim3 grid((unsigned)rows);
    if (D == 128)
        hipLaunchKernelGGL((combine_kernel<T, 128>), grid, dim3(kCombineThreads), 0, st, dp);
    else
        hipLaunchKernelGGL((combine_kernel<T, 64>), grid, dim3(kCombineThreads), 0, st, dp);
    return hipGetLastError();
}

// ------------------------------------------------------ static scratch --
//
// The split partials of rattn_decode_noalloc live here instead of in a caller
// workspace.  Each GPU the library runs on holds its own copy of the array,
// at its own address, until the process ends.  On the host the name `scratch`
// is only a stand-in for the symbol, not a device address: host code uses the
// address hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
    static std::atomic<void *> addr[64];
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> g(mu);
        p = addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            addr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

hipError_t launch_decode(int bf16_in, const DecodeParams &dp, int D, int cpad, size_t lds, unsigned stages,
                         hipStream_t st) {
    hipError_t e = hipSuccess;
    if (stages & 1u) {
        e = bf16_in ? launch_split_t<bf16>(dp, D, cpad, lds, st) : launch_split_t<float>(dp, D, cpad, lds, st);
        if (e != hipSuccess) return e;
    }
    if (stages & 2u) e = bf16_in ? launch_combine_t<bf16>(dp, D, st) : launch_combine_t<float>(dp, D, st);
    return e;
}

}  // namespace rattn
