// recon.hip -- decode with each agent's residual keys rebuilt in registers
// right before the score product (gfx950).
//
// This is the ForkKV Guide's own kernel design ("Fused ResidualAttention",
// section 2, On-the-Fly Register Fusion: base and residual keys are streamed
// and added in registers immediately before the matrix product).  The main
// decode path keeps the residual factored instead (score correction
// (q Bk^T) Lk^T, one base tile shared by every agent's rows in one MFMA); that
// factoring no longer holds once keys are rotated by position after the
// up-projection (rotary position embedding), because then the residual key of
// token j is rot_j(Lk_j Bk).  Here, per agent and 16-token step:
//   dK^T = Bk^T Lk^T                 (MFMA, 16 d-rows x 16 tokens per tile)
//   dK   = rot_j(dK)                 (rotate-half pairs (f, f + d/2), optional)
//   S^T  = K_base Q^T + dK Q^T       (dK as bf16 hi + lo halves)
// then the same online softmax and value products as the main path (the value
// residual keeps its factored form P Lv, Bv applied once per row in the
// merge, since values are not rotated).
//
// The output of the dK^T product leaves lane (n, j) holding d = 16 t + 4 j + i
// (i < 4) of token n for d-tile t, which is not the A-operand layout of the
// score product (8 consecutive d per lane).  The contraction does not care
// about the order of its terms as long as both operands use the same one, so
// the score takes its d slots in the order {32 s + 4 j + i, 32 s + 16 + 4 j + i}
// for step s: exactly what the lane holds for d-tiles 2s and 2s + 1, and what
// it reads of the base keys (two 8-byte LDS reads) and of the query row.  No
// transpose through LDS.  The rotation pairs d and d + 64 are d-tiles t and
// t + 4 of the same lane.
//
// Each workgroup stages the split's base keys and values and the low-rank rows
// of its agents through an LDS ring (direct loads, every wave filling 16-row
// groups of some regions), so the base tile is read from HBM once for up to
// eight agents.  An agent's rows take tg waves (token groups), which share out
// the stage's 16-token steps (wave tg_i takes steps tg_i, tg_i + tg, ...) and
// each keep their own softmax state, written as partial slot split * tg + tg_i:
// two waves per SIMD hide the long dependent chain of a step (rank product,
// conversion, score, softmax, value products); with the rotation at rank 32
// its state leaves room for one wave per SIMD (four waves).  Partials go to the decode
// workspace layout and the decode merge kernel finishes the call.
#include "device.h"
#include "internal.h"
#include "stage.h"

namespace rattn {

// sin and cos of 2 pi x for x in revolutions (gfx950's v_sin_f32 / v_cos_f32)
__device__ inline float sin_rev(float x) { return __builtin_amdgcn_sinf(x); }
__device__ inline float cos_rev(float x) { return __builtin_amdgcn_cosf(x); }

// fractional revolutions of pos * theta (theta in radians), formed in fp64
__device__ inline float rev_of(double pos, float theta) {
    const double r = pos * ((double)theta * 0.15915494309189533577);  // / (2 pi)
    return (float)(r - __builtin_floor(r));
}

template <int R, bool ROPE>
__global__ __launch_bounds__(64 * recon_waves(ROPE, R)) void recon_split_kernel(ReconParams p) {
    constexpr int D = 128, KS = D / 32, VPL = D / 16, ES = 2;
    constexpr int CPL = R / 16;  // residual column tiles of W
    const int T = p.T;
    using O = Ops<bf16>;
    using frag = O::frag;
    using frag4 = O::frag4;

    extern __shared__ __attribute__((aligned(16))) char smem[];
    touch_params<ReconParams>();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n16 = lane & 15, j4 = lane >> 4;

    // items: agent group fastest, then KV head, then split, so that the agent
    // groups of one (head, split) run back to back on one XCD and share its L2
    const int bid = blockIdx.x;
    const int li = (bid & 7) * p.per_xcd + (bid >> 3);
    if (li >= p.n_items) return;
    const int ag = li % p.n_ag, rest = li / p.n_ag;
    const int k = rest % p.HK, sp = rest / p.HK;
    const int a0 = ag * p.apg;
    const int na = p.N - a0 < p.apg ? p.N - a0 : p.apg;
    const int t0 = sp * p.tok_split;
    int t1 = t0 + p.tok_split < p.L ? t0 + p.tok_split : (int)p.L;
    if (t1 < t0) t1 = t0;
    const int wa = small_div(wave, p.tg), tgi = wave - wa * p.tg;  // this wave's agent (in the group), token group
    const int a = a0 + wa;
    const bool active = wa < na;

    // ---- stage geometry: one head's K and V rows, the agents' Lk and Lv rows
    Geo g;
    g.T = T;
    g.nst = p.nst;
    g.stage_bytes = p.stage_bytes;
    g.cpr_kv = D * ES / 16;
    g.lg_kv = ilog2(g.cpr_kv);
    g.cpr_k = g.cpr_kv;
    g.lg_k = g.lg_kv;
    g.cpa_lr = R * ES / 16;
    g.lg_lr = ilog2(g.cpa_lr);
    g.na_lr = p.shared_lr ? 1 : na;
    g.lr_grp = 16 * g.na_lr * g.cpa_lr;
    g.H = 1;
    g.ofs_v = T * g.cpr_kv;
    g.ofs_lk = 2 * T * g.cpr_kv;
    g.ofs_lv = g.ofs_lk + (T >> 4) * g.lr_grp;
    g.chunks = g.ofs_lv + (T >> 4) * g.lr_grp;

    Src<bf16> src;
    src.kb = static_cast<const bf16 *>(p.kb) + (int64_t)k * p.L * D;
    src.vb = static_cast<const bf16 *>(p.vb) + (int64_t)k * p.L * D;
    src.head_stride = p.L * D;
    src.page_stride = 0;
    src.k_head_stride = p.L * D;
    src.k_page_stride = 0;
    src.fps = FastDiv{((uint64_t)1 << 32) + 1, 32, 1};  // unused: contiguous rows
    src.pg0 = 0;
    src.pages = nullptr;
    const int64_t a_lr = p.shared_lr ? 0 : a0;
    src.lk = static_cast<const bf16 *>(p.lk) + a_lr * p.L * R;
    src.lv = static_cast<const bf16 *>(p.lv) + a_lr * p.L * R;
    src.lr_agent_stride = p.L * R;
    src.r = R;
    src.tlast = t1 > t0 ? t1 - 1 : t0;

    GroupFill fp;
    make_group_fill<bf16, D>(fp, g, src, true, wave, lane, recon_waves(ROPE, R));  // a multiple of T / 16
    const int n_tiles = (t1 - t0 + T - 1) / T;
    const int fpw = fp.fpw;
    auto fill = [&](int tile, int stage) {
        const int tt = t0 + tile * T;
        fill_group<bf16, D>(fp, g, src, tt, smem + (size_t)stage * g.stage_bytes, tt + T - 1 > src.tlast, lane);
    };
    for (int i = 0; i < g.nst - 1 && i < n_tiles; ++i) fill(i, i);

    // ---- this lane's query row (column n16 of the score tile) and operands
    const int rpa = p.rpa;
    const bool vm = active && n16 < rpa;
    const int ria = vm ? n16 : 0;
    const int tq = ria / p.g, hh = ria - tq * p.g;
    const int64_t qrow = ((int64_t)(active ? a : 0) * p.QL + tq) * p.HQ + (int64_t)k * p.g + hh;
    // query row, d slots {32 s + 4 j4 + i, 32 s + 16 + 4 j4 + i}
    frag qB[KS];
    {
        const bf16 *qp = static_cast<const bf16 *>(p.q) + qrow * D + 4 * j4;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (vm) {
                __builtin_memcpy(&w[0], __builtin_assume_aligned(qp + 32 * s, 8), 8);
                __builtin_memcpy(&w[2], __builtin_assume_aligned(qp + 32 * s + 16, 8), 8);
            }
            __builtin_memcpy(&qB[s], w, 16);
        }
    }
    // Bk^T as the A operand of dK^T = Bk^T Lk^T: d-row 16 t + n16, rank slots
    // 4 j4 .. + 3 (R = 16, 16x16x16 product) or 8 j4 .. + 7 (R = 32, 16x16x32)
    constexpr int BS = R == 16 ? 4 : 8;
    typedef bf16 bkvec __attribute__((ext_vector_type(BS)));
    bkvec bkt[VPL];
    {
        const bf16 *bk = static_cast<const bf16 *>(p.bk) + (int64_t)(active ? a : 0) * R * p.HK * D +
                         (int64_t)k * D + n16;
        const int64_t ldb = (int64_t)p.HK * D;
#pragma unroll
        for (int t = 0; t < VPL; ++t)
#pragma unroll
            for (int i = 0; i < BS; ++i) bkt[t][i] = bk[(int64_t)(BS * j4 + i) * ldb + 16 * t];
    }
    // rotation state: cos / sin of this wave's next token (t0 + 16 tgi + n16 first)
    // for f = 16 t + 4 j4 + i (t < 4), advanced by the 16 tg tokens between the
    // wave's steps with the angle-addition rule
    float cs[4][4], sn[4][4], c16[4][4], s16[4][4];
    if constexpr (ROPE) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float th = p.theta[16 * t + 4 * j4 + i];
                const float r0 = rev_of((double)(t0 + 16 * tgi + n16), th), r16 = rev_of(16.0 * p.tg, th);
                cs[t][i] = cos_rev(r0);
                sn[t][i] = sin_rev(r0);
                c16[t][i] = cos_rev(r16);
                s16[t][i] = sin_rev(r16);
            }
    }
    wait_vmcnt(0);  // every register load (and the first stages) landed

    // LDS read offsets (relative to a step's first row): base keys in the d
    // order above, transposed value reads, this agent's Lk and Lv rows
    uint32_t ko[KS][2];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        ko[s][0] = elem_ofs(0, n16, ES * (32 * s + 4 * j4), g.cpr_kv, g.lg_kv);
        ko[s][1] = elem_ofs(0, n16, ES * (32 * s + 16 + 4 * j4), g.cpr_kv, g.lg_kv);
    }
    uint32_t vtr[VPL];
#pragma unroll
    for (int jj = 0; jj < VPL; ++jj)
        vtr[jj] = elem_ofs(g.ofs_v, 4 * j4 + (n16 >> 2), ES * (16 * jj + 4 * (n16 & 3)), g.cpr_kv, g.lg_kv);
    const int la = p.shared_lr ? 0 : wa;  // this agent among the staged low-rank rows
    const uint32_t lko = lr_ofs(g, 0, la, n16, ES * BS * j4);  // rank slots of token n16
    uint32_t wtr[CPL];
#pragma unroll
    for (int jj = 0; jj < CPL; ++jj) wtr[jj] = lr_ofs(g, 0, la, 4 * j4 + (n16 >> 2), ES * (16 * jj + 4 * (n16 & 3)));

    f32x4 o[VPL], w[CPL], ls = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < VPL; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < CPL; ++i) w[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -1.0e30f;
    const float cl2 = p.c;

    for (int it = 0; it < n_tiles; ++it) {
        const int later = (n_tiles - 1 - it) < (g.nst - 2) ? (n_tiles - 1 - it) : (g.nst - 2);
        wait_vmcnt(later * fpw);
        ring_barrier();
        if (it + g.nst - 1 < n_tiles) fill(it + g.nst - 1, (it + g.nst - 1) % g.nst);
        if (!active) continue;
        const char *st = smem + (size_t)(it % g.nst) * g.stage_bytes;
        const int tt = t0 + it * T;
#pragma unroll 1
        for (int u = tgi; u < (T >> 4); u += p.tg) {
            const char *kvb = st + 16 * u * D * ES;
            const char *lkb = st + 16 * (g.ofs_lk + u * g.lr_grp);
            const char *lvb = st + 16 * (g.ofs_lv + u * g.lr_grp);
            const int tok = tt + 16 * u;
            // dK^T for the step's 16 tokens
            f32x4 dk[VPL];
            {
                bkvec lt;
                __builtin_memcpy(&lt, __builtin_assume_aligned(lkb + lko, 2 * BS), 2 * BS);
#pragma unroll
                for (int t = 0; t < VPL; ++t) {
                    if constexpr (R == 16)
                        dk[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bkt[t], lt, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                           0);
                    else
                        dk[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bkt[t], lt, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                         0);
                }
            }
            if constexpr (ROPE) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x1 = dk[t][i], x2 = dk[t + 4][i], c = cs[t][i], s = sn[t][i];
                        dk[t][i] = x1 * c - x2 * s;
                        dk[t + 4][i] = x2 * c + x1 * s;
                        cs[t][i] = c * c16[t][i] - s * s16[t][i];
                        sn[t][i] = s * c16[t][i] + c * s16[t][i];
                    }
            }
            // S^T = K_base Q^T + dK Q^T (dK as bf16 hi + lo), two accumulator chains
            f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                frag kf, dh, dl;
                __builtin_memcpy(&kf, __builtin_assume_aligned(kvb + ko[s][0], 8), 8);
                __builtin_memcpy(reinterpret_cast<char *>(&kf) + 8, __builtin_assume_aligned(kvb + ko[s][1], 8), 8);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x0 = dk[2 * s][i], x1 = dk[2 * s + 1][i];
                    const bf16 h0 = (bf16)x0, h1 = (bf16)x1;
                    dh.v[i] = h0;
                    dh.v[4 + i] = h1;
                    dl.v[i] = (bf16)(x0 - (float)h0);
                    dl.v[4 + i] = (bf16)(x1 - (float)h1);
                }
                acc = O::mma(kf, qB[s], acc);
                acc2 = O::mma(dh, qB[s], acc2);
                acc = O::mma(dl, qB[s], acc);
            }
            acc += acc2;
            if (tok + 16 > t1) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok + 4 * j4 + i >= t1) acc[i] = -__builtin_inff();
            }
            // online softmax (log2 domain) and the value products, as the main path
            bf16x4 va[VPL];
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) va[jj] = lds_tr4(kvb + vtr[jj]);
            bf16x4 wa[CPL];
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) wa[jj] = lds_tr4(lvb + wtr[jj]);
            // the cross-lane maximum only where some lane's own passes the slack
            const float lmx = amax3(acc[0], acc[1], amax(acc[2], acc[3]));
            if (__builtin_amdgcn_ballot_w64(lmx * cl2 > m + kRescaleSlack)) {
                const float mx = row_max4(lmx) * cl2;
                const bool grow = mx > m + kRescaleSlack;
                const float m_new = grow ? mx : m;
                const float alpha = fexp2(m - m_new);
                m = m_new;
#pragma unroll
                for (int i = 0; i < VPL; ++i) o[i] *= alpha;
#pragma unroll
                for (int i = 0; i < CPL; ++i) w[i] *= alpha;
                ls *= alpha;
            }
            frag4 pB;
            pB.v = to_bf16x4(fexp2(__builtin_fmaf(acc[0], cl2, -m)), fexp2(__builtin_fmaf(acc[1], cl2, -m)),
                             fexp2(__builtin_fmaf(acc[2], cl2, -m)), fexp2(__builtin_fmaf(acc[3], cl2, -m)));
            {
                frag4 ones;
                ones.v = bf16x4{(bf16)1.0f, (bf16)1.0f, (bf16)1.0f, (bf16)1.0f};
                ls = O::mma16(ones, pB, ls);
            }
#pragma unroll
            for (int jj = 0; jj < VPL; ++jj) {
                frag4 vA;
                vA.v = va[jj];
                o[jj] = O::mma16(vA, pB, o[jj]);
            }
#pragma unroll
            for (int jj = 0; jj < CPL; ++jj) {
                frag4 wA;
                wA.v = wa[jj];
                w[jj] = O::mma16(wA, pB, w[jj]);
            }
        }
    }

    // ---- partials of this agent's rows (split sp, token group tgi): O and W divided
    // by the weight sum, as fp16 (zeros when no token was visible)
    if (vm) {
        const int64_t rec = ((int64_t)k * p.N * rpa + (int64_t)a * rpa + ria) * p.n_slots + sp * p.tg + tgi;
        const float inv_l = ls[0] > 0.0f ? 1.0f / ls[0] : 0.0f;
        f16 *po = static_cast<f16 *>(p.p_o) + rec * D + 4 * j4;
#pragma unroll
        for (int jj = 0; jj < VPL; ++jj) *reinterpret_cast<f16x4 *>(po + 16 * jj) = to_f16x4(o[jj] * inv_l);
        f16 *pw = static_cast<f16 *>(p.p_w) + rec * R + 4 * j4;
#pragma unroll
        for (int jj = 0; jj < CPL; ++jj) *reinterpret_cast<f16x4 *>(pw + 16 * jj) = to_f16x4(w[jj] * inv_l);
        if (j4 == 0) *reinterpret_cast<float2 *>(p.p_ml + rec * 2) = float2{m, ls[0]};
    }
}

template <int R, bool ROPE>
struct ReconSlot {};

template <int R, bool ROPE>
static hipError_t launch_recon_one(const ReconParams &p, hipStream_t st) {
    auto *fn = recon_split_kernel<R, ROPE>;
    const size_t lds = (size_t)p.nst * p.stage_bytes;
    const hipError_t e = ensure_lds<ReconSlot<R, ROPE>>(reinterpret_cast<const void *>(fn), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3(8 * p.per_xcd), dim3(64 * recon_waves(ROPE, R)), lds, st, p);
    return hipGetLastError();
}

hipError_t launch_recon(const ReconParams &p, hipStream_t st) {
    const bool rope = p.theta != nullptr;
    if (p.r == 16) return rope ? launch_recon_one<16, true>(p, st) : launch_recon_one<16, false>(p, st);
    return rope ? launch_recon_one<32, true>(p, st) : launch_recon_one<32, false>(p, st);
}

}  // namespace rattn
