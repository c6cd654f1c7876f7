// gdn_prefill.hip -- chunk-64 prefill of the gated delta rule on gfx950.
//
// The token recurrence (S in R^{Dv x Dk}; q/k head g = h / (Hv/Hk))
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
// is evaluated 64 tokens at a time through an exact rewrite. Inside a chunk
// with start state S let g_t = sum_{s<=t} ln a_s (chunk-local, so every
// exponent below is g_t - g_s with t >= s and no factor exceeds 1),
// gamma_t = e^{g_t}, and
//     A_ts = b_t e^{g_t - g_s} (k_t . k_s)   for s < t,   T = (I + A)^{-1}
//     P_ts = e^{g_t - g_s} (q_t . k_s)       for s <= t
// Then, with R = diag(b) (V - diag(gamma) K S^T),
//     U     = T R                 (row t of U is b_t (v_t - a_t S_{t-1} k_t))
//     O^T   = S Q^T diag(gamma) + U^T P^T
//     S_end = gamma_C S + U^T diag(e^{g_C - g}) K
//
// Work decomposition. One workgroup owns one (sequence, value head, slice of
// DVS value columns) and walks that sequence's chunks in order; the rows of S
// it owns evolve independently of the other rows, so slices never talk to
// each other. Wave w owns DVW value columns and keeps S^T for them in MFMA
// accumulators (fp32) for the whole call. The state-free part of a chunk
// (Gram products, decay, T, P) is computed cooperatively and shared through
// LDS.
//
// Per chunk (barriers marked |):
//   | stage   registers -> LDS: K, Q row-major, K^T and V^T (bf16) or V
//             (fp32). Wave 0 turns its alpha/beta registers into the
//             chunk-local log decay. The next chunk's global loads are then
//             issued into registers so their latency overlaps this chunk.
//             Rows past the end of the sequence are staged as k = q = v = 0,
//             alpha = 1, beta = 0, which leaves the recurrence unchanged.
//   | gram    (K K^T)^T and (Q K^T)^T lower 16x16 tiles on MFMA; the decay
//             masks are applied in registers and A (fp32) / P rows written.
//   | solve   wave 0: T = (I + A)^{-1} (forward substitution on the four
//             16x16 diagonal blocks, one lane per column; block rows 1..3 on
//             MFMA with the finished blocks kept in registers). The other
//             waves meanwhile form K S^T and S Q^T for their columns.
//   | chain   R, U = T R, O^T += U^T P^T, store O, state update, all on MFMA
//             with fp32 accumulation.
#include <float.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kC = 64;  // chunk length

template <typename DT, int D, int NW, int DVW> struct PrefillCfg {
    static constexpr int NTH = NW * 64;
    static constexpr int DVS = NW * DVW;  // value columns per workgroup
    static constexpr int NKT = D / 16;    // key-dim tiles of S^T
    static constexpr int NB = DVW / 16;   // value-dim tiles per wave
    static constexpr int KS = D / 32;     // 32-deep steps over the key dim
    static constexpr bool BF = sizeof(DT) == 2;
    static constexpr int EPP = 16 / (int)sizeof(DT);  // elements per 16-byte piece
    static constexpr int PK = D + (BF ? 8 : 4);       // row pitch of K, Q
    static constexpr int PT = kC + 4;                 // row pitch of T, P, K^T, V^T
    static constexpr int PV = DVS + 4;                // row pitch of V (fp32 path)
    static constexpr int PA = kC + 4;                 // row pitch of fp32 A and E
    static constexpr int SZ_K = kC * PK * (int)sizeof(DT);
    static constexpr int SZ_KT = BF ? D * PT * 2 : 0;
    static constexpr int SZ_V = BF ? DVS * PT * 2 : kC * PV * 4;
    static constexpr int SZ_T = kC * PT * (int)sizeof(DT);
    static constexpr int SZ_A = kC * PA * 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_K;
    static constexpr int OFF_KT = OFF_Q + SZ_K;
    static constexpr int OFF_V = OFF_KT + SZ_KT;
    static constexpr int OFF_T = OFF_V + SZ_V;
    static constexpr int OFF_P = OFF_T + SZ_T;
    static constexpr int OFF_A = OFF_P + SZ_T;
    static constexpr int OFF_E = OFF_A + SZ_A;
    static constexpr int OFF_VEC = OFF_E + SZ_A;  // g, gamma, dec, beta: 4 x 64 floats
    static constexpr int LDS = OFF_VEC + 4 * kC * 4;
    // staging tasks: one task is one 16-byte piece of two consecutive rows
    static constexpr int PPR_K = D / EPP;
    static constexpr int PPR_V = DVS / EPP;
    static constexpr int TK = 32 * PPR_K;
    static constexpr int TV = 32 * PPR_V;
    static constexpr int NTK = (TK + NTH - 1) / NTH;
    static constexpr int NTV = (TV + NTH - 1) / NTH;
    static_assert(DVW % 16 == 0 && D % 32 == 0, "tile shapes");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// Task -> (row pair, piece). Within 64 consecutive tasks the row pair varies
// fastest over 16 (or 32) values, so the transposed LDS writes of a wave
// spread over all banks while each wave still reads whole 64-byte row
// segments from global memory.
template <int PPR>
__device__ __forceinline__ void task_coords(int task, int &rp, int &pc) {
    constexpr int PCB = PPR < 4 ? PPR : 4;  // pieces per 64-task group
    constexpr int RPB = 64 / PCB;           // row pairs per 64-task group
    constexpr int NRB = 32 / RPB;           // row-pair blocks
    const int li = task & 63, grp = task >> 6;
    rp = (li % RPB) + RPB * (grp % NRB);
    pc = (li / RPB) + PCB * (grp / NRB);
}

// Two rows (lo = row r, hi = row r+1) of 8 bf16 each, written transposed:
// column j of the pair goes to dst[j * PT .. +1] as one 32-bit word.
template <int PT>
__device__ __forceinline__ void store_pair_transposed(__bf16 *dst, const u32x4 &l, const u32x4 &h) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        *reinterpret_cast<uint32_t *>(dst + (2 * w) * PT) = (l[w] & 0xFFFFu) | (h[w] << 16);
        *reinterpret_cast<uint32_t *>(dst + (2 * w + 1) * PT) = (l[w] >> 16) | (h[w] & 0xFFFF0000u);
    }
}
template <int PT>
__device__ __forceinline__ void store_pair_transposed(float *, const u32x4 &, const u32x4 &) {}

// Lower 16x16 tile pairs (ti, tj), tj <= ti, of a 64x64 chunk matrix.
__device__ __forceinline__ constexpr int pair_i(int pr) {
    return pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
}
__device__ __forceinline__ constexpr int pair_j(int pr) { return pr - pair_i(pr) * (pair_i(pr) + 1) / 2; }

template <typename DT, int D, int NW, int DVW>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillParams p, int nsplit,
                                                          int remap_xcd) {
    using Cf = PrefillCfg<DT, D, NW, DVW>;
    constexpr int NTH = Cf::NTH, NKT = Cf::NKT, NB = Cf::NB, KS = Cf::KS;
    constexpr int PK = Cf::PK, PT = Cf::PT, PV = Cf::PV, PA = Cf::PA;
    constexpr bool BF = Cf::BF;
    using F = Frag<DT>;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS];
    DT *sK = reinterpret_cast<DT *>(smem + Cf::OFF_K);
    DT *sQ = reinterpret_cast<DT *>(smem + Cf::OFF_Q);
    DT *sKT = reinterpret_cast<DT *>(smem + Cf::OFF_KT);  // bf16 only: [D][PT]
    DT *sV = reinterpret_cast<DT *>(smem + Cf::OFF_V);    // bf16: V^T [DVS][PT]; fp32: V [kC][PV]
    DT *sT = reinterpret_cast<DT *>(smem + Cf::OFF_T);
    DT *sP = reinterpret_cast<DT *>(smem + Cf::OFF_P);
    float *sA = reinterpret_cast<float *>(smem + Cf::OFF_A);
    float *sE = reinterpret_cast<float *>(smem + Cf::OFF_E);
    float *sG = reinterpret_cast<float *>(smem + Cf::OFF_VEC);
    float *sGam = sG + kC;
    float *sDec = sG + 2 * kC;
    float *sBeta = sG + 3 * kC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    // ---- which (sequence, value head, slice) this workgroup owns
    int wg = blockIdx.x;
    if (remap_xcd) {
        // Workgroups are dispatched to the 8 XCDs round-robin; give each XCD
        // a contiguous range of logical ids so that the value heads (and
        // slices) sharing one q/k head share that XCD's L2.
        const int per = (int)(gridDim.x >> 3);
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int slice = wg % nsplit;
    const int nh = wg / nsplit;
    const int h = nh % p.Hv;
    const int n = nh / p.Hv;
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    if (p.cu_seqlens) {
        tok0 = p.cu_seqlens[n];
        len = (int64_t)p.cu_seqlens[n + 1] - tok0;
    } else {
        tok0 = (int64_t)n * p.seq_len;
        len = p.seq_len;
    }
    const int dv0 = slice * Cf::DVS;
    const int wdv = wave * DVW;  // this wave's first column inside the slice

    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const DT *qh = reinterpret_cast<const DT *>(p.q) + tok0 * sQK + (int64_t)grp * D;
    const DT *kh = reinterpret_cast<const DT *>(p.k) + tok0 * sQK + (int64_t)grp * D;
    const DT *vh = reinterpret_cast<const DT *>(p.v) + tok0 * sVO + (int64_t)h * D + dv0;
    DT *oh = reinterpret_cast<DT *>(p.out) + tok0 * sVO + (int64_t)h * D + dv0 + wdv;
    const float *ah = p.alpha + tok0 * p.Hv + h;
    const float *bh = p.beta + tok0 * p.Hv + h;

    // Upper blocks of T and P are never written: clear both once.
    for (int i = tid; i < 2 * Cf::SZ_T / 4; i += NTH)
        reinterpret_cast<float *>(smem + Cf::OFF_T)[i] = 0.f;

    // ---- state S^T for this wave's columns: st[a][b] = S^T tile (dk a, dv b)
    f32x4 st[NKT][NB];
    {
        const float *s0 = p.s0 ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                st[a][b] = s0 ? *reinterpret_cast<const f32x4 *>(
                                    s0 + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a + 4 * g4)
                              : zero4();
    }

    // ---- staging: per-thread task coordinates (fixed for the whole call)
    int kOffG[Cf::NTK], kOffL[Cf::NTK], kRow[Cf::NTK];
    int vOffG[Cf::NTV], vOffL[Cf::NTV], vRow[Cf::NTV];
#pragma unroll
    for (int i = 0; i < Cf::NTK; ++i) {
        int rp = 0, pc = 0;
        task_coords<Cf::PPR_K>(tid + i * NTH, rp, pc);
        kRow[i] = 2 * rp;
        kOffG[i] = pc * Cf::EPP;
        kOffL[i] = 2 * rp * PK + pc * Cf::EPP;
    }
#pragma unroll
    for (int i = 0; i < Cf::NTV; ++i) {
        int rp = 0, pc = 0;
        task_coords<Cf::PPR_V>(tid + i * NTH, rp, pc);
        vRow[i] = 2 * rp;
        vOffG[i] = pc * Cf::EPP;
        vOffL[i] = BF ? (pc * Cf::EPP) * PT + 2 * rp : 2 * rp * PV + pc * Cf::EPP;
    }
    u32x4 rK[Cf::NTK][2], rQ[Cf::NTK][2], rV[Cf::NTV][2];
    float rAl = 1.f, rBe = 0.f;  // wave 0: alpha, beta of token `lane` of the next chunk

    // The loads below are kept raw; rows past the end of the sequence are
    // read from a valid row and zeroed at store time, so nothing consumes
    // the loaded registers before the next chunk's store (the loads stay in
    // flight while this chunk computes).
    auto stage_load = [&](int64_t c) {
        const int64_t t0 = c * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
#pragma unroll
        for (int i = 0; i < Cf::NTK; ++i) {
            if (Cf::TK % NTH == 0 || tid + i * NTH < Cf::TK) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = kRow[i] + e;
                    const int rr = r < lenc ? r : lenc - 1;  // always a valid row
                    const int64_t off = (t0 + rr) * sQK + kOffG[i];
                    rK[i][e] = *reinterpret_cast<const u32x4 *>(kh + off);
                    rQ[i][e] = *reinterpret_cast<const u32x4 *>(qh + off);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NTV; ++i) {
            if (Cf::TV % NTH == 0 || tid + i * NTH < Cf::TV) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = vRow[i] + e;
                    const int rr = r < lenc ? r : lenc - 1;
                    rV[i][e] = *reinterpret_cast<const u32x4 *>(vh + (t0 + rr) * sVO + vOffG[i]);
                }
            }
        }
        if (wave == 0) {
            const int rr = lane < lenc ? lane : lenc - 1;
            rAl = ah[(t0 + rr) * p.Hv];
            rBe = bh[(t0 + rr) * p.Hv];
        }
    };

    const u32x4 z4 = {0u, 0u, 0u, 0u};
    auto stage_store = [&](int lenc) {
#pragma unroll
        for (int i = 0; i < Cf::NTK; ++i) {
            if (Cf::TK % NTH == 0 || tid + i * NTH < Cf::TK) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const bool ok = kRow[i] + e < lenc;
                    rK[i][e] = ok ? rK[i][e] : z4;
                    rQ[i][e] = ok ? rQ[i][e] : z4;
                    *reinterpret_cast<u32x4 *>(sK + kOffL[i] + e * PK) = rK[i][e];
                    *reinterpret_cast<u32x4 *>(sQ + kOffL[i] + e * PK) = rQ[i][e];
                }
                if constexpr (BF)  // K^T[col][row pair]: two rows per 32-bit word
                    store_pair_transposed<PT>(sKT + kOffG[i] * PT + kRow[i], rK[i][0], rK[i][1]);
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NTV; ++i) {
            if (Cf::TV % NTH == 0 || tid + i * NTH < Cf::TV) {
#pragma unroll
                for (int e = 0; e < 2; ++e) rV[i][e] = vRow[i] + e < lenc ? rV[i][e] : z4;
                if constexpr (BF) {
                    store_pair_transposed<PT>(sV + vOffL[i], rV[i][0], rV[i][1]);
                } else {
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        *reinterpret_cast<u32x4 *>(sV + vOffL[i] + e * PV) = rV[i][e];
                }
            }
        }
        if (wave == 0) {
            // chunk-local cumulative log decay: inclusive scan over the 64 lanes
            const bool ok = lane < lenc;
            const float al = ok ? rAl : 1.f;
            const float be = ok ? rBe : 0.f;
            float x = __logf(fmaxf(al, FLT_MIN));
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                x += lane >= off ? y : 0.f;
            }
            const float glast = __shfl(x, 63, 64);
            sG[lane] = x;
            sGam[lane] = __expf(x);
            sDec[lane] = __expf(glast - x);
            sBeta[lane] = be;
        }
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    if (nchunks > 0) stage_load(0);
    // Drain the initial-state and first-chunk loads here (the first store
    // needs them anyway). Without this, the state registers count as
    // possibly pending inside the loop and each chunk would wait for its own
    // prefetch before touching the state.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    for (int64_t c = 0; c < nchunks; ++c) {
        const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
        __syncthreads();  // the previous chunk is done with LDS
        stage_store(lenc);
        if (c + 1 < nchunks) stage_load(c + 1);
        __syncthreads();

        // ---- Gram tiles, transposed: X[s][t] = k_s . k_t and k_s . q_t for
        // the lower tile pair (ti, tj) (s in tile tj, t in tile ti); decay
        // masks applied in registers; rows of A (fp32) and P written.
#pragma unroll
        for (int pr = 0; pr < 10; ++pr) {
            if (pr % NW != wave) continue;
            const int ti = pair_i(pr), tj = pair_j(pr);
            f32x4 gk = zero4(), gq = zero4();
            F fks[KS], fkt[KS], fqt[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                ld_nat(sK + (16 * tj + c16) * PK + 32 * kk + 8 * g4, fks[kk]);
                ld_nat(sK + (16 * ti + c16) * PK + 32 * kk + 8 * g4, fkt[kk]);
                ld_nat(sQ + (16 * ti + c16) * PK + 32 * kk + 8 * g4, fqt[kk]);
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                gk = mma(fks[kk], fkt[kk], gk);
                gq = mma(fks[kk], fqt[kk], gq);
            }
            const int t = 16 * ti + c16;
            const float gt = sG[t];
            const float bt = sBeta[t];
            const f32x4 gs = *reinterpret_cast<const f32x4 *>(sG + 16 * tj + 4 * g4);
            f32x4 av;
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = 16 * tj + 4 * g4 + r;
                // for s > t (diagonal tiles only) the value is discarded below
                const float dec = __expf(gt - gs[r]);
                const float a = bt * dec * gk[r];
                const float pp = dec * gq[r];
                if (ti == tj) {
                    av[r] = s < t ? a : 0.f;
                    pv[r] = s <= t ? pp : 0.f;
                } else {
                    av[r] = a;
                    pv[r] = pp;
                }
            }
            *reinterpret_cast<f32x4 *>(sA + t * PA + 16 * tj + 4 * g4) = av;
            if constexpr (BF) {
                bf16x4 pb;
#pragma unroll
                for (int r = 0; r < 4; ++r) pb[r] = (__bf16)pv[r];
                *reinterpret_cast<bf16x4 *>(sP + t * PT + 16 * tj + 4 * g4) = pb;
            } else {
                *reinterpret_cast<f32x4 *>(sP + t * PT + 16 * tj + 4 * g4) =
                    f32x4{pv[0], pv[1], pv[2], pv[3]};
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1} on wave 0
        if (wave == 0) {
            // diagonal blocks E_b = (I + A_bb)^{-1}: lane = 16 b + column. Rows
            // are solved four at a time; a batch's rows of A are read before
            // any of its arithmetic so that one LDS latency covers the batch.
            {
                const int blk = g4, col = c16;
                const float *ab = sA + (16 * blk) * PA + 16 * blk;
                float x[16];
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    f32x4 arow[4][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int m4 = 0; m4 <= rb; ++m4)
                            arow[i][m4] = *reinterpret_cast<const f32x4 *>(ab + (4 * rb + i) * PA + 4 * m4);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = 4 * rb + i;
                        float acc = r == col ? 1.f : 0.f;
#pragma unroll
                        for (int m = 0; m < r; ++m) acc -= arow[i][m >> 2][m & 3] * x[m];
                        x[r] = acc;
                    }
                }
                float *eb = sE + (16 * blk) * PA + 16 * blk + col;
                DT *tb = sT + (16 * blk) * PT + 16 * blk + col;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    eb[r * PA] = x[r];
                    tb[r * PT] = from_f32<DT>(x[r]);
                }
            }
            // block rows 1..3: T_ij = -E_i * sum_{m=j}^{i-1} A_im T_mj, with the
            // off-diagonal T_mj kept in registers (accumulator layout).
            f32x4 Toff[4][4];
            // columns of E_0..E_2 as B operands (k = 4 g4 + e)
            float ecol[3][4];
#pragma unroll
            for (int m = 0; m < 3; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) ecol[m][e] = sE[(16 * m + 4 * g4 + e) * PA + 16 * m + c16];
#pragma unroll
            for (int ti = 1; ti < 4; ++ti) {
                f32x4 aim[3];
#pragma unroll
                for (int m = 0; m < ti; ++m)
                    aim[m] = *reinterpret_cast<const f32x4 *>(sA + (16 * ti + c16) * PA + 16 * m + 4 * g4);
                const f32x4 ev =
                    *reinterpret_cast<const f32x4 *>(sE + (16 * ti + c16) * PA + 16 * ti + 4 * g4);
#pragma unroll
                for (int tj = 0; tj < ti; ++tj) {
                    f32x4 X = zero4();
#pragma unroll
                    for (int m = tj; m < ti; ++m) {
                        float a4[4], b4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            a4[e] = aim[m][e];
                            b4[e] = m == tj ? ecol[m][e] : Toff[m][tj][e];
                        }
                        X = mma_k16(a4, b4, X, DT{});
                    }
                    float a4[4], b4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a4[e] = ev[e];
                        b4[e] = X[e];
                    }
                    const f32x4 Y = mma_k16(a4, b4, zero4(), DT{});
#pragma unroll
                    for (int r = 0; r < 4; ++r) Toff[ti][tj][r] = -Y[r];
                    DT *tb = sT + (16 * ti + 4 * g4) * PT + 16 * tj + c16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) tb[r * PT] = from_f32<DT>(-Y[r]);
                }
            }
        }

        // ---- chain, state-only half: R_raw = K S^T and O^T = S Q^T
        F sf[KS][NB];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(st[2 * kk][b], st[2 * kk + 1][b], sf[kk][b]);
        f32x4 racc[4][NB], oT[4][NB];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                racc[mt][b] = zero4();
                oT[mt][b] = zero4();
            }
            F fk[KS], fq[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                ld_chain(sK + (16 * mt + c16) * PK + 32 * kk + 4 * g4, fk[kk]);
                ld_chain(sQ + (16 * mt + c16) * PK + 32 * kk + 4 * g4, fq[kk]);
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    racc[mt][b] = mma(fk[kk], sf[kk][b], racc[mt][b]);  // C[t][dv]
                    oT[mt][b] = mma(sf[kk][b], fq[kk], oT[mt][b]);      // C[dv][t]
                }
            }
        }
        __syncthreads();  // T is ready

        // ---- R = beta (V - gamma K S^T)           (C layout [t][dv])
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int tb = 16 * mt + 4 * g4;
            const f32x4 bet = *reinterpret_cast<const f32x4 *>(sBeta + tb);
            const f32x4 gam = *reinterpret_cast<const f32x4 *>(sGam + tb);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int dvl = wdv + 16 * b + c16;
                float vv[4];
                if constexpr (BF) {
                    const bf16x4 v4 = *reinterpret_cast<const bf16x4 *>(sV + dvl * PT + tb);
#pragma unroll
                    for (int r = 0; r < 4; ++r) vv[r] = (float)v4[r];
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) vv[r] = to_f32(sV[(tb + r) * PV + dvl]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    racc[mt][b][r] = bet[r] * (vv[r] - gam[r] * racc[mt][b][r]);
            }
        }
        // ---- U = T R (T lower triangular: block row mt needs k steps 0..mt/2)
        F fr[2][NB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(racc[2 * k2][b], racc[2 * k2 + 1][b], fr[k2][b]);
        f32x4 u[4][NB];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int b = 0; b < NB; ++b) u[mt][b] = zero4();
#pragma unroll
            for (int k2 = 0; k2 <= (mt >> 1); ++k2) {
                F ft;
                ld_chain(sT + (16 * mt + c16) * PT + 32 * k2 + 4 * g4, ft);
#pragma unroll
                for (int b = 0; b < NB; ++b) u[mt][b] = mma(ft, fr[k2][b], u[mt][b]);
            }
        }
        // ---- O^T = (S Q^T) diag(gamma) + U^T P^T, stored for valid rows
        F fu[2][NB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(u[2 * k2][b], u[2 * k2 + 1][b], fu[k2][b]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float gam = sGam[16 * mt + c16];
#pragma unroll
            for (int b = 0; b < NB; ++b) oT[mt][b] *= gam;
#pragma unroll
            for (int k2 = 0; k2 <= (mt >> 1); ++k2) {
                F fp;
                ld_chain(sP + (16 * mt + c16) * PT + 32 * k2 + 4 * g4, fp);
#pragma unroll
                for (int b = 0; b < NB; ++b) oT[mt][b] = mma(fu[k2][b], fp, oT[mt][b]);
            }
        }
        {
            DT *oc = oh + (c * kC + c16) * sVO + 4 * g4;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                if (16 * mt + c16 < lenc) {
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        DT *dst = oc + (int64_t)(16 * mt) * sVO + 16 * b;
                        if constexpr (BF) {
                            bf16x4 ob;
#pragma unroll
                            for (int r = 0; r < 4; ++r) ob[r] = (__bf16)(p.scale * oT[mt][b][r]);
                            *reinterpret_cast<bf16x4 *>(dst) = ob;
                        } else {
                            *reinterpret_cast<f32x4 *>(dst) = p.scale * oT[mt][b];
                        }
                    }
                }
            }
        }
        // ---- S^T <- gamma_C S^T + K^T diag(e^{g_C - g}) U
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const f32x4 dec = *reinterpret_cast<const f32x4 *>(sDec + 16 * mt + 4 * g4);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) u[mt][b][r] *= dec[r];
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(u[2 * k2][b], u[2 * k2 + 1][b], fu[k2][b]);
        const float gC = sGam[kC - 1];
#pragma unroll
        for (int a0 = 0; a0 < NKT; a0 += 4) {
            F fkt[4][2];
#pragma unroll
            for (int a = a0; a < a0 + 4 && a < NKT; ++a)
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) {
                    if constexpr (BF)
                        ld_chain(sKT + (16 * a + c16) * PT + 32 * k2 + 4 * g4, fkt[a - a0][k2]);
                    else
                        ld_chain_col<DT>(sK + (32 * k2 + 4 * g4) * PK + 16 * a + c16, PK,
                                         fkt[a - a0][k2]);
                }
#pragma unroll
            for (int a = a0; a < a0 + 4 && a < NKT; ++a) {
#pragma unroll
                for (int b = 0; b < NB; ++b) st[a][b] *= gC;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                    for (int b = 0; b < NB; ++b) st[a][b] = mma(fkt[a - a0][k2], fu[k2][b], st[a][b]);
            }
        }
    }

    if (p.s_final) {
        float *sf = p.s_final + ((int64_t)n * p.Hv + h) * D * D;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<f32x4 *>(sf + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a +
                                           4 * g4) = st[a][b];
    }
}

template <typename DT, int D, int NW, int DVW>
static hipError_t launch_cfg(const PrefillParams &p, int nsplit, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.nseq * p.Hv * nsplit;
    if (nblocks <= 0 || nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int remap = (nblocks % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((prefill_kernel<DT, D, NW, DVW>), dim3((unsigned)nblocks), dim3(NW * 64), 0,
                       stream, p, nsplit, remap);
    return hipGetLastError();
}

// Choose the value-column slice per workgroup. With many chains
// (sequences x value heads) a workgroup takes a whole head; with few, the
// head is split so that more CUs work (each slice repeats the small
// state-free part of a chunk).
static int choose_split(int64_t chains, int D, int num_cus) {
    if (const char *env = getenv("GDN_PREFILL_NSPLIT")) {
        const int v = atoi(env);
        if (v == 1 || v == 2 || v == 4 || v == 8) return (D == 64 && v == 8) ? 4 : v;
    }
    if (chains >= num_cus) return 1;
    if (chains * 2 >= num_cus) return 2;
    return D == 128 ? 4 : 2;
}

hipError_t launch_prefill(const PrefillParams &p, int dtype, int D, int num_cus,
                          hipStream_t stream) {
    int ns = choose_split((int64_t)p.nseq * p.Hv, D, num_cus);
    if (dtype == 1) {
        if (D == 128) {
            switch (ns) {
            case 1: return launch_cfg<__bf16, 128, 8, 16>(p, 1, stream);
            case 2: return launch_cfg<__bf16, 128, 4, 16>(p, 2, stream);
            case 4: return launch_cfg<__bf16, 128, 2, 16>(p, 4, stream);
            default: return launch_cfg<__bf16, 128, 1, 16>(p, 8, stream);
            }
        } else if (D == 64) {
            switch (ns) {
            case 1: return launch_cfg<__bf16, 64, 4, 16>(p, 1, stream);
            case 2: return launch_cfg<__bf16, 64, 2, 16>(p, 2, stream);
            default: return launch_cfg<__bf16, 64, 1, 16>(p, 4, stream);
            }
        }
    } else if (dtype == 0) {
        if (D == 64) {
            switch (ns) {
            case 1: return launch_cfg<float, 64, 4, 16>(p, 1, stream);
            case 2: return launch_cfg<float, 64, 2, 16>(p, 2, stream);
            default: return launch_cfg<float, 64, 1, 16>(p, 4, stream);
            }
        } else if (D == 128) {
            // fp32 K, Q and V for a whole head exceed the LDS of a CU: at
            // least two slices.
            switch (ns) {
            case 1:
            case 2: return launch_cfg<float, 128, 4, 16>(p, 2, stream);
            case 4: return launch_cfg<float, 128, 2, 16>(p, 4, stream);
            default: return launch_cfg<float, 128, 1, 16>(p, 8, stream);
            }
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
