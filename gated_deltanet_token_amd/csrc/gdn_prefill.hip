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
//     U     = T R
//     O     = diag(gamma) Q S^T + P U
//     S_end = gamma_C S + U^T diag(e^{g_C - g}) K
// (U's row t is the token recurrence's b_t (v_t - a_t S_{t-1} k_t).)
//
// Work decomposition. One workgroup owns one (sequence, value head,
// slice of DVS value columns) and walks that sequence's chunks in order; the
// rows of S it owns evolve independently of the other rows, so slices never
// talk to each other. Inside the workgroup, wave w owns DVW value columns
// and keeps S^T for them in MFMA accumulators (fp32) for the whole call.
// The state-free part of a chunk (Gram products, decay, T, P) is computed
// cooperatively and shared through LDS.
//
// Per chunk:
//   stage   global -> LDS: K and Q row-major, K^T and V^T (bf16) or V (fp32),
//           alpha, beta. The next chunk's loads are issued into registers
//           right after, so HBM latency overlaps this chunk's math. Rows past
//           the end of the sequence are staged as k = q = v = 0, alpha = 1,
//           beta = 0, which leaves the recurrence unchanged.
//   gram    K K^T and Q K^T, lower 16x16 tiles only, on MFMA.
//   scan    chunk-local cumulative ln(alpha) (one wave).
//   mask    A (fp32) and P (operand type) into LDS.
//   solve   T = (I + A)^{-1}: the four 16x16 diagonal blocks by forward
//           substitution (one lane per column), then block rows 1..3 by
//           T_ij = -E_i sum_{m=j}^{i-1} A_im T_mj on MFMA (wave 0), while the
//           other waves already form K S^T and Q S^T for their columns.
//   chain   R, U = T R, O = gamma.(Q S^T) + P U, store O, then the state update,
//           all on MFMA with fp32 accumulation.
#include <float.h>

#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

constexpr int kC = 64;  // chunk length

template <typename DT, int D, int NW, int DVW> struct PrefillCfg {
    static constexpr int NTH = NW * 64;
    static constexpr int DVS = NW * DVW;   // value columns per workgroup
    static constexpr int NKT = D / 16;     // key-dim tiles of S^T
    static constexpr int NB = DVW / 16;    // value-dim tiles per wave
    static constexpr int KS = D / 32;      // 32-deep steps over the key dim
    static constexpr bool BF = sizeof(DT) == 2;
    static constexpr int EPP = 16 / (int)sizeof(DT);  // elements per 16-byte piece
    static constexpr int PK = D + (BF ? 8 : 4);       // row pitch of K, Q
    static constexpr int PT = kC + 4;                 // row pitch of T, P, K^T, V^T
    static constexpr int PV = DVS + 4;                // row pitch of V (fp32 path)
    static constexpr int PA = kC + 4;                 // row pitch of fp32 A and T
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
    static constexpr int OFF_TF = OFF_A + SZ_A;
    static constexpr int OFF_VEC = OFF_TF + SZ_A;  // 6 vectors of 64 floats
    static constexpr int LDS = OFF_VEC + 6 * kC * 4;
    // staging tasks: a task is one 16-byte piece of two consecutive rows
    static constexpr int PPR_K = D / EPP;
    static constexpr int PPR_V = DVS / EPP;
    static constexpr int TK = 32 * PPR_K;
    static constexpr int TV = 32 * PPR_V;
    static constexpr int NTK = (TK + NTH - 1) / NTH;
    static constexpr int NTV = (TV + NTH - 1) / NTH;
    static constexpr int NAB = (2 * kC + NTH - 1) / NTH;
    static constexpr int NPAIR = 10;                  // lower 16x16 tiles of a 64x64
    static constexpr int NPW = (NPAIR + NW - 1) / NW;  // tile pairs per wave
    static_assert(DVW % 16 == 0 && D % 32 == 0, "tile shapes");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// Task -> (row pair, piece). Within 64 consecutive tasks the row pair varies
// fastest over min(64, 32*...) values so the transposed LDS writes of a wave
// spread over all banks, while each wave still reads whole 64-byte row
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
    float *sTF = reinterpret_cast<float *>(smem + Cf::OFF_TF);
    float *sG = reinterpret_cast<float *>(smem + Cf::OFF_VEC);
    float *sGam = sG + kC;
    float *sDec = sG + 2 * kC;
    float *sBeta = sG + 3 * kC;
    float *sAraw = sG + 4 * kC;
    float *sBraw = sG + 5 * kC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    DT *oh = reinterpret_cast<DT *>(p.out) + tok0 * sVO + (int64_t)h * D + dv0;
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

    // ---- staging registers
    uint4 rK[Cf::NTK][2], rQ[Cf::NTK][2], rV[Cf::NTV][2];
    float rAB[Cf::NAB];
    auto stage_load = [&](int c) {
        const int64_t t0 = (int64_t)c * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
#pragma unroll
        for (int i = 0; i < Cf::NTK; ++i) {
            const int task = tid + i * NTH;
            if (task < Cf::TK) {
                int rp, pc;
                task_coords<Cf::PPR_K>(task, rp, pc);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * rp + e;
                    const int64_t off = (t0 + r) * sQK + pc * Cf::EPP;
                    rK[i][e] = r < lenc ? *reinterpret_cast<const uint4 *>(kh + off) : uint4{0, 0, 0, 0};
                    rQ[i][e] = r < lenc ? *reinterpret_cast<const uint4 *>(qh + off) : uint4{0, 0, 0, 0};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NTV; ++i) {
            const int task = tid + i * NTH;
            if (task < Cf::TV) {
                int rp, pc;
                task_coords<Cf::PPR_V>(task, rp, pc);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int r = 2 * rp + e;
                    const int64_t off = (t0 + r) * sVO + pc * Cf::EPP;
                    rV[i][e] = r < lenc ? *reinterpret_cast<const uint4 *>(vh + off) : uint4{0, 0, 0, 0};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NAB; ++i) {
            const int idx = tid + i * NTH;
            if (idx < kC)
                rAB[i] = idx < lenc ? ah[(t0 + idx) * p.Hv] : 1.f;
            else if (idx < 2 * kC)
                rAB[i] = idx - kC < lenc ? bh[(t0 + idx - kC) * p.Hv] : 0.f;
        }
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int i = 0; i < Cf::NTK; ++i) {
            const int task = tid + i * NTH;
            if (task < Cf::TK) {
                int rp, pc;
                task_coords<Cf::PPR_K>(task, rp, pc);
                const int r0 = 2 * rp, col = pc * Cf::EPP;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    *reinterpret_cast<uint4 *>(sK + (r0 + e) * PK + col) = rK[i][e];
                    *reinterpret_cast<uint4 *>(sQ + (r0 + e) * PK + col) = rQ[i][e];
                }
                if constexpr (BF) {
                    const uint32_t *lo = reinterpret_cast<const uint32_t *>(&rK[i][0]);
                    const uint32_t *hi = reinterpret_cast<const uint32_t *>(&rK[i][1]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t a = lo[w], b = hi[w];
                        *reinterpret_cast<uint32_t *>(sKT + (col + 2 * w) * PT + r0) =
                            (a & 0xFFFFu) | (b << 16);
                        *reinterpret_cast<uint32_t *>(sKT + (col + 2 * w + 1) * PT + r0) =
                            (a >> 16) | (b & 0xFFFF0000u);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NTV; ++i) {
            const int task = tid + i * NTH;
            if (task < Cf::TV) {
                int rp, pc;
                task_coords<Cf::PPR_V>(task, rp, pc);
                const int r0 = 2 * rp, col = pc * Cf::EPP;
                if constexpr (BF) {
                    const uint32_t *lo = reinterpret_cast<const uint32_t *>(&rV[i][0]);
                    const uint32_t *hi = reinterpret_cast<const uint32_t *>(&rV[i][1]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const uint32_t a = lo[w], b = hi[w];
                        *reinterpret_cast<uint32_t *>(sV + (col + 2 * w) * PT + r0) =
                            (a & 0xFFFFu) | (b << 16);
                        *reinterpret_cast<uint32_t *>(sV + (col + 2 * w + 1) * PT + r0) =
                            (a >> 16) | (b & 0xFFFF0000u);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 2; ++e)
                        *reinterpret_cast<uint4 *>(sV + (r0 + e) * PV + col) = rV[i][e];
                }
            }
        }
#pragma unroll
        for (int i = 0; i < Cf::NAB; ++i) {
            const int idx = tid + i * NTH;
            if (idx < kC)
                sAraw[idx] = rAB[i];
            else if (idx < 2 * kC)
                sBraw[idx - kC] = rAB[i];
        }
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    if (nchunks > 0) stage_load(0);

    for (int64_t c = 0; c < nchunks; ++c) {
        const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
        __syncthreads();  // the previous chunk is done with LDS
        stage_store();
        if (c + 1 < nchunks) stage_load((int)(c + 1));
        __syncthreads();

        // ---- Gram tiles: pair pr -> lower tile (i, j) of K K^T and Q K^T
        f32x4 gk[Cf::NPW], gq[Cf::NPW];
#pragma unroll
        for (int pi = 0; pi < Cf::NPW; ++pi) {
            const int pr = wave + pi * NW;
            gk[pi] = zero4();
            gq[pi] = zero4();
            if (pr < Cf::NPAIR) {
                const int ti = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
                const int tj = pr - ti * (ti + 1) / 2;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    F fki, fqi, fkj;
                    ld_nat(sK + (16 * ti + c16) * PK + 32 * kk + 8 * g4, fki);
                    ld_nat(sQ + (16 * ti + c16) * PK + 32 * kk + 8 * g4, fqi);
                    ld_nat(sK + (16 * tj + c16) * PK + 32 * kk + 8 * g4, fkj);
                    gk[pi] = mma(fki, fkj, gk[pi]);
                    gq[pi] = mma(fqi, fkj, gq[pi]);
                }
            }
        }
        // ---- chunk-local cumulative log decay (wave 0)
        if (wave == 0) {
            float x = logf(fmaxf(sAraw[lane], FLT_MIN));
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(x, off, 64);
                if (lane >= off) x += y;
            }
            const float glast = __shfl(x, 63, 64);
            sG[lane] = x;
            sGam[lane] = __expf(x);
            sDec[lane] = __expf(glast - x);
            sBeta[lane] = sBraw[lane];
        }
        __syncthreads();

        // ---- decay masks: A (fp32) and P (operand type)
#pragma unroll
        for (int pi = 0; pi < Cf::NPW; ++pi) {
            const int pr = wave + pi * NW;
            if (pr < Cf::NPAIR) {
                const int ti = pr < 1 ? 0 : pr < 3 ? 1 : pr < 6 ? 2 : 3;
                const int tj = pr - ti * (ti + 1) / 2;
                const int s = 16 * tj + c16;
                const float gs = sG[s];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * ti + 4 * g4 + r;
                    const float dec = s <= t ? __expf(sG[t] - gs) : 0.f;
                    sA[t * PA + s] = s < t ? sBeta[t] * dec * gk[pi][r] : 0.f;
                    sP[t * PT + s] = from_f32<DT>(dec * gq[pi][r]);
                }
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1} on wave 0
        if (wave == 0) {
            // diagonal 16x16 blocks: lane = 16*blk + column, forward substitution
            {
                const int blk = g4, col = c16;
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float acc = r == col ? 1.f : 0.f;
                    const float *ar = sA + (16 * blk + r) * PA + 16 * blk;
#pragma unroll
                    for (int m = 0; m < r; ++m) acc -= ar[m] * x[m];
                    x[r] = acc;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sTF[(16 * blk + r) * PA + 16 * blk + col] = x[r];
                    sT[(16 * blk + r) * PT + 16 * blk + col] = from_f32<DT>(x[r]);
                }
            }
            // block rows 1..3: T_ij = -E_i * sum_{m=j}^{i-1} A_im T_mj
#pragma unroll
            for (int ti = 1; ti < 4; ++ti) {
#pragma unroll
                for (int tj = 0; tj < ti; ++tj) {
                    f32x4 X = zero4();
#pragma unroll
                    for (int m = tj; m < ti; ++m) {
                        float a4[4], b4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            a4[e] = sA[(16 * ti + c16) * PA + 16 * m + 4 * g4 + e];
                            b4[e] = sTF[(16 * m + 4 * g4 + e) * PA + 16 * tj + c16];
                        }
                        X = mma_k16(a4, b4, X, DT{});
                    }
                    float a4[4], b4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        a4[e] = sTF[(16 * ti + c16) * PA + 16 * ti + 4 * g4 + e];
                        b4[e] = X[e];
                    }
                    const f32x4 Y = mma_k16(a4, b4, zero4(), DT{});
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * ti + 4 * g4 + r;
                        sTF[t * PA + 16 * tj + c16] = -Y[r];
                        sT[t * PT + 16 * tj + c16] = from_f32<DT>(-Y[r]);
                    }
                }
            }
        }

        // ---- chain, state-only half: K S^T and Q S^T for this wave's columns
        F sf[KS][NB];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(st[2 * kk][b], st[2 * kk + 1][b], sf[kk][b]);
        f32x4 racc[4][NB], oacc[4][NB];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                racc[mt][b] = zero4();
                oacc[mt][b] = zero4();
            }
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                F fk, fq;
                ld_chain(sK + (16 * mt + c16) * PK + 32 * kk + 4 * g4, fk);
                ld_chain(sQ + (16 * mt + c16) * PK + 32 * kk + 4 * g4, fq);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    racc[mt][b] = mma(fk, sf[kk][b], racc[mt][b]);
                    oacc[mt][b] = mma(fq, sf[kk][b], oacc[mt][b]);
                }
            }
        }
        __syncthreads();  // T is ready

        // ---- R = beta (V - gamma K S^T)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int dvl = wdv + 16 * b + c16;
                const int tb = 16 * mt + 4 * g4;
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
                    racc[mt][b][r] = sBeta[tb + r] * (vv[r] - sGam[tb + r] * racc[mt][b][r]);
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
        // ---- O = gamma (Q S^T) + P U, stored for valid rows
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) oacc[mt][b][r] *= sGam[16 * mt + 4 * g4 + r];
        F fu[2][NB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(u[2 * k2][b], u[2 * k2 + 1][b], fu[k2][b]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int k2 = 0; k2 <= (mt >> 1); ++k2) {
                F fp;
                ld_chain(sP + (16 * mt + c16) * PT + 32 * k2 + 4 * g4, fp);
#pragma unroll
                for (int b = 0; b < NB; ++b) oacc[mt][b] = mma(fp, fu[k2][b], oacc[mt][b]);
            }
        }
        {
            DT *oc = oh + c * kC * sVO + wdv + c16;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * mt + 4 * g4 + r;
                    if (t < lenc) {
#pragma unroll
                        for (int b = 0; b < NB; ++b)
                            oc[(int64_t)t * sVO + 16 * b] = from_f32<DT>(p.scale * oacc[mt][b][r]);
                    }
                }
        }
        // ---- S^T <- gamma_C S^T + K^T diag(e^{g_C - g}) U
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) u[mt][b][r] *= sDec[16 * mt + 4 * g4 + r];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(u[2 * k2][b], u[2 * k2 + 1][b], fu[k2][b]);
        const float gC = sGam[kC - 1];
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
#pragma unroll
            for (int b = 0; b < NB; ++b) st[a][b] *= gC;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                F fkt;
                if constexpr (BF)
                    ld_chain(sKT + (16 * a + c16) * PT + 32 * k2 + 4 * g4, fkt);
                else
                    ld_chain_col<DT>(sK + (32 * k2 + 4 * g4) * PK + 16 * a + c16, PK, fkt);
#pragma unroll
                for (int b = 0; b < NB; ++b) st[a][b] = mma(fkt, fu[k2][b], st[a][b]);
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
            case 1: return launch_cfg<__bf16, 128, 4, 32>(p, 1, stream);
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
