// gdn_prefill.hip -- chunk-64 prefill of the gated delta rule on gfx950.
//
// The token recurrence (S in R^{Dv x Dk}; q/k head g = h / (Hv/Hk))
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
// is evaluated 64 tokens at a time through the exact rewrite documented in
// gdn_chunk.hpp. Two ways to run it:
//
// Fused (no workspace). One workgroup owns one (sequence, value head, slice
// of DVS value columns) and walks that sequence's chunks in order; wave w
// owns DVW value columns and keeps S^T for them in MFMA accumulators for the
// whole call. Per chunk (barriers marked |):
//   | stage  registers -> LDS (K, Q row-major; K^T, V^T for bf16), wave 0
//            turns its alpha/beta registers into the chunk-local decay; the
//            next chunk's global loads are then issued into registers so
//            their latency overlaps this chunk. Rows past the end of the
//            sequence are staged as k = q = v = 0, alpha = 1, beta = 0, which
//            leaves the recurrence unchanged.
//   | gram   transposed Gram tiles on MFMA, decay masks, rows of A and P.
//   | solve  wave 0: T = (I + A)^{-1}; the other waves form K S^T, S Q^T.
//   | chain  R, U = T R, O, state update on MFMA.
// The rows of S a workgroup owns evolve independently of the other rows, so
// slices never talk to each other; they only repeat the state-free work.
//
// Two-pass (caller-provided workspace). The state-free work of every chunk
// (Gram products, decay, the solve) has no dependence on the state, so
// prep_kernel does it for all (chunk, value head) pairs at once and writes
// T, P and the decay vectors to the workspace; chain_kernel then walks the
// chunks in order doing only the MFMA state chain. This moves the solve's
// latency off the sequential path, which is what limits small batches.
#include <float.h>
#include <stdlib.h>

#include "gdn_chunk.hpp"
#include "gdn_seq.hpp"
#include <type_traits>

#include "gdn_launch.hpp"

namespace gdn {

// ----------------------------------------------------------------------------
// shared per-workgroup bookkeeping

// Sequence bounds of sequence n.
// ----------------------------------------------------------------------------
// staging of K, Q (row-major, K^T for bf16) and a V column slice (V^T for
// bf16, row-major for fp32) through registers, one chunk ahead.

template <typename DT, int D, int NTH, int DVS> struct Stager {
    using P = ChunkPitch<DT, D>;
    static constexpr bool BF = P::BF;
    static constexpr int EPP = 16 / (int)sizeof(DT);
    static constexpr int PPR_K = D / EPP;
    static constexpr int PPR_V = DVS / EPP;
    static constexpr int TK = 32 * PPR_K;
    static constexpr int TV = 32 * PPR_V;
    static constexpr int NTK = (TK + NTH - 1) / NTH;
    static constexpr int NTV = (TV + NTH - 1) / NTH;
    static constexpr int PV = DVS + 4;

    int kOffG[NTK], kOffL[NTK], kRow[NTK];
    int vOffG[NTV], vOffL[NTV], vRow[NTV];
    u32x4 rK[NTK][2], rQ[NTK][2], rV[NTV][2];

    // Threads past the last task take the last task again: every thread
    // issues every load (a load skipped by a whole wave would leave the
    // compiler unsure how many loads are in flight, and it would then wait for
    // all of them), and duplicate LDS writes store identical bytes.
    __device__ __forceinline__ void init(int tid) {
#pragma unroll
        for (int i = 0; i < NTK; ++i) {
            int rp = 0, pc = 0;
            task_coords<PPR_K>(min(tid + i * NTH, TK - 1), rp, pc);
            kRow[i] = 2 * rp;
            kOffG[i] = pc * EPP;
            kOffL[i] = 2 * rp * P::PK + pc * EPP;
        }
#pragma unroll
        for (int i = 0; i < NTV; ++i) {
            int rp = 0, pc = 0;
            task_coords<PPR_V>(min(tid + i * NTH, TV - 1), rp, pc);
            vRow[i] = 2 * rp;
            vOffG[i] = pc * EPP;
            vOffL[i] = BF ? (pc * EPP) * P::PT + 2 * rp : 2 * rp * PV + pc * EPP;
        }
    }
    // Raw loads of chunk rows [t0, t0 + 64); rows >= lenc are read from a
    // valid row and zeroed at store time, so nothing consumes the loaded
    // registers before the store (the loads stay in flight meanwhile).
    __device__ __forceinline__ void load(const DT *kh, const DT *qh, const DT *vh, int64_t t0,
                                         int lenc, int64_t sQK, int64_t sVO, int) {
#pragma unroll
        for (int i = 0; i < NTK; ++i) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = kRow[i] + e;
                const int rr = r < lenc ? r : lenc - 1;
                const int64_t off = (t0 + rr) * sQK + kOffG[i];
                rK[i][e] = *reinterpret_cast<const u32x4 *>(kh + off);
                rQ[i][e] = *reinterpret_cast<const u32x4 *>(qh + off);
            }
        }
#pragma unroll
        for (int i = 0; i < NTV; ++i) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int r = vRow[i] + e;
                const int rr = r < lenc ? r : lenc - 1;
                rV[i][e] = *reinterpret_cast<const u32x4 *>(vh + (t0 + rr) * sVO + vOffG[i]);
            }
        }
    }
    __device__ __forceinline__ void store(DT *sK, DT *sQ, DT *sKT, DT *sV, int lenc, int) {
        const u32x4 z4 = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NTK; ++i) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bool ok = kRow[i] + e < lenc;
                rK[i][e] = ok ? rK[i][e] : z4;
                rQ[i][e] = ok ? rQ[i][e] : z4;
                *reinterpret_cast<u32x4 *>(sK + kOffL[i] + e * P::PK) = rK[i][e];
                *reinterpret_cast<u32x4 *>(sQ + kOffL[i] + e * P::PK) = rQ[i][e];
            }
            if constexpr (BF)
                store_pair_transposed<P::PT>(sKT + kOffG[i] * P::PT + kRow[i], rK[i][0], rK[i][1]);
        }
#pragma unroll
        for (int i = 0; i < NTV; ++i) {
#pragma unroll
            for (int e = 0; e < 2; ++e) rV[i][e] = vRow[i] + e < lenc ? rV[i][e] : z4;
            if constexpr (BF) {
                store_pair_transposed<P::PT>(sV + vOffL[i], rV[i][0], rV[i][1]);
            } else {
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    *reinterpret_cast<u32x4 *>(sV + vOffL[i] + e * PV) = rV[i][e];
            }
        }
    }
};

// ----------------------------------------------------------------------------
// fused kernel

template <typename DT, int D, int NW, int DVW> struct FusedCfg {
    using P = ChunkPitch<DT, D>;
    static constexpr int NTH = NW * 64;
    static constexpr int DVS = NW * DVW;
    static constexpr int PV = DVS + 4;
    static constexpr int SZ_K = kC * P::PK * (int)sizeof(DT);
    static constexpr int SZ_KT = P::BF ? D * P::PT * 2 : 0;
    static constexpr int SZ_V = P::BF ? DVS * P::PT * 2 : kC * PV * 4;
    static constexpr int SZ_T = kC * P::PT * (int)sizeof(DT);
    static constexpr int SZ_A = kC * P::PA * 4;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_K;
    static constexpr int OFF_KT = OFF_Q + SZ_K;
    static constexpr int OFF_V = OFF_KT + SZ_KT;
    static constexpr int OFF_T = OFF_V + SZ_V;
    static constexpr int OFF_P = OFF_T + SZ_T;
    static constexpr int OFF_A = OFF_P + SZ_T;
    static constexpr int OFF_E = OFF_A + SZ_A;
    // g, gam, dec, beta, gamq, grA, grP, gc (the last four with raw q, k)
    static constexpr int OFF_VEC = OFF_E + SZ_A;
    static constexpr int LDS = OFF_VEC + 8 * kC * 4;
    static_assert(DVW % 16 == 0 && D % 32 == 0, "tile shapes");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// PREFIX: also write the block-aligned prefix states; RAWQK: q and k rows
// are raw and get L2-normalised here (their norms folded into the decay
// vectors). Each is a separate instantiation, so that the kernel without
// them carries no trace of either.
template <typename DT, int D, int NW, int DVW, bool PREFIX, bool RAWQK>
__global__ __launch_bounds__(NW * 64) void prefill_kernel(PrefillParams p, int nsplit,
                                                          int remap_xcd) {
    using Cf = FusedCfg<DT, D, NW, DVW>;
    using Pi = ChunkPitch<DT, D>;
    constexpr int NTH = Cf::NTH, NKT = D / 16, NB = DVW / 16, KS = D / 32;
    constexpr int PK = Pi::PK, PT = Pi::PT, PA = Pi::PA, PV = Cf::PV;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS];
    DT *sK = reinterpret_cast<DT *>(smem + Cf::OFF_K);
    DT *sQ = reinterpret_cast<DT *>(smem + Cf::OFF_Q);
    DT *sKT = reinterpret_cast<DT *>(smem + Cf::OFF_KT);
    DT *sV = reinterpret_cast<DT *>(smem + Cf::OFF_V);
    DT *sT = reinterpret_cast<DT *>(smem + Cf::OFF_T);
    DT *sP = reinterpret_cast<DT *>(smem + Cf::OFF_P);
    float *sA = reinterpret_cast<float *>(smem + Cf::OFF_A);
    float *sE = reinterpret_cast<float *>(smem + Cf::OFF_E);
    float *sG = reinterpret_cast<float *>(smem + Cf::OFF_VEC);
    float *sGam = sG + kC;
    float *sDec = sG + 2 * kC;
    float *sBeta = sG + 3 * kC;
    float *sGamQ = sG + 4 * kC;
    float *sGrA = sG + 5 * kC;
    float *sGrP = sG + 6 * kC;
    float *sGc = sG + 7 * kC;
    constexpr bool raw_qk = RAWQK;
    const bool logits = p.flags & kGateLogits;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    const int wg = logical_wg(remap_xcd);
    const int slice = wg % nsplit;
    const int nh = wg / nsplit;
    const int h = nh % p.Hv;
    const int n = nh / p.Hv;
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int dv0 = slice * Cf::DVS;
    const int wdv = wave * DVW;

    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const DT *qh = reinterpret_cast<const DT *>(p.q) + tok0 * sQK + (int64_t)grp * D;
    const DT *kh = reinterpret_cast<const DT *>(p.k) + tok0 * sQK + (int64_t)grp * D;
    const int64_t sVt = p.v_stride;
    const DT *vh = reinterpret_cast<const DT *>(p.v) + tok0 * sVt + (int64_t)h * D + dv0;
    DT *oh = reinterpret_cast<DT *>(p.out) + tok0 * sVO + (int64_t)h * D + dv0 + wdv;
    const float *ah = p.alpha + tok0 * p.Hv + h;
    const float *bh = p.beta + tok0 * p.Hv + h;

    // Upper blocks of T and P are never written: clear both once.
    for (int i = tid; i < 2 * Cf::SZ_T / 4; i += NTH)
        reinterpret_cast<float *>(smem + Cf::OFF_T)[i] = 0.f;

    f32x4 st[NKT][NB];
    {
        const float *s0 = p.s0 ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                st[a][b] = p.s0_identity ? eye4(dv0 + wdv + 16 * b + c16, 16 * a + 4 * g4)
                           : s0 ? *reinterpret_cast<const f32x4 *>(
                                      s0 + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a + 4 * g4)
                                : zero4();
    }

    Stager<DT, D, NTH, Cf::DVS> sg;
    sg.init(tid);
    float rAl = 1.f, rBe = 0.f;  // wave 0: alpha, beta of token `lane` of the next chunk
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
        sg.load(kh, qh, vh, t0, lenc, sQK, sVt, tid);
        if (wave == 0) {
            const int rr = lane < lenc ? lane : lenc - 1;
            rAl = ah[(t0 + rr) * p.Hv];
            rBe = bh[(t0 + rr) * p.Hv];
        }
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    PrefixRows pre(p, n, len);
    if (nchunks > 0) load_chunk(0);
    // Drain the initial-state and first-chunk loads here (the first store
    // needs them anyway). Otherwise the state registers count as possibly
    // pending inside the loop and each chunk would wait on its prefetch.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    for (int64_t c = 0; c < nchunks; ++c) {
        const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
        __syncthreads();  // the previous chunk is done with LDS
        sg.store(sK, sQ, sKT, sV, lenc, tid);
        if (wave == 0) {
            const bool ok = lane < lenc;
            const float la = logits ? neg_softplus(rAl) : __logf(fmaxf(rAl, FLT_MIN));
            const float x = wave_inclusive_scan(ok ? la : 0.f);
            const float glast = __shfl(x, 63, 64);
            sG[lane] = x;
            sGam[lane] = __expf(x);
            sDec[lane] = __expf(glast - x);
            sBeta[lane] = ok ? (logits ? sigmoid_f(rBe) : rBe) : 0.f;
        }
        if (c + 1 < nchunks) load_chunk(c + 1);
        __syncthreads();
        if constexpr (raw_qk) {
            fold_qk_norms<DT, D, PK, NTH>(sK, sQ, sG, sGam, sDec, sGamQ, sGrA, sGrP, sGc, tid);
            __syncthreads();
        }

#pragma unroll
        for (int pr = 0; pr < 10; ++pr) {
            if (pr % NW != wave) continue;
            f32x4 gk, gq;
            gram_pair<DT, D, PK>(sK, sQ, pair_i(pr), pair_j(pr), g4, c16, gk, gq);
            mask_pair<DT, PA, PT, false, raw_qk>(gk, gq, pair_i(pr), pair_j(pr), g4, c16,
                                                 raw_qk ? sGrA : sG,
                                  raw_qk ? sGrP : sG, raw_qk ? sGc : sG, sBeta, sA, sP);
        }
        __syncthreads();

        // T = (I + A)^{-1}: the diagonal blocks on wave 0 while the others
        // form their state-dependent half; then, with four or more waves, the
        // three block columns below the diagonal on waves 0 .. 2 at once
        constexpr bool PAR = NW >= 4;
        if (wave == 0) {
            if constexpr (PAR)
                solve_diag_blocks<DT, PA, PT, false>(sA, sE, sT, g4, c16);
            else
                solve_unit_lower<DT, PA, PT>(sA, sE, sT, g4, c16);
        }

        const ChainSmem<DT> m{sK,   sQ,   sKT,   sV,    sT,
                              sP,   sGam, sDec,  sBeta, raw_qk ? sGamQ : sGam};
        Frag<DT> sf[KS][NB];
        f32x4 racc[4][NB], oT[4][NB];
        chain_state_half<DT, D, NB, PK, (NW < 8)>(m, st, sf, racc, oT, g4, c16);
        if constexpr (PAR) {
            __syncthreads();  // the diagonal blocks E_b are ready
            if (wave < 3) solve_column<DT, PA, PT>(sA, sE, sT, wave, g4, c16);
        }
        __syncthreads();  // T is ready
        chain_finish<DT, D, NB, PK, PT, PV>(m, st, racc, oT, wdv, oh + c * kC * sVO, sVO, lenc,
                                            p.scale, g4, c16);
        const int64_t prow = PREFIX ? pre.take(p, c) : -1;
        if (prow >= 0) {
            float *ps = p.prefix + (prow * p.Hv + h) * D * D;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    __builtin_nontemporal_store(
                        st[a][b], reinterpret_cast<f32x4 *>(
                                      ps + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a + 4 * g4));
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

// ----------------------------------------------------------------------------
// two-pass path: per-chunk factors in the workspace
//
// Workspace record of one (chunk slot, value head), ws_bytes_per_chunk bytes:
//   T [64][64] DT | P [64][64] DT | gam [64] | dec [64] | beta [64] | gamq [64] (f32;
//   the decay vectors of ChainSmem)

template <typename DT> constexpr int ws_bytes_per_chunk() {
    return 2 * kC * kC * (int)sizeof(DT) + 4 * kC * 4;
}

// Fragment record (bf16, read by chain4_kernel and chain_db_kernel): T and P
// each as the kTriFrags MFMA fragments that cover their nonzero blocks, in
// lane order, the two with a zero half stored compact (5 KiB each), then
// gam [64] | dec [64] | beta [64] | gamq [64] (f32, 1 KiB): 11 KiB. The chain
// copies it into LDS unchanged and reads one fragment per lane with a single
// 16-byte (compact: 8-byte) load.
constexpr int kFragBytes = kTriFragBytes;
constexpr int ws_bytes_frag() { return 2 * kFragBytes + 1024; }
static_assert(ws_bytes_frag() <= ws_bytes_per_chunk<__bf16>(), "fragment record fits the query");

// value heads per q/k head that one prep workgroup serves at most
constexpr int kPrepGrpMax = 3;

template <typename DT, int D, bool FRAG> struct PrepCfg {
    using P = ChunkPitch<DT, D>;
    static constexpr int SZ_K = kC * P::PK * (int)sizeof(DT);
    static constexpr int SZ_A = kC * P::PA * 4;
    static constexpr int SZ_T = kC * P::PT * (int)sizeof(DT);
    // K and Q are dead once the Gram products are formed; A (and with FRAG
    // also T) then take their place. FRAG writes P straight to the workspace.
    static constexpr int AT = FRAG ? SZ_A + SZ_T : SZ_A;
    static constexpr int SZ_KQ = 2 * SZ_K > AT ? 2 * SZ_K : AT;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = SZ_K;
    static constexpr int OFF_A = 0;
    static constexpr int OFF_T = FRAG ? SZ_A : SZ_KQ;
    static constexpr int OFF_P = FRAG ? SZ_KQ : OFF_T + SZ_T;
    static constexpr int OFF_VEC = FRAG ? SZ_KQ : OFF_P + SZ_T;
    static constexpr int LDS = OFF_VEC + 8 * kC * 4;  // the eight vectors of prefill_kernel
    // a workgroup for all value heads of a q/k head: their vectors and the
    // inverse K, Q row norms
    static constexpr int LDS_GRP = OFF_VEC + kPrepGrpMax * 7 * kC * 4 + 2 * kC * 4;
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// T, P of one chunk and value head -> its workspace record: as fragments
// (FRAG) or as dense [64][64] rows; blocks above the diagonal (never written
// in LDS) are stored as zeros.
template <typename DT, int D, bool FRAG>
__device__ __forceinline__ void write_tp_record(unsigned char *rec, const DT *sT, const DT *sP, int tid) {
    using Pi = ChunkPitch<DT, D>;
    constexpr int PT = Pi::PT;
    constexpr int EPP = 16 / (int)sizeof(DT);
    if constexpr (FRAG) {
        // T (P is written by mask_pair): piece q is fragment i, lane l; its
        // halves are columns 32 k2 + 4 g4 .. +3 and 16 further of row
        // 16 rb + c16. The upper half lies above the diagonal (zero) exactly
        // for the compact fragments, which store the lower half alone.
        for (int q = tid; q < kTriFrags * 64; q += 256) {
            const int i = q / 64, l = q % 64, lg4 = l >> 4, lc16 = l & 15;
            const int rb = tri_rb(i), k2 = tri_k2(i);
            const DT *src = sT + (16 * rb + lc16) * PT + 32 * k2 + 4 * lg4;
            const u32x2 lo = *reinterpret_cast<const u32x2 *>(src);
            if (tri_frag_half(i)) {
                *reinterpret_cast<u32x2 *>(rec + tri_frag_at(i, l, 0)) = lo;
            } else {
                const u32x2 hi = *reinterpret_cast<const u32x2 *>(src + 16);
                *reinterpret_cast<u32x4 *>(rec + tri_frag_at(i, l, 0)) = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
    } else {
        constexpr int PPR = kC / EPP;
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        DT *gT = reinterpret_cast<DT *>(rec);
        DT *gP = gT + kC * kC;
        for (int i = tid; i < kC * PPR; i += 256) {
            const int r = i / PPR, pc = i % PPR;
            const bool upper = (pc * EPP) / 16 > r / 16;
            *reinterpret_cast<u32x4 *>(gT + r * kC + pc * EPP) =
                upper ? z4 : *reinterpret_cast<const u32x4 *>(sT + r * PT + pc * EPP);
            *reinterpret_cast<u32x4 *>(gP + r * kC + pc * EPP) =
                upper ? z4 : *reinterpret_cast<const u32x4 *>(sP + r * PT + pc * EPP);
        }
    }
}

// One workgroup (4 waves) per (chunk slot, value head): Gram products, decay,
// T = (I + A)^{-1}; writes T, P, gamma, dec, beta to the workspace (52 KiB
// of LDS for bf16, D = 128: three workgroups share a CU and hide each
// other's latencies). FRAG: the fragment record instead of dense rows, with
// T in the dead K/Q staging and P written from registers (35 KiB, at most
// 128 registers: four workgroups per CU). GRP (with FRAG): one workgroup per
// (chunk slot, q/k head) for its R = Hv / Hk <= kPrepGrpMax value heads: the
// K, Q staging, their row norms and the Gram products K K^T, Q K^T (which no
// gate enters) are formed once, the scans run on waves 0 .. R - 1 at once,
// and the masks, the solve and the record follow head by head.
template <typename DT, int D, bool FRAG, bool RAWQK, bool GRP>
__global__ __launch_bounds__(256, FRAG ? 4 : 1) void prep_kernel(PrefillParams p, unsigned char *ws,
                                                                 int remap_xcd) {
    static_assert(!FRAG || sizeof(DT) == 2, "fragment records are bf16");
    static_assert(!GRP || FRAG, "the grouped prep writes fragment records");
    using Cf = PrepCfg<DT, D, FRAG>;
    using Pi = ChunkPitch<DT, D>;
    constexpr int PK = Pi::PK, PT = Pi::PT, PA = Pi::PA;
    constexpr int EPP = 16 / (int)sizeof(DT);
    __shared__ __attribute__((aligned(16))) unsigned char smem[GRP ? Cf::LDS_GRP : Cf::LDS];
    DT *sK = reinterpret_cast<DT *>(smem + Cf::OFF_K);
    DT *sQ = reinterpret_cast<DT *>(smem + Cf::OFF_Q);
    float *sA = reinterpret_cast<float *>(smem + Cf::OFF_A);
    DT *sT = reinterpret_cast<DT *>(smem + Cf::OFF_T);
    DT *sP = reinterpret_cast<DT *>(smem + Cf::OFF_P);
    // the vectors of value head r of the group at sG0 + VS r: g, gamma, dec,
    // beta, gamq, grA, grP, gc; the grouped kernel keeps seven (gc takes
    // g's place once the norms are folded in), so that four workgroups fit a
    // CU's LDS
    constexpr int VS = (GRP ? 7 : 8) * kC;
    float *sG0 = reinterpret_cast<float *>(smem + Cf::OFF_VEC);
    float *sIK = sG0 + kPrepGrpMax * 7 * kC;  // GRP: inverse K row norms, then Q's
    float *sIQ = sIK + kC;
    static_assert(!GRP || !FRAG || 4 * Cf::LDS_GRP <= 160 * 1024, "four grouped workgroups per CU");
    constexpr bool raw_qk = RAWQK;
    const bool logits = p.flags & kGateLogits;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    // value heads of one chunk are consecutive logical ids: same XCD, so the
    // heads sharing a q/k head read K and Q through one L2
    const int wg = logical_wg(remap_xcd);
    const int nhg = GRP ? p.Hk : p.Hv;  // workgroups per chunk slot
    const int hw = wg % nhg;
    const int64_t slot = p.chunk0 + wg / nhg;  // chunk0 > 0 only for one dense sequence
    // which (sequence, chunk) owns this slot
    int n;
    if (p.cu_seqlens) {
        int lo = 0, hi = p.nseq - 1;  // largest n with slot_base(n) <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (slot_base(p, mid) <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        n = lo;
    } else {
        // chunks per sequence and slots both fit 32 bits (the ABI bounds them)
        const uint32_t per = (uint32_t)((p.seq_len + kC - 1) / kC);
        n = (int)((uint32_t)slot / per);
    }
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int64_t c = slot - slot_base(p, n);
    if (c < 0 || c * kC >= len) return;  // unused slot (uniform over the workgroup)
    const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
    const int64_t t0 = tok0 + c * kC;
    const int R = GRP ? p.Hv / p.Hk : 1;  // value heads of this workgroup: h0 .. h0 + R - 1
    const int grp = GRP ? hw : hw / (p.Hv / p.Hk);
    const int h0 = GRP ? hw * R : hw;
    const int64_t sQK = (int64_t)p.Hk * D;
    const DT *kh = reinterpret_cast<const DT *>(p.k) + t0 * sQK + (int64_t)grp * D;
    const DT *qh = reinterpret_cast<const DT *>(p.q) + t0 * sQK + (int64_t)grp * D;

    // alpha, beta (wave r: head h0 + r) and the K, Q rows are all requested
    // before any of them is used, so their latencies overlap
    float a_t = 1.f, b_t = 0.f;
    if (wave < R) {
        const int rr = lane < lenc ? lane : lenc - 1;
        a_t = p.alpha[(t0 + rr) * p.Hv + h0 + wave];
        b_t = p.beta[(t0 + rr) * p.Hv + h0 + wave];
    }
    // K, Q rows -> LDS (rows past the end of the sequence are zero)
    {
        constexpr int PPR = D / EPP;
        constexpr int NPC = kC * PPR / 256;  // pieces per thread
        static_assert(kC * PPR % 256 == 0, "whole pieces per thread");
        const u32x4 z4 = {0u, 0u, 0u, 0u};
        u32x4 kv[NPC], qv[NPC];
#pragma unroll
        for (int j = 0; j < NPC; ++j) {
            const int i = tid + 256 * j, r = i / PPR, pc = i % PPR;
            const int rr = r < lenc ? r : lenc - 1;
            kv[j] = *reinterpret_cast<const u32x4 *>(kh + (int64_t)rr * sQK + pc * EPP);
            qv[j] = *reinterpret_cast<const u32x4 *>(qh + (int64_t)rr * sQK + pc * EPP);
        }
#pragma unroll
        for (int j = 0; j < NPC; ++j) {
            const int i = tid + 256 * j, r = i / PPR, pc = i % PPR;
            *reinterpret_cast<u32x4 *>(sK + r * PK + pc * EPP) = r < lenc ? kv[j] : z4;
            *reinterpret_cast<u32x4 *>(sQ + r * PK + pc * EPP) = r < lenc ? qv[j] : z4;
        }
    }
    constexpr int WSB = FRAG ? ws_bytes_frag() : ws_bytes_per_chunk<DT>();
    auto rec_of = [&](int r) { return ws + (slot * p.Hv + h0 + r) * (int64_t)WSB; };
    auto vec_of = [&](int r) {
        return reinterpret_cast<float *>(rec_of(r) + (FRAG ? 2 * kFragBytes : 2 * kC * kC * (int)sizeof(DT)));
    };
    if (wave < R) {
        float *sG = sG0 + VS * wave, *sGam = sG + kC, *sDec = sG + 2 * kC, *sBeta = sG + 3 * kC;
        float *vec = vec_of(wave);
        const float a = a_t, b = b_t;
        const bool ok = lane < lenc;
        const float la = logits ? neg_softplus(a) : __logf(fmaxf(a, FLT_MIN));
        const float x = wave_inclusive_scan(ok ? la : 0.f);
        const float glast = __shfl(x, 63, 64);
        const float gam = __expf(x), dec = __expf(glast - x);
        const float bet = ok ? (logits ? sigmoid_f(b) : b) : 0.f;
        sG[lane] = x;
        sGam[lane] = gam;
        sDec[lane] = dec;
        sBeta[lane] = bet;
        if (!raw_qk) {  // otherwise written once the row norms are folded in
            vec[lane] = gam;
            vec[kC + lane] = dec;
            vec[2 * kC + lane] = bet;
            vec[3 * kC + lane] = gam;
        }
    }
    __syncthreads();
    if constexpr (raw_qk) {  // K and Q stay live until the barrier after the Gram products
        if constexpr (GRP) {
            qk_inv_norms<DT, D, PK, 256>(sK, sQ, sIK, sIQ, tid);
        } else {
            float *sG = sG0;
            fold_qk_norms<DT, D, PK, 256>(sK, sQ, sG, sG + kC, sG + 2 * kC, sG + 4 * kC, sG + 5 * kC,
                                          sG + 6 * kC, sG + 7 * kC, tid);
        }
    }
    // Gram products of this wave's lower tile pairs (pr = wave, wave + 4, ...)
    f32x4 gk[3], gq[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const int pr = wave + 4 * k;
        if (pr < 10) gram_pair<DT, D, PK>(sK, sQ, pair_i(pr), pair_j(pr), g4, c16, gk[k], gq[k]);
    }
    __syncthreads();  // K and Q are dead from here on: A overlays them
    if constexpr (raw_qk && GRP) {
        // the row norms folded into each head's vectors (as fold_qk_norms)
        for (int i = tid; i < R * kC; i += 256) {
            float *sG = sG0 + VS * (i / kC);
            const int t = i % kC;
            const float g = sG[t], ik = sIK[t], iq = sIQ[t];
            const float lk = logf(ik), lq = logf(iq), eg = __expf(g);
            sG[6 * kC + t] = g + lq;  // grP
            sG[4 * kC + t] = eg * iq; // gamq
            sG[5 * kC + t] = g + lk;  // grA
            sG[t] = g - lk;           // gc, in g's place
            sG[kC + t] = eg * ik;     // gamma
            sG[2 * kC + t] *= ik;     // dec
        }
        __syncthreads();
    }
    if constexpr (GRP) {
        // every head's P first (straight to its record), so that only the
        // K Gram products stay live through the solves
        for (int r = 0; r < R; ++r) {
            float *sG = sG0 + VS * r;  // gc in g's place
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int pr = wave + 4 * k;
                if (pr < 10)
                    mask_pair<DT, PA, PT, FRAG, raw_qk, 2>(gk[k], gq[k], pair_i(pr), pair_j(pr), g4, c16,
                                                   raw_qk ? sG + 5 * kC : sG, raw_qk ? sG + 6 * kC : sG,
                                                   sG, sG + 3 * kC, sA, sP, rec_of(r) + kFragBytes);
            }
        }
    }
    for (int r = 0; r < R; ++r) {
        float *sG = sG0 + VS * r;
        float *sGam = sG + kC, *sDec = sG + 2 * kC, *sBeta = sG + 3 * kC, *sGamQ = sG + 4 * kC;
        float *sGrA = sG + 5 * kC, *sGrP = sG + 6 * kC, *sGc = GRP ? sG : sG + 7 * kC;
        unsigned char *rec = rec_of(r);
        float *vec = vec_of(r);
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const int pr = wave + 4 * k;
            if (pr < 10)
                mask_pair<DT, PA, PT, FRAG, raw_qk, GRP ? 1 : 3>(gk[k], gq[k], pair_i(pr), pair_j(pr), g4, c16,
                                                         raw_qk ? sGrA : sG, raw_qk ? sGrP : sG,
                                                         raw_qk ? sGc : sG, sBeta, sA, sP, rec + kFragBytes);
        }
        __syncthreads();
        if (raw_qk && wave == 0) {  // raw_qk is a compile-time constant
            vec[lane] = sGam[lane];
            vec[kC + lane] = sDec[lane];
            vec[2 * kC + lane] = sBeta[lane];
            vec[3 * kC + lane] = sGamQ[lane];
        }
        // E_b overwrite the diagonal blocks of A (each is read in full first);
        // the grouped kernel reads each batch's rows when it needs them (the
        // K Gram products hold registers across its loop)
        if (wave == 0) solve_diag_blocks<DT, PA, PT, !GRP>(sA, sA, sT, g4, c16);
        __syncthreads();
        if (wave < 3) solve_column<DT, PA, PT>(sA, sA, sT, wave, g4, c16);
        __syncthreads();
        // T, P -> workspace (the next head's masks write only A; its solve
        // writes T after the barrier that follows them)
        write_tp_record<DT, D, FRAG>(rec, sT, sP, tid);
    }
}

template <typename DT, int D, int NC, int DVW> struct ChainCfg {
    using P = ChunkPitch<DT, D>;
    static constexpr int NTH = 256;
    static constexpr int DVS = NC * DVW;
    static constexpr int PV = DVS + 4;
    static constexpr int SZ_K = kC * P::PK * (int)sizeof(DT);
    static constexpr int SZ_KT = P::BF ? D * P::PT * 2 : 0;
    static constexpr int SZ_V = P::BF ? DVS * P::PT * 2 : kC * PV * 4;
    static constexpr int SZ_T = kC * P::PT * (int)sizeof(DT);
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_K;
    static constexpr int OFF_KT = OFF_Q + SZ_K;
    static constexpr int OFF_V = OFF_KT + SZ_KT;
    static constexpr int OFF_T = OFF_V + SZ_V;
    static constexpr int OFF_P = OFF_T + SZ_T;
    static constexpr int OFF_VEC = OFF_P + SZ_T;  // gamma, dec, beta
    static constexpr int LDS = OFF_VEC + 4 * kC * 4;
    // T and P pieces (16 bytes) per thread, decay-vector pieces
    static constexpr int EPP = 16 / (int)sizeof(DT);
    static constexpr int TP_PIECES = kC * kC / EPP;
    static constexpr int NTP = (TP_PIECES + NTH - 1) / NTH;
    static constexpr int VEC_PIECES = 4 * kC / 4;
    static_assert(NC >= 1 && NC <= 4 && DVW % 16 == 0, "chain waves");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// One workgroup (4 waves) per (sequence, value head, slice of DVS columns);
// waves 0..NC-1 own DVW columns each and run the state chain, all four waves
// stage the next chunk.
template <typename DT, int D, int NC, int DVW, bool PREFIX>
__global__ __launch_bounds__(256) void chain_kernel(PrefillParams p, const unsigned char *ws,
                                                    int nsplit, int remap_xcd) {
    using Cf = ChainCfg<DT, D, NC, DVW>;
    using Pi = ChunkPitch<DT, D>;
    constexpr int NKT = D / 16, NB = DVW / 16, KS = D / 32;
    constexpr int PK = Pi::PK, PT = Pi::PT, PV = Cf::PV, EPP = Cf::EPP;
    constexpr int WSB = ws_bytes_per_chunk<DT>();

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS];
    DT *sK = reinterpret_cast<DT *>(smem + Cf::OFF_K);
    DT *sQ = reinterpret_cast<DT *>(smem + Cf::OFF_Q);
    DT *sKT = reinterpret_cast<DT *>(smem + Cf::OFF_KT);
    DT *sV = reinterpret_cast<DT *>(smem + Cf::OFF_V);
    DT *sT = reinterpret_cast<DT *>(smem + Cf::OFF_T);
    DT *sP = reinterpret_cast<DT *>(smem + Cf::OFF_P);
    float *sVec = reinterpret_cast<float *>(smem + Cf::OFF_VEC);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    const int wg = logical_wg(remap_xcd);
    const int slice = wg % nsplit;
    const int nh = wg / nsplit;
    const int h = nh % p.Hv;
    const int n = nh / p.Hv;
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int dv0 = slice * Cf::DVS;
    const int wdv = (wave < NC ? wave : 0) * DVW;
    const int64_t base = slot_base(p, n);

    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const DT *qh = reinterpret_cast<const DT *>(p.q) + tok0 * sQK + (int64_t)grp * D;
    const DT *kh = reinterpret_cast<const DT *>(p.k) + tok0 * sQK + (int64_t)grp * D;
    const int64_t sVt = p.v_stride;
    const DT *vh = reinterpret_cast<const DT *>(p.v) + tok0 * sVt + (int64_t)h * D + dv0;
    DT *oh = reinterpret_cast<DT *>(p.out) + tok0 * sVO + (int64_t)h * D + dv0 + wdv;

    f32x4 st[NKT][NB];
    {
        const float *s0 = p.s0 && wave < NC ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                st[a][b] = p.s0_identity ? eye4(dv0 + wdv + 16 * b + c16, 16 * a + 4 * g4)
                           : s0 ? *reinterpret_cast<const f32x4 *>(
                                      s0 + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a + 4 * g4)
                                : zero4();
    }

    Stager<DT, D, 256, Cf::DVS> sg;
    sg.init(tid);
    u32x4 rT[Cf::NTP], rP[Cf::NTP], rVec = {0u, 0u, 0u, 0u};
    auto load_chunk = [&](int64_t c) {
        const int64_t t0 = c * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
        sg.load(kh, qh, vh, t0, lenc, sQK, sVt, tid);
        const unsigned char *rec = ws + ((base + c) * p.Hv + h) * (int64_t)WSB;
#pragma unroll
        for (int i = 0; i < Cf::NTP; ++i) {
            const int pc = tid + i * 256;
            if (Cf::TP_PIECES % 256 == 0 || pc < Cf::TP_PIECES) {
                rT[i] = reinterpret_cast<const u32x4 *>(rec)[pc];
                rP[i] = reinterpret_cast<const u32x4 *>(rec + kC * kC * sizeof(DT))[pc];
            }
        }
        if (tid < Cf::VEC_PIECES)
            rVec = reinterpret_cast<const u32x4 *>(rec + 2 * kC * kC * sizeof(DT))[tid];
    };

    const int64_t nchunks = (len + kC - 1) / kC;
    PrefixRows pre(p, n, len);
    if (nchunks > 0) load_chunk(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): see prefill_kernel

    for (int64_t c = 0; c < nchunks; ++c) {
        const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
        __syncthreads();  // the previous chunk is done with LDS
        sg.store(sK, sQ, sKT, sV, lenc, tid);
#pragma unroll
        for (int i = 0; i < Cf::NTP; ++i) {
            const int pc = tid + i * 256;
            if (Cf::TP_PIECES % 256 == 0 || pc < Cf::TP_PIECES) {
                const int r = pc / (kC / EPP), col = (pc % (kC / EPP)) * EPP;
                *reinterpret_cast<u32x4 *>(sT + r * PT + col) = rT[i];
                *reinterpret_cast<u32x4 *>(sP + r * PT + col) = rP[i];
            }
        }
        if (tid < Cf::VEC_PIECES) reinterpret_cast<u32x4 *>(sVec)[tid] = rVec;
        if (c + 1 < nchunks) load_chunk(c + 1);
        __syncthreads();

        if (wave < NC) {
            const ChainSmem<DT> m{sK,   sQ,        sKT,           sV,           sT,
                                  sP,   sVec,      sVec + kC,     sVec + 2 * kC, sVec + 3 * kC};
            Frag<DT> sf[KS][NB];
            f32x4 racc[4][NB], oT[4][NB];
            chain_state_half<DT, D, NB, PK>(m, st, sf, racc, oT, g4, c16);
            chain_finish<DT, D, NB, PK, PT, PV>(m, st, racc, oT, wdv, oh + c * kC * sVO, sVO, lenc,
                                                p.scale, g4, c16);
            const int64_t prow = PREFIX ? pre.take(p, c) : -1;
            if (prow >= 0) {
                float *ps = p.prefix + (prow * p.Hv + h) * D * D;
#pragma unroll
                for (int a = 0; a < NKT; ++a)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        __builtin_nontemporal_store(
                            st[a][b], reinterpret_cast<f32x4 *>(ps + (int64_t)(dv0 + wdv + 16 * b +
                                                                               c16) * D +
                                                                16 * a + 4 * g4));
            }
        }
    }

    if (p.s_final && wave < NC) {
        float *sf = p.s_final + ((int64_t)n * p.Hv + h) * D * D;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<f32x4 *>(sf + (int64_t)(dv0 + wdv + 16 * b + c16) * D + 16 * a +
                                           4 * g4) = st[a][b];
    }
}

// Double-buffered two-pass chain (bf16). Wave roles, per workgroup of
// NW = 2 NC + 1 + NH waves owning DVS = 16 NC value columns of one head:
//   waves 0 .. NC-1        chain: K S^T, R, U = T R, state update (the
//                          sequential part); each owns 16 value columns;
//   waves NC .. 2 NC-1     output: O for the same columns from the chain
//                          wave's S^T and U, handed over through LDS;
//   wave 2 NC              L2 prefetch: touches the lines of chunk
//                          c + 1 + DEPTH + PF_AHEAD once per owner workgroup;
//   the rest               helpers: copy chunk c + 1 into the other LDS buffer
//                          while chunk c is processed.
// One barrier per chunk. K, Q and V are staged as unpadded rows whose 16-byte
// pieces are permuted per row (swz_f); the copies apply the permutation
// through their source addresses. T, P and the decay vectors are the
// workspace record copied unchanged. Every copy is one LDS-DMA load per KiB.
template <int D, int NC, int NH> struct ChainDbCfg {
    using DT = __bf16;
    static constexpr int NW = 2 * NC + 1 + NH;
    static constexpr int NTHH = NH * 64;
    static constexpr int DVS = 16 * NC;
    static constexpr int DEPTH = 1;
    static constexpr int PF_AHEAD = 4;   // chunks a line is touched ahead of its load
    static constexpr int PF_LOADS = 8;   // line touches per lane per chunk (at most)
    static constexpr int KR = D * 2;     // K, Q row bytes
    static constexpr int VR = DVS * 2;   // V row bytes
    static constexpr int WSB = ws_bytes_frag();
    static constexpr int SZ_K = kC * KR;
    static constexpr int SZ_V = kC * VR;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_K;
    static constexpr int OFF_V = OFF_Q + SZ_K;
    static constexpr int OFF_REC = OFF_V + SZ_V;  // the workspace record: T, P, vectors
    static constexpr int OFF_T = OFF_REC;
    static constexpr int OFF_P = OFF_T + kFragBytes;
    static constexpr int OFF_VEC = OFF_P + kFragBytes;
    static constexpr int BUF = OFF_REC + WSB;
    static constexpr int OFF_HO = 2 * BUF;          // chain -> output handoff, per chain wave
    static constexpr int OFF_FLAG = OFF_HO + NC * Handoff<D, 1>::BYTES;
    static constexpr int LDS = OFF_FLAG + 64;
    // helper copies: LDS-DMA blocks of 64 16-byte slots
    static constexpr int BLK_K = SZ_K / 1024, BLK_V = SZ_V / 1024, BLK_R = WSB / 1024;
    static constexpr int NBLK = 2 * BLK_K + BLK_V + BLK_R;  // K, Q, V, record
    static_assert(SZ_K % 1024 == 0 && SZ_V % 1024 == 0 && WSB % 1024 == 0, "whole blocks");
    static_assert(NC >= 1 && NH >= 1 && NW <= 16, "wave roles");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
    // Role of hardware wave w. Waves w and w + 4 of a workgroup share a SIMD
    // (and its MFMA unit). With two chain waves they take hardware waves 2
    // and 3, alone on their SIMDs, and the P / prefetch wave and the helper
    // pair with the output waves, which mostly wait; otherwise roles follow
    // the wave order (with four chain waves each shares with its output wave).
    static __device__ __forceinline__ int role(int w) {
        return NC == 2 && NH == 1 ? (w < 2 ? w + 2 : w < 4 ? w - 2 : w) : w;
    }
};

// The LDS buffers allow one workgroup per CU.
template <int D, int NC, int NH, bool PREFIX>
__global__ __launch_bounds__((ChainDbCfg<D, NC, NH>::NW * 64)) __attribute__((amdgpu_waves_per_eu(1, 2)))
void chain_db_kernel(PrefillParams p, const unsigned char *ws, int nsplit, int remap_xcd) {
    using DT = __bf16;
    using Cf = ChainDbCfg<D, NC, NH>;
    constexpr int NKT = D / 16;
    constexpr int DEPTH = Cf::DEPTH;
    constexpr int WSB = Cf::WSB;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = Cf::role(__builtin_amdgcn_readfirstlane(tid >> 6));
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    const int wg = logical_wg(remap_xcd);
    const int slice = wg % nsplit;
    const int nh = wg / nsplit;
    const int h = nh % p.Hv;
    // dual: the second half of the chains reruns the sequences from the
    // identity state with the zero v row
    const bool second = p.dual && nh / p.Hv >= p.nseq;
    const int n = nh / p.Hv - (second ? p.nseq : 0);
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int dv0 = slice * Cf::DVS;
    const int64_t base = slot_base(p, n);
    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const int64_t nchunks = (len + kC - 1) / kC;
    // this launch's chunks [cb, cb + npc) of the sequence; loop indices below
    // count from cb (flags, handoff slots, LDS buffers), addresses use cb + c
    const int64_t cb = p.chunk0;
    const int64_t ce = p.chunk_end > 0 && p.chunk_end < nchunks ? p.chunk_end : nchunks;
    const int64_t npc = ce > cb ? ce - cb : 0;
    int *flags = reinterpret_cast<int *>(smem + Cf::OFF_FLAG);

    auto smem_view = [&](int64_t c) {
        const unsigned char *b = smem + (c & 1) * Cf::BUF;
        const float *vec = reinterpret_cast<const float *>(b + Cf::OFF_VEC);
        return DbSmem{reinterpret_cast<const DT *>(b + Cf::OFF_K),
                      reinterpret_cast<const DT *>(b + Cf::OFF_Q),
                      reinterpret_cast<const DT *>(b + Cf::OFF_V),
                      b + Cf::OFF_T, b + Cf::OFF_P,
                      vec, vec + kC, vec + 2 * kC, vec + 3 * kC};
    };

    if (wave < 2 * NC) {
        const int w = wave < NC ? wave : wave - NC;  // column group
        const int wdv = 16 * w;
        Handoff<D, 1> ho(smem + Cf::OFF_HO + w * Handoff<D, 1>::BYTES);
        int *flag = flags + w;
        if (wave < NC) {
            // chain wave: the sequential path, so it wins instruction issue
            // (and with it LDS request) arbitration against the other waves
            __builtin_amdgcn_s_setprio(3);
            f32x4 st[NKT][1];
            const float *s0 = p.s0 && !second ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                st[a][0] = p.s0_identity || second ? eye4(dv0 + wdv + c16, 16 * a + 4 * g4)
                           : s0 ? *reinterpret_cast<const f32x4 *>(
                                      s0 + (int64_t)(dv0 + wdv + c16) * D + 16 * a + 4 * g4)
                                : zero4();
            if (lane == 0) *flag = 0;
            PrefixRows pre(p, n, len);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): initial state; see prefill_kernel
            __syncthreads();
            for (int64_t c = 0; c < npc; ++c) {
                chain_core_db<D, Cf::DVS, 1, (Cf::NW > 8)>(smem_view(c), st, wdv, ho, flag, (int)c,
                                                           g4, c16, lane);
                const int64_t prow = PREFIX ? pre.take(p, cb + c) : -1;
                if (prow >= 0) {
                    float *ps = p.prefix + (prow * p.Hv + h) * D * D;
#pragma unroll
                    for (int a = 0; a < NKT; ++a)
                        __builtin_nontemporal_store(
                            st[a][0], reinterpret_cast<f32x4 *>(ps + (int64_t)(dv0 + wdv + c16) * D +
                                                                16 * a + 4 * g4));
                }
                __syncthreads();
            }
            float *sfin = second ? p.s_final2 : p.s_final;
            if (sfin) {
                float *sf = sfin + ((int64_t)n * p.Hv + h) * D * D;
#pragma unroll
                for (int a = 0; a < NKT; ++a)
                    *reinterpret_cast<f32x4 *>(sf + (int64_t)(dv0 + wdv + c16) * D + 16 * a +
                                               4 * g4) = st[a][0];
            }
        } else {
            // output wave
            DT *oh = reinterpret_cast<DT *>(second ? p.out2 : p.out) + tok0 * sVO + (int64_t)h * D +
                     dv0 + wdv;
            __syncthreads();
            OutCarry<D, 1> carry;
            auto lenc_of = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
            for (int64_t c = 0; c < npc; ++c) {
                const int64_t cp = cb + (c > 0 ? c - 1 : 0);
                out_step<D, 1, (Cf::NW > 8)>(smem_view(c), ho, flag, (int)c, carry, oh + cp * kC * sVO, sVO,
                               lenc_of(cp), p.scale, g4, c16, lane, p.status);
                __syncthreads();
            }
            if (npc > 0)
                out_tail<D, 1>(ho, flag, (int)npc - 1, carry, oh + (ce - 1) * kC * sVO,
                               sVO, lenc_of(ce - 1), p.scale, g4, c16, lane, p.status);
        }
        return;
    }

    if (wave == 2 * NC) {
        // L2 prefetch wave: the lines of chunk c + LEAD are touched in
        // iteration c, spread over the workgroups that share them (consecutive
        // logical ids, so one XCD and one L2): the K and Q lines of q/k head
        // grp over its G value heads x nsplit slices, the V and workspace-record
        // lines of head h over its slices. One CU misses L2 at a limited rate,
        // so lines left to a single owner would arrive late. A touch is a
        // 4-byte load whose value is folded into a dummy one iteration later
        // (the load has long completed by then).
        constexpr int NL = Cf::PF_LOADS;
        constexpr int LEAD = 1 + DEPTH + Cf::PF_AHEAD;  // chunk touched in iteration c: c + LEAD
        constexpr int QKL = D * 2 / 128;                // lines per K, Q or V (head) row
        constexpr int NQKL = 2 * QKL * kC, NVL = QKL * kC, NRL = WSB / 128;
        static_assert(D * 2 % 128 == 0 && WSB % 128 == 0, "whole lines");
        static_assert(NL * 64 >= NQKL + NVL + NRL, "touch budget of a workgroup alone");
        const int G = p.Hv / p.Hk;
        const int nsh = G * nsplit;               // workgroups sharing K and Q
        const int rq = (h % G) * nsplit + slice;  // this one among them
        const int nqk = (NQKL - rq + nsh - 1) / nsh;      // lines rq, rq + nsh, ...
        const int nv = (NVL - slice + nsplit - 1) / nsplit;  // lines slice, slice + nsplit, ...
        const int ntot = nqk + nv + (NRL - slice + nsplit - 1) / nsplit;
        const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k) +
                                  (tok0 * sQK + (int64_t)grp * D) * 2;
        const unsigned char *qb = reinterpret_cast<const unsigned char *>(p.q) +
                                  (tok0 * sQK + (int64_t)grp * D) * 2;
        const int64_t vstride = second ? 0 : p.v_stride;
        const unsigned char *vhb = reinterpret_cast<const unsigned char *>(second ? p.v2 : p.v) +
                                   (tok0 * vstride + (int64_t)h * D) * 2;
        const int64_t rowqk = sQK * 2, rowv = vstride * 2;
        uint32_t pend[NL], acc = 0;
#pragma unroll
        for (int j = 0; j < NL; ++j) pend[j] = 0;
        auto touch = [&](int64_t c) {
            const int64_t t0 = c * kC;
            const int rows = c < nchunks ? (int)((len - t0) < kC ? (len - t0) : kC) : 0;
            const unsigned char *rec = ws + ((base + c) * p.Hv + h) * (int64_t)WSB;
            // three waves per SIMD: line offsets recomputed per chunk (see copy_chunk)
            int ln = lane;
            if constexpr (Cf::NW > 8) asm volatile("" : "+v"(ln));
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                if (64 * j >= ntot) break;  // uniform over the wave
                const int i = ln + 64 * j;
                const unsigned char *a = kb;  // lanes without a line re-touch row 0
                if (i < nqk) {
                    const int L = rq + nsh * i, mat = L / (QKL * kC), w = L % (QKL * kC);
                    const int r = w / QKL, part = w % QKL;
                    if (r < rows) a = (mat ? qb : kb) + (t0 + r) * rowqk + part * 128;
                } else if (i < nqk + nv) {
                    const int L = slice + nsplit * (i - nqk), r = L / QKL, part = L % QKL;
                    if (r < rows) a = vhb + (t0 + r) * rowv + part * 128;
                } else if (i < ntot && rows > 0) {
                    a = rec + (int64_t)(slice + nsplit * (i - nqk - nv)) * 128;
                }
                acc ^= pend[j];
                pend[j] = *reinterpret_cast<const uint32_t *>(a);
            }
        };
        // chunk c + 1 + DEPTH is loaded by the helpers in iteration c and was
        // touched PF_AHEAD iterations earlier (chunks 1 + DEPTH .. LEAD - 1
        // here). The dummy line, row 0 of the sequence, exists only if the
        // sequence is not empty.
        if (npc > 0) {
#pragma unroll
            for (int j = 1 + DEPTH; j < LEAD; ++j) touch(cb + j);
        }
        __syncthreads();
        for (int64_t c = 0; c < npc; ++c) {
            touch(cb + c + LEAD);
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) acc ^= pend[j];
        asm volatile("" ::"v"(acc));  // keeps the touches
        return;
    }

    // the copies come next after the chain waves
    __builtin_amdgcn_s_setprio(2);
    // helper waves: copy chunk c + 1 into the other buffer with LDS-DMA loads
    // (global -> LDS without registers). Block j of a chunk is issued by
    // helper j % NH; rows past the end of the sequence repeat its last row
    // (finite values that the decay and beta of those rows cancel exactly).
    const int hw = wave - (2 * NC + 1);
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(p.q) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const int64_t vstride = second ? 0 : p.v_stride;
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(second ? p.v2 : p.v) +
                              (tok0 * vstride + (int64_t)h * D + dv0) * 2;
    const int64_t rowqk = sQK * 2, rowv = vstride * 2;
    // one 1 KiB block: slots 64 b .. 64 b + 63 of a swizzled region with rows
    // of ROWB bytes; LDS slot s of row r receives data piece s ^ swz_f(r),
    // src(row, piece) gives its address
    auto block = [&](unsigned char *dst, int b, int ln, auto rowb_c, auto src) {
        constexpr int ROWB = decltype(rowb_c)::value, NP = ROWB / 16;
        const int slot = 64 * b + ln;
        const int row = slot / NP;
        const int pc = (slot % NP) ^ swz_f<ROWB>(row % 16);
        dma16(src(row, pc), dst + 1024 * b);
    };
    using KR_c = std::integral_constant<int, Cf::KR>;
    using VR_c = std::integral_constant<int, Cf::VR>;
    auto copy_chunk = [&](int64_t c) {  // c counts from cb
        unsigned char *buf = smem + (c & 1) * Cf::BUF;
        const int64_t t0 = (cb + c) * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
        const unsigned char *rec = ws + ((base + cb + c) * p.Hv + h) * (int64_t)WSB;
        auto srcK = [&](int row, int pc) { return kb + (t0 + min(row, lenc - 1)) * rowqk + 16 * pc; };
        auto srcQ = [&](int row, int pc) { return qb + (t0 + min(row, lenc - 1)) * rowqk + 16 * pc; };
        auto srcV = [&](int row, int pc) { return vb + (t0 + min(row, lenc - 1)) * rowv + 16 * pc; };
        // With three waves per SIMD (168 registers each) the per-block
        // offsets do not fit when hoisted out of the chunk loop: there the
        // lane index is made opaque so that they are recomputed each chunk.
        int ln = lane;
        if constexpr (Cf::NW > 8) asm volatile("" : "+v"(ln));
        constexpr int J1 = Cf::BLK_K, J2 = 2 * Cf::BLK_K, J3 = J2 + Cf::BLK_V;
#pragma unroll
        for (int j = 0; j < Cf::NBLK; ++j) {
            if (j % NH != hw) continue;  // uniform over the wave
            if (j < J1) {
                block(buf + Cf::OFF_K, j, ln, KR_c{}, srcK);
            } else if (j < J2) {
                block(buf + Cf::OFF_Q, j - J1, ln, KR_c{}, srcQ);
            } else if (j < J3) {
                block(buf + Cf::OFF_V, j - J2, ln, VR_c{}, srcV);
            } else {
                dma16(rec + 1024 * (j - J3) + 16 * ln, buf + Cf::OFF_REC + 1024 * (j - J3));
            }
        }
    };
    if (npc > 0) copy_chunk(0);
    __syncthreads();  // waits for this wave's copies, then the workgroup barrier
    for (int64_t c = 0; c < npc; ++c) {
        if (c + 1 < npc) copy_chunk(c + 1);
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// launch

template <typename DT, int D, int NW, int DVW, bool PREFIX, bool RAWQK>
static void launch_fused_as(const PrefillParams &p, int nsplit, int64_t nblocks,
                            hipStream_t stream) {
    hipLaunchKernelGGL((prefill_kernel<DT, D, NW, DVW, PREFIX, RAWQK>), dim3((unsigned)nblocks),
                       dim3(NW * 64), 0, stream, p, nsplit, nblocks % 8 == 0 ? 1 : 0);
}

template <typename DT, int D, int NW, int DVW>
static hipError_t launch_fused(const PrefillParams &p, int nsplit, hipStream_t stream) {
    if (p.dual) return hipErrorInvalidValue;  // the double-buffered chain only
    const int64_t nblocks = (int64_t)p.nseq * p.Hv * nsplit;
    if (nblocks <= 0 || nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const bool raw = p.flags & kQkL2Norm;
    if (p.prefix) {
        if (raw) launch_fused_as<DT, D, NW, DVW, true, true>(p, nsplit, nblocks, stream);
        else launch_fused_as<DT, D, NW, DVW, true, false>(p, nsplit, nblocks, stream);
    } else {
        if (raw) launch_fused_as<DT, D, NW, DVW, false, true>(p, nsplit, nblocks, stream);
        else launch_fused_as<DT, D, NW, DVW, false, false>(p, nsplit, nblocks, stream);
    }
    return hipGetLastError();
}

// The records of nslots chunk slots. Fragment records for 2 .. kPrepGrpMax
// value heads per q/k head take one workgroup per (slot, q/k head), which
// shares the K, Q staging and Gram products among those heads (GDN_PREP=1:
// one workgroup per value head, as for every other case).
template <typename DT, int D, bool FRAG>
static hipError_t launch_prep(const PrefillParams &p, unsigned char *ws, int64_t nslots,
                              hipStream_t stream) {
    if (p.records_ready) return hipSuccess;
    const int R = p.Hv / p.Hk;
    const char *pe = getenv("GDN_PREP");
    const bool grp = FRAG && R >= 2 && R <= kPrepGrpMax && !(pe && pe[0] == '1');
    const int64_t nprep = nslots * (grp ? p.Hk : p.Hv);
    if (nprep <= 0 || nprep > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 g((unsigned)nprep), b(256);
    const int remap = nprep % 8 == 0 ? 1 : 0;
    const bool raw = p.flags & kQkL2Norm;
    if constexpr (FRAG) {
        if (grp) {
            if (raw)
                hipLaunchKernelGGL((prep_kernel<DT, D, FRAG, true, true>), g, b, 0, stream, p, ws, remap);
            else
                hipLaunchKernelGGL((prep_kernel<DT, D, FRAG, false, true>), g, b, 0, stream, p, ws, remap);
            return hipGetLastError();
        }
    }
    if (raw)
        hipLaunchKernelGGL((prep_kernel<DT, D, FRAG, true, false>), g, b, 0, stream, p, ws, remap);
    else
        hipLaunchKernelGGL((prep_kernel<DT, D, FRAG, false, false>), g, b, 0, stream, p, ws, remap);
    return hipGetLastError();
}

template <typename DT, int D, int NC, int DVW>
static hipError_t launch_split(const PrefillParams &p, unsigned char *ws, int64_t nslots,
                               int nsplit, hipStream_t stream) {
    if (p.dual) return hipErrorInvalidValue;  // the double-buffered chain only
    const int64_t nprep = nslots * p.Hv;
    const int64_t nchain = (int64_t)p.nseq * p.Hv * nsplit;
    if (nprep <= 0 || nprep > 0x7FFFFFFF || nchain <= 0 || nchain > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipError_t e = launch_prep<DT, D, false>(p, ws, nslots, stream);
    if (e != hipSuccess) return e;
    if (p.prefix)
        hipLaunchKernelGGL((chain_kernel<DT, D, NC, DVW, true>), dim3((unsigned)nchain), dim3(256),
                           0, stream, p, (const unsigned char *)ws, nsplit,
                           nchain % 8 == 0 ? 1 : 0);
    else
        hipLaunchKernelGGL((chain_kernel<DT, D, NC, DVW, false>), dim3((unsigned)nchain), dim3(256),
                           0, stream, p, (const unsigned char *)ws, nsplit,
                           nchain % 8 == 0 ? 1 : 0);
    return hipGetLastError();
}

template <int D, int NC, int NH>
static hipError_t launch_split_db(const PrefillParams &p, unsigned char *ws, int64_t nslots,
                                  int nsplit, hipStream_t stream) {
    const int64_t nprep = nslots * p.Hv;
    const int64_t nchain = (int64_t)p.nseq * p.Hv * nsplit * (p.dual ? 2 : 1);
    if (nprep <= 0 || nprep > 0x7FFFFFFF || nchain <= 0 || nchain > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    if (ChainDbCfg<D, NC, NH>::DVS * nsplit != D) return hipErrorInvalidValue;
    hipError_t e = launch_prep<__bf16, D, true>(p, ws, nslots, stream);
    if (e != hipSuccess) return e;
    // the one-wave-per-SIMD chain where it applies; GDN_CHAIN=db keeps this
    // kernel (for comparisons and the tests that cover both)
    const char *ck = getenv("GDN_CHAIN");
    if (!(ck && ck[0] == 'd') && chain4_supported(p, D, nsplit))
        return launch_chain4(p, ws, nchain, stream);
    if (p.prefix)
        hipLaunchKernelGGL((chain_db_kernel<D, NC, NH, true>), dim3((unsigned)nchain),
                           dim3(ChainDbCfg<D, NC, NH>::NW * 64), 0, stream, p,
                           (const unsigned char *)ws, nsplit, nchain % 8 == 0 ? 1 : 0);
    else
        hipLaunchKernelGGL((chain_db_kernel<D, NC, NH, false>), dim3((unsigned)nchain),
                           dim3(ChainDbCfg<D, NC, NH>::NW * 64), 0, stream, p,
                           (const unsigned char *)ws, nsplit, nchain % 8 == 0 ? 1 : 0);
    return hipGetLastError();
}

int64_t prefill_ws_slots(int64_t nseq, int64_t total_tokens, int64_t seq_len, bool packed) {
    if (!packed) return nseq * ((seq_len + kC - 1) / kC);
    return (total_tokens + kC - 1) / kC + nseq;
}

size_t prefill_ws_bytes(int64_t slots, int Hv, int dtype) {
    const int per = dtype == 1 ? ws_bytes_per_chunk<__bf16>() : ws_bytes_per_chunk<float>();
    return (size_t)slots * (size_t)Hv * (size_t)per;
}

static int env_int(const char *name, int dflt) {
    const char *e = getenv(name);
    return e ? atoi(e) : dflt;
}

// The two-pass path pays off when there are too few (sequence, value head)
// chains to fill the chip with one workgroup each. GDN_PREFILL_PATH=fused or
// =split overrides the choice (for tuning).
bool prefill_wants_workspace(int64_t chains, int num_cus) {
    const char *e = getenv("GDN_PREFILL_PATH");
    if (e && e[0] == 'f') return false;
    if (e && e[0] == 's') return true;
    return chains < 2 * (int64_t)num_cus;
}

static int pow2_floor(int v) {
    int r = 1;
    while (r * 2 <= v) r *= 2;
    return r;
}

// Value-column slices per head of the two-pass chain: about one workgroup
// per CU (the double-buffered chain kernel fills a CU's LDS), at most four.
static int chain_slices(int64_t chains, int num_cus) {
    int ns = env_int("GDN_PREFILL_NSPLIT", 0);
    if (ns != 1 && ns != 2 && ns != 4 && ns != 8) {
        const int64_t want = (int64_t)num_cus / (chains > 0 ? chains : 1);
        ns = pow2_floor((int)(want < 4 ? (want < 1 ? 1 : want) : 4));
    }
    return ns;
}

// ----------------------------------------------------------------------------
// segmented prefill (gdn_segment.hip): few long sequences, split into P
// segments of L tokens (L a multiple of 64) that run as a packed batch.

struct SegPlan {
    int32_t P = 0;  // segments per sequence (0: not segmented)
    int64_t L = 0;  // tokens per segment (the last may be shorter)
};

// Segments when the plain two-pass path would leave most CUs idle: at most
// num_cus / 8 (sequence, value head) chains and at least 8 chunks each. The
// two passes cost about 3 us per chunk of a segment and the scan about 2.3 us
// per segment (measured at D = 128), so P is near sqrt(1.3 * chunks), and at
// most what fills the chip at 4 value-column slices per chain.
// GDN_PREFILL_SEGMENTS = 0 disables it, = P forces P segments (any dense
// bf16 batch, for tests).
static SegPlan seg_plan(int64_t nseq, int64_t T, int Hv, int D, int dtype, int num_cus) {
    SegPlan sp;
    if (dtype != 1 || (D != 64 && D != 128) || T <= 0) return sp;
    const int64_t chains = nseq * Hv;
    const int64_t nchunks = (T + kC - 1) / kC;
    const int forced = env_int("GDN_PREFILL_SEGMENTS", -1);
    int64_t P;
    if (forced == 0) return sp;
    if (forced > 0) {
        P = forced;
    } else {
        if (chains * 8 > num_cus || nchunks < 8) return sp;
        // P from a cost model of the parts, measured on the MI355X: per
        // 64-token chunk of a segment ~1.6 / 2.4 / 5.8 us on the chain at
        // 4 / 2 / 1 value-column slices per head (twice that when the two
        // segment passes cannot run as one launch), ~1.9 us per scan step,
        // ~15 us of setup, scan start and corrections; against one pass.
        auto chunk_us = [](int ns) { return ns >= 4 ? 1.6 : ns == 2 ? 2.4 : 5.8; };
        const int64_t pmax = (int64_t)num_cus / 4 / chains < nchunks / 2
                                 ? (int64_t)num_cus / 4 / chains
                                 : nchunks / 2;
        double best_t = (double)nchunks * chunk_us(chain_slices(chains, num_cus));
        P = 0;
        for (int64_t q = 2; q <= pmax; ++q) {
            const int64_t lc = (nchunks + q - 1) / q;
            const int ns2 = chain_slices(2 * q * chains, num_cus);
            const bool merged = D == 64 || ns2 >= 2;
            const int ns = merged ? ns2 : chain_slices(q * chains, num_cus);
            const double t = (merged ? 1 : 2) * lc * chunk_us(ns) + 1.9 * q + 15.0;
            if (t < best_t) {
                best_t = t;
                P = q;
            }
        }
        if (P == 0) return sp;
    }
    if (P < 2 || P > nchunks) return sp;
    const int64_t lc = (nchunks + P - 1) / P;  // chunks per segment
    sp.P = (int32_t)((nchunks + lc - 1) / lc);
    sp.L = lc * kC;
    if (sp.P < 2 || nseq * sp.P > 0x7FFFFFFF / 8) sp.P = 0;
    return sp;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The two-pass chain on the double-buffered kernel: one prep launch over all
// chunks, then one chain launch.
template <int D, int NC, int NH>
static hipError_t run_split_db(const PrefillParams &p, unsigned char *ws, int64_t nslots,
                               int nsplit, hipStream_t stream) {
    return launch_split_db<D, NC, NH>(p, ws, nslots, nsplit, stream);
}

struct SegLayout {
    size_t rec, cu, zero_v, n_end, m_end, s_start, o_id, total;
};

static SegLayout seg_layout(int64_t nseq, int64_t T, int Hv, int D, const SegPlan &sp) {
    SegLayout l{};
    const int64_t nsegs = nseq * sp.P;
    const size_t states = (size_t)nsegs * Hv * D * D * 4;
    size_t off = 0;
    l.rec = off;
    off += align256(prefill_ws_bytes(prefill_ws_slots(nsegs, nseq * T, 0, true), Hv, 1));
    l.cu = off;
    off += align256((size_t)(nsegs + 1) * 4);
    l.zero_v = off;
    off += align256((size_t)Hv * D * 2);
    l.n_end = off;
    off += align256(states);
    l.m_end = off;
    off += align256(states);
    l.s_start = off;
    off += align256(states);
    l.o_id = off;
    off += align256((size_t)nseq * T * Hv * D * 2);
    l.total = off;
    return l;
}

size_t prefill_seg_ws_bytes(int64_t nseq, int64_t T, int Hv, int D, int dtype, int num_cus) {
    const SegPlan sp = seg_plan(nseq, T, Hv, D, dtype, num_cus);
    return sp.P ? seg_layout(nseq, T, Hv, D, sp).total : 0;
}

static hipError_t launch_prefill_ws(const PrefillParams &p, int dtype, int D, int num_cus,
                                   void *ws, size_t ws_bytes, int64_t nslots, hipStream_t stream);

static hipError_t launch_segmented(const PrefillParams &p, int D, int num_cus, unsigned char *ws,
                                   const SegPlan &sp, hipStream_t stream) {
    const int64_t B = p.nseq, T = p.seq_len;
    const int32_t nsegs = (int32_t)(B * sp.P);
    const SegLayout l = seg_layout(B, T, p.Hv, D, sp);
    int32_t *cu = reinterpret_cast<int32_t *>(ws + l.cu);
    __bf16 *zero_v = reinterpret_cast<__bf16 *>(ws + l.zero_v);
    float *n_end = reinterpret_cast<float *>(ws + l.n_end);
    float *m_end = reinterpret_cast<float *>(ws + l.m_end);
    float *s_start = reinterpret_cast<float *>(ws + l.s_start);
    __bf16 *o_id = reinterpret_cast<__bf16 *>(ws + l.o_id);
    hipError_t e = launch_segment_setup(cu, (int32_t)B, sp.P, T, sp.L, zero_v, p.Hv * D, stream);
    if (e != hipSuccess) return e;
    const int64_t slots = prefill_ws_slots(nsegs, B * T, 0, true);
    const size_t rec_bytes = prefill_ws_bytes(slots, p.Hv, 1);
    // 1. every segment from a zero state: outputs o^0 (into out), end states N_j
    PrefillParams pz = p;
    pz.cu_seqlens = cu;
    pz.total_tokens = B * T;
    pz.nseq = nsegs;
    pz.seq_len = 0;
    pz.s0 = nullptr;
    pz.s_final = n_end;
    // 2. every segment from the identity with v = 0: outputs M_{->t} q_t, end states M_j.
    // Steps 1 and 2 share the per-chunk records and are independent, so on
    // the double-buffered chain they run as one launch over twice the chains
    // (half the value-column slices each, so that the launch fits the chip
    // once); otherwise one after the other.
    const int64_t chains2 = (int64_t)2 * nsegs * p.Hv;
    const char *path = getenv("GDN_PREFILL_PATH");
    const bool merge = env_int("GDN_PREFILL_SEG_MERGE", 1) != 0 && !(path && path[0] == 'f') &&
                       prefill_wants_workspace(chains2, num_cus) &&
                       (D == 64 || chain_slices(chains2, num_cus) >= 2);
    if (merge) {
        pz.dual = true;
        pz.v2 = zero_v;
        pz.out2 = o_id;
        pz.s_final2 = m_end;
    }
    e = launch_prefill_ws(pz, 1, D, num_cus, ws + l.rec, rec_bytes, slots, stream);
    if (e != hipSuccess) return e;
    if (!merge) {
        PrefillParams pi = pz;
        pi.v = zero_v;
        pi.v_stride = 0;
        pi.s0_identity = true;
        pi.records_ready = true;  // same q, k, alpha, beta and slots as step 1
        pi.out = o_id;
        pi.s_final = m_end;
        e = launch_prefill_ws(pi, 1, D, num_cus, ws + l.rec, rec_bytes, slots, stream);
        if (e != hipSuccess) return e;
    }
    // 3. the scan over segments; 4. the corrections (segment 0 only from a
    // nonzero initial state)
    e = launch_segment_scan(p.s0, n_end, m_end, s_start, p.s_final, (int32_t)B, sp.P, p.Hv, D,
                            stream);
    if (e != hipSuccess) return e;
    return launch_segment_correct(static_cast<__bf16 *>(p.out), o_id, s_start, cu, (int32_t)B,
                                  sp.P, p.Hv, sp.L, p.s0 ? 0 : 1, D, stream);
}

static hipError_t launch_prefill_ws(const PrefillParams &p, int dtype, int D, int num_cus,
                                   void *ws, size_t ws_bytes, int64_t nslots, hipStream_t stream) {
    if (!p.cu_seqlens && !p.prefix && !p.s0_identity && ws) {
        const SegPlan sp = seg_plan(p.nseq, p.seq_len, p.Hv, D, dtype, num_cus);
        if (sp.P && ws_bytes >= seg_layout(p.nseq, p.seq_len, p.Hv, D, sp).total)
            return launch_segmented(p, D, num_cus, static_cast<unsigned char *>(ws), sp, stream);
    }
    const int64_t chains = (int64_t)p.nseq * p.Hv * (p.dual ? 2 : 1);
    const bool split = ws != nullptr && nslots > 0 &&
                       ws_bytes >= prefill_ws_bytes(nslots, p.Hv, dtype) &&
                       prefill_wants_workspace(chains, num_cus);
    if (split) {
        // Value-column slices per head: about one workgroup per CU (the
        // double-buffered chain kernel fills a CU's LDS), at most four.
        const int ns = chain_slices(chains, num_cus);
        unsigned char *w = static_cast<unsigned char *>(ws);
        if (dtype == 1 && D == 128) {
            switch (ns) {
            case 1: return launch_split<__bf16, 128, 4, 32>(p, w, nslots, 1, stream);
            case 2: return run_split_db<128, 4, 1>(p, w, nslots, 2, stream);
            case 4: return run_split_db<128, 2, 1>(p, w, nslots, 4, stream);
            default: return run_split_db<128, 1, 1>(p, w, nslots, 8, stream);
            }
        } else if (dtype == 1 && D == 64) {
            switch (ns) {
            case 1: return run_split_db<64, 4, 1>(p, w, nslots, 1, stream);
            case 2: return run_split_db<64, 2, 1>(p, w, nslots, 2, stream);
            default: return run_split_db<64, 1, 1>(p, w, nslots, 4, stream);
            }
        } else if (dtype == 0 && D == 64) {
            switch (ns) {
            case 1: return launch_split<float, 64, 4, 16>(p, w, nslots, 1, stream);
            case 2: return launch_split<float, 64, 2, 16>(p, w, nslots, 2, stream);
            default: return launch_split<float, 64, 1, 16>(p, w, nslots, 4, stream);
            }
        } else if (dtype == 0 && D == 128) {
            switch (ns) {
            case 1:
            case 2: return launch_split<float, 128, 4, 16>(p, w, nslots, 2, stream);
            case 4: return launch_split<float, 128, 2, 16>(p, w, nslots, 4, stream);
            default: return launch_split<float, 128, 1, 16>(p, w, nslots, 8, stream);
            }
        }
        return hipErrorInvalidValue;
    }

    // Fused: with many chains a workgroup takes a whole head; with few, the
    // head is split so that more CUs work.
    int ns = env_int("GDN_PREFILL_NSPLIT", 0);
    if (ns != 1 && ns != 2 && ns != 4 && ns != 8)
        ns = chains >= num_cus ? 1 : chains * 2 >= num_cus ? 2 : (D == 128 ? 4 : 2);
    if (D == 64 && ns == 8) ns = 4;
    if (dtype == 1) {
        if (D == 128) {
            switch (ns) {
            case 1: {
                // GDN_FUSED=old keeps the eight-wave kernel (for comparison)
                const char *fe = getenv("GDN_FUSED");
                if (!(fe && fe[0] == 'o') && fused2_supported(p, dtype, D)) return launch_fused2(p, stream);
                return launch_fused<__bf16, 128, 8, 16>(p, 1, stream);
            }
            case 2: return launch_fused<__bf16, 128, 4, 16>(p, 2, stream);
            case 4: return launch_fused<__bf16, 128, 2, 16>(p, 4, stream);
            default: return launch_fused<__bf16, 128, 1, 16>(p, 8, stream);
            }
        } else if (D == 64) {
            switch (ns) {
            case 1: return launch_fused<__bf16, 64, 4, 16>(p, 1, stream);
            case 2: return launch_fused<__bf16, 64, 2, 16>(p, 2, stream);
            default: return launch_fused<__bf16, 64, 1, 16>(p, 4, stream);
            }
        }
    } else if (dtype == 0) {
        if (D == 64) {
            switch (ns) {
            case 1: return launch_fused<float, 64, 4, 16>(p, 1, stream);
            case 2: return launch_fused<float, 64, 2, 16>(p, 2, stream);
            default: return launch_fused<float, 64, 1, 16>(p, 4, stream);
            }
        } else if (D == 128) {
            // fp32 K, Q and V of a whole head exceed a CU's LDS: two slices at
            // least; a one-wave workgroup would not fit its registers
            switch (ns) {
            case 1:
            case 2: return launch_fused<float, 128, 4, 16>(p, 2, stream);
            default: return launch_fused<float, 128, 2, 16>(p, 4, stream);
            }
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillParams &p, int dtype, int D, int num_cus, void *ws,
                          size_t ws_bytes, int64_t nslots, hipStream_t stream) {
    if (!ws || ws_bytes < kWsStatusBytes) return launch_prefill_ws(p, dtype, D, num_cus, nullptr, 0,
                                                                   nslots, stream);
    PrefillParams pw = p;
    pw.status = static_cast<int *>(ws);
    return launch_prefill_ws(pw, dtype, D, num_cus, static_cast<unsigned char *>(ws) + kWsStatusBytes,
                             ws_bytes - kWsStatusBytes, nslots, stream);
}

}  // namespace gdn
