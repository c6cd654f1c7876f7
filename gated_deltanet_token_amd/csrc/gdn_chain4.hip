// gdn_chain4.hip -- the sequential state chain of the two-pass prefill for
// 32 value columns of a head, one wave per SIMD.
//
// The chunk-64 rewrite of the gated delta rule (gdn_chunk.hpp) splits each
// chunk's work into a state-free part (the decay scan, T = (I + A)^{-1} and
// the masked Q K^T, which prep_kernel writes to the workspace for all chunks
// at once) and the part that needs the state S at the chunk's start:
//     R = diag(beta) (V - diag(gamma) K S^T),   U = T R,
//     O = diag(gamma) Q S^T + P U,              S' = gamma_63 S + U^T diag(dec) K.
// Only R, U and S' are on the sequential path. This kernel walks the chunks
// of one (sequence, value head, 32-column slice) with four waves, one per
// SIMD, so that each may hold up to 512 registers:
//   wave 0, 1  chain: S^T of 16 value columns in MFMA accumulators; per
//              chunk K S^T, R, U = T R and the state update. It publishes
//              S (at the chunk's start) and U to the output wave through
//              LDS, and reads the next chunk's K fragments while its state
//              update runs (the chunk after is already in LDS);
//   wave 2     output: O for all 32 columns from the staged Q and P and the
//              published S and U; it also touches the L2 lines of the
//              chunks after the ones being copied;
//   wave 3     copies: chunk c + NBUF - 1 into the LDS ring with LDS-DMA
//              loads while chunk c is processed.
// One barrier per chunk. The state's rows (the key dimension dk) are held
// in a permuted order: state tile a, lane group g, element r is key column
// 32 (a >> 1) + 8 g + 4 (a & 1) + r. With it the eight keys that a lane
// contributes to a 32-deep MFMA step are contiguous, so the K and Q
// operands of K S^T and Q S^T are single 16-byte LDS reads; the transposing
// reads of K for the state update take the same order through their
// addresses. Loads and stores of the state map the order back.
#include <float.h>
#include <stdint.h>

#include <type_traits>

#include "gdn_chunk.hpp"
#include "gdn_launch.hpp"
#include "gdn_seq.hpp"

namespace gdn {

namespace {

template <int NBUF> struct C4 {
    static constexpr int D = 128;
    static constexpr int NC = 2;         // chain waves, 16 value columns each
    static constexpr int DVS = 16 * NC;  // value columns of a workgroup
    static constexpr int NSPLIT = D / DVS;
    static constexpr int KR = D * 2;     // K, Q row bytes
    static constexpr int VR = DVS * 2;   // V row bytes
    static constexpr int WSB = 2 * kTriFrags * 64 * 16 + 1024;  // T, P fragments, 4 vectors
    static constexpr int SZ_K = kC * KR;
    static constexpr int SZ_V = kC * VR;
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = OFF_K + SZ_K;
    static constexpr int OFF_V = OFF_Q + SZ_K;
    static constexpr int OFF_REC = OFF_V + SZ_V;
    static constexpr int OFF_T = OFF_REC;
    static constexpr int OFF_P = OFF_T + kTriFrags * 1024;
    static constexpr int OFF_VEC = OFF_P + kTriFrags * 1024;  // gam, dec, beta, gamq [64] fp32
    static constexpr int BUF = OFF_REC + WSB;
    static constexpr int HO_S = (D / 32) * 1024;  // S^T fragments of one chain wave
    static constexpr int HO_U = 2 * 1024;         // U fragments of one chain wave
    static constexpr int HO = HO_S + HO_U;
    static constexpr int OFF_HO = NBUF * BUF;
    static constexpr int OFF_FLAG = OFF_HO + NC * HO;
    static constexpr int LDS = OFF_FLAG + 64;
    static constexpr int BLK_K = SZ_K / 1024, BLK_V = SZ_V / 1024, BLK_R = WSB / 1024;
    static constexpr int NBLK = 2 * BLK_K + BLK_V + BLK_R;
    static_assert(SZ_K % 1024 == 0 && SZ_V % 1024 == 0 && WSB % 1024 == 0, "whole DMA blocks");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
    static constexpr int PF_AHEAD = 3;   // chunks a line is touched before its copy
    static constexpr int PF_LOADS = 4;   // line touches per lane per chunk (at most)
};

// Key column of state tile a (16 virtual rows), lane group g, element 0.
__device__ __forceinline__ int st_key(int a, int g) { return 32 * (a >> 1) + 8 * g + 4 * (a & 1); }

template <int NBUF, bool PREFIX>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chain4_kernel(PrefillParams p, const unsigned char *ws, int remap_xcd) {
    using Cf = C4<NBUF>;
    using DT = __bf16;
    using F = bf16x8;
    constexpr int D = Cf::D, KR = Cf::KR, VR = Cf::VR, NSPLIT = Cf::NSPLIT;
    constexpr int KS = D / 32, NKT = D / 16;

    __shared__ __attribute__((aligned(16))) unsigned char smem[Cf::LDS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4;
    const int c16 = lane & 15;

    const int wg = logical_wg(remap_xcd);
    const int slice = wg % NSPLIT;
    const int nh = wg / NSPLIT;
    const int h = nh % p.Hv;
    const int n = nh / p.Hv;
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int dv0 = slice * Cf::DVS;
    const int64_t base = slot_base(p, n);
    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const int64_t npc = (len + kC - 1) / kC;
    int *flags = reinterpret_cast<int *>(smem + Cf::OFF_FLAG);
    auto buf = [&](int64_t c) { return smem + (int)(c % NBUF) * Cf::BUF; };

    if (wave < Cf::NC) {
        // ------------------------------------------------------------ chain
        __builtin_amdgcn_s_setprio(3);
        const int wdv = 16 * wave;
        bf16x8 *ho_s = reinterpret_cast<bf16x8 *>(smem + Cf::OFF_HO + wave * Cf::HO);
        bf16x8 *ho_u = ho_s + (D / 32) * 64;
        int *flag = flags + wave;
        f32x4 st[NKT];
        {
            const float *s0 = p.s0 ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
            const int64_t row = (int64_t)(dv0 + wdv + c16) * D;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                st[a] = s0 ? *reinterpret_cast<const f32x4 *>(s0 + row + st_key(a, g4)) : zero4();
        }
        if (lane == 0) *flag = 0;
        PrefixRows pre(p, n, len);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the initial state
        __syncthreads();                      // the first chunks are staged
        // K fragments of a chunk: row 16 mt + c16, keys 32 kk + 8 g4 .. +7
        auto load_fk = [&](const unsigned char *b, F (&fk)[KS][4]) {
            const DT *K = reinterpret_cast<const DT *>(b + Cf::OFF_K);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    fk[kk][mt] = *reinterpret_cast<const F *>(swz_at<KR>(K, 16 * mt, c16, 32 * kk + 8 * g4));
        };
        F fk[KS][4];
        if (npc > 0) load_fk(buf(0), fk);
        for (int64_t c = 0; c < npc; ++c) {
            const unsigned char *b = buf(c);
            const DT *K = reinterpret_cast<const DT *>(b + Cf::OFF_K);
            const DT *V = reinterpret_cast<const DT *>(b + Cf::OFF_V);
            const F *T = reinterpret_cast<const F *>(b + Cf::OFF_T);
            const float *vec = reinterpret_cast<const float *>(b + Cf::OFF_VEC);
            // S^T at the chunk's start as B fragments, published for the output wave
            F sf[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                c_to_frag(st[2 * kk], st[2 * kk + 1], sf[kk]);
                ho_s[kk * 64 + lane] = sf[kk];
            }
            set_flag(flag, 2 * (int)c + 1);
            // operands of R, U = T R and the state update (this chunk)
            F ft[kTriFrags];
#pragma unroll
            for (int i = 0; i < kTriFrags; ++i) ft[i] = T[i * 64 + lane];
            bf16x4 v4[4];
            f32x4 bet[4], gam[4], dec[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int tb = 16 * mt + 4 * g4;
                v4[mt] = ld_tr(swz_at<VR>(V, 16 * mt, 4 * g4 + (c16 >> 2), wdv + 4 * (c16 & 3)));
                bet[mt] = *reinterpret_cast<const f32x4 *>(vec + 2 * kC + tb);
                gam[mt] = *reinterpret_cast<const f32x4 *>(vec + tb);
                dec[mt] = *reinterpret_cast<const f32x4 *>(vec + kC + tb);
            }
            const float gC = vec[kC - 1] * __builtin_amdgcn_rcpf(vec[2 * kC - 1]);
            F fkt[NKT][2];
            {
                // transposing reads of K in the state's key order: sender
                // lane c16 of group g4 points at token row r0 + (c16 >> 2),
                // key st_key(a, c16 & 3); its receivers get keys + 0 .. 3
                const int rl = 4 * g4 + (c16 >> 2);
#pragma unroll
                for (int a = 0; a < NKT; ++a)
#pragma unroll
                    for (int k2 = 0; k2 < 2; ++k2) {
                        const int col = st_key(a, c16 & 3);
                        const bf16x4 lo = ld_tr(swz_at<KR>(K, 32 * k2, rl, col));
                        const bf16x4 hi = ld_tr(swz_at<KR>(K, 32 * k2 + 16, rl, col));
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            fkt[a][k2][e] = lo[e];
                            fkt[a][k2][e + 4] = hi[e];
                        }
                    }
            }
            // K S^T
            f32x4 racc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) racc[mt] = zero4();
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) racc[mt] = mma(fk[kk][mt], sf[kk], racc[mt]);
            phase_fence();
            // the next chunk's K fragments (its buffer was filled a step ago)
            load_fk(buf(c + 1), fk);
            // R = beta (V - gamma K S^T), U = T R
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    racc[mt][r] = bet[mt][r] * ((float)v4[mt][r] - gam[mt][r] * racc[mt][r]);
            F fr[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) c_to_frag(racc[2 * k2], racc[2 * k2 + 1], fr[k2]);
            f32x4 u[4];
            u[0] = mma(ft[0], fr[0], zero4());
            u[1] = mma(ft[1], fr[0], zero4());
            u[2] = mma(ft[2], fr[0], zero4());
            u[3] = mma(ft[4], fr[0], zero4());
            u[2] = mma(ft[3], fr[1], u[2]);
            u[3] = mma(ft[5], fr[1], u[3]);
            // publish U; S^T <- gamma_C S^T + K^T diag(dec) U
            F fd[2];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                F fu;
                c_to_frag(u[2 * k2], u[2 * k2 + 1], fu);
                ho_u[k2 * 64 + lane] = fu;
                f32x4 lo = u[2 * k2], hi = u[2 * k2 + 1];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    lo[r] *= dec[2 * k2][r];
                    hi[r] *= dec[2 * k2 + 1][r];
                }
                c_to_frag(lo, hi, fd[k2]);
            }
            set_flag(flag, 2 * (int)c + 2);
#pragma unroll
            for (int a = 0; a < NKT; ++a) {
                st[a] *= gC;
#pragma unroll
                for (int k2 = 0; k2 < 2; ++k2) st[a] = mma(fkt[a][k2], fd[k2], st[a]);
            }
            const int64_t prow = PREFIX ? pre.take(p, c) : -1;
            if (prow >= 0) {
                float *ps = p.prefix + (prow * p.Hv + h) * D * D + (int64_t)(dv0 + wdv + c16) * D;
#pragma unroll
                for (int a = 0; a < NKT; ++a)
                    __builtin_nontemporal_store(st[a], reinterpret_cast<f32x4 *>(ps + st_key(a, g4)));
            }
            __syncthreads();
        }
        if (p.s_final) {
            float *sf = p.s_final + ((int64_t)n * p.Hv + h) * D * D + (int64_t)(dv0 + wdv + c16) * D;
#pragma unroll
            for (int a = 0; a < NKT; ++a) *reinterpret_cast<f32x4 *>(sf + st_key(a, g4)) = st[a];
        }
        return;
    }

    if (wave == Cf::NC) {
        // ------------------------------------------------------------ output
        __builtin_amdgcn_s_setprio(1);
        __bf16 *oh = reinterpret_cast<__bf16 *>(p.out) + tok0 * sVO + (int64_t)h * D + dv0;
        const unsigned char *qb = reinterpret_cast<const unsigned char *>(p.q) +
                                  (tok0 * sQK + (int64_t)grp * D) * 2;
        const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k) +
                                  (tok0 * sQK + (int64_t)grp * D) * 2;
        const int64_t rowqk = sQK * 2, rowv = p.v_stride * 2;
        // L2 prefetch: the lines of chunk c are touched PF_AHEAD steps before
        // their copy, spread over the workgroups that share them (consecutive
        // logical ids, so one XCD): K and Q lines over the G value heads x
        // NSPLIT slices of the q/k head, V and record lines over the slices. A
        // touch is a 4-byte load whose value is folded in two steps later, so
        // this wave never waits for it (its barriers wait for LDS only).
        constexpr int NL = Cf::PF_LOADS;
        constexpr int QKL = D * 2 / 128;
        constexpr int NQKL = 2 * QKL * kC, NVL = QKL * kC, NRL = Cf::WSB / 128;
        const int G = p.Hv / p.Hk;
        const int nsh = G * NSPLIT;
        const int rq = (h % G) * NSPLIT + slice;
        const int nqk = (NQKL - rq + nsh - 1) / nsh;
        const int nv = (NVL - slice + NSPLIT - 1) / NSPLIT;
        const int ntot = nqk + nv + (NRL - slice + NSPLIT - 1) / NSPLIT;
        const unsigned char *vhb = reinterpret_cast<const unsigned char *>(p.v) +
                                   (tok0 * p.v_stride + (int64_t)h * D) * 2;
        uint32_t pend[2][NL], tacc = 0;  // values of the last two steps' touches
#pragma unroll
        for (int j = 0; j < NL; ++j) pend[0][j] = pend[1][j] = 0;
        auto touch = [&](int64_t c, int slot) {
            const int64_t t0 = c * kC;
            const int rows = c < npc ? (int)((len - t0) < kC ? (len - t0) : kC) : 0;
            const unsigned char *rec = ws + ((base + c) * p.Hv + h) * (int64_t)Cf::WSB;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                if (64 * j >= ntot) break;  // uniform over the wave
                const int i = lane + 64 * j;
                const unsigned char *a = kb;  // lanes without a line re-touch row 0
                if (i < nqk) {
                    const int L = rq + nsh * i, mat = L / (QKL * kC), w = L % (QKL * kC);
                    const int r = w / QKL, part = w % QKL;
                    if (r < rows) a = (mat ? qb : kb) + (t0 + r) * rowqk + part * 128;
                } else if (i < nqk + nv) {
                    const int L = slice + NSPLIT * (i - nqk), r = L / QKL, part = L % QKL;
                    if (r < rows) a = vhb + (t0 + r) * rowv + part * 128;
                } else if (i < ntot && rows > 0) {
                    a = rec + (int64_t)(slice + NSPLIT * (i - nqk - nv)) * 128;
                }
                tacc ^= pend[slot][j];
                pend[slot][j] = *reinterpret_cast<const uint32_t *>(a);
            }
        };
        constexpr int LEAD = NBUF - 1 + Cf::PF_AHEAD;  // chunk touched in step c: c + LEAD
        for (int j = NBUF - 1; j < LEAD; ++j) touch(j, j & 1);
        __syncthreads();
        auto load_q = [&](const unsigned char *b, F (&fq)[KS][4]) {
            const DT *Q = reinterpret_cast<const DT *>(b + Cf::OFF_Q);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    fq[kk][mt] = *reinterpret_cast<const F *>(swz_at<KR>(Q, 16 * mt, c16, 32 * kk + 8 * g4));
        };
        F fq[KS][4];
        if (npc > 0) load_q(buf(0), fq);
        for (int64_t c = 0; c < npc; ++c) {
            const unsigned char *b = buf(c);
            const F *P = reinterpret_cast<const F *>(b + Cf::OFF_P);
            const float *gamq = reinterpret_cast<const float *>(b + Cf::OFF_VEC + 3 * kC * 4);
            F fp[kTriFrags];
#pragma unroll
            for (int i = 0; i < kTriFrags; ++i) fp[i] = P[i * 64 + lane];
            float gq[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) gq[mt] = gamq[16 * mt + c16];
            // O^T = (S Q^T) diag(gamma) for both column groups
            f32x4 acc[Cf::NC][4];
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                const bf16x8 *hs = reinterpret_cast<const bf16x8 *>(smem + Cf::OFF_HO + j * Cf::HO);
                wait_flag(flags + j, 2 * (int)c + 1, p.status);
                F sf[KS];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) sf[kk] = hs[kk * 64 + lane];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[j][mt] = zero4();
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = mma(sf[kk], fq[kk][mt], acc[j][mt]);
            }
            phase_fence();
            load_q(buf(c + 1), fq);
            touch(c + LEAD, (int)(c & 1));
            // + U^T P^T, then the rows of this chunk that exist
            const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
            __bf16 *oc = oh + c * kC * sVO + (int64_t)c16 * sVO + 4 * g4;
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                const bf16x8 *hu =
                    reinterpret_cast<const bf16x8 *>(smem + Cf::OFF_HO + j * Cf::HO + Cf::HO_S);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[j][mt] *= gq[mt];
                wait_flag(flags + j, 2 * (int)c + 2, p.status);
                const F fu0 = hu[lane], fu1 = hu[64 + lane];
                acc[j][0] = mma(fu0, fp[0], acc[j][0]);
                acc[j][1] = mma(fu0, fp[1], acc[j][1]);
                acc[j][2] = mma(fu0, fp[2], acc[j][2]);
                acc[j][3] = mma(fu0, fp[4], acc[j][3]);
                acc[j][2] = mma(fu1, fp[3], acc[j][2]);
                acc[j][3] = mma(fu1, fp[5], acc[j][3]);
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) {
                    if (16 * mt + c16 < lenc) {
                        bf16x4 ob;
#pragma unroll
                        for (int r = 0; r < 4; ++r) ob[r] = (__bf16)(p.scale * acc[j][mt][r]);
                        *reinterpret_cast<bf16x4 *>(oc + (int64_t)(16 * mt) * sVO + 16 * j) = ob;
                    }
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) tacc ^= pend[0][j] ^ pend[1][j];
        asm volatile("" ::"v"(tacc));  // keeps the touches
        return;
    }

    // ---------------------------------------------------------------- copies
    __builtin_amdgcn_s_setprio(2);
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(p.q) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(p.v) +
                              (tok0 * p.v_stride + (int64_t)h * D + dv0) * 2;
    const int64_t rowqk = sQK * 2, rowv = p.v_stride * 2;
    // one 1 KiB block: slots 64 blk .. 64 blk + 63 of a swizzled region with
    // rows of ROWB bytes; LDS slot s of row r receives data piece s ^ swz_f(r)
    auto block = [&](unsigned char *dst, int blk, auto rowb_c, auto src) {
        constexpr int ROWB = decltype(rowb_c)::value, NP = ROWB / 16;
        const int slot = 64 * blk + lane;
        const int row = slot / NP;
        const int pc = (slot % NP) ^ swz_f<ROWB>(row % 16);
        dma16(src(row, pc), dst + 1024 * blk);
    };
    using KR_c = std::integral_constant<int, KR>;
    using VR_c = std::integral_constant<int, VR>;
    // rows past the end of the sequence repeat its last row: finite values
    // whose every contribution is multiplied by that row's beta = 0 (U rows
    // are zero there, and P masks those columns)
    auto copy_chunk = [&](int64_t c) {
        unsigned char *bf = smem + (int)(c % NBUF) * Cf::BUF;
        const int64_t t0 = c * kC;
        const int lenc = (int)((len - t0) < kC ? (len - t0) : kC);
        const unsigned char *rec = ws + ((base + c) * p.Hv + h) * (int64_t)Cf::WSB;
        auto srcK = [&](int row, int pc) { return kb + (t0 + min(row, lenc - 1)) * rowqk + 16 * pc; };
        auto srcQ = [&](int row, int pc) { return qb + (t0 + min(row, lenc - 1)) * rowqk + 16 * pc; };
        auto srcV = [&](int row, int pc) { return vb + (t0 + min(row, lenc - 1)) * rowv + 16 * pc; };
#pragma unroll
        for (int j = 0; j < Cf::BLK_K; ++j) block(bf + Cf::OFF_K, j, KR_c{}, srcK);
#pragma unroll
        for (int j = 0; j < Cf::BLK_K; ++j) block(bf + Cf::OFF_Q, j, KR_c{}, srcQ);
#pragma unroll
        for (int j = 0; j < Cf::BLK_V; ++j) block(bf + Cf::OFF_V, j, VR_c{}, srcV);
#pragma unroll
        for (int j = 0; j < Cf::BLK_R; ++j) dma16(rec + 1024 * j + 16 * lane, bf + Cf::OFF_REC + 1024 * j);
    };
    constexpr int LEAD = NBUF - 1;  // chunk c + LEAD is copied in step c
    for (int j = 0; j < LEAD && j < npc; ++j) copy_chunk(j);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first chunks have landed
    __syncthreads();
    for (int64_t c = 0; c < npc; ++c) {
        if (c + LEAD < npc) copy_chunk(c + LEAD);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's copies have landed
        __syncthreads();
    }
}

}  // namespace

bool chain4_supported(const PrefillParams &p, int D, int nsplit) {
    return D == 128 && nsplit == C4<3>::NSPLIT && !p.dual && !p.s0_identity;
}

hipError_t launch_chain4(const PrefillParams &p, const unsigned char *ws, int64_t nchain,
                         hipStream_t stream) {
    constexpr int NBUF = 3;
    if (nchain <= 0 || nchain > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int remap = nchain % 8 == 0 ? 1 : 0;
    if (p.prefix)
        hipLaunchKernelGGL((chain4_kernel<NBUF, true>), dim3((unsigned)nchain), dim3(256), 0,
                           stream, p, ws, remap);
    else
        hipLaunchKernelGGL((chain4_kernel<NBUF, false>), dim3((unsigned)nchain), dim3(256), 0,
                           stream, p, ws, remap);
    return hipGetLastError();
}

}  // namespace gdn
