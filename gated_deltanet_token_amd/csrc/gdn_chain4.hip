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
//              chunk K S^T, R, U = T R and the state update. S (at the
//              chunk's start) and U go to the output wave through LDS, in
//              one of two slots by chunk parity;
//   wave 2     output, one chunk behind: in step c it forms O of chunk c - 1
//              for all 32 columns from S and U of that chunk (complete at
//              the barrier that ended step c - 1, so no flag is needed) and
//              Q, P and the query decay of that chunk, which it read from
//              LDS into registers during step c - 1;
//   wave 3     copies with LDS-DMA loads: V and the workspace record of
//              chunk c + 1 and K, Q of chunk c + 2 in step c, so that the
//              larger part has two steps to land. (Measured on the MI355X:
//              one CU's LDS-DMA copies move ~16 bytes per cycle when each
//              chunk must land within the step that issues it, ~25 with two
//              in flight.) It also touches the lines of chunk c + 4 so that
//              those copies find them in L2: a CU takes in data at a rate set
//              by the latency of its requests, and the shared K, Q and record
//              lines otherwise make every workgroup that shares them wait for
//              the same HBM misses.
// One barrier per chunk. The state's rows (the key dimension dk) are held
// in a permuted order: state tile a, lane group g, element r is key column
// 32 (a >> 1) + 8 g + 4 (a & 1) + r. With it the eight keys that a lane
// contributes to a 32-deep MFMA step are contiguous, so the K and Q
// operands of K S^T and Q S^T are single 16-byte reads; the transposing
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

struct C4 {
    static constexpr int D = 128;
    static constexpr int NC = 2;         // chain waves, 16 value columns each
    static constexpr int DVS = 16 * NC;  // value columns of a workgroup
    static constexpr int NSPLIT = D / DVS;
    static constexpr int KR = D * 2;     // K, Q row bytes
    static constexpr int VR = DVS * 2;   // V row bytes
    static constexpr int FRAG = kTriFragBytes;  // T or P as (compact) MFMA fragments
    static constexpr int WSB = 2 * FRAG + 1024; // record: T, P, 4 vectors
    // K and Q are copied two chunks ahead (ring of 3: in use, landing,
    // issued); V and the record one chunk ahead (ring of 2: in use, issued)
    static constexpr int NKQ = 3, NVR = 2;
    static constexpr int SZ_K = kC * KR;
    static constexpr int SZ_V = kC * VR;
    static constexpr int OFF_K = 0, OFF_Q = SZ_K, SZ_KQ = 2 * SZ_K;
    static constexpr int OFF_V = 0, OFF_REC = SZ_V, SZ_VR = SZ_V + WSB;
    static constexpr int OFF_T = OFF_REC, OFF_P = OFF_REC + FRAG, OFF_VEC = OFF_REC + 2 * FRAG;
    static constexpr int OFF_KQR = 0;
    static constexpr int OFF_VRR = NKQ * SZ_KQ;
    static constexpr int HO_S = (D / 32) * 1024;  // S^T fragments of one chain wave
    static constexpr int HO_U = 2 * 1024;         // U fragments of one chain wave
    static constexpr int HO = HO_S + HO_U;
    static constexpr int OFF_HO = OFF_VRR + NVR * SZ_VR;  // [slot][chain wave]
    static constexpr int OFF_JUNK = OFF_HO + 2 * NC * HO;  // target of the L2 touches
    static constexpr int LDS = OFF_JUNK + 1024;
    static constexpr int PF_AHEAD = 4;  // chunks between an L2 touch and its copy
    static constexpr int NPF = 4;       // touch instructions per step
    static constexpr int BLK_KQ = SZ_KQ / 1024, BLK_V = SZ_V / 1024, BLK_R = WSB / 1024;
    static constexpr int BLK_VR = BLK_V + BLK_R;
    static_assert(SZ_K % 1024 == 0 && SZ_V % 1024 == 0 && WSB % 1024 == 0, "whole DMA blocks");
    static_assert(BLK_KQ + BLK_VR + NPF < 64, "a step's copies fit the vmcnt counter");
    static_assert(LDS <= 160 * 1024, "LDS budget of a gfx950 CU");
};

// s_waitcnt with only vmcnt(n) (n < 64), the other counters not waited for
template <int N> __device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Key column of state tile a (16 virtual rows), lane group g, element 0.
__device__ __forceinline__ int st_key(int a, int g) { return 32 * (a >> 1) + 8 * g + 4 * (a & 1); }

template <bool PREFIX>
__global__ __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chain4_kernel(PrefillParams p, const unsigned char *ws, int remap_xcd) {
    using Cf = C4;
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
    auto kslot = [&](int64_t c) { return smem + Cf::OFF_KQR + (int)(c % Cf::NKQ) * Cf::SZ_KQ; };
    auto vslot = [&](int64_t c) { return smem + Cf::OFF_VRR + (int)(c & 1) * Cf::SZ_VR; };
    auto hslot = [&](int64_t c, int j) { return smem + Cf::OFF_HO + ((int)(c & 1) * Cf::NC + j) * Cf::HO; };
    auto record = [&](int64_t c) { return ws + ((base + c) * p.Hv + h) * (int64_t)Cf::WSB; };

    if (wave < Cf::NC) {
        // ------------------------------------------------------------ chain
        __builtin_amdgcn_s_setprio(3);
        const int wdv = 16 * wave;
        f32x4 st[NKT];
        {
            const float *s0 = p.s0 ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
            const int64_t row = (int64_t)(dv0 + wdv + c16) * D;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
                st[a] = s0 ? *reinterpret_cast<const f32x4 *>(s0 + row + st_key(a, g4)) : zero4();
        }
        PrefixRows pre(p, n, len);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the initial state
        __syncthreads();                      // the first chunks are staged
        // K fragments of a chunk: row 16 mt + c16, keys 32 kk + 8 g4 .. +7
        auto load_fk = [&](const unsigned char *kb_, F (&fk)[KS][4]) {
            const DT *K = reinterpret_cast<const DT *>(kb_);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    fk[kk][mt] = *reinterpret_cast<const F *>(swz_at<KR>(K, 16 * mt, c16, 32 * kk + 8 * g4));
        };
        for (int64_t c = 0; c < npc; ++c) {
            const DT *K = reinterpret_cast<const DT *>(kslot(c) + Cf::OFF_K);
            const unsigned char *vt = vslot(c);
            const DT *V = reinterpret_cast<const DT *>(vt + Cf::OFF_V);
            const unsigned char *T = vt + Cf::OFF_T;
            const float *vec = reinterpret_cast<const float *>(vt + Cf::OFF_VEC);
            bf16x8 *ho_s = reinterpret_cast<bf16x8 *>(hslot(c, wave));
            bf16x8 *ho_u = ho_s + (D / 32) * 64;
            // S^T at the chunk's start as B fragments; a copy for the output wave
            F sf[KS];
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                c_to_frag(st[2 * kk], st[2 * kk + 1], sf[kk]);
                ho_s[kk * 64 + lane] = sf[kk];
            }
            F fk[KS][4];
            load_fk(kslot(c) + Cf::OFF_K, fk);
            // operands of R, U = T R and the state update (this chunk)
            F ft[kTriFrags];
#pragma unroll
            for (int i = 0; i < kTriFrags; ++i) ft[i] = ld_tri_frag(T, i, lane);
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
            // U for the output wave; S^T <- gamma_C S^T + K^T diag(dec) U
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
        // Q rows, P fragments and the query decay of one chunk, read from LDS
        // in the step that uses the chunk (the output of that chunk is formed
        // in the next step, when both slots may be overwritten)
        struct Ops {
            F fq[KS][4];
            F fp[kTriFrags];
            float gq[4];
        };
        Ops ops[2];
        auto load_ops = [&](int64_t c, Ops &o) {
            const DT *Q = reinterpret_cast<const DT *>(kslot(c) + Cf::OFF_Q);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt)
                    o.fq[kk][mt] = *reinterpret_cast<const F *>(swz_at<KR>(Q, 16 * mt, c16, 32 * kk + 8 * g4));
            const unsigned char *vr = vslot(c);
#pragma unroll
            for (int i = 0; i < kTriFrags; ++i) o.fp[i] = ld_tri_frag(vr + Cf::OFF_P, i, lane);
            const float *gamq = reinterpret_cast<const float *>(vr + Cf::OFF_VEC + 3 * kC * 4);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) o.gq[mt] = gamq[16 * mt + c16];
        };
        // O of chunk c from its operands and the S, U its chain waves left in LDS
        auto out_chunk = [&](int64_t c, const Ops &o) {
            const int lenc = (int)((len - c * kC) < kC ? (len - c * kC) : kC);
            f32x4 acc[Cf::NC][4];
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                const bf16x8 *hs = reinterpret_cast<const bf16x8 *>(hslot(c, j));
                F sf[KS];
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) sf[kk] = hs[kk * 64 + lane];
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[j][mt] = zero4();
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) acc[j][mt] = mma(sf[kk], o.fq[kk][mt], acc[j][mt]);
            }
            F fu[Cf::NC][2];
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                const bf16x8 *hu = reinterpret_cast<const bf16x8 *>(hslot(c, j) + Cf::HO_S);
                fu[j][0] = hu[lane];
                fu[j][1] = hu[64 + lane];
            }
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j)
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) acc[j][mt] *= o.gq[mt];
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                acc[j][0] = mma(fu[j][0], o.fp[0], acc[j][0]);
                acc[j][1] = mma(fu[j][0], o.fp[1], acc[j][1]);
                acc[j][2] = mma(fu[j][0], o.fp[2], acc[j][2]);
                acc[j][3] = mma(fu[j][0], o.fp[4], acc[j][3]);
            }
#pragma unroll
            for (int j = 0; j < Cf::NC; ++j) {
                acc[j][2] = mma(fu[j][1], o.fp[3], acc[j][2]);
                acc[j][3] = mma(fu[j][1], o.fp[5], acc[j][3]);
            }
            // Lane (g4, c16) holds columns 4 g4 .. + 3 of both chain waves' tiles
            // (j = 0, 1) for token 16 mt + c16. One exchange between lane rows
            // (row g4 odd <-> row g4 - 1, v_permlane16_swap) gives each lane 8
            // consecutive columns of one tile -- rows 0, 1, 2, 3: columns 0, 16,
            // 8, 24 .. + 7 -- so a token's 64 bytes leave as four 16-byte stores
            // instead of eight 8-byte ones: half the write requests, which
            // share the CU's memory path with the copies.
            static_assert(Cf::NC == 2, "two 16-column tiles per token row");
            __bf16 *o0 = oh + (c * kC + c16) * sVO + 8 * (g4 >> 1) + 16 * (g4 & 1);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                bf16x4 xb, yb;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    xb[r] = (__bf16)(p.scale * acc[0][mt][r]);
                    yb[r] = (__bf16)(p.scale * acc[1][mt][r]);
                }
                const u32x2 x = __builtin_bit_cast(u32x2, xb), y = __builtin_bit_cast(u32x2, yb);
                const auto s0 = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
                if (16 * mt + c16 < lenc)
                    *reinterpret_cast<u32x4 *>(o0 + (int64_t)(16 * mt) * sVO) = u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
        };
        __syncthreads();
        // step c: chunk c's operands into set c & 1, O of chunk c - 1 from set
        // (c - 1) & 1; two steps per iteration so that the sets are fixed
        // registers
        for (int64_t c = 0; c < npc; c += 2) {
            load_ops(c, ops[0]);
            if (c > 0) out_chunk(c - 1, ops[1]);
            __syncthreads();
            if (c + 1 < npc) {
                load_ops(c + 1, ops[1]);
                out_chunk(c, ops[0]);
                __syncthreads();
            }
        }
        if (npc > 0) {
            if ((npc - 1) & 1)
                out_chunk(npc - 1, ops[1]);
            else
                out_chunk(npc - 1, ops[0]);
        }
        return;
    }

    // ---------------------------------------------------------------- copies
    __builtin_amdgcn_s_setprio(2);
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(p.k) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(p.q) +
                              (tok0 * sQK + (int64_t)grp * D) * 2;
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(p.v) +
                              (tok0 * p.v_stride + (int64_t)h * D + dv0) * 2;
    const int64_t rowqk = sQK * 2, rowv = p.v_stride * 2;
    // One 1 KiB block b of a swizzled region with rows of ROWB bytes covers
    // slots 64 b .. 64 b + 63; LDS slot s of row r receives data piece
    // s ^ swz_f(r). The source offset of this lane's piece in a full chunk
    // does not change from chunk to chunk, so it is computed once.
    auto piece_off = [&](int blk, auto rowb_c, int64_t rowbytes, int lenc) {
        constexpr int ROWB = decltype(rowb_c)::value, NP = ROWB / 16;
        const int slot = 64 * blk + lane;
        const int row = slot / NP;
        const int pc = (slot % NP) ^ swz_f<ROWB>(row % 16);
        return (int64_t)min(row, lenc - 1) * rowbytes + 16 * pc;
    };
    using KR_c = std::integral_constant<int, KR>;
    using VR_c = std::integral_constant<int, VR>;
    int64_t offK[Cf::BLK_KQ / 2], offV[Cf::BLK_V];
#pragma unroll
    for (int j = 0; j < Cf::BLK_KQ / 2; ++j) offK[j] = piece_off(j, KR_c{}, rowqk, kC);
#pragma unroll
    for (int j = 0; j < Cf::BLK_V; ++j) offV[j] = piece_off(j, VR_c{}, rowv, kC);
    // Rows past the end of the sequence repeat its last row: finite values
    // whose every contribution is multiplied by that row's beta = 0 (U rows
    // are zero there, and P masks those columns). Only the last chunk of a
    // sequence can be partial; its offsets are recomputed with the clamp.
    auto lenc_of = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
    // NPF touches of the lines of chunk c (16-byte LDS-DMA loads into a
    // scratch KiB that nothing reads), so that its copies PF_AHEAD steps later
    // hit L2. Each K and Q line is touched by one of the workgroups that share
    // it (the value heads of this q/k head times the column slices), each
    // record line and each V line by one of the slices that share it; the
    // lanes beyond the lines repeat the first one. (Every workgroup
    // touching every line instead took longer than no touches at all: the
    // extra requests queue behind the same per-CU limit as the copies.)
    const int share = (h % (p.Hv / p.Hk)) * NSPLIT + slice;
    const int nshare = (p.Hv / p.Hk) * NSPLIT;
    auto touch = [&](int64_t c) {
        unsigned char *junk = smem + Cf::OFF_JUNK;
        const int lenc = lenc_of(c);
        int j = share + nshare * lane;  // line j of the chunk's K rows, and of its Q rows
        if (j >= 2 * kC) j = share;
        const int64_t okq = (int64_t)min(j >> 1, lenc - 1) * rowqk + 128 * (j & 1);
        dma16(kb + c * kC * rowqk + okq, junk);
        dma16(qb + c * kC * rowqk + okq, junk);
        int jr = slice + NSPLIT * lane;  // line of the record
        if (jr >= Cf::WSB / 128) jr = slice;
        dma16(record(c) + 128 * jr, junk);
        // V: a 128-byte line holds the columns of slices 2 i and 2 i + 1; each of
        // the two touches half of its rows (lanes 32 .. 63 repeat 0 .. 31)
        const int vrow = 32 * (slice & 1) + (lane & 31);
        dma16(vb - 2 * dv0 + 128 * (slice >> 1) + c * kC * rowv + (int64_t)min(vrow, lenc - 1) * rowv, junk);
    };
    static_assert(Cf::NPF == 4 && kC * KR / 128 == 2 * kC, "four touch instructions: K, Q, record, V");
    static_assert(Cf::WSB / 128 <= NSPLIT * 64, "the slices' lanes cover the record's lines");
    static_assert(NSPLIT == 4 && Cf::VR == 64, "two slices share each 128-byte V line");
    auto copy_kq = [&](int64_t c) {  // BLK_KQ copies
        unsigned char *dst = kslot(c);
        const unsigned char *k0 = kb + c * kC * rowqk, *q0 = qb + c * kC * rowqk;
        const int lenc = lenc_of(c);
#pragma unroll
        for (int j = 0; j < Cf::BLK_KQ / 2; ++j) {
            const int64_t o = lenc == kC ? offK[j] : piece_off(j, KR_c{}, rowqk, lenc);
            dma16(k0 + o, dst + Cf::OFF_K + 1024 * j);
            dma16(q0 + o, dst + Cf::OFF_Q + 1024 * j);
        }
    };
    auto copy_vr = [&](int64_t c) {  // BLK_VR copies
        unsigned char *dst = vslot(c);
        const unsigned char *v0 = vb + c * kC * rowv;
        const int lenc = lenc_of(c);
#pragma unroll
        for (int j = 0; j < Cf::BLK_V; ++j)
            dma16(v0 + (lenc == kC ? offV[j] : piece_off(j, VR_c{}, rowv, lenc)),
                  dst + Cf::OFF_V + 1024 * j);
        const unsigned char *rec = record(c);
#pragma unroll
        for (int j = 0; j < Cf::BLK_R; ++j) dma16(rec + 1024 * j + 16 * lane, dst + Cf::OFF_REC + 1024 * j);
    };
    // Before step 0: V and the record of chunk 0, then K, Q of chunks 0 and 1;
    // step 0 needs all but chunk 1's K, Q. In step c: V and the record of
    // chunk c + 1, then K, Q of chunk c + 2 and the touches of chunk c + 4
    // (clamped to the last chunk); at its end everything but the last two
    // groups has landed (loads complete in issue order). The barrier carries
    // no fence (a fence would make the compiler wait for every outstanding
    // copy): the explicit counts order this wave's copies before it, and the
    // other waves read after their own barriers. The last steps wait for
    // everything, so that no copy is in flight when the workgroup ends.
    for (int64_t c = 1; c < min<int64_t>(npc, 1 + Cf::PF_AHEAD); ++c) touch(c);
    if (npc > 0) {
        copy_vr(0);
        copy_kq(0);
    }
    if (npc > 1) {
        copy_kq(1);
        wait_vm<Cf::BLK_KQ>();
    } else {
        wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    for (int64_t c = 0; c < npc; ++c) {
        if (c + 1 < npc) copy_vr(c + 1);
        if (c + 2 < npc) {
            copy_kq(c + 2);
            touch(c + Cf::PF_AHEAD < npc ? c + Cf::PF_AHEAD : npc - 1);
            wait_vm<Cf::BLK_KQ + Cf::NPF>();
        } else {
            wait_vm<0>();
        }
        __builtin_amdgcn_s_barrier();
    }
}

}  // namespace

bool chain4_supported(const PrefillParams &p, int D, int nsplit) {
    return D == 128 && nsplit == C4::NSPLIT && !p.dual && !p.s0_identity;
}

hipError_t launch_chain4(const PrefillParams &p, const unsigned char *ws, int64_t nchain,
                         hipStream_t stream) {
    if (nchain <= 0 || nchain > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int remap = nchain % 8 == 0 ? 1 : 0;
    if (p.prefix)
        hipLaunchKernelGGL((chain4_kernel<true>), dim3((unsigned)nchain), dim3(256), 0, stream, p,
                           ws, remap);
    else
        hipLaunchKernelGGL((chain4_kernel<false>), dim3((unsigned)nchain), dim3(256), 0, stream, p,
                           ws, remap);
    return hipGetLastError();
}

}  // namespace gdn
