// gdn_fused2.hip -- single-pass chunked prefill for many (sequence, value
// head) chains: bf16, head dimension 128, one workgroup of four waves per
// chain, two workgroups per CU.
//
// The chunk-64 rewrite of the gated delta rule (gdn_chunk.hpp), per chunk of
// 64 tokens with state S in R^{Dv x Dk} at its start:
//     A_ts = b_t e^{g_t - g_s} (k_t . k_s) (s < t),  T = (I + A)^{-1},
//     P_ts = e^{g_t - g_s} (q_t . k_s)     (s <= t),
//     R = diag(b) (V - diag(gamma) K S^T),  U = T R,
//     O = diag(gamma) Q S^T + P U,          S' = gamma_63 S + U^T diag(dec) K.
// A workgroup walks one chain's chunks in order; each wave owns 32 value
// columns and keeps S^T of them in MFMA accumulators. Per chunk
// (| = workgroup barrier):
//   | wave 0: the chunk-local decay (scan of ln alpha)
//   | Gram tiles K K^T, Q K^T on MFMA and the decay masks: A (fp32), P as
//     MFMA fragments
//   | wave 0: the diagonal 16x16 blocks of T by forward substitution, while
//     waves 1..3 form K S^T, S Q^T and R for their columns (then start to
//     load their 32 columns of the next chunk's V)
//   | waves 1..3: the blocks below the diagonal, one block column each, on
//     MFMA (T as fragments), while wave 0 forms its K S^T, S Q^T and R
//   | the next chunk's K and Q start to load; every wave: U = T R, the
//     output O and the state update for its 32 columns.
// K, Q and V move by LDS-DMA (global_load_lds: no registers) into their LDS
// areas as soon as the current chunk is done with them: Q after the state
// products and the solve, V (per wave: its own column block) after R. K is needed until the
// state update, so K and A share two areas that swap roles every chunk: the
// next chunk's K lands in the area that held this chunk's A. No LDS read
// waits on the copies in flight; they are waited for once, at the barrier
// that opens the next chunk.
// One chunk needs 79 KiB of LDS, so two workgroups share a CU: while one
// waits in the latency-bound solve or on its loads, the other keeps the MFMA
// units busy.
//
// Layouts. K and Q: 64 rows of 256 bytes whose 16-byte pieces are permuted
// per row (swz_f); V: four column blocks of 64 rows x 64 bytes (one per wave),
// likewise; A: fp32 rows of 256 bytes, piece p of row r in slot p ^ (r % 16).
// Column reads of K and V use transposing LDS reads. The state's rows (keys)
// are held in a permuted order -- state tile a, lane group g, element r is
// key 32 (a >> 1) + 8 g + 4 (a & 1) + r -- which makes the K and Q operands
// of K S^T and S Q^T single 16-byte reads.
#include <float.h>
#include <stdint.h>

#include "gdn_chunk.hpp"
#include "gdn_launch.hpp"
#include "gdn_seq.hpp"

namespace gdn {

namespace {

constexpr int kF2D = 128;             // head dimension
constexpr int kF2Waves = 4;
constexpr int kF2NB = 2;              // 16-column tiles per wave
constexpr int kF2Row = 2 * kF2D;      // bytes per K / Q row
constexpr int kF2VRow = 64;           // bytes per row of a wave's V block
constexpr int kF2Area = kC * kF2Row;  // 16 KiB: K, Q, V, or A (fp32 64 x 64)
static_assert(kF2Area == kC * kC * 4, "K and A share an area");
constexpr int kF2MaxRankedSeqs = 2048;  // packed batches up to this size run longest first
static_assert(kF2MaxRankedSeqs * 8 <= kF2Area, "the sort keys fit an area");

__device__ __forceinline__ int st_key(int a, int g) { return 32 * (a >> 1) + 8 * g + 4 * (a & 1); }

// The lane id through an empty asm: values derived from it cannot be hoisted
// above this point. Each phase of the chunk loop derives its lane indices
// afresh, so that the compiler recomputes the phase's LDS addresses (a few
// integer operations) instead of hoisting all of them out of the loop, where
// they would hold dozens of registers across it.
__device__ __forceinline__ int fresh_lane(int lane) {
    asm volatile("" : "+v"(lane));
    return lane;
}

// LDS-DMA of 16 bytes per lane (lane l writes lds + 16 l), issued through
// inline asm so that the compiler does not track it: it would otherwise make
// LDS reads it cannot tell apart from the copy's target, and every workgroup
// barrier, wait for all copies in flight. The kernel waits for its copies
// itself (vmcnt(0) before the barrier that publishes them) and reads or
// writes no target area before then. The source is base + off (base
// workgroup-uniform, off a 32-bit lane offset: no 64-bit address arithmetic
// per lane). M0 holds the LDS address; one wait state separates its write from
// the load that reads it.
__device__ __forceinline__ void dma16_async(const unsigned char *base, uint32_t off,
                                            unsigned char *lds) {
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_u8 *)lds;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}

__device__ __forceinline__ bf16x4 to_bf4(const f32x4 &x) {
    bf16x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = (__bf16)x[e];
    return y;
}

// Byte offset of A[row][col] (fp32) in its area.
__device__ __forceinline__ int a_off(int row, int col) {
    return row * 256 + ((((col >> 2) ^ (row & 15))) << 4) + ((col & 3) << 2);
}
__device__ __forceinline__ float *a_at(unsigned char *A, int row, int col) {
    return reinterpret_cast<float *>(A + a_off(row, col));
}
__device__ __forceinline__ f32x4 a_row4(const unsigned char *A, int row, int col) {
    return *reinterpret_cast<const f32x4 *>(A + a_off(row, col));
}

// T fragment byte offset of element (row, col) of the lower-triangular 64x64
// T (fragment (rb, k2) = (row >> 4, col >> 5), lane 16 g4 + (row & 15) with
// col = 32 k2 + 4 g4 + (e & 3) + 16 (e >> 2)).
__device__ __forceinline__ int tfrag_off(int row, int col) {
    const int k2 = col >> 5, w = col & 31;
    const int g4 = (w & 15) >> 2, e = (w & 3) + 4 * (w >> 4);
    return ((tri_frag(row >> 4, k2) * 64 + 16 * g4 + (row & 15)) << 4) + 2 * e;
}

// Decay masks of one transposed Gram pair (accumulators X[s][t], s in tile
// tj, t in tile ti): A_ts = beta_t e^{grA_t - gc_s} k_t.k_s (s < t) into the
// A area, P_ts = scale e^{grP_t - gc_s} q_t.k_s (s <= t; the output scale
// rides on P and on gamq) into P's fragments (this
// lane's four values are one half of fragment (ti, tj / 2); pairs on even
// diagonal tiles also clear the other half). With q and k used as given the
// three exponent vectors are the log decay g; with raw rows (NORMS) they
// carry the row norms and P gets the row factor e^{grP_t - grA_t}.
template <bool NORMS>
__device__ __forceinline__ void mask_pair_f2(const f32x4 &gk, const f32x4 &gq, int ti, int tj, int g4,
                                             int c16, const float *sGrA, const float *sGrP,
                                             const float *sGc, const float *sBeta, unsigned char *A,
                                             unsigned char *pfr, float scale) {
    const int t = 16 * ti + c16;
    const float gt = sGrA[t];
    const float rt = NORMS ? __expf(sGrP[t] - gt) * scale : scale;
    const float bt = sBeta[t];
    const f32x4 gs = *reinterpret_cast<const f32x4 *>(sGc + 16 * tj + 4 * g4);
    f32x4 av;
    bf16x4 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int s = 16 * tj + 4 * g4 + r;
        const float dec = __expf(gt - gs[r]);  // for s > t discarded below
        const float a = bt * dec * gk[r];
        const float pp = dec * gq[r] * rt;
        av[r] = (ti != tj || s < t) ? a : 0.f;
        pb[r] = (__bf16)((ti != tj || s <= t) ? pp : 0.f);
    }
    *reinterpret_cast<f32x4 *>(A + a_off(t, 16 * tj + 4 * g4)) = av;
    unsigned char *f = pfr + (tri_frag(ti, tj >> 1) * 64 + 16 * g4 + c16) * 16;
    *reinterpret_cast<bf16x4 *>(f + (tj & 1) * 8) = pb;
    if (ti == tj && (tj & 1) == 0) *reinterpret_cast<uint2 *>(f + 8) = uint2{0u, 0u};
}

// Gram products and decay masks of this wave's lower tile pairs
// pr = wave + 4 k (three pairs on waves 0 and 1, two on waves 2 and 3). The
// twelve fragments of a pair (K rows of tile tj, K and Q rows of tile ti, four
// k steps each) are read one pair ahead, so that the MFMAs of a pair do not
// wait on LDS.
template <bool NORMS>
__device__ __forceinline__ void gram_masks_f2(const __bf16 *sK, const __bf16 *sQ, int wave, int g4,
                                              int c16, const float *sGrA, const float *sGrP,
                                              const float *sGc, const float *sBeta,
                                              unsigned char *A, unsigned char *pfr, float scale) {
    using F = bf16x8;
    F fr[2][3][kF2D / 32];
    auto load = [&](int k, F (&f)[3][kF2D / 32]) {
        const int pr = wave + 4 * k;
        const int ti = pair_i(pr), tj = pair_j(pr);
#pragma unroll
        for (int kk = 0; kk < kF2D / 32; ++kk) {
            f[0][kk] = *reinterpret_cast<const F *>(swz_at<kF2Row>(sK, 16 * tj, c16, 32 * kk + 8 * g4));
            f[1][kk] = *reinterpret_cast<const F *>(swz_at<kF2Row>(sK, 16 * ti, c16, 32 * kk + 8 * g4));
            f[2][kk] = *reinterpret_cast<const F *>(swz_at<kF2Row>(sQ, 16 * ti, c16, 32 * kk + 8 * g4));
        }
    };
    const int np = wave < 2 ? 3 : 2;
    load(0, fr[0]);
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        if (k < np) {
            if (k + 1 < np) load(k + 1, fr[(k + 1) & 1]);
            phase_fence();
            const int pr = wave + 4 * k;
            const int ti = pair_i(pr), tj = pair_j(pr);
            f32x4 gk = zero4(), gq = zero4();
#pragma unroll
            for (int kk = 0; kk < kF2D / 32; ++kk) {
                gk = mma(fr[k & 1][0][kk], fr[k & 1][1][kk], gk);
                gq = mma(fr[k & 1][0][kk], fr[k & 1][2][kk], gq);
            }
            mask_pair_f2<NORMS>(gk, gq, ti, tj, g4, c16, sGrA, sGrP, sGc, sBeta, A, pfr, scale);
        }
    }
}

// Diagonal blocks E_b = (I + A_bb)^{-1} of T (one wave; lane = 16 b + column)
// by forward substitution, four rows per batch: row r of the block is
// x_r = [r == col] - sum_{m<r} a_rm x_m, the part of the sum over earlier
// batches as four independent partial sums. E overwrites A's diagonal blocks
// (each is read in full first: a block's lanes are one lane group, whose
// reads all precede its writes) and goes to T's fragments.
__device__ __forceinline__ void solve_diag_f2(unsigned char *A, unsigned char *tf, int g4, int c16) {
    const int blk = g4, col = c16, r0 = 16 * blk;
    float x[16];
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
        f32x4 arow[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int m4 = 0; m4 <= rb; ++m4) arow[i][m4] = a_row4(A, r0 + 4 * rb + i, r0 + 4 * m4);
        float part[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < rb; ++m4) {
                p0 = fmaf(arow[i][m4][0], x[4 * m4 + 0], p0);
                p1 = fmaf(arow[i][m4][1], x[4 * m4 + 1], p1);
                p2 = fmaf(arow[i][m4][2], x[4 * m4 + 2], p2);
                p3 = fmaf(arow[i][m4][3], x[4 * m4 + 3], p3);
            }
            part[i] = (p0 + p1) + (p2 + p3);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * rb + i;
            float acc = (r == col ? 1.f : 0.f) - part[i];
#pragma unroll
            for (int m = 4 * rb; m < r; ++m) acc = fmaf(-arow[i][rb][m - 4 * rb], x[m], acc);
            x[r] = acc;
        }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        *a_at(A, r0 + r, r0 + col) = x[r];
        *reinterpret_cast<__bf16 *>(tf + tfrag_off(r0 + r, r0 + col)) = (__bf16)x[r];
    }
}

// Blocks T_ij, i > j, of block column j (one wave per column):
// T_ij = -E_i sum_{m=j}^{i-1} A_im T_mj on MFMA (bf16 operands, fp32
// accumulate); the finished blocks of the column stay in registers.
__device__ __forceinline__ void solve_column_f2(const unsigned char *A, unsigned char *tf, int j,
                                                int g4, int c16) {
    f32x4 Tc[4];
    float ecol[4];  // column of E_j as a B operand (k = 4 g4 + e)
#pragma unroll
    for (int e = 0; e < 4; ++e)
        ecol[e] = *reinterpret_cast<const float *>(A + a_off(16 * j + 4 * g4 + e, 16 * j + c16));
#pragma unroll
    for (int ti = 1; ti < 4; ++ti) {
        if (ti <= j) continue;
        f32x4 aim[3];
#pragma unroll
        for (int m = 0; m < ti; ++m)
            if (m >= j) aim[m] = a_row4(A, 16 * ti + c16, 16 * m + 4 * g4);
        const f32x4 ev = a_row4(A, 16 * ti + c16, 16 * ti + 4 * g4);
        f32x4 X = zero4();
#pragma unroll
        for (int m = 0; m < ti; ++m) {
            if (m < j) continue;
            float a4[4], b4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a4[e] = aim[m][e];
                b4[e] = m == j ? ecol[e] : Tc[m][e];
            }
            X = mma_k16(a4, b4, X, __bf16{});
        }
        float a4[4], b4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a4[e] = ev[e];
            b4[e] = X[e];
        }
        const f32x4 Y = mma_k16(a4, b4, zero4(), __bf16{});
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            Tc[ti][r] = -Y[r];
            *reinterpret_cast<__bf16 *>(tf + tfrag_off(16 * ti + 4 * g4 + r, 16 * j + c16)) =
                (__bf16)(-Y[r]);
        }
    }
}

// K S^T (C layout [t][dv]) and S Q^T (C layout [dv][t]) for one wave's
// value tiles, the k steps as the outer loop (16 independent accumulators).
// The state's keys 32 kk + 8 g4 .. +7 are one 16-byte piece of a K or Q row.
__device__ __forceinline__ void state_products_f2(const __bf16 *sK, const __bf16 *sQ,
                                                  const f32x4 (&st)[kF2D / 16][kF2NB],
                                                  f32x4 (&racc)[4][kF2NB], f32x4 (&oT)[4][kF2NB],
                                                  int g4, int c16) {
    using F = bf16x8;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int b = 0; b < kF2NB; ++b) {
            racc[mt][b] = zero4();
            oT[mt][b] = zero4();
        }
#pragma unroll
    for (int kk = 0; kk < kF2D / 32; ++kk) {
        // the state's bf16 fragments once per k step, for both products
        F sf[kF2NB], fk[4], fq[4];
#pragma unroll
        for (int b = 0; b < kF2NB; ++b) c_to_frag(st[2 * kk][b], st[2 * kk + 1][b], sf[b]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            fk[mt] = *reinterpret_cast<const F *>(swz_at<kF2Row>(sK, 16 * mt, c16, 32 * kk + 8 * g4));
            fq[mt] = *reinterpret_cast<const F *>(swz_at<kF2Row>(sQ, 16 * mt, c16, 32 * kk + 8 * g4));
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int b = 0; b < kF2NB; ++b) {
                racc[mt][b] = mma(fk[mt], sf[b], racc[mt][b]);
                oT[mt][b] = mma(sf[b], fq[mt], oT[mt][b]);
            }
    }
}

// Sequence processed by ranked workgroup slot r of a packed batch: the r-th
// longest (ties by index), so that the longest chains start first and the
// tail of the launch is short. All threads of the workgroup call this. The
// keys (length << 32 | ~index, sorted descending) go to `keys` (LDS, room
// for kF2MaxRankedSeqs), padded with zeros to a power of two, and are sorted
// by a bitonic network (log2(n) (log2(n) + 1) / 2 barrier-separated stages):
// a few microseconds even at the largest batch, where counting each
// sequence's rank would take O(N^2 / threads) steps.
__device__ __forceinline__ int ranked_seq(const PrefillParams &p, int r, uint64_t *keys) {
    const int N = p.nseq;
    int n2 = 1;
    while (n2 < N) n2 <<= 1;
    for (int m = threadIdx.x; m < n2; m += blockDim.x) {
        uint64_t key = 0;
        if (m < N) {
            int64_t t0, lm;
            seq_bounds(p, m, t0, lm);
            key = ((uint64_t)(lm < 0x7FFFFFFF ? lm : 0x7FFFFFFF) << 32) | (uint32_t)~(uint32_t)m;
        }
        keys[m] = key;
    }
    __syncthreads();
    // ascending sort of ~key, i.e. descending by length, then ascending index
    for (int k = 2; k <= n2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = threadIdx.x; i < n2; i += blockDim.x) {
                const int ixj = i ^ j;
                if (ixj > i) {
                    const uint64_t a = ~keys[i], b = ~keys[ixj];
                    if (((i & k) == 0) == (a > b)) {
                        keys[i] = ~b;
                        keys[ixj] = ~a;
                    }
                }
            }
            __syncthreads();
        }
    }
    const int n = (int)~(uint32_t)keys[r];
    __syncthreads();  // every thread has read its slot before the area is reused
    return n;
}

template <bool PREFIX, bool RAWQK>
__global__ __launch_bounds__(kF2Waves * 64, 2) void fused2_kernel(PrefillParams p, int remap_xcd,
                                                                 int ranked) {
    using DT = __bf16;
    using F = bf16x8;
    constexpr int D = kF2D, NB = kF2NB, NKT = D / 16, NTH = kF2Waves * 64;

    __shared__ __attribute__((aligned(16))) unsigned char X0[kF2Area];  // K or A
    __shared__ __attribute__((aligned(16))) unsigned char X1[kF2Area];  // A or K
    __shared__ __attribute__((aligned(16))) unsigned char Qs[kF2Area];
    __shared__ __attribute__((aligned(16))) unsigned char Vs[kF2Area];
    __shared__ __attribute__((aligned(16))) unsigned char Ts[kTriFrags * 1024];
    __shared__ __attribute__((aligned(16))) unsigned char Ps[kTriFrags * 1024];
    // decay vectors: g, grA, grP, gc (read up to the masks) and, per chunk
    // parity, gam, dec, beta, gamq (read up to the end of the chunk)
    __shared__ __attribute__((aligned(16))) float Vg[4 * kC];
    __shared__ __attribute__((aligned(16))) float Vf0[4 * kC];
    __shared__ __attribute__((aligned(16))) float Vf1[4 * kC];

    const bool logits = p.flags & kGateLogits;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // (sequence, value head) of this workgroup. Dense batches: the XCD-aware
    // order (the heads sharing a q/k head run on one XCD). Packed batches of
    // unequal lengths (ranked): longest sequences first, where a unit is the
    // Hv / Hk value heads of one q/k head of one sequence, units in rank order;
    // ranked == 2 (units a multiple of 8): unit u runs whole on XCD u % 8
    // (workgroups go to the XCDs round-robin), which balances the XCDs and
    // keeps each unit's shared K and Q in one L2; ranked == 1: units follow
    // the dispatch order directly.
    int h, n;
    if (ranked) {
        const int b = blockIdx.x, G3 = p.Hv / p.Hk;
        int u, j;
        if (ranked == 2) {
            const int s = b >> 3;
            u = (s / G3) * 8 + (b & 7);
            j = s % G3;
        } else {
            u = b / G3;
            j = b % G3;
        }
        h = (u % p.Hk) * G3 + j;
        // (the keys go to X1, which the first chunk uses only after its first barrier)
        n = ranked_seq(p, u / p.Hk, reinterpret_cast<uint64_t *>(X1));
    } else {
        const int wg = logical_wg(remap_xcd);
        h = wg % p.Hv;
        n = wg / p.Hv;
    }
    const int grp = h / (p.Hv / p.Hk);
    int64_t tok0, len;
    seq_bounds(p, n, tok0, len);
    const int wdv = 32 * wave;  // this wave's first value column

    const int64_t sQK = (int64_t)p.Hk * D;
    const int64_t sVO = (int64_t)p.Hv * D;
    const int64_t sVt = p.v_stride;
    const unsigned char *kb = reinterpret_cast<const unsigned char *>(
        reinterpret_cast<const DT *>(p.k) + tok0 * sQK + (int64_t)grp * D);
    const unsigned char *qb = reinterpret_cast<const unsigned char *>(
        reinterpret_cast<const DT *>(p.q) + tok0 * sQK + (int64_t)grp * D);
    const unsigned char *vb = reinterpret_cast<const unsigned char *>(
        reinterpret_cast<const DT *>(p.v) + tok0 * sVt + (int64_t)h * D + wdv);
    DT *oh = reinterpret_cast<DT *>(p.out) + tok0 * sVO + (int64_t)h * D + wdv;
    const float *ah = p.alpha + tok0 * p.Hv + h;
    const float *bh = p.beta + tok0 * p.Hv + h;

    // T's fragments: the halves above the diagonal of fragments (0, 0) and
    // (2, 1) are never written
    for (int i = tid; i < kTriFrags * 256; i += NTH) reinterpret_cast<uint32_t *>(Ts)[i] = 0u;

    // state S^T of this wave's columns (the key order of st_key)
    f32x4 st[NKT][NB];
    {
        const int g4 = lane >> 4, c16 = lane & 15;
        const float *s0 = p.s0 ? p.s0 + ((int64_t)n * p.Hv + h) * D * D : nullptr;
        if (s0 && !p.s0_identity) {
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    st[a][b] = *reinterpret_cast<const f32x4 *>(
                        s0 + (int64_t)(wdv + 16 * b + c16) * D + st_key(a, g4));
        } else {
            const float one = p.s0_identity ? 1.f : 0.f;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        st[a][b][r] = wdv + 16 * b + c16 == st_key(a, g4) + r ? one : 0.f;
        }
    }

    const int64_t nchunks = (len + kC - 1) / kC;
    auto chunk_len = [&](int64_t c) { return (int)((len - c * kC) < kC ? (len - c * kC) : kC); };
    // LDS-DMA of a chunk's K or Q rows 16 wave .. 16 wave + 15 (four KiB per
    // wave): instruction j fills rows 4 j' .. 4 j' + 3 (j' = 4 wave + j), lane l
    // piece (l % 16) ^ swz_f(row) of row 4 j' + l / 16. Rows past the end of the
    // sequence repeat its last row (finite values, weighted zero by beta = 0).
    const uint32_t rowQK = (uint32_t)(sQK * 2), rowV = (uint32_t)(sVt * 2);  // bytes per token
    auto copy_rows = [&](const unsigned char *src, unsigned char *dst, int64_t c) {
        const int ln = fresh_lane(lane);
        const int lc = chunk_len(c);
        const unsigned char *base = src + c * kC * (int64_t)rowQK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * wave + 4 * j + (ln >> 4);
            const int piece = (ln & 15) ^ swz_f<kF2Row>(row & 15);
            const uint32_t off = (uint32_t)(row < lc ? row : lc - 1) * rowQK + 16 * piece;
            dma16_async(base, off, dst + (16 * wave + 4 * j) * kF2Row);
        }
    };
    // LDS-DMA of this wave's 32 value columns of a chunk's V: a block of 64
    // rows x 64 bytes; instruction j fills rows 16 j .. 16 j + 15.
    auto copy_v = [&](int64_t c) {
        const int ln = fresh_lane(lane);
        const int lc = chunk_len(c);
        unsigned char *dst = Vs + wave * (kC * kF2VRow);
        const unsigned char *base = vb + c * kC * (int64_t)rowV;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of the block are done
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 16 * j + (ln >> 2);
            const int piece = (ln & 3) ^ swz_f<kF2VRow>(row & 15);
            const uint32_t off = (uint32_t)(row < lc ? row : lc - 1) * rowV + 16 * piece;
            dma16_async(base, off, dst + j * 1024);
        }
    };
    float rAl = 1.f, rBe = 0.f;  // wave 0: alpha, beta of token `lane` of the next chunk
    auto load_gates = [&](int64_t c) {
        if (wave == 0) {
            const int lc = chunk_len(c);
            const int rr = lane < lc ? lane : lc - 1;
            rAl = ah[(c * kC + rr) * p.Hv];
            rBe = bh[(c * kC + rr) * p.Hv];
        }
    };

    PrefixRows pre(p, n, len);
    if (nchunks > 0) {
        copy_rows(kb, X0, 0);
        copy_rows(qb, Qs, 0);
        copy_v(0);
        load_gates(0);
    }

    for (int64_t c = 0; c < nchunks; ++c) {
        // K in X0 and A in X1 for even chunks, the other way round for odd ones
        const bool odd = c & 1;
        unsigned char *Kc = odd ? X1 : X0;  // this chunk's K
        unsigned char *Ac = odd ? X0 : X1;  // this chunk's A; then the next chunk's K
        float *Vf = odd ? Vf1 : Vf0;
        const DT *sK = reinterpret_cast<const DT *>(Kc);
        const DT *sQ = reinterpret_cast<const DT *>(Qs);
        float *sG = Vg, *sGrA = Vg + kC, *sGrP = Vg + 2 * kC, *sGc = Vg + 3 * kC;
        float *sGam = Vf, *sDec = Vf + kC, *sBeta = Vf + 2 * kC, *sGamQ = Vf + 3 * kC;
        const int lenc = chunk_len(c);
        const bool more = c + 1 < nchunks;

        if (wave == 0) {
            const bool ok = lane < lenc;
            const float la = logits ? neg_softplus(rAl) : __logf(fmaxf(rAl, FLT_MIN));
            const float x = wave_inclusive_scan(ok ? la : 0.f);
            const float glast = __shfl(x, 63, 64);
            sG[lane] = x;
            sGam[lane] = __expf(x);
            sDec[lane] = __expf(glast - x);
            sBeta[lane] = ok ? (logits ? sigmoid_f(rBe) : rBe) : 0.f;
            if (!RAWQK) sGamQ[lane] = p.scale * __expf(x);  // the output scale rides on gamq and P
        }
        // this chunk's K, Q and V have landed (each wave waits for its own
        // copies; the barrier publishes them)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if constexpr (RAWQK) {
            fold_qk_norms<DT, D, D, NTH>(sK, sQ, sG, sGam, sDec, sGamQ, sGrA, sGrP, sGc, tid,
                                         p.scale);
            __syncthreads();
        }

        int g4 = fresh_lane(lane) >> 4, c16 = fresh_lane(lane) & 15;
        gram_masks_f2<RAWQK>(sK, sQ, wave, g4, c16, RAWQK ? sGrA : sG, RAWQK ? sGrP : sG,
                             RAWQK ? sGc : sG, sBeta, Ac, Ps, p.scale);
        __syncthreads();
        // the diagonal blocks of T on wave 0 while waves 1..3 form their
        // state products; then the blocks below the diagonal on waves 1..3
        // while wave 0 forms its own
        // (the accumulators start defined on every path: the register
        // allocator then keeps one set of them across both phases)
        f32x4 racc[4][NB], oT[4][NB];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int b = 0; b < NB; ++b) racc[mt][b] = oT[mt][b] = zero4();
        // R = beta (V - gamma K S^T) from this wave's V block, right after
        // the wave's state products (it needs no T); then the block is done
        // with and the next chunk's V block starts to load
        auto form_r = [&]() {
            const int g4r = fresh_lane(lane) >> 4, c16r = fresh_lane(lane) & 15;
            const DT *sVw = reinterpret_cast<const DT *>(Vs + wave * (kC * kF2VRow));
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int tb = 16 * mt + 4 * g4r;
                const f32x4 bet = *reinterpret_cast<const f32x4 *>(sBeta + tb);
                const f32x4 gam = *reinterpret_cast<const f32x4 *>(sGam + tb);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const bf16x4 v4 = ld_tr(
                        swz_at<kF2VRow>(sVw, 16 * mt, 4 * g4r + (c16r >> 2), 16 * b + 4 * (c16r & 3)));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        racc[mt][b][r] = bet[r] * ((float)v4[r] - gam[r] * racc[mt][b][r]);
                }
            }
            // (its reads have returned: R used them)
            if (more) copy_v(c + 1);
        };
        g4 = fresh_lane(lane) >> 4;
        c16 = fresh_lane(lane) & 15;
        if (wave == 0) {
            solve_diag_f2(Ac, Ts, g4, c16);
        } else {
            state_products_f2(sK, sQ, st, racc, oT, g4, c16);
            form_r();
        }
        __syncthreads();
        g4 = fresh_lane(lane) >> 4;
        c16 = fresh_lane(lane) & 15;
        if (wave == 0) {
            state_products_f2(sK, sQ, st, racc, oT, g4, c16);
            form_r();
        } else {
            solve_column_f2(Ac, Ts, wave - 1, g4, c16);
        }
        __syncthreads();
        // A and Q are done with: the next chunk's K goes to A's area, its Q
        // to Q's
        if (more) {
            copy_rows(kb, Ac, c + 1);
            copy_rows(qb, Qs, c + 1);
            load_gates(c + 1);
        }

        g4 = fresh_lane(lane) >> 4;
        c16 = fresh_lane(lane) & 15;
        // U = T R (T's fragments read as they are used)
        const F *Tf = reinterpret_cast<const F *>(Ts) + lane;
        F fr[2][NB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int b = 0; b < NB; ++b) c_to_frag(racc[2 * k2][b], racc[2 * k2 + 1][b], fr[k2][b]);
        f32x4 u[4][NB];
        {
            const F t0 = Tf[0], t1 = Tf[64], t2 = Tf[128], t4 = Tf[256];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                u[0][b] = mma(t0, fr[0][b], zero4());
                u[1][b] = mma(t1, fr[0][b], zero4());
                u[2][b] = mma(t2, fr[0][b], zero4());
                u[3][b] = mma(t4, fr[0][b], zero4());
            }
            const F t3 = Tf[192], t5 = Tf[320];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                u[2][b] = mma(t3, fr[1][b], u[2][b]);
                u[3][b] = mma(t5, fr[1][b], u[3][b]);
            }
        }
        // U as the B operand of the output (fu) and, scaled by dec, of the
        // state update (fd)
        F fu[2][NB], fd[2][NB];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            const f32x4 d0 = *reinterpret_cast<const f32x4 *>(sDec + 32 * k2 + 4 * g4);
            const f32x4 d1 = *reinterpret_cast<const f32x4 *>(sDec + 32 * k2 + 16 + 4 * g4);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 lo = u[2 * k2][b], hi = u[2 * k2 + 1][b];
                c_to_frag(lo, hi, fu[k2][b]);
                f32x4 dl, dh;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dl[r] = lo[r] * d0[r];
                    dh[r] = hi[r] * d1[r];
                }
                c_to_frag(dl, dh, fd[k2][b]);
            }
        }
        // O^T = (S Q^T) diag(gamq) + U^T P^T (the scale is in gamq and P),
        // stored for rows t < lenc
        const F *Pf = reinterpret_cast<const F *>(Ps) + lane;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const float gq = sGamQ[16 * mt + c16];
#pragma unroll
            for (int b = 0; b < NB; ++b) oT[mt][b] *= gq;
        }
        {
            const F p0 = Pf[0], p1 = Pf[64], p2 = Pf[128], p4 = Pf[256];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                oT[0][b] = mma(fu[0][b], p0, oT[0][b]);
                oT[1][b] = mma(fu[0][b], p1, oT[1][b]);
                oT[2][b] = mma(fu[0][b], p2, oT[2][b]);
                oT[3][b] = mma(fu[0][b], p4, oT[3][b]);
            }
            const F p3 = Pf[192], p5 = Pf[320];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                oT[2][b] = mma(fu[1][b], p3, oT[2][b]);
                oT[3][b] = mma(fu[1][b], p5, oT[3][b]);
            }
        }
        {
            // Lane (g4, c16) holds columns 4 g4 .. + 3 of both tiles (b = 0, 1)
            // for token 16 mt + c16. One exchange between lane rows (row g4 odd
            // <-> row g4 - 1, v_permlane16_swap) gives each lane 8 consecutive
            // columns of one tile -- rows 0, 1, 2, 3: columns 0, 16, 8, 24 .. + 7
            // -- so each token's 64 bytes go out as four 16-byte stores, not
            // eight 8-byte ones.
            const int dvo = 8 * (g4 >> 1) + 16 * (g4 & 1);
            DT *o0 = oh + (c * kC + c16) * sVO + dvo;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const u32x2 x = __builtin_bit_cast(u32x2, to_bf4(oT[mt][0]));
                const u32x2 y = __builtin_bit_cast(u32x2, to_bf4(oT[mt][1]));
                const auto s0 = __builtin_amdgcn_permlane16_swap(x[0], y[0], false, false);
                const auto s1 = __builtin_amdgcn_permlane16_swap(x[1], y[1], false, false);
                if (16 * mt + c16 < lenc)
                    *reinterpret_cast<u32x4 *>(o0 + (int64_t)(16 * mt) * sVO) =
                        u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
        }
        g4 = fresh_lane(lane) >> 4;
        c16 = fresh_lane(lane) & 15;
        // S^T <- gamma_C S^T + K^T diag(dec) U; K^T by transposing reads in
        // the state's key order (gamma_C = gam[63] / dec[63]: dec[63] = 1
        // unless the row norms are folded in)
        const float gC = sGam[kC - 1] * __builtin_amdgcn_rcpf(sDec[kC - 1]);
        const int rl = 4 * g4 + (c16 >> 2);
        // all of K^T's fragments first (64 registers), then the MFMAs
        F fkt[NKT][2];
#pragma unroll
        for (int a = 0; a < NKT; ++a) {
            const int col = st_key(a, c16 & 3);
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const bf16x4 lo = ld_tr(swz_at<kF2Row>(sK, 32 * k2, rl, col));
                const bf16x4 hi = ld_tr(swz_at<kF2Row>(sK, 32 * k2 + 16, rl, col));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    fkt[a][k2][e] = lo[e];
                    fkt[a][k2][e + 4] = hi[e];
                }
            }
        }
        // the decay in place first, then the 32 MFMAs with consecutive ones
        // independent (scaled as it goes, each tile went through one
        // temporary, and every product waited for the one before)
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b) st[a][b] *= gC;
        phase_fence();
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b) st[a][b] = mma(fkt[a][k2], fd[k2][b], st[a][b]);
        const int64_t prow = PREFIX ? pre.take(p, c) : -1;
        if (prow >= 0) {
            float *ps = p.prefix + (prow * p.Hv + h) * D * D;
#pragma unroll
            for (int a = 0; a < NKT; ++a)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    __builtin_nontemporal_store(
                        st[a][b], reinterpret_cast<f32x4 *>(ps + (int64_t)(wdv + 16 * b + c16) * D +
                                                            st_key(a, g4)));
        }
    }

    if (p.s_final) {
        const int g4 = lane >> 4, c16 = lane & 15;
        float *sfp = p.s_final + ((int64_t)n * p.Hv + h) * D * D;
#pragma unroll
        for (int a = 0; a < NKT; ++a)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<f32x4 *>(sfp + (int64_t)(wdv + 16 * b + c16) * D + st_key(a, g4)) =
                    st[a][b];
    }
}

}  // namespace

bool fused2_supported(const PrefillParams &p, int dtype, int D) {
    // the copies' lane offsets are 32-bit: a chunk's 64 rows of q, k or v must
    // span less than 4 GiB
    return dtype == 1 && D == kF2D && !p.dual && (int64_t)p.Hk * D * 2 * kC < ((int64_t)1 << 32) &&
           p.v_stride * 2 * kC < ((int64_t)1 << 32);
}

hipError_t launch_fused2(const PrefillParams &p, hipStream_t stream) {
    const int64_t nblocks = (int64_t)p.nseq * p.Hv;
    if (nblocks <= 0 || nblocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const int remap = nblocks % 8 == 0 ? 1 : 0;
    // packed batches: longest sequences first (2: units of one q/k head kept
    // on one XCD, which needs a multiple of 8 units)
    const int ranked = p.cu_seqlens && p.nseq > 1 && p.nseq <= kF2MaxRankedSeqs
                           ? ((int64_t)p.nseq * p.Hk % 8 == 0 ? 2 : 1)
                           : 0;
    const bool raw = p.flags & kQkL2Norm;
    const dim3 grid((unsigned)nblocks), block(kF2Waves * 64);
    if (p.prefix) {
        if (raw)
            hipLaunchKernelGGL((fused2_kernel<true, true>), grid, block, 0, stream, p, remap, ranked);
        else
            hipLaunchKernelGGL((fused2_kernel<true, false>), grid, block, 0, stream, p, remap, ranked);
    } else {
        if (raw)
            hipLaunchKernelGGL((fused2_kernel<false, true>), grid, block, 0, stream, p, remap, ranked);
        else
            hipLaunchKernelGGL((fused2_kernel<false, false>), grid, block, 0, stream, p, remap, ranked);
    }
    return hipGetLastError();
}

}  // namespace gdn
