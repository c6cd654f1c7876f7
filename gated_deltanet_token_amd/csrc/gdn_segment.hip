// gdn_segment.hip -- prefill of few long sequences split into segments that
// run in parallel (gfx950).
//
// The state after a chunk is an affine function of the state before it:
// S' = S M_c + N_c, with M_c in R^{Dk x Dk} (gamma_C I minus a rank-64 term
// built from the chunk's keys) and N_c the chunk's contribution from zero.
// Composing the chunks of a segment gives the same form, S_end = S_start M + N,
// and every output inside the segment is o_t = S_start (M_{->t} q_t) + o^0_t,
// where M_{->t} composes the segment up to token t and o^0_t is the output
// the segment gives from a zero state. So a sequence of P segments runs as
//   1. every segment from a zero state (outputs o^0, end states N_j);
//   2. every segment from the identity state with v = 0 (outputs o'_t =
//      M_{->t} q_t, end states M_j): the same chunked kernels, whose state
//      then holds the composed map;
//   3. the scan S_0 = initial state, S_{j+1} = S_j M_j + N_j, sequential over
//      the segments only (seg_scan_kernel);
//   4. o_t += S_j o'_t for the tokens of segment j (seg_correct_kernel).
// Steps 1 and 2 expose P times more chains to the chip than one pass over
// the whole sequence, at twice its chunk work. The same affine form is what
// lets a sequence be split across GPUs (context parallelism); here the
// segments stay on one GPU.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// Segment bounds as packed-sequence offsets: segment j of sequence b covers
// tokens [b T + j L, min(b T + (j + 1) L, (b + 1) T)), entry b P + j; and a
// zero row of v (Hv * D elements) for step 2.
__global__ __launch_bounds__(256) void seg_setup_kernel(int32_t *cu, int32_t B, int32_t P,
                                                        int64_t T, int64_t L, __bf16 *zero_v,
                                                        int32_t nzero) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i <= B * P) {
        const int b = i / P, j = i - b * P;
        const int64_t start = (int64_t)b * T + (int64_t)j * L;
        const int64_t end_b = (int64_t)(b + 1) * T;
        cu[i] = (int32_t)(i == B * P ? (int64_t)B * T : (start < end_b ? start : end_b));
    }
    for (int e = i; e < nzero; e += gridDim.x * 256) zero_v[e] = (__bf16)0.f;
}

// Operands of one scan step held in registers by a lane: B operands
// b[nt][q][e] = M_j[16 q + 4 g4 + e][col(nt)] and N_j in C layout.
template <int NT, int NQ> struct ScanOps {
    float b[NT][NQ][4];
    float n[NT][4];
};

template <int D, int NT, int NQ>
__device__ __forceinline__ void scan_load(ScanOps<NT, NQ> &o, const float *m, const float *n,
                                          int wave, int g4, int c16) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int col = (wave * NT + nt) * 16 + c16;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) o.b[nt][q][e] = m[(size_t)(16 * q + 4 * g4 + e) * D + col];
#pragma unroll
        for (int i = 0; i < 4; ++i) o.n[nt][i] = n[(size_t)(4 * g4 + i) * D + col];
    }
}

// acc = N_j + S_j M_j for this wave's columns; S_j rows in LDS (pitch PS).
template <int D, int NT, int NQ, int PS>
__device__ __forceinline__ void scan_product(const ScanOps<NT, NQ> &o, const float *sS,
                                             f32x4 (&acc)[NT], int g4, int c16) {
    f32x4 acc2[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = f32x4{o.n[nt][0], o.n[nt][1], o.n[nt][2], o.n[nt][3]};
        acc2[nt] = zero4();
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(sS + c16 * PS + 16 * q + 4 * g4);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (q & 1)
                    acc2[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], o.b[nt][q][e], acc2[nt],
                                                                    0, 0, 0);
                else
                    acc[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], o.b[nt][q][e], acc[nt],
                                                                   0, 0, 0);
            }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] += acc2[nt];
}

// The scan over segments for 16 state rows of one (sequence, value head):
//   S_0 = initial state (or 0), S_{j+1} = S_j M_j + N_j, j = 0 .. P-1,
// writing S_j (the start state of segment j) for the corrections and S_P as
// the final state. fp32 MFMA (16x16x4): wave w forms columns
// [w D/4, (w + 1) D/4) of the product. The k order inside each 16-deep block
// is permuted (MFMA step 4 q + e takes k = 16 q + 4 g4 + e on lane group g4),
// so a lane's A operands are four consecutive entries of S_j's row (one
// 16-byte LDS read per four steps) and its B operands are the entries of
// M_j's column at those k: each wave loads exactly its own B operands from
// memory into registers, two segments ahead (two register sets, used in
// turn), and no copy of M_j goes through LDS. Two accumulators per tile
// halve the dependent MFMA chain.
template <int D>
__global__ __launch_bounds__(256) void seg_scan_kernel(const float *s0, const float *n_end,
                                                       const float *m_end, float *s_start,
                                                       float *s_final, int32_t B, int32_t P,
                                                       int32_t Hv) {
    constexpr int RS = 16;        // rows per workgroup
    constexpr int NT = D / 64;    // 16-column tiles per wave
    constexpr int NQ = D / 16;    // 16-deep k blocks
    constexpr int PS = D + 4;     // padded LDS row of S: the 16 rows of an A read differ in bank
    __shared__ __attribute__((aligned(16))) float sS[RS * PS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15;
    const int slices = D / RS;
    const int bh = blockIdx.x / slices, slice = blockIdx.x - bh * slices;
    const int b = bh / Hv, h = bh - b * Hv;
    const size_t DD = (size_t)D * D;
    const int row0 = slice * RS;
    const size_t base = ((size_t)b * P * Hv + h) * DD;  // state (b, 0, h); + seg * Hv * DD
    const size_t seg_stride = (size_t)Hv * DD;

    // S_0 rows -> LDS and to the corrections (segment 0)
    {
        const float *src = s0 ? s0 + ((size_t)b * Hv + h) * DD : nullptr;
        for (int i = tid; i < RS * D; i += 256) {
            const float x = src ? src[(size_t)row0 * D + i] : 0.f;
            sS[(i / D) * PS + i % D] = x;
            s_start[base + (size_t)row0 * D + i] = x;
        }
    }
    ScanOps<NT, NQ> ops[2];
    auto load = [&](ScanOps<NT, NQ> &o, int seg) {
        scan_load<D>(o, m_end + base + seg * seg_stride,
                     n_end + base + seg * seg_stride + (size_t)row0 * D, wave, g4, c16);
    };
    load(ops[0], 0);
    if (P > 1) load(ops[1], 1);
    f32x4 acc[NT];
    // One step: S_{j+1} = N_j + S_j M_j from the operand set o, which is then
    // refilled with segment j + 2.
    auto step = [&](ScanOps<NT, NQ> &o, int j) {
        __syncthreads();  // S_j is in LDS
        scan_product<D, NT, NQ, PS>(o, sS, acc, g4, c16);
        if (j + 2 < P) load(o, j + 2);
        __syncthreads();  // every wave is done reading S_j
        float *dst = j + 1 < P ? s_start + base + (j + 1) * seg_stride + (size_t)row0 * D
                               : nullptr;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = (wave * NT + nt) * 16 + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sS[(4 * g4 + i) * PS + col] = acc[nt][i];
                if (dst) dst[(size_t)(4 * g4 + i) * D + col] = acc[nt][i];
            }
        }
    };
    for (int j = 0; j < P; j += 2) {
        step(ops[0], j);
        if (j + 1 < P) step(ops[1], j + 1);
    }
    if (s_final) {
        float *out = s_final + ((size_t)b * Hv + h) * DD + (size_t)row0 * D;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = (wave * NT + nt) * 16 + c16;
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(size_t)(4 * g4 + i) * D + col] = acc[nt][i];
        }
    }
}

// o_t += S_j o'_t for the tokens of segment j (bf16 out and o', fp32 S_j):
// one workgroup per (sequence, segment, value head, group of `tiles` 64-token
// tiles: more when there are many, so that staging S_j is amortised).
// S_j^T is staged in LDS as bf16 MFMA fragments once and reused for the
// group's tiles; wave w forms rows 16 w .. 16 w + 15 of a tile, all D
// columns: C[t][n] = sum_k o'[t][k] S_j[n][k]. C goes through a per-wave LDS
// block so that out is read and written as whole rows (16-byte accesses,
// 64 contiguous bytes per row and instruction); the next tile's o' and out
// rows are loaded before the current tile's products. Rows past the end of
// the segment re-read its last row and are never stored.
template <int D>
__global__ __launch_bounds__(256) void seg_correct_kernel(__bf16 *out, const __bf16 *o_id,
                                                          const float *s_start,
                                                          const int32_t *cu, int32_t B,
                                                          int32_t P, int32_t Hv, int32_t groups,
                                                          int32_t first_seg, int32_t tiles) {
    constexpr int NT = D / 16;     // 16-column tiles
    constexpr int KS = D / 32;     // k steps of 32
    constexpr int VP = D / 32;     // 16-byte pieces of a row per lane in the row pass
    constexpr int PC = D + 4;      // fp32 pitch of the staged C rows
    __shared__ bf16x8 sB[KS * NT * 64];  // fragment (ks, nt), lane l
    __shared__ __attribute__((aligned(16))) float sC[4 * 16 * PC];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, c16 = lane & 15;
    int rest = blockIdx.x;
    const int grp = rest % groups;
    rest /= groups;
    const int h = rest % Hv;
    rest /= Hv;
    const int seg = rest % (P - first_seg) + first_seg;
    const int b = rest / (P - first_seg);
    const int si = b * P + seg;
    const int64_t t_lo = cu[si], t_hi = cu[si + 1];
    const int64_t g0 = t_lo + (int64_t)grp * 64 * tiles;
    if (g0 >= t_hi) return;  // uniform over the workgroup
    const float *S = s_start + ((size_t)si * Hv + h) * D * D;

    // B fragments: B[k][n] = S[n][k]; lane (g4, c16) of fragment (ks, nt)
    // holds n = 16 nt + c16, k = 32 ks + 8 g4 .. + 7
    for (int f = tid; f < KS * NT * 64; f += 256) {
        const int l = f & 63, nt = (f >> 6) % NT, ks = (f >> 6) / NT;
        const int n = 16 * nt + (l & 15), k0 = 32 * ks + 8 * (l >> 4);
        const f32x4 a = *reinterpret_cast<const f32x4 *>(S + (size_t)n * D + k0);
        const f32x4 c = *reinterpret_cast<const f32x4 *>(S + (size_t)n * D + k0 + 4);
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[e] = (__bf16)a[e];
            v[4 + e] = (__bf16)c[e];
        }
        sB[f] = v;
    }
    __syncthreads();

    const int64_t sO = (int64_t)Hv * D;
    const __bf16 *oi = o_id + (int64_t)h * D;
    __bf16 *oo = out + (int64_t)h * D;
    // row pass: lane takes row rr of the wave's 16 and the 16-byte pieces
    // 4 v + q (v < VP) of it
    const int rr = lane & 15, q = lane >> 4;
    float *cw = sC + wave * 16 * PC;
    const int ntl = (int)((t_hi - g0 + 63) / 64 < tiles ? (t_hi - g0 + 63) / 64 : tiles);
    auto load_tile = [&](int tile, bf16x8 (&a)[KS], bf16x8 (&ov)[VP]) {
        const int64_t t0 = g0 + 64 * tile + 16 * wave;
        const int64_t ta = t0 + c16 < t_hi ? t0 + c16 : t_hi - 1;
        const int64_t tr = t0 + rr < t_hi ? t0 + rr : t_hi - 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            a[ks] = *reinterpret_cast<const bf16x8 *>(oi + ta * sO + 32 * ks + 8 * g4);
#pragma unroll
        for (int v = 0; v < VP; ++v)
            ov[v] = *reinterpret_cast<const bf16x8 *>(oo + tr * sO + 8 * (4 * v + q));
    };
    bf16x8 a[KS], ov[VP];
    load_tile(0, a, ov);
    for (int tile = 0; tile < ntl; ++tile) {
        const int64_t t0 = g0 + 64 * tile + 16 * wave;  // this wave's first row
        bf16x8 an[KS], on[VP];
        load_tile(tile + 1 < ntl ? tile + 1 : tile, an, on);  // the last re-reads its own rows
        f32x4 acc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt] = mma(a[ks], sB[(ks * NT + nt) * 64 + lane], acc[nt]);
        // C layout (rows 4 g4 + i, column 16 nt + c16) -> rows in LDS; the
        // wave reads back only what it wrote, in order
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) cw[(4 * g4 + i) * PC + 16 * nt + c16] = acc[nt][i];
        asm volatile("" ::: "memory");
        const int64_t t = t0 + rr;
        if (t < t_hi) {
#pragma unroll
            for (int v = 0; v < VP; ++v) {
                const int col = 8 * (4 * v + q);
                const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cw + rr * PC + col);
                const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cw + rr * PC + col + 4);
                bf16x8 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    r[e] = (__bf16)((float)ov[v][e] + c0[e]);
                    r[4 + e] = (__bf16)((float)ov[v][4 + e] + c1[e]);
                }
                *reinterpret_cast<bf16x8 *>(oo + t * sO + col) = r;
            }
        }
        asm volatile("" ::: "memory");  // this tile's C rows are read before the next tile's writes
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = an[ks];
#pragma unroll
        for (int v = 0; v < VP; ++v) ov[v] = on[v];
    }
}

hipError_t launch_segment_setup(int32_t *cu, int32_t B, int32_t P, int64_t T, int64_t L,
                                __bf16 *zero_v, int32_t nzero, hipStream_t stream) {
    const int n = B * P + 1 > nzero ? B * P + 1 : nzero;
    hipLaunchKernelGGL(seg_setup_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       cu, B, P, T, L, zero_v, nzero);
    return hipGetLastError();
}

hipError_t launch_segment_scan(const float *s0, const float *n_end, const float *m_end,
                               float *s_start, float *s_final, int32_t B, int32_t P, int32_t Hv,
                               int D, hipStream_t stream) {
    const unsigned grid = (unsigned)(B * Hv * (D / 16));
    if (D == 128)
        hipLaunchKernelGGL(seg_scan_kernel<128>, dim3(grid), dim3(256), 0, stream, s0, n_end,
                           m_end, s_start, s_final, B, P, Hv);
    else if (D == 64)
        hipLaunchKernelGGL(seg_scan_kernel<64>, dim3(grid), dim3(256), 0, stream, s0, n_end,
                           m_end, s_start, s_final, B, P, Hv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_segment_correct(__bf16 *out, const __bf16 *o_id, const float *s_start,
                                  const int32_t *cu, int32_t B, int32_t P, int32_t Hv,
                                  int64_t seg_len, int32_t first_seg, int D, hipStream_t stream) {
    // 64-token tiles per workgroup: 1 while that leaves under ~1024
    // workgroups, up to 8 for long segments
    const int64_t seg_tiles = (seg_len + 63) / 64;
    const int64_t all_tiles = (int64_t)B * (P - first_seg) * Hv * seg_tiles;
    int32_t tiles = (int32_t)(all_tiles / 1024);
    tiles = tiles < 1 ? 1 : tiles > 8 ? 8 : tiles;
    const int32_t groups = (int32_t)((seg_tiles + tiles - 1) / tiles);
    const int64_t grid = (int64_t)B * (P - first_seg) * Hv * groups;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
    if (D == 128)
        hipLaunchKernelGGL(seg_correct_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream,
                           out, o_id, s_start, cu, B, P, Hv, groups, first_seg, tiles);
    else if (D == 64)
        hipLaunchKernelGGL(seg_correct_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream,
                           out, o_id, s_start, cu, B, P, Hv, groups, first_seg, tiles);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
