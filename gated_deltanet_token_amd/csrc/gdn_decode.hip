// gdn_decode.hip -- one-token state update for a batch of sequences (gfx950).
//
// Per (sequence b, value head h) with state S in R^{D x D} (row i = value
// dimension i, contiguous over the key dimension), the gated delta rule for
// one token is, row by row,
//     sk_i = S_i . k,  sq_i = S_i . q
//     u_i  = beta * (v_i - alpha * sk_i)
//     S'_i = alpha * S_i + u_i * k                (written back in place)
//     o_i  = scale * (alpha * sq_i + u_i * (k . q))   (= scale * S'_i . q)
// Rows are independent, so the kernel is one pass over the state: every byte
// of S is read once and written once, which makes it bound by HBM bandwidth
// (4 flops per 8 bytes). This is the fixed per-token cost behind the flat
// decode speed reported in "The economics of hybrid attention" (section
// "Where the constraint moved").
//
// Mapping: one 256-thread workgroup per (b, h); wave w owns rows
// [w*D/4, (w+1)*D/4). Within a wave, 16 lanes share a row: lane j reads the
// float4 columns [4j, 4j+4) (and [64+4j, 64+4j+4) when D = 128), so one
// load instruction covers 4 rows x 256 contiguous bytes. All of a lane's row
// loads are issued before any arithmetic, keeping D/4 * D * 4 / 64 bytes per
// lane in flight. Dot products reduce over the 16 lanes with DPP.
#include "gdn_device.hpp"
#include "gdn_launch.hpp"

namespace gdn {

template <int D> struct DecodeShape {
    static constexpr int kWaves = 4;
    static constexpr int kV4 = D / 64;                       // float4 per lane per row
    static constexpr int kRowsPerWave = D / kWaves;          // 32 or 16
    static constexpr int kSteps = kRowsPerWave / 4;          // 4 rows per wave step
};

template <typename DT>
__device__ __forceinline__ void load4(const DT *p, float (&x)[4]) {
    if constexpr (sizeof(DT) == 2) {
        const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
    } else {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = v[e];
    }
}

template <typename DT, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecodeParams p) {
    using Sh = DecodeShape<D>;
    constexpr int V4 = Sh::kV4;
    constexpr int STEPS = Sh::kSteps;
    __shared__ float s_o[D];

    const int bh = blockIdx.x;
    const int b = bh / p.Hv;
    const int h = bh - b * p.Hv;
    const int g = h / (p.Hv / p.Hk);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int rsub = lane >> 4;

    float *S = p.state + (size_t)bh * D * D;
    const int row0 = wave * Sh::kRowsPerWave + rsub;

    // Issue the state loads first: STEPS * V4 float4 per lane.
    f32x4 s[STEPS][V4];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const float *rowp = S + (size_t)(row0 + 4 * st) * D + 4 * j;
#pragma unroll
        for (int c = 0; c < V4; ++c)
            s[st][c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(rowp + 64 * c));
    }

    const DT *qp = reinterpret_cast<const DT *>(p.q) + ((size_t)b * p.Hk + g) * D;
    const DT *kp = reinterpret_cast<const DT *>(p.k) + ((size_t)b * p.Hk + g) * D;
    const DT *vp = reinterpret_cast<const DT *>(p.v) + (size_t)bh * D;
    float kk[V4][4], qq[V4][4];
#pragma unroll
    for (int c = 0; c < V4; ++c) {
        load4<DT>(kp + 64 * c + 4 * j, kk[c]);
        load4<DT>(qp + 64 * c + 4 * j, qq[c]);
    }
    float vrow[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) vrow[st] = to_f32(vp[row0 + 4 * st]);
    float alpha = p.alpha[bh];
    float beta = p.beta[bh];
    if (p.flags & kGateLogits) {
        alpha = expf(neg_softplus(alpha));
        beta = sigmoid_f(beta);
    }
    if (p.flags & kQkL2Norm) {
        // the 16 lanes of a row hold all D elements of k and q
        float k2 = 0.f, q2 = 0.f;
#pragma unroll
        for (int c = 0; c < V4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k2 += kk[c][e] * kk[c][e];
                q2 += qq[c][e] * qq[c][e];
            }
        const float ik = inv_norm(row16_sum(k2), kL2Eps), iq = inv_norm(row16_sum(q2), kL2Eps);
#pragma unroll
        for (int c = 0; c < V4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[c][e] *= ik;
                qq[c][e] *= iq;
            }
    }

    float kq = 0.f;
#pragma unroll
    for (int c = 0; c < V4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e) kq += kk[c][e] * qq[c][e];
    kq = row16_sum(kq);

#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int c = 0; c < V4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += s[st][c][e] * kk[c][e];
                sq += s[st][c][e] * qq[c][e];
            }
        sk = row16_sum(sk);
        sq = row16_sum(sq);
        const float u = beta * (vrow[st] - alpha * sk);
        float *rowp = S + (size_t)(row0 + 4 * st) * D + 4 * j;
#pragma unroll
        for (int c = 0; c < V4; ++c) {
            f32x4 nv;
#pragma unroll
            for (int e = 0; e < 4; ++e) nv[e] = alpha * s[st][c][e] + u * kk[c][e];
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4 *>(rowp + 64 * c));
        }
        if (j == 0) s_o[row0 + 4 * st] = p.scale * (alpha * sq + u * kq);
    }
    __syncthreads();
    DT *op = reinterpret_cast<DT *>(p.out) + (size_t)bh * D;
    for (int i = threadIdx.x; i < D; i += 256) op[i] = from_f32<DT>(s_o[i]);
}

// ---------------------------------------------------------------------------
// Several tokens per sequence against a pool of state slots.
//
// The same row-wise step as above, applied K times in token order with the
// state held in registers in between: S is read once from slot src_slot[b]
// (or taken as zero when that index is negative), the K tokens run, and the
// final state is written once to slot dst_slot[b] (not at all when that index
// is negative). HBM traffic per (b, h) is therefore one state read and one
// state write for all K tokens, plus the optional per-token states. A padding
// token with alpha = 1, beta = 0 leaves the state unchanged.
//
// The token inputs (k, q, v, alpha, beta) of up to kStage tokens are staged
// in LDS once per workgroup, v permuted so that a lane's STEPS value rows are
// contiguous (one LDS read per token). Their global loads are issued before
// the state loads, so the wait for them leaves the state loads in flight.
// With the token inputs out of registers the kernel fits 128 VGPRs: four
// workgroups per CU, so one workgroup's arithmetic overlaps the others'
// state traffic. The state is kept as a scalar times a matrix so that the
// decay costs one multiply per row instead of one per element (three fp32
// operations per state element and token instead of four).
template <typename DT, int D> struct MultiShape {
    using Sh = DecodeShape<D>;
    static constexpr int kStage = 8;                       // tokens per LDS stage
    // v position of row r: lane group (wave, rsub) holds rows
    // wave*RPW + rsub + 4*st at [(wave*4 + rsub)*STEPS + st]
    static __device__ __forceinline__ int vpos(int r) {
        const int wave = r / Sh::kRowsPerWave, rem = r % Sh::kRowsPerWave;
        return (wave * 4 + (rem & 3)) * Sh::kSteps + (rem >> 2);
    }
};

template <typename DT, int D>
struct MultiSmem {
    DT k[MultiShape<DT, D>::kStage][D];
    DT q[MultiShape<DT, D>::kStage][D];
    DT v[MultiShape<DT, D>::kStage][D];
    float ab[MultiShape<DT, D>::kStage][2];
};

template <typename DT> struct Vec4Of;
template <> struct Vec4Of<__bf16> { using type = bf16x4; };
template <> struct Vec4Of<float> { using type = f32x4; };

// Global loads of tokens [t0, t0 + n) into registers: thread i covers the
// 4-element pieces i, i + 256, ... of the n*D/4 pieces of k, q and v each.
template <typename DT, int D> struct StageRegs {
    static constexpr int kPieces = MultiShape<DT, D>::kStage * D / 4;
    static constexpr int kPerThread = (kPieces + 255) / 256;
    typename Vec4Of<DT>::type k[kPerThread], q[kPerThread], v[kPerThread];
    float ab;
};

template <typename DT, int D>
__device__ __forceinline__ void stage_load(StageRegs<DT, D> &r, const DecodeMultiParams &p,
                                           size_t tok0, int g, int h, int n) {
    using V = typename Vec4Of<DT>::type;
    using R = StageRegs<DT, D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R::kPerThread; ++i) {
        // clamped to the last valid piece: every load is unconditional
        const int pc = min(tid + 256 * i, n * D / 4 - 1);
        const int t = pc / (D / 4), c4 = pc % (D / 4);
        const size_t tok = tok0 + t;
        r.k[i] = *reinterpret_cast<const V *>(reinterpret_cast<const DT *>(p.k) +
                                              (tok * p.Hk + g) * D + 4 * c4);
        r.q[i] = *reinterpret_cast<const V *>(reinterpret_cast<const DT *>(p.q) +
                                              (tok * p.Hk + g) * D + 4 * c4);
        r.v[i] = *reinterpret_cast<const V *>(reinterpret_cast<const DT *>(p.v) +
                                              (tok * p.Hv + h) * D + 4 * c4);
    }
    const int ta = min(tid >> 1, n - 1);
    r.ab = ((tid & 1) ? p.beta : p.alpha)[(tok0 + ta) * p.Hv + h];
}

template <typename DT, int D>
__device__ __forceinline__ void stage_store(MultiSmem<DT, D> &sm, const StageRegs<DT, D> &r,
                                            int n, uint32_t flags) {
    using V = typename Vec4Of<DT>::type;
    using R = StageRegs<DT, D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R::kPerThread; ++i) {
        const int pc = tid + 256 * i;
        if (pc < n * D / 4) {
            const int t = pc / (D / 4), c4 = pc % (D / 4);
            *reinterpret_cast<V *>(&sm.k[t][4 * c4]) = r.k[i];
            *reinterpret_cast<V *>(&sm.q[t][4 * c4]) = r.q[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.v[t][MultiShape<DT, D>::vpos(4 * c4 + e)] = r.v[i][e];
        }
    }
    if (tid < 2 * n) {
        float g = r.ab;
        if (flags & kGateLogits) g = (tid & 1) ? sigmoid_f(g) : expf(neg_softplus(g));
        sm.ab[tid >> 1][tid & 1] = g;
    }
}

template <typename DT, int D>
// fp32 token inputs need more registers: three workgroups per CU for them
__global__ __launch_bounds__(256, sizeof(DT) == 2 ? 4 : 3) void decode_multi_kernel(
    DecodeMultiParams p) {
    using Sh = DecodeShape<D>;
    using Ms = MultiShape<DT, D>;
    using V = typename Vec4Of<DT>::type;
    constexpr int V4 = Sh::kV4;
    constexpr int STEPS = Sh::kSteps;
    constexpr int KS = Ms::kStage;
    constexpr size_t DD = (size_t)D * D;
    __shared__ MultiSmem<DT, D> sm;

    const int bh = blockIdx.x;
    const int b = bh / p.Hv;
    const int h = bh - b * p.Hv;
    const int g = h / (p.Hv / p.Hk);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;
    const int rsub = lane >> 4;
    const int row0 = wave * Sh::kRowsPerWave + rsub;
    const int K = p.K;

    const int src = p.src_slot[b];
    const int dst = p.dst_slot[b];
    // Token t of this (b, h): q/k at ((b*K + t)*Hk + g)*D, v and out at
    // ((b*K + t)*Hv + h)*D, alpha/beta at (b*K + t)*Hv + h, per-token state
    // at ((b*K + t)*Hv + h)*D*D.
    const size_t tok0 = (size_t)b * K;
    const size_t v_step = (size_t)p.Hv * D;
    DT *o0 = reinterpret_cast<DT *>(p.out) + (tok0 * p.Hv + h) * D;
    float *st0 = p.steps ? p.steps + (tok0 * p.Hv + h) * DD : nullptr;

    if (src >= p.num_slots || dst >= p.num_slots) {
        // A slot index past the pool: no pool access; outputs (and the
        // per-token states) become NaN so the error cannot pass unseen.
        const float nan = __builtin_nanf("");
        for (int t = 0; t < K; ++t) {
            for (int i = threadIdx.x; i < D; i += 256) o0[t * v_step + i] = from_f32<DT>(nan);
            if (st0)
                for (int i = threadIdx.x; i < (int)DD; i += 256)
                    st0[(size_t)t * p.Hv * DD + i] = nan;
        }
        return;
    }

    // First stage's token loads, then the state loads.
    StageRegs<DT, D> sr;
    if (K > 0) stage_load<DT, D>(sr, p, tok0, g, h, min(K, KS));
    f32x4 s[STEPS][V4];
    if (src >= 0) {
        const float *S = p.pool + ((size_t)src * p.Hv + h) * DD;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int c = 0; c < V4; ++c)
                s[st][c] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(
                    S + (size_t)(row0 + 4 * st) * D + 64 * c + 4 * j));
    } else {
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int c = 0; c < V4; ++c) s[st][c] = zero4();
    }

    // The state is cs * s, and the decay goes into the scalar: with
    // cn = cs * alpha the update is one FMA per element, s += (u / cn) k,
    // then cs = cn. When cn would leave [2^-64, 2^64] (alpha = 0 restarts
    // the state), and for every token when per-token states are stored, a
    // pass s *= cn first folds cs and alpha into s; the token then runs with
    // cs = 1 and an effective alpha of 1, and s is the state itself after it.
    float cs = 1.f;
    for (int t0 = 0; t0 < K; t0 += KS) {
        const int n = min(K - t0, KS);
        if (t0 > 0) {
            __syncthreads();  // every wave is done with the previous stage
            stage_load<DT, D>(sr, p, tok0 + t0, g, h, n);
        }
        stage_store<DT, D>(sm, sr, n, p.flags);
        __syncthreads();
        for (int tl = 0; tl < n; ++tl) {
            const int t = t0 + tl;
            float kk[V4][4], qq[V4][4];
#pragma unroll
            for (int c = 0; c < V4; ++c) {
                const V kv = *reinterpret_cast<const V *>(&sm.k[tl][64 * c + 4 * j]);
                const V qv = *reinterpret_cast<const V *>(&sm.q[tl][64 * c + 4 * j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kk[c][e] = to_f32(kv[e]);
                    qq[c][e] = to_f32(qv[e]);
                }
            }
            if (p.flags & kQkL2Norm) {
                float k2 = 0.f, q2 = 0.f;
#pragma unroll
                for (int c = 0; c < V4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        k2 += kk[c][e] * kk[c][e];
                        q2 += qq[c][e] * qq[c][e];
                    }
                const float ik = inv_norm(row16_sum(k2), kL2Eps);
                const float iq = inv_norm(row16_sum(q2), kL2Eps);
#pragma unroll
                for (int c = 0; c < V4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kk[c][e] *= ik;
                        qq[c][e] *= iq;
                    }
            }
            float kq = 0.f;
#pragma unroll
            for (int c = 0; c < V4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) kq += kk[c][e] * qq[c][e];
            DT vr[STEPS];
#pragma unroll
            for (int st = 0; st < STEPS; ++st) vr[st] = sm.v[tl][(wave * 4 + rsub) * STEPS + st];
            const float beta = sm.ab[tl][1];
            float alpha = sm.ab[tl][0];
            float cn = cs * alpha;
            DT *ot = o0 + t * v_step;
            float *stt = st0 ? st0 + (size_t)t * p.Hv * DD : nullptr;
            if (stt || !(cn >= 0x1p-64f && cn <= 0x1p64f)) {
#pragma unroll
                for (int st = 0; st < STEPS; ++st)
#pragma unroll
                    for (int c = 0; c < V4; ++c) s[st][c] *= cn;
                cs = 1.f;
                alpha = 1.f;
                cn = 1.f;
            }
            const float inv = 1.f / cn;
            kq = row16_sum(kq);
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
                float sk = 0.f, sq = 0.f;
#pragma unroll
                for (int c = 0; c < V4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sk += s[st][c][e] * kk[c][e];
                        sq += s[st][c][e] * qq[c][e];
                    }
                sk = cs * row16_sum(sk);
                sq = cs * row16_sum(sq);
                const float u = beta * (to_f32(vr[st]) - alpha * sk);
                const float w = u * inv;
#pragma unroll
                for (int c = 0; c < V4; ++c)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[st][c][e] += w * kk[c][e];
                if (j == 0) ot[row0 + 4 * st] = from_f32<DT>(p.scale * (alpha * sq + u * kq));
                if (stt) {
#pragma unroll
                    for (int c = 0; c < V4; ++c)
                        __builtin_nontemporal_store(
                            s[st][c], reinterpret_cast<f32x4 *>(stt + (size_t)(row0 + 4 * st) * D +
                                                                64 * c + 4 * j));
                }
            }
            cs = cn;
        }
    }

    if (dst >= 0) {
        float *S = p.pool + ((size_t)dst * p.Hv + h) * DD;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int c = 0; c < V4; ++c)
                __builtin_nontemporal_store(
                    s[st][c] * cs,
                    reinterpret_cast<f32x4 *>(S + (size_t)(row0 + 4 * st) * D + 64 * c + 4 * j));
    }
}

hipError_t launch_decode_multi(const DecodeMultiParams &p, int dtype, int D,
                               hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hv));
    const dim3 block(256);
    if (dtype == 1 && D == 128)
        hipLaunchKernelGGL((decode_multi_kernel<__bf16, 128>), grid, block, 0, stream, p);
    else if (dtype == 1 && D == 64)
        hipLaunchKernelGGL((decode_multi_kernel<__bf16, 64>), grid, block, 0, stream, p);
    else if (dtype == 0 && D == 128)
        hipLaunchKernelGGL((decode_multi_kernel<float, 128>), grid, block, 0, stream, p);
    else if (dtype == 0 && D == 64)
        hipLaunchKernelGGL((decode_multi_kernel<float, 64>), grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, int dtype, int D, hipStream_t stream) {
    const dim3 grid((unsigned)((int64_t)p.B * p.Hv));
    const dim3 block(256);
    if (dtype == 1 && D == 128)
        hipLaunchKernelGGL((decode_kernel<__bf16, 128>), grid, block, 0, stream, p);
    else if (dtype == 1 && D == 64)
        hipLaunchKernelGGL((decode_kernel<__bf16, 64>), grid, block, 0, stream, p);
    else if (dtype == 0 && D == 128)
        hipLaunchKernelGGL((decode_kernel<float, 128>), grid, block, 0, stream, p);
    else if (dtype == 0 && D == 64)
        hipLaunchKernelGGL((decode_kernel<float, 64>), grid, block, 0, stream, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gdn
