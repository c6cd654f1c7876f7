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
    const float alpha = p.alpha[bh];
    const float beta = p.beta[bh];

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
// The inputs of token t + 1 are loaded while token t is computed (clamped to
// the last token, so every load is unconditional). Each of the 16 lanes that
// share a row holds the row's dot products after the DPP reduction, and lane
// j == 0 stores the output element.
template <typename DT> struct Vec4Of;
template <> struct Vec4Of<__bf16> { using type = bf16x4; };
template <> struct Vec4Of<float> { using type = f32x4; };

template <typename DT, int V4, int STEPS> struct TokenInputs {
    typename Vec4Of<DT>::type k[V4], q[V4];
    DT v[STEPS];
    float alpha, beta;
};

template <typename DT, int D>
__device__ __forceinline__ void load_token(TokenInputs<DT, D / 64, D / 16> &x, const DT *kp,
                                           const DT *qp, const DT *vp, const float *ap,
                                           const float *bp, int j, int row0) {
    using V = typename Vec4Of<DT>::type;
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
        x.k[c] = *reinterpret_cast<const V *>(kp + 64 * c + 4 * j);
        x.q[c] = *reinterpret_cast<const V *>(qp + 64 * c + 4 * j);
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x.v[st] = vp[row0 + 4 * st];
    x.alpha = *ap;
    x.beta = *bp;
}

template <typename DT, int D>
__global__ __launch_bounds__(256) void decode_multi_kernel(DecodeMultiParams p) {
    using Sh = DecodeShape<D>;
    constexpr int V4 = Sh::kV4;
    constexpr int STEPS = Sh::kSteps;
    constexpr size_t DD = (size_t)D * D;

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
    const size_t qk_step = (size_t)p.Hk * D, v_step = (size_t)p.Hv * D;
    const DT *q0 = reinterpret_cast<const DT *>(p.q) + (tok0 * p.Hk + g) * D;
    const DT *k0 = reinterpret_cast<const DT *>(p.k) + (tok0 * p.Hk + g) * D;
    const DT *v0 = reinterpret_cast<const DT *>(p.v) + (tok0 * p.Hv + h) * D;
    const float *a0 = p.alpha + tok0 * p.Hv + h;
    const float *b0 = p.beta + tok0 * p.Hv + h;
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

    TokenInputs<DT, V4, STEPS> cur, nxt;
    if (K > 0) load_token<DT, D>(cur, k0, q0, v0, a0, b0, j, row0);
    for (int t = 0; t < K; ++t) {
        const int tn = t + 1 < K ? t + 1 : t;
        load_token<DT, D>(nxt, k0 + tn * qk_step, q0 + tn * qk_step, v0 + tn * v_step,
                          a0 + (size_t)tn * p.Hv, b0 + (size_t)tn * p.Hv, j, row0);
        float kk[V4][4], qq[V4][4];
        float kq = 0.f;
#pragma unroll
        for (int c = 0; c < V4; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[c][e] = to_f32(cur.k[c][e]);
                qq[c][e] = to_f32(cur.q[c][e]);
                kq += kk[c][e] * qq[c][e];
            }
        kq = row16_sum(kq);
        const float alpha = cur.alpha, beta = cur.beta;
        DT *ot = o0 + t * v_step;
        float *stt = st0 ? st0 + (size_t)t * p.Hv * DD : nullptr;
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
            const float u = beta * (to_f32(cur.v[st]) - alpha * sk);
#pragma unroll
            for (int c = 0; c < V4; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[st][c][e] = alpha * s[st][c][e] + u * kk[c][e];
            if (j == 0) ot[row0 + 4 * st] = from_f32<DT>(p.scale * (alpha * sq + u * kq));
            if (stt) {
#pragma unroll
                for (int c = 0; c < V4; ++c)
                    __builtin_nontemporal_store(
                        s[st][c], reinterpret_cast<f32x4 *>(stt + (size_t)(row0 + 4 * st) * D +
                                                            64 * c + 4 * j));
            }
        }
        cur = nxt;
    }

    if (dst >= 0) {
        float *S = p.pool + ((size_t)dst * p.Hv + h) * DD;
#pragma unroll
        for (int st = 0; st < STEPS; ++st)
#pragma unroll
            for (int c = 0; c < V4; ++c)
                __builtin_nontemporal_store(
                    s[st][c],
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
