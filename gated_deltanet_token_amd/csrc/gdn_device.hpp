// gdn_device.hpp -- device-side building blocks for the gfx950 kernels.
//
// MFMA conventions used throughout (wave64, 16x16 output tiles):
//   * lane l, group g4 = l >> 4 (0..3), column c = l & 15;
//   * accumulator ("C layout"): lane l holds C[4*g4 + r][c], r = 0..3;
//   * an operand "fragment" is 8 k-values per lane. Lane l of the A operand
//     holds row c of A, lane l of the B operand holds column c of B; the 8
//     values of group g4 cover 8 k positions. Which 8 positions is free as
//     long as A and B agree, because the contraction sums over all of them.
//     Two assignments are used:
//       natural : k = 8*g4 + e              (e = 0..7)
//       chain   : k = 4*g4 + e (e < 4), 16 + 4*g4 + (e - 4) (e >= 4)
//     The chain assignment is exactly what two stacked accumulator tiles
//     hold, so a product whose B operand comes from registers (an
//     accumulator reused as the next operand) needs no lane exchange.
//   * bf16 fragments feed v_mfma_f32_16x16x32_bf16 (one instruction per
//     16x16x32 step); fp32 fragments feed eight v_mfma_f32_16x16x4_f32, the
//     e-th of which sees, in lane group g4, the k position of element e.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename DT> struct FragT;
template <> struct FragT<__bf16> { using type = bf16x8; };
template <> struct FragT<float> { using type = f32x8; };
template <typename DT> using Frag = typename FragT<DT>::type;

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// C += A * B over one 32-deep k step.
__device__ __forceinline__ f32x4 mma(const bf16x8 &a, const bf16x8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const f32x8 &a, const f32x8 &b, f32x4 c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// C += A * B over a 16-deep k step given as 4 values per lane (k = 4*g4 + e).
__device__ __forceinline__ f32x4 mma_k16(const float (&a)[4], const float (&b)[4], f32x4 c,
                                         __bf16) {
    bf16x8 fa, fb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        fa[e] = (__bf16)a[e];
        fb[e] = (__bf16)b[e];
        fa[e + 4] = (__bf16)0.f;
        fb[e + 4] = (__bf16)0.f;
    }
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(const float (&a)[4], const float (&b)[4], f32x4 c,
                                         float) {
#pragma unroll
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], c, 0, 0, 0);
    return c;
}

// Two stacked accumulator tiles (k rows 0..15 and 16..31 of a 32-deep step)
// as a B fragment in the chain assignment.
__device__ __forceinline__ void c_to_frag(const f32x4 &lo, const f32x4 &hi, bf16x8 &f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f[r] = (__bf16)lo[r];
        f[r + 4] = (__bf16)hi[r];
    }
}
__device__ __forceinline__ void c_to_frag(const f32x4 &lo, const f32x4 &hi, f32x8 &f) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        f[r] = lo[r];
        f[r + 4] = hi[r];
    }
}

// LDS fragment loads. `p` points at (row, k0 + offset of this lane group).
// natural: 8 consecutive elements at p.
__device__ __forceinline__ void ld_nat(const __bf16 *p, bf16x8 &f) {
    f = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void ld_nat(const float *p, f32x8 &f) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = a[e];
        f[e + 4] = b[e];
    }
}
// chain: elements p[0..3] and p[16..19].
__device__ __forceinline__ void ld_chain(const __bf16 *p, bf16x8 &f) {
    const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4 *>(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = a[e];
        f[e + 4] = b[e];
    }
}
__device__ __forceinline__ void ld_chain(const float *p, f32x8 &f) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = a[e];
        f[e + 4] = b[e];
    }
}
// chain assignment down a column: p[k * pitch] for the 8 chain positions.
template <typename DT>
__device__ __forceinline__ void ld_chain_col(const DT *p, int pitch, Frag<DT> &f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = p[e * pitch];
        f[e + 4] = p[(16 + e) * pitch];
    }
}

// Sum over the 16 lanes of each DPP row (lanes 16*i .. 16*i+15); every lane
// of the row receives the total.
#define GDN_DPP(x, ctrl)                                                                  \
    __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, (x)), (ctrl), \
                                                       0xF, 0xF, false))
__device__ __forceinline__ float row16_sum(float x) {
    x += GDN_DPP(x, 0xB1);   // quad_perm [1,0,3,2]
    x += GDN_DPP(x, 0x4E);   // quad_perm [2,3,0,1]
    x += GDN_DPP(x, 0x141);  // row_half_mirror
    x += GDN_DPP(x, 0x140);  // row_mirror
    return x;
}

// Four consecutive entries (row, col0 .. col0 + 3) of the identity matrix.
__device__ __forceinline__ f32x4 eye4(int row, int col0) {
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = row == col0 + e ? 1.f : 0.f;
    return r;
}

// Gates from logits: log(alpha) = -softplus(a) (stable for either sign of
// a), beta = sigmoid(b).
__device__ __forceinline__ float neg_softplus(float a) {
    return -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))));
}
__device__ __forceinline__ float sigmoid_f(float b) { return 1.f / (1.f + expf(-b)); }

// 1 / sqrt(x + eps) with an IEEE square root and division (x: a sum of squares).
__device__ __forceinline__ float inv_norm(float x, float eps) { return 1.f / sqrtf(x + eps); }

// Conversions between the storage type and fp32.
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename DT> __device__ __forceinline__ DT from_f32(float x);
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

}  // namespace gdn
