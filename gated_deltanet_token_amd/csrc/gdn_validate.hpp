// gdn_validate.hpp -- host-side argument checks of the C ABI (include/gdn.h).
//
// Plain C++ with no HIP runtime call, so that the same code is compiled into
// the library and into a host-only test program built with AddressSanitizer
// and UndefinedBehaviorSanitizer. Every function returns a status and has no
// side effects.
#pragma once
#include <stdint.h>
#include <stddef.h>

#include "../../include/gdn.h"

namespace gdn {
namespace val {

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

static inline Range range_of(const void *p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, bytes > 0 && p ? a + (uintptr_t)bytes : a};
}

static inline bool overlap(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

static inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// acc *= f with overflow detection (all factors >= 0).
static inline bool mul_ok(int64_t &acc, int64_t f) {
    if (f < 0 || acc < 0) return false;
    if (f != 0 && acc > INT64_MAX / f) return false;
    acc *= f;
    return true;
}

static inline gdn_status_t check_heads(int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv) {
    if (Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1) return GDN_ERR_BAD_SHAPE;
    if (Hv % Hk != 0) return GDN_ERR_BAD_SHAPE;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

static inline bool known_dtype(gdn_dtype_t d) { return d == GDN_F32 || d == GDN_BF16; }

// Shared checks of the two prefill entry points. `tokens` is B*T or total_T,
// `nstates` is B or N, `cu_count` the number of cu_seqlens entries (0 for a
// dense batch).
static inline gdn_status_t check_prefill(const void *q, const void *k, const void *v, const float *alpha,
                                  const float *beta, const float *s0, const void *out,
                                  const float *sf, const float *prefix, int64_t prefix_rows,
                                  const int32_t *cu, int64_t cu_count, int64_t tokens,
                                  int64_t nstates, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                  gdn_dtype_t dtype, const void *ws, size_t ws_bytes) {
    if (!known_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
    if (tokens < 0 || nstates < 1 || prefix_rows < 0) return GDN_ERR_BAD_SHAPE;
    const int64_t es = dtype == GDN_BF16 ? 2 : 4;
    int64_t nqk = tokens, nv = tokens, nab = tokens, nst = nstates;
    if (!mul_ok(nqk, Hk) || !mul_ok(nqk, Dk) || !mul_ok(nqk, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nv, Hv) || !mul_ok(nv, Dv) || !mul_ok(nv, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nab, Hv) || !mul_ok(nab, 4)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nst, Hv) || !mul_ok(nst, Dv) || !mul_ok(nst, Dk) || !mul_ok(nst, 4))
        return GDN_ERR_BAD_SHAPE;
    if (nstates * Hv > 0x7FFFFFFF / 8) return GDN_ERR_BAD_SHAPE;  // grid size
    int64_t npre = prefix ? prefix_rows : 0;
    if (!mul_ok(npre, Hv) || !mul_ok(npre, Dv) || !mul_ok(npre, Dk) || !mul_ok(npre, 4))
        return GDN_ERR_BAD_SHAPE;

    if (tokens > 0 && (!q || !k || !v || !alpha || !beta || !out)) return GDN_ERR_NULL_POINTER;
    if (cu_count > 0 && !cu) return GDN_ERR_NULL_POINTER;
    const void *ptrs[] = {q, k, v, alpha, beta, s0, out, sf, prefix, cu, ws};
    for (const void *ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;
    if (ws_bytes > (size_t)INT64_MAX) return GDN_ERR_BAD_SHAPE;

    const Range rq = range_of(q, nqk), rk = range_of(k, nqk), rv = range_of(v, nv);
    const Range ra = range_of(alpha, nab), rb = range_of(beta, nab);
    const Range rs0 = range_of(s0, nst), ro = range_of(out, nv), rsf = range_of(sf, nst);
    const Range rcu = range_of(cu, cu_count * 4);
    const Range inputs[] = {rq, rk, rv, ra, rb, rs0, rcu};
    for (const Range &r : inputs)
        if (overlap(ro, r) || overlap(ro, rsf)) return GDN_ERR_ALIAS;
    if (sf && sf != s0) {
        for (const Range &r : inputs)
            if (overlap(rsf, r)) return GDN_ERR_ALIAS;
    }
    if (sf && sf == s0) {
        const Range others[] = {rq, rk, rv, ra, rb, rcu};
        for (const Range &r : others)
            if (overlap(rsf, r)) return GDN_ERR_ALIAS;
    }
    const Range rws = range_of(ws, (int64_t)ws_bytes);
    const Range all[] = {rq, rk, rv, ra, rb, rs0, ro, rsf, rcu};
    for (const Range &r : all)
        if (overlap(rws, r)) return GDN_ERR_ALIAS;
    const Range rpre = range_of(prefix, npre);
    for (const Range &r : all)
        if (overlap(rpre, r)) return GDN_ERR_ALIAS;
    if (overlap(rpre, rws)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

static inline gdn_status_t check_decode(const void *q, const void *k, const void *v, const float *alpha,
                                 const float *beta, const float *state, const void *out,
                                 int32_t B, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                 gdn_dtype_t dtype) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (B < 1) return GDN_ERR_BAD_SHAPE;
    if (!known_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
    if (!q || !k || !v || !alpha || !beta || !state || !out) return GDN_ERR_NULL_POINTER;
    const int64_t es = dtype == GDN_BF16 ? 2 : 4;
    int64_t nqk = B, nv = B, nab = B, nst = B;
    if (!mul_ok(nqk, Hk) || !mul_ok(nqk, Dk) || !mul_ok(nqk, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nv, Hv) || !mul_ok(nv, Dv) || !mul_ok(nv, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nab, Hv) || !mul_ok(nab, 4)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nst, Hv) || !mul_ok(nst, Dv) || !mul_ok(nst, Dk) || !mul_ok(nst, 4))
        return GDN_ERR_BAD_SHAPE;
    if ((int64_t)B * Hv > 0x7FFFFFFF) return GDN_ERR_BAD_SHAPE;
    const void *ptrs[] = {q, k, v, alpha, beta, state, out};
    for (const void *ptr : ptrs)
        if (!aligned16(ptr)) return GDN_ERR_MISALIGNED;
    const Range rq = range_of(q, nqk), rk = range_of(k, nqk), rv = range_of(v, nv);
    const Range ra = range_of(alpha, nab), rb = range_of(beta, nab);
    const Range rs = range_of(state, nst), ro = range_of(out, nv);
    const Range inputs[] = {rq, rk, rv, ra, rb};
    for (const Range &r : inputs)
        if (overlap(ro, r) || overlap(rs, r)) return GDN_ERR_ALIAS;
    if (overlap(ro, rs)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

static inline gdn_status_t check_decode_multi(const void *q, const void *k, const void *v,
                                       const float *alpha, const float *beta,
                                       const float *state_pool, int32_t num_slots,
                                       const int32_t *src_slot, const int32_t *dst_slot,
                                       const void *out, const float *step_states, int32_t B,
                                       int32_t K, int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                       gdn_dtype_t dtype) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (B < 1 || K < 0 || num_slots < 1) return GDN_ERR_BAD_SHAPE;
    if (!known_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
    if (!state_pool || !src_slot || !dst_slot) return GDN_ERR_NULL_POINTER;
    if (K > 0 && (!q || !k || !v || !alpha || !beta || !out)) return GDN_ERR_NULL_POINTER;
    const int64_t es = dtype == GDN_BF16 ? 2 : 4;
    int64_t ntok = B;
    if (!mul_ok(ntok, K)) return GDN_ERR_BAD_SHAPE;
    int64_t nqk = ntok, nv = ntok, nab = ntok, nsteps = ntok, npool = num_slots;
    if (!mul_ok(nqk, Hk) || !mul_ok(nqk, Dk) || !mul_ok(nqk, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nv, Hv) || !mul_ok(nv, Dv) || !mul_ok(nv, es)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nab, Hv) || !mul_ok(nab, 4)) return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(nsteps, Hv) || !mul_ok(nsteps, Dv) || !mul_ok(nsteps, Dk) || !mul_ok(nsteps, 4))
        return GDN_ERR_BAD_SHAPE;
    if (!mul_ok(npool, Hv) || !mul_ok(npool, Dv) || !mul_ok(npool, Dk) || !mul_ok(npool, 4))
        return GDN_ERR_BAD_SHAPE;
    if ((int64_t)B * Hv > 0x7FFFFFFF) return GDN_ERR_BAD_SHAPE;
    const void *ptrs[] = {q, k, v, alpha, beta, state_pool, out, step_states};
    for (const void *ptr : ptrs)
        if (ptr && !aligned16(ptr)) return GDN_ERR_MISALIGNED;
    if ((reinterpret_cast<uintptr_t>(src_slot) | reinterpret_cast<uintptr_t>(dst_slot)) & 3u)
        return GDN_ERR_MISALIGNED;
    const Range rq = range_of(q, nqk), rk = range_of(k, nqk), rv = range_of(v, nv);
    const Range ra = range_of(alpha, nab), rb = range_of(beta, nab);
    const Range rss = range_of(src_slot, (int64_t)B * 4), rds = range_of(dst_slot, (int64_t)B * 4);
    const Range rp = range_of(state_pool, npool), ro = range_of(out, nv);
    const Range rst = range_of(step_states, nsteps);
    const Range reads[] = {rq, rk, rv, ra, rb, rss, rds};
    const Range writes[] = {rp, ro, rst};
    for (const Range &w : writes)
        for (const Range &r : reads)
            if (overlap(w, r)) return GDN_ERR_ALIAS;
    if (overlap(rp, ro) || overlap(rp, rst) || overlap(ro, rst)) return GDN_ERR_ALIAS;
    return GDN_OK;
}

// Contents of cu_seqlens (a host copy of its N + 1 entries): starts at 0,
// never decreases, ends at total_T. The library runs this only when the
// environment sets GDN_DEBUG=1 (it needs a synchronous device-to-host copy).
static inline gdn_status_t check_cu_seqlens(const int32_t *cu, int32_t N, int64_t total_T) {
    if (!cu) return GDN_ERR_NULL_POINTER;
    if (N < 1) return GDN_ERR_BAD_SHAPE;
    if (cu[0] != 0) return GDN_ERR_BAD_SHAPE;
    for (int32_t n = 0; n < N; ++n)
        if (cu[n + 1] < cu[n]) return GDN_ERR_BAD_SHAPE;
    if ((int64_t)cu[N] != total_T) return GDN_ERR_BAD_SHAPE;
    return GDN_OK;
}

}  // namespace val
}  // namespace gdn
