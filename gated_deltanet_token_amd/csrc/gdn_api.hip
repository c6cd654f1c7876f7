// gdn_api.hip -- the C ABI (include/gdn.h): argument validation and launch.
//
// Every entry point checks its arguments on the host before touching the HIP
// runtime, so a rejected call has no side effects and costs no device work.
// Accepted calls enqueue their kernels on the caller's stream and return.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/gdn.h"
#include "gdn_launch.hpp"

namespace {

thread_local char g_detail[256];

constexpr uint32_t kKnownFlags = GDN_QK_L2NORM | GDN_GATE_LOGITS;
static_assert(GDN_QK_L2NORM == gdn::kQkL2Norm && GDN_GATE_LOGITS == gdn::kGateLogits,
              "flag values of the ABI and the kernels");

struct Range {
    uintptr_t lo, hi;  // [lo, hi); empty when lo == hi
};

Range range_of(const void *p, int64_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, bytes > 0 && p ? a + (uintptr_t)bytes : a};
}

bool overlap(const Range &a, const Range &b) {
    if (a.lo == a.hi || b.lo == b.hi) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b*c*... as int64 with overflow detection (all factors >= 0)
bool mul_ok(int64_t &acc, int64_t f) {
    if (f < 0) return false;
    if (f != 0 && acc > INT64_MAX / f) return false;
    acc *= f;
    return true;
}

gdn_status_t check_heads(int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv) {
    if (Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1) return GDN_ERR_BAD_SHAPE;
    if (Hv % Hk != 0) return GDN_ERR_BAD_SHAPE;
    if (Dk != Dv || (Dk != 64 && Dk != 128)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status_t hip_fail(hipError_t e, const char *where) {
    snprintf(g_detail, sizeof g_detail, "HIP error in %s: %s (%d)", where, hipGetErrorString(e),
             (int)e);
    return GDN_ERR_HIP;
}

gdn_status_t device_cus(int *cus) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    e = hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    return GDN_OK;
}

// Shared checks of the two prefill entry points. `tokens` is B*T or total_T,
// `nstates` is B or N.
gdn_status_t check_prefill(const void *q, const void *k, const void *v, const float *alpha,
                           const float *beta, const float *s0, const void *out, const float *sf,
                           const float *prefix, int64_t prefix_rows,
                           const int32_t *cu, int64_t cu_count, int64_t tokens, int64_t nstates,
                           int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, gdn_dtype_t dtype,
                           const void *ws, size_t ws_bytes) {
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
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

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status_t s) {
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case GDN_ERR_UNSUPPORTED: return "unsupported dtype or head dimension (Dk == Dv in {64, 128})";
    case GDN_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case GDN_ERR_ALIAS: return "forbidden overlap between buffers";
    case GDN_ERR_HIP: return g_detail[0] ? g_detail : "HIP runtime error";
    }
    return "unknown status";
}

int32_t gdn_version(void) { return 500; }

size_t gdn_prefill_workspace_size(int32_t num_seqs, int64_t tokens, int32_t Hk, int32_t Hv,
                                  int32_t Dk, int32_t Dv, gdn_dtype_t dtype, int32_t packed) {
    if (check_heads(Hk, Hv, Dk, Dv) != GDN_OK) return 0;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return 0;
    if (num_seqs < 1 || tokens < 0 || (packed && tokens > 0x7FFFFFFF)) return 0;
    int64_t total = packed ? tokens : (int64_t)num_seqs;
    if (!packed && !mul_ok(total, tokens)) return 0;
    if (total == 0) return 0;
    int cus = 0;
    if (device_cus(&cus) != GDN_OK) return 0;
    if (!gdn::prefill_wants_workspace((int64_t)num_seqs * Hv, cus)) return 0;
    const int64_t slots = gdn::prefill_ws_slots(num_seqs, total, packed ? 0 : tokens, packed != 0);
    const size_t recs = gdn::prefill_ws_bytes(slots, Hv, dtype == GDN_BF16 ? 1 : 0);
    const size_t two_pass =
        packed ? recs
               : gdn::prefill_two_pass_ws_bytes(num_seqs, tokens, Hv, Dk,
                                                dtype == GDN_BF16 ? 1 : 0, cus, recs);
    // few long sequences: the segmented path, whose layout also holds the above
    const size_t seg = packed ? 0
                              : gdn::prefill_seg_ws_bytes(num_seqs, tokens, Hv, Dk,
                                                          dtype == GDN_BF16 ? 1 : 0, cus);
    return seg > two_pass ? seg : two_pass;
}

gdn_status_t gdn_prefill_chunked(const void *q, const void *k, const void *v, const float *alpha,
                                 const float *beta, const float *initial_state, void *out,
                                 float *final_state, float *prefix_states, int32_t prefix_interval,
                                 int32_t B, int64_t T, int32_t Hk, int32_t Hv, int32_t Dk,
                                 int32_t Dv, gdn_dtype_t dtype, float scale, uint32_t flags,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || T < 0) return GDN_ERR_BAD_SHAPE;
    if (prefix_states && prefix_interval < 1) return GDN_ERR_BAD_SHAPE;
    int64_t tokens = B;
    if (!mul_ok(tokens, T)) return GDN_ERR_BAD_SHAPE;
    // B * floor(T / (64 m)) prefix rows
    const int64_t prefix_rows = prefix_states ? (int64_t)B * (T / (64 * (int64_t)prefix_interval)) : 0;
    st = check_prefill(q, k, v, alpha, beta, initial_state, out, final_state, prefix_states,
                       prefix_rows, nullptr, 0, tokens, B, Hk, Hv, Dk, Dv, dtype, workspace,
                       workspace_bytes);
    if (st != GDN_OK) return st;
    if (tokens == 0 && !final_state) return GDN_OK;  // nothing to write
    int cus = 0;
    if ((st = device_cus(&cus)) != GDN_OK) return st;
    gdn::PrefillParams p{q,  k,     v,     alpha,         beta,
                         initial_state, out, final_state, nullptr, T,
                         B,  Hk,    Hv,    scale,         prefix_rows ? prefix_states : nullptr,
                         prefix_interval, flags, (int64_t)Hv * Dv, false, false};
    const int64_t slots = gdn::prefill_ws_slots(B, tokens, T, false);
    const hipError_t e = gdn::launch_prefill(p, dtype == GDN_BF16 ? 1 : 0, Dk, cus, workspace,
                                             workspace_bytes, slots, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_prefill_chunked launch");
    return GDN_OK;
}

gdn_status_t gdn_varlen_prefill(const void *q, const void *k, const void *v, const float *alpha,
                                const float *beta, const int32_t *cu_seqlens, int32_t N,
                                int64_t total_T, const float *initial_state, void *out,
                                float *final_state, float *prefix_states, int32_t prefix_interval,
                                int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv, gdn_dtype_t dtype,
                                float scale, uint32_t flags, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (N < 1 || total_T < 0 || total_T > 0x7FFFFFFF) return GDN_ERR_BAD_SHAPE;
    if (!cu_seqlens) return GDN_ERR_NULL_POINTER;
    if (prefix_states && prefix_interval < 1) return GDN_ERR_BAD_SHAPE;
    // floor(total_T / (64 m)) + N prefix rows
    const int64_t prefix_rows =
        prefix_states ? total_T / (64 * (int64_t)prefix_interval) + N : 0;
    st = check_prefill(q, k, v, alpha, beta, initial_state, out, final_state, prefix_states,
                       prefix_rows, cu_seqlens, (int64_t)N + 1, total_T, N, Hk, Hv, Dk, Dv, dtype,
                       workspace, workspace_bytes);
    if (st != GDN_OK) return st;
    if (total_T == 0 && !final_state) return GDN_OK;
    int cus = 0;
    if ((st = device_cus(&cus)) != GDN_OK) return st;
    gdn::PrefillParams p{q,          k,  v,  alpha, beta, initial_state, out, final_state,
                         cu_seqlens, 0,  N,  Hk,    Hv,   scale,         prefix_states,
                         prefix_interval, flags, (int64_t)Hv * Dv, false, false};
    const int64_t slots = gdn::prefill_ws_slots(N, total_T, 0, true);
    const hipError_t e = gdn::launch_prefill(p, dtype == GDN_BF16 ? 1 : 0, Dk, cus, workspace,
                                             workspace_bytes, slots, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_varlen_prefill launch");
    return GDN_OK;
}

gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *state, void *out, int32_t B, int32_t Hk,
                             int32_t Hv, int32_t Dk, int32_t Dv, gdn_dtype_t dtype, float scale,
                             uint32_t flags, hipStream_t stream) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B < 1) return GDN_ERR_BAD_SHAPE;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
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
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    gdn::DecodeParams p{q, k, v, alpha, beta, state, out, B, Hk, Hv, scale, flags};
    e = gdn::launch_decode(p, dtype == GDN_BF16 ? 1 : 0, Dk, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_decode_step launch");
    return GDN_OK;
}

gdn_status_t gdn_decode_multi(const void *q, const void *k, const void *v, const float *alpha,
                              const float *beta, float *state_pool, int32_t num_slots,
                              const int32_t *src_slot, const int32_t *dst_slot, void *out,
                              float *step_states, int32_t B, int32_t K, int32_t Hk, int32_t Hv,
                              int32_t Dk, int32_t Dv, gdn_dtype_t dtype, float scale,
                              uint32_t flags, hipStream_t stream) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || K < 0 || num_slots < 1) return GDN_ERR_BAD_SHAPE;
    if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
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
    gdn::DecodeMultiParams p{q,        k,        v,   alpha,       beta, state_pool,
                             src_slot, dst_slot, out, step_states, B,    K,
                             Hk,       Hv,       num_slots, scale, flags};
    hipError_t e = gdn::launch_decode_multi(p, dtype == GDN_BF16 ? 1 : 0, Dk, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_decode_multi launch");
    return GDN_OK;
}

}  // extern "C"
