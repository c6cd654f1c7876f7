// gdn_api.hip -- the C ABI (include/gdn.h): argument validation and launch.
//
// Every entry point checks its arguments on the host before touching the HIP
// runtime, so a rejected call has no side effects and costs no device work.
// Accepted calls enqueue their kernels on the caller's stream and return.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_launch.hpp"
#include "gdn_validate.hpp"

namespace {

using namespace gdn::val;

thread_local char g_detail[256];

constexpr uint32_t kKnownFlags = GDN_QK_L2NORM | GDN_GATE_LOGITS;
static_assert(GDN_QK_L2NORM == gdn::kQkL2Norm && GDN_GATE_LOGITS == gdn::kGateLogits,
              "flag values of the ABI and the kernels");

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

// GDN_DEBUG=1 in the environment turns on the synchronous checks: the
// contents of cu_seqlens before a packed prefill, and the workspace's status
// word (set by a kernel whose bounded wait for another wave ran out) after a
// prefill that used a workspace. They synchronise the stream, so they are
// skipped for a stream that is being captured into a graph.
bool debug_checks(hipStream_t stream) {
    const char *e = getenv("GDN_DEBUG");
    if (!e || e[0] != '1') return false;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cap) == hipSuccess && cap == hipStreamCaptureStatusNone;
}

gdn_status_t debug_cu_seqlens(const int32_t *cu, int32_t N, int64_t total_T, hipStream_t stream) {
    std::vector<int32_t> h((size_t)N + 1);
    hipError_t e = hipMemcpyAsync(h.data(), cu, h.size() * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "GDN_DEBUG copy of cu_seqlens");
    return check_cu_seqlens(h.data(), N, total_T);
}

gdn_status_t debug_clear_status(void *ws, hipStream_t stream) {
    const hipError_t e = hipMemsetAsync(ws, 0, gdn::kWsStatusBytes, stream);
    return e == hipSuccess ? GDN_OK : hip_fail(e, "GDN_DEBUG clear of the status word");
}

gdn_status_t debug_read_status(const void *ws, hipStream_t stream) {
    int32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, ws, 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "GDN_DEBUG read of the status word");
    if (word != 0) {
        snprintf(g_detail, sizeof g_detail,
                 "a prefill kernel's bounded wait for another wave ran out (status word 0x%x); "
                 "results of this call are invalid", (unsigned)word);
        return GDN_ERR_HIP;
    }
    return GDN_OK;
}

// Launch of a prefill with the debug checks around it.
gdn_status_t run_prefill(const gdn::PrefillParams &p, int dtype, int D, int cus, void *ws,
                         size_t ws_bytes, int64_t slots, hipStream_t stream, bool debug,
                         const char *where) {
    const bool ws_used = ws && ws_bytes >= gdn::kWsStatusBytes;
    if (debug && ws_used) {
        const gdn_status_t st = debug_clear_status(ws, stream);
        if (st != GDN_OK) return st;
    }
    const hipError_t e = gdn::launch_prefill(p, dtype, D, cus, ws, ws_bytes, slots, stream);
    if (e != hipSuccess) return hip_fail(e, where);
    if (debug && ws_used) return debug_read_status(ws, stream);
    return GDN_OK;
}

// Device scratch of gdn_prefill_chunked_noalloc: the workspace of callers
// that cannot allocate. Each device holds its own copy for the life of the
// process. In host code the array's name is only a stand-in; its device
// address on the current device comes from hipGetSymbolAddress, taken once
// per device and kept in scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> g_scratch_ptr[kMaxDevices];

gdn_status_t scratch_ptr(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return hip_fail(hipErrorInvalidDevice, "scratch device index");
    uintptr_t a = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (a == 0) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        a = reinterpret_cast<uintptr_t>(p);
        g_scratch_ptr[dev].store(a, std::memory_order_release);  // the same value from any thread
    }
    *ptr = reinterpret_cast<void *>(a);
    return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status_t s) {
    switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "a size is out of range or inconsistent";
    case GDN_ERR_UNSUPPORTED:
        return "unsupported dtype or head dimension (Dk == Dv in {64, 128}), or a shape whose "
               "scratch exceeds the static 64 MiB of gdn_prefill_chunked_noalloc";
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
    // few long sequences: the segmented path, whose layout also holds the above
    const size_t seg = packed ? 0
                              : gdn::prefill_seg_ws_bytes(num_seqs, tokens, Hv, Dk,
                                                          dtype == GDN_BF16 ? 1 : 0, cus);
    return gdn::kWsStatusBytes + (seg > recs ? seg : recs);
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
    return run_prefill(p, dtype == GDN_BF16 ? 1 : 0, Dk, cus, workspace, workspace_bytes, slots,
                       stream, debug_checks(stream), "gdn_prefill_chunked launch");
}

gdn_status_t gdn_prefill_chunked_noalloc(const void *q, const void *k, const void *v,
                                         const float *alpha, const float *beta,
                                         const float *initial_state, void *out,
                                         float *final_state, float *prefix_states,
                                         int32_t prefix_interval, int32_t B, int64_t T, int32_t Hk,
                                         int32_t Hv, int32_t Dk, int32_t Dv, gdn_dtype_t dtype,
                                         float scale, uint32_t flags, hipStream_t stream) {
    gdn_status_t st = check_heads(Hk, Hv, Dk, Dv);
    if (st != GDN_OK) return st;
    if (!known_dtype(dtype)) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || T < 0) return GDN_ERR_BAD_SHAPE;
    const size_t want = gdn_prefill_workspace_size(B, T, Hk, Hv, Dk, Dv, dtype, 0);
    if (want > kNoAllocScratchBytes) {
        snprintf(g_detail, sizeof g_detail,
                 "gdn_prefill_chunked_noalloc: this shape needs %zu bytes of scratch, the "
                 "library's static scratch holds %zu",
                 want, kNoAllocScratchBytes);
        return GDN_ERR_UNSUPPORTED;
    }
    void *ws = nullptr;
    if (want > 0 && (st = scratch_ptr(&ws)) != GDN_OK) return st;
    return gdn_prefill_chunked(q, k, v, alpha, beta, initial_state, out, final_state,
                               prefix_states, prefix_interval, B, T, Hk, Hv, Dk, Dv, dtype, scale,
                               flags, want > 0 ? ws : nullptr, want, stream);
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
    const bool debug = debug_checks(stream);
    if (debug && (st = debug_cu_seqlens(cu_seqlens, N, total_T, stream)) != GDN_OK) return st;
    int cus = 0;
    if ((st = device_cus(&cus)) != GDN_OK) return st;
    gdn::PrefillParams p{q,          k,  v,  alpha, beta, initial_state, out, final_state,
                         cu_seqlens, 0,  N,  Hk,    Hv,   scale,         prefix_states,
                         prefix_interval, flags, (int64_t)Hv * Dv, false, false};
    p.total_tokens = total_T;
    const int64_t slots = gdn::prefill_ws_slots(N, total_T, 0, true);
    return run_prefill(p, dtype == GDN_BF16 ? 1 : 0, Dk, cus, workspace, workspace_bytes, slots,
                       stream, debug, "gdn_varlen_prefill launch");
}

gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v, const float *alpha,
                             const float *beta, float *state, void *out, int32_t B, int32_t Hk,
                             int32_t Hv, int32_t Dk, int32_t Dv, gdn_dtype_t dtype, float scale,
                             uint32_t flags, hipStream_t stream) {
    gdn_status_t st = check_decode(q, k, v, alpha, beta, state, out, B, Hk, Hv, Dk, Dv, dtype);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
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
    gdn_status_t st = check_decode_multi(q, k, v, alpha, beta, state_pool, num_slots, src_slot,
                                         dst_slot, out, step_states, B, K, Hk, Hv, Dk, Dv, dtype);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_UNSUPPORTED;
    gdn::DecodeMultiParams p{q,        k,        v,   alpha,       beta, state_pool,
                             src_slot, dst_slot, out, step_states, B,    K,
                             Hk,       Hv,       num_slots, scale, flags};
    hipError_t e = gdn::launch_decode_multi(p, dtype == GDN_BF16 ? 1 : 0, Dk, stream);
    if (e != hipSuccess) return hip_fail(e, "gdn_decode_multi launch");
    return GDN_OK;
}

}  // extern "C"
