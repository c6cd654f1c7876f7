/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet token mixer.
 *
 * The layer: the Gated DeltaNet blocks that fill 48 of the 64 layers of the
 * hybrid stack in "The Hybrid Attention in Qwen3.8-27B" (section "Why 27B
 * parameters can carry 262K tokens": layout 16 x (3 x (Gated DeltaNet ->
 * FFN) -> 1 x (Gated Attention -> FFN)); section "Grouped-query attention
 * multiplies on top of that": 16 query/key heads, 48 value heads, head
 * dimension 128). Each value head keeps one fixed-size state whatever the
 * context length ("The economics of hybrid attention", TL;DR: the 48 blocks
 * hold a fixed ~150 MiB, i.e. 48 x 48 x 128 x 128 fp32).
 *
 * The pages name the layer but do not print its recurrence; this library
 * computes the published gated delta rule, for each sequence and value head
 * h (S in R^{Dv x Dk}, row-major; q/k head g = h / (Hv / Hk)):
 *
 *     S_t = alpha_t * S_{t-1} * (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers, contiguous, in the layouts
 *    stated per call, and 16-byte aligned. q, k, v and out have the element
 *    type `dtype` (GDN_BF16 or GDN_F32); alpha, beta and states are fp32.
 *  - Ownership: the caller owns every buffer. The library allocates and
 *    frees no memory, creates no stream or event, keeps no pointer after the
 *    call returns and holds no mutable global state; calls are re-entrant
 *    and thread-safe (two calls that share a workspace must not overlap in
 *    time on the device, like any two users of one buffer).
 *  - Asynchrony: each call validates its arguments on the host, enqueues
 *    kernels on `stream` and returns without synchronising. Results are
 *    ready when the stream reaches that point.
 *  - Validation happens before any HIP call; a call that fails validation
 *    has no side effects. GDN_ERR_HIP reports a failure of the HIP runtime
 *    (no device, launch error); gdn_status_string() then gives the detail
 *    for the calling thread.
 *  - Values are not validated: NaN or Inf inputs propagate. alpha and beta
 *    are meant to lie in [0, 1]; alpha is clamped to >= FLT_MIN before its
 *    logarithm is taken.
 *  - Debug checks: with GDN_DEBUG=1 in the environment, the prefill calls
 *    also run synchronous checks (they synchronise `stream`, and are skipped
 *    while the stream is being captured into a graph): the contents of
 *    cu_seqlens (GDN_ERR_BAD_SHAPE before any launch when malformed), and,
 *    after a call that used a workspace, its status word (GDN_ERR_HIP when a
 *    kernel's bounded wait for another wave of its workgroup ran out, which
 *    a correct run never does).
 *  - `out` must not overlap any input. `final_state` must either be the same
 *    pointer as `initial_state` (in-place update) or not overlap it, and it
 *    must not overlap any other argument.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_POINTER = 1, /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,    /* a size is out of range or inconsistent */
    GDN_ERR_UNSUPPORTED = 3,  /* a valid shape the library has no kernel for */
    GDN_ERR_MISALIGNED = 4,   /* a pointer is not 16-byte aligned */
    GDN_ERR_ALIAS = 5,        /* forbidden overlap between buffers */
    GDN_ERR_HIP = 6           /* HIP runtime error; see gdn_status_string */
} gdn_status_t;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype_t; /* type of q, k, v, out */

/*
 * Input preparation done inside the kernels: the `flags` argument of the
 * compute calls (bitwise OR; 0 = inputs used as given). The pages name the
 * layer but not these steps; they are the ones just before the recurrence in
 * the published Gated DeltaNet (Yang, Kautz & Hatamizadeh, ICLR 2025): q and k
 * L2-normalised per head, the write strength a sigmoid and the decay the
 * exponential of a negative softplus of per-token projections.
 *   GDN_QK_L2NORM    q and k hold raw rows; each row x is used as
 *                    x / sqrt(sum(x^2) + 1e-6) (fp32 arithmetic)
 *   GDN_GATE_LOGITS  alpha holds a, beta holds b (fp32 logits); the kernels
 *                    use alpha = exp(-softplus(a)), beta = sigmoid(b), taking
 *                    log(alpha) = -softplus(a) directly for the decay
 * Any other bit: GDN_ERR_UNSUPPORTED.
 */
enum { GDN_QK_L2NORM = 1, GDN_GATE_LOGITS = 2 };

/*
 * gdn_prefill_chunked -- chunked prefill of B equal-length sequences.
 *
 *   q, k          [B, T, Hk, Dk]  dtype
 *   v             [B, T, Hv, Dv]  dtype
 *   alpha, beta   [B, T, Hv]      fp32   per-token decay and write strength
 *   initial_state [B, Hv, Dv, Dk] fp32   S_0 per (sequence, value head);
 *                                        NULL means a zero state
 *   out           [B, T, Hv, Dv]  dtype  o_t (fp32 -> bf16 rounds to nearest even)
 *   final_state   [B, Hv, Dv, Dk] fp32   S_T; NULL means not written;
 *                                        may equal initial_state
 *   prefix_states [B, floor(T / L), Hv, Dv, Dk] fp32, or NULL: the state
 *                 after every block of L = 64 * prefix_interval tokens,
 *                 row i of sequence b holding S_{L (i + 1)} (whole blocks
 *                 only; the state after a partial last block is final_state).
 *                 These are the block-aligned prefix states of "PHBA:
 *                 Prefix-State Hybrid Block Attention" (Abstract, Figure 1),
 *                 formed by the gated recurrence at block boundaries, and the
 *                 states a prefix cache keeps. prefix_interval >= 1 when
 *                 prefix_states is set (ignored otherwise); must not overlap
 *                 any other argument.
 *
 * Sizes: B >= 1, T >= 0, Hk >= 1, Hv a multiple of Hk, Dk == Dv in {64, 128}.
 * T == 0 writes the initial state (or zeros) to final_state.
 * The sequence is processed in chunks of 64 tokens; the result equals the
 * token recurrence up to rounding (the chunked form is an exact rewrite).
 *
 * workspace: optional device scratch of workspace_bytes bytes (16-byte
 * aligned, disjoint from every other argument, contents ignored and
 * overwritten; the caller keeps ownership). Its first 256 bytes hold a status
 * word (see "Debug checks" above). When it holds at least
 * gdn_prefill_workspace_size() bytes the call may run in two passes: the
 * state-independent per-chunk factors of all chunks first, then the
 * sequential state chain. NULL (or too small) selects the single-pass
 * kernel. Both give the same result up to rounding. With few (sequence,
 * value head) chains, bf16 and no prefix states, a workspace of the size
 * query's answer also allows the segmented arrangement: each sequence is
 * split into segments run in parallel from zero and from the identity
 * state, joined by a scan of the segment maps and an output correction
 * (same result up to rounding).
 */
gdn_status_t gdn_prefill_chunked(const void *q, const void *k, const void *v,
                                 const float *alpha, const float *beta,
                                 const float *initial_state, void *out,
                                 float *final_state, float *prefix_states,
                                 int32_t prefix_interval, int32_t B, int64_t T,
                                 int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                 gdn_dtype_t dtype, float scale, uint32_t flags,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * gdn_prefill_chunked_noalloc -- gdn_prefill_chunked for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments and results as
 * gdn_prefill_chunked without the workspace pair: the call uses the
 * library's own static device scratch of 64 MiB per device (allocated when
 * the library's code is loaded on that device, held until the process ends)
 * as the workspace that gdn_prefill_workspace_size() names, and calls no
 * allocating routine. Shapes that need more scratch than 64 MiB are
 * rejected with GDN_ERR_UNSUPPORTED and no side effects (the scratch covers,
 * for example, one 4,096-token sequence at 16 q/k and 48 value heads of
 * dimension 128). Every call on a device shares that device's scratch, which
 * keeps the last call's contents: calls that may overlap in time on one
 * device (different streams, or threads) race and must be serialised by the
 * caller.
 */
gdn_status_t gdn_prefill_chunked_noalloc(const void *q, const void *k, const void *v,
                                         const float *alpha, const float *beta,
                                         const float *initial_state, void *out,
                                         float *final_state, float *prefix_states,
                                         int32_t prefix_interval, int32_t B, int64_t T,
                                         int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                                         gdn_dtype_t dtype, float scale, uint32_t flags,
                                         hipStream_t stream);

/*
 * gdn_decode_step -- one new token per sequence, state updated in place.
 *
 *   q, k         [B, Hk, Dk]     dtype
 *   v            [B, Hv, Dv]     dtype
 *   alpha, beta  [B, Hv]         fp32
 *   state        [B, Hv, Dv, Dk] fp32   read as S_{t-1}, overwritten with S_t
 *   out          [B, Hv, Dv]     dtype  o_t = scale * S_t q_t
 *
 * Sizes: B >= 1, Hk >= 1, Hv a multiple of Hk, Dk == Dv in {64, 128}.
 * This is the fixed-cost step the pages point to when they note that decode
 * speed stays flat as the context grows ("The economics of hybrid
 * attention", section "Where the constraint moved").
 */
gdn_status_t gdn_decode_step(const void *q, const void *k, const void *v,
                             const float *alpha, const float *beta, float *state,
                             void *out, int32_t B, int32_t Hk, int32_t Hv,
                             int32_t Dk, int32_t Dv, gdn_dtype_t dtype,
                             float scale, uint32_t flags, hipStream_t stream);

/*
 * gdn_decode_multi -- K new tokens per sequence against a pool of state
 * slots, for checking several drafted tokens in one call. "The economics of
 * hybrid attention" names the model's multi-token prediction head (section
 * "The stack, verified") and the speculation head's draft buffers served at
 * two slots (section "Where the constraint moved"); this call is the mixer's
 * side of that: the K tokens of each sequence run in order on one state that
 * crosses HBM once per call instead of once per token.
 *
 *   q, k         [B, K, Hk, Dk]      dtype
 *   v            [B, K, Hv, Dv]      dtype
 *   alpha, beta  [B, K, Hv]          fp32
 *   state_pool   [num_slots, Hv, Dv, Dk] fp32, DEVICE memory
 *   src_slot     [B] int32, DEVICE memory: sequence b starts from the state
 *                in slot src_slot[b]; a negative value means a zero state
 *   dst_slot     [B] int32, DEVICE memory: S_K of sequence b is written to
 *                slot dst_slot[b]; a negative value means it is not written
 *   out          [B, K, Hv, Dv]      dtype  o_t = scale * S_t q_t
 *   step_states  [B, K, Hv, Dv, Dk]  fp32 or NULL: S_t after each token t
 *                (for rolling back to any accepted prefix); NULL skips them
 *
 * Sizes: B >= 1, K >= 0, num_slots >= 1, Hk >= 1, Hv a multiple of Hk,
 * Dk == Dv in {64, 128}. K == 0 copies slot src_slot[b] (or zeros) to slot
 * dst_slot[b]. A token with alpha = 1 and beta = 0 leaves the state unchanged,
 * so a batch with fewer real tokens in some sequences can be padded with such
 * tokens.
 *
 * The slot indices are read on the device. An index >= num_slots is not
 * an error the call can return: that sequence touches no slot and its
 * outputs (and step states) are set to NaN. The caller guarantees that the
 * non-negative dst_slot values are distinct and that no sequence's dst slot
 * is another sequence's src slot (src_slot[b] == dst_slot[b] updates in
 * place); otherwise workgroups race and the result is unspecified. Slots not
 * named in dst_slot are left untouched. state_pool, out, step_states and the
 * slot arrays must not overlap each other or the inputs (GDN_ERR_ALIAS).
 */
gdn_status_t gdn_decode_multi(const void *q, const void *k, const void *v,
                              const float *alpha, const float *beta,
                              float *state_pool, int32_t num_slots,
                              const int32_t *src_slot, const int32_t *dst_slot,
                              void *out, float *step_states, int32_t B, int32_t K,
                              int32_t Hk, int32_t Hv, int32_t Dk, int32_t Dv,
                              gdn_dtype_t dtype, float scale, uint32_t flags,
                              hipStream_t stream);

/*
 * gdn_varlen_prefill -- chunked prefill of N packed sequences.
 *
 *   q, k          [total_T, Hk, Dk] dtype
 *   v, out        [total_T, Hv, Dv] dtype
 *   alpha, beta   [total_T, Hv]     fp32
 *   cu_seqlens    [N + 1] int32, DEVICE memory: sequence n spans tokens
 *                 cu_seqlens[n] .. cu_seqlens[n+1]-1; cu_seqlens[0] = 0,
 *                 non-decreasing, cu_seqlens[N] = total_T. Its contents are
 *                 checked only under GDN_DEBUG=1. Otherwise the kernels clamp
 *                 each sequence's start and end into [0, total_T] (end >=
 *                 start), so malformed offsets give meaningless results but
 *                 no access outside the caller's buffers.
 *   initial_state [N, Hv, Dv, Dk] fp32 or NULL (zero states)
 *   final_state   [N, Hv, Dv, Dk] fp32 or NULL; may equal initial_state
 *   prefix_states [floor(total_T / L) + N, Hv, Dv, Dk] fp32 or NULL, with
 *                 L = 64 * prefix_interval: as for gdn_prefill_chunked, the
 *                 state after each whole block of L tokens of a sequence;
 *                 block i of sequence n goes to row
 *                 floor(cu_seqlens[n] / L) + n + i (rows that no block maps
 *                 to are left untouched)
 *
 * Sizes: N >= 1, 0 <= total_T < 2^31, Hv a multiple of Hk, Dk == Dv in
 * {64, 128}. Chunks restart at every sequence boundary. workspace: as for
 * gdn_prefill_chunked.
 */
gdn_status_t gdn_varlen_prefill(const void *q, const void *k, const void *v,
                                const float *alpha, const float *beta,
                                const int32_t *cu_seqlens, int32_t N,
                                int64_t total_T, const float *initial_state,
                                void *out, float *final_state,
                                float *prefix_states, int32_t prefix_interval,
                                int32_t Hk,
                                int32_t Hv, int32_t Dk, int32_t Dv,
                                gdn_dtype_t dtype, float scale, uint32_t flags,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * gdn_prefill_workspace_size -- bytes of workspace the prefill calls can use.
 *
 *   packed = 0: gdn_prefill_chunked with num_seqs = B and tokens = T;
 *   packed = 1: gdn_varlen_prefill with num_seqs = N and tokens = total_T.
 *
 * Returns 0 when the library would not use a workspace for this shape on the
 * current device (enough (sequence, value head) pairs to fill it in one
 * pass), when an argument is invalid, or when no device is available. The
 * size is 256 bytes (the status word) plus 17,152 bytes (bf16) or 33,536
 * bytes (fp32) per (64-token chunk, value head): B * ceil(T/64) chunks, or
 * ceil(total_T/64) + N for packed batches. It is larger where
 * gdn_prefill_chunked would run segmented (the segment end states, maps,
 * start states and the identity-start outputs).
 */
size_t gdn_prefill_workspace_size(int32_t num_seqs, int64_t tokens, int32_t Hk,
                                  int32_t Hv, int32_t Dk, int32_t Dv,
                                  gdn_dtype_t dtype, int32_t packed);

/* Static description of a status; for GDN_ERR_HIP, the calling thread's
 * last HIP error detail. The pointer stays valid until the thread's next
 * call into the library. */
const char *gdn_status_string(gdn_status_t s);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
