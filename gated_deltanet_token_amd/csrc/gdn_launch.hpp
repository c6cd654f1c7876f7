// gdn_launch.hpp -- host-side launchers of the kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// One chunked-prefill launch. Dense batches pass cu_seqlens == nullptr and
// seq_len = T; packed batches pass the device offsets and seq_len = 0.
struct PrefillParams {
    const void *q, *k, *v;
    const float *alpha, *beta, *s0;
    void *out;
    float *s_final;
    const int32_t *cu_seqlens;
    int64_t seq_len;
    int32_t nseq, Hk, Hv;
    float scale;
    float *prefix;         // block-aligned prefix states, or nullptr
    int32_t prefix_every;  // block length in chunks (>= 1 when prefix is set)
    uint32_t flags;        // input preparation (kQkL2Norm | kGateLogits)
    int64_t v_stride;      // elements between consecutive tokens of v (Hv * Dv; 0: one row
                           // serves every token)
    bool s0_identity;      // initial state I (Dv == Dk) instead of s0 / zeros
    bool records_ready;    // two-pass: the workspace already holds this batch's per-chunk
                           // factors (they depend on q, k, alpha, beta only)
    int64_t chunk0;        // two-pass, one dense sequence: first chunk of this launch
    int64_t chunk_end;     // one past its last (0: to the end of the sequence)
    // Two-pass on the double-buffered chain only: with dual set, chains
    // nseq .. 2 nseq - 1 run sequence n - nseq a second time, from the
    // identity state with v = v2 (token stride 0), writing out2 and s_final2.
    bool dual;
    const void *v2;
    void *out2;
    float *s_final2;
    int64_t total_tokens;  // packed batches: tokens in the batch (offsets are clamped to it)
    int *status;           // the workspace's status word (nullptr without a workspace)
};

// The prefill workspace starts with a status word (padded to 256 bytes): a
// kernel whose bounded wait for another wave of its workgroup runs out ORs a
// nonzero code into it. The rest of the workspace follows.
constexpr size_t kWsStatusBytes = 256;
constexpr int kStatusWaitBound = 1;

// Input preparation flags (the ABI's GDN_QK_L2NORM, GDN_GATE_LOGITS).
constexpr uint32_t kQkL2Norm = 1, kGateLogits = 2;
constexpr float kL2Eps = 1e-6f;

struct DecodeParams {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *state;
    void *out;
    int32_t B, Hk, Hv;
    float scale;
    uint32_t flags;
};

// Several tokens per sequence; states live in a pool of slots.
struct DecodeMultiParams {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *pool;
    const int32_t *src_slot, *dst_slot;
    void *out;
    float *steps;  // per-token states, or nullptr
    int32_t B, K, Hk, Hv, num_slots;
    float scale;
    uint32_t flags;
};

// dtype: 0 = fp32, 1 = bf16. D: 64 or 128. Returns a hipError_t. `ws` is
// the caller's whole workspace (status word first). With at least
// kWsStatusBytes + prefill_ws_bytes(nslots, ...) bytes (and when
// prefill_wants_workspace agrees) the two-pass path runs; otherwise the
// fused kernel.
hipError_t launch_prefill(const PrefillParams &p, int dtype, int D, int num_cus, void *ws,
                          size_t ws_bytes, int64_t nslots, hipStream_t stream);
// Chunk records the two-pass workspace holds: B * ceil(T/64) for dense
// batches, ceil(total/64) + N for packed ones.
int64_t prefill_ws_slots(int64_t nseq, int64_t total_tokens, int64_t seq_len, bool packed);
size_t prefill_ws_bytes(int64_t slots, int Hv, int dtype);
bool prefill_wants_workspace(int64_t chains, int num_cus);
// Workspace bytes of the segmented prefill (dense bf16 batches with few
// chains), or 0 when it does not apply to these shapes.
size_t prefill_seg_ws_bytes(int64_t nseq, int64_t T, int Hv, int D, int dtype, int num_cus);

hipError_t launch_segment_setup(int32_t *cu, int32_t B, int32_t P, int64_t T, int64_t L,
                                __bf16 *zero_v, int32_t nzero, hipStream_t stream);
hipError_t launch_segment_scan(const float *s0, const float *n_end, const float *m_end,
                               float *s_start, float *s_final, int32_t B, int32_t P, int32_t Hv,
                               int D, hipStream_t stream);
hipError_t launch_segment_correct(__bf16 *out, const __bf16 *o_id, const float *s_start,
                                  const int32_t *cu, int32_t B, int32_t P, int32_t Hv,
                                  int64_t seg_len, int32_t first_seg, int D, hipStream_t stream);
// The two-pass chain with one wave per SIMD (gdn_chain4.hip): bf16, D = 128,
// four value-column slices per head, plain or identity-free calls.
// Single-pass prefill with one workgroup per (sequence, value head) chain and
// two workgroups per CU (gdn_fused2.hip): bf16, head dimension 128.
bool fused2_supported(const PrefillParams &p, int dtype, int D);
hipError_t launch_fused2(const PrefillParams &p, hipStream_t stream);
bool chain4_supported(const PrefillParams &p, int D, int nsplit);
hipError_t launch_chain4(const PrefillParams &p, const unsigned char *ws, int64_t nchain,
                         hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int dtype, int D, hipStream_t stream);
hipError_t launch_decode_multi(const DecodeMultiParams &p, int dtype, int D, hipStream_t stream);

}  // namespace gdn
