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
};

struct DecodeParams {
    const void *q, *k, *v;
    const float *alpha, *beta;
    float *state;
    void *out;
    int32_t B, Hk, Hv;
    float scale;
};

// dtype: 0 = fp32, 1 = bf16. D: 64 or 128. Returns a hipError_t.
hipError_t launch_prefill(const PrefillParams &p, int dtype, int D, int num_cus,
                          hipStream_t stream);
hipError_t launch_decode(const DecodeParams &p, int dtype, int D, hipStream_t stream);

}  // namespace gdn
