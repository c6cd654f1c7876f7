// gdn_seq.hpp -- per-workgroup bookkeeping shared by the prefill kernels:
// sequence bounds, workspace slots, the XCD-aware workgroup order and the
// LDS-DMA copy.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_chunk.hpp"
#include "gdn_launch.hpp"

namespace gdn {

// Packed offsets are clamped into [0, total_tokens] with end >= start, so
// malformed cu_seqlens cannot address memory outside the batch (the results
// are then meaningless, but no access leaves the caller's buffers).
__device__ __forceinline__ void seq_bounds(const PrefillParams &p, int n, int64_t &tok0,
                                           int64_t &len) {
    if (p.cu_seqlens) {
        const int64_t tot = p.total_tokens;
        int64_t a = p.cu_seqlens[n], b = p.cu_seqlens[n + 1];
        a = a < 0 ? 0 : a > tot ? tot : a;
        b = b < a ? a : b > tot ? tot : b;
        tok0 = a;
        len = b - a;
    } else {
        tok0 = (int64_t)n * p.seq_len;
        len = p.seq_len;
    }
}

// Workspace slot of chunk 0 of sequence n. Dense batches: n * ceil(T/64).
// Packed batches: floor(cu[n] / 64) + n, which is injective over all
// (sequence, chunk) pairs and below ceil(total/64) + N.
__device__ __forceinline__ int64_t packed_start(const PrefillParams &p, int n) {
    const int64_t a = p.cu_seqlens[n];
    return a < 0 ? 0 : a > p.total_tokens ? p.total_tokens : a;
}

__device__ __forceinline__ int64_t slot_base(const PrefillParams &p, int n) {
    if (p.cu_seqlens) return (packed_start(p, n) >> 6) + n;
    return (int64_t)n * ((p.seq_len + kC - 1) / kC);
}

// Prefix states: the state after every block of 64 * prefix_every tokens of
// a sequence (whole blocks only). Block i of sequence n goes to row
//   dense : n * floor(T / blk) + i
//   packed: floor(cu[n] / blk) + n + i   (injective, below floor(total/blk) + N)
// The divisions run once per workgroup; per chunk the check is one compare
// (this sits on the sequential path of the chain).
struct PrefixRows {
    int64_t next;  // chunk after which the next state is due; -1: none left
    int64_t row;   // its row
    int64_t left;  // states still due
    __device__ __forceinline__ PrefixRows(const PrefillParams &p, int n, int64_t len) {
        const int64_t every = p.prefix ? p.prefix_every : 1, blk = every * kC;
        left = p.prefix ? len / blk : 0;
        next = left > 0 ? every - 1 : -1;
        row = p.cu_seqlens ? packed_start(p, n) / blk + n : (int64_t)n * (p.seq_len / blk);
    }
    // Row for the state after chunk c, or -1; advances when one is due.
    __device__ __forceinline__ int64_t take(const PrefillParams &p, int64_t c) {
        if (c != next) return -1;
        const int64_t r = row++;
        next = --left > 0 ? next + p.prefix_every : -1;
        return r;
    }
};

// Logical workgroup id: workgroups are dispatched to the 8 XCDs round-robin;
// give each XCD a contiguous range of logical ids so that workgroups sharing
// a q/k head (and thus K, Q) share that XCD's L2.
// A select, not a branch: the compiler then loads the kernel arguments in
// one batch instead of waiting for remap_xcd before reading the grid size.
__device__ __forceinline__ int logical_wg(int remap_xcd) {
    const int wg = blockIdx.x;
    const int remapped = (wg & 7) * (int)(gridDim.x >> 3) + (wg >> 3);
    return remap_xcd ? remapped : wg;
}

// LDS-DMA load of 16 bytes per lane (global -> LDS without registers): lane l
// writes lds + 16 l, so a wave fills one contiguous KiB.
__device__ __forceinline__ void dma16(const unsigned char *src, unsigned char *lds) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint32_t *>(src), lds, 16, 0, 0);
}

}  // namespace gdn
