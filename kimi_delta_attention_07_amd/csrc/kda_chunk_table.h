// Chunk table lookup shared by the chunk-path kernels (forward and backward).
#pragma once

#include "kda_internal.h"

namespace kda {

// A chunk record as the kernels may use it: the table is built on the device
// from cu_seqlens_dev while grids are sized from the host copy; should the two
// ever disagree, out-of-range entries become empty chunks instead of stray
// memory accesses.
__device__ __forceinline__ ChunkInfo load_chunk(const ChunkParams &p, int cid) {
    if (p.plan_in_args) {
        // the sequence holding chunk cid: the last n with plan_off[n] <= cid
        // (empty sequences share their offset with the next one)
        int lo = 0, hi = p.n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.plan_off[mid] <= cid) lo = mid;
            else hi = mid - 1;
        }
        ChunkInfo ci;
        ci.seq = lo;
        ci.first = cid == p.plan_off[lo];
        ci.start = p.plan_cu[lo] + kChunk * (cid - p.plan_off[lo]);
        ci.len = max(0, min(kChunk, p.plan_cu[lo + 1] - ci.start));
        return ci;
    }
    ChunkInfo ci = p.chunk_info[cid];
    ci.start = __builtin_amdgcn_readfirstlane(ci.start);
    ci.len = __builtin_amdgcn_readfirstlane(ci.len);
    ci.seq = __builtin_amdgcn_readfirstlane(ci.seq);
    ci.first = __builtin_amdgcn_readfirstlane(ci.first);
    if (ci.start < 0 || ci.len < 0 || ci.len > kChunk || ci.start > p.T - ci.len || ci.seq < 0 ||
        ci.seq >= p.n_seqs) {
        ci.start = 0;
        ci.len = 0;
        ci.seq = 0;
        ci.first = 0;
    }
    return ci;
}

}  // namespace kda
