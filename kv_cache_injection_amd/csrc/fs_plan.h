// Device helpers that write an inject plan (the segment of a request's
// selected facts laid end to end from its start position, validated, and
// mapped token by token to an arena row and a cache slot).  Shared by the
// plan kernel and by the top-k kernel that plans as it selects.  Not part of
// the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fs.h"
#include "fs_internal.h"

namespace fsp {

// largest j < nf with off[j] <= t (off is non-decreasing, off[0] = 0)
__device__ __forceinline__ int find_fact(const int32_t* off, int nf, int t) {
    int lo = 0, hi = nf - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Checks of a segment of L tokens laid from position s: the position range
// fits int32, the block-table row has an entry for every block it touches
// (first = s >> lb .. last = (s + L - 1) >> lb, all below max_blocks), and
// each such entry names a block in [0, num_blocks).  Called by n threads with
// index i (a wave or a block) that split the entries; every caller gets the
// position and row-length bits, and the entry bits of the entries it read, so
// the caller ORs the results.  entry(j) returns bt[j] for first <= j <= last.
template <class Entry>
__device__ __forceinline__ uint32_t check_segment(int s, int L, int max_blocks, int num_blocks, int lb, int i,
                                                  int n, Entry entry) {
    if (s < 0 || int64_t(s) + L > int64_t(INT32_MAX)) return FS_ERR_START_POS;
    if (L == 0) return 0;
    const int first = s >> lb;
    const int last = (s + L - 1) >> lb;
    if (last >= max_blocks) return FS_ERR_BLOCK_SHORT;
    uint32_t bits = 0;
    // four entries per thread in flight at a time (indices clamped to the
    // range, so the loads need no branch and no wait between them)
    for (int j0 = first + i; j0 <= last; j0 += 4 * n) {
        int e[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = entry(min(j0 + n * q, last));
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (j0 + n * q <= last && (e[q] < 0 || e[q] >= num_blocks)) bits |= FS_ERR_BLOCK_ID;
    }
    return bits;
}

// The token map of an accepted segment: token t (0 <= t < L) lies in fact
// j = find_fact(off, nf, t), at arena row row0[j] + t - off[j], and goes to
// cache slot entry(p >> lb) * 2^lb + p % 2^lb for p = s + t.  n threads with
// index i split the tokens.
template <class Entry>
__device__ __forceinline__ void write_tokens(PlanTok* tok, const int32_t* off, const int64_t* row0, int nf, int L,
                                             int s, int lb, int i, int n, Entry entry) {
    const int mask = (1 << lb) - 1;
    for (int t = i; t < L; t += n) {
        const int j = find_fact(off, nf, t);
        const int p = s + t;
        tok[t] = PlanTok{row0[j] + (t - off[j]), (int64_t(entry(p >> lb)) << lb) | (p & mask)};
    }
}

__device__ __forceinline__ void write_header(PlanHeader* hdr, uint64_t key, uint32_t tag, int batch, int k,
                                             int seg_tokens, int num_blocks) {
    PlanHeader h{};
    h.key = key;
    h.magic = kPlanMagic;
    h.tag = tag;
    h.batch = batch;
    h.k = k;
    h.seg_tokens = seg_tokens;
    h.num_blocks = num_blocks;
    *hdr = h;
}

}  // namespace fsp
