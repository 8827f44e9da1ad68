// GPU-resident retrieval: embedding scores and top-k selection.
//
// InferScale keeps the retrieval index and the KV store on the GPU and picks
// the k most relevant facts per request (gist.science summary,
// "Contributions Clés" and "Problématique").  Here the similarity is the
// inner product of fp32 embeddings: each fp32*fp32 product is exact in fp64
// and the sum is accumulated in fp64, so two facts with identical embedding
// rows get bit-identical scores and the tie is settled by the lower fact id.
//
// score kernel   grid (row tiles, batch), 256 threads = 4 waves, 2 rows per
//                wave; each lane owns a fixed set of columns (float4 c, c+64,
//                ...), accumulates them in order, then a fixed butterfly
//                reduces the wave.  The reduction order depends only on the
//                column, never on the row, which is what makes equal rows tie.
//                Consecutive requests of one user (up to 8) are scored by one
//                block, which reads its rows once for all their queries: a
//                batch of one user's requests scans the table once, not once
//                per request.
// top-k kernel   one block per request: 256 threads when no request of the
//                launch has more than 2,048 scores (a small block starts
//                sooner beside a running inject), 1,024 above.  Users above
//                65,536 facts are selected in two phases: the top k of every
//                16,384-score chunk (one block each), then the top k of those
//                candidates, which is exact.  First try: the min and
//                max of the request's scores define 2048 equal-width value
//                bins (the bin is a monotone function of the score, so equal
//                scores share a bin); an LDS histogram and a block suffix scan
//                find the bin that holds the k-th best score, every score in
//                that bin or above becomes a candidate, and each candidate's
//                rank is the number of candidates that beat it on
//                (score desc, index asc).  That costs a few passes over the
//                scores whatever k is.  When the threshold bin holds too many
//                scores (heavy ties, clustered values) or a score is not
//                finite, the block falls back to an exact MSB-first radix
//                select on order-preserving 64-bit keys (8-bit digits, LDS
//                histogram; equal full keys keep the lowest indices through a
//                block-wide ordered scan) and a bitonic sort of the winners.
//                The same block sums the winners' lengths (the segment
//                length).

#include <hip/hip_runtime.h>

#include "fs_internal.h"
#include "fs_plan.h"

namespace {

constexpr int kScoreWaves = 4;
constexpr int kScoreRowsPerWave = 2;
constexpr int kScoreRowsPerBlock = kScoreWaves * kScoreRowsPerWave;
constexpr int kScoreGroup = 8;       // queries of one user scored per block
constexpr int kScoreChunks = 4;      // float4 chunks of a row a lane loads at once (E up to 1024)
constexpr int kTopkSmallN = 2048;     // up to this many scores a 256-thread block selects
constexpr int kBins = 2048;          // value bins of the threshold search
constexpr int kCandMax = 2048;       // largest candidate set ranked directly

__device__ __forceinline__ uint64_t order_key(double x) {
    uint64_t u = (x == 0.0) ? 0ull : static_cast<uint64_t>(__double_as_longlong(x));
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_value(uint64_t key) {
    uint64_t u = (key >> 63) ? (key & 0x7FFFFFFFFFFFFFFFull) : ~key;
    return __longlong_as_double(static_cast<long long>(u));
}

__device__ __forceinline__ bool better(uint64_t ka, int ia, uint64_t kb, int ib) {
    return ka > kb || (ka == kb && ia < ib);
}

// Bin of a score: (x - lo) * scale rounds monotonically, so x <= y implies
// bin(x) <= bin(y).  One definition serves both passes that need it.
__device__ __forceinline__ int value_bin(double x, double lo, double scale) {
    const int bin = static_cast<int>((x - lo) * scale);
    return bin < kBins - 1 ? bin : kBins - 1;
}

// The value of lane (lane ^ m) for m a power of two below 64, without an
// LDS round trip where the lane pattern allows: m = 1 and 2 by DPP quad
// permutes, 4, 8 and 16 by swizzles within 32 lanes, 32 by a bpermute.
// Folds to one instruction when m is a constant.
__device__ __forceinline__ int xor_lane(int v, int m) {
    switch (m) {
        case 1: return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
        case 2: return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
        case 4: return __builtin_amdgcn_ds_swizzle(v, 0x101F);
        case 8: return __builtin_amdgcn_ds_swizzle(v, 0x201F);
        case 16: return __builtin_amdgcn_ds_swizzle(v, 0x401F);
        default: return __shfl_xor(v, m, 64);
    }
}
__device__ __forceinline__ uint64_t xor_lane(uint64_t v, int m) {
    const int lo = xor_lane(static_cast<int>(static_cast<uint32_t>(v)), m);
    const int hi = xor_lane(static_cast<int>(v >> 32), m);
    return (uint64_t(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
__device__ __forceinline__ double xor_lane(double v, int m) {
    return __longlong_as_double(static_cast<long long>(xor_lane(static_cast<uint64_t>(__double_as_longlong(v)), m)));
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += xor_lane(v, m);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane i gets v_0 + ... +
// v_i), all lanes active: DPP shifts within each row of 16 lanes, then each
// row's running total carried into the following rows by the row broadcasts
// (no LDS round trip).
__device__ __forceinline__ int wave_incl_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2 and 3
    return v;
}

struct ScoreArgs {
    const float4* emb;        // [F][E/4]
    int32_t e4;               // E/4
    const int64_t* user_begin;
    const int32_t* user_count;  // live facts per user, or null: user_begin[u + 1] ends the user
    int32_t num_users;
    const int32_t* user;
    const float4* query;      // [B][E/4]
    int32_t batch;
    double* scores;           // [B][stride]
    int32_t stride;
};

__device__ __forceinline__ void fma4(double& acc, const float4& e, const float4& q) {
    acc = fma(double(e.x), double(q.x), acc);
    acc = fma(double(e.y), double(q.y), acc);
    acc = fma(double(e.z), double(q.z), acc);
    acc = fma(double(e.w), double(q.w), acc);
}

// Block (row tile, request b).  Requests of one user that follow each other
// (within an aligned group of kGroup) are scored together by the block
// of the first of them: its rows are read once for all their queries.  The
// other blocks of the run exit at once.  Every score still accumulates the
// same products in the same order, so it does not depend on the grouping.
// kGroup = 1 (launches of one request) loads all of its two rows' chunks
// before the first product, so the rows arrive in one round trip; kGroup =
// kScoreGroup loops over the chunks two at a time, with fewer registers.
// Both accumulate the same products in the same order.
template <int kGroup>
__global__ __launch_bounds__(256) void fs_score_kernel(ScoreArgs a) {
    const int b = blockIdx.y;
    const int u = a.user[b];
    if (u < 0 || u >= a.num_users) return;
    if (b % kGroup != 0 && a.user[b - 1] == u) return;   // scored by the run's first block
    int nq = 1;
    while (nq < kGroup && (b + nq) % kGroup != 0 && b + nq < a.batch && a.user[b + nq] == u) ++nq;
    const int64_t base = a.user_begin[u];
    const int32_t n = a.user_count ? a.user_count[u] : static_cast<int32_t>(a.user_begin[u + 1] - base);
    const int32_t row0 = blockIdx.x * kScoreRowsPerBlock;
    if (row0 >= n) return;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int32_t r0 = row0 + wave * kScoreRowsPerWave;
    const bool v0 = r0 < n, v1 = r0 + 1 < n;
    const float4* e0 = a.emb + (base + (v0 ? r0 : 0)) * a.e4;
    const float4* e1 = a.emb + (base + (v1 ? r0 + 1 : 0)) * a.e4;
    // the queries are read straight from global memory (cached after the
    // first wave touches them), so their loads overlap the embedding loads
    const float4* qv = a.query + int64_t(b) * a.e4;
    double acc[kGroup][2];
#pragma unroll
    for (int q = 0; q < kGroup; ++q) acc[q][0] = acc[q][1] = 0.0;
    auto accumulate = [&](int c, const float4& ea, const float4& eb) {
#pragma unroll
        for (int q = 0; q < kGroup; ++q) {
            if (q < nq) {
                const float4 qq = qv[int64_t(q) * a.e4 + c];
                fma4(acc[q][0], ea, qq);
                fma4(acc[q][1], eb, qq);
            }
        }
    };
    if (kGroup == 1 && a.e4 <= 64 * kScoreChunks) {
        // every chunk of both rows is loaded before the first product; the
        // products then run in column order as in the loop below
        float4 ea[kScoreChunks], eb[kScoreChunks];
#pragma unroll
        for (int j = 0; j < kScoreChunks; ++j) {
            const int c = lane + 64 * j;
            ea[j] = c < a.e4 ? e0[c] : float4{};
            eb[j] = c < a.e4 ? e1[c] : float4{};
        }
#pragma unroll
        for (int j = 0; j < kScoreChunks; ++j)
            if (lane + 64 * j < a.e4) accumulate(lane + 64 * j, ea[j], eb[j]);
    } else {
#pragma unroll 2
        for (int c = lane; c < a.e4; c += 64) {
            const float4 ea = e0[c];
            const float4 eb = e1[c];
#pragma unroll
            for (int q = 0; q < kGroup; ++q) {
                if (q < nq) {
                    const float4 qq = qv[int64_t(q) * a.e4 + c];
                    fma4(acc[q][0], ea, qq);
                    fma4(acc[q][1], eb, qq);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < kGroup; ++q) {
        if (q < nq) {
            const double s0 = wave_sum(acc[q][0]);
            const double s1 = wave_sum(acc[q][1]);
            if (lane == 0) {
                double* out = a.scores + int64_t(b + q) * a.stride;
                if (v0) out[r0] = s0;
                if (v1) out[r0 + 1] = s1;
            }
        }
    }
}

// ---- approximate retrieval: scan of the probed inverted lists -------------

struct ListArgs {
    const float4* emb_sorted;  // [N_u][E/4] rows in list order
    int32_t e4;
    const int32_t* list_begin; // [nlist+1]
    const int32_t* members;    // [N_u] global fact ids
    const int32_t* chosen;     // [B][np_stride] probed lists, best first
    int32_t np_stride, nprobe;
    int32_t* offs;             // [B][np_stride + 1] first candidate of each probed list
    const float4* query;       // [B][E/4]
    double* cand_scores;       // [B][stride]
    int32_t* cand_ids;         // [B][stride]
    int32_t* counts;           // [B]
    int32_t stride;
};

// One wave per request: where each probed list's candidates start (probe
// order), and how many candidates there are.
__global__ __launch_bounds__(64) void fs_list_offsets_kernel(ListArgs a) {
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t* ch = a.chosen + int64_t(b) * a.np_stride;
    int32_t* off = a.offs + int64_t(b) * (a.np_stride + 1);
    int32_t carry = 0;
    for (int j0 = 0; j0 < a.nprobe; j0 += 64) {
        const int j = j0 + lane;
        int32_t len = 0;
        if (j < a.nprobe) {
            const int c = ch[j];
            len = a.list_begin[c + 1] - a.list_begin[c];
        }
        int32_t incl = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int32_t y = __shfl_up(incl, o, 64);
            if (lane >= o) incl += y;
        }
        if (j < a.nprobe) off[j] = carry + incl - len;
        carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
        off[a.nprobe] = carry;
        a.counts[b] = carry;
    }
}

// Block (row tile, probed list pi, request b): scores 8 rows of list
// chosen[b][pi] with the arithmetic of fs_score_kernel (same column
// ownership, fma order and butterfly), so a fact scores the same bits here as
// in the flat scan.  Candidates of request b are the probed lists in probe
// order.
__global__ __launch_bounds__(256) void fs_list_score_kernel(ListArgs a) {
    const int b = blockIdx.z;
    const int pi = blockIdx.y;
    const int c = a.chosen[int64_t(b) * a.np_stride + pi];
    const int32_t off = a.offs[int64_t(b) * (a.np_stride + 1) + pi];
    const int32_t beg = a.list_begin[c];
    const int32_t n = a.list_begin[c + 1] - beg;
    const int32_t row0 = blockIdx.x * kScoreRowsPerBlock;
    if (row0 >= n) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int32_t r0 = row0 + wave * kScoreRowsPerWave;
    const bool v0 = r0 < n, v1 = r0 + 1 < n;
    const float4* e0 = a.emb_sorted + int64_t(beg + (v0 ? r0 : 0)) * a.e4;
    const float4* e1 = a.emb_sorted + int64_t(beg + (v1 ? r0 + 1 : 0)) * a.e4;
    const float4* qv = a.query + int64_t(b) * a.e4;
    double acc0 = 0.0, acc1 = 0.0;
#pragma unroll 2
    for (int cc = lane; cc < a.e4; cc += 64) {
        const float4 ea = e0[cc];
        const float4 eb = e1[cc];
        const float4 qq = qv[cc];
        fma4(acc0, ea, qq);
        fma4(acc1, eb, qq);
    }
    const double s0 = wave_sum(acc0);
    const double s1 = wave_sum(acc1);
    if (lane == 0) {
        const int64_t o = int64_t(b) * a.stride + off + r0;
        if (v0) {
            a.cand_scores[o] = s0;
            a.cand_ids[o] = a.members[beg + r0];
        }
        if (v1) {
            a.cand_scores[o + 1] = s1;
            a.cand_ids[o + 1] = a.members[beg + r0 + 1];
        }
    }
}

struct TopkArgs {
    const double* scores;     // [B][stride]
    int32_t stride;
    const int64_t* user_begin;
    const int32_t* user_count;  // live facts per user, or null: user_begin[u + 1] ends the user
    int32_t num_users;
    const int32_t* user;
    const int32_t* fact_len;
    int32_t k;
    int32_t* ids;             // [B][k] or null when k == 0
    double* out_scores;       // [B][k] or null
    int32_t* num_tokens;      // [B] or null
    uint32_t* err;
    // candidate mode (approximate retrieval): request b has counts[b]
    // candidates, candidate i is fact idmap[b * stride + i]; ties go to the
    // lower fact id
    const int32_t* counts;
    const int32_t* idmap;
    // chunk mode (first phase of a large user's selection): block
    // (request b, chunk c) selects the top k of the user's scores
    // [c * chunk, (c + 1) * chunk) and writes them, by global fact id, to
    // ids / out_scores at row b * nchunks + c; the request's last chunk
    // writes the number of candidates to out_counts[b]
    int32_t chunk;
    int32_t nchunks;
    int32_t* out_counts;
    // planning (the final selection of fs_retrieve_plan; never in chunk
    // mode): the inject plan of the selected ids, as the plan kernel
    // composes it from them; plan.hdr is null when not planning
    PlanView plan;
    uint64_t plan_key;
    uint32_t plan_tag;
    int32_t batch, seg_tokens, num_blocks, max_blocks, log2_block;
    const int32_t* block_table;   // [batch][max_blocks]
    const int32_t* start_pos;     // [batch]
    const int64_t* fact_begin;
};

// A value every lane of the block shares, loaded through the scalar unit
// (the data is not written while the kernel runs): its wait does not hold
// back the vector loads issued around it.
template <class T>
__device__ __forceinline__ T scalar_load(const T* p) { return *(const __attribute__((address_space(4))) T*)p; }

// block-table entries of a planning request fetched when its selection
// starts (from the block its start position falls in)
constexpr int kPlanWin = 256;

__device__ __forceinline__ int wave_or_u(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, 64);
    return static_cast<int>(v);
}

// The planning tail of fs_retrieve_plan: request b's inject plan from its kk
// selected ids (base + cand_idx[j], rank order), with the segment, checks,
// error bits and token map the plan kernel derives from the same ids.  Every
// id is a live fact of the request's user by construction, so only a bad
// user, the start position and the block table can reject the request.
// known: the selection left each rank's segment offset and first arena row
// in off / row0 and the segment length in *s_len.  win_e is this thread's
// block-table entry win_first + tid (tid < kPlanWin), fetched at the start.
template <int kT>
__device__ void plan_selected(const TopkArgs& a, int b, int kk, int64_t base, const int32_t* cand_idx, bool known,
                              bool bad_user, int s0, int win_first, int win_e, int32_t* off, int64_t* row0,
                              int32_t* win, const uint64_t* win_bad, int* s_len, int* s_bits) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int nwin = max(0, min(kPlanWin, a.max_blocks - win_first));
    if (known) {
        // The selection laid the segment out (off, row0, *s_len) before its
        // last barrier, and the block-table window and its bad-entry bits
        // (win_bad, one bit per entry) are in LDS since the first one.  When
        // the segment's blocks all fall inside the window, every thread takes
        // the same decision from them, with no further barrier.
        const int L = *s_len;
        const int64_t last_pos = int64_t(s0) + L - 1;
        const int last_blk = static_cast<int>(last_pos >> a.log2_block);
        // (the start-position and empty cases take the general path below,
        // which reports them exactly as the plan kernel does)
        if (s0 >= 0 && L > 0 && int64_t(s0) + L <= int64_t(INT32_MAX) && last_blk - win_first < nwin) {
            // entries first .. last of the segment are window entries
            // 0 .. last_blk - win_first (the window starts at the first)
            const int hi = last_blk - win_first;
            uint32_t bits = bad_user ? FS_ERR_USER : 0u;
            if (last_blk >= a.max_blocks) {
                bits |= FS_ERR_BLOCK_SHORT;
            } else {
#pragma unroll
                for (int w = 0; w < kPlanWin / 64; ++w) {
                    uint64_t m = 64 * w <= hi ? win_bad[w] : 0ull;
                    if (hi - 64 * w < 63) m &= (2ull << max(hi - 64 * w, 0)) - 1ull;
                    if (m) bits |= FS_ERR_BLOCK_ID;
                }
            }
            if (tid == 0) {
                if (bits) atomicOr(a.err, bits);
                a.plan.req[b] = PlanReq{bits ? 0 : L, s0};
                if (b == 0) fsp::write_header(a.plan.hdr, a.plan_key, a.plan_tag, a.batch, a.k, a.seg_tokens, a.num_blocks);
            }
            if (bits) return;
            PlanTok* tok = a.plan.tok + int64_t(b) * a.seg_tokens;
            const int mask = (1 << a.log2_block) - 1;
            const int G = kk > 0 && kk < kT ? kT / kk : 1;
            const int sub = tid % G;
            for (int j = tid / G; j < kk; j += kT / G) {
                const int o = off[j];
                const int n = (j + 1 < kk ? off[j + 1] : L) - o;
                const int64_t r = row0[j];
#pragma unroll 4
                for (int t = sub; t < n; t += G) {
                    const int p = s0 + o + t;
                    tok[o + t] = PlanTok{r + t, (int64_t(win[(p >> a.log2_block) - win_first]) << a.log2_block) | (p & mask)};
                }
            }
            return;
        }
    }
    if (!known && tid < 64) {
        // one dependent round: the selected facts' lengths and first rows
        int carry = 0;
        for (int c0 = 0; c0 < kk; c0 += 64) {
            const int j = c0 + lane;
            const int64_t id = j < kk ? base + cand_idx[j] : 0;
            const int len = j < kk ? a.fact_len[id] : 0;
            const int64_t r0 = j < kk ? a.fact_begin[id] : 0;
            int incl = len;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o, 64);
                if (lane >= o) incl += y;
            }
            if (j < kk) {
                off[j] = carry + incl - len;
                row0[j] = r0;
            }
            carry += __shfl(incl, 63, 64);
        }
        if (tid == 0) *s_len = carry;
    }
    if (tid < kPlanWin) win[tid] = win_e;
    if (tid == 0) *s_bits = 0;
    __syncthreads();
    const int L = *s_len;
    const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
    // The block-table entries come from the window when all the segment's
    // blocks fall inside it (the usual case), else from the table.  The
    // choice is uniform and each path has one kind of load: a per-token
    // choice between two loads becomes one flat load of a selected pointer,
    // which waits on the vector-memory counter.
    const int64_t last_pos = int64_t(s0) + L - 1;
    const bool in_win = s0 >= 0 && L > 0 && last_pos <= int64_t(INT32_MAX) &&
                        (static_cast<int>(last_pos >> a.log2_block) - win_first) < nwin;
    auto from_win = [&](int j) { return win[j - win_first]; };
    auto from_table = [&](int j) { return bt[j]; };
    uint32_t bits = in_win ? fsp::check_segment(s0, L, a.max_blocks, a.num_blocks, a.log2_block, tid, kT, from_win)
                           : fsp::check_segment(s0, L, a.max_blocks, a.num_blocks, a.log2_block, tid, kT, from_table);
    if (bad_user) bits |= FS_ERR_USER;
    bits = wave_or_u(bits);
    if (lane == 0 && bits) atomicOr(s_bits, static_cast<int>(bits));
    __syncthreads();
    bits = static_cast<uint32_t>(*s_bits);
    if (tid == 0) {
        if (bits) atomicOr(a.err, bits);
        a.plan.req[b] = PlanReq{bits ? 0 : L, s0};
        if (b == 0) fsp::write_header(a.plan.hdr, a.plan_key, a.plan_tag, a.batch, a.k, a.seg_tokens, a.num_blocks);
    }
    if (bits) return;
    // the token map: G threads per fact, each over every G-th token of it
    // (no search for a token's fact; a thread's lookups are independent)
    PlanTok* tok = a.plan.tok + int64_t(b) * a.seg_tokens;
    const int mask = (1 << a.log2_block) - 1;
    const int G = kk > 0 && kk < kT ? kT / kk : 1;
    const int sub = tid % G;
    auto write_map = [&](auto entry) {
        for (int j = tid / G; j < kk; j += kT / G) {
            const int o = off[j];
            const int n = (j + 1 < kk ? off[j + 1] : L) - o;
            const int64_t r = row0[j];
#pragma unroll 4
            for (int t = sub; t < n; t += G) {
                const int p = s0 + o + t;
                tok[o + t] = PlanTok{r + t, (int64_t(entry(p >> a.log2_block)) << a.log2_block) | (p & mask)};
            }
        }
    };
    if (in_win) write_map(from_win);
    else write_map(from_table);
}

// kT threads: 256 for stores of up to kTopkSmallN scores per request (a
// small block starts sooner beside a running inject and syncs faster),
// 1024 above.
// kPlan: the launch plans (a.plan set); the plain selection is built
// without any of the planning code.
template <int kT, bool kPlan>
__global__ __launch_bounds__(kT) void fs_topk_kernel(TopkArgs a) {
    constexpr int kTopkThreads = kT;
    constexpr int kTopkWaves = kT / 64;
    // scores per thread kept in registers: all of a small block's requests
    // (every kept slot costs unrolled code and registers, so no more), the
    // first 4096 of a large block's
    constexpr int kKeep = (kT == 256 ? kTopkSmallN : 4096) / kT;
    __shared__ int hist[256];
    __shared__ uint64_t cand_key[fsi::kMaxK];
    __shared__ int32_t cand_idx[fsi::kMaxK];
    __shared__ int wave_cnt[kTopkThreads / 64];
    __shared__ uint64_t s_prefix, s_mask;
    __shared__ int s_rem, s_done, s_ncand, s_tokens;
    extern __shared__ uint64_t keys_lds[];

    const bool chunked = a.chunk > 0;
    const int b = chunked ? blockIdx.x / a.nchunks : blockIdx.x;
    const int cidx = chunked ? blockIdx.x - b * a.nchunks : 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int k = a.k;
    const bool mapped = a.counts != nullptr;
    // planning: the request's start position (and, in candidate mode, which
    // reads no user otherwise, its user) in the first round of loads
    const int s0 = kPlan ? scalar_load(a.start_pos + b) : 0;
    const int pu = kPlan && mapped ? scalar_load(a.user + b) : 0;
    const int u = mapped ? 0 : a.user[b];
    const bool bad_user = !mapped && (u < 0 || u >= a.num_users);
    const int64_t ubase = (mapped || bad_user) ? 0 : a.user_begin[u];
    const int32_t n_all = mapped ? a.counts[b]
                                 : (bad_user ? 0 : (a.user_count ? a.user_count[u]
                                                                : static_cast<int32_t>(a.user_begin[u + 1] - ubase)));
    const int32_t c0 = cidx * a.chunk;              // first score of this block's chunk
    // scores i = tid + j*blockDim.x: the first kKeep of each thread stay in
    // registers for the later passes (the rest, for large users, are
    // re-read).  Their address depends only on the request, so they are
    // loaded before anything else, beside the user -> range chain; entries
    // past the request's count (inside the scratch row) are loaded and never
    // used.
    const double* sc = a.scores + int64_t(b) * a.stride + c0;
    double xv[kKeep];
    {
        const int32_t in_row = a.stride - c0;
#pragma unroll
        for (int j = 0; j < kKeep; ++j) {
            const int i = tid + j * kTopkThreads;
            xv[j] = i < in_row ? sc[i] : 0.0;
        }
    }
    const int32_t n = chunked ? max(0, min(a.chunk, n_all - c0)) : n_all;
    const int64_t base = ubase + c0;
    const int kk = n < k ? n : k;
    if (chunked && tid == 0) {
        // the request's last non-empty chunk (or chunk 0 of an empty user)
        // reports how many candidates the chunks hold
        const int last = n_all > 0 ? (n_all - 1) / a.chunk : 0;
        if (cidx == last) a.out_counts[b] = n_all > 0 ? last * k + min(k, n_all - last * a.chunk) : 0;
    }
    const int32_t* imap = mapped ? a.idmap + int64_t(b) * a.stride : nullptr;
    // the id a candidate is ranked and reported by
    auto cand_id = [&](int i) -> int32_t { return mapped ? imap[i] : i; };

    // planning: the user's validity and the request's block-table window,
    // fetched now, beside the scores
    constexpr bool planning = kPlan;
    // candidates of the threshold bin (score key, id, fact length; first
    // arena row when planning, for the one-wave sort's at most 64)
    __shared__ uint64_t s_ck[kCandMax];
    __shared__ int32_t s_ci[kCandMax];
    __shared__ int32_t s_cl[kCandMax];
    __shared__ int64_t s_cr[64];
    __shared__ int32_t s_win[kPlanWin];
    __shared__ uint64_t s_winbad[kPlanWin / 64];   // entries outside [0, num_blocks), one bit each
    __shared__ int s_plen, s_pbits;
    // the plan's per-rank segment offsets and first rows reuse the candidate
    // keys and ids, which are dead once the ranks are known
    static_assert(sizeof(int32_t) * fsi::kMaxK <= sizeof(s_ci) && sizeof(int64_t) * fsi::kMaxK <= sizeof(s_ck),
                  "plan arrays fit the candidate arrays");
    int32_t* const s_poff = s_ci;
    int64_t* const s_prow = reinterpret_cast<int64_t*>(s_ck);
    int win_first = 0, win_e = 0;
    bool plan_bad_user = false;
    if (planning) {
        win_first = s0 > 0 ? (s0 >> a.log2_block) : 0;
        const int j = win_first + tid;
        win_e = tid < kPlanWin && j < a.max_blocks ? a.block_table[int64_t(b) * a.max_blocks + j] : 0;
        plan_bad_user = mapped ? (pu < 0 || pu >= a.num_users) : bad_user;
    }

    if (__builtin_expect(bad_user, 0) && tid == 0 && cidx == 0) atomicOr(a.err, FS_ERR_USER);
    if (chunked && kk == 0) return;
    if (__builtin_expect(kk == 0, 0)) {
        for (int j = tid; j < k; j += blockDim.x) {
            a.ids[int64_t(b) * k + j] = -1;
            if (a.out_scores) a.out_scores[int64_t(b) * k + j] = -__builtin_huge_val();
        }
        if (a.num_tokens && tid == 0) a.num_tokens[b] = 0;
        if (planning)
            plan_selected<kT>(a, b, 0, base, cand_idx, false, plan_bad_user, s0, win_first, win_e, s_poff, s_prow,
                              s_win, s_winbad, &s_plen, &s_pbits);
        return;
    }

    bool tokens_known = false;           // the fast path sums the lengths itself
    bool plan_known = false;             // the fast path lays the plan's segment itself

    // ---- first try: threshold bin, then rank the candidates ---------------
    __shared__ int s_bin[kBins];
    __shared__ double s_wlo[kTopkWaves], s_whi[kTopkWaves];
    __shared__ int s_wbad[kTopkWaves], s_wsum[kTopkWaves];
    __shared__ int s_t, s_C, s_nc;
    __shared__ int s_wn[kTopkWaves];
    {
        // for plain requests, the kept scores' fact lengths, fetched once
        // the range is known: a candidate's length loaded only once it is
        // found costs a round trip per candidate a thread holds
        int32_t lv[kKeep];
        // and, when planning, their first arena rows
        int64_t rv[kKeep];
        const bool pre_len = !mapped && a.fact_len;
        const bool pre_row = pre_len && planning;
        const int tail0 = tid + kKeep * kTopkThreads;
        {
            // unpredicated, unbranched loads (the index clamped into the
            // user's range, n >= 1 here; with no lengths to fetch, a harmless
            // read of the request's first score instead): in straight-line
            // code the scores' wait below counts past these loads instead of
            // waiting for them too
            const int64_t last = base + n - 1;
            const int32_t* len_at = pre_len ? a.fact_len : reinterpret_cast<const int32_t*>(sc);
            const int64_t* row_at = pre_row ? a.fact_begin : reinterpret_cast<const int64_t*>(sc);
#pragma unroll
            for (int j = 0; j < kKeep; ++j) {
                const int64_t f = min(base + tid + j * kTopkThreads, last);
                lv[j] = len_at[pre_len ? f : 0];
                if (kPlan) rv[j] = row_at[pre_row ? f : 0];
                else rv[j] = 0;
            }
        }
        double lo = __builtin_huge_val(), hi = -__builtin_huge_val();
        int bad = 0;
        auto see = [&](double x) {
            if (!(fabs(x) < __builtin_huge_val())) bad = 1;     // NaN or infinite
            lo = fmin(lo, x);
            hi = fmax(hi, x);
        };
        // the kept scores by selects, not branches: in straight-line code
        // the wait for each score counts past the length loads issued after
        // it, instead of waiting for every load in flight
#pragma unroll
        for (int j = 0; j < kKeep; ++j) {
            const bool in = tid + j * kTopkThreads < n;
            const double x = xv[j];
            bad |= (in && !(fabs(x) < __builtin_huge_val())) ? 1 : 0;
            lo = fmin(lo, in ? x : __builtin_huge_val());
            hi = fmax(hi, in ? x : -__builtin_huge_val());
        }
        for (int i = tail0; i < n; i += kTopkThreads) see(sc[i]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            lo = fmin(lo, xor_lane(lo, m));
            hi = fmax(hi, xor_lane(hi, m));
            bad |= xor_lane(bad, m);
        }
        if (lane == 0) {
            s_wlo[wave] = lo;
            s_whi[wave] = hi;
            s_wbad[wave] = bad;
        }
        if (planning) {
            // the block-table window, loaded at the start, and which of its
            // entries name no cache block (entries past the table's row are
            // the plan's row-length check, not marked)
            if (tid < kPlanWin) s_win[tid] = win_e;
            const bool off_pool = tid < kPlanWin && win_first + tid < a.max_blocks && (win_e < 0 || win_e >= a.num_blocks);
            const uint64_t m = __builtin_amdgcn_ballot_w64(off_pool);
            if (lane == 0 && wave < kPlanWin / 64) s_winbad[wave] = m;
        }
        for (int i = tid; i < kBins; i += blockDim.x) s_bin[i] = 0;
        if (tid == 0) {
            s_nc = 0;
            s_tokens = 0;
        }
        __syncthreads();
        for (int w = 0; w < kTopkWaves; ++w) {
            lo = fmin(lo, s_wlo[w]);
            hi = fmax(hi, s_whi[w]);
            bad |= s_wbad[w];
        }
        const double range = hi - lo;
        const double scale = (kBins - 0.5) / range;
        if (__builtin_expect(!bad && range == 0.0 && !mapped, 0)) {
            // every score is equal: the lowest kk indices win, in order
            for (int j = tid; j < kk; j += blockDim.x) {
                cand_key[j] = order_key(lo);
                cand_idx[j] = j;
            }
            __syncthreads();
            goto outputs;
        }
        if (__builtin_expect(!bad && range < __builtin_huge_val() && scale < __builtin_huge_val(), 1)) {
#pragma unroll
            for (int j = 0; j < kKeep; ++j)
                if (tid + j * kTopkThreads < n) atomicAdd(&s_bin[value_bin(xv[j], lo, scale)], 1);
            for (int i = tail0; i < n; i += kTopkThreads) atomicAdd(&s_bin[value_bin(sc[i], lo, scale)], 1);
            __syncthreads();
            // suffix counts from the top bin down: thread tid owns the kBPT
            // bins at descending positions kBPT*tid .. kBPT*tid + kBPT - 1
            constexpr int kBPT = kBins / kTopkThreads;
            int cb[kBPT];
            int local = 0;
#pragma unroll
            for (int j = 0; j < kBPT; ++j) {
                cb[j] = s_bin[kBins - 1 - (kBPT * tid + j)];
                local += cb[j];
            }
            const int incl = wave_incl_sum(local);
            if (lane == 63) s_wsum[wave] = incl;
            __syncthreads();
            int before = incl - local;
            for (int w = 0; w < wave; ++w) before += s_wsum[w];
            // the k-th best score lies in the bin where the count of scores
            // above it first reaches kk
            {
                int cum = before;
#pragma unroll
                for (int j = 0; j < kBPT; ++j) {
                    if (cum < kk && kk <= cum + cb[j]) {
                        s_t = kBins - 1 - (kBPT * tid + j);
                        s_C = cum + cb[j];
                    }
                    cum += cb[j];
                }
            }
            __syncthreads();
            const int t = s_t, C = s_C;
            if (__builtin_expect(C <= kCandMax, 1)) {
                // len < 0: the length (and, planning, the first row) is loaded here
                auto put = [&](int slot, double x, int i, int32_t len, int64_t r0) {
                    const int32_t id = cand_id(i);
                    s_ck[slot] = order_key(x);
                    s_ci[slot] = id;
                    s_cl[slot] = len >= 0 ? len : (a.fact_len ? a.fact_len[base + id] : 0);
                    if (planning && slot < 64) s_cr[slot] = len >= 0 ? r0 : a.fact_begin[base + id];
                };
                if (__builtin_expect(C <= 64 && n <= kKeep * kTopkThreads, 1)) {
                    // few candidates, every score in registers: each wave
                    // counts its candidates by ballot, and after one barrier
                    // writes them at its offset in index order (no LDS
                    // atomics)
                    uint64_t cm[kKeep];
                    int wn = 0;
#pragma unroll
                    for (int j = 0; j < kKeep; ++j) {
                        cm[j] = __builtin_amdgcn_ballot_w64(tid + j * kTopkThreads < n &&
                                                            value_bin(xv[j], lo, scale) >= t);
                        wn += __popcll(cm[j]);
                    }
                    if (lane == 0) s_wn[wave] = wn;
                    __syncthreads();
                    int at = 0;
                    for (int w = 0; w < wave; ++w) at += s_wn[w];
                    if (__builtin_expect(pre_len && !mapped, 1)) {
                        // the usual request: ids are score indices and the
                        // lengths and rows are in registers, so each
                        // candidate is a few LDS writes (the general writer
                        // below carries the loads of the other cases, and its
                        // instructions, run for every kept slot, cost the
                        // phase a microsecond)
#pragma unroll
                        for (int j = 0; j < kKeep; ++j) {
                            if ((cm[j] >> lane) & 1ull) {
                                const int slot = at + __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(cm[j] >> 32),
                                                                                __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cm[j]), 0));
                                s_ck[slot] = order_key(xv[j]);
                                s_ci[slot] = tid + j * kTopkThreads;
                                s_cl[slot] = lv[j];
                                if (planning) s_cr[slot] = rv[j];   // slot < 64: at most 64 candidates
                            }
                            at += __popcll(cm[j]);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < kKeep; ++j) {
                            if ((cm[j] >> lane) & 1ull) {
                                const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(cm[j] >> 32),
                                                                            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cm[j]), 0));
                                put(at + below, xv[j], tid + j * kTopkThreads, pre_len ? lv[j] : -1, rv[j]);
                            }
                            at += __popcll(cm[j]);
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < kKeep; ++j)
                        if (tid + j * kTopkThreads < n && value_bin(xv[j], lo, scale) >= t)
                            put(atomicAdd(&s_nc, 1), xv[j], tid + j * kTopkThreads, pre_len ? lv[j] : -1, rv[j]);
                    for (int i = tail0; i < n; i += kTopkThreads) {
                        const double x = sc[i];
                        if (value_bin(x, lo, scale) >= t) put(atomicAdd(&s_nc, 1), x, i, -1, 0);
                    }
                }
                __syncthreads();
                if (__builtin_expect(C <= 64, 1)) {
                    // one wave sorts the candidates in registers (bitonic,
                    // best first): a lane per candidate, the padding lanes
                    // worse than any candidate
                    if (wave == 0) {
                        // each lane carries its candidate's slot
                        uint64_t key = lane < C ? s_ck[lane] : 0;
                        int32_t idx = lane < C ? s_ci[lane] : INT32_MAX;
                        int32_t slot = lane;
#pragma unroll
                        for (int kw = 2; kw <= 64; kw <<= 1) {
#pragma unroll
                            for (int jw = kw >> 1; jw > 0; jw >>= 1) {
                                const uint64_t ok = xor_lane(key, jw);
                                const int32_t oi = xor_lane(idx, jw);
                                const int32_t os = xor_lane(slot, jw);
                                // the lower lane of a pair keeps the better one in a
                                // best-first run, the worse one in a worst-first run
                                const bool lower = (lane & jw) == 0;
                                const bool best_first = (lane & kw) == 0;
                                const bool other_better = better(ok, oi, key, idx);
                                if (other_better == (lower == best_first)) {
                                    key = ok;
                                    idx = oi;
                                    slot = os;
                                }
                            }
                        }
                        const int tok = lane < kk ? s_cl[slot] : 0;
                        const int incl = wave_incl_sum(tok);
                        const int sum = __builtin_amdgcn_readlane(incl, 63);
                        if (lane < kk) {
                            cand_key[lane] = key;
                            cand_idx[lane] = idx;
                            if (planning) {
                                // rank lane's segment offset and first row
                                s_poff[lane] = incl - tok;
                                s_prow[lane] = s_cr[slot];
                            }
                        }
                        if (lane == 0) {
                            s_tokens = sum;
                            s_plen = sum;
                        }
                    }
                    __syncthreads();
                    tokens_known = true;
                    plan_known = true;
                    goto outputs;
                }
                int my_tokens = 0;
                for (int j = tid; j < C; j += blockDim.x) {
                    const uint64_t kj = s_ck[j];
                    const int ij = s_ci[j];
                    int r = 0;
#pragma unroll 8
                    for (int m = 0; m < C; ++m) r += better(s_ck[m], s_ci[m], kj, ij) ? 1 : 0;
                    if (r < kk) {
                        cand_key[r] = kj;
                        cand_idx[r] = ij;
                        my_tokens += s_cl[j];
                    }
                }
                if (my_tokens) atomicAdd(&s_tokens, my_tokens);
                __syncthreads();
                tokens_known = true;
                goto outputs;
            }
        }
    }

    if (__builtin_expect(mapped, 0)) {
        // exact fallback for candidate mode: the r-th winner is the best
        // candidate worse than the (r-1)-th on (score desc, fact id asc)
        __shared__ uint64_t s_rk[kTopkWaves];
        __shared__ int32_t s_ri[kTopkWaves];
        uint64_t pk = 0;
        int32_t pi = 0;
        for (int r = 0; r < kk; ++r) {
            uint64_t bk = 0;
            int32_t bi = INT32_MAX;
            for (int i = tid; i < n; i += kTopkThreads) {
                const uint64_t key = order_key(sc[i]);
                const int32_t id = imap[i];
                if ((r == 0 || better(pk, pi, key, id)) && better(key, id, bk, bi)) {
                    bk = key;
                    bi = id;
                }
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
                const uint64_t ok = __shfl_xor(bk, m, 64);
                const int32_t oi = __shfl_xor(bi, m, 64);
                if (better(ok, oi, bk, bi)) {
                    bk = ok;
                    bi = oi;
                }
            }
            if (lane == 0) {
                s_rk[wave] = bk;
                s_ri[wave] = bi;
            }
            __syncthreads();
            for (int w = 0; w < kTopkWaves; ++w)
                if (better(s_rk[w], s_ri[w], bk, bi)) {
                    bk = s_rk[w];
                    bi = s_ri[w];
                }
            if (tid == 0) {
                cand_key[r] = bk;
                cand_idx[r] = bi;
            }
            pk = bk;
            pi = bi;
            __syncthreads();
        }
        goto outputs;
    }

    {
    const bool in_lds = n <= fsi::kTopkLdsKeys;
    if (in_lds)
        for (int i = tid; i < n; i += blockDim.x) keys_lds[i] = order_key(sc[i]);
    auto key_at = [&](int i) -> uint64_t { return in_lds ? keys_lds[i] : order_key(sc[i]); };

    if (tid == 0) {
        s_prefix = 0;
        s_mask = 0;
        s_rem = kk;
        s_done = 0;
        s_ncand = 0;
        s_tokens = 0;
    }
    __syncthreads();

    // ---- MSB-first radix select of the kk-th largest key ------------------
    for (int shift = 56; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += blockDim.x) hist[i] = 0;
        __syncthreads();
        const uint64_t prefix = s_prefix, mask = s_mask;
        for (int i = tid; i < n; i += blockDim.x) {
            const uint64_t key = key_at(i);
            if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l holds digits 255-4l .. 252-4l (descending)
            int c[4];
            int sum = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                c[j] = hist[255 - 4 * lane - j];
                sum += c[j];
            }
            int incl = sum;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            const int excl = incl - sum;
            const int rem = s_rem;
            if (excl < rem && rem <= incl) {
                int cum = excl;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (cum + c[j] >= rem) {
                        const uint64_t digit = uint64_t(255 - 4 * lane - j);
                        const int left = rem - cum;       // still needed from this digit
                        s_prefix = prefix | (digit << shift);
                        s_mask = mask | (0xFFull << shift);
                        s_rem = left;
                        s_done = (c[j] == left);
                        break;
                    }
                    cum += c[j];
                }
            }
        }
        __syncthreads();
        if (s_done) break;
    }

    // ---- collect the winners ---------------------------------------------
    const uint64_t prefix = s_prefix, mask = s_mask;
    const bool done = s_done != 0;
    const int rem = s_rem;
    for (int i = tid; i < n; i += blockDim.x) {
        const uint64_t key = key_at(i);
        const uint64_t m = key & mask;
        if (m > prefix || (done && m == prefix)) {
            const int slot = atomicAdd(&s_ncand, 1);
            cand_key[slot] = key;
            cand_idx[slot] = i;
        }
    }
    __syncthreads();
    if (!done) {
        // equal full keys: keep the `rem` lowest indices, in index order
        const int first_slot = kk - rem;
        int taken = 0;
        for (int c0 = 0; c0 < n && taken < rem; c0 += blockDim.x) {
            const int i = c0 + tid;
            const bool eq = i < n && key_at(i) == prefix;
            const uint64_t bal = __ballot(eq);
            if (lane == 0) wave_cnt[wave] = __popcll(bal);
            __syncthreads();
            int before = 0, total = 0;
            for (int w = 0; w < kTopkThreads / 64; ++w) {
                if (w < wave) before += wave_cnt[w];
                total += wave_cnt[w];
            }
            const int rank = taken + before + __popcll(bal & ((1ull << lane) - 1ull));
            if (eq && rank < rem) {
                cand_key[first_slot + rank] = prefix;
                cand_idx[first_slot + rank] = i;
            }
            taken += total;
            __syncthreads();
        }
    }

    // ---- bitonic sort of the kk winners: key desc, index asc ---------------
    int P = 1;
    while (P < kk) P <<= 1;
    for (int i = kk + tid; i < P; i += blockDim.x) {
        cand_key[i] = 0;
        cand_idx[i] = 0x7FFFFFFF;
    }
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P; i += blockDim.x) {
                const int j = i ^ stride;
                if (j > i) {
                    const uint64_t ki = cand_key[i], kj = cand_key[j];
                    const int32_t ii = cand_idx[i], ij = cand_idx[j];
                    const bool j_first = (kj > ki) || (kj == ki && ij < ii);
                    const bool i_first = (ki > kj) || (ki == kj && ii < ij);
                    const bool ascending = (i & size) == 0;
                    if (ascending ? j_first : i_first) {
                        cand_key[i] = kj;
                        cand_key[j] = ki;
                        cand_idx[i] = ij;
                        cand_idx[j] = ii;
                    }
                }
            }
            __syncthreads();
        }
    }

    }

outputs:
    // ---- outputs -----------------------------------------------------------
    if (chunked) {
        const int64_t row = (int64_t(b) * a.nchunks + cidx) * k;
        for (int j = tid; j < kk; j += blockDim.x) {
            a.ids[row + j] = static_cast<int32_t>(base + cand_idx[j]);
            a.out_scores[row + j] = key_value(cand_key[j]);
        }
        return;
    }
    int my_tokens = 0;
    for (int j = tid; j < k; j += blockDim.x) {
        int32_t id = -1;
        double s = -__builtin_huge_val();
        if (j < kk) {
            id = static_cast<int32_t>(base + cand_idx[j]);
            s = key_value(cand_key[j]);
            if (!tokens_known && a.fact_len) my_tokens += a.fact_len[id];
        }
        a.ids[int64_t(b) * k + j] = id;
        if (a.out_scores) a.out_scores[int64_t(b) * k + j] = s;
    }
    if (a.num_tokens) {
        if (!tokens_known) {
            if (my_tokens) atomicAdd(&s_tokens, my_tokens);
            __syncthreads();
        }
        if (tid == 0) a.num_tokens[b] = s_tokens;
    }
    if (planning)
        plan_selected<kT>(a, b, kk, base, cand_idx, plan_known, plan_bad_user, s0, win_first, win_e, s_poff, s_prow,
                          s_win, s_winbad, &s_plen, &s_pbits);
}

}  // namespace


namespace {

// One block per request; n_max bounds the scores any request of the launch has.
void launch_topk(int64_t n_max, dim3 grid, size_t lds, hipStream_t stream, const TopkArgs& a) {
    const bool plan = a.plan.hdr != nullptr;
    if (n_max <= kTopkSmallN) {
        if (plan) fs_topk_kernel<256, true><<<grid, 256, lds, stream>>>(a);
        else fs_topk_kernel<256, false><<<grid, 256, lds, stream>>>(a);
    } else {
        if (plan) fs_topk_kernel<1024, true><<<grid, 1024, lds, stream>>>(a);
        else fs_topk_kernel<1024, false><<<grid, 1024, lds, stream>>>(a);
    }
}

}  // namespace

hipError_t fsi_launch_retrieve(const RetrieveLaunch& r) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    if (r.k > 0 && st->max_user_facts > 0) {
        ScoreArgs sa{};
        sa.emb = reinterpret_cast<const float4*>(st->emb);
        sa.e4 = d.embed_dim / 4;
        sa.user_begin = st->d_user_begin;
        sa.user_count = st->d_user_count;
        sa.num_users = d.num_users;
        sa.user = r.user;
        sa.query = reinterpret_cast<const float4*>(r.query);
        sa.batch = r.batch;
        sa.scores = st->d_scores;
        sa.stride = st->max_user_facts;
        dim3 grid((st->max_user_facts + kScoreRowsPerBlock - 1) / kScoreRowsPerBlock, r.batch);
        if (r.batch == 1) fs_score_kernel<1><<<grid, 256, 0, r.stream>>>(sa);
        else fs_score_kernel<kScoreGroup><<<grid, 256, 0, r.stream>>>(sa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    TopkArgs ta{};
    ta.scores = st->d_scores;
    ta.stride = st->max_user_facts;
    ta.user_begin = st->d_user_begin;
    ta.user_count = st->d_user_count;
    ta.num_users = d.num_users;
    ta.user = r.user;
    ta.fact_len = st->d_fact_len;
    ta.k = r.k;
    ta.ids = r.ids;
    ta.out_scores = r.scores;
    ta.num_tokens = r.num_tokens;
    ta.err = st->d_err;
    if (r.plan) {
        ta.plan = fsi_plan_view(st, r.batch, r.plan);
        ta.plan_key = fsi_plan_key(st->tag, r.batch, r.k, st->seg_tokens, r.num_blocks);
        ta.plan_tag = st->tag;
        ta.batch = r.batch;
        ta.seg_tokens = st->seg_tokens;
        ta.num_blocks = r.num_blocks;
        ta.max_blocks = r.max_blocks;
        ta.log2_block = st->log2_block;
        ta.block_table = r.block_table;
        ta.start_pos = r.start_pos;
        ta.fact_begin = st->d_fact_begin;
    }
    if (st->topk_chunks > 0 && r.k > 0) {
        // large users: the top k of every chunk, one block each, then the top
        // k of those candidates by (score desc, fact id asc).  Every fact of
        // the true top k is among its own chunk's top k, so this is exact.
        TopkArgs t1 = ta;
        t1.plan = PlanView{};
        t1.fact_len = nullptr;
        t1.num_tokens = nullptr;
        t1.ids = st->d_tk_ids;
        t1.out_scores = st->d_tk_scores;
        t1.chunk = fsi::kTopkChunk;
        t1.nchunks = st->topk_chunks;
        t1.out_counts = st->d_tk_counts;
        launch_topk(fsi::kTopkChunk, dim3(static_cast<unsigned>(r.batch) * st->topk_chunks),
                    sizeof(uint64_t) * size_t(fsi::kTopkLdsKeys), r.stream, t1);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        TopkArgs t2 = ta;
        t2.scores = st->d_tk_scores;
        t2.stride = st->topk_chunks * r.k;
        t2.counts = st->d_tk_counts;
        t2.idmap = st->d_tk_ids;
        launch_topk(int64_t(t2.stride), dim3(r.batch), 0, r.stream, t2);
        return hipGetLastError();
    }
    const int lds_keys = st->max_user_facts < fsi::kTopkLdsKeys ? st->max_user_facts : fsi::kTopkLdsKeys;
    size_t lds = sizeof(uint64_t) * size_t(lds_keys);
    launch_topk(st->max_user_facts, dim3(r.batch), lds, r.stream, ta);
    return hipGetLastError();
}

// Approximate retrieval through an inverted-file index: centroid scores,
// top-nprobe lists, scan of those lists, top-k of the candidates by
// (score desc, fact id asc).
hipError_t fsi_launch_ivf_probe(const IvfProbeLaunch& r) {
    const fs_ivf* ix = r.ivf;
    const fs_store* st = ix->store;
    const fs_store_desc& d = st->desc;
    const int e4 = d.embed_dim / 4;
    ScoreArgs sa{};
    sa.emb = reinterpret_cast<const float4*>(ix->d_cent);
    sa.e4 = e4;
    sa.user_begin = ix->d_cent_range;
    sa.num_users = 1;
    sa.user = ix->d_zero_users;
    sa.query = reinterpret_cast<const float4*>(r.query);
    sa.batch = r.batch;
    sa.scores = ix->d_cscores;
    sa.stride = ix->nlist;
    dim3 g1((ix->nlist + kScoreRowsPerBlock - 1) / kScoreRowsPerBlock, r.batch);
    if (r.batch == 1) fs_score_kernel<1><<<g1, 256, 0, r.stream>>>(sa);
    else fs_score_kernel<kScoreGroup><<<g1, 256, 0, r.stream>>>(sa);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    TopkArgs t1{};
    t1.scores = ix->d_cscores;
    t1.stride = ix->nlist;
    t1.user_begin = ix->d_cent_range;
    t1.num_users = 1;
    t1.user = ix->d_zero_users;
    t1.k = r.nprobe;
    t1.ids = ix->d_chosen;          // row stride nprobe: written as [B][nprobe]
    t1.err = st->d_err;
    const int lds1 = ix->nlist < fsi::kTopkLdsKeys ? ix->nlist : fsi::kTopkLdsKeys;
    launch_topk(ix->nlist, dim3(r.batch), sizeof(uint64_t) * size_t(lds1), r.stream, t1);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    ListArgs la{};
    la.emb_sorted = reinterpret_cast<const float4*>(ix->d_emb_sorted);
    la.e4 = e4;
    la.list_begin = ix->d_list_begin;
    la.members = ix->d_members;
    la.chosen = ix->d_chosen;
    la.np_stride = r.nprobe;
    la.nprobe = r.nprobe;
    la.query = reinterpret_cast<const float4*>(r.query);
    la.cand_scores = ix->d_cand_scores;
    la.cand_ids = ix->d_cand_ids;
    la.counts = ix->d_counts;
    la.stride = ix->cand_stride;
    la.offs = ix->d_offs;
    fs_list_offsets_kernel<<<dim3(r.batch), 64, 0, r.stream>>>(la);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 g3((ix->max_list + kScoreRowsPerBlock - 1) / kScoreRowsPerBlock, r.nprobe, r.batch);
    fs_list_score_kernel<<<g3, 256, 0, r.stream>>>(la);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    TopkArgs t2{};
    t2.scores = ix->d_cand_scores;
    t2.stride = ix->cand_stride;
    t2.fact_len = st->d_fact_len;
    t2.k = r.k;
    t2.ids = r.ids;
    t2.out_scores = r.scores;
    t2.num_tokens = r.num_tokens;
    t2.err = st->d_err;
    t2.counts = ix->d_counts;
    t2.idmap = ix->d_cand_ids;
    launch_topk(int64_t(r.nprobe) * ix->max_list, dim3(r.batch), 0, r.stream, t2);
    return hipGetLastError();
}
