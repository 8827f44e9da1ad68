// Compose -> Chunked RoPE -> paged scatter, and the host-memory fetch.
//
// InferScale's online phase (gist.science summary, "Phase En-ligne"): keys
// are stored before RoPE; at serving time the retrieved facts are composed
// into one contiguous segment, every stored key is rotated to its new
// serving-time position, and the composed K/V is scatter-copied into the
// paged KV cache.  Values are copied raw.  The re-rotation is exact under
// RoPE (Theorem 6 as the pages describe it), so the rotation is evaluated in
// fp64 and rounded once to bf16.
//
// Two kernels per injection:
//
// Plan (fs_plan_kernel, one block per request): composes the segment (prefix
// sums of the selected facts' lengths, ids checked against the user),
// validates the request (start position, block-table coverage and entries,
// for pinned stores the staging slot) and writes a plan: a header naming the
// store, batch, k and cache size it was checked for, the segment length (0
// for a rejected request) and start position, and every segment token's
// arena row and cache slot.
//
// Inject (fs_row_kernel, and fs_short_kernel for rows under 1 KB): a pure
// stream over the plan.  Each 256-thread workgroup moves whole token rows of
// K or of V (never both) for one request and layer, one 16-byte vector per
// lane, read once and written once, so a workgroup carries 4 KB and the
// launch holds tens of thousands of them.  K rows are rotated on the way
// through with cos/sin evaluated in fp64 while the row is in flight.
//
// HBM-bound gather/copy with a small amount of arithmetic; no dense
// contraction, so no MFMA.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "fs_device.h"
#include "fs_internal.h"
#include "fs_plan.h"

namespace {

using fsd::bf16_hi;
using fsd::bf16_lo;
using fsd::f64_to_bf16_bits;
using fsd::sincos_angle;
using fsd::wave_or;

constexpr int kThreads = 64;        // one wave per fetch block
constexpr int kFlatThreads = 256;   // 4 waves per inject workgroup
constexpr int kPlanThreads = 1024;

#define FS_GLOBAL __attribute__((address_space(1)))
#define FS_CONST __attribute__((address_space(4)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_stream(const FS_GLOBAL u32x4* p) { return __builtin_nontemporal_load(p); }
// A streaming store at device scope (sc1 nt).  Against the plain streaming
// store (nt alone), a gather of 2 KB rows into 32 KB cache blocks at the
// inject's size ran 2% faster: 67.4 against 68.9 us.
__device__ __forceinline__ void st_stream(FS_GLOBAL u32x4* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1 nt" ::"v"(p), "v"(v) : "memory");
}
// a cache row store: streaming, or through the caches when the launch's
// writes fit in the last-level cache (a compile-time choice: a branch per
// store cost the streaming launch 3%)
template <bool kCached>
__device__ __forceinline__ void st_row(FS_GLOBAL u32x4* p, u32x4 v) {
    if constexpr (kCached) *p = v;
    else st_stream(p, v);
}
// a load the caller knows is wave-uniform and not written during the kernel:
// through the scalar cache (its own counter, so it never waits on the
// vector loads in flight)
template <class T>
__device__ __forceinline__ T sload(const T* p) { return *(const FS_CONST T*)p; }
__device__ __forceinline__ PlanReq sload(const PlanReq* p) {
    const uint64_t v = sload(reinterpret_cast<const uint64_t*>(p));
    return PlanReq{static_cast<int32_t>(v & 0xFFFFFFFFu), static_cast<int32_t>(v >> 32)};
}
__device__ __forceinline__ PlanTok sload(const PlanTok* p) { return PlanTok{sload(&p->src), sload(&p->dst)}; }

struct PlanArgs {
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    int32_t batch;
    const int32_t* block_table;
    int32_t max_blocks;
    const int32_t* start_pos;
    int32_t num_blocks;
    int32_t log2_block;
    const int64_t* fact_begin;
    const int32_t* fact_len;
    const int64_t* user_begin;
    const int32_t* user_count;      // live facts per user (from user_begin[u])
    int32_t num_users;
    int64_t num_facts;
    int32_t layer_begin, layer_end;
    const int32_t* stage_ids;       // non-null for pinned stores
    const int32_t* stage_meta;
    int32_t staging_layers, max_batch, max_k;
    int32_t seg_tokens;
    uint32_t tag;
    uint64_t key;
    PlanView out;
    uint32_t* err;
};

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int y = __shfl_up(v, off, 64);
        if (lane >= off) v += y;
    }
    return v;
}

// Segment plan of request b, by one wave, into LDS.
//   off[j]  = first segment token of the j-th selected fact (j < nf)
//   row0[j] = its first arena row
// Returns the error bits (0 when the request can be served); *L and *nf get
// the segment length and the number of real (non-pad) ids.
__device__ uint32_t plan_request(const int32_t* user, const int32_t* ids, int k,
                                 const int64_t* user_begin, const int32_t* user_count, int num_users,
                                 int64_t num_facts, const int32_t* fact_len, const int64_t* fact_begin, int b,
                                 int32_t* off, int64_t* row0, int* L_out, int* nf_out) {
    const int lane = threadIdx.x & 63;
    uint32_t bits = 0;
    // the user and the first 64 ids are read together; the user's range and
    // each id's length and first row then together (an id outside the fact
    // table reads fact 0 and is rejected below): two dependent rounds
    const int u = user[b];
    const int id0 = lane < k ? ids[int64_t(b) * k + lane] : 0;
    const bool bad_user = (u < 0 || u >= num_users);
    if (bad_user) bits |= FS_ERR_USER;
    const int64_t ub0 = bad_user ? 0 : user_begin[u];
    const int64_t ub1 = bad_user ? 0 : ub0 + user_count[u];     // the user's live facts
    // Lengths are counted only up to the first -1 pad, so every token t < L
    // maps into a valid fact of the user even when the request is rejected.
    int carry = 0, first_pad = k, last_real = -1;
    for (int c0 = 0; c0 < k; c0 += 64) {
        const int j = c0 + lane;
        const int id = c0 == 0 ? id0 : (j < k ? ids[int64_t(b) * k + j] : 0);
        const int64_t idc = id >= 0 && id < num_facts ? id : 0;
        const int len_any = j < k ? fact_len[idc] : 0;
        const int64_t r0_any = j < k ? fact_begin[idc] : 0;
        int len = 0;
        int64_t r0 = 0;
        first_pad = wave_min(min(first_pad, (j < k && id < 0) ? j : k));
        if (j < k) {
            if (id < 0 || j > first_pad) {
                // pad, or an id after a pad (reported below)
            } else {
                if (bad_user) {
                    // reported once as FS_ERR_USER; ids cannot be judged
                } else if (id < ub0 || id >= ub1) {
                    bits |= FS_ERR_FACT_ID;
                } else {
                    len = len_any;
                    r0 = r0_any;
                }
            }
        }
        if (j < k && id >= 0) last_real = j;
        const int incl = wave_incl_scan(len, lane);
        if (j < k) {
            off[j] = carry + incl - len;
            row0[j] = r0;
        }
        carry += __shfl(incl, 63, 64);
    }
    last_real = wave_max(last_real);
    if (last_real > first_pad) bits |= FS_ERR_FACT_ID;
    *L_out = carry;
    *nf_out = first_pad;
    return bits;
}

// Validation of one composed request: start position, block-table coverage
// and entries, and for pinned stores that every staging slot holds these ids.
__device__ uint32_t check_request(const PlanArgs& a, int b, int L) {
    const int lane = threadIdx.x & 63;
    uint32_t bits = 0;
    const int s = a.start_pos[b];
    const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
    bits |= fsp::check_segment(s, L, a.max_blocks, a.num_blocks, a.log2_block, lane, 64,
                               [&](int j) { return bt[j]; });
    if (a.stage_ids) {
        for (int l = a.layer_begin; l < a.layer_end; ++l) {
            const int slot = l % a.staging_layers;
            const int32_t* meta = a.stage_meta + 4 * slot;
            if (meta[0] != a.k || meta[1] <= b || meta[2] != l) {
                bits |= FS_ERR_STAGING;
            } else {
                const int32_t* sid = a.stage_ids + (int64_t(slot) * a.max_batch + b) * a.max_k;
                for (int j = lane; j < a.k; j += 64)
                    if (sid[j] != a.ids[int64_t(b) * a.k + j]) bits |= FS_ERR_STAGING;
            }
        }
    }
    return bits;
}

// One block per request.  Wave 0 composes and validates into LDS, then the
// whole block writes the token map; a rejected request gets length 0.
// Block 0 also writes the plan header.
__global__ __launch_bounds__(kPlanThreads) void fs_plan_kernel(PlanArgs a) {
    extern __shared__ int64_t plan_lds[];
    __shared__ int s_len, s_nf;
    int64_t* row0 = plan_lds;
    int32_t* off = reinterpret_cast<int32_t*>(plan_lds + a.k);
    const int b = blockIdx.x;
    if (threadIdx.x < 64) {
        int L = 0, nf = 0;
        uint32_t bits = plan_request(a.user, a.ids, a.k, a.user_begin, a.user_count, a.num_users, a.num_facts, a.fact_len,
                                     a.fact_begin, b, off, row0, &L, &nf);
        bits |= check_request(a, b, L);
        bits = wave_or(bits);
        if (threadIdx.x == 0) {
            if (bits) atomicOr(a.err, bits);
            s_len = bits ? 0 : L;
            s_nf = nf;
            a.out.req[b] = PlanReq{bits ? 0 : L, a.start_pos[b]};
            if (b == 0) fsp::write_header(a.out.hdr, a.key, a.tag, a.batch, a.k, a.seg_tokens, a.num_blocks);
        }
    }
    __syncthreads();
    const int L = s_len, nf = s_nf;
    const int s = a.start_pos[b];
    const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
    fsp::write_tokens(a.out.tok + int64_t(b) * a.seg_tokens, off, row0, nf, L, s, a.log2_block, threadIdx.x,
                      blockDim.x, [&](int j) { return bt[j]; });
}

struct FlatArgs {
    // read by every wave first (kept together)
    const PlanHeader* hdr;
    const PlanReq* req;
    const PlanTok* tok;
    uint64_t key;                   // what the plan header must hold
    const void* const* src_kv;      // device table [num_layers][2] (device stores)
    const double* inv_freq;         // [D/2] w_i
    int64_t row_elems;              // heads * D
    int64_t num_rows;               // arena rows: every source row lies below
    int64_t cache_rows;             // num_blocks * block_size
    int32_t units;                  // workgroups per (kind, request, layer)
    int32_t layer_begin;
    int32_t seg_tokens;
    int32_t vpr;                    // the row's 16-byte vectors (heads * D / 8)
    // rarely read
    const uint16_t* stage_k;        // staging ring (pinned stores)
    const uint16_t* stage_v;
    int32_t staging_layers, stage_tokens, max_batch;
    uint32_t* err;
    void* cache[2 * FS_MAX_LAYERS]; // [layer][K, V]
};

// The lane's rotate-half partner: the same vector position in the other half
// of its head, D/16 lanes away (xor; heads start at multiples of D/8 lanes).
template <int D>
__device__ __forceinline__ uint32_t partner(uint32_t v) {
    if constexpr (D == 128) {
        // rotate each row of 16 lanes by 8: lane i receives lane i ^ 8
        return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false));
    } else if constexpr (D == 64) {
        // swizzle within 32 lanes: and 0x1f, or 0, xor 4
        return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x101F));
    } else {
        // xor 16
        return static_cast<uint32_t>(__builtin_amdgcn_ds_swizzle(static_cast<int>(v), 0x401F));
    }
}

// The first workgroup of the launch checks the plan's key even when its
// request is empty (a live one checks it on its way), so a plan that is not
// this call's is reported whatever its lengths hold.
__device__ __forceinline__ void plan_check_once(const FlatArgs& a) {
    if (threadIdx.x == 0 && sload(&a.hdr->key) != a.key) atomicOr(a.err, FS_ERR_PLAN);
}

// Rotate-half of one 16-byte vector (8 bf16) of a K row: the first half's
// lanes compute y_i = x_i c - x_{i+D/2} s, the second half's
// y_{i+D/2} = x_{i+D/2} c + x_i s, each from its own vector and its
// partner's; the vector holds pairs i = 8*tl .. 8*tl+7.  The row's cos/sin
// table is stored transposed (pair 8*tl + k at k * D/16 + tl), so the lanes
// of a half head read consecutive entries.  The sign is applied to the
// partner's bf16 sign bit (exact) rather than by a multiply.
//
// Narrowing to bf16: the fp64 value rounded to fp32 (nearest) and then to
// bf16 (nearest even) equals its direct rounding to bf16 unless the fp32
// value sits exactly on a bf16 midpoint (low 16 bits 0x8000), the one case
// a double rounding can decide wrongly; a wave with such a lane redoes the
// vector with the exact narrowing (round-to-odd to fp32 first).
template <int D>
__device__ __forceinline__ u32x4 rotate_vec(u32x4 x, int vec, const double2* row_cs) {
    constexpr int kHalfV = D / 16;
    const int vh = vec & (D / 8 - 1);
    const bool second = vh >= kHalfV;
    const int tl = second ? vh - kHalfV : vh;
    const uint32_t neg = second ? 0u : 0x80008000u;
    u32x4 p;
    p.x = partner<D>(x.x) ^ neg;
    p.y = partner<D>(x.y) ^ neg;
    p.z = partner<D>(x.z) ^ neg;
    p.w = partner<D>(x.w) ^ neg;
    const double2* cp = row_cs + tl;
    double yd[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double2 c0 = cp[(2 * e) * kHalfV], c1 = cp[(2 * e + 1) * kHalfV];
        yd[2 * e] = fma(static_cast<double>(bf16_lo(x[e])), c0.x, static_cast<double>(bf16_lo(p[e])) * c0.y);
        yd[2 * e + 1] = fma(static_cast<double>(bf16_hi(x[e])), c1.x, static_cast<double>(bf16_hi(p[e])) * c1.y);
    }
    u32x4 y;
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t u0 = __float_as_uint(static_cast<float>(yd[2 * e]));
        const uint32_t u1 = __float_as_uint(static_cast<float>(yd[2 * e + 1]));
        tie |= (u0 & 0xFFFFu) == 0x8000u || (u1 & 0xFFFFu) == 0x8000u;
        y[e] = ((u0 + 0x7FFFu + ((u0 >> 16) & 1u)) >> 16) | ((u1 + 0x7FFFu + ((u1 >> 16) & 1u)) & 0xFFFF0000u);
    }
    if (__builtin_amdgcn_ballot_w64(tie)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = f64_to_bf16_bits(yd[2 * e]) | (f64_to_bf16_bits(yd[2 * e + 1]) << 16);
    }
    return y;
}

// cos/sin(p * w_i) of kTok rows of the workgroup (row j at position
// start + min(t0 + j, L - 1)) into LDS, row j at j * D/2, pair i of it
// transposed as rotate_vec reads it.  The angle lies
// below 2^31, so a reduction by pi/2 in three parts covers it with no
// large-argument path (the library's sincos carries one, and computing it on
// every lane beside the short path cost the launch 3%).
template <int D, int kTok>
__device__ __forceinline__ void fill_cs(double2* s_cs, const double* w_e, int start, int t0, int L) {
    constexpr int kE = kTok * (D / 2);
    constexpr int kEPT = (kE + kFlatThreads - 1) / kFlatThreads;
#pragma unroll
    for (int q = 0; q < kEPT; ++q) {
        const int e = static_cast<int>(threadIdx.x) + q * kFlatThreads;
        if (e < kE) {
            const int tt = min(t0 + e / (D / 2), L - 1);
            const int i = e & (D / 2 - 1);
            double sv, cv;
            sincos_angle(static_cast<double>(start + tt) * w_e[q], &sv, &cv);
            s_cs[(e - i) + (i & 7) * (D / 16) + (i >> 3)] = make_double2(cv, sv);
        }
    }
}

// The (request, layer) segment's K rows or V rows are cut into workgroups
// of 256 16-byte vectors, one per lane: a row of 2^kLg vectors (the row's
// heads * D / 8, rounded up to a power of two; the lanes of the padding stay
// idle) gives each workgroup 256 >> kLg whole rows, or 2^(kLg-8)
// workgroups one row.  The grid covers a segment of k of the store's longest
// facts, so a workgroup past its request's real length exits; it reads only
// that length first (a workgroup that also loaded its plan entries before
// finding itself empty made the launch 5% slower), and a live one then
// reads the rest.  The workgroups of one launch number in the tens of
// thousands and a compute unit's scalar unit issues for all of them, so the
// prologue is short: compile-time shifts and masks, one 64-bit key rather
// than field-by-field plan checks, and one scalar load per request, row and
// layer.
//
// Rows of 64 vectors or more (fs_row_kernel): every wave lies inside one row,
// so the wave's plan entry comes through the scalar cache.  K workgroups
// first issue the loads of the inverse frequencies of the cos/sin entries
// they own, then the K row, then evaluate cos/sin(p * w_i) in fp64 into LDS
// while the row is in flight; a lane's rotate-half partner (D/16 lanes away,
// in the same head) arrives by a cross-lane move.  Per launch on the Llama
// shape: 68.8 us, against 80 us for a block of 8 tokens x all heads x K and V
// with a per-block plan and cos/sin table, and 73.8 us for the runtime's
// device copy of the same bytes.
template <int D, int kLg, bool kStaged, bool kCached>
__global__ __launch_bounds__(kFlatThreads) void fs_row_kernel(FlatArgs a) {
    constexpr int kSplit = kLg > 8 ? kLg - 8 : 0;              // log2 workgroups per row
    constexpr int kTok = kLg <= 8 ? kFlatThreads >> kLg : 1;   // rows per workgroup
    constexpr int kE = kTok * (D / 2);
    constexpr int kEPT = (kE + kFlatThreads - 1) / kFlatThreads;
    static_assert(kLg >= 6, "a wave lies inside one row");
    __shared__ double2 s_cs[kE];

    const int kind = blockIdx.x >= static_cast<unsigned>(a.units);
    const int unit = static_cast<int>(blockIdx.x) - kind * a.units;
    const int b = blockIdx.y;
    const int l = a.layer_begin + static_cast<int>(blockIdx.z);
    // the request's length and start first: a workgroup past the segment
    // leaves after this one load
    const PlanReq rq = sload(a.req + b);
    const int L = rq.len;
    const int t0 = kLg <= 8 ? unit * kTok : unit >> kSplit;    // first row of the workgroup
    if (t0 >= L) {
        if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0) plan_check_once(a);
        return;
    }
    const int r = kLg <= 8 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> kLg) : 0;
    const int vec = kLg <= 8 ? static_cast<int>(threadIdx.x) & ((1 << kLg) - 1)
                             : ((unit & ((1 << kSplit) - 1)) << 8) + static_cast<int>(threadIdx.x);
    const int tw = t0 + r;                                      // the wave's row
    // in range of the plan's token map whatever the header holds
    const PlanTok* te = a.tok + int64_t(b) * a.seg_tokens + min(tw, a.seg_tokens - 1);
    const int64_t stage_row = kStaged ? (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + tw : 0;

    if (kind == 1) {
        // V: a raw row copy
        if (tw >= L) return;
        const uint64_t key = sload(&a.hdr->key);
        const int64_t sr = kStaged ? stage_row : sload(&te->src);
        const int64_t dr = sload(&te->dst);
        const uint16_t* sb = kStaged ? a.stage_v : static_cast<const uint16_t*>(sload(a.src_kv + 2 * l + 1));
        if (key != a.key || L > a.seg_tokens) {
            // not a plan of this store, batch, k and cache size: nothing is written
            if (blockIdx.x == static_cast<unsigned>(a.units) && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
                atomicOr(a.err, FS_ERR_PLAN);
            return;
        }
        // a row outside the arena or the caches is never touched (a plan
        // this store wrote has none)
        if (!(kStaged || static_cast<uint64_t>(sr) < static_cast<uint64_t>(a.num_rows)) ||
            static_cast<uint64_t>(dr) >= static_cast<uint64_t>(a.cache_rows)) {
            if ((threadIdx.x & 63) == 0) atomicOr(a.err, FS_ERR_PLAN);
            return;
        }
        if (vec >= a.vpr) return;
        const u32x4 x = ld_stream((const FS_GLOBAL u32x4*)(sb + sr * a.row_elems) + vec);
        st_row<kCached>((FS_GLOBAL u32x4*)(static_cast<uint16_t*>(a.cache[2 * l + 1]) + dr * a.row_elems) + vec, x);
        return;
    }

    // K: the frequencies of the table entries this thread evaluates, then
    // the key, the wave's row entry and the layer's arena, all at once
    double w_e[kEPT];
#pragma unroll
    for (int q = 0; q < kEPT; ++q)
        w_e[q] = a.inv_freq[(static_cast<int>(threadIdx.x) + q * kFlatThreads) & (D / 2 - 1)];
    const uint64_t key = sload(&a.hdr->key);
    const int64_t sr = kStaged ? stage_row : sload(&te->src);
    const int64_t dr = sload(&te->dst);
    const uint16_t* sb = kStaged ? a.stage_k : static_cast<const uint16_t*>(sload(a.src_kv + 2 * l));
    // naming every loaded value here keeps the compiler from sinking the
    // loads into the branches below one round trip at a time
    asm volatile("" ::"s"(key), "s"(sr), "s"(dr), "s"(sb));
    if (key != a.key || L > a.seg_tokens) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) atomicOr(a.err, FS_ERR_PLAN);
        return;
    }
    const bool ok = (kStaged || static_cast<uint64_t>(sr) < static_cast<uint64_t>(a.num_rows)) &&
                    static_cast<uint64_t>(dr) < static_cast<uint64_t>(a.cache_rows);
    const bool act = tw < L && ok;
    // the row load is issued by every lane (a wave without a row reads the
    // arena's first row): a conditional load would leave the compiler unsure
    // how many loads are in flight, and it would then wait for the row
    // before the cos/sin evaluation instead of after it
    asm volatile("" ::: "memory");
    const u32x4 x = ld_stream((const FS_GLOBAL u32x4*)(sb + (act ? sr * a.row_elems : 0)) + min(vec, a.vpr - 1));
    asm volatile("" ::: "memory");
    fill_cs<D, kTok>(s_cs, w_e, rq.start, t0, L);
    __syncthreads();
    if (!act) {
        // reported after the loads: a memory operation between the plan
        // loads and the row load would make the compiler wait for every
        // load in flight
        if (tw < L && (threadIdx.x & 63) == 0) atomicOr(a.err, FS_ERR_PLAN);
        return;
    }
    const u32x4 y = rotate_vec<D>(x, vec, s_cs + r * (D / 2));
    if (vec < a.vpr)
        st_row<kCached>((FS_GLOBAL u32x4*)(static_cast<uint16_t*>(a.cache[2 * l]) + dr * a.row_elems) + vec, y);
}

// Rows of fewer than 64 vectors (fs_short_kernel): a wave holds 64 >> kLg
// rows and each lane takes the entry of its own row among the wave's.
template <int D, int kLg, bool kStaged, bool kCached>
__global__ __launch_bounds__(kFlatThreads) void fs_short_kernel(FlatArgs a) {
    constexpr int kVPR = 1 << kLg;
    constexpr int kRPW = 64 >> kLg;                    // rows per wave
    constexpr int kTok = kFlatThreads >> kLg;          // rows per workgroup
    constexpr int kE = kTok * (D / 2);
    constexpr int kEPT = (kE + kFlatThreads - 1) / kFlatThreads;
    static_assert(kLg < 6, "rows shorter than a wave");
    __shared__ double2 s_cs[kE];

    const int kind = blockIdx.x >= static_cast<unsigned>(a.units);
    const int unit = static_cast<int>(blockIdx.x) - kind * a.units;
    const int b = blockIdx.y;
    const int l = a.layer_begin + static_cast<int>(blockIdx.z);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int tf = unit * kTok;                        // first row of the workgroup
    const int tw0 = tf + wave * kRPW;                  // the wave's first row
    const PlanReq rq = sload(a.req + b);
    const int L = rq.len;
    if (tf >= L) {
        if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0) plan_check_once(a);
        return;
    }

    double w_e[kEPT];
    if (kind == 0) {
#pragma unroll
        for (int q = 0; q < kEPT; ++q)
            w_e[q] = a.inv_freq[(static_cast<int>(threadIdx.x) + q * kFlatThreads) & (D / 2 - 1)];
    }
    const uint64_t key = sload(&a.hdr->key);
    PlanTok tk[kRPW];
    const PlanTok* tb = a.tok + int64_t(b) * a.seg_tokens;
#pragma unroll
    for (int j = 0; j < kRPW; ++j) tk[j] = sload(tb + min(tw0 + j, a.seg_tokens - 1));
    const uint16_t* src_base =
        kStaged ? (kind == 0 ? a.stage_k : a.stage_v) : static_cast<const uint16_t*>(sload(a.src_kv + 2 * l + kind));
    asm volatile("" ::"s"(key), "s"(src_base));
#pragma unroll
    for (int j = 0; j < kRPW; ++j) asm volatile("" ::"s"(tk[j].src), "s"(tk[j].dst));
    if (key != a.key || L > a.seg_tokens) {
        if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) atomicOr(a.err, FS_ERR_PLAN);
        return;
    }
    uint16_t* dst_base = static_cast<uint16_t*>(a.cache[2 * l + kind]);

    // the lane's own row among the wave's
    const int tj = tf + (static_cast<int>(threadIdx.x) >> kLg);
    const int vj = static_cast<int>(threadIdx.x) & (kVPR - 1);
    int64_t sr = tk[0].src, dr = tk[0].dst;
#pragma unroll
    for (int j = 1; j < kRPW; ++j)
        if (tj - tw0 == j) {
            sr = tk[j].src;
            dr = tk[j].dst;
        }
    if (kStaged) sr = (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + tj;
    const bool ok = (kStaged || static_cast<uint64_t>(sr) < static_cast<uint64_t>(a.num_rows)) &&
                    static_cast<uint64_t>(dr) < static_cast<uint64_t>(a.cache_rows);
    const bool in = tj < L && vj < a.vpr;
    const bool bad = in && !ok;
    const bool act = in && ok;
    const u32x4 x = ld_stream((const FS_GLOBAL u32x4*)(src_base + (act ? sr * a.row_elems + int64_t(vj) * 8 : 0)));
    asm volatile("" ::: "memory");
    if (kind == 1) {
        if (act) st_row<kCached>((FS_GLOBAL u32x4*)(dst_base + dr * a.row_elems) + vj, x);
        if (bad) atomicOr(a.err, FS_ERR_PLAN);
        return;
    }
    fill_cs<D, kTok>(s_cs, w_e, rq.start, tf, L);
    __syncthreads();
    const u32x4 y = rotate_vec<D>(x, vj, s_cs + min(tj - tf, kTok - 1) * (D / 2));
    if (act) st_row<kCached>((FS_GLOBAL u32x4*)(dst_base + dr * a.row_elems) + vj, y);
    if (bad) atomicOr(a.err, FS_ERR_PLAN);
}

struct FetchArgs {
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    const int64_t* fact_begin;
    const int32_t* fact_len;
    const int64_t* user_begin;
    const int32_t* user_count;      // live facts per user (from user_begin[u])
    int32_t num_users;
    int64_t num_facts;
    int32_t heads;
    int32_t layer_begin, layer_end, layers_per_block;
    const void* const* src_k;       // device table of device-visible host addresses
    const void* const* src_v;
    uint16_t* stage_k;
    uint16_t* stage_v;
    int32_t* stage_ids;
    int32_t* stage_meta;
    int32_t staging_layers, stage_tokens, max_batch, max_k, batch;
    uint32_t* err;
};

template <int D>
__global__ __launch_bounds__(kThreads) void fs_fetch_kernel(FetchArgs a) {
    constexpr int kTok = kThreads / (D / 16);   // tokens per block
    extern __shared__ int64_t plan_lds[];
    int64_t* row0 = plan_lds;
    int32_t* off = reinterpret_cast<int32_t*>(plan_lds + a.k);

    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    int L = 0, nf = 0;
    uint32_t bits = plan_request(a.user, a.ids, a.k, a.user_begin, a.user_count, a.num_users, a.num_facts, a.fact_len,
                                 a.fact_begin, b, off, row0, &L, &nf);
    bits = wave_or(bits);
    const int l0 = a.layer_begin + blockIdx.z * a.layers_per_block;
    const int l1 = min(a.layer_end, l0 + a.layers_per_block);
    if (blockIdx.x == 0) {
        // record what this staging slot now holds (a failed request records
        // ids that can never match, so a later inject refuses it)
        for (int l = l0; l < l1; ++l) {
            const int slot = l % a.staging_layers;
            int32_t* sid = a.stage_ids + (int64_t(slot) * a.max_batch + b) * a.max_k;
            for (int j = lane; j < a.k; j += 64) sid[j] = bits ? INT32_MIN : a.ids[int64_t(b) * a.k + j];
            if (b == 0 && lane == 0) {
                a.stage_meta[4 * slot] = a.k;
                a.stage_meta[4 * slot + 1] = a.batch;
                a.stage_meta[4 * slot + 2] = l;
            }
        }
    }
    if (bits) {
        if (lane == 0 && blockIdx.x == 0 && blockIdx.z == 0) atomicOr(a.err, bits);
        return;
    }
    __syncthreads();

    // the whole wave copies one token row at a time, two tokens in flight:
    // each instruction reads 1 KiB of contiguous host memory, so the host
    // link carries large read requests (a team of lanes per token, each
    // instruction touching 8 rows, reached 88% of a DMA copy; this, 97%)
    const int t0 = blockIdx.x * kTok;
    const int tend = min(L, t0 + kTok);
    if (t0 >= tend) return;
    const int64_t row_elems = int64_t(a.heads) * D;
    const int vec_per_row = a.heads * (D / 8);
    for (int l = l0; l < l1; ++l) {
        for (int tt = t0; tt < tend; tt += 2) {
            const bool two = tt + 1 < tend;
            const int ja = fsp::find_fact(off, nf, tt);
            const int64_t rowa = row0[ja] + (tt - off[ja]);
            int64_t rowb = rowa;
            if (two) {
                const int jb = fsp::find_fact(off, nf, tt + 1);
                rowb = row0[jb] + (tt + 1 - off[jb]);
            }
            const int64_t sa = (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + tt;
            const uint4* ksa = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_k[l]) + rowa * row_elems);
            const uint4* vsa = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_v[l]) + rowa * row_elems);
            const uint4* ksb = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_k[l]) + rowb * row_elems);
            const uint4* vsb = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_v[l]) + rowb * row_elems);
            uint4* kda = reinterpret_cast<uint4*>(a.stage_k + sa * row_elems);
            uint4* vda = reinterpret_cast<uint4*>(a.stage_v + sa * row_elems);
            for (int o = lane; o < vec_per_row; o += 64) {
                const uint4 k0 = ksa[o], v0 = vsa[o];
                uint4 k1, v1;
                if (two) {
                    k1 = ksb[o];
                    v1 = vsb[o];
                }
                kda[o] = k0;
                vda[o] = v0;
                if (two) {
                    kda[row_elems / 8 + o] = k1;
                    vda[row_elems / 8 + o] = v1;
                }
            }
        }
    }
}

int layers_per_block(int nl, int64_t blocks_per_layer) {
    // enough blocks to fill 256 CUs several times over, while reusing each
    // block's plan over as many layers as possible
    int lpb = nl;
    while (lpb > 1 && blocks_per_layer * ((nl + lpb - 1) / lpb) < 4096) lpb = (lpb + 1) / 2;
    return lpb;
}

template <int D>
hipError_t launch_plan(const InjectLaunch& r, void* plan) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    PlanArgs pa{};
    pa.user = r.user;
    pa.ids = r.ids;
    pa.k = r.k;
    pa.batch = r.batch;
    pa.block_table = r.block_table;
    pa.max_blocks = r.max_blocks;
    pa.start_pos = r.start_pos;
    pa.num_blocks = r.num_blocks;
    pa.log2_block = st->log2_block;
    pa.fact_begin = st->d_fact_begin;
    pa.fact_len = st->d_fact_len;
    pa.user_begin = st->d_user_begin;
    pa.user_count = st->d_user_count;
    pa.num_users = d.num_users;
    pa.num_facts = d.num_facts;
    pa.layer_begin = r.layer_begin;
    pa.layer_end = r.layer_end;
    if (d.kv_location == FS_KV_PINNED_HOST) {
        pa.stage_ids = st->d_stage_ids;
        pa.stage_meta = st->d_stage_meta;
        pa.staging_layers = d.staging_layers;
    }
    pa.max_batch = d.max_batch;
    pa.max_k = d.max_k;
    pa.seg_tokens = st->seg_tokens;
    pa.tag = st->tag;
    pa.key = fsi_plan_key(st->tag, r.batch, r.k, st->seg_tokens, r.num_blocks);
    pa.out = fsi_plan_view(st, r.batch, plan);
    pa.err = st->d_err;
    const size_t plan_lds = sizeof(int64_t) * (size_t(r.k) + (size_t(r.k) + 2) / 2);
    fs_plan_kernel<<<dim3(r.batch), kPlanThreads, plan_lds, r.stream>>>(pa);
    return hipGetLastError();
}

// longest padded row the inject kernels are built for: 2^10 vectors (16 KB,
// e.g. 32 heads of 256 or 64 heads of 128)
constexpr int kFlatMaxLg = 10;
// launches expected to write at most this much store through the caches
constexpr double kCachedWriteBytes = 128.0 * (1 << 20);

template <int D, int kLg, bool kStaged, bool kCached>
void launch_flat_v(const FlatArgs& a, dim3 grid, hipStream_t s) {
    if constexpr (kLg >= 6) fs_row_kernel<D, kLg, kStaged, kCached><<<grid, kFlatThreads, 0, s>>>(a);
    else fs_short_kernel<D, kLg, kStaged, kCached><<<grid, kFlatThreads, 0, s>>>(a);
}

template <int D, int kLg>
void dispatch_flat(int lg, bool cached, const FlatArgs& a, dim3 grid, hipStream_t s) {
    if constexpr (kLg <= kFlatMaxLg) {
        if (lg != kLg) {
            dispatch_flat<D, kLg + 1>(lg, cached, a, grid, s);
        } else if (a.stage_k) {
            if (cached) launch_flat_v<D, kLg, true, true>(a, grid, s);
            else launch_flat_v<D, kLg, true, false>(a, grid, s);
        } else {
            if (cached) launch_flat_v<D, kLg, false, true>(a, grid, s);
            else launch_flat_v<D, kLg, false, false>(a, grid, s);
        }
    }
}

template <int D>
hipError_t launch_flat(const InjectLaunch& r, const void* plan) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    const PlanView v = fsi_plan_view(st, r.batch, plan);
    FlatArgs a{};
    a.hdr = v.hdr;
    a.req = v.req;
    a.tok = v.tok;
    a.key = fsi_plan_key(st->tag, r.batch, r.k, st->seg_tokens, r.num_blocks);
    a.src_kv = st->d_src_kv;
    a.inv_freq = st->d_inv_freq;
    a.row_elems = int64_t(d.num_kv_heads) * D;
    a.num_rows = d.num_tokens;
    a.cache_rows = int64_t(r.num_blocks) << st->log2_block;
    a.layer_begin = r.layer_begin;
    a.seg_tokens = st->seg_tokens;
    a.vpr = d.num_kv_heads * (D / 8);
    int lg = 0;
    while ((1 << lg) < a.vpr) ++lg;
    if (lg > kFlatMaxLg) return hipErrorInvalidValue;
    if (d.kv_location == FS_KV_PINNED_HOST) {
        a.stage_k = static_cast<const uint16_t*>(st->d_stage_k);
        a.stage_v = static_cast<const uint16_t*>(st->d_stage_v);
        a.staging_layers = d.staging_layers;
        a.stage_tokens = st->stage_tokens;
    }
    a.max_batch = d.max_batch;
    a.err = st->d_err;
    for (int l = 0; l < d.num_layers; ++l) {
        a.cache[2 * l] = r.k_cache[l];
        a.cache[2 * l + 1] = r.v_cache[l];
    }
    // units cover the longest possible segment of k facts (padded rows laid
    // end to end); a workgroup past its request's real length exits after
    // reading that length
    const int64_t seg = int64_t(r.k) * st->max_fact_len;
    // Stores: rows of a launch whose expected writes (k facts of the store's
    // mean length per request, K and V, every layer) fit in a half of the
    // 256 MB last-level cache go through the caches, and their write-back
    // overlaps what follows; larger launches stream past them.  On the
    // Qwen shape (86 MB) cached stores made the launch 4% faster, on the
    // Llama shape (195 MB) 8% slower.
    const double expect = double(r.k) * st->mean_fact_len * r.batch * (r.layer_end - r.layer_begin) * 2.0 *
                          double(a.row_elems) * 2.0;
    const bool cached = expect <= kCachedWriteBytes;
    const int64_t units = ((seg << lg) + kFlatThreads - 1) / kFlatThreads;
    if (units > INT32_MAX / 2) return hipErrorInvalidValue;
    a.units = static_cast<int32_t>(std::max<int64_t>(units, 1));
    const dim3 grid(static_cast<unsigned>(2 * a.units), static_cast<unsigned>(r.batch),
                    static_cast<unsigned>(r.layer_end - r.layer_begin));
    // a head is D/8 vectors, so rows start at 2^log2(D/8) vectors
    constexpr int kLg0 = D == 64 ? 3 : (D == 128 ? 4 : 5);
    dispatch_flat<D, kLg0>(lg, cached, a, grid, r.stream);
    return hipGetLastError();
}

template <int D>
hipError_t launch_inject(const InjectLaunch& r) {
    if (r.plan_out) {
        hipError_t e = launch_plan<D>(r, r.plan_out);
        if (e != hipSuccess || !r.inject) return e;
        return launch_flat<D>(r, r.plan_out);
    }
    return launch_flat<D>(r, r.plan_in);
}

template <int D>
hipError_t launch_fetch(const FetchLaunch& r) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    FetchArgs a{};
    a.user = r.user;
    a.ids = r.ids;
    a.k = r.k;
    a.fact_begin = st->d_fact_begin;
    a.fact_len = st->d_fact_len;
    a.user_begin = st->d_user_begin;
    a.user_count = st->d_user_count;
    a.num_users = d.num_users;
    a.num_facts = d.num_facts;
    a.heads = d.num_kv_heads;
    a.layer_begin = r.layer_begin;
    a.layer_end = r.layer_end;
    a.src_k = st->d_src_k;
    a.src_v = st->d_src_v;
    a.stage_k = static_cast<uint16_t*>(st->d_stage_k);
    a.stage_v = static_cast<uint16_t*>(st->d_stage_v);
    a.stage_ids = st->d_stage_ids;
    a.stage_meta = st->d_stage_meta;
    a.staging_layers = d.staging_layers;
    a.stage_tokens = st->stage_tokens;
    a.max_batch = d.max_batch;
    a.max_k = d.max_k;
    a.batch = r.batch;
    a.err = st->d_err;
    constexpr int kTok = kThreads / (D / 16);
    const int64_t max_tokens = int64_t(r.k) * st->max_fact_len;
    const int64_t tiles = (max_tokens + kTok - 1) / kTok;
    const int nl = r.layer_end - r.layer_begin;
    a.layers_per_block = layers_per_block(nl, tiles * r.batch);
    dim3 grid(static_cast<unsigned>(tiles), r.batch, (nl + a.layers_per_block - 1) / a.layers_per_block);
    size_t lds = sizeof(int64_t) * r.k + sizeof(int32_t) * (r.k + 1);
    fs_fetch_kernel<D><<<grid, kThreads, lds, r.stream>>>(a);
    return hipGetLastError();
}

}  // namespace

// The plan buffer of fs_inject_noalloc: FS_NOALLOC_PLAN_BYTES of device
// memory per GPU, in the code object (each device that loads the library holds
// its own copy until the process ends), so a call allocates nothing.  Host
// code never names the array: its device address comes from
// hipGetSymbolAddress, once per device with that device current.
static __device__ __align__(256) unsigned char scratch[FS_NOALLOC_PLAN_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t fsi_noalloc_scratch(int device, void** ptr, size_t* bytes) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != device) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *ptr = g_scratch_ptr[device];
    *bytes = sizeof(scratch);
    return hipSuccess;
}

hipError_t fsi_launch_inject(const InjectLaunch& r) {
    switch (r.st->desc.head_dim) {
        case 64: return launch_inject<64>(r);
        case 128: return launch_inject<128>(r);
        case 256: return launch_inject<256>(r);
        default: return hipErrorInvalidValue;
    }
}

hipError_t fsi_launch_fetch(const FetchLaunch& r) {
    switch (r.st->desc.head_dim) {
        case 64: return launch_fetch<64>(r);
        case 128: return launch_fetch<128>(r);
        case 256: return launch_fetch<256>(r);
        default: return hipErrorInvalidValue;
    }
}
