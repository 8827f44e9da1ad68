// Fused gather -> Chunked RoPE -> paged scatter, and the host-memory fetch.
//
// InferScale's online phase (gist.science summary, "Phase En-ligne"): keys
// are stored before RoPE; at serving time the retrieved facts are composed
// into one contiguous segment, every stored key is rotated to its new
// serving-time position, and the composed K/V is scatter-copied into the
// paged KV cache.  Values are copied raw.  The re-rotation is exact under
// RoPE (Theorem 6 as the pages describe it), so the kernel evaluates the
// rotation in fp64 and rounds once to bf16.
//
// Device stores: one fs_inject call is one launch of the inject kernel, one
// 256-thread block per (token group, request, layer).  Wave 0 plans the
// request in LDS (prefix sums of the selected facts' lengths, ids checked
// against the user) while the other waves evaluate cos/sin of p*w_i in fp64
// for every (token, frequency) of the group, one sincos per entry; the first
// K/V loads go out before the request's check (start position, block-table
// coverage and entries) completes, and a rejected request writes nothing.  A
// team of head_dim/16 lanes owns one token: lane tl holds the 8 rotate-half
// pairs i = 8*tl .. 8*tl+7 (one 16-byte vector from each half of the head
// row).  Each wave streams whole heads of the group: 4 non-temporal 16-byte
// loads per lane, rotation of K, 4 non-temporal stores.  Thousands of small
// blocks let the dispatcher keep every CU fed to the end of the launch (a
// persistent grid with equal shares per CU finished later: the CUs do not
// drain at the same rate).
//
// Pinned-host stores: a plan kernel (one block per request) validates each
// request, including that every layer's staging slot holds its ids, and
// writes a token map (arena row and cache slot of every segment token); the
// inject kernel then reads the staged rows through that map.  Device stores
// can take the same two steps with the map in a caller-owned plan
// (fs_plan_inject, fs_inject_planned): the injecting blocks then read their
// rows and slots instead of planning.  The fetch
// kernel fills the staging ring from host memory beforehand (fs_fetch_async),
// one wave per group of tokens, copying one whole token row per instruction
// pair so that the host link sees large contiguous reads.
//
// HBM-bound copy with a small amount of arithmetic; no dense contraction, so
// no MFMA.

#include <hip/hip_runtime.h>

#include <algorithm>

#include "fs_device.h"
#include "fs_internal.h"

namespace {

using fsd::bf16_hi;
using fsd::bf16_lo;
using fsd::f64_to_bf16_bits;
using fsd::wave_or;

constexpr int kThreads = 64;        // one wave per fetch block
constexpr int kInjectThreads = 256; // 4 waves per inject block
constexpr int kInjectOcc = 6;       // waves per SIMD the register budget allows
constexpr int kPlanThreads = 1024;

#define FS_GLOBAL __attribute__((address_space(1)))
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_stream(const FS_GLOBAL u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_stream(FS_GLOBAL u32x4* p, u32x4 v) { __builtin_nontemporal_store(v, p); }

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
    int32_t layer_begin, layer_end, heads;
    const int32_t* stage_ids;       // non-null for pinned stores
    const int32_t* stage_meta;
    int32_t staging_layers, max_batch, max_k;
    int32_t seg_tokens;
    int64_t* tok_src;
    int64_t* tok_dst;
    int32_t* req_len;
    int32_t* start_out;             // a caller-owned plan's copy of start_pos, or null
    uint32_t* err;
};

struct InjectArgs {
    const int32_t* start_pos;
    const int64_t* tok_src;
    const int64_t* tok_dst;
    const int32_t* req_len;
    int32_t seg_tokens;
    const double* inv_freq;         // [D/2] w_i
    int32_t heads;
    int32_t layer_begin;
    const void* const* src_k;       // device table [num_layers] (device store)
    const void* const* src_v;
    const uint16_t* stage_k;        // non-null: read the staging ring instead
    const uint16_t* stage_v;
    int32_t staging_layers, stage_tokens, max_batch;
    void* kc[FS_MAX_LAYERS];
    void* vc[FS_MAX_LAYERS];
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

// Segment plan of request b, shared by the block through LDS.
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
    // maps into a valid fact of the user even when the request is rejected
    // (the kernels may read before the verdict is in, never out of bounds).
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

__device__ __forceinline__ int find_fact(const int32_t* off, int nf, int t) {
    // largest j < nf with off[j] <= t (off is non-decreasing, off[0] = 0)
    int lo = 0, hi = nf - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ uint32_t rot_word(uint32_t wa, uint32_t wb, int e, const double* c,
                                             const double* s, uint32_t* out_b) {
    // two adjacent pairs: elements (2e, 2e+1) of this lane's first-half vector
    // and the same elements of its second-half vector
    const double a0 = bf16_lo(wa), a1 = bf16_hi(wa);
    const double b0 = bf16_lo(wb), b1 = bf16_hi(wb);
    const double y0 = fma(a0, c[2 * e], -(b0 * s[2 * e]));
    const double z0 = fma(b0, c[2 * e], a0 * s[2 * e]);
    const double y1 = fma(a1, c[2 * e + 1], -(b1 * s[2 * e + 1]));
    const double z1 = fma(b1, c[2 * e + 1], a1 * s[2 * e + 1]);
    *out_b = f64_to_bf16_bits(z0) | (f64_to_bf16_bits(z1) << 16);
    return f64_to_bf16_bits(y0) | (f64_to_bf16_bits(y1) << 16);
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

__device__ __forceinline__ void rot_v(const u32x4& xa, const u32x4& xb, const double* c,
                                      const double* s, u32x4& ya, u32x4& yb) {
    uint32_t b0, b1, b2, b3;
    ya.x = rot_word(xa.x, xb.x, 0, c, s, &b0);
    ya.y = rot_word(xa.y, xb.y, 1, c, s, &b1);
    ya.z = rot_word(xa.z, xb.z, 2, c, s, &b2);
    ya.w = rot_word(xa.w, xb.w, 3, c, s, &b3);
    yb.x = b0;
    yb.y = b1;
    yb.z = b2;
    yb.w = b3;
}

// Validation of one planned request, shared by the plan kernel and the
// single-request inject path: start position, block-table coverage and
// entries, and for pinned stores that every staging slot holds these ids.
__device__ uint32_t check_request(const PlanArgs& a, int b, int L) {
    const int lane = threadIdx.x & 63;
    uint32_t bits = 0;
    const int s = a.start_pos[b];
    const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
    if (s < 0 || int64_t(s) + L > int64_t(INT32_MAX)) {
        bits |= FS_ERR_START_POS;
    } else if (L > 0) {
        const int first = s >> a.log2_block;
        const int last = (s + L - 1) >> a.log2_block;
        if (last >= a.max_blocks) {
            bits |= FS_ERR_BLOCK_SHORT;
        } else {
            // four entries per lane in flight at a time (indices clamped to
            // the range, so the loads need no branch and no wait between them)
            for (int j0 = first + lane; j0 <= last; j0 += 256) {
                int e[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) e[q] = bt[min(j0 + 64 * q, last)];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (j0 + 64 * q <= last && (e[q] < 0 || e[q] >= a.num_blocks)) bits |= FS_ERR_BLOCK_ID;
            }
        }
    }
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

// Batches: one block per request.  Wave 0 plans into LDS, then the whole
// block writes the token map; a rejected request gets length 0.
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
            a.req_len[b] = bits ? 0 : L;
            if (a.start_out) a.start_out[b] = a.start_pos[b];
        }
    }
    __syncthreads();
    const int L = s_len, nf = s_nf;
    const int s = a.start_pos[b];
    const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
    const int bs_mask = (1 << a.log2_block) - 1;
    int64_t* src = a.tok_src + int64_t(b) * a.seg_tokens;
    int64_t* dst = a.tok_dst + int64_t(b) * a.seg_tokens;
    for (int t = threadIdx.x; t < L; t += blockDim.x) {
        const int j = find_fact(off, nf, t);
        src[t] = row0[j] + (t - off[j]);
        const int p = s + t;
        dst[t] = (int64_t(bt[p >> a.log2_block]) << a.log2_block) | (p & bs_mask);
    }
}

// One block per (token group g, request b, layer l).  The group's tokens are
// t = g*kTok + team.
//
// kPlanned = false (device stores): the block plans its request itself.  Wave 0
// reads the ids and prefix-sums the fact lengths into LDS while the other
// waves fill the cos/sin table.  After the first barrier every lane locates
// its token's arena row and cache slot and issues its first loads, while wave
// 0 validates the whole request (so a rejected request writes nothing in any
// block); the second barrier publishes the verdict before any store.  Reads
// before the verdict stay in bounds: the plan counts only valid facts of the
// user, and block-table reads are range-checked.  No launch is spent on
// planning.
//
// kPlanned = true (pinned stores): the plan kernel has validated the request
// (including every layer's staging slot) and written the token map.
template <int D, bool kPlanned>
__global__ __launch_bounds__(kInjectThreads, kInjectOcc) void fs_inject_kernel(InjectArgs a, PlanArgs pa) {
    constexpr int kTeam = D / 16;            // lanes per token
    constexpr int kTok = 64 / kTeam;         // tokens per group
    constexpr int kHalf = D / 16;            // 16-byte vectors per half head row
    constexpr int kCS = kTok * (D / 2);      // (cos, sin) entries of the group
    constexpr int kWaves = kInjectThreads / 64;
    __shared__ double2 s_cs[kCS];
    __shared__ int s_L, s_nf, s_bits;
    extern __shared__ int64_t plan_lds[];
    int64_t* row0 = plan_lds;
    int32_t* off = reinterpret_cast<int32_t*>(plan_lds + pa.k);
    const int b = blockIdx.y;
    const int g = blockIdx.x;
    const int l = a.layer_begin + blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int team = lane / kTeam;
    const int tl = lane % kTeam;
    const int t = g * kTok + team;
    const int64_t p0 = int64_t(a.start_pos[b]) + int64_t(g) * kTok;
    const bool reporter = !kPlanned && g == 0 && blockIdx.z == 0;

    int L;
    int64_t src_row = 0, dst_row = 0;
    if (kPlanned) {
        L = a.req_len[b];
        if (g * kTok >= L) return;           // uniform over the block
        if (t < L) {
            src_row = a.tok_src[int64_t(b) * a.seg_tokens + t];
            dst_row = a.tok_dst[int64_t(b) * a.seg_tokens + t];
        }
    } else if (wave == 0) {
        int Lr = 0, nf = 0;
        const uint32_t bits = plan_request(pa.user, pa.ids, pa.k, pa.user_begin, pa.user_count, pa.num_users, pa.num_facts,
                                           pa.fact_len, pa.fact_begin, b, off, row0, &Lr, &nf);
        const uint32_t any = wave_or(bits);
        if (lane == 0) {
            s_L = Lr;
            s_nf = nf;
            s_bits = any;
        }
    }
    constexpr int kCsBegin = kPlanned ? 0 : 64;             // threads filling the table
    constexpr int kCsStride = kInjectThreads - kCsBegin;
    // when the stride is a multiple of D/2 a thread meets one frequency only:
    // it is loaded once, not before every sincos
    constexpr bool kOneFreq = kCsStride % (D / 2) == 0;
    if (kPlanned || wave > 0) {
        const double w_own = kOneFreq ? a.inv_freq[(threadIdx.x - kCsBegin) % (D / 2)] : 0.0;
        for (int e = threadIdx.x - kCsBegin; e < kCS; e += kCsStride) {
            const int tt = e / (D / 2);
            const int i = e - tt * (D / 2);
            double sv, cv;
            sincos(static_cast<double>(p0 + tt) * (kOneFreq ? w_own : a.inv_freq[i]), &sv, &cv);
            s_cs[e] = make_double2(cv, sv);
        }
    }
    if (!kPlanned) {
        __syncthreads();                     // plan in LDS
        L = s_L;
        if (g * kTok >= L && !reporter) return;   // uniform over the block
        if (t < L) {
            const int j = find_fact(off, s_nf, t);
            src_row = row0[j] + (t - off[j]);
        }
    }
    const bool act = t < L;
    const int H = a.heads;
    const int64_t row_elems = int64_t(H) * D;
    const FS_GLOBAL u32x4* kbase;
    const FS_GLOBAL u32x4* vbase;
    if (a.stage_k) {
        const int64_t srow = (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + t;
        kbase = (const FS_GLOBAL u32x4*)(a.stage_k + srow * row_elems);
        vbase = (const FS_GLOBAL u32x4*)(a.stage_v + srow * row_elems);
    } else {
        kbase = (const FS_GLOBAL u32x4*)(static_cast<const uint16_t*>(a.src_k[l]) + src_row * row_elems);
        vbase = (const FS_GLOBAL u32x4*)(static_cast<const uint16_t*>(a.src_v[l]) + src_row * row_elems);
    }
    u32x4 ka, kb, va, vb;
    auto load_head = [&](int h) {
        if (act && h < H) {
            const int o = h * (D / 8) + tl;
            ka = ld_stream(kbase + o);
            kb = ld_stream(kbase + o + kHalf);
            va = ld_stream(vbase + o);
            vb = ld_stream(vbase + o + kHalf);
        }
    };
    load_head(wave);                         // in flight across the barrier
    // the token's cache slot: its block-table entry is read after the K/V
    // loads are out, by every thread (index clamped in range, so no branch
    // forces a wait on it here; a bad entry or a short table rejects the
    // request below, before any store)
    int blk_raw = 0;
    const int64_t p_tok = p0 + team;
    const int64_t bi_tok = p_tok >> pa.log2_block;
    if (!kPlanned)
        blk_raw = pa.block_table[int64_t(b) * pa.max_blocks +
                                 (p_tok >= 0 && bi_tok < pa.max_blocks ? bi_tok : 0)];
    if (!kPlanned && wave == 0) {
        const uint32_t bits = wave_or(check_request(pa, b, L)) | s_bits;
        if (lane == 0) {
            s_bits = bits;
            if (bits && reporter) atomicOr(pa.err, bits);
        }
    }
    __syncthreads();                         // reached by every thread still here
    if (!kPlanned && s_bits) return;
    if (!act) return;
    if (!kPlanned) dst_row = (int64_t(blk_raw) << pa.log2_block) | (p_tok & ((1 << pa.log2_block) - 1));
    FS_GLOBAL u32x4* kd = (FS_GLOBAL u32x4*)(static_cast<uint16_t*>(a.kc[l]) + dst_row * row_elems);
    FS_GLOBAL u32x4* vd = (FS_GLOBAL u32x4*)(static_cast<uint16_t*>(a.vc[l]) + dst_row * row_elems);
    double c[8], sn[8];
    const double2* cs = s_cs + team * (D / 2) + 8 * tl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const double2 v = cs[e];
        c[e] = v.x;
        sn[e] = v.y;
    }
    for (int h = wave; h < H; h += kWaves) {
        if (h != wave) load_head(h);
        const int o = h * (D / 8) + tl;
        u32x4 ya, yb;
        rot_v(ka, kb, c, sn, ya, yb);
        st_stream(kd + o, ya);
        st_stream(kd + o + kHalf, yb);
        st_stream(vd + o, va);
        st_stream(vd + o + kHalf, vb);
    }
}

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
            const int ja = find_fact(off, nf, tt);
            const int64_t rowa = row0[ja] + (tt - off[ja]);
            int64_t rowb = rowa;
            if (two) {
                const int jb = find_fact(off, nf, tt + 1);
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
    // team's cos/sin over as many layers as possible
    int lpb = nl;
    while (lpb > 1 && blocks_per_layer * ((nl + lpb - 1) / lpb) < 4096) lpb = (lpb + 1) / 2;
    return lpb;
}

template <int D>
hipError_t launch_inject(const InjectLaunch& r) {
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
    pa.heads = d.num_kv_heads;
    if (d.kv_location == FS_KV_PINNED_HOST) {
        pa.stage_ids = st->d_stage_ids;
        pa.stage_meta = st->d_stage_meta;
        pa.staging_layers = d.staging_layers;
    }
    pa.max_batch = d.max_batch;
    pa.max_k = d.max_k;
    pa.seg_tokens = st->seg_tokens;
    pa.tok_src = st->d_tok_src;
    pa.tok_dst = st->d_tok_dst;
    pa.req_len = st->d_req_len;
    pa.err = st->d_err;
    const size_t plan_lds = sizeof(int64_t) * (size_t(r.k) + (size_t(r.k) + 2) / 2);
    if (r.plan_out) {
        // compose and validate into the caller's plan, nothing else
        const PlanView v = fsi_plan_view(st, r.batch, r.plan_out);
        pa.tok_src = v.tok_src;
        pa.tok_dst = v.tok_dst;
        pa.req_len = v.req_len;
        pa.start_out = v.start;
        fs_plan_kernel<<<dim3(r.batch), kPlanThreads, plan_lds, r.stream>>>(pa);
        return hipGetLastError();
    }

    InjectArgs a{};
    a.start_pos = r.start_pos;
    a.tok_src = st->d_tok_src;
    a.tok_dst = st->d_tok_dst;
    a.req_len = st->d_req_len;
    a.seg_tokens = st->seg_tokens;
    a.inv_freq = st->d_inv_freq;
    a.heads = d.num_kv_heads;
    a.layer_begin = r.layer_begin;
    a.src_k = st->d_src_k;
    a.src_v = st->d_src_v;
    if (d.kv_location == FS_KV_PINNED_HOST) {
        a.stage_k = static_cast<const uint16_t*>(st->d_stage_k);
        a.stage_v = static_cast<const uint16_t*>(st->d_stage_v);
        a.staging_layers = d.staging_layers;
        a.stage_tokens = st->stage_tokens;
    }
    a.max_batch = d.max_batch;
    for (int l = 0; l < d.num_layers; ++l) {
        a.kc[l] = r.k_cache[l];
        a.vc[l] = r.v_cache[l];
    }
    // token groups of the longest possible segment (at least one, which
    // reports the request's errors); the blocks past a request's real length
    // exit once its length is known
    constexpr int kTok = 64 / (D / 16);
    const int64_t groups = std::max<int64_t>(1, (int64_t(r.k) * st->max_fact_len + kTok - 1) / kTok);
    const dim3 grid(static_cast<unsigned>(groups), static_cast<unsigned>(r.batch),
                    static_cast<unsigned>(r.layer_end - r.layer_begin));
    if (r.plan_in) {
        // inject from the caller's plan: the blocks read their tokens' rows
        // and slots instead of planning
        const PlanView v = fsi_plan_view(st, r.batch, r.plan_in);
        a.start_pos = v.start;
        a.tok_src = v.tok_src;
        a.tok_dst = v.tok_dst;
        a.req_len = v.req_len;
        fs_inject_kernel<D, true><<<grid, kInjectThreads, 0, r.stream>>>(a, pa);
    } else if (d.kv_location == FS_KV_PINNED_HOST) {
        fs_plan_kernel<<<dim3(r.batch), kPlanThreads, plan_lds, r.stream>>>(pa);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        fs_inject_kernel<D, true><<<grid, kInjectThreads, 0, r.stream>>>(a, pa);
    } else {
        fs_inject_kernel<D, false><<<grid, kInjectThreads, plan_lds, r.stream>>>(a, pa);
    }
    return hipGetLastError();
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
