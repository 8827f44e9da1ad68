// Fused gather -> Chunked RoPE -> paged scatter, and the host-memory fetch.
//
// InferScale's online phase (gist.science summary, "Phase En-ligne"): keys
// are stored before RoPE; at serving time the retrieved facts are composed
// into one contiguous segment, every stored key is rotated to its new
// serving-time position, and the composed K/V is scatter-copied into the
// paged KV cache.  Values are copied raw.  The re-rotation is exact under
// RoPE (Theorem 6 as the pages describe it), so this kernel evaluates the
// rotation in fp64 and rounds once to bf16.
//
// Work decomposition (HBM-bound copy with a small amount of arithmetic; no
// dense contraction, so no MFMA):
//   block = one wave (64 threads); grid = (token tiles, request, layer chunk)
//   team  = head_dim/16 lanes per segment token; lane `tl` of a team owns the
//           8 rotate-half pairs i = 8*tl .. 8*tl+7 (elements i and i + D/2),
//           i.e. one 16-byte vector from each half of a head row
//   a team computes cos/sin of p*w_i for its 8 frequencies ONCE (fp64) and
//   reuses them for every head of every layer in its chunk.
//   Per (layer, head): two 16-byte loads of K, two of V, two 16-byte stores
//   of each — rows are 2*head_dim bytes, read and written whole by the team.
//
// Every block first plans its request (prefix sums of the selected facts'
// lengths, validation of ids, start position and the used block-table
// entries).  A request that fails any check writes nothing; the first block
// of the request records the reason in the store's error word.

#include <hip/hip_runtime.h>

#include "fs_internal.h"

namespace {

constexpr int kThreads = 64;   // one wave per block

struct InjectArgs {
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    const int32_t* block_table;
    int32_t max_blocks;
    const int32_t* start_pos;
    int32_t num_blocks;
    int32_t log2_block;
    const int64_t* fact_begin;
    const int32_t* fact_len;
    const int64_t* user_begin;
    int32_t num_users;
    const double* inv_freq;
    int32_t heads;
    int32_t layer_begin, layer_end, layers_per_block;
    const void* const* src_k;       // device table [num_layers] (device store)
    const void* const* src_v;
    const uint16_t* stage_k;        // non-null: read the staging ring instead
    const uint16_t* stage_v;
    const int32_t* stage_ids;       // [staging_layers][max_batch][max_k]
    const int32_t* stage_meta;      // [staging_layers][4]: k, batch, layer
    int32_t staging_layers, stage_tokens, max_batch, max_k;
    uint32_t* err;
    void* kc[FS_MAX_LAYERS];
    void* vc[FS_MAX_LAYERS];
};

struct FetchArgs {
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    const int64_t* fact_begin;
    const int32_t* fact_len;
    const int64_t* user_begin;
    int32_t num_users;
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

__device__ __forceinline__ int wave_or(int v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, 64);
    return v;
}
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
                                 const int64_t* user_begin, int num_users,
                                 const int32_t* fact_len, const int64_t* fact_begin, int b,
                                 int32_t* off, int64_t* row0, int* L_out, int* nf_out) {
    const int lane = threadIdx.x;
    uint32_t bits = 0;
    const int u = user[b];
    const bool bad_user = (u < 0 || u >= num_users);
    if (bad_user) bits |= FS_ERR_USER;
    const int64_t ub0 = bad_user ? 0 : user_begin[u];
    const int64_t ub1 = bad_user ? 0 : user_begin[u + 1];
    int carry = 0, first_pad = k, last_real = -1;
    for (int c0 = 0; c0 < k; c0 += 64) {
        const int j = c0 + lane;
        int len = 0;
        int64_t r0 = 0;
        if (j < k) {
            const int id = ids[int64_t(b) * k + j];
            if (id < 0) {
                first_pad = min(first_pad, j);
            } else {
                last_real = j;
                if (bad_user) {
                    // reported once as FS_ERR_USER; ids cannot be judged
                } else if (id < ub0 || id >= ub1) {
                    bits |= FS_ERR_FACT_ID;
                } else {
                    len = fact_len[id];
                    r0 = fact_begin[id];
                }
            }
        }
        const int incl = wave_incl_scan(len, lane);
        if (j < k) {
            off[j] = carry + incl - len;
            row0[j] = r0;
        }
        carry += __shfl(incl, 63, 64);
    }
    first_pad = wave_min(first_pad);
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

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round an fp64 value to the nearest bf16, ties to even, without double
// rounding: narrow to fp32 with round-to-odd (Boldo & Melquiond, "Emulation of
// FMA and correctly rounded sums: proved algorithms using rounding to odd",
// IEEE Trans. Computers 2008: an intermediate format with >= 2 more bits,
// rounded to odd, makes the final round-to-nearest correct), then round the
// fp32 bits to 16 bits to nearest-even.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double y) {
    const float f = static_cast<float>(y);
    uint32_t u = __float_as_uint(f);
    const double back = static_cast<double>(f);
    if (back != y) {
        if (fabs(back) > fabs(y)) u -= 1u;   // rounded away from zero: step back
        u |= 1u;                             // sticky bit: round-to-odd
    }
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
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

__device__ __forceinline__ void rotate16(const uint4& xa, const uint4& xb, const double* c,
                                         const double* s, uint4& ya, uint4& yb) {
    ya.x = rot_word(xa.x, xb.x, 0, c, s, &yb.x);
    ya.y = rot_word(xa.y, xb.y, 1, c, s, &yb.y);
    ya.z = rot_word(xa.z, xb.z, 2, c, s, &yb.z);
    ya.w = rot_word(xa.w, xb.w, 3, c, s, &yb.w);
}

template <int D>
__global__ __launch_bounds__(kThreads) void fs_inject_kernel(InjectArgs a) {
    constexpr int kTeam = D / 16;            // lanes per token
    constexpr int kTok = kThreads / kTeam;   // tokens per block
    constexpr int kHalf = D / 16;            // uint4 per half head row
    extern __shared__ int64_t plan_lds[];
    int64_t* row0 = plan_lds;
    int32_t* off = reinterpret_cast<int32_t*>(plan_lds + a.k);

    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    int L = 0, nf = 0;
    uint32_t bits = plan_request(a.user, a.ids, a.k, a.user_begin, a.num_users, a.fact_len,
                                 a.fact_begin, b, off, row0, &L, &nf);
    const int s = a.start_pos[b];
    if (s < 0 || int64_t(s) + L > int64_t(INT32_MAX)) bits |= FS_ERR_START_POS;
    const int bs_mask = (1 << a.log2_block) - 1;
    if (!(bits & FS_ERR_START_POS) && L > 0) {
        const int first = s >> a.log2_block;
        const int last = (s + L - 1) >> a.log2_block;
        if (last >= a.max_blocks) {
            bits |= FS_ERR_BLOCK_SHORT;
        } else {
            const int32_t* bt = a.block_table + int64_t(b) * a.max_blocks;
            for (int j = first + lane; j <= last; j += 64) {
                const int e = bt[j];
                if (e < 0 || e >= a.num_blocks) bits |= FS_ERR_BLOCK_ID;
            }
        }
    }
    if (a.stage_k) {
        for (int l = a.layer_begin + blockIdx.z * a.layers_per_block;
             l < min(a.layer_end, a.layer_begin + (int(blockIdx.z) + 1) * a.layers_per_block); ++l) {
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
    bits = wave_or(bits);
    if (bits) {
        if (lane == 0 && blockIdx.x == 0 && blockIdx.z == 0) atomicOr(a.err, bits);
        return;
    }
    __syncthreads();   // plan in LDS visible to every lane

    const int team = lane / kTeam;
    const int tl = lane % kTeam;
    const int t = blockIdx.x * kTok + team;
    if (t >= L) return;
    const int j = find_fact(off, nf, t);
    const int64_t row = row0[j] + (t - off[j]);
    const int p = s + t;
    const int blk = a.block_table[int64_t(b) * a.max_blocks + (p >> a.log2_block)];
    const int64_t dst_row = (int64_t(blk) << a.log2_block) | (p & bs_mask);

    double c[8], sn[8];
    const double pd = static_cast<double>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) sincos(pd * a.inv_freq[8 * tl + e], &sn[e], &c[e]);

    const int H = a.heads;
    const int64_t row_elems = int64_t(H) * D;
    const int l0 = a.layer_begin + blockIdx.z * a.layers_per_block;
    const int l1 = min(a.layer_end, l0 + a.layers_per_block);
    for (int l = l0; l < l1; ++l) {
        const uint4* ks;
        const uint4* vs;
        if (a.stage_k) {
            const int64_t srow = (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + t;
            ks = reinterpret_cast<const uint4*>(a.stage_k + srow * row_elems);
            vs = reinterpret_cast<const uint4*>(a.stage_v + srow * row_elems);
        } else {
            ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_k[l]) + row * row_elems);
            vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_v[l]) + row * row_elems);
        }
        uint4* kd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.kc[l]) + dst_row * row_elems);
        uint4* vd = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.vc[l]) + dst_row * row_elems);
        int h = 0;
        for (; h + 2 <= H; h += 2) {
            const int o0 = h * (D / 8) + tl, o1 = o0 + D / 8;
            const uint4 xa0 = ks[o0], xb0 = ks[o0 + kHalf];
            const uint4 xa1 = ks[o1], xb1 = ks[o1 + kHalf];
            const uint4 va0 = vs[o0], vb0 = vs[o0 + kHalf];
            const uint4 va1 = vs[o1], vb1 = vs[o1 + kHalf];
            uint4 ya0, yb0, ya1, yb1;
            rotate16(xa0, xb0, c, sn, ya0, yb0);
            rotate16(xa1, xb1, c, sn, ya1, yb1);
            kd[o0] = ya0;
            kd[o0 + kHalf] = yb0;
            kd[o1] = ya1;
            kd[o1 + kHalf] = yb1;
            vd[o0] = va0;
            vd[o0 + kHalf] = vb0;
            vd[o1] = va1;
            vd[o1 + kHalf] = vb1;
        }
        for (; h < H; ++h) {
            const int o0 = h * (D / 8) + tl;
            const uint4 xa0 = ks[o0], xb0 = ks[o0 + kHalf];
            const uint4 va0 = vs[o0], vb0 = vs[o0 + kHalf];
            uint4 ya0, yb0;
            rotate16(xa0, xb0, c, sn, ya0, yb0);
            kd[o0] = ya0;
            kd[o0 + kHalf] = yb0;
            vd[o0] = va0;
            vd[o0 + kHalf] = vb0;
        }
    }
}

template <int D>
__global__ __launch_bounds__(kThreads) void fs_fetch_kernel(FetchArgs a) {
    constexpr int kTeam = D / 16;
    constexpr int kTok = kThreads / kTeam;
    extern __shared__ int64_t plan_lds[];
    int64_t* row0 = plan_lds;
    int32_t* off = reinterpret_cast<int32_t*>(plan_lds + a.k);

    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    int L = 0, nf = 0;
    uint32_t bits = plan_request(a.user, a.ids, a.k, a.user_begin, a.num_users, a.fact_len,
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

    const int team = lane / kTeam;
    const int tl = lane % kTeam;
    const int t = blockIdx.x * kTok + team;
    if (t >= L) return;
    const int j = find_fact(off, nf, t);
    const int64_t row = row0[j] + (t - off[j]);
    const int64_t row_elems = int64_t(a.heads) * D;
    const int vec_per_row = a.heads * (D / 8);
    for (int l = l0; l < l1; ++l) {
        const int64_t srow = (int64_t(l % a.staging_layers) * a.max_batch + b) * a.stage_tokens + t;
        const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_k[l]) + row * row_elems);
        const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.src_v[l]) + row * row_elems);
        uint4* kd = reinterpret_cast<uint4*>(a.stage_k + srow * row_elems);
        uint4* vd = reinterpret_cast<uint4*>(a.stage_v + srow * row_elems);
        int o = tl;
        for (; o + kTeam < vec_per_row; o += 2 * kTeam) {
            const uint4 k0 = ks[o], k1 = ks[o + kTeam];
            const uint4 v0 = vs[o], v1 = vs[o + kTeam];
            kd[o] = k0;
            kd[o + kTeam] = k1;
            vd[o] = v0;
            vd[o + kTeam] = v1;
        }
        for (; o < vec_per_row; o += kTeam) {
            kd[o] = ks[o];
            vd[o] = vs[o];
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
    InjectArgs a{};
    a.user = r.user;
    a.ids = r.ids;
    a.k = r.k;
    a.block_table = r.block_table;
    a.max_blocks = r.max_blocks;
    a.start_pos = r.start_pos;
    a.num_blocks = r.num_blocks;
    a.log2_block = st->log2_block;
    a.fact_begin = st->d_fact_begin;
    a.fact_len = st->d_fact_len;
    a.user_begin = st->d_user_begin;
    a.num_users = d.num_users;
    a.inv_freq = st->d_inv_freq;
    a.heads = d.num_kv_heads;
    a.layer_begin = r.layer_begin;
    a.layer_end = r.layer_end;
    a.src_k = st->d_src_k;
    a.src_v = st->d_src_v;
    if (d.kv_location == FS_KV_PINNED_HOST) {
        a.stage_k = static_cast<const uint16_t*>(st->d_stage_k);
        a.stage_v = static_cast<const uint16_t*>(st->d_stage_v);
        a.stage_ids = st->d_stage_ids;
        a.stage_meta = st->d_stage_meta;
        a.staging_layers = d.staging_layers;
        a.stage_tokens = st->stage_tokens;
    }
    a.max_batch = d.max_batch;
    a.max_k = d.max_k;
    a.err = st->d_err;
    for (int l = 0; l < d.num_layers; ++l) {
        a.kc[l] = r.k_cache[l];
        a.vc[l] = r.v_cache[l];
    }
    constexpr int kTok = kThreads / (D / 16);
    const int64_t max_tokens = int64_t(r.k) * st->max_fact_len;
    const int64_t tiles = (max_tokens + kTok - 1) / kTok;
    const int nl = r.layer_end - r.layer_begin;
    a.layers_per_block = layers_per_block(nl, tiles * r.batch);
    dim3 grid(static_cast<unsigned>(tiles), r.batch, (nl + a.layers_per_block - 1) / a.layers_per_block);
    size_t lds = sizeof(int64_t) * r.k + sizeof(int32_t) * (r.k + 1);
    fs_inject_kernel<D><<<grid, kThreads, lds, r.stream>>>(a);
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
    a.num_users = d.num_users;
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
