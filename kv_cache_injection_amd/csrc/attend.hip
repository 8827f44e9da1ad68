// Attention read of the injected cache: causal prefill of a request's own
// tokens over one layer's paged K/V cache.
//
// InferScale's retrieve-and-inject inference rests on Theorem 3 as the pages
// describe it (gist.science summary, "Contributions Clés"): for a causal
// decoder, attention over KV states injected at the intended positions equals
// attention over the same memory given as prompt.  This kernel is that read:
// query token j of request b sits at position q_pos[b] + j and attends to
// every cache position p with ctx_begin[b] <= p <= q_pos[b] + j, through the
// same block table the injection wrote with.  The caller has written the query
// tokens' own K/V at their positions (as an engine's prefill does).
//
// Queries arrive before RoPE; the kernel rotates them (rotate-half,
// w_i = theta^(-2i/D)) in fp64 and rounds once to bf16, as the injection does
// for keys, so Q and K carry the same rounding.
//
// One block = one KV head and 16 or 32 query tokens (all the query heads of
// its GQA group): for groups up to 4 and more than 16 tokens, two 16-token
// sub-tiles with two heads per wave; otherwise 16 tokens with one head per
// wave, two per wave for groups of 5..8.  Scores and P.V run
// on the matrix cores (gfx950 16x16x32 bf16 MFMA, fp32 accumulation);
// softmax is online in fp32 (exp2); the weights are rounded to bf16 for P.V
// and summed unrounded for the normaliser.  Both products are computed transposed,
// S^T = K Q^T and O^T += V^T P^T: a lane's scores are then exactly the P^T
// entries it supplies, and the O^T column it accumulates is the query whose
// softmax state it holds, so rescaling and normalising need no shuffles; only
// the running maximum is reduced across lanes (lane-swap moves), once per 64
// positions.  The maximum is raised only when a column's grows by more than
// 2^8, so unnormalised weights stay below 256 and O is rescaled on few
// tiles; the masked pass runs only on tiles that cross the diagonal.  The
// contraction index of P.V maps to positions in the order the score tiles
// produce them (any order works if both operands agree).  K/V tiles of 64
// positions go from global memory straight into LDS (gfx950's direct loads,
// no registers or LDS stores on the way), row-major with swizzled 16-byte
// chunks, into two buffers: the next tile lands in one while the current one
// is consumed from the other, with one barrier per tile.  The V^T operand
// comes from gfx950's transposing LDS reads.  A block's raw Q and first K/V
// tile are loaded before anything else (the block-table entries of that tile
// are range-checked where they are read), so their latency overlaps the
// request check and the (cos, sin) table.  Long contexts are split over
// several blocks whose partial results a second kernel merges.

#include <hip/hip_runtime.h>

#include "fs_device.h"
#include "fs_internal.h"

namespace {

using fsd::f64_to_bf16_bits;
using fsd::wave_or;

constexpr int kD = 128;               // head dim handled
constexpr int kQT = 16;               // query tokens per block
constexpr int kKT = 64;               // cache positions per tile
constexpr int kThreads = 256;         // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kRowB = kD * 2;         // one K or V row in LDS: 256 bytes, unpadded
constexpr int kHalfB = kKT * kRowB;   // the K (or V) half of a tile buffer
constexpr int kBufB = 2 * kHalfB;     // one tile buffer, K then V
// The direct loads fill 1 KB (four rows) per wave instruction, so rows cannot
// be padded; 16-byte chunks are XOR-swizzled within a row instead.  K chunk c
// of row r sits in slot c ^ (r & 15): the 16 rows a score fragment reads hit
// 16 different slots.  V chunk c sits in slot c ^ 2(r & 7): the 8 rows of a
// half-wave's transposing reads hit 8 different slot pairs.
__device__ __forceinline__ int k_slot(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_slot(int r, int c) { return c ^ ((r & 7) << 1); }

typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

struct AttendArgs {
    const uint16_t* q;                // [B][Tq][Hq][D] bf16, before RoPE
    int32_t tq, hq, hkv, group;
    const uint16_t* kc;               // [NB][bs][Hkv][D] bf16
    const uint16_t* vc;
    int32_t num_blocks, log2_block, max_blocks;
    const int32_t* bt;                // [B][max_blocks]
    const int32_t* ctx_begin;         // [B]
    const int32_t* q_pos;             // [B]
    const double* inv_freq;           // [D/2]
    const void* zero_row;             // 256+ bytes of zeros
    float scale_log2;                 // softmax scale * log2(e)
    float* out;                       // [B][Tq][Hq][D] fp32
    uint32_t* err;
    int32_t splits;                   // context split into this many ranges (1: no workspace)
    float* part_o;                    // [splits][B][Tq][Hq][D] unnormalised partial outputs
    float2* part_ml;                  // [splits][B][Tq][Hq] (running max, weight sum)
};

constexpr int kBtCache = 1024;        // block-table entries a block caches in LDS
constexpr unsigned kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), other counters untouched
constexpr int kMaxSplits = 16;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

__device__ __forceinline__ __bf16 as_bf16(uint16_t h) {
    __bf16 r;
    __builtin_memcpy(&r, &h, 2);
    return r;
}

typedef short s4 __attribute__((ext_vector_type(4)));

// maximum over the four lanes l, l^16, l^32, l^48 (the rows of one S^T
// column), by gfx950's lane-swap moves instead of LDS permutes: the first
// swap pairs 16-lane rows 0-1 and 2-3, the second the two halves
__device__ __forceinline__ float colmax(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// the running maximum (log2 units) is raised only when a tile's exceeds it
// by more than this, so unnormalised weights stay below 2^kLazy
constexpr float kLazy = 8.0f;

// gfx950's transposing LDS read (ds_read_b64_tr_b16): each group of 16 lanes
// supplies 16 chunks of 4 consecutive 16-bit values, R[c][0..3] at lane c's
// address, and lane i receives R[i/4 + 4e][i % 4] for e = 0..3.  When lane c
// points at V[p0 + c/4][d0 + 4*(c%4)], lane i receives V[p0 + e][d0 + i]:
// four consecutive positions of column d0 + i.  Two reads, 16 positions
// apart, give the 8 positions of one lane's A = V^T fragment.
__device__ __forceinline__ b8 tr_v(const uint16_t* p, int second) {
    const s4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p));
    const s4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4*)(p + second));
    struct { s4 a, b; } v{lo, hi};
    return __builtin_bit_cast(b8, v);
}

// kQS sub-tiles of 16 query tokens per block; the 4 waves form kQS teams of
// kWaves / kQS waves, team qs covering sub-tile qs.  Wave hb of a team holds
// the query heads hb, hb + kWaves / kQS, ... (kHS head slots): a team covers
// the whole GQA group when group <= kHS * kWaves / kQS.  A wave's head slots
// share every K and V fragment it reads from LDS.
template <int kHS, int kQS>
// Two tile buffers (64 KB) and the block-table cache hold two blocks per CU.
__global__ __launch_bounds__(kThreads, 2) void fs_attend_kernel(AttendArgs a) {
    constexpr int kWQ = kWaves / kQS;     // waves per team
    constexpr int kBQ = kQT * kQS;        // query tokens per block
    // the fp64 (cos, sin) table of the block's queries is only needed before
    // the first tile, so it shares storage with the K/V tiles
    constexpr int kCSBytes = kBQ * (kD / 2) * 16;
    static_assert(kCSBytes <= kBufB, "the (cos, sin) table fits one tile buffer");
    // two tile buffers as separate objects: the compiler then knows that
    // reads of one need not wait for the direct loads into the other
    __shared__ __attribute__((aligned(16))) unsigned char s_buf0[kBufB];
    __shared__ __attribute__((aligned(16))) unsigned char s_buf1[kBufB];
    __shared__ int s_bt[kBtCache];
    __shared__ int s_ok;
    // the fp64 (cos, sin) table of the block's queries is needed only
    // before the first tile: it lives in buffer 1, which the first tile
    // does not use
    auto s_cs = reinterpret_cast<double2(*)[kD / 2]>(s_buf1);                   // [query][i]

    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin, so
    // physical id P runs on XCD P mod 8.  Logical ids are handed out in 8
    // contiguous chunks, one per XCD: the query tiles of one (request, KV
    // head) then share their K/V tiles in one XCD's L2.  Within a (request,
    // KV head), the last query tiles go first: under the causal mask they
    // have the longest context, and starting the longest blocks first
    // shortens the tail of the launch.
    const int nblk = gridDim.x * gridDim.y * gridDim.z;
    const int pid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int xq = nblk >> 3, xr = nblk & 7, xcd = pid & 7;
    const int lid = xcd * xq + min(xcd, xr) + (pid >> 3);
    const int lx = gridDim.x - 1 - lid % gridDim.x;
    const int qt = lx / a.splits, sp = lx - qt * a.splits;
    const int hk = (lid / gridDim.x) % gridDim.y, b = lid / (gridDim.x * gridDim.y);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
    const int qs = wave / kWQ;        // the wave's query sub-tile
    const int hb = wave - qs * kWQ;   // its first head
    const int col = lane & 15;        // the query this lane's S^T / O^T column holds
    const int grp = lane >> 4;        // 4-row group of the MFMA layouts
    const int c0 = a.ctx_begin[b];
    const int qp0 = a.q_pos[b];
    const int32_t* bt = a.bt + int64_t(b) * a.max_blocks;
    const int jb = qt * kBQ;          // the block's first query
    const int j_lo = jb + qs * kQT;   // the wave's first query
    const int jq = j_lo + col;
    const bool q_real = jq < a.tq;
    const bool wave_live = j_lo < a.tq;
    auto head = [&](int hs) { return hb + kWQ * hs; };

    // ---- raw Q (the lane's 8 + 8 elements of each head slot), issued first
    uint4 qraw[kHS][4];
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        const int hw = head(hs);
        const bool hv = hw < a.group && q_real;
        const uint16_t* qrow = a.q + ((int64_t(b) * a.tq + (q_real ? jq : 0)) * a.hq + hk * a.group +
                                      (hw < a.group ? hw : 0)) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int i = (kk & 1) * 32 + 8 * grp + (kk >> 1) * (kD / 2);
            qraw[hs][kk] = hv ? *reinterpret_cast<const uint4*>(qrow + i) : make_uint4(0, 0, 0, 0);
        }
    }

    // ---- the block's tile range (positions checked in int64 first: the
    // first tile's loads go out before the block-table check below)
    const bool pos_ok = c0 >= 0 && c0 <= qp0 && int64_t(qp0) + a.tq - 1 <= int64_t(INT32_MAX);
    const int j_hi = min(a.tq, jb + kBQ) - 1;               // last real query of the block
    const int p_end = pos_ok ? qp0 + j_hi : 0;              // last position any of them reads
    const int ntiles = pos_ok ? (p_end - c0) / kKT + 1 : 0;
    const int tps = (ntiles + a.splits - 1) / a.splits;     // tiles per split
    const int t_begin = sp * tps;
    const int t_end = min(ntiles, t_begin + tps);
    const int qpos = qp0 + jq;
    const int wave_last = qp0 + min(a.tq - 1, j_lo + kQT - 1);   // the wave's last query position

    // ---- tile staging by direct loads: wave w fills rows 16w .. 16w+15 of
    // a tile, four rows (1 KB) per instruction; lane l of instruction i holds
    // row 16w + 4i + l/16, slot l % 16.  A row past the block's last
    // position or with a block id out of range reads the zero row.
    const int slot = lane & 15;
    const unsigned char* zrow = static_cast<const unsigned char*>(a.zero_row) + 16 * slot;
    // tile-invariant parts of the addresses: each of the lane's four rows,
    // and the byte offset of its K and V chunk within a cache position
    // (head hk, swizzled slot); a cache block is below 4 GiB (checked on
    // the host), so only the block's base needs 64-bit arithmetic
    const uint32_t row_b = uint32_t(a.hkv) * (kD * 2);
    const uint32_t blk_b = row_b << a.log2_block;
    const int pmask = (1 << a.log2_block) - 1;
    int rr[4];
    uint32_t ko[4], vo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        rr[i] = 16 * wave + 4 * i + (lane >> 4);
        ko[i] = uint32_t(hk) * (kD * 2) + 16 * k_slot(rr[i], slot);
        vo[i] = uint32_t(hk) * (kD * 2) + 16 * v_slot(rr[i], slot);
    }
    // when a wave's 16 rows lie in one cache block (blocks of 16 positions or
    // more, context start on a 16-position boundary) each lane's offset from
    // that block's first row is the same for every tile
    uint32_t lk[4], lv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lk[i] = uint32_t(4 * i + (lane >> 4)) * row_b + ko[i];
        lv[i] = uint32_t(4 * i + (lane >> 4)) * row_b + vo[i];
    }
    const unsigned char* kc_b = reinterpret_cast<const unsigned char*>(a.kc);
    const unsigned char* vc_b = reinterpret_cast<const unsigned char*>(a.vc);
    const int64_t dkv = vc_b - kc_b;
    auto dma_tile = [&](unsigned char* buf, int t, const int (&blk)[4]) {
        const uint32_t tb = uint32_t(c0) + uint32_t(t) * kKT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // position within its cache block (< 1024) times the position
            // stride (< 2^24, checked on the host): a 24-bit product
            const uint32_t in_blk = __umul24((tb + rr[i]) & pmask, row_b);
            const unsigned char* kb = kc_b + uint64_t(uint32_t(blk[i])) * blk_b;
            const unsigned char* ks = blk[i] >= 0 ? kb + (in_blk + ko[i]) : zrow;
            const unsigned char* vs = blk[i] >= 0 ? kb + dkv + (in_blk + vo[i]) : zrow;
            __builtin_amdgcn_global_load_lds(ks, (__attribute__((address_space(3))) void*)(buf + (16 * wave + 4 * i) * kRowB), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vs, (__attribute__((address_space(3))) void*)(buf + kHalfB + (16 * wave + 4 * i) * kRowB), 16, 0, 0);
        }
    };
    if (t_begin < t_end) {
        // entries read from the table and range-checked here, since the
        // request's check has not run yet (a rejected request discards the
        // tile); the four entries are read first (clamped in range, so the
        // reads need no branch), then the eight direct loads
        int blk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t ei = int64_t(c0 + t_begin * kKT + rr[i]) >> a.log2_block;
            blk[i] = __builtin_nontemporal_load(bt + (ei < a.max_blocks ? ei : a.max_blocks - 1));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = c0 + t_begin * kKT + rr[i];
            if (p > p_end || (int64_t(p) >> a.log2_block) >= a.max_blocks || blk[i] < 0 || blk[i] >= a.num_blocks)
                blk[i] = -1;
        }
        dma_tile(s_buf0, t_begin, blk);
    }

    // ---- validation of the request (every block checks, one block reports)
    if (wave == 0) {
        uint32_t bits = 0;
        const int64_t last = int64_t(qp0) + a.tq - 1;
        if (!pos_ok) {
            bits |= FS_ERR_START_POS;
        } else if ((last >> a.log2_block) >= a.max_blocks) {
            bits |= FS_ERR_BLOCK_SHORT;
        } else {
            for (int64_t j = (c0 >> a.log2_block) + lane; j <= (last >> a.log2_block); j += 64) {
                const int e = bt[j];
                if (e < 0 || e >= a.num_blocks) bits |= FS_ERR_BLOCK_ID;
            }
        }
        bits = wave_or(bits);
        if (lane == 0) {
            s_ok = bits == 0;
            if (bits && qt == 0 && hk == 0 && sp == 0) atomicOr(a.err, bits);
        }
    }
    __syncthreads();
    auto mark = [&](float2 v) {       // this split's (max, sum) of the wave's rows
        if (q_real && grp == 0) {
#pragma unroll
            for (int hs = 0; hs < kHS; ++hs) {
                const int hw = head(hs);
                if (hw < a.group)
                    a.part_ml[((int64_t(sp) * gridDim.z + b) * a.tq + jq) * a.hq + hk * a.group + hw] = v;
            }
        }
    };
    if (!s_ok) {
        // a split run marks its partials so the combine writes nothing
        if (a.splits > 1) mark(make_float2(__builtin_nanf(""), 0.0f));
        __builtin_amdgcn_s_waitcnt(kWaitVm0);               // no direct load outlives the block
        return;
    }
    if (t_begin >= t_end) {
        // nothing of the context falls in this split: an empty partial
        mark(make_float2(-1e30f, 0.0f));
        return;
    }

    // ---- block-table entries of this block's positions, cached in LDS
    const int64_t e_first = int64_t(c0 + t_begin * kKT) >> a.log2_block;
    const int64_t e_last = int64_t(min(p_end, c0 + t_end * kKT - 1)) >> a.log2_block;
    const bool bt_cached = e_last - e_first + 1 <= kBtCache;
    if (bt_cached)
        for (int64_t j = e_first + threadIdx.x; j <= e_last; j += kThreads) s_bt[j - e_first] = bt[j];

    // ---- fp64 (cos, sin) of (position of query jb + qq) * w_i, shared by the
    // heads.  A thread keeps one frequency i and takes every kStep-th query:
    // one sincos for its first query and one for the step angle, then the
    // angle-addition recurrence (at most kBQ / kStep - 1 steps, each adding
    // a few fp64 roundings, far below the bf16 rounding that follows)
    static_assert(kThreads % (kD / 2) == 0, "one frequency per thread");
    {
        constexpr int kStep = kThreads / (kD / 2);
        const int i = threadIdx.x % (kD / 2);
        const double w_i = a.inv_freq[i];
        int qq = threadIdx.x / (kD / 2);
        double sv, cv, ds, dc;
        sincos(static_cast<double>(qp0 + jb + qq) * w_i, &sv, &cv);
        sincos(static_cast<double>(kStep) * w_i, &ds, &dc);
        for (; qq < kBQ; qq += kStep) {
            s_cs[qq][i] = make_double2(cv, sv);
            const double cn = fma(cv, dc, -(sv * ds));
            sv = fma(sv, dc, cv * ds);
            cv = cn;
        }
    }
    __syncthreads();

    // ---- Q fragments (B operand of S^T = K Q^T), rotated and rounded to bf16:
    // lane holds Q[jq][kk*32 + 8*grp + e]; chunks kk and kk+2 pair i with i+64
    b8 qf[kHS][4];
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const uint32_t* w1 = &qraw[hs][kk].x;
            const uint32_t* w2 = &qraw[hs][kk + 2].x;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = kk * 32 + 8 * grp + e;
                const double x1 = bf16_to_f32(static_cast<uint16_t>(w1[e >> 1] >> (16 * (e & 1))));
                const double x2 = bf16_to_f32(static_cast<uint16_t>(w2[e >> 1] >> (16 * (e & 1))));
                const double2 cs = s_cs[qs * kQT + col][i];
                qf[hs][kk][e] = as_bf16(static_cast<uint16_t>(f64_to_bf16_bits(fma(x1, cs.x, -(x2 * cs.y)))));
                qf[hs][kk + 2][e] = as_bf16(static_cast<uint16_t>(f64_to_bf16_bits(fma(x2, cs.x, x1 * cs.y))));
            }
        }
    }

    // O^T chunks: o[hs][dc][i] = O[jq][dc*16 + 4*grp + i]
    f4 o[kHS][8];
    float m[kHS], lp[kHS];            // running max (uniform over a column), partial sum (this lane)
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        m[hs] = -1e30f;
        lp[hs] = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) o[hs][dc] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // the block ids of the four rows first (LDS or global, one uniform
    // branch), then the eight direct loads
    // entry indices are clamped to the block's range and read without a
    // branch; rows past the block's last position then take -1
    const int e_first32 = static_cast<int>(e_first), e_span = static_cast<int>(e_last - e_first);
    const bool wave_blocks = bt_cached && a.log2_block >= 4 && (c0 & 15) == 0;
    auto load_tile = [&](unsigned char* buf, int t) {
        int blk[4];
        const uint32_t tb = uint32_t(c0) + uint32_t(t) * kKT;
        if (wave_blocks && tb + kKT - 1 <= uint32_t(p_end)) {
            // every row of the tile is real and the wave's 16 rows share one
            // cache block: one table entry and one base address per wave
            const uint32_t p0 = tb + 16 * wave;
            const int v = __builtin_amdgcn_readfirstlane(s_bt[min(static_cast<int>(p0 >> a.log2_block) - e_first32, e_span)]);
            const unsigned char* kb = kc_b + uint64_t(uint32_t(v)) * blk_b + __umul24(p0 & pmask, row_b);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_global_load_lds(kb + lk[i], (__attribute__((address_space(3))) void*)(buf + (16 * wave + 4 * i) * kRowB), 16, 0, 0);
                __builtin_amdgcn_global_load_lds(kb + dkv + lv[i], (__attribute__((address_space(3))) void*)(buf + kHalfB + (16 * wave + 4 * i) * kRowB), 16, 0, 0);
            }
            return;
        }
        if (bt_cached) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = tb + rr[i];
                const int v = s_bt[min(static_cast<int>(p >> a.log2_block) - e_first32, e_span)];
                blk[i] = p <= uint32_t(p_end) ? v : -1;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t p = tb + rr[i];
                const int v = bt[min(static_cast<int>(p >> a.log2_block), e_first32 + e_span)];
                blk[i] = p <= uint32_t(p_end) ? v : -1;
            }
        }
        dma_tile(buf, t, blk);
    };

    auto tile_math = [&](int t, const unsigned char* buf) {
        const int tbase = c0 + t * kKT;
        // a tile wholly after the wave's queries changes nothing (every weight
        // is 0), so the wave skips it; so do waves without a real query
        if (wave_live && tbase <= wave_last) {
            // S^T for 4 sub-tiles of 16 positions: st[hs][sub][i] = S[jq][tbase + 16*sub + 4*grp + i]
            // the compiler's own interleave of matrix instructions with LDS
            // reads: 1-3% faster on every shape measured
            __builtin_amdgcn_iglp_opt(1);
            f4 st[kHS][4];
#pragma unroll
            for (int sub = 0; sub < 4; ++sub) {
#pragma unroll
                for (int hs = 0; hs < kHS; ++hs) st[hs][sub] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const b8 ka = *reinterpret_cast<const b8*>(buf + (16 * sub + col) * kRowB + 16 * k_slot(col, 4 * kk + grp));
                    // a slot past the group computes on zero Q and is never
                    // written: no branch between the matrix instructions
#pragma unroll
                    for (int hs = 0; hs < kHS; ++hs)
                        st[hs][sub] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[hs][kk], st[hs][sub], 0, 0, 0);
                }
            }
            // causal mask only on tiles that reach past the wave's first
            // query position (a uniform branch); columns of absent queries
            // are never written
            if (tbase + kKT - 1 > qp0 + j_lo) {
#pragma unroll
                for (int hs = 0; hs < kHS; ++hs)
#pragma unroll
                    for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (tbase + 16 * sub + 4 * grp + i > qpos) st[hs][sub][i] = -1e30f;
                __asm__ volatile("" ::: "memory");
            }
            b8 pb[kHS][2];
            bool rescale = false;
            float m_new[kHS];
#pragma unroll
            for (int hs = 0; hs < kHS; ++hs) {
                // raw scores; the scale (> 0) is applied to the maximum and
                // inside each exponent, fl(max(s) c) being max(fl(s c))
                float tmax = -1e30f;
#pragma unroll
                for (int sub = 0; sub < 4; ++sub)
#pragma unroll
                    for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, st[hs][sub][i]);
                tmax = colmax(tmax);
                m_new[hs] = fmaxf(m[hs], tmax * a.scale_log2);
                rescale |= m_new[hs] > m[hs] + kLazy;
            }
            // the running maximum moves only when some column's grows by
            // more than kLazy: weights stay below 2^kLazy, and the rescale of
            // O and the sums is skipped on most tiles
            if (__builtin_amdgcn_ballot_w64(rescale) != 0) {
#pragma unroll
                for (int hs = 0; hs < kHS; ++hs) {
                    const float alpha = __builtin_amdgcn_exp2f(m[hs] - m_new[hs]);
                    m[hs] = m_new[hs];
                    lp[hs] *= alpha;
#pragma unroll
                    for (int dc = 0; dc < 8; ++dc) o[hs][dc] *= alpha;
                }
            }
#pragma unroll
            for (int hs = 0; hs < kHS; ++hs) {
                // P^T fragments for the two 32-position halves: k = 8*grp + e maps to
                // position 32*hh + 16*(e/4) + 4*grp + e%4, the lane's own scores
                float psum = 0.0f;
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pe = __builtin_amdgcn_exp2f(fmaf(st[hs][2 * hh + e / 4][e % 4], a.scale_log2, -m[hs]));
                        pb[hs][hh][e] = static_cast<__bf16>(pe);
                        psum += pe;
                    }
                }
                lp[hs] += psum;
            }
#pragma unroll
            for (int dc = 0; dc < 8; ++dc) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    // A = V^T row dc*16 + col, in the position order of pb,
                    // by two transposing LDS reads of row-major V (see tr_v)
                    const int vr = 32 * hh + 4 * grp + (col >> 2);
                    const b8 va = tr_v(reinterpret_cast<const uint16_t*>(buf + kHalfB + vr * kRowB + 16 * v_slot(vr, 2 * dc + ((col & 3) >> 1))) + 4 * (col & 1),
                                       16 * kD);
#pragma unroll
                    for (int hs = 0; hs < kHS; ++hs)
                        o[hs][dc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hs][hh], o[hs][dc], 0, 0, 0);
                }
            }
        }
    };
    // one barrier per tile: after it, tile t has landed in its buffer (each
    // wave waited for its own direct loads first) and every wave is done
    // with the other buffer, which then takes tile t + 1
    auto step = [&](int t, const unsigned char* cur, unsigned char* nxt) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        if (t + 1 < t_end) load_tile(nxt, t + 1);
        tile_math(t, cur);
    };
    for (int t = t_begin; t < t_end; t += 2) {
        step(t, s_buf0, s_buf1);
        if (t + 1 < t_end) step(t + 1, s_buf1, s_buf0);
    }

    // ---- lane holds O[jq][dc*16 + 4*grp .. +3] (unnormalised)
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        const int hw = head(hs);
        if (hw >= a.group) continue;
        float l = lp[hs];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        if (!q_real) continue;
        const int64_t row = (int64_t(b) * a.tq + jq) * a.hq + hk * a.group + hw;
        if (a.splits == 1) {
            const float linv = 1.0f / l;
            float* orow = a.out + row * kD + 4 * grp;
#pragma unroll
            for (int dc = 0; dc < 8; ++dc) *reinterpret_cast<f4*>(orow + dc * 16) = o[hs][dc] * linv;
        } else {
            const int64_t prow = int64_t(sp) * gridDim.z * a.tq * a.hq + row;
            float* orow = a.part_o + prow * kD + 4 * grp;
#pragma unroll
            for (int dc = 0; dc < 8; ++dc) *reinterpret_cast<f4*>(orow + dc * 16) = o[hs][dc];
            if (grp == 0) a.part_ml[prow] = make_float2(m[hs], l);
        }
    }
}

// Merge of the split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s
// with M = max_s m_s.  One thread per (row, 4 consecutive d): every split's
// (max, sum) is loaded at once, then every contributing split's partial, and
// the sums run in split order.  A NaN max marks a rejected request, whose
// rows are left unwritten.
__global__ __launch_bounds__(256) void fs_attend_combine_kernel(AttendArgs a, int64_t rows) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row = idx / (kD / 4);
    if (row >= rows) return;
    const int d = 4 * static_cast<int>(idx - row * (kD / 4));
    float2 ml[kMaxSplits];
    float mx = -1e30f;
    bool bad = false;
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        ml[s2] = s2 < a.splits ? a.part_ml[int64_t(s2) * rows + row] : make_float2(-1e30f, 0.0f);
        if (ml[s2].x != ml[s2].x) bad = true;
        mx = fmaxf(mx, ml[s2].x);
    }
    if (bad) return;
    float w[kMaxSplits];
    f4 x[kMaxSplits];
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        w[s2] = s2 < a.splits ? __builtin_amdgcn_exp2f(ml[s2].x - mx) : 0.0f;
        // empty splits leave no partial output
        x[s2] = w[s2] > 0.0f ? *reinterpret_cast<const f4*>(a.part_o + (int64_t(s2) * rows + row) * kD + d)
                             : f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    f4 num = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        if (w[s2] > 0.0f) {
            den += w[s2] * ml[s2].y;
            num += w[s2] * x[s2];
        }
    }
    *reinterpret_cast<f4*>(a.out + row * kD + d) = num / den;
}

}  // namespace

namespace {

// Query sub-tiles per block: two when two waves' head slots hold the whole
// GQA group and the request has more than one sub-tile of queries.
int attend_qsub(int group, int32_t num_q_tokens) { return group <= 4 && num_q_tokens > kQT ? 2 : 1; }

}  // namespace

int fsi_attend_splits(const fs_store* st, int32_t batch, int32_t num_q_tokens, int32_t num_q_heads,
                      int32_t max_blocks) {
    const int bq = kQT * attend_qsub(num_q_heads / st->desc.num_kv_heads, num_q_tokens);
    const int64_t base = int64_t((num_q_tokens + bq - 1) / bq) * st->desc.num_kv_heads * batch;
    // at most two blocks per CU (what LDS allows): more would queue a
    // second round of blocks
    const int64_t cus = st->num_cus;
    const int64_t two = 2 * cus / base > 1 ? 2 * cus / base : 1;
    const int64_t one = cus / base > 1 ? cus / base : 1;
    int64_t sp = two;
    if (two == 2 && 4 * base >= 3 * cus) {
        // one block per CU and no combine beats two per CU and a combine
        sp = 1;
    } else if (max_blocks > 0) {
        // a split shorter than 4 tiles of the longest context the block
        // table can hold: one block per CU with twice the tiles is faster
        // (the prologue and the combine are paid once per split)
        const int64_t tiles = ((int64_t(max_blocks) << st->log2_block) + kKT - 1) / kKT;
        if (tiles < 4 * two) sp = one;
    }
    return static_cast<int>(sp < 1 ? 1 : (sp > kMaxSplits ? kMaxSplits : sp));
}

size_t fsi_attend_workspace_bytes(int splits, int32_t batch, int32_t num_q_tokens, int32_t num_q_heads) {
    if (splits <= 1) return 0;
    const size_t rows = size_t(batch) * num_q_tokens * num_q_heads;
    return size_t(splits) * rows * (kD * sizeof(float) + sizeof(float2));
}

hipError_t fsi_launch_attend(const AttendLaunch& r) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    AttendArgs a{};
    a.q = static_cast<const uint16_t*>(r.q);
    a.tq = r.num_q_tokens;
    a.hq = r.num_q_heads;
    a.hkv = d.num_kv_heads;
    a.group = r.num_q_heads / d.num_kv_heads;
    a.kc = static_cast<const uint16_t*>(r.k_cache);
    a.vc = static_cast<const uint16_t*>(r.v_cache);
    a.num_blocks = r.num_blocks;
    a.log2_block = st->log2_block;
    a.max_blocks = r.max_blocks;
    a.bt = r.block_table;
    a.ctx_begin = r.ctx_begin;
    a.q_pos = r.q_pos;
    a.inv_freq = st->d_inv_freq;
    a.zero_row = st->d_zero_row;
    a.scale_log2 = r.scale * 1.4426950408889634f;
    a.out = r.out;
    a.err = st->d_err;
    // split the context when one range per (query tile, KV head, request)
    // would leave the device idle and the workspace holds the partials
    int splits = fsi_attend_splits(st, r.batch, r.num_q_tokens, r.num_q_heads, r.max_blocks);
    while (splits > 1 && fsi_attend_workspace_bytes(splits, r.batch, r.num_q_tokens, r.num_q_heads) >
                             r.workspace_bytes)
        --splits;
    if (!r.workspace) splits = 1;
    a.splits = splits;
    if (splits > 1) {
        const size_t rows = size_t(r.batch) * r.num_q_tokens * r.num_q_heads;
        a.part_o = static_cast<float*>(r.workspace);
        a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(r.workspace) + size_t(splits) * rows * kD * sizeof(float));
    }
    const int qsub = attend_qsub(a.group, r.num_q_tokens);
    const int bq = kQT * qsub;
    const dim3 grid(static_cast<unsigned>((r.num_q_tokens + bq - 1) / bq * splits),
                    static_cast<unsigned>(d.num_kv_heads), static_cast<unsigned>(r.batch));
    if (qsub == 2) {
        if (a.group <= kWaves / 2)
            fs_attend_kernel<1, 2><<<grid, kThreads, 0, r.stream>>>(a);
        else
            fs_attend_kernel<2, 2><<<grid, kThreads, 0, r.stream>>>(a);
    } else if (a.group <= kWaves) {
        fs_attend_kernel<1, 1><<<grid, kThreads, 0, r.stream>>>(a);
    } else {
        fs_attend_kernel<2, 1><<<grid, kThreads, 0, r.stream>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t rows = int64_t(r.batch) * r.num_q_tokens * r.num_q_heads;
    fs_attend_combine_kernel<<<static_cast<unsigned>((rows * (kD / 4) + 255) / 256), 256, 0, r.stream>>>(a, rows);
    return hipGetLastError();
}
