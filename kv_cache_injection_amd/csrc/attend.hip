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
// One block = 16 query tokens x one KV head (all the query heads of its GQA
// group).  Scores and P.V run on the matrix cores (16x16x16 bf16 MFMA, fp32
// accumulation); softmax is online in fp32 (exp2).  Scores are computed
// transposed, S^T = K Q^T, so that each lane's four scores are exactly the
// four P entries it must supply as the A operand of P V: no shuffle of P.
// K tiles of 16 positions are staged in LDS row-major, V tiles transposed
// (d-major), double-buffered, with the next tile's global loads in flight
// while the current one is consumed.

#include <hip/hip_runtime.h>

#include "fs_device.h"
#include "fs_internal.h"

namespace {

using fsd::f64_to_bf16_bits;
using fsd::wave_or;

constexpr int kD = 128;               // head dim handled
constexpr int kQT = 16;               // query tokens per block
constexpr int kKT = 16;               // cache positions per tile
constexpr int kThreads = 256;         // 4 waves
constexpr int kWaves = kThreads / 64;

typedef short s4 __attribute__((ext_vector_type(4)));
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
    float scale_log2;                 // softmax scale * log2(e)
    float* out;                       // [B][Tq][Hq][D] fp32
    uint32_t* err;
};

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

template <int kHS>                    // head slots per wave: group <= 4 * kHS
__global__ __launch_bounds__(kThreads) void fs_attend_kernel(AttendArgs a) {
    __shared__ uint16_t sK[2][kKT][kD + 8];      // [pos][d], rows padded against bank conflicts
    __shared__ uint16_t sVt[2][kD][kKT + 4];     // [d][pos], rows padded against bank conflicts
    __shared__ int s_ok;

    const int qt = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;        // S^T column = query; O column = d within a chunk
    const int grp = lane >> 4;        // 4-row group of the MFMA layouts
    const int c0 = a.ctx_begin[b];
    const int qp0 = a.q_pos[b];
    const int64_t bs_mask = (int64_t(1) << a.log2_block) - 1;
    const int32_t* bt = a.bt + int64_t(b) * a.max_blocks;

    // ---- validation of the request (every block checks, block (0, 0) reports)
    if (wave == 0) {
        uint32_t bits = 0;
        const int64_t last = int64_t(qp0) + a.tq - 1;
        if (c0 < 0 || c0 > qp0 || last > int64_t(INT32_MAX)) {
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
            if (bits && qt == 0 && hk == 0) atomicOr(a.err, bits);
        }
    }
    __syncthreads();
    if (!s_ok) return;

    const int j_lo = qt * kQT;
    const int j_hi = min(a.tq, j_lo + kQT) - 1;            // last real query of the block
    const int p_end = qp0 + j_hi;                           // last position any of them reads
    const int ntiles = (p_end - c0) / kKT + 1;
    const int jq = j_lo + col;                              // this lane's query (S^T column)
    const bool q_real = jq < a.tq;
    const int qpos = qp0 + jq;

    // ---- Q fragments (B operand of S^T = K Q^T), rotated and rounded to bf16
    // lane holds Q[jq][kk*16 + 4*grp + e]; chunks kk and kk+4 pair i with i+64
    s4 qf[kHS][8];
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        const int hw = wave + kWaves * hs;
        const bool hv = hw < a.group && q_real;
        const uint16_t* qrow = a.q + ((int64_t(b) * a.tq + (q_real ? jq : 0)) * a.hq + hk * a.group +
                                      (hw < a.group ? hw : 0)) * kD;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = kk * 16 + 4 * grp + e;
                uint16_t y1 = 0, y2 = 0;
                if (hv) {
                    const double x1 = bf16_to_f32(qrow[i]);
                    const double x2 = bf16_to_f32(qrow[i + kD / 2]);
                    double sv, cv;
                    sincos(static_cast<double>(qpos) * a.inv_freq[i], &sv, &cv);
                    y1 = static_cast<uint16_t>(f64_to_bf16_bits(fma(x1, cv, -(x2 * sv))));
                    y2 = static_cast<uint16_t>(f64_to_bf16_bits(fma(x2, cv, x1 * sv)));
                }
                qf[hs][kk][e] = static_cast<short>(y1);
                qf[hs][kk + 4][e] = static_cast<short>(y2);
            }
        }
    }

    f4 o[kHS][8];
    float m[kHS], l[kHS];
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        m[hs] = -1e30f;
        l[hs] = 0.0f;
#pragma unroll
        for (int dc = 0; dc < 8; ++dc) o[hs][dc] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // ---- K/V tile staging: thread -> (position tid/16, 16-byte vector tid%16)
    const int lpos = threadIdx.x >> 4;
    const int lvec = threadIdx.x & 15;
    uint4 kreg = make_uint4(0, 0, 0, 0), vreg = make_uint4(0, 0, 0, 0);
    auto gload = [&](int t) {
        const int p = c0 + t * kKT + lpos;
        if (p <= p_end) {
            const int blk = bt[p >> a.log2_block];
            const int64_t row = (int64_t(blk) << a.log2_block) | (p & bs_mask);
            const int64_t off = (row * a.hkv + hk) * kD + lvec * 8;
            kreg = *reinterpret_cast<const uint4*>(a.kc + off);
            vreg = *reinterpret_cast<const uint4*>(a.vc + off);
        } else {
            kreg = make_uint4(0, 0, 0, 0);
            vreg = make_uint4(0, 0, 0, 0);
        }
    };
    auto lstore = [&](int buf) {
        *reinterpret_cast<uint4*>(&sK[buf][lpos][lvec * 8]) = kreg;
        const uint32_t w[4] = {vreg.x, vreg.y, vreg.z, vreg.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sVt[buf][lvec * 8 + 2 * e][lpos] = static_cast<uint16_t>(w[e] & 0xFFFFu);
            sVt[buf][lvec * 8 + 2 * e + 1][lpos] = static_cast<uint16_t>(w[e] >> 16);
        }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int buf = t & 1;
        if (t + 1 < ntiles) gload(t + 1);
        const int pbase = c0 + t * kKT + 4 * grp;           // positions of this lane's 4 scores
#pragma unroll
        for (int hs = 0; hs < kHS; ++hs) {
            if (wave + kWaves * hs >= a.group) continue;    // uniform over the wave
            f4 st = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const s4 ka = *reinterpret_cast<const s4*>(&sK[buf][col][kk * 16 + 4 * grp]);
                st = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, qf[hs][kk], st, 0, 0, 0);
            }
            // st[i] = S^T[position pbase + i][query jq]
            float sv[4];
            float tmax = -1e30f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = q_real && (pbase + i <= qpos);
                sv[i] = ok ? st[i] * a.scale_log2 : -1e30f;
                tmax = fmaxf(tmax, sv[i]);
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m[hs], tmax);
            const float alpha = exp2f(m[hs] - m_new);
            s4 pa;
            float psum = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint16_t pb = f32_to_bf16_rne(exp2f(sv[i] - m_new));
                pa[i] = static_cast<short>(pb);
                psum += bf16_to_f32(pb);                      // normalise with the weights used
            }
            psum += __shfl_xor(psum, 16, 64);
            psum += __shfl_xor(psum, 32, 64);
            l[hs] = l[hs] * alpha + psum;
            m[hs] = m_new;
            // O rows are queries 4*grp + i: their rescale factors sit in lanes
            // whose column is that query
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
                for (int dc = 0; dc < 8; ++dc) o[hs][dc][i] *= ai;
            }
#pragma unroll
            for (int dc = 0; dc < 8; ++dc) {
                const s4 vb = *reinterpret_cast<const s4*>(&sVt[buf][dc * 16 + col][4 * grp]);
                o[hs][dc] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, o[hs][dc], 0, 0, 0);
            }
        }
        if (t + 1 < ntiles) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- normalise and write: lane holds O[query j_lo + 4*grp + i][dc*16 + col]
#pragma unroll
    for (int hs = 0; hs < kHS; ++hs) {
        const int hw = wave + kWaves * hs;
        if (hw >= a.group) continue;
        const float linv = l[hs] > 0.0f ? 1.0f / l[hs] : 0.0f;
        const int h = hk * a.group + hw;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(linv, 4 * grp + i, 64);
            const int jo = j_lo + 4 * grp + i;
            if (jo < a.tq) {
                float* orow = a.out + ((int64_t(b) * a.tq + jo) * a.hq + h) * kD;
#pragma unroll
                for (int dc = 0; dc < 8; ++dc) orow[dc * 16 + col] = o[hs][dc][i] * li;
            }
        }
    }
}

}  // namespace

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
    a.scale_log2 = r.scale * 1.4426950408889634f;
    a.out = r.out;
    a.err = st->d_err;
    const dim3 grid(static_cast<unsigned>((r.num_q_tokens + kQT - 1) / kQT),
                    static_cast<unsigned>(d.num_kv_heads), static_cast<unsigned>(r.batch));
    if (a.group <= kWaves)
        fs_attend_kernel<1><<<grid, kThreads, 0, r.stream>>>(a);
    else
        fs_attend_kernel<2><<<grid, kThreads, 0, r.stream>>>(a);
    return hipGetLastError();
}
