// Inverted-file index over one user's fact embeddings, for approximate
// retrieval from stores far larger than a flat scan serves at low latency.
//
// The pages name a GPU-resident retrieval index ("Jasper", gist.science
// summary, "Contributions Clés") without describing it; this index is
// designed here.  Build: spherical k-means (inner product, unit-norm
// centroids), iterated a fixed number of times on the GPU, then the facts are
// grouped by their nearest centroid into lists (ascending fact id within a
// list) and their embedding rows copied in list order so that a probe streams
// each list contiguously.  Probe (retrieve.hip): score the centroids, take the
// nprobe best lists, scan them, keep the top k.
//
// Build kernels, all deterministic for a given input:
//   init     centroid c starts as the row floor(c * N / C), normalised in fp64
//   assign   tiled fp32 dot products of 64 rows x 64 centroids per block
//            (16 x 16 threads, 4 x 4 outputs each, 16-column LDS slices);
//            every row keeps its best centroid, ties to the lower index
//   lists    per 1024-row chunk an LDS histogram; per-list prefix over chunks;
//            one wave per chunk writes each row at list start + chunk prefix
//            + its rank among earlier rows of the chunk in the same list,
//            which keeps lists in ascending fact order
//   update   one block per list sums its rows in list order in fp64 and
//            normalises; an empty list keeps its centroid
// Index build is offline work; it is correct and reproducible rather than
// tuned.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "fs_internal.h"

namespace {

constexpr int kChunk = 1024;          // rows per list-building chunk

__global__ void ivf_init_kernel(const float* emb, int32_t n, int32_t e, int32_t nlist, float* cent) {
    const int c = blockIdx.x;
    const int64_t row = int64_t(c) * n / nlist;
    const float* src = emb + row * e;
    __shared__ double s_sum[256];
    double ss = 0.0;
    for (int j = threadIdx.x; j < e; j += blockDim.x) ss += double(src[j]) * double(src[j]);
    s_sum[threadIdx.x] = ss;
    __syncthreads();
    for (int h = blockDim.x / 2; h > 0; h >>= 1) {
        if (int(threadIdx.x) < h) s_sum[threadIdx.x] += s_sum[threadIdx.x + h];
        __syncthreads();
    }
    const double inv = s_sum[0] > 0.0 ? 1.0 / sqrt(s_sum[0]) : 0.0;
    for (int j = threadIdx.x; j < e; j += blockDim.x) cent[int64_t(c) * e + j] = static_cast<float>(src[j] * inv);
}

// 64 rows x all centroids, in 64-centroid tiles; E in slices of 16.
__global__ __launch_bounds__(256) void ivf_assign_kernel(const float* emb, int32_t n, int32_t e,
                                                         const float* cent, int32_t nlist, int32_t* assign) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t r0 = int64_t(blockIdx.x) * 64;
    float best[4];
    int bidx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        best[i] = -3.0e38f;
        bidx[i] = 0;
    }
    const int lr = tid >> 2, le = (tid & 3) * 4;   // loader: row/centroid lr, columns le..le+3
    for (int c0 = 0; c0 < nlist; c0 += 64) {
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
        for (int e0 = 0; e0 < e; e0 += 16) {
            const int64_t row = r0 + lr;
            const int cc = c0 + lr;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = e0 + le + j;
                As[le + j][lr] = (row < n && col < e) ? emb[row * e + col] : 0.0f;
                Bs[le + j][lr] = (cc < nlist && col < e) ? cent[int64_t(cc) * e + col] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                float av[4], bv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    av[i] = As[kk][ty * 4 + i];
                    bv[i] = Bs[kk][tx * 4 + i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
            }
            __syncthreads();
        }
        // best centroid of this tile per row, across the 16 threads of the row
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float bs = -3.0e38f;
            int bc = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cc = c0 + tx * 4 + j;
                if (cc < nlist && acc[i][j] > bs) {
                    bs = acc[i][j];
                    bc = cc;
                }
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
                const float os = __shfl_xor(bs, m, 64);
                const int oc = __shfl_xor(bc, m, 64);
                if (os > bs || (os == bs && oc < bc)) {
                    bs = os;
                    bc = oc;
                }
            }
            if (bs > best[i]) {            // tiles come in ascending order: ties keep the earlier
                best[i] = bs;
                bidx[i] = bc;
            }
        }
    }
    if (tx == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t row = r0 + ty * 4 + i;
            if (row < n) assign[row] = bidx[i];
        }
    }
}

__global__ __launch_bounds__(256) void ivf_count_kernel(const int32_t* assign, int32_t n, int32_t nlist,
                                                        int32_t* chunk_counts) {
    extern __shared__ int s_hist[];
    for (int c = threadIdx.x; c < nlist; c += blockDim.x) s_hist[c] = 0;
    __syncthreads();
    const int64_t r0 = int64_t(blockIdx.x) * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += blockDim.x)
        if (r0 + i < n) atomicAdd(&s_hist[assign[r0 + i]], 1);
    __syncthreads();
    for (int c = threadIdx.x; c < nlist; c += blockDim.x) chunk_counts[int64_t(blockIdx.x) * nlist + c] = s_hist[c];
}

// per list: counts over chunks become exclusive prefixes; totals[c] the list size
__global__ void ivf_chunk_prefix_kernel(int32_t* chunk_counts, int32_t nchunks, int32_t nlist, int32_t* totals) {
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= nlist) return;
    int32_t run = 0;
    for (int k = 0; k < nchunks; ++k) {
        const int32_t t = chunk_counts[int64_t(k) * nlist + c];
        chunk_counts[int64_t(k) * nlist + c] = run;
        run += t;
    }
    totals[c] = run;
}

// one block of 1024 threads: list_begin = exclusive scan of totals (nlist <= 4096)
__global__ __launch_bounds__(1024) void ivf_list_begin_kernel(const int32_t* totals, int32_t nlist,
                                                              int32_t* list_begin, int32_t* max_list) {
    __shared__ int32_t s_part[1024];
    __shared__ int32_t s_max[1024];
    const int t = threadIdx.x;
    int32_t v[4], sum = 0, mx = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = t * 4 + j;
        v[j] = c < nlist ? totals[c] : 0;
        sum += v[j];
        mx = max(mx, v[j]);
    }
    s_part[t] = sum;
    s_max[t] = mx;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {      // inclusive scan (Hillis-Steele)
        const int32_t x = t >= off ? s_part[t - off] : 0;
        const int32_t m = t >= off ? s_max[t - off] : 0;
        __syncthreads();
        s_part[t] += x;
        s_max[t] = max(s_max[t], m);
        __syncthreads();
    }
    int32_t run = t > 0 ? s_part[t - 1] : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = t * 4 + j;
        if (c < nlist) list_begin[c] = run;
        run += v[j];
    }
    if (t == 1023) {
        list_begin[nlist] = s_part[1023];
        *max_list = s_max[1023];
    }
}

// one wave per chunk: stable placement of the chunk's rows into their lists
__global__ __launch_bounds__(64) void ivf_scatter_kernel(const int32_t* assign, int32_t n, int32_t nlist,
                                                         const int32_t* chunk_prefix, const int32_t* list_begin,
                                                         int64_t fact_base, int32_t* members) {
    extern __shared__ int s_seen[];
    const int lane = threadIdx.x;
    for (int c = lane; c < nlist; c += 64) s_seen[c] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const int64_t r0 = int64_t(blockIdx.x) * kChunk;
    const int32_t* pre = chunk_prefix + int64_t(blockIdx.x) * nlist;
    for (int s0 = 0; s0 < kChunk; s0 += 64) {
        const int64_t row = r0 + s0 + lane;
        const bool v = row < n;
        const int c = v ? assign[row] : -1;
        int rank = 0;
        for (int j = 0; j < 64; ++j) {
            const int cj = __shfl(c, j, 64);
            if (j < lane && cj == c) ++rank;
        }
        int seen = 0;
        if (v) seen = s_seen[c];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (v) {
            members[list_begin[c] + pre[c] + seen + rank] = static_cast<int32_t>(fact_base + row);
            atomicAdd(&s_seen[c], 1);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

__global__ void ivf_gather_rows_kernel(const float* emb, int32_t e, const int32_t* members, int32_t n,
                                       int64_t fact_base, float* out) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t row = idx / e;
    if (row >= n) return;
    const int j = static_cast<int>(idx - row * e);
    out[idx] = emb[(int64_t(members[row]) - fact_base) * e + j];
}

// one block per list: fp64 sum of its rows in list order, normalised
__global__ __launch_bounds__(256) void ivf_update_kernel(const float* emb, int32_t e, const int32_t* members,
                                                         const int32_t* list_begin, int64_t fact_base,
                                                         float* cent) {
    extern __shared__ double s_acc[];          // [e]
    __shared__ double s_red[256];
    const int c = blockIdx.x;
    const int32_t beg = list_begin[c], end = list_begin[c + 1];
    if (beg == end) return;                    // an empty list keeps its centroid
    for (int j = threadIdx.x; j < e; j += blockDim.x) {
        double acc = 0.0;
        for (int32_t r = beg; r < end; ++r) acc += double(emb[(int64_t(members[r]) - fact_base) * e + j]);
        s_acc[j] = acc;
    }
    double ss = 0.0;
    for (int j = threadIdx.x; j < e; j += blockDim.x) ss += s_acc[j] * s_acc[j];
    s_red[threadIdx.x] = ss;
    __syncthreads();
    for (int h = blockDim.x / 2; h > 0; h >>= 1) {
        if (int(threadIdx.x) < h) s_red[threadIdx.x] += s_red[threadIdx.x + h];
        __syncthreads();
    }
    if (s_red[0] <= 0.0) return;
    const double inv = 1.0 / sqrt(s_red[0]);
    for (int j = threadIdx.x; j < e; j += blockDim.x) cent[int64_t(c) * e + j] = static_cast<float>(s_acc[j] * inv);
}

}  // namespace

hipError_t fsi_ivf_build(fs_ivf* ix, hipStream_t s) {
    const fs_store_desc& d = ix->store->desc;
    const int32_t e = d.embed_dim;
    const int32_t n = ix->num_facts;
    const int32_t C = ix->nlist;
    const float* emb = ix->store->emb + ix->fact_base * e;
    const int32_t nchunks = (n + kChunk - 1) / kChunk;
    int32_t* d_assign = nullptr;
    int32_t* d_chunk = nullptr;
    int32_t* d_tot = nullptr;
    int32_t* d_max = nullptr;
    hipError_t err = hipMalloc(&d_assign, sizeof(int32_t) * size_t(n));
    if (err == hipSuccess) err = hipMalloc(&d_chunk, sizeof(int32_t) * size_t(nchunks) * C);
    if (err == hipSuccess) err = hipMalloc(&d_tot, sizeof(int32_t) * size_t(C));
    if (err == hipSuccess) err = hipMalloc(&d_max, sizeof(int32_t));
    auto lists = [&]() -> hipError_t {
        ivf_assign_kernel<<<dim3((n + 63) / 64), 256, 0, s>>>(emb, n, e, ix->d_cent, C, d_assign);
        ivf_count_kernel<<<dim3(nchunks), 256, sizeof(int) * size_t(C), s>>>(d_assign, n, C, d_chunk);
        ivf_chunk_prefix_kernel<<<dim3((C + 255) / 256), 256, 0, s>>>(d_chunk, nchunks, C, d_tot);
        ivf_list_begin_kernel<<<1, 1024, 0, s>>>(d_tot, C, ix->d_list_begin, d_max);
        ivf_scatter_kernel<<<dim3(nchunks), 64, sizeof(int) * size_t(C), s>>>(
            d_assign, n, C, d_chunk, ix->d_list_begin, ix->fact_base, ix->d_members);
        return hipGetLastError();
    };
    if (err == hipSuccess) {
        ivf_init_kernel<<<dim3(C), 256, 0, s>>>(emb, n, e, C, ix->d_cent);
        err = hipGetLastError();
    }
    for (int it = 0; it < ix->iters && err == hipSuccess; ++it) {
        err = lists();
        if (err == hipSuccess) {
            ivf_update_kernel<<<dim3(C), 256, sizeof(double) * size_t(e), s>>>(
                emb, e, ix->d_members, ix->d_list_begin, ix->fact_base, ix->d_cent);
            err = hipGetLastError();
        }
    }
    if (err == hipSuccess) err = lists();            // final lists from the final centroids
    if (err == hipSuccess) {
        const int64_t tot = int64_t(n) * e;
        ivf_gather_rows_kernel<<<dim3(static_cast<unsigned>((tot + 255) / 256)), 256, 0, s>>>(
            emb, e, ix->d_members, n, ix->fact_base, ix->d_emb_sorted);
        err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipMemcpyAsync(&ix->max_list, d_max, sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    for (void* p : {static_cast<void*>(d_assign), static_cast<void*>(d_chunk), static_cast<void*>(d_tot),
                    static_cast<void*>(d_max)})
        if (p) (void)hipFree(p);
    return err;
}
