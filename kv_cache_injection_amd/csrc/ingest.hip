// Store ingest: the capture half of Context-Window Encoding.
//
// InferScale encodes each memory fact offline together with a window of the
// w preceding conversation turns and keeps only the KV of the fact itself,
// keys taken before RoPE (gist.science summary, "Phase Hors-ligne" and
// "Stockage Pré-RoPE").  The encoder is the serving model's own prefill over
// [w turns ; fact]; this kernel is what the store does with its output: for
// every layer it copies the fact's rows out of the window's pre-RoPE K and
// raw V into free arena rows, then records the fact's rows and length in its
// slot and copies its embedding row.  The context rows are discarded.
//
// Grid (row group, fact, layer); 256-thread blocks copy 16-byte vectors, a
// whole K and V row per token; block (0, f, 0) writes fact f's metadata.

#include <hip/hip_runtime.h>

#include "fs_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerBlock = 8;

struct IngestArgs {
    const IngestItem* items;
    int32_t row_vec;                       // 16-byte vectors per row (H * D / 8)
    int32_t e;                             // embedding width
    const uint4* kw[FS_MAX_LAYERS];
    const uint4* vw[FS_MAX_LAYERS];
    uint4* ka[FS_MAX_LAYERS];
    uint4* va[FS_MAX_LAYERS];
    int64_t* fact_begin;
    int32_t* fact_len;
    const float* emb_new;
    float* emb;
};

__global__ __launch_bounds__(kThreads) void fs_ingest_kernel(IngestArgs a) {
    const IngestItem it = a.items[blockIdx.y];
    const int l = blockIdx.z;
    const int r0 = blockIdx.x * kRowsPerBlock;
    if (blockIdx.x == 0 && l == 0) {
        if (threadIdx.x == 0) {
            a.fact_begin[it.slot] = it.dst_row;
            a.fact_len[it.slot] = it.len;
        }
        for (int j = threadIdx.x; j < a.e; j += kThreads)
            a.emb[int64_t(it.slot) * a.e + j] = a.emb_new[int64_t(it.emb_row) * a.e + j];
    }
    if (r0 >= it.len) return;
    const int rows = min(kRowsPerBlock, it.len - r0);
    const int64_t nvec = int64_t(rows) * a.row_vec;
    const int64_t src = (it.src_row + r0) * a.row_vec;
    const int64_t dst = (it.dst_row + r0) * a.row_vec;
    for (int64_t i = threadIdx.x; i < nvec; i += kThreads) {
        a.ka[l][dst + i] = a.kw[l][src + i];
        a.va[l][dst + i] = a.vw[l][src + i];
    }
}

}  // namespace

hipError_t fsi_launch_ingest(const IngestLaunch& r) {
    const fs_store* st = r.st;
    const fs_store_desc& d = st->desc;
    IngestArgs a{};
    a.items = static_cast<const IngestItem*>(st->d_ingest_items);
    a.row_vec = d.num_kv_heads * d.head_dim / 8;
    a.e = d.embed_dim;
    for (int l = 0; l < d.num_layers; ++l) {
        a.kw[l] = static_cast<const uint4*>(r.k_window[l]);
        a.vw[l] = static_cast<const uint4*>(r.v_window[l]);
        a.ka[l] = static_cast<uint4*>(const_cast<void*>(st->src_k[l]));
        a.va[l] = static_cast<uint4*>(const_cast<void*>(st->src_v[l]));
    }
    a.fact_begin = st->d_fact_begin;
    a.fact_len = st->d_fact_len;
    a.emb_new = r.emb_new;
    a.emb = const_cast<float*>(st->emb);
    const dim3 grid(static_cast<unsigned>((r.max_len + kRowsPerBlock - 1) / kRowsPerBlock),
                    static_cast<unsigned>(r.n), static_cast<unsigned>(d.num_layers));
    fs_ingest_kernel<<<grid, kThreads, 0, r.stream>>>(a);
    return hipGetLastError();
}
