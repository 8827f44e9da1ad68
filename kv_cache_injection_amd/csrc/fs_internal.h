// Internal declarations shared by the host runtime and the kernel files of the
// fact-store KV-injection library.  Not part of the ABI (include/fs.h is).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "fs.h"

namespace fsi {

// Largest segment-token count a block's prologue handles for one request in
// LDS: offsets [k+1] int32 + first rows [k] int64.
constexpr int kMaxK = FS_MAX_K;

// Top-k keeps a request's keys in LDS when the user has at most this many
// facts (48 KiB of uint64 keys); larger users are re-read from global memory.
constexpr int kTopkLdsKeys = 6144;
// users with more facts than kTopkChunkedN are selected in two phases: the
// top k of every chunk of kTopkChunk scores (one block each), then the top k
// of those candidates
constexpr int kTopkChunkedN = 65536;
constexpr int kTopkChunk = 16384;

}  // namespace fsi

struct fs_store {
    fs_store_desc desc;
    int device = 0;
    int32_t num_cus = 0;          // compute units of the device (attention split sizing)
    int32_t max_fact_len = 0;     // longest fact, tokens
    double mean_fact_len = 0;     // mean fact length at creation (inject grid sizing)
    int32_t seg_tokens = 0;       // max_k * max_fact_len: longest possible segment
    int32_t max_user_facts = 0;   // largest user, facts
    int32_t log2_block = 0;

    // library-owned device memory
    int64_t* d_fact_begin = nullptr;   // [F+1] first arena row of each fact
    int32_t* d_fact_len = nullptr;     // [F]
    int64_t* d_user_begin = nullptr;   // [U+1] first fact slot of each user
    int32_t* d_user_count = nullptr;   // [U] live facts of each user: slots user_begin[u] .. + count
    double* d_inv_freq = nullptr;      // [head_dim/2] theta^(-2i/D)
    void* d_zero_row = nullptr;        // kZeroRowBytes of zeros (rows past a tile's end read it)
    uint32_t* d_err = nullptr;         // device error word
    double* d_scores = nullptr;        // [max_batch][max_user_facts] score scratch
    int32_t topk_chunks = 0;           // chunks of the largest user (0: one-phase selection)
    int32_t* d_tk_ids = nullptr;       // [max_batch][topk_chunks * max_k] per-chunk winners
    double* d_tk_scores = nullptr;     // [max_batch][topk_chunks * max_k]
    int32_t* d_tk_counts = nullptr;    // [max_batch]
    const void** d_src_k = nullptr;    // [L] device-visible arena pointers
    const void** d_src_v = nullptr;
    const void** d_src_kv = nullptr;   // [L][2]: the same, K then V of each layer
    // identity written into every plan header this store makes (plans are
    // refused by another store)
    uint32_t tag = 0;
    // fs_inject's plan slots: each call composes its plan into a slot and
    // injects from it.  A slot is reused by the stream that used it last
    // without any synchronisation (stream order); handing it to another
    // stream first makes that stream wait for an event recorded on the last
    // one.  Pinned stores use slot 0 only (their calls must not overlap).
    struct PlanSlot {
        void* buf = nullptr;                 // fsi_plan_bytes(max_batch) bytes
        hipStream_t last = nullptr;          // stream of the last call that used it
        bool used = false;
        uint64_t stamp = 0;                  // last use (LRU choice)
        hipEvent_t ev = nullptr;             // recorded on `last` when the slot changes streams
    };
    mutable std::vector<PlanSlot> slots;
    mutable std::mutex slot_mu;
    mutable uint64_t slot_clock = 0;

    // pinned stores: staging ring
    int32_t stage_tokens = 0;          // max_k * max_fact_len
    void* d_stage_k = nullptr;         // [staging_layers][max_batch][stage_tokens][H][D] bf16
    void* d_stage_v = nullptr;
    int32_t* d_stage_ids = nullptr;    // [staging_layers][max_batch][max_k]
    int32_t* d_stage_meta = nullptr;   // [staging_layers][4]: k, batch, layer of the last fetch

    // host mirrors of the metadata that ingest and eviction change
    std::vector<int64_t> h_user_begin;     // [U+1]
    std::vector<int32_t> h_user_count;     // [U]
    std::vector<int64_t> h_fact_begin;     // [F]
    std::vector<int32_t> h_fact_len;       // [F]
    int64_t next_row = 0;                  // first arena row never handed out
    void* d_ingest_items = nullptr;        // [kIngestMax] per-call fact descriptors
    void* h_ingest_items = nullptr;        // pinned host staging of the descriptors (first ingest)
    int32_t* h_ingest_counts = nullptr;    // pinned host staging of the live counts [U]
    hipEvent_t ingest_copied = nullptr;    // recorded after the last ingest's host-to-device copies

    // caller-owned, referenced
    const float* emb = nullptr;
    std::vector<const void*> src_k, src_v;   // device-visible addresses
};

// ---- kernel launchers (one translation unit each) -------------------------

struct RetrieveLaunch {
    const fs_store* st;
    int32_t batch;
    const int32_t* user;
    const float* query;
    int32_t k;
    int32_t* ids;
    double* scores;
    int32_t* num_tokens;
    hipStream_t stream;
    // plan set (fs_retrieve_plan): the final selection also writes the inject
    // plan of the selected ids into it, checked against these
    void* plan = nullptr;
    const int32_t* block_table = nullptr;
    int32_t max_blocks = 0;
    const int32_t* start_pos = nullptr;
    int32_t num_blocks = 0;
};
hipError_t fsi_launch_retrieve(const RetrieveLaunch& a);

struct InjectLaunch {
    const fs_store* st;
    int32_t layer_begin, layer_end;   // [begin, end)
    int32_t batch;
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    const int32_t* block_table;
    int32_t max_blocks;
    const int32_t* start_pos;
    void* const* k_cache;             // host array [num_layers]
    void* const* v_cache;
    int32_t num_blocks;
    hipStream_t stream;
    // plan_out set: compose and validate into it (and inject from it when
    // inject is set); plan_in set: inject from it (user, ids, block_table,
    // start_pos unused)
    void* plan_out = nullptr;
    const void* plan_in = nullptr;
    bool inject = false;
};
hipError_t fsi_launch_inject(const InjectLaunch& a);
// fs_inject_noalloc's plan buffer on `device`: its device address (looked up
// once per device) and size in bytes
hipError_t fsi_noalloc_scratch(int device, void** ptr, size_t* bytes);

// Layout of an inject plan for `batch` requests:
//   PlanHeader (32 bytes); then per request {segment length (0 when
//   rejected), start position} as two int32 (padded to 16 bytes); then per
//   request seg_tokens entries {arena row, cache slot (block * block_size +
//   slot)} as two int64.  Each request's pair and each token's pair is one
//   scalar load for the injecting kernel.
constexpr uint32_t kPlanMagic = 0x4E414C50u;   // "PLAN"
struct PlanHeader {
    uint64_t key;          // fsi_plan_key of the call that wrote it
    uint32_t magic;
    uint32_t tag;          // fs_store::tag of the store that wrote it
    int32_t batch, k, seg_tokens;
    int32_t num_blocks;    // the cache size the block ids were checked against
};
static_assert(sizeof(PlanHeader) == 32, "plan header is 32 bytes");
struct PlanReq {
    int32_t len, start;
};
struct PlanTok {
    int64_t src, dst;
};
struct PlanView {
    PlanHeader* hdr;
    PlanReq* req;
    PlanTok* tok;          // [batch][seg_tokens]
};
inline size_t fsi_plan_header_bytes(int32_t batch) {
    return sizeof(PlanHeader) + (size_t(batch) * sizeof(PlanReq) + 15) / 16 * 16;
}
inline size_t fsi_plan_bytes(const fs_store* st, int32_t batch) {
    return fsi_plan_header_bytes(batch) + sizeof(PlanTok) * size_t(batch) * size_t(st->seg_tokens);
}
inline PlanView fsi_plan_view(const fs_store* st, int32_t batch, const void* plan) {
    (void)st;
    char* p = static_cast<char*>(const_cast<void*>(plan));
    return PlanView{reinterpret_cast<PlanHeader*>(p), reinterpret_cast<PlanReq*>(p + sizeof(PlanHeader)),
                    reinterpret_cast<PlanTok*>(p + fsi_plan_header_bytes(batch))};
}
// A 64-bit identity of (store, batch, k, segment bound, cache size): the plan
// kernel writes the key of its call, the inject kernel compares it with the
// key of its own call (FNV-1a over the six words)
inline uint64_t fsi_plan_key(uint32_t tag, int32_t batch, int32_t k, int32_t seg_tokens, int32_t num_blocks) {
    const uint32_t w[6] = {kPlanMagic, tag, uint32_t(batch), uint32_t(k), uint32_t(seg_tokens), uint32_t(num_blocks)};
    uint64_t h = 0xcbf29ce484222325ull;
    for (uint32_t x : w)
        for (int byte = 0; byte < 4; ++byte) {
            h ^= (x >> (8 * byte)) & 0xFFu;
            h *= 0x100000001b3ull;
        }
    return h;
}

constexpr size_t kZeroRowBytes = 512;
struct AttendLaunch {
    const fs_store* st;
    int32_t batch, num_q_tokens, num_q_heads;
    const void* q;
    const void* k_cache;
    const void* v_cache;
    int32_t num_blocks;
    const int32_t* block_table;
    int32_t max_blocks;
    const int32_t* ctx_begin;
    const int32_t* q_pos;
    float scale;
    float* out;
    void* workspace;
    size_t workspace_bytes;
    hipStream_t stream;
};
hipError_t fsi_launch_attend(const AttendLaunch& a);
// context splits the launch would use, and the workspace that many need
// max_blocks: the block table's width (the context bound), or 0 when unknown
int fsi_attend_splits(const fs_store* st, int32_t batch, int32_t num_q_tokens, int32_t num_q_heads,
                      int32_t max_blocks);
size_t fsi_attend_workspace_bytes(int splits, int32_t batch, int32_t num_q_tokens, int32_t num_q_heads);

// Inverted-file index over one user's facts (approximate retrieval).
struct fs_ivf {
    const fs_store* store = nullptr;
    int32_t user = 0, nlist = 0, num_facts = 0, max_nprobe = 0, max_list = 0, iters = 0;
    int32_t max_batch = 0;
    int64_t fact_base = 0;             // global id of the user's first fact
    float* d_cent = nullptr;           // [nlist][E] unit-norm centroids
    int32_t* d_list_begin = nullptr;   // [nlist+1] offsets into members
    int32_t* d_members = nullptr;      // [num_facts] global fact ids, by list, ascending within a list
    float* d_emb_sorted = nullptr;     // [num_facts][E] the members' embedding rows, same order
    int64_t* d_cent_range = nullptr;   // {0, nlist}: the centroids as one "user"
    int32_t* d_zero_users = nullptr;   // [max_batch] zeros
    double* d_cscores = nullptr;       // [max_batch][nlist] centroid scores
    int32_t* d_chosen = nullptr;       // [max_batch][max_nprobe] probed lists
    int32_t cand_stride = 0;           // max_nprobe lists of at most max_list facts
    double* d_cand_scores = nullptr;   // [max_batch][cand_stride]
    int32_t* d_cand_ids = nullptr;     // [max_batch][cand_stride]
    int32_t* d_counts = nullptr;       // [max_batch] candidates per request
    int32_t* d_offs = nullptr;         // [max_batch][max_nprobe + 1] list starts in the candidates
};

struct IvfProbeLaunch {
    const fs_ivf* ivf;
    int32_t batch;
    const float* query;
    int32_t nprobe, k;
    int32_t* ids;
    double* scores;
    int32_t* num_tokens;
    hipStream_t stream;
};
hipError_t fsi_launch_ivf_probe(const IvfProbeLaunch& a);
// builds ix's centroids, lists and sorted rows (index arrays already allocated)
hipError_t fsi_ivf_build(fs_ivf* ix, hipStream_t stream);

// one ingested fact: rows [src_row, src_row + len) of the window arrays go to
// arena rows [dst_row, dst_row + len), slot `slot`, embedding row `emb_row`
struct IngestItem {
    int64_t src_row, dst_row;
    int32_t len, slot, emb_row, pad;
};
constexpr int kIngestMax = 4096;          // facts per fs_ingest_facts call

struct IngestLaunch {
    const fs_store* st;
    int32_t n;
    int32_t max_len;
    const void* const* k_window;           // host array [num_layers] of device-visible [rows][H][D]
    const void* const* v_window;
    const float* emb_new;                  // device [n][E]
    hipStream_t stream;
};
hipError_t fsi_launch_ingest(const IngestLaunch& a);

struct FetchLaunch {
    const fs_store* st;
    int32_t layer_begin, layer_end;
    int32_t batch;
    const int32_t* user;
    const int32_t* ids;
    int32_t k;
    hipStream_t stream;
};
hipError_t fsi_launch_fetch(const FetchLaunch& a);
