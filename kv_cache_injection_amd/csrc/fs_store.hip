// Host runtime of the fact-store KV-injection library: argument validation,
// store creation/destruction, launch dispatch and error reporting.
//
// Every host-checkable condition is tested before the first HIP call of an
// entry point, so a rejected call enqueues nothing and writes nothing.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "fs_internal.h"

namespace {

thread_local char g_msg[512] = "";

fs_status fail(fs_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return st;
}

fs_status hip_fail(hipError_t e, const char* what) {
    return fail(FS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}

void free_store(fs_store* s) {
    if (!s) return;
    void* bufs[] = {s->d_fact_begin, s->d_fact_len, s->d_user_begin, s->d_user_count,
                    s->d_ingest_items, s->d_inv_freq, s->d_zero_row, s->d_err,
                    s->d_scores, s->d_tk_ids, s->d_tk_scores, s->d_tk_counts,
                    (void*)s->d_src_k, (void*)s->d_src_v, (void*)s->d_src_kv, s->d_stage_k,
                    s->d_stage_v, s->d_stage_ids, s->d_stage_meta};
    for (void* p : bufs)
        if (p) (void)hipFree(p);
    for (auto& sl : s->slots) {
        if (sl.buf) (void)hipFree(sl.buf);
        if (sl.ev) (void)hipEventDestroy(sl.ev);
    }
    if (s->ingest_copied) (void)hipEventDestroy(s->ingest_copied);
    if (s->h_ingest_items) (void)hipHostFree(s->h_ingest_items);
    if (s->h_ingest_counts) (void)hipHostFree(s->h_ingest_counts);
    delete s;
}

// A plan slot for one fs_inject call on stream s (caller holds slot_mu):
// the slot this stream used last, else an unused one, else the least
// recently used one, after making s wait for that slot's last use.
void* acquire_slot(const fs_store* st, hipStream_t s, hipError_t* err) {
    auto& slots = st->slots;
    int pick = -1;
    for (size_t i = 0; i < slots.size() && pick < 0; ++i)
        if (slots[i].used && slots[i].last == s) pick = static_cast<int>(i);
    for (size_t i = 0; i < slots.size() && pick < 0; ++i)
        if (!slots[i].used) pick = static_cast<int>(i);
    if (pick < 0) {
        pick = 0;
        for (size_t i = 1; i < slots.size(); ++i)
            if (slots[i].stamp < slots[pick].stamp) pick = static_cast<int>(i);
        fs_store::PlanSlot& sl = slots[pick];
        hipError_t e = hipEventRecord(sl.ev, sl.last);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, sl.ev, 0);
        if (e != hipSuccess) {
            *err = e;
            return nullptr;
        }
    }
    fs_store::PlanSlot& sl = slots[pick];
    sl.used = true;
    sl.last = s;
    sl.stamp = ++st->slot_clock;
    return sl.buf;
}

fs_status check_desc(const fs_store_desc* d) {
    if (d->num_layers < 1 || d->num_layers > FS_MAX_LAYERS)
        return fail(FS_E_ARG, "num_layers %d outside [1, %d]", d->num_layers, FS_MAX_LAYERS);
    if (d->num_kv_heads < 1) return fail(FS_E_ARG, "num_kv_heads must be >= 1");
    if (d->head_dim < 16 || d->head_dim % 16 != 0)
        return fail(FS_E_ARG, "head_dim %d must be a positive multiple of 16", d->head_dim);
    if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256)
        return fail(FS_E_UNSUPPORTED, "head_dim %d: built for 64, 128, 256", d->head_dim);
    if (int64_t(d->num_kv_heads) * d->head_dim > 8192)
        return fail(FS_E_UNSUPPORTED, "num_kv_heads * head_dim = %lld: token rows above 16 KB are not built",
                    static_cast<long long>(int64_t(d->num_kv_heads) * d->head_dim));
    if (d->embed_dim < 4 || d->embed_dim % 4 != 0)
        return fail(FS_E_ARG, "embed_dim %d must be a positive multiple of 4", d->embed_dim);
    if (d->embed_dim > 4096) return fail(FS_E_UNSUPPORTED, "embed_dim %d > 4096", d->embed_dim);
    if (!(d->rope_theta > 1.0) || !std::isfinite(d->rope_theta))
        return fail(FS_E_ARG, "rope_theta must be finite and > 1");
    if (!pow2(d->block_size) || d->block_size > 1024)
        return fail(FS_E_ARG, "block_size %d must be a power of two <= 1024", d->block_size);
    if (d->kv_location != FS_KV_DEVICE && d->kv_location != FS_KV_PINNED_HOST)
        return fail(FS_E_ARG, "kv_location %d unknown", d->kv_location);
    if (d->num_users < 1) return fail(FS_E_ARG, "num_users must be >= 1");
    if (d->max_batch < 1 || d->max_batch > 65535)
        return fail(FS_E_ARG, "max_batch %d outside [1, 65535]", d->max_batch);
    if (d->max_k < 1 || d->max_k > FS_MAX_K)
        return fail(FS_E_ARG, "max_k %d outside [1, %d]", d->max_k, FS_MAX_K);
    if (d->kv_location == FS_KV_PINNED_HOST &&
        (d->staging_layers < 1 || d->staging_layers > d->num_layers))
        return fail(FS_E_ARG, "staging_layers %d outside [1, num_layers]", d->staging_layers);
    if (d->num_facts < 1) return fail(FS_E_ARG, "num_facts must be >= 1");
    if (d->num_tokens < 1) return fail(FS_E_ARG, "num_tokens must be >= 1");
    return FS_OK;
}

}  // namespace

extern "C" {

const char* fs_last_error_message(void) { return g_msg; }

const char* fs_strerror(fs_status s) {
    switch (s) {
        case FS_OK: return "ok";
        case FS_E_ARG: return "invalid argument";
        case FS_E_RANGE: return "argument out of the store's range";
        case FS_E_BLOCKTABLE: return "unusable block table arguments";
        case FS_E_NOMEM: return "device allocation failed";
        case FS_E_HIP: return "HIP runtime error";
        case FS_E_DEVICE: return "device-side error bits set";
        case FS_E_UNSUPPORTED: return "unsupported configuration";
        default: return "unknown status";
    }
}

fs_status fs_create_store(const fs_store_desc* desc, const int64_t* user_fact_begin,
                          const int32_t* fact_len, const float* emb, const void* const* k_pre,
                          const void* const* v, void* stream, fs_store** out) {
    g_msg[0] = 0;
    if (!desc || !user_fact_begin || !fact_len || !emb || !k_pre || !v || !out)
        return fail(FS_E_ARG, "null pointer argument");
    if (fs_status st = check_desc(desc)) return st;
    const fs_store_desc& d = *desc;
    if (!aligned(emb, 16)) return fail(FS_E_ARG, "emb not 16-byte aligned");
    for (int l = 0; l < d.num_layers; ++l) {
        if (!k_pre[l] || !v[l]) return fail(FS_E_ARG, "layer %d arena pointer is null", l);
        if (!aligned(k_pre[l], 16) || !aligned(v[l], 16))
            return fail(FS_E_ARG, "layer %d arena not 16-byte aligned", l);
    }
    if (user_fact_begin[0] != 0) return fail(FS_E_ARG, "user_fact_begin[0] must be 0");
    int64_t max_user = 0;
    for (int u = 0; u < d.num_users; ++u) {
        int64_t n = user_fact_begin[u + 1] - user_fact_begin[u];
        if (n < 0) return fail(FS_E_ARG, "user_fact_begin decreases at user %d", u);
        if (n > max_user) max_user = n;
    }
    if (user_fact_begin[d.num_users] != d.num_facts)
        return fail(FS_E_ARG, "user_fact_begin[num_users] != num_facts");
    if (max_user > INT32_MAX) return fail(FS_E_UNSUPPORTED, "a user has more than 2^31-1 facts");
    int64_t total = 0;
    int32_t max_len = 0;
    for (int64_t f = 0; f < d.num_facts; ++f) {
        if (fact_len[f] < 1) return fail(FS_E_ARG, "fact_len[%lld] < 1", (long long)f);
        total += fact_len[f];
        if (fact_len[f] > max_len) max_len = fact_len[f];
    }
    if (total > d.num_tokens) return fail(FS_E_ARG, "sum(fact_len) exceeds num_tokens");
    if (int64_t(max_len) * d.max_k > INT32_MAX)
        return fail(FS_E_UNSUPPORTED, "max_k * longest fact exceeds 2^31-1 tokens");

    // ---- host checks done; from here on HIP calls ---------------------------
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    fs_store* st = new (std::nothrow) fs_store();
    if (!st) return fail(FS_E_NOMEM, "host allocation failed");
    st->desc = d;
    st->max_fact_len = max_len;
    st->mean_fact_len = double(total) / double(d.num_facts);
    st->max_user_facts = static_cast<int32_t>(max_user);
    st->log2_block = ilog2(d.block_size);
    st->emb = emb;
    hipError_t e = hipGetDevice(&st->device);
    if (e != hipSuccess) { free_store(st); return hip_fail(e, "hipGetDevice"); }
    e = hipDeviceGetAttribute(&st->num_cus, hipDeviceAttributeMultiprocessorCount, st->device);
    if (e != hipSuccess || st->num_cus < 1) { free_store(st); return hip_fail(e, "hipDeviceGetAttribute(CUs)"); }
    st->seg_tokens = max_len * d.max_k;

    // pointer kinds: a device store must hold device memory, a pinned store
    // page-locked host memory, and every kernel gets a device-visible address
    auto kind_ok = [&](const void* p, bool want_host, const void** dev, const char* what,
                       int l) -> fs_status {
        hipPointerAttribute_t at;
        hipError_t pe = hipPointerGetAttributes(&at, p);
        if (pe != hipSuccess) {
            (void)hipGetLastError();
            return fail(FS_E_ARG, "%s (layer %d): not HIP-registered memory", what, l);
        }
        if (want_host) {
            if (at.type != hipMemoryTypeHost)
                return fail(FS_E_ARG, "%s (layer %d): not page-locked host memory", what, l);
            void* dp = nullptr;
            hipError_t ge = hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0);
            if (ge != hipSuccess || !dp)
                return fail(FS_E_ARG, "%s (layer %d): no device mapping", what, l);
            *dev = dp;
        } else {
            if (at.type != hipMemoryTypeDevice)
                return fail(FS_E_ARG, "%s (layer %d): not device memory", what, l);
            *dev = p;
        }
        return FS_OK;
    };
    const bool pinned = d.kv_location == FS_KV_PINNED_HOST;
    {
        const void* dummy;
        if (fs_status ks = kind_ok(emb, false, &dummy, "emb", -1)) { free_store(st); return ks; }
    }
    st->src_k.resize(d.num_layers);
    st->src_v.resize(d.num_layers);
    for (int l = 0; l < d.num_layers; ++l) {
        if (fs_status ks = kind_ok(k_pre[l], pinned, &st->src_k[l], "k_pre", l)) { free_store(st); return ks; }
        if (fs_status ks = kind_ok(v[l], pinned, &st->src_v[l], "v", l)) { free_store(st); return ks; }
    }

    std::vector<int64_t> fb(d.num_facts + 1, 0);
    for (int64_t f = 0; f < d.num_facts; ++f) fb[f + 1] = fb[f] + fact_len[f];
    std::vector<double> inv(d.head_dim / 2);
    for (int i = 0; i < d.head_dim / 2; ++i)
        inv[i] = std::pow(d.rope_theta, -2.0 * double(i) / double(d.head_dim));

    const int H = d.num_kv_heads, D = d.head_dim;
    st->topk_chunks = max_user > fsi::kTopkChunkedN
                          ? static_cast<int32_t>((max_user + fsi::kTopkChunk - 1) / fsi::kTopkChunk) : 0;
    const size_t tk_elems = size_t(d.max_batch) * size_t(st->topk_chunks > 0 ? st->topk_chunks : 1) * size_t(d.max_k);
    struct { void** p; size_t bytes; const char* what; } allocs[] = {
        {(void**)&st->d_fact_begin, sizeof(int64_t) * (d.num_facts + 1), "fact offsets"},
        {(void**)&st->d_fact_len, sizeof(int32_t) * d.num_facts, "fact lengths"},
        {(void**)&st->d_user_begin, sizeof(int64_t) * (d.num_users + 1), "user offsets"},
        {(void**)&st->d_user_count, sizeof(int32_t) * d.num_users, "user counts"},
        {(void**)&st->d_ingest_items, sizeof(IngestItem) * kIngestMax, "ingest descriptors"},
        {(void**)&st->d_inv_freq, sizeof(double) * (D / 2), "frequency table"},
        {(void**)&st->d_zero_row, kZeroRowBytes, "zero row"},
        {(void**)&st->d_err, sizeof(uint32_t), "error word"},
        {(void**)&st->d_scores, sizeof(double) * size_t(d.max_batch) * size_t(max_user > 0 ? max_user : 1), "score scratch"},
        {(void**)&st->d_tk_ids, sizeof(int32_t) * tk_elems, "top-k chunk scratch"},
        {(void**)&st->d_tk_scores, sizeof(double) * tk_elems, "top-k chunk scratch"},
        {(void**)&st->d_tk_counts, sizeof(int32_t) * size_t(d.max_batch), "top-k chunk scratch"},
        {(void**)&st->d_src_k, sizeof(void*) * d.num_layers, "arena table"},
        {(void**)&st->d_src_v, sizeof(void*) * d.num_layers, "arena table"},
        {(void**)&st->d_src_kv, 2 * sizeof(void*) * d.num_layers, "arena table"},
    };
    for (auto& a : allocs) {
        e = hipMalloc(a.p, a.bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            free_store(st);
            return fail(FS_E_NOMEM, "hipMalloc(%s, %zu bytes): %s", a.what, a.bytes, hipGetErrorString(e));
        }
    }
    // plan slots of fs_inject (pinned stores: one, their calls never overlap)
    st->slots.resize(pinned ? 1 : FS_PLAN_SLOTS);
    for (auto& sl : st->slots) {
        e = hipMalloc(&sl.buf, fsi_plan_bytes(st, d.max_batch));
        if (e == hipSuccess) e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            free_store(st);
            return fail(FS_E_NOMEM, "plan slot (%zu bytes): %s", fsi_plan_bytes(st, d.max_batch),
                        hipGetErrorString(e));
        }
    }
    {
        // a process-unique identity for the plans this store writes
        static std::atomic<uint32_t> next_tag{0x2545F491u};
        st->tag = next_tag.fetch_add(0x9E3779B9u);
    }
    if (pinned) {
        st->stage_tokens = st->seg_tokens;
        size_t rows = size_t(d.staging_layers) * d.max_batch * size_t(st->stage_tokens);
        size_t bytes = rows * H * D * 2;
        struct { void** p; size_t bytes; } sa[] = {
            {&st->d_stage_k, bytes}, {&st->d_stage_v, bytes},
            {(void**)&st->d_stage_ids, sizeof(int32_t) * size_t(d.staging_layers) * d.max_batch * d.max_k},
            {(void**)&st->d_stage_meta, sizeof(int32_t) * 4 * size_t(d.staging_layers)}};
        for (auto& a : sa) {
            e = hipMalloc(a.p, a.bytes);
            if (e != hipSuccess) {
                (void)hipGetLastError();
                free_store(st);
                return fail(FS_E_NOMEM, "hipMalloc(staging, %zu bytes): %s", a.bytes, hipGetErrorString(e));
            }
        }
    }

    st->h_user_begin.assign(user_fact_begin, user_fact_begin + d.num_users + 1);
    st->h_user_count.resize(d.num_users);
    for (int u = 0; u < d.num_users; ++u)
        st->h_user_count[u] = static_cast<int32_t>(user_fact_begin[u + 1] - user_fact_begin[u]);
    st->h_fact_begin.assign(fb.begin(), fb.end() - 1);
    st->h_fact_len.assign(fact_len, fact_len + d.num_facts);
    st->next_row = total;                     // rows past the facts are free for ingest
    std::vector<const void*> src_kv(2 * size_t(d.num_layers));
    for (int l = 0; l < d.num_layers; ++l) {
        src_kv[2 * l] = st->src_k[l];
        src_kv[2 * l + 1] = st->src_v[l];
    }
    std::vector<int32_t> meta_init(4 * size_t(pinned ? d.staging_layers : 0), -1);
    uint32_t zero = 0;
    const std::vector<unsigned char> zero_row(kZeroRowBytes, 0);
    struct { void* dst; const void* src; size_t bytes; } cps[] = {
        {st->d_fact_begin, fb.data(), sizeof(int64_t) * fb.size()},
        {st->d_fact_len, fact_len, sizeof(int32_t) * d.num_facts},
        {st->d_user_begin, user_fact_begin, sizeof(int64_t) * (d.num_users + 1)},
        {st->d_user_count, st->h_user_count.data(), sizeof(int32_t) * d.num_users},
        {st->d_inv_freq, inv.data(), sizeof(double) * inv.size()},
        {st->d_err, &zero, sizeof(uint32_t)},
        {st->d_zero_row, zero_row.data(), kZeroRowBytes},
        {(void*)st->d_src_k, st->src_k.data(), sizeof(void*) * d.num_layers},
        {(void*)st->d_src_v, st->src_v.data(), sizeof(void*) * d.num_layers},
        {(void*)st->d_src_kv, src_kv.data(), 2 * sizeof(void*) * d.num_layers},
        {st->d_stage_meta, meta_init.data(), sizeof(int32_t) * meta_init.size()},
    };
    for (auto& c : cps) {
        if (!c.bytes) continue;
        e = hipMemcpyAsync(c.dst, c.src, c.bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) { free_store(st); return hip_fail(e, "hipMemcpyAsync(metadata)"); }
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) { free_store(st); return hip_fail(e, "hipStreamSynchronize"); }
    *out = st;
    return FS_OK;
}

fs_status fs_destroy_store(fs_store* store) {
    g_msg[0] = 0;
    if (!store) return FS_OK;
    hipError_t e = hipDeviceSynchronize();
    free_store(store);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    return FS_OK;
}

namespace {

// the host checks of fs_retrieve_topk and fs_retrieve_plan
fs_status check_retrieve(const fs_store* store, int32_t batch, const int32_t* user, const float* query, int32_t k,
                         const int32_t* ids, const double* scores, const int32_t* num_tokens) {
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_store_desc& d = store->desc;
    if (batch < 1 || batch > d.max_batch)
        return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, d.max_batch);
    if (k < 0 || k > d.max_k) return fail(FS_E_RANGE, "k %d outside [0, %d]", k, d.max_k);
    if (!user || !query) return fail(FS_E_ARG, "null user or query");
    if (!aligned(query, 16)) return fail(FS_E_ARG, "query not 16-byte aligned");
    if (!aligned(user, 4)) return fail(FS_E_ARG, "user not 4-byte aligned");
    if (k > 0 && !ids) return fail(FS_E_ARG, "null ids");
    if (ids && !aligned(ids, 4)) return fail(FS_E_ARG, "ids not 4-byte aligned");
    if (scores && !aligned(scores, 8)) return fail(FS_E_ARG, "scores not 8-byte aligned");
    if (num_tokens && !aligned(num_tokens, 4)) return fail(FS_E_ARG, "num_tokens not 4-byte aligned");
    return FS_OK;
}

}  // namespace

fs_status fs_retrieve_topk(const fs_store* store, int32_t batch, const int32_t* user,
                           const float* query, int32_t k, int32_t* ids, double* scores,
                           int32_t* num_tokens, void* stream) {
    g_msg[0] = 0;
    if (fs_status c = check_retrieve(store, batch, user, query, k, ids, scores, num_tokens)) return c;
    if (k == 0 && !num_tokens) return FS_OK;
    RetrieveLaunch a{store, batch, user, query, k, ids, scores, num_tokens,
                     reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = fsi_launch_retrieve(a);
    if (e != hipSuccess) return hip_fail(e, "retrieve launch");
    return FS_OK;
}

namespace {

// the host checks of fs_inject_layers and fs_inject_noalloc
fs_status check_inject(const fs_store* store, int32_t layer_begin, int32_t layer_end, int32_t batch,
                       const int32_t* user, const int32_t* ids, int32_t k, const int32_t* block_table,
                       int32_t max_blocks, const int32_t* start_pos, void* const* k_cache,
                       void* const* v_cache, int32_t num_blocks) {
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_store_desc& d = store->desc;
    if (layer_begin < 0 || layer_end > d.num_layers || layer_begin >= layer_end)
        return fail(FS_E_RANGE, "layer range [%d, %d) invalid for %d layers", layer_begin, layer_end,
                    d.num_layers);
    if (batch < 1 || batch > d.max_batch)
        return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, d.max_batch);
    if (k < 0 || k > d.max_k) return fail(FS_E_RANGE, "k %d outside [0, %d]", k, d.max_k);
    if (!user || !ids || !block_table || !start_pos || !k_cache || !v_cache)
        return fail(FS_E_ARG, "null pointer argument");
    if (!aligned(user, 4) || !aligned(ids, 4) || !aligned(block_table, 4) || !aligned(start_pos, 4))
        return fail(FS_E_ARG, "int32 argument not 4-byte aligned");
    if (max_blocks < 1) return fail(FS_E_BLOCKTABLE, "max_blocks %d < 1", max_blocks);
    if (num_blocks < 1) return fail(FS_E_BLOCKTABLE, "num_blocks %d < 1", num_blocks);
    for (int l = layer_begin; l < layer_end; ++l) {
        if (!k_cache[l] || !v_cache[l]) return fail(FS_E_ARG, "layer %d cache pointer is null", l);
        if (!aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
            return fail(FS_E_ARG, "layer %d cache not 16-byte aligned", l);
    }
    return FS_OK;
}

}  // namespace

fs_status fs_inject_layers(const fs_store* store, int32_t layer_begin, int32_t layer_end, int32_t batch,
                           const int32_t* user, const int32_t* ids, int32_t k, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* start_pos, void* const* k_cache,
                           void* const* v_cache, int32_t num_blocks, void* stream) {
    g_msg[0] = 0;
    const fs_status c = check_inject(store, layer_begin, layer_end, batch, user, ids, k, block_table, max_blocks,
                                     start_pos, k_cache, v_cache, num_blocks);
    if (c != FS_OK || k == 0) return c;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    InjectLaunch a{store, layer_begin, layer_end, batch, user, ids, k, block_table, max_blocks, start_pos,
                   k_cache, v_cache, num_blocks, s};
    a.inject = true;
    // the slot stays locked until both kernels are enqueued, so no other
    // call can hand it to another stream in between
    std::lock_guard<std::mutex> lock(store->slot_mu);
    hipError_t e = hipSuccess;
    a.plan_out = acquire_slot(store, s, &e);
    if (e != hipSuccess) return hip_fail(e, "plan slot hand-over");
    e = fsi_launch_inject(a);
    if (e != hipSuccess) return hip_fail(e, "inject launch");
    return FS_OK;
}

fs_status fs_inject_noalloc(const fs_store* store, int32_t layer, int32_t batch, const int32_t* user,
                            const int32_t* ids, int32_t k, const int32_t* block_table, int32_t max_blocks,
                            const int32_t* start_pos, void* const* k_cache, void* const* v_cache,
                            int32_t num_blocks, void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const int32_t nl = store->desc.num_layers;
    if (layer != FS_ALL_LAYERS && (layer < 0 || layer >= nl))
        return fail(FS_E_RANGE, "layer %d outside [0, %d)", layer, nl);
    const int32_t lb = layer == FS_ALL_LAYERS ? 0 : layer;
    const int32_t le = layer == FS_ALL_LAYERS ? nl : layer + 1;
    const fs_status c = check_inject(store, lb, le, batch, user, ids, k, block_table, max_blocks, start_pos,
                                     k_cache, v_cache, num_blocks);
    if (c != FS_OK) return c;
    const size_t need = fsi_plan_bytes(store, batch);
    if (need > FS_NOALLOC_PLAN_BYTES)
        return fail(FS_E_RANGE, "plan of %zu bytes for %d requests exceeds the %zu-byte static plan buffer", need,
                    batch, static_cast<size_t>(FS_NOALLOC_PLAN_BYTES));
    if (k == 0) return FS_OK;
    void* buf = nullptr;
    size_t bytes = 0;
    hipError_t e = fsi_noalloc_scratch(store->device, &buf, &bytes);
    if (e != hipSuccess) return hip_fail(e, "static plan buffer lookup");
    InjectLaunch a{store, lb, le, batch, user, ids, k, block_table, max_blocks, start_pos,
                   k_cache, v_cache, num_blocks, reinterpret_cast<hipStream_t>(stream)};
    a.inject = true;
    a.plan_out = buf;
    e = fsi_launch_inject(a);
    if (e != hipSuccess) return hip_fail(e, "inject launch");
    return FS_OK;
}

fs_status fs_inject_plan_size(const fs_store* store, int32_t batch, size_t* bytes) {
    g_msg[0] = 0;
    if (!store || !bytes) return fail(FS_E_ARG, "null argument");
    if (batch < 1 || batch > store->desc.max_batch)
        return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, store->desc.max_batch);
    *bytes = fsi_plan_bytes(store, batch);
    return FS_OK;
}

namespace {

// the checks a plan buffer must pass in both halves of the planned path
fs_status check_plan(const fs_store* store, int32_t batch, int32_t k, const void* plan, size_t plan_bytes) {
    const fs_store_desc& d = store->desc;
    if (d.kv_location != FS_KV_DEVICE) return fail(FS_E_UNSUPPORTED, "planned injection needs a device store");
    if (batch < 1 || batch > d.max_batch) return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, d.max_batch);
    if (k < 0 || k > d.max_k) return fail(FS_E_RANGE, "k %d outside [0, %d]", k, d.max_k);
    if (!plan) return fail(FS_E_ARG, "null plan");
    if (!aligned(plan, 16)) return fail(FS_E_ARG, "plan not 16-byte aligned");
    if (plan_bytes < fsi_plan_bytes(store, batch))
        return fail(FS_E_RANGE, "plan of %zu bytes, %zu needed for %d requests", plan_bytes,
                    fsi_plan_bytes(store, batch), batch);
    return FS_OK;
}

}  // namespace

fs_status fs_plan_inject(const fs_store* store, int32_t batch, const int32_t* user, const int32_t* ids, int32_t k,
                         const int32_t* block_table, int32_t max_blocks, const int32_t* start_pos,
                         int32_t num_blocks, void* plan, size_t plan_bytes, void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_status c = check_plan(store, batch, k, plan, plan_bytes);
    if (c != FS_OK) return c;
    if (!user || !ids || !block_table || !start_pos) return fail(FS_E_ARG, "null pointer argument");
    if (!aligned(user, 4) || !aligned(ids, 4) || !aligned(block_table, 4) || !aligned(start_pos, 4))
        return fail(FS_E_ARG, "int32 argument not 4-byte aligned");
    if (max_blocks < 1) return fail(FS_E_BLOCKTABLE, "max_blocks %d < 1", max_blocks);
    if (num_blocks < 1) return fail(FS_E_BLOCKTABLE, "num_blocks %d < 1", num_blocks);
    if (k == 0) return FS_OK;
    InjectLaunch a{store, 0, store->desc.num_layers, batch, user, ids, k, block_table, max_blocks, start_pos,
                   nullptr, nullptr, num_blocks, reinterpret_cast<hipStream_t>(stream)};
    a.plan_out = plan;
    hipError_t e = fsi_launch_inject(a);
    if (e != hipSuccess) return hip_fail(e, "plan launch");
    return FS_OK;
}

fs_status fs_retrieve_plan(const fs_store* store, int32_t batch, const int32_t* user, const float* query, int32_t k,
                           int32_t* ids, double* scores, int32_t* num_tokens, const int32_t* block_table,
                           int32_t max_blocks, const int32_t* start_pos, int32_t num_blocks, void* plan,
                           size_t plan_bytes, void* stream) {
    g_msg[0] = 0;
    if (fs_status c = check_retrieve(store, batch, user, query, k, ids, scores, num_tokens)) return c;
    if (fs_status c = check_plan(store, batch, k, plan, plan_bytes)) return c;
    if (!block_table || !start_pos) return fail(FS_E_ARG, "null pointer argument");
    if (!aligned(block_table, 4) || !aligned(start_pos, 4))
        return fail(FS_E_ARG, "int32 argument not 4-byte aligned");
    if (max_blocks < 1) return fail(FS_E_BLOCKTABLE, "max_blocks %d < 1", max_blocks);
    if (num_blocks < 1) return fail(FS_E_BLOCKTABLE, "num_blocks %d < 1", num_blocks);
    if (k == 0 && !num_tokens) return FS_OK;
    RetrieveLaunch a{store, batch, user, query, k, ids, scores, num_tokens,
                     reinterpret_cast<hipStream_t>(stream)};
    if (k > 0) {
        // k = 0 plans nothing, as fs_plan_inject
        a.plan = plan;
        a.block_table = block_table;
        a.max_blocks = max_blocks;
        a.start_pos = start_pos;
        a.num_blocks = num_blocks;
    }
    hipError_t e = fsi_launch_retrieve(a);
    if (e != hipSuccess) return hip_fail(e, "retrieve launch");
    return FS_OK;
}

fs_status fs_inject_planned(const fs_store* store, int32_t layer_begin, int32_t layer_end, int32_t batch, int32_t k,
                            const void* plan, size_t plan_bytes, void* const* k_cache, void* const* v_cache,
                            int32_t num_blocks, void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_status c = check_plan(store, batch, k, plan, plan_bytes);
    if (c != FS_OK) return c;
    const fs_store_desc& d = store->desc;
    if (layer_begin < 0 || layer_end > d.num_layers || layer_begin >= layer_end)
        return fail(FS_E_RANGE, "layer range [%d, %d) invalid for %d layers", layer_begin, layer_end,
                    d.num_layers);
    if (!k_cache || !v_cache) return fail(FS_E_ARG, "null pointer argument");
    if (num_blocks < 1) return fail(FS_E_BLOCKTABLE, "num_blocks %d < 1", num_blocks);
    for (int l = layer_begin; l < layer_end; ++l) {
        if (!k_cache[l] || !v_cache[l]) return fail(FS_E_ARG, "layer %d cache pointer is null", l);
        if (!aligned(k_cache[l], 16) || !aligned(v_cache[l], 16))
            return fail(FS_E_ARG, "layer %d cache not 16-byte aligned", l);
    }
    if (k == 0) return FS_OK;
    InjectLaunch a{store, layer_begin, layer_end, batch, nullptr, nullptr, k, nullptr, 0, nullptr,
                   k_cache, v_cache, num_blocks, reinterpret_cast<hipStream_t>(stream)};
    a.plan_in = plan;
    hipError_t e = fsi_launch_inject(a);
    if (e != hipSuccess) return hip_fail(e, "inject launch");
    return FS_OK;
}

fs_status fs_inject(const fs_store* store, int32_t layer, int32_t batch, const int32_t* user,
                    const int32_t* ids, int32_t k, const int32_t* block_table, int32_t max_blocks,
                    const int32_t* start_pos, void* const* k_cache, void* const* v_cache,
                    int32_t num_blocks, void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const int32_t L = store->desc.num_layers;
    if (layer != FS_ALL_LAYERS && (layer < 0 || layer >= L))
        return fail(FS_E_RANGE, "layer %d outside [0, %d)", layer, L);
    const int32_t lb = layer == FS_ALL_LAYERS ? 0 : layer;
    const int32_t le = layer == FS_ALL_LAYERS ? L : layer + 1;
    return fs_inject_layers(store, lb, le, batch, user, ids, k, block_table, max_blocks, start_pos, k_cache,
                            v_cache, num_blocks, stream);
}

fs_status fs_fetch_async(const fs_store* store, int32_t batch, const int32_t* user,
                         const int32_t* ids, int32_t k, int32_t layer_begin, int32_t layer_end,
                         void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_store_desc& d = store->desc;
    if (d.kv_location != FS_KV_PINNED_HOST)
        return fail(FS_E_UNSUPPORTED, "fs_fetch_async needs a pinned-host store");
    if (batch < 1 || batch > d.max_batch)
        return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, d.max_batch);
    if (k < 0 || k > d.max_k) return fail(FS_E_RANGE, "k %d outside [0, %d]", k, d.max_k);
    if (layer_begin < 0 || layer_end > d.num_layers || layer_begin >= layer_end)
        return fail(FS_E_RANGE, "layer range [%d, %d) invalid", layer_begin, layer_end);
    if (layer_end - layer_begin > d.staging_layers)
        return fail(FS_E_RANGE, "layer range wider than staging_layers %d", d.staging_layers);
    if (!user || !ids) return fail(FS_E_ARG, "null pointer argument");
    if (!aligned(user, 4) || !aligned(ids, 4)) return fail(FS_E_ARG, "int32 argument not 4-byte aligned");
    if (k == 0) return FS_OK;
    FetchLaunch a{store, layer_begin, layer_end, batch, user, ids, k,
                  reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = fsi_launch_fetch(a);
    if (e != hipSuccess) return hip_fail(e, "fetch launch");
    return FS_OK;
}

fs_status fs_attend_prefill(const fs_store* store, int32_t batch, int32_t num_q_tokens,
                            int32_t num_q_heads, const void* q, const void* k_cache,
                            const void* v_cache, int32_t num_blocks, const int32_t* block_table,
                            int32_t max_blocks, const int32_t* ctx_begin, const int32_t* q_pos,
                            float scale, float* out, void* workspace, size_t workspace_bytes,
                            void* stream) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_store_desc& d = store->desc;
    if (d.head_dim != 128) return fail(FS_E_UNSUPPORTED, "attention needs head_dim 128 (store has %d)", d.head_dim);
    if (batch < 1 || batch > 65535) return fail(FS_E_RANGE, "batch %d outside [1, 65535]", batch);
    if (num_q_tokens < 1) return fail(FS_E_RANGE, "num_q_tokens %d < 1", num_q_tokens);
    if (num_q_heads < 1 || num_q_heads % d.num_kv_heads != 0)
        return fail(FS_E_RANGE, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                    d.num_kv_heads);
    if (num_q_heads / d.num_kv_heads > 8)
        return fail(FS_E_UNSUPPORTED, "more than 8 query heads per KV head");
    if (uint64_t(d.num_kv_heads) * d.head_dim * 2 >= (uint64_t(1) << 24) ||
        uint64_t(d.num_kv_heads) * d.head_dim * 2 * uint64_t(d.block_size) >= (uint64_t(1) << 32))
        return fail(FS_E_UNSUPPORTED, "a cache position (%d KV heads) reaches 16 MiB or a block of %d reaches 4 GiB",
                    d.num_kv_heads, d.block_size);
    if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(FS_E_ARG, "scale must be finite and > 0");
    if (!q || !k_cache || !v_cache || !block_table || !ctx_begin || !q_pos || !out)
        return fail(FS_E_ARG, "null pointer argument");
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
        return fail(FS_E_ARG, "q, caches and out must be 16-byte aligned");
    if (!aligned(block_table, 4) || !aligned(ctx_begin, 4) || !aligned(q_pos, 4))
        return fail(FS_E_ARG, "int32 argument not 4-byte aligned");
    if (max_blocks < 1) return fail(FS_E_BLOCKTABLE, "max_blocks %d < 1", max_blocks);
    if (num_blocks < 1) return fail(FS_E_BLOCKTABLE, "num_blocks %d < 1", num_blocks);
    if (workspace && !aligned(workspace, 16)) return fail(FS_E_ARG, "workspace not 16-byte aligned");
    AttendLaunch a{store, batch, num_q_tokens, num_q_heads, q, k_cache, v_cache, num_blocks,
                   block_table, max_blocks, ctx_begin, q_pos, scale, out,
                   workspace, workspace ? workspace_bytes : 0, reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = fsi_launch_attend(a);
    if (e != hipSuccess) return hip_fail(e, "attend launch");
    return FS_OK;
}

fs_status fs_attend_workspace_size(const fs_store* store, int32_t batch, int32_t num_q_tokens,
                                   int32_t num_q_heads, size_t* bytes) {
    g_msg[0] = 0;
    if (!store || !bytes) return fail(FS_E_ARG, "null pointer argument");
    if (batch < 1 || num_q_tokens < 1 || num_q_heads < 1)
        return fail(FS_E_RANGE, "batch, num_q_tokens and num_q_heads must be >= 1");
    *bytes = fsi_attend_workspace_bytes(fsi_attend_splits(store, batch, num_q_tokens, num_q_heads, 0), batch,
                                        num_q_tokens, num_q_heads);
    return FS_OK;
}

fs_status fs_ingest_init(fs_store* store, const int32_t* live_counts, int64_t rows_used, void* stream) {
    g_msg[0] = 0;
    if (!store || !live_counts) return fail(FS_E_ARG, "null pointer argument");
    const fs_store_desc& d = store->desc;
    if (rows_used < 0 || rows_used > d.num_tokens)
        return fail(FS_E_RANGE, "rows_used %lld outside [0, num_tokens]", static_cast<long long>(rows_used));
    for (int u = 0; u < d.num_users; ++u) {
        const int64_t cap = store->h_user_begin[u + 1] - store->h_user_begin[u];
        if (live_counts[u] < 0 || live_counts[u] > cap)
            return fail(FS_E_RANGE, "user %d: %d live facts, capacity %lld", u, live_counts[u],
                        static_cast<long long>(cap));
        for (int32_t j = 0; j < live_counts[u]; ++j) {
            const int64_t f = store->h_user_begin[u] + j;
            if (store->h_fact_begin[f] + store->h_fact_len[f] > rows_used)
                return fail(FS_E_RANGE, "live fact %lld uses rows at or past rows_used", static_cast<long long>(f));
        }
    }
    store->h_user_count.assign(live_counts, live_counts + d.num_users);
    store->next_row = rows_used;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(store->d_user_count, live_counts, sizeof(int32_t) * d.num_users,
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "user counts upload");
    return FS_OK;
}

fs_status fs_ingest_facts(fs_store* store, int32_t n, const int32_t* user, const void* const* k_window,
                          const void* const* v_window, const int64_t* keep_begin, const int32_t* keep_len,
                          const float* emb, void* stream, int32_t* fact_ids) {
    g_msg[0] = 0;
    if (!store || !user || !k_window || !v_window || !keep_begin || !keep_len || !emb || !fact_ids)
        return fail(FS_E_ARG, "null pointer argument");
    const fs_store_desc& d = store->desc;
    if (n < 1 || n > kIngestMax) return fail(FS_E_RANGE, "n %d outside [1, %d]", n, kIngestMax);
    if (!aligned(emb, 16)) return fail(FS_E_ARG, "emb not 16-byte aligned");
    for (int l = 0; l < d.num_layers; ++l) {
        if (!k_window[l] || !v_window[l]) return fail(FS_E_ARG, "layer %d window pointer is null", l);
        if (!aligned(k_window[l], 16) || !aligned(v_window[l], 16))
            return fail(FS_E_ARG, "layer %d window not 16-byte aligned", l);
    }
    // plan every fact before touching anything: slots and rows
    std::vector<int32_t> count = store->h_user_count;
    int64_t row = store->next_row;
    std::vector<IngestItem> items(n);
    int32_t max_len = 0;
    for (int i = 0; i < n; ++i) {
        const int u = user[i];
        if (u < 0 || u >= d.num_users) return fail(FS_E_RANGE, "fact %d: user %d outside [0, %d)", i, u, d.num_users);
        if (keep_len[i] < 1 || keep_len[i] > store->max_fact_len)
            return fail(FS_E_RANGE, "fact %d: length %d outside [1, %d]", i, keep_len[i], store->max_fact_len);
        if (keep_begin[i] < 0) return fail(FS_E_RANGE, "fact %d: negative window row", i);
        const int64_t cap = store->h_user_begin[u + 1] - store->h_user_begin[u];
        if (count[u] >= cap) return fail(FS_E_RANGE, "user %d has no free fact slot", u);
        if (row + keep_len[i] > d.num_tokens) return fail(FS_E_RANGE, "arenas full (%lld rows)",
                                                          static_cast<long long>(d.num_tokens));
        items[i].src_row = keep_begin[i];
        items[i].dst_row = row;
        items[i].len = keep_len[i];
        items[i].slot = static_cast<int32_t>(store->h_user_begin[u] + count[u]);
        items[i].emb_row = i;
        items[i].pad = 0;
        ++count[u];
        row += keep_len[i];
        max_len = std::max(max_len, keep_len[i]);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // descriptors and counts go through pinned host buffers, so the copies
    // are asynchronous; a buffer is refilled only after the previous call's
    // copies out of it have completed
    hipError_t e = hipSuccess;
    if (!store->h_ingest_items) {
        e = hipHostMalloc(&store->h_ingest_items, sizeof(IngestItem) * kIngestMax, hipHostMallocDefault);
        if (e == hipSuccess)
            e = hipHostMalloc(reinterpret_cast<void**>(&store->h_ingest_counts), sizeof(int32_t) * d.num_users,
                              hipHostMallocDefault);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&store->ingest_copied, hipEventDisableTiming);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(FS_E_NOMEM, "ingest staging: %s", hipGetErrorString(e));
        }
    } else {
        e = hipEventSynchronize(store->ingest_copied);
        if (e != hipSuccess) return hip_fail(e, "ingest staging wait");
    }
    std::memcpy(store->h_ingest_items, items.data(), sizeof(IngestItem) * n);
    std::memcpy(store->h_ingest_counts, count.data(), sizeof(int32_t) * d.num_users);
    e = hipMemcpyAsync(store->d_ingest_items, store->h_ingest_items, sizeof(IngestItem) * n,
                       hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(ingest descriptors)");
    IngestLaunch a{store, n, max_len, k_window, v_window, emb, s};
    e = fsi_launch_ingest(a);
    if (e != hipSuccess) return hip_fail(e, "ingest launch");
    e = hipMemcpyAsync(store->d_user_count, store->h_ingest_counts, sizeof(int32_t) * d.num_users,
                       hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipEventRecord(store->ingest_copied, s);
    if (e != hipSuccess) return hip_fail(e, "ingest");
    for (int i = 0; i < n; ++i) {
        store->h_fact_begin[items[i].slot] = items[i].dst_row;
        store->h_fact_len[items[i].slot] = items[i].len;
        fact_ids[i] = items[i].slot;
    }
    store->h_user_count = count;
    store->next_row = row;
    return FS_OK;
}

fs_status fs_evict_fact(fs_store* store, int32_t fact_id, void* stream, int32_t* moved_from) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    const fs_store_desc& d = store->desc;
    if (fact_id < 0 || fact_id >= d.num_facts) return fail(FS_E_RANGE, "fact %d outside [0, %lld)", fact_id,
                                                            static_cast<long long>(d.num_facts));
    const auto it = std::upper_bound(store->h_user_begin.begin(), store->h_user_begin.end(), int64_t(fact_id));
    const int u = static_cast<int>(it - store->h_user_begin.begin()) - 1;
    const int64_t first = store->h_user_begin[u];
    if (fact_id >= first + store->h_user_count[u]) return fail(FS_E_RANGE, "fact %d is not live", fact_id);
    const int64_t last = first + store->h_user_count[u] - 1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    if (last != fact_id) {
        // the user's last live fact moves into the freed slot
        store->h_fact_begin[fact_id] = store->h_fact_begin[last];
        store->h_fact_len[fact_id] = store->h_fact_len[last];
        e = hipMemcpyAsync(store->d_fact_begin + fact_id, &store->h_fact_begin[fact_id], sizeof(int64_t),
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(store->d_fact_len + fact_id, &store->h_fact_len[fact_id], sizeof(int32_t),
                               hipMemcpyHostToDevice, s);
        if (e == hipSuccess)
            e = hipMemcpyAsync(const_cast<float*>(store->emb) + int64_t(fact_id) * d.embed_dim,
                               store->emb + last * d.embed_dim, sizeof(float) * d.embed_dim,
                               hipMemcpyDeviceToDevice, s);
    }
    --store->h_user_count[u];
    if (e == hipSuccess)
        e = hipMemcpyAsync(store->d_user_count + u, &store->h_user_count[u], sizeof(int32_t),
                           hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);   // the host sources above must stay unchanged until copied
    if (e != hipSuccess) return hip_fail(e, "eviction copies");
    if (moved_from) *moved_from = last != fact_id ? static_cast<int32_t>(last) : -1;
    return FS_OK;
}

fs_status fs_store_live(const fs_store* store, int32_t user, int32_t* live, int64_t* rows_used) {
    g_msg[0] = 0;
    if (!store) return fail(FS_E_ARG, "null store");
    if (user < 0 || user >= store->desc.num_users) return fail(FS_E_RANGE, "user %d out of range", user);
    if (live) *live = store->h_user_count[user];
    if (rows_used) *rows_used = store->next_row;
    return FS_OK;
}

static void free_ivf(fs_ivf* ix) {
    if (!ix) return;
    void* bufs[] = {ix->d_cent, ix->d_list_begin, ix->d_members, ix->d_emb_sorted, ix->d_cent_range,
                    ix->d_zero_users, ix->d_cscores, ix->d_chosen, ix->d_cand_scores, ix->d_cand_ids,
                    ix->d_counts, ix->d_offs};
    for (void* p : bufs)
        if (p) (void)hipFree(p);
    delete ix;
}

fs_status fs_ivf_build(const fs_store* store, int32_t user, int32_t nlist, int32_t iters,
                       int32_t max_nprobe, void* stream, fs_ivf** out) {
    g_msg[0] = 0;
    if (!store || !out) return fail(FS_E_ARG, "null pointer argument");
    *out = nullptr;
    const fs_store_desc& d = store->desc;
    if (user < 0 || user >= d.num_users) return fail(FS_E_RANGE, "user %d outside [0, %d)", user, d.num_users);
    if (nlist < 1 || nlist > 4096) return fail(FS_E_RANGE, "nlist %d outside [1, 4096]", nlist);
    if (iters < 0 || iters > 100) return fail(FS_E_RANGE, "iters %d outside [0, 100]", iters);
    if (max_nprobe < 1 || max_nprobe > nlist)
        return fail(FS_E_RANGE, "max_nprobe %d outside [1, nlist]", max_nprobe);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int64_t range[2] = {0, 0};
    hipError_t e = hipMemcpy(range, store->d_user_begin + user, sizeof(range), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(user range)");
    const int64_t n = store->h_user_count[user];
    if (n < nlist) return fail(FS_E_RANGE, "user %d has %lld facts, fewer than nlist %d", user,
                               static_cast<long long>(n), nlist);
    if (n > INT32_MAX / 2) return fail(FS_E_RANGE, "user too large for one index");
    fs_ivf* ix = new (std::nothrow) fs_ivf();
    if (!ix) return fail(FS_E_NOMEM, "host allocation");
    ix->store = store;
    ix->user = user;
    ix->nlist = nlist;
    ix->num_facts = static_cast<int32_t>(n);
    ix->max_nprobe = max_nprobe;
    ix->iters = iters;
    ix->max_batch = d.max_batch;
    ix->fact_base = range[0];
    const size_t E = d.embed_dim;
    struct { void** p; size_t bytes; } a1[] = {
        {(void**)&ix->d_cent, sizeof(float) * nlist * E},
        {(void**)&ix->d_list_begin, sizeof(int32_t) * (nlist + 1)},
        {(void**)&ix->d_members, sizeof(int32_t) * size_t(n)},
        {(void**)&ix->d_emb_sorted, sizeof(float) * size_t(n) * E},
        {(void**)&ix->d_cent_range, sizeof(int64_t) * 2},
        {(void**)&ix->d_zero_users, sizeof(int32_t) * size_t(d.max_batch)},
        {(void**)&ix->d_cscores, sizeof(double) * size_t(d.max_batch) * nlist},
        {(void**)&ix->d_chosen, sizeof(int32_t) * size_t(d.max_batch) * max_nprobe},
        {(void**)&ix->d_counts, sizeof(int32_t) * size_t(d.max_batch)},
        {(void**)&ix->d_offs, sizeof(int32_t) * size_t(d.max_batch) * (max_nprobe + 1)},
    };
    for (auto& a : a1) {
        e = hipMalloc(a.p, a.bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            free_ivf(ix);
            return fail(FS_E_NOMEM, "hipMalloc(index, %zu bytes): %s", a.bytes, hipGetErrorString(e));
        }
    }
    const int64_t cr[2] = {0, nlist};
    std::vector<int32_t> zeros(size_t(d.max_batch), 0);
    e = hipMemcpyAsync(ix->d_cent_range, cr, sizeof(cr), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(ix->d_zero_users, zeros.data(), sizeof(int32_t) * zeros.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = fsi_ivf_build(ix, s);       // synchronises s
    if (e != hipSuccess) {
        free_ivf(ix);
        return hip_fail(e, "index build");
    }
    const int64_t stride = int64_t(max_nprobe) * ix->max_list;
    ix->cand_stride = static_cast<int32_t>(std::min<int64_t>(stride, n));
    struct { void** p; size_t bytes; } a2[] = {
        {(void**)&ix->d_cand_scores, sizeof(double) * size_t(d.max_batch) * ix->cand_stride},
        {(void**)&ix->d_cand_ids, sizeof(int32_t) * size_t(d.max_batch) * ix->cand_stride},
    };
    for (auto& a : a2) {
        e = hipMalloc(a.p, a.bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            free_ivf(ix);
            return fail(FS_E_NOMEM, "hipMalloc(probe scratch, %zu bytes): %s", a.bytes, hipGetErrorString(e));
        }
    }
    *out = ix;
    return FS_OK;
}

fs_status fs_ivf_destroy(fs_ivf* ix) {
    g_msg[0] = 0;
    if (!ix) return FS_OK;
    free_ivf(ix);
    return FS_OK;
}

fs_status fs_ivf_arrays(const fs_ivf* ix, fs_ivf_view* view) {
    g_msg[0] = 0;
    if (!ix || !view) return fail(FS_E_ARG, "null pointer argument");
    view->user = ix->user;
    view->nlist = ix->nlist;
    view->num_facts = ix->num_facts;
    view->max_list = ix->max_list;
    view->max_nprobe = ix->max_nprobe;
    view->centroids = ix->d_cent;
    view->list_begin = ix->d_list_begin;
    view->members = ix->d_members;
    return FS_OK;
}

fs_status fs_ivf_retrieve_topk(const fs_store* store, const fs_ivf* ix, int32_t batch, const float* query,
                               int32_t nprobe, int32_t k, int32_t* ids, double* scores,
                               int32_t* num_tokens, void* stream) {
    g_msg[0] = 0;
    if (!store || !ix) return fail(FS_E_ARG, "null store or index");
    if (ix->store != store) return fail(FS_E_ARG, "index was built on another store");
    const fs_store_desc& d = store->desc;
    if (batch < 1 || batch > d.max_batch) return fail(FS_E_RANGE, "batch %d outside [1, %d]", batch, d.max_batch);
    if (nprobe < 1 || nprobe > ix->max_nprobe)
        return fail(FS_E_RANGE, "nprobe %d outside [1, %d]", nprobe, ix->max_nprobe);
    if (k < 0 || k > d.max_k) return fail(FS_E_RANGE, "k %d outside [0, %d]", k, d.max_k);
    if (!query) return fail(FS_E_ARG, "null query");
    if (!aligned(query, 16)) return fail(FS_E_ARG, "query not 16-byte aligned");
    if (k > 0 && !ids) return fail(FS_E_ARG, "null ids");
    if ((ids && !aligned(ids, 4)) || (scores && !aligned(scores, 8)) || (num_tokens && !aligned(num_tokens, 4)))
        return fail(FS_E_ARG, "output not aligned");
    if (k == 0 && !num_tokens) return FS_OK;
    IvfProbeLaunch a{ix, batch, query, nprobe, k, ids, scores, num_tokens, reinterpret_cast<hipStream_t>(stream)};
    hipError_t e = fsi_launch_ivf_probe(a);
    if (e != hipSuccess) return hip_fail(e, "index probe launch");
    return FS_OK;
}

fs_status fs_check_block_tables(int32_t batch, const int32_t* block_table, int32_t max_blocks,
                                const int32_t* start_pos, const int32_t* num_tokens, int32_t block_size,
                                int32_t num_blocks, int32_t* conflict) {
    g_msg[0] = 0;
    if (conflict)
        for (int i = 0; i < 4; ++i) conflict[i] = -1;
    if (batch < 0) return fail(FS_E_ARG, "batch %d < 0", batch);
    if (batch > 0 && (!block_table || !start_pos || !num_tokens)) return fail(FS_E_ARG, "null pointer argument");
    if (max_blocks < 1) return fail(FS_E_ARG, "max_blocks %d < 1", max_blocks);
    if (!pow2(block_size)) return fail(FS_E_ARG, "block_size %d is not a power of two", block_size);
    if (num_blocks < 1) return fail(FS_E_ARG, "num_blocks %d < 1", num_blocks);
    auto report = [&](int32_t b, int32_t j, int32_t id, int32_t other, const char* what) {
        if (conflict) {
            conflict[0] = b;
            conflict[1] = j;
            conflict[2] = id;
            conflict[3] = other;
        }
        return fail(FS_E_BLOCKTABLE, "request %d, logical block %d (block id %d): %s", b, j, id, what);
    };
    // every written (request, logical block) with its physical id, then
    // sorted by id: a repeated id is an alias
    struct Use {
        int32_t id, b, j;
    };
    std::vector<Use> uses;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t s = start_pos[b], L = num_tokens[b];
        if (L <= 0) continue;
        if (s < 0) return report(b, -1, -1, -1, "negative start position");
        const int64_t first = s / block_size, last = (s + L - 1) / block_size;
        if (last >= max_blocks) return report(b, static_cast<int32_t>(last), -1, -1, "beyond the block table");
        for (int64_t j = first; j <= last; ++j) {
            const int32_t id = block_table[int64_t(b) * max_blocks + j];
            if (id < 0 || id >= num_blocks)
                return report(b, static_cast<int32_t>(j), id, -1, "block id outside [0, num_blocks)");
            uses.push_back(Use{id, b, static_cast<int32_t>(j)});
        }
    }
    std::stable_sort(uses.begin(), uses.end(), [](const Use& x, const Use& y) { return x.id < y.id; });
    for (size_t i = 1; i < uses.size(); ++i)
        if (uses[i].id == uses[i - 1].id)
            return report(uses[i].b, uses[i].j, uses[i].id, uses[i - 1].b, "block also written by another entry");
    return FS_OK;
}

fs_status fs_poll_errors(const fs_store* store, void* stream, uint32_t* flags) {
    g_msg[0] = 0;
    if (!store || !flags) return fail(FS_E_ARG, "null pointer argument");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t v = 0, zero = 0;
    e = hipMemcpy(&v, store->d_err, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
    e = hipMemcpy(store->d_err, &zero, sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy(clear error word)");
    *flags = v;
    if (v) return fail(FS_E_DEVICE, "device error bits 0x%x", v);
    return FS_OK;
}

}  // extern "C"
