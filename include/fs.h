/*
 * fs.h — C ABI of the fact-store KV-injection library (AMD Instinct MI355X, gfx950).
 *
 * The library implements the serving-time hot path of KV injection as the
 * InferScale pages describe it ("InferScale: GPU-Native KV Injection for
 * Personalized LLM Serving", Li & Pandey, arXiv 2607.27090):
 *
 *   precompute each fact's KV, keep it on the GPU next to a semantic
 *   embedding, retrieve the relevant facts at serving time and inject their
 *   KV straight into the paged KV cache
 *       (astralor.com feed item, "Full text" = the paper's abstract);
 *   keys are stored before RoPE; at serving time the retrieved facts form one
 *   contiguous segment and every stored key is rotated to its new position
 *   (Chunked RoPE); the composed K/V is scatter-copied into the paged cache
 *       (gist.science technical summary, "Phase En-ligne" / "Fase Online");
 *   the store may live in host DRAM when the GPU is too small
 *       (gist.science summary, "Résultats" / "Resultados", scalability item).
 *
 * Conventions for every entry point
 *   - Plain pointers and sizes only.  "device" pointers are HIP device
 *     memory of the current device; "host" pointers are ordinary host memory
 *     read during the call and not kept.
 *   - The caller owns every buffer it passes (embeddings, K/V arenas, caches,
 *     ids, block tables, queries) and keeps the store's buffers alive until
 *     fs_destroy_store.  The library owns only what it allocates itself:
 *     metadata copies, the RoPE frequency table, an error word and scratch.
 *   - Stream arguments are hipStream_t values passed as void* (NULL = the
 *     legacy default stream).  Every call except create/destroy/poll only
 *     enqueues work and returns; results are ready when the stream reaches
 *     that point.
 *   - Concurrency on one store (not detected): fs_retrieve_topk calls share
 *     the score scratch, so they must not overlap one another; on pinned
 *     stores fs_inject calls share the plan scratch and the staging ring, so
 *     they must not overlap one another or an fs_fetch_async.  On device
 *     stores each fs_inject call composes its plan into one of the store's
 *     plan slots (FS_PLAN_SLOTS of them): a slot goes back to the stream that
 *     used it last with no synchronisation (stream order protects it), and
 *     to another stream only after that stream waits, on the device, for the
 *     slot's last use.  So one stream may inject while another retrieves for
 *     a later request (the caller orders each inject after the retrieval
 *     that produced its ids, e.g. with an event), and injects on up to
 *     FS_PLAN_SLOTS streams run side by side when they write disjoint cache
 *     blocks.  The slot choice is guarded by a mutex, so host threads may
 *     call fs_inject on one store.  Several stores may be created over the
 *     same arenas and embeddings (each with its own scratch, e.g. one per
 *     stream) while none of them ingests or evicts: each keeps its own copy
 *     of the metadata.
 *   - Errors: a call returns a status.  Host-checkable errors return before
 *     anything is enqueued and nothing is written.  Conditions only the GPU
 *     can see set bits in the store's device error word (fs_poll_errors) and
 *     the offending request writes nothing.  Nothing is thrown across the
 *     ABI.  fs_last_error_message() gives the detail of the last failure on
 *     the calling thread.
 *
 * Data layout (bf16 = 16-bit brain float; all bf16 buffers 16-byte aligned)
 *   fact f has fact_len[f] tokens; facts are stored back to back in fact
 *   order, so fact f occupies arena rows [sum_{g<f} fact_len[g], ... + fact_len[f]).
 *   user u owns facts [user_fact_begin[u], user_fact_begin[u+1]).
 *   K/V arena of one layer:   bf16 [num_tokens][num_kv_heads][head_dim]
 *                             (keys un-rotated, values raw)
 *   embeddings:               fp32 [num_facts][embed_dim], row-major
 *   paged cache of one layer: bf16 [num_blocks][block_size][num_kv_heads][head_dim]
 *   block table:              int32 [batch][max_blocks]; absolute position p of
 *                             request b lives in block block_table[b][p / block_size],
 *                             slot p % block_size.
 */
#ifndef FS_H_
#define FS_H_

#include <stddef.h>
#include <stdint.h>

/* the library is built with hidden visibility; only these entry points are exported */
#if defined(__GNUC__) || defined(__clang__)
#define FS_API __attribute__((visibility("default")))
#else
#define FS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fs_store fs_store;      /* opaque, library-owned */
typedef int32_t fs_status;

/* ---- status codes ---------------------------------------------------- */
#define FS_OK              0
#define FS_E_ARG           1   /* null/misaligned pointer, bad shape or size   */
#define FS_E_RANGE         2   /* layer, batch or k outside the store's limits */
#define FS_E_BLOCKTABLE    3   /* block table arguments unusable (host check)  */
#define FS_E_NOMEM         4   /* device allocation failed                     */
#define FS_E_HIP           5   /* a HIP runtime call failed                    */
#define FS_E_DEVICE        6   /* fs_poll_errors: device error bits were set   */
#define FS_E_UNSUPPORTED   7   /* valid request this build does not implement  */

/* ---- device error bits (fs_poll_errors) ------------------------------ */
#define FS_ERR_USER        0x01u  /* user index outside [0, num_users)            */
#define FS_ERR_FACT_ID     0x02u  /* id not a fact of the request's user, or a -1
                                     pad followed by a real id                     */
#define FS_ERR_START_POS   0x04u  /* start_pos < 0, or start_pos + L > INT32_MAX   */
#define FS_ERR_BLOCK_SHORT 0x08u  /* block table has fewer than
                                     ceil((start_pos + L) / block_size) entries   */
#define FS_ERR_BLOCK_ID    0x10u  /* a used block id outside [0, num_blocks)       */
#define FS_ERR_STAGING     0x20u  /* pinned store: inject ids differ from the ids
                                     the staging slot was fetched for              */
#define FS_ERR_PLAN        0x40u  /* fs_inject_planned: the plan was not written by
                                     fs_plan_inject of this store for this batch
                                     and k, or was checked against more cache
                                     blocks than the caches hold; nothing is
                                     written from it                               */

#define FS_ALL_LAYERS      (-1)
#define FS_MAX_LAYERS      128
#define FS_MAX_K           1024
#define FS_PLAN_SLOTS      4      /* fs_inject plan slots per device store     */
#define FS_NOALLOC_PLAN_BYTES 0x400000u  /* fs_inject_noalloc plan buffer per GPU (4 MiB) */

#define FS_KV_DEVICE       0      /* K/V arenas in device memory              */
#define FS_KV_PINNED_HOST  1      /* K/V arenas in page-locked host memory    */

typedef struct fs_store_desc {
    int32_t num_layers;      /* 1 .. FS_MAX_LAYERS                               */
    int32_t num_kv_heads;    /* >= 1; num_kv_heads * head_dim <= 8192          */
    int32_t head_dim;        /* 64, 128 or 256 (rotate-half pairs i, i+head_dim/2) */
    int32_t embed_dim;       /* multiple of 4, 4 .. 4096                         */
    double  rope_theta;      /* RoPE base, > 1 (w_i = theta^(-2i/head_dim))      */
    int32_t block_size;      /* paged-cache block size, power of two, 1 .. 1024  */
    int32_t kv_location;     /* FS_KV_DEVICE or FS_KV_PINNED_HOST                */
    int32_t num_users;       /* >= 1                                             */
    int32_t max_batch;       /* largest batch any call will pass, >= 1           */
    int32_t max_k;           /* largest k any call will pass, 1 .. FS_MAX_K      */
    int32_t staging_layers;  /* pinned stores: layers the device staging ring
                                holds (1 .. num_layers); ignored otherwise       */
    int64_t num_facts;       /* >= 1                                             */
    int64_t num_tokens;      /* arena rows, >= sum of fact_len; rows past the sum
                                are free for fs_ingest_facts                    */
} fs_store_desc;

/*
 * fs_create_store — register a fact store (InferScale abstract: each fact's KV
 * is precomputed and stored alongside a semantic embedding on the GPU;
 * "Stockage Pré-RoPE": keys intercepted before RoPE plus raw values).
 *
 *   desc             host; shapes and limits (see fs_store_desc)
 *   user_fact_begin  host int64 [num_users + 1]; 0, non-decreasing, ends at num_facts
 *   fact_len         host int32 [num_facts]; every length >= 1
 *   emb              device fp32 [num_facts][embed_dim], 16-byte aligned;
 *                    rows are expected L2-normalised (not checked)
 *   k_pre, v         host arrays of num_layers pointers to the per-layer K and V
 *                    arenas, bf16 [num_tokens][num_kv_heads][head_dim], 16-byte
 *                    aligned; device memory for FS_KV_DEVICE, page-locked host
 *                    memory (hipHostMalloc / pinned) for FS_KV_PINNED_HOST
 *   stream           stream used for the metadata uploads (synchronised before return)
 *   out              receives the handle; untouched on failure
 *
 * The store keeps the emb/k_pre/v pointers (not the data).  Allocates: fact
 * offsets and lengths, user offsets, the fp64 frequency table, the error word,
 * score scratch [max_batch][largest user], and for pinned stores the staging
 * ring [staging_layers][max_batch][max_k * longest fact][heads][head_dim] x2.
 * Errors: FS_E_ARG (bad desc/pointer/alignment/metadata), FS_E_UNSUPPORTED
 * (head_dim or embed_dim not built), FS_E_NOMEM, FS_E_HIP.
 */
FS_API fs_status fs_create_store(const fs_store_desc* desc,
                          const int64_t* user_fact_begin,
                          const int32_t* fact_len,
                          const float* emb,
                          const void* const* k_pre,
                          const void* const* v,
                          void* stream,
                          fs_store** out);

/* fs_destroy_store — free everything the library allocated for the store
 * (waits for the device).  NULL is accepted and ignored. */
FS_API fs_status fs_destroy_store(fs_store* store);

/*
 * fs_retrieve_topk — GPU-resident semantic retrieval with budget k
 * (gist.science summary, "Problématique": k retrieved facts;
 * "Contributions Clés": retrieval index and KV store both on the GPU).
 *
 * For each request b: s_i = <emb[i], query[b]> over the facts i of user[b],
 * each fp32*fp32 product exact and summed in fp64; selects the
 * k' = min(k, N_user) best facts ordered by (score descending, fact id
 * ascending).
 *
 *   batch       1 .. max_batch
 *   user        device int32 [batch]
 *   query       device fp32 [batch][embed_dim], 16-byte aligned
 *   k           0 .. max_k
 *   ids         device int32 [batch][k]: global fact ids in rank order, -1 past k'
 *   scores      device fp64 [batch][k] or NULL: the scores, -inf past k'
 *   num_tokens  device int32 [batch] or NULL: L_b = sum of the selected facts' lengths
 *
 * A bad user index sets FS_ERR_USER; that request gets ids -1, scores -inf
 * and num_tokens 0.  Errors: FS_E_ARG, FS_E_RANGE, FS_E_HIP.
 */
FS_API fs_status fs_retrieve_topk(const fs_store* store, int32_t batch,
                           const int32_t* user, const float* query, int32_t k,
                           int32_t* ids, double* scores, int32_t* num_tokens,
                           void* stream);

/*
 * fs_inject — Chunked RoPE + scatter-copy into the paged KV cache
 * (gist.science summary, "Phase En-ligne": "Rotation Dynamique" and
 * "Injection"; Theorem 6 as described there: the re-rotation is exact).
 *
 * For each request b the facts ids[b][0..] (up to the first -1) are laid end
 * to end from position start_pos[b]: token t of the segment has position
 * p = start_pos[b] + t.  For every written layer l and head h:
 *   K cache (block_table[b][p / bs], slot p % bs, h) =
 *       bf16_rne( R(p) * k_pre[l][row(t)][h] )     rotate-half RoPE,
 *       R(p) rotating (x_i, x_{i+D/2}) by angle p * theta^(-2i/D), evaluated in
 *       fp64 and rounded once to bf16 (round to nearest, ties to even)
 *   V cache (same address) = v[l][row(t)][h]            (bytes, unchanged)
 * Every other cache byte is left untouched.
 *
 * Enqueues two kernels on `stream`: the plan (composition and validation of
 * every request, one small block each) into a plan slot of the store, then
 * the injection, which streams K and V rows through that plan.
 *
 *   layer        0 .. num_layers-1, or FS_ALL_LAYERS
 *   batch        1 .. max_batch
 *   user         device int32 [batch]; ids must belong to the request's user
 *   ids          device int32 [batch][k] (e.g. fs_retrieve_topk's output)
 *   k            0 .. max_k (0: nothing is enqueued)
 *   block_table  device int32 [batch][max_blocks]
 *   start_pos    device int32 [batch]
 *   k_cache, v_cache  host arrays of num_layers device pointers, each
 *                bf16 [num_blocks][block_size][num_kv_heads][head_dim],
 *                16-byte aligned; entries of layers not written may be NULL
 *   num_blocks   physical blocks per layer cache, >= 1
 * Pinned stores read the staging slot layer % staging_layers filled by
 * fs_fetch_async with the same ids (else FS_ERR_STAGING).
 * Block ids used by one call must be distinct across its requests (caller's
 * contract, not checked).  Device-checked: FS_ERR_USER, FS_ERR_FACT_ID,
 * FS_ERR_START_POS, FS_ERR_BLOCK_SHORT, FS_ERR_BLOCK_ID, FS_ERR_STAGING — the
 * request then writes nothing.  Errors: FS_E_ARG, FS_E_RANGE, FS_E_BLOCKTABLE,
 * FS_E_HIP.
 */
FS_API fs_status fs_inject(const fs_store* store, int32_t layer, int32_t batch,
                    const int32_t* user, const int32_t* ids, int32_t k,
                    const int32_t* block_table, int32_t max_blocks,
                    const int32_t* start_pos,
                    void* const* k_cache, void* const* v_cache,
                    int32_t num_blocks, void* stream);

/*
 * fs_inject_layers — fs_inject over the layers [layer_begin, layer_end) in
 * one call (one plan, one inject launch; same passages, same per-layer
 * result, same checks and errors).  A layer-pipelined caller injects the
 * first layers alone and the rest in larger chunks: one call per chunk
 * instead of one per layer.
 *   0 <= layer_begin < layer_end <= num_layers, else FS_E_RANGE.  On pinned
 *   stores every layer of the range reads its own staging slot, so the range
 *   spans at most staging_layers layers (FS_ERR_STAGING otherwise).
 */
FS_API fs_status fs_inject_layers(const fs_store* store, int32_t layer_begin, int32_t layer_end,
                           int32_t batch, const int32_t* user, const int32_t* ids, int32_t k,
                           const int32_t* block_table, int32_t max_blocks,
                           const int32_t* start_pos,
                           void* const* k_cache, void* const* v_cache,
                           int32_t num_blocks, void* stream);

/*
 * fs_inject_noalloc — fs_inject for callers that cannot allocate device
 * memory while they run (code captured into a HIP graph, a serving loop that
 * must not call hipMalloc, a harness that forbids it).  Same arguments,
 * result, host checks and device-checked errors as fs_inject; the call
 * allocates nothing.  Its plan goes into one static device buffer of
 * FS_NOALLOC_PLAN_BYTES (4 MiB) per GPU instead of a plan slot of the store:
 *   - a batch whose plan (fs_inject_plan_size(batch) bytes) exceeds it
 *     returns FS_E_RANGE and enqueues nothing;
 *   - every fs_inject_noalloc call on a GPU, from any store, uses that one
 *     buffer, so calls that overlap on one GPU (different streams, or
 *     different host threads) race: the caller orders them;
 *   - the buffer keeps the last call's plan; each call writes every entry
 *     its injection reads, so nothing needs clearing.
 * The buffer's device address is looked up on the first call on each GPU.
 */
FS_API fs_status fs_inject_noalloc(const fs_store* store, int32_t layer, int32_t batch,
                                   const int32_t* user, const int32_t* ids, int32_t k,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* start_pos, void* const* k_cache,
                                   void* const* v_cache, int32_t num_blocks, void* stream);

/*
 * fs_plan_inject, fs_inject_planned — fs_inject's two kernels as two calls,
 * with the plan (the segment of ids[b] laid from start_pos[b], validated;
 * same passages as fs_inject) in a buffer the caller owns.  A serving loop
 * plans request i + 1 while request i injects, and one plan serves any
 * number of layer ranges (a layer-pipelined forward).  fs_plan_inject
 * followed by fs_inject_planned writes exactly what fs_inject_layers writes
 * with the same arguments.  Device stores only (FS_E_UNSUPPORTED otherwise).
 *
 * fs_inject_plan_size: bytes of a plan for `batch` requests (1 .. max_batch).
 * The plan holds a header (this store, batch, k and the num_blocks it was
 * checked against), per request its segment length (0 when rejected) and
 * start position, and every segment token's arena row and cache slot.
 *
 * fs_plan_inject: arguments as fs_inject's; plan is device memory of at least
 *   fs_inject_plan_size(batch) bytes, 16-byte aligned (else FS_E_RANGE /
 *   FS_E_ARG), owned by the caller.  Device-checked as fs_inject
 *   (FS_ERR_USER, FS_ERR_FACT_ID, FS_ERR_START_POS, FS_ERR_BLOCK_SHORT,
 *   FS_ERR_BLOCK_ID): a rejected request's length is 0, so no inject from
 *   the plan writes anything for it.  k = 0 enqueues nothing.
 *
 * fs_inject_planned: the layers [layer_begin, layer_end) from a plan that
 *   fs_plan_inject wrote earlier in stream order (or after an event) with the
 *   same batch and k; k_cache and v_cache as fs_inject's, each holding
 *   num_blocks blocks.  Device-checked: a plan whose header does not name
 *   this store, batch and k, or that was checked against more than
 *   num_blocks blocks (including a buffer fs_plan_inject never wrote), sets
 *   FS_ERR_PLAN and writes nothing; every row the inject touches is also
 *   bounds-checked against the arenas and caches (FS_ERR_PLAN).  A plan may
 *   be used for any number of layer ranges; it must not be rewritten while
 *   an inject reads it, and a plan of earlier requests stays valid for them
 *   only (the caller's responsibility).  Errors: FS_E_ARG, FS_E_RANGE,
 *   FS_E_BLOCKTABLE, FS_E_UNSUPPORTED, FS_E_HIP.
 */
FS_API fs_status fs_inject_plan_size(const fs_store* store, int32_t batch, size_t* bytes);
FS_API fs_status fs_plan_inject(const fs_store* store, int32_t batch, const int32_t* user,
                                const int32_t* ids, int32_t k, const int32_t* block_table,
                                int32_t max_blocks, const int32_t* start_pos, int32_t num_blocks,
                                void* plan, size_t plan_bytes, void* stream);
FS_API fs_status fs_inject_planned(const fs_store* store, int32_t layer_begin, int32_t layer_end,
                                   int32_t batch, int32_t k, const void* plan, size_t plan_bytes,
                                   void* const* k_cache, void* const* v_cache, int32_t num_blocks,
                                   void* stream);

/*
 * fs_retrieve_plan — retrieval and planning of one serving step in one call
 * (gist.science summary, "Phase En-ligne": the retrieved facts' segment is
 * what gets re-rotated and injected; "Résultats", Latence: the per-request
 * path stays short).  Writes exactly what fs_retrieve_topk writes (ids,
 * scores, num_tokens) and the plan that fs_plan_inject would write from
 * those ids with the same user, block_table, max_blocks, start_pos and
 * num_blocks; the selection's last kernel composes the plan itself, so
 * fs_inject_planned can follow at once.  Device stores only.
 *
 *   arguments as fs_retrieve_topk's, then as fs_plan_inject's (block_table
 *   device int32 [batch][max_blocks], start_pos device int32 [batch], plan
 *   caller-owned device memory of fs_inject_plan_size(batch) bytes, 16-byte
 *   aligned).  k = 0 writes num_tokens (when given) and no plan.
 * Device-checked: FS_ERR_USER (ids -1, length 0), FS_ERR_START_POS,
 * FS_ERR_BLOCK_SHORT, FS_ERR_BLOCK_ID (the request's plan length is then 0;
 * its ids are still written).  Errors: FS_E_ARG, FS_E_RANGE,
 * FS_E_BLOCKTABLE, FS_E_UNSUPPORTED, FS_E_HIP.
 */
FS_API fs_status fs_retrieve_plan(const fs_store* store, int32_t batch, const int32_t* user,
                                  const float* query, int32_t k, int32_t* ids, double* scores,
                                  int32_t* num_tokens, const int32_t* block_table, int32_t max_blocks,
                                  const int32_t* start_pos, int32_t num_blocks, void* plan,
                                  size_t plan_bytes, void* stream);

/*
 * fs_fetch_async — host-DRAM offload (gist.science summary, "Résultats":
 * the KV store can be offloaded to host DRAM at a small TTFT cost).
 * Pinned stores only.  Gathers the selected facts' K and V rows of layers
 * [layer_begin, layer_end) from the page-locked host arenas, over the host
 * link, into the device staging ring (slot = layer % staging_layers), in
 * composed segment order; fs_inject then reads the slot.  Enqueued on
 * `stream` (typically a side stream): the caller orders the later fs_inject
 * after it (e.g. with an event).  layer_end - layer_begin <= staging_layers.
 * Device-checked: FS_ERR_USER, FS_ERR_FACT_ID (that request stages nothing).
 * Errors: FS_E_ARG, FS_E_RANGE, FS_E_UNSUPPORTED (device store), FS_E_HIP.
 */
FS_API fs_status fs_fetch_async(const fs_store* store, int32_t batch,
                         const int32_t* user, const int32_t* ids, int32_t k,
                         int32_t layer_begin, int32_t layer_end, void* stream);

/*
 * fs_attend_prefill — the attention read of one layer's injected cache: a
 * causal prefill of each request's own tokens over the paged K/V cache.
 * Retrieve-and-inject inference rests on the equivalence of KV states
 * injected at the intended positions with the same memory given as prompt,
 * for causal decoders (Theorem 3 as the gist.science summary states it,
 * "Contributions Clés").
 *   batch          requests, 1 .. 65535
 *   num_q_tokens   Tq >= 1 query tokens per request
 *   num_q_heads    Hq, a multiple of the store's num_kv_heads (at most 8
 *                  query heads per KV head); query head h reads KV head
 *                  h / (Hq / num_kv_heads)
 *   q              device bf16 [batch][Tq][Hq][head_dim], BEFORE RoPE; token
 *                  j of request b is at position q_pos[b] + j and is rotated
 *                  here (the store's theta, rotate-half, fp64, one rounding
 *                  to bf16)
 *   k_cache, v_cache  device bf16 [num_blocks][block_size][num_kv_heads]
 *                  [head_dim] of ONE layer, holding rotated K and raw V for
 *                  every attended position, the query tokens' own included
 *                  (the caller writes those, as an engine's prefill does)
 *   block_table    device int32 [batch][max_blocks]: position p lives in
 *                  block block_table[b][p / block_size], slot p % block_size
 *   ctx_begin      device int32 [batch]: first attended position
 *   q_pos          device int32 [batch]: position of query token 0
 *   scale          softmax scale (typically 1/sqrt(head_dim)), finite, > 0
 *   out            device fp32 [batch][Tq][Hq][head_dim]: for token j,
 *                  softmax over p in [ctx_begin, q_pos + j] of
 *                  scale * <q_j, k_p>, applied to v_p
 *   workspace      device memory of workspace_bytes bytes (16-byte aligned),
 *                  or NULL.  When one pass per (16 query tokens, KV head,
 *                  request) would leave the device idle, the context is split
 *                  into ranges whose partial results go here and are merged
 *                  by a second launch; fs_attend_workspace_size gives the
 *                  bytes for the full split.  A smaller workspace splits less,
 *                  NULL not at all; the result is the same up to rounding.
 *                  Calls that share a workspace must not overlap.
 * head_dim must be 128, one cache position (num_kv_heads * 256 bytes) below
 * 16 MiB and one cache block below 4 GiB (else FS_E_UNSUPPORTED).
 * Precision: Q, K, V bf16; scores and accumulation fp32 on the matrix cores;
 * the softmax weights are rounded to bf16 before they multiply V (the
 * normaliser sums them in fp32).  Device-checked (the request's output rows
 * are then not written):
 * FS_ERR_START_POS (ctx_begin < 0, ctx_begin > q_pos, or q_pos + Tq past
 * INT32_MAX), FS_ERR_BLOCK_SHORT, FS_ERR_BLOCK_ID.  Errors: FS_E_ARG
 * (null or misaligned: q, caches and out 16-byte aligned), FS_E_RANGE,
 * FS_E_BLOCKTABLE, FS_E_UNSUPPORTED, FS_E_HIP.  Uses no library scratch, so
 * it may overlap any other call on the store.
 */
FS_API fs_status fs_attend_prefill(const fs_store* store, int32_t batch, int32_t num_q_tokens,
                                   int32_t num_q_heads, const void* q, const void* k_cache,
                                   const void* v_cache, int32_t num_blocks,
                                   const int32_t* block_table, int32_t max_blocks,
                                   const int32_t* ctx_begin, const int32_t* q_pos, float scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * fs_attend_workspace_size — bytes of workspace fs_attend_prefill uses for
 * this batch shape at its full context split (0 when it would not split).
 * Errors: FS_E_ARG, FS_E_RANGE.
 */
FS_API fs_status fs_attend_workspace_size(const fs_store* store, int32_t batch,
                                          int32_t num_q_tokens, int32_t num_q_heads,
                                          size_t* bytes);

/* ---- store ingest and eviction (Context-Window Encoding capture) -------- */

/*
 * Facts are encoded offline with a window of the w conversation turns before
 * them, and only the fact's own KV is kept: keys taken before RoPE, values
 * raw (gist.science summary, "Phase Hors-ligne" and "Stockage Pré-RoPE").
 * The encoder is the serving model's own prefill over [w turns ; fact]; these
 * calls take its per-layer output and maintain the store.
 *
 * Slots: user u owns fact ids user_fact_begin[u] .. user_fact_begin[u+1]-1
 * (its capacity); the first live_count[u] of them are live.  Retrieval and
 * injection see live facts only.  Arena rows are handed out in order from
 * rows_used and are not reused after an eviction (rebuild the store to
 * compact).  An inverted-file index is not updated: rebuild it after ingest
 * or eviction.  These calls write the caller's embedding matrix and arenas
 * and must not overlap any other call on the store.  fs_ingest_init and
 * fs_evict_fact synchronise `stream` before they return; fs_ingest_facts is
 * asynchronous on `stream` like the compute calls, so the caller orders any
 * later call on the store after it (the same stream, or an event).
 */

/*
 * fs_ingest_init — declare the live facts per user (host [num_users], each
 * at most the user's capacity) and the first free arena row (every live
 * fact's rows lie below it).  At creation every slot is live and every row
 * used.  Errors: FS_E_ARG, FS_E_RANGE, FS_E_HIP.
 */
FS_API fs_status fs_ingest_init(fs_store* store, const int32_t* live_counts, int64_t rows_used,
                                void* stream);

/*
 * fs_ingest_facts — append n facts (1 .. 4096) in one launch.  Fact i goes to
 * user user[i] (host array), into that user's next free slot.  k_window /
 * v_window: host arrays [num_layers] of device-visible bf16 [rows][H][D]
 * holding the encoder's pre-RoPE keys and raw values of the windows (all
 * facts' windows in one array per layer); fact i keeps rows keep_begin[i] ..
 * keep_begin[i] + keep_len[i] - 1 (host arrays; 1 <= keep_len <= the longest
 * fact at creation), the rest of its window is discarded.  emb: device fp32
 * [n][embed_dim], fact i's embedding.  fact_ids (host [n], out): the ids
 * given, assigned at once (fs_store_live counts them on return).  The window
 * arrays and emb must stay valid until `stream` has run the call.
 * All-or-nothing: a host-checked error (no free slot, arenas full, a length
 * out of range) writes nothing.  Errors: FS_E_ARG, FS_E_RANGE, FS_E_NOMEM
 * (host staging of the first call), FS_E_HIP.
 */
FS_API fs_status fs_ingest_facts(fs_store* store, int32_t n, const int32_t* user,
                                 const void* const* k_window, const void* const* v_window,
                                 const int64_t* keep_begin, const int32_t* keep_len,
                                 const float* emb, void* stream, int32_t* fact_ids);

/*
 * fs_evict_fact — remove a live fact.  Its user's last live fact moves into
 * the freed slot (metadata and embedding row), so live ids stay dense;
 * *moved_from (optional) receives the moved fact's former id, or -1.  Ids
 * held by the caller for the moved fact change.  Errors: FS_E_ARG,
 * FS_E_RANGE (not a live fact), FS_E_HIP.
 */
FS_API fs_status fs_evict_fact(fs_store* store, int32_t fact_id, void* stream, int32_t* moved_from);

/* fs_store_live — live facts of `user` and the first free arena row. */
FS_API fs_status fs_store_live(const fs_store* store, int32_t user, int32_t* live,
                               int64_t* rows_used);

/* ---- approximate retrieval: inverted-file index ------------------------- */

/*
 * The pages keep a GPU-resident semantic retrieval index beside the KV store
 * (gist.science summary, "Contributions Clés") and name it without
 * describing it.  This is an index of its own design for users whose fact
 * tables are too large for the flat scan of fs_retrieve_topk: the user's
 * embeddings are clustered (spherical k-means, inner product) into nlist
 * lists; a probe scores the nlist centroids, scans the nprobe best lists and
 * returns the top k of their facts.
 *
 * What a probe returns, exactly: with the lists ranked by (centroid score
 * desc, list index asc), the k best facts of the union of the first nprobe
 * lists by (score desc, fact id asc), scored exactly as fs_retrieve_topk
 * scores them (same bits).  With nprobe = nlist it equals fs_retrieve_topk.
 */
typedef struct fs_ivf fs_ivf;

typedef struct {
    int32_t user;            /* the indexed user                              */
    int32_t nlist;           /* lists (= centroids)                           */
    int32_t num_facts;       /* the user's facts, all in exactly one list     */
    int32_t max_list;        /* longest list                                  */
    int32_t max_nprobe;
    const float* centroids;  /* device fp32 [nlist][embed_dim], unit norm     */
    const int32_t* list_begin; /* device [nlist + 1]: list c is members[list_begin[c] ..
                                  list_begin[c+1])                          */
    const int32_t* members;  /* device [num_facts] global fact ids, ascending within a list */
} fs_ivf_view;

/*
 * fs_ivf_build — cluster user `user`'s embeddings into `nlist` lists
 * (1 .. 4096, at most the user's fact count) with `iters` k-means
 * iterations (0 .. 100; centroids start at the rows floor(c * N / nlist)),
 * and allocate probe scratch for up to `max_nprobe` lists and the store's
 * max_batch requests.  Runs on `stream` and synchronises it; deterministic
 * for a given store.  The index keeps a copy of the rows in list order (4 *
 * N * embed_dim bytes) and reads the store's embeddings only while building.
 * Errors: FS_E_ARG, FS_E_RANGE, FS_E_NOMEM, FS_E_HIP.
 */
FS_API fs_status fs_ivf_build(const fs_store* store, int32_t user, int32_t nlist, int32_t iters,
                              int32_t max_nprobe, void* stream, fs_ivf** out);

/* fs_ivf_destroy — free an index (NULL is a no-op); no call may be in flight. */
FS_API fs_status fs_ivf_destroy(fs_ivf* ivf);

/* fs_ivf_arrays — sizes and read-only device pointers of a built index. */
FS_API fs_status fs_ivf_arrays(const fs_ivf* ivf, fs_ivf_view* view);

/*
 * fs_ivf_retrieve_topk — approximate retrieval for `batch` requests of the
 * indexed user (query device fp32 [batch][embed_dim], 16-byte aligned),
 * probing `nprobe` lists (1 .. max_nprobe).  ids / scores / num_tokens as in
 * fs_retrieve_topk (rank order, -1 / -inf pads when the probed lists hold
 * fewer than k facts).  Uses the index's probe scratch: calls on one index
 * must not overlap.  Errors: FS_E_ARG, FS_E_RANGE, FS_E_HIP.
 */
FS_API fs_status fs_ivf_retrieve_topk(const fs_store* store, const fs_ivf* ivf, int32_t batch,
                                      const float* query, int32_t nprobe, int32_t k, int32_t* ids,
                                      double* scores, int32_t* num_tokens, void* stream);

/*
 * fs_check_block_tables — opt-in debug check, on the host, that the cache
 * blocks a call writes are its own: fs_inject writes request b's segment of
 * num_tokens[b] tokens at positions start_pos[b] .. start_pos[b] +
 * num_tokens[b] - 1, through block_table[b][p / block_size] (gist.science
 * summary, "Phase En-ligne", item "Injection").  The GPU path checks each
 * entry's range but not that two requests, or two logical blocks of one
 * request, name the same physical block; this call does, so a caller can
 * find aliased tables before they corrupt each other's cache.
 *   All arrays are host memory, read only: block_table [batch][max_blocks],
 *   start_pos [batch], num_tokens [batch] (e.g. fs_retrieve_topk's output
 *   copied to the host).  block_size: a power of two; num_blocks >= 1.
 *   Returns FS_OK when every written block is named once and lies in
 *   [0, num_blocks); FS_E_BLOCKTABLE on the first violation, with conflict
 *   (int32 [4], may be null) set to {request, logical block, block id, the
 *   earlier request naming it or -1 for a range error}; FS_E_ARG on bad
 *   arguments.  Needs no store and no GPU.
 */
FS_API fs_status fs_check_block_tables(int32_t batch, const int32_t* block_table, int32_t max_blocks,
                                       const int32_t* start_pos, const int32_t* num_tokens,
                                       int32_t block_size, int32_t num_blocks, int32_t* conflict);

/*
 * fs_poll_errors — synchronise `stream`, return the device error bits
 * accumulated since the last poll in *flags, and clear them.  Returns
 * FS_E_DEVICE when any bit was set, FS_OK otherwise (FS_E_ARG, FS_E_HIP).
 */
FS_API fs_status fs_poll_errors(const fs_store* store, void* stream, uint32_t* flags);

/* fs_strerror — static text for a status code. */
FS_API const char* fs_strerror(fs_status status);

/* fs_last_error_message — detail of the last failing call on this thread
 * (static per thread; empty string if none). */
FS_API const char* fs_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* FS_H_ */
