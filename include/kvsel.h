/*
 * kvsel.h - query-oriented KV selection (QuoKA) + compacted attention for
 * chunked prefill, as a C ABI over hand-written gfx950 (MI355X) HIP kernels.
 *
 * What is computed (QuoKA article, "Qualcomm QuoKA", itsolotime.com, Fig. 1(a)
 * and 1(b) and the method paragraph after Fig. 1): a prompt is processed one
 * chunk at a time; for each chunk of C queries at positions [T, T+C)
 *   1. per query head h, the chunk's mean query m_h is formed and the n_q
 *      queries with the smallest cosine to m_h are kept (ties: lower token);
 *   2. every prior cache key j < T of KV head g is scored
 *      S[g][j] = mean over the G = h_q / h_kv query heads h of g of
 *                max over kept queries i of h of cos(q_{h,i}, k_{g,j});
 *   3. the `budget` highest-scoring keys are kept per KV head (ties: lower
 *      index; indices reported ascending); when T <= budget every prior key
 *      is kept and steps 1-2 are skipped;
 *   4. the kept K/V rows are compacted and
 *   5. every chunk query attends, with softmax scale 1/sqrt(d) (or `scale`),
 *      to the compacted prior keys (all visible) plus the chunk's own keys
 *      under the causal mask; KV head of query head h is h / G (grouped and
 *      multi-query attention, multi-query attention page, "Teknisk innsikt").
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns all
 *     device memory, including the workspace; the library allocates nothing
 *     and keeps no per-call state.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues kernel launches on it (no memset, copy or host wait) and
 *     returns without synchronising, so calls can be captured in a HIP graph
 *     while kernel tracing is off; a replay reads the argument values of the
 *     captured calls, so their buffers must stay allocated.
 *   - Arguments are checked on the host before anything is enqueued; on an
 *     error the call returns a non-zero kvsel_status with nothing enqueued and
 *     kvsel_last_error() describes it.  A failed launch returns
 *     KVSEL_ERR_HIP.  Errors during execution surface at the caller's next
 *     synchronisation.  No C++ exception crosses this boundary.
 *   - Tensors are dense row-major with the shapes given; element type is
 *     `heads->dtype` for q/k/v (fp32 or bf16 bit patterns), accumulation is
 *     always fp32.
 *   - The same inputs give bitwise-identical outputs (no floating-point
 *     atomics anywhere).
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVSEL_OK = 0,
    KVSEL_ERR_INVALID_ARG = 1,   /* a null pointer, a bad shape, an out-of-range value */
    KVSEL_ERR_UNSUPPORTED = 2,   /* a valid request the library does not implement (e.g. d = 96) */
    KVSEL_ERR_WORKSPACE = 3,     /* workspace missing or smaller than kvsel_workspace_size() */
    KVSEL_ERR_HIP = 4            /* a HIP launch failed; kvsel_last_error() has the HIP message */
} kvsel_status;

typedef enum { KVSEL_F32 = 0, KVSEL_BF16 = 1 } kvsel_dtype;

/* Attention heads of one layer.  h_q % h_kv == 0; d in {64, 128};
 * scale == 0 means 1/sqrt(d). */
typedef struct {
    int32_t h_q, h_kv, d;
    int32_t dtype;               /* kvsel_dtype of q, k, v */
    float scale;
} kvsel_heads;

/* Order of the two poolings of step 2.
 *   KVSEL_POOL_HEAD (0): as above - mean over the group's query heads of each
 *     head's max over its own kept queries (steps 1-2 as listed).
 *   KVSEL_POOL_GROUP (1): the group is pooled first.  QuoKA article, Table 4
 *     caption: the method's cost is stated with the number of KV heads in
 *     place of the number of query heads.  For every KV head g and chunk
 *     token i, qbar[g][i] = mean over the G query heads of g of q/|q| (a zero
 *     row contributes 0); step 1 runs on the pooled rows (n_q tokens kept per
 *     KV head) and S[g][j] = max over kept i of qbar[g][i] . k_j / |k_j|, the
 *     max over kept tokens of the mean over heads of the cosine.  With
 *     chunk_len == 1 both orders give the same score. */
typedef enum { KVSEL_POOL_HEAD = 0, KVSEL_POOL_GROUP = 1 } kvsel_pooling;

/* Selection budget.  n_q >= 1 queries kept per query head (per KV head with
 * KVSEL_POOL_GROUP; all when n_q >= chunk_len); budget >= 1 prior keys kept
 * per KV head; pooling is a kvsel_pooling. */
typedef struct {
    int32_t n_q, budget;
    int32_t pooling;
} kvsel_params;

/* One layer's KV cache.
 *   contiguous (block_size == 0): k, v are [batch][h_kv][capacity][d]; the
 *     prior tokens of sequence b are rows [0, T_b).
 *   paged (block_size > 0): k, v are [capacity][h_kv][block_size][d]
 *     (capacity = number of physical blocks); position p of sequence b lives
 *     in block block_table[b * max_blocks_per_seq + p / block_size], row
 *     p % block_size.  Every block a call touches must be mapped. */
typedef struct {
    void *k, *v;
    int64_t capacity;
    int32_t block_size;
    int32_t max_blocks_per_seq;
    const int32_t *block_table;  /* paged only: [batch][max_blocks_per_seq] */
} kvsel_cache;

/* The sequences of one call.  Every sequence contributes chunk_len new tokens
 * (chunk_len == 1 is a decode step). */
typedef struct {
    int32_t batch, chunk_len;
    const int64_t *prior_len_host;   /* [host][batch] T_b: sizes the grids, no device->host copy */
    const int64_t *prior_len_dev;    /* [batch] the same values in device memory */
} kvsel_batch;

/* Limits shared by kvsel_workspace_size, kvsel_select and kvsel_prefill_chunk:
 * max_b T_b and budget are at most KVSEL_MAX_SELECT_KEYS (the exact top-B
 * keeps one counter pair per 2048-key segment on chip); larger requests
 * return KVSEL_ERR_UNSUPPORTED with nothing enqueued. */
#define KVSEL_MAX_SELECT_KEYS (2048 * 1024)

/* Workspace bytes that kvsel_select and kvsel_prefill_chunk need for these
 * shapes (the larger of the two) on the current device (some launch shapes
 * follow its compute-unit count).  Writes *bytes; returns a status (so that
 * an invalid or unsupported shape is reported, not sized). */
kvsel_status kvsel_workspace_size(const kvsel_heads *heads, const kvsel_batch *batch,
                                  const kvsel_params *params, size_t *bytes);

/* Workspace bytes that kvsel_sparse_attn needs (it lays the caller's
 * compacted set and the chunk's keys out for the MFMA kernel and may split
 * long key lists over several workgroups, whose partial results live here). */
kvsel_status kvsel_sparse_attn_workspace_size(const kvsel_heads *heads, const kvsel_batch *batch,
                                              int32_t n_sel_max, size_t *bytes);

/* Steps 1-3 (and the compaction of step 4 when k_sel/v_sel are given) for one
 * chunk of every sequence, against the prior cache rows [0, T_b).
 * QuoKA article, Fig. 1(b): queries filtered by cosine dissimilarity to the
 * mean query, then keys by query-key cosine similarity; the method paragraph
 * after Fig. 1: max pooling over the kept queries, mean pooling over the query
 * heads of a KV head (GQA); Fig. 1(a): the cache of each chunk is
 * sub-selected before attention.  The pages give no formula; the steps above
 * are the plain reading of those passages.
 * Errors: every argument and size check returns before anything is enqueued
 * (KVSEL_ERR_INVALID_ARG, _UNSUPPORTED, _WORKSPACE); a failed launch returns
 * KVSEL_ERR_HIP and may leave earlier launches of the call enqueued.
 *   q       [batch][h_q][chunk_len][d]
 *   cache   read only
 *   idx     out [batch][h_kv][budget] int32: kept prior positions, ascending,
 *           -1 past min(budget, T_b)
 *   k_sel, v_sel  optional out [batch][h_kv][budget][d]: the kept rows, copied
 *           bit for bit; rows past min(budget, T_b) are not written.  Both or
 *           neither.
 *   q_keep  optional debug out [batch][h_q][min(n_q, chunk_len)] int32: the
 *           kept query tokens, ascending; written only for sequences with
 *           T_b > budget.  With KVSEL_POOL_GROUP and chunk_len > 1 the rows
 *           are per KV head: [batch][h_kv][min(n_q, chunk_len)].
 *   scores  optional debug out [batch][h_kv][score_stride] fp32 with
 *           score_stride = max_b T_b: S[g][j] for j < T_b; written only for
 *           sequences with T_b > budget. */
kvsel_status kvsel_select(const kvsel_heads *heads, const kvsel_batch *batch,
                          const kvsel_params *params, const void *q, const kvsel_cache *cache,
                          int32_t *idx, void *k_sel, void *v_sel, int32_t *q_keep, float *scores,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Step 5 alone, on a compacted set supplied by the caller.
 * QuoKA article, Fig. 1(a): the compacted cache is fed to a dense attention
 * kernel; every chunk query attends to all compacted prior keys and, under
 * the causal mask, to the chunk's own keys, with softmax scale 1/sqrt(d).
 * QUILT page, "In parole semplici": the queries sharing one selected set
 * load its entries once (here: all G query heads of a KV head and all chunk
 * tokens read each staged key tile once per workgroup).  Multi-query
 * attention page, "Teknisk innsikt": query head h uses KV head h / G.
 *   q                [batch][h_q][chunk_len][d]
 *   k_sel, v_sel     [batch][h_kv][n_sel_max][d]: compacted prior keys, all visible
 *   n_sel            [batch] int32 (device): rows of k_sel used per sequence, 0..n_sel_max
 *   k_chunk, v_chunk [batch][h_kv][chunk_len][d]: the chunk's own keys, causal
 *   out              [batch][h_q][chunk_len][d], element type out_dtype
 * batch->prior_len_* are not read and may be NULL. */
kvsel_status kvsel_sparse_attn(const kvsel_heads *heads, const kvsel_batch *batch,
                               const void *q, const void *k_sel, const void *v_sel,
                               const int32_t *n_sel, int32_t n_sel_max,
                               const void *k_chunk, const void *v_chunk,
                               void *out, int32_t out_dtype,
                               void *workspace, size_t workspace_bytes, void *stream);

/* One chunk of chunked prefill for every sequence: steps 1-5, then append the
 * chunk's K/V to the cache at positions [T_b, T_b + chunk_len) (the cache
 * grows by one chunk; the caller advances T_b).
 * QuoKA article, introduction and Fig. 1(a): a long prompt is processed one
 * chunk after another, each chunk's cache sub-selected (kvsel_select) and
 * the compacted cache fed to dense attention (kvsel_sparse_attn); the cache
 * grows by one chunk per step.  When T_b <= budget every prior key is kept
 * and steps 1-3 are skipped for that sequence.
 * Errors: as kvsel_select.
 *   q, k_chunk, v_chunk, out  as in kvsel_sparse_attn
 *   cache   prior rows are read, rows [T_b, T_b + chunk_len) are written;
 *           capacity (contiguous) or the block table (paged) must cover them
 *   idx     optional out [batch][h_kv][budget] int32 as in kvsel_select */
kvsel_status kvsel_prefill_chunk(const kvsel_heads *heads, const kvsel_batch *batch,
                                 const kvsel_params *params, const void *q,
                                 const void *k_chunk, const void *v_chunk,
                                 const kvsel_cache *cache, void *out, int32_t out_dtype,
                                 int32_t *idx, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* The selected-entry cache of decode with cross-step reuse (SQD page,
 * rit.work, the paragraph on sparse attention: the top-k selection scans the
 * whole cache each step, the values at the selected positions are kept from
 * one step to the next and only the misses are fetched).  The page gives no
 * slot policy; the one used: after a step's top-B (n_b = min(budget, T_b)
 * positions per KV head), a slot below n_b whose position is selected again
 * keeps its rows (a hit); the selected positions held by no such slot (the
 * misses), in ascending order, are fetched from the KV cache into the other
 * slots below n_b, in ascending order; slots from n_b on become empty.
 * Caller-owned device memory, kept from one call to the next:
 *   k, v     [batch][h_kv][budget][d], element type heads->dtype
 *   pos      [batch][h_kv][budget] int32: the position each slot holds, -1 =
 *            empty.  Set every entry to -1 before a sequence's first step (and
 *            when a batch entry starts another sequence); after that only the
 *            library writes it.
 *   counts   optional [batch][h_kv][2] int32: hits and misses of the last call */
typedef struct {
    void *k, *v;
    int32_t *pos;
    int32_t *counts;
} kvsel_sel_cache;

#define KVSEL_REUSE_MAX_BUDGET 8192

/* One decode step of every sequence (chunk_len tokens each, with
 * (h_q / h_kv) * chunk_len <= 128) with the selected-entry cache `sel`:
 * steps 1-3 as in kvsel_prefill_chunk, then the update of `sel` above, then
 * attention of every query over the slots [0, n_b) of its KV head plus the
 * step's own tokens (causal), then the cache append at [T_b, T_b + chunk_len).
 * The output is kvsel_prefill_chunk's up to floating-point summation order
 * (softmax attention does not depend on the order of its keys; QuoKA
 * article, Fig. 1(a)).  bf16 only; budget <= KVSEL_REUSE_MAX_BUDGET;
 * workspace as sized by kvsel_workspace_size.  idx: optional out as in
 * kvsel_select.  Errors: as kvsel_select. */
kvsel_status kvsel_decode_reuse(const kvsel_heads *heads, const kvsel_batch *batch,
                                const kvsel_params *params, const void *q, const void *k_new,
                                const void *v_new, const kvsel_cache *cache, const kvsel_sel_cache *sel,
                                void *out, int32_t out_dtype, int32_t *idx, void *workspace,
                                size_t workspace_bytes, void *stream);

/* kvsel_prefill_chunk for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation and outputs as kvsel_prefill_chunk, with
 * the workspace taken from a fixed device array inside the library instead of
 * a caller buffer: KVSEL_NOALLOC_SCRATCH_BYTES per GPU, held from the first
 * call on that GPU until the process ends.  Shapes whose workspace
 * (kvsel_workspace_size) is larger return KVSEL_ERR_UNSUPPORTED with nothing
 * enqueued.  The call allocates nothing (no hipMalloc / hipFree) and records
 * no trace events.  Every call on one GPU uses that GPU's one array, which
 * keeps the last call's contents: calls that overlap in time on one GPU (two
 * streams, two threads) race on it and must be serialised by the caller. */
#define KVSEL_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
kvsel_status kvsel_prefill_chunk_noalloc(const kvsel_heads *heads, const kvsel_batch *batch,
                                         const kvsel_params *params, const void *q,
                                         const void *k_chunk, const void *v_chunk,
                                         const kvsel_cache *cache, void *out, int32_t out_dtype,
                                         int32_t *idx, void *stream);

/* Where kvsel_prefill_chunk leaves the compacted key list of step 4 in the
 * workspace, so that a caller can read it back after the call (QuoKA article,
 * Fig. 1(a): the compacted cache handed to attention).  For the shapes and
 * cache given (only its layout is read):
 *   *packed = 1 when the call builds the lists in the workspace, 0 when its
 *     attention reads the kept rows in place (no lists; the other outputs are
 *     then left unwritten): through their cache row numbers (chunks of G x
 *     chunk_len <= 128 query rows per KV head), or, when no sequence selects
 *     (every T_b <= budget) on a contiguous bf16 cache, as the cache prefix
 *     [0, T_b) followed by the chunk's rows, which the call appends first;
 *   keys at byte offset *k_offset: [batch][h_kv][*slots][d] (one row per slot);
 *   values at *v_offset: [batch][h_kv][d][*slots] (transposed) when
 *     *v_transposed, else [batch][h_kv][*slots][d];
 *   slot s of sequence b holds, for s < n_b = min(budget, T_b), the prior row
 *   at idx[b][g][s]; for n_b <= s < n_b + chunk_len, the chunk's row s - n_b;
 *   beyond, zeros.
 * The lists are valid until the next call that uses the workspace.  Returns a
 * status; pure host arithmetic (nothing is enqueued). */
kvsel_status kvsel_compacted_view(const kvsel_heads *heads, const kvsel_batch *batch,
                                  const kvsel_params *params, const kvsel_cache *cache,
                                  int32_t *packed, size_t *k_offset, size_t *v_offset,
                                  int32_t *slots, int32_t *v_transposed);

/* Per-kernel timing (a tracing aid for benchmarks).  After
 * kvsel_trace_start(mask), every launch of a kernel whose bit (1 << id) is
 * set in `mask` is bracketed by two hipEvents recorded on its launch stream;
 * kvsel_trace_stop() ends recording.  kvsel_trace_read() waits for the
 * recorded events and writes, for every kernel id < n, the number of launches
 * and their summed duration in milliseconds into the [host] arrays
 * `launches` and `total_ms`, then clears the record.  The library creates the
 * events itself (no device memory) and reuses them.  Tracing state is global
 * to the process and guarded by a mutex. */
typedef enum {
    KVSEL_K_QSTATS = 0,   /* step 1: query cosines to the mean query, 1/|q| */
    KVSEL_K_QTOPK = 1,    /* step 1: the kept queries (exact top-k) */
    KVSEL_K_QPACK = 2,    /* step 1: kept query rows packed per KV head */
    KVSEL_K_SCAN = 3,     /* step 2: cosine key scores over the prior cache */
    KVSEL_K_TOPB = 4,     /* step 3: per-KV-head top-B (in kvsel_prefill_chunk's bf16 packed path its
                             threshold launch also writes the chunk's list slots and appends the chunk) */
    KVSEL_K_GATHER = 5,   /* step 4 (kvsel_select): k_sel/v_sel rows */
    KVSEL_K_PACK = 6,     /* step 4: compacted keys (+ chunk keys and the cache append, unless the
                             top-B launch wrote them) for attention */
    KVSEL_K_ATTN = 7,     /* step 5: attention */
    KVSEL_K_APPEND = 8,   /* cache append on its own (gathering attention path; otherwise inside the pack kernel) */
    KVSEL_K_QPOOL = 9,    /* step 1 with KVSEL_POOL_GROUP: the group's unit queries averaged per token */
    KVSEL_K_REUSE = 10,   /* kvsel_decode_reuse: slot update and miss fetch of the selected-entry cache */
    KVSEL_K_COUNT = 11
} kvsel_kernel;

kvsel_status kvsel_trace_start(uint32_t kernel_mask);
kvsel_status kvsel_trace_stop(void);
kvsel_status kvsel_trace_read(int32_t *launches, float *total_ms, int32_t n);
/* Short name of kernel id (e.g. "attn"); "" for an unknown id. */
const char *kvsel_kernel_name(int32_t id);

/* Text of the last error on the calling thread ("" if none); valid until the
 * next kvsel_* call on that thread. */
const char *kvsel_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t kvsel_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
