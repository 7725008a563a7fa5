// C-ABI entry points of libkvsel: argument checks, workspace carving and the
// launch sequence of one chunk.  Every check runs on the host before anything
// is enqueued; no C++ exception leaves this file.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "kvsel.h"
#include "launch.h"

using namespace kvsel;

namespace kvsel {
int device_cus() {
    static std::atomic<int> cus[64];          // 0: not queried yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}
}  // namespace kvsel

namespace {

thread_local std::string g_err;

kvsel_status fail(kvsel_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

kvsel_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return KVSEL_OK;
    return fail(KVSEL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define KVSEL_TRY(expr, what)                          \
    do {                                               \
        kvsel_status _s = hip_check((expr), (what));   \
        if (_s != KVSEL_OK) return _s;                 \
    } while (0)

constexpr int64_t kMaxLen = int64_t(1) << 30;   // positions fit int32 kernel arithmetic

// ----------------------------------------------------------------------------- tracing

const char* const kKernelNames[KVSEL_K_COUNT] = {"qstats", "qtopk", "qpack", "scan", "topb", "gather",
                                                 "pack", "attn", "append", "qpool", "reuse"};

struct Trace {
    std::mutex mu;
    uint32_t mask = 0;
    struct Rec { int id; hipEvent_t a, b; };
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
    hipEvent_t take() {
        if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
        // timing only, read after the caller's synchronisation: no system-scope
        // fence (its cache writeback and invalidation would slow the launches
        // being timed)
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
        return e;
    }
};
Trace g_trace;

// Set while a call must not create trace events (the no-allocation entry point).
thread_local bool g_no_trace = false;
struct NoTraceScope {
    bool prev;
    NoTraceScope() : prev(g_no_trace) { g_no_trace = true; }
    ~NoTraceScope() { g_no_trace = prev; }
};

// Launch `fn` (returning hipError_t), bracketed by events when kernel `id` is traced.
template <typename F>
hipError_t traced(int id, hipStream_t st, F&& fn) {
    hipEvent_t a = nullptr, b = nullptr;
    if (!g_no_trace) {
        std::lock_guard<std::mutex> lk(g_trace.mu);
        if (g_trace.mask & (1u << id)) {
            a = g_trace.take();
            b = g_trace.take();
            if (!a || !b) {                    // an event could not be created: this launch is not timed
                if (a) g_trace.pool.push_back(a);
                if (b) g_trace.pool.push_back(b);
                a = b = nullptr;
            }
        }
    }
    if (a) (void)hipEventRecord(a, st);
    const hipError_t e = fn();
    if (a) {
        (void)hipEventRecord(b, st);
        std::lock_guard<std::mutex> lk(g_trace.mu);
        g_trace.recs.push_back({id, a, b});
    }
    return e;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ----------------------------------------------------------------------------- checks

kvsel_status check_heads(const kvsel_heads* h) {
    if (!h) return fail(KVSEL_ERR_INVALID_ARG, "heads is NULL");
    if (h->h_q < 1 || h->h_kv < 1) return fail(KVSEL_ERR_INVALID_ARG, "h_q=%d h_kv=%d must be >= 1", h->h_q, h->h_kv);
    if (h->h_q % h->h_kv) return fail(KVSEL_ERR_INVALID_ARG, "h_q=%d is not a multiple of h_kv=%d", h->h_q, h->h_kv);
    if (h->dtype != KVSEL_F32 && h->dtype != KVSEL_BF16) return fail(KVSEL_ERR_INVALID_ARG, "dtype=%d unknown", h->dtype);
    if (h->d != 64 && h->d != 128) return fail(KVSEL_ERR_UNSUPPORTED, "head dim d=%d (supported: 64, 128)", h->d);
    if (!std::isfinite(h->scale) || h->scale < 0.0f) return fail(KVSEL_ERR_INVALID_ARG, "scale must be finite and >= 0");
    return KVSEL_OK;
}

kvsel_status check_batch(const kvsel_batch* b, bool need_lens, int64_t* t_max) {
    if (!b) return fail(KVSEL_ERR_INVALID_ARG, "batch is NULL");
    if (b->batch < 1) return fail(KVSEL_ERR_INVALID_ARG, "batch=%d must be >= 1", b->batch);
    if (b->chunk_len < 1 || b->chunk_len > kMaxLen) return fail(KVSEL_ERR_INVALID_ARG, "chunk_len=%d out of range", b->chunk_len);
    *t_max = 0;
    if (!need_lens) return KVSEL_OK;
    if (!b->prior_len_host || !b->prior_len_dev) return fail(KVSEL_ERR_INVALID_ARG, "prior_len_host/prior_len_dev is NULL");
    for (int i = 0; i < b->batch; ++i) {
        const int64_t T = b->prior_len_host[i];
        if (T < 0 || T + b->chunk_len > kMaxLen) return fail(KVSEL_ERR_INVALID_ARG, "prior_len[%d]=%lld out of range", i, (long long)T);
        if (T > *t_max) *t_max = T;
    }
    return KVSEL_OK;
}

kvsel_status check_params(const kvsel_params* p) {
    if (!p) return fail(KVSEL_ERR_INVALID_ARG, "params is NULL");
    if (p->n_q < 1) return fail(KVSEL_ERR_INVALID_ARG, "n_q=%d must be >= 1", p->n_q);
    if (p->budget < 1) return fail(KVSEL_ERR_INVALID_ARG, "budget=%d must be >= 1", p->budget);
    if (p->pooling != KVSEL_POOL_HEAD && p->pooling != KVSEL_POOL_GROUP)
        return fail(KVSEL_ERR_INVALID_ARG, "pooling=%d must be KVSEL_POOL_HEAD or KVSEL_POOL_GROUP", p->pooling);
    return KVSEL_OK;
}

// Selection limits: the top-B's per-segment counters (kTopbMaxSegments
// segments of kTopbSegKeys keys) bound the prior length and the budget.
kvsel_status check_select(int64_t t_max, const kvsel_params* p) {
    if (topb_segments(t_max, p->budget) > kTopbMaxSegments)
        return fail(KVSEL_ERR_UNSUPPORTED, "prior length %lld / budget %d: at most %lld keys per sequence can be selected from",
                    (long long)t_max, p->budget, (long long)kTopbSegKeys * kTopbMaxSegments);
    return KVSEL_OK;
}

// extra = rows past T_b that the call writes (chunk_len for prefill, 0 for select)
kvsel_status check_cache(const kvsel_cache* c, const kvsel_batch* b, int extra) {
    if (!c) return fail(KVSEL_ERR_INVALID_ARG, "cache is NULL");
    if (!c->k || !c->v) return fail(KVSEL_ERR_INVALID_ARG, "cache k/v is NULL");
    if (!aligned16(c->k) || !aligned16(c->v)) return fail(KVSEL_ERR_INVALID_ARG, "cache k/v must be 16-byte aligned");
    if (c->block_size < 0) return fail(KVSEL_ERR_INVALID_ARG, "block_size=%d < 0", c->block_size);
    if (c->capacity < 1) return fail(KVSEL_ERR_INVALID_ARG, "cache capacity=%lld < 1", (long long)c->capacity);
    for (int i = 0; i < b->batch; ++i) {
        const int64_t need = b->prior_len_host[i] + extra;
        if (c->block_size == 0) {
            if (need > c->capacity)
                return fail(KVSEL_ERR_INVALID_ARG, "sequence %d needs %lld cache rows, capacity is %lld", i, (long long)need, (long long)c->capacity);
        } else {
            if (!c->block_table) return fail(KVSEL_ERR_INVALID_ARG, "paged cache without block_table");
            const int64_t blocks = (need + c->block_size - 1) / c->block_size;
            if (blocks > c->max_blocks_per_seq)
                return fail(KVSEL_ERR_INVALID_ARG, "sequence %d needs %lld blocks, block table holds %d", i, (long long)blocks, c->max_blocks_per_seq);
        }
    }
    return KVSEL_OK;
}

// The gathering attention carries cache row numbers as int32.
bool cache_rows_fit(const kvsel_cache* c, const kvsel_heads* h, const kvsel_batch* b) {
    const int64_t per = c->block_size == 0 ? int64_t(b->batch) * c->capacity : c->capacity * c->block_size;
    return per * h->h_kv < (int64_t(1) << 31);
}

CacheView make_view(const kvsel_cache* c, const kvsel_heads* h) {
    CacheView v;
    v.k = static_cast<char*>(c->k);
    v.v = static_cast<char*>(c->v);
    v.capacity = c->capacity;
    v.block_size = c->block_size;
    v.max_blocks = c->max_blocks_per_seq;
    v.block_table = c->block_table;
    v.h_kv = h->h_kv;
    v.row_bytes = h->d * (h->dtype == KVSEL_BF16 ? 2 : 4);
    return v;
}

SelShape make_shape(const kvsel_heads* h, const kvsel_batch* b, const kvsel_params* p, int64_t t_max) {
    SelShape s;
    s.batch = b->batch;
    s.h_q = h->h_q;
    s.h_kv = h->h_kv;
    s.G = h->h_q / h->h_kv;
    s.d = h->d;
    s.C = b->chunk_len;
    s.esz = h->dtype == KVSEL_BF16 ? 2 : 4;
    s.nqp = p ? (p->n_q < b->chunk_len ? p->n_q : b->chunk_len) : 0;
    if (s.esz == 4) s.nq_pad = s.nqp;                                     // VALU scan: exact rows
    else if (s.nqp == 1 && s.G <= 16) s.nq_pad = 1;                       // one query row per head
    else s.nq_pad = static_cast<int>(round_up(s.nqp, 32));                // MFMA scan: 32-row blocks
    s.budget = p ? p->budget : 0;
    s.t_max = t_max;
    s.nsplit = (s.esz == 2 && s.nq_pad % 32 == 0) ? scan_splits(s.batch, s.h_kv, s.G, t_max) : 1;
    // a single chunk token makes both pooling orders the same score: the
    // group-pooled path is only taken for chunk_len > 1
    s.pool = (p && p->pooling == KVSEL_POOL_GROUP && s.C > 1) ? 1 : 0;
    s.qsplit = 0;
    return s;
}

// Scan shape of the group-pooled order: one pooled row stream per KV head
// (G = 1), bf16 scans take the rows as [hi | lo] pairs on the MFMA path.
SelShape pooled_shape(const SelShape& s) {
    SelShape p = s;
    p.h_q = s.h_kv;
    p.G = 1;
    p.nq_pad = s.esz == 4 ? s.nqp : static_cast<int>(round_up(s.nqp, 32));
    p.nsplit = 1;
    p.qsplit = s.esz == 2 ? 1 : 0;
    return p;
}

// ----------------------------------------------------------------------------- workspace layout

struct Layout {
    size_t qpart, qcos, qrn, keep, qsel, rq, qbar, scores, topb, idx, rowidx, nsel, kall, vall, apart, total;
    int nk_pad;
};

Layout layout(const SelShape& s, bool with_attn) {
    Layout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += align256(bytes); return o; };
    const size_t bh = size_t(s.batch) * s.h_q, bg = size_t(s.batch) * s.h_kv;
    L.qpart = take(size_t(qstats_part_elems(s)) * 8);
    L.qcos = take(bh * s.C * 4);
    L.qrn = take(bh * s.C * 4);
    L.keep = take(bh * s.nqp * 4);
    size_t qsel_bytes = bg * s.G * s.nq_pad * s.d * s.esz, rq_rows = bg * s.G * s.nq_pad;
    if (s.pool) {                                   // pooled rows: 4*d bytes ([hi | lo] bf16 or fp32)
        const SelShape p = pooled_shape(s);
        qsel_bytes = std::max(qsel_bytes, bg * p.nq_pad * s.d * 4);
        rq_rows = std::max(rq_rows, bg * p.nq_pad);
    }
    L.qsel = take(qsel_bytes);
    L.rq = take(rq_rows * 4);
    L.qbar = s.pool ? take(bg * s.C * s.d * 4) : 0;
    L.scores = take(bg * (s.t_max > 0 ? s.t_max : 1) * 4 * s.nsplit);
    L.topb = take(topb_scratch_bytes(static_cast<int>(bg), s.t_max, s.budget));
    L.idx = take(bg * s.budget * 4);
    L.rowidx = take(bg * s.budget * 4);
    L.nsel = take(size_t(s.batch) * 4);
    const int64_t nsel_max = s.budget < s.t_max ? s.budget : s.t_max;
    L.nk_pad = static_cast<int>(round_up(nsel_max + s.C, 64));
    if (with_attn) {
        if (!attn_use_gather(s)) {           // the gathering attention reads the kept rows in place
            L.kall = take(bg * L.nk_pad * s.d * s.esz);
            L.vall = take(bg * L.nk_pad * s.d * s.esz);
        }
        L.apart = take(attn_part_bytes(s));
    }
    L.total = off;
    return L;
}

// Whether kvsel_prefill_chunk takes the gathering attention (kept rows read in
// place through their cache row numbers, no packed lists) for these shapes.
// (A gathering shape whose cache holds 2^31 rows or more is refused, see
// check_gather_rows: its workspace has no room for packed lists.)
bool prefill_uses_gather(const SelShape& s) { return attn_use_gather(s); }

// Whether kvsel_prefill_chunk attends to the cache prefix in place: nothing is
// selected (every T_b <= budget, so the key list is cache rows [0, T_b) then
// the chunk's rows, which the call appends at [T_b, T_b + C) first) and the
// cache is contiguous; bf16 shapes of the packed attention, with the list's
// byte size and the capacity within the kernel's 32-bit offsets.
bool prefill_inplace(const SelShape& s, const kvsel_cache* c) {
    return s.esz == 2 && !attn_use_gather(s) && c->block_size == 0 && s.t_max <= s.budget &&
           (s.t_max + s.C) * s.d * 2 < (int64_t(1) << 31) && c->capacity < (int64_t(1) << 31) / (s.d * 2);
}

kvsel_status check_gather_rows(const SelShape& s, const kvsel_cache* c, const kvsel_heads* h, const kvsel_batch* b) {
    if (attn_use_gather(s) && !cache_rows_fit(c, h, b))
        return fail(KVSEL_ERR_UNSUPPORTED, "chunks of %d tokens x %d query heads per KV head read the cache through "
                    "int32 row numbers: a cache of 2^31 rows or more is not supported", s.C, s.G);
    return KVSEL_OK;
}

template <typename P> P* at(void* ws, size_t off) { return reinterpret_cast<P*>(static_cast<char*>(ws) + off); }

kvsel_status check_ws(void* ws, size_t have, size_t need) {
    if (need > have) return fail(KVSEL_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    if (!ws) return fail(KVSEL_ERR_WORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(KVSEL_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    return KVSEL_OK;
}

// Steps 1-3 into idx (shared by select and prefill_chunk).
kvsel_status run_select(const SelShape& s, const kvsel_batch* b, const void* q, const CacheView& cv, void* ws,
                        const Layout& L, int32_t* idx, int32_t* q_keep, float* scores, hipStream_t st,
                        int32_t* rowidx = nullptr, const ChunkPack* cp = nullptr, bool* hosted = nullptr) {
    bool any = false;
    for (int i = 0; i < b->batch; ++i) any |= b->prior_len_host[i] > s.budget;
    const int64_t* T = b->prior_len_dev;
    // the scan writes into the workspace (its split partials when s.nsplit > 1);
    // the top-B kernel adds the splits and stores the sum in `scores` if asked
    const SelShape sc = s.pool ? pooled_shape(s) : s;     // the scan's shape
    float* S = (scores && sc.nsplit == 1) ? scores : at<float>(ws, L.scores);
    const int64_t split_stride = int64_t(s.batch) * s.h_kv * s.t_max;
    if (any && s.pool) {
        // group-pooled: the group's unit rows averaged per token, then steps
        // 1-2 on the pooled rows as one head per KV head
        int32_t* keep = q_keep ? q_keep : at<int32_t>(ws, L.keep);
        float* qbar = at<float>(ws, L.qbar);
        SelShape sq = sc;
        sq.esz = 4;                                          // qbar is fp32
        KVSEL_TRY(traced(KVSEL_K_QPOOL, st, [&] { return launch_qpool(s, q, T, qbar, st); }), "query pooling");
        KVSEL_TRY(traced(KVSEL_K_QSTATS, st, [&] { return launch_qstats(sq, qbar, T, at<double>(ws, L.qpart), at<float>(ws, L.qcos), at<float>(ws, L.qrn), at<uint32_t>(ws, L.topb), int64_t(topb_zero_words(s.batch * s.h_kv)), st); }), "query statistics");
        KVSEL_TRY(traced(KVSEL_K_QTOPK, st, [&] { return launch_topk(s.batch * s.h_kv, s.h_kv, at<float>(ws, L.qcos), s.C, 1, 0, nullptr, T, s.C, s.budget, s.nqp, keep, s.nqp,
                              1, s.C, st); }), "query top-k");
        KVSEL_TRY(traced(KVSEL_K_QPACK, st, [&] { return launch_pack_pooled(sc, qbar, keep, s.nqp, T, at<void>(ws, L.qsel), at<float>(ws, L.rq), st); }), "query packing");
        KVSEL_TRY(traced(KVSEL_K_SCAN, st, [&] { return launch_scan(sc, at<void>(ws, L.qsel), at<float>(ws, L.rq), cv, T, S, s.t_max, st, b->prior_len_host); }), "key scan");
    } else if (any) {
        int32_t* keep = q_keep ? q_keep : at<int32_t>(ws, L.keep);
        const bool keep_all = s.nqp == s.C;   // every query kept: no statistics to take (decode)
        if (!keep_all) {
            KVSEL_TRY(traced(KVSEL_K_QSTATS, st, [&] { return launch_qstats(s, q, T, at<double>(ws, L.qpart), at<float>(ws, L.qcos), at<float>(ws, L.qrn), at<uint32_t>(ws, L.topb), int64_t(topb_zero_words(s.batch * s.h_kv)), st); }), "query statistics");
            KVSEL_TRY(traced(KVSEL_K_QTOPK, st, [&] { return launch_topk(s.batch * s.h_q, s.h_q, at<float>(ws, L.qcos), s.C, 1, 0, nullptr, T, s.C, s.budget, s.nqp, keep, s.nqp,
                                  1, s.C, st); }), "query top-k");
        }
        KVSEL_TRY(traced(KVSEL_K_QPACK, st, [&] { return launch_pack_qsel(s, q, keep, s.nqp, at<float>(ws, L.qrn), T, at<void>(ws, L.qsel), at<float>(ws, L.rq), st,
                                                                         keep_all, at<uint32_t>(ws, L.topb), int64_t(topb_zero_words(s.batch * s.h_kv))); }),
                  "query packing");
        KVSEL_TRY(traced(KVSEL_K_SCAN, st, [&] { return launch_scan(s, at<void>(ws, L.qsel), at<float>(ws, L.rq), cv, T, S, s.t_max, st, b->prior_len_host); }), "key scan");
    }
    float* comb = scores ? scores : S;
    KVSEL_TRY(traced(KVSEL_K_TOPB, st, [&] { return launch_topb_hosting(s.batch * s.h_kv, s.h_kv, S, sc.nsplit, split_stride, comb, s.t_max, T,
                                                                        s.budget, s.t_max, any, at<uint32_t>(ws, L.topb), idx, st,
                                                                        rowidx ? &cv : nullptr, rowidx, b->prior_len_host, cp, hosted); }),
              "key top-B");
    return KVSEL_OK;
}

// Checks shared by kvsel_prefill_chunk and kvsel_prefill_chunk_noalloc.
kvsel_status check_prefill(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params,
                           const void* q, const void* k_chunk, const void* v_chunk, const kvsel_cache* cache,
                           int32_t out_dtype, const void* out, int64_t* t_max) {
    kvsel_status st;
    if ((st = check_heads(heads)) || (st = check_batch(batch, true, t_max)) || (st = check_params(params)) ||
        (st = check_select(*t_max, params)) || (st = check_cache(cache, batch, batch->chunk_len)))
        return st;
    if (!q || !k_chunk || !v_chunk || !out) return fail(KVSEL_ERR_INVALID_ARG, "q/k_chunk/v_chunk/out is NULL");
    if (!aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(out))
        return fail(KVSEL_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (out_dtype != KVSEL_F32 && out_dtype != KVSEL_BF16) return fail(KVSEL_ERR_INVALID_ARG, "out_dtype=%d unknown", out_dtype);
    return KVSEL_OK;
}

// One chunk of every sequence on a checked workspace: steps 1-5 and the append.
kvsel_status run_prefill(const kvsel_heads* heads, const kvsel_batch* batch, const SelShape& s, const Layout& L,
                         const void* q, const void* k_chunk, const void* v_chunk, const kvsel_cache* cache,
                         void* out, int32_t out_dtype, int32_t* idx, void* workspace, hipStream_t hs) {
    kvsel_status st;
    const CacheView cv = make_view(cache, heads);
    int32_t* idx_buf = idx ? idx : at<int32_t>(workspace, L.idx);
    const bool gather = prefill_uses_gather(s);
    int32_t* rowidx = gather ? at<int32_t>(workspace, L.rowidx) : nullptr;
    const bool inplace = !gather && prefill_inplace(s, cache);
    // bf16 key lists: their chunk slots and the cache append run in spare
    // workgroups of the top-B threshold launch (most compute units are idle
    // there), the pack launch then copies only the kept prior keys
    ChunkPack cp{};
    const bool host_chunk = !gather && !inplace && s.esz == 2;
    if (host_chunk) {
        cp.cv = cv;
        cp.prior_len = batch->prior_len_dev;
        cp.budget = s.budget;
        cp.k_chunk = static_cast<const char*>(k_chunk);
        cp.v_chunk = static_cast<const char*>(v_chunk);
        cp.kall = at<char>(workspace, L.kall);
        cp.vall = at<char>(workspace, L.vall);
        cp.batch = s.batch;
        cp.h_kv = s.h_kv;
        cp.C = s.C;
        cp.nk_pad = L.nk_pad;
        cp.row_bytes = s.d * s.esz;
        cp.wgs = chunk_pack_wgs(s.batch, s.h_kv, s.C);
    }
    bool hosted = false;
    // nothing to select and no index output asked for: the in-place attention
    // reads no index, so the identity index write is skipped
    if (!(inplace && !idx) &&
        (st = run_select(s, batch, q, cv, workspace, L, idx_buf, nullptr, nullptr, hs, rowidx,
                         host_chunk ? &cp : nullptr, &hosted)))
        return st;
    PackSrc src{};
    src.cache = &cv;
    src.prior_len = batch->prior_len_dev;
    src.budget = s.budget;
    src.idx = idx_buf;
    src.idx_stride = s.budget;
    src.append = !hosted;
    src.chunk_hosted = hosted;
    int32_t* nsel = at<int32_t>(workspace, L.nsel);
    const float scale = heads->scale > 0.0f ? heads->scale : 1.0f / std::sqrt(static_cast<float>(heads->d));
    if (gather) {
        // fused gather: the attention reads the kept rows from the cache itself
        // (row numbers from the top-B); the append runs on its own (it writes
        // rows [T_b, T_b + C), which neither the selection nor the attention reads)
        AttnGather ga{cv, batch->prior_len_dev, s.budget, rowidx, s.budget, k_chunk, v_chunk};
        KVSEL_TRY(traced(KVSEL_K_ATTN, hs, [&] { return launch_attn(s, q, nullptr, nullptr, nullptr, 0, scale, out, out_dtype == KVSEL_F32,
                              at<float>(workspace, L.apart), hs, &ga); }), "attention");
        KVSEL_TRY(traced(KVSEL_K_APPEND, hs, [&] { return launch_append(s, cv, batch->prior_len_dev, k_chunk, v_chunk, hs); }), "cache append");
        return KVSEL_OK;
    }
    if (inplace) {
        // nothing selected: append the chunk, then the key list of every
        // (sequence, KV head) is its cache rows [0, T_b + C), read in place
        KVSEL_TRY(traced(KVSEL_K_APPEND, hs, [&] { return launch_append(s, cv, batch->prior_len_dev, k_chunk, v_chunk, hs); }), "cache append");
        AttnGather ga{cv, batch->prior_len_dev, s.budget, nullptr, 0, k_chunk, v_chunk};
        KVSEL_TRY(traced(KVSEL_K_ATTN, hs, [&] { return launch_attn(s, q, cache->k, cache->v, nullptr, static_cast<int>(cache->capacity), scale,
                                                                    out, out_dtype == KVSEL_F32, at<float>(workspace, L.apart), hs, &ga, true); }),
                  "attention");
        return KVSEL_OK;
    }
    KVSEL_TRY(traced(KVSEL_K_PACK, hs, [&] { return launch_pack(s, src, k_chunk, v_chunk, L.nk_pad, at<void>(workspace, L.kall), at<void>(workspace, L.vall),
                          nsel, hs); }), "pack");
    KVSEL_TRY(traced(KVSEL_K_ATTN, hs, [&] { return launch_attn(s, q, at<void>(workspace, L.kall), at<void>(workspace, L.vall), nsel, L.nk_pad, scale, out,
                          out_dtype == KVSEL_F32, at<float>(workspace, L.apart), hs); }), "attention");
    // here the cache append happens inside the pack kernel (it reads the chunk's rows anyway)
    return KVSEL_OK;
}

// ----------------------------------------------------------------------------- fixed scratch (no-allocation entry)
//
// kvsel_prefill_chunk_noalloc takes its workspace from this array instead of
// a caller buffer.  Each GPU the library runs on holds its own copy (from the
// first call on that GPU until the process ends).  In host code `scratch` only
// names the symbol: its device address, different on every GPU, comes from
// hipGetSymbolAddress once per device (with that device current) and only
// that address is handed to kernels.  Nothing here requires the array to
// start zeroed: every kernel writes what a later one reads (the top-B
// histogram is cleared by the first selection kernel of each call).
constexpr size_t kNoAllocScratchBytes = KVSEL_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

kvsel_status scratch_address(void** out) {
    int dev = -1;
    KVSEL_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(KVSEL_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void* p = nullptr;
        KVSEL_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return fail(KVSEL_ERR_HIP, "scratch address %p not 256-byte aligned", p);
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return KVSEL_OK;
}

}  // namespace

extern "C" {

const char* kvsel_last_error(void) { return g_err.c_str(); }

kvsel_status kvsel_trace_start(uint32_t kernel_mask) {
    g_err.clear();
    std::lock_guard<std::mutex> lk(g_trace.mu);
    g_trace.mask = kernel_mask;
    return KVSEL_OK;
}

kvsel_status kvsel_trace_stop(void) {
    g_err.clear();
    std::lock_guard<std::mutex> lk(g_trace.mu);
    g_trace.mask = 0;
    return KVSEL_OK;
}

kvsel_status kvsel_trace_read(int32_t* launches, float* total_ms, int32_t n) {
    g_err.clear();
    if (!launches || !total_ms || n < 0) return fail(KVSEL_ERR_INVALID_ARG, "launches/total_ms is NULL or n < 0");
    for (int i = 0; i < n; ++i) { launches[i] = 0; total_ms[i] = 0.0f; }
    std::lock_guard<std::mutex> lk(g_trace.mu);
    kvsel_status st = KVSEL_OK;
    for (auto& r : g_trace.recs) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == KVSEL_OK) st = hip_check(e, "trace event");
        if (r.id < n) { launches[r.id] += 1; total_ms[r.id] += ms; }
        g_trace.pool.push_back(r.a);
        g_trace.pool.push_back(r.b);
    }
    g_trace.recs.clear();
    return st;
}

const char* kvsel_kernel_name(int32_t id) { return (id >= 0 && id < KVSEL_K_COUNT) ? kKernelNames[id] : ""; }

int32_t kvsel_version(void) { return 102; }

kvsel_status kvsel_workspace_size(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params,
                                  size_t* bytes) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_heads(heads)) || (st = check_batch(batch, true, &t_max)) || (st = check_params(params)) ||
        (st = check_select(t_max, params)))
        return st;
    if (!bytes) return fail(KVSEL_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = layout(make_shape(heads, batch, params, t_max), true).total;
    return KVSEL_OK;
}

kvsel_status kvsel_compacted_view(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params,
                                  const kvsel_cache* cache, int32_t* packed, size_t* k_offset, size_t* v_offset,
                                  int32_t* slots, int32_t* v_transposed) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_heads(heads)) || (st = check_batch(batch, true, &t_max)) || (st = check_params(params)) ||
        (st = check_select(t_max, params)) || (st = check_cache(cache, batch, batch->chunk_len)))
        return st;
    if (!packed || !k_offset || !v_offset || !slots || !v_transposed)
        return fail(KVSEL_ERR_INVALID_ARG, "an output pointer is NULL");
    const SelShape s = make_shape(heads, batch, params, t_max);
    const Layout L = layout(s, true);
    if ((st = check_gather_rows(s, cache, heads, batch))) return st;
    *packed = (prefill_uses_gather(s) || prefill_inplace(s, cache)) ? 0 : 1;
    *k_offset = L.kall;
    *v_offset = L.vall;
    *slots = L.nk_pad;
    *v_transposed = s.esz == 2 ? 1 : 0;
    return KVSEL_OK;
}

kvsel_status kvsel_sparse_attn_workspace_size(const kvsel_heads* heads, const kvsel_batch* batch, int32_t n_sel_max,
                                              size_t* bytes) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_heads(heads)) || (st = check_batch(batch, false, &t_max))) return st;
    if (n_sel_max < 0 || n_sel_max > kMaxLen) return fail(KVSEL_ERR_INVALID_ARG, "n_sel_max=%d out of range", n_sel_max);
    if (!bytes) return fail(KVSEL_ERR_INVALID_ARG, "bytes is NULL");
    SelShape s = make_shape(heads, batch, nullptr, 0);
    const int nk_pad = static_cast<int>(round_up(int64_t(n_sel_max) + s.C, 64));
    const size_t kv = size_t(s.batch) * s.h_kv * nk_pad * s.d * s.esz;
    *bytes = align256(size_t(s.batch) * 4) + 2 * align256(kv) + align256(attn_part_bytes(s));
    return KVSEL_OK;
}

kvsel_status kvsel_select(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params, const void* q,
                          const kvsel_cache* cache, int32_t* idx, void* k_sel, void* v_sel, int32_t* q_keep,
                          float* scores, void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_heads(heads)) || (st = check_batch(batch, true, &t_max)) || (st = check_params(params)) ||
        (st = check_select(t_max, params)) || (st = check_cache(cache, batch, 0)))
        return st;
    if (!q || !aligned16(q)) return fail(KVSEL_ERR_INVALID_ARG, "q is NULL or not 16-byte aligned");
    if (!idx) return fail(KVSEL_ERR_INVALID_ARG, "idx is NULL");
    if ((k_sel == nullptr) != (v_sel == nullptr)) return fail(KVSEL_ERR_INVALID_ARG, "give both k_sel and v_sel, or neither");
    if (k_sel && (!aligned16(k_sel) || !aligned16(v_sel))) return fail(KVSEL_ERR_INVALID_ARG, "k_sel/v_sel must be 16-byte aligned");
    const SelShape s = make_shape(heads, batch, params, t_max);
    const Layout L = layout(s, false);
    if ((st = check_ws(workspace, workspace_bytes, L.total))) return st;
    const CacheView cv = make_view(cache, heads);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if ((st = run_select(s, batch, q, cv, workspace, L, idx, q_keep, scores, hs))) return st;
    if (k_sel) KVSEL_TRY(traced(KVSEL_K_GATHER, hs, [&] { return launch_gather(s, cv, batch->prior_len_dev, idx, s.budget, k_sel, v_sel, hs); }), "gather");
    return KVSEL_OK;
}

kvsel_status kvsel_sparse_attn(const kvsel_heads* heads, const kvsel_batch* batch, const void* q, const void* k_sel,
                               const void* v_sel, const int32_t* n_sel, int32_t n_sel_max, const void* k_chunk,
                               const void* v_chunk, void* out, int32_t out_dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_heads(heads)) || (st = check_batch(batch, false, &t_max))) return st;
    if (n_sel_max < 0 || n_sel_max > kMaxLen) return fail(KVSEL_ERR_INVALID_ARG, "n_sel_max=%d out of range", n_sel_max);
    if (!q || !k_chunk || !v_chunk || !out || !n_sel) return fail(KVSEL_ERR_INVALID_ARG, "q/k_chunk/v_chunk/out/n_sel is NULL");
    if (n_sel_max > 0 && (!k_sel || !v_sel)) return fail(KVSEL_ERR_INVALID_ARG, "k_sel/v_sel is NULL");
    if (!aligned16(q) || !aligned16(k_chunk) || !aligned16(v_chunk) || !aligned16(out) || !aligned16(k_sel) || !aligned16(v_sel))
        return fail(KVSEL_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if (out_dtype != KVSEL_F32 && out_dtype != KVSEL_BF16) return fail(KVSEL_ERR_INVALID_ARG, "out_dtype=%d unknown", out_dtype);
    size_t need;
    if ((st = kvsel_sparse_attn_workspace_size(heads, batch, n_sel_max, &need))) return st;
    if ((st = check_ws(workspace, workspace_bytes, need))) return st;
    const SelShape s = make_shape(heads, batch, nullptr, 0);
    const int nk_pad = static_cast<int>(round_up(int64_t(n_sel_max) + s.C, 64));
    const size_t kv = size_t(s.batch) * s.h_kv * nk_pad * s.d * s.esz;
    int32_t* nsel_ws = at<int32_t>(workspace, 0);
    void* kall = at<void>(workspace, align256(size_t(s.batch) * 4));
    void* vall = at<void>(workspace, align256(size_t(s.batch) * 4) + align256(kv));
    float* apart = at<float>(workspace, align256(size_t(s.batch) * 4) + 2 * align256(kv));
    PackSrc src{};
    src.k_compact = k_sel;
    src.v_compact = v_sel;
    src.n_sel = n_sel;
    src.n_sel_max = n_sel_max;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const float scale = heads->scale > 0.0f ? heads->scale : 1.0f / std::sqrt(static_cast<float>(heads->d));
    KVSEL_TRY(traced(KVSEL_K_PACK, hs, [&] { return launch_pack(s, src, k_chunk, v_chunk, nk_pad, kall, vall, nsel_ws, hs); }), "pack");
    KVSEL_TRY(traced(KVSEL_K_ATTN, hs, [&] { return launch_attn(s, q, kall, vall, nsel_ws, nk_pad, scale, out, out_dtype == KVSEL_F32, apart, hs); }), "attention");
    return KVSEL_OK;
}

kvsel_status kvsel_prefill_chunk(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params,
                                 const void* q, const void* k_chunk, const void* v_chunk, const kvsel_cache* cache,
                                 void* out, int32_t out_dtype, int32_t* idx, void* workspace, size_t workspace_bytes,
                                 void* stream) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_prefill(heads, batch, params, q, k_chunk, v_chunk, cache, out_dtype, out, &t_max))) return st;
    const SelShape s = make_shape(heads, batch, params, t_max);
    if ((st = check_gather_rows(s, cache, heads, batch))) return st;
    const Layout L = layout(s, true);
    if ((st = check_ws(workspace, workspace_bytes, L.total))) return st;
    return run_prefill(heads, batch, s, L, q, k_chunk, v_chunk, cache, out, out_dtype, idx, workspace,
                       static_cast<hipStream_t>(stream));
}

kvsel_status kvsel_decode_reuse(const kvsel_heads* heads, const kvsel_batch* batch, const kvsel_params* params,
                                const void* q, const void* k_new, const void* v_new, const kvsel_cache* cache,
                                const kvsel_sel_cache* sel, void* out, int32_t out_dtype, int32_t* idx,
                                void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_prefill(heads, batch, params, q, k_new, v_new, cache, out_dtype, out, &t_max))) return st;
    if (!sel || !sel->k || !sel->v || !sel->pos) return fail(KVSEL_ERR_INVALID_ARG, "sel / sel->k / sel->v / sel->pos is NULL");
    if (!aligned16(sel->k) || !aligned16(sel->v)) return fail(KVSEL_ERR_INVALID_ARG, "sel->k / sel->v must be 16-byte aligned");
    if (heads->dtype != KVSEL_BF16) return fail(KVSEL_ERR_UNSUPPORTED, "the selected-entry cache is implemented for bf16");
    if (params->budget > kReuseMaxBudget)
        return fail(KVSEL_ERR_UNSUPPORTED, "budget=%d: the selected-entry cache holds at most %d slots", params->budget, kReuseMaxBudget);
    const SelShape s = make_shape(heads, batch, params, t_max);
    if (!attn_use_gather(s))
        return fail(KVSEL_ERR_UNSUPPORTED, "decode reuse needs (h_q / h_kv) * chunk_len <= 128 (got %d)", s.G * s.C);
    if ((st = check_gather_rows(s, cache, heads, batch))) return st;
    if (int64_t(s.batch) * s.h_kv * s.budget >= (int64_t(1) << 31))
        return fail(KVSEL_ERR_UNSUPPORTED, "the selected-entry cache holds 2^31 slots or more");
    const Layout L = layout(s, true);
    if ((st = check_ws(workspace, workspace_bytes, L.total))) return st;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const CacheView cv = make_view(cache, heads);
    int32_t* idx_buf = idx ? idx : at<int32_t>(workspace, L.idx);
    if ((st = run_select(s, batch, q, cv, workspace, L, idx_buf, nullptr, nullptr, hs))) return st;
    KVSEL_TRY(traced(KVSEL_K_REUSE, hs, [&] { return launch_reuse(s, cv, batch->prior_len_dev, idx_buf, sel->k, sel->v, sel->pos,
                                                                  sel->counts, hs); }), "selected-entry cache update");
    // the slot buffer as a contiguous cache of `budget` rows per (sequence, KV head)
    CacheView sv = cv;
    sv.k = static_cast<char*>(sel->k);
    sv.v = static_cast<char*>(sel->v);
    sv.capacity = s.budget;
    sv.block_size = 0;
    sv.block_table = nullptr;
    AttnGather ga{sv, batch->prior_len_dev, s.budget, nullptr, s.budget, k_new, v_new, 1};
    const float scale = heads->scale > 0.0f ? heads->scale : 1.0f / std::sqrt(static_cast<float>(heads->d));
    KVSEL_TRY(traced(KVSEL_K_ATTN, hs, [&] { return launch_attn(s, q, nullptr, nullptr, nullptr, 0, scale, out, out_dtype == KVSEL_F32,
                                                                at<float>(workspace, L.apart), hs, &ga); }), "attention");
    KVSEL_TRY(traced(KVSEL_K_APPEND, hs, [&] { return launch_append(s, cv, batch->prior_len_dev, k_new, v_new, hs); }), "cache append");
    return KVSEL_OK;
}

kvsel_status kvsel_prefill_chunk_noalloc(const kvsel_heads* heads, const kvsel_batch* batch,
                                         const kvsel_params* params, const void* q, const void* k_chunk,
                                         const void* v_chunk, const kvsel_cache* cache, void* out,
                                         int32_t out_dtype, int32_t* idx, void* stream) {
    g_err.clear();
    kvsel_status st;
    int64_t t_max;
    if ((st = check_prefill(heads, batch, params, q, k_chunk, v_chunk, cache, out_dtype, out, &t_max))) return st;
    const SelShape s = make_shape(heads, batch, params, t_max);
    if ((st = check_gather_rows(s, cache, heads, batch))) return st;
    const Layout L = layout(s, true);
    if (L.total > kNoAllocScratchBytes)
        return fail(KVSEL_ERR_UNSUPPORTED, "these shapes need %zu bytes of workspace; the fixed scratch array holds %zu "
                    "(use kvsel_prefill_chunk with a caller workspace)", L.total, kNoAllocScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_address(&ws))) return st;
    NoTraceScope no_trace;                        // trace events are created lazily: none on this path
    return run_prefill(heads, batch, s, L, q, k_chunk, v_chunk, cache, out, out_dtype, idx, ws,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
