// Internal launchers of the kvsel kernels (host side).  Each returns the HIP
// status of its launch(es).  Shapes are validated by the C-ABI layer first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace kvsel {

struct SelShape {
    int batch, h_q, h_kv, G, d, C;   // heads, chunk length
    int esz;                          // element bytes (2 = bf16, 4 = fp32)
    int nqp;                          // kept queries per head = min(n_q, C)
    int nq_pad;                       // rows reserved per head in Q_sel (>= nqp)
    int64_t budget;
    int64_t t_max;                    // max_b T_b
    int nsplit;                       // MFMA scan: query-head groups per key tile (1 = no split)
    int pool;                         // 0: per-head max then group mean; 1: group-pooled rows first
    int qsplit;                       // MFMA scan rows are [hi | lo] bf16 pairs of fp32 rows (2*d elements)
};

// Choose how many query-head groups the MFMA scan splits a KV head into: a
// power of two dividing G (at most 8), the smallest that gives >= 512
// workgroups for the largest prior length (counted in 256-key tiles whatever
// the scan's per-launch tile is: every split adds a pass of the top-B over the
// scores, so the split count is not raised with the tile).
inline int scan_splits(int batch, int h_kv, int G, int64_t t_max) {
    const int64_t tiles = (t_max + 255) / 256;
    int ns = 1;
    while (ns < 8 && G % (2 * ns) == 0 && int64_t(batch) * h_kv * tiles * ns < 512) ns *= 2;
    return ns;
}

// Step 1: per (b, h) cosine of each chunk query to the mean query (selection
// key) and 1/|q| of each query.  Sequences with T_b <= budget are skipped.
// part: fp64 scratch of qstats_part_elems(s) elements.  The first pass also
// clears zero[0..zero_n) (the top-B histogram) for the kernels that follow.
hipError_t launch_qstats(const SelShape& s, const void* q, const int64_t* prior_len, double* part,
                         float* qcos, float* qrn, uint32_t* zero, int64_t zero_n, hipStream_t st);
// query rows per statistics workgroup: 64 when that still gives fewer than
// about 1024 workgroups (more loads in flight per CU), else 128
constexpr int kQRowsMin = 64;
inline int64_t qstats_part_elems(const SelShape& s) {
    return int64_t(s.batch) * s.h_q * ((s.C + kQRowsMin - 1) / kQRowsMin) * s.d;
}

// Exact top-k with lower-index tie-break, indices ascending, -1 padded to k.
//   mode 0: the k largest of scores[p][0..n_p)      (n_p = prior_len[p / heads_per_seq])
//   mode 1: the k smallest of scores[p][0..n_fixed) (query keep); problems
//           whose sequence has T_b <= budget are skipped
// When n_p <= k every index [0, n_p) is taken.  max_n bounds every n_p.
// The score of key j is the sum, in split order, of nsplit partial arrays
// scores + s * split_stride; when s_out is given that sum is also stored there
// (same indexing as scores).
hipError_t launch_topk(int problems, int heads_per_seq, const float* scores, int64_t score_stride,
                       int nsplit, int64_t split_stride, float* s_out,
                       const int64_t* prior_len, int n_fixed, int64_t budget, int k,
                       int32_t* out, int64_t out_stride, int mode, int64_t max_n, hipStream_t st);

// Per-KV-head top-B of the (split-partial) key scores on many workgroups:
// writes out[p][0..budget) (kept indices ascending, -1 past T_p) for every
// problem p = b * heads_per_seq + g, and with cv / rowidx given the cache row
// number of every kept position (rowidx[p][r], for the gathering attention).  comb receives the summed scores (may be
// `part` itself).  scratch: topb_scratch_bytes(); its first
// topb_zero_words(problems) words (the histogram) must be zero on entry when
// any_select (launch_qstats or launch_pack_qsel clears them).
// Compute units of the current device (queried once per device; 256 if the
// query fails).  Launch shapes that run in rounds are sized with it.
int device_cus();

// A ragged batch's workgroups listed per sequence in the launch arguments
// (built on the host from the prior lengths), so that a grid holds only the
// workgroups with work: sequence b owns workgroups [first[b], first[b+1]),
// heads x its per-head count, in (head, item) order; len[b] is its prior
// length.  n == 0: no list, the grid spans every sequence up to the longest.
constexpr int kMapSeqs = 256;
struct TileMap {
    int32_t n;
    int32_t first[kMapSeqs + 1];
    int32_t len[kMapSeqs];
};
// Fill m for per-sequence item counts count(T_b) (times heads); false (m.n = 0)
// when the batch is too long to list or the list would not be shorter.
template <typename F>
bool build_tile_map(TileMap& m, const int64_t* prior_len_host, int batch, int heads, int64_t full_grid, F count) {
    m.n = 0;
    if (!prior_len_host || batch > kMapSeqs) return false;
    int64_t acc = 0;
    for (int i = 0; i < batch; ++i) {
        m.first[i] = static_cast<int32_t>(acc);
        m.len[i] = static_cast<int32_t>(prior_len_host[i]);
        acc += count(prior_len_host[i]) * heads;
    }
    m.first[batch] = static_cast<int32_t>(acc);
    if (acc > full_grid || acc > INT32_MAX) return false;
    m.n = batch;
    return true;
}
// Workgroup blockIdx.x of a listed grid -> (sequence b, head g, item t).
__device__ __forceinline__ void tile_map_slot(const TileMap& m, int heads, int& b, int& g, int& t) {
    const int slot = blockIdx.x;
    int lo = 0, hi = m.n;               // the largest b with first[b] <= slot (first[n] > slot)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (m.first[mid] <= slot) lo = mid;
        else hi = mid;
    }
    const int per = (m.first[lo + 1] - m.first[lo]) / heads;
    const int r = slot - m.first[lo];
    b = lo;
    g = r / per;
    t = r % per;
}
// The top-B counts kept keys per 2048-key segment in LDS, for at most
// kTopbMaxSegments segments: max(T_max, budget) <= 2^21.
constexpr int kTopbSegKeys = 2048;
constexpr int kTopbMaxSegments = 1024;
int topb_segments(int64_t t_max, int64_t budget);
size_t topb_scratch_bytes(int problems, int64_t t_max, int64_t budget);
// Words at the start of the top-B scratch that must be zero on entry.
size_t topb_zero_words(int problems);
// The chunk's slots of the packed bf16 key lists ([bg][nk_pad][d] keys,
// [bg][d][nk_pad] values) and the cache append, for a launch to run beside
// its own work (chunk_pack.h); wgs = 0: nothing to run.
struct ChunkPack {
    CacheView cv;
    const int64_t* prior_len;
    int64_t budget;
    const char* k_chunk;
    const char* v_chunk;
    char* kall;
    char* vall;
    int batch, h_kv, C, nk_pad, row_bytes;
    int wgs;                          // workgroups added to the host launch
};
// Workgroups to add for `cp` (its item count, at most one per compute unit).
int chunk_pack_wgs(int batch, int h_kv, int C);
hipError_t launch_topb(int problems, int heads_per_seq, const float* part, int nsplit, int64_t split_stride,
                       float* comb, int64_t s_stride, const int64_t* prior_len, int64_t budget, int64_t t_max,
                       bool any_select, uint32_t* scratch, int32_t* out, hipStream_t st,
                       const CacheView* cv = nullptr, int32_t* rowidx = nullptr,
                       const int64_t* prior_len_host = nullptr);
// The same, with the chunk's part of the key lists run by extra workgroups of
// the threshold launch when that launch happens (*hosted says whether it did;
// if not, nothing of `cp` ran).
hipError_t launch_topb_hosting(int problems, int heads_per_seq, const float* part, int nsplit, int64_t split_stride,
                               float* comb, int64_t s_stride, const int64_t* prior_len, int64_t budget, int64_t t_max,
                               bool any_select, uint32_t* scratch, int32_t* out, hipStream_t st,
                               const CacheView* cv, int32_t* rowidx, const int64_t* prior_len_host,
                               const ChunkPack* cp, bool* hosted);

// Gather the kept query rows of every head into Q_sel[b][g][hh*nq_pad + r][d]
// (raw rows) and rq = 1/|q|; rows r >= nqp repeat row 0 of that head.  With
// keep_all (every chunk query kept, nqp == C: step 1 has nothing to choose and
// launch_qstats / launch_topk are not run) the kept list is the identity,
// written to keep when keep is not NULL, 1/|q| is computed here, and
// zero[0..zero_n) is cleared in place of launch_qstats.
hipError_t launch_pack_qsel(const SelShape& s, const void* q, int32_t* keep, int64_t keep_stride,
                            const float* qrn, const int64_t* prior_len, void* qsel, float* rq,
                            hipStream_t st, bool keep_all = false, uint32_t* zero = nullptr, int64_t zero_n = 0);

// Group-pooled step 1 (s.pool == 1): qbar[b][g][i][d] fp32 = mean over the G
// query heads of g of the unit query rows (sequences with T_b <= budget
// skipped).
hipError_t launch_qpool(const SelShape& s, const void* q, const int64_t* prior_len, float* qbar, hipStream_t st);
// Q_sel of the pooled scan (sp: one "head" per KV head, G = 1): the kept qbar
// rows, as [hi | lo] bf16 pairs when sp.qsplit, else fp32; rq = 1.
hipError_t launch_pack_pooled(const SelShape& sp, const float* qbar, const int32_t* keep, int64_t keep_stride,
                              const int64_t* prior_len, void* qsel, float* rq, hipStream_t st);

// Step 2: S[b][g][j] for j < T_b (sequences with T_b > budget only).  With
// s.nsplit > 1 the MFMA scan writes s.nsplit partial arrays, split k at
// S + k * (batch * h_kv * s_stride), whose sum is the score.
// prior_len_host (optional): the prior lengths on the host; the one-query scan
// then launches only the workgroups that have keys to score
hipError_t launch_scan(const SelShape& s, const void* qsel, const float* rq, const CacheView& cv,
                       const int64_t* prior_len, float* S, int64_t s_stride, hipStream_t st,
                       const int64_t* prior_len_host = nullptr);

// Step 4 for the select API: k_sel[b][g][r] = cache row idx[b][g][r], r < min(budget, T_b).
hipError_t launch_gather(const SelShape& s, const CacheView& cv, const int64_t* prior_len,
                         const int32_t* idx, int64_t idx_stride, void* k_sel, void* v_sel,
                         hipStream_t st);

// Compacted key/value layout consumed by the attention kernels:
//   kall [b][g][nk_pad][d]; vall [b][g][d][nk_pad] (bf16, transposed) or
//   [b][g][nk_pad][d] (fp32).  Slot s < nsel_b: prior key, s < nsel_b + C: the
//   chunk's key s - nsel_b, beyond: zeros.  With src.append the chunk's rows
//   are also written into the cache (the prior rows it reads are [0, T_b), so
//   the two never overlap).
struct PackSrc {
    // prior keys from the cache through idx (cache != nullptr) ...
    const CacheView* cache;
    const int64_t* prior_len;
    int64_t budget;
    const int32_t* idx;
    int64_t idx_stride;
    // ... or, with cache == nullptr, from a caller-supplied compacted array
    // [b][g][n_sel_max][d] (k_compact / v_compact may be NULL when n_sel_max == 0)
    const void* k_compact;
    const void* v_compact;
    const int32_t* n_sel;
    int n_sel_max;
    // cache mode only: also append the chunk's rows to the cache at [T_b, T_b + C)
    bool append;
    // the tiles from n_b to n_b + C (chunk rows only) were written by the
    // top-B launch (ChunkPack): skip them
    bool chunk_hosted;
};
hipError_t launch_pack(const SelShape& s, const PackSrc& src, const void* k_chunk, const void* v_chunk,
                       int nk_pad, void* kall, void* vall, int32_t* nsel_out, hipStream_t st);

// Gathering attention: the key list is read straight from its sources, slot
// s < n_b = min(T_b, budget) from cache row rowidx[b][g][s] (row number as
// written by launch_topb), the chunk's rows after it, no packed copy.
struct AttnGather {
    CacheView cv;
    const int64_t* prior_len;
    int64_t budget;
    const int32_t* rowidx;
    int64_t ri_stride;
    const void* k_chunk;             // [b][h_kv][C][d]
    const void* v_chunk;
    // slot s of (b, g) is row (b * h_kv + g) * ri_stride + s of cv (a contiguous
    // slot buffer, the selected-entry cache); rowidx is then not read
    int identity;
};

// Cross-step reuse of the selected entries (decode): after the top-B wrote idx
// (ascending, n_b = min(budget, T_b) per (b, g)), update the slot buffer
// sel_k / sel_v [b][g][budget][d] and its positions pos [b][g][budget]: a slot
// below n_b whose position is selected again keeps it, the other selected
// positions (misses, ascending) fill the remaining slots below n_b (ascending)
// and their rows are copied from the cache; slots from n_b on become -1.
// counts (optional) [b][g][2]: hits, misses.  budget <= kReuseMaxBudget.
constexpr int kReuseMaxBudget = 8192;
hipError_t launch_reuse(const SelShape& s, const CacheView& cv, const int64_t* prior_len, const int32_t* idx,
                        void* sel_k, void* sel_v, int32_t* pos, int32_t* counts, hipStream_t st);
// bf16 KV heads with a single 128-row block (G * C <= 128: decode, short
// chunks) take the gathering attention: each key row is read by one workgroup
// only, so packing it first is pure extra traffic.
bool attn_use_gather(const SelShape& s);

// Step 5 (packed layout, or gathering when `gather` is given); out is fp32
// (out_f32) or bf16.  When the grid would hold fewer than two workgroups per
// CU (gathering: always) the key tiles of every row block are split over
// attn_ksplit(s) workgroups whose partials (fp32 scratch `part` of
// attn_part_bytes(s) bytes) a merge kernel combines.
// With inplace (every prior key kept, contiguous cache, the chunk already
// appended): kall / vall are the cache's K / V and nk_pad its capacity; the key
// list of (b, g) is cache rows [0, T_b + C) read in place, n_b = T_b from
// gather->prior_len (gather->budget >= every T_b); the 4-wave kernel runs it.
int attn_ksplit(const SelShape& s, bool inplace = false);
size_t attn_part_bytes(const SelShape& s);
hipError_t launch_attn(const SelShape& s, const void* q, const void* kall, const void* vall,
                       const int32_t* nsel, int nk_pad, float scale, void* out, bool out_f32,
                       float* part, hipStream_t st, const AttnGather* gather = nullptr,
                       bool inplace = false);

// Cache append without packing: chunk rows -> cache rows [T_b, T_b + C).
hipError_t launch_append(const SelShape& s, const CacheView& cv, const int64_t* prior_len, const void* k_chunk,
                         const void* v_chunk, hipStream_t st);

}  // namespace kvsel
