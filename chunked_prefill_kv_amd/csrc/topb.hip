// Per-KV-head top-B over the key scores, spread over many workgroups.
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(a)-(b): the
// best-scoring keys of the cache are kept.  Exact: the B largest scores, ties
// to the lower index, indices written ascending (the same result as the
// single-workgroup radix select in select.hip).
//
//   topb_hist    (problem x segment)  sum the scan's split partials into the
//                score, store it, and count it into a 4096-bin value
//                histogram (bin = floor((s + 1) * 2048), monotone in s);
//   topb_thresh  (problem)            boundary bin from the histogram, the keys
//                of that bin collected in one pass, the exact threshold key tau
//                and the number of keys equal to tau that are kept, and per
//                segment the number of kept keys above / equal to tau;
//   topb_write   (problem x segment)  ordered write of the kept indices.
// For few short problems topb_thresh also does topb_hist's work (its
// workgroup holds the problem's scores in registers).  With the prior lengths
// on the host, the segment grids list only the segments that have keys.
#include <algorithm>

#include "chunk_pack.h"

namespace kvsel {

namespace {

constexpr int kBins = 4096;
constexpr int kSeg = kTopbSegKeys;   // keys per segment (one workgroup of 256 threads, 8 keys each)
static_assert(kSeg == 8 * 256, "a segment is 8 keys per thread of a 256-thread workgroup");
constexpr int kCap = 6144;        // boundary-bin keys kept in LDS by topb_thresh

// floor((v + 1) * 2048) clamped to [0, kBins): the product is exact (a power
// of two), so one fma rounds as the sum does, and clamping before the floor
// gives the same bin (scores are finite)
__device__ __forceinline__ int value_bin(float v) {
    const float x = __builtin_amdgcn_fmed3f(fmaf(v, 2048.0f, 2048.0f), 0.0f, float(kBins - 1));
    return static_cast<int>(floorf(x));
}

struct TopbArgs {
    const float* part;        // scan output: split s at part + s * split_stride
    int nsplit;
    int64_t split_stride;
    float* comb;              // summed scores (== part when nsplit == 1)
    int64_t s_stride;         // per problem
    const int64_t* prior_len;
    int heads_per_seq;
    int64_t budget;
    int nseg;
    uint32_t* hist;           // [problem][kBins]
    uint32_t* thr;            // [problem][2]: tau, need_eq
    uint32_t* segc;           // [problem][nseg][2]: kept above tau, equal to tau
    int32_t* out;             // [problem][budget]
    CacheView cv;             // with rowidx: the cache the positions index
    int32_t* rowidx;          // optional [problem][budget]: cache row number of each kept position
    int problems;             // threshold workgroups; those past them run the ChunkPack items
};

}  // namespace

// Workgroup -> (problem, segment): through the per-sequence list, or the full
// problems x segments grid.
__device__ __forceinline__ void segment_of(const TopbArgs& a, const TileMap& m, int& p, int& seg) {
    if (m.n > 0) {
        int b, g;
        tile_map_slot(m, a.heads_per_seq, b, g, seg);
        p = b * a.heads_per_seq + g;
    } else {
        p = blockIdx.x / a.nseg;
        seg = blockIdx.x % a.nseg;
    }
}

// SPLIT: the scan left more than one split partial (the one-split form keeps
// no registers for the other splits' loads).
template <bool SPLIT>
__global__ __launch_bounds__(256) void topb_hist_kernel(TopbArgs a, TileMap m) {
    int p, seg;
    segment_of(a, m, p, seg);
    const int j0 = seg * kSeg;
    // the first split's scores are requested before the prior length is known
    // (inside the problem's row of s_stride entries; keys past T are dropped)
    const float* x = a.part + static_cast<int64_t>(p) * a.s_stride;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t j = j0 + i * 256 + threadIdx.x;
        v[i] = x[j < a.s_stride ? j : a.s_stride - 1];
    }
    const int64_t T = a.prior_len[p / a.heads_per_seq];
    if (T <= a.budget) return;
    if (j0 >= T) return;
    __shared__ uint32_t lh[kBins];
    for (int i = threadIdx.x; i < kBins; i += 256) lh[i] = 0;
    __syncthreads();
    // the other splits' partials, four splits' loads in flight at a time,
    // added in split order
    if (SPLIT)
    for (int sp0 = 1; sp0 < a.nsplit; sp0 += 4) {
        float w[4][8];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = j0 + i * 256 + threadIdx.x;
                w[q][i] = (sp0 + q < a.nsplit && j < T) ? x[(sp0 + q) * a.split_stride + j] : 0.0f;
            }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (sp0 + q < a.nsplit) v[i] += w[q][i];
    }
    float* c = a.comb + static_cast<int64_t>(p) * a.s_stride;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = j0 + i * 256 + threadIdx.x;
        if (j < T) {
            if (a.nsplit > 1 || c != x) c[j] = v[i];
            atomicAdd(&lh[value_bin(v[i])], 1u);
        }
    }
    __syncthreads();
    uint32_t* h = a.hist + static_cast<int64_t>(p) * kBins;
    for (int i = threadIdx.x; i < kBins; i += 256)
        if (lh[i]) atomicAdd(&h[i], lh[i]);
}

// Exclusive scan over the 1024 threads of the workgroup (ascending thread id).
__device__ __forceinline__ uint32_t excl_scan_1024(uint32_t v, uint32_t* wsum) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t off = 0;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    __syncthreads();
    return off + incl - v;
}

// FUSED (problems of at most kFusedKeys keys): the workgroup also sums the
// scan's split partials and counts the histogram itself, with every score of
// the problem held in registers (no histogram launch, one read of the scores).
constexpr int kFusedSteps = 4;                  // 8192-key steps held in registers
constexpr int kFusedKeys = kFusedSteps * 8192;
template <bool FUSED, int NST>
__global__ __launch_bounds__(1024) void topb_thresh_kernel(TopbArgs a, ChunkPack cp) {
    static_assert(!FUSED || NST == kFusedSteps, "the fused form holds every step");
    __shared__ uint32_t hs[kBins];
    __shared__ uint32_t ck[kCap];
    __shared__ int cj[kCap];
    __shared__ uint32_t sgt[kTopbMaxSegments], seq_[kTopbMaxSegments];   // per-segment counts
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t s_bin, s_need, s_cnt, s_digit, s_rem, s_full;
    static_assert(sizeof(hs) >= 64 * 128 * 2, "the histogram holds a 64 x 128 bf16 staging tile");
    if (static_cast<int>(blockIdx.x) >= a.problems) {      // spare workgroups: the chunk's key-list slots
        chunk_pack_wg(cp, static_cast<int>(blockIdx.x) - a.problems, reinterpret_cast<uint16_t*>(hs));
        return;
    }
    const int p = blockIdx.x;
    const int64_t T64 = a.prior_len[p / a.heads_per_seq];
    if (T64 <= a.budget) return;
    const int T = static_cast<int>(T64);
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const float* c = a.comb + static_cast<int64_t>(p) * a.s_stride;
    // The scores pass over the keys in 8192-key steps (wave w takes
    // [base0 + 512 w, +512) in 8 loads of 64), held in a ring of NST steps of
    // registers: FUSED holds every step; otherwise the first NST steps are
    // requested before the histogram (they arrive while the boundary bin is
    // found) and each later step NST steps ahead.
    float vs[NST][8];                              // key 8192 st + 512 wave + 64 i + lane
    auto load_step = [&](int st, float (&dst)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = st * 8192 + wave * 512 + i * kWave + lane;
            dst[i] = c[j < T ? j : T - 1];
        }
    };
    if constexpr (FUSED) {
        // the scan's partials added in split order (as the histogram launch
        // does), the sum kept in registers and stored as the score
        const float* x = a.part + static_cast<int64_t>(p) * a.s_stride;
        float* cw = a.comb + static_cast<int64_t>(p) * a.s_stride;
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = st * 8192 + wave * 512 + i * kWave + lane;
                vs[st][i] = x[j < T ? j : T - 1];
            }
        for (int sp = 1; sp < a.nsplit; ++sp)
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int j = st * 8192 + wave * 512 + i * kWave + lane;
                    if (j < T) vs[st][i] += x[sp * a.split_stride + j];
                }
        if (a.nsplit > 1 || cw != x) {
#pragma unroll
            for (int st = 0; st < NST; ++st)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int j = st * 8192 + wave * 512 + i * kWave + lane;
                    if (j < T) cw[j] = vs[st][i];
                }
        }
        for (int i = tid; i < kBins; i += 1024) hs[i] = 0;
    } else {
#pragma unroll
        for (int st = 0; st < NST; ++st)
            if (st * 8192 < T) load_step(st, vs[st]);
        const uint32_t* h = a.hist + static_cast<int64_t>(p) * kBins;
        for (int i = tid; i < kBins; i += 1024) hs[i] = h[i];
    }
    for (int i = tid; i < a.nseg; i += 1024) { sgt[i] = 0; seq_[i] = 0; }
    if (tid == 0) { s_cnt = 0; s_bin = 0; s_need = 1; s_digit = 0; s_rem = 1; }
    __syncthreads();
    if constexpr (FUSED) {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            if ((st + 1) * 8192 <= T) {          // a whole step of keys: no per-key test
#pragma unroll
                for (int i = 0; i < 8; ++i) atomicAdd(&hs[value_bin(vs[st][i])], 1u);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int j = st * 8192 + wave * 512 + i * kWave + lane;
                    if (j < T) atomicAdd(&hs[value_bin(vs[st][i])], 1u);
                }
            }
        }
        __syncthreads();
    }
    // boundary bin: thread t owns bins 4(1023-t) .. +3, scanned from the top
    {
        const int t = 1023 - tid;
        uint32_t hb[4], hsum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { hb[i] = hs[4 * t + i]; hsum += hb[i]; }
        uint32_t above = excl_scan_1024(hsum, wsum);
        const uint32_t k = static_cast<uint32_t>(a.budget);
#pragma unroll
        for (int i = 3; i >= 0; --i) {
            if (above < k && above + hb[i] >= k) { s_bin = 4 * t + i; s_need = k - above; }
            above += hb[i];
        }
    }
    __syncthreads();
    const int bstar = static_cast<int>(s_bin);
    const uint32_t need = s_need;                 // keys kept from the boundary bin
    // one pass: keys above the boundary bin are counted per segment, boundary
    // keys collected.  Wave w takes keys [base0 + 512 w, +512) in 8 slices of
    // 64 (one segment: the count stays in a register, one LDS atomic per wave
    // and pass).  With several steps in registers (FUSED or NST > 1) a step's
    // boundary keys reserve their slots with one atomic for all 8 slices (base
    // broadcast by readfirstlane) and are written in slice order: 5-10% off the
    // top-B of the prefill layers.  With one step in flight (many problems,
    // decode) the per-slice form, one atomic per slice that holds boundary
    // keys, measured faster (93 against 102 us per 64-sequence decode step).
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int st0 = 0; st0 * 8192 < T; st0 += NST)
#pragma unroll
    for (int r = 0; r < NST; ++r) {
        const int st = st0 + r;
        const int base0 = st * 8192;
        if (base0 >= T) break;
        const int wbase = base0 + wave * 512;
        float cur[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = vs[r][i];
        if (!FUSED && (st + NST) * 8192 < T) load_step(st + NST, vs[r]);
        uint32_t ngt = 0;
        if constexpr (FUSED || NST > 1) {
            uint32_t neq = 0;
            int bn[8];
            uint64_t beq[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = wbase + i * kWave + lane;
                bn[i] = j < T ? value_bin(cur[i]) : -1;
                ngt += static_cast<uint32_t>(__popcll(__ballot(bn[i] > bstar)));
                beq[i] = __ballot(bn[i] == bstar);
                neq += static_cast<uint32_t>(__popcll(beq[i]));
            }
            if (neq) {                               // (uniform) this step's boundary keys
                uint32_t first = 0;
                if (lane == 0) first = atomicAdd(&s_cnt, neq);
                uint32_t pos = __builtin_amdgcn_readfirstlane(first);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    if (bn[i] == bstar) {
                        const uint32_t at = pos + static_cast<uint32_t>(__popcll(beq[i] & lt));
                        if (at < kCap) { ck[at] = order_key(cur[i]); cj[at] = wbase + i * kWave + lane; }
                    }
                    pos += static_cast<uint32_t>(__popcll(beq[i]));
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int j = wbase + i * kWave + lane;
                const int bn = j < T ? value_bin(cur[i]) : -1;
                ngt += static_cast<uint32_t>(__popcll(__ballot(bn > bstar)));
                const uint64_t beq = __ballot(bn == bstar);
                if (beq) {
                    uint32_t first = 0;
                    if (lane == 0) first = atomicAdd(&s_cnt, static_cast<uint32_t>(__popcll(beq)));
                    first = __shfl(first, 0, kWave);
                    if (bn == bstar) {
                        const uint32_t pos = first + static_cast<uint32_t>(__popcll(beq & lt));
                        if (pos < kCap) { ck[pos] = order_key(cur[i]); cj[pos] = j; }
                    }
                }
            }
        }
        if (lane == 0 && ngt) atomicAdd(&sgt[wbase / kSeg], ngt);
    }
    __syncthreads();
    const uint32_t cnt = s_cnt;
    const bool in_lds = cnt <= kCap;
    // exact radix select of the need-th largest key among the boundary keys
    auto bkey = [&](int i, bool& ok) -> uint32_t {   // i-th boundary key (LDS), or key i of the problem (global)
        if (in_lds) { ok = i < static_cast<int>(cnt); return ok ? ck[i] : 0u; }
        const float v = c[i];
        ok = i < T && value_bin(v) == bstar;
        return ok ? order_key(v) : 0u;
    };
    const int n_scan = in_lds ? static_cast<int>(cnt) : T;
    uint32_t prefix = 0, remaining = need;
    int bits0 = 32;
    if (in_lds) {
        // the boundary keys share one value bin, so their leading bits agree:
        // the radix passes start below the highest bit in which any differs
        const uint32_t first = ck[0];
        uint32_t diff = 0;
        for (int i = tid; i < n_scan; i += 1024) diff |= ck[i] ^ first;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) diff |= __shfl_xor(diff, o, kWave);
        if (lane == 0) wsum[wave] = diff;
        __syncthreads();
        diff = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) diff |= wsum[w];
        __syncthreads();
        bits0 = diff ? 32 - __clz(diff) : 0;
        prefix = bits0 == 32 ? 0u : (first >> bits0) << bits0;
    }
    for (int bits = bits0; bits > 0;) {
        const int w = bits < 11 ? bits : 11, shift = bits - w;
        for (int i = tid; i < 2048; i += 1024) hs[i] = 0;
        __syncthreads();
        for (int i = tid; i < n_scan; i += 1024) {
            bool ok;
            const uint32_t u = bkey(i, ok);
            if (ok && (bits == 32 || (u >> bits) == (prefix >> bits))) atomicAdd(&hs[(u >> shift) & ((1u << w) - 1u)], 1u);
        }
        __syncthreads();
        const int t = 1023 - tid;
        const uint32_t h0 = hs[2 * t], h1 = hs[2 * t + 1];
        const uint32_t above = excl_scan_1024(h0 + h1, wsum);
        if (above < remaining && above + h1 >= remaining) {
            s_digit = 2 * t + 1;
            s_rem = remaining - above;
            s_full = remaining - above == h1 ? 1u : 0u;          // every key of the bin is kept
        } else if (above + h1 < remaining && above + h1 + h0 >= remaining) {
            s_digit = 2 * t;
            s_rem = remaining - above - h1;
            s_full = remaining - above - h1 == h0 ? 1u : 0u;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        remaining = s_rem;
        bits = shift;
        if (s_full && bits > 0 && prefix > 0) {
            // the kept boundary keys are exactly those >= prefix: tau sits just
            // below them and no key equal to it is kept
            prefix -= 1;
            remaining = 0;
            bits = 0;
        }
        __syncthreads();
    }
    const uint32_t tau = prefix, need_eq = remaining;
    // boundary keys above tau / equal to tau, per segment
    for (int i = tid; i < n_scan; i += 1024) {
        bool ok;
        const uint32_t u = bkey(i, ok);
        if (!ok) continue;
        const int j = in_lds ? cj[i] : i;
        if (u > tau) atomicAdd(&sgt[j / kSeg], 1u);
        else if (u == tau) atomicAdd(&seq_[j / kSeg], 1u);
    }
    __syncthreads();
    uint32_t* sc = a.segc + static_cast<int64_t>(p) * a.nseg * 2;
    for (int i = tid; i < a.nseg; i += 1024) { sc[2 * i] = sgt[i]; sc[2 * i + 1] = seq_[i]; }
    if (tid == 0) {
        a.thr[2 * p] = tau;
        a.thr[2 * p + 1] = need_eq;
    }
}

__global__ __launch_bounds__(256) void topb_write_kernel(TopbArgs a, TileMap m) {
    int p, seg;
    segment_of(a, m, p, seg);
    // wave w owns keys [j0 + 512 w, j0 + 512 (w + 1)) in 8 steps of 64; the
    // scores are requested first, before the prior length, the threshold and
    // the earlier segments' counts (inside the problem's row of s_stride
    // entries; keys past T are not used)
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const float* c = a.comb + static_cast<int64_t>(p) * a.s_stride;
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t j = seg * kSeg + wave * 512 + i * kWave + lane;
        sv[i] = c[j < a.s_stride ? j : a.s_stride - 1];
    }
    const int64_t T64 = a.prior_len[p / a.heads_per_seq];
    int32_t* o = a.out + static_cast<int64_t>(p) * a.budget;
    const int j0 = seg * kSeg;
    const int bq = p / a.heads_per_seq, gq = p % a.heads_per_seq;
    int32_t* ri = a.rowidx ? a.rowidx + static_cast<int64_t>(p) * a.budget : nullptr;
    if (T64 <= a.budget) {                     // everything is kept: iota, then -1 up to budget
        for (int i = threadIdx.x; i < kSeg; i += 256) {
            const int64_t j = j0 + i;
            if (j < a.budget) o[j] = j < T64 ? static_cast<int32_t>(j) : -1;
            if (ri && j < T64) ri[j] = static_cast<int32_t>(a.cv.row_index(bq, gq, j));
        }
        return;
    }
    const int T = static_cast<int>(T64);
    if (j0 >= T) return;
    const uint32_t tau = a.thr[2 * p], need_eq = a.thr[2 * p + 1];
    const uint32_t* sc = a.segc + static_cast<int64_t>(p) * a.nseg * 2;
    __shared__ uint32_t wcnt[2][4], wbase[2][4];
    {                                          // kept keys in earlier segments, summed by all threads
        uint32_t g = 0, e = 0;
        for (int s = threadIdx.x; s < seg; s += 256) { g += sc[2 * s]; e += sc[2 * s + 1]; }
#pragma unroll
        for (int o2 = 32; o2 >= 1; o2 >>= 1) {
            g += __shfl_xor(g, o2, kWave);
            e += __shfl_xor(e, o2, kWave);
        }
        if (lane == 0) { wbase[0][wave] = g; wbase[1][wave] = e; }
    }
    uint32_t u[8];
    bool in[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        in[i] = j0 + wave * 512 + i * kWave + lane < T;
        u[i] = in[i] ? order_key(sv[i]) : 0u;
    }
    uint32_t ng = 0, ne = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ng += __popcll(__ballot(in[i] && u[i] > tau));
        ne += __popcll(__ballot(in[i] && u[i] == tau));
    }
    if (lane == 0) { wcnt[0][wave] = ng; wcnt[1][wave] = ne; }
    __syncthreads();
    uint32_t gt_run = wbase[0][0] + wbase[0][1] + wbase[0][2] + wbase[0][3];
    uint32_t eq_run = wbase[1][0] + wbase[1][1] + wbase[1][2] + wbase[1][3];
    for (int w = 0; w < wave; ++w) { gt_run += wcnt[0][w]; eq_run += wcnt[1][w]; }
    const uint64_t lt = (1ull << lane) - 1ull;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = j0 + wave * 512 + i * kWave + lane;
        const bool gt = in[i] && u[i] > tau, eq = in[i] && u[i] == tau;
        const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
        const uint32_t gb = gt_run + __popcll(bgt & lt), eb = eq_run + __popcll(beq & lt);
        const uint32_t pos = gt ? gb + min(eb, need_eq) : gb + eb;
        if ((gt || (eq && eb < need_eq)) && pos < static_cast<uint32_t>(a.budget)) {
            o[pos] = j;
            if (ri) ri[pos] = static_cast<int32_t>(a.cv.row_index(bq, gq, j));
        }
        gt_run += __popcll(bgt);
        eq_run += __popcll(beq);
    }
}

int topb_segments(int64_t t_max, int64_t budget) {
    const int64_t n = t_max > budget ? t_max : budget;
    return static_cast<int>((n + kSeg - 1) / kSeg);
}

size_t topb_zero_words(int problems) { return size_t(problems) * kBins; }

size_t topb_scratch_bytes(int problems, int64_t t_max, int64_t budget) {
    const int nseg = topb_segments(t_max, budget);
    return size_t(problems) * (kBins + 2 + 2 * size_t(nseg)) * 4;
}

int chunk_pack_wgs(int batch, int h_kv, int C) {
    const int64_t items = int64_t(batch) * h_kv * ((C + 63) / 64 + 1);
    return static_cast<int>(std::min<int64_t>(items, device_cus()));
}

hipError_t launch_topb(int problems, int heads_per_seq, const float* part, int nsplit, int64_t split_stride,
                       float* comb, int64_t s_stride, const int64_t* prior_len, int64_t budget, int64_t t_max,
                       bool any_select, uint32_t* scratch, int32_t* out, hipStream_t st, const CacheView* cv,
                       int32_t* rowidx, const int64_t* prior_len_host) {
    return launch_topb_hosting(problems, heads_per_seq, part, nsplit, split_stride, comb, s_stride, prior_len, budget,
                               t_max, any_select, scratch, out, st, cv, rowidx, prior_len_host, nullptr, nullptr);
}

hipError_t launch_topb_hosting(int problems, int heads_per_seq, const float* part, int nsplit, int64_t split_stride,
                               float* comb, int64_t s_stride, const int64_t* prior_len, int64_t budget, int64_t t_max,
                               bool any_select, uint32_t* scratch, int32_t* out, hipStream_t st, const CacheView* cv,
                               int32_t* rowidx, const int64_t* prior_len_host, const ChunkPack* cp, bool* hosted) {
    if (hosted) *hosted = false;
    TopbArgs a;
    a.cv = cv ? *cv : CacheView{};
    a.rowidx = cv ? rowidx : nullptr;
    a.part = part;
    a.nsplit = nsplit;
    a.split_stride = split_stride;
    a.comb = comb;
    a.s_stride = s_stride;
    a.prior_len = prior_len;
    a.heads_per_seq = heads_per_seq;
    a.budget = budget;
    a.nseg = topb_segments(t_max, budget);
    a.hist = scratch;
    a.thr = scratch + size_t(problems) * kBins;
    a.segc = a.thr + size_t(problems) * 2;
    a.out = out;
    if (a.nseg > kTopbMaxSegments) return hipErrorInvalidValue;   // rejected on the host before any launch
    // few problems of at most kFusedKeys keys: one fused threshold launch
    // (sums, histogram and threshold from registers) in place of two
    // (and at most two split partials: the workgroup adds them alone)
    const bool fused = problems <= 64 && t_max <= kFusedKeys && nsplit <= 2;
    // with the prior lengths on the host, only the segments with keys (the
    // histogram: of selecting sequences; the write: up to max(T_b, budget))
    const int64_t full = int64_t(problems) * a.nseg;
    const int batch = problems / heads_per_seq;
    TileMap mh, mw;
    dim3 grid_h(static_cast<unsigned>(full)), grid_w(static_cast<unsigned>(full));
    if (build_tile_map(mh, prior_len_host, batch, heads_per_seq, full,
                       [&](int64_t T) -> int64_t { return T > budget ? (T + kSeg - 1) / kSeg : 0; }))
        grid_h = dim3(static_cast<unsigned>(mh.first[batch]));
    if (build_tile_map(mw, prior_len_host, batch, heads_per_seq, full,
                       [&](int64_t T) -> int64_t { return ((T > budget ? T : budget) + kSeg - 1) / kSeg; }))
        grid_w = dim3(static_cast<unsigned>(mw.first[batch]));
    a.problems = problems;
    if (any_select && grid_h.x > 0) {
        // the threshold launch hosts the chunk's key-list slots when asked
        // (at most one workgroup per compute unit beside the thresholds')
        ChunkPack c = cp ? *cp : ChunkPack{};
        if (!cp) c.wgs = 0;
        else if (problems < device_cus()) c.wgs = std::min(c.wgs, device_cus() - problems);
        const dim3 grid_t(static_cast<unsigned>(problems + c.wgs));
        if (hosted) *hosted = c.wgs > 0;
        if (fused) {
            hipLaunchKernelGGL((topb_thresh_kernel<true, kFusedSteps>), grid_t, dim3(1024), 0, st, a, c);
        } else {
            if (nsplit > 1) hipLaunchKernelGGL(topb_hist_kernel<true>, grid_h, dim3(256), 0, st, a, mh);
            else hipLaunchKernelGGL(topb_hist_kernel<false>, grid_h, dim3(256), 0, st, a, mh);
            // fewer problems than CUs: each workgroup keeps four steps of
            // loads in flight (its latency is the launch's); otherwise one
            // step, and more workgroups share each CU (on the 512-problem
            // decode batch: 101 us per step against 113 with four)
            if (problems < device_cus())
                hipLaunchKernelGGL((topb_thresh_kernel<false, 4>), grid_t, dim3(1024), 0, st, a, c);
            else
                hipLaunchKernelGGL((topb_thresh_kernel<false, 1>), grid_t, dim3(1024), 0, st, a, c);
        }
    }
    if (grid_w.x > 0) hipLaunchKernelGGL(topb_write_kernel, grid_w, dim3(256), 0, st, a, mw);
    return hipGetLastError();
}

}  // namespace kvsel
