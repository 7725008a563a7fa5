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
#include "launch.h"

namespace kvsel {

namespace {

constexpr int kBins = 4096;
constexpr int kSeg = 2048;        // keys per segment (one workgroup of 256 threads, 8 keys each)
constexpr int kCap = 8192;        // boundary-bin keys kept in LDS by topb_thresh

__device__ __forceinline__ int value_bin(float v) {
    const float f = floorf((v + 1.0f) * 2048.0f);
    return f < 0.0f ? 0 : (f > float(kBins - 1) ? kBins - 1 : static_cast<int>(f));
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
};

}  // namespace

__global__ __launch_bounds__(256) void topb_hist_kernel(TopbArgs a) {
    const int p = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
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
    for (int sp = 1; sp < a.nsplit; ++sp) {          // partials added in split order
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = j0 + i * 256 + threadIdx.x;
            if (j < T) v[i] += x[sp * a.split_stride + j];
        }
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

__global__ __launch_bounds__(1024) void topb_thresh_kernel(TopbArgs a) {
    const int p = blockIdx.x;
    const int64_t T64 = a.prior_len[p / a.heads_per_seq];
    if (T64 <= a.budget) return;
    const int T = static_cast<int>(T64);
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    __shared__ uint32_t hs[kBins];
    __shared__ uint32_t ck[kCap];
    __shared__ int cj[kCap];
    __shared__ uint32_t sgt[1024], seq_[1024];      // per-segment counts (nseg <= 1024)
    __shared__ uint32_t wsum[16];
    __shared__ uint32_t s_bin, s_need, s_cnt, s_digit, s_rem;
    const float* c = a.comb + static_cast<int64_t>(p) * a.s_stride;
    // the pass's first scores are requested before the histogram, so they
    // arrive while the boundary bin is found; each later step's scores are
    // requested one step ahead (wave w reads [base0 + 512 w, +512) in 8
    // loads of 64)
    float v[8];
    auto load_step = [&](int base0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = base0 + wave * 512 + i * kWave + lane;
            v[i] = c[j < T ? j : T - 1];
        }
    };
    load_step(0);
    const uint32_t* h = a.hist + static_cast<int64_t>(p) * kBins;
    for (int i = tid; i < kBins; i += 1024) hs[i] = h[i];
    for (int i = tid; i < a.nseg; i += 1024) { sgt[i] = 0; seq_[i] = 0; }
    if (tid == 0) { s_cnt = 0; s_bin = 0; s_need = 1; s_digit = 0; s_rem = 1; }
    __syncthreads();
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
    // keys collected.  Wave w takes keys [base0 + 512 w, +512) in 8 steps of
    // 64 (one segment: the count stays in a register, one LDS atomic per wave
    // and pass), boundary keys are appended with one atomic per wave and step.
    const uint64_t lt = (1ull << lane) - 1ull;
    for (int base0 = 0; base0 < T; base0 += 8 * 1024) {
        const int wbase = base0 + wave * 512;
        float cur[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) cur[i] = v[i];
        if (base0 + 8 * 1024 < T) load_step(base0 + 8 * 1024);
        uint32_t ngt = 0;
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
        if (above < remaining && above + h1 >= remaining) { s_digit = 2 * t + 1; s_rem = remaining - above; }
        else if (above + h1 < remaining && above + h1 + h0 >= remaining) { s_digit = 2 * t; s_rem = remaining - above - h1; }
        __syncthreads();
        prefix |= s_digit << shift;
        remaining = s_rem;
        bits = shift;
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

__global__ __launch_bounds__(256) void topb_write_kernel(TopbArgs a) {
    const int p = blockIdx.x / a.nseg, seg = blockIdx.x % a.nseg;
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
    __shared__ uint32_t wcnt[2][4];
    __shared__ uint32_t base_gt, base_eq;
    if (threadIdx.x == 0) {                    // kept keys in earlier segments
        uint32_t g = 0, e = 0;
        for (int s = 0; s < seg; ++s) { g += sc[2 * s]; e += sc[2 * s + 1]; }
        base_gt = g;
        base_eq = e;
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
    uint32_t gt_run = base_gt, eq_run = base_eq;
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

size_t topb_scratch_bytes(int problems, int64_t t_max, int64_t budget) {
    const int nseg = topb_segments(t_max, budget);
    return size_t(problems) * (kBins + 2 + 2 * size_t(nseg)) * 4;
}

hipError_t launch_topb(int problems, int heads_per_seq, const float* part, int nsplit, int64_t split_stride,
                       float* comb, int64_t s_stride, const int64_t* prior_len, int64_t budget, int64_t t_max,
                       bool any_select, uint32_t* scratch, int32_t* out, hipStream_t st, const CacheView* cv,
                       int32_t* rowidx) {
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
    if (a.nseg > 1024) return hipErrorInvalidValue;    // per-segment counters live in LDS
    const dim3 grid_seg(problems * a.nseg);
    if (any_select) {
        hipLaunchKernelGGL(topb_hist_kernel, grid_seg, dim3(256), 0, st, a);
        hipLaunchKernelGGL(topb_thresh_kernel, dim3(problems), dim3(1024), 0, st, a);
    }
    hipLaunchKernelGGL(topb_write_kernel, grid_seg, dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace kvsel
