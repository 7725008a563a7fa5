// Query sub-selection statistics, exact radix top-k, and Q_sel packing.
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(b) and Fig. 2:
// queries are filtered by their cosine dissimilarity to the chunk's mean
// query (high S_q = low cosine kept); Fig. 1(a): the best-scoring keys of the
// cache are kept.  Both selections here are exact (no bucketing): a radix
// select finds the k-th key, ties go to the lower index, and the kept indices
// are written in ascending order.
#include "launch.h"

namespace kvsel {

// ----------------------------------------------------------------------------- helpers

template <typename T> struct Vec8;
template <> struct Vec8<uint16_t> {   // 8 bf16 = one 16-byte load
    static __device__ __forceinline__ void load(const uint16_t* p, float* out) {
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(v[i] << 16);
            out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
        }
    }
};
template <> struct Vec8<float> {      // 8 fp32 = two 16-byte loads
    static __device__ __forceinline__ void load(const float* p, float* out) {
        f32x4 a = *reinterpret_cast<const f32x4*>(p);
        f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { out[i] = a[i]; out[4 + i] = b[i]; }
    }
};

// ----------------------------------------------------------------------------- step 1 statistics
//
// Two passes over the chunk's queries, both spread over (head, 256-row block)
// workgroups with coalesced 16-byte loads.  Sums, dot products and norms are
// accumulated in fp64 (the inputs are exact in fp32), so the selection key
// carries only its final fp32 rounding.


// pass 1: per (head, row block) column sums of the query rows -> part[bh][blk][D] (fp64)
template <typename T, int D, int QR>
__global__ __launch_bounds__(256) void qsum_kernel(const T* __restrict__ q, int h_q, int C, int nblk,
                                                   const int64_t* __restrict__ prior_len, int64_t budget,
                                                   double* __restrict__ part, uint32_t* __restrict__ zero,
                                                   int64_t zero_n) {
    constexpr int G8 = D / 8;                 // 8-column groups per row
    constexpr int RPP = 256 / G8;             // rows per pass
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < zero_n; i += int64_t(gridDim.x) * 256) zero[i] = 0;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const T* qh = q + static_cast<int64_t>(bh) * C * D;
    const int c8 = threadIdx.x % G8, sub = threadIdx.x / G8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int r1 = min(C, (blk + 1) * QR);
    constexpr int NIT = QR / RPP;
    float x[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {           // all loads in flight first, before the prior length
        const int r = blk * QR + sub + it * RPP;
        if (r < r1) Vec8<T>::load(qh + static_cast<int64_t>(r) * D + c8 * 8, x[it]);
        else for (int i = 0; i < 8; ++i) x[it][i] = 0.0f;
    }
    if (prior_len[bh / h_q] <= budget) return;
#pragma unroll
    for (int it = 0; it < NIT; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += static_cast<double>(x[it][i]);
    __shared__ double red[RPP][D];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[sub][c8 * 8 + i] = acc[i];
    __syncthreads();
    if (threadIdx.x < D) {
        double s = 0.0;
        for (int k = 0; k < RPP; ++k) s += red[k][threadIdx.x];
        part[(static_cast<int64_t>(bh) * nblk + blk) * D + threadIdx.x] = s;
    }
}

// pass 2: mean query from the partial sums, then cos(q_i, mean) and 1/|q_i| per row
template <typename T, int D, int QR>
__global__ __launch_bounds__(256) void qcos_kernel(const T* __restrict__ q, int h_q, int C, int nblk,
                                                   const int64_t* __restrict__ prior_len, int64_t budget,
                                                   const double* __restrict__ part, float* __restrict__ qcos,
                                                   float* __restrict__ qrn) {
    constexpr int G8 = D / 8;
    constexpr int RPP = 256 / G8;
    const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    // this block's query rows are loaded first (before the prior length), so
    // they arrive while the mean is formed
    const int c8 = threadIdx.x % G8, sub = threadIdx.x / G8;
    const T* qh = q + static_cast<int64_t>(bh) * C * D;
    const int r1 = min(C, (blk + 1) * QR);
    constexpr int NIT = QR / RPP;
    float x[NIT][8];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int r = blk * QR + sub + it * RPP;
        if (r < r1) Vec8<T>::load(qh + static_cast<int64_t>(r) * D + c8 * 8, x[it]);
        else for (int i = 0; i < 8; ++i) x[it][i] = 0.0f;
    }
    if (prior_len[bh / h_q] <= budget) return;
    __shared__ double mean[D];
    __shared__ double mnorm;
    {
        // column sums of the partials: every thread takes one column and every
        // NS-th block, 16 loads in flight.  fp64 sums of bf16 rows are exact,
        // so the order of the additions does not change the mean; for fp32
        // rows it can only move the last bits of the fp64 mean.
        constexpr int NS = 256 / D;
        __shared__ double red[NS][D];
        const int c = threadIdx.x % D, j = threadIdx.x / D;
        double s = 0.0;
        for (int k0 = j; k0 < nblk; k0 += 16 * NS) {
            double v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int k = k0 + i * NS;
                v[i] = k < nblk ? part[(static_cast<int64_t>(bh) * nblk + k) * D + c] : 0.0;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) s += v[i];
        }
        red[j][c] = s;
        __syncthreads();
        if (threadIdx.x < D) {
            double m = 0.0;
#pragma unroll
            for (int i = 0; i < NS; ++i) m += red[i][threadIdx.x];
            mean[threadIdx.x] = m / C;
        }
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        double s = 0.0;
        for (int e = threadIdx.x; e < D; e += kWave) s += mean[e] * mean[e];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
        if (threadIdx.x == 0) mnorm = sqrt(s);
    }
    __syncthreads();
    double m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = mean[c8 * 8 + i];
    const double mn = mnorm;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {           // uniform trip count: shuffles stay converged
        const int r = blk * QR + sub + it * RPP;
        double dot = 0.0, n2 = 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double xd = x[it][i];
            dot += xd * m[i];
            n2 += xd * xd;
        }
#pragma unroll
        for (int o = G8 / 2; o >= 1; o >>= 1) {               // reduce over the row's lanes
            dot += __shfl_xor(dot, o, kWave);
            n2 += __shfl_xor(n2, o, kWave);
        }
        if (c8 == 0 && r < r1) {
            const double nq = sqrt(n2);
            const double den = nq * mn;
            qcos[static_cast<int64_t>(bh) * C + r] = den > 0.0 ? static_cast<float>(dot / den) : 0.0f;
            qrn[static_cast<int64_t>(bh) * C + r] = nq > 0.0 ? static_cast<float>(1.0 / nq) : 0.0f;
        }
    }
}

// ----------------------------------------------------------------------------- exact top-k

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kHistBins = 2048;   // 11-bit digits

// Exclusive scan of one uint32 per thread across the workgroup (ascending thread id).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) {
        const uint32_t s = wsum[w];
        off += (w < wave) ? s : 0u;
        tot += s;
    }
    __syncthreads();
    *total = tot;
    return off + incl - v;
}

constexpr int kLdsKeys = 30720;   // problems up to this size keep their keys in LDS

template <bool kLds>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int64_t score_stride,
                                                            int nsplit, int64_t split_stride, float* __restrict__ s_out,
                                                            int heads_per_seq, const int64_t* __restrict__ prior_len,
                                                            int n_fixed, int64_t budget, int k,
                                                            int32_t* __restrict__ out, int64_t out_stride, int mode) {
    const int p = blockIdx.x;
    const int b = p / heads_per_seq;
    const int64_t T = prior_len[b];
    // mode 1: the problem size does not depend on T, so the keys are requested
    // before T is checked (sequences with T <= budget return after the first pass)
    const int n = mode == 0 ? static_cast<int>(T) : n_fixed;
    const float* x = scores + static_cast<int64_t>(p) * score_stride;
    int32_t* o = out + static_cast<int64_t>(p) * out_stride;
    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;

    if (n <= k) {   // everything is kept
        if (mode == 1 && T <= budget) return;
        for (int j = tid; j < k; j += kTopkThreads) o[j] = j < n ? j : -1;
        return;
    }
    const uint32_t flip = mode ? 0xFFFFFFFFu : 0u;   // mode 1 keeps the smallest
    __shared__ uint32_t kc[kLds ? kLdsKeys : 1];      // the problem's order keys when they fit
    auto gval = [&](int j) -> float {                  // partial scores summed in split order
        float v = x[j];
        for (int sp = 1; sp < nsplit; ++sp) v += x[j + sp * split_stride];
        return v;
    };
    auto gkey = [&](int j) -> uint32_t { return order_key(gval(j)) ^ flip; };
    float* so = s_out ? s_out + static_cast<int64_t>(p) * score_stride : nullptr;
    auto key = [&](int j) -> uint32_t { return kLds ? kc[j] : gkey(j); };

    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t wsum[kTopkWaves];
    __shared__ uint32_t wtot[2][kTopkWaves];
    __shared__ uint32_t s_digit, s_rem, s_full;

    // bits shared by every key need no histogram pass
    const uint32_t first = gkey(0);
    uint32_t diff = 0;
    for (int j0 = tid; j0 < n; j0 += 8 * kTopkThreads) {     // 8 independent loads in flight per thread
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = j0 + i * kTopkThreads;
            v[i] = j < n ? gval(j) : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = j0 + i * kTopkThreads;
            const uint32_t u = j < n ? order_key(v[i]) ^ flip : first;
            if (kLds && j < n) kc[j] = u;
            if (so && j < n) so[j] = v[i];
            diff |= u ^ first;
        }
    }
    if (mode == 1 && T <= budget) return;             // the whole workgroup: before any barrier
#pragma unroll
    for (int o2 = 32; o2 >= 1; o2 >>= 1) diff |= __shfl_xor(diff, o2, kWave);
    if (lane == 0) wsum[wave] = diff;
    __syncthreads();
    diff = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) diff |= wsum[w];
    __syncthreads();

    int bits = diff ? 32 - __clz(diff) : 0;        // low bits still unresolved
    uint32_t prefix = bits == 32 ? 0u : (first >> bits) << bits;
    uint32_t remaining = static_cast<uint32_t>(k);
    while (bits > 0) {
        const int w = bits < 11 ? bits : 11;
        const int shift = bits - w;
        const uint32_t dmask = (1u << w) - 1u;
        for (int i = tid; i < kHistBins; i += kTopkThreads) hist[i] = 0;
        __syncthreads();
        for (int j0 = tid; j0 < n; j0 += 4 * kTopkThreads) {
            uint32_t u[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + i * kTopkThreads;
                u[i] = j < n ? key(j) : 0u;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + i * kTopkThreads;
                const bool match = (bits == 32) || ((u[i] >> bits) == (prefix >> bits));
                if (j < n && match) atomicAdd(&hist[(u[i] >> shift) & dmask], 1u);
            }
        }
        __syncthreads();
        // thread t owns bins [BPT*t, BPT*t + BPT); counts of all higher bins via a reversed scan
        constexpr int BPT = kHistBins / kTopkThreads;
        const int t = kTopkThreads - 1 - tid;               // reversed order
        uint32_t hb[BPT], hsum = 0;
#pragma unroll
        for (int i = 0; i < BPT; ++i) { hb[i] = hist[BPT * t + i]; hsum += hb[i]; }
        uint32_t tot;
        uint32_t above = block_excl_scan(hsum, wsum, &tot);   // keys in bins above BPT*t + BPT - 1
#pragma unroll
        for (int i = BPT - 1; i >= 0; --i) {
            if (above < remaining && above + hb[i] >= remaining) {
                s_digit = BPT * t + i;
                s_rem = remaining - above;
                s_full = remaining - above == hb[i] ? 1u : 0u;   // every key of the bin is kept
            }
            above += hb[i];
        }
        __syncthreads();
        prefix |= s_digit << shift;
        remaining = s_rem;
        bits = shift;
        if (s_full && bits > 0 && prefix > 0) {
            // the kept keys are exactly those >= prefix (the bin's lowest key):
            // no further digits are needed, tau sits just below the bin and
            // no key equal to it is kept
            prefix -= 1;
            remaining = 0;
            bits = 0;
        }
        __syncthreads();
    }
    const uint32_t tau = prefix;          // the k-th largest key (or just below the kept range)
    const uint32_t need = remaining;      // keys equal to tau that are kept (lowest indices)

    // Ordered compaction: wave w owns the contiguous segment [w*seg, (w+1)*seg).
    // Pass 1 counts keys above tau and equal to tau per wave; after one barrier
    // every wave knows how many of each precede its segment, and pass 2 writes
    // each kept index at (#above before it) + min(#equal before it, need).
    const uint64_t lt = (1ull << lane) - 1ull;
    const int seg = ((n + kTopkWaves - 1) / kTopkWaves + kWave - 1) / kWave * kWave;
    const int j0 = wave * seg, j1 = min(n, j0 + seg);
    uint32_t n_gt = 0, n_eq = 0;
    for (int base = j0; base < j1; base += kWave) {
        const int j = base + lane;
        const uint32_t u = j < j1 ? key(j) : 0u;
        n_gt += __popcll(__ballot(j < j1 && u > tau));
        n_eq += __popcll(__ballot(j < j1 && u == tau));
    }
    if (lane == 0) {
        wtot[0][wave] = n_gt;
        wtot[1][wave] = n_eq;
    }
    __syncthreads();
    uint32_t gt_run = 0, eq_run = 0;
    for (int w = 0; w < wave; ++w) {
        gt_run += wtot[0][w];
        eq_run += wtot[1][w];
    }
    for (int base = j0; base < j1 && gt_run + min(eq_run, need) < static_cast<uint32_t>(k); base += kWave) {
        const int j = base + lane;
        const uint32_t u = j < j1 ? key(j) : 0u;
        const bool gt = j < j1 && u > tau;
        const bool eq = j < j1 && u == tau;
        const uint64_t bgt = __ballot(gt), beq = __ballot(eq);
        const uint32_t gt_before = gt_run + __popcll(bgt & lt);
        const uint32_t eq_before = eq_run + __popcll(beq & lt);
        if (gt) o[gt_before + min(eq_before, need)] = j;
        else if (eq && eq_before < need) o[gt_before + eq_before] = j;
        gt_run += __popcll(bgt);
        eq_run += __popcll(beq);
    }
}

// ----------------------------------------------------------------------------- Q_sel packing

template <typename T, int D>
__global__ __launch_bounds__(256) void pack_qsel_kernel(const T* __restrict__ q, int h_q, int G, int C, int nqp,
                                                        int nq_pad, int rblocks, int32_t* __restrict__ keep,
                                                        int64_t keep_stride, const float* __restrict__ qrn,
                                                        const int64_t* __restrict__ prior_len, int64_t budget,
                                                        T* __restrict__ qsel, float* __restrict__ rq, int keep_all,
                                                        uint32_t* __restrict__ zero, int64_t zero_n) {
    constexpr int kPieces = D * sizeof(T) / 16;          // 16-byte pieces per row
    constexpr int kRows = 32;                            // rows per workgroup
    constexpr int PPT = kRows * kPieces / 256;           // pieces per thread
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < zero_n; i += int64_t(gridDim.x) * 256) zero[i] = 0;
    const int bh = blockIdx.x / rblocks, rb = blockIdx.x % rblocks;
    const int b = bh / h_q, h = bh % h_q;
    const int g = h / G, hh = h % G;
    const int h_kv = h_q / G;
    const int64_t dst_row0 = (static_cast<int64_t>(b) * h_kv + g) * G * nq_pad + static_cast<int64_t>(hh) * nq_pad;
    int32_t* kp = keep + static_cast<int64_t>(bh) * keep_stride;
    // kept token of row r (rows past nqp repeat row 0); with every query kept
    // (nqp == C) the list is the identity and the statistics were not run.
    // The list entries are read before the prior length (the list is written
    // only for selecting sequences, so the rows themselves are read after).
    auto kept = [&](int r) { return keep_all ? (r < nqp ? r : 0) : kp[r < nqp ? r : 0]; };
    int rr[PPT], tk[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = threadIdx.x + 256 * i;
        rr[i] = rb * kRows + p / kPieces;
        tk[i] = rr[i] < nq_pad ? kept(rr[i]) : 0;
    }
    if (prior_len[b] <= budget) return;
    u32x4 v[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = threadIdx.x + 256 * i;
        const int r = rr[i], pc = p % kPieces;
        if (r < nq_pad) v[i] = reinterpret_cast<const u32x4*>(q + (static_cast<int64_t>(bh) * C + tk[i]) * D)[pc];
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = threadIdx.x + 256 * i;
        const int r = rr[i], pc = p % kPieces;
        if (r < nq_pad) reinterpret_cast<u32x4*>(qsel + (dst_row0 + r) * D)[pc] = v[i];
    }
    if (keep_all) {
        // 1/|q| of each row from its pieces: squares summed in fp64 (exact for
        // bf16 and fp32 inputs at these sizes), reduced over the row's lanes
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + 256 * i;
            const int r = rr[i], pc = p % kPieces;
            double n2 = 0.0;
            if (r < nq_pad) {
                float x[16 / sizeof(T)];
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[2 * e] = __uint_as_float(v[i][e] << 16);
                        x[2 * e + 1] = __uint_as_float(v[i][e] & 0xFFFF0000u);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(v[i][e]);
                }
#pragma unroll
                for (int e = 0; e < 16 / static_cast<int>(sizeof(T)); ++e) n2 += static_cast<double>(x[e]) * x[e];
            }
#pragma unroll
            for (int o = kPieces / 2; o >= 1; o >>= 1) n2 += __shfl_xor(n2, o, kWave);
            if (pc == 0 && r < nq_pad) {
                const double nq = sqrt(n2);
                rq[dst_row0 + r] = nq > 0.0 ? static_cast<float>(1.0 / nq) : 0.0f;
                if (keep && r < nqp) kp[r] = r;
            }
        }
    } else if (threadIdx.x < kRows) {
        const int r = rb * kRows + threadIdx.x;
        if (r < nq_pad) rq[dst_row0 + r] = qrn[static_cast<int64_t>(bh) * C + kept(r)];
    }
}

// ----------------------------------------------------------------------------- launchers

hipError_t launch_qstats(const SelShape& s, const void* q, const int64_t* prior_len, double* part, float* qcos,
                         float* qrn, uint32_t* zero, int64_t zero_n, hipStream_t st) {
    const int qr = int64_t(s.batch) * s.h_q * ((s.C + 127) / 128) < 1024 ? kQRowsMin : 128;
    const int nblk = (s.C + qr - 1) / qr;
    dim3 grid(s.batch * s.h_q * nblk), block(256);
#define KVSEL_QSTATS(T, D, QR)                                                                                     \
    do {                                                                                                           \
        hipLaunchKernelGGL((qsum_kernel<T, D, QR>), grid, block, 0, st, (const T*)q, s.h_q, s.C, nblk, prior_len,  \
                           s.budget, part, zero, zero_n);                                                          \
        hipLaunchKernelGGL((qcos_kernel<T, D, QR>), grid, block, 0, st, (const T*)q, s.h_q, s.C, nblk, prior_len,  \
                           s.budget, part, qcos, qrn);                                                             \
    } while (0)
#define KVSEL_QSTATS_R(T, D)                                                                                       \
    do {                                                                                                           \
        if (qr == kQRowsMin) KVSEL_QSTATS(T, D, kQRowsMin);                                                        \
        else KVSEL_QSTATS(T, D, 128);                                                                              \
    } while (0)
    if (s.esz == 2) {
        if (s.d == 128) KVSEL_QSTATS_R(uint16_t, 128);
        else KVSEL_QSTATS_R(uint16_t, 64);
    } else {
        if (s.d == 128) KVSEL_QSTATS_R(float, 128);
        else KVSEL_QSTATS_R(float, 64);
    }
#undef KVSEL_QSTATS_R
#undef KVSEL_QSTATS
    return hipGetLastError();
}

hipError_t launch_topk(int problems, int heads_per_seq, const float* scores, int64_t score_stride,
                       int nsplit, int64_t split_stride, float* s_out,
                       const int64_t* prior_len, int n_fixed, int64_t budget, int k, int32_t* out,
                       int64_t out_stride, int mode, int64_t max_n, hipStream_t st) {
    if (max_n <= kLdsKeys)
        hipLaunchKernelGGL(topk_kernel<true>, dim3(problems), dim3(kTopkThreads), 0, st, scores, score_stride, nsplit,
                           split_stride, s_out, heads_per_seq, prior_len, n_fixed, budget, k, out, out_stride, mode);
    else
        hipLaunchKernelGGL(topk_kernel<false>, dim3(problems), dim3(kTopkThreads), 0, st, scores, score_stride, nsplit,
                           split_stride, s_out, heads_per_seq, prior_len, n_fixed, budget, k, out, out_stride, mode);
    return hipGetLastError();
}

hipError_t launch_pack_qsel(const SelShape& s, const void* q, int32_t* keep, int64_t keep_stride,
                            const float* qrn, const int64_t* prior_len, void* qsel, float* rq, hipStream_t st,
                            bool keep_all, uint32_t* zero, int64_t zero_n) {
    const int rblocks = (s.nq_pad + 31) / 32;
    dim3 grid(s.batch * s.h_q * rblocks), block(256);
    const int ka = keep_all ? 1 : 0;
    if (!keep_all) zero_n = 0;
#define KVSEL_PACKQ(T, D) hipLaunchKernelGGL((pack_qsel_kernel<T, D>), grid, block, 0, st, (const T*)q, s.h_q, s.G, s.C, s.nqp, s.nq_pad, rblocks, keep, keep_stride, qrn, prior_len, s.budget, (T*)qsel, rq, ka, zero, zero_n)
    if (s.esz == 2) {
        if (s.d == 128) KVSEL_PACKQ(uint16_t, 128);
        else KVSEL_PACKQ(uint16_t, 64);
    } else {
        if (s.d == 128) KVSEL_PACKQ(float, 128);
        else KVSEL_PACKQ(float, 64);
    }
#undef KVSEL_PACKQ
    return hipGetLastError();
}

}  // namespace kvsel
