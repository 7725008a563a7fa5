// Cross-step reuse of the selected entries in decode.
//
// SQD page (rit.work, the paragraph on sparse attention): the top-k selection
// scans the whole cache every step, the values of the selected positions are
// kept from one step to the next, and only the misses are fetched.  Here the
// kept entries live in a caller-owned slot buffer per (sequence, KV head);
// after the step's top-B, one workgroup per (sequence, KV head) decides which
// slots keep their entry and fetches the misses' rows from the KV cache:
//   * a slot s < n = min(B, T_b) whose position is selected again keeps it (hit);
//   * the selected positions held by no hit slot (misses), in ascending order,
//     fill the other slots below n in ascending order; slots >= n end empty (-1).
// The attention then reads slots [0, n) of the buffer (its order does not
// matter to the softmax).
#include "launch.h"

namespace kvsel {

namespace {

constexpr int kReuseThreads = 256;
constexpr int kPer = kReuseMaxBudget / kReuseThreads;    // list entries per thread in the scans

// Exclusive scan of one value per thread over the 256 threads (ascending thread id);
// *total receives the sum.
__device__ __forceinline__ uint32_t excl_scan_256(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += t;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kReuseThreads / kWave; ++w) {
        off += w < wave ? wsum[w] : 0u;
        tot += wsum[w];
    }
    __syncthreads();
    *total = tot;
    return off + incl - v;
}

// Index of p in the ascending list a[0, n), or -1.
__device__ __forceinline__ int find_sorted(const int32_t* a, int n, int32_t p) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < p) lo = mid + 1;
        else hi = mid;
    }
    return (lo < n && a[lo] == p) ? lo : -1;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kReuseThreads) void reuse_kernel(CacheView cv, const int64_t* __restrict__ prior_len,
                                                              int budget, const int32_t* __restrict__ idx,
                                                              int h_kv, char* __restrict__ sk, char* __restrict__ sv,
                                                              int32_t* __restrict__ pos, int32_t* __restrict__ counts) {
    __shared__ int32_t sidx[kReuseMaxBudget];     // this step's kept positions (ascending); later the misses
    __shared__ int32_t spos[kReuseMaxBudget];     // slot contents: previous, then new
    __shared__ uint8_t held[kReuseMaxBudget];     // kept position i is held by a hit slot
    __shared__ uint8_t hitf[kReuseMaxBudget];     // slot s is a hit
    __shared__ int32_t fslot[kReuseMaxBudget];    // the r-th free slot below n
    __shared__ uint32_t wsum[kReuseThreads / kWave];
    const int bg = blockIdx.x, b = bg / h_kv, g = bg % h_kv;
    const int tid = threadIdx.x;
    const int64_t T = prior_len[b];
    const int n = static_cast<int>(T < budget ? T : budget);
    const int32_t* ib = idx + static_cast<int64_t>(bg) * budget;
    int32_t* pb = pos + static_cast<int64_t>(bg) * budget;
    for (int i = tid; i < budget; i += kReuseThreads) {
        sidx[i] = i < n ? ib[i] : 0;
        spos[i] = pb[i];
        held[i] = 0;
    }
    __syncthreads();
    // hits: slots below n whose position is selected again
    for (int s = tid; s < budget; s += kReuseThreads) {
        const int32_t p = spos[s];
        const int at = (s < n && p >= 0) ? find_sorted(sidx, n, p) : -1;
        hitf[s] = at >= 0 ? 1 : 0;
        if (at >= 0) held[at] = 1;
    }
    __syncthreads();
    // ranks: the r-th miss (ascending position) goes to the r-th free slot below n
    const int e0 = tid * kPer;
    uint32_t nm = 0, nf = 0;
    for (int e = e0; e < e0 + kPer && e < n; ++e) {
        nm += held[e] ? 0u : 1u;
        nf += hitf[e] ? 0u : 1u;
    }
    uint32_t tot_m, tot_f;
    uint32_t rm = excl_scan_256(nm, wsum, &tot_m);
    uint32_t rf = excl_scan_256(nf, wsum, &tot_f);
    // the misses' positions are moved to the front of sidx below, so read them first
    int32_t mine[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) mine[k] = (e0 + k < n) ? sidx[e0 + k] : 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {              // unrolled: mine[] stays in registers
        const int e = e0 + k;
        if (e < n) {
            if (!held[e]) sidx[rm++] = mine[k];
            if (!hitf[e]) fslot[rf++] = e;
        }
    }
    __syncthreads();
    // both counts are n minus the hits for a slot state this kernel produced
    // (distinct positions); min() keeps any other state inside the lists
    const int misses = static_cast<int>(tot_m < tot_f ? tot_m : tot_f);
    for (int r = tid; r < misses; r += kReuseThreads) spos[fslot[r]] = sidx[r];
    for (int s = n + tid; s < budget; s += kReuseThreads) spos[s] = -1;
    __syncthreads();
    for (int s = tid; s < budget; s += kReuseThreads) pb[s] = spos[s];
    if (counts && tid == 0) {
        counts[2 * bg] = n - misses;
        counts[2 * bg + 1] = misses;
    }
    // fetch the misses' key and value rows into their slots (16-byte pieces)
    constexpr int PPR = D * 2 / 16;
    const int64_t slot0 = static_cast<int64_t>(bg) * budget;
    for (int it = tid; it < misses * PPR; it += kReuseThreads) {
        const int r = it / PPR, c = it % PPR;
        const int64_t src = cv.row_offset(b, g, sidx[r]);
        const int64_t dst = (slot0 + fslot[r]) * (D * 2);
        reinterpret_cast<u32x4*>(sk + dst)[c] = reinterpret_cast<const u32x4*>(cv.k + src)[c];
        reinterpret_cast<u32x4*>(sv + dst)[c] = reinterpret_cast<const u32x4*>(cv.v + src)[c];
    }
}

hipError_t launch_reuse(const SelShape& s, const CacheView& cv, const int64_t* prior_len, const int32_t* idx,
                        void* sel_k, void* sel_v, int32_t* pos, int32_t* counts, hipStream_t st) {
    const dim3 grid(s.batch * s.h_kv), block(kReuseThreads);
    const int budget = static_cast<int>(s.budget);
    if (s.d == 128)
        hipLaunchKernelGGL(reuse_kernel<128>, grid, block, 0, st, cv, prior_len, budget, idx, s.h_kv,
                           static_cast<char*>(sel_k), static_cast<char*>(sel_v), pos, counts);
    else
        hipLaunchKernelGGL(reuse_kernel<64>, grid, block, 0, st, cv, prior_len, budget, idx, s.h_kv,
                           static_cast<char*>(sel_k), static_cast<char*>(sel_v), pos, counts);
    return hipGetLastError();
}

}  // namespace kvsel
