// Group-pooled query rows for the group-first scoring order.
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Table 4 caption: the
// method's cost is stated with the number of KV heads in place of the number
// of query heads.  Read as pooling the G query heads of a KV head before the
// scan: qbar[b][g][i] = (1/G) * sum_h q[b][gG+h][i] / |q[b][gG+h][i]| (a zero
// row contributes 0).  Query sub-selection then runs on qbar as if it were one
// head per KV head, and the scan scores max_i qbar_i . k_j / |k_j|.
//
// qbar is kept in fp32.  The bf16 MFMA scan takes each kept row as the pair
// (hi, lo) = (bf16(x), bf16(x - bf16(x))): |x - hi - lo| <= 2^-18 |x| per
// element, so with |qbar| <= 1 the score error is at most 2^-18 (Cauchy-
// Schwarz) plus fp32 accumulation.
#include "launch.h"

namespace kvsel {

// A wave covers TPW consecutive tokens of one (b, g): every head's rows of
// those tokens are contiguous, so each lane loads 16 bytes (LPR lanes per
// row), the sum of squares is reduced within the row's lanes, and the unit
// rows are added in head order.  Four heads are loaded before any is used.
template <typename E, int D>
__global__ __launch_bounds__(256) void qpool_kernel(const E* __restrict__ q, int h_kv, int G, int C, int tblocks,
                                                    const int64_t* __restrict__ prior_len, int64_t budget,
                                                    float* __restrict__ qbar) {
    constexpr int EPL = 16 / static_cast<int>(sizeof(E));   // elements per lane
    constexpr int LPR = D / EPL;                            // lanes per row
    constexpr int TPW = kWave / LPR;                        // tokens per wave
    const int bg = blockIdx.x / tblocks, tb = blockIdx.x % tblocks;
    const int b = bg / h_kv, g = bg % h_kv;
    if (prior_len[b] <= budget) return;
    const int lane = lane_id();
    const int i = (tb * 4 + static_cast<int>(threadIdx.x) / kWave) * TPW + lane / LPR;
    const int e0 = (lane % LPR) * EPL;
    const bool valid = i < C;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.0f;
    const int64_t head0 = (static_cast<int64_t>(b) * h_kv + g) * G;
    for (int h0 = 0; h0 < G; h0 += 4) {
        u32x4 raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int hh = h0 + u;
            raw[u] = (valid && hh < G) ? *reinterpret_cast<const u32x4*>(q + ((head0 + hh) * C + i) * D + e0)
                                       : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            float x[EPL];
            if constexpr (sizeof(E) == 2) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    x[2 * w] = __uint_as_float(raw[u][w] << 16);
                    x[2 * w + 1] = __uint_as_float(raw[u][w] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int w = 0; w < 4; ++w) x[w] = __uint_as_float(raw[u][w]);
            }
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) ss = fmaf(x[e], x[e], ss);
#pragma unroll
            for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, kWave);
            const float inv = ss > 0.0f ? 1.0f / sqrtf(ss) : 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] = fmaf(x[e], inv, acc[e]);
        }
    }
    if (!valid) return;
    float* dst = qbar + (static_cast<int64_t>(bg) * C + i) * D + e0;
    const float gf = static_cast<float>(G);
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{acc[e] / gf, acc[e + 1] / gf, acc[e + 2] / gf, acc[e + 3] / gf};
}

// Q_sel rows of the pooled scan: row r of (b, g) is qbar[b][g][keep[r]] (rows
// r >= nqp repeat the first kept row, which leaves every max unchanged), as
// [hi | lo] bf16 (2*D elements, SPLIT) or fp32 (D elements); rq = 1 (the
// pooled row is not normalised: its dot product is already a mean of cosines
// once divided by |k|).
template <int D, bool SPLIT>
__global__ __launch_bounds__(256) void pack_pooled_kernel(const float* __restrict__ qbar, int h_kv, int C, int nqp,
                                                          int nq_pad, int rblocks, const int32_t* __restrict__ keep,
                                                          int64_t keep_stride, const int64_t* __restrict__ prior_len,
                                                          int64_t budget, void* __restrict__ qsel,
                                                          float* __restrict__ rq) {
    constexpr int TPR = D / 4;              // threads per row (4 elements each)
    constexpr int PASSES = 32 * TPR / 256;  // 32 rows per workgroup
    const int bg = blockIdx.x / rblocks, rb = blockIdx.x % rblocks;
    const int b = bg / h_kv;
    if (prior_len[b] <= budget) return;
    const int32_t* kp = keep + static_cast<int64_t>(bg) * keep_stride;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
        const int p = static_cast<int>(threadIdx.x) + 256 * pass;
        const int r = rb * 32 + p / TPR, c = (p % TPR) * 4;
        if (r >= nq_pad) continue;
        const int t = kp[r < nqp ? r : 0];
        const f32x4 x = *reinterpret_cast<const f32x4*>(qbar + (static_cast<int64_t>(bg) * C + t) * D + c);
        const int64_t row = static_cast<int64_t>(bg) * nq_pad + r;
        if (SPLIT) {
            uint16_t* dst = static_cast<uint16_t*>(qsel) + row * 2 * D;
            const uint32_t h01 = pack_bf16x2(x[0], x[1]), h23 = pack_bf16x2(x[2], x[3]);
            const float r0 = x[0] - bf16_to_f32(static_cast<uint16_t>(h01 & 0xFFFFu));
            const float r1 = x[1] - bf16_to_f32(static_cast<uint16_t>(h01 >> 16));
            const float r2 = x[2] - bf16_to_f32(static_cast<uint16_t>(h23 & 0xFFFFu));
            const float r3 = x[3] - bf16_to_f32(static_cast<uint16_t>(h23 >> 16));
            uint32_t* hi = reinterpret_cast<uint32_t*>(dst + c);
            uint32_t* lo = reinterpret_cast<uint32_t*>(dst + D + c);
            hi[0] = h01;
            hi[1] = h23;
            lo[0] = pack_bf16x2(r0, r1);
            lo[1] = pack_bf16x2(r2, r3);
        } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(qsel) + row * D + c) = x;
        }
    }
    if (threadIdx.x < 32) {
        const int r = rb * 32 + static_cast<int>(threadIdx.x);
        if (r < nq_pad) rq[static_cast<int64_t>(bg) * nq_pad + r] = 1.0f;
    }
}

hipError_t launch_qpool(const SelShape& s, const void* q, const int64_t* prior_len, float* qbar, hipStream_t st) {
    const int tpw = kWave / (s.d / (16 / s.esz));        // tokens per wave (as in qpool_kernel)
    const int tblocks = (s.C + 4 * tpw - 1) / (4 * tpw);
    dim3 grid(s.batch * s.h_kv * tblocks), block(256);
    if (s.esz == 2) {
        if (s.d == 128) hipLaunchKernelGGL((qpool_kernel<uint16_t, 128>), grid, block, 0, st, (const uint16_t*)q, s.h_kv, s.G, s.C, tblocks, prior_len, s.budget, qbar);
        else hipLaunchKernelGGL((qpool_kernel<uint16_t, 64>), grid, block, 0, st, (const uint16_t*)q, s.h_kv, s.G, s.C, tblocks, prior_len, s.budget, qbar);
    } else {
        if (s.d == 128) hipLaunchKernelGGL((qpool_kernel<float, 128>), grid, block, 0, st, (const float*)q, s.h_kv, s.G, s.C, tblocks, prior_len, s.budget, qbar);
        else hipLaunchKernelGGL((qpool_kernel<float, 64>), grid, block, 0, st, (const float*)q, s.h_kv, s.G, s.C, tblocks, prior_len, s.budget, qbar);
    }
    return hipGetLastError();
}

hipError_t launch_pack_pooled(const SelShape& sp, const float* qbar, const int32_t* keep, int64_t keep_stride,
                              const int64_t* prior_len, void* qsel, float* rq, hipStream_t st) {
    const int rblocks = (sp.nq_pad + 31) / 32;
    dim3 grid(sp.batch * sp.h_kv * rblocks), block(256);
    if (sp.qsplit) {
        if (sp.d == 128) hipLaunchKernelGGL((pack_pooled_kernel<128, true>), grid, block, 0, st, qbar, sp.h_kv, sp.C, sp.nqp, sp.nq_pad, rblocks, keep, keep_stride, prior_len, sp.budget, qsel, rq);
        else hipLaunchKernelGGL((pack_pooled_kernel<64, true>), grid, block, 0, st, qbar, sp.h_kv, sp.C, sp.nqp, sp.nq_pad, rblocks, keep, keep_stride, prior_len, sp.budget, qsel, rq);
    } else {
        if (sp.d == 128) hipLaunchKernelGGL((pack_pooled_kernel<128, false>), grid, block, 0, st, qbar, sp.h_kv, sp.C, sp.nqp, sp.nq_pad, rblocks, keep, keep_stride, prior_len, sp.budget, qsel, rq);
        else hipLaunchKernelGGL((pack_pooled_kernel<64, false>), grid, block, 0, st, qbar, sp.h_kv, sp.C, sp.nqp, sp.nq_pad, rblocks, keep, keep_stride, prior_len, sp.budget, qsel, rq);
    }
    return hipGetLastError();
}

}  // namespace kvsel
