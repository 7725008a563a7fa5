// Key-scoring scan over the whole prior cache.
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(b) and the method
// paragraph: each cache key is scored by its cosine similarity with the kept
// queries, max-pooled over the queries of a head and mean-pooled over the
// query heads that share the KV head (GQA):
//   S[g][j] = (1/G) * sum_h max_i (q_{h,i} . k_j) / (|q_{h,i}| |k_j|)
// The raw bf16 products are accumulated in fp32 by MFMA and scaled by the
// fp32 reciprocal norms afterwards (normalised vectors are never rounded to
// bf16); 1/|k_j| is common to every query so it is applied after the max.
#include "launch.h"

namespace kvsel {

constexpr int kRows16Groups = 4;   // 16-key groups per wave of the one-query scan

// ----------------------------------------------------------------------------- prefill scan (MFMA 32x32x16)
//
// Workgroup = 4 waves x NB blocks of 32 keys.  Each wave keeps its keys'
// bf16 fragments in registers for the whole kernel (the B operand, loaded from
// HBM exactly once) and streams the packed kept queries Q_sel (the A operand,
// G * nq_pad rows, L2-resident) through a double-buffered LDS stage.  The
// MFMA result tile has queries on rows and keys on columns, so each lane holds
// 16 query rows of one key: the max over queries is in-register plus one
// exchange between the two half-waves at the end of every head.
//
// With QK = 2 every Q_sel row is a pair [hi | lo] of bf16 rows whose sum is an
// fp32 row (the group-pooled rows); both halves multiply the same key
// fragments and accumulate into one fp32 product.
//
// The G query heads may be split over `nsplit` workgroups per key tile (more
// workgroups when the cache or the KV head count is small); split s writes
// the sum over its heads, scaled by 1/G, to S + s * split_stride and the top-B
// kernel adds the splits in order.
constexpr double kScanW4 = 0.78;   // time per key of four 32-key blocks per wave, relative to two
constexpr int kScanOcc = 2;        // workgroups per CU the register budget is sized for
template <int D, int NB, int QK>
__global__ __launch_bounds__(256, kScanOcc) void scan_mfma_kernel(const uint16_t* __restrict__ qsel,
                                                           const float* __restrict__ rq, CacheView cv,
                                                           const int64_t* __restrict__ prior_len, int64_t budget,
                                                           int h_kv, int G, int nq_pad, int tiles, int nsplit,
                                                           float* __restrict__ S, int64_t s_stride,
                                                           int64_t split_stride) {
    constexpr int KS = D / 16;              // MFMA k-steps over the head dim
    constexpr int KQ = D * QK;              // elements per Q_sel row ([hi | lo] pairs when QK = 2)
    constexpr int KSQ = KQ / 16;            // k-steps per query row; key fragment ks % KS
    constexpr int KEYS = 4 * NB * 32;       // keys per workgroup
    constexpr int STAGE = 64;               // query rows per LDS stage
    constexpr int LDQ = KQ + 8;             // padded LDS row (bf16 elements)
    constexpr int PIECES = STAGE * KQ / 8;  // 16-byte pieces per stage
    constexpr int PPT = PIECES / 256;       // pieces per thread
    __shared__ __attribute__((aligned(16))) uint16_t qs[2][STAGE * LDQ];
    __shared__ __attribute__((aligned(16))) float rqs[2][STAGE];

    const int slot = xcd_slot(blockIdx.x, gridDim.x);
    const int tile = slot % tiles;
    const int split = (slot / tiles) % nsplit;
    const int bg = slot / tiles / nsplit;
    const int b = bg / h_kv, g = bg % h_kv;
    const int64_t T = prior_len[b];
    if (T <= budget) return;
    const int64_t key0 = static_cast<int64_t>(tile) * KEYS;
    if (key0 >= T) return;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int half = lane >> 5, col = lane & 31;

    const int R = G / nsplit * nq_pad;                  // this split's query rows
    const int nstage = (R + STAGE - 1) / STAGE;
    const uint16_t* qb = qsel + (static_cast<int64_t>(bg) * G * nq_pad + static_cast<int64_t>(split) * R) * KQ;
    const float* rqb = rq + static_cast<int64_t>(bg) * G * nq_pad + static_cast<int64_t>(split) * R;

    u32x4 pre[PPT];
    float prq = 0.0f;
    auto fetch = [&](int s) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            const int r = p / (KQ / 8), c8 = p % (KQ / 8);
            // rows past R (R is a multiple of 32) are never multiplied: their
            // loads read row R-1, so every load is unconditional
            const int row = min(s * STAGE + r, R - 1);
            pre[i] = *reinterpret_cast<const u32x4*>(qb + static_cast<int64_t>(row) * KQ + c8 * 8);
        }
        if (tid < STAGE) prq = rqb[min(s * STAGE + tid, R - 1)];
    };
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = tid + 256 * i;
            const int r = p / (KQ / 8), c8 = p % (KQ / 8);
            *reinterpret_cast<u32x4*>(&qs[buf][r * LDQ + c8 * 8]) = pre[i];
        }
        if (tid < STAGE) rqs[buf][tid] = prq;
    };

    float run[NB], sum[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) { run[kb] = -INFINITY; sum[kb] = 0.0f; }

    // the first query stage is requested before the keys: staging it waits
    // for those loads only, and the first MFMAs for the first key block only
    fetch(0);
    // ---- this wave's keys: fragments (their reciprocal norms are taken after
    // the stage loop, so the first stages do not wait for every key row)
    // Keys past T read key T-1 (their scores are never written), so every
    // load is unconditional and the compiler's waits count them exactly.
    // (Row offsets first: in a paged cache each one waits for a block-table
    // entry, and no key load then waits behind another block's.)
    bf16x8 kf[NB][KS];
    int64_t koff[NB];
    if (cv.block_size == 0) {
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) koff[kb] = cv.row_offset(b, g, min(key0 + (wave * NB + kb) * 32 + col, T - 1));
    } else {
        const uint32_t bs = static_cast<uint32_t>(cv.block_size);
        int32_t blk[NB];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const uint32_t p = static_cast<uint32_t>(min(key0 + (wave * NB + kb) * 32 + col, T - 1));
            blk[kb] = cv.block_table[static_cast<int64_t>(b) * cv.max_blocks + p / bs];
        }
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) {
            const uint32_t p = static_cast<uint32_t>(min(key0 + (wave * NB + kb) * 32 + col, T - 1));
            koff[kb] = ((static_cast<int64_t>(blk[kb]) * cv.h_kv + g) * cv.block_size + p % bs) * static_cast<int64_t>(cv.row_bytes);
        }
    }
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kf[kb][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(cv.k + koff[kb] + (16 * ks + 8 * half) * 2));

    stash(0);
    __syncthreads();
    for (int s = 0; s < nstage; ++s) {
        const int buf = s & 1;
        if (s + 1 < nstage) fetch(s + 1);
#pragma unroll
        for (int rb = 0; rb < STAGE / 32; ++rb) {
            const int row0 = s * STAGE + rb * 32;
            if (row0 < R) {
                bf16x8 a[KSQ];
#pragma unroll
                for (int ks = 0; ks < KSQ; ++ks)
                    a[ks] = *reinterpret_cast<const bf16x8*>(&qs[buf][(rb * 32 + col) * LDQ + 16 * ks + 8 * half]);
                float rv[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(&rqs[buf][rb * 32 + 8 * q4 + 4 * half]);
                    rv[4 * q4 + 0] = v[0]; rv[4 * q4 + 1] = v[1]; rv[4 * q4 + 2] = v[2]; rv[4 * q4 + 3] = v[3];
                }
#pragma unroll
                for (int kb = 0; kb < NB; ++kb) {
                    f32x16 acc = {};
#pragma unroll
                    for (int ks = 0; ks < KSQ; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], kf[kb][ks % KS], acc, 0, 0, 0);
                    float m = run[kb];
#pragma unroll
                    for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[r] * rv[r]);
                    run[kb] = m;
                }
                if ((row0 + 32) % nq_pad == 0) {      // last 32-row block of a head
#pragma unroll
                    for (int kb = 0; kb < NB; ++kb) {
                        const float m = fmaxf(run[kb], __shfl_xor(run[kb], 32, kWave));
                        sum[kb] += m;
                        run[kb] = -INFINITY;
                    }
                }
            }
        }
        if (s + 1 < nstage) stash(buf ^ 1);
        __syncthreads();
    }

    float rk[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
        float n2 = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 raw = __builtin_bit_cast(u32x4, kf[kb][ks]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(raw[i] << 16), hi = __uint_as_float(raw[i] & 0xFFFF0000u);
                n2 = fmaf(lo, lo, n2);
                n2 = fmaf(hi, hi, n2);
            }
        }
        n2 += __shfl_xor(n2, 32, kWave);
        rk[kb] = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    }
    const float inv_g = 1.0f / static_cast<float>(G);
    float* Sb = S + static_cast<int64_t>(split) * split_stride + static_cast<int64_t>(bg) * s_stride;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
        const int64_t key = key0 + (wave * NB + kb) * 32 + col;
        if (half == 0 && key < T) Sb[key] = sum[kb] * inv_g * rk[kb];
    }
}

// ----------------------------------------------------------------------------- one kept query per head (MFMA 16x16x32)
//
// With a single query per head (decode, or N_q = 1) the G <= 16 query heads of
// a KV head form the 16 rows of one MFMA tile; keys stream through registers
// straight from HBM (this scan is bandwidth-bound: 4 useful rows per key).
template <int D, int GROUPS>
__global__ __launch_bounds__(256) void scan_rows16_kernel(const uint16_t* __restrict__ qsel,
                                                         const float* __restrict__ rq, CacheView cv,
                                                         const int64_t* __restrict__ prior_len, int64_t budget,
                                                         int h_kv, int G, int tiles, float* __restrict__ S,
                                                         int64_t s_stride, TileMap map) {
    constexpr int KS = D / 32;          // k-steps of 32
    constexpr int KEYS = 4 * GROUPS * 16;
    // slots follow the launch order, so every XCD receives an even share of
    // the key tiles whatever the sequence lengths (grouping a sequence's tiles
    // on one XCD, as the prefill scan does for L2 reuse, buys nothing here:
    // every key is read once)
    int b, g, tile;
    int64_t T;
    if (map.n > 0) {                    // only workgroups with keys were launched
        tile_map_slot(map, h_kv, b, g, tile);
        T = map.len[b];
    } else {
        const int bg0 = blockIdx.x / tiles;
        tile = blockIdx.x % tiles;
        b = bg0 / h_kv;
        g = bg0 % h_kv;
        T = prior_len[b];
        if (T <= budget) return;
        if (static_cast<int64_t>(tile) * KEYS >= T) return;
    }
    const int bg = b * h_kv + g;
    const int64_t key0 = static_cast<int64_t>(tile) * KEYS;
    const int lane = lane_id(), wave = threadIdx.x / kWave;
    const int quad = lane >> 4, col = lane & 15;

    // A: query rows (row m = query head m of the group, zero past G)
    bf16x8 a[KS];
    {
        const bool valid = col < G;
        const uint16_t* qrow = qsel + (static_cast<int64_t>(bg) * G + (valid ? col : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 raw = {0u, 0u, 0u, 0u};
            if (valid) raw = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * quad);
            a[ks] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    float rv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * quad + r;
        rv[r] = row < G ? rq[static_cast<int64_t>(bg) * G + row] : 0.0f;
    }

    u32x4 raw[GROUPS][KS];
#pragma unroll
    for (int gr = 0; gr < GROUPS; ++gr) {
        const int64_t key = key0 + wave * GROUPS * 16 + gr * 16 + col;
        const bool valid = key < T;
        const char* row = cv.k + (valid ? cv.row_offset(b, g, key) : 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            raw[gr][ks] = valid ? *reinterpret_cast<const u32x4*>(row + (32 * ks + 8 * quad) * 2) : u32x4{0u, 0u, 0u, 0u};
    }
    const float inv_g = 1.0f / static_cast<float>(G);
    float* Sb = S + static_cast<int64_t>(bg) * s_stride;
#pragma unroll
    for (int gr = 0; gr < GROUPS; ++gr) {
        f32x4 acc = {};
        float n2 = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], __builtin_bit_cast(bf16x8, raw[gr][ks]), acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = __uint_as_float(raw[gr][ks][i] << 16), hi = __uint_as_float(raw[gr][ks][i] & 0xFFFF0000u);
                n2 = fmaf(lo, lo, n2);
                n2 = fmaf(hi, hi, n2);
            }
        }
        float v = acc[0] * rv[0] + acc[1] * rv[1] + acc[2] * rv[2] + acc[3] * rv[3];
        v += __shfl_xor(v, 16, kWave);
        v += __shfl_xor(v, 32, kWave);
        n2 += __shfl_xor(n2, 16, kWave);
        n2 += __shfl_xor(n2, 32, kWave);
        const float rkv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
        const int64_t key = key0 + wave * GROUPS * 16 + gr * 16 + col;
        if (quad == 0 && key < T) Sb[key] = v * inv_g * rkv;
    }
}

// ----------------------------------------------------------------------------- VALU scan (fp32 inputs)
//
// 16 lanes per key, each holding D/16 consecutive elements of the key row; a
// workgroup scores 16 keys.  The kept query rows of the KV head pass through
// LDS in stages of 32; each lane forms its part of q . k and the 16 lanes of
// the key add their parts with DPP (every lane gets the dot product), so the
// max over a head's queries and the mean over the heads run in every lane.
template <int D>
__global__ __launch_bounds__(256) void scan_valu_kernel(const float* __restrict__ qsel, const float* __restrict__ rq,
                                                        CacheView cv, const int64_t* __restrict__ prior_len,
                                                        int64_t budget, int h_kv, int G, int nqp, int tiles,
                                                        float* __restrict__ S, int64_t s_stride) {
    constexpr int DPL = D / 16;             // elements per lane
    constexpr int KPW = 16;                 // keys per workgroup
    constexpr int QR = 32;                  // query rows per LDS stage
    __shared__ __attribute__((aligned(16))) float qs[QR][D];
    __shared__ float rqs[QR];
    const int bg = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bg / h_kv, g = bg % h_kv;
    const int64_t T = prior_len[b];
    if (T <= budget) return;
    const int64_t key0 = static_cast<int64_t>(tile) * KPW;
    if (key0 >= T) return;
    const int c = threadIdx.x & 15;
    const int64_t key = key0 + (threadIdx.x >> 4);
    const bool valid = key < T;             // lanes past T score row 0 and write nothing
    float k[DPL];
    {
        const float* row = reinterpret_cast<const float*>(cv.k + (valid ? cv.row_offset(b, g, key) : cv.row_offset(b, g, 0)));
#pragma unroll
        for (int e = 0; e < DPL; e += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(row + c * DPL + e);
            k[e] = x[0]; k[e + 1] = x[1]; k[e + 2] = x[2]; k[e + 3] = x[3];
        }
    }
    float n2 = 0.0f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) n2 = fmaf(k[e], k[e], n2);
    n2 = row16_sum(n2);
    const float rkv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    const float* qb = qsel + static_cast<int64_t>(bg) * G * nqp * D;
    const float* rqb = rq + static_cast<int64_t>(bg) * G * nqp;
    float sum = 0.0f;
    for (int hh = 0; hh < G; ++hh) {
        float run = -INFINITY;
        for (int r0 = 0; r0 < nqp; r0 += QR) {
            const int nr = min(QR, nqp - r0);
            __syncthreads();
            for (int i = threadIdx.x; i < nr * D / 4; i += 256)
                reinterpret_cast<f32x4*>(&qs[0][0])[i] =
                    reinterpret_cast<const f32x4*>(qb + (static_cast<int64_t>(hh) * nqp + r0) * D)[i];
            if (threadIdx.x < nr) rqs[threadIdx.x] = rqb[hh * nqp + r0 + threadIdx.x];
            __syncthreads();
            for (int r = 0; r < nr; ++r) {
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < DPL; ++e) dot = fmaf(qs[r][c * DPL + e], k[e], dot);
                run = fmaxf(run, row16_sum(dot) * rqs[r]);
            }
        }
        sum += run;
    }
    if (valid && c == 0) S[static_cast<int64_t>(bg) * s_stride + key] = sum * (1.0f / static_cast<float>(G)) * rkv;
}

// ----------------------------------------------------------------------------- launcher

hipError_t launch_scan(const SelShape& s, const void* qsel, const float* rq, const CacheView& cv,
                       const int64_t* prior_len, float* S, int64_t s_stride, hipStream_t st,
                       const int64_t* prior_len_host) {
    const int bgs = s.batch * s.h_kv;
    if (s.esz == 2 && s.nq_pad == 1 && !s.qsplit) {   // one query per head, G <= 16
        constexpr int GR = kRows16Groups;
        constexpr int KEYS = 64 * GR;
        const int tiles = static_cast<int>((s.t_max + KEYS - 1) / KEYS);
        dim3 grid(bgs * tiles), block(256);
        // With the lengths on the host, list only the workgroups that have keys
        // (a ragged batch otherwise launches batch x h_kv x the longest
        // sequence's tiles, most of them empty).
        TileMap map;
        if (build_tile_map(map, prior_len_host, s.batch, s.h_kv, grid.x,
                           [&](int64_t T) -> int64_t { return T > s.budget ? (T + KEYS - 1) / KEYS : 0; })) {
            if (map.first[s.batch] == 0) return hipSuccess;   // nothing to score
            grid = dim3(static_cast<unsigned>(map.first[s.batch]));
        }
        if (s.d == 128) hipLaunchKernelGGL((scan_rows16_kernel<128, GR>), grid, block, 0, st, (const uint16_t*)qsel, rq, cv, prior_len, s.budget, s.h_kv, s.G, tiles, S, s_stride, map);
        else hipLaunchKernelGGL((scan_rows16_kernel<64, GR>), grid, block, 0, st, (const uint16_t*)qsel, rq, cv, prior_len, s.budget, s.h_kv, s.G, tiles, S, s_stride, map);
    } else if (s.esz == 2) {
        // 32-key blocks per wave: 2 for [hi | lo] query pairs (twice the query
        // fragments per key block); for bf16 rows 3 or 2, whichever gives the
        // shorter launch: the workgroups of a launch run in rounds of two per
        // CU, and a last round that is mostly empty costs a whole round, so
        // the estimate is rounds x keys per wave, with 3 blocks counted 15%
        // faster per key than 2 (this weight matches the measured choice on
        // the three prefill layers: 3 blocks always won on the 128K layer,
        // whose launches span many rounds)
        int nb = 2;
        if (!s.qsplit) {
            const int64_t slots = 2 * int64_t(device_cus());
            auto est = [&](int b) {
                const int64_t wgs = int64_t(bgs) * ((s.t_max + 128 * b - 1) / (128 * b)) * s.nsplit;
                return double((wgs + slots - 1) / slots) * b * (b == 4 ? kScanW4 : b == 3 ? 0.85 : 1.0);
            };
            nb = est(3) <= est(2) ? 3 : 2;
            if (est(4) < est(nb)) nb = 4;
        }
        const int tiles = static_cast<int>((s.t_max + 4 * nb * 32 - 1) / (4 * nb * 32));
        dim3 grid(bgs * tiles * s.nsplit), block(256);
        const int64_t split_stride = int64_t(bgs) * s_stride;
#define KVSEL_SCAN(D, NB, QK) hipLaunchKernelGGL((scan_mfma_kernel<D, NB, QK>), grid, block, 0, st, (const uint16_t*)qsel, rq, cv, prior_len, s.budget, s.h_kv, s.G, s.nq_pad, tiles, s.nsplit, S, s_stride, split_stride)
        if (s.qsplit) {
            if (s.d == 128) KVSEL_SCAN(128, 2, 2); else KVSEL_SCAN(64, 2, 2);
        } else if (nb == 4) {
            if (s.d == 128) KVSEL_SCAN(128, 4, 1); else KVSEL_SCAN(64, 4, 1);
        } else if (nb == 3) {
            if (s.d == 128) KVSEL_SCAN(128, 3, 1); else KVSEL_SCAN(64, 3, 1);
        } else {
            if (s.d == 128) KVSEL_SCAN(128, 2, 1); else KVSEL_SCAN(64, 2, 1);
        }
#undef KVSEL_SCAN
    } else {
        const int tiles = static_cast<int>((s.t_max + 15) / 16);
        dim3 grid(bgs * tiles), block(256);
        if (s.d == 128) hipLaunchKernelGGL((scan_valu_kernel<128>), grid, block, 0, st, (const float*)qsel, rq, cv, prior_len, s.budget, s.h_kv, s.G, s.nq_pad, tiles, S, s_stride);
        else hipLaunchKernelGGL((scan_valu_kernel<64>), grid, block, 0, st, (const float*)qsel, rq, cv, prior_len, s.budget, s.h_kv, s.G, s.nq_pad, tiles, S, s_stride);
    }
    return hipGetLastError();
}

}  // namespace kvsel
