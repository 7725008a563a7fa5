// Attention of every chunk query over its KV head's compacted prior keys (all
// visible) plus the chunk's own keys (causal), online softmax in fp32.
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(a): the compacted
// cache feeds a dense attention kernel.  QUILT page (chiosa.app, "In parole
// semplici"): queries that selected the same KV entries are grouped so those
// entries are loaded once and reused.  Here every query of a chunk that maps
// to one KV head shares the same compacted set, so a workgroup packs
// (token, head-in-group) rows of all G heads of a KV head and stages each key
// tile in LDS once for all of them.  Multi-query attention page, "Teknisk
// innsikt": each query head uses its own query against the shared K/V.
#include <algorithm>
#include <type_traits>

#include "launch.h"

namespace kvsel {

namespace {

// MFMA row m of the key tile is loaded from key sigma(m): with this order the
// 32x32x16 result tile S^T (keys x queries) leaves, in every lane, 8
// consecutive keys per 16-key block in 8 consecutive registers - exactly the
// B operand of the P.V MFMA, so P never leaves registers.
// max over lanes l and l ^ 32 (v_permlane32_swap exchanges the two half-waves)
__device__ __forceinline__ float half_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row sum of the softmax weights as rounded for the P.V MFMAs: one v_dot2
// with (1, 1) per packed bf16 pair (half the adds of summing the fp32 values;
// the normaliser is then the sum of the weights the products use).  The
// 4-wave kernel sums this way (1% faster there); the ping-pong kernel adds
// the fp32 values (1% slower with the pairs).
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float add_pair(uint32_t w, float acc) {
    const bf16x2v ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, w), ones, acc, false);
}
__device__ __forceinline__ int sigma(int m) {
    const int a = m >> 3, hb = (m >> 2) & 1, c = m & 3;
    return 16 * (a >> 1) + 8 * hb + 4 * (a & 1) + c;
}

}  // namespace

// ----------------------------------------------------------------------------- bf16 MFMA kernel
//
// Workgroup: WAVES waves x 32 query rows; rows are (token, head-in-group)
// pairs, row = token * G + head, so a workgroup covers 32 * WAVES / G tokens of
// all G heads, and every wave reads the same staged K/V tiles.
// Per 64-key tile: S^T = K . Q^T (2 x KS MFMAs), online softmax on the lane's
// query column, O^T += V^T . P^T (DB x 4 MFMAs).  K tiles are row-major
// [key][d] and V tiles are [d][key] (written transposed by the pack kernel).
constexpr int kAttnKT = 64;           // keys per staged tile
// wave priority: MFMA issue runs at priority 1, the softmax at 0 (it yields
// the issue slot to the other wave of the SIMD)
#define KVSEL_SETPRIO(p) __builtin_amdgcn_s_setprio(p)

//
// GATHER: the key list is read from its sources (kept cache rows through idx,
// then the chunk's rows) instead of the packed copy; V then arrives row-major
// and is staged [key][d], its V^T fragments read with LDS transpose loads.
// INPLACE: every prior key is kept (T_b <= budget) and the chunk's rows have
// been appended to a contiguous cache, so rows [0, T_b + C) of the cache are
// the key list itself: kall / vall are the cache's K and V ([b][g][nk_pad][d],
// nk_pad = capacity), read in place (V row-major as with GATHER); loads past
// row T_b + C return zeros (the cache beyond is not part of the list).
template <int D, bool OUT_F32, int KT, int WAVES, bool GATHER, bool INPLACE>
__global__ __launch_bounds__(64 * WAVES, 2) void attn_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ kall,
                                                           const uint16_t* __restrict__ vall,
                                                           const int32_t* __restrict__ nsel, int nk_pad, int C, int G,
                                                           int h_kv, int row_blocks, float cl2,
                                                           void* __restrict__ out, int ksplit,
                                                           float* __restrict__ part, AttnGather ga, int cu_pair) {
    static_assert(!(GATHER && INPLACE), "one key-list source");
    constexpr bool VR = GATHER || INPLACE;  // V tile staged row-major
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int NKB = KT / 32;            // 32-key MFMA blocks per tile
    constexpr int LDK = D + 8;
    constexpr int LDV = VR ? D + 16 : KT + 8;   // V tile row: [key][d] (pitch spreads a transpose
                                                 // load over 4 bank groups) or [d][key]
    constexpr int KSZ = KT * LDK;               // stage sizes in elements
    constexpr int VSZ = VR ? KT * LDV : D * LDV;
    constexpr int NT = 64 * WAVES;          // threads per workgroup
    constexpr int ROWS = 32 * WAVES;        // query rows per workgroup
    constexpr int PK = KT * D / 8 / NT;     // 16-byte K pieces per thread per tile
    constexpr int PV = D * KT / 8 / NT;     // 16-byte V^T pieces per thread per tile
    // the two stages as two arrays (a stage is picked by a select)
    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[KSZ], k_lds1[KSZ];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[VSZ], v_lds1[VSZ];
    auto kl = [&](int buf) -> uint16_t* { return buf ? k_lds1 : k_lds0; };
    auto vl = [&](int buf) -> uint16_t* { return buf ? v_lds1 : v_lds0; };

    // slot -> (KV head, row block, key split); later row blocks (more keys) first
    const int slot = xcd_slot(blockIdx.x, gridDim.x);
    int bg = slot / (row_blocks * ksplit);
    const int rem = slot % (row_blocks * ksplit);
    int rblk = row_blocks - 1 - rem / ksplit;
    const int ksp = rem % ksplit;
    if (cu_pair) {
        // One round, two workgroups per CU: an XCD's m workgroups are placed
        // on its CUs in dispatch order, so workgroups p and p + m/2 of the XCD
        // share a CU, and a CU lasts about as long as the tiles of both.  The
        // p-th heaviest row block is paired with the p-th lightest (KV heads
        // of the XCD: m / row_blocks; ksplit is 1 here).
        const int m = gridDim.x / kXcds, k = m / row_blocks;
        const int x = slot / m, pp = slot % m;
        const int q = pp < m / 2 ? pp : m - 1 - (pp - m / 2);
        rblk = row_blocks - 1 - q / k;
        bg = x * k + q % k;
    }
    const int b = bg / h_kv, g = bg % h_kv;
    const int nrows = G * C;
    const int64_t T_b = (GATHER || INPLACE) ? ga.prior_len[b] : 0;
    const int n_s = (GATHER || INPLACE) ? static_cast<int>(T_b < ga.budget ? T_b : ga.budget) : nsel[b];
    const int row_wg0 = rblk * ROWS;
    const int wg_tmax = min(row_wg0 + ROWS - 1, nrows - 1) / G;
    const int ntiles_all = (n_s + wg_tmax + 1 + KT - 1) / KT;
    // with ksplit > 1 this workgroup takes tiles [t_beg, t_end) and leaves an
    // unnormalised partial (O, running max, row sum) for the merge kernel
    const int per = (ntiles_all + ksplit - 1) / ksplit;
    const int t_beg = min(ntiles_all, ksp * per);
    const int ntiles = min(ntiles_all, t_beg + per) - t_beg;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int half = lane >> 5, col = lane & 31;
    const int wrow0 = row_wg0 + wave * 32;
    const bool wave_active = wrow0 < nrows;
    const int w_tmin = min(wrow0, nrows - 1) / G;
    const int w_tmax = min(wrow0 + 31, nrows - 1) / G;
    const int qrow = wrow0 + col;
    const bool rvalid = qrow < nrows;
    const int tok = rvalid ? qrow / G : 0;
    const int hh = rvalid ? qrow % G : 0;
    const int64_t qoff = ((static_cast<int64_t>(b) * h_kv * G + g * G + hh) * C + tok) * D;

    // (a lane past the last row reads the head's first row: qoff points there)
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + qoff + 16 * ks + 8 * half));
    // The Q loads are completed before the tile loop, on every path: otherwise
    // the loop header merges a path on which they may still be in flight and
    // the compiler's wait analysis puts a wait for every outstanding load
    // (including the next tile's, just issued) in front of each tile's first
    // MFMA.  The packed path completes them after requesting its first tile.
    auto complete_q = [&] {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    };
    if constexpr (GATHER) complete_q();

    const uint16_t* kb = kall + static_cast<int64_t>(bg) * nk_pad * D;
    const uint16_t* vb = vall + static_cast<int64_t>(bg) * D * nk_pad;   // [d][slot] packed, [row][d] in place
    // Staging with a full tile of latency for every load (t counts tiles in
    // the order this workgroup reads them): V(t+1) is fetched at the start of
    // tile t and written to LDS at its end; K(t+1), fetched in the middle of
    // tile t-1, is written after t's S MFMAs and K(t+2) is fetched then.
    // Buffer (t+1)&1 was last read in tile t-1 and buffer t&1 (K(t+2)) in
    // tile t, each closed by a barrier before the write.
    u32x4 rk[PK], rv[PV];
    // Per-thread byte offsets inside a tile, fixed for the whole loop: a load
    // is a buffer load with this lane offset and the tile's uniform offset
    // (no per-load 64-bit address arithmetic on the VALU).
    uint32_t koff[PK], voff[PV];
#pragma unroll
    for (int i = 0; i < PK; ++i) {
        const int p = tid + NT * i;
        koff[i] = static_cast<uint32_t>(((p / (D / 8)) * D + (p % (D / 8)) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < PV; ++i) {
        const int p = tid + NT * i;
        voff[i] = static_cast<uint32_t>(((p / (KT / 8)) * nk_pad + (p % (KT / 8)) * 8) * 2);
    }
    // buffer descriptors over this KV head's packed K and V^T, or its cache
    // rows [0, T_b + C) in place (reads past the end return 0); the tile
    // offset is the uniform soffset operand
    const int list_bytes = (INPLACE ? n_s + C : nk_pad) * D * 2;
    const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), 0, list_bytes, kBufferFormat);
    const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), 0, list_bytes, kBufferFormat);
    // the tile index is the same in every lane; readfirstlane hands it to the
    // scalar offset operand directly (no per-lane waterfall over its values)
    auto fetch_k = [&](int t) {
        const int so = __builtin_amdgcn_readfirstlane(t * KT * D * 2);
#pragma unroll
        for (int i = 0; i < PK; ++i) rk[i] = __builtin_amdgcn_raw_buffer_load_b128(rsk, koff[i], so, 0);
    };
    // Gathering: slot s < n_s is cache row rowidx[s], then the chunk's rows
    // (coded -1 - chunk row); slots past the list read the chunk's last row
    // (finite values that the causal mask removes).  The row numbers of the
    // next two tiles are held in registers (R1: tile t+1, R2: tile t+2 at the
    // start of tile t), so no row load waits on an index load.
    int32_t R1[PK], R2[PK];
    auto rows_of = [&](int t, int32_t (&rr)[PK]) {
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int sl = t * KT + (tid + NT * i) / (D / 8);
            rr[i] = sl < n_s ? (ga.identity ? static_cast<int32_t>(bg * ga.ri_stride + sl)
                                            : ga.rowidx[static_cast<int64_t>(bg) * ga.ri_stride + sl])
                             : -1 - (bg * C + min(sl - n_s, C - 1));
        }
    };
    auto gfetch = [&](const int32_t (&rr)[PK], bool v, u32x4 (&dst)[PK]) {
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int32_t r = rr[i];
            const char* base = r >= 0 ? (v ? ga.cv.v : ga.cv.k) + static_cast<int64_t>(r) * (D * 2)
                                      : static_cast<const char*>(v ? ga.v_chunk : ga.k_chunk) +
                                            static_cast<int64_t>(-1 - r) * (D * 2);
            dst[i] = *reinterpret_cast<const u32x4*>(base + ((tid + NT * i) % (D / 8)) * 16);
        }
    };
    auto stash_k = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PK; ++i) {
            const int p = tid + NT * i;
            const int r = p / (D / 8), c = p % (D / 8);
            *reinterpret_cast<u32x4*>(&kl(buf)[r * LDK + c * 8]) = rk[i];
        }
    };
    auto fetch_v = [&](int t) {
        if constexpr (INPLACE) {              // row-major rows, the same pieces as K
            const int so = __builtin_amdgcn_readfirstlane(t * KT * D * 2);
#pragma unroll
            for (int i = 0; i < PV; ++i) rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rsv, koff[i], so, 0);
        } else {
            const int so = __builtin_amdgcn_readfirstlane(t * KT * 2);
#pragma unroll
            for (int i = 0; i < PV; ++i) rv[i] = __builtin_amdgcn_raw_buffer_load_b128(rsv, voff[i], so, 0);
        }
    };
    auto stash_v = [&](int buf) {
#pragma unroll
        for (int i = 0; i < PV; ++i) {
            const int p = tid + NT * i;
            if (VR) {
                const int r = p / (D / 8), c = p % (D / 8);
                *reinterpret_cast<u32x4*>(&vl(buf)[r * LDV + c * 8]) = rv[i];
            } else {
                const int d = p / (KT / 8), j = p % (KT / 8);
                *reinterpret_cast<u32x4*>(&vl(buf)[d * LDV + j * 8]) = rv[i];
            }
        }
    };
    // V^T fragment of the P.V MFMA: d = 32*db + (lane & 31), keys kb + 8*half
    // .. +7.  Row-major V: two transpose loads; in each 16-lane group, lane j
    // receives element (j & 3) of the 8 bytes addressed by lanes 4r + (j >> 2),
    // r = 0..3, so lane s of the group points at key kb + 8*half + (s >> 2),
    // d = 32*db + 16*((lane >> 4) & 1) + 4*(s & 3), and gets keys +0..3 of
    // column d (+4..7 from the second load).
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef short v8s __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    auto vfrag = [&](int buf, int db, int k0) -> bf16x8 {
        if (VR) {
            const int j = lane & 15;
            const int row = k0 + 8 * half + (j >> 2);
            const int colv = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
            const v4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)&vl(buf)[row * LDV + colv]);
            const v4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)&vl(buf)[(row + 4) * LDV + colv]);
            const v8s x = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            return __builtin_bit_cast(bf16x8, x);
        }
        return *reinterpret_cast<const bf16x8*>(&vl(buf)[(32 * db + col) * LDV + k0 + 8 * half]);
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m = -INFINITY, l = 0.0f;
    // kept beside m, updated only when it moves: the value the block max must
    // pass to move it (m + 2^8 in log2 units) and -m * cl2 for the exponents
    // (0 while no key is visible, so masked scores give 0)
    float m_thr = -INFINITY, nmc = 0.0f;
    const float step8 = 8.0f / cl2;
    float l2[2] = {0.0f, 0.0f};                 // row sum in two chains (l: their total at the end)
    const int krow = sigma(col);
    // K fragment of the S MFMA: key 32*kb2 + krow, elements 16*ks + 8*half .. +7
    auto kfrag = [&](int buf, int kb2, int ks) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(&kl(buf)[(32 * kb2 + krow) * LDK + 16 * ks + 8 * half]);
    };
    const int lim = n_s + tok;                  // last visible slot of this lane's query

    // One KT-key tile: S^T, online softmax, O^T += V^T P^T.  MASK applies the
    // causal limit (only tiles that reach past the wave's first token need it).
    // The running max is only moved when it grows by more than 2^8 (log2
    // units): p = exp2(s*cl2 - m*cl2) then stays <= 256 and O, l share the same
    // reference, so the result is unchanged while most tiles skip the rescale.
    auto tile = [&](const int buf, const int s0, auto mask_tag, auto&& mid) {
        constexpr bool MASK = decltype(mask_tag)::value;
        f32x16 sacc[NKB];
        KVSEL_SETPRIO(1);                  // MFMA issue first; softmax yields to the other wave
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {          // every S MFMA of the tile is issued first
            sacc[kb2] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = kfrag(buf, kb2, ks);
                sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kb2], 0, 0, 0);
            }
        }
        KVSEL_SETPRIO(0);
        mid();
        // Online softmax per 32-key block, so block kb2's softmax overlaps the
        // MFMAs still running for the next block and its P.V MFMAs overlap the
        // next block's softmax.
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
            // this block's V^T fragments are read now so they land during the softmax
            bf16x8 vf[DB][2];
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int k16 = 0; k16 < 2; ++k16)
                    vf[db][k16] = vfrag(buf, db, 32 * kb2 + 16 * k16);
            // register r holds slot s0 + 32*kb2 + 16*(r>>3) + 8*half + (r&7)
            if (MASK) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int sl = s0 + 32 * kb2 + 16 * (r >> 3) + 8 * half + (r & 7);
                    if (sl > lim) sacc[kb2][r] = -INFINITY;
                }
            }
            float mt = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb2][r]);
            mt = half_max(mt);
            const float m_new = fmaxf(m, mt);
            if (__ballot(m_new > m_thr) != 0ull) {
                const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m - m_new) * cl2);
                l2[0] *= alpha;
                l2[1] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
                m = m_new;
                m_thr = m + step8;
                nmc = m == -INFINITY ? 0.0f : -m * cl2;   // no visible key yet: every p is 0
            }
            bf16x8 pf[2];
            KVSEL_SETPRIO(0);
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][8 * k16 + 2 * e], cl2, nmc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][8 * k16 + 2 * e + 1], cl2, nmc));
                    w[e] = pack_bf16x2(p0, p1);
                    l2[e & 1] = add_pair(w[e], l2[e & 1]);
                }
                pf[k16] = __builtin_bit_cast(bf16x8, w);
            }
            KVSEL_SETPRIO(1);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int k16 = 0; k16 < 2; ++k16)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db][k16], pf[k16], o[db], 0, 0, 0);
            KVSEL_SETPRIO(0);
        }
    };

    // Every prefetch is unconditional, with its tile index clamped to the last
    // tile this workgroup reads (always in bounds; the extra copy is never
    // stashed): the same loads are then in flight on every path, so the
    // compiler's waits count them exactly and each load keeps its full tile of
    // latency.
    const int t_last = max(t_beg + ntiles - 1, 0);
    auto tc = [&](int t) { return min(t, t_last); };
    // Packed path: the row blocks of one KV head (all on one XCD) start their
    // tile sequence at evenly spaced tiles and wrap around, so at any moment
    // they read different tiles rather than all requesting the same lines from
    // the L2 at once (the softmax is order-independent; the per-tile mask
    // tests take the tile's own position).  tix(u) is the u-th tile read;
    // past the last one it repeats the last one (always in bounds).
    const int rot = ntiles > 0 ? (rblk * ntiles) / row_blocks : 0;
    auto tix = [&](int uu) {
        const int v = min(uu, max(ntiles - 1, 0)) + rot;
        return t_beg + (v >= ntiles ? v - ntiles : v);
    };
    if constexpr (GATHER) {
        static_assert(PK == PV, "K and V rows are fetched together");
        rows_of(tc(t_beg), R1);
        if (ntiles > 0) {
            gfetch(R1, false, rk);
            gfetch(R1, true, rv);
            stash_k(0);
            stash_v(0);
        }
        rows_of(tc(t_beg + 1), R1);
        gfetch(R1, false, rk);
        rows_of(tc(t_beg + 2), R2);
    } else {
        if (ntiles > 0) {
            fetch_k(tix(0));
            fetch_v(tix(0));
            complete_q();
            stash_k(0);
            stash_v(0);
        } else {
            complete_q();
        }
        fetch_k(tix(1));
    }
    __syncthreads();
    // one tile: u counts tiles within this workgroup's range, buf is its stage
    auto step = [&](const int u, const int buf) {
        const int t = GATHER ? t_beg + u : tix(u);
        if constexpr (GATHER) {
            gfetch(R1, true, rv);                // V(t+1)
#pragma unroll
            for (int i = 0; i < PK; ++i) R1[i] = R2[i];
            rows_of(tc(t + 3), R2);
        } else {
            fetch_v(tix(u + 1));
        }
        auto mid = [&] {
            if (u + 1 < ntiles) stash_k(buf ^ 1);
            if constexpr (GATHER) gfetch(R1, false, rk);   // K(t+2)
            else fetch_k(tix(u + 2));
        };
        const int s0 = t * KT;
        if (wave_active && s0 <= n_s + w_tmax) {
            if (s0 + KT > n_s + w_tmin + 1) tile(buf, s0, std::true_type{}, mid);
            else tile(buf, s0, std::false_type{}, mid);
        } else {
            mid();
        }
        if (u + 1 < ntiles) stash_v(buf ^ 1);
        __syncthreads();
    };
    for (int u = 0; u < ntiles; ++u) step(u, u & 1);

    l = half_sum(l2[0] + l2[1]);
    if (!rvalid) return;
    if (ksplit > 1) {                            // partial: O unnormalised, (m, l) per row
        const int64_t rows_total = static_cast<int64_t>(gridDim.x / (row_blocks * ksplit)) * nrows;
        float* po = part + static_cast<int64_t>(ksp) * rows_total * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * half;
                *reinterpret_cast<f32x4*>(po + qoff + d0) =
                    f32x4{o[db][4 * a4 + 0], o[db][4 * a4 + 1], o[db][4 * a4 + 2], o[db][4 * a4 + 3]};
            }
        if (half == 0) {
            float* pml = part + static_cast<int64_t>(ksplit) * rows_total * D + (static_cast<int64_t>(ksp) * rows_total + qoff / D) * 2;
            pml[0] = m;
            pml[1] = l;
        }
        return;
    }
    const float inv = 1.0f / l;
    // O^T tile: register r of block db holds d = 32*db + 8*(r>>2) + 4*half + (r&3)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d0 = 32 * db + 8 * a4 + 4 * half;
            const float v0 = o[db][4 * a4 + 0] * inv, v1 = o[db][4 * a4 + 1] * inv;
            const float v2 = o[db][4 * a4 + 2] * inv, v3 = o[db][4 * a4 + 3] * inv;
            if (OUT_F32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(out) + qoff + d0) = f32x4{v0, v1, v2, v3};
            } else {
                uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + qoff + d0);
                dst[0] = pack_bf16x2(v0, v1);
                dst[1] = pack_bf16x2(v2, v3);
            }
        }
}

// ----------------------------------------------------------------------------- ping-pong MFMA kernel
//
// Packed path, 8 waves x 32 query rows.  Waves w and w + 4 share a SIMD; the
// two groups of four (A = waves 0-3, B = waves 4-7) run the same tile loop
// half a tile apart, so that on every SIMD one wave issues MFMAs while the
// other computes a softmax.  For tile t a wave runs
//   M(t): O += P(t-1) V(t-1) (if t >= 1), then S(t) = K(t) Q^T (if t < n)
//   X(t): online softmax of S(t) -> P(t), running max and sum, rescale of O
// each followed by a workgroup barrier; group B passes one barrier before
// the loop and group A one after it, so M(t) of one group runs beside X(t-1)
// (or X(t)) of the other and every wave passes the same 2n+4 barriers.  The
// rescale of O by X(t) comes after M(t) has added P(t-1) V(t-1) and before
// M(t+1) adds P(t) V(t), the order of the sequential recurrence.
// Staging: each thread owns pieces tid and tid + 512 of every K and V^T tile
// (16 bytes each) and writes one piece in each half of its loop, 2 barriers
// after fetching it.  Between barriers 2u and 2u+1 (counted from the first
// loop barrier of group A) the workgroup writes half of K(u+1) and of V(u),
// the other halves in the next interval, while K(u) and V(u-1) are read.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(512, 1) void attn_pp_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kall,
                                                       const uint16_t* __restrict__ vall,
                                                       const int32_t* __restrict__ nsel, int nk_pad, int C, int G,
                                                       int h_kv, int row_blocks, float cl2, void* __restrict__ out,
                                                       int ksplit, float* __restrict__ part) {
    constexpr int KT = 64, NT = 512, ROWS = 256;
    constexpr int KS = D / 16;
    constexpr int DB = D / 32;
    constexpr int NKB = KT / 32;
    constexpr int LDK = D + 8;
    constexpr int LDV = KT + 8;
    constexpr int PK = KT * D / 8 / NT;     // 16-byte pieces per thread per K (or V^T) tile
    __shared__ __attribute__((aligned(16))) uint16_t k_lds0[KT * LDK], k_lds1[KT * LDK];
    __shared__ __attribute__((aligned(16))) uint16_t v_lds0[D * LDV], v_lds1[D * LDV];
    auto kl = [&](int buf) -> uint16_t* { return buf ? k_lds1 : k_lds0; };
    auto vl = [&](int buf) -> uint16_t* { return buf ? v_lds1 : v_lds0; };

    const int slot = xcd_slot(blockIdx.x, gridDim.x);
    const int bg = slot / (row_blocks * ksplit);
    const int rem = slot % (row_blocks * ksplit);
    const int rblk = row_blocks - 1 - rem / ksplit;
    const int ksp = rem % ksplit;
    const int b = bg / h_kv, g = bg % h_kv;
    const int nrows = G * C;
    const int n_s = nsel[b];
    const int row_wg0 = rblk * ROWS;
    const int wg_tmax = min(row_wg0 + ROWS - 1, nrows - 1) / G;
    const int ntiles_all = (n_s + wg_tmax + 1 + KT - 1) / KT;
    const int per = (ntiles_all + ksplit - 1) / ksplit;
    const int t_beg = min(ntiles_all, ksp * per);
    const int ntiles = min(ntiles_all, t_beg + per) - t_beg;

    const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);   // 0: group A, 1: group B (half a tile later)
    const int half = lane >> 5, col = lane & 31;
    const int wrow0 = row_wg0 + wave * 32;
    const bool wave_active = wrow0 < nrows;
    const int w_tmin = min(wrow0, nrows - 1) / G;
    const int w_tmax = min(wrow0 + 31, nrows - 1) / G;
    const int qrow = wrow0 + col;
    const bool rvalid = qrow < nrows;
    const int tok = rvalid ? qrow / G : 0;
    const int hh = rvalid ? qrow % G : 0;
    const int64_t qoff = ((static_cast<int64_t>(b) * h_kv * G + g * G + hh) * C + tok) * D;

    // (a lane past the last row reads the head's first row: qoff points there);
    // the loads are completed after the first tile is requested (prologue)
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q + qoff + 16 * ks + 8 * half));
    auto complete_q = [&] {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
    };

    const uint16_t* kb = kall + static_cast<int64_t>(bg) * nk_pad * D;
    const uint16_t* vb = vall + static_cast<int64_t>(bg) * D * nk_pad;
    // piece h of this thread is tile piece tid + NT*h (h = 0, 1); a K piece is
    // row p / (D/8), chunk p % (D/8), a V^T piece row p / (KT/8), chunk p % (KT/8)
    static_assert(PK == 2, "two 16-byte pieces per thread per tile (d = 128)");
    u32x4 rk[2], rv[2];
    uint32_t koff[2], voff[2], kst[2], vst[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int p = tid + NT * h;
        koff[h] = static_cast<uint32_t>(((p / (D / 8)) * D + (p % (D / 8)) * 8) * 2);
        voff[h] = static_cast<uint32_t>(((p / (KT / 8)) * nk_pad + (p % (KT / 8)) * 8) * 2);
        kst[h] = static_cast<uint32_t>((p / (D / 8)) * LDK + (p % (D / 8)) * 8);
        vst[h] = static_cast<uint32_t>((p / (KT / 8)) * LDV + (p % (KT / 8)) * 8);
    }
    const __amdgpu_buffer_rsrc_t rsk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kb), 0, nk_pad * D * 2, kBufferFormat);
    const __amdgpu_buffer_rsrc_t rsv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vb), 0, nk_pad * D * 2, kBufferFormat);
    // piece h of K tile tk and V^T tile tv into registers / from registers to stages
    auto fetch = [&](int h, int tk, int tv) {
        rk[h] = __builtin_amdgcn_raw_buffer_load_b128(rsk, koff[h], __builtin_amdgcn_readfirstlane(tk * KT * D * 2), 0);
        rv[h] = __builtin_amdgcn_raw_buffer_load_b128(rsv, voff[h], __builtin_amdgcn_readfirstlane(tv * KT * 2), 0);
    };
    auto stash = [&](int h, int kbuf, int vbuf) {
        *reinterpret_cast<u32x4*>(kl(kbuf) + kst[h]) = rk[h];
        *reinterpret_cast<u32x4*>(vl(vbuf) + vst[h]) = rv[h];
    };
    // tiles in a rotated order per row block (as in attn_mfma_kernel); past
    // the last tile the index repeats the last one (always in bounds)
    const int rot = ntiles > 0 ? (rblk * ntiles) / row_blocks : 0;
    auto tix = [&](int uu) {
        const int v = min(uu, max(ntiles - 1, 0)) + rot;
        return t_beg + (v >= ntiles ? v - ntiles : v);
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m = -INFINITY, l = 0.0f;
    float m_thr = -INFINITY, nmc = 0.0f;    // as in attn_mfma_kernel
    const float step8 = 8.0f / cl2;
    const int krow = sigma(col);
    const int lim = n_s + tok;
    f32x16 sacc[NKB];                       // S(t), from M(t) to X(t)
    bf16x8 pf[NKB][2];                      // P(t), from X(t) to M(t+1)
    auto live = [&](int t) { return t < ntiles && wave_active && tix(t) * KT <= n_s + w_tmax; };

    // M(t) as four groups of 8 MFMAs (P.V for each 32-key block, then S for
    // each); a group's 8 fragments are read from LDS before the previous
    // group's MFMAs are issued, so the reads' latency hides behind them
    auto rd_v = [&](int buf, int kb2, bf16x8 (&f)[8]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16)
                f[2 * db + k16] = *reinterpret_cast<const bf16x8*>(
                    &vl(buf)[(32 * db + col) * LDV + 32 * kb2 + 16 * k16 + 8 * half]);
    };
    auto rd_k = [&](int buf, int kb2, bf16x8 (&f)[8]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            f[ks] = *reinterpret_cast<const bf16x8*>(&kl(buf)[(32 * kb2 + krow) * LDK + 16 * ks + 8 * half]);
    };
    auto mm_v = [&](int kb2, const bf16x8 (&f)[8]) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[2 * db + k16], pf[kb2][k16], o[db], 0, 0, 0);
    };
    auto mm_k = [&](int kb2, const bf16x8 (&f)[8]) {
        sacc[kb2] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks], qf[ks], sacc[kb2], 0, 0, 0);
    };
    static_assert(2 * DB == 8 && KS == 8, "8 fragments per group (d = 128)");
    auto phase_m = [&](int t) {
        KVSEL_SETPRIO(1);
        const bool pv = t >= 1 && live(t - 1), sk = live(t);   // O += P(t-1) V(t-1); S(t)^T = K(t) Q^T
        const int vb_ = (t - 1) & 1, kb_ = t & 1;
        bf16x8 fa[8], fb[8];
        // (sched_barrier: the scheduler would otherwise sink each read to just
        // before its MFMA and expose the LDS latency)
        if (pv && sk) {
            rd_v(vb_, 0, fa);
            rd_v(vb_, 1, fb);
            __builtin_amdgcn_sched_barrier(0);
            mm_v(0, fa);
            rd_k(kb_, 0, fa);
            __builtin_amdgcn_sched_barrier(0);
            mm_v(1, fb);
            rd_k(kb_, 1, fb);
            __builtin_amdgcn_sched_barrier(0);
            mm_k(0, fa);
            mm_k(1, fb);
        } else if (pv) {
            rd_v(vb_, 0, fa);
            rd_v(vb_, 1, fb);
            __builtin_amdgcn_sched_barrier(0);
            mm_v(0, fa);
            mm_v(1, fb);
        } else if (sk) {
            rd_k(kb_, 0, fa);
            rd_k(kb_, 1, fb);
            __builtin_amdgcn_sched_barrier(0);
            mm_k(0, fa);
            mm_k(1, fb);
        }
        KVSEL_SETPRIO(0);
    };
    // X(t): the running max moves only when it grows by more than 2^8 (log2
    // units), as in attn_mfma_kernel
    auto phase_x = [&](int t) {
        if (!live(t)) return;
        const int s0 = tix(t) * KT;
        if (s0 + KT > n_s + w_tmin + 1) {    // causal limit reaches into this tile
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int sl = s0 + 32 * kb2 + 16 * (r >> 3) + 8 * half + (r & 7);
                    if (sl > lim) sacc[kb2][r] = -INFINITY;
                }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb2][r]);
        mt = half_max(mt);
        const float m_new = fmaxf(m, mt);
        if (__ballot(m_new > m_thr) != 0ull) {
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m - m_new) * cl2);
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m = m_new;
            m_thr = m + step8;
            nmc = m == -INFINITY ? 0.0f : -m * cl2;
        }
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
            for (int k16 = 0; k16 < 2; ++k16) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][8 * k16 + 2 * e], cl2, nmc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[kb2][8 * k16 + 2 * e + 1], cl2, nmc));
                    l += p0 + p1;
                    w[e] = pack_bf16x2(p0, p1);
                }
                pf[kb2][k16] = __builtin_bit_cast(bf16x8, w);
            }
    };

    // prologue: K(0) staged whole; registers hold K(1) and V(0) (both pieces)
    if (ntiles > 0) {
        fetch(0, tix(0), tix(0));
        fetch(1, tix(0), tix(0));
        complete_q();
        stash(0, 0, 0);
        stash(1, 0, 0);                      // V(0) also lands in stage 0 here (rewritten below)
        fetch(0, tix(1), tix(0));
        fetch(1, tix(1), tix(0));
    } else {
        complete_q();
    }
    __syncthreads();
    if (ntiles > 0 && grp == 1) {            // group B: the second half of the interval before the loop
        stash(1, 1, 0);                      // K(1), V(0) piece 1
        fetch(1, tix(2), tix(1));
        __syncthreads();
    }
    const int nloop = ntiles > 0 ? ntiles + 1 : 0;
    for (int t = 0; t < nloop; ++t) {
        stash(0, (t + 1) & 1, t & 1);        // K(t+1), V(t) piece 0
        fetch(0, tix(t + 2), tix(t + 1));
        phase_m(t);
        __syncthreads();
        stash(1, (t + 1 + grp) & 1, (t + grp) & 1);   // group A: K(t+1), V(t); B: K(t+2), V(t+1)
        fetch(1, tix(t + 2 + grp), tix(t + 1 + grp));
        phase_x(t);
        __syncthreads();
    }
    if (ntiles > 0 && grp == 0) __syncthreads();   // group A: the interval after the loop

    l = half_sum(l);
    if (!rvalid) return;
    if (ksplit > 1) {
        const int64_t rows_total = static_cast<int64_t>(gridDim.x / (row_blocks * ksplit)) * nrows;
        float* po = part + static_cast<int64_t>(ksp) * rows_total * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = 32 * db + 8 * a4 + 4 * half;
                *reinterpret_cast<f32x4*>(po + qoff + d0) =
                    f32x4{o[db][4 * a4 + 0], o[db][4 * a4 + 1], o[db][4 * a4 + 2], o[db][4 * a4 + 3]};
            }
        if (half == 0) {
            float* pml = part + static_cast<int64_t>(ksplit) * rows_total * D + (static_cast<int64_t>(ksp) * rows_total + qoff / D) * 2;
            pml[0] = m;
            pml[1] = l;
        }
        return;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
            const int d0 = 32 * db + 8 * a4 + 4 * half;
            const float v0 = o[db][4 * a4 + 0] * inv, v1 = o[db][4 * a4 + 1] * inv;
            const float v2 = o[db][4 * a4 + 2] * inv, v3 = o[db][4 * a4 + 3] * inv;
            if (OUT_F32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(out) + qoff + d0) = f32x4{v0, v1, v2, v3};
            } else {
                uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + qoff + d0);
                dst[0] = pack_bf16x2(v0, v1);
                dst[1] = pack_bf16x2(v2, v3);
            }
        }
}

// ----------------------------------------------------------------------------- split merge
//
// out = sum_s w_s O_s / sum_s w_s l_s with w_s = exp2((m_s - max_s m_s) * cl2):
// the key-split partials of one row combined as one softmax over all its keys.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part, int64_t rows, int ksplit,
                                                         float cl2, void* __restrict__ out) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (row, 4-column group)
    if (i >= rows * (D / 4)) return;
    const int64_t row = i / (D / 4);
    const int c4 = static_cast<int>(i % (D / 4));
    const float* pml = part + static_cast<int64_t>(ksplit) * rows * D;
    float mx = -INFINITY;
    for (int s = 0; s < ksplit; ++s) mx = fmaxf(mx, pml[(s * rows + row) * 2]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
    for (int s = 0; s < ksplit; ++s) {
        const float ms = pml[(s * rows + row) * 2], ls = pml[(s * rows + row) * 2 + 1];
        const float w = ls > 0.0f ? __builtin_amdgcn_exp2f((ms - mx) * cl2) : 0.0f;
        const f32x4 v = *reinterpret_cast<const f32x4*>(part + (s * rows + row) * D + 4 * c4);
        acc += w * v;
        den += w * ls;
    }
    const float inv = 1.0f / den;
    if (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + row * D + 4 * c4) = acc * inv;
    } else {
        uint32_t* dst = reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(out) + row * D + 4 * c4);
        dst[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
        dst[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    }
}

// ----------------------------------------------------------------------------- fp32 VALU kernel
//
// 16 lanes per query row, each holding D/16 consecutive elements of q and of
// the output; a workgroup takes 16 rows ((token, head-in-group) pairs as in
// the MFMA kernels) and stages 32-key tiles of K and V in LDS.  Each lane
// forms its part of q . k, the 16 lanes of the row add their parts with DPP,
// and every lane runs the row's online softmax and accumulates its slice of
// P.V.
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void attn_valu_kernel(const float* __restrict__ q, const float* __restrict__ kall,
                                                        const float* __restrict__ vall,
                                                        const int32_t* __restrict__ nsel, int nk_pad, int C, int G,
                                                        int h_kv, int row_blocks, float scale,
                                                        void* __restrict__ out) {
    constexpr int KT = 32;
    constexpr int DPL = D / 16;             // elements per lane
    constexpr int RPW = 16;                 // rows per workgroup
    constexpr int PPT = KT * D / 4 / 256;   // float4 pieces per thread per tile
    __shared__ __attribute__((aligned(16))) float kt[KT][D];
    __shared__ __attribute__((aligned(16))) float vt[KT][D];
    const int bg = blockIdx.x / row_blocks;
    const int rblk = row_blocks - 1 - blockIdx.x % row_blocks;
    const int b = bg / h_kv, g = bg % h_kv;
    const int nrows = G * C;
    const int n_s = nsel[b];
    const int row0 = rblk * RPW;
    const int wg_tmax = min(row0 + RPW - 1, nrows - 1) / G;
    const int ntiles = (n_s + wg_tmax + 1 + KT - 1) / KT;
    const int c = threadIdx.x & 15;
    const int qrow = row0 + (threadIdx.x >> 4);
    const bool rvalid = qrow < nrows;
    const int tok = rvalid ? qrow / G : 0, hh = rvalid ? qrow % G : 0;
    const int64_t qoff = ((static_cast<int64_t>(b) * h_kv * G + g * G + hh) * C + tok) * D;
    float qv[DPL], acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; e += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(q + qoff + c * DPL + e);
        qv[e] = x[0]; qv[e + 1] = x[1]; qv[e + 2] = x[2]; qv[e + 3] = x[3];
    }
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.0f;
    const float* kb = kall + static_cast<int64_t>(bg) * nk_pad * D;
    const float* vb = vall + static_cast<int64_t>(bg) * nk_pad * D;
    float m = -INFINITY, l = 0.0f;
    const int lim = n_s + tok;                  // slot 0 is always visible, so m is finite after tile 0
    for (int t = 0; t < ntiles; ++t) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int p = threadIdx.x + 256 * i;
            reinterpret_cast<f32x4*>(&kt[0][0])[p] = reinterpret_cast<const f32x4*>(kb + static_cast<int64_t>(t) * KT * D)[p];
            reinterpret_cast<f32x4*>(&vt[0][0])[p] = reinterpret_cast<const f32x4*>(vb + static_cast<int64_t>(t) * KT * D)[p];
        }
        __syncthreads();
        float s[KT];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) dot = fmaf(qv[e], kt[j][c * DPL + e], dot);
            dot = row16_sum(dot);
            s[j] = (t * KT + j <= lim) ? dot * scale : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        const float m_new = fmaxf(m, mt);
        const float alpha = expf(m - m_new);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
        m = m_new;
#pragma unroll
        for (int j = 0; j < KT; ++j) {
            const float p = expf(s[j] - m);
            l += p;
#pragma unroll
            for (int e = 0; e < DPL; ++e) acc[e] = fmaf(p, vt[j][c * DPL + e], acc[e]);
        }
    }
    if (!rvalid) return;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        if (OUT_F32) static_cast<float*>(out)[qoff + c * DPL + e] = acc[e] * inv;
        else static_cast<uint16_t*>(out)[qoff + c * DPL + e] = f32_to_bf16(acc[e] * inv);
    }
}

// ----------------------------------------------------------------------------- launcher

bool attn_use_gather(const SelShape& s) { return s.esz == 2 && s.G * s.C <= 128; }
// Ping-pong kernel: packed bf16 path with d = 128 (two staged pieces per
// thread), where its 256-row grid either splits keys (fewer workgroups than
// CUs) or holds two or more workgroups per CU.  In between (one round of one
// workgroup per CU) the 4-wave kernel measured faster (2% on 8 KV heads x 32
// row blocks); with splits and with several rounds the ping-pong kernel was
// 1.7-3% faster.
static bool attn_use_pp(const SelShape& s) {
    if (!(s.esz == 2 && s.d == 128 && !attn_use_gather(s))) return false;
    const int64_t wgs = int64_t(s.batch) * s.h_kv * ((s.G * s.C + 255) / 256);
    return wgs < 256 || wgs >= 512;
}

int attn_ksplit(const SelShape& s, bool inplace) {
    if (s.esz != 2) return 1;
    // gathering (one row block per KV head): split the key list only as far as
    // needed for one round of two workgroups per CU (at most 4 ways); on the
    // 64-sequence decode batch (512 KV heads) no split, and no merge pass,
    // measured 105 us per step against 116 with 2 and 133 with 4 ways
    if (attn_use_gather(s)) {
        const int64_t wgs = int64_t(s.batch) * s.h_kv;
        int k = 1;
        while (k < 4 && wgs * k < 2 * int64_t(device_cus())) k *= 2;
        return k;
    }
    // at least two 4-wave workgroups, or one 8-wave ping-pong workgroup, per CU
    // (the in-place list is read by the 4-wave kernel only)
    const bool pp = !inplace && attn_use_pp(s);
    const int rows = pp ? 256 : 128, target = pp ? 256 : 512;
    const int64_t wgs = int64_t(s.batch) * s.h_kv * ((s.G * s.C + rows - 1) / rows);
    int k = 1;
    while (k < 4 && wgs * k < target) k *= 2;
    return k;
}

size_t attn_part_bytes(const SelShape& s) {
    const int k = std::max(attn_ksplit(s, false), attn_ksplit(s, true));
    if (k == 1) return 0;
    const size_t rows = size_t(s.batch) * s.h_q * s.C;
    return size_t(k) * rows * (s.d + 2) * 4;
}

hipError_t launch_attn(const SelShape& s, const void* q, const void* kall, const void* vall, const int32_t* nsel,
                       int nk_pad, float scale, void* out, bool out_f32, float* part, hipStream_t st,
                       const AttnGather* gather, bool inplace) {
    const int bgs = s.batch * s.h_kv;
    if (s.esz == 2) {
        // with inplace, `gather` only carries the prior lengths and the budget
        const bool gathering = gather && !inplace;
        const bool pp = !gather && attn_use_pp(s);                // 8 waves x 32 rows, else 4 waves
        const int row_blocks = (s.G * s.C + (pp ? 255 : 127)) / (pp ? 256 : 128);
        const int ksplit = attn_ksplit(s, inplace);
        dim3 grid(bgs * row_blocks * ksplit), block(pp ? 512 : 256);
        // 4-wave packed kernel in one round of two workgroups per CU, whole KV
        // heads per XCD: pair long with short row blocks on each CU
        const int64_t per_xcd = grid.x / kXcds;
        const int cu_pair = (!gathering && !pp && ksplit == 1 && row_blocks > 1 &&
                             grid.x % kXcds == 0 && per_xcd % row_blocks == 0 &&
                             int64_t(grid.x) <= 2 * int64_t(device_cus())) ? 1 : 0;
        const float cl2 = scale * 1.4426950408889634f;
        const uint16_t *qq = (const uint16_t*)q, *kk = (const uint16_t*)kall, *vv = (const uint16_t*)vall;
        const AttnGather ga = gather ? *gather : AttnGather{};
#define KVSEL_ATTN(D, F32, W) hipLaunchKernelGGL((attn_mfma_kernel<D, F32, kAttnKT, W, false, false>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, cl2, out, ksplit, part, ga, cu_pair)
#define KVSEL_ATTN_I(D, F32) hipLaunchKernelGGL((attn_mfma_kernel<D, F32, kAttnKT, 4, false, true>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, cl2, out, ksplit, part, ga, cu_pair)
#define KVSEL_ATTN_G(D, F32) hipLaunchKernelGGL((attn_mfma_kernel<D, F32, kAttnKT, 4, true, false>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, cl2, out, ksplit, part, ga, 0)
#define KVSEL_ATTN_PPK(D, F32) hipLaunchKernelGGL((attn_pp_kernel<D, F32>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, cl2, out, ksplit, part)
        if (gathering) {
            if (s.d == 128) { if (out_f32) KVSEL_ATTN_G(128, true); else KVSEL_ATTN_G(128, false); }
            else { if (out_f32) KVSEL_ATTN_G(64, true); else KVSEL_ATTN_G(64, false); }
        } else if (inplace) {
            if (s.d == 128) { if (out_f32) KVSEL_ATTN_I(128, true); else KVSEL_ATTN_I(128, false); }
            else { if (out_f32) KVSEL_ATTN_I(64, true); else KVSEL_ATTN_I(64, false); }
        } else if (pp) {
            if (out_f32) KVSEL_ATTN_PPK(128, true); else KVSEL_ATTN_PPK(128, false);
        } else if (s.d == 128) {
            if (out_f32) KVSEL_ATTN(128, true, 4); else KVSEL_ATTN(128, false, 4);
        } else {
            if (out_f32) KVSEL_ATTN(64, true, 4); else KVSEL_ATTN(64, false, 4);
        }
#undef KVSEL_ATTN
#undef KVSEL_ATTN_I
#undef KVSEL_ATTN_G
#undef KVSEL_ATTN_PPK
        if (ksplit > 1) {
            const int64_t rows = int64_t(s.batch) * s.h_q * s.C;
            const dim3 mg(static_cast<unsigned>((rows * (s.d / 4) + 255) / 256));
            if (s.d == 128) {
                if (out_f32) hipLaunchKernelGGL((attn_merge_kernel<128, true>), mg, dim3(256), 0, st, part, rows, ksplit, cl2, out);
                else hipLaunchKernelGGL((attn_merge_kernel<128, false>), mg, dim3(256), 0, st, part, rows, ksplit, cl2, out);
            } else {
                if (out_f32) hipLaunchKernelGGL((attn_merge_kernel<64, true>), mg, dim3(256), 0, st, part, rows, ksplit, cl2, out);
                else hipLaunchKernelGGL((attn_merge_kernel<64, false>), mg, dim3(256), 0, st, part, rows, ksplit, cl2, out);
            }
        }
    } else {
        const int row_blocks = (s.G * s.C + 15) / 16;
        dim3 grid(bgs * row_blocks), block(256);
        const float *qq = (const float*)q, *kk = (const float*)kall, *vv = (const float*)vall;
        if (s.d == 128) {
            if (out_f32) hipLaunchKernelGGL((attn_valu_kernel<128, true>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, scale, out);
            else hipLaunchKernelGGL((attn_valu_kernel<128, false>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, scale, out);
        } else {
            if (out_f32) hipLaunchKernelGGL((attn_valu_kernel<64, true>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, scale, out);
            else hipLaunchKernelGGL((attn_valu_kernel<64, false>), grid, block, 0, st, qq, kk, vv, nsel, nk_pad, s.C, s.G, s.h_kv, row_blocks, scale, out);
        }
    }
    return hipGetLastError();
}

}  // namespace kvsel
