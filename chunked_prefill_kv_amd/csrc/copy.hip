// Compaction, gather and cache append (pure data movement, bit-exact).
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(a): the cache kept
// for a chunk is compacted and handed to a dense attention kernel, and the
// cache grows by one chunk per step.
//
// The attention kernels read one key list per (sequence, KV head): the
// compacted prior keys followed by the chunk's own keys, padded with zeros to
// a multiple of 64 slots.  For bf16 the value rows are written transposed
// ([d][slot]) so that the P.V MFMA reads 8 consecutive slots per lane with a
// single 16-byte LDS load; the transpose happens here, once, through LDS.
#include "launch.h"

namespace kvsel {

constexpr int kTile = 64;   // slots per workgroup

struct PackArgs {
    CacheView cv;
    const int64_t* prior_len;
    int64_t budget;
    const int32_t* idx;
    int64_t idx_stride;
    const char* k_compact;
    const char* v_compact;
    const int32_t* n_sel;
    int n_sel_max;
    bool compact;            // prior keys from k_compact / v_compact (else from the cache through idx)
    const char* k_chunk;
    const char* v_chunk;
    int C, h_kv, nk_pad, tiles, row_bytes;
    char* kall;
    char* vall;
    int32_t* nsel_out;
    bool append;             // also write the chunk's rows into the cache at [T_b, T_b + C)
    bool chunk_hosted;       // tiles in [n_b, n_b + C) were written by the top-B launch
};

// Source rows of slot s (nullptr = zero row).
__device__ __forceinline__ void slot_source(const PackArgs& a, int b, int g, int s, int nsel_b, int64_t T,
                                            const char** kp, const char** vp) {
    const int64_t bg = static_cast<int64_t>(b) * a.h_kv + g;
    if (s < nsel_b) {
        if (a.compact) {
            const int64_t off = (bg * a.n_sel_max + s) * a.row_bytes;
            *kp = a.k_compact + off;
            *vp = a.v_compact + off;
        } else {
            const int64_t pos = (T <= a.budget) ? s : a.idx[bg * a.idx_stride + s];
            const int64_t off = a.cv.row_offset(b, g, pos);
            *kp = a.cv.k + off;
            *vp = a.cv.v + off;
        }
    } else if (s < nsel_b + a.C) {
        const int64_t off = (bg * a.C + (s - nsel_b)) * a.row_bytes;
        *kp = a.k_chunk + off;
        *vp = a.v_chunk + off;
    } else {
        *kp = nullptr;
        *vp = nullptr;
    }
}

__device__ __forceinline__ int seq_nsel(const PackArgs& a, int b, int64_t* T) {
    if (a.compact) {             // caller-supplied count, clamped to the array it indexes
        *T = 0;
        const int v = a.n_sel[b];
        return v < 0 ? 0 : (v > a.n_sel_max ? a.n_sel_max : v);
    }
    *T = a.prior_len[b];
    return static_cast<int>(*T < a.budget ? *T : a.budget);
}

// Natural layout for both K and V (fp32 path): kall/vall [bg][nk_pad][d].
__global__ __launch_bounds__(256) void pack_rows_kernel(PackArgs a) {
    const int bg = blockIdx.x / a.tiles, tile = blockIdx.x % a.tiles;
    const int b = bg / a.h_kv, g = bg % a.h_kv;
    int64_t T;
    const int nsel_b = seq_nsel(a, b, &T);
    if (a.nsel_out && g == 0 && tile == 0 && threadIdx.x == 0) a.nsel_out[b] = nsel_b;
    const int ppr = a.row_bytes / 16;
    for (int p = threadIdx.x; p < kTile * ppr; p += 256) {
        const int r = p / ppr, c = p % ppr;
        const int s = tile * kTile + r;
        const char *kp, *vp;
        slot_source(a, b, g, s, nsel_b, T, &kp, &vp);
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 kv = kp ? reinterpret_cast<const u32x4*>(kp)[c] : z;
        const u32x4 vv = vp ? reinterpret_cast<const u32x4*>(vp)[c] : z;
        const int64_t dst = (static_cast<int64_t>(bg) * a.nk_pad + s) * a.row_bytes;
        reinterpret_cast<u32x4*>(a.kall + dst)[c] = kv;
        reinterpret_cast<u32x4*>(a.vall + dst)[c] = vv;
        if (a.append && s >= nsel_b && s < nsel_b + a.C) {
            const int64_t off = a.cv.row_offset(b, g, T + (s - nsel_b));
            reinterpret_cast<u32x4*>(a.cv.k + off)[c] = kv;
            reinterpret_cast<u32x4*>(a.cv.v + off)[c] = vv;
        }
    }
}

// bf16: kall [bg][nk_pad][D], vall transposed [bg][D][nk_pad].
template <int D>
__global__ __launch_bounds__(256) void pack_bf16_kernel(PackArgs a) {
    constexpr int PPR = D / 8;            // 16-byte pieces per row
    // LDS tile of V rows [slot][D]; piece c of row r sits at piece c ^ ((r / 8) % PPR),
    // so the transposed reads below (8 rows 8 apart, one piece column) hit 8
    // different pieces and the row writes stay a permutation of the row
    __shared__ __attribute__((aligned(16))) uint16_t vt[kTile * D];
    static_assert(PPR >= 8, "the swizzle needs 8 distinct pieces per row");
    const int bg = blockIdx.x / a.tiles, tile = blockIdx.x % a.tiles;
    const int b = bg / a.h_kv, g = bg % a.h_kv;
    int64_t T;
    const int nsel_b = seq_nsel(a, b, &T);
    if (a.nsel_out && g == 0 && tile == 0 && threadIdx.x == 0) a.nsel_out[b] = nsel_b;
    if (a.chunk_hosted && tile * kTile >= nsel_b && tile * kTile < nsel_b + a.C) return;
    constexpr int PPT = kTile * PPR / 256;
    u32x4 kv[PPT], vv[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {              // every load in flight before the first store
        const int p = threadIdx.x + 256 * i;
        const int r = p / PPR, c = p % PPR;
        const char *kp, *vp;
        slot_source(a, b, g, tile * kTile + r, nsel_b, T, &kp, &vp);
        const u32x4 z = {0u, 0u, 0u, 0u};
        kv[i] = kp ? reinterpret_cast<const u32x4*>(kp)[c] : z;
        vv[i] = vp ? reinterpret_cast<const u32x4*>(vp)[c] : z;
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = threadIdx.x + 256 * i;
        const int r = p / PPR, c = p % PPR;
        const int s = tile * kTile + r;
        reinterpret_cast<u32x4*>(a.kall + (static_cast<int64_t>(bg) * a.nk_pad + s) * (D * 2))[c] = kv[i];
        *reinterpret_cast<u32x4*>(&vt[r * D + ((c ^ ((r >> 3) & (PPR - 1))) * 8)]) = vv[i];
        if (a.append && s >= nsel_b && s < nsel_b + a.C) {
            const int64_t off = a.cv.row_offset(b, g, T + (s - nsel_b));
            reinterpret_cast<u32x4*>(a.cv.k + off)[c] = kv[i];
            reinterpret_cast<u32x4*>(a.cv.v + off)[c] = vv[i];
        }
    }
    __syncthreads();
    // transposed write: thread piece = (d, 8-slot group j)
    uint16_t* vout = reinterpret_cast<uint16_t*>(a.vall) + static_cast<int64_t>(bg) * D * a.nk_pad + tile * kTile;
    for (int p = threadIdx.x; p < D * (kTile / 8); p += 256) {
        const int d = p / (kTile / 8), j = p % (kTile / 8);
        const int col = (((d >> 3) ^ j) << 3) + (d & 7);     // rows 8j .. 8j+7 share the swizzle j
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = vt[(8 * j + 2 * i) * D + col];
            const uint32_t hi = vt[(8 * j + 2 * i + 1) * D + col];
            w[i] = lo | (hi << 16);
        }
        *reinterpret_cast<u32x4*>(vout + static_cast<int64_t>(d) * a.nk_pad + 8 * j) = w;
    }
}

// k_sel[bg][r] = cache row idx[bg][r] for r < min(budget, T_b).
__global__ __launch_bounds__(256) void gather_kernel(CacheView cv, const int64_t* __restrict__ prior_len,
                                                     int64_t budget, const int32_t* __restrict__ idx,
                                                     int64_t idx_stride, int h_kv, int tiles, char* k_sel,
                                                     char* v_sel, int64_t out_rows) {
    const int bg = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bg / h_kv, g = bg % h_kv;
    const int64_t T = prior_len[b];
    const int n = static_cast<int>(T < budget ? T : budget);
    const int ppr = cv.row_bytes / 16;
    for (int p = threadIdx.x; p < kTile * ppr; p += 256) {
        const int r = tile * kTile + p / ppr, c = p % ppr;
        if (r >= n) continue;
        const int64_t pos = idx[static_cast<int64_t>(bg) * idx_stride + r];
        const int64_t off = cv.row_offset(b, g, pos);
        const int64_t dst = (static_cast<int64_t>(bg) * out_rows + r) * cv.row_bytes;
        reinterpret_cast<u32x4*>(k_sel + dst)[c] = reinterpret_cast<const u32x4*>(cv.k + off)[c];
        reinterpret_cast<u32x4*>(v_sel + dst)[c] = reinterpret_cast<const u32x4*>(cv.v + off)[c];
    }
}

// Cache append on its own (the gathering attention path packs nothing):
// K/V rows t < C of (b, g) to cache positions T_b + t.
__global__ __launch_bounds__(256) void append_kernel(CacheView cv, const int64_t* __restrict__ prior_len,
                                                     const char* __restrict__ k_chunk, const char* __restrict__ v_chunk,
                                                     int C, int h_kv, int tiles) {
    const int bg = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int b = bg / h_kv, g = bg % h_kv;
    const int64_t T = prior_len[b];
    const int ppr = cv.row_bytes / 16;
    for (int p = threadIdx.x; p < kTile * ppr; p += 256) {
        const int t = tile * kTile + p / ppr, c = p % ppr;
        if (t >= C) continue;
        const int64_t src = (static_cast<int64_t>(bg) * C + t) * cv.row_bytes;
        const int64_t dst = cv.row_offset(b, g, T + t);
        reinterpret_cast<u32x4*>(cv.k + dst)[c] = reinterpret_cast<const u32x4*>(k_chunk + src)[c];
        reinterpret_cast<u32x4*>(cv.v + dst)[c] = reinterpret_cast<const u32x4*>(v_chunk + src)[c];
    }
}

hipError_t launch_append(const SelShape& s, const CacheView& cv, const int64_t* prior_len, const void* k_chunk,
                         const void* v_chunk, hipStream_t st) {
    const int tiles = (s.C + kTile - 1) / kTile;
    hipLaunchKernelGGL(append_kernel, dim3(s.batch * s.h_kv * tiles), dim3(256), 0, st, cv, prior_len,
                       static_cast<const char*>(k_chunk), static_cast<const char*>(v_chunk), s.C, s.h_kv, tiles);
    return hipGetLastError();
}

hipError_t launch_pack(const SelShape& s, const PackSrc& src, const void* k_chunk, const void* v_chunk, int nk_pad,
                       void* kall, void* vall, int32_t* nsel_out, hipStream_t st) {
    PackArgs a;
    if (src.cache) a.cv = *src.cache;
    else a.cv = CacheView{};
    a.prior_len = src.prior_len;
    a.budget = src.budget;
    a.idx = src.idx;
    a.idx_stride = src.idx_stride;
    a.k_compact = static_cast<const char*>(src.k_compact);
    a.v_compact = static_cast<const char*>(src.v_compact);
    a.n_sel = src.n_sel;
    a.n_sel_max = src.n_sel_max;
    a.compact = src.cache == nullptr;    // no cache given: the caller's compacted arrays (possibly empty)
    a.k_chunk = static_cast<const char*>(k_chunk);
    a.v_chunk = static_cast<const char*>(v_chunk);
    a.C = s.C;
    a.h_kv = s.h_kv;
    a.nk_pad = nk_pad;
    a.tiles = nk_pad / kTile;
    a.row_bytes = s.d * s.esz;
    a.kall = static_cast<char*>(kall);
    a.vall = static_cast<char*>(vall);
    a.nsel_out = nsel_out;
    a.append = src.append;
    a.chunk_hosted = src.chunk_hosted && s.esz == 2;
    dim3 grid(s.batch * s.h_kv * a.tiles), block(256);
    if (s.esz == 2) {
        if (s.d == 128) hipLaunchKernelGGL(pack_bf16_kernel<128>, grid, block, 0, st, a);
        else hipLaunchKernelGGL(pack_bf16_kernel<64>, grid, block, 0, st, a);
    } else {
        hipLaunchKernelGGL(pack_rows_kernel, grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const SelShape& s, const CacheView& cv, const int64_t* prior_len, const int32_t* idx,
                         int64_t idx_stride, void* k_sel, void* v_sel, hipStream_t st) {
    const int64_t rows = s.budget < s.t_max ? s.budget : s.t_max;
    const int tiles = static_cast<int>((rows + kTile - 1) / kTile);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3(s.batch * s.h_kv * tiles), dim3(256), 0, st, cv, prior_len, s.budget, idx,
                       idx_stride, s.h_kv, tiles, static_cast<char*>(k_sel), static_cast<char*>(v_sel), s.budget);
    return hipGetLastError();
}

}  // namespace kvsel
