// The chunk's part of the packed bf16 key lists, run by spare workgroups of a
// launch that leaves most compute units idle (the top-B threshold launch).
//
// QuoKA article ("Qualcomm QuoKA", itsolotime.com), Fig. 1(a): the attention
// of a chunk reads the compacted cache followed by the chunk's own keys, and
// the cache grows by the chunk.  Neither the chunk's slots of the key list nor
// the cache append depend on which prior keys the selection keeps: slot n_b + t
// holds chunk row t, where n_b = min(T_b, budget) is the number of kept prior
// keys, known before the selection ends.  So these copies can run beside the
// selection instead of after it; the pack launch that follows writes only the
// kept prior keys (and the tile, if any, that mixes them with chunk rows).
#pragma once

#include "launch.h"

namespace kvsel {

// Work item i = (bg, j): 64-slot tile floor(n_b / 64) + j of KV head bg.  A
// tile that starts at or past n_b and before n_b + C is written whole (chunk K
// rows, chunk V rows transposed, zeros past n_b + C); in every item the chunk
// rows it holds are also appended to the cache at T_b + t.  Every workgroup of
// the host launch with index w takes items w, w + wgs, ...  lds: a 64 x D
// bf16 staging tile (16 KiB at D = 128).
__device__ inline void chunk_pack_wg(const ChunkPack& c, int w, uint16_t* lds) {
    const int D = c.row_bytes / 2, PPR = D / 8;        // bf16 elements and 16-byte pieces per row
    const int jt = (c.C + 63) / 64 + 1;                // tiles a chunk can touch
    const int64_t items = static_cast<int64_t>(c.batch) * c.h_kv * jt;
    const int nt = blockDim.x, tid = threadIdx.x;
    for (int64_t i = w; i < items; i += c.wgs) {       // uniform per workgroup
        const int bg = static_cast<int>(i / jt), j = static_cast<int>(i % jt);
        const int b = bg / c.h_kv, g = bg % c.h_kv;
        const int64_t T = c.prior_len[b];
        const int n = static_cast<int>(T < c.budget ? T : c.budget);
        const int64_t s0l = (static_cast<int64_t>(n) / 64 + j) * 64;
        if (s0l >= static_cast<int64_t>(n) + c.C || s0l >= c.nk_pad) continue;
        const int s0 = static_cast<int>(s0l);
        const bool whole = s0 >= n;                    // no kept prior key in this tile
        for (int p = tid; p < 64 * PPR; p += nt) {
            const int r = p / PPR, cc = p % PPR;
            const int s = s0 + r;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (s >= n && s < n + c.C) {
                const int t = s - n;
                const int64_t src = (static_cast<int64_t>(bg) * c.C + t) * c.row_bytes;
                kv = reinterpret_cast<const u32x4*>(c.k_chunk + src)[cc];
                vv = reinterpret_cast<const u32x4*>(c.v_chunk + src)[cc];
                const int64_t off = c.cv.row_offset(b, g, T + t);
                reinterpret_cast<u32x4*>(c.cv.k + off)[cc] = kv;
                reinterpret_cast<u32x4*>(c.cv.v + off)[cc] = vv;
            }
            if (whole) {
                reinterpret_cast<u32x4*>(c.kall + (static_cast<int64_t>(bg) * c.nk_pad + s) * c.row_bytes)[cc] = kv;
                // piece cc of row r at piece cc ^ (r / 8): the transposed reads
                // below (8 rows of one 8-row group, one piece column) then fall
                // in 8 different pieces
                *reinterpret_cast<u32x4*>(&lds[r * D + ((cc ^ ((r >> 3) & (PPR - 1))) * 8)]) = vv;
            }
        }
        if (whole) {
            __syncthreads();
            uint16_t* vout = reinterpret_cast<uint16_t*>(c.vall) + static_cast<int64_t>(bg) * D * c.nk_pad + s0;
            for (int p = tid; p < D * 8; p += nt) {
                const int d = p / 8, jj = p % 8;
                const int col = (((d >> 3) ^ jj) << 3) + (d & 7);
                u32x4 wv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = lds[(8 * jj + 2 * e) * D + col];
                    const uint32_t hi = lds[(8 * jj + 2 * e + 1) * D + col];
                    wv[e] = lo | (hi << 16);
                }
                *reinterpret_cast<u32x4*>(vout + static_cast<int64_t>(d) * c.nk_pad + 8 * jj) = wv;
            }
            __syncthreads();
        }
    }
}

}  // namespace kvsel
