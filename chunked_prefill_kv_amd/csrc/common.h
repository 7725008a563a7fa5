// Shared device helpers for the kvsel kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvsel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Word 3 of a raw buffer resource (untyped loads/stores, 32-bit data format).
constexpr int kBufferFormat = 0x00020000;

// ---------------------------------------------------------------- element access

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950: v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xFFFFu);
}

// ---------------------------------------------------------------- cache addressing

// Where row `pos` of sequence b, KV head g lives (contiguous or paged cache).
struct CacheView {
    char* k;                  // base pointers (bytes)
    char* v;
    int64_t capacity;         // contiguous: rows per (b, g); paged: number of blocks
    int32_t block_size;       // 0 = contiguous
    int32_t max_blocks;
    const int32_t* block_table;
    int32_t h_kv;
    int32_t row_bytes;        // d * element bytes

    // row number (row_offset / row_bytes)
    __device__ __forceinline__ int64_t row_index(int b, int g, int64_t pos) const {
        if (block_size == 0) return (static_cast<int64_t>(b) * h_kv + g) * capacity + pos;
        const uint32_t p = static_cast<uint32_t>(pos), bs = static_cast<uint32_t>(block_size);   // pos < 2^30
        const int64_t blk = block_table[static_cast<int64_t>(b) * max_blocks + p / bs];
        return (blk * h_kv + g) * block_size + p % bs;
    }
    __device__ __forceinline__ int64_t row_offset(int b, int g, int64_t pos) const {
        if (block_size == 0) {
            return ((static_cast<int64_t>(b) * h_kv + g) * capacity + pos) * row_bytes;
        }
        const uint32_t p = static_cast<uint32_t>(pos), bs = static_cast<uint32_t>(block_size);   // pos < 2^30
        const int64_t blk = block_table[static_cast<int64_t>(b) * max_blocks + p / bs];
        return ((blk * h_kv + g) * block_size + p % bs) * static_cast<int64_t>(row_bytes);
    }
};

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, kWave);
    return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, kWave));
    return x;
}

// Sum over the 16 lanes of each DPP row (lanes 16r .. 16r+15); every lane of
// the row receives the total.  Rotations by 8 and 4 inside the row, then swaps
// of lane pairs 2 and 1 apart inside each group of four.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x = dpp_add<0x128>(x);     // row_ror:8
    x = dpp_add<0x124>(x);     // row_ror:4
    x = dpp_add<0x4E>(x);      // quad_perm [2,3,0,1]
    return dpp_add<0xB1>(x);   // quad_perm [1,0,3,2]
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 is
// folded onto +0 first so that equal values compare equal.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The 8 workgroup-dispatch queues of MI355X place consecutive workgroup ids on
// consecutive XCDs (each with its own L2).  remap so that the workgroups one
// XCD receives are consecutive slots (sharing the same head's data).
constexpr int kXcds = 8;   // MI355X: 8 XCDs, workgroups dealt to them round-robin
__device__ __forceinline__ int xcd_slot(int linear, int n) {
    if (n % kXcds != 0) return linear;
    return (linear % kXcds) * (n / kXcds) + linear / kXcds;
}

}  // namespace kvsel
