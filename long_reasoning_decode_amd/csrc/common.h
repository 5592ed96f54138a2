// Shared device helpers and launch-argument records for the TriAttention
// pruning kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

constexpr int kWave = 64;

// ---------------------------------------------------------------- stored elements
// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e of a 16-byte chunk holding E stored values (E = 8 bf16 or 4 fp32).
template <bool BF16>
__device__ __forceinline__ float chunk_elem(const uint4& c, int e) {
    const uint32_t w = e < (BF16 ? 2 : 1) ? c.x : e < (BF16 ? 4 : 2) ? c.y : e < (BF16 ? 6 : 3) ? c.z : c.w;
    if (BF16) return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    return __uint_as_float(w);
}

// Orderable 32-bit key of an fp32 score: larger score <=> larger key.
// -0 is folded onto +0 so the two compare equal (IEEE comparison semantics).
__device__ __forceinline__ uint32_t order_key(float a) {
    uint32_t u = __float_as_uint(a);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- cache addressing
// Where slot n of segment s lives, as a row index into k/v (rows of head_dim
// elements) and pos (one int32 per row).
struct CacheView {
    const uint8_t* k;
    const uint8_t* v;
    const int32_t* pos;
    const int32_t* page_table;   // paged only
    int64_t capacity;            // dense: rows per segment
    int32_t page_size;           // paged only (>0 means paged)
    int32_t page_shift;          // log2(page_size) for a power of two, else -1
    int32_t max_pages;
    int32_t row_bytes;           // head_dim * element size

    // Slot n (< 2^31) of a paged segment sits in page-table entry
    // page_entry(n), row page_within(n) of that page.
    __device__ __forceinline__ int page_entry(int n) const {
        return page_shift >= 0 ? n >> page_shift : (int)((uint32_t)n / (uint32_t)page_size);
    }
    __device__ __forceinline__ int page_within(int n) const {
        return page_shift >= 0 ? n & (page_size - 1) : (int)((uint32_t)n % (uint32_t)page_size);
    }
    __device__ __forceinline__ int64_t row(int64_t s, int64_t n) const {
        if (page_size > 0) {
            const int64_t page = page_table[s * max_pages + page_entry((int)n)];
            return page * page_size + page_within((int)n);
        }
        return s * capacity + n;
    }
};

struct CacheOut {
    uint8_t* k;
    uint8_t* v;
    int32_t* pos;
    const int32_t* page_table;
    int64_t capacity;
    int32_t page_size;
    int32_t page_shift;
    int32_t max_pages;

    __device__ __forceinline__ int64_t row(int64_t s, int64_t n) const {
        if (page_size > 0) {
            const uint32_t un = (uint32_t)n;
            const uint32_t e = page_shift >= 0 ? un >> page_shift : un / (uint32_t)page_size;
            const uint32_t w = page_shift >= 0 ? un & (uint32_t)(page_size - 1) : un - e * (uint32_t)page_size;
            const int64_t page = page_table[s * max_pages + e];
            return page * page_size + w;
        }
        return s * capacity + n;
    }
};

// Segment s -> (layer, sequence, kv head) for s = (l * n_seq + b) * Hkv + h.
struct SegShape {
    int32_t n_seq;
    int32_t n_kv_heads;
    __device__ __forceinline__ int layer(int s) const { return s / (n_seq * n_kv_heads); }
    __device__ __forceinline__ int seq(int s) const { return (s / n_kv_heads) % n_seq; }
    __device__ __forceinline__ int head(int s) const { return s % n_kv_heads; }
};

// ---------------------------------------------------------------- matrix cores and LDS DMA
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));    // operand type of the 16x16x16 bf16 MFMA
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8): wait until at most n vector-memory operations (LDS-DMA
// loads included) are outstanding, or for all LDS operations.
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitVm0 = wait_vm(0);
constexpr int kWaitLgkm0 = 0xC07F;

// ---------------------------------------------------------------- wave reductions
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m, kWave));
    return x;
}
__device__ __forceinline__ float wave_sumf(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, kWave);
    return x;
}

// Inclusive prefix sum of a uint32 across the wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    return x;
}

}  // namespace tri
