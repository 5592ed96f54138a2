// Block-level merge of per-chunk score statistics into the per-head
// population mean and standard deviation of a segment, and the z-score /
// GQA-max aggregation built on them.
#pragma once

#include "common.h"

namespace tri {

// Sum of G doubles over a block of NT threads; the result is returned to
// every thread.  `scratch` holds (NT/64 + 1) * G doubles of LDS.
template <int G, int NT>
__device__ __forceinline__ void block_sum(double (&v)[G], double* scratch) {
    constexpr int NW = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = wave_sum(v[g]);
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) scratch[w * G + g] = v[g];
    }
    __syncthreads();
    if ((int)threadIdx.x < G) {
        double t = 0.0;
        for (int i = 0; i < NW; ++i) t += scratch[i * G + threadIdx.x];
        scratch[NW * G + threadIdx.x] = t;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) v[g] = scratch[NW * G + g];
    __syncthreads();
}

// Per-head z-score parameters of one segment, in the form the aggregation uses:
// z = ((S - mu_hi) - mu_lo) * inv_sigma, inv_sigma = 0 when sigma = 0.
template <int G>
struct ZParams {
    float mu_hi[G], mu_lo[G], inv[G];
};

// Chunk c of a segment of N keys holds n_c = clamp(N - c*chunk, 0, chunk)
// keys with mean m_c and sum of squared deviations M2_c.  The segment's
//   mean = sum n_c m_c / N,   M2 = sum (M2_c + n_c (m_c - mean)^2),
// both as plain sums (no per-merge division), sigma = sqrt(M2 / N).
// When mu_sigma is given, threads 0..G-1 also store (mu_h, sigma_h) there as fp32.
template <int G, int NT>
__device__ __forceinline__ ZParams<G> merge_stats(const double2* st, int n_chunks, int chunk, int N,
                                                  double* scratch, float* mu_sigma = nullptr) {
    double acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.0;
    for (int c = threadIdx.x; c < n_chunks; c += NT) {
        const int nc = min(max(N - c * chunk, 0), chunk);
        if (nc > 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] += (double)nc * st[c * G + g].x;
        }
    }
    block_sum<G, NT>(acc, scratch);
    double mean[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mean[g] = N > 0 ? acc[g] / (double)N : 0.0;
        acc[g] = 0.0;
    }
    for (int c = threadIdx.x; c < n_chunks; c += NT) {
        const int nc = min(max(N - c * chunk, 0), chunk);
        if (nc > 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const double2 v = st[c * G + g];
                const double dm = v.x - mean[g];
                acc[g] += v.y + (double)nc * dm * dm;
            }
        }
    }
    block_sum<G, NT>(acc, scratch);
    ZParams<G> z;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const double sig = N > 0 ? sqrt(acc[g] / (double)N) : 0.0;
        if (mu_sigma && (int)threadIdx.x == g) {
            mu_sigma[2 * g] = (float)mean[g];
            mu_sigma[2 * g + 1] = (float)sig;
        }
        z.mu_hi[g] = (float)mean[g];
        z.mu_lo[g] = (float)(mean[g] - (double)z.mu_hi[g]);
        z.inv[g] = sig > 0.0 ? (float)(1.0 / sig) : 0.0f;
    }
    return z;
}

// The same merge by one wave, for at most 64 chunks (lane c holds chunk c):
// no barrier and no LDS, so each wave of a block can run it by itself.  Its
// sums are exactly those of merge_stats: there, too, every chunk sits in wave
// 0 (thread c), the butterfly is the same, and the other waves add zeros.
template <int G>
__device__ __forceinline__ ZParams<G> merge_stats_wave(const double2* st, int n_chunks, int chunk, int N) {
    const int c = threadIdx.x & (kWave - 1);
    const int nc = c < n_chunks ? min(max(N - c * chunk, 0), chunk) : 0;
    ZParams<G> z;
#pragma unroll
    for (int g = 0; g < G; ++g) {                 // one head at a time: few registers live
        const double2 v = nc > 0 ? st[c * G + g] : make_double2(0.0, 0.0);
        double acc = 0.0;
        if (nc > 0) acc += (double)nc * v.x;
        acc = wave_sum(acc);
        const double mean = N > 0 ? acc / (double)N : 0.0;
        acc = 0.0;
        if (nc > 0) {
            const double dm = v.x - mean;
            acc += v.y + (double)nc * dm * dm;
        }
        acc = wave_sum(acc);
        const double sig = N > 0 ? sqrt(acc / (double)N) : 0.0;
        z.mu_hi[g] = (float)mean;
        z.mu_lo[g] = (float)(mean - (double)z.mu_hi[g]);
        z.inv[g] = sig > 0.0 ? (float)(1.0 / sig) : 0.0f;
    }
    return z;
}

// A = max over the G query heads of their z-scores.
template <int G>
__device__ __forceinline__ float aggregate(const float (&S)[G], const ZParams<G>& z) {
    float a = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < G; ++g) a = fmaxf(a, ((S[g] - z.mu_hi[g]) - z.mu_lo[g]) * z.inv[g]);
    return a;
}

}  // namespace tri
