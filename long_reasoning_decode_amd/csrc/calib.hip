// Offline calibration kernels for gfx950: per (layer, query head, band), the
// centre magnitude M = mean |q_f|, phase phi = arg sum q_f and concentration
// R = | mean q_f / |q_f| | (mean resultant length) of sampled pre-RoPE queries
// (yeyulingfeng.com TriAttention page, section 主要方法: pre-RoPE queries gather
// around fixed non-zero centres; the concentration of a band is its mean
// resultant length).  These are the inputs tri_calib_load folds.
//
// Layout: q [L][n_samples][Hq][d] (one row per sample and head); band f of a row
// is q[f] + i q[f+F].  Pass 1: one wave per (layer, chunk of chunk_len samples,
// block of 64 (head, 4-band) groups), up to eight such waves of one (layer,
// chunk) in a workgroup; lane t owns one group and loads
// the 4 real parts and the matching 4 imaginary parts per sample, so the wave
// reads 1 KB of each sample's rows contiguously (four heads at head_dim 128).
// Per sample and band it forms |q_f| and q_f/|q_f| in fp32 and adds them to
// the five sums (|q|, Re, Im, unit Re, unit Im): in fp32 over one batch of at
// most eight samples (within about eight ulps of the terms' magnitude), each
// batch then added to fp64 sums, which cuts the fp64-rate work eightfold.
// Four bands per lane keep the sums to 60 registers, so four waves share a
// SIMD, each with eight samples' loads in flight.  Pass 2 adds the chunks in order
// (deterministic) and forms M, phi, R.
#include "launch.h"

namespace tri {

// Waves per pass-1 workgroup: neighbouring blocks of 64 band groups of one
// (layer, chunk) run together, so a sample's rows are read by co-resident waves.
constexpr int kCalibWavesPerGroup = 8;

// Samples are read once: non-temporal loads keep them from displacing cached lines.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint2 ldnt(const uint2* p) {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    return make_uint2(v.x, v.y);
}
__device__ inline float4 ldnt(const float4* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

template <bool BF16>
__global__ __launch_bounds__(64 * kCalibWavesPerGroup) __attribute__((amdgpu_waves_per_eu(BF16 ? 4 : 1))) void k_calib_partial(CalibArgs a) {
    constexpr int ES = BF16 ? 2 : 4, NB = kCalibBands;
    using raw_t = typename std::conditional<BF16, uint2, float4>::type;   // one lane's NB stored values
    const int F = a.head_dim / 2, gpr = F / NB;          // band groups per head
    const int l = blockIdx.x / a.n_chunks, c = blockIdx.x - l * a.n_chunks;
    const int g = blockIdx.y * blockDim.x + threadIdx.x; // (head, band group)
    if (g >= a.n_q_heads * gpr) return;
    const int h = g / gpr, f0 = (g - h * gpr) * NB;
    const int s0 = c * a.chunk_len, s1 = min(s0 + a.chunk_len, a.n_samples);
    const int64_t rowb = (int64_t)a.head_dim * ES;
    const uint8_t* base = a.q + (((int64_t)l * a.n_samples) * a.n_q_heads + h) * rowb;
    const int64_t sstride = (int64_t)a.n_q_heads * rowb;
    double sm[NB], sr[NB], si[NB], ur[NB], ui[NB];
    float bm[NB], br[NB], bi[NB], bu[NB], bv[NB];      // the current batch's sums
#pragma unroll
    for (int e = 0; e < NB; ++e) {
        sm[e] = sr[e] = si[e] = ur[e] = ui[e] = 0.0;
        bm[e] = br[e] = bi[e] = bu[e] = bv[e] = 0.0f;
    }
    auto unpack = [&](const raw_t& v, float (&x)[NB]) {
        if constexpr (BF16) {
            x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        } else {
            x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
        }
    };
    auto add = [&](const raw_t& rv, const raw_t& iv) {
        float re[NB], im[NB];
        unpack(rv, re);
        unpack(iv, im);
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            const float r2 = fmaf(re[e], re[e], im[e] * im[e]);
            const float rs = r2 > 0.0f ? __builtin_amdgcn_rsqf(r2) : 0.0f;
            bm[e] += r2 * rs;
            br[e] += re[e];
            bi[e] += im[e];
            bu[e] += re[e] * rs;
            bv[e] += im[e] * rs;
        }
    };
    auto fold = [&]() {                                  // batch sums -> fp64 sums
#pragma unroll
        for (int e = 0; e < NB; ++e) {
            sm[e] += (double)bm[e];
            sr[e] += (double)br[e];
            si[e] += (double)bi[e];
            ur[e] += (double)bu[e];
            ui[e] += (double)bv[e];
            bm[e] = br[e] = bi[e] = bu[e] = bv[e] = 0.0f;
        }
    };
    const uint8_t* pr = base + (int64_t)f0 * ES;         // the lane's real parts in sample 0
    const uint8_t* pi = base + (int64_t)(F + f0) * ES;   // and imaginary parts
    int s = s0;
    // eight samples' raw loads in flight, unpacked as they are added
    constexpr int U = 8;
    for (; s + U <= s1; s += U) {
        raw_t rv[U], iv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            rv[u] = ldnt(reinterpret_cast<const raw_t*>(pr + (int64_t)(s + u) * sstride));
            iv[u] = ldnt(reinterpret_cast<const raw_t*>(pi + (int64_t)(s + u) * sstride));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) add(rv[u], iv[u]);
        fold();
    }
    for (; s < s1; ++s)
        add(ldnt(reinterpret_cast<const raw_t*>(pr + (int64_t)s * sstride)),
            ldnt(reinterpret_cast<const raw_t*>(pi + (int64_t)s * sstride)));
    fold();
    // partials [L][chunk][Hq][F][5]
    double* out = a.part + ((((int64_t)l * a.n_chunks + c) * a.n_q_heads + h) * F + f0) * 5;
#pragma unroll
    for (int e = 0; e < NB; ++e) {
        out[5 * e] = sm[e];
        out[5 * e + 1] = sr[e];
        out[5 * e + 2] = si[e];
        out[5 * e + 3] = ur[e];
        out[5 * e + 4] = ui[e];
    }
}

__global__ __launch_bounds__(256) void k_calib_final(CalibArgs a) {
    const int F = a.head_dim / 2;
    const int64_t per_l = (int64_t)a.n_q_heads * F;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (l, h, f)
    if (i >= (int64_t)a.n_layers * per_l) return;
    const int l = (int)(i / per_l);
    const int64_t hf = i - l * per_l;
    double t[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    for (int c = 0; c < a.n_chunks; ++c) {
        const double* p = a.part + (((int64_t)l * a.n_chunks + c) * per_l + hf) * 5;
#pragma unroll
        for (int k = 0; k < 5; ++k) t[k] += p[k];
    }
    const double n = (double)a.n_samples;
    a.mag[i] = (float)(t[0] / n);
    a.phase[i] = (t[1] == 0.0 && t[2] == 0.0) ? 0.0f : (float)atan2(t[2], t[1]);
    a.conc[i] = (float)(sqrt(t[3] * t[3] + t[4] * t[4]) / n);
}

hipError_t launch_calibrate(const CalibArgs& a, bool bf16, hipStream_t stream) {
    const int groups = a.n_q_heads * (a.head_dim / 2 / kCalibBands);
    {
        TimedLaunch tl(KID_CALIB, stream);
        const int blocks = (groups + 63) / 64;
        const int waves = blocks < kCalibWavesPerGroup ? blocks : kCalibWavesPerGroup;
        const dim3 grid((unsigned)(a.n_layers * a.n_chunks), (unsigned)((blocks + waves - 1) / waves));
        if (bf16) hipLaunchKernelGGL(k_calib_partial<true>, grid, dim3(64 * waves), 0, stream, a);
        else hipLaunchKernelGGL(k_calib_partial<false>, grid, dim3(64 * waves), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    TimedLaunch tl(KID_CALIB_FINAL, stream);
    const int64_t total = (int64_t)a.n_layers * a.n_q_heads * (a.head_dim / 2);
    hipLaunchKernelGGL(k_calib_final, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tri
