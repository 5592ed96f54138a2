// Offline calibration kernels for gfx950: per (layer, query head, band), the
// centre magnitude M = mean |q_f|, phase phi = arg sum q_f and concentration
// R = | mean q_f / |q_f| | (mean resultant length) of sampled pre-RoPE queries
// (yeyulingfeng.com TriAttention page, section 主要方法: pre-RoPE queries gather
// around fixed non-zero centres; the concentration of a band is its mean
// resultant length).  These are the inputs tri_calib_load folds.
//
// Layout: q [L][n_samples][Hq][d] (one row per sample and head); band f of a row
// is q[f] + i q[f+F].  Pass 1: one-wave workgroup (layer, chunk of kCalibChunk
// samples, block of 64 (head, 8-band) groups); lane t owns one group and loads
// 16 bytes of real parts and the matching 16 bytes of imaginary parts per
// sample (eight bf16 samples in flight), so the wave reads 2 KB of each sample's rows
// contiguously.  Per sample and band it
// forms |q_f| and q_f/|q_f| in fp32 and adds the five sums (|q|, Re, Im, unit
// Re, unit Im) in fp64.  Pass 2 adds the chunks in order (deterministic) and
// forms M, phi, R.
#include "launch.h"

namespace tri {

template <bool BF16>
__device__ __forceinline__ void load8(const uint8_t* p, float (&x)[8]) {
    if constexpr (BF16) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bf16_lo(w[e]);
            x[2 * e + 1] = bf16_hi(w[e]);
        }
    } else {
        const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
}

template <bool BF16>
__global__ __launch_bounds__(64) void k_calib_partial(CalibArgs a) {
    constexpr int ES = BF16 ? 2 : 4;
    const int F = a.head_dim / 2, gpr = F / 8;          // 8-band groups per head
    const int l = blockIdx.x / a.n_chunks, c = blockIdx.x - l * a.n_chunks;
    const int g = blockIdx.y * 64 + threadIdx.x;         // (head, band group)
    if (g >= a.n_q_heads * gpr) return;
    const int h = g / gpr, f0 = (g - h * gpr) * 8;
    const int s0 = c * kCalibChunk, s1 = min(s0 + kCalibChunk, a.n_samples);
    const int64_t rowb = (int64_t)a.head_dim * ES;
    const uint8_t* base = a.q + (((int64_t)l * a.n_samples) * a.n_q_heads + h) * rowb;
    const int64_t sstride = (int64_t)a.n_q_heads * rowb;
    double sm[8], sr[8], si[8], ur[8], ui[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sm[e] = sr[e] = si[e] = ur[e] = ui[e] = 0.0;
    auto add = [&](const float (&re)[8], const float (&im)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float r2 = fmaf(re[e], re[e], im[e] * im[e]);
            const float rs = r2 > 0.0f ? __builtin_amdgcn_rsqf(r2) : 0.0f;
            sm[e] += (double)(r2 * rs);
            sr[e] += (double)re[e];
            si[e] += (double)im[e];
            ur[e] += (double)(re[e] * rs);
            ui[e] += (double)(im[e] * rs);
        }
    };
    int s = s0;
    if constexpr (BF16) {
        // eight samples' raw 16-byte loads in flight, unpacked as they are added
        constexpr int U = 8;
        for (; s + U <= s1; s += U) {
            uint4 rv[U], iv[U];
            const uint8_t* p0 = base + (int64_t)s * sstride;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                rv[u] = *reinterpret_cast<const uint4*>(p0 + u * sstride + f0 * ES);
                iv[u] = *reinterpret_cast<const uint4*>(p0 + u * sstride + (F + f0) * ES);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float re[8], im[8];
                const uint32_t rw[4] = {rv[u].x, rv[u].y, rv[u].z, rv[u].w}, iw[4] = {iv[u].x, iv[u].y, iv[u].z, iv[u].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    re[2 * e] = bf16_lo(rw[e]);
                    re[2 * e + 1] = bf16_hi(rw[e]);
                    im[2 * e] = bf16_lo(iw[e]);
                    im[2 * e + 1] = bf16_hi(iw[e]);
                }
                add(re, im);
            }
        }
    } else {
        for (; s + 4 <= s1; s += 4) {                    // four samples' loads in flight
            float re0[8], im0[8], re1[8], im1[8], re2[8], im2[8], re3[8], im3[8];
            const uint8_t* p0 = base + (int64_t)s * sstride;
            load8<BF16>(p0 + f0 * ES, re0);
            load8<BF16>(p0 + (F + f0) * ES, im0);
            load8<BF16>(p0 + sstride + f0 * ES, re1);
            load8<BF16>(p0 + sstride + (F + f0) * ES, im1);
            load8<BF16>(p0 + 2 * sstride + f0 * ES, re2);
            load8<BF16>(p0 + 2 * sstride + (F + f0) * ES, im2);
            load8<BF16>(p0 + 3 * sstride + f0 * ES, re3);
            load8<BF16>(p0 + 3 * sstride + (F + f0) * ES, im3);
            add(re0, im0);
            add(re1, im1);
            add(re2, im2);
            add(re3, im3);
        }
    }
    for (; s < s1; ++s) {
        float re0[8], im0[8];
        const uint8_t* p0 = base + (int64_t)s * sstride;
        load8<BF16>(p0 + f0 * ES, re0);
        load8<BF16>(p0 + (F + f0) * ES, im0);
        add(re0, im0);
    }
    // partials [L][chunk][Hq][F][5]
    double* out = a.part + ((((int64_t)l * a.n_chunks + c) * a.n_q_heads + h) * F + f0) * 5;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
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
    const int groups = a.n_q_heads * (a.head_dim / 16);
    {
        TimedLaunch tl(KID_CALIB, stream);
        const dim3 grid((unsigned)(a.n_layers * a.n_chunks), (unsigned)((groups + 63) / 64));
        if (bf16) hipLaunchKernelGGL(k_calib_partial<true>, grid, dim3(64), 0, stream, a);
        else hipLaunchKernelGGL(k_calib_partial<false>, grid, dim3(64), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    TimedLaunch tl(KID_CALIB_FINAL, stream);
    const int64_t total = (int64_t)a.n_layers * a.n_q_heads * (a.head_dim / 2);
    hipLaunchKernelGGL(k_calib_final, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tri
