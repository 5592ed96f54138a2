// Key scoring kernels for gfx950.
//
// The score of a post-RoPE key x for query head h (yeyulingfeng.com TriAttention
// page, section 主要方法: a trigonometric-series term from the offline query
// centre, averaged over geometric future offsets, fused with a norm term whose
// weight rises as the band's concentration falls) is
//     S_h = (1/|O|) sum_o sum_f Re( M e^{i phi} e^{i w_f (t+o)} conj(x_f) ) + sum_f (1-R) M |x_f|.
// The offset average only touches e^{i w_f o}, so per (sequence, head, band) it
// collapses to one complex coefficient C_f = P_f e^{i w_f t} with P_f folded at
// calibration time; the trig term is then the real dot product
//     sum_f (Re C_f x[f] + Im C_f x[f+F]),
// a fixed number of FMAs per key with no transcendental on the key.  The phase
// e^{i w_f t} is evaluated in fp64 (w_0 t reaches 1e5 rad) and rounded once.
#include "launch.h"
#include "stats.h"

namespace tri {

// ------------------------------------------------------------------ phase
__global__ __launch_bounds__(256) void k_phase(PhaseArgs a) {
    const int F = a.head_dim / 2;
    const int64_t total = (int64_t)a.n_layers * a.n_seq * F;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int f = (int)(i % F);
    const int b = (int)((i / F) % a.n_seq);
    const int l = (int)(i / ((int64_t)F * a.n_seq));
    double sn, cs;
    sincos(a.omega[f] * (double)a.t[b], &sn, &cs);
    const double2* P = a.P + ((int64_t)(a.layer0 + l) * a.n_q_heads) * F + f;
    float* out = a.ctab + ((int64_t)(l * a.n_seq + b) * a.n_q_heads) * a.head_dim + f;
    for (int hq = 0; hq < a.n_q_heads; ++hq) {
        const double2 p = P[(int64_t)hq * F];
        out[(int64_t)hq * a.head_dim] = (float)(p.x * cs - p.y * sn);
        out[(int64_t)hq * a.head_dim + F] = (float)(p.x * sn + p.y * cs);
    }
}

hipError_t launch_phase(const PhaseArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.n_layers * a.n_seq * (a.head_dim / 2);
    if (total == 0) return hipSuccess;
    TimedLaunch tl(KID_PHASE, stream);
    hipLaunchKernelGGL(k_phase, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ score
// One workgroup of 256 threads scores `chunk` consecutive keys of one segment,
// one key per lane per iteration.  The per-band coefficients of the G query
// heads (Re C, Im C, (1-R)M) sit in LDS, ordered so that one 16-byte chunk of
// the key's first half (E bands' real parts) and the matching chunk of its
// second half (their imaginary parts) meet 3*E/4 broadcast float4 reads per head.
template <int D, int G, bool BF16>
__global__ __launch_bounds__(256) void k_score(ScoreArgs a) {
    constexpr int F = D / 2;
    constexpr int E = BF16 ? 8 : 4;          // elements per 16-byte chunk
    constexpr int NP = F / E;                // chunks per half row
    constexpr int ROWB = D * (BF16 ? 2 : 4);
    __shared__ float4 coef[NP][G][3][E / 4];
    __shared__ float sh_shift[G];
    __shared__ double red[5 * 2 * G];

    const int tid = threadIdx.x;
    const int s = blockIdx.x / a.n_chunks;
    const int c = blockIdx.x - s * a.n_chunks;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int start = c * a.chunk;
    if (start >= N) return;                  // uniform: whole block exits
    const int cnt = min(a.chunk, N - start);

    {
        const int l = a.shape.layer(s), b = a.shape.seq(s), h = a.shape.head(s);
        const float* cb = a.ctab + ((int64_t)(l * a.shape.n_seq + b) * a.n_q_heads + h * G) * D;
        const float* wb = a.wtab + ((int64_t)l * a.n_q_heads + h * G) * F;
        float* dst = reinterpret_cast<float*>(&coef[0][0][0][0]);
        for (int i = tid; i < NP * G * 3 * E; i += 256) {
            const int e = i % E, comp = (i / E) % 3, g = (i / (3 * E)) % G, q = i / (3 * E * G);
            const int f = q * E + e;
            dst[i] = comp == 0 ? cb[g * D + f] : comp == 1 ? cb[g * D + F + f] : wb[g * F + f];
        }
    }
    __syncthreads();

    float shift[G], sd[G], sd2[G];
#pragma unroll
    for (int g = 0; g < G; ++g) shift[g] = sd[g] = sd2[g] = 0.0f;

    const int iters = (cnt + 255) / 256;
    for (int j = 0; j < iters; ++j) {
        const int local = j * 256 + tid;
        const bool valid = local < cnt;
        const int n = start + local;
        float S[G];
#pragma unroll
        for (int g = 0; g < G; ++g) S[g] = 0.0f;
        if (valid) {
            const uint4* row = reinterpret_cast<const uint4*>(a.kv.k + a.kv.row(s, n) * ROWB);
            uint4 lo[NP], hi[NP];
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                lo[q] = row[q];
                hi[q] = row[NP + q];
            }
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                float re[E], im[E], nr[E];
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    re[e] = chunk_elem<BF16>(lo[q], e);
                    im[e] = chunk_elem<BF16>(hi[q], e);
                    nr[e] = __builtin_amdgcn_sqrtf(fmaf(re[e], re[e], im[e] * im[e]));
                }
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float acc = S[g];
#pragma unroll
                    for (int e4 = 0; e4 < E / 4; ++e4) {
                        const float4 cr = coef[q][g][0][e4];
                        const float4 ci = coef[q][g][1][e4];
                        const float4 w = coef[q][g][2][e4];
                        const int e = 4 * e4;
                        acc = fmaf(cr.x, re[e + 0], acc); acc = fmaf(ci.x, im[e + 0], acc); acc = fmaf(w.x, nr[e + 0], acc);
                        acc = fmaf(cr.y, re[e + 1], acc); acc = fmaf(ci.y, im[e + 1], acc); acc = fmaf(w.y, nr[e + 1], acc);
                        acc = fmaf(cr.z, re[e + 2], acc); acc = fmaf(ci.z, im[e + 2], acc); acc = fmaf(w.z, nr[e + 2], acc);
                        acc = fmaf(cr.w, re[e + 3], acc); acc = fmaf(ci.w, im[e + 3], acc); acc = fmaf(w.w, nr[e + 3], acc);
                    }
                    S[g] = acc;
                }
            }
            if (a.s_raw) {
#pragma unroll
                for (int g = 0; g < G; ++g) a.s_raw[((int64_t)s * G + g) * a.cap + n] = S[g];
            }
            if (a.s_int) {
                float* o = a.s_int + ((int64_t)s * a.cap + n) * G;
                if constexpr (G % 4 == 0) {
#pragma unroll
                    for (int g = 0; g < G; g += 4)
                        *reinterpret_cast<float4*>(o + g) = make_float4(S[g], S[g + 1], S[g + 2], S[g + 3]);
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g) o[g] = S[g];
                }
            }
        }
        if (j == 0) {
            // The chunk's first key shifts the running sums: cancellation stays
            // bounded, and equal scores give exactly zero spread.
            if (tid == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) sh_shift[g] = S[g];
            }
            __syncthreads();
#pragma unroll
            for (int g = 0; g < G; ++g) shift[g] = sh_shift[g];
        }
        if (valid) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float dv = S[g] - shift[g];
                sd[g] += dv;
                sd2[g] = fmaf(dv, dv, sd2[g]);
            }
        }
    }

    double v[2 * G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        v[g] = (double)sd[g];
        v[G + g] = (double)sd2[g];
    }
    block_sum<2 * G, 256>(v, red);
    if (tid < G) {
        const int g = tid;
        const double n = (double)cnt;
        const double m = (double)shift[g] + v[g] / n;
        const double m2 = fmax(v[G + g] - v[g] * v[g] / n, 0.0);
        a.stats[((int64_t)s * a.n_chunks + c) * G + g] = make_double2(m, m2);
    }
}

template <int D, int G, bool BF16>
static void score_kernel(const ScoreArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((k_score<D, G, BF16>), dim3((unsigned)((int64_t)a.n_seg * a.n_chunks)), dim3(256), 0,
                       stream, a);
}

template <int D, int G>
static void score_dtype(const ScoreArgs& a, bool bf16, hipStream_t stream) {
    if (bf16) score_kernel<D, G, true>(a, stream);
    else score_kernel<D, G, false>(a, stream);
}

template <int D>
static bool score_group(const ScoreArgs& a, int group, bool bf16, hipStream_t stream) {
    switch (group) {
        case 1: score_dtype<D, 1>(a, bf16, stream); return true;
        case 2: score_dtype<D, 2>(a, bf16, stream); return true;
        case 4: score_dtype<D, 4>(a, bf16, stream); return true;
        case 8: score_dtype<D, 8>(a, bf16, stream); return true;
        default: return false;
    }
}

hipError_t launch_score(const ScoreArgs& a, int head_dim, int group, bool bf16, hipStream_t stream) {
    if ((int64_t)a.n_seg * a.n_chunks == 0) return hipSuccess;
    TimedLaunch tl(KID_SCORE, stream);
    bool ok = head_dim == 64 ? score_group<64>(a, group, bf16, stream)
            : head_dim == 128 ? score_group<128>(a, group, bf16, stream) : false;
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

// ------------------------------------------------------------------ z-score + max
// One workgroup per (segment, chunk): merge the segment's chunk statistics,
// then write A = max_h z_h for the chunk's keys.
template <int G>
__global__ __launch_bounds__(256) void k_zmax(ZmaxArgs a) {
    __shared__ double scratch[5 * G];
    const int s = blockIdx.x / a.n_chunks;
    const int c = blockIdx.x - s * a.n_chunks;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int start = c * a.chunk;
    if (start >= N) return;
    const ZParams<G> z = merge_stats<G, 256>(a.stats + (int64_t)s * a.n_chunks * G, a.n_chunks, a.chunk, N,
                                             scratch, (c == 0 && a.mu_sigma) ? a.mu_sigma + (int64_t)s * G * 2
                                                                              : nullptr);
    const int end = min(start + a.chunk, N);
    for (int n = start + threadIdx.x; n < end; n += 256) {
        float S[G];
        if (a.s_int) {
            const float* p = a.s_int + ((int64_t)s * a.cap + n) * G;
#pragma unroll
            for (int g = 0; g < G; ++g) S[g] = p[g];
        } else {
#pragma unroll
            for (int g = 0; g < G; ++g) S[g] = a.s_raw[((int64_t)s * G + g) * a.cap + n];
        }
        a.agg[(int64_t)s * a.cap + n] = aggregate<G>(S, z);
    }
}

hipError_t launch_zmax(const ZmaxArgs& a, int group, hipStream_t stream) {
    if ((int64_t)a.n_seg * a.n_chunks == 0) return hipSuccess;
    TimedLaunch tl(KID_ZMAX, stream);
    const dim3 grid((unsigned)((int64_t)a.n_seg * a.n_chunks)), block(256);
    switch (group) {
        case 1: hipLaunchKernelGGL(k_zmax<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(k_zmax<2>, grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(k_zmax<4>, grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL(k_zmax<8>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tri
