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
// One thread per (layer, sequence, query head, band): C = P e^{i w_f t} in
// fp64, rounded once to fp32.  The same threads (grid-stride) clear the words
// a later kernel of the pass accumulates into.
__global__ __launch_bounds__(256) void k_phase(PhaseArgs a) {
    const int F = a.head_dim / 2;
    const int64_t total = (int64_t)a.n_layers * a.n_seq * a.n_q_heads * F;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i == 0 && a.fb_reset) *a.fb_reset = 0;
    for (int64_t z = i; z < a.zero_words; z += (int64_t)gridDim.x * blockDim.x) a.zero[z] = 0u;
    if (i >= total) return;
    const int f = (int)(i % F);
    const int64_t r = i / F;                       // (l, b, hq)
    const int hq = (int)(r % a.n_q_heads);
    const int b = (int)((r / a.n_q_heads) % a.n_seq);
    const int l = (int)(r / ((int64_t)a.n_q_heads * a.n_seq));
    double sn, cs;
    sincos(a.omega[f] * (double)a.t[b], &sn, &cs);
    const double2 p = a.P[((int64_t)(a.layer0 + l) * a.n_q_heads + hq) * F + f];
    float* out = a.ctab + r * a.head_dim + f;
    out[0] = (float)(p.x * cs - p.y * sn);
    out[F] = (float)(p.x * sn + p.y * cs);
}

hipError_t launch_phase(const PhaseArgs& a, hipStream_t stream) {
    const int64_t total = (int64_t)a.n_layers * a.n_seq * a.n_q_heads * (a.head_dim / 2);
    const int64_t zb = (a.zero_words + 1023) / 1024;           // four words per thread
    int64_t blocks = (total + 255) / 256;
    if (zb > blocks) blocks = zb < 4096 ? zb : 4096;
    if (blocks == 0) return hipSuccess;
    TimedLaunch tl(KID_PHASE, stream);
    hipLaunchKernelGGL(k_phase, dim3((unsigned)blocks), dim3(256), 0, stream, a);
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

// ------------------------------------------------------------------ score (bf16, MFMA)
// The same score as a skinny dense contraction on the matrix cores.  Per 16-key
// tile, with k-steps of 32 along the row:
//   S[key][col] += K[key][dims] . Bc[dims][col]        (trig: head_dim/32 steps)
//   S[key][col] += |K|[key][bands] . Bw[bands][col]    (norm: F/32 steps, |K| as a
//                                                       bf16 hi + lo pair)
// Columns are (split q, head h): each fp32 coefficient is carried as the sum of
// three bf16 values (hi, mid, lo), so the bf16 products keep fp32-level
// accuracy; the three partial sums of a head are added afterwards.  The key
// rows feed the A operand straight from HBM (16 rows x 64 contiguous bytes per
// load); the coefficient fragments are loop-invariant registers.  |k_f| needs
// the band's real and imaginary parts, which sit in the same lane and slot of
// two A fragments (dims f and f + F), so the norm operand is built in registers.

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Component q (0: hi, 1: mid, 2: lo) of the three-way bf16 split of x
// (all three parts are formed and one is selected: no branch on q).
__device__ __forceinline__ uint32_t bf16_split3(float x, int q) {
    const uint32_t h = bf16_rne_bits(x);
    const float r1 = x - __uint_as_float(h << 16);
    const uint32_t m = bf16_rne_bits(r1);
    const uint32_t l = bf16_rne_bits(r1 - __uint_as_float(m << 16));
    return q == 0 ? h : (q == 1 ? m : l);
}

// Chan merge of (n, mean, M2) summaries.
__device__ __forceinline__ void chan_merge(double& n, double& m, double& m2, double nb, double mb, double m2b) {
    if (nb == 0.0) return;
    if (n == 0.0) {
        n = nb; m = mb; m2 = m2b;
        return;
    }
    const double nt = n + nb, dl = mb - m;
    m += dl * (nb / nt);
    m2 += m2b + dl * dl * (n * nb / nt);
    n = nt;
}



// B fragments of one segment's G query heads for v_mfma_f32_16x16x32_bf16:
// column 16t + (lane % 16) is (split q, head h) = ((16t + lane%16) / G, % G),
// k-slot (lane / 16, e); trig fragments cover the head_dim row elements,
// norm fragments the F bands.  Coefficients are carried as three bf16 parts.
template <int D, int G>
__device__ __forceinline__ void mfma_coef_fragments(const float* ctab, const float* wtab, const SegShape& shape,
                                                    int n_q_heads, int s, bf16x8_t (&bt)[D / 32][(3 * G + 15) / 16],
                                                    bf16x8_t (&bn)[D / 64][(3 * G + 15) / 16]) {
    constexpr int F = D / 2, TS = D / 32, NS = F / 32, NCOL = 3 * G, NT = (NCOL + 15) / 16;
    const int lane = threadIdx.x & 63, row = lane & 15, grp = lane >> 4;
    const int l = shape.layer(s), b = shape.seq(s), hk = shape.head(s);
    const float* cb = ctab + ((int64_t)(l * shape.n_seq + b) * n_q_heads + hk * G) * D;
    const float* wb = wtab + ((int64_t)l * n_q_heads + hk * G) * F;
    // All of a column's coefficients are loaded first (8 consecutive floats per
    // fragment, two 16-byte loads; h < G, so unused columns read valid rows and
    // are zeroed afterwards), then split: one wait instead of one per element.
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int jg = 16 * t + row;
        const bool used = jg < NCOL;
        const int q = jg / G, h = jg % G;
        float4 cv[TS][2], wv[NS][2];
#pragma unroll
        for (int st = 0; st < TS; ++st)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                cv[st][x] = *reinterpret_cast<const float4*>(cb + h * D + 32 * st + 8 * grp + 4 * x);
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int x = 0; x < 2; ++x)
                wv[st][x] = *reinterpret_cast<const float4*>(wb + h * F + 32 * st + 8 * grp + 4 * x);
        auto pack = [&](const float4 (&v)[2]) {
            const float e[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
            uint32_t w[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
                w[e2] = used ? (bf16_split3(e[2 * e2], q) | (bf16_split3(e[2 * e2 + 1], q) << 16)) : 0u;
            return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        };
#pragma unroll
        for (int st = 0; st < TS; ++st) bt[st][t] = pack(cv[st]);
#pragma unroll
        for (int st = 0; st < NS; ++st) bn[st][t] = pack(wv[st]);
    }
}

// Scores of one 16-key tile.  av[st] is lane (grp, row)'s A fragment: the
// 16-byte chunk 4*st + grp of key row `row`.  On return, lanes with
// row < G hold S_row of keys 4*grp + r in S4[r].
template <int D, int G>
__device__ __forceinline__ void mfma_tile_scores(const uint4 (&av)[D / 32],
                                                 const bf16x8_t (&bt)[D / 32][(3 * G + 15) / 16],
                                                 const bf16x8_t (&bn)[D / 64][(3 * G + 15) / 16], float (&S4)[4]) {
    constexpr int TS = D / 32, NS = D / 64, NT = (3 * G + 15) / 16;
    const int lane = threadIdx.x & 63, row = lane & 15;
    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int st = 0; st < TS; ++st)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[st]), bt[st][t], acc[t], 0,
                                                             0, 0);
    // |k_f|: the band's real and imaginary parts sit in the same lane and slot
    // of fragments st and st + NS; fed as a bf16 hi + lo pair
#pragma unroll
    for (int st = 0; st < NS; ++st) {
        const uint4 rv = av[st], iv = av[st + NS];
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w}, iw[4] = {iv.x, iv.y, iv.z, iv.w};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float r0 = bf16_lo(rw[e2]), r1 = bf16_hi(rw[e2]);
            const float i0 = bf16_lo(iw[e2]), i1 = bf16_hi(iw[e2]);
            const float m0 = __builtin_amdgcn_sqrtf(fmaf(r0, r0, i0 * i0));
            const float m1 = __builtin_amdgcn_sqrtf(fmaf(r1, r1, i1 * i1));
            const bf16x2_t hp = __builtin_convertvector(f32x2_t{m0, m1}, bf16x2_t);
            const uint32_t hb = __builtin_bit_cast(uint32_t, hp);
            const f32x2_t res = {m0 - bf16_lo(hb), m1 - bf16_hi(hb)};
            hw[e2] = hb;
            lw[e2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(res, bf16x2_t));
        }
        const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        const bf16x8_t al = __builtin_bit_cast(bf16x8_t, make_uint4(lw[0], lw[1], lw[2], lw[3]));
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bn[st][t], acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bn[st][t], acc[t], 0, 0, 0);
        }
    }
    // lane (grp, row) holds rows 4*grp + r of column row; add the three split
    // columns of head `row`
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = 0.0f;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const int t = (q * G) / 16;
            const int src = (lane & 48) | ((q * G + row) & 15);
            v += __shfl(acc[t][r], src, kWave);
        }
        S4[r] = v;
    }
}

constexpr int kMaxChunkBlocks = 2048 / 32;   // 32-key mask words per chunk
// LDS per scoring workgroup that still lets four of them share a CU.
constexpr int kScoreLds = 40960;

// Scores chunk c of segment s.  CAND = false: every key's G scores go to the
// interleaved scratch (and/or the head-major output).  CAND = true: only the
// (key, head) pairs with S_h >= L_h (the segment's thresholds) are kept: the
// score S_h, key-major then head-major, in a per-wave list, plus G mask words
// per 32-key block (word h: which keys of the block passed head h).  Wave w of
// a chunk scores blocks w, w+4, w+8, ..., so its list holds at most
// G * wave_keys(w, cnt) floats; the four lists sit back to back in the scratch
// rows of the chunk's keys.  The chunk statistics always cover every key.
template <int D, int G, bool CAND, bool PAGED>
__device__ __forceinline__ void score_chunk_mfma(const ScoreArgs& a, const int s, const int c) {
    constexpr int F = D / 2;
    constexpr int TS = D / 32;               // trig k-steps = 16-byte A fragments per key
    constexpr int NS = F / 32;               // norm k-steps
    constexpr int NCOL = 3 * G;              // (split, head) columns
    constexpr int NT = (NCOL + 15) / 16;     // 16-column MFMA tiles
    constexpr int UT = 2;                    // 16-key tiles per wave stage
    constexpr int ROWB = D * 2;
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per key row
    constexpr int SKEYS = 16 * UT;           // keys per wave stage
    constexpr int NDMA = SKEYS * CPR / 64;   // LDS-DMA instructions per stage
    // Each wave stages its keys through its own LDS region: global_load_lds
    // writes 64 x 16 bytes per instruction (4 whole 256-byte rows for head_dim
    // 128), with the non-temporal hint; chunk lc of stage key k sits at chunk
    // position lc ^ (k mod CPR) so the fragment reads below are conflict-free.
    static_assert(SKEYS == 32, "one stage is one 32-key mask block");
    // Candidate mode: each wave keeps its kept scores in LDS and writes them
    // out only when the buffer cannot stage another 32 keys, and at the end of
    // the chunk; the buffer takes whatever LDS four workgroups per CU leave
    // (1824 floats per wave for head_dim 128, G = 4).  Every record store
    // mixed into the key stream slows it on some page placements.
    constexpr int FIXED = (int)sizeof(uint4) * 4 * SKEYS * CPR + 4 * G * 3 * 8 + kMaxChunkBlocks * G * 4;
    constexpr int CAPF0 = (kScoreLds - FIXED) / (4 * 4);
    constexpr int CAPF = CAND ? (CAPF0 > 2 * SKEYS * G ? CAPF0 : 2 * SKEYS * G) : 1;   // floats per wave buffer
    __shared__ uint4 stage[4][SKEYS * CPR];
    __shared__ float tileS[CAND ? 1 : 4][CAND ? 1 : 16 * G];      // one tile's scores, key-major
    __shared__ double part[4][G][3];
    __shared__ float cbuf[CAND ? 4 : 1][CAND ? CAPF : 1];
    __shared__ uint32_t maskbuf[CAND ? kMaxChunkBlocks * G : 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = lane & 15, grp = lane >> 4;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int start = c * a.chunk;
    if (start >= N) return;
    const int cnt = min(a.chunk, N - start);

    float thr[CAND ? G : 1];
    int nb = 0, nw = 0;            // floats staged in LDS / already written (wave-uniform)
    float* list = nullptr;
    if constexpr (CAND) {
#pragma unroll
        for (int g = 0; g < G; ++g) thr[g] = a.thr[(int64_t)s * G + g];
        list = a.s_int + ((int64_t)s * a.cap + start + wave_list_base(wave, cnt)) * G;
    }

    bf16x8_t bt[TS][NT], bn[NS][NT];           // loop-invariant B fragments, loaded below

    // per-lane running statistics for head `row` (lanes row < G), shifted by
    // the lane's first score
    float shift = 0.0f, sd = 0.0f, sd2 = 0.0f;
    int cntl = 0;
    const int n_tiles = (cnt + 15) / 16;
    uint4* region = &stage[wave][0];
    // Paged caches: lane l holds the page of key l of the next stage to issue
    // (loaded one stage ahead, so the page-table read completes under the
    // current stage instead of delaying the next stage's DMA); each DMA lane
    // takes its row's page from that lane.
    int pg = 0;
    auto fetch_pages = [&](int tb) {
        if constexpr (PAGED) {
            const int key = min(tb * 16 + (lane & (SKEYS - 1)), cnt - 1);
            pg = a.kv.page_table[(int64_t)s * a.kv.max_pages + a.kv.page_entry(start + key)];
        }
    };
    // DMA of the stage whose first tile is tb: instruction i, lane l fills
    // chunk position P = 64 i + l, i.e. key P / CPR, chunk (P mod CPR) ^ key.
    auto issue_stage = [&](int tb) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int P = 64 * i + lane;
            const int kl = P / CPR;
            const int lc = (P % CPR) ^ (kl % CPR);
            const int key = min(tb * 16 + kl, cnt - 1);            // clamped: tail rows re-read a valid row
            int64_t r;
            if constexpr (PAGED) r = (int64_t)__shfl(pg, kl, kWave) * a.kv.page_size + a.kv.page_within(start + key);
            else r = (int64_t)s * a.kv.capacity + start + key;
            const uint8_t* src = a.kv.k + r * ROWB + 16 * lc;
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(region + 64 * i), 16, 0, 2 /* nt */);
        }
    };
    // all nb buffered floats -> list[nw ..]
    auto flush_records = [&]() {
        if constexpr (CAND) {
            for (int i = lane; i < nb; i += kWave) list[nw + i] = cbuf[wave][i];
            nw += nb;
            nb = 0;
            __builtin_amdgcn_wave_barrier();
        }
    };
    if (wave * UT < n_tiles) {
        fetch_pages(wave * UT);
        issue_stage(wave * UT);
        fetch_pages(wave * UT + 4 * UT);
    }
    // the coefficient loads follow the first stage's DMA, so the two latencies overlap
    mfma_coef_fragments<D, G>(a.ctab, a.wtab, a.shape, a.n_q_heads, s, bt, bn);
    for (int tb = wave * UT; tb < n_tiles; tb += 4 * UT) {
        uint4 av[UT][TS];
            __builtin_amdgcn_s_waitcnt(kWaitVm0);                      // this stage's DMA has landed
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < UT; ++u) {
            const int kl = 16 * u + row;
#pragma unroll
            for (int st = 0; st < TS; ++st) av[u][st] = region[kl * CPR + ((4 * st + grp) ^ (kl % CPR))];
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                    // fragments are in registers
        __builtin_amdgcn_wave_barrier();
        if (tb + 4 * UT < n_tiles) {                               // next stage loads under this compute
            issue_stage(tb + 4 * UT);
            fetch_pages(tb + 8 * UT);
        }
        if constexpr (CAND) {
            if (nb + SKEYS * G > CAPF) flush_records();              // no room to stage this stage's scores
        }
#pragma unroll
        for (int u = 0; u < UT; ++u) {
            if (tb + u >= n_tiles) break;
            float S4[4];
            mfma_tile_scores<D, G>(av[u], bt, bn, S4);
            const int tile0 = (tb + u) * 16;
            if (row < G) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = tile0 + 4 * grp + r;
                    // candidate mode: the stage's 32 keys are staged after the kept records
                    if constexpr (CAND) cbuf[wave][nb + (16 * u + 4 * grp + r) * G + row] = S4[r];
                    else tileS[wave][(4 * grp + r) * G + row] = S4[r];
                    if (key < cnt) {
                        if (cntl == 0) shift = S4[r];
                        const float dv = S4[r] - shift;
                        sd += dv;
                        sd2 = fmaf(dv, dv, sd2);
                        ++cntl;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
            // Scores leave through LDS so every store instruction writes whole
            // lines: key-major scratch (lanes 0..15 store one key's G scores,
            // 16 keys x 4G bytes contiguous) or head-major output (lane (h, k)
            // stores S_h(k)).  Scattered 4-byte stores mixed into the key stream
            // made the stream's speed depend on where the scratch was allocated.
            if (!CAND && a.s_int && lane < 16 && tile0 + lane < cnt) {
                float* o = a.s_int + ((int64_t)s * a.cap + start + tile0 + lane) * G;
                if constexpr (G % 4 == 0) {
#pragma unroll
                    for (int g = 0; g < G; g += 4)
                        *reinterpret_cast<float4*>(o + g) = *reinterpret_cast<const float4*>(&tileS[wave][lane * G + g]);
                } else {
#pragma unroll
                    for (int g = 0; g < G; ++g) o[g] = tileS[wave][lane * G + g];
                }
            }
            if (!CAND && a.s_raw) {
                for (int i = lane; i < 16 * G; i += kWave) {
                    const int h = i / 16, k = i % 16;
                    if (tile0 + k < cnt) a.s_raw[((int64_t)s * G + h) * a.cap + start + tile0 + k] = tileS[wave][k * G + h];
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        if constexpr (CAND) {
            // lanes 0..31: which heads of staged key tb*16 + lane pass (S_h >= L_h)?
            // The passing scores move down onto the kept floats (reads before
            // writes; a key's floats never pass a later key's record).
            const int key0 = tb * 16;
            float rec[G];
            uint32_t hb = 0u;
            if (lane < 32) {
#pragma unroll
                for (int g = 0; g < G; ++g) rec[g] = cbuf[wave][nb + lane * G + g];
                if (key0 + lane < cnt) {
#pragma unroll
                    for (int g = 0; g < G; ++g) hb |= (rec[g] >= thr[g] ? 1u : 0u) << g;
                }
            }
            const uint32_t below = (1u << (lane & 31)) - 1u;
            int off = 0, tot = 0;
            uint32_t mwd[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                mwd[g] = (uint32_t)__ballot((hb >> g) & 1u);
                off += __popc(mwd[g] & below);
                tot += __popc(mwd[g]);
            }
            __builtin_amdgcn_wave_barrier();
            if (hb) {
                int p = nb + off;
#pragma unroll
                for (int g = 0; g < G; ++g)
                    if ((hb >> g) & 1u) cbuf[wave][p++] = rec[g];
            }
            nb += tot;
            if (lane == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) maskbuf[(tb / UT) * G + g] = mwd[g];
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
    if constexpr (CAND) {
        if (nb > 0) flush_records();
    }

    // merge the lane summaries of each head: across the 4 lane groups, then waves
    double n = (double)cntl, m = 0.0, m2 = 0.0;
    if (cntl > 0) {
        m = (double)shift + (double)sd / n;
        m2 = fmax((double)sd2 - (double)sd * (double)sd / n, 0.0);
    }
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
        const double nb = __shfl_xor(n, x, kWave), mb = __shfl_xor(m, x, kWave), m2b = __shfl_xor(m2, x, kWave);
        chan_merge(n, m, m2, nb, mb, m2b);
    }
    if (lane < G) {
        part[wave][lane][0] = n;
        part[wave][lane][1] = m;
        part[wave][lane][2] = m2;
    }
    __syncthreads();
    if (tid < G) {
        double tn = 0.0, tm = 0.0, tm2 = 0.0;
        for (int w = 0; w < 4; ++w) chan_merge(tn, tm, tm2, part[w][tid][0], part[w][tid][1], part[w][tid][2]);
        a.stats[((int64_t)s * a.n_chunks + c) * G + tid] = make_double2(tm, tm2);
    }
    if constexpr (CAND) {
        for (int i = tid; i < (cnt + 31) / 32 * G; i += 256)
            a.masks[((int64_t)s * a.mask_stride + start / 32) * G + i] = maskbuf[i];
    }
}

// (at most 128 VGPRs for head_dim 128 with G <= 4, so four workgroups share a CU)
// Paged pools are sized for the longest segment, so many of a ragged batch's
// (segment, chunk) workgroups have no keys.  There the grid runs chunk-major
// (chunk 0 of every segment first): the workgroups with keys are dispatched
// first and the empty ones, which return at once, come last.
template <int D, int G, bool CAND, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(G <= 4 ? 4 : 1))) void k_score_mfma(ScoreArgs a) {
    if constexpr (PAGED) {
        const int c = blockIdx.x / a.n_seg;
        score_chunk_mfma<D, G, CAND, PAGED>(a, blockIdx.x - c * a.n_seg, c);
    } else {
        const int s = blockIdx.x / a.n_chunks;
        score_chunk_mfma<D, G, CAND, PAGED>(a, s, blockIdx.x - s * a.n_chunks);
    }
}

// Full scoring of the segments whose candidate pass failed its certificate:
// work items (listed segment, chunk), grid-strided.
template <int D, int G, bool PAGED>
__global__ __launch_bounds__(256) void k_score_mfma_fallback(ScoreArgs a) {
    const int64_t items = (int64_t)(*a.fb_count) * a.n_chunks;
    for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
        __syncthreads();                      // LDS of the previous item is no longer read
        const int s = a.fb_list[it / a.n_chunks];
        score_chunk_mfma<D, G, false, PAGED>(a, s, (int)(it % a.n_chunks));
    }
}

// ------------------------------------------------------------------ candidate thresholds
// One workgroup per segment scores an evenly spaced sample of kSample keys in
// fp32, estimates each head's mean and spread and the aggregated score at rank
// (kCandNum / kCandDen) * B/N of the sample, and stores per-head score thresholds
// L_h = mean_h + tau * spread_h.  Keys with no S_h >= L_h are left out of the
// candidate list; the select kernel then proves with the exact statistics that
// none of them can be among the B kept (else the segment is redone in full).
// The thresholds only decide how much work is skipped, never the result.
constexpr int kSample = 256;
static_assert(kSample <= 256, "sample index fits the low 8 bits of a rank key");
// rank 2.5 B/N: about 2.5 B candidates per segment, a margin of about 3.4
// threshold errors to the cut (rank 2 B/N left 19 of the main workload's 4608
// segments to the fallback; 3 B/N lists a fifth more records)
constexpr int kCandNum = 5, kCandDen = 2;

template <int D, int G>
__global__ __launch_bounds__(kSample) void k_sample(SampleArgs a) {
    constexpr int TS = D / 32, NS = D / 64, NT = (3 * G + 15) / 16;
    constexpr int ROWB = D * 2, CPR = ROWB / 16, NDMA = 32 * CPR / 64;
    static_assert(kSample == 256, "four waves of two 32-key stages");
    __shared__ uint4 stage[4][32 * CPR];
    __shared__ float sS[kSample][G];
    __shared__ __align__(16) uint32_t ak[kSample];
    __shared__ float red[kSample / kWave][G];
    __shared__ float tau_s;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int row = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x;
    if (s == 0 && tid == 0) *a.fb_count = 0;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    float* thr = a.thr + (int64_t)s * G;
    if (!candidate_mode(N, a.budget)) {
        if (tid < G) thr[tid] = -__builtin_inff();
        return;
    }
    // Sample j = 64 w + 32 h + k (stage h of wave w, stage key k) sits in
    // stratum j of N/kSample keys, at an offset that varies with j and the
    // segment.  Its row comes in through LDS like the scoring pass's keys
    // (whole rows per DMA instruction, the same swizzle), and its scores come
    // from the same tile contraction, so they are the exact fp32 scores.
    const int stride = N / kSample;           // >= 16 in candidate mode
    uint4* region = &stage[w][0];
    auto issue = [&](int h) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int P = 64 * i + lane;
            const int kl = P / CPR;
            const int lc = (P % CPR) ^ (kl % CPR);
            const int j = w * (kSample / 4) + 32 * h + kl;
            const int slot = j * stride + (int)(((uint32_t)j * 2654435761u + (uint32_t)s * 40503u) >> 8) % stride;
            const uint8_t* src = a.kv.k + a.kv.row(s, slot) * ROWB + 16 * lc;
            __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(region + 64 * i), 16, 0, 0);
        }
    };
    issue(0);
    bf16x8_t bt[TS][NT], bn[NS][NT];
    mfma_coef_fragments<D, G>(a.ctab, a.wtab, a.shape, a.n_q_heads, s, bt, bn);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint4 av[2][TS];
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int kl = 16 * u + row;
#pragma unroll
            for (int st = 0; st < TS; ++st) av[u][st] = region[kl * CPR + ((4 * st + grp) ^ (kl % CPR))];
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_wave_barrier();
        if (h == 0) issue(1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float S4[4];
            mfma_tile_scores<D, G>(av[u], bt, bn, S4);
            if (row < G) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sS[w * (kSample / 4) + 32 * h + 16 * u + 4 * grp + r][row] = S4[r];
            }
        }
    }
    __syncthreads();
    float S[G];
#pragma unroll
    for (int g = 0; g < G; ++g) S[g] = sS[tid][g];

    // sample mean and spread per head (two passes)
    float mu[G], sg[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float t = wave_sumf(S[g]);
        if (lane == 0) red[w][g] = t;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float t = 0.0f;
        for (int i = 0; i < kSample / kWave; ++i) t += red[i][g];
        mu[g] = t / kSample;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float dv = S[g] - mu[g];
        const float t = wave_sumf(dv * dv);
        if (lane == 0) red[w][g] = t;
    }
    __syncthreads();
    float A = -__builtin_inff();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float t = 0.0f;
        for (int i = 0; i < kSample / kWave; ++i) t += red[i][g];
        sg[g] = sqrtf(t / kSample);
        A = fmaxf(A, sg[g] > 0.0f ? (S[g] - mu[g]) / sg[g] : 0.0f);
    }
    // Distinct ordered keys: the sample index replaces the low 8 bits of the
    // order-preserving pattern of A (a relative change below 2^-15, immaterial
    // for a threshold), so a rank is one unsigned compare per sample.
    const uint32_t mykey = (order_key(A) & ~0xFFu) | (uint32_t)(kSample - 1 - tid);
    ak[tid] = mykey;
    if (tid == 0) tau_s = -__builtin_inff();   // (every rank is taken once)
    __syncthreads();
    // tau = the r-th largest sample aggregate, r = ceil(kCandNum B kSample / (kCandDen N))
    const int64_t r64 = ((int64_t)kCandNum * a.budget * kSample + (int64_t)kCandDen * N - 1) / ((int64_t)kCandDen * N);
    const int r = (int)(r64 < 1 ? 1 : r64 > kSample ? kSample : r64);
    int rank = 0;
    const uint4* ak4 = reinterpret_cast<const uint4*>(ak);
#pragma unroll 8
    for (int j4 = 0; j4 < kSample / 4; ++j4) {
        const uint4 q = ak4[j4];
        rank += (q.x > mykey) + (q.y > mykey) + (q.z > mykey) + (q.w > mykey);
    }
    if (rank == r - 1) tau_s = A;
    __syncthreads();
    if (tid < G) {
        float m = 0.0f, sd = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g)
            if (g == tid) { m = mu[g]; sd = sg[g]; }
        // a head with no spread in the sample admits every key (its scores here
        // and in the scoring pass may differ in the last bit)
        thr[tid] = sd > 0.0f ? fmaf(tau_s, sd, m) : -__builtin_inff();
    }
}

template <int D>
static bool sample_group(const SampleArgs& a, int group, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_seg), block(kSample);
    switch (group) {
        case 1: hipLaunchKernelGGL((k_sample<D, 1>), grid, block, 0, stream, a); return true;
        case 2: hipLaunchKernelGGL((k_sample<D, 2>), grid, block, 0, stream, a); return true;
        case 4: hipLaunchKernelGGL((k_sample<D, 4>), grid, block, 0, stream, a); return true;
        case 8: hipLaunchKernelGGL((k_sample<D, 8>), grid, block, 0, stream, a); return true;
        default: return false;
    }
}

hipError_t launch_sample(const SampleArgs& a, int head_dim, int group, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    TimedLaunch tl(KID_SAMPLE, stream);
    const bool ok = head_dim == 64 ? sample_group<64>(a, group, stream)
                  : head_dim == 128 ? sample_group<128>(a, group, stream) : false;
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int D, int G, bool BF16>
static void score_kernel(const ScoreArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((k_score<D, G, BF16>), dim3((unsigned)((int64_t)a.n_seg * a.n_chunks)), dim3(256), 0,
                       stream, a);
}

template <int D, int G, bool PAGED>
static void score_mfma_launch(const ScoreArgs& a, int mode, int64_t items, hipStream_t stream) {
    if (mode == SCORE_FULL)
        hipLaunchKernelGGL((k_score_mfma<D, G, false, PAGED>), dim3((unsigned)items), dim3(256), 0, stream, a);
    else if (mode == SCORE_CANDIDATES)
        hipLaunchKernelGGL((k_score_mfma<D, G, true, PAGED>), dim3((unsigned)items), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((k_score_mfma_fallback<D, G, PAGED>), dim3((unsigned)(items < 2048 ? items : 2048)),
                           dim3(256), 0, stream, a);
}

template <int D, int G>
static bool score_dtype(const ScoreArgs& a, bool bf16, int mode, hipStream_t stream) {
    const int64_t items = (int64_t)a.n_seg * a.n_chunks;
    if (!bf16) {
        if (mode != SCORE_FULL) return false;         // candidate lists are a bf16 (MFMA) feature
        score_kernel<D, G, false>(a, stream);
        return true;
    }
    if (a.kv.page_size > 0) score_mfma_launch<D, G, true>(a, mode, items, stream);
    else score_mfma_launch<D, G, false>(a, mode, items, stream);
    return true;
}

template <int D>
static bool score_group(const ScoreArgs& a, int group, bool bf16, int mode, hipStream_t stream) {
    switch (group) {
        case 1: return score_dtype<D, 1>(a, bf16, mode, stream);
        case 2: return score_dtype<D, 2>(a, bf16, mode, stream);
        case 4: return score_dtype<D, 4>(a, bf16, mode, stream);
        case 8: return score_dtype<D, 8>(a, bf16, mode, stream);
        default: return false;
    }
}

hipError_t launch_score(const ScoreArgs& a, int head_dim, int group, bool bf16, int mode, hipStream_t stream) {
    if ((int64_t)a.n_seg * a.n_chunks == 0) return hipSuccess;
    if (a.chunk % 512 || a.chunk > 2048) return hipErrorInvalidValue;
    TimedLaunch tl(mode == SCORE_FALLBACK ? KID_SCORE_FALLBACK : KID_SCORE, stream);
    const bool ok = head_dim == 64 ? score_group<64>(a, group, bf16, mode, stream)
                  : head_dim == 128 ? score_group<128>(a, group, bf16, mode, stream) : false;
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
