// Decode-loop kernels for gfx950: appending a generated token to every
// segment, and single-query decode attention over the (pruned) cache.
//
// Between two pruning passes the cache grows by one token per step and every
// step re-attends to the whole cache (zingnex.cn TriAttention page, section
// 长推理的内存困境); the attention here is plain softmax(scale q.K^T) V per
// query head, over the keys the pruning kept plus those appended since.
#include "launch.h"

namespace tri {

// ------------------------------------------------------------------ append
// 256 threads append the new rows of 256 / TPS segments: TPS = 2 * row_bytes
// / 16 threads per segment, one 16-byte chunk of the K or V row each (a step
// appends a few hundred KB in all, so the launch is latency-bound and fewer,
// fuller workgroups finish it sooner than one small workgroup per segment).
__global__ __launch_bounds__(256) void k_append(AppendArgs a) {
    const int cpr = a.row_bytes >> 4;              // chunks per row
    const int tps = 2 * cpr;                       // threads per segment (power of two, <= 256)
    const int s = (int)(((int64_t)blockIdx.x * 256 + threadIdx.x) / tps);
    const int j = threadIdx.x & (tps - 1);
    const int n = s < a.n_seg ? a.lengths[s] : -1;
    __syncthreads();                               // every lane has read its segment's length
    if (s >= a.n_seg || n < 0 || n >= a.kv.capacity) return;   // full (or corrupt) segment: unchanged
    const int64_t r = a.kv.row(s, n);
    if (j < cpr)
        reinterpret_cast<uint4*>(a.kv.k + r * a.row_bytes)[j] =
            reinterpret_cast<const uint4*>(a.k_new + (int64_t)s * a.row_bytes)[j];
    else
        reinterpret_cast<uint4*>(a.kv.v + r * a.row_bytes)[j - cpr] =
            reinterpret_cast<const uint4*>(a.v_new + (int64_t)s * a.row_bytes)[j - cpr];
    if (j == 0) {
        a.kv.pos[r] = a.pos_new[a.shape.seq(s)];
        a.lengths[s] = n + 1;
    }
}

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    const int tps = 2 * (a.row_bytes >> 4);
    if (a.row_bytes % 16 || tps < 1 || tps > 256 || (tps & (tps - 1))) return hipErrorInvalidValue;
    const int64_t blocks = ((int64_t)a.n_seg * tps + 255) / 256;
    TimedLaunch tl(KID_APPEND, stream);
    hipLaunchKernelGGL(k_append, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------ decode attention
// One 256-thread workgroup per segment (the G query heads sharing one KV head).
// Each wave walks 64-key tiles with an online softmax:
//  * logits: lane = key; the key row is held in registers and the G query
//    vectors are wave-uniform (scalar operands of the FMAs);
//  * probabilities go through a per-wave LDS tile;
//  * P.V: lane = output dimension (D/64 dims per lane), broadcast LDS reads of
//    four probabilities at a time.
// The four waves' (max, sum, partial output) are merged at the end.
template <int D, int G, bool BF16>
__global__ __launch_bounds__(256) void k_decode_attn(AttnArgs a) {
    constexpr int E = BF16 ? 8 : 4;     // elements per 16-byte chunk
    constexpr int NC = D / E;           // chunks per row
    constexpr int DPL = D / kWave;      // output dims per lane
    constexpr int ES = BF16 ? 2 : 4;
    constexpr float kLog2e = 1.4426950408889634f;
    __shared__ float4 ptile[4][G][kWave / 4];
    __shared__ float wm[4][G], wl[4][G];
    __shared__ float wo[4][G][D];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int s = blockIdx.x;
    const int N = min(max(a.lengths[s], 0), (int)a.kv.capacity);
    const int l = a.shape.layer(s), b = a.shape.seq(s), h = a.shape.head(s);
    const uint8_t* qb = a.q + (((int64_t)l * a.shape.n_seq + b) * a.n_q_heads + (int64_t)h * G) * D * ES;
    const float sl2 = a.scale * kLog2e;

    float m[G], lsum[G], o[G][DPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -__builtin_inff();
        lsum[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[g][d] = 0.0f;
    }

    for (int t0 = w * kWave; t0 < N; t0 += 4 * kWave) {
        const int n = t0 + lane;
        const bool valid = n < N;
        float lg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) lg[g] = 0.0f;
        if (valid) {
            const uint4* row = reinterpret_cast<const uint4*>(a.kv.k + a.kv.row(s, n) * (D * ES));
            uint4 kc[NC];
#pragma unroll
            for (int q = 0; q < NC; ++q) kc[q] = row[q];
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                float kf[E];
#pragma unroll
                for (int e = 0; e < E; ++e) kf[e] = chunk_elem<BF16>(kc[q], e);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const uint4 qc = reinterpret_cast<const uint4*>(qb + (int64_t)g * D * ES)[q];
                    float acc = lg[g];
#pragma unroll
                    for (int e = 0; e < E; ++e) acc = fmaf(chunk_elem<BF16>(qc, e), kf[e], acc);
                    lg[g] = acc;
                }
            }
        }
        // online softmax update (base 2); the tile's first key is valid, so the
        // new running maximum is finite
        float* pt = reinterpret_cast<float*>(&ptile[w][0][0]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float x = valid ? lg[g] * sl2 : -__builtin_inff();
            const float mn = fmaxf(m[g], wave_max(x));
            const float alpha = __builtin_amdgcn_exp2f(m[g] - mn);
            const float p = valid ? __builtin_amdgcn_exp2f(x - mn) : 0.0f;
            lsum[g] = lsum[g] * alpha + wave_sumf(p);
            m[g] = mn;
#pragma unroll
            for (int d = 0; d < DPL; ++d) o[g][d] *= alpha;
            pt[g * kWave + lane] = p;
        }
        __builtin_amdgcn_wave_barrier();
        const int cnt = min(kWave, N - t0);
        for (int i4 = 0; i4 < cnt; i4 += 4) {
            float4 p4[G];
#pragma unroll
            for (int g = 0; g < G; ++g) p4[g] = ptile[w][g][i4 >> 2];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (i4 + u < cnt) {
                    const uint8_t* vrow = a.kv.v + a.kv.row(s, t0 + i4 + u) * (D * ES);
#pragma unroll
                    for (int d = 0; d < DPL; ++d) {
                        const int dim = lane + d * kWave;
                        float v;
                        if (BF16) v = bf16_lo((uint32_t)reinterpret_cast<const uint16_t*>(vrow)[dim]);
                        else v = reinterpret_cast<const float*>(vrow)[dim];
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            const float pg = u == 0 ? p4[g].x : u == 1 ? p4[g].y : u == 2 ? p4[g].z : p4[g].w;
                            o[g][d] = fmaf(pg, v, o[g][d]);
                        }
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    }

    // merge the four waves
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            wm[w][g] = m[g];
            wl[w][g] = lsum[g];
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int d = 0; d < DPL; ++d) wo[w][g][lane + d * kWave] = o[g][d];
    __syncthreads();
    float* out = a.out + (((int64_t)l * a.shape.n_seq + b) * a.n_q_heads + (int64_t)h * G) * D;
    for (int i = tid; i < G * D; i += 256) {
        const int g = i / D, d = i - g * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, wm[v][g]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float sc = wl[v][g] > 0.0f ? __builtin_amdgcn_exp2f(wm[v][g] - M) : 0.0f;
            num = fmaf(wo[v][g][d], sc, num);
            den = fmaf(wl[v][g], sc, den);
        }
        out[(int64_t)g * D + d] = den > 0.0f ? num / den : 0.0f;
    }
}

// bf16 caches.  One workgroup of NW waves per segment; wave w takes the key
// tiles w, w+NW, ... (TK keys each: 32 for head_dim 64, 16 for 128, so a K or
// V tile is 4 KB).  A tile comes in through LDS DMA, whole rows per
// instruction, rows chunk-swizzled (16-byte chunk lc of tile key k at
// lc ^ (k mod CPR)).  The compiler makes every LDS access wait for all LDS
// DMA in flight, so a wave reads its whole tile into registers as soon as it
// lands, refills the buffer with its next tile, and then computes from
// registers only: one tile in flight per wave during all of its compute.
//  * logits q.K^T on the matrix cores: A = 16 key rows, B = the G query
//    vectors as columns (bf16, so the products are exact; fp32 accumulation);
//  * online softmax per head (base 2) on the fragment layout: lane (grp, row)
//    holds head `row`'s logits of keys 4 grp + r;
//  * P.V on the matrix cores too (v_mfma_f32_16x16x16_bf16, one per 16-key
//    unit, 16-dim block and split part): A = the probabilities in the logits'
//    own fragment layout, each carried as three bf16 parts (24 bits), B = the
//    V tile, whose fragments are copied from LDS to registers right after the
//    tile lands, so the compute touches no LDS while the next tile loads.  On
//    the vector units (a readlane and an FMA per key, head and dim) this was
//    about 80% of the SIMDs' issue cycles at head_dim 64, GQA 8.
// The waves' (max, sum, partial output) are merged at the end.
// Paged caches: lane l holds the page of key l of the tile the wave issues
// next, loaded (a plain load into a register) one compute phase ahead.
// P.V goes to the matrix cores where its vector form is the larger cost: G
// heads x D dims of multiply-adds (and G readlanes) per key against 4 D bytes
// of K and V, i.e. G >= 8 at head_dim 64.  At head_dim 128 (G <= 8) the
// vector form is cheaper than the registers the MFMA form needs (its
// accumulators and V fragments would not fit four waves per SIMD).
constexpr bool pv_on_mfma(int D, int G) { return G * 64 / D >= 8; }

template <int D, int G, bool PAGED, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(pv_on_mfma(D, G) && NW == 4 ? (PAGED ? 4 : 5) : 1))) void k_decode_attn_mfma(AttnArgs a) {
    constexpr int ROWB = D * 2, CPR = ROWB / 16;
    constexpr int TK = 2048 / D;               // keys per tile
    constexpr int NU = TK / 16;                // 16-key MFMA tiles per tile
    constexpr int TS = D / 32;                 // k-steps
    constexpr int NDMA = TK * CPR / 64;        // DMA instructions per operand and tile
    constexpr int NDB = D / 16;                // 16-dim output blocks
    constexpr int DPL = D / kWave;             // vector path: output dims per lane
    constexpr bool PV_MFMA = pv_on_mfma(D, G);
    constexpr float kLog2e = 1.4426950408889634f;
    static_assert(G <= 16 && NU >= 1, "one 16-column B fragment holds the group");
    static_assert(DPL == 1 || DPL == 2, "one or two output dims per lane");
    __shared__ uint4 kt[NW][TK * CPR];
    __shared__ uint4 vt[NW][TK * CPR];

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: the tile loop runs on scalar registers
    const int row = lane & 15, grp = lane >> 4;
    const int s = blockIdx.x;
    const int N = min(max(a.lengths[s], 0), (int)a.kv.capacity);
    const int l = a.shape.layer(s), b = a.shape.seq(s), h = a.shape.head(s);
    const uint8_t* qb = a.q + (((int64_t)l * a.shape.n_seq + b) * a.n_q_heads + (int64_t)h * G) * ROWB;
    const float sl2 = a.scale * kLog2e;
    const int nt = (N + TK - 1) / TK;

    int pg = 0;                                // paged: page of key (lane mod TK) of the next tile
    auto fetch_pages = [&](int t) {
        if constexpr (PAGED) {
            const int key = min(t * TK + lane % TK, N - 1);
            pg = a.kv.page_table[(int64_t)s * a.kv.max_pages + a.kv.page_entry(key)];
        }
    };
    auto issue = [&](int t) {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) {
            const int P = 64 * i + lane;
            const int kl = P / CPR;
            const int lc = (P % CPR) ^ (kl % CPR);
            const int key = min(t * TK + kl, N - 1);          // tail rows re-read a valid row
            int64_t r;
            if constexpr (PAGED) r = (int64_t)__shfl(pg, kl, kWave) * a.kv.page_size + a.kv.page_within(key);
            else r = (int64_t)s * a.kv.capacity + key;
            const int64_t off = r * ROWB + 16 * lc;
            __builtin_amdgcn_global_load_lds(a.kv.k + off, (lds_void_t*)(&kt[w][0] + 64 * i), 16, 0, 2 /* nt */);
            __builtin_amdgcn_global_load_lds(a.kv.v + off, (lds_void_t*)(&vt[w][0] + 64 * i), 16, 0, 2 /* nt */);
        }
    };
    if (w < nt) {
        fetch_pages(w);
        issue(w);
        if (w + NW < nt) fetch_pages(w + NW);              // arrives while tile w is awaited and computed
    }

    // B fragments: column row = head row (zero past G), k-slot (grp, e)
    bf16x8_t bq[TS];
#pragma unroll
    for (int st = 0; st < TS; ++st) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (row < G) v = reinterpret_cast<const uint4*>(qb + (int64_t)row * ROWB)[4 * st + grp];
        bq[st] = __builtin_bit_cast(bf16x8_t, v);
    }

    float m = -__builtin_inff(), lsum = 0.0f;              // head `row`'s running max and sum
    // output accumulators, the D layout of v_mfma_f32_16x16x16_bf16 per block
    // of 16 dims: lane (row, grp) holds O[head 4 grp + r][dim 16 c + row]
    f32x4_t oacc[PV_MFMA ? NDB : 1];
#pragma unroll
    for (int c = 0; c < (PV_MFMA ? NDB : 1); ++c) oacc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // otherwise (vector-unit P.V) lane = output dimension(s) DPL * lane + d
    float o[PV_MFMA ? 1 : G][DPL];
#pragma unroll
    for (int g = 0; g < (PV_MFMA ? 1 : G); ++g)
#pragma unroll
        for (int d = 0; d < DPL; ++d) o[g][d] = 0.0f;
    constexpr int VW = TK * DPL / 2;                       // vector path: 32-bit words of the lane's V values per tile

    // Byte offsets of the lane's fragment reads inside its wave's tile.  The
    // swizzle's XOR splits into a lane part and a compile-time part, so every
    // read is one of these registers plus an immediate offset.
    //  K, A fragment (row 16u + row, chunk 4 st + grp): the row's chunk is
    //  (4 st + grp) ^ (row mod CPR), the same for every u (16 is a multiple of CPR);
    static_assert(16 % CPR == 0, "a 16-key unit spans whole swizzle periods");
    int kofs[TS];
#pragma unroll
    for (int st = 0; st < TS; ++st) kofs[st] = 16 * (row * CPR + ((4 * st + grp) ^ (row % CPR)));
    //  V, B fragment (key 16u + 4grp + r, dim 16c + row, head_dim 64: CPR = 8):
    //  the chunk (2c + row/8) ^ (4 (grp mod 2) + r) has bit 0 = row/8 ^ r mod 2,
    //  bit 1 = c mod 2 ^ r/2 and bit 2 = c/2 ^ grp mod 2; the lane parts of
    //  bits 0 and 2 give four bases, the rest is constant.
    static_assert(!PV_MFMA || D == 64, "the V fragment offsets assume head_dim 64");
    int vofs[2][2];
#pragma unroll
    for (int r0 = 0; r0 < 2; ++r0)
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1)
            vofs[r0][c1] = 16 * CPR * 4 * grp + 2 * (row & 7) + 16 * ((row >> 3) ^ r0) + 64 * (c1 ^ (grp & 1));

    for (int t = w; t < nt; t += NW) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);              // this tile has landed
        __builtin_amdgcn_wave_barrier();
        // Everything the tile needs from LDS goes to registers first: the K
        // fragments and this lane's V values (key pairs packed at head_dim 64,
        // a dim pair per key at 128).  The buffers are then refilled with the
        // next tile while this one is computed, and the compute touches no LDS
        // (the probabilities and rescale factors are broadcast with readlane).
        const uint4* kr = &kt[w][0];
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(&vt[w][0]);
        uint4 af[NU][TS];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int st = 0; st < TS; ++st)
                af[u][st] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint8_t*>(kr) + kofs[st] +
                                                            16 * CPR * 16 * u);
        // V as B fragments: for 16-key unit u and dim block c, lane (row,
        // grp) holds V[16 u + 4 grp + r][16 c + row], r = 0..3 (bf16 pairs)
        // (vector path: the lane's own dims, every key of the tile)
        uint32_t vf[PV_MFMA ? NU : 1][PV_MFMA ? NDB : 1][2];
        uint32_t vw[PV_MFMA ? 1 : VW];
        if constexpr (PV_MFMA) {
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int c = 0; c < NDB; ++c)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        // key 16u + 4grp + r, dim 16c + row: vofs plus a constant
                        const uint8_t* cp = vb + vofs[r & 1][c >> 1] + 16 * CPR * (16 * u + r) + 32 * ((c & 1) ^ (r >> 1));
                        const uint32_t h = *reinterpret_cast<const uint16_t*>(cp);
                        if (r & 1) vf[u][c][r >> 1] |= h << 16;
                        else vf[u][c][r >> 1] = h;
                    }
        } else {
            const int dim = DPL * lane;                    // the lane's dims share one 16-byte chunk
#pragma unroll
            for (int k = 0; k < TK; ++k) {
                const uint8_t* cp = vb + 16 * (k * CPR + ((dim >> 3) ^ (k % CPR))) + 2 * (dim & 7);
                if constexpr (DPL == 2) {
                    vw[k] = *reinterpret_cast<const uint32_t*>(cp);
                } else {
                    const uint32_t h = *reinterpret_cast<const uint16_t*>(cp);
                    if (k & 1) vw[k >> 1] |= h << 16;
                    else vw[k >> 1] = h;
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);            // the reads are done: the buffers may be refilled
        __builtin_amdgcn_wave_barrier();
        if (t + NW < nt) issue(t + NW);
        if (t + 2 * NW < nt) fetch_pages(t + 2 * NW);      // the tile after next: arrives under this compute
        float x[NU][4];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            f32x4_t acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int st = 0; st < TS; ++st)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, af[u][st]), bq[st], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = t * TK + 16 * u + 4 * grp + r;
                x[u][r] = key < N ? acc[r] * sl2 : -__builtin_inff();
            }
        }
        // online softmax: head `row` over the tile's keys (4 lanes x NU*4 values);
        // the tile's first key is valid, so the new maximum is finite
        float tm = -__builtin_inff();
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) tm = fmaxf(tm, x[u][r]);
        tm = fmaxf(tm, __shfl_xor(tm, 16, kWave));
        tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
        const float mn = fmaxf(m, tm);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        float ts = 0.0f;
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                x[u][r] = __builtin_amdgcn_exp2f(x[u][r] - mn);   // probability, head `row`, key 16u + 4grp + r
                ts += x[u][r];
            }
        ts += __shfl_xor(ts, 16, kWave);
        ts += __shfl_xor(ts, 32, kWave);
        lsum = lsum * alpha + ts;
        m = mn;
        if constexpr (!PV_MFMA) {
            // P.V on the vector units: head g's probability of key 16u + 4q + r
            // sits in lane 16q + g, register x[u][r]
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float al = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), g));
#pragma unroll
                for (int d = 0; d < DPL; ++d) o[g][d] *= al;
            }
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int k = 16 * u + 4 * q + r;
                        float v[DPL];
                        if constexpr (DPL == 2) {
                            v[0] = bf16_lo(vw[k]);
                            v[1] = bf16_hi(vw[k]);
                        } else {
                            v[0] = (k & 1) ? bf16_hi(vw[k >> 1]) : bf16_lo(vw[k >> 1]);
                        }
#pragma unroll
                        for (int g = 0; g < G; ++g) {
                            const float p = __int_as_float(
                                __builtin_amdgcn_readlane(__float_as_int(x[u][r]), 16 * q + g));
#pragma unroll
                            for (int d = 0; d < DPL; ++d) o[g][d] = fmaf(p, v[d], o[g][d]);
                        }
                    }
            continue;
        }
        // rescale: the lane's output rows are heads 4 grp + r, whose factors
        // sit in lanes 4 grp + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float al = __shfl(alpha, 4 * grp + r, kWave);
#pragma unroll
            for (int c = 0; c < NDB; ++c) oacc[c][r] *= al;
        }
        // P.V on the matrix cores: A = P (16 heads x 16 keys of unit u) is the
        // logits' own layout (lane (row, grp) holds head row's probabilities of
        // keys 16 u + 4 grp + r); each probability is carried as the sum of
        // three bf16 parts (hi, mid, lo: 24 bits), so the bf16 products keep
        // fp32-level accuracy
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            bf16x4_t pa[3];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const __bf16 hi = (__bf16)x[u][r];
                const float r1 = x[u][r] - (float)hi;
                const __bf16 mid = (__bf16)r1;
                pa[0][r] = hi;
                pa[1][r] = mid;
                pa[2][r] = (__bf16)(r1 - (float)mid);
            }
#pragma unroll
            for (int c = 0; c < NDB; ++c) {
                const s16x4_t b = __builtin_bit_cast(s16x4_t, make_uint2(vf[u][c][0], vf[u][c][1]));
#pragma unroll
                for (int q = 0; q < 3; ++q)
                    oacc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, pa[q]), b,
                                                                       oacc[c], 0, 0, 0);
            }
        }
    }

    // merge the waves (their tile buffers hold the partial outputs, maxima and sums)
    __syncthreads();
    float* wo = reinterpret_cast<float*>(&kt[0][0]);      // [NW][G][D]
    float (*wm)[G] = reinterpret_cast<float (*)[G]>(&vt[0][0]);
    float (*wl)[G] = wm + NW;
    static_assert(sizeof(vt) >= sizeof(float) * 2 * NW * G, "maxima and sums fit the V tiles");
    static_assert(sizeof(kt) >= sizeof(float) * NW * G * D, "partial outputs fit the K tiles");
    if (grp == 0 && row < G) {
        wm[w][row] = m;
        wl[w][row] = lsum;
    }
    if constexpr (PV_MFMA) {
#pragma unroll
        for (int c = 0; c < NDB; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * grp + r < G) wo[(w * G + 4 * grp + r) * D + 16 * c + row] = oacc[c][r];
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int d = 0; d < DPL; ++d) wo[(w * G + g) * D + DPL * lane + d] = o[g][d];
    }
    __syncthreads();
    float* out = a.out + (((int64_t)l * a.shape.n_seq + b) * a.n_q_heads + (int64_t)h * G) * D;
    for (int i = tid; i < G * D; i += NW * 64) {
        const int g = i / D, d = i - g * D;
        float M = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < NW; ++v) M = fmaxf(M, wm[v][g]);
        float num = 0.0f, den = 0.0f;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float sc = wl[v][g] > 0.0f ? __builtin_amdgcn_exp2f(wm[v][g] - M) : 0.0f;
            num = fmaf(wo[(v * G + g) * D + d], sc, num);
            den = fmaf(wl[v][g], sc, den);
        }
        out[(int64_t)g * D + d] = den > 0.0f ? num / den : 0.0f;
    }
}

// Waves per decode-attention workgroup.  Four single-buffered waves (32 KB of
// LDS) let four or five workgroups share a CU, with more tiles per wave to
// amortise each workgroup's start and a cheaper final merge than 2 x 8 or
// 1 x 16 (measured fastest of 4, 8 and 16 on a batch that fills the GPU many
// times over, and no slower from 288 segments up).  A batch with fewer
// segments than CUs leaves most SIMDs without waves at four per segment: it
// takes 8 waves per segment (25-75% faster at 192 segments, head_dim 64 and
// 128), and 16 when at most half the CUs have a segment.
constexpr int kAttnWaves = 4;

static int attn_waves(int64_t n_seg) {
    static int cus = -1;
    if (cus < 0) {
        int dev = 0, n = 0;
        cus = hipGetDevice(&dev) == hipSuccess &&
                      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                  ? n
                  : 256;
    }
    if (n_seg >= cus) return kAttnWaves;
    return 2 * n_seg > cus ? 8 : 16;
}

template <int D, int G, bool PAGED>
static void attn_mfma(const AttnArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_seg);
    switch (attn_waves(a.n_seg)) {
        case kAttnWaves:
            hipLaunchKernelGGL((k_decode_attn_mfma<D, G, PAGED, kAttnWaves>), grid, dim3(kAttnWaves * 64), 0, stream, a);
            break;
        case 8: hipLaunchKernelGGL((k_decode_attn_mfma<D, G, PAGED, 8>), grid, dim3(8 * 64), 0, stream, a); break;
        default: hipLaunchKernelGGL((k_decode_attn_mfma<D, G, PAGED, 16>), grid, dim3(16 * 64), 0, stream, a); break;
    }
}

template <int D, int G>
static void attn_dtype(const AttnArgs& a, bool bf16, hipStream_t stream) {
    if (bf16 && a.kv.page_size > 0) attn_mfma<D, G, true>(a, stream);
    else if (bf16) attn_mfma<D, G, false>(a, stream);
    else hipLaunchKernelGGL((k_decode_attn<D, G, false>), dim3((unsigned)a.n_seg), dim3(256), 0, stream, a);
}

template <int D>
static bool attn_group(const AttnArgs& a, int group, bool bf16, hipStream_t stream) {
    switch (group) {
        case 1: attn_dtype<D, 1>(a, bf16, stream); return true;
        case 2: attn_dtype<D, 2>(a, bf16, stream); return true;
        case 4: attn_dtype<D, 4>(a, bf16, stream); return true;
        case 8: attn_dtype<D, 8>(a, bf16, stream); return true;
        default: return false;
    }
}

hipError_t launch_decode_attn(const AttnArgs& a, int head_dim, int group, bool bf16, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    TimedLaunch tl(KID_DECODE_ATTN, stream);
    bool ok = head_dim == 64 ? attn_group<64>(a, group, bf16, stream)
            : head_dim == 128 ? attn_group<128>(a, group, bf16, stream) : false;
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace tri
