// Top-B selection and compaction kernels for gfx950.
//
// Selection (yeyulingfeng.com TriAttention page, section 主要方法: when the cache
// exceeds its budget, keep only the top-B keys): one 1024-thread workgroup per
// segment holds the segment's aggregated scores in registers as order-preserving
// 32-bit keys, finds the exact B-th largest key T with an MSB-first radix select
// (11 + 11 + 10 bit digits, 2048-bin LDS histograms, one block scan per digit),
// then keeps every key > T and the lowest-slot keys equal to T.  The kept slots
// are emitted in ascending order from wave ballots plus one block scan over
// (register index, wave) counts, so the result is identical run to run.
//
// In gather mode the same workgroup then copies the kept K/V rows and positions
// (bit-exact, slot order) into the destination cache: the fused pruning pass.
// In place, only the kept rows at or above the kept count move, into the slots
// freed below it.
#include "launch.h"
#include "stats.h"

namespace tri {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxBudget = 8192;

// Inclusive scan of one uint32 per thread over the 1024-thread block.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t x, uint32_t* wsum) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    x = wave_incl_scan(x);
    if (lane == kWave - 1) wsum[w] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < w; ++i) before += wsum[i];
    __syncthreads();
    return x + before;
}

// Candidate lists of one segment (written by the scoring pass in candidate
// mode) -> order keys and slots held in registers, in slot order: entry k sits
// in register k / 1024 of thread k % 1024.  Returns the number of candidates,
// or -1 when they do not fit in J * 1024 registers.
// Block b (keys 32b .. 32b+31) was scored by wave w = (b mod bpc) mod 4 of chunk
// c = b / bpc (bpc = chunk / 32 blocks per chunk), whose list (at
// wave_list_base in the chunk's scratch rows) holds its blocks' candidates
// block after block.  Two block scans give, per block, the rank of
// its first candidate in slot order (pre) and, in the order of the wave lists,
// the running count (lpos) from which its offset inside its list follows.
// Block of candidate k (the last block whose first candidate rank is <= k) and
// k's rank q inside it.
__device__ __forceinline__ void cand_block(int k, int nbk, const uint32_t* pre, int& b, int& q) {
    int lo = 0, hi = nbk;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int)pre[mid] <= k) lo = mid;
        else hi = mid;
    }
    b = lo;
    q = k - (int)pre[lo];
}

// Position (0..31) of the q-th set bit (0-based) of m.
__device__ __forceinline__ int nth_bit(uint32_t m, int q) {
    for (int i = 0; i < q; ++i) m &= m - 1u;
    return __builtin_ctz(m);
}

// Candidate lists of one segment (written by the scoring pass in candidate
// mode) -> order keys held in registers, in slot order: entry k sits in
// register k / 1024 of thread k % 1024.  Returns the number of candidate keys
// (keys with at least one listed head), or -1 when they do not fit in
// J * 1024 registers.
// Block b (keys 32b .. 32b+31) has G mask words (word h: keys whose head h
// passed) and was scored by wave w = (b mod bpc) mod 4 of chunk c = b / bpc
// (bpc = chunk / 32), whose list (at wave_list_base in the chunk's scratch
// rows) holds, block after block and key after key, the passing heads' scores.
// Two block scans give, per block, the slot-order rank of its first candidate
// key (pre, from the union of its words) and, in the order of the wave lists,
// the running float count (lpos) from which its offset inside its list follows.
// The mask words are staged in LDS (hwl) as they are read, so each candidate
// then needs one global load (its scores), not two.
// A key's entry is A' = the largest z-score over its listed heads.
// NB: the blocks the per-block LDS arrays hold (>= nbk; a multiple of 64, so a
// chunk's wave-list positions stay inside them).
template <int J, int G, int NB>
__device__ __forceinline__ int load_candidates(const SelectArgs& a, const int s, const int N, const ZParams<G>& z,
                                               uint32_t (&key)[J], uint32_t* pre, uint32_t* lpos, uint32_t* mw,
                                               uint32_t* hwl, uint32_t* wsum, uint32_t* bcast) {
    constexpr int BPT = NB >= kSelThreads ? NB / kSelThreads : 1;   // blocks per thread: tid * BPT + i
    const int tid = threadIdx.x;
    const int nbk = (N + 31) / 32;                     // <= NB
    const int bpc = a.chunk / 32, q4 = bpc / 4;
    auto perm = [&](int b) {                           // block -> position in wave-list order
        const int c = b / bpc, r = b - c * bpc;
        return c * bpc + (r & 3) * q4 + (r >> 2);
    };
    const uint32_t* mp = a.masks + (int64_t)s * a.mask_stride * G;
    uint32_t cu[BPT], cf[BPT], ct = 0u;                // per block: candidate keys, listed floats
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = tid * BPT + i;
        uint32_t u = 0u, f = 0u;
        if (b < nbk) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint32_t wd = mp[b * G + g];
                hwl[b * G + g] = wd;
                u |= wd;
                f += __popc(wd);
            }
        }
        if (b < NB) {
            mw[b] = u;
            lpos[b] = 0u;
        }
        cu[i] = __popc(u);
        cf[i] = f;
        ct += cu[i];
    }
    const uint32_t inc = block_incl_scan(ct, wsum);     // (synchronises)
    {
        uint32_t run = inc - ct;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid * BPT + i;
            if (b < NB) pre[b] = run;
            run += cu[i];
        }
    }
    if (tid == kSelThreads - 1) bcast[0] = inc;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = tid * BPT + i;
        if (b < nbk) lpos[perm(b)] = cf[i];
    }
    __syncthreads();
    uint32_t tv[BPT], tt = 0u;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = tid * BPT + i;
        tv[i] = b < NB ? lpos[b] : 0u;
        tt += tv[i];
    }
    const uint32_t inc2 = block_incl_scan(tt, wsum);
    {
        uint32_t run = inc2 - tt;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid * BPT + i;
            if (b < NB) lpos[b] = run;
            run += tv[i];
        }
    }
    __syncthreads();
    const int nc = (int)bcast[0];
    if (nc > J * kSelThreads) return -1;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int k = j * kSelThreads + tid;
        if (k < nc) {
            int lo, q;
            cand_block(k, nbk, pre, lo, q);
            const int kb = nth_bit(mw[lo], q);
            const uint32_t below = (1u << kb) - 1u;
            uint32_t hw[G];
            if constexpr (G % 4 == 0) {
#pragma unroll
                for (int g = 0; g < G; g += 4) {
                    const uint4 v = *reinterpret_cast<const uint4*>(hwl + lo * G + g);
                    hw[g] = v.x; hw[g + 1] = v.y; hw[g + 2] = v.z; hw[g + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int g = 0; g < G; ++g) hw[g] = hwl[lo * G + g];
            }
            int foff = 0;
#pragma unroll
            for (int g = 0; g < G; ++g) foff += __popc(hw[g] & below);
            const int c = lo / bpc, r = lo - c * bpc;
            const int head = c * bpc + (r & 3) * q4;
            const int base = wave_list_base(r & 3, min(a.chunk, N - c * a.chunk));
            const float* p = a.s_int + ((int64_t)s * a.cap + (int64_t)c * a.chunk + base) * G +
                             (lpos[head + (r >> 2)] - lpos[head]) + foff;
            float A = -__builtin_inff();
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if ((hw[g] >> kb) & 1u) {
                    const float S = *p++;
                    A = fmaxf(A, ((S - z.mu_hi[g]) - z.mu_lo[g]) * z.inv[g]);
                }
            }
            key[j] = order_key(A);
        }
        if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    return nc;
}

// Top-B of segment s.  MODE: SELECT_A reads aggregated scores, SELECT_S the
// interleaved per-head scores and chunk statistics, SELECT_C the candidate
// lists.  In mode C the result stands only if it provably equals mode S's: an
// unlisted (key, head) pair has S_h < L_h, and z_h = ((S - mu_hi) - mu_lo) * inv
// is monotone in S_h in fp32 as well, so its z-score is at most U = max_h z_h(L_h).
// A key's true A is therefore A' (the max over its listed heads) whenever
// A' > U, and at most U otherwise (keys with no listed head included).  If the
// cut T (the B-th largest A') exceeds U, the keys at or above it, their A and
// their tie order are exactly those of the full computation.  Otherwise the
// segment goes on the fallback list and nothing is written for it here.
template <int J, int G, int MODE>
__device__ __forceinline__ void select_segment(const SelectArgs& a, const int s) {
    constexpr bool CAND = MODE == SELECT_C;
    // mode C holds at most J*1024 >= N/2 candidates (launch_select), so a segment
    // has at most 64 J blocks of 32 keys (and at most 2048, N <= 65536)
    constexpr int NB = CAND ? (64 * J < 2048 ? 64 * J : 2048) : 1;
    constexpr int GZ = G > 0 ? G : 1;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ uint32_t pick[2];
    __shared__ uint32_t cnt_gt[J * kSelWaves], cnt_eq[J * kSelWaves];
    __shared__ int32_t kept[kMaxBudget];
    __shared__ double scratch[(kSelWaves + 1) * GZ];
    __shared__ uint32_t pre[NB], lpos[NB], mw[NB];
    __shared__ __align__(16) uint32_t hwl[CAND ? NB * GZ : 1];      // mode C: the segment's mask words
    __shared__ uint32_t bcast[1];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), w = tid / kWave;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int B = a.budget;
    const bool all = N <= B;

    uint32_t key[J];
#pragma unroll
    for (int j = 0; j < J; ++j) key[j] = 0u;
    uint32_t T = 0u;
    int need = 0;
    int nv = N;                                         // register entries, in slot order

    if (!all) {
        ZParams<GZ> z;
        if constexpr (G > 0) {
            // the segment's mean and spread per head: each wave merges the chunk
            // statistics by itself when a wave holds them all (no barrier)
            const double2* st = a.stats + (int64_t)s * a.n_chunks * G;
            auto merge = [&]() {
                return a.n_chunks <= kWave ? merge_stats_wave<G>(st, a.n_chunks, a.chunk, N)
                                           : merge_stats<G, kSelThreads>(st, a.n_chunks, a.chunk, N, scratch);
            };
            if constexpr (CAND) {
                z = merge();
                nv = load_candidates<J, G, NB>(a, s, N, z, key, pre, lpos, mw, hwl, wsum, bcast);
                if (nv < B) {                           // overflow (-1) or too few to hold the cut
                    if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1)] = s;
                    return;
                }
            } else {
                // Key j's G scores; loaded LB keys at a time (the scheduler would
                // otherwise hoist every key's loads at once).  Where one block
                // per CU leaves the registers (J >= 32), batches are 16 keys and
                // the first is requested before the merge, which does not need it.
                constexpr bool WIDE = J >= 32 && G <= 4;
                constexpr int LB = WIDE ? 16 : 8;
                constexpr int L0 = WIDE ? LB : 0;                  // keys loaded before the merge
                auto load_scores = [&](int j, float (&S)[G]) {
                    const float* p = a.s_int + ((int64_t)s * a.cap + j * kSelThreads + tid) * G;
                    if constexpr (G % 4 == 0) {
#pragma unroll
                        for (int g = 0; g < G; g += 4) {
                            const float4 v = *reinterpret_cast<const float4*>(p + g);
                            S[g] = v.x; S[g + 1] = v.y; S[g + 2] = v.z; S[g + 3] = v.w;
                        }
                    } else {
#pragma unroll
                        for (int g = 0; g < G; ++g) S[g] = p[g];
                    }
                };
                float S0[L0 > 0 ? L0 : 1][G];
#pragma unroll
                for (int j = 0; j < L0; ++j)
                    if (j * kSelThreads + tid < N) load_scores(j, S0[j]);
                z = merge();
#pragma unroll
                for (int j = 0; j < L0; ++j)
                    if (j * kSelThreads + tid < N) key[j] = order_key(aggregate<G>(S0[j], z));
#pragma unroll
                for (int j = L0; j < J; ++j) {
                    if (j * kSelThreads + tid < N) {
                        float S[G];
                        load_scores(j, S);
                        key[j] = order_key(aggregate<G>(S, z));
                    }
                    if (j % LB == LB - 1) __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int n = j * kSelThreads + tid;
                if (n < N) key[j] = order_key(a.agg[(int64_t)s * a.agg_stride + n]);
                if ((j & 15) == 15) __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- radix select of the B-th largest key
        uint32_t prefix = 0u, pmask = 0u;
        need = B;
#pragma unroll
        for (int pass = 0; pass < 3; ++pass) {
            const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
            const uint32_t dmask = pass < 2 ? 0x7ffu : 0x3ffu;
            hist[tid] = 0u;
            hist[tid + kSelThreads] = 0u;
            if (tid == 0) {
                pick[0] = 0u;
                pick[1] = 0u;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int n = j * kSelThreads + tid;
                if (n < nv && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
            }
            __syncthreads();
            // Thread t owns bins 2047-2t and 2046-2t: a scan in thread order is a
            // cumulative count from the top bin down.
            const int b0 = 2047 - 2 * tid, b1 = b0 - 1;
            const uint32_t h0 = hist[b0], h1 = hist[b1];
            const uint32_t incl = block_incl_scan(h0 + h1, wsum);
            const uint32_t above0 = incl - (h0 + h1);
            const uint32_t above1 = above0 + h0;
            const uint32_t un = (uint32_t)need;
            if (above0 < un && above0 + h0 >= un) {
                pick[0] = (uint32_t)b0;
                pick[1] = above0;
            } else if (above1 < un && above1 + h1 >= un) {
                pick[0] = (uint32_t)b1;
                pick[1] = above1;
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            pmask |= dmask << shift;
            need -= (int)pick[1];
            __syncthreads();
        }
        T = prefix;

        if constexpr (CAND) {
            if (nv < N) {                               // certificate for the keys left out
                float L[GZ];
#pragma unroll
                for (int g = 0; g < GZ; ++g) L[g] = a.thr[(int64_t)s * GZ + g];
                if (!(T > order_key(aggregate<GZ>(L, z)))) {
                    if (tid == 0) a.fb_list[atomicAdd(a.fb_count, 1)] = s;
                    return;
                }
            }
        }
    }

    // ---- ordered emission: entry k = j*1024 + w*64 + lane, in (j, w, lane) order
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int n = j * kSelThreads + tid;
        const bool valid = n < nv;
        const bool gt = valid && (all || key[j] > T);
        const bool eq = valid && !all && key[j] == T;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        if (lane == 0) {
            cnt_gt[j * kSelWaves + w] = (uint32_t)__popcll(bg);
            cnt_eq[j * kSelWaves + w] = (uint32_t)__popcll(be);
        }
    }
    __syncthreads();
    {
        const uint32_t vg = tid < J * kSelWaves ? cnt_gt[tid] : 0u;
        const uint32_t ve = tid < J * kSelWaves ? cnt_eq[tid] : 0u;
        const uint32_t ig = block_incl_scan(vg, wsum);
        const uint32_t ie = block_incl_scan(ve, wsum);
        if (tid < J * kSelWaves) {
            cnt_gt[tid] = ig - vg;
            cnt_eq[tid] = ie - ve;
        }
    }
    __syncthreads();
    const int nk = min(N, B);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int n = j * kSelThreads + tid;
        const bool valid = n < nv;
        const bool gt = valid && (all || key[j] > T);
        const bool eq = valid && !all && key[j] == T;
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const int eb = (int)cnt_eq[j * kSelWaves + w] + __popcll(be & below);
        const int gb = (int)cnt_gt[j * kSelWaves + w] + __popcll(bg & below);
        const int out = gb + min(eb, need);
        if ((gt || (eq && eb < need)) && out < nk) {
            int slot = n;
            if constexpr (CAND) {
                if (!all) {                             // candidate n -> its slot
                    int b, q;
                    cand_block(n, (N + 31) / 32, pre, b, q);
                    slot = 32 * b + nth_bit(mw[b], q);
                }
            }
            if (a.gather) kept[out] = slot;
            else a.idx_out[(int64_t)s * a.idx_stride + out] = slot;
        }
    }
    __syncthreads();                                    // every wave has read lengths[s] (n_kept may alias it)
    if (a.n_kept && tid == 0) a.n_kept[s] = nk;
    if (!a.gather) return;

    const int cpr = a.row_bytes >> 4;
    const int lg = 31 - __clz(cpr);
    if (a.gather == GATHER_IN_PLACE) {
        // kept[0..c) are below nk and stay; kept[c..nk) fill the freed slots
        // below nk in ascending order.  The r-th freed slot is r + p, where p
        // counts the kept slots below it, i.e. the entries i < c with
        // kept[i] - i <= r (kept[i] - i, the freed slots below kept[i], does
        // not decrease with i).  Freed slots are found in batches of 2048
        // (the histogram's LDS, no longer needed).
        int lo = 0, hi = nk;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kept[mid] < nk) lo = mid + 1;
            else hi = mid;
        }
        const int c = lo, m = nk - c;
        for (int base = 0; base < m; base += 2048) {
            const int nb = min(2048, m - base);
            for (int r = tid; r < nb; r += kSelThreads) {
                int l2 = 0, h2 = c;
                while (l2 < h2) {
                    const int mid = (l2 + h2) >> 1;
                    if (kept[mid] - mid <= base + r) l2 = mid + 1;
                    else h2 = mid;
                }
                hist[r] = (uint32_t)(base + r + l2);
            }
            __syncthreads();
            for (int u = tid; u < nb * cpr; u += kSelThreads) {
                const int jr = u >> lg, q = u & (cpr - 1);
                const int64_t sr = a.src.row(s, kept[c + base + jr]);
                const int64_t dr = a.dst.row(s, (int)hist[jr]);
                const uint4 kv = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[q];
                const uint4 vv = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[q];
                reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[q] = kv;
                reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[q] = vv;
            }
            for (int jr = tid; jr < nb; jr += kSelThreads)
                a.dst.pos[a.dst.row(s, (int)hist[jr])] = a.src.pos[a.src.row(s, kept[c + base + jr])];
            __syncthreads();                            // hist is refilled by the next batch
        }
        return;
    }

    // ---- compaction of the kept rows (16-byte copies), then positions
    const int total = nk * cpr;
    for (int u = tid; u < total; u += kSelThreads) {
        const int jrow = u >> lg, q = u & (cpr - 1);
        const int64_t sr = a.src.row(s, kept[jrow]);
        const int64_t dr = a.dst.row(s, jrow);
        const uint4 kv = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[q];
        const uint4 vv = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[q];
        reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[q] = kv;
        reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[q] = vv;
    }
    for (int jrow = tid; jrow < nk; jrow += kSelThreads)
        a.dst.pos[a.dst.row(s, jrow)] = a.src.pos[a.src.row(s, kept[jrow])];
}

// J <= 16, G <= 4: two workgroups per CU (at most 64 VGPRs and the SGPRs of 8 waves per
// SIMD), so one workgroup's gather overlaps the other's select phase.
template <int J, int G, int MODE>
__global__ __launch_bounds__(kSelThreads) __attribute__((amdgpu_waves_per_eu((J <= 16 && G <= 4) || (J <= 2 && G == 8) ? 8 : 1))) void k_select(
    SelectArgs a) {
    select_segment<J, G, MODE>(a, blockIdx.x);
}

// Mode S over the segments whose candidate pass failed its certificate.
template <int J, int G>
__global__ __launch_bounds__(kSelThreads) void k_select_fallback(SelectArgs a) {
    const int n = *a.fb_count;
    for (int i = blockIdx.x; i < n; i += gridDim.x) {
        __syncthreads();                                // LDS of the previous segment is no longer read
        select_segment<J, G, SELECT_S>(a, a.fb_list[i]);
    }
}

template <int J, int G>
static bool select_launch(const SelectArgs& a, int mode, hipStream_t stream) {
    const dim3 block(kSelThreads);
    if (mode == SELECT_S_FALLBACK) {
        if constexpr (G > 0)
            hipLaunchKernelGGL((k_select_fallback<J, G>), dim3((unsigned)(a.n_seg < 512 ? a.n_seg : 512)), block, 0, stream, a);
        return G > 0;
    }
    const dim3 grid((unsigned)a.n_seg);
    if constexpr (G == 0) {
        hipLaunchKernelGGL((k_select<J, 0, SELECT_A>), grid, block, 0, stream, a);
    } else if (mode == SELECT_C) {
        hipLaunchKernelGGL((k_select<J, G, SELECT_C>), grid, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL((k_select<J, G, SELECT_S>), grid, block, 0, stream, a);
    }
    return true;
}

template <int J>
static bool select_group(const SelectArgs& a, int group, int mode, hipStream_t stream) {
    if ((group == 0) != (mode == SELECT_A)) return false;
    switch (group) {
        case 0: return select_launch<J, 0>(a, mode, stream);
        case 1: return select_launch<J, 1>(a, mode, stream);
        case 2: return select_launch<J, 2>(a, mode, stream);
        case 4: return select_launch<J, 4>(a, mode, stream);
        case 8: return select_launch<J, 8>(a, mode, stream);
        default: return false;
    }
}

hipError_t launch_select(const SelectArgs& a, int group, int mode, int64_t max_len, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    if (a.budget > kMaxBudget || max_len > 64 * kSelThreads) return hipErrorInvalidValue;
    int64_t held = max_len;                             // entries one thread block holds in registers
    if (mode == SELECT_C) {
        // every key of a segment outside candidate mode (N < max(4096, 8B)), or
        // half of the longest segment's keys (the sampled threshold admits about
        // 3 B/N of them, at most 3/8 since N >= 8 B); a longer list sends its
        // segment to the fallback (full rescoring, mode S)
        const int64_t small = 8 * (int64_t)a.budget > 4096 ? 8 * (int64_t)a.budget : 4096;
        const int64_t half = (max_len + 1) / 2 > small ? (max_len + 1) / 2 : small;
        held = half < max_len ? half : max_len;
        if (a.chunk % 512 || a.chunk > 2048) return hipErrorInvalidValue;
    }
    const KernelId id = mode == SELECT_S_FALLBACK ? KID_SELECT_FALLBACK : a.gather ? KID_SELECT_GATHER : KID_SELECT;
    TimedLaunch tl(id, stream);
    bool ok;
    if (held <= 2 * kSelThreads) ok = select_group<2>(a, group, mode, stream);
    else if (held <= 8 * kSelThreads) ok = select_group<8>(a, group, mode, stream);
    else if (mode == SELECT_C && held <= 16 * kSelThreads) ok = select_group<16>(a, group, mode, stream);
    else if (held <= 32 * kSelThreads) ok = select_group<32>(a, group, mode, stream);
    // a 32K-key cache plus a window of up to 4K appended keys
    else if (held <= 36 * kSelThreads) ok = select_group<36>(a, group, mode, stream);
    else ok = select_group<64>(a, group, mode, stream);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

// ------------------------------------------------------------------ gather
// Unfused compaction: workgroup (segment, block of rows) copies kept rows.
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
    const int s = blockIdx.x / a.blocks_per_seg;
    const int rb = blockIdx.x - s * a.blocks_per_seg;
    const int nk = min(max(a.n_kept[s], 0), (int)min(a.idx_stride, a.dst.capacity));
    const int r0 = rb * a.rows_per_block;
    if (r0 >= nk) return;
    const int rows = min(a.rows_per_block, nk - r0);
    const int cpr = a.row_bytes >> 4;
    const int lg = 31 - __clz(cpr);
    const int32_t* idx = a.idx + (int64_t)s * a.idx_stride + r0;
    for (int u = threadIdx.x; u < rows * cpr; u += 256) {
        const int jrow = u >> lg, q = u & (cpr - 1);
        const int32_t i = idx[jrow];
        if (i < 0 || i >= a.src.capacity) continue;      // out-of-range index: row skipped
        const int64_t sr = a.src.row(s, i);
        const int64_t dr = a.dst.row(s, r0 + jrow);
        const uint4 kv = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[q];
        const uint4 vv = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[q];
        reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[q] = kv;
        reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[q] = vv;
    }
    for (int jrow = threadIdx.x; jrow < rows; jrow += 256) {
        const int32_t i = idx[jrow];
        if (i >= 0 && i < a.src.capacity) a.dst.pos[a.dst.row(s, r0 + jrow)] = a.src.pos[a.src.row(s, i)];
    }
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.n_seg * a.blocks_per_seg;
    if (blocks == 0) return hipSuccess;
    TimedLaunch tl(KID_GATHER, stream);
    hipLaunchKernelGGL(k_gather, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace tri
