// Top-B selection and compaction kernels for gfx950.
//
// Selection (yeyulingfeng.com TriAttention page, section 主要方法: when the cache
// exceeds its budget, keep only the top-B keys): one 1024-thread workgroup per
// segment holds the segment's aggregated scores in registers as order-preserving
// 32-bit keys, finds the exact B-th largest key T with an MSB-first radix select
// (11 + 11 + 10 bit digits, 2048-bin LDS histograms, one block scan per digit),
// then keeps every key > T and, of the keys equal to T, those at the earliest
// positions (a second radix select over their positions, run only when more
// keys tie at T than fit; equal positions, and callers without positions, go
// by lower slot).  The kept slots are emitted in ascending order from wave
// ballots plus one block scan over (register index, wave) counts, so the
// result is identical run to run.
//
// In gather mode the same workgroup then copies the kept K/V rows and positions
// (bit-exact, slot order) into the destination cache: the fused pruning pass.
// In place, the kept rows move down to their slot-order slots in batches; or,
// in the fill mode, only the kept rows at or above the kept count move, into
// the slots freed below it.
#include "launch.h"
#include "stats.h"

namespace tri {

constexpr int kSelThreads = 1024;

// 16-byte loads and stores with the non-temporal hint, for rows the pass
// touches once (the gather's source rows and the destination rows it writes).
using u32x4_t = unsigned int __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
    const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4 v) {
    const u32x4_t x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<u32x4_t*>(p));
}
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kMaxBudget = 8192;

// Inclusive scan of one uint32 per thread over a block of NT threads.
template <int NT = kSelThreads>
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

// MSB-first radix select over the block's register entries (entry j of a
// thread: key[j], entry number j * 1024 + tid).  Among the entries below nv
// (and, with use_sel, whose bit j of sel is set), finds the need-th largest
// key: 11 + 11 + 10 bit digits, one 2048-bin LDS histogram and one block scan
// per digit.  On return T is that key, need the number of entries equal to T
// that rank within the first `need` (entries > T plus that many entries == T
// make up the original need), and n_eq the number of such entries equal to T.
template <int J, int NT>
__device__ __forceinline__ void radix_select(const uint32_t (&key)[J], int nv, uint64_t sel, bool use_sel,
                                             int& need, uint32_t& T, uint32_t& n_eq, uint32_t* hist,
                                             uint32_t* wsum, uint32_t* pick) {
    constexpr int HB = 2048 / NT;                       // histogram bins per thread
    const int tid = threadIdx.x;
    uint32_t prefix = 0u, pmask = 0u;
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
        const uint32_t dmask = pass < 2 ? 0x7ffu : 0x3ffu;
#pragma unroll
        for (int i = 0; i < HB; ++i) hist[tid + i * NT] = 0u;
        if (tid == 0) {
            pick[0] = 0u;
            pick[1] = 0u;
            pick[2] = 0u;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const bool in = j * NT + tid < nv && (!use_sel || ((sel >> j) & 1u));
            if (in && (key[j] & pmask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
        }
        __syncthreads();
        // Thread t owns bins 2047 - HB t down to 2048 - HB (t + 1): a scan in
        // thread order is a cumulative count from the top bin down.
        uint32_t h[HB], hs = 0u;
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            h[i] = hist[2047 - HB * tid - i];
            hs += h[i];
        }
        uint32_t above = block_incl_scan<NT>(hs, wsum) - hs;
        const uint32_t un = (uint32_t)need;
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            if (above < un && above + h[i] >= un) {
                pick[0] = (uint32_t)(2047 - HB * tid - i);
                pick[1] = above;
                pick[2] = h[i];
            }
            above += h[i];
        }
        __syncthreads();
        prefix |= pick[0] << shift;
        pmask |= dmask << shift;
        need -= (int)pick[1];
        n_eq = pick[2];
        __syncthreads();
    }
    T = prefix;
}

// Slot of candidate entry n of a segment of N keys (mode C: entry n is the
// n-th candidate key in slot order).
__device__ __forceinline__ int cand_slot(int n, int N, const uint32_t* pre, const uint32_t* mw) {
    int b, q;
    cand_block(n, (N + 31) / 32, pre, b, q);
    return 32 * b + nth_bit(mw[b], q);
}

// Instances built for 8 waves per SIMD (at most 64 VGPRs), so two workgroups
// share a CU and one's gather overlaps the other's select phase.
constexpr bool select_low_regs(int J, int G, int NT = 1024) {
    return NT < 1024 || (J <= 16 && G <= 4);
}

// Orderable key of a position for the tie rule: an earlier (smaller, signed)
// position gives a larger key.
__device__ __forceinline__ uint32_t pos_order_key(int32_t p) { return ~((uint32_t)p ^ 0x80000000u); }

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
template <int J, int G, int MODE, int NT = kSelThreads>
__device__ __forceinline__ void select_segment(const SelectArgs& a, const int s) {
    constexpr bool CAND = MODE == SELECT_C;
    constexpr bool LOW_REGS = select_low_regs(J, G, NT);
    constexpr int NW = NT / kWave;
    // kept slots: at most the budget, and at most the J * NT entries held
    constexpr int KEPT = J * NT < kMaxBudget ? J * NT : kMaxBudget;
    static_assert(NT == kSelThreads || !CAND, "candidate lists are read by 1024-thread blocks");
    // mode C holds at most J*1024 >= N/2 candidates (launch_select), so a segment
    // has at most 64 J blocks of 32 keys (and at most 2048, N <= 65536)
    constexpr int NB = CAND ? (64 * J < 2048 ? 64 * J : 2048) : 1;
    constexpr int GZ = G > 0 ? G : 1;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[NW];
    __shared__ uint32_t pick[3];
    __shared__ uint32_t cnt_gt[J * NW], cnt_eq[J * NW];
    __shared__ int32_t kept[KEPT];
    __shared__ double scratch[(NW + 1) * GZ];
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
    uint32_t T = 0u, n_eq = 0u;
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
                                           : merge_stats<G, NT>(st, a.n_chunks, a.chunk, N, scratch);
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
                    const float* p = a.s_int + ((int64_t)s * a.cap + j * NT + tid) * G;
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
                    if (j * NT + tid < N) load_scores(j, S0[j]);
                z = merge();
#pragma unroll
                for (int j = 0; j < L0; ++j)
                    if (j * NT + tid < N) key[j] = order_key(aggregate<G>(S0[j], z));
#pragma unroll
                for (int j = L0; j < J; ++j) {
                    if (j * NT + tid < N) {
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
                const int n = j * NT + tid;
                if (n < N) key[j] = order_key(a.agg[(int64_t)s * a.agg_stride + n]);
                if ((j & 15) == 15) __builtin_amdgcn_sched_barrier(0);
            }
        }

        // ---- radix select of the B-th largest key
        need = B;
        radix_select<J, NT>(key, nv, 0ull, false, need, T, n_eq, hist, wsum, pick);

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

    // ---- ties at the cut: when more keys equal T than fit, the earliest
    // positions among them are kept.  Their register entries (bit j of eqm)
    // are overwritten with the order keys of their positions (earlier = larger)
    // and a second radix select finds the position cut P: tied keys above it
    // are kept, and of those at it (a shared position) the lowest slots.
    const bool by_pos = !all && a.tie != TIE_SLOT && (int)n_eq > need;   // block-uniform
    uint64_t eqm = 0ull;
    uint32_t P = 0u;
    if (by_pos) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int n = j * NT + tid;
            if (n < nv && key[j] == T) {
                int slot = n;
                if constexpr (CAND) slot = cand_slot(n, N, pre, mw);
                const int32_t p = a.tie == TIE_POS_ARRAY ? a.tie_pos[(int64_t)s * a.tie_stride + slot]
                                                         : a.src.pos[a.src.row(s, slot)];
                key[j] = pos_order_key(p);
                eqm |= 1ull << j;
            }
        }
        uint32_t n_eq2 = 0u;
        radix_select<J, NT>(key, nv, eqm, true, need, P, n_eq2, hist, wsum, pick);
    }
#define TRI_CLASSIFY(j, gt, eq)                                             \
    const bool valid_##j = (j) * NT + tid < nv;                    \
    bool gt, eq;                                                            \
    if (by_pos && ((eqm >> (j)) & 1u)) {                                    \
        gt = key[j] > P;                                                    \
        eq = key[j] == P;                                                   \
    } else {                                                                \
        gt = valid_##j && (all || key[j] > T);                              \
        eq = valid_##j && !all && !by_pos && key[j] == T;                   \
    }

    // ---- ordered emission: entry k = j*1024 + w*64 + lane, in (j, w, lane) order
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
    for (int j = 0; j < J; ++j) {
        TRI_CLASSIFY(j, gt, eq)
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        if (lane == 0) {
            cnt_gt[j * NW + w] = (uint32_t)__popcll(bg);
            cnt_eq[j * NW + w] = (uint32_t)__popcll(be);
        }
    }
    __syncthreads();
    {
        const uint32_t vg = tid < J * NW ? cnt_gt[tid] : 0u;
        const uint32_t ve = tid < J * NW ? cnt_eq[tid] : 0u;
        const uint32_t ig = block_incl_scan<NT>(vg, wsum);
        const uint32_t ie = block_incl_scan<NT>(ve, wsum);
        if (tid < J * NW) {
            cnt_gt[tid] = ig - vg;
            cnt_eq[tid] = ie - ve;
        }
    }
    __syncthreads();
    const int nk = min(N, B);
#pragma unroll
    for (int j = 0; j < J; ++j) {
        TRI_CLASSIFY(j, gt, eq)
        const uint64_t bg = __ballot(gt), be = __ballot(eq);
        const int eb = (int)cnt_eq[j * NW + w] + __popcll(be & below);
        const int gb = (int)cnt_gt[j * NW + w] + __popcll(bg & below);
        const int out = gb + min(eb, need);
        if ((gt || (eq && eb < need)) && out < nk) {
            int slot = j * NT + tid;
            if constexpr (CAND) {
                if (!all) slot = cand_slot(slot, N, pre, mw);
            }
            if (a.gather) kept[out] = slot;
            else a.idx_out[(int64_t)s * a.idx_stride + out] = slot;
        }
    }
#undef TRI_CLASSIFY
    __syncthreads();                                    // every wave has read lengths[s] (n_kept may alias it)
    if (a.n_kept && tid == 0) a.n_kept[s] = nk;
    if (!a.gather) return;

    const int cpr = a.row_bytes >> 4;
    const int lg = 31 - __clz(cpr);
    if (a.gather == GATHER_IN_PLACE) {
        // kept[j] >= j, and kept[j] - j does not decrease: rows j < c (kept[j] ==
        // j) stay, and every row from c on moves down to slot j.  Batches of
        // rows [j0, j0 + nb): all of a batch's rows are read into registers
        // (four 16-byte K and V pieces per thread), then, after a barrier,
        // written.  A batch writes slots below j0 + nb and later batches read
        // slots kept[j] >= j >= j0 + nb, so no row is overwritten before it is
        // read.
        int lo = 0, hi = nk;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (kept[mid] == mid) lo = mid + 1;
            else hi = mid;
        }
        // (pieces held in named registers: a local array here was placed in
        // scratch and LDS, with a wait after every load; two pieces in the
        // instances built for 64 registers)
        constexpr int UP = LOW_REGS ? 2 : 4;
        const int per = (NT * UP) >> lg;       // rows per batch (<= 512: rows are >= 128 bytes)
        for (int j0 = lo; j0 < nk; j0 += per) {
            const int lim = min(per, nk - j0) * cpr;    // 16-byte pieces in the batch
            uint4 k0, k1, k2, k3, v0, v1, v2, v3;
            int32_t pv = 0;
#define TRI_IP_LOAD(u, kx, vx)                                                              \
            if ((u) * NT + tid < lim) {                                            \
                const int e = (u) * NT + tid;                                      \
                const int64_t sr = a.src.row(s, kept[j0 + (e >> lg)]);                     \
                kx = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[e & (cpr - 1)]; \
                vx = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[e & (cpr - 1)]; \
            }
#define TRI_IP_STORE(u, kx, vx)                                                             \
            if ((u) * NT + tid < lim) {                                            \
                const int e = (u) * NT + tid;                                      \
                const int64_t dr = a.dst.row(s, j0 + (e >> lg));                           \
                reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[e & (cpr - 1)] = kx;  \
                reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[e & (cpr - 1)] = vx;  \
            }
            TRI_IP_LOAD(0, k0, v0)
            TRI_IP_LOAD(1, k1, v1)
            if constexpr (UP == 4) {
                TRI_IP_LOAD(2, k2, v2)
                TRI_IP_LOAD(3, k3, v3)
            }
            if (tid * cpr < lim) pv = a.src.pos[a.src.row(s, kept[j0 + tid])];
            // every row of the batch has been read: the loads have returned
            // (the barrier alone does not wait for them) before any wave writes
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            __syncthreads();
            TRI_IP_STORE(0, k0, v0)
            TRI_IP_STORE(1, k1, v1)
            if constexpr (UP == 4) {
                TRI_IP_STORE(2, k2, v2)
                TRI_IP_STORE(3, k3, v3)
            }
            if (tid * cpr < lim) a.dst.pos[a.dst.row(s, j0 + tid)] = pv;
#undef TRI_IP_LOAD
#undef TRI_IP_STORE
        }
        return;
    }
    if (a.gather == GATHER_IN_PLACE_FILL) {
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
            for (int r = tid; r < nb; r += NT) {
                int l2 = 0, h2 = c;
                while (l2 < h2) {
                    const int mid = (l2 + h2) >> 1;
                    if (kept[mid] - mid <= base + r) l2 = mid + 1;
                    else h2 = mid;
                }
                hist[r] = (uint32_t)(base + r + l2);
            }
            __syncthreads();
            for (int u = tid; u < nb * cpr; u += NT) {
                const int jr = u >> lg, q = u & (cpr - 1);
                const int64_t sr = a.src.row(s, kept[c + base + jr]);
                const int64_t dr = a.dst.row(s, (int)hist[jr]);
                const uint4 kv = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[q];
                const uint4 vv = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[q];
                reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[q] = kv;
                reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[q] = vv;
            }
            for (int jr = tid; jr < nb; jr += NT)
                a.dst.pos[a.dst.row(s, (int)hist[jr])] = a.src.pos[a.src.row(s, kept[c + base + jr])];
            __syncthreads();                            // hist is refilled by the next batch
        }
        return;
    }

    // ---- compaction of the kept rows (16-byte copies), then positions.  Each
    // thread issues all the loads of a batch (UG K and UG V pieces, in named
    // registers) before its stores, so a workgroup keeps UG times more bytes in
    // flight than a load-store loop, which waits out one memory round trip per
    // 16-byte piece: the gather of one workgroup then keeps up with HBM while
    // the other workgroup on its CU is in its select phase.  The copies carry
    // the non-temporal hint: nothing in the pass reads these rows again (on
    // the main workload, in one process alternating the two builds: select +
    // gather 2.01 -> 1.97 ms on one GPU, the stores' hint giving the gain;
    // unchanged on another).
    constexpr int UG = LOW_REGS ? 4 : 8;
    const int total = nk * cpr;
    for (int u0 = 0; u0 < total; u0 += NT * UG) {
        uint4 k0, k1, k2, k3, k4, k5, k6, k7, v0, v1, v2, v3, v4, v5, v6, v7;
#define TRI_G_LOAD(i, kx, vx)                                                                  \
        if (u0 + (i) * NT + tid < total) {                                            \
            const int u = u0 + (i) * NT + tid;                                        \
            const int64_t sr = a.src.row(s, kept[u >> lg]);                                    \
            kx = ld_nt(reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes) + (u & (cpr - 1))); \
            vx = ld_nt(reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes) + (u & (cpr - 1))); \
        }
#define TRI_G_STORE(i, kx, vx)                                                                 \
        if (u0 + (i) * NT + tid < total) {                                            \
            const int u = u0 + (i) * NT + tid;                                        \
            const int64_t dr = a.dst.row(s, u >> lg);                                          \
            st_nt(reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes) + (u & (cpr - 1)), kx);  \
            st_nt(reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes) + (u & (cpr - 1)), vx);  \
        }
        TRI_G_LOAD(0, k0, v0)
        TRI_G_LOAD(1, k1, v1)
        TRI_G_LOAD(2, k2, v2)
        TRI_G_LOAD(3, k3, v3)
        if constexpr (UG == 8) {
            TRI_G_LOAD(4, k4, v4)
            TRI_G_LOAD(5, k5, v5)
            TRI_G_LOAD(6, k6, v6)
            TRI_G_LOAD(7, k7, v7)
        }
        TRI_G_STORE(0, k0, v0)
        TRI_G_STORE(1, k1, v1)
        TRI_G_STORE(2, k2, v2)
        TRI_G_STORE(3, k3, v3)
        if constexpr (UG == 8) {
            TRI_G_STORE(4, k4, v4)
            TRI_G_STORE(5, k5, v5)
            TRI_G_STORE(6, k6, v6)
            TRI_G_STORE(7, k7, v7)
        }
#undef TRI_G_LOAD
#undef TRI_G_STORE
    }
    for (int jrow = tid; jrow < nk; jrow += NT)
        a.dst.pos[a.dst.row(s, jrow)] = a.src.pos[a.src.row(s, kept[jrow])];
}

// J <= 16, G <= 4 (and the 256-thread instances): at most 64 VGPRs and the
// SGPRs of 8 waves per SIMD, so two 1024-thread (or eight 256-thread)
// workgroups share a CU and one's gather overlaps another's select phase.
// The 256-thread G = 8 instances (eight heads' statistics) spill at 64 VGPRs:
// they get 5 waves per SIMD (five workgroups per CU; measured as fast on the
// GPT-OSS-shaped window prune).
constexpr int select_waves(int J, int G, int NT) { return NT < kSelThreads && G == 8 ? 5 : select_low_regs(J, G, NT) ? 8 : 1; }
template <int J, int G, int MODE, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(select_waves(J, G, NT)))) void k_select(
    SelectArgs a) {
    select_segment<J, G, MODE, NT>(a, blockIdx.x);
}

// Mode S over the segments whose candidate pass failed its certificate:
// workgroup i takes list entry i (the grid covers every segment, the most the
// list can hold; the rest exit at once).  A grid-strided loop over the list
// made the compiler keep the per-thread key arrays in scratch memory.
template <int J, int G>
__global__ __launch_bounds__(kSelThreads) void k_select_fallback(SelectArgs a) {
    if ((int)blockIdx.x < *a.fb_count) select_segment<J, G, SELECT_S>(a, a.fb_list[blockIdx.x]);
}

template <int J, int G, int NT>
static bool select_launch(const SelectArgs& a, int mode, hipStream_t stream) {
    const dim3 block(NT);
    if (mode == SELECT_S_FALLBACK) {
        if constexpr (G > 0 && NT == kSelThreads)
            hipLaunchKernelGGL((k_select_fallback<J, G>), dim3((unsigned)a.n_seg), block, 0, stream, a);
        return G > 0 && NT == kSelThreads;
    }
    const dim3 grid((unsigned)a.n_seg);
    if constexpr (G == 0) {
        hipLaunchKernelGGL((k_select<J, 0, SELECT_A, NT>), grid, block, 0, stream, a);
    } else if (mode == SELECT_C) {
        if constexpr (NT == kSelThreads) hipLaunchKernelGGL((k_select<J, G, SELECT_C, NT>), grid, block, 0, stream, a);
        else return false;
    } else {
        hipLaunchKernelGGL((k_select<J, G, SELECT_S, NT>), grid, block, 0, stream, a);
    }
    return true;
}

template <int J, int NT = kSelThreads>
static bool select_group(const SelectArgs& a, int group, int mode, hipStream_t stream) {
    if ((group == 0) != (mode == SELECT_A)) return false;
    switch (group) {
        case 0: return select_launch<J, 0, NT>(a, mode, stream);
        case 1: return select_launch<J, 1, NT>(a, mode, stream);
        case 2: return select_launch<J, 2, NT>(a, mode, stream);
        case 4: return select_launch<J, 4, NT>(a, mode, stream);
        case 8: return select_launch<J, 8, NT>(a, mode, stream);
        default: return false;
    }
}

// Segments of at most this many keys are selected by 256-thread workgroups:
// eight of them share a CU, so the latency-bound select phases (statistics
// merge, three radix passes, emission, each a chain of block barriers) of
// many short segments overlap, where a 1024-thread workgroup would hold a
// quarter of a CU for a segment that fills a fraction of its threads.
constexpr int64_t kSmallSegKeys = 4096;

hipError_t launch_select(const SelectArgs& a, int group, int mode, int64_t max_len, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    if (a.budget > kMaxBudget || max_len > 64 * kSelThreads) return hipErrorInvalidValue;
    int64_t held = max_len;                             // entries one thread block holds in registers
    if (mode == SELECT_C) {
        held = candidate_select_held(max_len, a.budget);   // a longer list: fallback (full rescoring, mode S)
        if (a.chunk % 512 || a.chunk > 2048) return hipErrorInvalidValue;
    }
    const KernelId id = mode == SELECT_S_FALLBACK ? KID_SELECT_FALLBACK : a.gather ? KID_SELECT_GATHER : KID_SELECT;
    TimedLaunch tl(id, stream);
    bool ok;
    constexpr int ST = 256;
    if (mode != SELECT_C && mode != SELECT_S_FALLBACK && held <= kSmallSegKeys) {
        if (held <= 4 * ST) ok = select_group<4, ST>(a, group, mode, stream);
        else if (held <= 8 * ST) ok = select_group<8, ST>(a, group, mode, stream);
        else ok = select_group<16, ST>(a, group, mode, stream);
    }
    else if (held <= 2 * kSelThreads) ok = select_group<2>(a, group, mode, stream);
    else if (held <= 8 * kSelThreads) ok = select_group<8>(a, group, mode, stream);
    else if (mode == SELECT_C && held <= 16 * kSelThreads) ok = select_group<16>(a, group, mode, stream);
    else if (held <= 32 * kSelThreads) ok = select_group<32>(a, group, mode, stream);
    // a 32K-key cache plus a window of up to 4K appended keys
    else if (held <= 36 * kSelThreads) ok = select_group<36>(a, group, mode, stream);
    else ok = select_group<64>(a, group, mode, stream);
    if (!ok) return hipErrorInvalidValue;
    return hipGetLastError();
}

// ------------------------------------------------------------------ split select
// The top-B of a segment computed by one 256-thread workgroup per (segment,
// chunk of keys) instead of one workgroup per segment, for batches with few or
// uneven segments, where one workgroup per segment leaves most of the chip
// idle.  Same radix select as select_segment (11 + 11 + 10 bit digits of the
// aggregate's order key), with the histograms summed over a segment's chunks
// in the workspace, one launch per digit:
//   1. each chunk forms its keys' aggregates (exactly as select_segment: the
//      same statistics merge and aggregate, so the same bits), stores their
//      order keys and adds its first-digit histogram to the segment's;
//   2, 3. each chunk reads the finished histograms of the digits before, picks
//      the digit holding the B-th key, and histograms the next digit of its
//      keys that match;
//   4. the cut T, how many keys at T to keep, and each chunk's counts of keys
//      above and at T; a segment with more keys at T than fit (the tie rule
//      needs positions) or, in candidate mode, a failed certificate goes to
//      the fallback list;
//   5. each chunk emits its kept slots at their places in slot order.
constexpr int kSplitThreads = 256;
constexpr int kSplitState = 8;     // words of per-segment state
constexpr int kSplitHist = 3 * 2048;

// Digit level lv of the radix select: shift and mask of its bits.
__device__ __forceinline__ int split_shift(int lv) { return lv == 0 ? 21 : lv == 1 ? 10 : 0; }
__device__ __forceinline__ uint32_t split_mask(int lv) { return lv < 2 ? 0x7ffu : 0x3ffu; }

// Walks the segment's finished histograms of levels 0..levels-1: the prefix
// of the cut, its mask, the keys at or above the cut still needed, and the
// count of keys in the last picked bin.
__device__ __forceinline__ void split_walk(const uint32_t* hist, int levels, int budget, uint32_t& prefix,
                                           uint32_t& pmask, int& need, uint32_t& n_at, uint32_t* wsum,
                                           uint32_t* pick) {
    constexpr int HB = 2048 / kSplitThreads;
    const int tid = threadIdx.x;
    prefix = 0u;
    pmask = 0u;
    need = budget;
    n_at = 0u;
    for (int lv = 0; lv < levels; ++lv) {
        const uint32_t* h = hist + lv * 2048;
        if (tid == 0) {
            pick[0] = 0u;
            pick[1] = 0u;
            pick[2] = 0u;
        }
        uint32_t hv[HB], hs = 0u;
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            hv[i] = h[2047 - HB * tid - i];
            hs += hv[i];
        }
        uint32_t above = block_incl_scan<kSplitThreads>(hs, wsum) - hs;     // (synchronises)
        const uint32_t un = (uint32_t)need;
#pragma unroll
        for (int i = 0; i < HB; ++i) {
            if (above < un && above + hv[i] >= un) {
                pick[0] = (uint32_t)(2047 - HB * tid - i);
                pick[1] = above;
                pick[2] = hv[i];
            }
            above += hv[i];
        }
        __syncthreads();
        prefix |= pick[0] << split_shift(lv);
        pmask |= split_mask(lv) << split_shift(lv);
        need -= (int)pick[1];
        n_at = pick[2];
        __syncthreads();
    }
}

// Segment statistics as select_segment merges them (bit for bit).
template <int G>
__device__ __forceinline__ ZParams<G> split_zparams(const SplitSelArgs& a, int s, int N, double* scratch) {
    const double2* st = a.stats + (int64_t)s * a.n_chunks * G;
    return a.n_chunks <= kWave ? merge_stats_wave<G>(st, a.n_chunks, a.chunk, N)
                               : merge_stats<G, kSplitThreads>(st, a.n_chunks, a.chunk, N, scratch);
}

__global__ __launch_bounds__(256) void k_split_fill(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

// Launch 1: aggregates of chunk (blockIdx.x) of segment (blockIdx.y), their
// order keys, and the segment's first-digit histogram.
template <int G, bool CAND>
__global__ __launch_bounds__(kSplitThreads) void k_split_first(SplitSelArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ double scratch[(kSplitThreads / kWave + 1) * G];
    __shared__ uint32_t hw[64 * G], fl[64], lp[64], unl[1];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int c0 = c * a.chunk;
    if (N <= a.budget || c0 >= N) return;
    const int cnt = min(a.chunk, N - c0);
    const ZParams<G> z = split_zparams<G>(a, s, N, scratch);
    for (int b = tid; b < 2048; b += kSplitThreads) hist[b] = 0u;
    if constexpr (CAND) {
        // the chunk's mask words and, per block, the floats listed before it in
        // its wave's list (blocks r, r - 4, ... were scored by the same wave)
        const int nbk = (cnt + 31) / 32;
        if (tid < nbk) {
            const uint32_t* mp = a.masks + ((int64_t)s * a.mask_stride + c0 / 32 + tid) * G;
            uint32_t f = 0u;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                hw[tid * G + g] = mp[g];
                f += __popc(mp[g]);
            }
            fl[tid] = f;
        }
        if (tid == 0) unl[0] = 0u;
        __syncthreads();
        if (tid < nbk) {
            uint32_t before = 0u;
            for (int r = tid - 4; r >= 0; r -= 4) before += fl[r];
            lp[tid] = before;
        }
    }
    __syncthreads();
    uint32_t unlisted = 0u;
    for (int i = tid; i < cnt; i += kSplitThreads) {
        const int k = c0 + i;
        uint32_t key;
        if constexpr (CAND) {
            const int r = i >> 5, bit = i & 31;
            const uint32_t below = (1u << bit) - 1u;
            uint32_t any = 0u;
            int foff = 0;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                any |= hw[r * G + g] >> bit;
                foff += __popc(hw[r * G + g] & below);
            }
            if (any & 1u) {
                const int base = wave_list_base(r & 3, cnt);
                const float* p = a.s_int + ((int64_t)s * a.cap + c0 + base) * G + lp[r] + foff;
                float A = -__builtin_inff();
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    if ((hw[r * G + g] >> bit) & 1u) {
                        const float S = *p++;
                        A = fmaxf(A, ((S - z.mu_hi[g]) - z.mu_lo[g]) * z.inv[g]);
                    }
                }
                key = order_key(A);
            } else {
                key = 0u;                                 // below every listed key; covered by the certificate
                ++unlisted;
            }
        } else {
            float S[G];
            const float* p = a.s_int + ((int64_t)s * a.cap + k) * G;
#pragma unroll
            for (int g = 0; g < G; ++g) S[g] = p[g];
            key = order_key(aggregate<G>(S, z));
        }
        a.akey[(int64_t)s * a.cap + k] = key;
        atomicAdd(&hist[key >> 21], 1u);
    }
    if constexpr (CAND) {
        if (unlisted) atomicAdd(&unl[0], unlisted);
    }
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)s * kSplitHist;
    for (int b = tid; b < 2048; b += kSplitThreads)
        if (hist[b]) atomicAdd(&gh[b], hist[b]);
    if constexpr (CAND) {
        if (tid == 0 && unl[0]) atomicAdd(&a.state[(int64_t)s * kSplitState + 4], unl[0]);
    }
}

// Launches 2 and 3: histogram of digit LV of the keys matching the cut's
// prefix so far.
template <int LV>
__global__ __launch_bounds__(kSplitThreads) void k_split_next(SplitSelArgs a) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kSplitThreads / kWave], pick[3];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    const int c0 = c * a.chunk;
    if (N <= a.budget || c0 >= N) return;
    const int cnt = min(a.chunk, N - c0);
    uint32_t* gh = a.hist + (int64_t)s * kSplitHist;
    uint32_t prefix, pmask, n_at;
    int need;
    split_walk(gh, LV, a.budget, prefix, pmask, need, n_at, wsum, pick);
    for (int b = tid; b < 2048; b += kSplitThreads) hist[b] = 0u;
    __syncthreads();
    const uint32_t* ak = a.akey + (int64_t)s * a.cap + c0;
    for (int i = tid; i < cnt; i += kSplitThreads) {
        const uint32_t key = ak[i];
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> split_shift(LV)) & split_mask(LV)], 1u);
    }
    __syncthreads();
    for (int b = tid; b < 2048; b += kSplitThreads)
        if (hist[b]) atomicAdd(&gh[LV * 2048 + b], hist[b]);
}

// Launch 4: the cut, the fallback decision, and each chunk's counts of keys
// above and at the cut.
template <int G, bool CAND>
__global__ __launch_bounds__(kSplitThreads) void k_split_count(SplitSelArgs a) {
    __shared__ uint32_t wsum[kSplitThreads / kWave], pick[3], red[2 * kSplitThreads / kWave];
    __shared__ double scratch[(kSplitThreads / kWave + 1) * G];
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid / kWave;
    const int N = (int)min((int64_t)max(a.lengths[s], 0), a.cap);
    uint32_t* st = a.state + (int64_t)s * kSplitState;
    if (c == 0 && tid == 0) st[0] = (uint32_t)N;      // launch 5 reads N here (n_kept may alias lengths)
    const int c0 = c * a.chunk;
    if (N <= a.budget || c0 >= N) return;
    const int cnt = min(a.chunk, N - c0);
    uint32_t T, pmask, n_at;
    int need;
    split_walk(a.hist + (int64_t)s * kSplitHist, 3, a.budget, T, pmask, need, n_at, wsum, pick);
    bool fallback = (int)n_at > need;                 // keys tied at the cut beyond the budget: by position
    if constexpr (CAND) {
        if (!fallback && st[4] > 0u) {                // some keys unlisted: the certificate
            const ZParams<G> z = split_zparams<G>(a, s, N, scratch);
            float L[G];
#pragma unroll
            for (int g = 0; g < G; ++g) L[g] = a.thr[(int64_t)s * G + g];
            fallback = !(T > order_key(aggregate<G>(L, z)));
        }
    }
    if (fallback) {
        if (c == 0 && tid == 0) {
            st[3] = 1u;
            a.fb_list[atomicAdd(a.fb_count, 1)] = s;
        }
        return;
    }
    if (c == 0 && tid == 0) {
        st[1] = T;
        st[2] = (uint32_t)need;
    }
    const uint32_t* ak = a.akey + (int64_t)s * a.cap + c0;
    uint32_t ngt = 0u, neq = 0u;
    for (int i = tid; i < cnt; i += kSplitThreads) {
        const uint32_t key = ak[i];
        ngt += key > T;
        neq += key == T;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        ngt += __shfl_xor(ngt, m, kWave);
        neq += __shfl_xor(neq, m, kWave);
    }
    if (lane == 0) {
        red[2 * w] = ngt;
        red[2 * w + 1] = neq;
    }
    __syncthreads();
    if (tid == 0) {
        uint32_t g2 = 0u, e2 = 0u;
        for (int i = 0; i < kSplitThreads / kWave; ++i) {
            g2 += red[2 * i];
            e2 += red[2 * i + 1];
        }
        a.ccnt[((int64_t)s * a.n_chunks + c) * 2] = g2;
        a.ccnt[((int64_t)s * a.n_chunks + c) * 2 + 1] = e2;
    }
}

// Copy of kept rows [o0, o0 + n) of segment s, whose source slots are
// src_of[0 .. n), by the whole workgroup (16-byte chunks; positions after).
__device__ __forceinline__ void split_copy_rows(const SplitSelArgs& a, int s, int o0, int n, const int32_t* src_of) {
    const int cpr = a.row_bytes >> 4;
    const int lg = 31 - __clz(cpr);
    for (int u = threadIdx.x; u < n * cpr; u += kSplitThreads) {
        const int jrow = u >> lg, q = u & (cpr - 1);
        const int64_t sr = a.src.row(s, src_of[jrow]);
        const int64_t dr = a.dst.row(s, o0 + jrow);
        const uint4 kv = reinterpret_cast<const uint4*>(a.src.k + sr * a.row_bytes)[q];
        const uint4 vv = reinterpret_cast<const uint4*>(a.src.v + sr * a.row_bytes)[q];
        reinterpret_cast<uint4*>(a.dst.k + dr * a.row_bytes)[q] = kv;
        reinterpret_cast<uint4*>(a.dst.v + dr * a.row_bytes)[q] = vv;
    }
    for (int jrow = threadIdx.x; jrow < n; jrow += kSplitThreads)
        a.dst.pos[a.dst.row(s, o0 + jrow)] = a.src.pos[a.src.row(s, src_of[jrow])];
}

// Launch 5: kept slots of the chunk, each at its place in slot order
// (out = keys above the cut before it + min(keys at the cut before it, need)).
// A chunk's kept keys take consecutive places, so with `gather` the
// workgroup then copies that run of rows.
__global__ __launch_bounds__(kSplitThreads) void k_split_emit(SplitSelArgs a) {
    __shared__ uint32_t wsum[kSplitThreads / kWave], bg_w[kSplitThreads / kWave], be_w[kSplitThreads / kWave];
    __shared__ uint32_t base[2];
    __shared__ int32_t src_of[2048];                  // gather: source slot of the chunk's kept place o0 + j
    const int s = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), w = tid / kWave;
    const uint32_t* st = a.state + (int64_t)s * kSplitState;
    const int N = (int)st[0];
    const int c0 = c * a.chunk;
    int32_t* idx = a.idx + (int64_t)s * a.idx_stride;
    if (N <= a.budget) {                              // every key kept, in slot order
        const int end = min(N, c0 + a.chunk);
        for (int i = c0 + tid; i < end; i += kSplitThreads) {
            idx[i] = i;
            if (a.gather) src_of[i - c0] = i;
        }
        if (c == 0 && tid == 0 && a.n_kept) a.n_kept[s] = N;
        if (a.gather && end > c0) {
            __syncthreads();
            split_copy_rows(a, s, c0, end - c0, src_of);
        }
        return;
    }
    if (c0 >= N || st[3]) return;                     // no keys here, or left to the fallback
    const int cnt = min(a.chunk, N - c0);
    const uint32_t T = st[1];
    const int need = (int)st[2];
    // keys above and at the cut in the chunks before this one
    {
        uint32_t g2 = 0u, e2 = 0u;
        for (int cc = tid; cc < c; cc += kSplitThreads) {
            g2 += a.ccnt[((int64_t)s * a.n_chunks + cc) * 2];
            e2 += a.ccnt[((int64_t)s * a.n_chunks + cc) * 2 + 1];
        }
        const uint32_t gi = block_incl_scan<kSplitThreads>(g2, wsum);
        if (tid == kSplitThreads - 1) base[0] = gi;
        const uint32_t ei = block_incl_scan<kSplitThreads>(e2, wsum);
        if (tid == kSplitThreads - 1) base[1] = ei;
        __syncthreads();
    }
    uint32_t gb = base[0], eb = base[1];
    const int o0 = (int)min(gb + min(eb, (uint32_t)need), (uint32_t)a.budget);   // the chunk's first place
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const uint32_t* ak = a.akey + (int64_t)s * a.cap + c0;
    for (int i0 = 0; i0 < cnt; i0 += kSplitThreads) {   // block-uniform
        const int i = i0 + tid;
        const uint32_t key = i < cnt ? ak[i] : 0u;
        const bool gt = i < cnt && key > T, eq = i < cnt && key == T;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        if (lane == 0) {
            bg_w[w] = (uint32_t)__popcll(mg);
            be_w[w] = (uint32_t)__popcll(me);
        }
        __syncthreads();
        uint32_t g_before = gb + (uint32_t)__popcll(mg & below), e_before = eb + (uint32_t)__popcll(me & below);
        uint32_t g_all = 0u, e_all = 0u;
        for (int v = 0; v < kSplitThreads / kWave; ++v) {
            if (v < w) {
                g_before += bg_w[v];
                e_before += be_w[v];
            }
            g_all += bg_w[v];
            e_all += be_w[v];
        }
        if (gt || (eq && (int)e_before < need)) {
            const uint32_t out = g_before + min(e_before, (uint32_t)need);
            if (out < (uint32_t)a.budget) {
                idx[out] = c0 + i;
                if (a.gather) src_of[out - o0] = c0 + i;
            }
        }
        gb += g_all;
        eb += e_all;
        __syncthreads();                                // bg_w / be_w are rewritten next pass
    }
    if (c == 0 && tid == 0 && a.n_kept) a.n_kept[s] = a.budget;
    if (a.gather) {
        const int o1 = (int)min(gb + min(eb, (uint32_t)need), (uint32_t)a.budget);   // past the chunk's last place
        if (o1 > o0) split_copy_rows(a, s, o0, o1 - o0, src_of);      // (src_of complete: the loop's last barrier)
    }
}

// Histograms, then the state words, from SplitSelArgs::hist.
int64_t split_select_zero_words(int64_t n_seg) {
    static_assert(kSplitHist % 64 == 0, "the state words follow the histograms");
    return n_seg * (kSplitHist + kSplitState);
}

template <int G>
static void split_launch_g(const SplitSelArgs& a, bool cand, hipStream_t stream) {
    const dim3 grid((unsigned)a.n_chunks, (unsigned)a.n_seg), block(kSplitThreads);
    if (cand) hipLaunchKernelGGL((k_split_first<G, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_split_first<G, false>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(k_split_next<1>, grid, block, 0, stream, a);
    hipLaunchKernelGGL(k_split_next<2>, grid, block, 0, stream, a);
    if (cand) hipLaunchKernelGGL((k_split_count<G, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((k_split_count<G, false>), grid, block, 0, stream, a);
    hipLaunchKernelGGL(k_split_emit, grid, block, 0, stream, a);
}

hipError_t launch_split_select(const SplitSelArgs& a, int group, bool cand, hipStream_t stream) {
    if (a.n_seg == 0) return hipSuccess;
    if (a.budget > kMaxBudget || a.chunk % 32 || a.chunk > 2048 || a.n_chunks > 65535) return hipErrorInvalidValue;
    TimedLaunch tl(KID_SPLIT_SELECT, stream);
    // histograms and state start at zero
    if (!a.zeroed) {
        const int64_t words = split_select_zero_words(a.n_seg);
        const int64_t fill_blocks = (words + 255) / 256 < 4096 ? (words + 255) / 256 : 4096;
        hipLaunchKernelGGL(k_split_fill, dim3((unsigned)fill_blocks), dim3(256), 0, stream, a.hist, words);
    }
    switch (group) {
        case 1: split_launch_g<1>(a, cand, stream); break;
        case 2: split_launch_g<2>(a, cand, stream); break;
        case 4: split_launch_g<4>(a, cand, stream); break;
        case 8: split_launch_g<8>(a, cand, stream); break;
        default: return hipErrorInvalidValue;
    }
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
