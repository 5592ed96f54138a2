// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace tri {

// Kernel ids for the timing instrumentation (order = tri_timing_name).
enum KernelId : int {
    KID_PHASE = 0,
    KID_SCORE,
    KID_ZMAX,
    KID_SELECT,
    KID_SELECT_GATHER,
    KID_GATHER,
    KID_APPEND,
    KID_DECODE_ATTN,
    KID_SAMPLE,
    KID_SCORE_FALLBACK,
    KID_SELECT_FALLBACK,
    KID_CALIB,
    KID_CALIB_FINAL,
    KID_SPLIT_SELECT,
    KID_COUNT
};

// Whether the fused pass of a segment with N keys and budget B runs on a
// candidate list (keys whose score can reach the top B) instead of every key.
// Small segments, and budgets above 1/8 of the segment, keep every key.
__host__ __device__ inline bool candidate_mode(int64_t N, int64_t B) { return N >= 4096 && N >= 8 * B; }
// Entries the candidate-mode select holds per workgroup for segments of up to
// max_len keys: every key of a segment outside candidate mode (N < max(4096,
// 8B)), or half of the longest segment's keys (the sampled threshold admits
// about 2.5B/N of them, at most 5/16 since N >= 8B); a longer list sends its
// segment to the fallback.
inline int64_t candidate_select_held(int64_t max_len, int64_t budget) {
    const int64_t small = 8 * budget > 4096 ? 8 * budget : 4096;
    const int64_t half = (max_len + 1) / 2 > small ? (max_len + 1) / 2 : small;
    return half < max_len ? half : max_len;
}

// In candidate mode, wave w of a scoring workgroup scores the 32-key blocks
// w, w+4, w+8, ... of its chunk; its candidate list starts after the keys of
// waves 0..w-1, so the four lists of a chunk of cnt keys fill at most the
// scratch rows of those cnt keys.
__device__ inline int wave_keys(int w, int cnt) {
    const int full = cnt / 32, rem = cnt % 32;
    int n = full > w ? (full - w + 3) / 4 * 32 : 0;
    if (rem && (full & 3) == w) n += rem;
    return n;
}
__device__ inline int wave_list_base(int w, int cnt) {
    int b = 0;
    for (int i = 0; i < w; ++i) b += wave_keys(i, cnt);
    return b;
}

// Brackets one launch with HIP events when timing is enabled.
struct TimedLaunch {
    TimedLaunch(int id, hipStream_t stream);
    ~TimedLaunch();
    int id;
    hipStream_t stream;
    int device = 0;
    hipEvent_t start = nullptr, stop = nullptr;
};

// --- phase: ctab[l][b][hq][0..F) = Re C, [F..D) = Im C, with
//     C = P[layer0 + l][hq][f] * e^{i w_f t_b} evaluated in fp64.
struct PhaseArgs {
    const double2* P;       // [L_calib][Hq][F]
    const double* omega;    // [F]
    const int32_t* t;       // [n_seq]
    float* ctab;            // [n_layers][n_seq][Hq][D]
    int32_t* fb_reset;      // optional: a pruning pass without candidate mode zeroes its fallback count
    uint32_t* zero;         // optional: words [0, zero_words) cleared (the split select's histograms)
    int64_t zero_words;
    int32_t layer0, n_layers, n_seq, n_q_heads, head_dim;
};
hipError_t launch_phase(const PhaseArgs& a, hipStream_t stream);

// --- candidate thresholds: per segment and head, L_h from a key sample.
struct SampleArgs {
    CacheView kv;
    SegShape shape;
    const int32_t* lengths;
    const float* ctab;
    const float* wtab;
    float* thr;             // [n_seg][G]
    int32_t* fb_count;      // zeroed here (the pass's fallback counter)
    int64_t cap;
    int32_t n_q_heads, budget, n_seg;
};
hipError_t launch_sample(const SampleArgs& a, int head_dim, int group, hipStream_t stream);

// --- score: raw per-head scores of every key, plus per-chunk (mean, M2).
struct ScoreArgs {
    CacheView kv;
    SegShape shape;
    const int32_t* lengths;
    const float* ctab;      // [n_layers][n_seq][Hq][D]
    const float* wtab;      // [n_layers][Hq][F]  ((1 - R) M, from layer0)
    float* s_raw;           // optional [n_seg][G][cap]
    float* s_int;           // optional [n_seg][cap][G]; candidate mode: per-wave candidate lists
    double2* stats;         // [n_seg][n_chunks][G]
    const float* thr;       // candidate mode: [n_seg][G] thresholds L_h
    uint32_t* masks;        // candidate mode: [n_seg][mask_stride][G], bit i of word (b, h): key 32 b + i passed head h
    int64_t mask_stride;
    const int32_t* fb_list; // fallback mode: segments to redo, and their count
    const int32_t* fb_count;
    int64_t cap;
    int32_t n_q_heads;
    int32_t chunk;          // keys per block (multiple of 512)
    int32_t n_chunks;
    int32_t n_seg;
};
enum ScoreMode : int { SCORE_FULL = 0, SCORE_CANDIDATES = 1, SCORE_FALLBACK = 2 };
hipError_t launch_score(const ScoreArgs& a, int head_dim, int group, bool bf16, int mode, hipStream_t stream);

// --- zmax: merge chunk statistics, A = max_h z_h for every key.
struct ZmaxArgs {
    const float* s_raw;     // one of s_raw / s_int
    const float* s_int;
    const double2* stats;
    const int32_t* lengths;
    float* agg;             // [n_seg][cap]
    float* mu_sigma;        // optional [n_seg][G][2]
    int64_t cap;
    int32_t chunk, n_chunks, n_seg;
};
hipError_t launch_zmax(const ZmaxArgs& a, int group, hipStream_t stream);

// --- select (and, in gather mode, compaction) with one workgroup per segment.
struct SelectArgs {
    const float* agg;       // mode A: [n_seg][agg_stride]
    int64_t agg_stride;
    const float* s_int;     // mode S: [n_seg][cap][G] + chunk stats; mode C: candidate lists
    const double2* stats;
    const float* thr;       // mode C: thresholds, candidate masks, fallback list
    const uint32_t* masks;
    int64_t mask_stride;
    int32_t* fb_list;
    int32_t* fb_count;
    int32_t n_chunks, chunk;
    int64_t cap;
    const int32_t* lengths;
    int32_t budget;
    int32_t* idx_out;       // optional [n_seg][idx_stride]
    int64_t idx_stride;
    int32_t* n_kept;        // optional [n_seg]
    int32_t gather;         // GatherMode
    int32_t tie;            // TieMode: how keys tied at the cut are ordered
    const int32_t* tie_pos; // TIE_POS_ARRAY: positions [n_seg][tie_stride]
    int64_t tie_stride;
    CacheView src;
    CacheOut dst;
    int32_t row_bytes;
    int32_t n_seg;
};
// GATHER_COPY: kept row j of each segment -> dst slot j (dst is another cache).
// GATHER_IN_PLACE: dst is src; kept row j -> slot j as in GATHER_COPY (slot
// order kept).  kept[j] >= j, so rows move down only; the rows before the
// first freed slot stay, and the rest move in batches: each batch reads all
// its rows, then (after a barrier) writes them, and later batches read only
// slots at or above what earlier ones wrote.
// GATHER_IN_PLACE_FILL: dst is src; kept rows below n_kept stay, the kept rows
// at or above n_kept move into the freed slots below it, in ascending order
// (reads only from slots >= n_kept, writes only to slots < n_kept: no overlap).
enum GatherMode : int { GATHER_NONE = 0, GATHER_COPY = 1, GATHER_IN_PLACE = 2, GATHER_IN_PLACE_FILL = 3 };
// Order among keys tied at the cut: the lower slot (TIE_SLOT), or the earlier
// position, then the lower slot; positions from tie_pos (TIE_POS_ARRAY) or
// from the source cache (TIE_POS_CACHE).
enum TieMode : int { TIE_SLOT = 0, TIE_POS_ARRAY = 1, TIE_POS_CACHE = 2 };
// mode A: select on aggregated scores (group 0); S: on interleaved scores;
// C: on candidate lists, with the certificate and fallback list; S_FALLBACK:
// mode S over the segments listed in fb_list.
enum SelectMode : int { SELECT_A = 0, SELECT_S = 1, SELECT_C = 2, SELECT_S_FALLBACK = 3 };
hipError_t launch_select(const SelectArgs& a, int group, int mode, int64_t max_len, hipStream_t stream);

// --- split select: the top-B of each segment over many workgroups, one per
// (segment, chunk of keys), in five launches (aggregate + first digit
// histogram, second digit, third digit, per-chunk counts, ordered emission).
// Kept slots go to idx (rows idx_stride apart) and n_kept; the rows are then
// copied by launch_gather.  A segment whose keys tie at the cut with more
// keys than fit (the position rule needs the single-workgroup select), or in
// candidate mode whose certificate fails, is listed in fb_list and left to
// the fallback kernels.
struct SplitSelArgs {
    const float* s_int;     // mode S: [n_seg][cap][G]; mode C: the chunks' candidate lists
    const double2* stats;   // [n_seg][n_chunks][G]
    const float* thr;       // mode C: [n_seg][G]
    const uint32_t* masks;  // mode C: [n_seg][mask_stride][G]
    int64_t mask_stride;
    int32_t chunk, n_chunks;
    int64_t cap;
    const int32_t* lengths;
    int32_t budget;
    uint32_t* akey;         // workspace [n_seg][cap]: order keys of the aggregates
    uint32_t* hist;         // workspace [n_seg][3][2048]: digit histograms (zeroed by the first launch's fill,
                            // or beforehand when `zeroed`: split_select_zero_words words from hist)
    uint32_t* ccnt;         // workspace [n_seg][n_chunks][2]: keys above / at the cut per chunk
    uint32_t* state;        // workspace [n_seg][4]: N, cut, how many at the cut to keep, fallback flag
    int32_t* fb_list;
    int32_t* fb_count;
    int32_t* idx;           // [n_seg][idx_stride]
    int64_t idx_stride;
    int32_t* n_kept;
    int32_t n_seg;
    bool zeroed;            // hist and state already cleared (by the phase kernel of the same pass)
    bool gather;            // the emission also copies each kept row (K, V, position) from src to dst
    CacheView src;
    CacheOut dst;
    int32_t row_bytes;
};
int64_t split_select_zero_words(int64_t n_seg);
hipError_t launch_split_select(const SplitSelArgs& a, int group, bool cand, hipStream_t stream);

// --- gather (unfused compaction)
struct GatherArgs {
    CacheView src;
    CacheOut dst;
    const int32_t* idx;
    int64_t idx_stride;
    const int32_t* n_kept;
    int32_t row_bytes;
    int32_t rows_per_block;
    int32_t blocks_per_seg;
    int32_t n_seg;
};
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

// --- decode-loop helpers
struct AppendArgs {
    CacheOut kv;
    int32_t* lengths;
    const uint8_t* k_new;
    const uint8_t* v_new;
    const int32_t* pos_new;
    SegShape shape;
    int32_t row_bytes, n_seg;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

struct AttnArgs {
    CacheView kv;
    SegShape shape;
    const int32_t* lengths;
    const uint8_t* q;       // [n_layers][n_seq][Hq][D]
    float* out;             // same shape, fp32
    float scale;
    int32_t n_q_heads, n_seg;
};
hipError_t launch_decode_attn(const AttnArgs& a, int head_dim, int group, bool bf16,
                              hipStream_t stream);

// --- offline calibration from sampled pre-RoPE queries
constexpr int kCalibBands = 4;             // bands per pass-1 lane
// Samples per pass-1 wave: sized so the waves (layers x chunks x blocks of 64
// band groups) are about one round of what the chip holds at once (256 CUs x
// 4 SIMDs x 4 waves); a second, partial round
// would take as long as the first.  At least 64 samples (the fp64 partials
// then stay under a sixth of the samples' bytes), a multiple of 8 (one batch).
constexpr int kCalibResidentWaves = 4096;
inline int calib_chunk_len(int n_layers, int n_samples, int n_q_heads, int head_dim) {
    const int64_t blocks = (int64_t)n_layers * ((n_q_heads * (head_dim / 2 / kCalibBands) + 63) / 64);
    const int64_t chunks = blocks >= kCalibResidentWaves ? 1 : kCalibResidentWaves / blocks;
    int64_t len = (n_samples + chunks - 1) / chunks;
    len = len < 64 ? 64 : (len + 7) / 8 * 8;
    return (int)len;
}
struct CalibArgs {
    const uint8_t* q;       // [L][n_samples][Hq][d] stored rows
    double* part;           // [L][n_chunks][Hq][F][5] fp64 partial sums
    float* mag;             // [L][Hq][F]
    float* phase;
    float* conc;
    int32_t n_layers, n_samples, n_q_heads, head_dim, n_chunks, chunk_len;
};
hipError_t launch_calibrate(const CalibArgs& a, bool bf16, hipStream_t stream);

}  // namespace tri
