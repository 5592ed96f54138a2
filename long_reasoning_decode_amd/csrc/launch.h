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
    KID_COUNT
};

// Brackets one launch with HIP events when timing is enabled.
struct TimedLaunch {
    TimedLaunch(int id, hipStream_t stream);
    ~TimedLaunch();
    int id;
    hipStream_t stream;
    hipEvent_t start = nullptr, stop = nullptr;
};

// --- phase: ctab[l][b][hq][0..F) = Re C, [F..D) = Im C, with
//     C = P[layer0 + l][hq][f] * e^{i w_f t_b} evaluated in fp64.
struct PhaseArgs {
    const double2* P;       // [L_calib][Hq][F]
    const double* omega;    // [F]
    const int32_t* t;       // [n_seq]
    float* ctab;            // [n_layers][n_seq][Hq][D]
    int32_t layer0, n_layers, n_seq, n_q_heads, head_dim;
};
hipError_t launch_phase(const PhaseArgs& a, hipStream_t stream);

// --- score: raw per-head scores of every key, plus per-chunk (mean, M2).
struct ScoreArgs {
    CacheView kv;
    SegShape shape;
    const int32_t* lengths;
    const float* ctab;      // [n_layers][n_seq][Hq][D]
    const float* wtab;      // [n_layers][Hq][F]  ((1 - R) M, from layer0)
    float* s_raw;           // optional [n_seg][G][cap]
    float* s_int;           // optional [n_seg][cap][G]
    double2* stats;         // [n_seg][n_chunks][G]
    int64_t cap;
    int32_t n_q_heads;
    int32_t chunk;          // keys per block (multiple of 256)
    int32_t n_chunks;
    int32_t n_seg;
};
hipError_t launch_score(const ScoreArgs& a, int head_dim, int group, bool bf16, hipStream_t stream);

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
    const float* s_int;     // mode S: [n_seg][cap][G] + chunk stats
    const double2* stats;
    int32_t n_chunks, chunk;
    int64_t cap;
    const int32_t* lengths;
    int32_t budget;
    int32_t* idx_out;       // optional [n_seg][idx_stride]
    int64_t idx_stride;
    int32_t* n_kept;        // optional [n_seg]
    int32_t gather;         // 1: copy kept rows src -> dst
    CacheView src;
    CacheOut dst;
    int32_t row_bytes;
    int32_t n_seg;
};
hipError_t launch_select(const SelectArgs& a, int group /*0 = mode A*/, int64_t max_len,
                         hipStream_t stream);

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

}  // namespace tri
