// C ABI of the TriAttention pruning library: argument validation, the
// calibration handle, workspace planning, kernel dispatch and the optional
// kernel timing.  Declarations and contracts: include/triattn.h.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <map>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/triattn.h"
#include "launch.h"

using namespace tri;

struct tri_calib_s {
    int L, Hq, Hkv, G, D, F, n_off;
    double theta;
    void* dev;         // one device allocation holding the three tables below
    double2* P;        // [L][Hq][F]  M e^{i phi} * mean_o e^{i w_f o}
    float* wnorm;      // [L][Hq][F]  (1 - R) M
    double* omega;     // [F]
};

namespace {

constexpr int kMaxLen = 65536;
constexpr int kMaxBudget = 8192;
constexpr int kMinChunk = 512;

// ---------------------------------------------------------------- timing
struct PendingTiming {
    int id, device;
    hipEvent_t start, stop;
};
std::mutex g_tmu;
bool g_timing = false;
uint32_t g_timing_mask = ~0u;                   // kernel ids timed when enabled
std::vector<PendingTiming> g_pending;
// Timing events are reused (per device): creating two events for every launch
// cost the host more than a small pass's kernels take.
std::map<int, std::vector<hipEvent_t>> g_free_events;

hipEvent_t take_event_locked(int device) {
    auto& f = g_free_events[device];
    if (!f.empty()) {
        hipEvent_t e = f.back();
        f.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
}
int64_t g_launches[KID_COUNT] = {};
double g_ms[KID_COUNT] = {};
const char* kKernelNames[KID_COUNT] = {"phase",  "score",  "zmax",   "select",         "select_gather",
                                       "gather", "append", "decode_attn", "sample", "score_fallback",
                                       "select_fallback", "calibrate", "calibrate_final", "split_select"};

void drain_timing_locked() {
    for (auto& p : g_pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.stop) == hipSuccess && hipEventElapsedTime(&ms, p.start, p.stop) == hipSuccess) {
            g_ms[p.id] += ms;
            g_launches[p.id] += 1;
        }
        g_free_events[p.device].push_back(p.start);
        g_free_events[p.device].push_back(p.stop);
    }
    g_pending.clear();
}

// ---------------------------------------------------------------- helpers
int device_present() {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    return 1;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Workspaces start on a 256-byte boundary (every device allocation does):
// their regions sit at 256-byte offsets and are read with vector loads.
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int elem_size(int dtype) { return dtype == TRI_DTYPE_BF16 ? 2 : 4; }

int64_t n_segments(const tri_cache_desc* kv) {
    return (int64_t)kv->n_layers * kv->n_seq * kv->n_kv_heads;
}

// Validates the shape and pointers of a cache descriptor.
int check_cache(const tri_cache_desc* kv) {
    if (!kv) return TRI_ERR_INVALID_ARG;
    if (kv->dtype != TRI_DTYPE_F32 && kv->dtype != TRI_DTYPE_BF16) return TRI_ERR_INVALID_ARG;
    if (kv->layout != TRI_LAYOUT_DENSE && kv->layout != TRI_LAYOUT_PAGED) return TRI_ERR_INVALID_ARG;
    if (kv->n_layers < 1 || kv->layer0 < 0 || kv->n_seq < 1 || kv->n_kv_heads < 1) return TRI_ERR_INVALID_ARG;
    if (kv->head_dim <= 0 || (kv->head_dim & 1) || kv->capacity < 1) return TRI_ERR_INVALID_ARG;
    if (!kv->k || !kv->v || !kv->pos || !kv->lengths) return TRI_ERR_INVALID_ARG;
    if (kv->layout == TRI_LAYOUT_PAGED) {
        if (kv->page_size < 1 || kv->max_pages < 1 || !kv->page_table) return TRI_ERR_INVALID_ARG;
        if ((int64_t)kv->page_size * kv->max_pages != kv->capacity) return TRI_ERR_INVALID_ARG;
    }
    if (n_segments(kv) > (int64_t)0x7fffffff) return TRI_ERR_UNSUPPORTED;
    if (kv->head_dim != 64 && kv->head_dim != 128) return TRI_ERR_UNSUPPORTED;
    return TRI_OK;
}

int check_calib_vs_cache(const tri_calib_s* c, const tri_cache_desc* kv) {
    if (!c) return TRI_ERR_INVALID_ARG;
    if (kv->head_dim != c->D || kv->n_kv_heads != c->Hkv) return TRI_ERR_INVALID_ARG;
    if ((int64_t)kv->layer0 + kv->n_layers > c->L) return TRI_ERR_INVALID_ARG;
    return TRI_OK;
}

int page_shift_of(const tri_cache_desc* kv) {
    if (kv->layout != TRI_LAYOUT_PAGED) return -1;
    const int ps = kv->page_size;
    if (ps <= 0 || (ps & (ps - 1))) return -1;
    int sh = 0;
    while ((1 << sh) < ps) ++sh;
    return sh;
}

CacheView view_of(const tri_cache_desc* kv) {
    CacheView v;
    v.k = static_cast<const uint8_t*>(kv->k);
    v.v = static_cast<const uint8_t*>(kv->v);
    v.pos = kv->pos;
    v.page_table = kv->layout == TRI_LAYOUT_PAGED ? kv->page_table : nullptr;
    v.capacity = kv->capacity;
    v.page_size = kv->layout == TRI_LAYOUT_PAGED ? kv->page_size : 0;
    v.page_shift = page_shift_of(kv);
    v.max_pages = kv->layout == TRI_LAYOUT_PAGED ? kv->max_pages : 0;
    v.row_bytes = kv->head_dim * elem_size(kv->dtype);
    return v;
}

CacheOut out_of(const tri_cache_desc* kv) {
    CacheOut o;
    o.k = static_cast<uint8_t*>(kv->k);
    o.v = static_cast<uint8_t*>(kv->v);
    o.pos = kv->pos;
    o.page_table = kv->layout == TRI_LAYOUT_PAGED ? kv->page_table : nullptr;
    o.capacity = kv->capacity;
    o.page_size = kv->layout == TRI_LAYOUT_PAGED ? kv->page_size : 0;
    o.page_shift = page_shift_of(kv);
    o.max_pages = kv->layout == TRI_LAYOUT_PAGED ? kv->max_pages : 0;
    return o;
}

SegShape shape_of(const tri_cache_desc* kv) {
    SegShape s;
    s.n_seq = kv->n_seq;
    s.n_kv_heads = kv->n_kv_heads;
    return s;
}

// Keys per scoring workgroup: 2048 when that still gives >= 2048 workgroups,
// else smaller (down to 512) so small caches spread over the chip.  Paged
// caches start at 1024: they hold sequences of unequal length, and on such a
// batch (lengths 4K..64K) 1024-key chunks scored 13% faster than 2048 (512:
// 10%), while on equal 32K segments 2048 is the faster one.
int pick_chunk(const tri_cache_desc* kv) {
    const int64_t n_seg = n_segments(kv), cap = kv->capacity;
    int chunk = kv->layout == TRI_LAYOUT_PAGED ? 1024 : 2048;
    while (chunk > kMinChunk && n_seg * ((cap + chunk - 1) / chunk) < 2048) chunk >>= 1;
    return chunk;
}

// Workspace layout.  The fallback counter of the last pruning pass sits at
// offset 0 so tri_prune_fallbacks can find it without the cache shape.
struct WsPlan {
    size_t fb_count, fb_list, ctab, stats, thr, masks, s_int, idx, akey, shist, ccnt, total;
    int64_t mask_stride;
};

// Fewer segments than CUs: one select+gather workgroup per segment would copy
// each segment's kept rows with one workgroup while most of the chip idles.
// The pruning pass then has the select kernels write the kept slots to the
// workspace, and the unfused gather copies them with B/64 workgroups per
// segment.
constexpr int64_t kSplitGatherSegs = 256;
bool split_gather(const tri_cache_desc* kv) { return n_segments(kv) < kSplitGatherSegs; }

// Fewer segments than CUs, of many keys: the select runs one workgroup per
// (segment, chunk) (launch_split_select) instead of one per segment, which
// would leave most CUs idle (one 32K-key layer: 8 workgroups; its select 57 ->
// about 40 us).  Out of place only; the kept rows are then copied by the
// many-workgroup gather.  Not for batches that fill the GPU: on the ragged
// batch (512 segments of 4K..64K keys) the split select and the separate
// gather took 0.55 + 0.46 ms against 0.75 ms for the fused select + gather.
constexpr int64_t kSplitSelectMinCap = 8192;
bool split_select(const tri_cache_desc* kv) {
    return n_segments(kv) < kSplitGatherSegs && kv->capacity >= kSplitSelectMinCap;
}
constexpr int kSplitHistWords = 3 * 2048 + 8;      // per segment: three digit histograms, then its state

WsPlan plan_workspace(const tri_calib_s* c, const tri_cache_desc* kv) {
    const int64_t n_seg = n_segments(kv);
    const int64_t max_chunks = (kv->capacity + kMinChunk - 1) / kMinChunk;
    WsPlan p;
    p.mask_stride = (kv->capacity + 31) / 32;
    p.fb_count = 0;
    p.fb_list = 256;
    p.ctab = p.fb_list + align256((size_t)n_seg * sizeof(int32_t));
    p.stats = p.ctab + align256((size_t)kv->n_layers * kv->n_seq * c->Hq * c->D * sizeof(float));
    p.thr = p.stats + align256((size_t)n_seg * max_chunks * c->G * sizeof(double2));
    p.masks = p.thr + align256((size_t)n_seg * c->G * sizeof(float));
    p.s_int = p.masks + align256((size_t)n_seg * p.mask_stride * c->G * sizeof(uint32_t));
    p.idx = p.s_int + align256((size_t)n_seg * kv->capacity * c->G * sizeof(float));
    const int64_t idx_len = kv->capacity < kMaxBudget ? kv->capacity : kMaxBudget;   // budget <= both
    const bool ssel = split_select(kv);
    p.akey = p.idx + (split_gather(kv) || ssel ? align256((size_t)n_seg * idx_len * sizeof(int32_t)) : 0);
    p.shist = p.akey + (ssel ? align256((size_t)n_seg * kv->capacity * sizeof(uint32_t)) : 0);
    p.ccnt = p.shist + (ssel ? align256((size_t)n_seg * kSplitHistWords * sizeof(uint32_t)) : 0);
    p.total = p.ccnt + (ssel ? align256((size_t)n_seg * max_chunks * 2 * sizeof(uint32_t)) : 0);
    return p;
}

// Detail of the most recent TRI_ERR_HIP on this thread (see tri_last_error).
thread_local char t_last_error[192] = "";

int hip_status(hipError_t e, const char* step = "launch") {
    if (e == hipSuccess) return TRI_OK;
    snprintf(t_last_error, sizeof t_last_error, "%s: %s (%d)", step, hipGetErrorString(e), (int)e);
    return TRI_ERR_HIP;
}

// phase + score shared by tri_score and tri_prune_window.
// With `cand` (bf16 pruning pass): the sample kernel sets candidate thresholds
// and the score kernel writes candidate lists and masks instead of every score.
int run_phase_and_score(const tri_calib_s* c, const tri_cache_desc* kv, const int32_t* t, float* s_raw,
                        float* s_int, double2* stats, float* ctab, int chunk, hipStream_t st,
                        const WsPlan* cand = nullptr, char* ws = nullptr, int budget = 0,
                        int32_t* fb_reset = nullptr, uint32_t* zero = nullptr, int64_t zero_words = 0) {
    PhaseArgs pa;
    pa.fb_reset = fb_reset;
    pa.zero = zero;
    pa.zero_words = zero ? zero_words : 0;
    pa.P = c->P;
    pa.omega = c->omega;
    pa.t = t;
    pa.ctab = ctab;
    pa.layer0 = kv->layer0;
    pa.n_layers = kv->n_layers;
    pa.n_seq = kv->n_seq;
    pa.n_q_heads = c->Hq;
    pa.head_dim = c->D;
    int rc = hip_status(launch_phase(pa, st), "phase kernel");
    if (rc) return rc;

    ScoreArgs sa;
    sa.kv = view_of(kv);
    sa.shape = shape_of(kv);
    sa.lengths = kv->lengths;
    sa.ctab = ctab;
    sa.wtab = c->wnorm + (int64_t)kv->layer0 * c->Hq * c->F;
    sa.s_raw = s_raw;
    sa.s_int = s_int;
    sa.stats = stats;
    sa.cap = kv->capacity;
    sa.n_q_heads = c->Hq;
    sa.chunk = chunk;
    sa.n_chunks = (int)((kv->capacity + chunk - 1) / chunk);
    sa.n_seg = (int)n_segments(kv);
    sa.thr = nullptr;
    sa.masks = nullptr;
    sa.mask_stride = 0;
    sa.fb_list = nullptr;
    sa.fb_count = nullptr;
    int mode = SCORE_FULL;
    if (cand) {
        SampleArgs pa2;
        pa2.kv = sa.kv;
        pa2.shape = sa.shape;
        pa2.lengths = kv->lengths;
        pa2.ctab = ctab;
        pa2.wtab = sa.wtab;
        pa2.thr = reinterpret_cast<float*>(ws + cand->thr);
        pa2.fb_count = reinterpret_cast<int32_t*>(ws + cand->fb_count);
        pa2.cap = kv->capacity;
        pa2.n_q_heads = c->Hq;
        pa2.budget = budget;
        pa2.n_seg = sa.n_seg;
        if ((rc = hip_status(launch_sample(pa2, c->D, c->G, st), "sample kernel"))) return rc;
        sa.thr = pa2.thr;
        sa.masks = reinterpret_cast<uint32_t*>(ws + cand->masks);
        sa.mask_stride = cand->mask_stride;
        mode = SCORE_CANDIDATES;
    }
    return hip_status(launch_score(sa, c->D, c->G, kv->dtype == TRI_DTYPE_BF16, mode, st), "score kernel");
}

}  // namespace

// ---------------------------------------------------------------- timing hooks
namespace tri {
TimedLaunch::TimedLaunch(int id_, hipStream_t s) : id(id_), stream(s) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (!g_timing || !((g_timing_mask >> id) & 1u) || hipGetDevice(&device) != hipSuccess) return;
    start = take_event_locked(device);
    stop = take_event_locked(device);
    if (!start || !stop) {
        if (start) g_free_events[device].push_back(start);
        if (stop) g_free_events[device].push_back(stop);
        start = stop = nullptr;
        return;
    }
    (void)hipEventRecord(start, stream);
}
TimedLaunch::~TimedLaunch() {
    if (!start) return;
    std::lock_guard<std::mutex> lk(g_tmu);
    (void)hipEventRecord(stop, stream);
    g_pending.push_back({id, device, start, stop});
}
}  // namespace tri

extern "C" {

const char* tri_strerror(int code) {
    switch (code) {
        case TRI_OK: return "ok";
        case TRI_ERR_INVALID_ARG: return "invalid argument";
        case TRI_ERR_UNSUPPORTED: return "unsupported shape or type";
        case TRI_ERR_WORKSPACE: return "workspace missing or too small";
        case TRI_ERR_HIP: return "HIP runtime or launch error";
        case TRI_ERR_NO_DEVICE: return "no GPU device";
        default: return "unknown status";
    }
}

int tri_calib_load(tri_calib_t* out, int n_layers, int n_q_heads, int n_kv_heads, int head_dim,
                   double rope_theta, const float* mag, const float* phase, const float* conc,
                   const int32_t* offsets, int n_offsets, tri_stream_t stream) {
    return tri_calib_load_ex(out, n_layers, n_q_heads, n_kv_heads, head_dim, rope_theta, mag, phase, conc, offsets,
                             n_offsets, 0, stream);
}

int tri_calib_load_ex(tri_calib_t* out, int n_layers, int n_q_heads, int n_kv_heads, int head_dim,
                      double rope_theta, const float* mag, const float* phase, const float* conc,
                      const int32_t* offsets, int n_offsets, int variant, tri_stream_t stream) {
    if (!out || n_layers < 1 || n_q_heads < 1 || n_kv_heads < 1 || head_dim <= 0 || (head_dim & 1))
        return TRI_ERR_INVALID_ARG;
    if ((variant & ~(TRI_VARIANT_TRIG_ONLY | TRI_VARIANT_NORM_ONLY | TRI_VARIANT_FIXED_WEIGHT |
                     TRI_VARIANT_R_WEIGHTED_TRIG)) ||
        ((variant & TRI_VARIANT_TRIG_ONLY) && (variant & TRI_VARIANT_NORM_ONLY)))
        return TRI_ERR_INVALID_ARG;
    if (n_q_heads % n_kv_heads) return TRI_ERR_INVALID_ARG;
    if (!(rope_theta > 0.0) || !isfinite(rope_theta)) return TRI_ERR_INVALID_ARG;
    if (!mag || !phase || !conc || !offsets || n_offsets < 1) return TRI_ERR_INVALID_ARG;
    const int F = head_dim / 2;
    const int64_t n = (int64_t)n_layers * n_q_heads * F;
    for (int64_t i = 0; i < n; ++i) {
        if (!isfinite(mag[i]) || mag[i] < 0.0f || !isfinite(phase[i])) return TRI_ERR_INVALID_ARG;
        if (!(conc[i] >= 0.0f && conc[i] <= 1.0f)) return TRI_ERR_INVALID_ARG;
    }
    for (int i = 0; i < n_offsets; ++i)
        if (offsets[i] < 0) return TRI_ERR_INVALID_ARG;
    const int G = n_q_heads / n_kv_heads;
    if ((head_dim != 64 && head_dim != 128) || !supported_group(G)) return TRI_ERR_UNSUPPORTED;
    if (!device_present()) return TRI_ERR_NO_DEVICE;

    // Host-side fp64 folding of the offset average into one coefficient per band.
    std::vector<double> omega(F);
    std::vector<double2> A(F);
    for (int f = 0; f < F; ++f) {
        omega[f] = pow(rope_theta, -2.0 * (double)f / (double)head_dim);
        double re = 0.0, im = 0.0;
        for (int o = 0; o < n_offsets; ++o) {
            re += cos(omega[f] * (double)offsets[o]);
            im += sin(omega[f] * (double)offsets[o]);
        }
        A[f] = make_double2(re / n_offsets, im / n_offsets);
    }
    std::vector<double2> P((size_t)n);
    std::vector<float> wn((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
        const int f = (int)(i % F);
        double m = (double)mag[i];
        if (variant & TRI_VARIANT_R_WEIGHTED_TRIG) m *= (double)conc[i];
        if (variant & TRI_VARIANT_NORM_ONLY) m = 0.0;
        const double cr = m * cos((double)phase[i]);
        const double ci = m * sin((double)phase[i]);
        P[i] = make_double2(cr * A[f].x - ci * A[f].y, cr * A[f].y + ci * A[f].x);
        const double wt = (variant & TRI_VARIANT_FIXED_WEIGHT) ? 1.0 : 1.0 - (double)conc[i];
        wn[i] = (variant & TRI_VARIANT_TRIG_ONLY) ? 0.0f : (float)(wt * (double)mag[i]);
    }

    tri_calib_s* c = new (std::nothrow) tri_calib_s();
    if (!c) return TRI_ERR_INVALID_ARG;
    const size_t bP = align256(sizeof(double2) * (size_t)n);
    const size_t bW = align256(sizeof(float) * (size_t)n);
    const size_t bO = align256(sizeof(double) * (size_t)F);
    if (hipMalloc(&c->dev, bP + bW + bO) != hipSuccess) {
        delete c;
        return TRI_ERR_HIP;
    }
    c->P = static_cast<double2*>(c->dev);
    c->wnorm = reinterpret_cast<float*>(static_cast<char*>(c->dev) + bP);
    c->omega = reinterpret_cast<double*>(static_cast<char*>(c->dev) + bP + bW);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(c->P, P.data(), sizeof(double2) * n, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(c->wnorm, wn.data(), sizeof(float) * n, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(c->omega, omega.data(), sizeof(double) * F, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        (void)hipFree(c->dev);
        delete c;
        return TRI_ERR_HIP;
    }
    c->L = n_layers;
    c->Hq = n_q_heads;
    c->Hkv = n_kv_heads;
    c->G = G;
    c->D = head_dim;
    c->F = F;
    c->n_off = n_offsets;
    c->theta = rope_theta;
    *out = c;
    return TRI_OK;
}

int tri_calib_free(tri_calib_t calib) {
    if (!calib) return TRI_OK;
    int rc = TRI_OK;
    if (hipDeviceSynchronize() != hipSuccess) rc = TRI_ERR_HIP;
    if (hipFree(calib->dev) != hipSuccess) rc = TRI_ERR_HIP;
    delete calib;
    return rc;
}

int tri_workspace_size(tri_calib_t calib, const tri_cache_desc* kv, int budget, size_t* bytes) {
    if (!bytes || !calib) return TRI_ERR_INVALID_ARG;
    int rc = check_cache(kv);
    if (rc) return rc;
    if ((rc = check_calib_vs_cache(calib, kv))) return rc;
    if (budget < 1) return TRI_ERR_INVALID_ARG;
    *bytes = plan_workspace(calib, kv).total;
    return TRI_OK;
}

int tri_score(tri_calib_t calib, const tri_cache_desc* kv, const int32_t* t, float* scores, float* agg,
              float* mu_sigma, void* ws, size_t ws_bytes, tri_stream_t stream) {
    int rc = check_cache(kv);
    if (rc) return rc;
    if ((rc = check_calib_vs_cache(calib, kv))) return rc;
    if (!t || !agg) return TRI_ERR_INVALID_ARG;
    if (kv->capacity > kMaxLen) return TRI_ERR_UNSUPPORTED;
    const WsPlan p = plan_workspace(calib, kv);
    if (!ws || ws_bytes < p.total || !aligned256(ws)) return TRI_ERR_WORKSPACE;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    float* ctab = reinterpret_cast<float*>(w + p.ctab);
    double2* stats = reinterpret_cast<double2*>(w + p.stats);
    float* s_int = scores ? nullptr : reinterpret_cast<float*>(w + p.s_int);
    const int chunk = pick_chunk(kv);
    if ((rc = run_phase_and_score(calib, kv, t, scores, s_int, stats, ctab, chunk, st))) return rc;
    ZmaxArgs za;
    za.s_raw = scores;
    za.s_int = s_int;
    za.stats = stats;
    za.lengths = kv->lengths;
    za.agg = agg;
    za.mu_sigma = mu_sigma;
    za.cap = kv->capacity;
    za.chunk = chunk;
    za.n_chunks = (int)((kv->capacity + chunk - 1) / chunk);
    za.n_seg = (int)n_segments(kv);
    return hip_status(launch_zmax(za, calib->G, st), "aggregation kernel");
}

int tri_select_topb(const float* agg, const int32_t* lengths, int n_seg, int capacity, int budget,
                    int32_t* idx, int32_t* n_kept, void* ws, size_t ws_bytes, tri_stream_t stream) {
    return tri_select_topb_ex(agg, nullptr, lengths, n_seg, capacity, budget, idx, n_kept, ws, ws_bytes, stream);
}

int tri_select_topb_ex(const float* agg, const int32_t* pos, const int32_t* lengths, int n_seg, int capacity,
                       int budget, int32_t* idx, int32_t* n_kept, void* ws, size_t ws_bytes, tri_stream_t stream) {
    (void)ws;
    (void)ws_bytes;
    if (!agg || !lengths || !idx || n_seg < 0 || capacity < 1 || budget < 1) return TRI_ERR_INVALID_ARG;
    if (capacity > kMaxLen || budget > kMaxBudget) return TRI_ERR_UNSUPPORTED;
    if (n_seg == 0) return TRI_OK;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    SelectArgs a;
    memset(&a, 0, sizeof a);
    a.agg = agg;
    a.agg_stride = capacity;
    a.lengths = lengths;
    a.budget = budget;
    a.idx_out = idx;
    a.idx_stride = budget;
    a.n_kept = n_kept;
    a.gather = 0;
    a.tie = pos ? TIE_POS_ARRAY : TIE_SLOT;
    a.tie_pos = pos;
    a.tie_stride = capacity;
    a.n_seg = n_seg;
    a.cap = capacity;
    return hip_status(launch_select(a, 0, SELECT_A, capacity, static_cast<hipStream_t>(stream)), "select kernel");
}

// dst names exactly the storage of src (same rows for every slot).
static bool same_storage(const tri_cache_desc* s, const tri_cache_desc* d) {
    if (s->k != d->k || s->v != d->v || s->pos != d->pos) return false;
    if (s->layout != d->layout || s->capacity != d->capacity || s->layer0 != d->layer0) return false;
    if (s->layout == TRI_LAYOUT_PAGED)
        return s->page_table == d->page_table && s->page_size == d->page_size && s->max_pages == d->max_pages;
    return true;
}

// Bytes a dense cache's k (or v) array spans, and its pos array.
static int64_t dense_kv_bytes(const tri_cache_desc* c) {
    return n_segments(c) * (int64_t)c->capacity * c->head_dim * elem_size(c->dtype);
}
static bool ranges_meet(const void* a, int64_t na, const void* b, int64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

// Whether dst's storage may overlap src's where a compaction writes.  Dense
// caches: any byte of dst's k, v or pos arrays inside src's (their extents
// are known).  Paged caches: a pool's size is not in the descriptor, so only
// the base addresses are compared; two paged caches on the same pool with
// different page tables are accepted (the caller guarantees that dst's pages
// are not src's pages: fresh pages of a shared pool), any other shared base is
// refused.
static bool storage_overlaps(const tri_cache_desc* s, const tri_cache_desc* d) {
    if (s->layout == TRI_LAYOUT_DENSE && d->layout == TRI_LAYOUT_DENSE) {
        const int64_t ns = dense_kv_bytes(s), nd = dense_kv_bytes(d);
        const int64_t ps = n_segments(s) * (int64_t)s->capacity * 4, pd = n_segments(d) * (int64_t)d->capacity * 4;
        const void* sa[3] = {s->k, s->v, s->pos};
        const int64_t sn[3] = {ns, ns, ps};
        const void* da[3] = {d->k, d->v, d->pos};
        const int64_t dn[3] = {nd, nd, pd};
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                if (ranges_meet(sa[i], sn[i], da[j], dn[j])) return true;
        return false;
    }
    const bool same_base = d->k == s->k || d->v == s->v || d->pos == s->pos || d->k == s->v || d->v == s->k;
    if (s->layout == TRI_LAYOUT_PAGED && d->layout == TRI_LAYOUT_PAGED && same_base)
        return !(d->k == s->k && d->v == s->v && d->pos == s->pos && d->page_table != s->page_table);
    return same_base;
}

// src -> dst compaction arguments.  With `in_place` non-null, a dst that names
// src's storage is accepted (and reported); any other overlap is an error.
// dst must hold `budget` rows per segment for tri_compact (its kept counts
// come from the caller), and min(budget, src capacity) for a pruning pass,
// which keeps at most that many (a cache smaller than the budget is copied
// through, or left as it is in place).
static int check_pair(const tri_cache_desc* src, const tri_cache_desc* dst, int budget, bool* in_place = nullptr,
                      bool pruning = false) {
    int rc = check_cache(src);
    if (rc) return rc;
    if ((rc = check_cache(dst))) return rc;
    if (src->dtype != dst->dtype || src->head_dim != dst->head_dim || src->n_layers != dst->n_layers ||
        src->n_seq != dst->n_seq || src->n_kv_heads != dst->n_kv_heads)
        return TRI_ERR_INVALID_ARG;
    if (budget < 1) return TRI_ERR_INVALID_ARG;
    const int64_t rows = pruning && src->capacity < budget ? src->capacity : budget;
    if (dst->capacity < rows) return TRI_ERR_INVALID_ARG;
    if (in_place) *in_place = same_storage(src, dst);
    if (!(in_place && *in_place) && storage_overlaps(src, dst)) return TRI_ERR_INVALID_ARG;
    if (budget > kMaxBudget) return TRI_ERR_UNSUPPORTED;
    return TRI_OK;
}

int tri_compact(const tri_cache_desc* src, const int32_t* idx, const int32_t* n_kept, int budget,
                const tri_cache_desc* dst, tri_stream_t stream) {
    int rc = check_pair(src, dst, budget);
    if (rc) return rc;
    if (!idx || !n_kept) return TRI_ERR_INVALID_ARG;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    GatherArgs a;
    a.src = view_of(src);
    a.dst = out_of(dst);
    a.idx = idx;
    a.idx_stride = budget;
    a.n_kept = n_kept;
    a.row_bytes = src->head_dim * elem_size(src->dtype);
    a.rows_per_block = 64;
    a.blocks_per_seg = (budget + 63) / 64;
    a.n_seg = (int)n_segments(src);
    return hip_status(launch_gather(a, static_cast<hipStream_t>(stream)), "gather kernel");
}

// Segments below which the automatic path scores every key: they cannot fill
// the GPU, and the candidate pass's sample and fallback launches then cost
// more than the score writes it saves (one 32K-key layer, 8 segments: 0.17 ms
// with the candidate pass, 0.13 ms without).
constexpr int64_t kCandidateMinSegs = 256;
// Candidate lists the automatic path lets one select workgroup hold: up to
// 16 entries per thread, two workgroups share a CU and one's gather hides the
// other's list rebuild.  Longer lists (segments below 8B keep every key, so
// a cache of 64K-key capacity at B = 4096 holds 32K) leave one workgroup per
// CU, where rebuilding the lists costs more than the score writes the pass
// saves (the ragged batch: 1.74 ms with the candidate pass, 1.65 ms without).
constexpr int64_t kCandidateMaxHeld = 16 * 1024;

// ---------------------------------------------------------------- library-owned scratch
// Workspace of tri_prune_window_static: a file-scope device array, so the
// entry point allocates nothing.  The loader places one copy on every device
// the library runs on, held until the process ends.  In host code `scratch`
// is only a stand-in for the symbol: its device address on the current device
// comes from hipGetSymbolAddress, taken once per device on the first call
// there, and only that address is ever handed to kernels.
static __device__ __align__(256) unsigned char scratch[TRI_STATIC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;    // device -> address of that device's copy of `scratch`

static int static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "scratch: current device");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it == g_scratch_addr.end()) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "scratch: symbol address");
        if (!p || !aligned256(p)) {
            snprintf(t_last_error, sizeof t_last_error, "scratch: symbol address %p not 256-byte aligned", p);
            return TRI_ERR_HIP;
        }
        it = g_scratch_addr.emplace(dev, p).first;
    }
    *out = it->second;
    return TRI_OK;
}

// use_static: the workspace is the library's `scratch` on the current device
// (ws and ws_bytes are ignored), for caches whose workspace fits in it.
static int prune_window(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                        const tri_cache_desc* dst, int32_t* n_kept, void* ws, size_t ws_bytes, int path,
                        tri_stream_t stream, bool use_static = false) {
    const bool fill = (path & TRI_INPLACE_FILL_FREED) != 0;
    path &= ~TRI_INPLACE_FILL_FREED;
    if (path != TRI_PATH_AUTO && path != TRI_PATH_FULL && path != TRI_PATH_CANDIDATES) return TRI_ERR_INVALID_ARG;
    bool in_place = false;
    int rc = check_pair(src, dst, budget, &in_place, true);
    if (rc) return rc;
    if ((rc = check_calib_vs_cache(calib, src))) return rc;
    if (!t || !n_kept) return TRI_ERR_INVALID_ARG;
    if (src->capacity > kMaxLen) return TRI_ERR_UNSUPPORTED;
    const WsPlan p = plan_workspace(calib, src);
    if (use_static) {
        if (p.total > (size_t)TRI_STATIC_SCRATCH_BYTES) {
            snprintf(t_last_error, sizeof t_last_error,
                     "the pass needs %zu bytes of workspace; the library's scratch holds %zu", p.total,
                     (size_t)TRI_STATIC_SCRATCH_BYTES);
            return TRI_ERR_WORKSPACE;
        }
        if (!device_present()) return TRI_ERR_NO_DEVICE;
        if ((rc = static_scratch(&ws))) return rc;
        ws_bytes = TRI_STATIC_SCRATCH_BYTES;
    }
    if (!ws || ws_bytes < p.total || !aligned256(ws)) return TRI_ERR_WORKSPACE;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(ws);
    float* ctab = reinterpret_cast<float*>(w + p.ctab);
    double2* stats = reinterpret_cast<double2*>(w + p.stats);
    float* s_int = reinterpret_cast<float*>(w + p.s_int);
    const int chunk = pick_chunk(src);
    // bf16 caches that can hold a segment long enough for candidate mode:
    // candidate pass (sample -> score lists -> certified select), then the full
    // path for any segment whose certificate failed (both fallback kernels exit
    // at once when none did); the automatic choice also wants enough segments
    // to fill the GPU.  Otherwise (fp32, capacity below what candidate mode
    // needs, or the full path asked for): the full path.
    const bool cand = src->dtype == TRI_DTYPE_BF16 && candidate_mode(src->capacity, budget) &&
                      (path == TRI_PATH_CANDIDATES ||
                       (path == TRI_PATH_AUTO && n_segments(src) >= kCandidateMinSegs &&
                        candidate_select_held(src->capacity, budget) <= kCandidateMaxHeld));
    // (without candidate mode nothing falls back: the phase kernel zeroes the count tri_prune_fallbacks reads;
    // with the split select it also clears that select's histograms)
    const bool ssel = !in_place && split_select(src);
    if ((rc = run_phase_and_score(calib, src, t, nullptr, s_int, stats, ctab, chunk, st, cand ? &p : nullptr, w,
                                  budget, cand ? nullptr : reinterpret_cast<int32_t*>(w + p.fb_count),
                                  ssel ? reinterpret_cast<uint32_t*>(w + p.shist) : nullptr,
                                  ssel ? split_select_zero_words(n_segments(src)) : 0)))
        return rc;
    SelectArgs a;
    memset(&a, 0, sizeof a);
    a.s_int = s_int;
    a.stats = stats;
    a.chunk = chunk;
    a.n_chunks = (int)((src->capacity + chunk - 1) / chunk);
    a.cap = src->capacity;
    a.lengths = src->lengths;
    a.budget = budget;
    a.n_kept = n_kept;
    const bool split = !in_place && (split_gather(src) || ssel);
    a.gather = in_place ? (fill ? GATHER_IN_PLACE_FILL : GATHER_IN_PLACE) : split ? GATHER_NONE : GATHER_COPY;
    a.tie = TIE_POS_CACHE;
    a.src = view_of(src);
    a.dst = out_of(dst);
    a.row_bytes = src->head_dim * elem_size(src->dtype);
    a.n_seg = (int)n_segments(src);
    // split: kept-slot rows min(budget, capacity) apart (a segment keeps at most that many)
    const int64_t idx_stride = budget < src->capacity ? budget : src->capacity;
    if (split) {
        a.idx_out = reinterpret_cast<int32_t*>(w + p.idx);
        a.idx_stride = idx_stride;
    }
    // split: every select kernel has written its segments' kept slots; copy them
    // (the split select's emission copies its rows itself, and its fallback
    // select gathers the segments it takes)
    auto gather_split = [&]() -> int {
        if (!split || ssel) return TRI_OK;
        GatherArgs ga;
        ga.src = a.src;
        ga.dst = a.dst;
        ga.idx = a.idx_out;
        ga.idx_stride = idx_stride;
        ga.n_kept = n_kept;
        ga.row_bytes = a.row_bytes;
        ga.rows_per_block = 64;
        ga.blocks_per_seg = (budget + 63) / 64;
        ga.n_seg = a.n_seg;
        return hip_status(launch_gather(ga, st), "gather kernel");
    };
    if (ssel) {
        // split select; segments it lists (ties at the cut beyond the budget,
        // failed certificates) go through the fallback kernels below
        SplitSelArgs ss;
        ss.s_int = s_int;
        ss.stats = stats;
        ss.thr = reinterpret_cast<const float*>(w + p.thr);
        ss.masks = reinterpret_cast<const uint32_t*>(w + p.masks);
        ss.mask_stride = p.mask_stride;
        ss.chunk = chunk;
        ss.n_chunks = a.n_chunks;
        ss.cap = src->capacity;
        ss.lengths = src->lengths;
        ss.budget = budget;
        ss.akey = reinterpret_cast<uint32_t*>(w + p.akey);
        ss.hist = reinterpret_cast<uint32_t*>(w + p.shist);
        ss.ccnt = reinterpret_cast<uint32_t*>(w + p.ccnt);
        ss.state = ss.hist + (int64_t)a.n_seg * 3 * 2048;
        ss.fb_list = reinterpret_cast<int32_t*>(w + p.fb_list);
        ss.fb_count = reinterpret_cast<int32_t*>(w + p.fb_count);
        ss.idx = a.idx_out;
        ss.idx_stride = idx_stride;
        ss.n_kept = n_kept;
        ss.n_seg = a.n_seg;
        ss.zeroed = true;
        ss.gather = true;
        ss.src = a.src;
        ss.dst = a.dst;
        ss.row_bytes = a.row_bytes;
        if ((rc = hip_status(launch_split_select(ss, calib->G, cand, st), "split select kernels"))) return rc;
        a.fb_list = ss.fb_list;
        a.fb_count = ss.fb_count;
        a.gather = GATHER_COPY;                       // the fallback select copies its segments' rows
        if (!cand) {
            if ((rc = hip_status(launch_select(a, calib->G, SELECT_S_FALLBACK, src->capacity, st),
                                 "fallback select kernel")))
                return rc;
            return gather_split();
        }
    } else if (!cand) {
        if ((rc = hip_status(launch_select(a, calib->G, SELECT_S, src->capacity, st), "select+gather kernel")))
            return rc;
        return gather_split();
    }
    a.thr = reinterpret_cast<const float*>(w + p.thr);
    a.masks = reinterpret_cast<const uint32_t*>(w + p.masks);
    a.mask_stride = p.mask_stride;
    a.fb_list = reinterpret_cast<int32_t*>(w + p.fb_list);
    a.fb_count = reinterpret_cast<int32_t*>(w + p.fb_count);
    if (!ssel && (rc = hip_status(launch_select(a, calib->G, SELECT_C, src->capacity, st), "select+gather kernel")))
        return rc;
    ScoreArgs sa;
    memset(&sa, 0, sizeof sa);
    sa.kv = a.src;
    sa.shape = shape_of(src);
    sa.lengths = src->lengths;
    sa.ctab = ctab;
    sa.wtab = calib->wnorm + (int64_t)src->layer0 * calib->Hq * calib->F;
    sa.s_int = s_int;
    sa.stats = stats;
    sa.fb_list = a.fb_list;
    sa.fb_count = a.fb_count;
    sa.cap = src->capacity;
    sa.n_q_heads = calib->Hq;
    sa.chunk = chunk;
    sa.n_chunks = a.n_chunks;
    sa.n_seg = a.n_seg;
    if ((rc = hip_status(launch_score(sa, calib->D, calib->G, true, SCORE_FALLBACK, st), "fallback score kernel")))
        return rc;
    if ((rc = hip_status(launch_select(a, calib->G, SELECT_S_FALLBACK, src->capacity, st), "fallback select kernel")))
        return rc;
    return gather_split();
}

int tri_prune_window(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                     const tri_cache_desc* dst, int32_t* n_kept, void* ws, size_t ws_bytes,
                     tri_stream_t stream) {
    return prune_window(calib, src, t, budget, dst, n_kept, ws, ws_bytes, TRI_PATH_AUTO, stream);
}

int tri_prune_window_ex(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                        const tri_cache_desc* dst, int32_t* n_kept, void* ws, size_t ws_bytes, int path,
                        tri_stream_t stream) {
    return prune_window(calib, src, t, budget, dst, n_kept, ws, ws_bytes, path, stream);
}

int tri_prune_window_static(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                            const tri_cache_desc* dst, int32_t* n_kept, int path, tri_stream_t stream) {
    return prune_window(calib, src, t, budget, dst, n_kept, nullptr, 0, path, stream, true);
}

int tri_prune_fallbacks(const void* ws, size_t ws_bytes, int32_t* count, tri_stream_t stream) {
    if (!ws || !count || ws_bytes < sizeof(int32_t)) return TRI_ERR_INVALID_ARG;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(count, ws, sizeof(int32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    return hip_status(e, "fallback count read");
}

int tri_append(const tri_cache_desc* kv, const void* k_new, const void* v_new, const int32_t* pos_new,
               tri_stream_t stream) {
    int rc = check_cache(kv);
    if (rc) return rc;
    if (!k_new || !v_new || !pos_new) return TRI_ERR_INVALID_ARG;
    if (kv->layout != TRI_LAYOUT_DENSE) return TRI_ERR_UNSUPPORTED;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    AppendArgs a;
    a.kv = out_of(kv);
    a.lengths = kv->lengths;
    a.k_new = static_cast<const uint8_t*>(k_new);
    a.v_new = static_cast<const uint8_t*>(v_new);
    a.pos_new = pos_new;
    a.shape = shape_of(kv);
    a.row_bytes = kv->head_dim * elem_size(kv->dtype);
    a.n_seg = (int)n_segments(kv);
    return hip_status(launch_append(a, static_cast<hipStream_t>(stream)), "append kernel");
}

int tri_decode_attn(const tri_cache_desc* kv, int n_q_heads, const void* q, float scale, float* out,
                    tri_stream_t stream) {
    int rc = check_cache(kv);
    if (rc) return rc;
    if (!q || !out || n_q_heads < 1 || n_q_heads % kv->n_kv_heads || !isfinite(scale)) return TRI_ERR_INVALID_ARG;
    const int G = n_q_heads / kv->n_kv_heads;
    if (!supported_group(G)) return TRI_ERR_UNSUPPORTED;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    AttnArgs a;
    a.kv = view_of(kv);
    a.shape = shape_of(kv);
    a.lengths = kv->lengths;
    a.q = static_cast<const uint8_t*>(q);
    a.out = out;
    a.scale = scale;
    a.n_q_heads = n_q_heads;
    a.n_seg = (int)n_segments(kv);
    return hip_status(launch_decode_attn(a, kv->head_dim, G, kv->dtype == TRI_DTYPE_BF16,
                                         static_cast<hipStream_t>(stream)), "decode attention kernel");
}

static int check_calib_shape(int n_layers, int n_samples, int n_q_heads, int head_dim) {
    if (n_layers < 1 || n_samples < 1 || n_q_heads < 1 || head_dim <= 0 || (head_dim & 1)) return TRI_ERR_INVALID_ARG;
    if (head_dim != 64 && head_dim != 128) return TRI_ERR_UNSUPPORTED;
    return TRI_OK;
}

static size_t calib_ws_bytes(int n_layers, int n_samples, int n_q_heads, int head_dim) {
    const int len = calib_chunk_len(n_layers, n_samples, n_q_heads, head_dim);
    const int64_t chunks = (n_samples + len - 1) / len;
    return align256((size_t)n_layers * chunks * n_q_heads * (head_dim / 2) * 5 * sizeof(double));
}

int tri_calibrate_workspace_size(int n_layers, int n_samples, int n_q_heads, int head_dim, size_t* bytes) {
    if (!bytes) return TRI_ERR_INVALID_ARG;
    const int rc = check_calib_shape(n_layers, n_samples, n_q_heads, head_dim);
    if (rc) return rc;
    *bytes = calib_ws_bytes(n_layers, n_samples, n_q_heads, head_dim);
    return TRI_OK;
}

int tri_calibrate(const void* q, int dtype, int n_layers, int n_samples, int n_q_heads, int head_dim, float* mag,
                  float* phase, float* conc, void* ws, size_t ws_bytes, tri_stream_t stream) {
    int rc = check_calib_shape(n_layers, n_samples, n_q_heads, head_dim);
    if (rc) return rc;
    if (!q || !mag || !phase || !conc || (reinterpret_cast<uintptr_t>(q) & 15)) return TRI_ERR_INVALID_ARG;
    if (dtype != TRI_DTYPE_F32 && dtype != TRI_DTYPE_BF16) return TRI_ERR_INVALID_ARG;
    if (!ws || ws_bytes < calib_ws_bytes(n_layers, n_samples, n_q_heads, head_dim) || !aligned256(ws))
        return TRI_ERR_WORKSPACE;
    if (!device_present()) return TRI_ERR_NO_DEVICE;
    CalibArgs a;
    a.q = static_cast<const uint8_t*>(q);
    a.part = static_cast<double*>(ws);
    a.mag = mag;
    a.phase = phase;
    a.conc = conc;
    a.n_layers = n_layers;
    a.n_samples = n_samples;
    a.n_q_heads = n_q_heads;
    a.head_dim = head_dim;
    a.chunk_len = calib_chunk_len(n_layers, n_samples, n_q_heads, head_dim);
    a.n_chunks = (n_samples + a.chunk_len - 1) / a.chunk_len;
    return hip_status(launch_calibrate(a, dtype == TRI_DTYPE_BF16, static_cast<hipStream_t>(stream)),
                      "calibration kernel");
}

int tri_timing_enable(int enable) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing = enable != 0;
    return TRI_OK;
}

int tri_timing_mask(uint32_t mask) {
    std::lock_guard<std::mutex> lk(g_tmu);
    g_timing_mask = mask;
    return TRI_OK;
}

int tri_timing_reset(void) {
    std::lock_guard<std::mutex> lk(g_tmu);
    drain_timing_locked();
    for (int i = 0; i < KID_COUNT; ++i) {
        g_ms[i] = 0.0;
        g_launches[i] = 0;
    }
    return TRI_OK;
}

int tri_timing_read(int which, int64_t* launches, double* total_ms) {
    if (which < 0 || which >= KID_COUNT || !launches || !total_ms) return TRI_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_tmu);
    drain_timing_locked();
    *launches = g_launches[which];
    *total_ms = g_ms[which];
    return TRI_OK;
}

const char* tri_last_error(void) { return t_last_error; }

const char* tri_timing_name(int which) {
    if (which < 0 || which >= KID_COUNT) return nullptr;
    return kKernelNames[which];
}

}  // extern "C"
