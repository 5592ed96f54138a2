/*
 * triattn.h — C ABI of the MI355X (gfx950) TriAttention KV-cache pruning library.
 *
 * Method (web pages describing TriAttention; formulas there were lost, the
 * prose is restated here):
 *   [YY] yeyulingfeng.com, "实现单卡4090跑通OpenClaw!英伟达&浙大等提出长上下文推理KV
 *        压缩新方法TriAttention", section 主要方法.
 *   [ZN] zingnex.cn, "TriAttention：用三角级数压缩KV缓存，让长推理模型跑在消费级显卡上",
 *        sections 预RoPE空间的发现 and TriAttention的核心机制：三角级数距离建模.
 *
 * Offline, each query head h of each layer gets per-band centre statistics:
 * magnitude M[h][f], phase phi[h][f] and concentration R[h][f] (mean resultant
 * length).  Online, every cached key is scored by
 *     S_h = (1/|O|) sum_{o in O} sum_f M |k_f| cos(w_f (t + o - p) + phi - psi_f)
 *         + sum_f (1 - R) M |k_f|
 * (the centre query's RoPE logit at future positions t + o, averaged over a
 * geometric offset set, plus a norm term that grows where the band is not
 * concentrated), z-scored inside each query head, max-aggregated over the GQA
 * group, and when a segment holds more than B keys only the B best survive
 * (ties at the cut to the earlier position) and K/V/positions are compacted in
 * slot order.
 *
 * Conventions shared by every entry point
 *  - Rotary layout: half-split pairing.  Band f of a row x is x[f] + i x[f+F],
 *    F = head_dim/2, frequency w_f = rope_theta^(-2f/head_dim).  The cache holds
 *    post-RoPE keys.
 *  - A segment is one (layer, sequence, KV head).  Segments are numbered
 *    s = (l * n_seq + b) * n_kv_heads + h; query heads h*G .. h*G+G-1 share it.
 *  - Pointers marked "device" are device memory owned by the caller; pointers
 *    marked "host" are host memory read during the call.  The library never
 *    allocates per call; only tri_calib_load allocates (a small table it owns),
 *    and the timing instrumentation, when enabled, creates HIP events once and
 *    reuses them.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = null stream).
 *    Return codes report host-side validation and launch errors only; on a
 *    validation error nothing is launched and outputs are untouched (a launch
 *    error part way through a multi-kernel call can leave earlier kernels'
 *    writes behind).
 *  - Supported: head_dim 64 or 128, GQA group 1, 2, 4 or 8, bf16 or fp32
 *    storage, segments of at most 65536 keys, budget at most 8192.
 */
#ifndef TRIATTN_H
#define TRIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define TRI_OK 0
#define TRI_ERR_INVALID_ARG (-1) /* malformed argument (null, negative, inconsistent shape) */
#define TRI_ERR_UNSUPPORTED (-2) /* well-formed but outside the supported set above        */
#define TRI_ERR_WORKSPACE (-3)   /* workspace missing or smaller than tri_workspace_size   */
#define TRI_ERR_HIP (-4)         /* a HIP runtime call or kernel launch failed             */
#define TRI_ERR_NO_DEVICE (-5)   /* no GPU visible to the process                          */

/* ---- storage types and layouts ---- */
#define TRI_DTYPE_F32 0
#define TRI_DTYPE_BF16 1
#define TRI_LAYOUT_DENSE 0
#define TRI_LAYOUT_PAGED 1

typedef void* tri_stream_t;                 /* hipStream_t */
typedef struct tri_calib_s* tri_calib_t;    /* opaque calibration handle */

/*
 * A KV cache.  All pointers are device memory owned by the caller.
 *  dense : k, v are [n_seg][capacity][head_dim] (row = head_dim elements),
 *          pos is int32 [n_seg][capacity].
 *  paged : k, v are a pool [n_pages][page_size][head_dim], pos is int32
 *          [n_pages][page_size]; slot i of segment s lives in row i % page_size
 *          of page page_table[s * max_pages + i / page_size].
 *  lengths : int32 [n_seg], valid keys per segment (slots 0..lengths[s]-1).
 *  layer0  : calibration layer of this cache's layer 0 (layer l uses
 *            calibration layer layer0 + l).
 */
typedef struct tri_cache_desc {
    int32_t dtype;        /* TRI_DTYPE_*                         */
    int32_t layout;       /* TRI_LAYOUT_*                        */
    int32_t n_layers;
    int32_t layer0;
    int32_t n_seq;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t capacity;     /* dense: slots per segment; paged: max_pages * page_size */
    void* k;
    void* v;
    int32_t* pos;
    int32_t* lengths;
    int32_t page_size;    /* paged only */
    int32_t max_pages;    /* paged only */
    const int32_t* page_table; /* paged only: int32 [n_seg][max_pages] */
} tri_cache_desc;

/*
 * Offline calibration -> device constants ([YY] 主要方法: centres, norms and
 * concentration are gathered offline; the future offsets are a geometric set).
 *   mag, phase, conc : host fp32 [n_layers][n_q_heads][head_dim/2]
 *                      (M >= 0, phase in radians, 0 <= conc <= 1).
 *   offsets          : host int32 [n_offsets], each >= 0.
 * Folds the offset average into one complex coefficient per band in fp64
 * (the average of e^{i w_f (t+o)} over o factors as e^{i w_f t} times a
 * constant), and stores it with the weights (1 - R) M on the device.
 * n_q_heads must be a multiple of n_kv_heads (group G = n_q_heads/n_kv_heads).
 * *out receives a handle (freed with tri_calib_free).  Synchronous.
 */
int tri_calib_load(tri_calib_t* out, int n_layers, int n_q_heads, int n_kv_heads, int head_dim,
                   double rope_theta, const float* mag, const float* phase, const float* conc,
                   const int32_t* offsets, int n_offsets, tri_stream_t stream);

/*
 * Score variants ([YY] 主实验结果: the ablations name the trigonometric score,
 * the adaptive weighting and the geometric offsets as key components), folded
 * into the handle at load time, so every entry point scores with them:
 *   TRI_VARIANT_TRIG_ONLY        drop the norm term
 *   TRI_VARIANT_NORM_ONLY        drop the trigonometric term (not with TRIG_ONLY)
 *   TRI_VARIANT_FIXED_WEIGHT     norm weight M instead of (1 - R) M
 *   TRI_VARIANT_R_WEIGHTED_TRIG  trigonometric term with centre magnitude R M
 *                                (the reading |E q_f| = R mean |q_f|)
 * Linear instead of geometric offsets need no flag: pass that offset set.
 * variant 0 is tri_calib_load.  Any other bit, or TRIG_ONLY with NORM_ONLY,
 * gives TRI_ERR_INVALID_ARG.
 */
#define TRI_VARIANT_TRIG_ONLY 1
#define TRI_VARIANT_NORM_ONLY 2
#define TRI_VARIANT_FIXED_WEIGHT 4
#define TRI_VARIANT_R_WEIGHTED_TRIG 8
int tri_calib_load_ex(tri_calib_t* out, int n_layers, int n_q_heads, int n_kv_heads, int head_dim,
                      double rope_theta, const float* mag, const float* phase, const float* conc,
                      const int32_t* offsets, int n_offsets, int variant, tri_stream_t stream);

/* Releases a handle (NULL is a no-op).  Waits for the device to be idle. */
int tri_calib_free(tri_calib_t calib);

/*
 * Offline calibration statistics from sampled pre-RoPE queries ([YY] 主要方法:
 * pre-RoPE queries gather around fixed non-zero centres, and a band's
 * concentration is the mean resultant length R, closer to 1 meaning more
 * concentrated).  For every layer, query head and band f (band = q[f] + i q[f+F]):
 *   mag   = mean of |q_f|,
 *   phase = arg of the sum of q_f (0 when that sum is 0),
 *   conc  = | mean of q_f / |q_f| |   (a sample with q_f = 0 adds no direction).
 *   q     : device [n_layers][n_samples][n_q_heads][head_dim], dtype TRI_DTYPE_*
 *           (pre-RoPE rows: one per sampled token and query head), 16-byte
 *           aligned (TRI_ERR_INVALID_ARG otherwise).
 *   mag, phase, conc : device fp32 [n_layers][n_q_heads][head_dim/2] outputs,
 *           the layout tri_calib_load takes (copy them to the host for it).
 *   ws    : device workspace of tri_calibrate_workspace_size bytes, 256-byte
 *           aligned (TRI_ERR_WORKSPACE otherwise).
 * Per-sample arithmetic is fp32; each run of at most eight samples is summed
 * in fp32 and added to fp64 sums, in a fixed order that depends only on the
 * shape (results do not depend on scheduling).  head_dim 64 or 128.
 */
int tri_calibrate_workspace_size(int n_layers, int n_samples, int n_q_heads, int head_dim, size_t* bytes);
int tri_calibrate(const void* q, int dtype, int n_layers, int n_samples, int n_q_heads, int head_dim, float* mag,
                  float* phase, float* conc, void* ws, size_t ws_bytes, tri_stream_t stream);

/*
 * Bytes of device workspace tri_score / tri_select_topb / tri_prune_window
 * need for this cache and budget (host-only; no device call).
 */
int tri_workspace_size(tri_calib_t calib, const tri_cache_desc* kv, int budget, size_t* bytes);

/*
 * Key scores and GQA aggregation ([YY] 主要方法: two-part key score fused into
 * one, averaged over future offsets; z-score inside each query head and max
 * over the heads sharing a KV head).
 *   t        : device int32 [n_seq], position of the next query of each sequence.
 *   scores   : optional device fp32 [n_seg][G][capacity]: raw S_h per key.
 *   agg      : device fp32 [n_seg][capacity]: A = max_h (S_h - mu_h) / sigma_h
 *              (population statistics over the segment's valid keys; a head
 *              with sigma = 0 contributes 0).  Slots >= lengths[s] untouched.
 *   mu_sigma : optional device fp32 [n_seg][G][2]: (mu_h, sigma_h).
 *   ws       : device workspace of tri_workspace_size bytes, 256-byte aligned
 *              (as every device allocation is; TRI_ERR_WORKSPACE otherwise).
 */
int tri_score(tri_calib_t calib, const tri_cache_desc* kv, const int32_t* t, float* scores,
              float* agg, float* mu_sigma, void* ws, size_t ws_bytes, tri_stream_t stream);

/*
 * Top-B selection per segment ([YY] 主要方法: keep only the top-B keys).
 *   agg     : device fp32 [n_seg][capacity] aggregated scores.
 *   lengths : device int32 [n_seg].
 *   idx     : device int32 [n_seg][budget]; row s receives the kept slots in
 *             ascending order: the budget largest scores (-0 and +0 are
 *             equal); all slots when lengths[s] <= budget.
 *   n_kept  : device int32 [n_seg], min(lengths[s], budget).
 * Keys tied at the cut: the earlier position is kept.  tri_select_topb has no
 * positions and takes slot order as position order (true of every cache this
 * library appends to and prunes, which stay in position order); the lower
 * slot wins.  tri_select_topb_ex takes the slots' positions, pos: device
 * int32 [n_seg][capacity] (NULL: as tri_select_topb); keys that tie at the
 * cut in score and position as well go by lower slot.  ws and ws_bytes are
 * not used (may be NULL, 0).
 */
int tri_select_topb(const float* agg, const int32_t* lengths, int n_seg, int capacity, int budget,
                    int32_t* idx, int32_t* n_kept, void* ws, size_t ws_bytes, tri_stream_t stream);
int tri_select_topb_ex(const float* agg, const int32_t* pos, const int32_t* lengths, int n_seg, int capacity,
                       int budget, int32_t* idx, int32_t* n_kept, void* ws, size_t ws_bytes, tri_stream_t stream);

/*
 * Compaction: for each segment, dst slot j <- src slot idx[s][j] for
 * j < n_kept[s] (K row, V row and position, bit-exact).  Out of place: dst
 * must not share memory with src (TRI_ERR_INVALID_ARG when dense arrays
 * overlap by any byte, or paged caches share a base address), except that a
 * paged dst may use src's pool through a different page table: its pages
 * must then be pages src does not use (fresh pages of a shared pool; not
 * checked).  dst describes a cache with the same
 * n_layers/n_seq/n_kv_heads/head_dim/dtype; its lengths are not written
 * (n_kept holds them).  idx rows are budget apart.
 */
int tri_compact(const tri_cache_desc* src, const int32_t* idx, const int32_t* n_kept, int budget,
                const tri_cache_desc* dst, tri_stream_t stream);

/*
 * One pruning pass over every segment ([YY] 主要方法: windowed batch pruning
 * every 128 generated tokens when the cache exceeds its budget): score,
 * aggregate, select and compact in one call, the fused hot path.  Segments
 * with lengths[s] <= budget are copied through unchanged, so dst is always a
 * complete cache; n_kept (device int32 [n_seg]) gets min(lengths[s], budget).
 *
 * Keys tied at the cut keep the earlier position (read from the cache's
 * positions; equal positions go by lower slot), so the kept set does not
 * depend on how the cache's slots are arranged.
 *
 * In place: when dst names src's storage (same k, v, pos, layout, capacity,
 * layer0 and, if paged, the same page table), the cache is pruned where it
 * is, with the same result as out of place: the kept rows end up in slots
 * 0..n_kept[s]-1 in their old slot order.  Rows before the first dropped slot
 * stay where they are and are not copied; every later kept row moves down.
 * Segments with lengths[s] <= budget are not touched.  n_kept may then be
 * src->lengths itself.  Out of place, dst and src share memory only as
 * tri_compact allows (fresh pages of src's pool); any other overlap is
 * TRI_ERR_INVALID_ARG.  dst must hold min(budget, src->capacity) rows per
 * segment (else TRI_ERR_INVALID_ARG); a cache whose capacity is below the
 * budget is copied through, or left as it is in place.
 */
int tri_prune_window(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                     const tri_cache_desc* dst, int32_t* n_kept, void* ws, size_t ws_bytes,
                     tri_stream_t stream);
/*
 * How the pass runs (the result does not depend on it).  The full-score path
 * keeps every key's G scores for the select step.  The candidate pass, for
 * bf16 caches, first gives segments with N >= 4096 and N >= 8 B per-head
 * score thresholds from a 256-key sample, and only keys reaching a threshold
 * in some head keep their scores.  The select step proves, with the exact
 * per-head statistics, that every other key ranks below the cut; segments
 * where that proof fails are scored and selected again over all of their
 * keys within the same call.  The kept set is always the one the full-score
 * path gives.
 *
 * tri_prune_window takes TRI_PATH_AUTO: the candidate pass when the cache is
 * bf16, its capacity allows candidate mode (>= 4096 and >= 8 B) and it has at
 * least 256 segments.  Fewer segments cannot fill the GPU: there the sample
 * and fallback launches cost more than the score writes the pass saves.
 * tri_prune_window_ex takes the path as an argument: TRI_PATH_FULL, or
 * TRI_PATH_CANDIDATES (the candidate pass whenever the cache allows it,
 * whatever its segment count).  Any other value is TRI_ERR_INVALID_ARG.
 *
 * TRI_INPLACE_FILL_FREED, or'ed into path, changes only the arrangement an
 * in-place prune leaves (no effect out of place): a kept key already below
 * n_kept[s] stays in its slot, and the kept keys at or above it move into the
 * freed slots below, lowest key into lowest freed slot.  Fewer rows move (at
 * most lengths[s] - budget per segment, against every kept row after the
 * first dropped slot), but slot order no longer follows position order, so
 * a later tri_select_topb (which has no positions) would break ties by a
 * different order; tri_prune_window itself reads positions and keeps the
 * same set either way.
 *
 * tri_prune_fallbacks: number of segments the last tri_prune_window on this
 * workspace had to redo in full (host int32 *count; 0 after a full-score
 * pass).  Synchronises `stream`.
 */
#define TRI_PATH_AUTO 0
#define TRI_PATH_FULL 1
#define TRI_PATH_CANDIDATES 2
#define TRI_INPLACE_FILL_FREED 16
int tri_prune_window_ex(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                        const tri_cache_desc* dst, int32_t* n_kept, void* ws, size_t ws_bytes, int path,
                        tri_stream_t stream);
int tri_prune_fallbacks(const void* ws, size_t ws_bytes, int32_t* count, tri_stream_t stream);

/*
 * tri_prune_window_ex without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a device array the
 * library holds, TRI_STATIC_SCRATCH_BYTES per device, on every device it
 * runs on, until the process ends.  This call allocates nothing.
 *  - Same arguments and result as tri_prune_window_ex (path included), minus
 *    ws/ws_bytes.
 *  - A cache whose tri_workspace_size exceeds TRI_STATIC_SCRATCH_BYTES is
 *    refused with TRI_ERR_WORKSPACE (tri_last_error gives both sizes); 64 MiB
 *    holds, e.g., one 32K-key layer of 8 KV heads at GQA 4.
 *  - Every call on one device shares that device's array, which keeps what
 *    the last call left; nothing in it needs to start at zero (each pass
 *    writes what it reads).  Calls whose work overlaps on one device (two
 *    streams, or two threads) race on it: serialise them.
 *  - The first call on a device looks up that device's copy of the array
 *    (hipGetSymbolAddress); later calls reuse the address.
 */
#define TRI_STATIC_SCRATCH_BYTES (64u << 20)
int tri_prune_window_static(tri_calib_t calib, const tri_cache_desc* src, const int32_t* t, int budget,
                            const tri_cache_desc* dst, int32_t* n_kept, int path, tri_stream_t stream);

/*
 * Appends one token to every segment: row lengths[s] of segment s receives
 * k_new[s], v_new[s] (device [n_seg][head_dim], cache dtype) and position
 * pos_new[b] (device int32 [n_seq]); lengths[s] then grows by one.  A segment
 * already at capacity is left unchanged (its length stays at capacity).
 * Dense caches only.
 */
int tri_append(const tri_cache_desc* kv, const void* k_new, const void* v_new,
               const int32_t* pos_new, tri_stream_t stream);

/*
 * Single-query decode attention over the current cache, for every layer,
 * sequence and query head ([ZN] 长推理的内存困境: each decode step re-attends
 * to the whole cache):  out = softmax(scale * q . K^T) V over the segment's
 * valid keys.  q : device [n_layers][n_seq][n_q_heads][head_dim] (cache dtype);
 * out : device fp32, same shape.  Dense or paged caches (a pruned paged cache
 * is read in place through its page table); lengths[s] >= 1.  Arithmetic:
 * fp32 sums of exact products (bf16 q and K on the matrix cores; the
 * probabilities times V either in fp32 or, for eight-head groups at head_dim
 * 64, on the matrix cores with each probability carried as three bf16 parts,
 * 24 bits), base-2 online softmax in fp32.
 */
int tri_decode_attn(const tri_cache_desc* kv, int n_q_heads, const void* q, float scale, float* out,
                    tri_stream_t stream);

/* Static description of a status code. */
const char* tri_strerror(int code);

/* For the calling thread's most recent TRI_ERR_HIP: which step failed and the
 * HIP error string; for a tri_prune_window_static refused for size: the
 * workspace needed and the scratch size ("" if none).  Valid until the next
 * failing call. */
const char* tri_last_error(void);

/*
 * Kernel timing (instrumentation).  When enabled, every kernel launched by
 * the library whose id is in the mask (bit i = kernel id i; all kernels
 * until tri_timing_mask says otherwise) is bracketed by HIP events on its
 * stream; each event record costs a few microseconds of GPU time, so a
 * caller timing a short pass can restrict the mask to the kernels it needs.
 * tri_timing_read synchronises those events and returns, for kernel id
 * `which` (0-based, see tri_timing_name), the number of launches and their
 * summed duration in ms since the last reset.  Returns TRI_ERR_INVALID_ARG
 * past the last id.
 */
int tri_timing_enable(int enable);
int tri_timing_mask(uint32_t mask);
int tri_timing_reset(void);
int tri_timing_read(int which, int64_t* launches, double* total_ms);
const char* tri_timing_name(int which);

#ifdef __cplusplus
}
#endif
#endif /* TRIATTN_H */
