/*
 * bkv.h -- beacon-guided KV-cache compression on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbkv.so.  The operations follow "BeaconKV: Key-Value Cache Compression
 * Guided by Beacon Queries for Efficient Large Reasoning Model Inference"
 * (thelatestinai.com/papers/2609.04971):
 *
 *   bkv_update_beacons  keeps per-KV-head beacon queries by continual farthest-point
 *                       sampling (Figure 7 caption; Abstract: compact representatives of
 *                       the global query clusters, no full query history);
 *   bkv_update_beacons_policy  the same, or the earliest queries kept (Table 3);
 *   bkv_score           attention-based score of every cached key from the recent queries
 *                       and the beacon queries (Figure 5 (b)), max-aggregated over queries
 *                       and heads (Figure 5 (c); Table 2 caption);
 *   bkv_score_agg       the same scores with max or mean aggregation (Table 2);
 *   bkv_select_topk     top-K under the cache budget (Figure 5 (c)), the recent window
 *                       always kept;
 *   bkv_compact         eviction: the kept K/V rows gathered into a compacted cache
 *                       (Abstract);
 *   bkv_compact_into    the same into a cache with room for the next decoded tokens;
 *   bkv_compress        bkv_score + bkv_select_topk + bkv_compact in one call;
 *   bkv_compress_static the same without a workspace, for callers that cannot allocate;
 *   bkv_decode_attention  one decoding step of attention over the (compacted) cache.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * Unit.  A unit is one (layer, sequence b, KV head h).  Query head h*G + r (r < G,
 * G = n_q_heads / n_kv_heads) belongs to KV head h.
 *
 * Layers.  Every per-layer argument is a HOST array of shape->n_layers DEVICE pointers,
 * one per layer, so one call covers a whole model.  The arrays are read during the call
 * only.  Layer pointers may differ in anything but shape.
 *
 * Layouts (all row-major, contiguous, bf16 = raw IEEE bfloat16 bit patterns):
 *   K, V cache     bf16  [batch][n_kv_heads][capacity][head_dim]
 *   queries        bf16  [batch][n_q_heads][q_len][head_dim]   (newest query last)
 *   beacons        bf16  [batch][n_kv_heads][nb_max][head_dim]
 *   beacon counts  int32 [batch][n_kv_heads]
 *   scores         fp32  [batch][n_kv_heads][capacity]
 *   kept positions int32 [batch][n_kv_heads][budget]
 *   kept counts    int32 [batch][n_kv_heads]
 *   compacted K, V bf16  [batch][n_kv_heads][budget][head_dim]
 * Row j of a cache is valid for j < L_b = min(seq_len[b], capacity).
 * Alignment: every bf16 array above (each layer's pointer) starts on a 16-byte boundary,
 * since the kernels move rows in 16-byte pieces; fp32 and int32 arrays (seq_len
 * included) on a 4-byte boundary.  A misaligned pointer is BKV_EINVAL.
 *
 * Memory and ordering.  Every pointer is device memory owned by the caller unless stated
 * otherwise.  The library never allocates, frees or synchronises; it keeps no pointer
 * after returning.  (Its one piece of memory of its own is the static scratch array of
 * bkv_compress_static, part of its code object.)  All work is enqueued on `stream`
 * (0 = the null stream) and runs in stream order; results are visible after the caller
 * synchronises.  Calls are thread-safe; concurrent calls must not share output or
 * workspace buffers, and bkv_compress_static calls on one device must not overlap.
 *
 * Overlap.  No output of a call (nor its workspace) may overlap anything else the call
 * touches: an input of any layer, seq_len, the workspace or another output, counted as
 * whole per-layer arrays of the layouts above.  Inputs may share memory.  A call that
 * breaks this returns BKV_EALIAS.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a failing call
 * enqueues nothing and returns a negative bkv_status.  Device-resident values are not
 * errors: seq_len[b] is clamped to [0, capacity] and beacon counts to [0, nb_max] inside
 * the kernels.  A failed launch returns BKV_EHIP (the stream may then hold part of the
 * call's work).
 */
#ifndef BKV_H_
#define BKV_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bkv_status {
  BKV_OK = 0,
  BKV_EINVAL = -1,        /* null or misaligned pointer, non-positive size,            */
                          /* window > budget, ...                                      */
  BKV_EUNSUPPORTED = -2,  /* valid but outside what the kernels support (head_dim,      */
                          /* observation rows, beacon pool size)                        */
  BKV_EALIAS = -3,        /* an output overlaps an input, the workspace or an output    */
  BKV_EWORKSPACE = -4,    /* workspace missing or smaller than the *_workspace_bytes    */
  BKV_EHIP = -5           /* a HIP launch or runtime call failed                        */
} bkv_status;

typedef struct bkv_shape {
  int32_t n_layers;        /* >= 1: length of every per-layer pointer array             */
  int32_t batch;           /* >= 1 sequences                                           */
  int32_t n_q_heads;       /* >= 1, a multiple of n_kv_heads                             */
  int32_t n_kv_heads;      /* >= 1                                                     */
  int32_t head_dim;        /* 64 or 128                                                */
  int32_t capacity;        /* >= 1 rows allocated per (sequence, KV head)               */
  const int32_t* seq_len;  /* DEVICE int32 [batch]: valid rows per sequence (all layers) */
} bkv_shape;

/* Largest number of observation rows (n_q_heads/n_kv_heads * window + nb_max) that
 * bkv_score / bkv_compress accept. */
#define BKV_MAX_OBS 512
/* Largest beacon pool (nb_max + n_q_heads/n_kv_heads * t_new) bkv_update_beacons accepts
 * (pools above 768 rows, e.g. a whole query history, take a slower streaming kernel). */
#define BKV_MAX_POOL 16384

/* Human-readable name of a status code, a bkv_status value (static string, never NULL;
 * any other value names an unknown status).  Enumerated arguments throughout this header
 * are passed as int32_t, so a caller may pass any value and get an error back. */
const char* bkv_status_string(int32_t status);

/* Library version, e.g. "0.2.0" (static string). */
const char* bkv_version(void);

/* Which HIP call failed, and how, for this thread's most recent BKV_EHIP, or why
 * bkv_compress_static last returned BKV_EUNSUPPORTED for lack of scratch (a thread-local
 * string valid until the thread's next failing call; "no HIP error recorded" if none). */
const char* bkv_last_error(void);

/* ------------------------------------------------------------------------------------
 * Continual farthest-point sampling of beacon queries.
 * BeaconKV page, Figure 7 caption ("Continual FPS") and Abstract (beacons are compact
 * representatives of each global query cluster, maintained without the full query
 * history); Figure 4 (a) measures query similarity by cosine similarity.
 *
 * Per unit, the candidate pool is the live beacons beacons_in[b][h][0 .. c) in stored
 * order, c = clamp(n_in[b][h], 0, nb_max), followed by the new queries of the group's
 * query heads h*G .. h*G+G-1, head-major, each head contributing its last t_new stored
 * rows (of q_len) in time order.  If the pool has at most nb_max rows all of them are
 * kept in pool order; otherwise nb_max rows are chosen greedily: first pool row 0, then
 * repeatedly the not-yet-chosen row whose cosine distance (1 - cos) to its nearest chosen
 * row is largest, ties to the lower pool index.  Distances are computed in fp32 from the
 * bf16 rows.
 *
 * beacons_out[b][h][0 .. n_out) receive bit copies of the chosen rows in choice order;
 * slots from n_out up are left untouched.  n_out[b][h] = min(nb_max, pool size).
 *
 * q_new:   per layer bf16 [batch][n_q_heads][q_len][head_dim]; 0 <= t_new <= q_len.
 * n_in:    per layer int32 [batch][n_kv_heads].
 * Errors:  BKV_EINVAL for null arrays/pointers or bad sizes; BKV_EUNSUPPORTED if
 *          nb_max + G * t_new > BKV_MAX_POOL or head_dim is not 64/128; BKV_EALIAS if
 *          beacons_out or n_out overlaps an input (beacons_in, n_in, q_new) or each other.
 * ---------------------------------------------------------------------------------- */
bkv_status bkv_update_beacons(const bkv_shape* shape,
                              const void* const* beacons_in, const int32_t* const* n_in,
                              int32_t nb_max,
                              const void* const* q_new, int32_t q_len, int32_t t_new,
                              void* const* beacons_out, int32_t* const* n_out,
                              hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Beacon update with a chosen policy.
 * BeaconKV page, Figure 7 caption (Continual FPS) and Table 3 (the Initial+Recent
 * baseline: the observation set is the earliest queries plus the recent ones).
 *
 *   BKV_BEACON_FPS:     identical to bkv_update_beacons.
 *   BKV_BEACON_INITIAL: the live rows beacons_in[b][h][0 .. c) stay in place and the new
 *                       queries fill the free slots in time order (for each of the t_new
 *                       steps, the group's heads in head order) until nb_max rows are
 *                       held; once full the set never changes.  n_out = min(nb_max,
 *                       c + G * t_new).  No pool-size limit applies.
 * Same arguments and errors as bkv_update_beacons, plus BKV_EINVAL for an unknown
 * policy.
 * ---------------------------------------------------------------------------------- */
typedef enum {
  BKV_BEACON_FPS = 0,     /* continual farthest-point sampling (the method) */
  BKV_BEACON_INITIAL = 1  /* first queries kept (Table 3's Initial+Recent) */
} bkv_beacon_policy;

bkv_status bkv_update_beacons_policy(const bkv_shape* shape,
                                     const void* const* beacons_in, const int32_t* const* n_in,
                                     int32_t nb_max,
                                     const void* const* q_new, int32_t q_len, int32_t t_new,
                                     int32_t policy /* bkv_beacon_policy */,
                                     void* const* beacons_out, int32_t* const* n_out,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Attention-based key scores, max-aggregated.
 * BeaconKV page, Figure 5 (b) (scores from beacon queries and recent queries),
 * Figure 5 (c) and Table 2 caption (max aggregation across heads and queries).
 *
 * Per unit the observation set is, in this order, the last `window` stored queries of
 * each query head of the group (head-major, time order) and the live beacons
 * beacons[b][h][0 .. nb), nb = clamp(n_beacons[b][h], 0, nb_max).  With
 * s_ij = q_i . k_j / sqrt(head_dim) (bf16 inputs, fp32 accumulation) and the softmax
 * over all valid keys j < L_b (no causal mask), the score of key j is
 *     scores[b][h][j] = max_i exp(s_ij - logsumexp_j' s_ij'),
 * i.e. the largest attention weight any observation query gives it.  Entries j >= L_b
 * are not written.  With an empty observation set every valid score is 0.
 *
 * window:      0 <= window <= q_len; n_q_heads/n_kv_heads * window + nb_max <= BKV_MAX_OBS.
 * beacons, n_beacons: may be NULL arrays when nb_max == 0.
 * workspace:   device scratch of at least bkv_score_workspace_bytes(...) bytes (256-byte
 *              aligned), contents irrelevant on entry and undefined on exit.
 * Errors:      BKV_EINVAL, BKV_EUNSUPPORTED (head_dim, observation rows), BKV_EWORKSPACE,
 *              BKV_EALIAS if scores or the workspace overlaps an input (K, queries, beacons,
 *              beacon counts, seq_len), each other or another scores layer.
 * ---------------------------------------------------------------------------------- */
size_t bkv_score_workspace_bytes(const bkv_shape* shape, int32_t window, int32_t nb_max);

/* How the observation rows' attention weights of a key combine into its score. */
typedef enum {
  BKV_AGG_MAX = 0,  /* largest weight (the method's choice; Figure 5 (c)) */
  BKV_AGG_MEAN = 1  /* mean weight over the observation rows (Table 2's alternative) */
} bkv_aggregation;

bkv_status bkv_score(const bkv_shape* shape,
                     const void* const* k,
                     const void* const* q, int32_t q_len, int32_t window,
                     const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                     float* const* scores,
                     void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Attention-based key scores with a chosen aggregation.
 * BeaconKV page, Table 2 (max vs. mean aggregation, applied alike across heads and
 * queries).
 *
 * As bkv_score, with the score of key j
 *     BKV_AGG_MAX:  max_i w_ij                      (identical to bkv_score)
 *     BKV_AGG_MEAN: (1 / n_obs) * sum_i w_ij
 * where w_ij = exp(s_ij - logsumexp_j' s_ij') over the unit's n_obs observation rows
 * (G * window recent queries and the live beacons); with n_obs = 0 every valid score is
 * 0.  Under BKV_AGG_MEAN a unit's scores sum to 1 over its valid keys.  Same arguments,
 * workspace and errors as bkv_score, plus BKV_EINVAL for an unknown aggregation.
 * ---------------------------------------------------------------------------------- */
bkv_status bkv_score_agg(const bkv_shape* shape,
                         const void* const* k,
                         const void* const* q, int32_t q_len, int32_t window,
                         const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                         int32_t aggregation /* bkv_aggregation */,
                         float* const* scores,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Top-K selection under the budget with the recent window always kept.
 * BeaconKV page, Figure 5 (c) (top-K selection via max aggregation of the scores).
 *
 * Per unit with L = L_b: if L <= budget every position 0 .. L-1 is kept.  Otherwise the
 * last `window` positions L-window .. L-1 are kept, and the budget - window positions
 * before them with the largest scores (compared as fp32; equal scores go to the lower
 * position).  idx[b][h][0 .. n) receives the kept positions in ascending order and
 * n_kept[b][h] = n = min(budget, L); idx slots from n up are left untouched.
 * Scores must be non-negative (as bkv_score produces); NaN ordering is unspecified.
 *
 * 1 <= budget, 0 <= window <= budget.  workspace may be NULL when
 * bkv_select_workspace_bytes(...) returns 0.
 * Errors: BKV_EINVAL, BKV_EWORKSPACE, BKV_EALIAS if idx or n_kept overlaps scores,
 *         seq_len or each other.
 * ---------------------------------------------------------------------------------- */
size_t bkv_select_workspace_bytes(const bkv_shape* shape, int32_t budget);

bkv_status bkv_select_topk(const bkv_shape* shape,
                           const float* const* scores, int32_t budget, int32_t window,
                           int32_t* const* idx, int32_t* const* n_kept,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Eviction by compaction: kept rows gathered into a new cache.
 * BeaconKV page, Abstract (the cache keeps only the selected KV pairs).
 *
 * For r < n = clamp(n_kept[b][h], 0, budget):
 *     k_out[b][h][r] = k[b][h][idx[b][h][r]],  v_out[b][h][r] = v[b][h][idx[b][h][r]]
 * as bit copies; rows from n up are left untouched.  Positions outside [0, capacity) are
 * clamped into it (bkv_select_topk never produces them).  Out of place: outputs must not
 * overlap K or V.
 * Errors: BKV_EINVAL, BKV_EUNSUPPORTED (head_dim; budget * head_dim / 8 >= 2^30),
 *         BKV_EALIAS if k_out or v_out overlaps K, V, idx, n_kept or each other.
 * ---------------------------------------------------------------------------------- */
bkv_status bkv_compact(const bkv_shape* shape,
                       const void* const* k, const void* const* v,
                       const int32_t* const* idx, const int32_t* const* n_kept, int32_t budget,
                       void* const* k_out, void* const* v_out,
                       hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Compaction into a cache with room to grow.
 * BeaconKV page, Abstract (the cache keeps only the selected KV pairs) and the serving
 * setting of Table 4 (decoding continues after each compression).
 *
 * As bkv_compact, but k_out / v_out are laid out [batch][n_kv_heads][out_capacity]
 * [head_dim] (out_capacity >= budget): the kept rows land in rows 0 .. n-1 of each
 * (sequence, KV head) and rows from n up are left untouched, so a caller can append the
 * next decoded tokens after them and compress again from that buffer (double buffering:
 * the outputs must not overlap K or V).  bkv_compact is the case out_capacity = budget.
 * Errors: as bkv_compact, plus BKV_EINVAL if out_capacity < budget.
 * ---------------------------------------------------------------------------------- */
bkv_status bkv_compact_into(const bkv_shape* shape,
                            const void* const* k, const void* const* v,
                            const int32_t* const* idx, const int32_t* const* n_kept, int32_t budget,
                            int32_t out_capacity,
                            void* const* k_out, void* const* v_out,
                            hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * One compression event: bkv_score, then bkv_select_topk, then bkv_compact, with the
 * arguments of those three calls (same meaning, same errors).  Writes scores, idx,
 * n_kept, k_out and v_out exactly as the three calls would.  The stages' outputs and the
 * workspace must not overlap each other either (BKV_EALIAS), since later stages read them.
 * workspace: at least bkv_compress_workspace_bytes(...) bytes.
 * ---------------------------------------------------------------------------------- */
size_t bkv_compress_workspace_bytes(const bkv_shape* shape, int32_t window, int32_t nb_max,
                                    int32_t budget);

bkv_status bkv_compress(const bkv_shape* shape,
                        const void* const* k, const void* const* v,
                        const void* const* q, int32_t q_len, int32_t window,
                        const void* const* beacons, const int32_t* const* n_beacons, int32_t nb_max,
                        int32_t budget,
                        float* const* scores, int32_t* const* idx, int32_t* const* n_kept,
                        void* const* k_out, void* const* v_out,
                        void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): bkv_compress without a workspace
 * argument.  Same arguments otherwise, same errors (no BKV_EWORKSPACE), and bit-identical
 * results wherever the default launches' partials fit the scratch.
 *
 * The score stage's statistics partials go to a static device array of
 * BKV_STATIC_SCRATCH_BYTES bytes that the library's code object holds on every device it
 * is loaded on, until the process ends; the call itself allocates and frees nothing.
 * Where the default launches' partials would not fit, the score stage goes out in groups
 * of fewer layers and sequences per launch (more launches; the scores may then differ from
 * bkv_compress's in the last bits, since the keys are summed in pieces that follow the
 * launch size, and a top-K can flip at such a near-tie).  If even one layer of one
 * sequence does not fit, the call returns BKV_EUNSUPPORTED and enqueues nothing;
 * bkv_last_error() then says how many bytes it would need.
 *
 * Every call on one device shares that device's array, and each call's partials are
 * written before they are read in the same call, so nothing needs clearing between calls.
 * Two calls whose work overlaps in time on one device (different streams, different host
 * threads) race on the array and may return wrong scores: the caller serialises them,
 * e.g. by issuing them on one stream.
 * ---------------------------------------------------------------------------------- */
#define BKV_STATIC_SCRATCH_BYTES ((size_t)32 << 20)

bkv_status bkv_compress_static(const bkv_shape* shape,
                               const void* const* k, const void* const* v,
                               const void* const* q, int32_t q_len, int32_t window,
                               const void* const* beacons, const int32_t* const* n_beacons,
                               int32_t nb_max, int32_t budget,
                               float* const* scores, int32_t* const* idx, int32_t* const* n_kept,
                               void* const* k_out, void* const* v_out,
                               hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * One decoding step of attention over a cache (typically the compacted one).
 * BeaconKV page, Abstract and Table 4: after compression decoding attends over the kept
 * KV pairs only, which is where the method's memory and throughput gains come from.
 *
 * For every sequence b and query head hq (KV head h = hq / G):
 *     out[b][hq] = sum_j w_j v[b][h][j],  w = softmax_j(q[b][hq] . k[b][h][j] / sqrt(d))
 * over the valid rows j < L_b (fp32 accumulation; out = 0 when L_b = 0).
 *
 * q:    per layer bf16 [batch][n_q_heads][head_dim] (one new query per head).
 * k, v: per layer bf16 [batch][n_kv_heads][capacity][head_dim] (e.g. bkv_compact_into's
 *       output with capacity = its out_capacity and seq_len = the kept counts).
 * out:  per layer fp32 [batch][n_q_heads][head_dim].
 * workspace: at least bkv_decode_workspace_bytes(shape) bytes, 256-byte aligned.
 * Errors: BKV_EINVAL, BKV_EUNSUPPORTED (head_dim; more than 8 query heads per KV head),
 *         BKV_EWORKSPACE, BKV_EALIAS if out or the workspace overlaps q, k, v, seq_len or
 *         each other.
 * ---------------------------------------------------------------------------------- */
size_t bkv_decode_workspace_bytes(const bkv_shape* shape);

bkv_status bkv_decode_attention(const bkv_shape* shape,
                                const void* const* q,
                                const void* const* k, const void* const* v,
                                float* const* out,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* BKV_H_ */
