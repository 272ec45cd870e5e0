/*
 * libsnapstream: the data-parallel hot path of SnapStream (fixed-size KV cache
 * built at prefill, ring-buffer decode over it) for AMD Instinct MI355X
 * (gfx950).  Plain C ABI; every buffer is caller-owned.  Tensor and workspace
 * pointers are device addresses aligned to 16 bytes (SS_ERR_INVALID_ARG
 * otherwise): the kernels move data in 16-byte vectors.
 *
 * Sources, by page title and section:
 *   "SnapStream: Efficient Long Sequence Decoding on Dataflow Accelerators",
 *     abstract: StreamingLLM sinks/recency fused with SnapKV selection into a
 *     fixed-size cache that works under static graphs and continuous batching.
 *   "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators" (episode
 *     companion), sections
 *       "Fixed-Size Cache Layout"  - built once at prefill: sink tokens +
 *                                    SnapKV top-K middle + recent window;
 *                                    L_sink, K, L_recent are hyperparameters;
 *       "Ring Buffer vs. Naive Slicing" - decode rotates only the recent
 *                                    window: a scatter into a fixed index, no
 *                                    gather, no concatenation;
 *       "Why This Wasn't Already Standard" - static shapes; requests of one
 *                                    batch at different points of their life;
 *       "Prefill / Decode Pipeline" - decode is memory-bound on the cache;
 *       "Infinity-Bench KV Retrieval" - pooling-based top-K selection.
 *
 * Conventions that the pages leave open (the library's reading):
 *   - score of middle key i: sum over the G q-heads of its kv-head and over
 *     the last W prompt queries of that query's causal softmax probability of
 *     key i (softmax over every prompt key up to the query's own position);
 *   - max-pool of odd width `pool`, stride 1, window clipped to the middle
 *     region [L_sink, L - L_recent);
 *   - top-K in the order (pooled score descending, position ascending); the K
 *     kept tokens occupy slots L_sink .. L_sink+K-1 in ascending position;
 *   - ring: position t >= L_sink+K lives in slot
 *     L_sink + K + ((t - L_sink - K) mod L_recent); a prompt with L <= C is
 *     stored uncompressed with token t in slot t;
 *   - rotary embedding (rotate-half, pairs (i, i + d_rot/2) of the range
 *     [rope_begin, rope_end), inv_freq_i = rope_theta^(-2i/d_rot)) is applied
 *     at the token's absolute position before the key is cached; angles are
 *     computed in fp64 and the rotated key is rounded once to the cache dtype;
 *   - decode writes the new token first, then attends over slots
 *     [0, min(pos + 1, C)), the new token included.
 */
#ifndef SNAPSTREAM_H
#define SNAPSTREAM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SS_OK = 0,
  SS_ERR_INVALID_ARG = 1,  /* a scalar or pointer argument is invalid; nothing was launched */
  SS_ERR_UNSUPPORTED = 2,  /* valid, but this build has no kernel for the shape/dtype */
  SS_ERR_WORKSPACE = 3,    /* ws_bytes is smaller than the matching *_workspace_bytes() */
  SS_ERR_HIP = 4,          /* a HIP launch failed (hipGetLastError after the launch) */
  SS_ERR_SCRATCH_LIMIT = 5 /* ss_decode_step_noalloc: the shapes need more scratch than the
                              library's static array holds; nothing was launched */
} ss_status;

typedef enum { SS_F32 = 0, SS_BF16 = 1 } ss_dtype;

/* One attention layer and its fixed cache.  C = L_sink + K + L_recent slots,
 * at most 2^24 (larger C: SS_ERR_INVALID_ARG).
 * Supported (d_qk, d_v, dtype): (64, 64, f32|bf16), (128, 128, f32|bf16),
 * (576, 512, bf16) with v_aliases_k = 1 (MLA absorbed latent; its rotary range,
 * if any, must start on a multiple of 8 dims and span a multiple of 16).  G = n_q_heads /
 * n_kv_heads must be an integer <= 16; G * W <= 256.  n_kv_heads, the cache's
 * B_max and a prefill call's b are at most 65535 (they index launch grid
 * dimensions): SS_ERR_UNSUPPORTED beyond, and the workspace sizes are 0. */
typedef struct {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t d_qk;
  int32_t d_v;
  int32_t v_aliases_k;  /* 1: value = first d_v dims of the cached key (MLA) */
  int32_t L_sink;       /* >= 0 */
  int32_t K;            /* >= 0, top-K budget of the middle region */
  int32_t L_recent;     /* >= 1, ring length */
  int32_t W;            /* >= 1, observation window (last W prompt queries) */
  int32_t pool;         /* odd, >= 1, max-pool width */
  float scale;          /* softmax scale; 0 -> 1/sqrt(d_qk) */
  float rope_theta;     /* 0 -> no rotary embedding at decode */
  int32_t rope_begin;   /* rotate dims [rope_begin, rope_end) (even length) */
  int32_t rope_end;
  int32_t dtype;        /* ss_dtype of q/k/v, cache and out */
} ss_config;

/* The fixed-shape cache of B_max request rows; device memory, caller-owned,
 * never resized.  Layouts (row-major):
 *   k        [B_max, n_kv_heads, C, d_qk]
 *   v        [B_max, n_kv_heads, C, d_v]   (NULL when v_aliases_k)
 *   slot_pos [B_max, n_kv_heads, C] int32  absolute position held by a slot, -1 empty
 *   n_tokens [B_max] int32                 tokens seen by the row (prompt + decoded)
 * The valid slots of row b are [0, min(n_tokens[b], C)). */
typedef struct {
  void* k;
  void* v;
  int32_t* slot_pos;
  int32_t* n_tokens;
  int32_t B_max;
} ss_cache;

/* Number of cache slots C = L_sink + K + L_recent, or -1 if cfg is invalid. */
int32_t ss_cache_slots(const ss_config* cfg);

/* Workspace (device bytes) needed by ss_prefill_compress for b requests of
 * L prompt tokens, and by ss_decode_step for a cache of B_max rows.  0 if the
 * arguments are invalid.  The prefill size depends on the current device (the
 * score passes split the keys to fill whole rounds of its compute units):
 * query it with the device current that the prefill call will run on. */
size_t ss_prefill_workspace_bytes(const ss_config* cfg, int32_t b, int32_t L);
size_t ss_decode_workspace_bytes(const ss_config* cfg, int32_t B_max);

/* Prepare a decode workspace before its first ss_decode_step: zero the
 * per-(row, kv-head) completion counters at its start (one small kernel on
 * `stream`, no memset, so it may be captured in a graph).  A zero-filled
 * allocation needs no init.  Every ss_decode_step leaves the counters zero
 * again, so the workspace stays ready as long as it is used only by
 * ss_decode_step calls of the same (cfg, B_max), one at a time. */
ss_status ss_decode_workspace_init(const ss_config* cfg, int32_t B_max, void* ws,
                                   size_t ws_bytes, hipStream_t stream);

/* Build the fixed cache of b requests at prefill ("Fixed-Size Cache Layout":
 * built once at prefill; SnapKV scoring of the middle by the observation
 * window, sinks and the recent window always kept).
 *
 *   q_obs  [b, n_q_heads, W, d_qk]   queries of prompt positions L-W .. L-1 (post-RoPE)
 *   k      [b, n_kv_heads, L, d_qk]  prompt keys (post-RoPE)
 *   v      [b, n_kv_heads, L, d_v]   prompt values (NULL when v_aliases_k)
 *   rows   device int32 [b]: destination cache row of each request, or NULL
 *          for rows 0 .. b-1 (continuous-batching admission into chosen rows);
 *          distinct (two requests into one row leave it undefined); a row
 *          outside [0, B_max) is skipped
 *   raw_out    optional device float [b, n_kv_heads, m], m = L - L_sink - L_recent:
 *              the middle-key scores (written only when L > C)
 *   pooled_out optional device float [b, n_kv_heads, m]: the pooled scores
 *   sel_out    optional device int32 [b, n_kv_heads, K]: kept middle tokens as
 *              indices into the middle region, ascending
 *   ws, ws_bytes  device workspace of >= ss_prefill_workspace_bytes(cfg, b, L)
 *
 * Writes, for every request i and kv-head h: cache->k/v rows of slots [0, C)
 * (L > C) or [0, L) (L <= C), slot_pos of all C slots, n_tokens[row] = L.
 * Requires W <= L_recent when L > C (the window lies in the recent region).
 * Enqueued on `stream`; no host synchronisation, no allocation. */
ss_status ss_prefill_compress(const ss_config* cfg, const void* q_obs, const void* k,
                              const void* v, int32_t b, int32_t L, const int32_t* rows,
                              const ss_cache* cache, float* raw_out, float* pooled_out,
                              int32_t* sel_out, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* ss_prefill_compress for a caller that already holds the log-sum-exp of
 * every observation row, as the prefill's own attention (a flash-attention
 * forward) returns it.  The scoring then makes one pass over the middle keys
 * instead of two (the row-statistics pass over all L keys is skipped); the
 * result is the same reading of the score ("Two Ingredients, Fused": SnapKV's
 * attention-based selection, here fed by the attention the prefill computed
 * anyway).
 *
 *   lse_obs  device float [b, n_q_heads, W]: natural-log log-sum-exp of row r
 *            of q-head j, log sum_{i <= L-W+r} exp(scale * q_obs[j, r] . k[i]),
 *            with the config's softmax scale.  Required (NULL:
 *            SS_ERR_INVALID_ARG) and read only when L > C.
 *
 * Every other argument, the workspace size and the results are those of
 * ss_prefill_compress.  The scores follow the given lse: an lse off by d
 * scales that row's probabilities by exp(-d). */
ss_status ss_prefill_compress_lse(const ss_config* cfg, const void* q_obs, const void* k,
                                  const void* v, int32_t b, int32_t L, const float* lse_obs,
                                  const int32_t* rows, const ss_cache* cache, float* raw_out,
                                  float* pooled_out, int32_t* sel_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* ss_prefill_compress for a batch of prompts of different lengths in one
 * call (continuous-batching admissions: "Why This Wasn't Already Standard",
 * requests at different points of their life share one static batch).
 *
 *   k, v        packed per kv-head: [n_kv_heads, T, d_qk] / [n_kv_heads, T, d_v]
 *               (v NULL when v_aliases_k), where request i holds tokens
 *               cu_seqlens[i] .. cu_seqlens[i+1]-1 of every head, T = cu_seqlens[b]
 *   cu_seqlens  device int32 [b+1], non-decreasing, cu_seqlens[0] = 0
 *   max_L       host bound on every prompt length L_i = cu_seqlens[i+1] -
 *               cu_seqlens[i]; it sizes the launch and the workspace
 *               (ss_prefill_workspace_bytes(cfg, b, max_L))
 *   q_obs       [b, n_q_heads, W, d_qk]: the last W queries of each request
 *               (read only for requests with L_i > C)
 *   lse_obs     optional device float [b, n_q_heads, W]: given, the scoring
 *               makes one pass as in ss_prefill_compress_lse; NULL: two passes
 *   raw_out / pooled_out  optional [b, n_kv_heads, max_L - L_sink - L_recent];
 *               request i fills its first L_i - L_sink - L_recent entries
 *   sel_out     optional [b, n_kv_heads, K]
 *
 * Request i is stored uncompressed when L_i <= C and compressed otherwise,
 * exactly as a single-request ss_prefill_compress of its L_i tokens would
 * store it; n_tokens[row] = L_i.  A request whose offsets are not
 * non-decreasing within [0, T], or longer than max_L, is stored as empty
 * (every slot -1, n_tokens 0). */
ss_status ss_prefill_compress_varlen(const ss_config* cfg, const void* q_obs, const void* k,
                                     const void* v, int32_t b, const int32_t* cu_seqlens,
                                     int32_t max_L, const float* lse_obs, const int32_t* rows,
                                     const ss_cache* cache, float* raw_out, float* pooled_out,
                                     int32_t* sel_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* One decode step of every cache row ("Ring Buffer vs. Naive Slicing": write
 * the new key/value into its fixed ring slot, evicting position pos -
 * L_recent; then memory-bound attention over the fixed cache).
 *
 *   q      [B_max, n_q_heads, d_qk]   pre-RoPE query of the new token
 *   k_new  [B_max, n_kv_heads, d_qk]  pre-RoPE key of the new token
 *   v_new  [B_max, n_kv_heads, d_v]   value of the new token (NULL when v_aliases_k)
 *   pos    device int32 [B_max]: absolute position of the new token; < 0 marks
 *          an inactive row (no state change, out row = 0)
 *   out    [B_max, n_q_heads, d_v]    attention output, cache dtype
 *   err_flag  optional device int32: set to 1 when an active row has
 *          pos != n_tokens (the step is still applied at pos); never cleared
 *   ws, ws_bytes  device workspace of >= ss_decode_workspace_bytes(cfg, B_max),
 *          zero-filled or prepared by ss_decode_workspace_init before the
 *          first call (see there); calls sharing a workspace must not overlap
 *
 * One kernel: rotary embedding, ring scatter, split-C attention and the merge
 * of the splits.  Enqueued on `stream`; no host synchronisation, no
 * allocation. */
ss_status ss_decode_step(const ss_config* cfg, const void* q, const void* k_new,
                         const void* v_new, const int32_t* pos, const ss_cache* cache,
                         void* out, int32_t* err_flag, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* ss_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and single kernel as ss_decode_step, without the
 * workspace: the split partials and completion counters live in a static
 * device array of the library (16 MiB per GPU, held until the process ends,
 * looked up on the first call on each device; that first call also enqueues
 * one small kernel on `stream` that zeroes the counters).  No call allocates
 * or frees memory.
 *
 * Limit: B_max * n_kv_heads <= 16384 and the partials of
 * B_max * n_q_heads * n_split * (d_v + 2) fp32 values (n_split as
 * ss_decode_step plans it for the cache shape) within 16 MiB - 64 KiB; larger
 * shapes return SS_ERR_SCRATCH_LIMIT before any launch.  Every shape the
 * workloads of this library use fits (e.g. 64 rows x 32 q-heads x 32768 slots,
 * or 32 rows x 8 latent heads x 32768 slots: about 8.6 MB).
 *
 * All calls on one GPU share the array, which keeps the last call's partials:
 * calls that overlap on one GPU (other streams, other threads, graph replays
 * in flight) race and must be serialised by the caller. */
ss_status ss_decode_step_noalloc(const ss_config* cfg, const void* q, const void* k_new,
                                 const void* v_new, const int32_t* pos, const ss_cache* cache,
                                 void* out, int32_t* err_flag, hipStream_t stream);

/* Profiling variants: identical to the calls above, and additionally record
 * `begin` / `end` on `stream` immediately before and after the dominant
 * kernels - the split-C attention kernel of ss_decode_step, the two score
 * passes (row statistics through column scores) of ss_prefill_compress, the
 * lse conversion and column-score pass of ss_prefill_compress_lse.
 * Either event may be NULL.  The events are caller-created (hipEventCreate);
 * the caller reads hipEventElapsedTime after its own synchronisation.  When a
 * prompt is stored uncompressed (L <= C) no score kernel runs and the two
 * events are recorded back to back. */
ss_status ss_prefill_compress_timed(const ss_config* cfg, const void* q_obs, const void* k,
                                    const void* v, int32_t b, int32_t L, const int32_t* rows,
                                    const ss_cache* cache, float* raw_out, float* pooled_out,
                                    int32_t* sel_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream, hipEvent_t begin, hipEvent_t end);
ss_status ss_prefill_compress_lse_timed(const ss_config* cfg, const void* q_obs, const void* k,
                                        const void* v, int32_t b, int32_t L,
                                        const float* lse_obs, const int32_t* rows,
                                        const ss_cache* cache, float* raw_out,
                                        float* pooled_out, int32_t* sel_out, void* ws,
                                        size_t ws_bytes, hipStream_t stream, hipEvent_t begin,
                                        hipEvent_t end);
ss_status ss_prefill_compress_varlen_timed(const ss_config* cfg, const void* q_obs,
                                           const void* k, const void* v, int32_t b,
                                           const int32_t* cu_seqlens, int32_t max_L,
                                           const float* lse_obs, const int32_t* rows,
                                           const ss_cache* cache, float* raw_out,
                                           float* pooled_out, int32_t* sel_out, void* ws,
                                           size_t ws_bytes, hipStream_t stream,
                                           hipEvent_t begin, hipEvent_t end);
ss_status ss_decode_step_timed(const ss_config* cfg, const void* q, const void* k_new,
                               const void* v_new, const int32_t* pos, const ss_cache* cache,
                               void* out, int32_t* err_flag, void* ws, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t begin, hipEvent_t end);

/* Static description of a status code. */
const char* ss_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SNAPSTREAM_H */
