// C ABI of libsnapstream: argument checks, workspace carving and kernel
// launches.  No allocation, no host synchronisation, no global state.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "snapstream.h"
#include "launch.h"

namespace {

constexpr size_t ALIGN = 256;
// Cache rows, requests and kv-heads index launch grid dimensions y / z,
// whose extent is at most 65535.
constexpr int MAX_GRID_YZ = 65535;
size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

bool supported_shape(const ss_config* c) {
  if (c->v_aliases_k)  // MLA absorbed latent: 512 value dims + rotary dims, bf16; the
                       // rotary range starts and splits on multiples of 8 dims
    return c->dtype == SS_BF16 && c->d_qk == 576 && c->d_v == 512 &&
           (c->rope_theta == 0.f ||
            (c->rope_begin % 8 == 0 && (c->rope_end - c->rope_begin) % 16 == 0));
  if (c->dtype != SS_F32 && c->dtype != SS_BF16) return false;
  return (c->d_qk == 64 && c->d_v == 64) || (c->d_qk == 128 && c->d_v == 128);
}

// Structural validity of a configuration (independent of the call).
ss_status check_config(const ss_config* c) {
  if (c == nullptr) return SS_ERR_INVALID_ARG;
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
    return SS_ERR_INVALID_ARG;
  if (c->d_qk < 1 || c->d_v < 1) return SS_ERR_INVALID_ARG;
  if (c->v_aliases_k && c->d_v > c->d_qk) return SS_ERR_INVALID_ARG;
  if (c->L_sink < 0 || c->K < 0 || c->L_recent < 1 || c->W < 1) return SS_ERR_INVALID_ARG;
  if (c->pool < 1 || c->pool % 2 == 0) return SS_ERR_INVALID_ARG;
  if (!(c->scale >= 0.f) || !isfinite(c->scale)) return SS_ERR_INVALID_ARG;
  if (!(c->rope_theta >= 0.f) || !isfinite(c->rope_theta)) return SS_ERR_INVALID_ARG;
  if (c->rope_theta > 0.f) {
    if (c->rope_begin < 0 || c->rope_end > c->d_qk || c->rope_end <= c->rope_begin ||
        (c->rope_end - c->rope_begin) % 2 != 0)
      return SS_ERR_INVALID_ARG;
  }
  // at most 2^24 slots: keeps every per-head partial range of the decode
  // workspace addressable with 32-bit byte offsets
  const long long C = static_cast<long long>(c->L_sink) + c->K + c->L_recent;
  if (C > ss::MAX_CACHE_SLOTS) return SS_ERR_INVALID_ARG;
  if (c->dtype != SS_F32 && c->dtype != SS_BF16) return SS_ERR_INVALID_ARG;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (!supported_shape(c) || G > 16 || G * c->W > 256 || c->n_kv_heads > MAX_GRID_YZ)
    return SS_ERR_UNSUPPORTED;
  if (c->rope_theta > 0.f && c->rope_end - c->rope_begin > 2 * ss::ROPE_MAX_PAIRS)
    return SS_ERR_UNSUPPORTED;
  return SS_OK;
}

// Tensors are read and written in 16-byte vectors.
bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

int cache_slots(const ss_config* c) { return c->L_sink + c->K + c->L_recent; }
float scale_log2(const ss_config* c) {
  const float s = c->scale > 0.f ? c->scale : 1.0f / sqrtf(static_cast<float>(c->d_qk));
  return s * 1.4426950408889634f;
}

// ---------------------------------------------------------------- prefill
struct PrefillPlan {
  bool compressed;
  int m, Rg, chunk1, n_chunk1, chunk2, n_chunk2, n_part, part_len;
  size_t off_part1, off_rowstat, off_raw, off_pooled, off_sel, off_shist, off_sstate, off_scnt,
      total;
};

PrefillPlan plan_prefill(const ss_config* c, int b, int L) {
  PrefillPlan p{};
  const int C = cache_slots(c);
  p.compressed = L > C;
  if (!p.compressed) return p;
  const int G = c->n_q_heads / c->n_kv_heads;
  p.m = L - c->L_sink - c->L_recent;
  p.Rg = (G * c->W + 15) / 16 * 16;
  const size_t groups = static_cast<size_t>(b) * c->n_kv_heads;
  // chunk lengths that fill whole rounds of the current device; the
  // compile-time defaults when it cannot be queried
  int slots1 = 0, slots2 = 0;
  // the register-query passes stage at most DIRECT_STAGE_KEYS column sums
  // per wave in pass 2
  const int max2 = ss::direct_scores_supported(c->dtype, c->d_qk, p.Rg)
                       ? ss::DIRECT_WAVES * ss::DIRECT_STAGE_KEYS
                       : 0;
  if (ss::prefill_score_slots(c->dtype, c->d_qk, p.Rg, &slots1, &slots2) == hipSuccess) {
    p.chunk1 = ss::score_chunk(L, static_cast<long long>(groups), slots1);
    p.chunk2 = ss::score_chunk(p.m, static_cast<long long>(groups), slots2, max2);
  } else {
    (void)hipGetLastError();  // a failed query leaves no error for later calls
    p.chunk1 = ss::SCORE_CHUNK1;
    p.chunk2 = max2 > 0 && ss::SCORE_CHUNK2 > max2 ? max2 : ss::SCORE_CHUNK2;
  }
  p.n_chunk1 = (L + p.chunk1 - 1) / p.chunk1;
  p.n_chunk2 = (p.m + p.chunk2 - 1) / p.chunk2;
  size_t off = 0;
  p.off_part1 = off;
  off += align_up(groups * p.Rg * p.n_chunk1 * 2 * sizeof(float));
  p.off_rowstat = off;
  off += align_up(groups * p.Rg * 2 * sizeof(float));
  p.off_raw = off;
  off += align_up(groups * p.m * sizeof(float));
  p.off_pooled = off;
  off += align_up(groups * p.m * sizeof(float));
  p.off_sel = off;
  off += align_up(groups * (c->K > 0 ? c->K : 1) * sizeof(int32_t));
  // select: groups longer than SEL_KEEP middle keys are split into parts so
  // that the grid has about SEL_TARGET_WG workgroups
  p.n_part = 1;
  p.part_len = (p.m + 63) / 64 * 64;
  if (p.m > ss::SEL_KEEP) {
    const long long want = (ss::SEL_TARGET_WG + static_cast<long long>(groups) - 1) /
                           static_cast<long long>(groups);
    const long long most = (p.m + ss::SEL_MIN_PART - 1) / ss::SEL_MIN_PART;
    const long long parts = want < most ? want : most;
    if (parts > 1) {
      p.part_len = static_cast<int>((p.m + parts - 1) / parts + 63) / 64 * 64;
      p.n_part = (p.m + p.part_len - 1) / p.part_len;
    }
  }
  p.off_shist = off;
  off += align_up(groups * p.n_part * ss::SEL_HIST_BINS * sizeof(uint32_t));
  p.off_sstate = off;
  off += align_up(groups * 6 * sizeof(uint32_t));
  p.off_scnt = off;
  off += align_up(groups * p.n_part * 2 * sizeof(uint32_t));
  p.total = off;
  return p;
}

// ----------------------------------------------------------------- decode
struct DecodePlan {
  int split, n_split;
  size_t off_cnt, n_cnt, off_o, off_ml, total;
};

// cnt_region: bytes reserved for the counters at the start of the workspace
// (at least what they need): the static scratch keeps a fixed region so that
// its partials never overlap counters of a call of another shape.
DecodePlan plan_decode(const ss_config* c, int B_max, size_t cnt_region = 0) {
  DecodePlan p{};
  const int C = cache_slots(c);
  const long long groups = static_cast<long long>(B_max) * c->n_kv_heads;
  // Each workgroup of DECODE_WAVES waves takes a split of the C slots, dealt
  // to its waves round-robin in tiles of 32 slots, 1 to DECODE_MAX_TILES per
  // wave, so that the grid holds about DECODE_TARGET_WAVES waves when every
  // slot is valid (short splits balance rows of very different valid
  // lengths).
  const long long tiles = (C + ss::DECODE_TILE - 1) / ss::DECODE_TILE;
  if (c->v_aliases_k) {
    // latent (MLA) kernel: the 4 waves of a workgroup share each tile
    long long want_wg = (ss::MLA_TARGET_WG + groups - 1) / groups;
    long long tpg = (tiles + want_wg - 1) / want_wg;
    if (tpg > ss::MLA_MAX_TILES) tpg = ss::MLA_MAX_TILES;
    if (tpg < 1) tpg = 1;
    p.split = static_cast<int>(tpg) * ss::DECODE_TILE;
  } else {
    long long want = (ss::DECODE_TARGET_WAVES + groups - 1) / groups;  // waves per group
    if (want < 1) want = 1;
    long long tpw = (tiles + want - 1) / want;
    if (tpw > ss::DECODE_MAX_TILES) tpw = ss::DECODE_MAX_TILES;
    if (tpw < 1) tpw = 1;
    p.split = ss::DECODE_WAVES * static_cast<int>(tpw) * ss::DECODE_TILE;
  }
  p.n_split = (C + p.split - 1) / p.split;
  const size_t rows_q = static_cast<size_t>(B_max) * c->n_q_heads;
  size_t off = 0;
  p.off_cnt = off;
  p.n_cnt = static_cast<size_t>(groups);
  off += align_up(p.n_cnt * sizeof(int32_t) > cnt_region ? p.n_cnt * sizeof(int32_t) : cnt_region);
  p.off_o = off;
  off += align_up(rows_q * p.n_split * c->d_v * sizeof(float));
  p.off_ml = off;
  off += align_up(rows_q * p.n_split * 2 * sizeof(float));
  p.total = off;
  return p;
}

}  // namespace

extern "C" {

int32_t ss_cache_slots(const ss_config* cfg) {
  const ss_status s = check_config(cfg);
  if (s == SS_ERR_INVALID_ARG) return -1;
  return cache_slots(cfg);
}

size_t ss_prefill_workspace_bytes(const ss_config* cfg, int32_t b, int32_t L) {
  if (check_config(cfg) != SS_OK || b < 1 || b > MAX_GRID_YZ || L < 1) return 0;
  const PrefillPlan p = plan_prefill(cfg, b, L);
  return p.compressed ? p.total : ALIGN;  // a non-zero size keeps the pointer rule uniform
}

size_t ss_decode_workspace_bytes(const ss_config* cfg, int32_t B_max) {
  if (check_config(cfg) != SS_OK || B_max < 1 || B_max > MAX_GRID_YZ) return 0;
  return plan_decode(cfg, B_max).total;
}

ss_status ss_decode_workspace_init(const ss_config* cfg, int32_t B_max, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  const ss_status cs = check_config(cfg);
  if (cs != SS_OK) return cs;
  if (B_max < 1) return SS_ERR_INVALID_ARG;
  if (B_max > MAX_GRID_YZ) return SS_ERR_UNSUPPORTED;
  const DecodePlan p = plan_decode(cfg, B_max);
  if (ws == nullptr || ws_bytes < p.total) return SS_ERR_WORKSPACE;
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.off_cnt);
  if (ss::launch_zero_counters(cnt, static_cast<int>(p.n_cnt), stream) != hipSuccess)
    return SS_ERR_HIP;
  return SS_OK;
}

}  // extern "C"

namespace {

// lse_call: the row log-sum-exp is given (required when a prompt is
// compressed).  cu: request token offsets of a packed varlen batch (device,
// [b+1]); L is then the longest prompt allowed.
ss_status prefill_impl(const ss_config* cfg, const void* q_obs, const void* k, const void* v,
                       int32_t b, int32_t L, bool lse_call, const float* lse,
                       const int32_t* cu, const int32_t* rows, const ss_cache* cache,
                       float* raw_out, float* pooled_out, int32_t* sel_out, void* ws,
                       size_t ws_bytes, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const ss_status cs = check_config(cfg);
  if (cs != SS_OK) return cs;
  if (cache == nullptr || b < 1 || L < 1 || k == nullptr || cache->k == nullptr ||
      cache->slot_pos == nullptr || cache->n_tokens == nullptr || cache->B_max < 1)
    return SS_ERR_INVALID_ARG;
  if (!cfg->v_aliases_k && (v == nullptr || cache->v == nullptr)) return SS_ERR_INVALID_ARG;
  if (misaligned(q_obs) || misaligned(k) || misaligned(v) || misaligned(cache->k) ||
      misaligned(cache->v) || misaligned(ws))
    return SS_ERR_INVALID_ARG;
  if (rows == nullptr && b > cache->B_max) return SS_ERR_INVALID_ARG;
  if (b > MAX_GRID_YZ) return SS_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(cu) & 3) != 0) return SS_ERR_INVALID_ARG;
  const int C = cache_slots(cfg);
  const bool compressed = L > C;  // with cu: some request may be compressed
  if (compressed) {
    if (q_obs == nullptr) return SS_ERR_INVALID_ARG;
    if (cfg->W > L || cfg->W > cfg->L_recent) return SS_ERR_INVALID_ARG;
    if (lse_call && (lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3) != 0))
      return SS_ERR_INVALID_ARG;
  }
  const PrefillPlan p = plan_prefill(cfg, b, L);
  if (ws == nullptr || ws_bytes < (compressed ? p.total : ALIGN)) return SS_ERR_WORKSPACE;

  ss::PrefillArgs a{};
  a.q_obs = q_obs;
  a.k = k;
  a.v = cfg->v_aliases_k ? nullptr : v;
  a.rows = rows;
  a.kc = cache->k;
  a.vc = cfg->v_aliases_k ? nullptr : cache->v;
  a.slot_pos = cache->slot_pos;
  a.n_tokens = cache->n_tokens;
  a.b = b;
  a.B_max = cache->B_max;
  a.L = L;
  a.Hq = cfg->n_q_heads;
  a.Hkv = cfg->n_kv_heads;
  a.G = cfg->n_q_heads / cfg->n_kv_heads;
  a.W = cfg->W;
  a.C = C;
  a.S = cfg->L_sink;
  a.K = cfg->K;
  a.R = cfg->L_recent;
  a.pool = cfg->pool;
  a.scale_log2 = scale_log2(cfg);
  a.cu = cu;
  if (compressed) {
    char* w = static_cast<char*>(ws);
    a.m = p.m;
    a.Rg = p.Rg;
    a.chunk1 = p.chunk1;
    a.n_chunk1 = p.n_chunk1;
    a.chunk2 = p.chunk2;
    a.n_chunk2 = p.n_chunk2;
    a.lse = lse_call ? lse : nullptr;
    a.part1 = reinterpret_cast<float*>(w + p.off_part1);
    a.rowstat = reinterpret_cast<float*>(w + p.off_rowstat);
    a.raw = raw_out ? raw_out : reinterpret_cast<float*>(w + p.off_raw);
    a.pooled = pooled_out ? pooled_out : reinterpret_cast<float*>(w + p.off_pooled);
    a.sel = sel_out ? sel_out : reinterpret_cast<int32_t*>(w + p.off_sel);
    a.n_part = p.n_part;
    a.part_len = p.part_len;
    a.sel_hist = reinterpret_cast<uint32_t*>(w + p.off_shist);
    a.sel_state = reinterpret_cast<uint32_t*>(w + p.off_sstate);
    a.sel_cnt = reinterpret_cast<uint32_t*>(w + p.off_scnt);
    if (ss::launch_prefill_scores(cfg->dtype, cfg->d_qk, a, stream, ev0, ev1) != hipSuccess)
      return SS_ERR_HIP;
    if (ss::launch_prefill_select(a, stream) != hipSuccess) return SS_ERR_HIP;
  } else {
    if (ev0 != nullptr && hipEventRecord(ev0, stream) != hipSuccess) return SS_ERR_HIP;
    if (ev1 != nullptr && hipEventRecord(ev1, stream) != hipSuccess) return SS_ERR_HIP;
  }
  if (ss::launch_prefill_gather(cfg->dtype, cfg->d_qk, cfg->d_v, cfg->v_aliases_k, compressed, a,
                                stream) != hipSuccess)
    return SS_ERR_HIP;
  return SS_OK;
}

// use_static: the workspace is the library's static scratch (ws, ws_bytes
// ignored).
ss_status decode_impl(const ss_config* cfg, const void* q, const void* k_new, const void* v_new,
                      const int32_t* pos, const ss_cache* cache, void* out, int32_t* err_flag,
                      void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t ev0,
                      hipEvent_t ev1, bool use_static = false) {
  const ss_status cs = check_config(cfg);
  if (cs != SS_OK) return cs;
  if (cache == nullptr || q == nullptr || k_new == nullptr || pos == nullptr || out == nullptr ||
      cache->k == nullptr || cache->slot_pos == nullptr || cache->n_tokens == nullptr ||
      cache->B_max < 1)
    return SS_ERR_INVALID_ARG;
  if (!cfg->v_aliases_k && (v_new == nullptr || cache->v == nullptr)) return SS_ERR_INVALID_ARG;
  if (misaligned(q) || misaligned(k_new) || misaligned(v_new) || misaligned(cache->k) ||
      misaligned(cache->v) || (!use_static && misaligned(ws)))
    return SS_ERR_INVALID_ARG;
  if (cache->B_max > MAX_GRID_YZ) return SS_ERR_UNSUPPORTED;
  const DecodePlan p =
      plan_decode(cfg, cache->B_max, use_static ? ss::STATIC_SCRATCH_PARTIALS_OFF : 0);
  if (use_static) {
    if (p.n_cnt > static_cast<size_t>(ss::STATIC_SCRATCH_COUNTERS) ||
        p.total > ss::STATIC_SCRATCH_BYTES)
      return SS_ERR_SCRATCH_LIMIT;
    if (ss::static_scratch(&ws, stream) != hipSuccess) return SS_ERR_HIP;
    ws_bytes = ss::STATIC_SCRATCH_BYTES;
  }
  if (ws == nullptr || ws_bytes < p.total) return SS_ERR_WORKSPACE;

  ss::DecodeArgs a{};
  char* w = static_cast<char*>(ws);
  a.q = q;
  a.k_new = k_new;
  a.v_new = cfg->v_aliases_k ? nullptr : v_new;
  a.pos = pos;
  a.kc = cache->k;
  a.vc = cfg->v_aliases_k ? nullptr : cache->v;
  a.slot_pos = cache->slot_pos;
  a.n_tokens = cache->n_tokens;
  a.out = out;
  a.err = err_flag;
  a.counter = reinterpret_cast<int32_t*>(w + p.off_cnt);
  a.part_o = reinterpret_cast<float*>(w + p.off_o);
  a.part_ml = reinterpret_cast<float*>(w + p.off_ml);
  a.B = cache->B_max;
  a.Hq = cfg->n_q_heads;
  a.Hkv = cfg->n_kv_heads;
  a.G = cfg->n_q_heads / cfg->n_kv_heads;
  a.C = cache_slots(cfg);
  a.S = cfg->L_sink;
  a.K = cfg->K;
  a.R = cfg->L_recent;
  a.split = p.split;
  a.n_split = p.n_split;
  a.scale_log2 = scale_log2(cfg);
  a.rope_begin = cfg->rope_begin;
  a.rope_half = cfg->rope_theta > 0.f ? (cfg->rope_end - cfg->rope_begin) / 2 : 0;
  for (int i = 0; i < a.rope_half; ++i)  // libm pow, as in the oracle
    a.inv_freq[i] = pow(static_cast<double>(cfg->rope_theta),
                        -2.0 * i / (cfg->rope_end - cfg->rope_begin));
  if (ss::launch_decode(cfg->dtype, cfg->d_qk, cfg->d_v, cfg->v_aliases_k, a, stream, ev0, ev1) !=
      hipSuccess)
    return SS_ERR_HIP;
  return SS_OK;
}

}  // namespace

extern "C" {

ss_status ss_prefill_compress(const ss_config* cfg, const void* q_obs, const void* k,
                              const void* v, int32_t b, int32_t L, const int32_t* rows,
                              const ss_cache* cache, float* raw_out, float* pooled_out,
                              int32_t* sel_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(cfg, q_obs, k, v, b, L, false, nullptr, nullptr, rows, cache, raw_out,
                      pooled_out, sel_out, ws, ws_bytes, stream, nullptr, nullptr);
}

ss_status ss_prefill_compress_timed(const ss_config* cfg, const void* q_obs, const void* k,
                                    const void* v, int32_t b, int32_t L, const int32_t* rows,
                                    const ss_cache* cache, float* raw_out, float* pooled_out,
                                    int32_t* sel_out, void* ws, size_t ws_bytes,
                                    hipStream_t stream, hipEvent_t begin, hipEvent_t end) {
  return prefill_impl(cfg, q_obs, k, v, b, L, false, nullptr, nullptr, rows, cache, raw_out,
                      pooled_out, sel_out, ws, ws_bytes, stream, begin, end);
}

ss_status ss_prefill_compress_lse(const ss_config* cfg, const void* q_obs, const void* k,
                                  const void* v, int32_t b, int32_t L, const float* lse_obs,
                                  const int32_t* rows, const ss_cache* cache, float* raw_out,
                                  float* pooled_out, int32_t* sel_out, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  return prefill_impl(cfg, q_obs, k, v, b, L, true, lse_obs, nullptr, rows, cache, raw_out,
                      pooled_out, sel_out, ws, ws_bytes, stream, nullptr, nullptr);
}

ss_status ss_prefill_compress_lse_timed(const ss_config* cfg, const void* q_obs, const void* k,
                                        const void* v, int32_t b, int32_t L,
                                        const float* lse_obs, const int32_t* rows,
                                        const ss_cache* cache, float* raw_out,
                                        float* pooled_out, int32_t* sel_out, void* ws,
                                        size_t ws_bytes, hipStream_t stream, hipEvent_t begin,
                                        hipEvent_t end) {
  return prefill_impl(cfg, q_obs, k, v, b, L, true, lse_obs, nullptr, rows, cache, raw_out,
                      pooled_out, sel_out, ws, ws_bytes, stream, begin, end);
}

ss_status ss_prefill_compress_varlen(const ss_config* cfg, const void* q_obs, const void* k,
                                     const void* v, int32_t b, const int32_t* cu_seqlens,
                                     int32_t max_L, const float* lse_obs, const int32_t* rows,
                                     const ss_cache* cache, float* raw_out, float* pooled_out,
                                     int32_t* sel_out, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  if (cu_seqlens == nullptr) return SS_ERR_INVALID_ARG;
  return prefill_impl(cfg, q_obs, k, v, b, max_L, lse_obs != nullptr, lse_obs, cu_seqlens, rows,
                      cache, raw_out, pooled_out, sel_out, ws, ws_bytes, stream, nullptr,
                      nullptr);
}

ss_status ss_prefill_compress_varlen_timed(const ss_config* cfg, const void* q_obs,
                                           const void* k, const void* v, int32_t b,
                                           const int32_t* cu_seqlens, int32_t max_L,
                                           const float* lse_obs, const int32_t* rows,
                                           const ss_cache* cache, float* raw_out,
                                           float* pooled_out, int32_t* sel_out, void* ws,
                                           size_t ws_bytes, hipStream_t stream,
                                           hipEvent_t begin, hipEvent_t end) {
  if (cu_seqlens == nullptr) return SS_ERR_INVALID_ARG;
  return prefill_impl(cfg, q_obs, k, v, b, max_L, lse_obs != nullptr, lse_obs, cu_seqlens, rows,
                      cache, raw_out, pooled_out, sel_out, ws, ws_bytes, stream, begin, end);
}

ss_status ss_decode_step(const ss_config* cfg, const void* q, const void* k_new,
                         const void* v_new, const int32_t* pos, const ss_cache* cache, void* out,
                         int32_t* err_flag, void* ws, size_t ws_bytes, hipStream_t stream) {
  return decode_impl(cfg, q, k_new, v_new, pos, cache, out, err_flag, ws, ws_bytes, stream,
                     nullptr, nullptr);
}

ss_status ss_decode_step_timed(const ss_config* cfg, const void* q, const void* k_new,
                               const void* v_new, const int32_t* pos, const ss_cache* cache,
                               void* out, int32_t* err_flag, void* ws, size_t ws_bytes,
                               hipStream_t stream, hipEvent_t begin, hipEvent_t end) {
  return decode_impl(cfg, q, k_new, v_new, pos, cache, out, err_flag, ws, ws_bytes, stream, begin,
                     end);
}

ss_status ss_decode_step_noalloc(const ss_config* cfg, const void* q, const void* k_new,
                                 const void* v_new, const int32_t* pos, const ss_cache* cache,
                                 void* out, int32_t* err_flag, hipStream_t stream) {
  return decode_impl(cfg, q, k_new, v_new, pos, cache, out, err_flag, nullptr, 0, stream, nullptr,
                     nullptr, true);
}

const char* ss_status_string(int32_t status) {
  switch (status) {
    case SS_OK: return "ok";
    case SS_ERR_INVALID_ARG: return "invalid argument";
    case SS_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SS_ERR_WORKSPACE: return "workspace too small";
    case SS_ERR_HIP: return "HIP launch error";
    case SS_ERR_SCRATCH_LIMIT: return "shapes need more than the static decode scratch";
    default: return "unknown status";
  }
}

}  // extern "C"
