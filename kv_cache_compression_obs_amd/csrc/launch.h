// Internal launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ss {

constexpr int ROPE_MAX_PAIRS = 64;  // rotary range of at most 128 dims
constexpr long long MAX_CACHE_SLOTS = 1LL << 24;

struct DecodeArgs {
  const void* q;         // [B, Hq, D] pre-RoPE
  const void* k_new;     // [B, Hkv, D] pre-RoPE
  const void* v_new;     // [B, Hkv, DV] or null (aliased)
  const int32_t* pos;    // [B]
  void* kc;              // cache k [B, Hkv, C, D]
  void* vc;              // cache v [B, Hkv, C, DV] or null (aliased)
  int32_t* slot_pos;     // [B, Hkv, C]
  int32_t* n_tokens;     // [B]
  void* out;             // [B, Hq, DV]
  int32_t* err;          // optional
  float* part_o;         // ws: [B, Hq, n_split, DV] unnormalised partial outputs
  float* part_ml;        // ws: [B, Hq, n_split, 2] (running max in log2 units, sum)
  int32_t* counter;      // ws: [B, Hkv] finished-split counters, zero between calls
  int B, Hq, Hkv, G, C, S, K, R;
  int split, n_split;    // slots per workgroup split, number of splits
  float scale_log2;      // softmax scale * log2(e)
  int rope_begin;        // rotated dims [rope_begin, rope_begin + 2*rope_half)
  int rope_half;         // rotation pairs; 0: no rotation
  double inv_freq[ROPE_MAX_PAIRS];  // theta^(-2i/d_rot), computed on the host
};

struct PrefillArgs {
  const void* q_obs;     // [b, Hq, W, D]
  const void* k;         // [b, Hkv, L, D]
  const void* v;         // [b, Hkv, L, DV] or null (aliased)
  const int32_t* rows;   // [b] destination rows or null
  void* kc;              // cache k [B_max, Hkv, C, D]
  void* vc;              // cache v or null
  int32_t* slot_pos;
  int32_t* n_tokens;
  const float* lse;      // [b, Hq, W] given row log-sum-exp (natural log) or null
  const int32_t* cu;     // [b+1] request token offsets (packed [Hkv, cu[b], d] keys) or null
  float* part1;          // ws: [b, Hkv, Rg, n_chunk1, 2] per-chunk (max, sum)
  float* rowstat;        // ws: [b, Hkv, Rg, 2] (max, 1/sum)
  float* raw;            // [b, Hkv, m]
  float* pooled;         // [b, Hkv, m]
  int32_t* sel;          // [b, Hkv, K]
  int b, B_max, L, Hq, Hkv, G, W, C, S, K, R, pool, m;
  int Rg;                // rows per group padded to a multiple of 16
  int chunk1, n_chunk1;  // keys per row-stat workgroup, count
  int chunk2, n_chunk2;  // middle keys per column-score workgroup, count
  float scale_log2;
  // select split over several workgroups per group (n_part > 1): parts of
  // part_len middle keys (a multiple of 64), per-part digit histograms
  // [b, Hkv, n_part, SEL_HIST_BINS], the radix state after each digit
  // [b, Hkv, 3, 2] and per-part (greater, equal) counts [b, Hkv, n_part, 2]
  int n_part, part_len;
  uint32_t* sel_hist;
  uint32_t* sel_state;
  uint32_t* sel_cnt;
};

// The prompt of request bi: its length and the row of k (and of v) that
// holds its first token for kv-head h.  Without `cu` every request has a.L
// tokens in [b, Hkv, L, d] layout; with `cu` the requests are packed per
// kv-head ([Hkv, cu[b], d]) and a.L is the longest allowed.  Offsets that are
// not non-decreasing, or a request longer than a.L, make that request empty.
struct Prompt {
  int L;
  size_t row0;
};
__device__ __forceinline__ Prompt prompt_of(const PrefillArgs& a, int bi, int h) {
  if (a.cu == nullptr) return {a.L, (static_cast<size_t>(bi) * a.Hkv + h) * a.L};
  const int c0 = a.cu[bi], c1 = a.cu[bi + 1], T = a.cu[a.b];
  const bool ok = c0 >= 0 && c0 <= c1 && c1 <= T && c1 - c0 <= a.L;
  return {ok ? c1 - c0 : 0, static_cast<size_t>(h) * T + (ok ? c0 : 0)};
}

// Returns hipErrorInvalidValue when no kernel exists for (dtype, D, DV).
// ev0/ev1 (nullable) are recorded right before/after the dominant kernels.
hipError_t launch_decode(int dtype, int D, int DV, int alias, const DecodeArgs& a,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_prefill_scores(int dtype, int D, const PrefillArgs& a, hipStream_t st,
                                 hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_decode_mla(int dtype, int D, int DV, const DecodeArgs& a, hipStream_t st,
                             hipEvent_t ev0, hipEvent_t ev1);
// bf16 K/V caches of D = DV = 64 or 128 dims (decode_ring.hip).
hipError_t launch_decode_ring(int D, const DecodeArgs& a, hipStream_t st, hipEvent_t ev0,
                              hipEvent_t ev1);
hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t st);

// The library's own decode scratch for callers that cannot allocate: a
// device array of STATIC_SCRATCH_BYTES per GPU, held until the process ends.
// Its first STATIC_SCRATCH_COUNTERS int32 are the completion counters (this
// region is never used for anything else, so the counters stay zero between
// calls whatever their shapes); the split partials follow from
// STATIC_SCRATCH_PARTIALS_OFF.  static_scratch returns the array's device
// address on the current device, looking it up (and zeroing the counters on
// `st`) the first time it is asked for on that device.
constexpr size_t STATIC_SCRATCH_BYTES = size_t(16) << 20;
constexpr int STATIC_SCRATCH_COUNTERS = 16384;
constexpr size_t STATIC_SCRATCH_PARTIALS_OFF = STATIC_SCRATCH_COUNTERS * sizeof(int32_t);
hipError_t static_scratch(void** ptr, hipStream_t st);
hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t st);
hipError_t launch_prefill_gather(int dtype, int D, int DV, int alias, bool compressed,
                                 const PrefillArgs& a, hipStream_t st);

// Tiling constants the host uses to size workspaces.
constexpr int DECODE_TILE = 32;   // slots per decode tile
constexpr int DECODE_WAVES = 4;   // waves per decode workgroup
// Decode grid: aim for this many waves when every slot is valid, with at most
// this many tiles per wave (compile-time tunables).
#ifndef SS_DECODE_TARGET_WAVES
#define SS_DECODE_TARGET_WAVES 2048
#endif
#ifndef SS_DECODE_MAX_TILES
#define SS_DECODE_MAX_TILES 32
#endif
// Latent (MLA) decode grid: aim for this many workgroups when every slot is
// valid, with at most SS_MLA_MAX_TILES tiles per workgroup.
#ifndef SS_MLA_TARGET_WG
#define SS_MLA_TARGET_WG 512
#endif
#ifndef SS_MLA_MAX_TILES
#define SS_MLA_MAX_TILES 64
#endif
constexpr int MLA_TARGET_WG = SS_MLA_TARGET_WG;
constexpr int MLA_MAX_TILES = SS_MLA_MAX_TILES;
// bf16 K/V decode through the direct-load LDS ring (decode_ring.hip); 0 keeps
// it on decode_kernel (register tiles), as fp32 caches are.
#ifndef SS_DECODE_RING
#define SS_DECODE_RING 1
#endif
constexpr int DECODE_TARGET_WAVES = SS_DECODE_TARGET_WAVES;
constexpr int DECODE_MAX_TILES = SS_DECODE_MAX_TILES;
// LDS row stride of the decode V tile (bytes) for value rows of `row_bytes`
// (+32 B keeps the transposed 16-bit reads of the 4 lane groups on disjoint
// banks).
constexpr int decode_vrow_stride(int row_bytes) { return row_bytes + 32; }
constexpr int SCORE_KT_MAX = 64;  // keys per score tile (chunks are multiples of it)
// Keys per workgroup of the two score passes when the device cannot be
// queried (multiples of SCORE_KT_MAX); otherwise the host sizes the chunks so
// that the workgroups fill whole rounds of the device (see score_chunk).
#ifndef SS_SCORE_CHUNK1
#define SS_SCORE_CHUNK1 2048
#endif
#ifndef SS_SCORE_CHUNK2
#define SS_SCORE_CHUNK2 1024
#endif
constexpr int SCORE_CHUNK1 = SS_SCORE_CHUNK1;
constexpr int SCORE_CHUNK2 = SS_SCORE_CHUNK2;
// Fixed cost of one score workgroup (start, queries, final reduction) in
// keys, for the chunk choice.
constexpr int SCORE_WG_OVERHEAD_KEYS = 128;
// Key tiles in flight per score workgroup (ring slots in LDS), capped by an
// LDS budget per workgroup.
#ifndef SS_SCORE_NBUF
#define SS_SCORE_NBUF 2
#endif
constexpr int SCORE_NBUF = SS_SCORE_NBUF;
// Score key tiles in LDS: 1 = XOR-permuted bf16 rows of 128 or 256 bytes,
// 0 = padded rows (affine fragment addresses; see KeyRing::pitch).
#ifndef SS_SCORE_SWIZZLE
#define SS_SCORE_SWIZZLE 1
#endif
constexpr bool SCORE_SWIZZLE = SS_SCORE_SWIZZLE != 0;
constexpr int SCORE_LDS_BUDGET = 156 * 1024;
// Select: a group's pooled scores stay in LDS (one workgroup) up to this many
// middle keys; longer groups are split over several workgroups, of at least
// SEL_MIN_PART keys each, aiming at SEL_TARGET_WG workgroups in all.
constexpr int SEL_KEEP = 16384;
constexpr int SEL_MIN_PART = 4096;
constexpr int SEL_TARGET_WG = 256;
constexpr int SEL_HIST_BINS = 2048 + 2048 + 512;  // the three radix digits

// Score passes with the group's query rows in registers (score.hip), for
// groups of at most 128 rows of 64 or 128 dims: DIRECT_WAVES waves per
// workgroup, each with a ring of DIRECT_RING1 (pass 1) / DIRECT_RING2
// (pass 2) 16-key tiles in LDS; pass 2 stages the sums of at most
// DIRECT_STAGE_KEYS keys per wave, which bounds its chunk at
// DIRECT_WAVES * DIRECT_STAGE_KEYS keys.  DIRECT_CPOL: cache-policy bits of
// the direct key loads (2: nt, non-temporal; each key is read once per pass).
#ifndef SS_DIRECT_RING1
#define SS_DIRECT_RING1 4
#endif
#ifndef SS_DIRECT_RING2
#define SS_DIRECT_RING2 4
#endif
#ifndef SS_DIRECT_CPOL
#define SS_DIRECT_CPOL 2
#endif
constexpr int DIRECT_WAVES = 4;
constexpr int DIRECT_RING1 = SS_DIRECT_RING1;
constexpr int DIRECT_RING2 = SS_DIRECT_RING2;
constexpr int DIRECT_CPOL = SS_DIRECT_CPOL;
#ifndef SS_DIRECT_STAGE_KEYS
#define SS_DIRECT_STAGE_KEYS 1024
#endif
constexpr int DIRECT_STAGE_KEYS = SS_DIRECT_STAGE_KEYS;
bool direct_scores_supported(int dtype, int D, int Rg);
hipError_t launch_direct_scores(int dtype, int D, const PrefillArgs& a, hipStream_t st,
                                hipEvent_t ev0, hipEvent_t ev1);
hipError_t direct_score_slots(int dtype, int D, int Rg, int* slots1, int* slots2);
// the row-statistics kernels shared by both score paths (prefill.hip)
void launch_lse_rowstat(const PrefillArgs& a, unsigned grid, hipStream_t st);
void launch_rowstat_combine(const PrefillArgs& a, unsigned grid, hipStream_t st);

// Workgroups of score pass 1 / pass 2 that run at once on the current
// device (compute units x resident workgroups per unit) for this dtype, head
// size and padded group row count; hipErrorInvalidValue for a shape without
// kernels, or the HIP error of the device query.
hipError_t prefill_score_slots(int dtype, int D, int Rg, int* slots1, int* slots2);

// Keys per workgroup for `keys` keys in each of `groups` groups when `slots`
// workgroups run at once: the multiple of SCORE_KT_MAX that minimises
// rounds x (chunk + SCORE_WG_OVERHEAD_KEYS).
// max_chunk (> 0): no chunk longer than that many keys.
inline int score_chunk(int keys, long long groups, int slots, int max_chunk = 0) {
  const int tiles = (keys + SCORE_KT_MAX - 1) / SCORE_KT_MAX;
  const int max_ct = max_chunk > 0 ? max_chunk / SCORE_KT_MAX : tiles;
  int best = -1;
  long long best_cost = -1;
  for (int n = 1; n <= tiles; ++n) {
    const int ct = (tiles + n - 1) / n;  // tiles per chunk
    if (ct > max_ct) continue;
    const int n_eff = (tiles + ct - 1) / ct;
    const long long rounds = (groups * n_eff + slots - 1) / slots;
    const long long cost =
        rounds * (static_cast<long long>(ct) * SCORE_KT_MAX + SCORE_WG_OVERHEAD_KEYS);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = ct * SCORE_KT_MAX;
    }
  }
  return best > 0 ? best : max_ct * SCORE_KT_MAX;
}

}  // namespace ss
