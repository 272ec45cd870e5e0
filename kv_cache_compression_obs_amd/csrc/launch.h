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
  int wsplit;            // slots per wave (multiple of 32); split = DECODE_WAVES * wsplit
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
hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t st);
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
constexpr int DECODE_TARGET_WAVES = SS_DECODE_TARGET_WAVES;
constexpr int DECODE_MAX_TILES = SS_DECODE_MAX_TILES;
// LDS row stride of the decode V tile (bytes) for value rows of `row_bytes`
// (+32 B keeps the transposed 16-bit reads of the 4 lane groups on disjoint
// banks).
constexpr int decode_vrow_stride(int row_bytes) { return row_bytes + 32; }
constexpr int SCORE_KT_MAX = 64;  // keys per score tile (chunks are multiples of it)
// Keys per workgroup of the two score passes (multiples of SCORE_KT_MAX).
#ifndef SS_SCORE_CHUNK1
#define SS_SCORE_CHUNK1 2048
#endif
#ifndef SS_SCORE_CHUNK2
#define SS_SCORE_CHUNK2 1024
#endif
constexpr int SCORE_CHUNK1 = SS_SCORE_CHUNK1;
constexpr int SCORE_CHUNK2 = SS_SCORE_CHUNK2;

}  // namespace ss
