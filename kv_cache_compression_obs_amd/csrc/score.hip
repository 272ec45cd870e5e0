// Observation-window scoring with the query rows of a group held in
// registers: the two score passes for groups of at most 128 query rows
// (G * W <= 128) of 64 or 128 dims.
//
// "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators", section
// "Two Ingredients, Fused": SnapKV's attention-based selection.  The score of
// middle key i sums, over the G q-heads of its kv-head and the last W prompt
// queries, that query's causal softmax probability of key i.  Pass 1
// (row statistics over every prompt key) and pass 2 (column sums over the
// middle keys) compute the same quantities as the shared-tile kernels in
// prefill.hip (which serve the latent and the 256-row groups), with another
// division of the work:
//
//  - each wave owns its own keys: 16-key tiles are dealt to the NW waves of a
//    workgroup round-robin (wave w: tiles w, w + NW, ...), so a workgroup
//    streams one compact window of keys and no key is read twice;
//  - every wave holds all NQB*16 query rows of the group in registers, as the
//    B operand (columns) of v_mfma_f32_16x16x32_bf16 (16x16x4 f32 for fp32);
//    the keys are the A operand (rows), so the accumulator of q-block qb in
//    lane (col, qg), register r, holds the logit of key 4*qg + r of the tile
//    for query row 16*qb + col;
//  - a wave's tiles land in a ring of NS slots of its own in LDS through
//    direct global->LDS loads (no registers), issued NS - 1 tiles ahead and
//    awaited with the wave's own vmcnt: no workgroup barrier in the loop, so
//    the waves drift apart and one wave's exponentials overlap another's
//    MFMAs;
//  - pass 2 sums a key's probabilities over the rows inside one wave: over
//    the q-blocks in registers, then over the 16 columns of a lane row with
//    four DPP steps (row mirror, row half-mirror, two quad permutes);
//  - the direct loads carry the non-temporal cache policy (DIRECT_CPOL): each
//    key is read once per pass.  Measured on llama8b-shaped prefill (16 x 8
//    groups of 16384 keys), pass 1 took 142 us with the default policy and
//    100 us with nt, and a loads-only build of the same passes reached
//    6.8 TB/s with it.
//
// Key rows in a ring slot: unit u (16 bytes) of tile row r is stored at
// position r * UPK + (u ^ swz(r)), which makes the A-fragment reads (16 lanes
// = 16 rows, the same unit) conflict-free: a 16-byte LDS read is served in
// groups of 32 lanes over 512 bytes of banks, and the 32 lanes' positions
// differ modulo 32.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace ss {

namespace {

typedef const __attribute__((address_space(1))) void* gptr;
typedef __attribute__((address_space(3))) void* lptr;

// Operand pieces of a 16-byte vector: bf16 -> one 8-element fragment; fp32
// -> four single-element fragments (MFMA steps).
template <typename T> struct Piece;
template <> struct Piece<bf16_t> {
  static constexpr int N = 1;
  static __device__ __forceinline__ bf16x8_t get(u32x4_t v, int) {
    return __builtin_bit_cast(bf16x8_t, v);
  }
};
template <> struct Piece<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ float get(u32x4_t v, int e) { return __uint_as_float(v[e]); }
};

template <typename T, int D>
struct Geo {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int UPK = D * ES / 16;         // 16-byte units per key row
  static constexpr int NJ = UPK / 4;              // units per lane per key row (lane group qg: 4j + qg)
  static constexpr int NI = 16 * UPK / 64;        // 1 KB direct loads per 16-key tile
  static constexpr int TB = 16 * UPK * 16;        // bytes per tile
  static_assert(UPK == 8 || UPK == 16 || UPK == 32, "key rows of 128, 256 or 512 bytes");
  // unit permutation of tile row r (see the file comment)
  static __device__ __forceinline__ int swz(int r) {
    if constexpr (UPK == 8) return 2 * ((r >> 2) & 3);
    else if constexpr (UPK == 16) return r & 15;
    else return (2 * r) & 31;
  }

  static constexpr int ROWB = D * ES;              // bytes per key row

  // Byte offset, from the tile's first key row, of the unit that lane
  // `lane` of direct load i brings (the ring position it writes is
  // i * 1024 + 16 * lane).
  static __device__ __forceinline__ void lane_offsets(int (&lo)[NI], int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = i * 64 + lane;
      const int r = p / UPK;
      lo[i] = r * ROWB + ((p % UPK) ^ swz(r)) * 16;
    }
  }

  // Tile of 16 keys t0 .. t0+15 (rows clamped to kend-1) into ring slot
  // `slot`.  A whole tile is addressed as one wave-uniform base plus the
  // lane offsets; only a tile that crosses kend clamps per lane.
  static __device__ __forceinline__ void issue_tile(char* slot, const T* kbase, int t0, int kend,
                                                    int lane, const int (&lo)[NI]) {
    if (t0 + 16 <= kend) {  // wave-uniform
      const char* base = reinterpret_cast<const char*>(kbase) + static_cast<size_t>(t0) * ROWB;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        __builtin_amdgcn_global_load_lds((gptr)(base + lo[i]), (lptr)(slot + i * 1024), 16, 0,
                                         DIRECT_CPOL);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int p = i * 64 + lane;
        const int r = p / UPK;
        const int u = (p % UPK) ^ swz(r);
        const int key = min(t0 + r, kend - 1);
        const char* src = reinterpret_cast<const char*>(kbase) + static_cast<size_t>(key) * ROWB +
                          u * 16;
        __builtin_amdgcn_global_load_lds((gptr)src, (lptr)(slot + i * 1024), 16, 0, DIRECT_CPOL);
      }
    }
  }

  // The group's query rows as B operands: q[qb][j] = unit 4j + qg of row
  // 16*qb + col (zero past G*W).
  template <int NQB>
  static __device__ __forceinline__ void load_q(u32x4_t (&q)[NQB][NJ], const PrefillArgs& a, int bi,
                                                int h, int col, int qg) {
    const char* q0 = reinterpret_cast<const char*>(
        static_cast<const T*>(a.q_obs) +
        (static_cast<size_t>(bi) * a.Hq + static_cast<size_t>(h) * a.G) * a.W * D);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int row = 16 * qb + col;
      const bool ok = row < a.G * a.W;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        q[qb][j] = ok ? *reinterpret_cast<const u32x4_t*>(q0 + static_cast<size_t>(row) * D * ES +
                                                          (4 * j + qg) * 16)
                      : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // This lane's A-operand units of the tile in `slot`.
  static __device__ __forceinline__ void read_a(u32x4_t (&av)[NJ], const char* slot,
                                                const int (&aoff)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) av[j] = *reinterpret_cast<const u32x4_t*>(slot + aoff[j]);
  }

  // Logits of the tile's 16 keys against the 16 query rows of one q-block.
  static __device__ __forceinline__ f32x4_t logits(const u32x4_t (&av)[NJ], const u32x4_t (&qv)[NJ]) {
    using MM = Mma<T>;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < Piece<T>::N; ++e)
        acc = MM::mma(Piece<T>::get(av[j], e), Piece<T>::get(qv[j], e), acc);
    return acc;
  }

  // Logits of the tile against every q-block, the MFMAs issued slice by
  // slice over all q-blocks: NQB independent accumulators between two MFMAs
  // of one chain, where logits() runs each q-block's chain back to back.
  // The same MFMAs in the same order per q-block, so the same logits.
  template <int NQB>
  static __device__ __forceinline__ void logits_all(f32x4_t (&acc)[NQB], const u32x4_t (&av)[NJ],
                                                    const u32x4_t (&qv)[NQB][NJ]) {
    using MM = Mma<T>;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < Piece<T>::N; ++e)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          acc[qb] = MM::mma(Piece<T>::get(av[j], e), Piece<T>::get(qv[qb][j], e),
                            (j == 0 && e == 0) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[qb]);
  }

  // Byte offsets of this lane's A-operand units in a ring slot.
  static __device__ __forceinline__ void a_offsets(int (&aoff)[NJ], int col, int qg) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) aoff[j] = (col * UPK + ((4 * j + qg) ^ swz(col))) * 16;
  }
};

// Wait until at most N direct loads of this wave are in flight (vector
// memory operations of one wave complete in issue order while only loads
// are in flight; no store is issued inside the loops).
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <- 15 - i within a row of 16
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- 7 - i within each half row
constexpr int DPP_XOR1 = 0xB1;              // quad_perm [1, 0, 3, 2]
constexpr int DPP_XOR2 = 0x4E;              // quad_perm [2, 3, 0, 1]

constexpr float EMPTY = -0x1p126f;  // reference max of a row that has seen no key (finite)

// Pass 1.  Grid (n_chunk1, Hkv, b), NW waves.  Per lane and query row (one
// per q-block: row 16*qb + col) a reference value m (log2 units) and the sum
// of 2^(x - m) over the keys the lane sees (fp32 per tile, fp64 across
// tiles).  The terms are computed with the current m; only when a tile's
// four terms sum past 2^OVER (or overflow: m starts at -2^126) does the lane
// raise m to the tile's largest logit and recompute them.  m is therefore
// always a logit the lane has seen, the terms stay below 2^OVER, and no
// per-tile maximum is needed on the common path, so the exponentials of one
// q-block can run while the MFMAs of the next are in flight.  The lanes and
// waves of a row are merged at the end; the workgroup writes one (max, sum)
// per row and chunk.
template <typename T, int D, int NQB, int NW, int NS>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW * NS * Geo<T, D>::TB <= 80 * 1024 ? 2 : 1)))
void direct_rowstat_kernel(PrefillArgs a) {
  using GG = Geo<T, D>;
  constexpr float OVER = 0x1p64f;
  constexpr int WB = NS * GG::TB;
  static_assert(NW * 16 * NQB * 12 <= NW * WB, "row merge fits in the rings");
  __shared__ __attribute__((aligned(1024))) char lds[NW * WB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const Prompt pr = prompt_of(a, bi, h);
  if (pr.L <= a.C || chunk * a.chunk1 >= pr.L) return;  // stored as is / past the prompt
  const int k0 = chunk * a.chunk1, k1 = min(k0 + a.chunk1, pr.L);
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;
  char* ring = lds + wave * WB;
  const int first = k0 + 16 * wave;  // this wave's tiles: first, first + 16*NW, ...
  const int ntile = first < k1 ? (k1 - first + 16 * NW - 1) / (16 * NW) : 0;

  u32x4_t q[NQB][GG::NJ];
  GG::template load_q<NQB>(q, a, bi, h, col, qg);
  int aoff[GG::NJ], lo[GG::NI];
  GG::a_offsets(aoff, col, qg);
  GG::lane_offsets(lo, lane);
  const float sc = a.scale_log2;
  float m[NQB];
  double s[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = EMPTY;
    s[qb] = 0.0;
  }
  // tiles wholly below this bound are visible to every row and real
  const int open_end = min(k1, pr.L - a.W + 1);

  if (ntile > 0) {
#pragma unroll
    for (int i = 0; i < NS - 1; ++i)
      GG::issue_tile(ring + i * GG::TB, kbase, first + i * 16 * NW, k1, lane, lo);
    for (int it = 0; it < ntile; ++it) {
      const int t0 = first + it * 16 * NW;
      wait_loads<(NS - 2) * GG::NI>();  // tile `it` has landed
      GG::issue_tile(ring + ((it + NS - 1) % NS) * GG::TB, kbase, t0 + (NS - 1) * 16 * NW, k1,
                     lane, lo);
      u32x4_t av[GG::NJ];
      GG::read_a(av, ring + (it % NS) * GG::TB, aoff);
      // logits of q-block qb, masked (MASK) to the keys of the chunk each row
      // may see
      auto logits = [&](int qb, auto mask) __attribute__((always_inline)) {
        f32x4_t acc = GG::logits(av, q[qb]);
        if constexpr (decltype(mask)::value) {
          const int row = 16 * qb + col;
          const int lim = row < a.G * a.W ? pr.L - a.W + row % a.W : -1;  // last visible key
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + 4 * qg + r;
            if (!(key < k1 && key <= lim)) acc[r] = -INFINITY;
          }
        }
        return acc;
      };
      // the tile's terms with the current m: straight-line over the
      // q-blocks, so each block's exponentials overlap the next block's
      // MFMAs; a block whose sum passed 2^OVER is redone after the loop
      auto tile = [&](auto mask) __attribute__((always_inline)) {
        float add[NQB];
        float big = 0.f;  // the largest tile sum (terms are positive)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const f32x4_t acc = logits(qb, mask);
          add[qb] = fast_exp2(__builtin_fmaf(acc[0], sc, -m[qb]));
#pragma unroll
          for (int r = 1; r < 4; ++r) add[qb] += fast_exp2(__builtin_fmaf(acc[r], sc, -m[qb]));
          big = fmaxf(big, add[qb]);
        }
        // wave-uniform; rare once m settles (an overflowed sum is +inf)
        if (__builtin_amdgcn_ballot_w64(!(big <= OVER)) != 0) {
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const f32x4_t acc = logits(qb, mask);
            const bool up = !(add[qb] <= OVER);
            const float mn = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3])) * sc;
            const float mu = up ? mn : m[qb];
            s[qb] *= up ? static_cast<double>(fast_exp2(m[qb] - mn)) : 1.0;
            m[qb] = mu;
            float again = 0.f;
#pragma unroll
            for (int r = 0; r < 4; ++r) again += fast_exp2(__builtin_fmaf(acc[r], sc, -mu));
            add[qb] = up ? again : add[qb];
          }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) s[qb] += static_cast<double>(add[qb]);
      };
      if (t0 + 16 > open_end)  // (uniform) the ragged end or the causal window
        tile(std::true_type{});
      else
        tile(std::false_type{});
    }
    wait_loads<0>();  // no direct load may still write this wave's ring
  }
  // merge the 4 lane groups of each row, then the waves (in wave order, fp64)
  float* wm = reinterpret_cast<float*>(lds);                                 // [NW][16*NQB]
  double* wsum = reinterpret_cast<double*>(lds + NW * 16 * NQB * 4);         // [NW][16*NQB]
  __syncthreads();  // every wave is done with its ring
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    float M = fmaxf(m[qb], __shfl_xor(m[qb], 16, WAVE));
    M = fmaxf(M, __shfl_xor(M, 32, WAVE));
    double sv = s[qb] * exp2(static_cast<double>(m[qb]) - static_cast<double>(M));
    sv += __shfl_xor(sv, 16, WAVE);
    sv += __shfl_xor(sv, 32, WAVE);
    if (qg == 0) {
      wm[wave * 16 * NQB + 16 * qb + col] = M;
      wsum[wave * 16 * NQB + 16 * qb + col] = sv;
    }
  }
  __syncthreads();
  if (tid < 16 * NQB && tid < a.Rg) {
    float M = EMPTY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w * 16 * NQB + tid]);
    double S = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      S += wsum[w * 16 * NQB + tid] *
           exp2(static_cast<double>(wm[w * 16 * NQB + tid]) - static_cast<double>(M));
    const size_t idx = ((static_cast<size_t>(bi) * a.Hkv + h) * a.Rg + tid) * a.n_chunk1 + chunk;
    a.part1[2 * idx] = M == EMPTY ? -INFINITY : M;
    a.part1[2 * idx + 1] = static_cast<float>(S);
  }
}

// Pass 2.  Grid (n_chunk2, Hkv, b) over the middle keys [S, L-R).  Every
// middle key is visible to every observation row (the window lies inside the
// recent region): no causal mask.  Per tile and lane: for each of the lane's
// 4 keys, sum over the q-blocks of 2^(x - M) * w (rows past G*W have zero
// queries and w = 0: exact zeros); then over the 16 columns of the lane row
// by DPP.  The loop is pipelined over tiles: the next tile's MFMAs (slice by
// slice over all q-blocks) are issued among this tile's exponentials, so no
// exponential waits on an MFMA issued just before it (with the key loads
// switched off, 91 -> 62 us over 16 x 8 groups of 14272 middle keys; 1-3%
// with them on, where the key stream bounds the pass).  The sums of a
// wave's keys are staged in LDS and written once its loads have drained (no
// store may sit between the loads whose count the wave waits for).
template <typename T, int D, int NQB, int NW, int NS>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(NW * (NS * Geo<T, D>::TB + DIRECT_STAGE_KEYS * 4) <= 80 * 1024
                                       ? 2 : 1)))
void direct_columns_kernel(PrefillArgs a) {
  using GG = Geo<T, D>;
  constexpr int WB = NS * GG::TB + DIRECT_STAGE_KEYS * 4;
  __shared__ __attribute__((aligned(1024))) char lds[NW * WB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const Prompt pr = prompt_of(a, bi, h);
  const int mend = pr.L - a.R;
  const int k0 = a.S + chunk * a.chunk2, k1 = min(k0 + a.chunk2, mend);
  if (pr.L <= a.C || k0 >= k1) return;  // stored as is / past the middle region
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;
  char* ring = lds + wave * WB;
  float* stage = reinterpret_cast<float*>(ring + NS * GG::TB);
  const int first = k0 + 16 * wave;
  const int ntile = first < k1 ? (k1 - first + 16 * NW - 1) / (16 * NW) : 0;

  u32x4_t q[NQB][GG::NJ];
  GG::template load_q<NQB>(q, a, bi, h, col, qg);
  int aoff[GG::NJ], lo[GG::NI];
  GG::a_offsets(aoff, col, qg);
  GG::lane_offsets(lo, lane);
  const size_t gidx = static_cast<size_t>(bi) * a.Hkv + h;
  float nM[NQB], w[NQB];  // -M and the weight 1/sum of each row (0, 0 past G*W)
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int row = 16 * qb + col;
    const bool ok = row < a.G * a.W;
    nM[qb] = ok ? -a.rowstat[2 * (gidx * a.Rg + row)] : 0.f;
    w[qb] = ok ? a.rowstat[2 * (gidx * a.Rg + row) + 1] : 0.f;
  }
  const float sc = a.scale_log2;
  const bool b3 = (col & 8) != 0, b2 = (col & 4) != 0;

  if (ntile > 0) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
      GG::issue_tile(ring + i * GG::TB, kbase, first + i * 16 * NW, k1, lane, lo);
    // the logits of tile 0; every later tile's logits are computed one
    // iteration early, their MFMAs issued among the previous tile's
    // exponentials
    wait_loads<(NS - 1) * GG::NI>();
    u32x4_t av[GG::NJ];
    GG::read_a(av, ring, aoff);
    f32x4_t acc[NQB];
    GG::template logits_all<NQB>(acc, av, q);
    for (int it = 0; it < ntile; ++it) {
      const int t0 = first + it * 16 * NW;
      // slot it % NS held tile it, whose fragments are in registers (the
      // MFMAs that read them waited for the LDS reads); tile it + NS goes
      // there, then tile it + 1 must have landed (tiles past the last one
      // are clamped re-reads: their logits are unused)
      GG::issue_tile(ring + (it % NS) * GG::TB, kbase, t0 + NS * 16 * NW, k1, lane, lo);
      wait_loads<(NS - 1) * GG::NI>();
      GG::read_a(av, ring + ((it + 1) % NS) * GG::TB, aoff);
      float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cs[r] = __builtin_fmaf(fast_exp2(__builtin_fmaf(acc[qb][r], sc, nM[qb])), w[qb], cs[r]);
      }
      GG::template logits_all<NQB>(acc, av, q);
      // over the 16 columns: halves keep keys {0,1} / {2,3}, quarters one
      // key, then two quad steps; lane (col, qg) ends with key 4*qg + col/4
      const float sa = b3 ? cs[0] : cs[2], sb = b3 ? cs[1] : cs[3];
      const float ta = (b3 ? cs[2] : cs[0]) + dpp<DPP_ROW_MIRROR>(sa);
      const float tb = (b3 ? cs[3] : cs[1]) + dpp<DPP_ROW_MIRROR>(sb);
      float u = (b2 ? tb : ta) + dpp<DPP_ROW_HALF_MIRROR>(b2 ? ta : tb);
      u += dpp<DPP_XOR1>(u);
      u += dpp<DPP_XOR2>(u);
      if ((col & 3) == 0) stage[16 * it + 4 * qg + (col >> 2)] = u;
    }
    wait_loads<0>();
  }
  // this wave's sums, in its own staging area: no other wave reads them
  float* raw = a.raw + gidx * a.m - a.S;  // indexed by absolute key
  for (int i = lane; i < 16 * ntile; i += 64) {
    const int key = first + (i / 16) * 16 * NW + i % 16;
    if (key < k1) raw[key] = stage[i];
  }
}

// Ring depth: `want` tiles per wave, fewer where a workgroup's rings (and
// pass 2's staging) would not fit in LDS.
template <typename T, int D>
constexpr int ring_depth(int want, int stage_bytes) {
  const int fit = (SCORE_LDS_BUDGET / DIRECT_WAVES - stage_bytes) / Geo<T, D>::TB;
  return want < fit ? want : fit;
}

template <typename T, int D>
constexpr int ring1() { return ring_depth<T, D>(DIRECT_RING1, 0); }
template <typename T, int D>
constexpr int ring2() { return ring_depth<T, D>(DIRECT_RING2, DIRECT_STAGE_KEYS * 4); }

template <typename T, int D, int NQB>
hipError_t run_direct(const PrefillArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int NW = DIRECT_WAVES, NS1 = ring1<T, D>(), NS2 = ring2<T, D>();
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(a.b) * a.Hkv * a.Rg;
  const unsigned rgrid = static_cast<unsigned>(cdiv(static_cast<int>(rows), 256));
  if (a.lse != nullptr) {
    launch_lse_rowstat(a, rgrid, st);
  } else {
    direct_rowstat_kernel<T, D, NQB, NW, NS1><<<dim3(a.n_chunk1, a.Hkv, a.b), 64 * NW, 0, st>>>(a);
    launch_rowstat_combine(a, rgrid, st);
  }
  direct_columns_kernel<T, D, NQB, NW, NS2><<<dim3(a.n_chunk2, a.Hkv, a.b), 64 * NW, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int D, int NQB>
hipError_t slots_direct(int* slots1, int* slots2) {
  constexpr int NW = DIRECT_WAVES, NS1 = ring1<T, D>(), NS2 = ring2<T, D>();
  int dev = 0, cus = 0, b1 = 0, b2 = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b1, reinterpret_cast<const void*>(direct_rowstat_kernel<T, D, NQB, NW, NS1>), 64 * NW, 0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b2, reinterpret_cast<const void*>(direct_columns_kernel<T, D, NQB, NW, NS2>), 64 * NW, 0);
  if (e != hipSuccess) return e;
  *slots1 = cus * b1;
  *slots2 = cus * b2;
  return (*slots1 > 0 && *slots2 > 0) ? hipSuccess : hipErrorInvalidValue;
}

}  // namespace

bool direct_scores_supported(int dtype, int D, int Rg) {
  if (Rg > 128) return false;
  if (dtype == 1) return D == 64 || D == 128;
  if (dtype == 0) return D == 64 || (D == 128 && Rg <= 64);  // query registers <= 128
  return false;
}

// q-blocks for Rg padded rows: 2, 4 or 8
#define SS_BY_ROWS(FN, T, D, ...)                                     \
  (a_Rg <= 32 ? FN<T, D, 2>(__VA_ARGS__)                              \
              : a_Rg <= 64 ? FN<T, D, 4>(__VA_ARGS__) : FN<T, D, 8>(__VA_ARGS__))

hipError_t launch_direct_scores(int dtype, int D, const PrefillArgs& a, hipStream_t st,
                                hipEvent_t ev0, hipEvent_t ev1) {
  if (!direct_scores_supported(dtype, D, a.Rg)) return hipErrorInvalidValue;
  // a wave stages the sums of at most DIRECT_STAGE_KEYS keys in pass 2
  if (a.chunk2 > DIRECT_WAVES * DIRECT_STAGE_KEYS || a.chunk2 % (16 * DIRECT_WAVES) != 0 ||
      a.chunk1 % (16 * DIRECT_WAVES) != 0)
    return hipErrorInvalidValue;
  const int a_Rg = a.Rg;
  if (dtype == 1 && D == 64) return SS_BY_ROWS(run_direct, bf16_t, 64, a, st, ev0, ev1);
  if (dtype == 1 && D == 128) return SS_BY_ROWS(run_direct, bf16_t, 128, a, st, ev0, ev1);
  if (dtype == 0 && D == 64) return SS_BY_ROWS(run_direct, float, 64, a, st, ev0, ev1);
  if (dtype == 0 && D == 128) return SS_BY_ROWS(run_direct, float, 128, a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

hipError_t direct_score_slots(int dtype, int D, int Rg, int* slots1, int* slots2) {
  if (!direct_scores_supported(dtype, D, Rg)) return hipErrorInvalidValue;
  const int a_Rg = Rg;
  if (dtype == 1 && D == 64) return SS_BY_ROWS(slots_direct, bf16_t, 64, slots1, slots2);
  if (dtype == 1 && D == 128) return SS_BY_ROWS(slots_direct, bf16_t, 128, slots1, slots2);
  if (dtype == 0 && D == 64) return SS_BY_ROWS(slots_direct, float, 64, slots1, slots2);
  if (dtype == 0 && D == 128) return SS_BY_ROWS(slots_direct, float, 128, slots1, slots2);
  return hipErrorInvalidValue;
}

#undef SS_BY_ROWS

}  // namespace ss
