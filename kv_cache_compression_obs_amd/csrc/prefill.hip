// Prefill-time compression: observation-window scoring of the prompt keys
// and the gather that builds the fixed-size cache.
//
// "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators", sections
// "Two Ingredients, Fused" (SnapKV attention-based selection fused with
// StreamingLLM sinks + window) and "Fixed-Size Cache Layout" (built once at
// prefill: sinks + top-K middle + recent window).
//
// Score of middle key i = sum over the G q-heads of the kv-head and the W
// observation queries of that query's causal softmax probability of key i.
// Two passes over the keys, both a dense Q_obs . K^T contraction on MFMA:
//   pass 1 (score_rowstat): per query row and chunk of keys, a reference
//            maximum m and the sum of 2^(x - m), x = scale*log2(e) * q.k;
//            combined in fp64 across chunks (score_rowstat_combine) into
//            (M, weight w = 1/sum of 2^(x - M));
//   pass 2 (score_columns): over the middle keys only, recompute x and sum
//            2^(x - M) * w over the rows of the group, per key.
// Both passes form the exponent with one fma of the raw dot product
// (fma(q.k, scale*log2(e), -m)).  Exponentials use the hardware exp2
// (fast_exp2): results below 2^-126 flush to zero, a negligible share of a
// sum whose largest term is at least 1.
#include "common.h"
#include "launch.h"

namespace ss {

namespace {

// A ring of NBUF key tiles (KT rows each) in LDS, filled by direct
// global->LDS loads: lane l of one load writes bytes [16 l, 16 l + 16) of a
// 1 KB LDS block, so a tile takes NI such loads and no registers.
//
// Layout in 16-byte units (KCH units per key row):
//  - bf16 rows of 8 or 16 units: unit u = row * KCH + j is stored at
//    u ^ (u / 16 mod 16), a permutation inside each 256-byte group.  The 16
//    lanes that read one B fragment (16 consecutive rows, the same unit of
//    each) land on 16 different groups of 4 banks, and the fragment address
//    is a per-lane term plus a constant per 16-row block;
//  - any other row (fp32, whose fragments are single dwords, or a row size
//    that is not a power of two): rows padded to KCH + 1 units, so fragment
//    addresses stay affine (immediate offsets); the pad unit gets a copy of
//    the row's last unit.
// Loads i = w, w + NWV, ... of a tile belong to wave w, which counts them on
// its own vmcnt: after waiting for its loads of tile t and meeting the
// workgroup barrier, every wave sees the whole of tile t.
typedef const __attribute__((address_space(1))) void* global_ptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

template <typename T, int D, int KT, int NWV, int NBUF>
struct KeyRing {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int KCH = D * ES / 16;  // 16-byte units per key row
  static constexpr bool SWZ = SCORE_SWIZZLE && ES == 2 && (KCH == 8 || KCH == 16);
  // Units per row in LDS.  gfx950 serves a ds_read_b128 in groups of 32
  // lanes over 512 bytes of banks (an LDS probe of these fragment patterns:
  // the conflict counter reads 0 exactly where the 32 lanes' 16-byte units
  // differ modulo 32).  The bf16 fragment reads (lane (col, qg): unit
  // col*RU + qg, qg < 2 within a group) meet that when RU = 2 mod 4: 74 for
  // d = 576, where the odd pitch 73 spent 47% of the read time in
  // conflicts.  fp32 fragments are 4-byte reads, conflict-free at any odd
  // pitch.
  static constexpr int pitch() {
    if (SWZ) return KCH;
    if (ES != 2) return KCH + 1;
    int ru = KCH + 1;
    while (ru % 4 != 2) ++ru;
    return ru;
  }
  static constexpr int RU = pitch();
  static constexpr int NI = cdiv(KT * RU, 64);   // 1 KB loads per tile
  static constexpr int BYTES = NI * 1024;        // one ring slot
  static constexpr int LO = NI / NWV;            // loads per wave and tile (LO + 1
  static constexpr int HI_WAVES = NI % NWV;      // for the first HI_WAVES waves)
  static_assert(NBUF >= 2 && (NBUF - 2) * (LO + 1) <= 63, "vmcnt range");
  static_assert(D * ES % 16 == 0, "key rows are whole 16-byte units");

  static __device__ __forceinline__ int perm(int u) { return u ^ ((u >> 4) & 15); }
  static __device__ __forceinline__ int unit(int row, int j) {
    if constexpr (SWZ) return perm(row * KCH + j);
    else return row * RU + j;
  }

  // keys t0 .. t0+KT-1 of kbase (rows clamped to kend-1) into ring slot `slot`
  static __device__ __forceinline__ void issue(char* slot, const T* kbase, int t0, int kend,
                                               int wave, int lane) {
#pragma unroll
    for (int k = 0; k <= LO; ++k) {
      const int i = wave + k * NWV;
      if (k < LO || i < NI) {  // wave-uniform
        const int p = i * 64 + lane;
        int row, j;
        if constexpr (SWZ) {
          const int u = perm(p);
          row = u / KCH;
          j = u % KCH;
        } else {
          row = p / RU;
          j = min(p % RU, KCH - 1);
        }
        const int key = min(t0 + row, kend - 1);
        const char* src =
            reinterpret_cast<const char*>(kbase + static_cast<size_t>(key) * D) + j * 16;
        __builtin_amdgcn_global_load_lds((global_ptr)src, (lds_ptr)(slot + i * 1024), 16, 0, 0);
      }
    }
  }

  // Called once the first NBUF - 1 tiles are issued: wait for every load of
  // this wave, those tiles and the loads before them (queries, row
  // statistics).  The compiler sees this wait, so it keeps no wait for those
  // loads inside the loop (where it cannot count the tile loads in flight).
  static __device__ __forceinline__ void wait_all() {
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  }

  // Wait until this wave's loads of the oldest tile in flight have landed
  // (NBUF - 2 newer tiles may still be loading), then the workgroup barrier.
  // lgkmcnt(0): this wave's LDS reads and writes are done as well.
  static __device__ __forceinline__ void wait_barrier(int wave) {
    if (wave < HI_WAVES)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NBUF - 2) * (LO + 1)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NBUF - 2) * LO) : "memory");
    asm volatile("s_barrier" ::: "memory");
  }
  // no load may still write LDS when the workgroup ends
  static __device__ __forceinline__ void drain() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // B operand (K^T) fragment: lane (col, qg) takes key 16*kb + col, dims
  // c*KSTEP + qg*KPL ..  Its byte address in a slot is a constant per (kb, c)
  // plus a lane term that repeats every KBP blocks of 16 rows and, padded,
  // is the same for every c: NL = KBP * NCL lane terms in registers.
  static constexpr int NCB = D / Mma<T>::KSTEP;              // fragments per row
  static constexpr int KBP = SWZ ? 16 / KCH : 1;
  static constexpr int NCL = SWZ ? NCB : 1;
  static constexpr int BLOCK = KBP * 16 * RU * 16;          // bytes of KBP blocks of 16 rows
  static __device__ __forceinline__ int frag_byte(int row, int c, int qg) {
    const int byte = (c * Mma<T>::KSTEP + qg * Mma<T>::KPL) * ES;
    return unit(row, byte >> 4) * 16 + (byte & 15);
  }
  static __device__ __forceinline__ void lane_terms(int (&lt)[KBP][NCL], int col, int qg) {
#pragma unroll
    for (int p = 0; p < KBP; ++p)
#pragma unroll
      for (int c = 0; c < NCL; ++c) lt[p][c] = frag_byte(16 * p + col, c, qg);
  }
  static __device__ __forceinline__ typename Mma<T>::frag bfrag(const char* slot,
                                                                const int (&lt)[KBP][NCL], int kb,
                                                                int c) {
    const int off = SWZ ? (kb / KBP) * BLOCK + lt[kb % KBP][c]
                        : kb * BLOCK + c * Mma<T>::KSTEP * ES + lt[0][0];
    return Mma<T>::load(reinterpret_cast<const T*>(slot + off));
  }
};

// One tile's contraction as NS steps (step s: key block s / NC, k-chunk
// s % NC; one fragment read from LDS and NMF MFMAs that use it).  With
// GS > 0 the fragments are double-buffered in groups of GS steps: the reads
// of group g + 1 are issued right after the MFMAs of the first step of group
// g, an order pinned with sched_group_barrier.  The pinning matters because
// the compiler drains every outstanding LDS read (lgkmcnt(0)) before the
// first use of any fragment while direct global->LDS loads are in flight (it
// cannot tell their LDS writes from the reads); placed this way, that drain
// finds reads issued a group earlier.  GS = 0: each fragment is read where
// it is used.
#ifndef SS_SCORE_GS
#define SS_SCORE_GS 3
#endif
// steps per fragment group for the two-block (latent) shape; 0 elsewhere
template <int RB>
constexpr int contract_group() { return RB == 2 ? SS_SCORE_GS : 0; }

template <int NS, int GS, typename Frag, typename Read, typename Step>
__device__ __forceinline__ void contract_steps(Read&& read, Step&& step) {
  if constexpr (GS == 0) {
#pragma unroll
    for (int st = 0; st < NS; ++st) step(read(st), st);
  } else {
    static_assert(NS % GS == 0, "steps per group");
    constexpr int NG = NS / GS;
    Frag kb[2][GS];
#pragma unroll
    for (int c = 0; c < GS; ++c) kb[0][c] = read(c);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
      for (int c = 0; c < GS; ++c) {
        step(kb[g & 1][c], g * GS + c);
        if (c == 0 && g + 1 < NG) {
#pragma unroll
          for (int c2 = 0; c2 < GS; ++c2) kb[(g + 1) & 1][c2] = read((g + 1) * GS + c2);
        }
      }
    }
  }
}

template <int NS, int GS, int NMF>
__device__ __forceinline__ void pin_contract_order() {
  if constexpr (GS > 0) {
    constexpr int NG = NS / GS;
#pragma unroll
    for (int c = 0; c < GS; ++c) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);                     // MFMA
      if (g + 1 < NG) __builtin_amdgcn_sched_group_barrier(0x100, GS, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NMF * (GS - 1), 0);
    }
  }
}

// Q_obs rows of the group (G heads x W rows, contiguous) as A fragments.
template <typename T, int D>
__device__ __forceinline__ void load_q(typename Mma<T>::frag (&qf)[D / Mma<T>::KSTEP],
                                       const PrefillArgs& a, int bi, int h, int row, int qg) {
  const T* qbase = static_cast<const T*>(a.q_obs) +
                   (static_cast<size_t>(bi) * a.Hq + static_cast<size_t>(h) * a.G) * a.W * D;
  const bool ok = row < a.G * a.W;
#pragma unroll
  for (int c = 0; c < D / Mma<T>::KSTEP; ++c)
    qf[c] = ok ? Mma<T>::load(qbase + static_cast<size_t>(row) * D + c * Mma<T>::KSTEP +
                              qg * Mma<T>::KPL)
               : Mma<T>::zero();
}

// Pass 1.  Grid (n_chunk1, Hkv, b), NWV waves of RB row blocks.  Wave w owns
// rows 16*RB*w .. 16*RB*(w+1)-1 of the group, as RB blocks of 16 that share
// every key fragment read from LDS; in block rb the accumulator lane
// (col, qg) register r holds row 16*(RB*w + rb) + 4qg + r and key 16kb + col
// of the tile.  Each lane keeps, per row, a reference maximum m (log2 units)
// and the sum of 2^(x - m) over the keys it sees; the 16 lanes of a row are
// merged at the end.  m is raised only when a tile's maximum exceeds it by
// more than 2^LAZY, so the terms stay below 2^LAZY and the rescale (one exp2
// per row) is skipped by the whole wave on most tiles.
//
// The bf16 single-block shape is held to 80 VGPRs (6 waves per SIMD, 3
// workgroups of 8 waves per CU); it fits without spilling, and one register
// more costs a workgroup per CU (6% at 131072 keys).
template <typename T, int D, int KT, int NWV, int NBUF, int RB>
__global__ __launch_bounds__(64 * NWV)
__attribute__((amdgpu_waves_per_eu(RB == 1 && sizeof(T) == 2 ? 6 : 1)))
void score_rowstat_kernel(PrefillArgs a) {
  using MM = Mma<T>;
  using Ring = KeyRing<T, D, KT, NWV, NBUF>;
  constexpr int NC = D / MM::KSTEP;
  constexpr int NKB = KT / 16;
  constexpr int GS = contract_group<RB>();
  constexpr float LAZY = 8.f;
  constexpr float EMPTY = -0x1p126f;  // m of a row that has seen no key yet (finite: no inf - inf)
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * Ring::BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const bool active = 16 * RB * wave < a.G * a.W;  // wave-uniform
  const Prompt pr = prompt_of(a, bi, h);
  if (pr.L <= a.C || chunk * a.chunk1 >= pr.L) return;  // stored as is / past the prompt

  typename MM::frag qf[RB][NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) load_q<T, D>(qf[rb], a, bi, h, 16 * (RB * wave + rb) + col, qg);
  int lt[Ring::KBP][Ring::NCL];
  Ring::lane_terms(lt, col, qg);
  const int k0 = chunk * a.chunk1, k1 = min(k0 + a.chunk1, pr.L);
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;

  const float sc = a.scale_log2;
  const float lazy_raw = LAZY / sc;  // LAZY in raw dot-product units
  // the row sums accumulate one fp32 tile sum (NKB terms) per tile in fp64:
  // a chunk can hold thousands of keys per lane, too many for an fp32 sum to
  // stay within the 1e-6 selection band
  float m[RB][4], thr[RB][4];
  double s[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      m[rb][r] = EMPTY;
      s[rb][r] = 0.0;
      thr[rb][r] = -INFINITY;  // the first visible key raises m
    }
  // keys of a tile wholly below this bound are visible to every row and real
  const int open_end = min(k1, pr.L - a.W + 1);
  // the first NBUF - 1 tiles in flight; each step then refills the slot its
  // predecessor used (tiles past the chunk read its last key)
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    Ring::issue(lds + i * Ring::BYTES, kbase, k0 + i * KT, k1, wave, lane);
  Ring::wait_all();
  for (int base = k0; base < k1; base += NBUF * KT) {
#pragma unroll
    for (int sl = 0; sl < NBUF; ++sl) {  // tile at t0 sits in slot sl (a constant here)
      const int t0 = base + sl * KT;
      if (t0 >= k1) break;
      Ring::wait_barrier(wave);  // tile t0 in LDS; every wave is done with the previous one
      Ring::issue(lds + ((sl + NBUF - 1) % NBUF) * Ring::BYTES, kbase, t0 + (NBUF - 1) * KT, k1,
                  wave, lane);
      if (!active) continue;
      const char* cur = lds + sl * Ring::BYTES;
      f32x4_t acc[RB][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      contract_steps<NKB * NC, GS, typename MM::frag>(
          [&](int st) __attribute__((always_inline)) { return Ring::bfrag(cur, lt, st / NC, st % NC); },
          [&](typename MM::frag kf, int st) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[rb][st / NC] = MM::mma(qf[rb][st % NC], kf, acc[rb][st / NC]);
          });
      pin_contract_order<NKB * NC, GS, RB>();
      if (t0 + KT > open_end) {  // (uniform) the ragged end or the causal window
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * (RB * wave + rb) + 4 * qg + r;
            const int lim = row < a.G * a.W ? pr.L - a.W + row % a.W : -1;  // last visible key
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
              const int key = t0 + 16 * kb + col;
              if (!(key < k1 && key <= lim)) acc[rb][kb][r] = -INFINITY;
            }
          }
      }
      // raise m when the tile's largest raw dot product passes thr, the
      // raw-units image of m + LAZY
      auto tile_max = [&](int rb, int r) {
        float tm = acc[rb][0][r];
#pragma unroll
        for (int kb = 1; kb < NKB; ++kb) tm = fmaxf(tm, acc[rb][kb][r]);
        return tm;
      };
      bool raise = false;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) raise |= tile_max(rb, r) > thr[rb][r];
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform; rare once m settles
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float tm = tile_max(rb, r);
            if (tm > thr[rb][r]) {
              const float mn = tm * sc;
              s[rb][r] *= static_cast<double>(fast_exp2(m[rb][r] - mn));
              m[rb][r] = mn;
              thr[rb][r] = tm + lazy_raw;
            }
          }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float add = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            add += fast_exp2(__builtin_fmaf(acc[rb][kb][r], sc, -m[rb][r]));
          s[rb][r] += static_cast<double>(add);
        }
    }
  }
  Ring::drain();
  if (!active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float M = m[rb][r];
      M = xor_max(M, 1);
      M = xor_max(M, 2);
      M = xor_max(M, 4);
      M = xor_max(M, 8);
      double sv = s[rb][r] * static_cast<double>(fast_exp2(m[rb][r] - M));
      sv += __shfl_xor(sv, 1, WAVE);
      sv += __shfl_xor(sv, 2, WAVE);
      sv += __shfl_xor(sv, 4, WAVE);
      sv += __shfl_xor(sv, 8, WAVE);
      const int row = 16 * (RB * wave + rb) + 4 * qg + r;
      if (col == 0 && row < a.Rg) {
        const size_t idx =
            ((static_cast<size_t>(bi) * a.Hkv + h) * a.Rg + row) * a.n_chunk1 + chunk;
        a.part1[2 * idx] = M == EMPTY ? -INFINITY : M;
        a.part1[2 * idx + 1] = static_cast<float>(sv);
      }
    }
}

// Merge the per-chunk (max, sum) of every query row in fp64.
__global__ __launch_bounds__(256) void score_rowstat_combine_kernel(PrefillArgs a) {
  const size_t n = static_cast<size_t>(a.b) * a.Hkv * a.Rg;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const size_t gidx = idx / a.Rg;
  const Prompt pr = prompt_of(a, static_cast<int>(gidx / a.Hkv), static_cast<int>(gidx % a.Hkv));
  if (pr.L <= a.C) return;
  const int nc = cdiv(pr.L, a.chunk1);  // chunks pass 1 wrote for this request
  const float* p = a.part1 + 2 * idx * a.n_chunk1;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, p[2 * c]);
  double S = 0.0;
  if (M != -INFINITY)
    for (int c = 0; c < nc; ++c)
      if (p[2 * c] != -INFINITY)
        S += static_cast<double>(p[2 * c + 1]) * exp2(static_cast<double>(p[2 * c]) - M);
  a.rowstat[2 * idx] = M;
  a.rowstat[2 * idx + 1] = S > 0.0 ? static_cast<float>(1.0 / S) : 0.f;
}

// Row statistics from a given log-sum-exp instead of pass 1.  With lse in
// natural-log units, p = exp(z - lse) = 2^(x - lse*log2(e)); the row keeps
// M = fp32(lse*log2(e)) and the weight w = 2^(M - lse*log2(e)) (both from
// fp64), so p = 2^(x - M) * w carries the given lse to fp32 accuracy whatever
// its magnitude.
__global__ __launch_bounds__(256) void lse_rowstat_kernel(PrefillArgs a) {
  const size_t n = static_cast<size_t>(a.b) * a.Hkv * a.Rg;
  const size_t idx = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int row = static_cast<int>(idx % a.Rg);
  const size_t gidx = idx / a.Rg;  // (request, kv-head)
  if (row >= a.G * a.W) return;    // padding rows are never read
  const size_t bi = gidx / a.Hkv, h = gidx % a.Hkv;
  if (prompt_of(a, static_cast<int>(bi), static_cast<int>(h)).L <= a.C) return;
  // q-heads h*G .. h*G+G-1 of request bi, W rows each, contiguous: row = g*W + r
  const double l2 = static_cast<double>(a.lse[(bi * a.Hq + h * a.G) * a.W + row]) *
                    1.4426950408889634074;
  const float M = static_cast<float>(l2);
  a.rowstat[2 * idx] = M;
  a.rowstat[2 * idx + 1] = static_cast<float>(exp2(static_cast<double>(M) - l2));
}

// Pass 2.  Grid (n_chunk2, Hkv, b) over the middle keys [S, L-R).  Every
// middle key is visible to every observation row (the window lies inside the
// recent region), so no causal mask.  Rows as in pass 1 (RB blocks of 16 per
// wave).  Column sums: the RB*4 rows of a lane in registers, then the 4 lane
// groups (lane swaps across 16 and 32), then the NWV waves through LDS in
// wave order.  Rows past G*W have zero queries and weight 0, so they add
// exact zeros.
template <typename T, int D, int KT, int NWV, int NBUF, int RB>
__global__ __launch_bounds__(64 * NWV) void score_columns_kernel(PrefillArgs a) {
  using MM = Mma<T>;
  using Ring = KeyRing<T, D, KT, NWV, NBUF>;
  constexpr int NC = D / MM::KSTEP;
  constexpr int NKB = KT / 16;
  constexpr int GS = contract_group<RB>();
  // one LDS object: the ring, then the column partials red[NBUF][NWV][KT]
  // (with a second object the compiler adds a full vmcnt wait before every
  // read of the ring)
  __shared__ __attribute__((aligned(1024))) char lds[NBUF * Ring::BYTES + NBUF * NWV * KT * 4];
  float(*red)[NWV][KT] = reinterpret_cast<float(*)[NWV][KT]>(lds + NBUF * Ring::BYTES);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int nwa = cdiv(a.G * a.W, 16 * RB);  // waves holding real rows
  const bool active = wave < nwa;

  typename MM::frag qf[RB][NC];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) load_q<T, D>(qf[rb], a, bi, h, 16 * (RB * wave + rb) + col, qg);
  int lt[Ring::KBP][Ring::NCL];
  Ring::lane_terms(lt, col, qg);
  float nM[RB][4], w[RB][4];  // -M and the weight 1/sum of each row (0, 0 past G*W)
  const size_t gidx = static_cast<size_t>(bi) * a.Hkv + h;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 16 * (RB * wave + rb) + 4 * qg + r;
      const bool ok = row < a.G * a.W;
      nM[rb][r] = ok ? -a.rowstat[2 * (gidx * a.Rg + row)] : 0.f;
      w[rb][r] = ok ? a.rowstat[2 * (gidx * a.Rg + row) + 1] : 0.f;
    }
  const Prompt pr = prompt_of(a, bi, h);
  const int mend = pr.L - a.R;
  const int k0 = a.S + chunk * a.chunk2, k1 = min(k0 + a.chunk2, mend);
  if (pr.L <= a.C || k0 >= k1) return;  // stored as is / past the middle region
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;
  float* raw = a.raw + gidx * a.m - a.S;  // indexed by absolute key
  const float sc = a.scale_log2;
  // column sums of the tile at tb from partial buffer b: the waves in order
  auto columns_out = [&](int tb, int b) {
    if (tid < KT && tb + tid < k1) {
      float v = 0.f;
      for (int wv = 0; wv < nwa; ++wv) v += red[b][wv][tid];
      raw[tb + tid] = v;
    }
  };

#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    Ring::issue(lds + i * Ring::BYTES, kbase, k0 + i * KT, k1, wave, lane);
  Ring::wait_all();
  for (int base = k0; base < k1; base += NBUF * KT) {
#pragma unroll
    for (int sl = 0; sl < NBUF; ++sl) {  // tile at t0: ring slot and partial buffer sl
      const int t0 = base + sl * KT;
      if (t0 >= k1) break;
      Ring::wait_barrier(wave);  // tile t0 in LDS; the previous tile's partials in red
      Ring::issue(lds + ((sl + NBUF - 1) % NBUF) * Ring::BYTES, kbase, t0 + (NBUF - 1) * KT, k1,
                  wave, lane);
      if (t0 > k0) columns_out(t0 - KT, (sl + NBUF - 1) % NBUF);
      if (!active) continue;
      const char* cur = lds + sl * Ring::BYTES;
      f32x4_t acc[RB][NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      contract_steps<NKB * NC, GS, typename MM::frag>(
          [&](int st) __attribute__((always_inline)) { return Ring::bfrag(cur, lt, st / NC, st % NC); },
          [&](typename MM::frag kf, int st) __attribute__((always_inline)) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              acc[rb][st / NC] = MM::mma(qf[rb][st % NC], kf, acc[rb][st / NC]);
          });
      pin_contract_order<NKB * NC, GS, RB>();
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float cs = 0.f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            cs = __builtin_fmaf(fast_exp2(__builtin_fmaf(acc[rb][kb][r], sc, nM[rb][r])), w[rb][r],
                                cs);
        cs = sum_across_16(cs);
        cs = sum_across_32(cs);
        if (qg == 0) red[sl][wave][16 * kb + col] = cs;
      }
    }
  }
  Ring::drain();
  __syncthreads();
  const int last = (k1 - 1 - k0) / KT;  // the last tile, in partial buffer last % NBUF
  columns_out(k0 + last * KT, last % NBUF);
}

// Build the cache rows of one request: slots [0, S) <- tokens 0..S-1, slots
// [S, S+K) <- the selected middle tokens (ascending), ring slots <- the last R
// tokens at S+K + ((t-S-K) mod R).  Uncompressed prompts (L <= C) map token t
// to slot t.  Grid (cdiv(C, GATHER_SLOTS), Hkv, b), 256 threads.  Each
// thread issues all of its 16-byte loads (K, then V rows) before its first
// store, so a workgroup has its whole 64-slot block in flight at once; the
// prompt rows are read once, with the non-temporal hint.  A destination row
// outside [0, B_max) is skipped.
constexpr int GATHER_SLOTS = 64;

template <typename T, int D, int DV, bool ALIAS>
__global__ __launch_bounds__(256) void gather_kernel(PrefillArgs a, int compressed) {
  constexpr int SLOTS = GATHER_SLOTS;
  constexpr int KCH = D * static_cast<int>(sizeof(T)) / 16;
  constexpr int VCH = ALIAS ? 0 : DV * static_cast<int>(sizeof(T)) / 16;
  constexpr int NK = SLOTS * KCH / 256, NV = SLOTS * VCH / 256;  // units per thread
  static_assert(SLOTS * KCH % 256 == 0 && SLOTS * VCH % 256 == 0, "whole units per thread");
  __shared__ int tok[SLOTS];
  const int tid = threadIdx.x;
  const int sb = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int row = a.rows ? a.rows[bi] : bi;
  if (row < 0 || row >= a.B_max) return;  // rows outside the cache are ignored
  const size_t gsrc = static_cast<size_t>(bi) * a.Hkv + h;
  const size_t gdst = static_cast<size_t>(row) * a.Hkv + h;
  const Prompt pr = prompt_of(a, bi, h);
  const int L = pr.L;
  const bool cmp = a.cu != nullptr ? L > a.C : compressed != 0;
  if (tid < SLOTS) {
    const int s = sb * SLOTS + tid;
    int t = -1;
    if (s < a.C) {
      if (!cmp) {
        t = s < L ? s : -1;
      } else if (s < a.S) {
        t = s;
      } else if (s < a.S + a.K) {
        const int j = a.sel[gsrc * a.K + (s - a.S)];
        t = (j >= 0 && j < L - a.S - a.R) ? a.S + j : -1;
      } else {
        int r = (s - L) % a.R;
        if (r < 0) r += a.R;
        t = L - a.R + r;
      }
      a.slot_pos[gdst * a.C + s] = t;
    }
    tok[tid] = t;
  }
  if (sb == 0 && h == 0 && tid == 0) a.n_tokens[row] = L;
  __syncthreads();
  const char* ksrc = reinterpret_cast<const char*>(static_cast<const T*>(a.k) + pr.row0 * D);
  char* kdst = reinterpret_cast<char*>(static_cast<T*>(a.kc) + gdst * a.C * D);
  const char* vsrc = ALIAS ? nullptr
                           : reinterpret_cast<const char*>(static_cast<const T*>(a.v) + pr.row0 * DV);
  char* vdst = ALIAS ? nullptr : reinterpret_cast<char*>(static_cast<T*>(a.vc) + gdst * a.C * DV);
  // unit id = i * 256 + tid: slot id / KCH of the block, chunk id % KCH
  u32x4_t kv[NK], vv[NV > 0 ? NV : 1];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int id = i * 256 + tid, t = tok[id / KCH];
    if (t >= 0)
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          ksrc + static_cast<size_t>(t) * KCH * 16 + (id % KCH) * 16));
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = i * 256 + tid, t = tok[id / VCH];
    if (t >= 0)
      vv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
          vsrc + static_cast<size_t>(t) * VCH * 16 + (id % VCH) * 16));
  }
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int id = i * 256 + tid;
    if (tok[id / KCH] >= 0)
      *reinterpret_cast<u32x4_t*>(kdst + (static_cast<size_t>(sb) * SLOTS + id / KCH) * KCH * 16 +
                                  (id % KCH) * 16) = kv[i];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int id = i * 256 + tid;
    if (tok[id / VCH] >= 0)
      *reinterpret_cast<u32x4_t*>(vdst + (static_cast<size_t>(sb) * SLOTS + id / VCH) * VCH * 16 +
                                  (id % VCH) * 16) = vv[i];
  }
}

// Ring depth: SS_SCORE_NBUF slots, fewer where they would not fit in LDS.
template <typename T, int D, int KT, int NWV>
constexpr int score_nbuf() {
  constexpr int bytes = KeyRing<T, D, KT, NWV, 2>::BYTES;
  constexpr int fit = SCORE_LDS_BUDGET / (bytes + NWV * KT * 4);  // a ring slot + its partials
  return SCORE_NBUF < fit ? SCORE_NBUF : fit;
}

template <typename T, int D, int KT, int NWV, int RB>
hipError_t run_scores_w(const PrefillArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr int NB = score_nbuf<T, D, KT, NWV>();
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(a.b) * a.Hkv * a.Rg;
  const unsigned rgrid = static_cast<unsigned>(cdiv(static_cast<int>(rows), 256));
  if (a.lse != nullptr) {
    lse_rowstat_kernel<<<rgrid, 256, 0, st>>>(a);
  } else {
    score_rowstat_kernel<T, D, KT, NWV, NB, RB>
        <<<dim3(a.n_chunk1, a.Hkv, a.b), 64 * NWV, 0, st>>>(a);
    score_rowstat_combine_kernel<<<rgrid, 256, 0, st>>>(a);
  }
  score_columns_kernel<T, D, KT, NWV, NB, RB>
      <<<dim3(a.n_chunk2, a.Hkv, a.b), 64 * NWV, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

// One 16-row block per wave: 8 waves cover G*W <= 128 rows, 16 waves <= 256.
// (The latent shape uses 8 waves of two blocks each: every key fragment read
// from LDS then feeds two MFMAs, halving the LDS reads that bound it.)
template <typename T, int D, int KT>
hipError_t run_scores(const PrefillArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.Rg <= 128) return run_scores_w<T, D, KT, 8, 1>(a, st, ev0, ev1);
  if (a.Rg <= 256) return run_scores_w<T, D, KT, 16, 1>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

template <typename T, int D, int DV, bool ALIAS>
hipError_t run_gather(bool compressed, const PrefillArgs& a, hipStream_t st) {
  gather_kernel<T, D, DV, ALIAS>
      <<<dim3(cdiv(a.C, GATHER_SLOTS), a.Hkv, a.b), 256, 0, st>>>(a, compressed);
  return hipGetLastError();
}

}  // namespace

namespace {

template <typename T, int D, int KT, int NWV, int RB>
hipError_t score_slots_w(int* slots1, int* slots2) {
  constexpr int NB = score_nbuf<T, D, KT, NWV>();
  int dev = 0, cus = 0, b1 = 0, b2 = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b1, reinterpret_cast<const void*>(score_rowstat_kernel<T, D, KT, NWV, NB, RB>), 64 * NWV,
        0);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &b2, reinterpret_cast<const void*>(score_columns_kernel<T, D, KT, NWV, NB, RB>), 64 * NWV,
        0);
  if (e != hipSuccess) return e;
  *slots1 = cus * b1;
  *slots2 = cus * b2;
  return (*slots1 > 0 && *slots2 > 0) ? hipSuccess : hipErrorInvalidValue;
}

template <typename T, int D, int KT>
hipError_t score_slots(int Rg, int* slots1, int* slots2) {
  if (Rg <= 128) return score_slots_w<T, D, KT, 8, 1>(slots1, slots2);
  if (Rg <= 256) return score_slots_w<T, D, KT, 16, 1>(slots1, slots2);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t prefill_score_slots(int dtype, int D, int Rg, int* slots1, int* slots2) {
  if (direct_scores_supported(dtype, D, Rg)) return direct_score_slots(dtype, D, Rg, slots1, slots2);
  if (dtype == 0 && D == 64) return score_slots<float, 64, 64>(Rg, slots1, slots2);
  if (dtype == 0 && D == 128) return score_slots<float, 128, 64>(Rg, slots1, slots2);
  if (dtype == 1 && D == 64) return score_slots<bf16_t, 64, 64>(Rg, slots1, slots2);
  if (dtype == 1 && D == 128) return score_slots<bf16_t, 128, 64>(Rg, slots1, slots2);
  if (dtype == 1 && D == 576) return score_slots_w<bf16_t, 576, 32, 8, 2>(slots1, slots2);
  return hipErrorInvalidValue;
}

void launch_lse_rowstat(const PrefillArgs& a, unsigned grid, hipStream_t st) {
  lse_rowstat_kernel<<<grid, 256, 0, st>>>(a);
}
void launch_rowstat_combine(const PrefillArgs& a, unsigned grid, hipStream_t st) {
  score_rowstat_combine_kernel<<<grid, 256, 0, st>>>(a);
}

hipError_t launch_prefill_scores(int dtype, int D, const PrefillArgs& a, hipStream_t st,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  if (direct_scores_supported(dtype, D, a.Rg)) return launch_direct_scores(dtype, D, a, st, ev0, ev1);
  if (dtype == 0 && D == 64) return run_scores<float, 64, 64>(a, st, ev0, ev1);
  if (dtype == 0 && D == 128) return run_scores<float, 128, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 64) return run_scores<bf16_t, 64, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 128) return run_scores<bf16_t, 128, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 576) return run_scores_w<bf16_t, 576, 32, 8, 2>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_gather(int dtype, int D, int DV, int alias, bool compressed,
                                 const PrefillArgs& a, hipStream_t st) {
  if (alias) {
    if (dtype == 1 && D == 576 && DV == 512)
      return run_gather<bf16_t, 576, 512, true>(compressed, a, st);
    return hipErrorInvalidValue;
  }
  if (dtype == 0 && D == 64 && DV == 64) return run_gather<float, 64, 64, false>(compressed, a, st);
  if (dtype == 0 && D == 128 && DV == 128)
    return run_gather<float, 128, 128, false>(compressed, a, st);
  if (dtype == 1 && D == 64 && DV == 64) return run_gather<bf16_t, 64, 64, false>(compressed, a, st);
  if (dtype == 1 && D == 128 && DV == 128)
    return run_gather<bf16_t, 128, 128, false>(compressed, a, st);
  return hipErrorInvalidValue;
}

}  // namespace ss
