// Decode step over the fixed-size cache for bf16 K/V caches (GQA): rotary
// embedding of the new token, its ring-buffer scatter, split-C flash-decode
// attention on MFMA and the merge of the split partials, as one kernel whose
// cache tiles stream through LDS by direct global->LDS loads.
//
// "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators", sections
// "Ring Buffer vs. Naive Slicing" (the new key/value is scattered into a fixed
// slot of the recent window, nothing is gathered or concatenated) and
// "Prefill / Decode Pipeline" (decode is bound by the cache bytes it reads
// every step).
//
// One workgroup of 4 waves per (split of the slots, kv-head, row).  The split
// goes by in tiles of 64 slots: the K and V rows of a tile arrive in one half
// of a two-tile LDS ring by direct loads (1 KB per wave instruction, whole
// rows, streaming hint; no registers, no LDS write instructions) while the
// other half is in use.  Wave w takes tile rows [16w, 16w + 16):
//   S^T[slot, head] = K[slot, :] . Q[head, :]^T    v_mfma_f32_16x16x32_bf16
//   online softmax over the wave's slots per head (log2 domain)
//   O^T[dv, head] += V^T[dv, slot] . P^T[slot, head]  v_mfma_f32_16x16x16_bf16
// The Q.K^T accumulator of lane (head, g) holds slots 4g .. 4g + 3 of the
// wave's 16, which is the P^T operand layout of the 16-slot contraction, and
// the V^T operand comes from transposing LDS reads, so nothing is shuffled.
// The fp32 query and probabilities enter as bf16 hi + lo pairs (exact
// products): only the cache itself is bf16.
//
// Prologue: each thread rotates one 16-byte unit (8 dims) of the G queries
// and, below RU, of the new k row (fp64 angles; the rotary table and the
// rotated queries pass through LDS behind the ring) while the first tile
// streams in; the second is issued after that work.  The workgroup whose split holds the ring slot of pos patches the
// rotated key and the value from registers into the tile that holds the slot
// (nothing reads back what this launch writes to HBM), and once its loop is
// done writes them into that slot (evicting pos - L_recent), sets slot_pos
// and (kv-head 0) checks and advances n_tokens.  Epilogue: the 4 wave
// partials merge in LDS into the workgroup's partial, written through to the
// level shared by all XCDs; the last workgroup of the (row, kv-head) to take a
// ticket merges every split in split order (merge_splits).
//
// While direct loads are in flight the compiler would wait for all of them
// before any LDS read it cannot tell apart from them, so the fragment reads
// are asm blocks that wait for their own results, the workgroup barriers
// inside the loop wait for LDS accesses only, and all LDS data is one object.
#include "decode_common.h"

namespace ss {

namespace {

using namespace dec;

constexpr int RW = 4;          // waves per workgroup
constexpr int RNT = 64 * RW;   // threads per workgroup
constexpr int RTS = 16 * RW;   // slots per tile: 16 per wave
constexpr int CPOL_NT = 2;     // cache policy nt: each cache row is read once per step
static_assert((DECODE_WAVES * DECODE_TILE) % RTS == 0, "splits hold whole tiles");

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int D> struct Ring {
  static constexpr int RB = 2 * D;          // bytes of one K (or V) row
  static constexpr int RU = RB / 16;        // 16-byte units per row
  static constexpr int TB = RTS * RB;       // bytes of the K (or V) rows of a tile
  static constexpr int NL = 2 * TB / 1024;  // 1 KB direct loads per tile (K, then V)
  static constexpr int LW = NL / RW;        // ... per wave
  static constexpr int RPB = 512 / RB;      // rows per 512 bytes (one sweep of the banks)
  static constexpr int NC = D / 32;         // 32-dim chunks of the Q.K^T contraction
  static constexpr int NDB = D / 16;        // 16-dim value blocks
  static_assert(NL % (2 * RW) == 0 && RU % 2 == 0 && RPB >= 1, "tile shape");
  // Unit u of tile row r sits at unit r * RU + (u ^ swz(r)).  gfx950 serves
  // a 16-byte LDS read in groups of 32 lanes over 512 bytes of banks, which
  // is conflict-free when the group's units differ modulo 32: the 16 rows x 2
  // units of a K fragment read meet that, and the 16 rows x 32 bytes of a
  // transposing V read cover all 512 bytes once.  (rocprof's LDSBankConflict
  // still reads ~4.5% for the kernel.)
  static __device__ __forceinline__ int swz(int r) { return 2 * ((r / RPB) % (RU / 2)); }
  static __device__ __forceinline__ int byte(int r, int u) { return (r * RU + (u ^ swz(r))) * 16; }
};

// K fragments (A operands of S^T = K . Q^T) of a wave: lane (m, g) takes
// dims 32 c + 8 g .. + 7 of tile row `row` (= 16 w + m), c < NC.
template <int D>
__device__ __forceinline__ void kfrags(const char* kt, int row, int g, bf16x8_t (&out)[Ring<D>::NC]) {
  using RG = Ring<D>;
  int ad[RG::NC];
#pragma unroll
  for (int c = 0; c < RG::NC; ++c) ad[c] = lds_addr(kt + RG::byte(row, 4 * c + g));
  u32x4_t r[RG::NC];
  lds_read16<RG::NC>(ad, r);
#pragma unroll
  for (int c = 0; c < RG::NC; ++c) out[c] = __builtin_bit_cast(bf16x8_t, r[c]);
}

// Four V^T fragments (A operands of the 16-slot P.V contraction), value
// blocks db0 .. db0 + 3: lane (m, g) of block db takes value dim 16 db + m of
// tile rows 16 w + 4 g + j, j < 4.  ds_read_b64_tr_b16: within each group of
// 16 lanes, lane 4a + b receives element b of the 8-byte chunks that lanes
// a + 4k (k < 4) address, so lane (l = 4k + a, g) addresses dims
// 16 db + 4a .. + 3 of row 16 w + 4 g + k.
template <int D>
__device__ __forceinline__ void vfrags4(const char* vt, int wrow, int lane, int db0,
                                        s16x4_t (&out)[4]) {
  using RG = Ring<D>;
  const int g = lane >> 4, l = lane & 15, a = l & 3, k = l >> 2;
  const int row = wrow + 4 * g + k;
  int ad[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    ad[q] = lds_addr(vt + RG::byte(row, 2 * (db0 + q) + (a >> 1)) + (a & 1) * 8);
  u32x2_t r[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
      : "memory");
#pragma unroll
  for (int q = 0; q < 4; ++q) out[q] = __builtin_bit_cast(s16x4_t, r[q]);
}

__device__ __forceinline__ f32x4_t mma16(s16x4_t a, s16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 4 fp32 probabilities as bf16 hi + lo operands of the 16-slot contraction
__device__ __forceinline__ void split4(const float* v, s16x4_t& hi, s16x4_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const bf16_t h = f32_to_bf16(v[e]);
    hi[e] = static_cast<short>(h);
    lo[e] = static_cast<short>(f32_to_bf16(v[e] - bf16_to_f32(h)));
  }
}

template <int D>
__global__ __launch_bounds__(RNT) void decode_ring_kernel(DecodeArgs a) {
  using RG = Ring<D>;
  using MM = Mma<bf16_t>;
  using frag = MM::frag;
  constexpr int RB = RG::RB, RU = RG::RU, TB = RG::TB, LW = RG::LW;
  constexpr int NC = RG::NC, NDB = RG::NDB;
  // One LDS object (73 KB at 128 dims: two workgroups per CU): the two-tile
  // ring (each half: K rows, then V rows), then the prologue's rotary table
  // and rotated queries; the epilogue's wave partials reuse the ring.
  constexpr int CSN_OFF = 4 * TB;                      // [pair] (cos, sin), fp64
  constexpr int QS_OFF = CSN_OFF + ROPE_MAX_PAIRS * 16;  // [thread] 8 rotated query dims, fp32
  constexpr int LDS_BYTES = QS_OFF + RNT * 32;
  constexpr int WM_OFF = RW * 16 * D * 4;              // after the wave partials
  static_assert(WM_OFF + 2 * RW * 16 * 4 + 4 <= 4 * TB, "epilogue fits in the ring");
  static_assert(16 * RU <= RNT && D / 2 <= ROPE_MAX_PAIRS, "one query unit / rotary pair per thread");
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  float(*wm)[16] = reinterpret_cast<float(*)[16]>(lds + WM_OFF);
  float(*wl)[16] = reinterpret_cast<float(*)[16]>(lds + WM_OFF + RW * 16 * 4);
  int* sh_ticket = reinterpret_cast<int*>(lds + WM_OFF + 2 * RW * 16 * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Grid (kv-head, row, split), split slowest: workgroup ids fall on the XCDs
  // round-robin, so each XCD holds whole kv-heads of every row (work that
  // short rows keep spreads over all XCDs), and when the grid fills the device
  // twice over, the two workgroups that share a CU are splits of the same
  // (row, kv-head).
  const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = a.G;
  // pos as a vector load: waiting for it does not wait for the loads after it
  const int pv = __hip_atomic_load(a.pos + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t gh = static_cast<size_t>(b) * a.Hkv + h;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(h) * G;
  const int col = lane & 15, qg = lane >> 4;
  // Split sizes: when the splits hold at least 32 tiles, the first half of
  // them (the workgroups dispatched first: each shares its CU with one of
  // the second half, and runs its loop some 2-5% faster) takes one tile
  // more and the second half one tile less.  Fixed by the split index, so
  // results stay deterministic.
  const int zh = static_cast<int>(gridDim.z) / 2;
  const int sd = (static_cast<int>(gridDim.z) % 2 == 0 && a.split >= 32 * RTS) ? RTS : 0;
  const int s0 = split < zh ? split * (a.split + sd) : zh * (a.split + sd) + (split - zh) * (a.split - sd);
  const int ssz = split < zh ? a.split + sd : a.split - sd;

  const char* kbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.kc) + gh * a.C * D);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.vc) + gh * a.C * D);
  // Tile [t0, t0 + 64) into ring half `dst`; rows at or past `hi` read row
  // hi - 1.  Load k of wave w covers LDS units 64 (w + RW k) .. + 63 of the
  // tile's K rows, and likewise of its V rows; a lane's tile row and source
  // unit do not depend on the tile, so they are computed once.
  int lrow[LW / 2], lsrc[LW / 2];
#pragma unroll
  for (int k = 0; k < LW / 2; ++k) {
    const int p = (wave + RW * k) * 64 + lane;
    lrow[k] = p / RU;
    lsrc[k] = ((p % RU) ^ RG::swz(lrow[k])) * 16;
  }
  auto issue_tile = [&](char* dst, int t0, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < LW / 2; ++k) {
      const size_t srow = static_cast<size_t>(min(t0 + lrow[k], hi - 1));
      __builtin_amdgcn_global_load_lds((gptr_t)(kbase + srow * RB + lsrc[k]),
                                       (lptr_t)(dst + (wave + RW * k) * 1024), 16, 0, CPOL_NT);
    }
#pragma unroll
    for (int k = 0; k < LW / 2; ++k) {
      const size_t srow = static_cast<size_t>(min(t0 + lrow[k], hi - 1));
      __builtin_amdgcn_global_load_lds((gptr_t)(vbase + srow * RB + lsrc[k]),
                                       (lptr_t)(dst + TB + (wave + RW * k) * 1024), 16, 0,
                                       CPOL_NT);
    }
  };

  // ---------------------------------------------------------------- loads
  // All unconditional (clamped indices), in this order (vector loads
  // complete in issue order): pos; this thread's 16-byte unit of the G query
  // rows (8 dims) and the 8 dims it pairs with under the rotation; the same
  // for the new k row (threads < RU: unit tid) and the new v unit; the rotary
  // frequency of pair tid; the row's token count.  Then (once pos has given
  // the split's valid end) the first tile, whose latency covers the rotary
  // work.  The rotary range starts and splits
  // on multiples of 8 dims (checked on the host), so the 8 partners of 8
  // aligned dims are 8 aligned consecutive dims; outside the range the
  // partner load reads the neighbouring 8 dims of the row, unused.
  const int half = a.rope_half;
  const bool rope = half > 0;
  const int rb = a.rope_begin, re = rb + 2 * half;
  const int qu = min(tid, G * RU - 1);      // query unit: head qu / RU, dims d0 .. d0 + 7
  const int d0 = 8 * (qu % RU);
  const int ku = min(tid, RU - 1);          // k / v unit: dims 8 ku .. + 7
  const bool qin = rope && d0 >= rb && d0 < re;
  const bool qup = qin && d0 - rb >= half;
  const int qpd = qin ? (qup ? d0 - half : d0 + half) : (d0 ^ 8);
  const bool kin = rope && 8 * ku >= rb && 8 * ku < re;
  const int kpd = kin ? (8 * ku - rb >= half ? 8 * ku - half : 8 * ku + half) : ((8 * ku) ^ 8);
  const bf16_t* qrow = static_cast<const bf16_t*>(a.q) + (head0 + qu / RU) * D;
  const bf16_t* krow = static_cast<const bf16_t*>(a.k_new) + gh * D;
  const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(qrow + d0);
  const u32x4_t qpv = *reinterpret_cast<const u32x4_t*>(qrow + qpd);
  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(krow + 8 * ku);
  const u32x4_t kpv = *reinterpret_cast<const u32x4_t*>(krow + kpd);
  const u32x4_t vld =
      *reinterpret_cast<const u32x4_t*>(static_cast<const bf16_t*>(a.v_new) + gh * D + 8 * ku);
  const double fq = a.inv_freq[min(tid, ROPE_MAX_PAIRS - 1)];
  const int ntok = a.n_tokens[b];

  const int p = __builtin_amdgcn_readfirstlane(pv);
  if (p < 0) {  // inactive row: output 0, no state change
    if (split == 0) {
      bf16_t* o = static_cast<bf16_t*>(a.out) + head0 * D;
      for (int i = tid; i < G * D; i += RNT) o[i] = 0;
    }
    return;
  }
  const int n_valid = min(p + 1, a.C);
  const int ns = n_valid <= zh * (a.split + sd) ? cdiv(n_valid, a.split + sd)
                                                 : zh + cdiv(n_valid - zh * (a.split + sd), a.split - sd);
  if (split >= ns) return;
  const int s1 = min(s0 + ssz, n_valid);
  const double ang = static_cast<double>(p) * fq;
  // Every load above has landed before the first tile is issued: the
  // compiler cannot count direct loads together with ordinary ones, so a
  // value loaded before them and used after would wait for the whole tile.
  asm volatile("" : : "v"(qv), "v"(qpv), "v"(kv), "v"(kpv), "v"(vld), "v"(ang) : "memory");
  // the first tile, in flight during the rotary work
  issue_tile(lds, s0, s1);
  const int SK = a.S + a.K;
  const int slot = p < SK ? p : SK + (p - SK) % a.R;
  const bool own = slot >= s0 && slot < s1;

  // cos, sin of pair tid (fp64 angle) into LDS, 16 bytes per pair
  if (tid < half) {
    double sv, cv;
    sincos(ang, &sv, &cv);
    lds_write16(lds_addr(lds + CSN_OFF + 16 * tid),
                __builtin_bit_cast(u32x4_t, double2{cv, sv}));
  }
  lds_barrier();
  // those of the 8 pairs of this thread's query unit (for tid < RU also its
  // k unit: the same dims); a unit outside the rotary range reads pairs 0..7,
  // unused
  const int i0 = qin ? (qup ? d0 - rb - half : d0 - rb) : 0;
  double cs[8], sn[8];
  {
    int ad[8];
    u32x4_t r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ad[e] = lds_addr(lds + CSN_OFF + 16 * min(i0 + e, ROPE_MAX_PAIRS - 1));
    lds_read16<8>(ad, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double2 t = __builtin_bit_cast(double2, r[e]);
      cs[e] = t.x;
      sn[e] = t.y;
    }
  }
  // the rotated query unit (fp32) into LDS at 32 bytes per thread
  {
    float qr[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16_t x = static_cast<bf16_t>(qv[e >> 1] >> (16 * (e & 1)));
      const bf16_t xp = static_cast<bf16_t>(qpv[e >> 1] >> (16 * (e & 1)));
      qr[e] = rot_dim<float>(x, xp, qin, qup, cs[e], sn[e]);
    }
    const int ad = lds_addr(lds + QS_OFF + 32 * tid);
    lds_write16(ad, __builtin_bit_cast(u32x4_t, f32x4_t{qr[0], qr[1], qr[2], qr[3]}));
    lds_write16(ad + 16, __builtin_bit_cast(u32x4_t, f32x4_t{qr[4], qr[5], qr[6], qr[7]}));
  }
  // the rotated new k unit (threads < RU; their query unit has the same
  // dims, so cs / sn apply): kept in registers, with the v unit, to patch
  // both into the tile that holds the slot
  u32x4_t knew_v;
  {
    bf16_t e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16_t x = static_cast<bf16_t>(kv[e >> 1] >> (16 * (e & 1)));
      const bf16_t xp = static_cast<bf16_t>(kpv[e >> 1] >> (16 * (e & 1)));
      e8[e] = rot_dim<bf16_t>(x, xp, kin, kin && 8 * ku - rb >= half, cs[e], sn[e]);
    }
    knew_v = __builtin_bit_cast(u32x4_t, pack_bf16x8(e8));
  }
  lds_barrier();  // rotated queries in LDS
  // the rotated queries as B operands (hi + lo parts): lane (head col, g)
  // holds dims 32 c + 8 g .. + 7, i.e. query unit col * RU + 4 c + g;
  // heads >= G are zero
  frag qf[2][NC];
  {
    int ad[2 * NC];
    u32x4_t r[2 * NC];
    const int qh = min(col, G - 1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ad[2 * c] = lds_addr(lds + QS_OFF + 32 * (qh * RU + 4 * c + qg));
      ad[2 * c + 1] = ad[2 * c] + 16;
    }
    lds_read16<2 * NC>(ad, r);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const f32x4_t lo4 = __builtin_bit_cast(f32x4_t, r[2 * c]);
      const f32x4_t hi4 = __builtin_bit_cast(f32x4_t, r[2 * c + 1]);
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = col < G ? lo4[e] : 0.f;
        v[4 + e] = col < G ? hi4[e] : 0.f;
      }
      frag parts[2];
      Split<bf16_t>::make(v, parts);
      qf[0][c] = parts[0];
      qf[1][c] = parts[1];
    }
  }

  // the second tile once the rotary work is done (issued right behind the
  // first, its loads stalled the wave until queue space freed: 46.5 against
  // 47.2 us per launch at 16 x 8 x 4096 slots)
  if (s0 + RTS < s1) issue_tile(lds + 2 * TB, s0 + RTS, s1);
  // ------------------------------------------------------------ main loop
  const int wrow = 16 * wave;  // this wave's tile rows
  f32x4_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = s0, it = 0; t0 < s1; t0 += RTS, ++it) {
    char* cur = lds + (it & 1) * 2 * TB;
    // this wave's direct loads of the tile have landed (and its reads of the
    // previous tile, and of the staged queries, are done); after the barrier
    // the whole tile is in LDS and every wave is done with the other half
    // (this wave issues no vector-memory operation but the direct loads
    // between the first tile and the end of the loop, so vmcnt counts tiles:
    // in the first iteration the second tile may still be in flight)
    if (it == 0 && t0 + RTS < s1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(LW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // from the second iteration on, the next tile streams into the other
    // half during this one (the first two were issued before the loop)
    if (it > 0 && t0 + RTS < s1) issue_tile(lds + ((it + 1) & 1) * 2 * TB, t0 + RTS, s1);
    if (own && slot >= t0 && slot < t0 + RTS) {
      // (uniform) the new token: every tile row whose (clamped) slot is
      // `slot` takes it from registers, never from the cache memory this
      // launch wrote
      if (tid < RU)
        for (int r = slot - t0; r < RTS; ++r)
          if (min(t0 + r, s1 - 1) == slot) {
            lds_write16(lds_addr(cur + RG::byte(r, tid)), knew_v);
            lds_write16(lds_addr(cur + TB + RG::byte(r, tid)), vld);
          }
      lds_barrier();
    }
    if (t0 + wrow >= s1) continue;  // (uniform per wave) none of its rows is valid

    frag kfr[NC];
    kfrags<D>(cur, wrow + col, qg, kfr);
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sacc = MM::mma(kfr[c], qf[0][c], sacc);
      sacc = MM::mma(kfr[c], qf[1][c], sacc);
    }
    // lane (col, qg) holds slots t0 + wrow + 4 qg + r of head col
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = t0 + wrow + 4 * qg + r < s1 ? sacc[r] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[r]);
    }
    tmax = max_across_16(tmax);
    tmax = max_across_32(tmax);
    const float mnew = fmaxf(m_run, tmax);  // finite: row wrow of the tile is valid
    const float alpha = fast_exp2(m_run - mnew);
    m_run = mnew;
    float pf[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pf[r] = fast_exp2(x[r] - mnew);
      psum += pf[r];
    }
    l_run = l_run * alpha + psum;
    s16x4_t phi, plo;
    split4(pf, phi, plo);
#pragma unroll
    for (int d0 = 0; d0 < NDB; d0 += 4) {
      s16x4_t vfr[4];
      vfrags4<D>(cur + TB, wrow, lane, d0, vfr);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        oacc[d0 + q] *= alpha;
        oacc[d0 + q] = mma16(vfr[q], phi, oacc[d0 + q]);
        oacc[d0 + q] = mma16(vfr[q], plo, oacc[d0 + q]);
      }
    }
  }
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);

  // the new token into its ring slot of the cache, after the loop (so that
  // vmcnt counted only tiles there): rotated k and v, slot_pos, and (kv-head
  // 0) the token-count check and advance
  if (own) {
    if (tid < RU) {
      const size_t off = (gh * a.C + slot) * D + 8 * tid;
      *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(a.kc) + off) = knew_v;
      *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(a.vc) + off) = vld;
    }
    if (tid == 0) {
      a.slot_pos[gh * a.C + slot] = p;
      if (h == 0) {
        if (a.err != nullptr && ntok != p) atomicOr(a.err, 1);
        a.n_tokens[b] = p + 1;
      }
    }
  }
  // ------------------------------------------------------------ epilogue
  lds_barrier();  // every wave is done with the last tile
  // the wave's partial, [G][D] fp32, into the ring
  float* wo = reinterpret_cast<float*>(lds) + wave * 16 * D;
  if (col < G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4_t*>(wo + col * D + 16 * db + 4 * qg) = oacc[db];
    if (qg == 0) {
      wm[wave][col] = m_run;  // -inf for a wave without slots
      wl[wave][col] = l_run;
    }
  }
  __syncthreads();
  // workgroup partial = merge of the RW wave partials; written with
  // device-scope stores (see st_dev)
  for (int idx = tid; idx < G * (D / 4); idx += RNT) {
    const int g = idx / (D / 4), d4 = idx % (D / 4);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < RW; ++w) M = fmaxf(M, wm[w][g]);
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < RW; ++w)
      o += exp2f(wm[w][g] - M) *
           *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(lds) + w * 16 * D +
                                            g * D + 4 * d4);
    st_dev4(a.part_o + ((head0 + g) * a.n_split + split) * D + 4 * d4, o);
  }
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < RW; ++w) M = fmaxf(M, wm[w][tid]);
#pragma unroll
    for (int w = 0; w < RW; ++w) L += exp2f(wm[w][tid] - M) * wl[w][tid];
    const size_t pidx = (head0 + tid) * a.n_split + split;
    st_dev(a.part_ml + 2 * pidx, M);
    st_dev(a.part_ml + 2 * pidx + 1, L);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();                // ... and every other thread's
  if (tid == 0)
    *sh_ticket = __hip_atomic_fetch_add(a.counter + gh, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*sh_ticket != ns - 1) return;
  merge_splits<bf16_t, D>(a, head0, G, ns, tid, RNT);
  if (tid == 0) a.counter[gh] = 0;  // ready for the next call
}

template <int D>
hipError_t run(const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.split % RTS != 0) return hipErrorInvalidValue;
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  decode_ring_kernel<D><<<dim3(a.Hkv, a.B, a.n_split), RNT, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_ring(int D, const DecodeArgs& a, hipStream_t st, hipEvent_t ev0,
                              hipEvent_t ev1) {
  if (D == 64) return run<64>(a, st, ev0, ev1);
  if (D == 128) return run<128>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

}  // namespace ss
