// Decode step over the fixed-size cache for absorbed multi-head latent
// attention (DeepSeek MLA): the G q-heads of one tensor-parallel rank share
// one cached latent row of 576 dims, whose first 512 dims are the value.
//
// "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators", sections
// "Ring Buffer vs. Naive Slicing" (scatter into a fixed slot of the recent
// window) and "16-Socket Deployment: Prefill vs. Decode Parallelism" (MLA
// changes how the compressed cache is laid out across sockets; here one
// rank's share: G heads against the rank's whole latent cache).
//
// One workgroup of 4 waves per (split of the slots, row).  Per 32-slot tile
// the latent rows are brought into LDS by direct global->LDS loads (no
// registers: the next tile streams into the other half of a two-tile ring
// while this one is used) and used twice:
//   S^T[slot, head] = Lat[slot, 0:576] . Q[head, :]^T   - the 18 d-chunks of
//       32 are spread over the 4 waves and the partial sums added through LDS
//       (every wave adds them in the same order, so all hold the same S);
//   O^T[dv, head] += Lat[slot, 0:512]^T . P^T[slot, head] - wave w produces
//       value dims [128w, 128w + 128).
// Rotary embedding at pos covers dims 512..575 (the rope range of the config);
// the rotated latent row is written into the ring slot and patched into the
// tile from registers.  Partials, ticket and merge as in decode.hip.
//
// LDS round trips set the pace of a tile, so the fragment reads go out in
// batches: all K fragments of a wave at once, the V fragments four at a time
// with the gfx950 transposing reads (two per fragment instead of eight 2-byte
// reads).  With direct loads in flight the compiler drains every vector-memory
// load before an LDS read it cannot tell apart from them, so these batches
// are asm blocks that also wait for their own reads, and the workgroup
// barriers inside a tile wait for LDS accesses only.
#include "decode_common.h"

namespace ss {

namespace {

using namespace dec;

constexpr int MW = 4;                   // waves per workgroup
constexpr int MNT = 64 * MW;            // threads per workgroup
constexpr int MD = 576, MDV = 512;      // latent dims, value dims
constexpr int MTS = DECODE_TILE;        // slots per tile
constexpr int MROW = MD * 2;            // bytes of one latent row (bf16)
constexpr int MCH = MROW / 16;          // 16-byte units per row
constexpr int MTB = MTS * MROW;         // bytes of one tile in LDS (rows not padded)
constexpr int MNL = MTB / 1024;         // 1 KB direct loads per tile
constexpr int MLW = MNL / MW;           // ... per wave
static_assert(MTB % 1024 == 0 && MNL % MW == 0, "whole direct loads per wave");
static_assert(MCH % 8 == 0, "the unit swizzle stays inside a row");
constexpr int MNC = MD / 32;            // d-chunks of the Q.K^T contraction
constexpr int MCW = cdiv(MNC, MW);      // at most this many chunks per wave
constexpr int MNDB = MDV / 16 / MW;     // 16-wide value blocks per wave
constexpr int CPOL_NT = 2;              // cache policy nt: non-temporal (each row is read once)

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Tile layout in LDS: unit u (16 bytes) of tile row r sits at unit
// r * MCH + (u ^ (r & 7)).  The rows are not padded (two tiles and the score
// exchange fill exactly half of a CU's LDS, so two workgroups share a CU);
// the XOR spreads the 16 rows that one fragment read touches over more
// banks than the plain layout does.
__device__ __forceinline__ int lat_byte(int r, int u) { return (r * MCH + (u ^ (r & 7))) * 16; }

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// V^T operands of the P.V contraction from the swizzled tile: lane
// (col, qg) of fragment db takes value dim 16 db + col of tile rows 4 i + qg,
// i < 8 (the slots the Q.K^T accumulator left in its P^T layout).  Two
// transposing LDS reads (ds_read_b64_tr_b16) build one: within each group of
// 16 lanes, lane 4a + b receives element b of the 8-byte chunks that lanes
// a + 4k (k < 4) address.  So lane (qg, a = lane % 4, k = lane / 4 % 4)
// addresses dims 16 db + 4a .. + 3 of row 4k + qg (elements i = k) and of row
// 16 + 4k + qg (i = 4 + k).  The NV fragments' reads go out in one asm
// block that ends by waiting for them: the compiler, which cannot tell these
// reads from the direct loads still writing the other half of the ring,
// would otherwise wait for every outstanding vector-memory load first.
template <int NV>
__device__ __forceinline__ void vfrags(const char* t, int db0, int lane, bf16x8_t (&out)[NV]) {
  static_assert(NV == 4, "one asm block of 8 reads");
  const int qg = lane >> 4, a = lane & 3, k = (lane >> 2) & 3;
  int ad[2 * NV];
#pragma unroll
  for (int q = 0; q < NV; ++q) {
    const int u = 2 * (db0 + q) + (a >> 1), byte = (a & 1) * 8;
    const char* p0 = t + lat_byte(4 * k + qg, u) + byte;
    const char* p1 = t + lat_byte(16 + 4 * k + qg, u) + byte;
    ad[2 * q] = static_cast<int>((uintptr_t)((const __attribute__((address_space(3))) char*)p0));
    ad[2 * q + 1] = static_cast<int>((uintptr_t)((const __attribute__((address_space(3))) char*)p1));
  }
  u32x2_t r[2 * NV];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7])
      : "memory");
#pragma unroll
  for (int q = 0; q < NV; ++q)
    out[q] = __builtin_bit_cast(bf16x8_t, u32x4_t{r[2 * q].x, r[2 * q].y, r[2 * q + 1].x,
                                                  r[2 * q + 1].y});
}

// The 2 x MCW K fragments (A operands of S^T = K . Q^T) of a wave: tile
// rows 16 h2 + koff, 16-byte unit 4 c + qg of d-chunk c = clo + j (clamped
// to the last chunk).  One asm block issues the reads and waits for them,
// for the reason given above.
__device__ __forceinline__ void kfrags(const char* t, int koff, int clo, int qg,
                                       bf16x8_t (&out)[2][MCW]) {
  static_assert(MCW == 5, "one asm block of 10 reads");
  int ad[2 * MCW];
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int j = 0; j < MCW; ++j)
      ad[h2 * MCW + j] = static_cast<int>((uintptr_t)((const __attribute__((address_space(3))) char*)(
          t + lat_byte(16 * h2 + koff, 4 * min(clo + j, MNC - 1) + qg))));
  u32x4_t r[2 * MCW];
  asm volatile(
      "ds_read_b128 %0, %10\n\t"
      "ds_read_b128 %1, %11\n\t"
      "ds_read_b128 %2, %12\n\t"
      "ds_read_b128 %3, %13\n\t"
      "ds_read_b128 %4, %14\n\t"
      "ds_read_b128 %5, %15\n\t"
      "ds_read_b128 %6, %16\n\t"
      "ds_read_b128 %7, %17\n\t"
      "ds_read_b128 %8, %18\n\t"
      "ds_read_b128 %9, %19\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9])
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
        "v"(ad[7]), "v"(ad[8]), "v"(ad[9])
      : "memory");
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int j = 0; j < MCW; ++j) out[h2][j] = __builtin_bit_cast(bf16x8_t, r[h2 * MCW + j]);
}

#ifndef SS_MLA_WAVES_PER_EU
#define SS_MLA_WAVES_PER_EU 2
#endif
__global__ __launch_bounds__(MNT) __attribute__((amdgpu_waves_per_eu(SS_MLA_WAVES_PER_EU))) void
decode_mla_kernel(DecodeArgs a) {
  using MM = Mma<bf16_t>;
  using frag = MM::frag;
  // 80 KB in all: the two-tile ring and the partial-score exchange, as one
  // LDS object (with two, the compiler waits for every direct load before
  // each read of the other object).  The prologue's rotary table (cos, sin
  // of each pair, 16 bytes) lives in the exchange area (unused until the
  // loop), the ticket in the ring (unused after it).
  constexpr int SXB = MW * 2 * 64 * 16;
  __shared__ __attribute__((aligned(1024))) char lds[2 * MTB + SXB];
  char* ring = lds;
  f32x4_t(*sx)[2][64] = reinterpret_cast<f32x4_t(*)[2][64]>(lds + 2 * MTB);
  static_assert(ROPE_MAX_PAIRS * 16 <= SXB, "prologue staging");
  const char* csn = lds + 2 * MTB;
  int* sh_ticket = reinterpret_cast<int*>(ring);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Grid (latent head, row, split), split slowest, as in decode_kernel:
  // workgroup ids fall on the XCDs round-robin, so each XCD holds whole rows
  // (work that short rows keep spreads over all XCDs)
  const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = a.G;
  // pos as a vector load: waiting for it does not wait for the loads after it
  const int pv = __hip_atomic_load(a.pos + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t gh = static_cast<size_t>(b) * a.Hkv + h;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(h) * G;
  const int col = lane & 15, qg = lane >> 4;
  const int clo = MNC * wave / MW, chi = MNC * (wave + 1) / MW;  // this wave's d-chunks
  // Split sizes: when the splits hold at least 32 tiles, the first half of
  // them (the workgroups dispatched first: each shares its CU with one of
  // the second half, and runs its loop some 2-5% faster) takes one tile
  // more and the second half one tile less.  Fixed by the split index, so
  // results stay deterministic.
  const int zh = static_cast<int>(gridDim.z) / 2;
  const int sd = (static_cast<int>(gridDim.z) % 2 == 0 && a.split >= 32 * MTS) ? MTS : 0;
  const int s0 = split < zh ? split * (a.split + sd) : zh * (a.split + sd) + (split - zh) * (a.split - sd);
  const int ssz = split < zh ? a.split + sd : a.split - sd;

  const bf16_t* lb = static_cast<const bf16_t*>(a.kc) + gh * a.C * MD;
  // tile [t0, t0 + 32) into ring half `dst` (streaming hint); rows at or past
  // `hi` read row hi - 1.  Load k of wave w covers LDS units 64 (w + MW k)
  // .. + 63 of the tile; a lane's tile row and source unit do not depend on
  // the tile, so they are computed once.
  int lrow[MLW], lsrc[MLW];
#pragma unroll
  for (int k = 0; k < MLW; ++k) {
    const int p = (wave + MW * k) * 64 + lane;
    lrow[k] = p / MCH;
    lsrc[k] = ((p % MCH) ^ (lrow[k] & 7)) * 16;
  }
  const char* lbb = reinterpret_cast<const char*>(lb);
  auto issue_tile = [&](char* dst, int t0, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < MLW; ++k) {
      const int srow = min(t0 + lrow[k], hi - 1);
      __builtin_amdgcn_global_load_lds(
          (gptr_t)(lbb + static_cast<size_t>(srow) * MROW + lsrc[k]),
          (lptr_t)(dst + (wave + MW * k) * 1024), 16, 0, CPOL_NT);
    }
  };

  // ---------------------------------------------------------------- loads
  // All unconditional (clamped indices), in this order (vector loads
  // complete in issue order): pos; each lane's 8 query dims of the Q.K^T
  // contraction (head col, dims c*32 + qg*8 .. +8 of this wave's chunks) and
  // the 8 dims they pair with under the rotation; thread tid's 16-byte unit
  // of the new latent row and its partner unit; the rotary frequency of pair
  // tid; the row's token count.  They all land before the tiles are issued:
  // the compiler cannot count direct loads together with ordinary ones, so a
  // value loaded before the tiles and used after them would wait for the
  // tiles.  The rotary range starts and splits on multiples of 8 dims
  // (checked on the host), so the 8 partners of 8 aligned dims are 8 aligned
  // consecutive dims; outside the range the partner load reads the
  // neighbouring 8 dims (d0 ^ 8, same row), unused.
  const int half = a.rope_half;
  const bool rope = half > 0;
  const int rb = a.rope_begin, re = rb + 2 * half;
  auto in_rope = [&](int d0) __attribute__((always_inline)) { return rope && d0 >= rb && d0 < re; };
  auto partner8 = [&](int d0) __attribute__((always_inline)) {
    return in_rope(d0) ? (d0 - rb < half ? d0 + half : d0 - half) : (d0 ^ 8);
  };
  const bool qlane = col < G;
  const bf16_t* qrow = static_cast<const bf16_t*>(a.q) + (head0 + (qlane ? col : 0)) * MD;
  u32x4_t qv[MCW], qpv[MCW];
#pragma unroll
  for (int j = 0; j < MCW; ++j) {
    const int d0 = min(clo + j, chi - 1) * 32 + qg * 8;
    qv[j] = *reinterpret_cast<const u32x4_t*>(qrow + d0);
    qpv[j] = *reinterpret_cast<const u32x4_t*>(qrow + partner8(d0));
  }
  const int kd0 = 8 * min(tid, MCH - 1);
  const bf16_t* krow = static_cast<const bf16_t*>(a.k_new) + gh * MD;
  const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(krow + kd0);
  const u32x4_t kpv = *reinterpret_cast<const u32x4_t*>(krow + partner8(kd0));
  const double fq = a.inv_freq[min(tid, ROPE_MAX_PAIRS - 1)];
  const int ntok = a.n_tokens[b];

  const int p = __builtin_amdgcn_readfirstlane(pv);
  if (p < 0) {  // inactive row: output 0, no state change
    if (split == 0) {
      bf16_t* o = static_cast<bf16_t*>(a.out) + head0 * MDV;
      for (int i = tid; i < G * MDV; i += MNT) o[i] = 0;
    }
    return;
  }
  const int n_valid = min(p + 1, a.C);
  const int ns = n_valid <= zh * (a.split + sd) ? cdiv(n_valid, a.split + sd)
                                                 : zh + cdiv(n_valid - zh * (a.split + sd), a.split - sd);
  if (split >= ns) return;
  const int s1 = min(s0 + ssz, n_valid);
  const double ang = static_cast<double>(p) * fq;
  asm volatile("" : : "v"(qv[0]), "v"(qv[1]), "v"(qv[2]), "v"(qv[3]), "v"(qv[4]), "v"(qpv[0]),
               "v"(qpv[1]), "v"(qpv[2]), "v"(qpv[3]), "v"(qpv[4]), "v"(kv), "v"(kpv), "v"(ang)
               : "memory");
  static_assert(MCW == 5, "the dependency list above names every query load");
  // The split's tiles go by starting at tile krot and wrapping round: the
  // splits of a row start evenly spread over their tile range instead of all
  // at its first tile (measured 1.7% faster: 194.7 against 198.1 us per
  // launch; a fixed function of the split, so results stay deterministic).
  const int ntile = cdiv(s1 - s0, MTS);
  const int krot = (split * (a.split / MTS) / static_cast<int>(gridDim.z)) % ntile;
  auto tile_at = [&](int i) __attribute__((always_inline)) {
    const int k = krot + i;
    return s0 + (k < ntile ? k : k - ntile) * MTS;
  };
  // the first tile, in flight during the rotary work
  issue_tile(ring, tile_at(0), s1);
  const int SK = a.S + a.K;
  const int slot = p < SK ? p : SK + (p - SK) % a.R;
  const bool own = slot >= s0 && slot < s1;
  // cos, sin of pair tid (fp64 angle) into the table
  static_assert(ROPE_MAX_PAIRS <= MNT, "one rotary pair per thread");
  if (tid < half) {
    double sv, cv;
    sincos(ang, &sv, &cv);
    lds_write16(lds_addr(csn + 16 * tid), __builtin_bit_cast(u32x4_t, double2{cv, sv}));
  }
  lds_barrier();
  // cos, sin of the 8 pairs of the 8 dims at d0 (pairs past the table's end
  // are clamped: they belong to dims outside the rotary range, unused)
  auto pairs8 = [&](int d0, double (&cs)[8], double (&sn)[8]) __attribute__((always_inline)) {
    const int i0 = in_rope(d0) ? (d0 - rb < half ? d0 - rb : d0 - rb - half) : 0;
    int ad[8];
    u32x4_t r[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ad[e] = lds_addr(csn + 16 * min(i0 + e, ROPE_MAX_PAIRS - 1));
    lds_read16<8>(ad, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double2 t = __builtin_bit_cast(double2, r[e]);
      cs[e] = t.x;
      sn[e] = t.y;
    }
  };
  auto elem = [](u32x4_t v, int e) __attribute__((always_inline)) {
    return static_cast<bf16_t>(v[e >> 1] >> (16 * (e & 1)));
  };
  // the rotated new latent row: thread tid < MCH keeps its 16 bytes (8 dims)
  // in registers, to patch them into the tile that holds the slot and write
  // them to the cache once the loop is done
  u32x4_t knew_v;
  {
    double cs[8], sn[8];
    pairs8(kd0, cs, sn);
    const bool kin = in_rope(kd0), kup = kin && kd0 - rb >= half;
    bf16_t e8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e8[e] = rot_dim<bf16_t>(elem(kv, e), elem(kpv, e), kin, kup, cs[e], sn[e]);
    knew_v = __builtin_bit_cast(u32x4_t, pack_bf16x8(e8));
  }
  // this wave's rotated query chunks as B operands (hi + lo parts); lanes of
  // heads >= G and chunks past the wave's range hold zeros.  A chunk that
  // lies wholly outside the rotary range (a test uniform over the wave)
  // needs no table.
  frag qf[2][MCW];
#pragma unroll
  for (int j = 0; j < MCW; ++j) {
    const int c = min(clo + j, chi - 1);
    const int d0 = c * 32 + qg * 8;
    const bool live = qlane && clo + j < chi;
    double cs[8], sn[8];
    if (rope && 32 * c + 32 > rb && 32 * c < re) {
      pairs8(d0, cs, sn);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = sn[e] = 0.0;
    }
    const bool qin = in_rope(d0), qup = qin && d0 - rb >= half;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = live ? rot_dim<float>(elem(qv[j], e), elem(qpv[j], e), qin, qup, cs[e], sn[e]) : 0.f;
    frag parts[2];
    Split<bf16_t>::make(v, parts);
    qf[0][j] = parts[0];
    qf[1][j] = parts[1];
  }

  // the second tile once the rotary work is done: issued right behind the
  // first, its loads stalled the wave until queue space freed, i.e. until
  // the first tile's data was coming back, and the rotary work waited with
  // them (193.5 against 195.3 us per launch)
  if (ntile > 1) issue_tile(ring + MTB, tile_at(1), s1);
  // ------------------------------------------------------------ main loop
  const int koff = 4 * (col & 3) + (col >> 2);
  f32x4_t oacc[MNDB];
#pragma unroll
  for (int db = 0; db < MNDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int it = 0; it < ntile; ++it) {
    const int t0 = tile_at(it);
    char* cur = ring + (it & 1) * MTB;
    // this wave's direct loads of the tile have landed; after the barrier
    // the whole tile is in LDS and every wave is done with the previous one
    // (this wave issues no vector-memory operation but the direct loads
    // between the first tile and the end of the loop, so vmcnt counts tiles:
    // in the first iteration the second tile may still be in flight)
    if (it == 0 && ntile > 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(MLW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (own && slot >= t0 && slot < t0 + MTS) {
      // (uniform) the new token: every tile row whose (clamped) slot is
      // `slot` takes it from registers, never from the cache memory this
      // launch wrote
      if (tid < MCH)
        for (int r = slot - t0; r < MTS; ++r)
          if (min(t0 + r, s1 - 1) == slot)
            lds_write16(lds_addr(cur + lat_byte(r, tid)), knew_v);
      lds_barrier();
    }

    // all of this wave's K fragments first, then the MFMAs: one LDS round
    // trip (chunks past the wave's range have zero queries and add nothing;
    // their reads stay inside the row)
    frag kfr[2][MCW];
    kfrags(cur, koff, clo, qg, kfr);
    f32x4_t sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      sacc[h2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < MCW; ++j) {
        sacc[h2] = MM::mma(kfr[h2][j], qf[0][j], sacc[h2]);
        sacc[h2] = MM::mma(kfr[h2][j], qf[1][j], sacc[h2]);
      }
      sx[wave][h2][lane] = sacc[h2];
    }
    lds_barrier();  // partial scores visible
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x4_t s = sx[0][h2][lane];
#pragma unroll
      for (int w = 1; w < MW; ++w) s += sx[w][h2][lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * h2 + r;  // slot t0 + 16*h2 + 4*r + qg = t0 + 4*i + qg
        x[i] = t0 + 4 * i + qg < s1 ? s[r] * a.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[i]);
      }
    }
    tmax = max_across_16(tmax);
    tmax = max_across_32(tmax);
    const float mnew = fmaxf(m_run, tmax);
    const float alpha = fast_exp2(m_run - mnew);
    m_run = mnew;
    float pf[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pf[i] = fast_exp2(x[i] - mnew);
      psum += pf[i];
    }
    l_run = l_run * alpha + psum;
    frag pfr[2];
    Split<bf16_t>::make(pf, pfr);
    // V fragments in batches of VB (VB reads in flight per round trip)
    constexpr int VB = 4;
    static_assert(MNDB % VB == 0, "value-block batches");
#pragma unroll
    for (int d0 = 0; d0 < MNDB; d0 += VB) {
      frag vfr[VB];
      vfrags<VB>(cur, MNDB * wave + d0, lane, vfr);
      // From the second iteration on, the next tile streams into the other
      // half from here (the first two were issued before the loop).  Where
      // in the iteration its loads go out matters: measured per launch,
      // right after the barrier 193.1 us, after the K fragment reads 191.8,
      // after the score exchange 191.1, after the softmax 190.6, here (after
      // the first value-fragment batch) 189.5, after the second 204.6, at
      // the end of the iteration 202.0.
      if (d0 == 0 && it > 0 && it + 1 < ntile)
        issue_tile(ring + ((it + 1) & 1) * MTB, tile_at(it + 1), s1);
#pragma unroll
      for (int q = 0; q < VB; ++q) {
        oacc[d0 + q] *= alpha;
        oacc[d0 + q] = MM::mma(vfr[q], pfr[0], oacc[d0 + q]);
        oacc[d0 + q] = MM::mma(vfr[q], pfr[1], oacc[d0 + q]);
      }
    }
  }
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);

  // the new latent row into its ring slot of the cache, after the loop (so
  // that vmcnt counted only tiles there), slot_pos, and (latent head 0) the
  // token-count check and advance
  if (own) {
    if (tid < MCH)
      *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(a.kc) + (gh * a.C + slot) * MD + 8 * tid) =
          knew_v;
    if (tid == 0) {
      a.slot_pos[gh * a.C + slot] = p;
      if (h == 0) {
        if (a.err != nullptr && ntok != p) atomicOr(a.err, 1);
        a.n_tokens[b] = p + 1;
      }
    }
  }

  // ------------------------------------------------------------ epilogue
  // every wave holds the same (m, l); wave w holds value dims [128w, 128w+128)
  if (col < G) {
    const size_t pidx = (head0 + col) * a.n_split + split;
    float* po = a.part_o + pidx * MDV + (MDV / MW) * wave;
#pragma unroll
    for (int db = 0; db < MNDB; ++db) st_dev4(po + 16 * db + 4 * qg, oacc[db]);
    if (wave == 0 && qg == 0) {
      st_dev(a.part_ml + 2 * pidx, m_run);
      st_dev(a.part_ml + 2 * pidx + 1, l_run);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();                // ... and every other thread's
  if (tid == 0)
    *sh_ticket = __hip_atomic_fetch_add(a.counter + gh, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*sh_ticket != ns - 1) return;
  merge_splits_wide<bf16_t, MDV, 4>(a, head0, G, ns, tid, MNT);
  if (tid == 0) a.counter[gh] = 0;  // ready for the next call
}

}  // namespace

hipError_t launch_decode_mla(int dtype, int D, int DV, const DecodeArgs& a, hipStream_t st,
                             hipEvent_t ev0, hipEvent_t ev1) {
  if (dtype != 1 || D != MD || DV != MDV) return hipErrorInvalidValue;
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  decode_mla_kernel<<<dim3(a.Hkv, a.B, a.n_split), MNT, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ss
