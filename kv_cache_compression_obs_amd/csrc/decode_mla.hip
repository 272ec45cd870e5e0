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
// the latent rows are staged once in LDS and used twice:
//   S^T[slot, head] = Lat[slot, 0:576] . Q[head, :]^T   - the 18 d-chunks of
//       32 are spread over the 4 waves and the partial sums added through LDS
//       (every wave adds them in the same order, so all hold the same S);
//   O^T[dv, head] += Lat[slot, 0:512]^T . P^T[slot, head] - wave w produces
//       value dims [128w, 128w + 128).
// Rotary embedding at pos covers dims 512..575 (the rope range of the config);
// the rotated latent row is written into the ring slot and patched into the
// tile from LDS.  Partials, ticket and merge as in decode.hip.
#include "decode_common.h"

namespace ss {

namespace {

using namespace dec;

constexpr int MW = 4;                   // waves per workgroup
constexpr int MNT = 64 * MW;            // threads per workgroup
constexpr int MD = 576, MDV = 512;      // latent dims, value dims
constexpr int MTS = DECODE_TILE;        // slots per tile
constexpr int MROW = MD * 2;            // bytes of one latent row (bf16)
constexpr int MLROW = MROW + 16;        // LDS row stride
constexpr int MCH = MROW / 16;          // 16-byte chunks per row
constexpr int MLD = MTS * MCH / MNT;    // chunks per thread per tile
constexpr int MNC = MD / 32;            // d-chunks of the Q.K^T contraction
constexpr int MCW = cdiv(MNC, MW);      // at most this many chunks per wave
constexpr int MNDB = MDV / 16 / MW;     // 16-wide value blocks per wave
static_assert(MTS * MCH % MNT == 0, "tile split");

#ifndef SS_MLA_WAVES_PER_EU
#define SS_MLA_WAVES_PER_EU 2
#endif
__global__ __launch_bounds__(MNT) __attribute__((amdgpu_waves_per_eu(SS_MLA_WAVES_PER_EU))) void
decode_mla_kernel(DecodeArgs a) {
  using MM = Mma<bf16_t>;
  using frag = MM::frag;
  __shared__ __attribute__((aligned(16))) char lat[MTS * MLROW];
  __shared__ __attribute__((aligned(16))) f32x4_t sx[MW][2][64];
  __shared__ double csn[2 * ROPE_MAX_PAIRS];
  __shared__ __attribute__((aligned(16))) bf16_t knew[MD];
  __shared__ __attribute__((aligned(16))) bf16_t kraw[MD];
  __shared__ int sh_ticket;

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
  const int s0 = split * a.split;

  const bf16_t* lb = static_cast<const bf16_t*>(a.kc) + gh * a.C * MD;
  u32x4_t pre[MLD];
  // tile [t0, t0 + 32) into registers (streaming hint); rows at or past `hi`
  // read row hi - 1
  auto load_tile = [&](int t0, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MLD; ++i) {
      const int id = i * MNT + tid;
      const int s = min(t0 + id / MCH, hi - 1);
      pre[i] = ld_stream(reinterpret_cast<const char*>(lb + static_cast<size_t>(s) * MD) +
                         (id % MCH) * 16);
    }
  };

  // ---------------------------------------------------------------- loads
  // In this order (vector loads complete in issue order): pos; each lane's 8
  // query dims of the Q.K^T contraction (head col, dims c*32 + qg*8 .. +8 of
  // this wave's chunks) and, inside the rotary range, the dims they pair
  // with; the new latent row; then (once pos has given the split's valid
  // end) the first tile, whose latency covers the rotary work.
  const int half = a.rope_half;
  const bool rope = half > 0;
  const int rb = a.rope_begin, re = rb + 2 * half;
  auto partner = [&](int d) __attribute__((always_inline)) {
    if (!rope || d < rb || d >= re) return d;
    return d - rb < half ? d + half : d - half;
  };
  const bool qlane = col < G;
  const bf16_t* qrow = static_cast<const bf16_t*>(a.q) + (head0 + (qlane ? col : 0)) * MD;
  // Unconditional loads (a lane past the wave's chunks rereads its last one;
  // lanes of heads >= G read head 0): no branch, so no wait is forced here.
  // The rotary range starts and splits on multiples of 8 dims (checked on the
  // host), so the 8 partners of 8 aligned dims are 8 aligned consecutive dims.
  // Outside the range the partner value is not used; the load then reads the
  // neighbouring 8 dims (d0 ^ 8, same row), an address the compiler cannot
  // fold into the query load.
  u32x4_t qv[MCW], qpv[MCW];
#pragma unroll
  for (int j = 0; j < MCW; ++j) {
    const int d0 = min(clo + j, chi - 1) * 32 + qg * 8;
    const bool inr = rope && d0 >= rb && d0 < re;
    const int pd = inr ? (d0 - rb < half ? d0 + half : d0 - half) : (d0 ^ 8);
    qv[j] = *reinterpret_cast<const u32x4_t*>(qrow + d0);
    qpv[j] = *reinterpret_cast<const u32x4_t*>(qrow + pd);
  }
  // the new latent row as given, 16 bytes per thread (threads past the row
  // reread its last chunk)
  const u32x4_t kld = *reinterpret_cast<const u32x4_t*>(static_cast<const bf16_t*>(a.k_new) +
                                                         gh * MD + 8 * min(tid, MCH - 1));
  // this thread's first rotary frequency and the row's token count (for the
  // consistency check) are loaded here too: a load issued after the tile
  // could only be waited for by waiting for the whole tile
  const double fq = tid < half ? a.inv_freq[tid] : 0.0;
  const int ntok = tid == 0 && h == 0 && a.err != nullptr ? a.n_tokens[b] : 0;

  const int p = __builtin_amdgcn_readfirstlane(pv);
  if (p < 0) {  // inactive row: output 0, no state change
    if (split == 0) {
      bf16_t* o = static_cast<bf16_t*>(a.out) + head0 * MDV;
      for (int i = tid; i < G * MDV; i += MNT) o[i] = 0;
    }
    return;
  }
  const int n_valid = min(p + 1, a.C);
  const int ns = cdiv(n_valid, a.split);
  if (split >= ns) return;
  const int s1 = min(s0 + a.split, n_valid);
  load_tile(s0, s1);  // the first tile, in flight during the rotary work
  const int SK = a.S + a.K;
  const int slot = p < SK ? p : SK + (p - SK) % a.R;
  const bool own = slot >= s0 && slot < s1;
  if (tid < MCH) reinterpret_cast<u32x4_t*>(kraw)[tid] = kld;
  if (tid < half) {
    const double ang = static_cast<double>(p) * fq;
    double sv, cv;
    sincos(ang, &sv, &cv);
    csn[tid] = cv;
    csn[half + tid] = sv;
  }
  // rotary ranges wider than 2*MNT dims: the remaining pairs (their
  // frequencies are loaded late, so this path waits for the tile)
  for (int i = tid + MNT; i < half; i += MNT) {
    const double ang = static_cast<double>(p) * a.inv_freq[i];
    double sv, cv;
    sincos(ang, &sv, &cv);
    csn[i] = cv;
    csn[half + i] = sv;
  }
  __syncthreads();
  if (own) {
    bf16_t* kdst = static_cast<bf16_t*>(a.kc) + (gh * a.C + slot) * MD;
    for (int d = tid; d < MD; d += MNT) {
      const bf16_t kv = rotate_pair<bf16_t, bf16_t>(kraw[d], kraw[partner(d)], d, rope, rb, half,
                                                    csn, csn + half);
      knew[d] = kv;
      kdst[d] = kv;
    }
    if (tid == 0) {
      a.slot_pos[gh * a.C + slot] = p;
      if (h == 0) {
        if (a.err != nullptr && ntok != p) atomicOr(a.err, 1);
        a.n_tokens[b] = p + 1;
      }
    }
  }
  // this wave's rotated query chunks as B operands (hi + lo parts); lanes of
  // heads >= G and chunks past the wave's range hold zeros
  frag qf[2][MCW];
#pragma unroll
  for (int j = 0; j < MCW; ++j) {
    const int d0 = (clo + j) * 32 + qg * 8;
    const bool live = qlane && clo + j < chi;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bf16_t x = static_cast<bf16_t>(qv[j][e >> 1] >> (16 * (e & 1)));
      const bf16_t xp = static_cast<bf16_t>(qpv[j][e >> 1] >> (16 * (e & 1)));
      v[e] = live ? rotate_pair<bf16_t, float>(x, xp, d0 + e, rope, rb, half, csn, csn + half) : 0.f;
    }
    frag parts[2];
    Split<bf16_t>::make(v, parts);
    qf[0][j] = parts[0];
    qf[1][j] = parts[1];
  }

  // ------------------------------------------------------------ main loop
  const int koff = 4 * (col & 3) + (col >> 2);
  f32x4_t oacc[MNDB];
#pragma unroll
  for (int db = 0; db < MNDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = s0; t0 < s1; t0 += MTS) {
    __syncthreads();  // the previous tile is no longer read; knew is visible
    // the new token: a tile row whose (clamped) slot is `slot` takes it from
    // LDS, never from the cache memory this launch just wrote; the thread that
    // stores a chunk also decides its source, so no two stores race
    const bool patch = own && slot >= t0 && slot < t0 + MTS;
#pragma unroll
    for (int i = 0; i < MLD; ++i) {
      const int id = i * MNT + tid;
      const int r = id / MCH, c = id % MCH;
      u32x4_t v = pre[i];
      if (patch && min(t0 + r, s1 - 1) == slot) v = reinterpret_cast<const u32x4_t*>(knew)[c];
      *reinterpret_cast<u32x4_t*>(lat + r * MLROW + c * 16) = v;
    }
    __syncthreads();  // tile visible
    if (t0 + MTS < s1) load_tile(t0 + MTS, s1);  // next tile in flight during this one

    f32x4_t sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      sacc[h2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const char* row = lat + (16 * h2 + koff) * MLROW + qg * 16;
#pragma unroll
      for (int j = 0; j < MCW; ++j)
        if (clo + j < chi) {
          const frag kfr = MM::load(reinterpret_cast<const bf16_t*>(row + (clo + j) * 64));
          sacc[h2] = MM::mma(kfr, qf[0][j], sacc[h2]);
          sacc[h2] = MM::mma(kfr, qf[1][j], sacc[h2]);
        }
      sx[wave][h2][lane] = sacc[h2];
    }
    __syncthreads();  // partial scores visible
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
    tmax = xor_max(tmax, 16);
    tmax = xor_max(tmax, 32);
    const float mnew = fmaxf(m_run, tmax);
    const float alpha = exp2f(m_run - mnew);
    m_run = mnew;
    float pf[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pf[i] = exp2f(x[i] - mnew);
      psum += pf[i];
    }
    l_run = l_run * alpha + psum;
    frag pfr[2];
    Split<bf16_t>::make(pf, pfr);
#pragma unroll
    for (int db = 0; db < MNDB; ++db) {
      oacc[db] *= alpha;
      const frag vfr = PvOps<bf16_t>::vfrag(lat, MLROW, MNDB * wave + db, col, qg, 0);
      oacc[db] = MM::mma(vfr, pfr[0], oacc[db]);
      oacc[db] = MM::mma(vfr, pfr[1], oacc[db]);
    }
  }
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);

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
    sh_ticket = __hip_atomic_fetch_add(a.counter + gh, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sh_ticket != ns - 1) return;
  merge_splits<bf16_t, MDV, 4>(a, head0, G, ns, tid, MNT);
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
