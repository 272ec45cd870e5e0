// Decode step over the fixed-size cache, as one kernel: rotary embedding of
// the new token, its ring-buffer scatter, split-C flash-decode attention with
// GQA head grouping on MFMA, and the merge of the split partials.  This
// register-tile kernel serves fp32 caches and rotary ranges that do not start
// and split on multiples of 8 dims; bf16 caches otherwise go through the
// direct-load ring kernel (decode_ring.hip), latent caches through
// decode_mla.hip.
//
// Follows "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators",
// sections "Ring Buffer vs. Naive Slicing" (decode rotates only the recent
// window: the new key/value is scattered into a fixed slot, nothing is
// gathered or concatenated) and "Prefill / Decode Pipeline" (decode is bound
// by the bytes of cache it reads every step).
#include <mutex>

#include "decode_common.h"

namespace ss {

namespace {

using namespace dec;

constexpr int DW = DECODE_WAVES;  // waves per decode workgroup


// One workgroup of DW waves per (split of the slots, kv-head, row).  The
// split's 32-slot tiles go to its waves round-robin (wave w: tiles w,
// w + DW, ...), so the waves of a workgroup read one compact window of K and
// of V at a time.
//
// Prologue (whole workgroup): rotate the G queries of the kv-head at pos (fp64
// angles) into LDS; the workgroup whose split holds the ring slot of pos also
// rotates k_new, writes it and v_new into that slot of the cache (evicting
// pos - L_recent), sets slot_pos, and (kv-head 0) checks and advances
// n_tokens.  The wave that meets the new row in its tiles takes it from LDS,
// so nothing reads back what this launch wrote to HBM.
//
// Main loop, per wave and 32-slot tile (the G q-heads share every K/V byte):
//   S^T[slot, head] = K[slot, :] . Q[head, :]^T     MFMA, K rows straight from HBM
//   online softmax over slots per head (log2 domain)
//   O^T[dv, head] += V^T[dv, slot] . P^T[slot, head]  MFMA, V staged in LDS
// K rows are loaded in the order slot = t0 + 16*h2 + 4*(m%4) + m/4 for A-row m,
// so accumulator register r of lane group qg holds slot t0 + 16*h2 + 4*r + qg:
// the probabilities are already in the P^T operand layout.
//
// Epilogue: the DW wave partials are merged in LDS into the workgroup's
// (max, sum, unnormalised output) partial, written through to the level
// shared by all XCDs; the last workgroup of the (row, kv-head) to take a
// ticket (device-scope counter) merges every split in split order and resets
// the counter.
template <typename T, int D, int DV>
__global__ __launch_bounds__(64 * DW) void decode_kernel(DecodeArgs a) {
  using MM = Mma<T>;
  using frag = typename MM::frag;
  constexpr int KPL = MM::KPL, KSTEP = MM::KSTEP;
  constexpr int NC = D / KSTEP;
  constexpr int NDB = DV / 16;
  constexpr int TS = DECODE_TILE;
  constexpr int VROW = DV * static_cast<int>(sizeof(T));
  constexpr int LROW = decode_vrow_stride(VROW);
  constexpr int VCH = VROW / 16;
  constexpr int VLD = TS * VCH / 64;
  constexpr int NP = Split<T>::N;
  constexpr int WBYTES = TS * LROW;  // one wave's V tile
  static_assert(D % KSTEP == 0 && DV % 64 == 0 && (TS * VCH) % 64 == 0, "tile shape");
  static_assert(DW * WBYTES >= 16 * D * 4 + 17 * D * static_cast<int>(sizeof(T)),
                "query staging must fit in the V tiles");
  static_assert(VROW <= 64 * DW * 16 && D * static_cast<int>(sizeof(T)) <= 64 * DW * 16,
                "one 16-byte load per thread covers a k / v row");
  static_assert(WBYTES >= 16 * DV * 4, "a wave's partial must fit in its V tile");
  __shared__ __attribute__((aligned(16))) char vt_all[DW * WBYTES];
  __shared__ double csn[D];
  __shared__ __attribute__((aligned(16))) T knew[D];
  __shared__ __attribute__((aligned(16))) T vnew[DV];
  __shared__ float wm[DW][16], wl[DW][16];
  __shared__ int sh_ticket;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Grid (kv-head, row, split), split slowest.  Workgroup ids fall on the
  // XCDs round-robin, so each XCD holds whole kv-heads of every row (work
  // that short rows keep spreads over all XCDs), and when the grid fills the
  // device twice over, the two workgroups that share a CU are splits of the
  // same (row, kv-head).
  const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
  const int G = a.G;
  // pos as a vector load: waiting for it does not wait for the loads after it
  const int pv = __hip_atomic_load(a.pos + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const size_t gh = static_cast<size_t>(b) * a.Hkv + h;
  const size_t head0 = static_cast<size_t>(b) * a.Hq + static_cast<size_t>(h) * G;
  const int col = lane & 15, qg = lane >> 4;
  const T* kb = static_cast<const T*>(a.kc) + gh * a.C * D;
  const T* vb = static_cast<const T*>(a.vc) + gh * a.C * DV;
  const int koff = 4 * (col & 3) + (col >> 2);
  frag kf[2][NC];
  u32x4_t vr[VLD];
  // Tile [t0, t0 + 32) into registers; rows at or past `hi` read row hi - 1.
  // V rows are whole-line loads with the streaming hint; K rows keep the
  // default policy (each K line is read in two 64-byte halves by two load
  // instructions).
  // Always inlined: the register arrays it fills must not become stack memory.
  auto load_tile = [&](int t0, int hi) __attribute__((always_inline)) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int s = min(t0 + 16 * h2 + koff, hi - 1);
      const T* kr = kb + static_cast<size_t>(s) * D + qg * KPL;
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[h2][c] = MM::load(kr + c * KSTEP);
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int id = i * 64 + lane;
      const int s = min(t0 + id / VCH, hi - 1);
      vr[i] = ld_stream(reinterpret_cast<const char*>(vb + static_cast<size_t>(s) * DV) +
                        (id % VCH) * 16);
    }
  };
  // ---------------------------------------------------------------- loads
  // In this order (vector loads complete in issue order): pos, the G queries
  // and the new token's k / v rows as 16-byte vectors, then (once pos has
  // given this wave's slots) the first tile, whose latency covers the rotary
  // work.  If the tile holds the new token's slot, the stale row it reads is
  // replaced from LDS in the main loop.
  const int half = a.rope_half;
  const bool rope = half > 0;
  const int rb = a.rope_begin;
  auto partner = [&](int d) __attribute__((always_inline)) {
    if (!rope || d < rb || d >= rb + 2 * half) return d;
    return d - rb < half ? d + half : d - half;
  };
  constexpr int NT = 64 * DW;
  constexpr int KROW = D * static_cast<int>(sizeof(T));   // bytes of one q / k row
  constexpr int QLD = cdiv(16 * KROW, NT * 16);           // 16-byte query loads per thread
  const int qbytes = G * KROW;
  const char* qsrc = reinterpret_cast<const char*>(static_cast<const T*>(a.q) + head0 * D);
  const char* ksrc = reinterpret_cast<const char*>(static_cast<const T*>(a.k_new) + gh * D);
  u32x4_t qld[QLD], kld, vld;
#pragma unroll
  for (int j = 0; j < QLD; ++j) {
    const int off = (tid + j * NT) * 16;
    if (off < qbytes) qld[j] = *reinterpret_cast<const u32x4_t*>(qsrc + off);
  }
  if (tid * 16 < KROW) kld = *reinterpret_cast<const u32x4_t*>(ksrc + tid * 16);
  if (tid * 16 < VROW)
    vld = *reinterpret_cast<const u32x4_t*>(
        reinterpret_cast<const char*>(static_cast<const T*>(a.v_new) + gh * DV) + tid * 16);
  // this thread's rotary frequency and the row's token count (for the
  // consistency check) are loaded here too: a load issued after the tile
  // could only be waited for by waiting for the whole tile
  static_assert(D / 2 <= NT, "one rotary pair per thread");
  const double fq = tid < half ? a.inv_freq[tid] : 0.0;
  const int ntok = tid == 0 && h == 0 && a.err != nullptr ? a.n_tokens[b] : 0;

  const int p = __builtin_amdgcn_readfirstlane(pv);
  if (p < 0) {  // inactive row: output 0, no state change
    if (split == 0) {
      T* o = static_cast<T*>(a.out) + head0 * DV;
      for (int i = tid; i < G * DV; i += 64 * DW) o[i] = from_f32<T>(0.f);
    }
    return;
  }
  const int n_valid = min(p + 1, a.C);
  const int ns = cdiv(n_valid, a.split);
  if (split >= ns) return;
  const int s0 = split * a.split;
  const int s1 = min(s0 + a.split, n_valid);
  const int w0 = s0 + wave * TS;  // this wave's tiles start at w0, w0 + DW*TS, ... below s1
  const int w1 = s1;              // valid slots of the split end here (rows past it clamp)
  if (w0 < w1) load_tile(w0, w1);  // the first tile, in flight during the rotary work
  const int SK = a.S + a.K;
  const int slot = p < SK ? p : SK + (p - SK) % a.R;
  const bool own = slot >= s0 && slot < s1;
  const bool wown = own && ((slot - s0) / TS) % DW == wave;
  // raw query / k_new rows into LDS behind the rotated-query area (all of it
  // is V tile space again once the main loop starts); v_new straight to vnew
  float* qs = reinterpret_cast<float*>(vt_all);                  // [G, D] rotated, fp32
  T* qraw = reinterpret_cast<T*>(vt_all + 16 * D * 4);          // [G, D] as given
  T* kraw = qraw + 16 * D;                                       // [D] as given
#pragma unroll
  for (int j = 0; j < QLD; ++j) {
    const int off = (tid + j * NT) * 16;
    if (off < qbytes) *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(qraw) + off) = qld[j];
  }
  if (tid * 16 < KROW) *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(kraw) + tid * 16) = kld;
  if (tid * 16 < VROW) *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(vnew) + tid * 16) = vld;
  if (tid < half) {
    const double ang = static_cast<double>(p) * fq;
    double sv, cv;
    sincos(ang, &sv, &cv);
    csn[tid] = cv;
    csn[half + tid] = sv;
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int d = idx % D;
    qs[idx] = rotate_pair<T, float>(qraw[idx], qraw[idx - d + partner(d)], d, rope, rb, half, csn,
                                    csn + half);
  }
  if (own) {
    T* kdst = static_cast<T*>(a.kc) + (gh * a.C + slot) * D;
    for (int d = tid; d < D; d += NT) {
      const T kv = rotate_pair<T, T>(kraw[d], kraw[partner(d)], d, rope, rb, half, csn, csn + half);
      knew[d] = kv;
      kdst[d] = kv;
    }
    if (tid * 16 < VROW)
      *reinterpret_cast<u32x4_t*>(reinterpret_cast<char*>(static_cast<T*>(a.vc) +
                                                          (gh * a.C + slot) * DV) + tid * 16) = vld;
    if (tid == 0) {
      a.slot_pos[gh * a.C + slot] = p;
      if (h == 0) {
        if (a.err != nullptr && ntok != p) atomicOr(a.err, 1);
        a.n_tokens[b] = p + 1;
      }
    }
  }
  __syncthreads();

  frag qf[NP][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float qv[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) qv[e] = col < G ? qs[col * D + c * KSTEP + qg * KPL + e] : 0.f;
    frag parts[NP];
    Split<T>::make(qv, parts);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) qf[pp][c] = parts[pp];
  }
  __syncthreads();  // queries read (their LDS is the V tiles) and vnew ready

  // ------------------------------------------------- main loop (per wave)
  char* vt = vt_all + wave * WBYTES;
  f32x4_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t0 = w0; t0 < w1; t0 += DW * TS) {
    wave_sync();  // the previous tile's LDS reads are done
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int id = i * 64 + lane;
      *reinterpret_cast<u32x4_t*>(vt + (id / VCH) * LROW + (id % VCH) * 16) = vr[i];
    }
    frag kcur[2][NC];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int c = 0; c < NC; ++c) kcur[h2][c] = kf[h2][c];
    if (wown && slot >= t0 && slot < t0 + TS) {
      // the new token: every tile row whose (clamped) slot is `slot` takes it
      // from LDS, never from the cache memory this launch just wrote
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        if (min(t0 + 16 * h2 + koff, w1 - 1) == slot)
#pragma unroll
          for (int c = 0; c < NC; ++c) kcur[h2][c] = MM::load(knew + c * KSTEP + qg * KPL);
      for (int r = 0; r < TS; ++r)
        if (min(t0 + r, w1 - 1) == slot)
          for (int i = lane; i < VROW / 4; i += 64)
            reinterpret_cast<uint32_t*>(vt + r * LROW)[i] = reinterpret_cast<const uint32_t*>(vnew)[i];
    }
    if (t0 + DW * TS < w1) load_tile(t0 + DW * TS, w1);  // next tile in flight during this one

    f32x4_t sacc[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      sacc[h2] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) sacc[h2] = MM::mma(kcur[h2][c], qf[pp][c], sacc[h2]);
    }
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int s = t0 + 4 * i + qg;  // i = 4*h2 + r  ->  slot t0 + 16*h2 + 4*r + qg
      x[i] = s < w1 ? sacc[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
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
    constexpr int PST = PvOps<T>::STEPS;
    frag pfr[PST][NP];
#pragma unroll
    for (int st = 0; st < PST; ++st) Split<T>::make(pf + st * KPL, pfr[st]);
    wave_sync();  // V tile written before the transposed reads
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] *= alpha;
#pragma unroll
      for (int st = 0; st < PST; ++st) {
        const frag vfr = PvOps<T>::vfrag(vt, LROW, db, col, qg, st);
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) oacc[db] = MM::mma(vfr, pfr[st][pp], oacc[db]);
      }
    }
  }
  l_run = xor_sum(l_run, 16);
  l_run = xor_sum(l_run, 32);

  // ------------------------------------------------------------ epilogue
  // the wave's partial into its own V tile (its loop is over), [G][DV] fp32
  wave_sync();
  float* wo = reinterpret_cast<float*>(vt);
  if (col < G) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<f32x4_t*>(wo + col * DV + 16 * db + 4 * qg) = oacc[db];
    if (qg == 0) {
      wm[wave][col] = m_run;  // -inf for a wave without slots
      wl[wave][col] = l_run;
    }
  }
  __syncthreads();
  // workgroup partial = merge of the DW wave partials; written with
  // device-scope stores (see st_dev)
  for (int idx = tid; idx < G * (DV / 4); idx += 64 * DW) {
    const int g = idx / (DV / 4), d4 = idx % (DV / 4);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DW; ++w) M = fmaxf(M, wm[w][g]);
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < DW; ++w)
      o += exp2f(wm[w][g] - M) *
           *reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(vt_all + w * WBYTES) +
                                            g * DV + 4 * d4);
    st_dev4(a.part_o + ((head0 + g) * a.n_split + split) * DV + 4 * d4, o);
  }
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
#pragma unroll
    for (int w = 0; w < DW; ++w) M = fmaxf(M, wm[w][tid]);
#pragma unroll
    for (int w = 0; w < DW; ++w) L += exp2f(wm[w][tid] - M) * wl[w][tid];
    const size_t pidx = (head0 + tid) * a.n_split + split;
    st_dev(a.part_ml + 2 * pidx, M);
    st_dev(a.part_ml + 2 * pidx + 1, L);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();                // ... and every other thread's
  if (tid == 0)
    sh_ticket = __hip_atomic_fetch_add(a.counter + gh, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (sh_ticket != ns - 1) return;
  merge_splits<T, DV>(a, head0, G, ns, tid, 64 * DW);
  if (tid == 0) a.counter[gh] = 0;  // ready for the next call
}

__global__ __launch_bounds__(256) void zero_counters_kernel(int32_t* c, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) c[i] = 0;
}

template <typename T, int D, int DV>
hipError_t run_decode(const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  decode_kernel<T, D, DV><<<dim3(a.Hkv, a.B, a.n_split), 64 * DW, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int D, int DV, int alias, const DecodeArgs& a,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (alias) return launch_decode_mla(dtype, D, DV, a, st, ev0, ev1);
  if (dtype == 0 && D == 64 && DV == 64) return run_decode<float, 64, 64>(a, st, ev0, ev1);
  if (dtype == 0 && D == 128 && DV == 128)
    return run_decode<float, 128, 128>(a, st, ev0, ev1);
#if SS_DECODE_RING
  // (its rotation takes 8 aligned dims at a time: the rotary range must start
  // and split on multiples of 8 dims)
  if (dtype == 1 && D == DV && (D == 64 || D == 128) &&
      (a.rope_half == 0 || (a.rope_begin % 8 == 0 && a.rope_half % 8 == 0)))
    return launch_decode_ring(D, a, st, ev0, ev1);
#endif
  if (dtype == 1 && D == 64 && DV == 64) return run_decode<bf16_t, 64, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 128 && DV == 128)
    return run_decode<bf16_t, 128, 128>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

hipError_t launch_zero_counters(int32_t* counters, int n, hipStream_t st) {
  zero_counters_kernel<<<cdiv(n, 256), 256, 0, st>>>(counters, n);
  return hipGetLastError();
}

// Decode scratch of ss_decode_step_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: host code only ever uses the device
// address that hipGetSymbolAddress returns for the current device (each GPU
// holds its own copy of the array).
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void** ptr, hipStream_t st) {
  constexpr int MAX_DEVICES = 64;
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    // The loader zero-fills the array; the counters are cleared once more
    // here, by a kernel on the caller's stream (also valid under capture),
    // before the first decode that uses them.  Every decode leaves them zero.
    e = launch_zero_counters(static_cast<int32_t*>(p), STATIC_SCRATCH_COUNTERS, st);
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace ss
