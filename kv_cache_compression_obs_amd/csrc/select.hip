// Max-pool of the middle-key scores and top-K selection per (request,
// kv-head): "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators",
// sections "Fixed-Size Cache Layout" (the SnapKV top-K middle segment) and
// "Infinity-Bench KV Retrieval" (pooling-based top-K selection).
//
// pooled[i] = max raw[u] over the middle region, |u - i| <= (pool-1)/2.
// The kept set is the first K of the order (pooled descending, index
// ascending), written in ascending index order.
//
// One 1024-thread workgroup per group.  Scores are non-negative floats, so
// their bit patterns order like the values (bit 31 is 0).  The raw scores are
// staged through LDS in chunks for the pooling; the pooled scores stay in LDS
// when the group has at most KEEP of them (else they are re-read from the
// pooled output).  A 3-pass radix select (bits 30..20, 19..9, 8..0, LDS
// histograms) finds the K-th largest value T and how many of the keys equal
// to T are kept (the lowest-indexed ones); an ordered compaction (ballot +
// popcount per wave, wave order across the group) then writes the kept
// indices ascending.  Integer work only after the pooling max, so the result
// is exact for the given scores.
#include "common.h"
#include "launch.h"

namespace ss {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int KEEP = 16384;  // pooled scores held in LDS
constexpr int CH = 16384;    // raw scores pooled per LDS chunk
constexpr int PMAX = 256;    // largest pooling half-width staged in LDS
constexpr int UNR = 16;      // loads in flight per thread in the global passes

// Inclusive prefix sum over the 1024 threads of the workgroup.
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t n = __shfl_up(v, off, 64);
    if (lane >= off) v += n;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < NW ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < NW; off <<= 1) {
      const uint32_t n = __shfl_up(w, off, 64);
      if (lane >= off) w += n;
    }
    if (lane < NW) wsum[lane] = w;
  }
  __syncthreads();
  if (wave > 0) v += wsum[wave - 1];
  __syncthreads();
  return v;
}

// Given a histogram of nb bins, find the bin holding the krem-th largest
// element (bins ordered by value).  Thread t owns bins nb-1-2t and nb-2-2t.
__device__ __forceinline__ void pick_bin(const uint32_t* hist, int nb, uint32_t* wsum,
                                         uint32_t* sh_digit, uint32_t* sh_krem, uint32_t krem) {
  const int t = threadIdx.x;
  const int hi = nb - 1 - 2 * t, lo = nb - 2 - 2 * t;
  const uint32_t chi = hi >= 0 ? hist[hi] : 0u;
  const uint32_t clo = lo >= 0 ? hist[lo] : 0u;
  const uint32_t incl = block_scan_incl(chi + clo, wsum);
  const uint32_t above = incl - chi - clo;
  if (hi >= 0 && above < krem && krem <= above + chi) {
    *sh_digit = static_cast<uint32_t>(hi);
    *sh_krem = krem - above;
  } else if (lo >= 0 && above + chi < krem && krem <= incl) {
    *sh_digit = static_cast<uint32_t>(lo);
    *sh_krem = krem - above - chi;
  }
  __syncthreads();
}

// f(v) for every pooled score v of the group: from LDS (kept) or from the
// pooled output, UNR loads in flight per thread.
template <typename F>
__device__ __forceinline__ void for_pooled(bool kept, const uint32_t* keep, const uint32_t* pbits,
                                           int m, F&& f) {
  if (kept) {
    for (int i = threadIdx.x; i < m; i += NT) f(keep[i]);
    return;
  }
  for (int i0 = threadIdx.x; i0 < m; i0 += UNR * NT) {
    uint32_t v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = i0 + u * NT;
      v[u] = i < m ? pbits[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (i0 + u * NT < m) f(v[u]);
  }
}

__global__ __launch_bounds__(NT) void pool_select_kernel(PrefillArgs a) {
  __shared__ uint32_t keep[KEEP];
  __shared__ float stage[CH + 2 * PMAX];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t sh_digit, sh_krem;
  __shared__ uint32_t cnt_gt[NW], cnt_eq[NW], eq_before[NW], out_before[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, bi = blockIdx.y;
  const size_t g = static_cast<size_t>(bi) * a.Hkv + h;
  const int L = prompt_of(a, bi, h).L;
  if (L <= a.C) return;  // stored as is: nothing to select
  // m: this request's middle keys; a.m: the row stride of raw / pooled / sel
  const int m = L - a.S - a.R, p = (a.pool - 1) / 2, K = a.K;
  const float* raw = a.raw + g * a.m;
  float* pooled = a.pooled + g * a.m;
  const uint32_t* pbits = reinterpret_cast<const uint32_t*>(pooled);
  const bool kept = m <= KEEP;

  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  // pooling + histogram of bits [30:20]
  auto pool_out = [&](int i, float v) {
    pooled[i] = v;
    const uint32_t b = __float_as_uint(v);
    if (kept) keep[i] = b;
    atomicAdd(&hist[b >> 20], 1u);
  };
  if (p <= PMAX) {
    // a chunk's staged scores (at most CH + 2*PMAX) arrive in one round of SL
    // loads per thread, and the next chunk's round is issued before this
    // chunk is pooled (131072-token prompts: 88 -> 78 us for this phase)
    constexpr int SL = cdiv(CH + 2 * PMAX, NT);
    float nx[SL];
    auto stage_load = [&](int c0) __attribute__((always_inline)) {
      const int s0 = max(0, c0 - p), s1 = min(m, c0 + CH + p);
#pragma unroll
      for (int u = 0; u < SL; ++u) {
        const int i = s0 + tid + u * NT;
        nx[u] = i < s1 ? raw[i] : 0.f;
      }
    };
    stage_load(0);
    for (int c0 = 0; c0 < m; c0 += CH) {
      const int s0 = max(0, c0 - p), s1 = min(m, c0 + CH + p);  // staged raw[s0, s1)
      __syncthreads();  // the previous chunk's reads of stage are done (and hist is clear)
#pragma unroll
      for (int u = 0; u < SL; ++u)
        if (s0 + tid + u * NT < s1) stage[tid + u * NT] = nx[u];
      if (c0 + CH < m) stage_load(c0 + CH);
      __syncthreads();
      for (int i = c0 + tid; i < min(m, c0 + CH); i += NT) {
        const int lo = max(0, i - p), hi = min(m - 1, i + p);
        float v = stage[lo - s0];
        for (int u = lo + 1; u <= hi; ++u) v = fmaxf(v, stage[u - s0]);
        pool_out(i, v);
      }
    }
  } else {
    __syncthreads();
    for (int i = tid; i < m; i += NT) {
      const int lo = max(0, i - p), hi = min(m - 1, i + p);
      float v = raw[lo];
      for (int u = lo + 1; u <= hi; ++u) v = fmaxf(v, raw[u]);
      pool_out(i, v);
    }
  }
  __syncthreads();
  if (K == 0) return;
  pick_bin(hist, 2048, wsum, &sh_digit, &sh_krem, static_cast<uint32_t>(K));
  uint32_t prefix = sh_digit << 20;
  uint32_t krem = sh_krem;

  // bits [19:9] among keys whose bits [30:20] match (a kept pooled score is
  // visible to every thread after the barriers in pick_bin; one re-read from
  // the pooled output needs this workgroup's own stores, which it sees)
  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
  for_pooled(kept, keep, pbits, m, [&](uint32_t v) {
    if ((v >> 20) == (prefix >> 20)) atomicAdd(&hist[(v >> 9) & 0x7ffu], 1u);
  });
  __syncthreads();
  pick_bin(hist, 2048, wsum, &sh_digit, &sh_krem, krem);
  prefix |= sh_digit << 9;
  krem = sh_krem;

  // bits [8:0] among keys whose bits [30:9] match
  for (int i = tid; i < 512; i += NT) hist[i] = 0u;
  __syncthreads();
  for_pooled(kept, keep, pbits, m, [&](uint32_t v) {
    if ((v >> 9) == (prefix >> 9)) atomicAdd(&hist[v & 0x1ffu], 1u);
  });
  __syncthreads();
  pick_bin(hist, 512, wsum, &sh_digit, &sh_krem, krem);
  const uint32_t T = prefix | sh_digit;
  const uint32_t need_eq = sh_krem;  // keys equal to T that are kept (lowest indices)

  // ordered compaction: wave w scans [w*seg, (w+1)*seg), UNR rows of 64
  // scores per batch of loads
  const int seg = cdiv(cdiv(m, NW), 64) * 64;
  const int beg = wave * seg, end = min(beg + seg, m);
  auto load_rows = [&](int base, uint32_t (&v)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + 64 * u + lane;
      v[u] = i < end ? (kept ? keep[i] : pbits[i]) : 0u;
    }
  };
  uint32_t ngt = 0, neq = 0;
  for (int base = beg; base < end; base += 64 * UNR) {
    uint32_t v[UNR];
    load_rows(base, v);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const bool in = base + 64 * u + lane < end;
      ngt += __popcll(__ballot(in && v[u] > T));
      neq += __popcll(__ballot(in && v[u] == T));
    }
  }
  if (lane == 0) {
    cnt_gt[wave] = ngt;
    cnt_eq[wave] = neq;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t e = 0, o = 0;
    for (int w = 0; w < NW; ++w) {
      eq_before[w] = e;
      out_before[w] = o;
      const uint32_t take_eq = e >= need_eq ? 0u : min(need_eq - e, cnt_eq[w]);
      o += cnt_gt[w] + take_eq;
      e += cnt_eq[w];
    }
  }
  __syncthreads();
  uint32_t eq_run = eq_before[wave], out_run = out_before[wave];
  const unsigned long long below = (1ull << lane) - 1ull;
  int32_t* sel = a.sel + g * K;
  for (int base = beg; base < end; base += 64 * UNR) {
    uint32_t v[UNR];
    load_rows(base, v);
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + 64 * u + lane;
      const bool gt = i < end && v[u] > T;
      const bool eq = i < end && v[u] == T;
      const unsigned long long eqm = __ballot(eq);
      const bool take = gt || (eq && eq_run + __popcll(eqm & below) < need_eq);
      const unsigned long long tm = __ballot(take);
      const uint32_t at = out_run + __popcll(tm & below);
      if (take && at < static_cast<uint32_t>(K)) sel[at] = i;
      eq_run += __popcll(eqm);
      out_run += __popcll(tm);
    }
  }
}

}  // namespace

hipError_t launch_prefill_select(const PrefillArgs& a, hipStream_t st) {
  pool_select_kernel<<<dim3(a.Hkv, a.b), NT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ss
