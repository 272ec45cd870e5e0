// Max-pool of the middle-key scores and top-K selection per (request,
// kv-head): "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators",
// sections "Fixed-Size Cache Layout" (the SnapKV top-K middle segment) and
// "Infinity-Bench KV Retrieval" (pooling-based top-K selection).
//
// pooled[i] = max raw[u] over the middle region, |u - i| <= (pool-1)/2.
// The kept set is the first K of the order (pooled descending, index
// ascending), written in ascending index order.
//
// Groups of at most SEL_KEEP middle keys: one 1024-thread workgroup per
// group (pool_select_kernel).  Scores are non-negative floats, so
// their bit patterns order like the values (bit 31 is 0).  The raw scores are
// staged through LDS in chunks for the pooling; the pooled scores stay in LDS
// when the group has at most KEEP of them (else they are re-read from the
// pooled output).  A 3-pass radix select (bits 30..20, 19..9, 8..0, LDS
// histograms) finds the K-th largest value T and how many of the keys equal
// to T are kept (the lowest-indexed ones); an ordered compaction (ballot +
// popcount per wave, wave order across the group) then writes the kept
// indices ascending.  Integer work only after the pooling max, so the result
// is exact for the given scores.
//
// Longer groups are split into n_part parts of part_len keys, one workgroup
// each, and the same steps run as five launches over (part, kv-head,
// request): pool + digit-1 histogram of the part; then, per digit, every
// workgroup sums the group's part histograms of the previous digit, picks
// its bin (part 0 records the pick for the next launch) and builds its part's
// histogram of the next digit; the fourth launch counts the part's keys
// above and equal to T; the fifth gives each part its output offset (the
// counts of the parts before it) and compacts it.  Every buffer is written
// in full before it is read, so the workspace needs no clearing, and the
// result is the single-workgroup result.
#include "common.h"
#include "launch.h"

namespace ss {

namespace {

constexpr int NT = 1024;
constexpr int NW = NT / 64;
constexpr int KEEP = SEL_KEEP;  // pooled scores held in LDS
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

// out(i, pooled[i]) for i in [i0, i1) of a middle region of m raw scores
// (windows clipped to [0, m)), by the whole workgroup; stage holds
// CH + 2*PMAX floats.  Windows up to PMAX wide on each side are staged
// through LDS in CH-key chunks: each chunk arrives in one round of SL loads
// per thread, and the next chunk's round is issued before this one is
// pooled (131072-token prompts: 88 -> 78 us for this phase).  Wider windows
// read the raw scores directly.
template <typename F>
__device__ __forceinline__ void pool_range(const float* raw, int m, int p, int i0, int i1,
                                           float* stage, F&& out) {
  const int tid = threadIdx.x;
  if (p <= PMAX) {
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
    if (i0 < i1) stage_load(i0);
    for (int c0 = i0; c0 < i1; c0 += CH) {
      const int s0 = max(0, c0 - p), s1 = min(m, c0 + CH + p);  // staged raw[s0, s1)
      __syncthreads();  // the previous chunk's reads of stage are done
#pragma unroll
      for (int u = 0; u < SL; ++u)
        if (s0 + tid + u * NT < s1) stage[tid + u * NT] = nx[u];
      if (c0 + CH < i1) stage_load(c0 + CH);
      __syncthreads();
      for (int i = c0 + tid; i < min(i1, c0 + CH); i += NT) {
        const int lo = max(0, i - p), hi = min(m - 1, i + p);
        float v = stage[lo - s0];
        for (int u = lo + 1; u <= hi; ++u) v = fmaxf(v, stage[u - s0]);
        out(i, v);
      }
    }
  } else {
    for (int i = i0 + tid; i < i1; i += NT) {
      const int lo = max(0, i - p), hi = min(m - 1, i + p);
      float v = raw[lo];
      for (int u = lo + 1; u <= hi; ++u) v = fmaxf(v, raw[u]);
      out(i, v);
    }
  }
  __syncthreads();
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
  __syncthreads();
  // pooling + histogram of bits [30:20]
  pool_range(raw, m, p, 0, m, stage, [&](int i, float v) {
    pooled[i] = v;
    const uint32_t b = __float_as_uint(v);
    if (kept) keep[i] = b;
    atomicAdd(&hist[b >> 20], 1u);
  });
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

// ------------------------------------------------ groups split into parts
// One workgroup per (part j, kv-head, request); part j holds the middle keys
// [j*part_len, (j+1)*part_len) of its group, clipped to the request's m.
struct Part {
  size_t g;
  int m, i0, i1;
  bool live;  // the request is compressed
};
__device__ __forceinline__ Part part_of(const PrefillArgs& a) {
  const int j = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  Part pt;
  pt.g = static_cast<size_t>(bi) * a.Hkv + h;
  const int L = prompt_of(a, bi, h).L;
  pt.live = L > a.C;
  pt.m = pt.live ? L - a.S - a.R : 0;
  pt.i0 = min(pt.m, j * a.part_len);
  pt.i1 = min(pt.m, pt.i0 + a.part_len);
  return pt;
}

// digit d (1..3) of the radix select: bins, bit shift, offset of its
// histogram inside a part's SEL_HIST_BINS block
__host__ __device__ constexpr int digit_bins(int d) { return d == 3 ? 512 : 2048; }
__host__ __device__ constexpr int digit_shift(int d) { return d == 1 ? 20 : (d == 2 ? 9 : 0); }
__host__ __device__ constexpr int digit_off(int d) { return d == 1 ? 0 : (d == 2 ? 2048 : 4096); }
static_assert(digit_off(3) + digit_bins(3) == SEL_HIST_BINS, "histogram block");

// f(i, bits of pooled[i]) for i in [i0, i1), UNR loads in flight per thread
template <typename F>
__device__ __forceinline__ void for_range(const uint32_t* pbits, int i0, int i1, F&& f) {
  for (int b0 = i0 + static_cast<int>(threadIdx.x); b0 < i1; b0 += UNR * NT) {
    uint32_t v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = b0 + u * NT;
      v[u] = i < i1 ? pbits[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (b0 + u * NT < i1) f(b0 + u * NT, v[u]);
  }
}

// launch 1: pool the part, histogram of digit 1
__global__ __launch_bounds__(NT) void sel_part_pool_kernel(PrefillArgs a) {
  __shared__ float stage[CH + 2 * PMAX];
  __shared__ uint32_t hist[2048];
  const int tid = threadIdx.x;
  const Part pt = part_of(a);
  if (!pt.live) return;
  float* pooled = a.pooled + pt.g * a.m;
  for (int i = tid; i < 2048; i += NT) hist[i] = 0u;
  __syncthreads();
  pool_range(a.raw + pt.g * a.m, pt.m, (a.pool - 1) / 2, pt.i0, pt.i1, stage,
             [&](int i, float v) {
               pooled[i] = v;
               atomicAdd(&hist[__float_as_uint(v) >> 20], 1u);
             });
  uint32_t* out = a.sel_hist + (pt.g * a.n_part + blockIdx.x) * SEL_HIST_BINS + digit_off(1);
  for (int i = tid; i < 2048; i += NT) out[i] = hist[i];
}

// launches 2, 3 (D = digit 2, 3): pick digit D-1 from the summed part
// histograms, then this part's histogram of digit D among the keys that
// match the prefix so far.  Launch 4 (D = 4): pick digit 3 (T and how many
// keys equal to T are kept), then count this part's keys above and at T.
template <int D>
__global__ __launch_bounds__(NT) void sel_part_digit_kernel(PrefillArgs a) {
  constexpr int DP = D - 1;  // the digit picked here
  constexpr int NBP = digit_bins(DP), SHP = digit_shift(DP);
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t sh_digit, sh_krem;
  __shared__ uint32_t red[2][NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Part pt = part_of(a);
  if (!pt.live || a.K == 0) return;
  uint32_t* state = a.sel_state + pt.g * 6;
  const uint32_t* hb = a.sel_hist + pt.g * a.n_part * SEL_HIST_BINS + digit_off(DP);
  for (int i = tid; i < NBP; i += NT) {
    uint32_t sum = 0u;
    for (int q = 0; q < a.n_part; ++q) sum += hb[static_cast<size_t>(q) * SEL_HIST_BINS + i];
    hist[i] = sum;
  }
  __syncthreads();
  uint32_t prefix = DP == 1 ? 0u : state[2 * (DP - 2)];
  const uint32_t krem_in = DP == 1 ? static_cast<uint32_t>(a.K) : state[2 * (DP - 2) + 1];
  pick_bin(hist, NBP, wsum, &sh_digit, &sh_krem, krem_in);
  prefix |= sh_digit << SHP;
  const uint32_t krem = sh_krem;
  if (blockIdx.x == 0 && tid == 0) {
    state[2 * (DP - 1)] = prefix;
    state[2 * (DP - 1) + 1] = krem;
  }
  const uint32_t* pbits = reinterpret_cast<const uint32_t*>(a.pooled + pt.g * a.m);
  if constexpr (D <= 3) {
    constexpr int NB = digit_bins(D), SH = digit_shift(D);
    for (int i = tid; i < NB; i += NT) hist[i] = 0u;  // pick_bin's reads ended at its barrier
    __syncthreads();
    for_range(pbits, pt.i0, pt.i1, [&](int, uint32_t v) {
      if ((v >> SHP) == (prefix >> SHP)) atomicAdd(&hist[(v >> SH) & (NB - 1)], 1u);
    });
    __syncthreads();
    uint32_t* out = a.sel_hist + (pt.g * a.n_part + blockIdx.x) * SEL_HIST_BINS + digit_off(D);
    for (int i = tid; i < NB; i += NT) out[i] = hist[i];
  } else {
    uint32_t ngt = 0u, neq = 0u;
    for_range(pbits, pt.i0, pt.i1, [&](int, uint32_t v) {
      ngt += v > prefix;
      neq += v == prefix;
    });
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      ngt += __shfl_xor(ngt, off, 64);
      neq += __shfl_xor(neq, off, 64);
    }
    if (lane == 0) {
      red[0][wave] = ngt;
      red[1][wave] = neq;
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t tg = 0u, te = 0u;
      for (int w = 0; w < NW; ++w) {
        tg += red[0][w];
        te += red[1][w];
      }
      a.sel_cnt[(pt.g * a.n_part + blockIdx.x) * 2] = tg;
      a.sel_cnt[(pt.g * a.n_part + blockIdx.x) * 2 + 1] = te;
    }
  }
}

// launch 5: this part's kept indices, ascending, at the offset the parts
// before it fill (the ties kept are the lowest-indexed ones)
__global__ __launch_bounds__(NT) void sel_part_compact_kernel(PrefillArgs a) {
  __shared__ uint32_t cnt_gt[NW], cnt_eq[NW], eq_before[NW], out_before[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const Part pt = part_of(a);
  const int K = a.K;
  if (!pt.live || K == 0) return;
  const uint32_t* state = a.sel_state + pt.g * 6;
  const uint32_t T = state[4], need_eq = state[5];
  const uint32_t* pbits = reinterpret_cast<const uint32_t*>(a.pooled + pt.g * a.m);
  const int seg = cdiv(cdiv(pt.i1 - pt.i0, NW), 64) * 64;
  const int beg = min(pt.i1, pt.i0 + wave * seg), end = min(beg + seg, pt.i1);
  auto load_rows = [&](int base, uint32_t (&v)[UNR]) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int i = base + 64 * u + lane;
      v[u] = i < end ? pbits[i] : 0u;
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
    uint32_t e = 0, o = 0;  // the parts before this one, in part order
    const uint32_t* pc = a.sel_cnt + pt.g * a.n_part * 2;
    for (int q = 0; q < static_cast<int>(blockIdx.x); ++q) {
      const uint32_t gq = pc[2 * q], eqq = pc[2 * q + 1];
      o += gq + (e >= need_eq ? 0u : min(need_eq - e, eqq));
      e += eqq;
    }
    for (int w = 0; w < NW; ++w) {
      eq_before[w] = e;
      out_before[w] = o;
      o += cnt_gt[w] + (e >= need_eq ? 0u : min(need_eq - e, cnt_eq[w]));
      e += cnt_eq[w];
    }
  }
  __syncthreads();
  uint32_t eq_run = eq_before[wave], out_run = out_before[wave];
  const unsigned long long below = (1ull << lane) - 1ull;
  int32_t* sel = a.sel + pt.g * K;
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
  if (a.n_part <= 1) {
    pool_select_kernel<<<dim3(a.Hkv, a.b), NT, 0, st>>>(a);
    return hipGetLastError();
  }
  const dim3 grid(a.n_part, a.Hkv, a.b);
  sel_part_pool_kernel<<<grid, NT, 0, st>>>(a);
  sel_part_digit_kernel<2><<<grid, NT, 0, st>>>(a);
  sel_part_digit_kernel<3><<<grid, NT, 0, st>>>(a);
  sel_part_digit_kernel<4><<<grid, NT, 0, st>>>(a);
  sel_part_compact_kernel<<<grid, NT, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace ss
