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
//   pass 1 (score_rowstat): per query row, running max and sum of 2^x over
//            key chunks, x = scale*log2(e) * q.k; combined in fp64 across
//            chunks (score_rowstat_combine) into (max M, weight w = 1/sum);
//   pass 2 (score_columns): over the middle keys only, recompute x and sum
//            2^(x - M) * w over the rows of the group, per key.
// Both passes form x - M with the same fma (x = scale*log2(e) * q.k), so pass 2
// sees the logits pass 1 normalised.  Exponentials use the hardware exp2
// (fast_exp2): results below 2^-126 of a row's maximum flush to zero, a
// negligible share of a sum whose largest term is 1.
#include "common.h"
#include "launch.h"

namespace ss {

namespace {

// A key tile of KT rows staged in LDS by the NT threads of a score workgroup.
template <typename T, int D, int KT, int NT>
struct KeyTile {
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int KROW = D * ES;      // bytes of one key row
  static constexpr int LROW = KROW + 16;   // LDS row stride (bytes)
  static constexpr int KCH = KROW / 16;    // 16-byte chunks per row
  static constexpr int NLD = cdiv(KT * KCH, NT);
  static constexpr int BYTES = KT * LROW;

  // rows t0 .. t0+KT-1 of kbase (clamped to kend-1) into registers
  static __device__ __forceinline__ void load(u32x4_t (&r)[NLD], const T* kbase, int t0, int kend,
                                              int tid) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = i * NT + tid;
      if (id < KT * KCH) {
        const int key = min(t0 + id / KCH, kend - 1);
        r[i] = *reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const char*>(kbase + static_cast<size_t>(key) * D) + (id % KCH) * 16);
      }
    }
  }
  static __device__ __forceinline__ void store(char* buf, const u32x4_t (&r)[NLD], int tid) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int id = i * NT + tid;
      if (id < KT * KCH)
        *reinterpret_cast<u32x4_t*>(buf + (id / KCH) * LROW + (id % KCH) * 16) = r[i];
    }
  }
  // B operand (K^T) fragment: lane (col, qg) takes key 16*kb + col, dims
  // c*KSTEP + qg*KPL ..
  static __device__ __forceinline__ typename Mma<T>::frag bfrag(const char* buf, int kb, int c,
                                                                int col, int qg) {
    return Mma<T>::load(reinterpret_cast<const T*>(
        buf + (16 * kb + col) * LROW + (c * Mma<T>::KSTEP + qg * Mma<T>::KPL) * ES));
  }
};

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

// Pass 1.  Grid (n_chunk1, Hkv, b), NWV waves.  Wave w owns rows 16w .. 16w+15
// of the group; accumulator lane (col, qg) register r holds row 16w + 4qg + r
// and key 16kb + col of the tile.  Each lane keeps running (max, sum) of its
// rows over the keys it sees; the 16 lanes of a row are merged at the end.
template <typename T, int D, int KT, int NWV>
__global__ __launch_bounds__(64 * NWV) void score_rowstat_kernel(PrefillArgs a) {
  using MM = Mma<T>;
  using KTile = KeyTile<T, D, KT, 64 * NWV>;
  constexpr int NC = D / MM::KSTEP;
  constexpr int NKB = KT / 16;
  __shared__ __attribute__((aligned(16))) char lds[2 * KTile::BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const bool active = 16 * wave < a.G * a.W;  // wave-uniform
  const Prompt pr = prompt_of(a, bi, h);
  if (pr.L <= a.C || chunk * a.chunk1 >= pr.L) return;  // stored as is / past the prompt

  typename MM::frag qf[NC];
  load_q<T, D>(qf, a, bi, h, 16 * wave + col, qg);
  int lim[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * wave + 4 * qg + r;
    lim[r] = row < a.G * a.W ? pr.L - a.W + row % a.W : -1;  // last visible key
  }
  const int k0 = chunk * a.chunk1, k1 = min(k0 + a.chunk1, pr.L);
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;

  // Per lane and row: running max of the raw dot products (ma), the same in
  // log2 units (m = ma * scale_log2) and the sum of 2^(x - m).
  float ma[4], m[4], s[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    ma[r] = m[r] = -INFINITY;
    s[r] = 0.f;
  }
  const float sc = a.scale_log2;
  // keys of a tile wholly below this bound are visible to every row and real
  const int open_end = min(k1, pr.L - a.W + 1);
  u32x4_t ld[KTile::NLD];
  KTile::load(ld, kbase, k0, k1, tid);
  KTile::store(lds, ld, tid);
  __syncthreads();
  int t = 0;
  for (int t0 = k0; t0 < k1; t0 += KT, ++t) {
    const char* cur = lds + (t & 1) * KTile::BYTES;
    const bool more = t0 + KT < k1;
    if (more) KTile::load(ld, kbase, t0 + KT, k1, tid);
    if (active) {
      f32x4_t acc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        acc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[kb] = MM::mma(qf[c], KTile::bfrag(cur, kb, c, col, qg), acc[kb]);
      }
      if (t0 + KT > open_end) {  // (uniform) the ragged end or the causal window
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const int key = t0 + 16 * kb + col;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (!(key < k1 && key <= lim[r])) acc[kb][r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float tm = acc[0][r];
#pragma unroll
        for (int kb = 1; kb < NKB; ++kb) tm = fmaxf(tm, acc[kb][r]);
        const float mn = fmaxf(ma[r], tm);
        // x - m = fma(acc, sc, -m); a row with no visible key yet keeps
        // (m, s) = (-inf, 0): its exponents are -inf (with m taken as 0)
        const float mx = mn == -INFINITY ? 0.f : mn * sc;
        float add = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) add += fast_exp2(__builtin_fmaf(acc[kb][r], sc, -mx));
        s[r] = s[r] * fast_exp2(m[r] - mx) + add;
        ma[r] = mn;
        m[r] = mn == -INFINITY ? -INFINITY : mx;
      }
    }
    if (more) KTile::store(lds + ((t + 1) & 1) * KTile::BYTES, ld, tid);
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float M = m[r];
    M = xor_max(M, 1);
    M = xor_max(M, 2);
    M = xor_max(M, 4);
    M = xor_max(M, 8);
    float sv = m[r] == -INFINITY ? 0.f : s[r] * fast_exp2(m[r] - M);
    sv = xor_sum(sv, 1);
    sv = xor_sum(sv, 2);
    sv = xor_sum(sv, 4);
    sv = xor_sum(sv, 8);
    const int row = 16 * wave + 4 * qg + r;
    if (col == 0 && row < a.Rg) {
      const size_t idx = ((static_cast<size_t>(bi) * a.Hkv + h) * a.Rg + row) * a.n_chunk1 + chunk;
      a.part1[2 * idx] = M;
      a.part1[2 * idx + 1] = sv;
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
// recent region), so no causal mask.  Column sums: 4 rows in registers, then
// the 4 lane groups (xor 16, 32), then the NWV waves through LDS in wave order.
template <typename T, int D, int KT, int NWV>
__global__ __launch_bounds__(64 * NWV) void score_columns_kernel(PrefillArgs a) {
  using MM = Mma<T>;
  using KTile = KeyTile<T, D, KT, 64 * NWV>;
  constexpr int NC = D / MM::KSTEP;
  constexpr int NKB = KT / 16;
  __shared__ __attribute__((aligned(16))) char lds[2 * KTile::BYTES];
  __shared__ float red[2][NWV][KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, qg = lane >> 4;
  const int chunk = blockIdx.x, h = blockIdx.y, bi = blockIdx.z;
  const int nrb = cdiv(a.G * a.W, 16);
  const bool active = wave < nrb;

  typename MM::frag qf[NC];
  load_q<T, D>(qf, a, bi, h, 16 * wave + col, qg);
  float M[4], w[4];
  bool ok[4];
  const size_t gidx = static_cast<size_t>(bi) * a.Hkv + h;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 16 * wave + 4 * qg + r;
    ok[r] = row < a.G * a.W;
    M[r] = ok[r] ? a.rowstat[2 * (gidx * a.Rg + row)] : 0.f;
    w[r] = ok[r] ? a.rowstat[2 * (gidx * a.Rg + row) + 1] : 0.f;
  }
  const Prompt pr = prompt_of(a, bi, h);
  const int mend = pr.L - a.R;
  const int k0 = a.S + chunk * a.chunk2, k1 = min(k0 + a.chunk2, mend);
  if (pr.L <= a.C || k0 >= k1) return;  // stored as is / past the middle region
  const T* kbase = static_cast<const T*>(a.k) + pr.row0 * D;
  float* raw = a.raw + gidx * a.m - a.S;  // indexed by absolute key

  u32x4_t ld[KTile::NLD];
  KTile::load(ld, kbase, k0, k1, tid);
  KTile::store(lds, ld, tid);
  __syncthreads();
  int t = 0;
  for (int t0 = k0; t0 < k1; t0 += KT, ++t) {
    const char* cur = lds + (t & 1) * KTile::BYTES;
    const bool more = t0 + KT < k1;
    if (more) KTile::load(ld, kbase, t0 + KT, k1, tid);
    if (active) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) acc = MM::mma(qf[c], KTile::bfrag(cur, kb, c, col, qg), acc);
        float cs = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          cs += ok[r] ? fast_exp2(__builtin_fmaf(acc[r], a.scale_log2, -M[r])) * w[r] : 0.f;
        cs = xor_sum(cs, 16);
        cs = xor_sum(cs, 32);
        if (qg == 0) red[t & 1][wave][16 * kb + col] = cs;
      }
    }
    if (more) KTile::store(lds + ((t + 1) & 1) * KTile::BYTES, ld, tid);
    __syncthreads();
    if (tid < KT && t0 + tid < k1) {
      float v = 0.f;
      for (int wv = 0; wv < nrb; ++wv) v += red[t & 1][wv][tid];
      raw[t0 + tid] = v;
    }
  }
}

// Build the cache rows of one request: slots [0, S) <- tokens 0..S-1, slots
// [S, S+K) <- the selected middle tokens (ascending), ring slots <- the last R
// tokens at S+K + ((t-S-K) mod R).  Uncompressed prompts (L <= C) map token t
// to slot t.  Grid (cdiv(C, 16), Hkv, b); copies are 16-byte coalesced.
// A destination row outside [0, B_max) is skipped.
template <typename T, int D, int DV, bool ALIAS>
__global__ __launch_bounds__(256) void gather_kernel(PrefillArgs a, int compressed) {
  constexpr int SLOTS = 16;
  constexpr int KCH = D * static_cast<int>(sizeof(T)) / 16;
  constexpr int VCH = DV * static_cast<int>(sizeof(T)) / 16;
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
  for (int id = tid; id < SLOTS * KCH; id += blockDim.x) {
    const int j = id / KCH, ch = id % KCH;
    const int t = tok[j];
    if (t < 0) continue;
    const size_t s = static_cast<size_t>(sb) * SLOTS + j;
    *reinterpret_cast<u32x4_t*>(kdst + s * KCH * 16 + ch * 16) =
        *reinterpret_cast<const u32x4_t*>(ksrc + static_cast<size_t>(t) * KCH * 16 + ch * 16);
  }
  if (ALIAS) return;
  const char* vsrc = reinterpret_cast<const char*>(static_cast<const T*>(a.v) + pr.row0 * DV);
  char* vdst = reinterpret_cast<char*>(static_cast<T*>(a.vc) + gdst * a.C * DV);
  for (int id = tid; id < SLOTS * VCH; id += blockDim.x) {
    const int j = id / VCH, ch = id % VCH;
    const int t = tok[j];
    if (t < 0) continue;
    const size_t s = static_cast<size_t>(sb) * SLOTS + j;
    *reinterpret_cast<u32x4_t*>(vdst + s * VCH * 16 + ch * 16) =
        *reinterpret_cast<const u32x4_t*>(vsrc + static_cast<size_t>(t) * VCH * 16 + ch * 16);
  }
}

template <typename T, int D, int KT, int NWV>
hipError_t run_scores_w(const PrefillArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  const size_t rows = static_cast<size_t>(a.b) * a.Hkv * a.Rg;
  const unsigned rgrid = static_cast<unsigned>(cdiv(static_cast<int>(rows), 256));
  if (a.lse != nullptr) {
    lse_rowstat_kernel<<<rgrid, 256, 0, st>>>(a);
  } else {
    score_rowstat_kernel<T, D, KT, NWV><<<dim3(a.n_chunk1, a.Hkv, a.b), 64 * NWV, 0, st>>>(a);
    score_rowstat_combine_kernel<<<rgrid, 256, 0, st>>>(a);
  }
  score_columns_kernel<T, D, KT, NWV><<<dim3(a.n_chunk2, a.Hkv, a.b), 64 * NWV, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  return hipGetLastError();
}

// One 16-row block per wave: 8 waves cover G*W <= 128 rows, 16 waves <= 256.
template <typename T, int D, int KT>
hipError_t run_scores(const PrefillArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.Rg <= 128) return run_scores_w<T, D, KT, 8>(a, st, ev0, ev1);
  if (a.Rg <= 256) return run_scores_w<T, D, KT, 16>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

template <typename T, int D, int DV, bool ALIAS>
hipError_t run_gather(bool compressed, const PrefillArgs& a, hipStream_t st) {
  gather_kernel<T, D, DV, ALIAS><<<dim3(cdiv(a.C, 16), a.Hkv, a.b), 256, 0, st>>>(a, compressed);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_scores(int dtype, int D, const PrefillArgs& a, hipStream_t st,
                                 hipEvent_t ev0, hipEvent_t ev1) {
  if (dtype == 0 && D == 64) return run_scores<float, 64, 64>(a, st, ev0, ev1);
  if (dtype == 0 && D == 128) return run_scores<float, 128, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 64) return run_scores<bf16_t, 64, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 128) return run_scores<bf16_t, 128, 64>(a, st, ev0, ev1);
  if (dtype == 1 && D == 576) return run_scores_w<bf16_t, 576, 32, 16>(a, st, ev0, ev1);
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
