// Decode step over the fixed-size cache: rotary embedding + ring-buffer
// scatter of the new token, split-C flash-decode attention with GQA head
// grouping on MFMA, and a fixed-order combine of the split partials.
//
// Follows "SnapStream: Taming KV-Cache Eviction for Dataflow Accelerators",
// sections "Ring Buffer vs. Naive Slicing" (decode rotates only the recent
// window: the new key/value is scattered into a fixed slot, nothing is
// gathered or concatenated) and "Prefill / Decode Pipeline" (decode is bound
// by the bytes of cache it reads every step).
#include "common.h"
#include "launch.h"

namespace ss {

namespace {

// Rotate-half rotary embedding of element d of a row, computed in fp64 from
// the stored values and rounded once to O (the cache dtype for keys, fp32 for
// queries).  cs/sn hold cos/sin of the pair angles (pair i couples dims
// begin+i and begin+i+half).
template <typename T, typename O>
__device__ __forceinline__ O rotate_elem(const T* row, int d, bool rope, int begin, int half,
                                         const double* cs, const double* sn) {
  if (!rope || d < begin || d >= begin + 2 * half) return from_f32<O>(to_f32<T>(row[d]));
  const int i = d - begin;
  if (i < half) {
    const double x1 = to_f32<T>(row[d]), x2 = to_f32<T>(row[d + half]);
    return from_f64<O>(x1 * cs[i] - x2 * sn[i]);
  }
  const double x2 = to_f32<T>(row[d]), x1 = to_f32<T>(row[d - half]);
  return from_f64<O>(x2 * cs[i - half] + x1 * sn[i - half]);
}

// One workgroup per cache row: rotate q (into the workspace) and k_new at the
// absolute position, write k_new/v_new into the ring slot, update slot_pos
// and n_tokens.  Inactive rows (pos < 0) are left untouched.
template <typename T, int D, int DV, bool ALIAS>
__global__ __launch_bounds__(256) void decode_scatter_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int p = a.pos[b];
  if (p < 0) return;
  __shared__ double cs[D / 2], sn[D / 2];
  const bool rope = a.rope_theta > 0.0;
  const int d_rot = a.rope_end - a.rope_begin;
  const int half = rope ? d_rot / 2 : 0;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double ang = static_cast<double>(p) * pow(a.rope_theta, -2.0 * i / d_rot);
    double s, c;
    sincos(ang, &s, &c);
    cs[i] = c;
    sn[i] = s;
  }
  if (threadIdx.x == 0) {
    if (a.err != nullptr && a.n_tokens[b] != p) atomicOr(a.err, 1);
    a.n_tokens[b] = p + 1;
  }
  __syncthreads();
  const int SK = a.S + a.K;
  const int slot = p < SK ? p : SK + (p - SK) % a.R;

  const T* q = static_cast<const T*>(a.q) + static_cast<size_t>(b) * a.Hq * D;
  float* qr = a.q_rot + static_cast<size_t>(b) * a.Hq * D;
  for (int idx = threadIdx.x; idx < a.Hq * D; idx += blockDim.x) {
    const int d = idx % D;
    qr[idx] = rotate_elem<T, float>(q + (idx - d), d, rope, a.rope_begin, half, cs, sn);
  }
  const T* kn = static_cast<const T*>(a.k_new) + static_cast<size_t>(b) * a.Hkv * D;
  T* kc = static_cast<T*>(a.kc);
  for (int idx = threadIdx.x; idx < a.Hkv * D; idx += blockDim.x) {
    const int h = idx / D, d = idx % D;
    const size_t dst = ((static_cast<size_t>(b) * a.Hkv + h) * a.C + slot) * D + d;
    kc[dst] = rotate_elem<T, T>(kn + (idx - d), d, rope, a.rope_begin, half, cs, sn);
  }
  if (!ALIAS) {
    const T* vn = static_cast<const T*>(a.v_new) + static_cast<size_t>(b) * a.Hkv * DV;
    T* vc = static_cast<T*>(a.vc);
    for (int idx = threadIdx.x; idx < a.Hkv * DV; idx += blockDim.x) {
      const int h = idx / DV, d = idx % DV;
      vc[((static_cast<size_t>(b) * a.Hkv + h) * a.C + slot) * DV + d] = vn[idx];
    }
  }
  for (int h = threadIdx.x; h < a.Hkv; h += blockDim.x)
    a.slot_pos[(static_cast<size_t>(b) * a.Hkv + h) * a.C + slot] = p;
}

// Operands of the P.V contraction.  The contraction index of lane group qg,
// element i is the tile-local slot 4*i + qg (i < 8), which is exactly where
// the Q.K^T accumulator left that slot's probability (see decode_attend).
template <typename T> struct PvOps;

template <> struct PvOps<bf16_t> {
  static constexpr int STEPS = 1;
  static __device__ __forceinline__ bf16x8_t vfrag(const char* vt, int lrow, int db, int col,
                                                   int qg, int) {
    bf16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      e[i] = *reinterpret_cast<const bf16_t*>(vt + (4 * i + qg) * lrow + (16 * db + col) * 2);
    return pack_bf16x8(e);
  }
};

template <> struct PvOps<float> {
  static constexpr int STEPS = 8;
  static __device__ __forceinline__ float vfrag(const char* vt, int lrow, int db, int col, int qg,
                                                int st) {
    return *reinterpret_cast<const float*>(vt + (4 * st + qg) * lrow + (16 * db + col) * 4);
  }
};

// fp32 values (the rotated query, the probabilities) as MFMA operands of the
// storage type.  For bf16 each value becomes hi + lo with hi = bf16(x) and
// lo = bf16(x - hi): two MFMAs with exact bf16 x bf16 products carry x to
// about 2^-17 relative, so only the cache itself is bf16.
template <typename T> struct Split;

template <> struct Split<float> {
  static constexpr int N = 1;
  static __device__ __forceinline__ void make(const float* v, float (&out)[1]) { out[0] = v[0]; }
};

template <> struct Split<bf16_t> {
  static constexpr int N = 2;
  static __device__ __forceinline__ void make(const float* v, bf16x8_t (&out)[2]) {
    bf16_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = f32_to_bf16(v[e]);
      lo[e] = f32_to_bf16(v[e] - bf16_to_f32(hi[e]));
    }
    out[0] = pack_bf16x8(hi);
    out[1] = pack_bf16x8(lo);
  }
};

// Split-C flash-decode.  One wave per (split, kv-head, row); the G q-heads of
// the kv-head share every K/V byte read.  Per 32-slot tile:
//   S^T[slot, head] = K[slot, :] . Q[head, :]^T    (MFMA, K rows straight from HBM)
//   online softmax over slots per head (log2 domain)
//   O^T[dv, head] += V^T[dv, slot] . P^T[slot, head]  (MFMA, V staged in LDS)
// K rows are loaded in the order slot = t0 + 16*h2 + 4*(m%4) + m/4 for A-row m,
// so accumulator register r of lane group qg holds slot t0 + 16*h2 + 4*r + qg:
// the probabilities are already in the P^T operand layout, no shuffle needed.
template <typename T, int D, int DV, bool ALIAS>
__global__ __launch_bounds__(64) void decode_attend_kernel(DecodeArgs a) {
  using MM = Mma<T>;
  using frag = typename MM::frag;
  constexpr int KPL = MM::KPL, KSTEP = MM::KSTEP;
  constexpr int NC = D / KSTEP;
  constexpr int NDB = DV / 16;
  constexpr int TS = DECODE_TILE;
  constexpr int VROW = DV * static_cast<int>(sizeof(T));
  constexpr int VSTRIDE = ALIAS ? D : DV;
  constexpr int LROW = VROW + 32;
  constexpr int VCH = VROW / 16;
  constexpr int VLD = TS * VCH / 64;
  static_assert(D % KSTEP == 0 && DV % 64 == 0 && (TS * VCH) % 64 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) char vt[TS * LROW];

  const int lane = threadIdx.x;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int p = a.pos[b];
  if (p < 0) return;
  const int n_valid = min(p + 1, a.C);
  const int s0 = split * a.split;
  if (s0 >= n_valid) return;
  const int s1 = min(s0 + a.split, n_valid);
  const int col = lane & 15, qg = lane >> 4;

  constexpr int NP = Split<T>::N;
  const float* qrow =
      a.q_rot + (static_cast<size_t>(b) * a.Hq + static_cast<size_t>(h) * a.G + col) * D;
  frag qf[NP][NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float qv[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) qv[e] = (col < a.G) ? qrow[c * KSTEP + qg * KPL + e] : 0.f;
    frag parts[NP];
    Split<T>::make(qv, parts);
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) qf[pp][c] = parts[pp];
  }

  const size_t gh = static_cast<size_t>(b) * a.Hkv + h;
  const T* kb = static_cast<const T*>(a.kc) + gh * a.C * D;
  const T* vb = ALIAS ? kb : static_cast<const T*>(a.vc) + gh * a.C * DV;
  const int koff = 4 * (col & 3) + (col >> 2);

  frag kf[2][NC];
  u32x4_t vr[VLD];
  // always inlined: the register arrays it fills must not become stack memory
  auto load_tile = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int s = min(t0 + 16 * h2 + koff, s1 - 1);
      const T* kr = kb + static_cast<size_t>(s) * D + qg * KPL;
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[h2][c] = MM::load(kr + c * KSTEP);
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int id = i * 64 + lane;
      const int s = min(t0 + id / VCH, s1 - 1);
      vr[i] = *reinterpret_cast<const u32x4_t*>(
          reinterpret_cast<const char*>(vb + static_cast<size_t>(s) * VSTRIDE) + (id % VCH) * 16);
    }
  };

  f32x4_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  load_tile(s0);
  for (int t0 = s0; t0 < s1; t0 += TS) {
    __syncthreads();  // the previous tile's LDS reads are done
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
    if (t0 + TS < s1) load_tile(t0 + TS);  // next tile in flight during this one

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
      x[i] = s < s1 ? sacc[i >> 2][i & 3] * a.scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, x[i]);
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
    constexpr int PST = PvOps<T>::STEPS;
    frag pfr[PST][NP];
#pragma unroll
    for (int st = 0; st < PST; ++st) Split<T>::make(pf + st * KPL, pfr[st]);
    __syncthreads();  // V tile visible in LDS
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
  if (col < a.G) {
    const size_t pidx =
        (static_cast<size_t>(b) * a.Hq + static_cast<size_t>(h) * a.G + col) * a.n_split + split;
    float* po = a.part_o + pidx * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<float4*>(po + 16 * db + 4 * qg) =
          make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    if (qg == 0) {
      a.part_ml[2 * pidx] = m_run;
      a.part_ml[2 * pidx + 1] = l_run;
    }
  }
}

// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s over the non-empty
// splits of the row, in split order (deterministic).  Inactive rows get 0.
template <typename T, int DV>
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  constexpr int PER = DV / 64;
  const int hq = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  T* out = static_cast<T*>(a.out) + (static_cast<size_t>(b) * a.Hq + hq) * DV + lane * PER;
  const int p = a.pos[b];
  if (p < 0) {
#pragma unroll
    for (int e = 0; e < PER; ++e) out[e] = from_f32<T>(0.f);
    return;
  }
  const int ns = cdiv(min(p + 1, a.C), a.split);
  const size_t base = (static_cast<size_t>(b) * a.Hq + hq) * a.n_split;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[2 * (base + s)]);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f(a.part_ml[2 * (base + s)] - M);
    wsum += w * a.part_ml[2 * (base + s) + 1];
    const float* po = a.part_o + (base + s) * DV + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += w * po[e];
  }
  const float inv = 1.f / wsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[e] = from_f32<T>(acc[e] * inv);
}

template <typename T, int D, int DV, bool ALIAS>
hipError_t run_decode(const DecodeArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  decode_scatter_kernel<T, D, DV, ALIAS><<<a.B, 256, 0, st>>>(a);
  if (ev0 != nullptr && hipEventRecord(ev0, st) != hipSuccess) return hipErrorInvalidValue;
  decode_attend_kernel<T, D, DV, ALIAS><<<dim3(a.n_split, a.Hkv, a.B), 64, 0, st>>>(a);
  if (ev1 != nullptr && hipEventRecord(ev1, st) != hipSuccess) return hipErrorInvalidValue;
  decode_combine_kernel<T, DV><<<dim3(a.Hq, a.B), 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(int dtype, int D, int DV, int alias, const DecodeArgs& a,
                         hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  if (alias) return hipErrorInvalidValue;
  if (dtype == 0 && D == 64 && DV == 64) return run_decode<float, 64, 64, false>(a, st, ev0, ev1);
  if (dtype == 0 && D == 128 && DV == 128)
    return run_decode<float, 128, 128, false>(a, st, ev0, ev1);
  if (dtype == 1 && D == 64 && DV == 64) return run_decode<bf16_t, 64, 64, false>(a, st, ev0, ev1);
  if (dtype == 1 && D == 128 && DV == 128)
    return run_decode<bf16_t, 128, 128, false>(a, st, ev0, ev1);
  return hipErrorInvalidValue;
}

}  // namespace ss
