// Helpers shared by the decode kernels (decode.hip, decode_ring.hip, decode_mla.hip).
#pragma once

#include "common.h"
#include "launch.h"

namespace ss {
namespace dec {

// Rotate-half rotary embedding of element d of a row (value x, and xp = the
// element it pairs with), computed in fp64 from the stored values and rounded
// once to O (the cache dtype for keys, fp32 for queries).  cs/sn hold cos/sin
// of the pair angles (pair i couples dims begin+i and begin+i+half).
template <typename T, typename O>
__device__ __forceinline__ O rotate_pair(T x, T xp, int d, bool rope, int begin, int half,
                                         const double* cs, const double* sn) {
  if (!rope || d < begin || d >= begin + 2 * half) return from_f32<O>(to_f32<T>(x));
  const int i = d - begin;
  const double v = to_f32<T>(x), w = to_f32<T>(xp);
  if (i < half) return from_f64<O>(v * cs[i] - w * sn[i]);
  return from_f64<O>(v * cs[i - half] + w * sn[i - half]);
}

// Device-scope stores: written through to the level shared by all XCDs (the
// sc1 policy the compiler uses for agent-scope atomic stores), so publishing
// them needs no whole-L2 write-back.  Completion is awaited with s_waitcnt.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Device-scope load (the access the compiler emits for an agent-scope relaxed
// atomic load: it is served by the level shared by all XCDs, never by a stale
// line of this XCD's L2).
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16-byte device-scope loads: a raw buffer over [p, p + bytes) whose loads
// carry the same device-scope (sc1) cache policy.
constexpr int CPOL_SC1 = 16;
constexpr int BUF_RSRC_WORD3 = 0x00020000;  // 32-bit data format, raw (stride 0) addressing
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_buffer(const float* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, bytes, BUF_RSRC_WORD3);
}
__device__ __forceinline__ f32x4_t ld_dev4(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CPOL_SC1));
}
__device__ __forceinline__ void st_dev4(float* p, f32x4_t v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}

// 16-byte load of cache bytes that this launch reads once, with the
// non-temporal cache policy (nt: a hint that the data will not be reused).
__device__ __forceinline__ u32x4_t ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// Operands of the P.V contraction.  The contraction index of lane group qg,
// element i is the tile-local slot 4*i + qg (i < 8), which is exactly where
// the Q.K^T accumulator left that slot's probability (see decode_kernel).
template <typename T> struct PvOps;

// bf16: two transposing LDS reads (gfx950 ds_read_b64_tr_b16) build the
// fragment.  Within each group of 16 lanes, lane 4a + b receives element b
// of the 8-byte chunks that lanes a + 4k (k < 4) address; so lane (col, qg)
// addresses dims 16 db + 4 (col % 4) .. + 3 of slot 4 (col / 4) + qg
// (elements i < 4) and of slot 16 + 4 (col / 4) + qg (i >= 4), and receives
// dim 16 db + col of slots 4 i + qg.  lrow must be a multiple of 8 bytes.
template <> struct PvOps<bf16_t> {
  static constexpr int STEPS = 1;
  static __device__ __forceinline__ bf16x8_t vfrag(const char* vt, int lrow, int db, int col,
                                                   int qg, int) {
    typedef short v4i16_t __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v4i16_t* lds_v4;
    const char* base = vt + (4 * (col >> 2) + qg) * lrow + (16 * db + 4 * (col & 3)) * 2;
    const u32x2_t lo = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)base));
    const u32x2_t hi =
        __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4)(base + 16 * lrow)));
    return __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
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

// ---- LDS access behind direct global->LDS loads.  While such loads are in
// flight the compiler waits for all of them before any LDS access it cannot
// tell apart from them (it does not count them together with ordinary loads
// and stores either), so kernels that stream tiles by direct loads make
// their other LDS accesses with these asm helpers, which wait for their own
// results only.

__device__ __forceinline__ int lds_addr(const char* p) {
  return static_cast<int>((uintptr_t)((const __attribute__((address_space(3))) char*)p));
}

// N 16-byte LDS reads in one asm block that also waits for them.
template <int N>
__device__ __forceinline__ void lds_read16(const int (&ad)[N], u32x4_t (&r)[N]) {
  if constexpr (N == 8) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
          "=&v"(r[6]), "=&v"(r[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]),
          "v"(ad[7])
        : "memory");
  } else if constexpr (N == 4) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  } else {
    static_assert(N == 2, "2, 4 or 8 reads");
    asm volatile(
        "ds_read_b128 %0, %2\n\t"
        "ds_read_b128 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1])
        : "v"(ad[0]), "v"(ad[1])
        : "memory");
  }
}

// 16-byte LDS store (its completion is awaited by the next lds_barrier or
// asm wait).
__device__ __forceinline__ void lds_write16(int ad, u32x4_t v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(ad), "v"(v) : "memory");
}

// Rotate-half rotary embedding of one dim from the stored value x and its
// partner xp, in fp64, rounded once to O: upper = the dim lies in the second
// half of the rotary range; c, s = cos, sin of the pair's angle.  Outside the
// range the value passes through.
template <typename O>
__device__ __forceinline__ O rot_dim(bf16_t x, bf16_t xp, bool in, bool upper, double c, double s) {
  if (!in) return from_f32<O>(bf16_to_f32(x));
  const double v = bf16_to_f32(x), w = bf16_to_f32(xp);
  if (!upper) return from_f64<O>(v * c - w * s);
  return from_f64<O>(v * c + w * s);
}

// Workgroup barrier for LDS data only (__syncthreads() would also wait for
// every outstanding direct load, e.g. of the next tile, just issued).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Orders LDS accesses of one wave (a wave executes its LDS instructions in
// order; this keeps the compiler from moving them across the point).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The last workgroup of a (row, kv-head) group merges every split's partial
// (max m_s, sum l_s, unnormalised o_s, written with st_dev/st_dev4).
// Ordering: every writer waits for its partial stores to complete at the
// device-coherent level before it takes its ticket; the merging workgroup
// holds the last ticket, so all partials are there before it issues its
// device-scope loads (ld_dev, ld_dev4).  No acquire fence is used: a fence would
// invalidate this XCD's whole L2 and slow every workgroup still streaming on
// it.  This rests on the gfx942/gfx950 cache policy rather than on the HIP
// memory model's release/acquire pair: sc1 stores (agent-scope atomic stores
// and st_dev4) write through the XCD's L2, s_waitcnt vmcnt(0) returns once
// they are acknowledged at the device-coherent level, and sc1 loads
// (agent-scope atomic loads and ld_dev4) never hit a stale line of this
// XCD's L2.  Checked with the ROCm 7.2 toolchain; the determinism, many-split and
// graph-replay decode tests guard it.  The merge computes
//   out[head, dv] = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// in split order.
template <typename T, int DV, int NI, int MB>
__device__ __forceinline__ void merge_splits_mb(const DecodeArgs& a, size_t head0, int G, int ns,
                                                int tid, int nthreads) {
  // Each thread merges NI outputs of one head (4 dims each, NO = DV/4/NI
  // apart so that every load instruction stays coalesced; they share the
  // splits' (m, l)) at once, MB splits per batch: one memory round trip per
  // batch.  Loads are unconditional (a split index
  // past ns rereads the last split), so no wait is forced between them; the
  // surplus gets weight 0.
  static_assert((DV / 4) % NI == 0, "an output group stays within one head");
  constexpr int NO = DV / 4 / NI;
  const int ngrp = G * NO;
  for (int q = tid; q < ngrp; q += nthreads) {
    const int g = q / NO, d40 = q % NO;
    const size_t base = (head0 + g) * a.n_split;
    const __amdgpu_buffer_rsrc_t ob = dev_buffer(a.part_o + base * DV, a.n_split * DV * 4);
    float M = -INFINITY, L = 0.f;
    f32x4_t acc[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < ns; sb += MB) {
      float mv[MB], lv[MB];
      f32x4_t ov[MB][NI];
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int sp = min(sb + j, ns - 1);
        mv[j] = ld_dev(a.part_ml + 2 * (base + sp));
        lv[j] = ld_dev(a.part_ml + 2 * (base + sp) + 1);
#pragma unroll
        for (int k = 0; k < NI; ++k) ov[j][k] = ld_dev4(ob, (sp * DV + 4 * (d40 + k * NO)) * 4);
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < MB; ++j)
        if (sb + j < ns) Mn = fmaxf(Mn, mv[j]);
      // a batch of splits without slots leaves Mn at -inf: nothing to add
      const float Mr = Mn == -INFINITY ? 0.f : Mn;
      const float r = exp2f(M - Mr);
      L *= r;
#pragma unroll
      for (int k = 0; k < NI; ++k) acc[k] *= r;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float w = sb + j < ns ? exp2f(mv[j] - Mr) : 0.f;
        L += w * lv[j];
#pragma unroll
        for (int k = 0; k < NI; ++k) acc[k] += w * ov[j][k];
      }
      M = Mn;
    }
    const float inv = 1.f / L;
    T* o = static_cast<T*>(a.out) + (head0 + g) * DV + 4 * d40;
#pragma unroll
    for (int k = 0; k < NI; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * k * NO + e] = from_f32<T>(acc[k][e] * inv);
  }
}

// Batches of 4 splits when there are at most 4, of 8 up to 8, else of 16 (a
// batch rereads the last split up to its size: at 4 splits, 48 loads per
// thread where 12 do; llama8b_c4k 46.5 -> 45.4 us per launch, llama8b_128k
// 158.9 -> 158.2 us).
template <typename T, int DV>
__device__ __forceinline__ void merge_splits(const DecodeArgs& a, size_t head0, int G, int ns,
                                             int tid, int nthreads) {
  if (ns <= 4) {
    merge_splits_mb<T, DV, 1, 4>(a, head0, G, ns, tid, nthreads);
  } else if (ns <= 8) {
    merge_splits_mb<T, DV, 1, 8>(a, head0, G, ns, tid, nthreads);
  } else {
    merge_splits_mb<T, DV, 1, 16>(a, head0, G, ns, tid, nthreads);
  }
}

template <typename T, int DV, int NI>
__device__ __forceinline__ void merge_splits_wide(const DecodeArgs& a, size_t head0, int G, int ns,
                                             int tid, int nthreads) {
  // (the latent kernel's merge: 8 heads x 512 dims of 16 splits; its (m, l)
  // as two 4-byte loads, which measured faster there than one 8-byte load)
  // Each thread merges NI outputs of one head (4 dims each, NO = DV/4/NI
  // apart so that every load instruction stays coalesced; they share the
  // splits' (m, l)) at once, MB splits per batch: one memory round trip per
  // batch.  Loads are unconditional (a split index past ns rereads
  // the last split), so no wait is forced between them; the surplus gets
  // weight 0.
  static_assert((DV / 4) % NI == 0, "an output group stays within one head");
  constexpr int MB = NI > 1 ? 8 : 16;
  constexpr int NO = DV / 4 / NI;
  const int ngrp = G * NO;
  for (int q = tid; q < ngrp; q += nthreads) {
    const int g = q / NO, d40 = q % NO;
    const size_t base = (head0 + g) * a.n_split;
    const __amdgpu_buffer_rsrc_t ob = dev_buffer(a.part_o + base * DV, a.n_split * DV * 4);
    float M = -INFINITY, L = 0.f;
    f32x4_t acc[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) acc[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < ns; sb += MB) {
      float mv[MB], lv[MB];
      f32x4_t ov[MB][NI];
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int sp = min(sb + j, ns - 1);
        mv[j] = ld_dev(a.part_ml + 2 * (base + sp));
        lv[j] = ld_dev(a.part_ml + 2 * (base + sp) + 1);
#pragma unroll
        for (int k = 0; k < NI; ++k) ov[j][k] = ld_dev4(ob, (sp * DV + 4 * (d40 + k * NO)) * 4);
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < MB; ++j)
        if (sb + j < ns) Mn = fmaxf(Mn, mv[j]);
      // a batch of splits without slots leaves Mn at -inf: nothing to add
      const float Mr = Mn == -INFINITY ? 0.f : Mn;
      const float r = exp2f(M - Mr);
      L *= r;
#pragma unroll
      for (int k = 0; k < NI; ++k) acc[k] *= r;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const float w = sb + j < ns ? exp2f(mv[j] - Mr) : 0.f;
        L += w * lv[j];
#pragma unroll
        for (int k = 0; k < NI; ++k) acc[k] += w * ov[j][k];
      }
      M = Mn;
    }
    const float inv = 1.f / L;
    T* o = static_cast<T*>(a.out) + (head0 + g) * DV + 4 * d40;
#pragma unroll
    for (int k = 0; k < NI; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * k * NO + e] = from_f32<T>(acc[k][e] * inv);
  }
}

}  // namespace dec
}  // namespace ss
