// Device-side helpers shared by the mixer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jm {

typedef uint16_t bf16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the high half of the fp32); narrowing rounds to
// nearest-even through the hardware converter (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ __forceinline__ bf16_t f2bf(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}
// two values rounded the same way and packed (lo in bits 0-15): one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

template <typename T> struct io;
template <> struct io<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ float cvt(float v) { return v; }
  static __device__ __forceinline__ float from(float v) { return v; }
};
template <> struct io<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
  static __device__ __forceinline__ float cvt(bf16_t v) { return bf2f(v); }
  static __device__ __forceinline__ bf16_t from(float v) { return f2bf(v); }
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x on the transcendental unit (v_exp_f32, about 1 ulp; flushes to 0 far below the normal range).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// 1/x on the transcendental unit (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// SiLU(u) = u / (1 + e^-u).  For u -> -inf the exp overflows to inf and the reciprocal gives 0.
__device__ __forceinline__ float silu(float u) { return u * rcp_fast(1.0f + exp2_fast(-u * kLog2e)); }

// max(v, 0) as one instruction: a signed-integer max of the bits (negative floats, -0 included, are
// negative integers; zero and positive floats keep their order).  fmaxf on a value the compiler cannot prove
// canonical (a matrix-core result, a load) first runs it through a second v_max_f32 to quiet signalling
// NaNs, which the inputs here never carry.  Plain code, not inline asm: the compiler must see the read to
// keep the wait states a matrix-core result needs before a vector instruction reads it.
__device__ __forceinline__ float relu(float v) { return __int_as_float(max(__float_as_int(v), 0)); }

// softplus(v) = log(1 + e^v) = max(v, 0) + log(1 + e^-|v|), without overflow, on the transcendental unit
// (v_exp_f32, v_log_f32).  For v below about -17, 1 + e^v rounds to 1 and the result is 0 instead of
// e^v < 4e-8: an absolute error far below anything a delta of that size can change downstream.
__device__ __forceinline__ float softplus(float v) {
  const float e = exp2_fast(-fabsf(v) * kLog2e);
  return relu(v) + __builtin_amdgcn_logf(1.0f + e) * kLn2;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The exact zero-order-hold input coefficient (exp(dt A) - 1) / A (the discretisation equation's first form,
// (dt A)^-1 (exp(dt A) - 1) dt, for a diagonal A), given e = exp(dt A) and 1 / A.  For |dt A| < 1/16, where
// e - 1 would lose digits, it is the series dt (1 + z/2 + z^2/6 + z^3/24), z = dt A (truncation < 2e-7).
__device__ __forceinline__ float zoh_coef(float dt, float e, float A, float iA) {
  const float z = dt * A;
  const float series = dt * fmaf(z, fmaf(z, fmaf(z, 1.0f / 24.0f, 1.0f / 6.0f), 0.5f), 1.0f);
  return fabsf(z) < 0.0625f ? series : fmaf(e, iA, -iA);   // (e - 1) / A as one FMA
}

// Packed variable-length batches: sequence s holds packed tokens [cu[s], cu[s+1]).  The sequence holding
// token t is the last s in [0, nseq) with cu[s] <= t, which skips empty sequences; the search stays in
// [0, nseq) whatever the offsets hold.  cu is read-only and wave-uniform here (scalar loads).
__device__ __forceinline__ int seq_of(const int32_t* cu, int nseq, int t) {
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid;
    else hi = mid;
  }
  return lo;
}

// The state row of sequence s: s itself without a pool, else its slot, -1 for a slot outside [0, pool).
__device__ __forceinline__ int64_t state_row(const int32_t* slots, int pool, int s) {
  if (!slots) return s;
  const int r = slots[s];
  return r >= 0 && r < pool ? r : -1;
}

// A wave's 64 channels of a [rows, C, 16] fp32 state are 4 KB of contiguous memory.  They move between HBM
// and registers through a 4 KB LDS tile, as four 1 KB rows of contiguous 16-byte lanes: per-lane 64-byte
// strides would make each 16-byte access instruction touch 32 cache lines for 1 KB of data (this is the
// whole traffic of a one-token step).  In LDS, chunk q of lane l sits in slot q ^ ((l >> 2) & 3) of the
// lane's 64 bytes, which keeps the per-lane 16-byte reads and writes free of bank conflicts.  The HBM side
// uses non-temporal loads and stores: a state is read once and written once per call, and keeping it out
// of the caches leaves them to the weights and activations that are reused (the B = 256 decode step went
// from 86 to 75 us with its four state sets rotated, i.e. with cold states).
__device__ __forceinline__ int hslot(int l, int q) { return l * 16 + ((q ^ ((l >> 2) & 3)) << 2); }
__device__ __forceinline__ void state_load(const float* src, float* hs, int lane, float* h) {
  __builtin_amdgcn_wave_barrier();                    // the tile may still be in use by an earlier store
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = q * 64 + lane;                      // 16-byte chunk g of the wave's 4 KB
    *reinterpret_cast<f32x4*>(&hs[hslot(g >> 2, g & 3)]) =
        __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + g * 4));
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(&hs[hslot(lane, q)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) h[q * 4 + i] = v[i];
  }
}
__device__ __forceinline__ void state_store(float* dst, float* hs, int lane, const float* h) {
  __builtin_amdgcn_wave_barrier();                    // the tile may still be in use by an earlier load
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(&hs[hslot(lane, q)]) = f32x4{h[q * 4], h[q * 4 + 1], h[q * 4 + 2], h[q * 4 + 3]};
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int g = q * 64 + lane;
    __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&hs[hslot(g >> 2, g & 3)]),
                                 reinterpret_cast<f32x4*>(dst + g * 4));
  }
}

}  // namespace jm
