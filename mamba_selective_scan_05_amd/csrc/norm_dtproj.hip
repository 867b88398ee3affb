// Jamba's RMSNorms on the selective parameters, then dt_proj + bias + softplus.
//
// norm: one wave per token adds the x_proj partial sums in slice order, then RMSNorms the dt slice (R
// values), the B slice and the C slice (N values each) separately: v / sqrt(mean(v^2) + eps) * w.  The
// normalised dt goes out in the I/O dtype (it is the next contraction's operand), B and C in fp32.
//
// dt_proj: delta[m, c] = softplus(sum_r dln[m, r] * W[c, r] + b[c]).  bf16 path on matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation): a workgroup of 4 waves computes a 64-token x 256-channel
// tile, each wave 64 x 64, with the bias and softplus fused into the epilogue.  fp32 path on the vector
// ALU.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kMaxCols = 9;   // ceil((512 + 32) / 64): columns of dbc per lane

template <typename T>
__global__ __launch_bounds__(256) void norm_kernel(const float* __restrict__ part, int splits, int M, int R, int N,
                                                   const T* __restrict__ wdt, const T* __restrict__ wb,
                                                   const T* __restrict__ wc, float eps, T* __restrict__ dln,
                                                   float* __restrict__ bc) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (m >= M) return;
  const int W = R + 2 * N;
  float v[kMaxCols];
  float ss_dt = 0.f, ss_b = 0.f, ss_c = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxCols; ++i) {
    const int col = lane + 64 * i;
    float s = 0.f;
    if (col < W)
      for (int p = 0; p < splits; ++p) s += part[((int64_t)p * M + m) * W + col];
    v[i] = s;
    const float sq = s * s;
    if (col < R) ss_dt += sq;
    else if (col < R + N) ss_b += sq;
    else if (col < W) ss_c += sq;
  }
  ss_dt = wave_sum(ss_dt);
  ss_b = wave_sum(ss_b);
  ss_c = wave_sum(ss_c);
  const float r_dt = 1.0f / sqrtf(ss_dt / R + eps);
  const float r_b = 1.0f / sqrtf(ss_b / N + eps);
  const float r_c = 1.0f / sqrtf(ss_c / N + eps);
#pragma unroll
  for (int i = 0; i < kMaxCols; ++i) {
    const int col = lane + 64 * i;
    if (col < R) {
      io<T>::st(dln + (int64_t)m * R + col, v[i] * r_dt * io<T>::ld(wdt + col));
    } else if (col < R + N) {
      bc[(int64_t)m * 2 * N + (col - R)] = v[i] * r_b * io<T>::ld(wb + (col - R));
    } else if (col < W) {
      bc[(int64_t)m * 2 * N + (col - R)] = v[i] * r_c * io<T>::ld(wc + (col - R - N));
    }
  }
}

__device__ __forceinline__ bf16x8 ld_bf16x8_guard(const bf16_t* p, bool ok) {
  uint4 raw = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  return __builtin_bit_cast(bf16x8, raw);
}

// 64 tokens x 256 channels per workgroup; wave w owns channels [64w, 64w + 64) of the tile.
__global__ __launch_bounds__(256) void dtproj_mfma_kernel(const bf16_t* __restrict__ dln,
                                                          const bf16_t* __restrict__ w,
                                                          const bf16_t* __restrict__ bias,
                                                          bf16_t* __restrict__ delta, int M, int C, int R) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int c0 = blockIdx.x * 256 + wave * 64;
  const int m0 = blockIdx.y * 64;
  f32x4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (c0 >= C) return;
  for (int k = 0; k < R; k += 32) {
    const bool kok = k + lk < R;   // R % 8 == 0: an 8-wide k group is wholly in or out
    bf16x8 a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + r * 16 + lr;
      a[r] = ld_bf16x8_guard(dln + (int64_t)m * R + k + lk, kok && m < M);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = ld_bf16x8_guard(w + (int64_t)(c0 + t * 16 + lr) * R + k + lk, kok);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], b[t], acc[r][t], 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = c0 + t * 16 + lr;
    const float bc_ = bf2f(bias[c]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + r * 16 + (lane >> 4) * 4 + i;
        if (m < M) delta[(int64_t)m * C + c] = f2bf(softplus(acc[r][t][i] + bc_));
      }
  }
}

__global__ __launch_bounds__(256) void dtproj_f32_kernel(const float* __restrict__ dln, const float* __restrict__ w,
                                                         const float* __restrict__ bias, float* __restrict__ delta,
                                                         int M, int C, int R) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int m = blockIdx.y;
  if (c >= C) return;
  float acc = 0.f;
  for (int r = 0; r < R; ++r) acc = fmaf(dln[(int64_t)m * R + r], w[(int64_t)c * R + r], acc);
  delta[(int64_t)m * C + c] = softplus(acc + bias[c]);
}

}  // namespace

void launch_norm(bool bf16, const float* part, int splits, int M, int R, int N, const void* wdt, const void* wb,
                 const void* wc, float eps, void* dln, float* bc, hipStream_t st) {
  if (M == 0) return;
  dim3 grid((M + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(norm_kernel<bf16_t>, grid, dim3(256), 0, st, part, splits, M, R, N, (const bf16_t*)wdt,
                       (const bf16_t*)wb, (const bf16_t*)wc, eps, (bf16_t*)dln, bc);
  else
    hipLaunchKernelGGL(norm_kernel<float>, grid, dim3(256), 0, st, part, splits, M, R, N, (const float*)wdt,
                       (const float*)wb, (const float*)wc, eps, (float*)dln, bc);
}

void launch_dtproj(bool bf16, const void* dln, const void* w, const void* b, void* delta, int M, int C, int R,
                   hipStream_t st) {
  if (M == 0) return;
  if (bf16) {
    dim3 grid((C + 255) / 256, (M + 63) / 64);
    hipLaunchKernelGGL(dtproj_mfma_kernel, grid, dim3(256), 0, st, (const bf16_t*)dln, (const bf16_t*)w,
                       (const bf16_t*)b, (bf16_t*)delta, M, C, R);
  } else {
    dim3 grid((C + 255) / 256, M);
    hipLaunchKernelGGL(dtproj_f32_kernel, grid, dim3(256), 0, st, (const float*)dln, (const float*)w,
                       (const float*)b, (float*)delta, M, C, R);
  }
}

}  // namespace jm
