// x_proj: dbc[m, n] = sum_k xc[m, k] * W[n, k]   (M tokens, N = dt_rank + 2*d_state, K = d_inner).
//
// bf16 path: matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.  A workgroup owns a 64-token
// tile and the whole N; its waves split N into 16-wide tiles, so every xc element is read from HBM once.
// The xc tile of each 64-wide K block is staged through LDS (double-buffered, rows padded by 16 bytes
// against bank conflicts) and shared by the waves; each wave streams its own rows of W straight from
// L2.  When there are too few token tiles to fill the GPU the K range is split over `splits` workgroups
// that write fp32 partial sums; the norm step adds them in a fixed order, so results are deterministic.
//
// fp32 path: plain fp32 dot products on the vector ALU (the fp32 I/O mode must not round xc to bf16).
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kMT = 64;          // tokens per workgroup tile
constexpr int kKB = 64;          // K block staged in LDS
constexpr int kLda = kKB + 8;    // padded LDS row, bf16 elements
constexpr int kNT = 9;           // 16-wide N tiles per wave

__device__ __forceinline__ bf16x8 ld_bf16x8(const bf16_t* p) {
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, raw);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// MFMA 16x16x32 operand layout used here: lane l supplies row (l % 16) of A and column (l % 16) of B,
// both over the 8 consecutive k values 8*(l / 16) .. +7 (the same k set for A and B, so the product is
// independent of how the hardware orders k).  The accumulator holds rows 4*(l / 16) + i, column l % 16.
__global__ __launch_bounds__(256) void xproj_mfma_kernel(const bf16_t* __restrict__ xc, const bf16_t* __restrict__ w,
                                                         float* __restrict__ part, int M, int N, int K,
                                                         int k_per_split) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kMT * kLda];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nthreads = blockDim.x;
  const int m0 = blockIdx.x * kMT;
  const int s = blockIdx.y;
  const int kbeg = s * k_per_split;
  const int nblocks = k_per_split / kKB;
  const int lr = lane & 15, lk = (lane >> 4) * 8;

  f32x4 acc[4][kNT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A tile loader: 64 rows x 64 k = 512 chunks of 16 bytes.
  auto load_a = [&](int kb, int buf) {
    for (int q = tid; q < kMT * (kKB / 8); q += nthreads) {
      const int row = q >> 3, kc = (q & 7) * 8;
      const int m = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M) v = *reinterpret_cast<const uint4*>(xc + (int64_t)m * K + kb + kc);
      *reinterpret_cast<uint4*>(&As[buf][row * kLda + kc]) = v;
    }
  };

  const int ntile0 = wave * kNT;
  load_a(kbeg, 0);
  __syncthreads();
  for (int ib = 0; ib < nblocks; ++ib) {
    const int kb = kbeg + ib * kKB;
    const int buf = ib & 1;
    if (ib + 1 < nblocks) load_a(kb + kKB, buf ^ 1);
#pragma unroll
    for (int ks = 0; ks < kKB; ks += 32) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = *reinterpret_cast<const bf16x8*>(&As[buf][(r * 16 + lr) * kLda + ks + lk]);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const int n = (ntile0 + t) * 16 + lr;
        const bf16x8 bv = n < N ? ld_bf16x8(w + (int64_t)n * K + kb + ks + lk) : zero_bf16x8();
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv, acc[r][t], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  float* dst = part + (int64_t)s * M * N;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int n = (ntile0 + t) * 16 + lr;
    if (n >= N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + r * 16 + (lane >> 4) * 4 + i;
        if (m < M) dst[(int64_t)m * N + n] = acc[r][t][i];
      }
  }
}

// fp32: one thread per (m, n); the xc row is staged through LDS in 1024-element pieces.
__global__ __launch_bounds__(64) void xproj_f32_kernel(const float* __restrict__ xc, const float* __restrict__ w,
                                                       float* __restrict__ part, int M, int N, int K) {
  __shared__ float row[1024];
  const int m = blockIdx.x;
  const int n = blockIdx.y * 64 + threadIdx.x;
  float acc = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 1024) {
    const int kn = min(1024, K - k0);
    __syncthreads();
    for (int i = threadIdx.x; i < kn; i += 64) row[i] = xc[(int64_t)m * K + k0 + i];
    __syncthreads();
    if (n < N)
      for (int i = 0; i < kn; ++i) acc = fmaf(row[i], w[(int64_t)n * K + k0 + i], acc);
  }
  if (n < N) part[(int64_t)m * N + n] = acc;
}

}  // namespace

void launch_xproj(bool bf16, const void* xc, const void* w, float* part, int M, int N, int K, int splits,
                  hipStream_t st) {
  if (M == 0) return;
  if (bf16) {
    const int ntiles = (N + 15) / 16;
    const int waves = (ntiles + kNT - 1) / kNT;
    dim3 grid((M + kMT - 1) / kMT, splits);
    hipLaunchKernelGGL(xproj_mfma_kernel, grid, dim3(64 * waves), 0, st, (const bf16_t*)xc, (const bf16_t*)w,
                       part, M, N, K, K / splits);
  } else {
    dim3 grid(M, (N + 63) / 64);
    hipLaunchKernelGGL(xproj_f32_kernel, grid, dim3(64), 0, st, (const float*)xc, (const float*)w, part, M, N, K);
  }
}

}  // namespace jm
