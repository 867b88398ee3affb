// The fp32 I/O mode's two contractions on the matrix cores (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums):
//   x_proj   part[s, m, n] = sum over channel slice s of xc[m, k] * w[n, k]   (the norm step adds the slices)
//   dt_proj  delta[m, n]   = softplus(sum_k dln[m, k] * w[n, k] + b[n])
// (TransformerLens "supported_architectures.jamba", the Mamba-1 mixer: x_proj to dt / B / C, then dt_proj with
// its bias and softplus.)  Both are Y = X W^T with K contiguous in both operands.
//
// A workgroup of 4 waves owns a 128-row x TN-column tile of Y (TN = 96 for x_proj's 288 columns, else 128), each
// wave 64 x TN / 2 (4 x TN / 32 MFMA tiles).  32-wide K blocks of X and W pass through double-buffered LDS, the
// next block's global loads in flight in registers while the current block multiplies; one barrier per
// block.  The tile size sets the arithmetic per byte the workgroup pulls from L2 (128 x 128: 32 flops per
// byte, against 16 for 64 x 64 tiles).  The MFMA's K slot of lane group g = lane / 16 takes K index 4g + q of a
// 16-wide chunk at step q (any assignment works as long as both operands use the same one), so a lane reads its
// A and B fragments of four steps as one 16-byte LDS load; rows are padded by 16 bytes, which spreads the 16
// rows of a fragment read over distinct banks.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

constexpr int kFM = 128;         // rows of X per tile
constexpr int kFK = 32;          // K block
constexpr int kFLd = kFK + 4;    // LDS row stride in floats
constexpr int kFThreads = 256;

// the column tile for N output columns: 96 when it divides N (x_proj's 288), else 128
constexpr int f32_cols(int N) { return N % 96 == 0 ? 96 : 128; }

// Y (+ blockIdx.z * M * N: the K slice's partial sums) over K range [blockIdx.z * kslice, + kslice).
// Requirements (checked by the launcher's callers): K and kslice multiples of 4, 16-byte aligned X and W.
template <bool kSoftplus, int TN>
__global__ __launch_bounds__(kFThreads) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                             const float* __restrict__ bias, float* __restrict__ Y,
                                                             int M, int N, int K, int kslice) {
  constexpr int kWT = TN / 32;                         // 16-column MFMA tiles per wave
  constexpr int kXL = kFM * (kFK / 4) / kFThreads;     // 16-byte X loads per thread per block
  constexpr int kWL = TN * (kFK / 4) / kFThreads;      // 16-byte W loads per thread per block
  static_assert(kXL * kFThreads == kFM * (kFK / 4) && kWL * kFThreads == TN * (kFK / 4), "whole loads");
  __shared__ __attribute__((aligned(16))) float xs[2][kFM * kFLd];
  __shared__ __attribute__((aligned(16))) float ws[2][TN * kFLd];
  const int m0 = blockIdx.x * kFM, n0 = blockIdx.y * TN;
  const int kb = blockIdx.z * kslice, ke = min(K, kb + kslice);
  float* out = Y + (int64_t)blockIdx.z * M * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // loader: 16-byte chunk id = tid + j * 256 of the tile is row id / 8, floats 4 (id % 8) .. + 3; rows past M / N
  // re-read the last row (their products are never stored)
  f32x4 gx[kXL], gw[kWL];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXL; ++j) {
      const int id = tid + j * kFThreads, r = id >> 3, k = k0 + (id & 7) * 4;
      const bool ok = k < ke;   // k and ke are multiples of 4: a 16-byte group is all in or all out
      gx[j] = ok ? *reinterpret_cast<const f32x4*>(X + (int64_t)min(m0 + r, M - 1) * K + k)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
      const int id = tid + j * kFThreads, r = id >> 3, k = k0 + (id & 7) * 4;
      const bool ok = k < ke;
      gw[j] = ok ? *reinterpret_cast<const f32x4*>(W + (int64_t)min(n0 + r, N - 1) * K + k)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXL; ++j) {
      const int id = tid + j * kFThreads;
      *reinterpret_cast<f32x4*>(&xs[buf][(id >> 3) * kFLd + (id & 7) * 4]) = gx[j];
    }
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
      const int id = tid + j * kFThreads;
      *reinterpret_cast<f32x4*>(&ws[buf][(id >> 3) * kFLd + (id & 7) * 4]) = gw[j];
    }
  };

  const int wm = (wave & 1) * 64, wn = (wave >> 1) * (TN / 2);
  const int fr = lane & 15, fg = lane >> 4;
  f32x4 acc[4][kWT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kWT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblk = (ke - kb + kFK - 1) / kFK;
  gload(kb);
  lstore(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int cur = b & 1;
    if (b + 1 < nblk) gload(kb + (b + 1) * kFK);
#pragma unroll
    for (int c = 0; c < kFK / 16; ++c) {
      f32x4 a[4], w[kWT];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const f32x4*>(&xs[cur][(wm + i * 16 + fr) * kFLd + c * 16 + fg * 4]);
#pragma unroll
      for (int j = 0; j < kWT; ++j)
        w[j] = *reinterpret_cast<const f32x4*>(&ws[cur][(wn + j * 16 + fr) * kFLd + c * 16 + fg * 4]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < kWT; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][q], w[j][q], acc[i][j], 0, 0, 0);
    }
    // the other buffer was last read in block b - 1, before the barrier that ended it
    if (b + 1 < nblk) lstore(cur ^ 1);
    __syncthreads();
  }

  // lane l holds rows 4 (l / 16) + r of each 16 x 16 tile at column l % 16: sixteen lanes store 64 contiguous
  // bytes of a row
#pragma unroll
  for (int j = 0; j < kWT; ++j) {
    const int n = n0 + wn + j * 16 + fr;
    if (n >= N) continue;
    const float bn = kSoftplus ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + i * 16 + fg * 4 + r;
        if (m < M) out[(int64_t)m * N + n] = kSoftplus ? softplus(acc[i][j][r] + bn) : acc[i][j][r];
      }
  }
}

template <int TN>
void launch_cols(const float* X, const float* W, const float* bias, float* Y, int M, int N, int K, int splits,
                 hipStream_t st) {
  dim3 grid((M + kFM - 1) / kFM, (N + TN - 1) / TN, splits);
  const int kslice = K / splits;
  if (bias)
    hipLaunchKernelGGL((gemm_f32_kernel<true, TN>), grid, dim3(kFThreads), 0, st, X, W, bias, Y, M, N, K, kslice);
  else
    hipLaunchKernelGGL((gemm_f32_kernel<false, TN>), grid, dim3(kFThreads), 0, st, X, W, nullptr, Y, M, N, K,
                       kslice);
}

}  // namespace

int64_t gemm_f32_tiles(int64_t M, int N) {
  const int tn = f32_cols(N);
  return ((M + kFM - 1) / kFM) * ((N + tn - 1) / tn);
}

void launch_gemm_f32(const float* X, const float* W, const float* bias, float* Y, int M, int N, int K, int splits,
                     hipStream_t st) {
  if (M == 0 || N == 0) return;
  if (f32_cols(N) == 96)
    launch_cols<96>(X, W, bias, Y, M, N, K, splits, st);
  else
    launch_cols<128>(X, W, bias, Y, M, N, K, splits, st);
}

}  // namespace jm
