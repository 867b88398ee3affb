// The fp32 I/O mode's two contractions on the matrix cores (v_mfma_f32_16x16x4_f32: fp32 products, fp32 sums):
//   x_proj   part[s, m, n] = sum over channel slice s of xc[m, k] * w[n, k]   (the norm step adds the slices)
//   dt_proj  delta[m, n]   = softplus(sum_k dln[m, k] * w[n, k] + b[n])
// (TransformerLens "supported_architectures.jamba", the Mamba-1 mixer: x_proj to dt / B / C, then dt_proj with
// its bias and softplus.)  Both are Y = X W^T with K contiguous in both operands.
//
// A workgroup of 4 waves owns a 64 x 64 tile of Y, each wave 32 x 32 (2 x 2 MFMA tiles).  32-wide K blocks of X
// and W pass through double-buffered LDS, the next block's global loads in flight in registers while the
// current block multiplies; one barrier per block.  The MFMA's K slot of lane group g = lane / 16 takes K index
// 4g + q of a 16-wide chunk at step q (any assignment works as long as both operands use the same one), so a
// lane reads its A and B fragments of four steps as one 16-byte LDS load; rows are padded by 16 bytes, which
// spreads the 16 rows of a fragment read over distinct banks.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {


constexpr int kFT = 64;          // rows of X and of W per tile
constexpr int kFK = 32;          // K block
constexpr int kFLd = kFK + 4;    // LDS row stride in floats

// Y (+ blockIdx.z * M * N: the K slice's partial sums) over K range [blockIdx.z * kslice, + kslice).
// Requirements (checked by the launcher's callers): K and kslice multiples of 4, 16-byte aligned X and W.
template <bool kSoftplus>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X, const float* __restrict__ W,
                                                       const float* __restrict__ bias, float* __restrict__ Y,
                                                       int M, int N, int K, int kslice) {
  __shared__ __attribute__((aligned(16))) float xs[2][kFT * kFLd];
  __shared__ __attribute__((aligned(16))) float ws[2][kFT * kFLd];
  const int m0 = blockIdx.x * kFT, n0 = blockIdx.y * kFT;
  const int kb = blockIdx.z * kslice, ke = min(K, kb + kslice);
  float* out = Y + (int64_t)blockIdx.z * M * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // loader: thread t moves 8 floats of row t / 4 (32 contiguous bytes; four threads cover a 128-byte row);
  // rows past M / N re-read the last row (their products are never stored)
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const float* xp = X + (int64_t)min(m0 + lr, M - 1) * K;
  const float* wp = W + (int64_t)min(n0 + lr, N - 1) * K;
  f32x4 gx[2], gw[2];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k = k0 + lk + 4 * j;
      const bool ok = k < ke;   // k and ke are multiples of 4: a 16-byte group is all in or all out
      gx[j] = ok ? *reinterpret_cast<const f32x4*>(xp + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      gw[j] = ok ? *reinterpret_cast<const f32x4*>(wp + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    f32x4* x = reinterpret_cast<f32x4*>(&xs[buf][lr * kFLd + lk]);
    f32x4* w = reinterpret_cast<f32x4*>(&ws[buf][lr * kFLd + lk]);
    x[0] = gx[0];
    x[1] = gx[1];
    w[0] = gw[0];
    w[1] = gw[1];
  };

  const int wm = (wave & 1) * 32, wn = (wave >> 1) * 32;
  const int fr = lane & 15, fg = lane >> 4;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nblk = (ke - kb + kFK - 1) / kFK;
  gload(kb);
  lstore(0);
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int cur = b & 1;
    if (b + 1 < nblk) gload(kb + (b + 1) * kFK);
#pragma unroll
    for (int c = 0; c < kFK / 16; ++c) {
      f32x4 a[2], w[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const f32x4*>(&xs[cur][(wm + i * 16 + fr) * kFLd + c * 16 + fg * 4]);
        w[i] = *reinterpret_cast<const f32x4*>(&ws[cur][(wn + i * 16 + fr) * kFLd + c * 16 + fg * 4]);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][q], w[j][q], acc[i][j], 0, 0, 0);
    }
    // the other buffer was last read in block b - 1, before the barrier that ended it
    if (b + 1 < nblk) lstore(cur ^ 1);
    __syncthreads();
  }

  // lane l holds rows 4 (l / 16) + r of each 16 x 16 tile at column l % 16: sixteen lanes store 64 contiguous
  // bytes of a row
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + j * 16 + fr;
      if (n >= N) continue;
      const float bn = kSoftplus ? bias[n] : 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm + i * 16 + fg * 4 + r;
        if (m < M) out[(int64_t)m * N + n] = kSoftplus ? softplus(acc[i][j][r] + bn) : acc[i][j][r];
      }
    }
}

}  // namespace

int64_t gemm_f32_tiles(int64_t M, int N) { return ((M + kFT - 1) / kFT) * ((N + kFT - 1) / kFT); }

void launch_gemm_f32(const float* X, const float* W, const float* bias, float* Y, int M, int N, int K, int splits,
                     hipStream_t st) {
  if (M == 0 || N == 0) return;
  dim3 grid((M + kFT - 1) / kFT, (N + kFT - 1) / kFT, splits);
  const int kslice = K / splits;
  if (bias)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, dim3(256), 0, st, X, W, bias, Y, M, N, K, kslice);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, dim3(256), 0, st, X, W, nullptr, Y, M, N, K, kslice);
}

}  // namespace jm
