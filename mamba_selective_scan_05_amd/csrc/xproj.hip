// x_proj: dbc[m, n] = sum_k xc[m, k] * W[n, k]   (M tokens, N = dt_rank + 2*d_state, K = d_inner).
//
// bf16 path: matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.  A workgroup of 4 waves owns a
// 128-token x 288-column output tile: wave (mg, ng) computes rows [64 mg, 64 mg + 64) x 16-wide column
// tiles [9 ng, 9 ng + 9), so every xc element is read from HBM once and every W_x element once per
// 128 tokens.  With few tokens (decode) the workgroups take 32-column groups instead (one tile per wave),
// which multiplies the grid by 9 without adding partial sums; xc is then re-read from L2 per group.  Both
// operands of each 64-wide K block are staged through LDS (double-buffered, rows padded by 32 bytes against
// bank conflicts); the next block's global loads are in flight while the
// current block's MFMAs run.  When there are too few token tiles to fill the GPU, the K range is split
// over `splits` workgroups that write fp32 partial sums (added in a fixed order by the norm step, so the
// result is deterministic).  Split s of token tile t runs as workgroup t * splits + s: workgroups are
// handed to the 8 XCDs round-robin, so each XCD works on a fixed subset of K slices and keeps their
// W_x rows in its own L2.  Wider projections (N > 288) run as several column groups (grid z).
//
// fp32 path: plain fp32 dot products on the vector ALU (the fp32 I/O mode must not round xc to bf16).
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
// 16 bytes in registers as a native vector (HIP's uint4 class does not always stay in registers when copied)
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kMT = 128;         // tokens per workgroup tile
constexpr int kKB = 64;           // K block staged in LDS
constexpr int kLd = kKB + 16;     // padded LDS row, bf16 elements (32 bytes of pad: conflict-free 16-byte fragment reads)
constexpr int kThreads = 256;
constexpr int kAChunks = kMT * (kKB / 8) / kThreads;   // 16-byte chunks per thread: 4
// Column tiles per wave: 9 (a workgroup covers 288 columns) normally; 1 (32 columns, grid z walks the
// column groups) when there are too few token tiles to fill the GPU even with the K range split.
constexpr int kNTWide = 9, kNTNarrow = 1;

__device__ __forceinline__ bf16x8 lds_frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// MFMA 16x16x32 operand layout used here: lane l supplies row (l % 16) of A and column (l % 16) of B,
// both over the 8 consecutive k values 8*(l / 16) .. +7 (the same k set for A and B, so the product is
// independent of how the hardware orders k).  The accumulator holds rows 4*(l / 16) + i, column l % 16.
template <int kNT>
__global__ __launch_bounds__(kThreads) void xproj_mfma_kernel(const bf16_t* __restrict__ xc,
                                                              const bf16_t* __restrict__ w,
                                                              float* __restrict__ part, int M, int N, int K,
                                                              int splits) {
  constexpr int kNG = 32 * kNT;                               // columns per workgroup
  constexpr int kBChunks = kNG * (kKB / 8) / kThreads;        // 16-byte W_x chunks per thread
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kMT * kLd];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kNG * kLd];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int s = blockIdx.x % splits;
  const int m0 = (blockIdx.x / splits) * kMT;
  const int n0 = blockIdx.z * kNG;
  const int kps = K / splits;
  const int kbeg = s * kps;
  const int nblocks = kps / kKB;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int mg = wave & 1, ng = wave >> 1;

  f32x4 acc[4][kNT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // xc (from HBM) is loaded two K blocks ahead, W_x (from L2) one block ahead.  Rows past M (tokens) or
  // N (columns) are clamped to the last valid row: they only feed outputs that are never stored, and
  // branch-free loads let the memory counter be waited on precisely.
  // Per-thread chunk addresses: chunk q of a block is row (tid + q * 256) / 8, k offset ((tid + q*256) % 8)*8.
  const int kc = (tid & 7) * 8;
  const bf16_t* pa[kAChunks];
  const bf16_t* pb[kBChunks];
  int la[kAChunks], lb[kBChunks];
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) {
    const int row = (tid >> 3) + q * (kThreads / 8);
    pa[q] = xc + (int64_t)min(m0 + row, M - 1) * K + kc;
    la[q] = row * kLd + kc;
  }
#pragma unroll
  for (int q = 0; q < kBChunks; ++q) {
    const int row = (tid >> 3) + q * (kThreads / 8);
    pb[q] = w + (int64_t)min(n0 + row, N - 1) * K + kc;
    lb[q] = row * kLd + kc;
  }
  // K blocks go in pairs (even block from LDS buffer 0, odd from buffer 1) with two register sets for xc
  // (X, Y), so a prefetched block never has to be copied between registers.  While block b computes:
  // W_x of b + 1 and xc of b + 2 are requested (W_x first: the memory counter drains in issue order, so
  // the LDS store at the end of the block waits for W_x and the older xc only); afterwards xc of b + 1
  // (already in registers) and W_x of b + 1 go to the other LDS buffer.  Loads past the last block re-read
  // it, and the LDS stores are unconditional (the last one fills the idle buffer): conditional loads or
  // stores would let the compiler sink the loads past the MFMAs.
  u32x4 rx[kAChunks], ry[kAChunks], rb[kBChunks];
  auto blk = [&](int b) { return kbeg + min(b, nblocks - 1) * kKB; };
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) ry[q] = *reinterpret_cast<const u32x4*>(pa[q] + blk(0));
#pragma unroll
  for (int q = 0; q < kBChunks; ++q) rb[q] = *reinterpret_cast<const u32x4*>(pb[q] + blk(0));
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) rx[q] = *reinterpret_cast<const u32x4*>(pa[q] + blk(1));
#pragma unroll
  for (int q = 0; q < kAChunks; ++q) *reinterpret_cast<u32x4*>(&As[0][la[q]]) = ry[q];
#pragma unroll
  for (int q = 0; q < kBChunks; ++q) *reinterpret_cast<u32x4*>(&Bs[0][lb[q]]) = rb[q];
  __syncthreads();

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kKB; ks += 32) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = lds_frag(&As[buf][(mg * 64 + r * 16 + lr) * kLd + ks + lk]);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const bf16x8 bv = lds_frag(&Bs[buf][((ng * kNT + t) * 16 + lr) * kLd + ks + lk]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv, acc[r][t], 0, 0, 0);
      }
    }
  };

  for (int ib = 0; ib < nblocks; ib += 2) {
    // even block ib (buffer 0); rx holds xc of ib + 1
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) rb[q] = *reinterpret_cast<const u32x4*>(pb[q] + blk(ib + 1));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kAChunks; ++q) ry[q] = *reinterpret_cast<const u32x4*>(pa[q] + blk(ib + 2));
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
#pragma unroll
    for (int q = 0; q < kAChunks; ++q) *reinterpret_cast<u32x4*>(&As[1][la[q]]) = rx[q];
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) *reinterpret_cast<u32x4*>(&Bs[1][lb[q]]) = rb[q];
    __syncthreads();
    if (ib + 1 >= nblocks) break;
    // odd block ib + 1 (buffer 1); ry holds xc of ib + 2
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) rb[q] = *reinterpret_cast<const u32x4*>(pb[q] + blk(ib + 2));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < kAChunks; ++q) rx[q] = *reinterpret_cast<const u32x4*>(pa[q] + blk(ib + 3));
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
#pragma unroll
    for (int q = 0; q < kAChunks; ++q) *reinterpret_cast<u32x4*>(&As[0][la[q]]) = ry[q];
#pragma unroll
    for (int q = 0; q < kBChunks; ++q) *reinterpret_cast<u32x4*>(&Bs[0][lb[q]]) = rb[q];
    __syncthreads();
  }

  float* dst = part + (int64_t)s * M * N;
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    const int n = n0 + (ng * kNT + t) * 16 + lr;
    if (n >= N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mg * 64 + r * 16 + (lane >> 4) * 4 + i;
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

int xproj_token_tile() { return kMT; }

int xproj_column_groups(int N, bool narrow) {
  const int cols = 32 * (narrow ? kNTNarrow : kNTWide);
  return (N + cols - 1) / cols;
}

void launch_xproj(bool bf16, const void* xc, const void* w, float* part, int M, int N, int K, int splits,
                  bool narrow, hipStream_t st) {
  if (M == 0) return;
  if (bf16) {
    dim3 grid(((M + kMT - 1) / kMT) * splits, 1, xproj_column_groups(N, narrow));
    if (narrow)
      hipLaunchKernelGGL(xproj_mfma_kernel<kNTNarrow>, grid, dim3(kThreads), 0, st, (const bf16_t*)xc,
                         (const bf16_t*)w, part, M, N, K, splits);
    else
      hipLaunchKernelGGL(xproj_mfma_kernel<kNTWide>, grid, dim3(kThreads), 0, st, (const bf16_t*)xc,
                         (const bf16_t*)w, part, M, N, K, splits);
  } else {
    dim3 grid(M, (N + 63) / 64);
    hipLaunchKernelGGL(xproj_f32_kernel, grid, dim3(64), 0, st, (const float*)xc, (const float*)w, part, M, N, K);
  }
}

}  // namespace jm
