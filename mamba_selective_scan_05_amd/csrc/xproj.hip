// x_proj: dbc[m, n] = sum_k xc[m, k] * W[n, k]   (M tokens, N = dt_rank + 2*d_state, K = d_inner).
//
// bf16 path: matrix cores (v_mfma_f32_16x16x32_bf16), fp32 accumulation.  A workgroup of 4 waves owns a
// 128-token x 288-column output tile: wave (mg, ng) computes rows [64 mg, 64 mg + 64) x 16-wide column
// tiles [9 ng, 9 ng + 9), so every xc element is read from HBM once and every W_x element once per
// 128 tokens.  With few tokens (decode) the workgroups take 32-column groups instead (one tile per wave),
// which multiplies the grid by 9 without adding partial sums; xc is then re-read from L2 per group.  The
// operands of each 64-wide K block reach LDS by direct global-to-LDS loads in a three-stage pipeline (see
// below).  When there are too few token tiles to fill the GPU, the K range is split over `splits`
// workgroups that write fp32 partial sums (added in a fixed order by the norm step, so the result is
// deterministic).  Split s of token tile t runs as workgroup t * splits + s: workgroups are handed to the
// 8 XCDs round-robin, so each XCD works on a fixed subset of K slices and keeps their W_x rows in its own
// L2.  Wider projections (N > 288) run as several column groups (grid z).
//
// fp32 path: the fp32 matrix-core GEMM of gemm_f32.hip (the fp32 I/O mode must not round xc to bf16), split
// over channel slices like the bf16 path.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

constexpr int kMT = 128;         // tokens per workgroup tile
constexpr int kKB = 64;           // K block staged in LDS (one 128-byte LDS row per token / column)
constexpr int kThreads = 256;
// Column tiles per wave: 9 (a workgroup covers 288 columns) normally; 1 (32 columns, grid z walks the
// column groups) when there are too few token tiles to fill the GPU even with the K range split.
constexpr int kNTWide = 9, kNTNarrow = 1;

__device__ __forceinline__ bf16x8 lds_frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// MFMA 16x16x32 operand layout used here: lane l supplies row (l % 16) of A and column (l % 16) of B,
// both over the 8 consecutive k values 8*(l / 16) .. +7 (the same k set for A and B, so the product is
// independent of how the hardware orders k).  The accumulator holds rows 4*(l / 16) + i, column l % 16.
//
// Operands reach LDS by direct global-to-LDS loads (16 bytes per lane, lane i of an instruction lands at
// byte 16 i of its destination), three K blocks deep: while block b multiplies, blocks b + 1 and b + 2 are
// in flight, with no staging registers.  LDS rows are 128 bytes (64 k) with no padding; 16-byte chunk j of
// row r sits in slot j ^ (r & 7), which makes the fragment reads conflict-free (measured: 12 conflict cycles
// per read without the swizzle, none with it).  A lane loads whichever global chunk belongs in its slot.
constexpr int kStages = 3;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;
__device__ __forceinline__ int swz(int r, int j) { return r * kKB + ((j ^ (r & 7)) << 3); }
// Workgroup barrier without __syncthreads' release fence: that fence would wait for every direct-to-LDS
// load in flight (they count as LDS writes).  Each wave has already waited for the loads of the block it
// hands over; the asm statements keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt operand (gfx9 encoding): vector-memory count n, the other counters at their maxima
__device__ __forceinline__ constexpr int wait_vm(int n) { return ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF); }

template <int kNT>
__global__ __launch_bounds__(kThreads) void xproj_mfma_kernel(const bf16_t* __restrict__ xc,
                                                              const bf16_t* __restrict__ w,
                                                              float* __restrict__ part, int M, int N, int K,
                                                              int splits) {
  constexpr int kNG = 32 * kNT;                               // columns per workgroup
  constexpr int kAL = kMT / 8 / 4;                            // direct loads per wave per block: A rows / 8 / waves
  constexpr int kBL = kNG / 8 / 4;
  // one array per stage, so the compiler can tell the loads in flight into one stage from reads of another
  __shared__ __attribute__((aligned(16))) bf16_t As0[kMT * kKB], As1[kMT * kKB], As2[kMT * kKB];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[kNG * kKB], Bs1[kNG * kKB], Bs2[kNG * kKB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS destinations in SGPRs
  const int s = blockIdx.x % splits;
  const int m0 = (blockIdx.x / splits) * kMT;
  const int n0 = blockIdx.z * kNG;
  const int kps = K / splits;
  const int kbeg = s * kps;
  const int nblocks = kps / kKB;
  const int lr = lane & 15, lk = lane >> 4;
  const int mg = wave & 1, ng = wave >> 1;

  f32x4 acc[4][kNT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Load q of this wave fills LDS rows 8 (wave * count + q) .. + 7; lane l takes row + l / 8, slot l % 8, so
  // it reads the global chunk (l % 8) ^ (row & 7).  Rows past M (tokens) or N (columns) re-read the last
  // valid row: they only feed outputs that are never stored.
  // Addresses are a wave-uniform tile base plus a 32-bit per-lane byte offset (one SGPR base per load).
  const char* abase = reinterpret_cast<const char*>(xc + (int64_t)m0 * K);
  const char* bbase = reinterpret_cast<const char*>(w + (int64_t)n0 * K);
  uint32_t oa[kAL], ob[kBL];
#pragma unroll
  for (int q = 0; q < kAL; ++q) {
    const int row = (wave * kAL + q) * 8 + (lane >> 3);
    oa[q] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
#pragma unroll
  for (int q = 0; q < kBL; ++q) {
    const int row = (wave * kBL + q) * 8 + (lane >> 3);
    ob[q] = (uint32_t)(((int64_t)(min(n0 + row, N - 1) - n0) * K + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
  // block b (past the last one: the last again, into a stage nobody reads) -> stage (A, B).  The W_x rows
  // (L2 hits) are requested before the xc rows (from HBM): measured ~3% faster than the other order.
  auto issue = [&](int b, bf16_t* A, bf16_t* B) {
    const int64_t kb = (int64_t)(kbeg + min(b, nblocks - 1) * kKB) * 2;
#pragma unroll
    for (int q = 0; q < kBL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(bbase + kb + ob[q]),
                                       (lds_void_t*)(B + (wave * kBL + q) * 8 * kKB), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kAL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(abase + kb + oa[q]),
                                       (lds_void_t*)(A + (wave * kAL + q) * 8 * kKB), 16, 0, 0);
  };
  auto compute = [&](const bf16_t* A, const bf16_t* B) {
#pragma unroll
    for (int ks = 0; ks < kKB / 8; ks += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = lds_frag(&A[swz(mg * 64 + r * 16 + lr, ks + lk)]);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const bf16x8 bv = lds_frag(&B[swz((ng * kNT + t) * 16 + lr, ks + lk)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv, acc[r][t], 0, 0, 0);
      }
    }
  };
  // Block b: wait until this thread's loads of block b have landed (block b + 1's may still be in flight),
  // then a barrier (everyone's have, and everyone is done with block b - 1), then refill block b - 1's
  // stage with block b + 2 and multiply block b.  Unrolled by three so every stage index is a constant.
  issue(0, As0, Bs0);
  issue(1, As1, Bs1);
  auto step = [&](int b, const bf16_t* A, const bf16_t* B, bf16_t* An, bf16_t* Bn) {
    __builtin_amdgcn_s_waitcnt(wait_vm(kAL + kBL));
    stage_barrier();
    issue(b + 2, An, Bn);
    compute(A, B);
  };
  for (int b = 0;; b += 3) {
    step(b, As0, Bs0, As2, Bs2);
    if (b + 1 >= nblocks) break;
    step(b + 1, As1, Bs1, As0, Bs0);
    if (b + 2 >= nblocks) break;
    step(b + 2, As2, Bs2, As1, Bs1);
    if (b + 3 >= nblocks) break;
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));   // the surplus loads must land before the workgroup's LDS is reused

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

// Long inputs: 256-token x 288-column tiles per workgroup of 8 waves (wave (mg, ng) computes rows
// [64 mg, 64 mg + 64) x column tiles [9 ng, 9 ng + 9)), so W_x is read once per 256 tokens instead of once per
// 128: the operands reach LDS through the direct global-to-LDS path, whose delivery rate from L2 bounds
// this kernel, and W_x is most of what it delivers (4.7 MB per token tile against 4 MB of xc per 256
// tokens).  Two LDS stages of one 64-wide K block each (144 KB: 32 KB of xc, 40 KB of W_x rows padded to
// 320 so that every wave issues five loads; the padding rows re-read the last row and are never used).
constexpr int kMT2 = 256;
constexpr int kNB2 = 320;          // W_x rows loaded per K block (kNG = 288 used)
constexpr int kThreads2 = 512;

__global__ __launch_bounds__(kThreads2) void xproj_mfma_tall_kernel(const bf16_t* __restrict__ xc,
                                                                    const bf16_t* __restrict__ w,
                                                                    float* __restrict__ part, int M, int N,
                                                                    int K, int splits) {
  constexpr int kNT = kNTWide;
  constexpr int kAL = kMT2 / 8 / 8;   // direct loads per wave per block
  constexpr int kBL = kNB2 / 8 / 8;
  __shared__ __attribute__((aligned(16))) bf16_t As0[kMT2 * kKB], As1[kMT2 * kKB];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[kNB2 * kKB], Bs1[kNB2 * kKB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x % splits;
  const int m0 = (blockIdx.x / splits) * kMT2;
  const int n0 = blockIdx.z * 32 * kNT;
  const int kps = K / splits;
  const int kbeg = s * kps;
  const int nblocks = kps / kKB;
  const int lr = lane & 15, lk = lane >> 4;
  const int mg = wave & 3, ng = wave >> 2;

  f32x4 acc[4][kNT];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const char* abase = reinterpret_cast<const char*>(xc + (int64_t)m0 * K);
  const char* bbase = reinterpret_cast<const char*>(w + (int64_t)n0 * K);
  uint32_t oa[kAL], ob[kBL];
#pragma unroll
  for (int q = 0; q < kAL; ++q) {
    const int row = (wave * kAL + q) * 8 + (lane >> 3);
    oa[q] = (uint32_t)(((int64_t)(min(m0 + row, M - 1) - m0) * K + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
#pragma unroll
  for (int q = 0; q < kBL; ++q) {
    const int row = (wave * kBL + q) * 8 + (lane >> 3);
    ob[q] = (uint32_t)(((int64_t)(min(n0 + row, N - 1) - n0) * K + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
  auto issue = [&](int b, bf16_t* A, bf16_t* B) {
    const int64_t kb = (int64_t)(kbeg + min(b, nblocks - 1) * kKB) * 2;
#pragma unroll
    for (int q = 0; q < kBL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(bbase + kb + ob[q]),
                                       (lds_void_t*)(B + (wave * kBL + q) * 8 * kKB), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kAL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(abase + kb + oa[q]),
                                       (lds_void_t*)(A + (wave * kAL + q) * 8 * kKB), 16, 0, 0);
  };
  auto compute = [&](const bf16_t* A, const bf16_t* B) {
#pragma unroll
    for (int ks = 0; ks < kKB / 8; ks += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = lds_frag(&A[swz(mg * 64 + r * 16 + lr, ks + lk)]);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const bf16x8 bv = lds_frag(&B[swz((ng * kNT + t) * 16 + lr, ks + lk)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv, acc[r][t], 0, 0, 0);
      }
    }
  };
  // Block b: wait for this thread's loads of block b, barrier (everyone's have landed, and everyone is done
  // with block b - 1), refill block b - 1's stage with block b + 1, multiply block b.
  issue(0, As0, Bs0);
  auto step = [&](int b, const bf16_t* A, const bf16_t* B, bf16_t* An, bf16_t* Bn) {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    stage_barrier();
    issue(b + 1, An, Bn);
    compute(A, B);
  };
  for (int b = 0;; b += 2) {
    step(b, As0, Bs0, As1, Bs1);
    if (b + 1 >= nblocks) break;
    step(b + 1, As1, Bs1, As0, Bs0);
    if (b + 2 >= nblocks) break;
  }
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

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

}  // namespace

int xproj_token_tile(bool tall) { return tall ? kMT2 : kMT; }

int xproj_column_groups(int N, bool narrow) {
  const int cols = 32 * (narrow ? kNTNarrow : kNTWide);
  return (N + cols - 1) / cols;
}

void launch_xproj(bool bf16, const void* xc, const void* w, float* part, int M, int N, int K, int splits,
                  bool narrow, hipStream_t st, bool tall) {
  if (M == 0) return;
  if (bf16 && tall) {
    dim3 grid(((M + kMT2 - 1) / kMT2) * splits, 1, xproj_column_groups(N, false));
    hipLaunchKernelGGL(xproj_mfma_tall_kernel, grid, dim3(kThreads2), 0, st, (const bf16_t*)xc, (const bf16_t*)w,
                       part, M, N, K, splits);
    return;
  }
  if (bf16) {
    dim3 grid(((M + kMT - 1) / kMT) * splits, 1, xproj_column_groups(N, narrow));
    if (narrow)
      hipLaunchKernelGGL(xproj_mfma_kernel<kNTNarrow>, grid, dim3(kThreads), 0, st, (const bf16_t*)xc,
                         (const bf16_t*)w, part, M, N, K, splits);
    else
      hipLaunchKernelGGL(xproj_mfma_kernel<kNTWide>, grid, dim3(kThreads), 0, st, (const bf16_t*)xc,
                         (const bf16_t*)w, part, M, N, K, splits);
  } else {
    launch_gemm_f32((const float*)xc, (const float*)w, nullptr, part, M, N, K, splits, st);
  }
}

}  // namespace jm
