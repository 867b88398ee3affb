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

// The plain prefill at the tall layout's lengths: the causal conv1d + SiLU computed inside x_proj.  Each
// 64-channel K block of the raw input x reaches LDS by the same direct loads as xc would, with 8 rows of left
// context above the 256-token tile, and the block's conv weights and biases beside it.  The workgroup then
// runs the conv in place: every thread keeps the 3 rows above its 4 rows x 8 channels in registers, all
// threads meet at a barrier, and each converts its own rows in registers and writes the SiLU outputs over
// them; the block is then multiplied as if xc had been loaded, and its rows go to xc (the scan reads xc) one
// block later, just before the stage is refilled.  x is read from HBM once and xc written once; the separate
// conv pass and x_proj's read of xc are gone.  The arithmetic per element is conv_silu_kernel's (the same FMA order and SiLU, rounded once to
// bf16), so xc matches it bit for bit.  The first 3 tokens of every sequence, whose left context is the conv
// state, are computed beforehand by the conv kernel itself (launch_conv_xproj) and copied in from xc.
constexpr int kHalo = 8;              // left-context rows staged above the tile (3 used; one whole load group)
constexpr int kAR = kHalo + kMT2;     // staged x rows per K block

__global__ __launch_bounds__(kThreads2) void conv_xproj_tall_kernel(
    const bf16_t* __restrict__ x, int64_t xs, const bf16_t* __restrict__ conv_w, const bf16_t* __restrict__ conv_b,
    bf16_t* __restrict__ xc, const bf16_t* __restrict__ w,
    float* __restrict__ part, int M, int N, int K, int splits, int L) {
  constexpr int kNT = kNTWide;
  constexpr int kAL = kMT2 / 8 / 8;   // direct loads of 8 tile rows per wave per block (wave 0 adds the halo)
  constexpr int kBL = kNB2 / 8 / 8;
  __shared__ __attribute__((aligned(16))) bf16_t As0[kAR * kKB], As1[kAR * kKB];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[kNB2 * kKB], Bs1[kNB2 * kKB];
  // per block: the 64 channels' taps (4 bf16 each, bytes 0..511), their biases (bytes 512..639), filler
  __shared__ __attribute__((aligned(16))) uint32_t Ps0[256], Ps1[256];
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

  // staged row slot r holds token m0 - kHalo + r, clamped to [0, M): rows outside are never used (a tile row
  // fewer than 3 positions into its sequence reads the conv state instead, and rows past M are not stored)
  const int rbase = m0 >= kHalo ? m0 - kHalo : 0;
  const char* abase = reinterpret_cast<const char*>(x + (int64_t)rbase * xs);
  const char* bbase = reinterpret_cast<const char*>(w + (int64_t)n0 * K);
  auto aoff = [&](int slot) {
    const int tok = min(max(m0 - kHalo + slot, 0), M - 1);
    return (uint32_t)(((int64_t)(tok - rbase) * xs + (((lane & 7) ^ (slot & 7)) << 3)) * 2);
  };
  uint32_t oa[kAL], ob[kBL];
#pragma unroll
  for (int q = 0; q < kAL; ++q) oa[q] = aoff((1 + wave * kAL + q) * 8 + (lane >> 3));
  const uint32_t oh = aoff(lane >> 3);
#pragma unroll
  for (int q = 0; q < kBL; ++q) {
    const int row = (wave * kBL + q) * 8 + (lane >> 3);
    ob[q] = (uint32_t)(((int64_t)(min(n0 + row, N - 1) - n0) * K + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
  // conv parameters: lanes 0..31 bring two channels' taps each, lanes 32..39 eight biases each (without a
  // bias, the taps of lanes 0..7 again), lanes 40..63 the taps of lanes 8..31 again (filler, never read)
  const bool has_bias = conv_b != nullptr;
  const char* pbase = lane >= 32 && lane < 40 && has_bias
                          ? reinterpret_cast<const char*>(conv_b) + (int64_t)(lane - 32) * 16
                          : reinterpret_cast<const char*>(conv_w) + (int64_t)(lane & 31) * 16;
  const int pscale = lane >= 32 && lane < 40 && has_bias ? 2 : 8;   // bytes per channel in the source
  auto issue = [&](int b, bf16_t* A, bf16_t* B, uint32_t* P) {
    const int64_t kc = kbeg + min(b, nblocks - 1) * kKB;   // first channel of the block
    const int64_t kb = kc * 2;
#pragma unroll
    for (int q = 0; q < kBL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(bbase + kb + ob[q]),
                                       (lds_void_t*)(B + (wave * kBL + q) * 8 * kKB), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kAL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(abase + kb + oa[q]),
                                       (lds_void_t*)(A + (1 + wave * kAL + q) * 8 * kKB), 16, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_global_load_lds((global_void_t*)(abase + kb + oh), (lds_void_t*)A, 16, 0, 0);
    if (wave == 1)
      __builtin_amdgcn_global_load_lds((global_void_t*)(pbase + kc * pscale), (lds_void_t*)P, 16, 0, 0);
  };
  auto compute = [&](const bf16_t* A, const bf16_t* B) {
#pragma unroll
    for (int ks = 0; ks < kKB / 8; ks += 4) {
      bf16x8 a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = lds_frag(&A[swz(kHalo + mg * 64 + r * 16 + lr, ks + lk)]);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const bf16x8 bv = lds_frag(&B[swz((ng * kNT + t) * 16 + lr, ks + lk)]);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv, acc[r][t], 0, 0, 0);
      }
    }
  };

  // conv roles: thread (g, j) computes tile rows 4g .. 4g+3 of channels 8j .. 8j+7 of each block
  const int cj = tid & 7, cg = tid >> 3;
  bool edge = false;   // one of the rows is fewer than 3 positions into its sequence
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = m0 + 4 * cg + i;
    edge = edge || (t < M && t % L < 3);
  }
  // uint32 index of (row slot r, 16-byte chunk cj) in a staged block
  auto widx = [&](int r) { return r * (kKB / 2) + ((cj ^ (r & 7)) << 2); };
  auto lo = [](uint32_t v) { return __uint_as_float(v << 16); };
  auto hi = [](uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); };
  auto conv = [&](int b, bf16_t* A, const uint32_t* P) {
    const int c0 = kbeg + b * kKB + cj * 8;   // the thread's first channel
    uint32_t* A32 = reinterpret_cast<uint32_t*>(A);
    // the three rows above the thread's group belong to the group above, which overwrites them: they are
    // read before the barrier; after it every thread rewrites only its own rows
    uint4 up[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) up[k] = *reinterpret_cast<const uint4*>(&A32[widx(kHalo + 4 * cg - 3 + k)]);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    stage_barrier();
    auto dw = [](const uint4& v, int d) { return d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w; };
    auto set_dw = [](uint4& v, int d, uint32_t x) {
      if (d == 0) v.x = x;
      else if (d == 1) v.y = x;
      else if (d == 2) v.z = x;
      else v.w = x;
    };
    // the SiLU outputs of channels c0 + 2d, c0 + 2d + 1 for one row, given its four inputs per channel
    auto conv2 = [&](int d, const float (&in)[2][4]) __attribute__((always_inline)) {
      const uint4 wv = *reinterpret_cast<const uint4*>(&P[(cj * 8 + 2 * d) * 2]);
      const uint32_t bv = P[128 + cj * 4 + d];
      const float wt[2][4] = {{lo(wv.x), hi(wv.x), lo(wv.y), hi(wv.y)}, {lo(wv.z), hi(wv.z), lo(wv.w), hi(wv.w)}};
      float o[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        float u = has_bias ? (e == 0 ? lo(bv) : hi(bv)) : 0.0f;
        u = fmaf(wt[e][0], in[e][0], u);
        u = fmaf(wt[e][1], in[e][1], u);
        u = fmaf(wt[e][2], in[e][2], u);
        u = fmaf(wt[e][3], in[e][3], u);
        o[e] = silu(u);
      }
      return f2bf2(o[0], o[1]);
    };
    // the own rows as whole 16-byte chunks (8 lanes cover a row: no bank conflicts; per-dword accesses put
    // the 64 lanes on 8 banks), converted in registers from the last row up: each output replaces an input
    // that no row still to be converted reads
    uint4 own[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) own[i] = *reinterpret_cast<const uint4*>(&A32[widx(kHalo + 4 * cg + i)]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {   // channels c0 + 2d, c0 + 2d + 1 (one dword of each row)
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        auto src = [&](int j) { return j < 3 ? dw(up[j], d) : dw(own[j - 3], d); };   // input i - 3 + k
        const float in[2][4] = {{lo(src(i)), lo(src(i + 1)), lo(src(i + 2)), lo(src(i + 3))},
                                {hi(src(i)), hi(src(i + 1)), hi(src(i + 2)), hi(src(i + 3))}};
        set_dw(own[i], d, conv2(d, in));
      }
      __builtin_amdgcn_sched_barrier(0);   // one channel pair at a time: bounded register use
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&A32[widx(kHalo + 4 * cg + i)]) = own[i];
    if (edge) {
      // a row fewer than 3 positions into its sequence needs its conv state as left context: launch_conv_xproj
      // has already written those rows of xc (with the conv kernel itself); they replace what was computed
      // here from the rows above
      __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = m0 + 4 * cg + i;
        if (t < M && t % L < 3)
          *reinterpret_cast<uint4*>(&A32[widx(kHalo + 4 * cg + i)]) =
              *reinterpret_cast<const uint4*>(xc + (int64_t)t * K + c0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // the outputs are in LDS before the matrix cores read them
    stage_barrier();
  };
  // xc rows of block b for the scan: the thread's own rows, read back whole from the block's stage.  This runs
  // one step later, just before the stage is refilled: the rows wave w reads back are exactly those its own
  // direct loads refill (tile rows 32w .. 32w + 31), so waiting for the reads is the only ordering needed,
  // and the stores are not waited for until the step after (waiting for them at once, together with the
  // next block's loads, exposed their latency every block).
  const bool writes_xc = blockIdx.z == 0;   // other column groups compute the same rows
  auto store_xc = [&](int b, const bf16_t* A) {
    __builtin_amdgcn_sched_barrier(0);
    const int c0 = kbeg + b * kKB + cj * 8;
    const uint32_t* A32 = reinterpret_cast<const uint32_t*>(A);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = m0 + 4 * cg + i;
      const uint4 v = *reinterpret_cast<const uint4*>(&A32[widx(kHalo + 4 * cg + i)]);
      if (writes_xc && t < M) *reinterpret_cast<uint4*>(xc + (int64_t)t * K + c0) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // read back before the refill lands
    __builtin_amdgcn_sched_barrier(0);
  };

  // Block b: wait for this thread's loads of block b, barrier (everyone's have landed, and everyone is done
  // with block b - 1), store block b - 1's xc rows and refill its stage with block b + 1, conv block b in
  // place, multiply it.
  issue(0, As0, Bs0, Ps0);
  auto step = [&](int b, bf16_t* A, const bf16_t* B, const uint32_t* P, bf16_t* An, bf16_t* Bn, uint32_t* Pn) {
    __builtin_amdgcn_s_waitcnt(wait_vm(0));
    stage_barrier();
    if (b > 0) store_xc(b - 1, An);
    issue(b + 1, An, Bn, Pn);
    conv(b, A, P);
    compute(A, B);
  };
  for (int b = 0;; b += 2) {
    step(b, As0, Bs0, Ps0, As1, Bs1, Ps1);
    if (b + 1 >= nblocks) break;
    step(b + 1, As1, Bs1, Ps1, As0, Bs0, Ps0);
    if (b + 2 >= nblocks) break;
  }
  store_xc(nblocks - 1, (nblocks - 1) & 1 ? As1 : As0);
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

bool conv_xproj_fits(int64_t x_stride) {
  // the staged rows of a tile lie within 32-bit byte offsets of the tile's first row
  return (int64_t)(kAR - 1) * x_stride * 2 + 2 * kKB < ((int64_t)1 << 32);
}

void launch_conv_xproj(const void* x, int64_t x_stride, const void* conv_w, const void* conv_b, const void* conv_in,
                       void* xc, const void* w, float* part, int B, int L, int N, int K, int splits, hipStream_t st) {
  const int M = B * L;
  if (M == 0) return;
  // the first 3 tokens of every sequence (their left context is the conv state): the conv kernel, first
  launch_conv_head(true, x, x_stride, conv_w, conv_b, conv_in, xc, B, L, K, st);
  dim3 grid(((M + kMT2 - 1) / kMT2) * splits, 1, xproj_column_groups(N, false));
  hipLaunchKernelGGL(conv_xproj_tall_kernel, grid, dim3(kThreads2), 0, st, (const bf16_t*)x, x_stride,
                     (const bf16_t*)conv_w, (const bf16_t*)conv_b, (bf16_t*)xc, (const bf16_t*)w, part, M, N, K,
                     splits, L);
}

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
