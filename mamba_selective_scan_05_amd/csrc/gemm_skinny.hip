// The whole layer's projections for a decode-sized batch (at most 256 tokens): Y[m, n] = sum_k X[m, k] W[n, k]
// (+ R[m, n]), bf16 operands and result, fp32 accumulation on the matrix cores (v_mfma_f32_16x16x32_bf16).
//
// With so few tokens the product is bound by streaming W (in_proj 4096 x 16384, out_proj 8192 x 4096 at
// Jamba v0.1's widths: 201 MB together), so the layout is chosen for W: a workgroup owns one 64-column block
// of W (64 rows of the [N, K] weight) for every token, over a slice of K, and W's bytes are read from HBM
// exactly once.  X (at most 256 x K, a few MB) is read by every workgroup and stays in the L2 caches.  Both
// operands reach LDS through direct global-to-LDS loads in a three-stage pipeline with the swizzled
// 128-byte rows of the x_proj kernel (16-byte chunk j of row r in slot j ^ (r & 7)).  Each wave computes
// 64 tokens x 64 columns: four waves for a 64-column block, eight for a 128-column block.  When the column
// blocks alone leave the GPU short of workgroups (out_proj: 64 of them) the K range is split and fp32 partial
// sums are added in split order by a second kernel, which also adds the residual; the result does not depend
// on timing.
//
// What bounds it is the rate at which L2 delivers X to the CUs (every workgroup re-reads X over its K slice:
// for in_proj with 64-column blocks 512 MB of X against 134 MB of W).  Whenever 128-column blocks still give a
// workgroup per CU over whole K slices, the workgroups take 128 columns: half the X re-reads of 64-column
// blocks, for splits x M x N x 4 bytes of partial sums.  256-column blocks (sixteen waves; two LDS stages of
// 64 KB, since three do not fit) measured slower at Jamba's widths: in_proj 49-54 against 44.6 us, out_proj
// 30 against 27.4 us, with twice the partial sums to add (one stage in flight does not hide the delivery).
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_void_t;

constexpr int kGM = 256;       // tokens per workgroup (the whole batch)
constexpr int kGK = 64;        // K block staged in LDS

__device__ __forceinline__ int gswz(int r, int j) { return r * kGK + ((j ^ (r & 7)) << 3); }
__device__ __forceinline__ bf16x8 gfrag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
// barrier without __syncthreads' release fence (it would wait for every direct-to-LDS load in flight)
__device__ __forceinline__ void gbarrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ constexpr int gwait_vm(int n) {
  return ((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 0xF);
}

// Workgroup w computes column block w / splits (GN columns) over K slice w % splits.  PARTIAL: fp32 partial
// sums to part[s, m, n]; otherwise bf16(acc + R) to Y.  Wave v: tokens 64 (v % 4) .., columns 64 (v / 4) ..
template <bool PARTIAL, int GN>
__global__ __launch_bounds__(GN * 4) void skinny_gemm_kernel(const bf16_t* __restrict__ X, int64_t ldx,
                                                             const bf16_t* __restrict__ W, int64_t ldw,
                                                             const bf16_t* R, int64_t ldr, bf16_t* Y,
                                                             int64_t ldy, float* __restrict__ part, int M,
                                                             int N, int K, int splits) {
  constexpr int kWaves = GN / 16;
  constexpr int kGAL = kGM / 8 / kWaves;   // direct loads per wave per block: X rows / 8 per load / waves
  constexpr int kGBL = GN / 8 / kWaves;    // W rows / 8 / waves
  static_assert(kGAL * 8 * kWaves == kGM && kGBL * 8 * kWaves == GN, "whole loads per wave");
  __shared__ __attribute__((aligned(16))) bf16_t As0[kGM * kGK], As1[kGM * kGK], As2[kGM * kGK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs0[GN * kGK], Bs1[GN * kGK], Bs2[GN * kGK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;   // the wave's 64 tokens and 64 columns
  const int s = blockIdx.x % splits;
  const int n0 = (blockIdx.x / splits) * GN;
  const int kps = K / splits;
  const int kbeg = s * kps;
  const int nblocks = kps / kGK;
  const int lr = lane & 15, lk = lane >> 4;
  // each workgroup starts at another K block (X is read by every workgroup; spreading the reads over X
  // measured ~4 us faster for the B = 256 layer decode step)
  const int rot = (int)((blockIdx.x * 7u) % (unsigned)nblocks);

  f32x4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Load q of a wave fills 8 LDS rows; lane l takes row + l / 8, slot l % 8, i.e. global chunk
  // (l % 8) ^ (row & 7).  X rows past M re-read row M - 1 (they feed outputs that are never stored).
  const char* xb = reinterpret_cast<const char*>(X);
  const char* wb = reinterpret_cast<const char*>(W + (int64_t)n0 * ldw);
  uint32_t ox[kGAL], ow[kGBL];
#pragma unroll
  for (int q = 0; q < kGAL; ++q) {
    const int row = (wave * kGAL + q) * 8 + (lane >> 3);
    ox[q] = (uint32_t)(((int64_t)min(row, M - 1) * ldx + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
#pragma unroll
  for (int q = 0; q < kGBL; ++q) {
    const int row = (wave * kGBL + q) * 8 + (lane >> 3);
    ow[q] = (uint32_t)(((int64_t)row * ldw + (((lane & 7) ^ (row & 7)) << 3)) * 2);
  }
  // block b (past the last one: the last again, into a stage nobody reads).  W (from HBM) is requested
  // before X (from L2).
  auto issue = [&](int b, bf16_t* A, bf16_t* B) {
    const int bb = min(b, nblocks - 1) + rot;
    const int64_t kb = (int64_t)(kbeg + (bb >= nblocks ? bb - nblocks : bb) * kGK) * 2;
#pragma unroll
    for (int q = 0; q < kGBL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(wb + kb + ow[q]),
                                       (lds_void_t*)(B + (wave * kGBL + q) * 8 * kGK), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < kGAL; ++q)
      __builtin_amdgcn_global_load_lds((global_void_t*)(xb + kb + ox[q]),
                                       (lds_void_t*)(A + (wave * kGAL + q) * 8 * kGK), 16, 0, 0);
  };
  auto compute = [&](const bf16_t* A, const bf16_t* B) {
#pragma unroll
    for (int ks = 0; ks < kGK / 8; ks += 4) {
      bf16x8 a[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = gfrag(&A[gswz(wm * 64 + r * 16 + lr, ks + lk)]);
#pragma unroll
      for (int t = 0; t < 4; ++t) bv[t] = gfrag(&B[gswz(wn * 64 + t * 16 + lr, ks + lk)]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], bv[t], acc[r][t], 0, 0, 0);
    }
  };
  // Block b: wait for this thread's loads of block b (block b + 1's may be in flight), barrier (everyone's
  // have landed and everyone is done with block b - 1), refill block b - 1's stage with block b + 2, multiply.
  issue(0, As0, Bs0);
  issue(1, As1, Bs1);
  auto step = [&](int b, const bf16_t* A, const bf16_t* B, bf16_t* An, bf16_t* Bn) {
    __builtin_amdgcn_s_waitcnt(gwait_vm(kGAL + kGBL));
    gbarrier();
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
  __builtin_amdgcn_s_waitcnt(gwait_vm(0));   // the surplus loads land before the workgroup's LDS is reused

  // accumulator (r, t) element i: token wm * 64 + r * 16 + (lane / 16) * 4 + i, column n0 + wn * 64 + t * 16 +
  // lane % 16
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 64 + r * 16 + lk * 4 + i;
      if (m >= M) continue;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + wn * 64 + t * 16 + lr;
        if (PARTIAL) {
          part[((int64_t)s * M + m) * N + n] = acc[r][t][i];
        } else {
          const float v = acc[r][t][i] + (R ? bf2f(R[(int64_t)m * ldr + n]) : 0.0f);
          Y[(int64_t)m * ldy + n] = f2bf(v);
        }
      }
    }
}

// Y[m, n] = bf16(sum over s in order of part[s, m, n] + R[m, n]); 8 columns (16 bytes of Y) per thread.
__global__ __launch_bounds__(256) void skinny_reduce_kernel(const float* __restrict__ part, int splits, int M,
                                                            int N, const bf16_t* R, int64_t ldr, bf16_t* Y,
                                                            int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over (m, n / 8)
  const int per = N / 8;
  if (i >= (int64_t)M * per) return;
  const int m = (int)(i / per), n = (int)(i % per) * 8;
  float v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  for (int s = 0; s < splits; ++s) {
    const f32x4* p = reinterpret_cast<const f32x4*>(part + ((int64_t)s * M + m) * N + n);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] += a[j];
      v[4 + j] += b[j];
    }
  }
  if (R) {
    typedef __attribute__((__vector_size__(16))) unsigned u32x4;
    const u32x4 raw = *reinterpret_cast<const u32x4*>(R + (int64_t)m * ldr + n);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] += __uint_as_float(raw[j] << 16);
      v[2 * j + 1] += __uint_as_float(raw[j] & 0xffff0000u);
    }
  }
  typedef __attribute__((__vector_size__(16))) unsigned u32x4;
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = f2bf2(v[2 * j], v[2 * j + 1]);
  *reinterpret_cast<u32x4*>(Y + (int64_t)m * ldy + n) = o;
}

}  // namespace

// Column-block width and K split for a shape.  Every workgroup re-reads X over its K slice, so the wider the
// column block the fewer X bytes per W byte: 128-column blocks (eight waves) are taken whenever a split of K
// into whole slices of at least 4 blocks gives the GPU a workgroup per CU and the partial sums fit (in_proj at
// Jamba's widths: 128 blocks over 2 slices; out_proj: 32 blocks over 8 slices), otherwise 64-column blocks,
// split the same way (shapes with at least 256 of them run unsplit).
struct SkinnyPlan {
  int gn, splits;
};
static SkinnyPlan skinny_plan(int M, int N, int K, int64_t ws_bytes) {
  if (M < 1 || M > kGM || N % 64 != 0 || K % kGK != 0) return {0, 0};
  const int kb = K / kGK;
  auto splits_for = [&](int gn) {
    int s = 1;
    while ((int64_t)(N / gn) * s < 256 && kb % (s * 2) == 0 && kb / (s * 2) >= 4 &&
           (int64_t)s * 2 * M * N * 4 <= ws_bytes)
      s *= 2;
    return s;
  };
  if (N % 128 == 0) {
    const int s = splits_for(128);
    if ((int64_t)(N / 128) * s >= 256) return {128, s};
  }
  return {64, splits_for(64)};
}

int skinny_gemm_splits(int M, int N, int K, int64_t ws_bytes) { return skinny_plan(M, N, K, ws_bytes).splits; }

void launch_skinny_gemm(const void* X, int64_t ldx, const void* W, int64_t ldw, const void* R, int64_t ldr, void* Y,
                        int64_t ldy, int M, int N, int K, int splits, float* part, hipStream_t st) {
  // as skinny_gemm_splits planned it (the workspace bound only limits the split, which the caller passes)
  const int gn = skinny_plan(M, N, K, (int64_t)splits * M * N * 4).gn;
  dim3 grid((unsigned)((N / gn) * splits));
  if (splits == 1) {
    if (gn == 128)
      hipLaunchKernelGGL((skinny_gemm_kernel<false, 128>), grid, dim3(512), 0, st, (const bf16_t*)X, ldx,
                         (const bf16_t*)W, ldw, (const bf16_t*)R, ldr, (bf16_t*)Y, ldy, part, M, N, K, 1);
    else
      hipLaunchKernelGGL((skinny_gemm_kernel<false, 64>), grid, dim3(256), 0, st, (const bf16_t*)X, ldx,
                         (const bf16_t*)W, ldw, (const bf16_t*)R, ldr, (bf16_t*)Y, ldy, part, M, N, K, 1);
    return;
  }
  if (gn == 128) {
    hipLaunchKernelGGL((skinny_gemm_kernel<true, 128>), grid, dim3(512), 0, st, (const bf16_t*)X, ldx,
                       (const bf16_t*)W, ldw, (const bf16_t*)R, ldr, (bf16_t*)Y, ldy, part, M, N, K, splits);
  } else {
    hipLaunchKernelGGL((skinny_gemm_kernel<true, 64>), grid, dim3(256), 0, st, (const bf16_t*)X, ldx,
                       (const bf16_t*)W, ldw, (const bf16_t*)R, ldr, (bf16_t*)Y, ldy, part, M, N, K, splits);
  }
  const int64_t n = (int64_t)M * (N / 8);
  hipLaunchKernelGGL(skinny_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, splits, M,
                     N, (const bf16_t*)R, ldr, (bf16_t*)Y, ldy);
}

}  // namespace jm
