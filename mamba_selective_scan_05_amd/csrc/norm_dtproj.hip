// Jamba's RMSNorms on the selective parameters, then dt_proj + bias + softplus.
//
// norm: one wave per token adds the x_proj partial sums in slice order (all slices of a column are loaded
// together, then added in order, so the result does not depend on timing), then RMSNorms the dt slice
// (R values), the B slice and the C slice (N values each) separately: v / sqrt(mean(v^2) + eps) * w.
// The normalised dt goes out in the I/O dtype (it is the next contraction's operand), B and C in fp32.
//
// dt_proj: delta[m, c] = softplus(sum_r dln[m, r] * W[c, r] + b[c]).  bf16 path on matrix cores
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation): for dt_rank <= 256 persistent 8-wave workgroups keep W_dt in
// registers and stream 64-token dln tiles (dtproj_mfma_stream_kernel); larger ranks take a tiled kernel in
// which a workgroup of 4 waves computes a 64-token x 256-channel tile and transposes it through LDS for
// 16-byte stores.  Bias and softplus are fused into both epilogues.  fp32 I/O: the fp32 matrix-core GEMM
// (gemm_f32.hip) with the same epilogue.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;

// norm: WPT waves per token (1, or 4 when there are few tokens), each summing S / WPT of the x_proj slices;
// with a single slice (long inputs) a wave takes TPW = 4 consecutive tokens, since a wave per token moves only a
// few hundred bytes (256K tokens: 136 -> 113 us; two tokens per wave with two slices, B = 8 x 4K, measured
// 1 us slower, so they keep a wave per token).  S (the number of slices) and COLS (columns per lane, 64 columns apart) are
// compile-time so that every partial-sum load is unconditional (columns past W re-read column W - 1 and tokens
// past M re-read token M - 1; both are dropped): all of a lane's loads are in flight together, then added in
// slice order; with WPT = 4 the four waves' sums are added in wave order through LDS (a fixed order: the
// result does not depend on timing).
template <typename T, int S, int COLS, int WPT, int TPW = 1>
__global__ __launch_bounds__(256) void norm_kernel(const float* __restrict__ part, int M, int R, int N,
                                                   const T* __restrict__ wdt, const T* __restrict__ wb,
                                                   const T* __restrict__ wc, float eps, T* __restrict__ dln,
                                                   float* __restrict__ bc) {
  static_assert(WPT == 1 || WPT == 4, "one wave per token or a whole workgroup per token");
  static_assert(WPT == 1 || TPW == 1, "several tokens per wave only with one wave per token");
  constexpr int SW = S / WPT;                          // slices per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m0 = WPT == 1 ? (blockIdx.x * 4 + wave) * TPW : blockIdx.x;
  if (WPT == 1 && m0 >= M) return;
  const int sub = WPT == 1 ? 0 : wave;
  const int W = R + 2 * N;
  const int64_t slice = (int64_t)M * W;
  float pv[TPW][COLS][SW], wn[COLS];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const float* src = part + (int64_t)min(m0 + t, M - 1) * W + (int64_t)sub * SW * slice;
#pragma unroll
    for (int i = 0; i < COLS; ++i) {
      const int col = min(lane + 64 * i, W - 1);
#pragma unroll
      for (int p = 0; p < SW; ++p) pv[t][i][p] = src[p * slice + col];
    }
  }
  // the norm weight of each column, loaded with the partial sums (clamped indices, no branches) so that it
  // is not a second round trip to memory after the reduction
#pragma unroll
  for (int i = 0; i < COLS; ++i) {
    const int col = lane + 64 * i;
    const float a = io<T>::ld(wdt + min(col, R - 1));
    const float b = io<T>::ld(wb + min(max(col - R, 0), N - 1));
    const float c = io<T>::ld(wc + min(max(col - R - N, 0), N - 1));
    wn[i] = col < R ? a : col < R + N ? b : c;
  }
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int m = m0 + t;
    if (TPW > 1 && m >= M) break;
    float v[COLS];
#pragma unroll
    for (int i = 0; i < COLS; ++i) {
      float s = 0.f;
#pragma unroll
      for (int p = 0; p < SW; ++p) s += pv[t][i][p];
      v[i] = s;
    }
    if (WPT > 1) {
      __shared__ float red[4][COLS * 64];
#pragma unroll
      for (int i = 0; i < COLS; ++i) red[wave][i * 64 + lane] = v[i];
      __syncthreads();
      if (wave != 0) return;
#pragma unroll
      for (int i = 0; i < COLS; ++i)
        v[i] = ((red[0][i * 64 + lane] + red[1][i * 64 + lane]) + red[2][i * 64 + lane]) + red[3][i * 64 + lane];
    }
    float ss_dt = 0.f, ss_b = 0.f, ss_c = 0.f;
#pragma unroll
    for (int i = 0; i < COLS; ++i) {
      const int col = lane + 64 * i;
      const float sq = v[i] * v[i];
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
    for (int i = 0; i < COLS; ++i) {
      const int col = lane + 64 * i;
      if (col < R) {
        io<T>::st(dln + (int64_t)m * R + col, v[i] * r_dt * wn[i]);
      } else if (col < R + N) {
        bc[(int64_t)m * 2 * N + (col - R)] = v[i] * r_b * wn[i];
      } else if (col < W) {
        bc[(int64_t)m * 2 * N + (col - R)] = v[i] * r_c * wn[i];
      }
    }
  }
}

template <typename T, int COLS, int WPT>
void launch_norm_cols(int splits, dim3 grid, hipStream_t st, const float* part, int M, int R, int N, const T* wdt,
                      const T* wb, const T* wc, float eps, T* dln, float* bc) {
  switch (splits) {
#define JM_NORM_CASE(S)                                                                                       \
  case S: {                                                                                                   \
    constexpr int wpt = S >= WPT ? WPT : 1;                                                                   \
    constexpr int tpw = wpt == 1 && S == 1 ? 4 : 1;                                                           \
    const dim3 g = wpt == 1 ? dim3((unsigned)((M + 4 * tpw - 1) / (4 * tpw))) : grid;                         \
    hipLaunchKernelGGL((norm_kernel<T, S, COLS, wpt, tpw>), g, dim3(256), 0, st, part, M, R, N, wdt, wb, wc,  \
                       eps, dln, bc);                                                                         \
    break;                                                                                                    \
  }
    JM_NORM_CASE(1)
    JM_NORM_CASE(2)
    JM_NORM_CASE(4)
    JM_NORM_CASE(8)
    JM_NORM_CASE(16)
#undef JM_NORM_CASE
    default: break;   // the plan only makes power-of-two slice counts up to kMaxXprojSplits
  }
}

template <typename T, int COLS>
void launch_norm_w(int splits, int M, int R, int N, const T* wdt, const T* wb, const T* wc, float eps, T* dln,
                   float* bc, const float* part, hipStream_t st) {
  // few tokens with many slices (decode): a workgroup per token, so that enough waves are in flight
  if (M <= 1024 && splits >= 4)
    launch_norm_cols<T, COLS, 4>(splits, dim3(M), st, part, M, R, N, wdt, wb, wc, eps, dln, bc);
  else
    launch_norm_cols<T, COLS, 1>(splits, dim3((M + 3) / 4), st, part, M, R, N, wdt, wb, wc, eps, dln, bc);
}

template <typename T>
void launch_norm_t(int splits, int M, int R, int N, const T* wdt, const T* wb, const T* wc, float eps, T* dln,
                   float* bc, const float* part, hipStream_t st) {
  if (R + 2 * N <= 5 * 64)
    launch_norm_w<T, 5>(splits, M, R, N, wdt, wb, wc, eps, dln, bc, part, st);
  else
    launch_norm_w<T, 9>(splits, M, R, N, wdt, wb, wc, eps, dln, bc, part, st);
}

constexpr int kDtMaxR = 256;            // dt_rank of the staged bf16 path (larger ranks loop in slices)
constexpr int kDtLd = kDtMaxR + 16;     // padded LDS row of the dln tile (32 bytes of pad: conflict-free fragment reads)
constexpr int kDtOutLd = 64 + 8;        // padded LDS row of a wave's output tile (bf16)

__device__ __forceinline__ bf16x8 ld16_guard(const bf16_t* p, bool ok) {
  uint4 raw = ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  return __builtin_bit_cast(bf16x8, raw);
}

// 64 tokens x 256 channels per workgroup; wave w owns channels [64w, 64w + 64) of the tile.  The LDS of
// the dln tile is reused for the output transpose once the products are done.
constexpr int kDtLdsBytes = (64 * kDtLd * 2 > 4 * 64 * kDtOutLd * 2) ? 64 * kDtLd * 2 : 4 * 64 * kDtOutLd * 2;
__global__ __launch_bounds__(256, 2) void dtproj_mfma_kernel(const bf16_t* __restrict__ dln,
                                                             const bf16_t* __restrict__ w,
                                                             const bf16_t* __restrict__ bias,
                                                             bf16_t* __restrict__ delta, int M, int C, int R) {
  __shared__ __attribute__((aligned(16))) char lds[kDtLdsBytes];
  bf16_t* As = reinterpret_cast<bf16_t*>(lds);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  // XCD-aware order: workgroup i runs on XCD i % 8; XCD x takes channel blocks x, x + 8, ... and walks
  // all token tiles of one channel block before the next.
  const int ncb = (C + 255) / 256, nmt = (M + 63) / 64;
  const int i = blockIdx.x;
  int cb, mt;
  if (ncb % 8 == 0) {
    const int x = i % 8, j = i / 8;
    cb = x + 8 * (j / nmt);
    mt = j % nmt;
  } else {
    cb = i / nmt;
    mt = i % nmt;
  }
  const int c0 = cb * 256 + wave * 64;
  const int m0 = mt * 64;

  f32x4 acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kr = 0; kr < R; kr += kDtMaxR) {
    const int rk = min(kDtMaxR, R - kr);
    __syncthreads();
    // stage the dln tile [64 x rk] (rk % 8 == 0)
    for (int q = tid; q < 64 * (kDtMaxR / 8); q += 256) {
      const int row = q / (kDtMaxR / 8), kc = (q % (kDtMaxR / 8)) * 8;
      const int m = m0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M && kc < rk) v = *reinterpret_cast<const uint4*>(dln + (int64_t)m * R + kr + kc);
      *reinterpret_cast<uint4*>(&As[row * kDtLd + kc]) = v;
    }
    __syncthreads();
    if (c0 < C) {
      // W_dt fragments two k-steps at a time: the next pair is in flight while the current pair multiplies
      auto ldb = [&](int ks, bf16x8* b) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          b[t] = ld16_guard(w + (int64_t)(c0 + t * 16 + lr) * R + kr + ks * 32 + lk, ks * 32 + lk < rk);
      };
      bf16x8 b0[4], b1[4], n0[4], n1[4];
      ldb(0, b0);
      ldb(1, b1);
#pragma unroll
      for (int ks = 0; ks < kDtMaxR / 32; ks += 2) {
        if (ks + 2 < kDtMaxR / 32) {
          ldb(ks + 2, n0);
          ldb(ks + 3, n1);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 a[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            a[r] = *reinterpret_cast<const bf16x8*>(&As[(r * 16 + lr) * kDtLd + (ks + h) * 32 + lk]);
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r], h ? b1[t] : b0[t], acc[r][t], 0, 0, 0);
        }
        if (ks + 2 < kDtMaxR / 32) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            b0[t] = n0[t];
            b1[t] = n1[t];
          }
        }
      }
    }
  }
  // epilogue: bias + softplus, bf16, through LDS so that each lane stores 16 contiguous bytes.  Waves past
  // the last channel block only take part in the barriers.
  const bool active = c0 < C;
  __syncthreads();   // every wave is done reading the dln tile: its LDS now holds the output tiles
  bf16_t* os = reinterpret_cast<bf16_t*>(lds) + wave * 64 * kDtOutLd;
  if (active) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float bc_ = bf2f(bias[c0 + t * 16 + lr]);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
          os[(r * 16 + (lane >> 4) * 4 + i2) * kDtOutLd + t * 16 + lr] = f2bf(softplus(acc[r][t][i2] + bc_));
    }
  }
  __syncthreads();
  if (!active) return;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int id = lane + 64 * q, row = id >> 3, cc = (id & 7) * 8;
    const int m = m0 + row;
    if (m < M) *reinterpret_cast<uint4*>(delta + (int64_t)m * C + c0 + cc) = *reinterpret_cast<const uint4*>(&os[row * kDtOutLd + cc]);
  }
}

// dt_rank <= 256: persistent workgroups of 8 waves (two per SIMD).  Each wave holds the W_dt rows of its 32
// channels for the whole K (dt_rank) in registers and walks a contiguous range of 64-token tiles; the dln
// tiles stream through double-buffered LDS with the next two tiles in flight in registers.  W_dt is the A
// operand and the dln tile the B operand, so a lane's accumulator holds four consecutive channels of one
// token.  The waves are software-pipelined: the MFMAs of tile t + 1 (into a second set of accumulators) are
// interleaved with the bias + softplus of tile t, so the matrix cores and the vector ALU work at the same
// time.  The softplus results go to a double-buffered LDS tile (64 tokens x 256 channels) and, after the next
// barrier, the workgroup writes them as whole 512-byte delta rows with 16-byte lanes: one store instruction
// then covers 8 full cache lines instead of 16 partial ones (the memory pipeline, not the math, bounded the
// kernel with per-lane 8-byte stores).  Stores go through a per-tile buffer resource whose range ends at the
// last token, so there are no branches.  Workgroup i runs on XCD i % 8 and takes token-tile group i % G, so
// each XCD keeps its group's dln tiles in its L2.
// NW waves per workgroup, 32 channels per wave: 256 channels per workgroup for long inputs, 128 for a few
// token tiles (decode), where twice as many workgroups each load half as much of W_dt.
constexpr int kDtWaveCh = 32;                            // channels per wave
constexpr int kDtWaveT = kDtWaveCh / 16;                 // 16-channel MFMA tiles per wave
constexpr int kDtBufferFlags = 0x00020000;               // dword 3 of a raw buffer descriptor on gfx9-family GPUs
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void dtproj_mfma_stream_kernel(const bf16_t* __restrict__ dln,
                                                                        const bf16_t* __restrict__ w,
                                                                        const bf16_t* __restrict__ bias,
                                                                        bf16_t* __restrict__ delta, int M, int C,
                                                                        int R, int groups, int tiles_per_group) {
  constexpr int kDtStreamThreads = 64 * NW;
  constexpr int kCB = kDtWaveCh * NW;                    // channels per workgroup
  constexpr int kDtStreamOutLd = kCB + 8;                // padded row of the LDS output tile (bf16)
  __shared__ __attribute__((aligned(16))) bf16_t As[2 * 64 * kDtLd];
  __shared__ __attribute__((aligned(16))) bf16_t Os[2 * 64 * kDtStreamOutLd];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4, lk = lq * 8;
  const int nmt = (M + 63) / 64;
  // Workgroup i runs on XCD i % 8.  With a multiple of 8 channel blocks, XCD x takes channel blocks x, x + 8,
  // ... (every token group of each), so its L2 holds only those blocks' W_dt rows: one eighth of W_dt per XCD
  // instead of all of it (measured: the start-up W_dt load took ~3 us with every XCD fetching the whole).
  const int ncb = (C + kCB - 1) / kCB;
  int g, cb;
  if (ncb % 8 == 0) {
    const int x = blockIdx.x % 8, j = blockIdx.x / 8;
    cb = x + 8 * (j / groups);
    g = j % groups;
  } else {
    g = blockIdx.x % groups;
    cb = blockIdx.x / groups;
  }
  const int mt_beg = g * tiles_per_group, mt_end = min(nmt, mt_beg + tiles_per_group);
  if (mt_beg >= mt_end) return;                      // uniform over the workgroup
  const int ntiles = mt_end - mt_beg;
  const int c0 = cb * kCB + wave * kDtWaveCh;
  const bool active = c0 < C;
  const int cw = active ? c0 : 0;                    // waves past C read valid rows and store nothing

  // this wave's W_dt fragments for all of K (zero past dt_rank): A operand, row = channel, 8 k per lane
  bf16x8 wa[kDtMaxR / 32][kDtWaveT];
#pragma unroll
  for (int ks = 0; ks < kDtMaxR / 32; ++ks)
#pragma unroll
    for (int t = 0; t < kDtWaveT; ++t)
      wa[ks][t] = ld16_guard(w + (int64_t)(cw + t * 16 + lr) * R + ks * 32 + lk, ks * 32 + lk < R);
  // bias of the four channels this lane's accumulators hold in each channel tile: the accumulators start
  // from it, so the products come out with the bias already added
  f32x4 bs[kDtWaveT];
#pragma unroll
  for (int t = 0; t < kDtWaveT; ++t)
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) bs[t][i2] = bf2f(bias[cw + t * 16 + lq * 4 + i2]);

  // dln tile loader: 64 rows x 256 k = 2048 chunks of 16 bytes, 2048 / threads per thread.  Rows past M
  // re-read row M - 1 (their products are never stored) and k past R re-reads column R - 8 (finite values that meet
  // the zero W_dt fragments), so the loads need no select, which would stall on them at issue.  Tiles past
  // the group re-read its last tile.
  typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
  constexpr int kQ = 64 * (kDtMaxR / 8) / kDtStreamThreads;
  auto load_tile = [&](int i, u32x4* r) {
    const int mt = mt_beg + min(i, ntiles - 1);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int id = tid + q * kDtStreamThreads, row = id >> 5, kc = (id & 31) * 8;
      const int m = min(mt * 64 + row, M - 1);
      r[q] = *reinterpret_cast<const u32x4*>(dln + (int64_t)m * R + min(kc, R - 8));
    }
  };
  auto store_tile = [&](int buf, const u32x4* r) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int id = tid + q * kDtStreamThreads, row = id >> 5, kc = (id & 31) * 8;
      *reinterpret_cast<u32x4*>(&As[buf * 64 * kDtLd + row * kDtLd + kc]) = r[q];
    }
  };
  typedef f32x4 Acc[4][kDtWaveT];
  auto mfma_ks = [&](const bf16_t* At, int ks, Acc& acc) {
    bf16x8 a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = *reinterpret_cast<const bf16x8*>(&At[(r * 16 + lr) * kDtLd + ks * 32 + lk]);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < kDtWaveT; ++t)
        acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[ks][t], a[r], acc[r][t], 0, 0, 0);
  };
  auto zero = [&](Acc& acc) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < kDtWaveT; ++t) acc[r][t] = bs[t];
  };
  auto mfma_tile = [&](int buf, Acc& acc) {
    zero(acc);
#pragma unroll
    for (int ks = 0; ks < kDtMaxR / 32; ++ks) mfma_ks(As + buf * 64 * kDtLd, ks, acc);
  };
  // acc[r][t][i2] is channel t*16 + 4*lq + i2 of token r*16 + lr: bias + softplus, four bf16 channels to
  // the LDS output tile in one 8-byte write
  auto epilogue_part = [&](bf16_t* O, const Acc& acc, int r, int t) {
    uint32_t pk[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) pk[h2] = f2bf2(softplus(acc[r][t][2 * h2]), softplus(acc[r][t][2 * h2 + 1]));
    *reinterpret_cast<uint2*>(&O[(r * 16 + lr) * kDtStreamOutLd + wave * kDtWaveCh + t * 16 + lq * 4]) =
        make_uint2(pk[0], pk[1]);
  };
  // the LDS output tile of tile i as whole rows: 64 rows x 2 kCB bytes, 16 bytes per lane, 4 per thread;
  // the buffer range ends at the last token and at the last channel of the workgroup's block
  auto store_out = [&](int i, const bf16_t* O) {
    const int64_t m0 = (int64_t)(mt_beg + i) * 64;
    const int rows = min(64, (int)(M - m0));
    const __amdgpu_buffer_rsrc_t out =
        __builtin_amdgcn_make_buffer_rsrc(delta + m0 * C, (short)0, rows * C * 2, kDtBufferFlags);
    constexpr int kRowChunks = kCB / 8;                  // 16-byte chunks per output row
    const int ch = (tid % kRowChunks) * 8, cbase = cb * kCB;
#pragma unroll
    for (int q = 0; q < 64 * kRowChunks / kDtStreamThreads; ++q) {
      const int row = tid / kRowChunks + q * (kDtStreamThreads / kRowChunks);
      const u32x4 v = *reinterpret_cast<const u32x4*>(&O[row * kDtStreamOutLd + ch]);
      if (cbase + ch < C)
        __builtin_amdgcn_raw_buffer_store_b128(v, out, (uint32_t)((row * C + cbase + ch) * 2), 0, 0);
    }
  };
  // MFMAs of the tile in LDS buffer buf into acc, interleaved with the epilogue of the previous tile from
  // prev into output buffer O: K step ks carries epilogue part ks (there are as many parts as K steps)
  static_assert(4 * kDtWaveT == kDtMaxR / 32, "one epilogue part per K step");
  auto mfma_and_epilogue = [&](int buf, Acc& acc, bf16_t* O, const Acc& prev) {
    zero(acc);
#pragma unroll
    for (int ks = 0; ks < kDtMaxR / 32; ++ks) {
      mfma_ks(As + buf * 64 * kDtLd, ks, acc);
      epilogue_part(O, prev, ks / kDtWaveT, ks % kDtWaveT);
    }
  };
  // the epilogue of the group's last tile, which has no next tile to overlap with
  auto epilogue_all = [&](bf16_t* O, const Acc& prev) {
#pragma unroll
    for (int ks = 0; ks < kDtMaxR / 32; ++ks) epilogue_part(O, prev, ks / kDtWaveT, ks % kDtWaveT);
  };

  // Tile i lives in LDS buffer i & 1 and its output in LDS output buffer i & 1.  Prologue: tile 0 to LDS,
  // tiles 1 and 2 in flight, MFMAs of tile 0, tile 1 to LDS.  Step i: stores of tile i - 1's output, MFMAs
  // of tile i + 1 with the epilogue of tile i, tile i + 2 (in registers) into the buffer tile i used, tile
  // i + 4 requested, barrier.  Unrolled by two, so accumulators and register sets alternate without copies.
  u32x4 rt0[kQ], rt1[kQ];
  Acc accA, accB;
  load_tile(0, rt0);
  store_tile(0, rt0);
  load_tile(1, rt0);
  load_tile(2, rt1);
  __syncthreads();
  mfma_tile(0, accA);
  store_tile(1, rt0);
  load_tile(3, rt0);
  __syncthreads();
  for (int i = 0;; i += 2) {
    if (i > 0) store_out(i - 1, Os + 64 * kDtStreamOutLd);
    if (i + 1 >= ntiles) {                           // tile i is the group's last
      epilogue_all(Os, accA);
      __syncthreads();
      store_out(i, Os);
      break;
    }
    mfma_and_epilogue(1, accB, Os, accA);            // MFMAs of tile i + 1, epilogue of tile i
    store_tile(0, rt1);                              // tile i + 2
    load_tile(i + 4, rt1);
    __syncthreads();
    store_out(i, Os);
    if (i + 2 >= ntiles) {                           // tile i + 1 is the group's last
      epilogue_all(Os + 64 * kDtStreamOutLd, accB);
      __syncthreads();
      store_out(i + 1, Os + 64 * kDtStreamOutLd);
      break;
    }
    mfma_and_epilogue(0, accA, Os + 64 * kDtStreamOutLd, accB);   // MFMAs of tile i + 2, epilogue of tile i + 1
    store_tile(1, rt0);                              // tile i + 3
    load_tile(i + 5, rt0);
    __syncthreads();
  }
}


}  // namespace

void launch_norm(bool bf16, const float* part, int splits, int M, int R, int N, const void* wdt, const void* wb,
                 const void* wc, float eps, void* dln, float* bc, hipStream_t st) {
  if (M == 0) return;
  if (bf16)
    launch_norm_t<bf16_t>(splits, M, R, N, (const bf16_t*)wdt, (const bf16_t*)wb, (const bf16_t*)wc, eps,
                          (bf16_t*)dln, bc, part, st);
  else
    launch_norm_t<float>(splits, M, R, N, (const float*)wdt, (const float*)wb, (const float*)wc, eps,
                         (float*)dln, bc, part, st);
}

void launch_dtproj(bool bf16, const void* dln, const void* w, const void* b, void* delta, int M, int C, int R,
                   hipStream_t st) {
  if (M == 0) return;
  if (bf16) {
    const int ncb = (C + 255) / 256, nmt = (M + 63) / 64;
    if (R <= kDtMaxR) {
      // one workgroup per CU: enough token-tile groups for ~256 workgroups, 8 when possible (one per XCD).
      // With at most 8 token tiles the workgroups take 128 channels instead of 256.
      const bool narrow = nmt <= 8;
      const int nb = narrow ? (C + 127) / 128 : ncb;
      int groups = nb >= 256 ? 1 : 256 / nb;
      if (groups > 8) groups = groups / 8 * 8;
      if (groups > nmt) groups = nmt;
      const int per = (nmt + groups - 1) / groups;
      if (narrow)
        hipLaunchKernelGGL(dtproj_mfma_stream_kernel<4>, dim3(nb * groups), dim3(256), 0, st, (const bf16_t*)dln,
                           (const bf16_t*)w, (const bf16_t*)b, (bf16_t*)delta, M, C, R, groups, per);
      else
        hipLaunchKernelGGL(dtproj_mfma_stream_kernel<8>, dim3(nb * groups), dim3(512), 0, st, (const bf16_t*)dln,
                           (const bf16_t*)w, (const bf16_t*)b, (bf16_t*)delta, M, C, R, groups, per);
    } else {
      hipLaunchKernelGGL(dtproj_mfma_kernel, dim3(ncb * nmt), dim3(256), 0, st, (const bf16_t*)dln, (const bf16_t*)w,
                         (const bf16_t*)b, (bf16_t*)delta, M, C, R);
    }
  } else {
    launch_gemm_f32((const float*)dln, (const float*)w, (const float*)b, (float*)delta, M, C, R, 1, st);
  }
}

}  // namespace jm
