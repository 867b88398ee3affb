// The one-token decode step as a single kernel (bf16 I/O).
//
// A decode step is the mixer run on one new token per sequence against that sequence's cached conv window and
// recurrent state (TransformerLens "supported_architectures.jamba": generation carries the conv and SSM
// caches from step to step; the arithmetic is the Jamba Guide's "Inside the Mamba State-Space Layers" with one
// token).  Its only dependence across channels is x_proj, a contraction over all of them, followed by the
// RMSNorms of its output rows; everything else is independent per (sequence, channel).  So one cooperative
// launch (every workgroup resident at once, one 8-wave workgroup per CU) runs three phases separated by two
// grid-wide barriers:
//   1  per unit of 32 sequences x 256 channels: conv + bias + SiLU and the shifted conv state, then the unit's
//      x_proj partial sums over its 256 channels on the matrix cores (v_mfma_f32_16x16x32_bf16);
//   2  per sequence: the partial sums added in slice order, then the dt / B / C RMSNorms;
//   3  per unit: dt_proj + bias + softplus on the matrix cores into LDS, then the state update, the D skip
//      and the SiLU(z) gate; the unit's states stream through HBM as 4 KB rows (a wave's 64 channels of one
//      sequence), three sequences' rows in flight per wave (one with the exact hold, for registers).
// Between the phases nothing goes back to the host, and with one unit per workgroup the unit's xc stays in
// LDS from phase 1 to phase 3.  Each step computes what the separate kernels do (conv_silu.hip,
// norm_dtproj.hip, scan.hip) up to summation order (x_proj slices of 256 channels here, the norms' sums of
// squares reduced across waves) and, for the exact hold, A and 1 / A derived from A log2(e).
//
// Barrier: one flag per workgroup in the workspace, set to a token unique to the launch and the barrier (see
// grid_barrier), so nothing needs zeroing between calls.  Every workgroup reaches both barriers (none returns
// early); the runtime refuses a cooperative launch that would not have every workgroup resident; and each
// wait gives up after a bounded number of polls (about a second), so the kernel always ends — with undefined
// results if a wait ever gave up, which a cooperative launch rules out.
#include <atomic>
#include <chrono>
#include <mutex>

#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kN = 16;
constexpr int kTaps = 4;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;   // one workgroup per CU, two waves per SIMD
constexpr int kUT = 32;                 // sequences per unit
constexpr int kUC = 256;                // channels per unit (one x_proj slice)
constexpr int kMaxR = 256;
constexpr int kMaxBatch = 1024;         // the partial sums take C / 256 * B * (R + 32) floats
constexpr int kXsLd = kUC + 8;          // bf16 row of the xc tile (16 bytes of pad)
constexpr int kDlLd = kMaxR + 8;        // bf16 row of the dln tile
constexpr int kDsLd = kUC + 4;          // fp32 row of the delta tile
constexpr int kSeqAhead = 3;            // sequences whose state rows a wave has in flight
constexpr int kXT = (kMaxR / 16 + 2 + kWaves - 1) / kWaves;   // x_proj column tiles per wave
constexpr int kDT = kUC / 16 / kWaves;                        // dt_proj channel tiles per wave
constexpr int kSeqPerWave = kUT / (kWaves / 4);               // phase 3: sequences per wave
constexpr int kSpinLimit = 1 << 20;     // polls of one barrier wait (far beyond any real wait)
constexpr int kWaitVmem0 = 0x0F70;      // s_waitcnt operand (gfx9 encoding): vector-memory count 0, others any
constexpr int kMaxSlices = 32;          // channel slices (d_inner / 256) the norm phase loads at once

__device__ __forceinline__ void unpack8(uint4 r, float* f) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(f2bf2(f[0], f[1]), f2bf2(f[2], f[3]), f2bf2(f[4], f[5]), f2bf2(f[6], f[7]));
}

// Buffer resource over [base, base + bytes): raw accesses with 32-bit offsets; loads past the range return 0
// and stores past it are dropped, so a sequence without a state (no input state, or a slot outside the pool)
// takes a zero-length range instead of a branch.
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a raw buffer descriptor on gfx9-family GPUs
constexpr int kNonTemporal = 2;            // cache policy of the state accesses: streamed once per call
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}

// Unit u -> its first sequence and first channel.  With a multiple of 8 channel slices, workgroup i (on XCD
// i % 8) gets slices congruent to i mod 8, so each XCD's L2 holds one eighth of W_x and W_dt.
__device__ __forceinline__ void unit_of(int u, int nT, int nC, int& b0, int& cs) {
  int tt;
  if (nC % 8 == 0) {
    const int x = u % 8, j = u / 8;
    cs = x + 8 * (j / nT);
    tt = j % nT;
  } else {
    cs = u / nT;
    tt = u % nT;
  }
  b0 = tt * kUT;
}

// Grid barrier k of launch L: workgroup g publishes the token 4 L + k in its own flag, then its threads poll
// all flags until every one holds that token.  Launch ids are unique, so a flag left by an earlier call (or
// whatever the workspace held) never matches, and nothing needs zeroing.  Before publishing, every thread
// waits for its own stores (they have reached L2), the workgroup meets, and one thread makes the workgroup's
// writes visible device-wide (one L2 write-back per workgroup, not one per wave); after the wait, one
// device-scope acquire per workgroup drops stale lines from the CU's L1 and the XCD's L2.  No atomic
// read-modify-writes: the waits read G flags in parallel instead of contending for one counter.
__device__ __forceinline__ void grid_barrier(uint64_t* flags, uint64_t token) {
  __builtin_amdgcn_s_waitcnt(kWaitVmem0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __hip_atomic_store(flags + blockIdx.x, token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  for (int i = 0; i < kSpinLimit; ++i) {
    int mine = 1;
    for (int g = threadIdx.x; g < (int)gridDim.x; g += blockDim.x)
      mine &= __hip_atomic_load(flags + g, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == token;
    if (__syncthreads_and(mine)) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (threadIdx.x == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();
}

template <bool ZOH>
__global__ __launch_bounds__(kThreads, 1) void decode_step_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t xs[kUT * kXsLd];     // the unit's xc
  __shared__ __attribute__((aligned(16))) bf16_t zs[kUT * kXsLd];     // the unit's gate inputs z
  __shared__ __attribute__((aligned(16))) bf16_t dls[kUT * kDlLd];    // the unit's normalised dt rows
  __shared__ __attribute__((aligned(16))) float ds[kUT * kDsLd];      // the unit's delta
  __shared__ __attribute__((aligned(16))) float bcs[kUT * 2 * kN];    // the unit's B and C rows
  __shared__ __attribute__((aligned(16))) float hst[kWaves * 64 * kN];   // a 4 KB state tile per wave
  __shared__ float red[kWaves][4];
  __shared__ int srow[kUT];                                           // the unit's state rows (-1: none)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: per-wave bases in SGPRs
  const int lr = lane & 15, lq = lane >> 4;
  const int B = a.B, C = a.C, R = a.R, W = R + 2 * kN;
  const int nT = (B + kUT - 1) / kUT, nC = C / kUC, U = nT * nC;
  const int G = gridDim.x;
  const bool keep_xc = U <= G;            // one unit per workgroup: its xc stays in LDS for phase 3
  const bf16_t* X = (const bf16_t*)a.x;
  const bf16_t* Z = (const bf16_t*)a.z;
  const bf16_t* CW = (const bf16_t*)a.conv_w;
  const bf16_t* CB = (const bf16_t*)a.conv_b;
  const bf16_t* CI = (const bf16_t*)a.conv_in;
  bf16_t* CO = (bf16_t*)a.conv_out;
  const bf16_t* WX = (const bf16_t*)a.x_proj_w;
  const bf16_t* WDT = (const bf16_t*)a.dt_proj_w;
  const bf16_t* BDT = (const bf16_t*)a.dt_proj_b;
  bf16_t* XC = (bf16_t*)a.xc;
  bf16_t* DLN = (bf16_t*)a.dln;
  bf16_t* OUT = (bf16_t*)a.out;

  // ---- phase 1: conv + SiLU, x_proj partial sums
  const int NTc = W / 16;                 // x_proj column tiles: wave w takes tiles w, w + 8, w + 16
  for (int u = blockIdx.x; u < U; u += G) {
    int b0, cs;
    unit_of(u, nT, nC, b0, cs);
    const int c0 = cs * kUC;
    // the W_x fragments of the wave's column tiles, requested before the conv so that they arrive during it
    bf16x8 wf[kXT][kUC / 32];
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const int nt = min(wave + kWaves * t, NTc - 1);
#pragma unroll
      for (int ks = 0; ks < kUC / 32; ++ks)
        wf[t][ks] = *reinterpret_cast<const bf16x8*>(WX + (int64_t)(nt * 16 + lr) * C + c0 + ks * 32 + lq * 8);
    }
    if (tid < kUT) srow[tid] = b0 + tid < B ? (int)state_row(a.slots, a.pool, b0 + tid) : -1;
    __syncthreads();                      // the previous unit's fragment reads of xs are done; srow is set
    // item -> (row r of the unit, 8 channels g): 32 rows x 32 groups.  Rows past B read the last sequence's
    // input with a zero state (their srow is -1) and store nothing but their (unused) LDS row.
    for (int it = tid; it < kUT * (kUC / 8); it += kThreads) {
      const int r = it >> 5, g = it & 31;
      const int bb = b0 + r, b = min(bb, B - 1);
      const int c = c0 + g * 8;
      const int row = srow[r];             // a wave spans two rows: per-lane state addresses
      const int64_t so = ((int64_t)max(row, 0) * C + c) * (kTaps - 1);
      const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
      const uint4 xr = *reinterpret_cast<const uint4*>(X + (int64_t)b * a.xs + c);
      uint4 sr[kTaps - 1] = {z4, z4, z4};
      if (CI != nullptr && row >= 0) {
        const uint4* sp = reinterpret_cast<const uint4*>(CI + so);
#pragma unroll
        for (int q = 0; q < kTaps - 1; ++q) sr[q] = sp[q];
      }
      const uint4* wp = reinterpret_cast<const uint4*>(CW + (int64_t)c * kTaps);
      uint4 wr[kTaps];
#pragma unroll
      for (int q = 0; q < kTaps; ++q) wr[q] = wp[q];
      const uint4 br = CB ? *reinterpret_cast<const uint4*>(CB + c) : z4;
      float xf[8], st[8 * (kTaps - 1)], wv[8 * kTaps], bv[8];
      unpack8(xr, xf);
#pragma unroll
      for (int q = 0; q < kTaps - 1; ++q) unpack8(sr[q], st + 8 * q);
#pragma unroll
      for (int q = 0; q < kTaps; ++q) unpack8(wr[q], wv + 8 * q);
      unpack8(br, bv);
      float o[8], ns[8 * (kTaps - 1)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float* s3 = st + i * (kTaps - 1);
        float v = bv[i];
        v = fmaf(wv[i * kTaps + 0], s3[0], v);
        v = fmaf(wv[i * kTaps + 1], s3[1], v);
        v = fmaf(wv[i * kTaps + 2], s3[2], v);
        v = fmaf(wv[i * kTaps + 3], xf[i], v);
        o[i] = silu(v);
        ns[i * 3 + 0] = s3[1];
        ns[i * 3 + 1] = s3[2];
        ns[i * 3 + 2] = xf[i];
      }
      const uint4 xo = pack8(o);
      *reinterpret_cast<uint4*>(&xs[r * kXsLd + g * 8]) = xo;
      if (!keep_xc && bb < B) *reinterpret_cast<uint4*>(XC + (int64_t)bb * C + c) = xo;
      if (row >= 0) {                      // rows past B have row -1 too
        uint4* op = reinterpret_cast<uint4*>(CO + so);
#pragma unroll
        for (int q = 0; q < kTaps - 1; ++q) op[q] = pack8(ns + 8 * q);
      }
    }
    __syncthreads();
    // part[cs, b, n] = sum over the unit's channels of xc[b, c] * W_x[n, c]: xc rows are the A operand
    // (tokens), W_x rows the B operand (columns); lane l holds tokens 4 (l / 16) + i of a tile, column l % 16
    f32x4 acc[kXT][2];
#pragma unroll
    for (int t = 0; t < kXT; ++t)
#pragma unroll
      for (int m = 0; m < 2; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kUC / 32; ++ks) {
      bf16x8 av[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        av[m] = *reinterpret_cast<const bf16x8*>(&xs[(m * 16 + lr) * kXsLd + ks * 32 + lq * 8]);
#pragma unroll
      for (int t = 0; t < kXT; ++t) {
        if (wave + kWaves * t >= NTc) continue;
#pragma unroll
        for (int m = 0; m < 2; ++m)
          acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], wf[t][ks], acc[t][m], 0, 0, 0);
      }
    }
    float* dst = a.part + (int64_t)cs * B * W;
#pragma unroll
    for (int t = 0; t < kXT; ++t) {
      const int nt = wave + kWaves * t;
      if (nt >= NTc) continue;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int bb = b0 + m * 16 + lq * 4 + i;
          if (bb < B) dst[(int64_t)bb * W + nt * 16 + lr] = acc[t][m][i];
        }
    }
  }

  // ---- phase 2: per sequence, add the slices in order and RMSNorm dt, B, C
  grid_barrier(a.flags, a.launch * 4 + 1);
  for (int b = blockIdx.x; b < B; b += G) {
    const int col = tid;
    float v = 0.0f;
    if (col < W) {
      const float* src = a.part + (int64_t)b * W + col;
      const int64_t sl = (int64_t)B * W;
      // all slices in flight (slice indices past nC re-read the last), then added in slice order
      for (int s0 = 0; s0 < nC; s0 += kMaxSlices) {
        float t[kMaxSlices];
#pragma unroll
        for (int j = 0; j < kMaxSlices; ++j) t[j] = src[min(s0 + j, nC - 1) * sl];
#pragma unroll
        for (int j = 0; j < kMaxSlices; ++j)
          if (s0 + j < nC) v += t[j];
      }
    }
    const float sq = v * v;
    float s_dt = col < R ? sq : 0.0f;
    float s_b = col >= R && col < R + kN ? sq : 0.0f;
    float s_c = col >= R + kN && col < W ? sq : 0.0f;
    s_dt = wave_sum(s_dt);
    s_b = wave_sum(s_b);
    s_c = wave_sum(s_c);
    if (lane == 0) {
      red[wave][0] = s_dt;
      red[wave][1] = s_b;
      red[wave][2] = s_c;
    }
    __syncthreads();
    float t_dt = 0.0f, t_b = 0.0f, t_c = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      t_dt += red[w][0];
      t_b += red[w][1];
      t_c += red[w][2];
    }
    const float r_dt = 1.0f / sqrtf(t_dt / R + a.eps);
    const float r_b = 1.0f / sqrtf(t_b / kN + a.eps);
    const float r_c = 1.0f / sqrtf(t_c / kN + a.eps);
    if (col < R) {
      DLN[(int64_t)b * R + col] = f2bf(v * r_dt * bf2f(((const bf16_t*)a.dt_norm_w)[col]));
    } else if (col < R + kN) {
      a.bc[(int64_t)b * 2 * kN + (col - R)] = v * r_b * bf2f(((const bf16_t*)a.b_norm_w)[col - R]);
    } else if (col < W) {
      a.bc[(int64_t)b * 2 * kN + (col - R)] = v * r_c * bf2f(((const bf16_t*)a.c_norm_w)[col - R - kN]);
    }
    __syncthreads();                      // red is reused by the next sequence
  }

  // ---- phase 3: dt_proj + softplus, then the state update and the gated output
  grid_barrier(a.flags, a.launch * 4 + 2);
  const int KS = R / 32;
  for (int u = blockIdx.x; u < U; u += G) {
    int b0, cs;
    unit_of(u, nT, nC, b0, cs);
    const int c0 = cs * kUC;
    // W_dt fragments of the wave's channel tiles (the A operand: rows are channels)
    bf16x8 wd[kDT][kMaxR / 32];
#pragma unroll
    for (int t = 0; t < kDT; ++t)
#pragma unroll
      for (int ks = 0; ks < kMaxR / 32; ++ks)
        if (ks < KS)
          wd[t][ks] = *reinterpret_cast<const bf16x8*>(WDT + (int64_t)(c0 + (wave * kDT + t) * 16 + lr) * R +
                                                       ks * 32 + lq * 8);
    __syncthreads();                      // the previous unit's readers of dls, ds and bcs are done
    for (int q = tid; q < kUT * (R / 8); q += kThreads) {
      const int r = q / (R / 8), k = (q % (R / 8)) * 8;
      const int b = min(b0 + r, B - 1);
      *reinterpret_cast<uint4*>(&dls[r * kDlLd + k]) = *reinterpret_cast<const uint4*>(DLN + (int64_t)b * R + k);
    }
    for (int q = tid; q < kUT * 2 * kN; q += kThreads) {
      const int r = q / (2 * kN), n = q % (2 * kN);
      bcs[q] = a.bc[(int64_t)min(b0 + r, B - 1) * 2 * kN + n];
    }
    if (tid < kUT) srow[tid] = b0 + tid < B ? (int)state_row(a.slots, a.pool, b0 + tid) : -1;
    for (int q = tid; q < kUT * (kUC / 8); q += kThreads) {
      const int r = q >> 5, k = (q & 31) * 8;
      *reinterpret_cast<uint4*>(&zs[r * kXsLd + k]) =
          *reinterpret_cast<const uint4*>(Z + (int64_t)min(b0 + r, B - 1) * a.zs + c0 + k);
    }
    if (!keep_xc) {                       // xc of this unit back from HBM (the LDS tile held another unit's)
      for (int q = tid; q < kUT * (kUC / 8); q += kThreads) {
        const int r = q >> 5, k = (q & 31) * 8;
        *reinterpret_cast<uint4*>(&xs[r * kXsLd + k]) =
            *reinterpret_cast<const uint4*>(XC + (int64_t)min(b0 + r, B - 1) * C + c0 + k);
      }
    }
    __syncthreads();
    // delta[c, b] = softplus(bias[c] + sum_r W_dt[c, r] dln[b, r]): lane l holds channels 4 (l / 16) + i of a
    // channel tile for token l % 16 of token tile m; rounded to bf16 like the I/O-dtype delta elsewhere
#pragma unroll
    for (int t = 0; t < kDT; ++t) {
      const int ch = (wave * kDT + t) * 16 + lq * 4;   // within the unit
      f32x4 bias4;
#pragma unroll
      for (int i = 0; i < 4; ++i) bias4[i] = bf2f(BDT[c0 + ch + i]);
      f32x4 dacc[2] = {bias4, bias4};
#pragma unroll
      for (int ks = 0; ks < kMaxR / 32; ++ks) {
        if (ks >= KS) break;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&dls[(m * 16 + lr) * kDlLd + ks * 32 + lq * 8]);
          dacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wd[t][ks], bv, dacc[m], 0, 0, 0);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x4 d;
#pragma unroll
        for (int i = 0; i < 4; ++i) d[i] = bf2f(f2bf(softplus(dacc[m][i])));
        *reinterpret_cast<f32x4*>(&ds[(m * 16 + lr) * kDsLd + ch]) = d;
      }
    }
    __syncthreads();

    // wave -> 64 channels (cg) x kSeqPerWave sequences (tq); lane = channel
    const int cg = wave & 3, tq = wave >> 2;
    const int c = c0 + cg * 64 + lane;
    float a2[kN];
    {
      const uint4* ap = reinterpret_cast<const uint4*>((const bf16_t*)a.A_log + (int64_t)c * kN);
      float al[kN];
      unpack8(ap[0], al);
      unpack8(ap[1], al + 8);
#pragma unroll
      for (int n = 0; n < kN; ++n) a2[n] = -exp2_fast(al[n] * kLog2e) * kLog2e;
    }
    const float Dc = bf2f(((const bf16_t*)a.D)[c]);
    float* hs = hst + wave * 64 * kN;
    const int jb = b0 + tq * kSeqPerWave;
    const int jn = min(kSeqPerWave, B - jb);   // this wave's sequences (none when jn <= 0)
    // this wave's 64 channels of state row 0 ([rows, C, 16] fp32)
    const float* h0w = a.h0 ? a.h0 + (int64_t)(c0 + cg * 64) * kN : nullptr;
    float* h1w = a.h_out + (int64_t)(c0 + cg * 64) * kN;
    constexpr int kRowBytes = 64 * kN * 4;
    // Sequence slot j of the wave (all kSeqPerWave slots run; slots past jn touch no memory): its 4 KB state
    // row as four 16-byte lanes per lane (global chunk q * 64 + lane).
    auto fetch = [&](int j, f32x4* rw) __attribute__((always_inline)) {
      const int jj = max(min(j, jn - 1), 0);
      const int row = __builtin_amdgcn_readfirstlane(srow[tq * kSeqPerWave + jj]);   // -1 past B
      const __amdgpu_buffer_rsrc_t in =
          rsrc(h0w + (int64_t)max(row, 0) * C * kN, h0w != nullptr && row >= 0 && j < jn ? kRowBytes : 0);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        rw[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(in, (q * 64 + lane) * 16, 0,
                                                                                 kNonTemporal));
    };
    auto process = [&](int j, const f32x4* rw) __attribute__((always_inline)) {
      const int r = tq * kSeqPerWave + j;
      const bool live = j < jn;
      const int row = __builtin_amdgcn_readfirstlane(srow[r]);
      float h[kN];
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = q * 64 + lane;
        *reinterpret_cast<f32x4*>(&hs[hslot(g >> 2, g & 3)]) = rw[q];
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&hs[hslot(lane, q)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) h[q * 4 + i] = v[i];
      }
      const float dt = ds[r * kDsLd + cg * 64 + lane];
      const float xv = bf2f(xs[r * kXsLd + cg * 64 + lane]);
      const float* Bt = &bcs[r * 2 * kN];
      const float* Ct = Bt + kN;
      float e[kN];
#pragma unroll
      for (int n = 0; n < kN; ++n) e[n] = dt * a2[n];
#pragma unroll
      for (int n = 0; n < kN; ++n) e[n] = exp2_fast(e[n]);
      const float uu = dt * xv;
      float y = 0.0f;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        float in;
        if (ZOH) {
          const float An = a2[n] * kLn2;
          in = zoh_coef(dt, e[n], An, rcp_fast(An)) * (xv * Bt[n]);
        } else {
          in = uu * Bt[n];
        }
        h[n] = fmaf(e[n], h[n], in);
        y = fmaf(Ct[n], h[n], y);
      }
      y = fmaf(Dc, xv, y);
      const float zv = bf2f(zs[r * kXsLd + cg * 64 + lane]);
      const float gate = zv * rcp_fast(1.0f + exp2_fast(zv * -kLog2e));
      const __amdgpu_buffer_rsrc_t o = rsrc(OUT + (int64_t)(jb + j) * C + c0 + cg * 64, live ? 64 * 2 : 0);
      __builtin_amdgcn_raw_buffer_store_b16(f2bf(y * gate), o, lane * 2, 0, 0);
      // the new state: lane-owned 64 bytes into the tile, then out as contiguous 16-byte lanes
      const __amdgpu_buffer_rsrc_t out =
          rsrc(h1w + (int64_t)max(row, 0) * C * kN, live && row >= 0 ? kRowBytes : 0);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(&hs[hslot(lane, q)]) = f32x4{h[q * 4], h[q * 4 + 1], h[q * 4 + 2], h[q * 4 + 3]};
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int g = q * 64 + lane;
        __builtin_amdgcn_raw_buffer_store_b128(
            __builtin_bit_cast(u32x4, *reinterpret_cast<const f32x4*>(&hs[hslot(g >> 2, g & 3)])), out, g * 16, 0,
            kNonTemporal);
      }
    };
    // Straight-line software pipeline over the wave's slots: slot j computes from ring entry j % D while
    // the next D - 1 slots' rows are in flight.  No branches, so the compiler's wait before each entry's
    // use counts exactly the accesses issued after it.
    constexpr int D = ZOH ? 1 : kSeqAhead;   // the exact hold needs more registers per sequence
    f32x4 raw[D][4];
#pragma unroll
    for (int d = 0; d < D; ++d) fetch(d, raw[d]);
#pragma unroll
    for (int j = 0; j < kSeqPerWave; ++j) {
      process(j, raw[j % D]);
      if (j + D < kSeqPerWave) fetch(j + D, raw[j % D]);
    }
  }
}

// Launch ids: distinct for every launch of the process (a 64-bit counter from a start that differs between
// processes), never 0.
uint64_t next_launch_id() {
  static std::atomic<uint64_t> next{(uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
  uint64_t id;
  do {
    id = next.fetch_add(1, std::memory_order_relaxed);
  } while (id == 0);
  return id;
}

struct DeviceInfo {
  bool init = false;
  bool ok = false;
  int max_groups = 0;
};
constexpr int kMaxDevices = 64;
std::mutex g_info_mu;
DeviceInfo g_info[kMaxDevices];

// Cooperative launch support and the resident workgroups of the kernel on the current device (both variants
// use the same resources; the smaller count is kept), looked up once per device.
const DeviceInfo* device_info() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_info_mu);
  DeviceInfo& d = g_info[dev];
  if (!d.init) {
    d.init = true;
    int coop = 0, cus = 0, n0 = 0, n1 = 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n0, decode_step_kernel<false>, kThreads, 0) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&n1, decode_step_kernel<true>, kThreads, 0) == hipSuccess) {
      d.max_groups = cus * (n0 < n1 ? n0 : n1);
      d.ok = coop != 0 && d.max_groups > 0;
    }
    (void)hipGetLastError();
  }
  return &d;
}

}  // namespace

bool decode_fused_shape_ok(int B, int C, int R) {
  return B >= 1 && B <= kMaxBatch && C % kUC == 0 && R % 32 == 0 && R <= kMaxR;
}

int decode_fused_slices(int C) { return C / kUC; }

bool decode_fused_available() {
  const DeviceInfo* d = device_info();
  return d && d->ok;
}

hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t st) {
  const DeviceInfo* d = device_info();
  if (!d || !d->ok) return hipErrorNotSupported;
  const int units = (a.B + kUT - 1) / kUT * (a.C / kUC);
  int groups = units > a.B ? units : a.B;
  if (groups > d->max_groups) groups = d->max_groups;
  if (groups > kDecodeMaxGroups) groups = kDecodeMaxGroups;
  DecodeArgs arg = a;
  arg.launch = next_launch_id();
  void* params[] = {&arg};
  const void* fn = a.zoh ? reinterpret_cast<const void*>(&decode_step_kernel<true>)
                         : reinterpret_cast<const void*>(&decode_step_kernel<false>);
  return hipLaunchCooperativeKernel(fn, dim3(groups), dim3(kThreads), params, 0, st);
}

}  // namespace jm
