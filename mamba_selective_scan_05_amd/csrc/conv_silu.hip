// Causal depthwise conv1d (kernel 4) + bias + SiLU: the mixer's first step.
//
// Each thread owns 16 bytes of channels (8 bf16 or 4 fp32) of one sequence and walks a run of tokens,
// keeping the three previous raw inputs in registers, so every input row is read once (plus a 3-row halo
// per run) with 16-byte loads and every output row written once with 16-byte stores: one coalesced pass
// at HBM speed.  The conv state supplies the left context of token 0.
#include <string.h>

#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

constexpr int kTaps = 4;

template <typename T>
struct Vec16 {
  static constexpr int n = 16 / sizeof(T);
  T v[n];
};

template <typename T>
__device__ __forceinline__ void load16(const T* p, float* out) {
  Vec16<T> r;
  uint4 raw = *reinterpret_cast<const uint4*>(p);
  memcpy(&r, &raw, 16);
#pragma unroll
  for (int i = 0; i < Vec16<T>::n; ++i) out[i] = io<T>::cvt(r.v[i]);
}

template <typename T>
__device__ __forceinline__ void unpack16(uint4 raw, float* out) {
  Vec16<T> r;
  memcpy(&r, &raw, 16);
#pragma unroll
  for (int i = 0; i < Vec16<T>::n; ++i) out[i] = io<T>::cvt(r.v[i]);
}

// rows per prefetch batch (B = 1, L = 4096, d_inner 8192: 29.6 us with 4, 33.1 with 8, 88 with 16)
constexpr int kRows = 4;

template <typename T>
__device__ __forceinline__ void store16(T* p, const float* in) {
  Vec16<T> r;
#pragma unroll
  for (int i = 0; i < Vec16<T>::n; ++i) r.v[i] = io<T>::from(in[i]);
  uint4 raw;
  memcpy(&raw, &r, 16);
  *reinterpret_cast<uint4*>(p) = raw;
}

template <typename T>
__global__ __launch_bounds__(256) void conv_silu_kernel(const T* __restrict__ x, int64_t xs,
                                                        const T* __restrict__ conv_w, const T* __restrict__ conv_b,
                                                        const T* __restrict__ conv_in, T* __restrict__ xc,
                                                        int L, int C, int run) {
  constexpr int V = Vec16<T>::n;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (c0 >= C) return;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * run;
  const int t1 = min(L, t0 + run);

  float w[V][kTaps], bias[V];
  {
    float wf[V * kTaps];
#pragma unroll
    for (int q = 0; q < V * kTaps; q += V) load16(conv_w + (int64_t)c0 * kTaps + q, wf + q);
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < kTaps; ++j) w[i][j] = wf[i * kTaps + j];
  }
  if (conv_b) {
    load16(conv_b + c0, bias);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) bias[i] = 0.0f;
  }

  // prev[j] = extended input at t - 3 + j
  float prev[kTaps - 1][V];
  if (t0 == 0) {
    if (conv_in) {
      // the state of these V channels is 3V contiguous elements (48 bytes): three 16-byte loads
      float st[(kTaps - 1) * V];
#pragma unroll
      for (int q = 0; q < kTaps - 1; ++q) load16(conv_in + ((int64_t)b * C + c0) * (kTaps - 1) + q * V, st + q * V);
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < kTaps - 1; ++j) prev[j][i] = st[i * (kTaps - 1) + j];
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < kTaps - 1; ++j) prev[j][i] = 0.0f;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTaps - 1; ++j) load16(x + ((int64_t)b * L + t0 - (kTaps - 1) + j) * xs + c0, prev[j]);
  }

  // Rows arrive in batches of kRows; the next batch's 16-byte loads are in flight while the current one is
  // computed (two register buffers used in turn).  Prefetch rows are clamped to the run, so they stay in
  // bounds without branches.
  const T* xb = x + (int64_t)b * L * xs + c0;
  T* ob = xc + (int64_t)b * L * C + c0;
  auto load_rows = [&](int tb, uint4* buf) {
#pragma unroll
    for (int j = 0; j < kRows; ++j) buf[j] = *reinterpret_cast<const uint4*>(xb + (int64_t)min(tb + j, t1 - 1) * xs);
  };
  auto conv_rows = [&](int tb, const uint4* buf) {
    const int count = min(kRows, t1 - tb);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
      if (j >= count) break;
      float cur[V], o[V];
      unpack16<T>(buf[j], cur);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        float u = bias[i];
        u = fmaf(w[i][0], prev[0][i], u);
        u = fmaf(w[i][1], prev[1][i], u);
        u = fmaf(w[i][2], prev[2][i], u);
        u = fmaf(w[i][3], cur[i], u);
        o[i] = silu(u);
        prev[0][i] = prev[1][i];
        prev[1][i] = prev[2][i];
        prev[2][i] = cur[i];
      }
      store16(ob + (int64_t)(tb + j) * C, o);
    }
  };
  uint4 bufA[kRows], bufB[kRows];
  load_rows(t0, bufA);
  for (int tb = t0; tb < t1; tb += 2 * kRows) {
    if (tb + kRows < t1) load_rows(tb + kRows, bufB);
    conv_rows(tb, bufA);
    if (tb + kRows >= t1) break;
    if (tb + 2 * kRows < t1) load_rows(tb + 2 * kRows, bufA);
    conv_rows(tb + kRows, bufB);
  }
}

// Packed batches: x is one axis of L tokens holding several sequences (v.cu).  A thread's run of tokens is
// walked as segments that each lie in one sequence, the rows of a segment as in conv_silu_kernel; a
// segment's left context comes from the sequence's earlier tokens or, at its start, from its conv state.
template <typename T>
__global__ __launch_bounds__(256) void conv_silu_varlen_kernel(const T* __restrict__ x, int64_t xs,
                                                               const T* __restrict__ conv_w,
                                                               const T* __restrict__ conv_b,
                                                               const T* __restrict__ conv_in, T* __restrict__ xc,
                                                               int L, int C, int run, VarSeqs v) {
  constexpr int V = Vec16<T>::n;
  constexpr int S3 = kTaps - 1;
  const int c0 = (blockIdx.x * blockDim.x + threadIdx.x) * V;
  if (c0 >= C) return;
  const int t0 = blockIdx.y * run;
  const int t1 = min(L, t0 + run);

  float w[V][kTaps], bias[V];
  {
    float wf[V * kTaps];
#pragma unroll
    for (int q = 0; q < V * kTaps; q += V) load16(conv_w + (int64_t)c0 * kTaps + q, wf + q);
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < kTaps; ++j) w[i][j] = wf[i * kTaps + j];
  }
  if (conv_b) {
    load16(conv_b + c0, bias);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) bias[i] = 0.0f;
  }
  const T* xb = x + c0;
  T* ob = xc + c0;

  // segments (offsets clamped so that every segment makes progress and every access stays in [0, L))
  for (int u0 = t0; u0 < t1;) {
    const int s = seq_of(v.cu, v.nseq, u0);
    const int S = min(max(v.cu[s], 0), u0);
    const int u1 = min(max(v.cu[s + 1], u0 + 1), t1);
    // prev[j] = extended input at u0 - 3 + j: the sequence's own tokens, else entries of its conv state
    // (3V contiguous elements for these V channels: three 16-byte loads)
    float prev[S3][V];
    if (u0 - S3 >= S) {
#pragma unroll
      for (int j = 0; j < S3; ++j) load16(xb + (int64_t)(u0 - S3 + j) * xs, prev[j]);
    } else {
      const int64_t srow = state_row(v.slots, v.pool, s);
      float st[S3 * V];
      if (conv_in && srow >= 0) {
#pragma unroll
        for (int q = 0; q < S3; ++q) load16(conv_in + (srow * C + c0) * S3 + q * V, st + q * V);
      } else {
#pragma unroll
        for (int q = 0; q < S3 * V; ++q) st[q] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < S3; ++j) {
        const int idx = u0 - S3 + j;
        if (idx >= S) {
          load16(xb + (int64_t)idx * xs, prev[j]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i) prev[j][i] = st[i * S3 + (idx - S + S3)];
        }
      }
    }
    // the segment's rows in batches of kRows, the next batch in flight while one is computed
    uint4 bufA[kRows], bufB[kRows];
    auto load_rows = [&](int tb, uint4* buf) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < kRows; ++j)
        buf[j] = *reinterpret_cast<const uint4*>(xb + (int64_t)min(tb + j, u1 - 1) * xs);
    };
    auto conv_rows = [&](int tb, const uint4* buf) __attribute__((always_inline)) {
      const int count = min(kRows, u1 - tb);
#pragma unroll
      for (int j = 0; j < kRows; ++j) {
        if (j >= count) break;
        float cur[V], o[V];
        unpack16<T>(buf[j], cur);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          float u = bias[i];
          u = fmaf(w[i][0], prev[0][i], u);
          u = fmaf(w[i][1], prev[1][i], u);
          u = fmaf(w[i][2], prev[2][i], u);
          u = fmaf(w[i][3], cur[i], u);
          o[i] = silu(u);
          prev[0][i] = prev[1][i];
          prev[1][i] = prev[2][i];
          prev[2][i] = cur[i];
        }
        store16(ob + (int64_t)(tb + j) * C, o);
      }
    };
    load_rows(u0, bufA);
    for (int tb = u0; tb < u1; tb += 2 * kRows) {
      if (tb + kRows < u1) load_rows(tb + kRows, bufB);
      conv_rows(tb, bufA);
      if (tb + kRows >= u1) break;
      if (tb + 2 * kRows < u1) load_rows(tb + 2 * kRows, bufA);
      conv_rows(tb + kRows, bufB);
    }
    u0 = u1;
  }
}

// One token per sequence (decode): each thread takes 16 bytes of channels; a workgroup takes 256 such groups
// of SPB consecutive sequences.  The conv weights (64 bytes per thread) are read once per workgroup, as
// contiguous 16-byte lanes into LDS, and kept in registers for all its sequences.  A sequence's conv state
// (48 bytes per thread) likewise arrives as contiguous 16-byte lanes, goes through LDS to the thread that
// owns it, and the shifted state goes back the same way: per-lane 48- or 64-byte strides would make every
// load instruction touch 3-4x as many cache lines.  The next sequence's state and input are in flight while
// the current one computes (with SPB > 1).  Each sequence's whole block is read before any of it is
// written, so conv_out may alias conv_in.
template <typename T, int SPB>
__global__ __launch_bounds__(256) void conv_step_kernel(const T* __restrict__ x, int64_t xs,
                                                        const T* __restrict__ conv_w, const T* __restrict__ conv_b,
                                                        const T* conv_in, T* __restrict__ xc, T* conv_out, int B,
                                                        int C, const int32_t* __restrict__ slots, int pool) {
  constexpr int V = Vec16<T>::n;
  constexpr int S3 = kTaps - 1;
  __shared__ uint4 sst[256 * S3], sw[256 * kTaps];
  const int tid = threadIdx.x;
  const int cbase = blockIdx.x * 256 * V;
  const int ng = min(256 * V, C - cbase) / V;          // channel groups of this block (C % 64 == 0)
  const int b0 = blockIdx.y * SPB;
  const int nb = min(SPB, B - b0);
  const int own = min(tid, ng - 1);                     // threads past the block recompute its last group
  {
    const uint4* gw = reinterpret_cast<const uint4*>(conv_w + (int64_t)cbase * kTaps);
    for (int k = tid; k < ng * kTaps; k += 256) sw[k] = gw[k];
  }
  float bias[V];
  if (conv_b) {
    load16(conv_b + cbase + own * V, bias);
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) bias[i] = 0.0f;
  }
  __syncthreads();
  float wf[V * kTaps];
#pragma unroll
  for (int q = 0; q < kTaps; ++q) unpack16<T>(sw[own * kTaps + q], wf + q * V);

  // sequence s: state chunks tid, tid + 256, tid + 512 (clamped to the block; zeros without a state) and the
  // thread's 16 bytes of input
  uint4 rs[S3], rx;
  // the state row of sequence b: b itself, or its slot in the pool (-1: none, a zero state stored nowhere)
  auto load_seq = [&](int s) {
    const int b = b0 + s;
    const int64_t row = state_row(slots, pool, b);
    const uint4* gst = reinterpret_cast<const uint4*>(conv_in + (max(row, (int64_t)0) * C + cbase) * S3);
#pragma unroll
    for (int q = 0; q < S3; ++q)
      rs[q] = conv_in && row >= 0 ? gst[min(tid + 256 * q, ng * S3 - 1)] : make_uint4(0u, 0u, 0u, 0u);
    rx = *reinterpret_cast<const uint4*>(x + b * xs + cbase + own * V);
  };
  load_seq(0);
  for (int s = 0; s < nb; ++s) {
    const int64_t b = b0 + s;
#pragma unroll
    for (int q = 0; q < S3; ++q)
      if (tid + 256 * q < ng * S3) sst[tid + 256 * q] = rs[q];
    const uint4 xcur = rx;
    __syncthreads();
    if (SPB > 1) load_seq(min(s + 1, nb - 1));         // the last sequence re-reads itself
    float st[S3 * V], cur[V];
#pragma unroll
    for (int q = 0; q < S3; ++q) unpack16<T>(sst[own * S3 + q], st + q * V);
    unpack16<T>(xcur, cur);
    float o[V], ns[S3 * V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float* s3 = st + i * S3;
      float u = bias[i];
      u = fmaf(wf[i * kTaps + 0], s3[0], u);
      u = fmaf(wf[i * kTaps + 1], s3[1], u);
      u = fmaf(wf[i * kTaps + 2], s3[2], u);
      u = fmaf(wf[i * kTaps + 3], cur[i], u);
      o[i] = silu(u);
      ns[i * S3 + 0] = s3[1];
      ns[i * S3 + 1] = s3[2];
      ns[i * S3 + 2] = cur[i];
    }
    __syncthreads();                                    // every thread has read its state from sst
    if (tid < ng) {
      store16(xc + b * C + cbase + tid * V, o);
#pragma unroll
      for (int q = 0; q < S3; ++q) store16(reinterpret_cast<T*>(&sst[tid * S3 + q]), ns + q * V);
    }
    __syncthreads();
    const int64_t row = state_row(slots, pool, (int)b);
    if (row < 0) continue;
    uint4* gout = reinterpret_cast<uint4*>(conv_out + (row * C + cbase) * S3);
#pragma unroll
    for (int q = 0; q < S3; ++q)
      if (tid + 256 * q < ng * S3) gout[tid + 256 * q] = sst[tid + 256 * q];
  }
}

template <typename T>
__global__ void state_passthrough_kernel(const T* __restrict__ conv_in, T* __restrict__ conv_out,
                                         const float* __restrict__ h0, float* __restrict__ h_out, int B, int C) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nc = (int64_t)B * C * (kTaps - 1), nh = (int64_t)B * C * 16;
  if (i < nc) {
    T v = conv_in ? conv_in[i] : io<T>::from(0.0f);
    conv_out[i] = v;
  }
  if (i < nh) {
    float v = h0 ? h0[i] : 0.0f;
    h_out[i] = v;
  }
}

// Per sequence of a packed batch (grid.x) and channel (grid.y blocks of 256): the conv state out, i.e. the
// last K-1 entries of the sequence's extended input (x after its conv state), and for an empty sequence
// the SSM state carried over.  Each thread reads its entries before it writes them and no two threads
// touch one element, so the outputs may alias the inputs.
template <typename T>
__global__ __launch_bounds__(256) void varlen_states_kernel(const T* x, int64_t xs, const T* conv_in, T* conv_out,
                                                            const float* h0, float* h_out, int C, int L,
                                                            VarSeqs v) {
  constexpr int S3 = kTaps - 1;
  const int s = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= C) return;
  const int64_t row = state_row(v.slots, v.pool, s);
  if (row < 0) return;
  const int S = min(max(v.cu[s], 0), L);
  const int E = min(max(v.cu[s + 1], S), L);
  const int len = E - S;
  const int64_t base = (row * C + c) * S3;
  T e[S3];
#pragma unroll
  for (int j = 0; j < S3; ++j) {
    const int idx = len - S3 + j;   // position in the sequence; negative: an entry of the old state
    if (idx >= 0) e[j] = x[(int64_t)(S + idx) * xs + c];
    else e[j] = conv_in ? conv_in[base + idx + S3] : io<T>::from(0.0f);
  }
#pragma unroll
  for (int j = 0; j < S3; ++j) conv_out[base + j] = e[j];
  if (len == 0) {
    const int64_t hb = (row * C + c) * 16;
    float hv[16];
#pragma unroll
    for (int n = 0; n < 16; ++n) hv[n] = h0 ? h0[hb + n] : 0.0f;
#pragma unroll
    for (int n = 0; n < 16; ++n) h_out[hb + n] = hv[n];
  }
}

}  // namespace

void launch_varlen_states(bool bf16, const void* x, int64_t xs, const void* conv_in, void* conv_out,
                          const float* h0, float* h_out, int C, int L, const VarSeqs& v, hipStream_t st) {
  dim3 grid((unsigned)v.nseq, (unsigned)((C + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(varlen_states_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x, xs,
                       (const bf16_t*)conv_in, (bf16_t*)conv_out, h0, h_out, C, L, v);
  else
    hipLaunchKernelGGL(varlen_states_kernel<float>, grid, dim3(256), 0, st, (const float*)x, xs,
                       (const float*)conv_in, (float*)conv_out, h0, h_out, C, L, v);
}

void launch_conv_silu(bool bf16, const void* x, int64_t xs, const void* conv_w, const void* conv_b,
                      const void* conv_in, void* xc, int B, int L, int C, hipStream_t st, const VarSeqs& v) {
  const int V = bf16 ? 8 : 4;
  const int run = 32;   // tokens per thread (16: 34.5 us, 64: 32.4 us with 8-row batches)
  dim3 block(256);
  dim3 grid((C / V + 255) / 256, (L + run - 1) / run, B);
  if (v.cu) {   // a packed batch: B == 1
    if (bf16)
      hipLaunchKernelGGL(conv_silu_varlen_kernel<bf16_t>, grid, block, 0, st, (const bf16_t*)x, xs,
                         (const bf16_t*)conv_w, (const bf16_t*)conv_b, (const bf16_t*)conv_in, (bf16_t*)xc, L, C,
                         run, v);
    else
      hipLaunchKernelGGL(conv_silu_varlen_kernel<float>, grid, block, 0, st, (const float*)x, xs,
                         (const float*)conv_w, (const float*)conv_b, (const float*)conv_in, (float*)xc, L, C, run,
                         v);
  } else if (bf16) {
    hipLaunchKernelGGL(conv_silu_kernel<bf16_t>, grid, block, 0, st, (const bf16_t*)x, xs,
                       (const bf16_t*)conv_w, (const bf16_t*)conv_b, (const bf16_t*)conv_in, (bf16_t*)xc, L, C,
                       run);
  } else {
    hipLaunchKernelGGL(conv_silu_kernel<float>, grid, block, 0, st, (const float*)x, xs, (const float*)conv_w,
                       (const float*)conv_b, (const float*)conv_in, (float*)xc, L, C, run);
  }
}

void launch_conv_head(bool bf16, const void* x, int64_t xs, const void* conv_w, const void* conv_b,
                      const void* conv_in, void* xc, int B, int L, int C, hipStream_t st) {
  const int V = bf16 ? 8 : 4;
  const int run = kTaps - 1;   // one run per sequence: its first 3 tokens
  dim3 grid((C / V + 255) / 256, 1, B);
  if (bf16)
    hipLaunchKernelGGL(conv_silu_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x, xs,
                       (const bf16_t*)conv_w, (const bf16_t*)conv_b, (const bf16_t*)conv_in, (bf16_t*)xc, L, C,
                       run);
  else
    hipLaunchKernelGGL(conv_silu_kernel<float>, grid, dim3(256), 0, st, (const float*)x, xs, (const float*)conv_w,
                       (const float*)conv_b, (const float*)conv_in, (float*)xc, L, C, run);
}

void launch_conv_step(bool bf16, const void* x, int64_t xs, const void* conv_w, const void* conv_b,
                      const void* conv_in, void* xc, void* conv_out, int B, int C, hipStream_t st,
                      const int32_t* slots, int pool) {
  constexpr int kSeqPerBlock = 1;   // measured at B = 256: 7.1 us, against 7.8 (2) and 9.5 (4): parallelism wins
  const int V = bf16 ? 8 : 4;
  dim3 grid((C / V + 255) / 256, (B + kSeqPerBlock - 1) / kSeqPerBlock);
  if (bf16)
    hipLaunchKernelGGL((conv_step_kernel<bf16_t, kSeqPerBlock>), grid, dim3(256), 0, st, (const bf16_t*)x, xs,
                       (const bf16_t*)conv_w, (const bf16_t*)conv_b, (const bf16_t*)conv_in, (bf16_t*)xc,
                       (bf16_t*)conv_out, B, C, slots, pool);
  else
    hipLaunchKernelGGL((conv_step_kernel<float, kSeqPerBlock>), grid, dim3(256), 0, st, (const float*)x, xs,
                       (const float*)conv_w, (const float*)conv_b, (const float*)conv_in, (float*)xc,
                       (float*)conv_out, B, C, slots, pool);
}

void launch_state_passthrough(bool bf16, const void* conv_in, void* conv_out, const float* h0, float* h_out,
                              int B, int C, hipStream_t st) {
  const int64_t n = (int64_t)B * C * 16;
  dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(state_passthrough_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)conv_in,
                       (bf16_t*)conv_out, h0, h_out, B, C);
  else
    hipLaunchKernelGGL(state_passthrough_kernel<float>, grid, dim3(256), 0, st, (const float*)conv_in,
                       (float*)conv_out, h0, h_out, B, C);
}

}  // namespace jm
