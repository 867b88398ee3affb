// The selective scan with the D skip and the SiLU(z) gate.
//
// Recurrence (Jamba Guide, "Inside the Mamba State-Space Layers", discretisation and recurrent state
// update):  h_t = exp(delta_t * A) * h_{t-1} + delta_t * B_t * xc_t,  y_t = C_t . h_t + D * xc_t,
// out_t = y_t * SiLU(z_t),  A = -exp(A_log).
//
// One lane owns one channel of one sequence and keeps its 16-wide fp32 state in registers; B_t and C_t
// are shared by every channel, so a wave reads them as wave-uniform (scalar) loads.  exp(delta * A) is
// evaluated as 2^(delta * A * log2 e) with A * log2 e precomputed per state.  Tokens are processed in
// batches of 4 whose per-channel loads (delta, xc, z) are issued one batch ahead, so HBM latency hides
// behind the arithmetic of the current batch.  The kernel is bound by the vector ALU (16 exponentials
// and about 64 other operations per token and channel), not by HBM.
//
// Two levels, so that short batches still fill the GPU: each sequence is cut into P pieces of Lp tokens.
//   local  : every piece but the last runs the recurrence from a zero state (piece 0 from the initial
//            state) and records its end state and the sum of its deltas;
//   carry  : per (sequence, channel, state) the pieces' incoming states follow from composing the affine
//            maps h -> exp(A * sum(delta)) * h + h_end_local in piece order;
//   full   : every piece reruns from its incoming state, producing the gated output; the last piece
//            writes the final SSM state and the conv state.
// With P = 1 only the full pass runs.
//
// A workgroup holds up to four waves: adjacent 64-channel groups of the same piece, one per SIMD of a CU, so
// that the four share the piece's B / C rows in the CU's scalar cache (measured against one-wave workgroups:
// the 256K prefill's local pass 15% faster, the whole scan 8%).
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

constexpr int kN = 16;
constexpr int kTaps = 4;
constexpr int kMaxScanWaves = 4;   // waves per workgroup of the local and full passes
constexpr int kBatch = 4;   // tokens per prefetch batch (keeps the pass under 128 VGPRs: 4 waves per SIMD)
// s_waitcnt operand (gfx9 encoding): scalar-memory count 0, vector-memory and export counts at their maxima
constexpr int kWaitScalar = 0xC07F;

// Buffer resource over [base, base + bytes): raw (untyped) accesses, 32-bit byte offsets.
constexpr int kBufferFlags = 0x00020000;   // dword 3 of a raw buffer descriptor on gfx9-family GPUs
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferFlags);
}

// A raw element held in a full 32-bit register: bf16 zero-extended (widened with a shift when used),
// fp32 as is.  Loads and stores go through a buffer resource with a per-lane byte offset (the channel)
// and a wave-uniform byte offset (the token row), so no per-access vector address arithmetic is needed.
template <typename T> struct Raw;
template <> struct Raw<bf16_t> {
  typedef uint32_t type;
  static __device__ __forceinline__ uint32_t ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  }
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b16(f2bf(v), r, voff, soff, 0);
  }
  static __device__ __forceinline__ float f(uint32_t v) { return __uint_as_float(v << 16); }
};
template <> struct Raw<float> {
  typedef float type;
  // the b32 buffer builtins move 32-bit integers: reinterpret, never convert
  static __device__ __forceinline__ float ld(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
  }
  static __device__ __forceinline__ void st(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
  }
  static __device__ __forceinline__ float f(float v) { return v; }
};

// a2[n] = A[c, n] * log2(e) = -exp(A_log[c, n]) * log2(e), with the hardware exp (about 1 ulp)
template <typename T>
__device__ __forceinline__ void load_a2(const T* A_log, int c, float* a2) {
#pragma unroll
  for (int n = 0; n < kN; ++n) a2[n] = -exp2_fast(io<T>::ld(A_log + (int64_t)c * kN + n) * kLog2e) * kLog2e;
}

// FULL = false: the local pass (end state + delta sum of a piece); FULL = true: the output pass.
// VAR: one packed axis of several sequences (a.cu).  A piece is walked as segments that each lie in one
// sequence; at a sequence start the state is reset to that sequence's initial state, and the local pass
// marks the piece as reset (its end state then no longer depends on the incoming state).  The full pass
// stores a sequence's final state where it ends.
// ZOH: the input matrix is the exact zero-order hold instead of dt * B (a variant of the same recurrence).
// SAVE (full pass of a plain batch): also write the state entering every backward piece, for the backward.
// A workgroup is blockDim.x / 64 waves over adjacent 64-channel groups; each wave has its own 4 KB LDS tile
// in the dynamic shared memory (blockDim.x / 64 tiles).
template <typename T, bool FULL, bool VAR, bool ZOH = false, bool SAVE = false>
__global__ __launch_bounds__(kMaxScanWaves * 64) void scan_pass_kernel(ScanArgs a) {
  const int lane = threadIdx.x & 63;
  const int cg = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);   // the wave's 64-channel group
  const int c = cg * 64 + lane;
  const int p = blockIdx.y;
  const int b = blockIdx.z;
  const int L = a.L, C = a.C, P = a.P;
  const int t0 = p * a.Lp, t1 = min(L, t0 + a.Lp);

  extern __shared__ __attribute__((aligned(16))) float scan_tiles[];
  float* hs = scan_tiles + (threadIdx.x >> 6) * 64 * kN;
  float a2[kN], h[kN];
  load_a2((const T*)a.A_log, c, a2);
  float Av[ZOH ? kN : 1], iA[ZOH ? kN : 1];
  if (ZOH) {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      Av[n] = -exp2_fast(io<T>::ld((const T*)a.A_log + (int64_t)c * kN + n) * kLog2e);
      iA[n] = 1.0f / Av[n];
    }
  }
  // the SSM state row of sequence b (VAR: of the sequence holding the piece's first token): b itself, or
  // its slot in a state pool (-1: none)
  int s = 0;
  int64_t srow = b;
  if (VAR) {
    s = seq_of(a.cu, a.nseq, t0);
    srow = state_row(a.slots, a.pool, s);
  } else if (a.slots) {
    srow = state_row(a.slots, a.pool, b);
  }
  auto init_state = [&](int64_t row) __attribute__((always_inline)) {
    if (a.h0 && row >= 0) {
      state_load(a.h0 + (row * C + cg * 64) * kN, hs, lane, h);
    } else {
#pragma unroll
      for (int n = 0; n < kN; ++n) h[n] = 0.0f;
    }
  };
  bool reset = false;
  if (FULL && P > 1) {
    const float* src = a.cin + ((int64_t)b * P + p) * kN * C + c;
#pragma unroll
    for (int n = 0; n < kN; ++n) h[n] = src[(int64_t)n * C];
  } else if (VAR ? a.cu[s] == t0 : p == 0) {
    init_state(srow);
    reset = true;
  } else {
#pragma unroll
    for (int n = 0; n < kN; ++n) h[n] = 0.0f;
  }
  const float Dc = FULL ? io<T>::ld((const T*)a.D + c) : 0.0f;
  // the state entering backward piece q (saved after the token before it; a boundary at this piece's start
  // is written here, one inside it after its token, so each boundary has a single writer)
  auto save_state = [&](int q) __attribute__((always_inline)) {
    float* dst = a.saved + ((int64_t)b * a.saved_P + q) * kN * C + c;
#pragma unroll
    for (int n = 0; n < kN; ++n) dst[(int64_t)n * C] = h[n];
  };
  if (SAVE && t0 % kBwdPiece == 0) save_state(t0 / kBwdPiece);

  // Per-piece buffer resources (the plan keeps a piece under 2 GiB), a per-lane channel offset and a
  // wave-uniform token offset.
  const int64_t row0 = (int64_t)b * L + t0;
  const int n_tok = t1 - t0;
  const int64_t zs = a.z_stride;
  const int64_t rows = n_tok > 0 ? n_tok : 1;
  const __amdgpu_buffer_rsrc_t dres = make_rsrc((const T*)a.delta + row0 * C, rows * C * (int64_t)sizeof(T));
  const __amdgpu_buffer_rsrc_t xres = make_rsrc((const T*)a.xc + row0 * C, rows * C * (int64_t)sizeof(T));
  const __amdgpu_buffer_rsrc_t zres = make_rsrc((const T*)a.z + row0 * zs, rows * zs * (int64_t)sizeof(T));
  const __amdgpu_buffer_rsrc_t ores = make_rsrc((T*)a.out + row0 * C, rows * C * (int64_t)sizeof(T));
  const uint32_t voff = (uint32_t)c * sizeof(T);
  const uint32_t row_bytes = (uint32_t)(C * sizeof(T)), zrow_bytes = (uint32_t)(zs * sizeof(T));
  // B and C were written by an earlier kernel and are read-only here: reading them through the constant
  // address space lets every wave fetch them with scalar loads.
  const __attribute__((address_space(4))) float* bcp =
      (const __attribute__((address_space(4))) float*)(a.bc + row0 * (2 * kN));

  // Raw per-channel inputs are held as 32-bit words (zero-extended for bf16) so that a load in flight
  // never has to be merged into a half register before it is needed.  Prefetch indices are clamped to the
  // piece, so loads past its end re-read its last token instead of branching.
  typedef typename Raw<T>::type R;
  auto load_batch = [&](int i0, R* d, R* x, R* z) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const uint32_t i = (uint32_t)min(i0 + j, n_tok - 1);
      d[j] = Raw<T>::ld(dres, voff, i * row_bytes);
      x[j] = Raw<T>::ld(xres, voff, i * row_bytes);
      if (FULL) z[j] = Raw<T>::ld(zres, voff, i * zrow_bytes);
    }
  };
  float sdt = 0.0f;
  // The decay factors exp(delta_t * A) of a token are computed as one group: the multiplies, then all the
  // exponentials back to back.  Issued one by one between the dependent FMAs, each exponential costs the
  // vector ALU noticeably more (measured: the full pass 7% and the local pass 9% slower).
  auto decay = [&](R d, float* e) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < kN; ++n) e[n] = Raw<T>::f(d) * a2[n];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < kN; ++n) e[n] = exp2_fast(e[n]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // SiLU(z) of a batch of tokens, each transcendental kind as one group
  auto gates = [&](const R* z, float* g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) g[j] = Raw<T>::f(z[j]) * -kLog2e;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) g[j] = 1.0f + exp2_fast(g[j]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) g[j] = Raw<T>::f(z[j]) * rcp_fast(g[j]);
    __builtin_amdgcn_sched_barrier(0);
  };
  // one token given its decay factors e and gate g: B_t / C_t come in as wave-uniform values
  auto step = [&](int i, R draw, R xraw, const float* e, float g, const float* Bt, const float* Ct) __attribute__((always_inline)) {
    const float dt = Raw<T>::f(draw);
    const float xv = Raw<T>::f(xraw);
    const float u = dt * xv;
    // the input term of state n: dt * x * B_n, or with ZOH (exp(dt A_n) - 1) / A_n * x * B_n
    auto input = [&](int n) __attribute__((always_inline)) {
      if (ZOH) return zoh_coef(dt, e[n], Av[ZOH ? n : 0], iA[ZOH ? n : 0]) * (xv * Bt[n]);
      return u * Bt[n];
    };
    if (FULL) {
      float y = 0.0f;
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        h[n] = fmaf(e[n], h[n], input(n));
        y = fmaf(Ct[n], h[n], y);
      }
      y = fmaf(Dc, xv, y);
      Raw<T>::st(ores, voff, (uint32_t)i * row_bytes, y * g);
      if (SAVE && (t0 + i + 1) % kBwdPiece == 0 && i + 1 < n_tok) save_state((t0 + i + 1) / kBwdPiece);
    } else {
#pragma unroll
      for (int n = 0; n < kN; ++n) h[n] = fmaf(e[n], h[n], input(n));
      sdt += dt;
    }
  };
  // B / C of the token being computed, fetched one token ahead.  Scalar loads may complete out of order,
  // so the only wait for them is "all scalar loads done": each token first waits for its own B / C, then
  // requests the next token's, then computes, and the request stays in flight for a whole token.
  float Bc[kN], Cc[kN];
  auto load_bc = [&](int i, float* Bt, float* Ct) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      Bt[n] = bcp[(int64_t)i * (2 * kN) + n];
      Ct[n] = FULL ? bcp[(int64_t)i * (2 * kN) + kN + n] : 0.0f;
    }
  };
  // A full batch of kBatch tokens starting at i0 whose inputs are in d/x/z; on entry Bc/Cc hold token i0's
  // B/C, on exit token i0 + kBatch's (clamped to the piece).
  auto run_full = [&](int i0, const R* d, const R* x, const R* z) __attribute__((always_inline)) {
    float g[kBatch];
    if (FULL) gates(z, g);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      float e[kN];
      decay(d[j], e);
      __builtin_amdgcn_s_waitcnt(kWaitScalar);
      __builtin_amdgcn_sched_barrier(0);
      float Bn[kN], Cn[kN];
      load_bc(min(i0 + j + 1, n_tok - 1), Bn, Cn);   // clamped: the last token re-reads its own row
      __builtin_amdgcn_sched_barrier(0);
      step(i0 + j, d[j], x[j], e, FULL ? g[j] : 0.0f, Bc, Cc);
#pragma unroll
      for (int n = 0; n < kN; ++n) {
        Bc[n] = Bn[n];
        Cc[n] = Cn[n];
      }
    }
  };

  // The steady state runs pairs of full batches with no branch inside: batch k computes from one register
  // set while batch k + 1 loads into the other.  The prefetches are unconditional (a batch past the end
  // re-reads the last token): a conditional one would make the compiler's wait at the join assume the
  // no-prefetch path, i.e. wait for the loads just issued.  Fewer than kBatch leftover tokens run one at a
  // time afterwards.
  R dA[kBatch], xA[kBatch], zA[kBatch], dB[kBatch], xB[kBatch], zB[kBatch];
  // tokens [i0, i1) of the piece
  auto run_range = [&](int i0, int i1) __attribute__((always_inline)) {
    const int nfull = (i1 - i0) / kBatch;
    if (i1 > i0) {
      load_batch(i0, dA, xA, zA);
      load_bc(i0, Bc, Cc);
    }
    int k = 0;
    for (; k + 2 <= nfull; k += 2) {
      load_batch(i0 + (k + 1) * kBatch, dB, xB, zB);
      run_full(i0 + k * kBatch, dA, xA, zA);
      load_batch(i0 + (k + 2) * kBatch, dA, xA, zA);
      run_full(i0 + (k + 1) * kBatch, dB, xB, zB);
    }
    if (k < nfull) {   // an odd last full batch, already loaded into dA / xA / zA
      run_full(i0 + k * kBatch, dA, xA, zA);
      ++k;
    }
    for (int i = i0 + k * kBatch; i < i1; ++i) {
      const R d = Raw<T>::ld(dres, voff, (uint32_t)i * row_bytes);
      const R x = Raw<T>::ld(xres, voff, (uint32_t)i * row_bytes);
      float e[kN];
#pragma unroll
      for (int n = 0; n < kN; ++n) e[n] = exp2_fast(Raw<T>::f(d) * a2[n]);
      const float g = FULL ? silu(Raw<T>::f(Raw<T>::ld(zres, voff, (uint32_t)i * zrow_bytes))) : 0.0f;
      float Bt[kN], Ct[kN];
      load_bc(i, Bt, Ct);
      step(i, d, x, e, g, Bt, Ct);
    }
  };

  if (!VAR) {
    run_range(0, n_tok);
  } else {
    // Segments, each inside one sequence (offsets clamped so every segment makes progress).  A sequence
    // that starts inside the piece and runs past it has its initial state read by the local pass (before
    // any final state is written) and saved in snap for the full pass: the piece that writes its final
    // state may run concurrently with this one, and the state rows may be updated in place.
    float* snap = a.snap + (int64_t)p * kN * C + c;
    for (int u = 0; u < n_tok;) {
      const int end = a.cu[s + 1] - t0;            // the sequence's end, relative to the piece
      const int u1 = min(max(end, u + 1), n_tok);
      run_range(u, u1);
      if (FULL && end <= n_tok && srow >= 0)      // the sequence ends in this piece
        state_store(a.h_out + (srow * C + cg * 64) * kN, hs, lane, h);
      u = u1;
      if (u >= n_tok) break;
      s = seq_of(a.cu, a.nseq, t0 + u);            // the next non-empty sequence starts at u
      srow = state_row(a.slots, a.pool, s);
      const bool spans = a.cu[s + 1] - t0 > n_tok;
      if (FULL && spans) {
#pragma unroll
        for (int n = 0; n < kN; ++n) h[n] = snap[(int64_t)n * C];
      } else {
        init_state(srow);
        if (!FULL && spans) {
#pragma unroll
          for (int n = 0; n < kN; ++n) snap[(int64_t)n * C] = h[n];
        }
      }
      reset = true;
    }
  }

  if (!FULL) {
    // the delta sum, or -1 when the piece resets the state (its end state is then independent of its
    // incoming state)
    float* dst = a.loc + ((int64_t)b * P + p) * (kN + 1) * C + c;
#pragma unroll
    for (int n = 0; n < kN; ++n) dst[(int64_t)n * C] = h[n];
    dst[(int64_t)kN * C] = VAR && reset ? -1.0f : sdt;
    return;
  }
  if (!VAR && p == P - 1) {
    if (srow < 0) return;
    state_store(a.h_out + (srow * C + cg * 64) * kN, hs, lane, h);
    // conv state (unless the conv step wrote it): the last K-1 entries of the extended input (old state
    // entries when L < K-1).  All three are read before any is written, so conv_out may alias conv_in.
    if (!a.conv_out) return;
    const T* x = (const T*)a.x;
    const T* ci = (const T*)a.conv_in;
    T v[kTaps - 1];
#pragma unroll
    for (int j = 0; j < kTaps - 1; ++j) {
      const int tau = L - (kTaps - 1) + j;
      if (tau >= 0) v[j] = x[((int64_t)b * L + tau) * a.x_stride + c];
      else v[j] = ci ? ci[((int64_t)b * C + c) * (kTaps - 1) + tau + (kTaps - 1)] : io<T>::from(0.0f);
    }
    T* co = (T*)a.conv_out + ((int64_t)b * C + c) * (kTaps - 1);
#pragma unroll
    for (int j = 0; j < kTaps - 1; ++j) co[j] = v[j];
  }
}

// VAR: a piece whose first token starts a sequence takes that sequence's initial state as its incoming
// state, and a piece marked as reset (delta sum -1) passes on its local end state alone.
template <typename T, bool VAR>
__global__ __launch_bounds__(256) void scan_carry_kernel(const float* __restrict__ loc, const T* __restrict__ A_log,
                                                         const float* __restrict__ h0, float* __restrict__ cin,
                                                         int B, int C, int P, ScanArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over (b, n, c)
  if (i >= (int64_t)B * kN * C) return;
  const int c = (int)(i % C);
  const int n = (int)((i / C) % kN);
  const int b = (int)(i / ((int64_t)C * kN));
  const float a2 = -exp2_fast(io<T>::ld(A_log + (int64_t)c * kN + n) * kLog2e) * kLog2e;
  const float* lb = loc + (int64_t)b * P * (kN + 1) * C;
  float* cb = cin + (int64_t)b * P * kN * C;
  float H = 0.0f;
  if (!VAR) {
    const int64_t row = state_row(a.slots, a.pool, b);
    cb[(int64_t)n * C + c] = h0 && row >= 0 ? h0[(row * C + c) * kN + n] : 0.0f;
    H = lb[(int64_t)n * C + c];   // piece 0 started from h0: its end state is exact
  }
  // pieces in groups (16 for plain batches; 8 for packed batches, which also look up each piece's sequence):
  // all loads of a group are issued before its serial combine, so a group costs one memory latency.  With
  // 128 pieces (256K tokens) groups of 16 against 8 took the pass from 38.5 to 29.4 us (rocprofv3); groups of
  // 32 made the 16-piece B = 8 case slower (30 -> 37 us: the clamped surplus loads and the registers).
  constexpr int kG = VAR ? 8 : 16;
  for (int p0 = VAR ? 0 : 1; p0 < P; p0 += kG) {
    float hl[kG], sd[kG], hi[kG];
    bool starts[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int p = min(p0 + j, P - 1);
      const float* lp = lb + (int64_t)p * (kN + 1) * C;
      hl[j] = lp[(int64_t)n * C + c];
      sd[j] = lp[(int64_t)kN * C + c];
      starts[j] = false;
      hi[j] = 0.0f;
      if (VAR) {
        const int tp = p * a.Lp;
        const int s = seq_of(a.cu, a.nseq, tp);
        starts[j] = a.cu[s] == tp;
        const int64_t row = state_row(a.slots, a.pool, s);
        if (starts[j] && h0 && row >= 0) hi[j] = h0[(row * C + c) * kN + n];
      }
    }
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int p = p0 + j;
      if (p < P) {
        if (VAR && starts[j]) H = hi[j];
        cb[((int64_t)p * kN + n) * C + c] = H;
        // unused after the last piece
        H = VAR && sd[j] < 0.0f ? hl[j] : fmaf(exp2_fast(sd[j] * a2), H, hl[j]);
      }
    }
  }
}

// Waves per workgroup of the passes: four when d_inner allows it (a multiple of 256), else two or one.
int scan_waves(int C) { return C % (64 * 4) == 0 ? 4 : C % (64 * 2) == 0 ? 2 : 1; }

template <typename T, bool VAR, bool ZOH>
void run_scan(const ScanArgs& a, hipStream_t st, void* const* marks) {
  const int wpb = scan_waves(a.C);
  const dim3 block(64 * wpb);
  const size_t lds = (size_t)wpb * 64 * kN * sizeof(float);
  auto mark = [&](int i) {
    if (marks) (void)hipEventRecord((hipEvent_t)marks[i], st);
  };
  mark(0);
  if (a.P > 1) {
    dim3 gl(a.C / (64 * wpb), a.P - 1, a.B);
    hipLaunchKernelGGL((scan_pass_kernel<T, false, VAR, ZOH>), gl, block, lds, st, a);
  }
  mark(1);
  if (a.P > 1) {
    const int64_t n = (int64_t)a.B * kN * a.C;
    hipLaunchKernelGGL((scan_carry_kernel<T, VAR>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.loc,
                       (const T*)a.A_log, a.h0, a.cin, a.B, a.C, a.P, a);
  }
  mark(2);
  dim3 gf(a.C / (64 * wpb), a.P, a.B);
  if constexpr (!VAR && !ZOH) {
    if (a.saved) {
      hipLaunchKernelGGL((scan_pass_kernel<T, true, false, false, true>), gf, block, lds, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((scan_pass_kernel<T, true, VAR, ZOH>), gf, block, lds, st, a);
}

template <typename T>
void run_scan_t(const ScanArgs& a, hipStream_t st, void* const* marks) {
  if (a.cu) {
    if (a.zoh) run_scan<T, true, true>(a, st, marks);
    else run_scan<T, true, false>(a, st, marks);
  } else {
    if (a.zoh) run_scan<T, false, true>(a, st, marks);
    else run_scan<T, false, false>(a, st, marks);
  }
}

}  // namespace

void launch_scan_carries(bool bf16, const ScanArgs& a, hipStream_t st) {
  if (a.P <= 1) return;
  const int64_t n = (int64_t)a.B * kN * a.C;
  const int wpb = scan_waves(a.C);
  const size_t lds = (size_t)wpb * 64 * kN * sizeof(float);
  dim3 gl(a.C / (64 * wpb), a.P - 1, a.B);
  if (bf16) {
    hipLaunchKernelGGL((scan_pass_kernel<bf16_t, false, false>), gl, dim3(64 * wpb), lds, st, a);
    hipLaunchKernelGGL((scan_carry_kernel<bf16_t, false>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.loc,
                       (const bf16_t*)a.A_log, a.h0, a.cin, a.B, a.C, a.P, a);
  } else {
    hipLaunchKernelGGL((scan_pass_kernel<float, false, false>), gl, dim3(64 * wpb), lds, st, a);
    hipLaunchKernelGGL((scan_carry_kernel<float, false>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.loc,
                       (const float*)a.A_log, a.h0, a.cin, a.B, a.C, a.P, a);
  }
}

void launch_scan(bool bf16, const ScanArgs& a, hipStream_t st, void* const* marks) {
  if (bf16) run_scan_t<bf16_t>(a, st, marks);
  else run_scan_t<float>(a, st, marks);
}

}  // namespace jm
