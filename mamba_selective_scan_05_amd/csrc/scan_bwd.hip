// Backward of the gated selective scan (the training direction).
//
// Forward (Jamba Guide, "Inside the Mamba State-Space Layers", discretisation and recurrent state update):
//   a_t = exp(delta_t * A),  h_t = a_t * h_{t-1} + delta_t * B_t * x_t,  y_t = C_t . h_t + D * x_t,
//   out_t = y_t * SiLU(z_t),  A = -exp(A_log).
// Backward (the chain rule in reverse time): with dy_t = dout_t * SiLU(z_t) and u_t the gradient reaching h_t
// from later tokens, g_t = u_t + C_t * dy_t is h_t's total gradient and u_{t-1} = a_t * g_t; then
//   d delta_t = sum_n g (h_{t-1} a A + B x),  d x_t = sum_n g delta B + D dy,  d z_t = dout y SiLU'(z),
//   d B_t = sum_c g delta x,  d C_t = sum_c dy h_t,  d A = sum_t g h_{t-1} a delta,  d D = sum_t dy x.
//
// Layout: four lanes per channel, each holding four of its 16 states (lane 4c + q holds states 4q..4q+3), so
// a workgroup of 256 lanes covers 64 channels.  Sums over a channel's states (y, d delta, d x) are quad DPP
// reductions; the sums over channels of d B / d C are DPP row reductions (the four lanes of a row that hold
// the same states), then a sum over the block's 16 rows in LDS, then over blocks in a reduce kernel.
//
// Time is cut into pieces of kPiece tokens, as in the forward: the forward's local and carry passes give
// every piece its incoming state; a backward local pass runs each piece's gradient recurrence from zero and
// records what leaves its first token (and the piece's delta sum); a backward carry composes those in reverse
// piece order; the full pass then reruns each piece with both its incoming state and incoming gradient.
// Inside a piece the full pass first runs forward, keeping the state at every kSub-th token in LDS, then
// walks the sub-chunks last to first: it recomputes a sub-chunk's states into registers and runs the
// gradient recurrence backwards through them.
#include "jm_device.h"
#include "jm_launch.h"

namespace jm {

namespace {

constexpr int kN = 16;
constexpr int kQ = 4;                  // states per lane
constexpr int kSub = 16;               // tokens per recomputed sub-chunk
constexpr int kPiece = kBwdPiece;      // tokens per piece (a multiple of kSub)
constexpr int kNSub = kPiece / kSub;
static_assert(kPiece % kSub == 0, "pieces hold whole sub-chunks");

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// sum over the four lanes of a quad (the four state groups of one channel), in every lane
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  return v;
}
// sum over the four lanes of a 16-lane row holding the same state group (stride 4), in every lane
__device__ __forceinline__ float row_q_sum(float v) {
  v += dpp<0x124>(v);  // row_ror:4
  v += dpp<0x128>(v);  // row_ror:8
  return v;
}

struct Lane {
  int c;       // channel
  int q;       // state group: states 4q .. 4q+3
};

__device__ __forceinline__ Lane lane_of() {
  Lane l;
  l.c = blockIdx.x * 64 + (threadIdx.x >> 2);
  l.q = threadIdx.x & 3;
  return l;
}

template <typename T>
__device__ __forceinline__ void load_A(const T* A_log, const Lane& l, float* A, float* a2) {
#pragma unroll
  for (int i = 0; i < kQ; ++i) {
    A[i] = -exp2_fast(io<T>::ld(A_log + (int64_t)l.c * kN + l.q * kQ + i) * kLog2e);
    a2[i] = A[i] * kLog2e;
  }
}

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void st4(float* p, const float* v) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}

// Backward local pass: pieces 1 .. P-1 run the gradient recurrence from zero at their end and record
// u at their first token (what flows into the previous piece) and their delta sum:
// bloc [B, P, N + 1, C] (state n at row n, the delta sum at row N).
template <typename T>
__global__ __launch_bounds__(256) void bwd_local_kernel(BwdArgs a) {
  const Lane l = lane_of();
  const int p = blockIdx.y + 1;
  const int b = blockIdx.z;
  const int C = a.C, L = a.L, P = a.P;
  const int t0 = p * kPiece, t1 = min(L, t0 + kPiece);
  float A[kQ], a2[kQ];
  load_A((const T*)a.A_log, l, A, a2);
  const int64_t row0 = (int64_t)b * L;
  float u[kQ] = {0.0f, 0.0f, 0.0f, 0.0f};
  float sdt = 0.0f;
  for (int t = t1 - 1; t >= t0; --t) {
    const int64_t r = row0 + t;
    const float d = io<T>::ld((const T*)a.delta + r * C + l.c);
    const float zv = io<T>::ld((const T*)a.z + r * C + l.c);
    const float dout = io<T>::ld((const T*)a.dout + r * C + l.c);
    const f32x4 Cv = ld4(a.bc + r * (2 * kN) + kN + l.q * kQ);
    const float dy = dout * silu(zv);
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
      const float g = fmaf(Cv[i], dy, u[i]);
      u[i] = exp2_fast(d * a2[i]) * g;
    }
    sdt += d;
  }
  float* dst = a.bloc + ((int64_t)b * P + p) * (kN + 1) * C + l.c;
#pragma unroll
  for (int i = 0; i < kQ; ++i) dst[(int64_t)(l.q * kQ + i) * C] = u[i];
  if (l.q == 0) dst[(int64_t)kN * C] = sdt;
}

// Backward carry: per (b, n, c), the gradient entering each piece from later tokens:
// gin[p] = dh_final for the last piece, gin[p-1] = exp(A * sum(delta_p)) * gin[p] + u_local[p].
template <typename T>
__global__ __launch_bounds__(256) void bwd_carry_kernel(BwdArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over (b, n, c)
  const int C = a.C, P = a.P;
  if (i >= (int64_t)a.B * kN * C) return;
  const int c = (int)(i % C);
  const int n = (int)((i / C) % kN);
  const int b = (int)(i / ((int64_t)C * kN));
  const float a2 = -exp2_fast(io<T>::ld((const T*)a.A_log + (int64_t)c * kN + n) * kLog2e) * kLog2e;
  const float* lb = a.bloc + (int64_t)b * P * (kN + 1) * C;
  float* gb = a.gin + (int64_t)b * P * kN * C;
  float U = a.dh_final ? a.dh_final[((int64_t)b * C + c) * kN + n] : 0.0f;
  constexpr int kG = 8;
  for (int p0 = P - 1; p0 >= 0; p0 -= kG) {
    float ul[kG], sd[kG];
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int p = max(p0 - j, 1);     // piece 0 has no local record (its u leaves the sequence)
      const float* lp = lb + (int64_t)p * (kN + 1) * C;
      ul[j] = lp[(int64_t)n * C + c];
      sd[j] = lp[(int64_t)kN * C + c];
    }
#pragma unroll
    for (int j = 0; j < kG; ++j) {
      const int p = p0 - j;
      if (p >= 0) {
        gb[((int64_t)p * kN + n) * C + c] = U;
        U = fmaf(exp2_fast(sd[j] * a2), U, ul[j]);   // unused after piece 0
      }
    }
  }
}

// Full backward pass of one piece (see the file comment).  Partial sums leave through the workspace:
//   pA [B*P, C, N]  per-piece sums of g h_{t-1} a delta (d A before the factor A)
//   pD [B*P, C]     per-piece sums of dy x
//   pbc [C/64, B*L, 2N]  per-block sums over its 64 channels of d B (columns 0..N-1) and d C (N..2N-1)
template <typename T>
__global__ __launch_bounds__(256, 2) void bwd_full_kernel(BwdArgs a) {
  const Lane l = lane_of();
  const int p = blockIdx.y;
  const int b = blockIdx.z;
  const int C = a.C, L = a.L, P = a.P;
  const int t0 = p * kPiece, t1 = min(L, t0 + kPiece);
  const int n_tok = t1 - t0;
  const int nsub = (n_tok + kSub - 1) / kSub;
  const int64_t row0 = (int64_t)b * L + t0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ __attribute__((aligned(16))) float ck[kNSub][256][kQ];       // state at each sub-chunk start
  __shared__ float red[kSub][16][2 * kQ * 4 + 1];                          // per-row d B / d C sums (+1 pad)

  float A[kQ], a2[kQ];
  load_A((const T*)a.A_log, l, A, a2);
  const float Dc = io<T>::ld((const T*)a.D + l.c);
  const T* dl = (const T*)a.delta + row0 * C + l.c;
  const T* xl = (const T*)a.xc + row0 * C + l.c;
  const T* zl = (const T*)a.z + row0 * C + l.c;
  const T* ol = (const T*)a.dout + row0 * C + l.c;
  const float* bcl = a.bc + row0 * (2 * kN) + l.q * kQ;

  // incoming state and incoming gradient of the piece
  float h[kQ], u[kQ];
  {
    const int64_t base = ((int64_t)b * P + p) * kN * C + l.c;
#pragma unroll
    for (int i = 0; i < kQ; ++i) {
      const int n = l.q * kQ + i;
      if (P > 1) {
        h[i] = a.cin[base + (int64_t)n * C];
        u[i] = a.gin[base + (int64_t)n * C];
      } else {
        h[i] = a.h0 ? a.h0[((int64_t)b * C + l.c) * kN + n] : 0.0f;
        u[i] = a.dh_final ? a.dh_final[((int64_t)b * C + l.c) * kN + n] : 0.0f;
      }
    }
  }

  // forward through the piece, saving the state at each sub-chunk start
  for (int k = 0; k < nsub; ++k) {
    *reinterpret_cast<f32x4*>(&ck[k][threadIdx.x][0]) = f32x4{h[0], h[1], h[2], h[3]};
    const int j1 = min(kSub, n_tok - k * kSub);
    for (int j = 0; j < j1; ++j) {
      const int i = k * kSub + j;
      const float d = io<T>::ld(dl + (int64_t)i * C);
      const float dx = d * io<T>::ld(xl + (int64_t)i * C);
      const f32x4 Bv = ld4(bcl + (int64_t)i * (2 * kN));
#pragma unroll
      for (int s = 0; s < kQ; ++s) h[s] = fmaf(exp2_fast(d * a2[s]), h[s], dx * Bv[s]);
    }
  }

  float dA[kQ] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dD = 0.0f;
  for (int k = nsub - 1; k >= 0; --k) {
    const int len = min(kSub, n_tok - k * kSub);
    // recompute the sub-chunk's states: hist[j] = state after its token j; keep delta, x and the gate terms
    float hist[kSub][kQ], dv[kSub], xv[kSub], dyv[kSub], dzf[kSub];
    float hs[kQ];
    {
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(&ck[k][threadIdx.x][0]);
#pragma unroll
      for (int s = 0; s < kQ; ++s) hs[s] = c4[s];
    }
#pragma unroll
    for (int s = 0; s < kQ; ++s) h[s] = hs[s];
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if (j < len) {
        const int i = k * kSub + j;
        const float d = io<T>::ld(dl + (int64_t)i * C);
        const float x = io<T>::ld(xl + (int64_t)i * C);
        const float zv = io<T>::ld(zl + (int64_t)i * C);
        const float dout = io<T>::ld(ol + (int64_t)i * C);
        const f32x4 Bv = ld4(bcl + (int64_t)i * (2 * kN));
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          h[s] = fmaf(exp2_fast(d * a2[s]), h[s], d * x * Bv[s]);
          hist[j][s] = h[s];
        }
        const float sg = rcp_fast(1.0f + exp2_fast(-zv * kLog2e));   // sigmoid(z)
        dv[j] = d;
        xv[j] = x;
        dyv[j] = dout * zv * sg;                                     // dout * SiLU(z)
        dzf[j] = dout * sg * fmaf(zv, 1.0f - sg, 1.0f);              // dout * SiLU'(z)
      }
    }
    // the gradient recurrence backwards through the sub-chunk
#pragma unroll
    for (int j = kSub - 1; j >= 0; --j) {
      if (j < len) {
        const int i = k * kSub + j;
        const f32x4 Bv = ld4(bcl + (int64_t)i * (2 * kN));
        const f32x4 Cv = ld4(bcl + (int64_t)i * (2 * kN) + kN);
        const float d = dv[j], x = xv[j], dy = dyv[j];
        float pdd = 0.0f, pdx = 0.0f, py = 0.0f;
        float vb[kQ], vc[kQ];
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          const float hp = j > 0 ? hist[j > 0 ? j - 1 : 0][s] : hs[s];
          const float e = exp2_fast(d * a2[s]);
          const float g = fmaf(Cv[s], dy, u[s]);
          const float ghe = g * hp * e;
          pdd = fmaf(ghe, A[s], fmaf(g * Bv[s], x, pdd));
          pdx = fmaf(g * d, Bv[s], pdx);
          dA[s] = fmaf(ghe, d, dA[s]);
          vb[s] = g * d * x;
          vc[s] = dy * hist[j][s];
          py = fmaf(Cv[s], hist[j][s], py);
          u[s] = e * g;
        }
        pdd = quad_sum(pdd);
        pdx = quad_sum(pdx);
        py = quad_sum(py);
        if (l.q == 0) {
          const int64_t r = (row0 + i) * C + l.c;
          io<T>::st((T*)a.ddelta + r, pdd);
          io<T>::st((T*)a.dxc + r, fmaf(Dc, dy, pdx));
          io<T>::st((T*)a.dz + r, fmaf(Dc, x, py) * dzf[j]);
        }
        dD = fmaf(dy, x, dD);
        // d B / d C of this token summed over the row's four channels; lanes 0..3 of each row keep them
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          vb[s] = row_q_sum(vb[s]);
          vc[s] = row_q_sum(vc[s]);
        }
        if ((lane & 15) < 4) {
          float* rr = &red[j][wave * 4 + (lane >> 4)][l.q * 2 * kQ];
#pragma unroll
          for (int s = 0; s < kQ; ++s) {
            rr[s] = vb[s];
            rr[kQ + s] = vc[s];
          }
        }
      }
    }
    __syncthreads();
    // sum the block's 16 rows and write this block's partial d B / d C for the sub-chunk's tokens
    for (int o = threadIdx.x; o < len * 2 * kN; o += 256) {
      const int j = o / (2 * kN), col = o % (2 * kN);
      // column col: d B (col < N) or d C of state n = col % N, held by state group n / 4 at slot n % 4
      const int n = col % kN, q = n / kQ;
      const int slot = q * 2 * kQ + (col < kN ? 0 : kQ) + n % kQ;
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += red[j][r][slot];
      a.pbc[((int64_t)blockIdx.x * a.B * L + row0 + k * kSub + j) * (2 * kN) + col] = sum;
    }
    __syncthreads();
  }

  // per-piece partials of d A and d D, and d h0 from the first piece
  const int64_t bp = (int64_t)b * P + p;
  st4(a.pA + (bp * C + l.c) * kN + l.q * kQ, dA);
  if (l.q == 0) a.pD[bp * C + l.c] = dD;
  if (p == 0 && a.dh0) st4(a.dh0 + ((int64_t)b * C + l.c) * kN + l.q * kQ, u);
}

// d B / d C = sum of the per-block partials; d A_log = A * sum over pieces; d D = sum over pieces.
__global__ __launch_bounds__(256) void bwd_reduce_bc_kernel(const float* __restrict__ pbc, float* __restrict__ dbc,
                                                            int64_t rows, int nblk) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over rows * 2N
  if (i >= rows * 2 * kN) return;
  float s = 0.0f;
  for (int k = 0; k < nblk; ++k) s += pbc[(int64_t)k * rows * 2 * kN + i];
  dbc[i] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(const float* __restrict__ pA,
                                                                const float* __restrict__ pD,
                                                                const T* __restrict__ A_log, float* __restrict__ dA_log,
                                                                float* __restrict__ dD, int C, int npieces) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // over C * N
  if (i >= C * kN) return;
  float s = 0.0f;
  for (int k = 0; k < npieces; ++k) s += pA[(int64_t)k * C * kN + i];
  const float A = -exp2_fast(io<T>::ld(A_log + i) * kLog2e);
  dA_log[i] = s * A;
  if (i < C) {
    float sd = 0.0f;
    for (int k = 0; k < npieces; ++k) sd += pD[(int64_t)k * C + i];
    dD[i] = sd;
  }
}

template <typename T>
void run_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.P > 1) {
    hipLaunchKernelGGL(bwd_local_kernel<T>, dim3(a.C / 64, a.P - 1, a.B), dim3(256), 0, st, a);
    const int64_t n = (int64_t)a.B * kN * a.C;
    hipLaunchKernelGGL(bwd_carry_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  }
  hipLaunchKernelGGL(bwd_full_kernel<T>, dim3(a.C / 64, a.P, a.B), dim3(256), 0, st, a);
  const int64_t rows = (int64_t)a.B * a.L;
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3((unsigned)((rows * 2 * kN + 255) / 256)), dim3(256), 0, st, a.pbc,
                     a.dbc, rows, a.C / 64);
  hipLaunchKernelGGL(bwd_reduce_params_kernel<T>, dim3((a.C * kN + 255) / 256), dim3(256), 0, st, a.pA, a.pD,
                     (const T*)a.A_log, a.dA_log, a.dD, a.C, a.B * a.P);
}

}  // namespace

void launch_scan_backward(bool bf16, const BwdArgs& a, hipStream_t st) {
  if (bf16) run_bwd<bf16_t>(a, st);
  else run_bwd<float>(a, st);
}

}  // namespace jm
