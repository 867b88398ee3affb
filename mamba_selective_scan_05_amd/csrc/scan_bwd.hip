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
// reductions; the sums over channels of d B / d C take one DPP step over pairs of channels, then a sum over the
// block's 32 pairs in LDS after each sub-chunk, then over blocks in a reduce kernel.
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
// Tile sizes measured at B=1, L=4096, d_inner 8192 (bf16): sub-chunks of 4 tokens in pieces of 32 (registers for four
// waves per SIMD) took 1073 us for the whole backward, against 1106 (8 / 64, two waves), 1174 (4 / 16) and
// 1244 (8 / 32, three waves); keeping the decay factors and prefetching every input won over recomputing.
constexpr int kSub = 4;                // tokens per recomputed sub-chunk
// The second __launch_bounds__ argument: it caps the registers at 128.  The LDS (53 KB per workgroup) then
// holds three workgroups per CU, i.e. three waves per SIMD, so the compiler reports its target of four unmet; a
// target of three (130 registers) measured the same (backward 827-830 against 830-835 us).
constexpr int kBwdWavesPerSimd = 4;
constexpr int kPiece = kBwdPiece;      // tokens per piece (a multiple of kSub)
constexpr int kNSub = kPiece / kSub;
static_assert(kPiece % kSub == 0, "pieces hold whole sub-chunks");

template <bool B> struct Flag { static constexpr bool value = B; };

// v read from another lane of the same row (every lane valid for these controls); as a plain DPP move with
// full masks the compiler folds it into the add that consumes it (v_add_f32 with a DPP source)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// sum over the four lanes of a quad (the four state groups of one channel), in every lane.  Contraction is
// off so that the product feeding a sum is not folded into it: each step stays one add with a DPP source.
__device__ __forceinline__ float quad_sum(float v) {
#pragma clang fp contract(off)
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  return v;
}
// lane r of a 16-lane row plus lane r + 4 (mod 16): the sum over a pair of channels of one state group; lanes
// 0..3 and 8..11 of a row hold the sums of channel pairs (0, 1) and (2, 3)
__device__ __forceinline__ float pair_sum(float v) {
#pragma clang fp contract(off)
  return v + dpp<0x124>(v);  // row_ror:4
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

// One channel's column of a [rows, C] io-dtype tensor over a piece's rows, through a raw buffer resource:
// the lane's channel is the vector offset and the token row a wave-uniform scalar offset, so a load or
// store needs no per-lane address arithmetic.
constexpr int kBufFlags = 0x00020000;   // dword 3 of a raw buffer descriptor on gfx9-family GPUs
template <typename T>
struct Col {
  __amdgpu_buffer_rsrc_t r;
  uint32_t voff, row_bytes;
  __device__ __forceinline__ Col(const void* base, int64_t row0, int rows, int C, int c) {
    const int64_t bytes = (int64_t)(rows > 0 ? rows : 1) * C * sizeof(T);
    r = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>((const T*)base + row0 * C), (short)0, (int)bytes,
                                          kBufFlags);
    voff = (uint32_t)c * sizeof(T);
    row_bytes = (uint32_t)C * sizeof(T);
  }
  __device__ __forceinline__ float ld(int i) const;
  __device__ __forceinline__ void st(int i, float v) const;
};
template <>
__device__ __forceinline__ float Col<bf16_t>::ld(int i) const {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, (uint32_t)i * row_bytes, 0) << 16);
}
template <>
__device__ __forceinline__ void Col<bf16_t>::st(int i, float v) const {
  __builtin_amdgcn_raw_buffer_store_b16(f2bf(v), r, voff, (uint32_t)i * row_bytes, 0);
}
template <>
__device__ __forceinline__ float Col<float>::ld(int i) const {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, (uint32_t)i * row_bytes, 0));
}
template <>
__device__ __forceinline__ void Col<float>::st(int i, float v) const {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, (uint32_t)i * row_bytes, 0);
}

// Backward local pass: pieces 1 .. P-1 run the gradient recurrence from zero at their end and record
// u at their first token (what flows into the previous piece) and their delta sum:
// bloc [B, P, N + 1, C] (state n at row n, the delta sum at row N).  Only the recurrence of u runs here, so a
// lane takes a whole channel (all 16 states), and the piece's C rows, shared by every channel, are read from
// LDS as broadcasts.
template <typename T>
__global__ __launch_bounds__(64) void bwd_local_kernel(BwdArgs a) {
  const int c = blockIdx.x * 64 + threadIdx.x;
  const int p = blockIdx.y + 1;
  const int b = blockIdx.z;
  const int C = a.C, L = a.L, P = a.P;
  const int t0 = p * kPiece, t1 = min(L, t0 + kPiece);
  const int n_tok = t1 - t0;
  const int64_t row0 = (int64_t)b * L + t0;
  __shared__ f32x4 sc[kPiece][kN / 4];
  for (int o = threadIdx.x; o < n_tok * (kN / 4); o += 64)
    sc[o / (kN / 4)][o % (kN / 4)] = ld4(a.bc + (row0 + o / (kN / 4)) * (2 * kN) + kN + (o % (kN / 4)) * 4);
  float a2[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) a2[n] = -exp2_fast(io<T>::ld((const T*)a.A_log + (int64_t)c * kN + n) * kLog2e) * kLog2e;
  const Col<T> dl(a.delta, row0, n_tok, C, c), zl(a.z, row0, n_tok, C, c), ol(a.dout, row0, n_tok, C, c);
  __syncthreads();
  float u[kN];
#pragma unroll
  for (int n = 0; n < kN; ++n) u[n] = 0.0f;
  float sdt = 0.0f;
  // tokens last to first in batches whose loads are all issued first (indices clamped to the piece)
  constexpr int kBatch = 8;
  for (int ib = n_tok - 1; ib >= 0; ib -= kBatch) {
    float dd[kBatch], dy[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int i = max(ib - j, 0);
      dd[j] = dl.ld(i);
      dy[j] = zl.ld(i);
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) dy[j] = ol.ld(max(ib - j, 0)) * silu(dy[j]);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (ib - j >= 0) {
        const int i = ib - j;
#pragma unroll
        for (int q = 0; q < kN / 4; ++q) {
          const f32x4 Cv = sc[i][q];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const int n = q * 4 + s;
            u[n] = exp2_fast(dd[j] * a2[n]) * fmaf(Cv[s], dy[j], u[n]);
          }
        }
        sdt += dd[j];
      }
    }
  }
  float* dst = a.bloc + ((int64_t)b * P + p) * (kN + 1) * C + c;
#pragma unroll
  for (int n = 0; n < kN; ++n) dst[(int64_t)n * C] = u[n];
  dst[(int64_t)kN * C] = sdt;
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
  // pieces in groups of 16: all loads of a group are issued before its serial combine (one memory latency
  // per group)
  constexpr int kG = 16;
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
// B / C of the piece (shared by every channel) are staged in LDS once; the per-channel inputs of the next
// sub-chunk are loaded while the current one computes (indices clamped, so no load is conditional).
template <typename T>
__global__ __launch_bounds__(256, kBwdWavesPerSimd) void bwd_full_kernel(BwdArgs a) {
  const Lane l = lane_of();
  const int p = blockIdx.y;
  const int b = blockIdx.z;
  const int C = a.C, L = a.L, P = a.P;
  const int t0 = p * kPiece, t1 = min(L, t0 + kPiece);
  const int n_tok = t1 - t0;
  const int nsub = (n_tok + kSub - 1) / kSub;
  const int64_t row0 = (int64_t)b * L + t0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ f32x4 ck[kNSub][256];                 // state at each sub-chunk start, per lane
  __shared__ f32x4 red[kSub][32][2 * kQ];          // per channel pair: d B / d C sums (4 x B, 4 x C float4)
  __shared__ f32x4 sbc[kPiece][2 * kQ];            // B (4 x float4) then C (4 x float4) of each token

  for (int o = threadIdx.x; o < n_tok * 2 * kQ; o += 256)
    sbc[o / (2 * kQ)][o % (2 * kQ)] = ld4(a.bc + row0 * (2 * kN) + (int64_t)o * 4);

  float A[kQ], a2[kQ];
  load_A((const T*)a.A_log, l, A, a2);
  const float Dc = io<T>::ld((const T*)a.D + l.c);
  const Col<T> dl(a.delta, row0, n_tok, C, l.c), xl(a.xc, row0, n_tok, C, l.c), zl(a.z, row0, n_tok, C, l.c),
      ol(a.dout, row0, n_tok, C, l.c);
  const Col<T> gdd(a.ddelta, row0, n_tok, C, l.c), gdx(a.dxc, row0, n_tok, C, l.c), gdz(a.dz, row0, n_tok, C, l.c);

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
  auto load2 = [&](int k, float* d, float* x) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const int i = min(k * kSub + j, n_tok - 1);
      d[j] = dl.ld(i);
      x[j] = xl.ld(i);
    }
  };
  auto load2zo = [&](int k, float* z, float* o) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      const int i = min(k * kSub + j, n_tok - 1);
      z[j] = zl.ld(i);
      o[j] = ol.ld(i);
    }
  };
  __syncthreads();   // sbc

  // forward through the piece, saving the state at each sub-chunk start (the last sub-chunk's own tokens are
  // not needed here)
  ck[0][threadIdx.x] = f32x4{h[0], h[1], h[2], h[3]};
  if (nsub > 1) {
    float dn[kSub], xn[kSub];
    load2(0, dn, xn);
    for (int k = 0; k + 1 < nsub; ++k) {
      float dd[kSub], xx[kSub];
#pragma unroll
      for (int j = 0; j < kSub; ++j) {
        dd[j] = dn[j];
        xx[j] = xn[j];
      }
      load2(min(k + 1, nsub - 1), dn, xn);
#pragma unroll
      for (int j = 0; j < kSub; ++j) {   // a sub-chunk before the last is always whole
        const f32x4 Bv = sbc[k * kSub + j][l.q];
        const float dx = dd[j] * xx[j];
#pragma unroll
        for (int s = 0; s < kQ; ++s) h[s] = fmaf(exp2_fast(dd[j] * a2[s]), h[s], dx * Bv[s]);
      }
      ck[k + 1][threadIdx.x] = f32x4{h[0], h[1], h[2], h[3]};
    }
  }

  float dA[kQ] = {0.0f, 0.0f, 0.0f, 0.0f};
  float dD = 0.0f;
  float pd[kSub], px[kSub];   // the next sub-chunk's per-channel inputs
  load2(nsub - 1, pd, px);
  float pz[kSub], po[kSub];
  load2zo(nsub - 1, pz, po);
  // One sub-chunk of len tokens.  WHOLE (len == kSub: every sub-chunk but a ragged last one) drops the
  // per-token conditions, which otherwise make the compiler shuffle registers between the paths.
  auto sub_chunk = [&](auto whole, int k, int len) __attribute__((always_inline)) {
    constexpr bool kWhole = decltype(whole)::value;
    float dv[kSub], xv[kSub], dyv[kSub], dzf[kSub];
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      dyv[j] = pz[j];
      dzf[j] = po[j];
    }
    load2zo(max(k - 1, 0), pz, po);
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      dv[j] = pd[j];
      xv[j] = px[j];
    }
    load2(max(k - 1, 0), pd, px);
    // recompute the sub-chunk's states: hist[j] = state after its token j, ehist[j] its decay factors; the
    // gate terms
    float hist[kSub][kQ];
    float ehist[kSub][kQ];
    const f32x4 c4 = ck[k][threadIdx.x];
    float hs[kQ];
#pragma unroll
    for (int s = 0; s < kQ; ++s) {
      hs[s] = c4[s];
      h[s] = c4[s];
    }
#pragma unroll
    for (int j = 0; j < kSub; ++j) {
      if (kWhole || j < len) {
        const f32x4 Bv = sbc[k * kSub + j][l.q];
        const float d = dv[j], x = xv[j];
        const float dx = d * x;
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          const float e = exp2_fast(d * a2[s]);
          ehist[j][s] = e;
          h[s] = fmaf(e, h[s], dx * Bv[s]);
          hist[j][s] = h[s];
        }
        const float zv = dyv[j], dout = dzf[j];
        const float sg = rcp_fast(1.0f + exp2_fast(-zv * kLog2e));   // sigmoid(z)
        dyv[j] = dout * zv * sg;                                     // dout * SiLU(z)
        dzf[j] = dout * sg * fmaf(zv, 1.0f - sg, 1.0f);              // dout * SiLU'(z)
      }
    }
    // the gradient recurrence backwards through the sub-chunk
#pragma unroll
    for (int j = kSub - 1; j >= 0; --j) {
      if (kWhole || j < len) {
        const int i = k * kSub + j;
        const f32x4 Bv = sbc[i][l.q], Cv = sbc[i][kQ + l.q];
        const float d = dv[j], x = xv[j], dy = dyv[j];
        const float dx = d * x;
        // per state: g, sum g B (-> d delta's B x term and d x), g h_{t-1} a (-> d delta's A term and d A)
        float gB = 0.0f, pdA = 0.0f, py = 0.0f;
        float vb[kQ], vc[kQ];
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          const float hp = j > 0 ? hist[j > 0 ? j - 1 : 0][s] : hs[s];
          const float e = ehist[j][s];
          const float g = fmaf(Cv[s], dy, u[s]);
          gB = fmaf(g, Bv[s], gB);
          const float ghe = g * hp * e;
          pdA = fmaf(ghe, A[s], pdA);
          dA[s] = fmaf(ghe, d, dA[s]);
          vb[s] = g * dx;
          vc[s] = dy * hist[j][s];
          py = fmaf(Cv[s], hist[j][s], py);
          u[s] = e * g;
        }
        gB = quad_sum(gB);
        pdA = quad_sum(pdA);
        py = quad_sum(py);
        if (l.q == 0) {
          gdd.st(i, fmaf(gB, x, pdA));
          gdx.st(i, fmaf(Dc, dy, gB * d));
          gdz.st(i, fmaf(Dc, x, py) * dzf[j]);
        }
        dD = fmaf(dy, x, dD);
        // d B / d C of this token summed over pairs of channels (one cross-lane step; the block's 32 pairs are
        // added after the sub-chunk, from LDS)
#pragma unroll
        for (int s = 0; s < kQ; ++s) {
          vb[s] = pair_sum(vb[s]);
          vc[s] = pair_sum(vc[s]);
        }
        if ((lane & 4) == 0) {
          const int pr = wave * 8 + (lane >> 3);   // channel pair (lanes 0..3 and 8..11 of a row: pairs 2r, 2r + 1)
          red[j][pr][l.q * 2] = f32x4{vb[0], vb[1], vb[2], vb[3]};
          red[j][pr][l.q * 2 + 1] = f32x4{vc[0], vc[1], vc[2], vc[3]};
        }
      }
    }
    __syncthreads();
    // sum the block's 32 channel pairs and write this block's partial d B / d C for the sub-chunk's tokens
    for (int o = threadIdx.x; o < len * 2 * kN; o += 256) {
      const int j = o / (2 * kN), col = o % (2 * kN);
      // column col: d B (col < N) or d C of state n = col % N, held by state group n / 4, element n % 4
      const int n = col % kN, q = n / kQ;
      const float* base = reinterpret_cast<const float*>(&red[j][0][q * 2 + (col < kN ? 0 : 1)]) + n % kQ;
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < 32; ++r) sum += base[r * (2 * kQ) * 4];
      a.pbc[((int64_t)blockIdx.x * a.B * L + row0 + k * kSub + j) * (2 * kN) + col] = sum;
    }
    __syncthreads();
  };
  for (int k = nsub - 1; k >= 0; --k) {
    const int len = min(kSub, n_tok - k * kSub);
    if (len == kSub) sub_chunk(Flag<true>{}, k, len);
    else sub_chunk(Flag<false>{}, k, len);
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
  // sixteen loads in flight per step (the partials are summed in block order)
  float s = 0.0f;
  int k = 0;
  for (; k + 16 <= nblk; k += 16) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = pbc[(int64_t)(k + j) * rows * 2 * kN + i];
#pragma unroll
    for (int j = 0; j < 16; ++j) s += v[j];
  }
  for (; k < nblk; ++k) s += pbc[(int64_t)k * rows * 2 * kN + i];
  dbc[i] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_params_kernel(const float* __restrict__ pA,
                                                                const float* __restrict__ pD,
                                                                const T* __restrict__ A_log, float* __restrict__ dA_log,
                                                                float* __restrict__ dD, int C, int npieces) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;   // over C * N
  if (i >= C * kN) return;
  // sixteen loads in flight per step (the partials are summed in piece order; with 2 waves per SIMD the pass
  // waits on one memory latency per step)
  auto sum = [&](const float* part, int64_t stride) __attribute__((always_inline)) {
    float s = 0.0f;
    int k = 0;
    for (; k + 16 <= npieces; k += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = part[(int64_t)(k + j) * stride + i];
#pragma unroll
      for (int j = 0; j < 16; ++j) s += v[j];
    }
    for (; k < npieces; ++k) s += part[(int64_t)k * stride + i];
    return s;
  };
  const float A = -exp2_fast(io<T>::ld(A_log + i) * kLog2e);
  dA_log[i] = sum(pA, (int64_t)C * kN) * A;
  if (i < C) dD[i] = sum(pD, C);
}

template <typename T>
void run_bwd(const BwdArgs& a, hipStream_t st) {
  if (a.P > 1) {
    hipLaunchKernelGGL(bwd_local_kernel<T>, dim3(a.C / 64, a.P - 1, a.B), dim3(64), 0, st, a);
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
