// The whole Jamba Mamba layer around the mixer (jm_layer.h): pre-norm RMSNorm, in_proj, the mixer,
// out_proj and the residual add.  The two projections are plain GEMMs: for a decode-sized batch (at most 256
// tokens, bf16) they run on this library's weight-streaming kernel (gemm_skinny.hip), otherwise through
// hipBLASLt; the norm is a kernel here; the mixer is this library's own.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <tuple>

#include "jm_device.h"
#include "jm_launch.h"
#include "jm_layer.h"

namespace {

constexpr int64_t kAlign = 256;
constexpr int64_t kGemmWorkspace = 32ll << 20;   // hipBLASLt workspace carved from the caller's
constexpr int kMaxDevices = 64;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------------------------------------- RMSNorm

// One workgroup per token: out = x / sqrt(mean(x^2) + eps) * w, with 16-byte accesses (8 bf16 or 4 fp32
// per chunk).  Sum of squares in fp32: per thread, per wave (shuffles), then across the 4 waves in LDS.
template <typename T>
__global__ __launch_bounds__(256) void rms_norm_kernel(const T* __restrict__ x, const T* __restrict__ w,
                                                       T* __restrict__ out, int D, float eps) {
  constexpr int V = 16 / sizeof(T);
  typedef __attribute__((__vector_size__(16))) unsigned u32x4;
  const int64_t row = blockIdx.x;
  const T* xr = x + row * D;
  T* orow = out + row * D;
  const int chunks = D / V;
  float ss = 0.0f;
  for (int k = threadIdx.x; k < chunks; k += 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + k * V);
    const T* e = reinterpret_cast<const T*>(&raw);
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const float v = jm::io<T>::cvt(e[i]);
      ss = fmaf(v, v, ss);
    }
  }
  ss = jm::wave_sum(ss);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float r = 1.0f / sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / D + eps);
  for (int k = threadIdx.x; k < chunks; k += 256) {
    const u32x4 raw = *reinterpret_cast<const u32x4*>(xr + k * V);
    const u32x4 wraw = *reinterpret_cast<const u32x4*>(w + k * V);
    const T* e = reinterpret_cast<const T*>(&raw);
    const T* we = reinterpret_cast<const T*>(&wraw);
    u32x4 o;
    T* oe = reinterpret_cast<T*>(&o);
#pragma unroll
    for (int i = 0; i < V; ++i) oe[i] = jm::io<T>::from(jm::io<T>::cvt(e[i]) * r * jm::io<T>::cvt(we[i]));
    *reinterpret_cast<u32x4*>(orow + k * V) = o;
  }
}

// ---------------------------------------------------------------------------------------------- GEMMs

// One hipBLASLt handle per device, and the algorithm chosen for each GEMM shape, created on first use.
struct GemmKey {
  int dev, dtype;
  int64_t m, n, k, lda, ldb, ldc, ldd;
  bool beta;
  bool operator<(const GemmKey& o) const {
    return std::tie(dev, dtype, m, n, k, lda, ldb, ldc, ldd, beta) <
           std::tie(o.dev, o.dtype, o.m, o.n, o.k, o.lda, o.ldb, o.ldc, o.ldd, o.beta);
  }
};
std::mutex g_gemm_mu;
hipblasLtHandle_t g_handle[kMaxDevices];
std::map<GemmKey, hipblasLtMatmulAlgo_t> g_algos;

// Row-major Y[T, N] = X[T, K] . W[N, K]^T (+ R[T, N] when there is a residual), all of the I/O type, fp32
// accumulation.  In hipBLASLt's column-major terms: D[N, T] = op(A)[N, K] . B[K, T] + C with A = W (its
// row-major [N, K] is column-major [K, N], transposed), B = X (column-major [K, T]), C = R, D = Y.
// A GEMM is prepared (descriptors, the device's handle, the algorithm for its shape) before the layer
// enqueues any work, so that every failure of hipBLASLt's set-up is reported with nothing enqueued; only
// the launch itself remains.
struct Gemm {
  hipblasLtMatmulDesc_t op = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr, ld = nullptr;
  hipblasLtHandle_t handle = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool residual = false;
  Gemm() = default;
  Gemm(const Gemm&) = delete;
  Gemm& operator=(const Gemm&) = delete;
  ~Gemm() {
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lc) hipblasLtMatrixLayoutDestroy(lc);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (op) hipblasLtMatmulDescDestroy(op);
  }
};

int gemm_prepare(Gemm* g, bool bf16, int64_t ldx, int64_t ldw, int64_t ldy, bool residual, int64_t ldr, int64_t T,
                 int64_t N, int64_t K) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return JM_ERR_HIP;
  const hipDataType ty = bf16 ? HIP_R_16BF : HIP_R_32F;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  const uint64_t wsz = kGemmWorkspace;
  g->residual = residual;
  if (hipblasLtMatmulDescCreate(&g->op, HIPBLAS_COMPUTE_32F, HIP_R_32F) != HIPBLAS_STATUS_SUCCESS) return JM_ERR_HIP;
  if (hipblasLtMatmulDescSetAttribute(g->op, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) !=
          HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatmulDescSetAttribute(g->op, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) !=
          HIPBLAS_STATUS_SUCCESS)
    return JM_ERR_HIP;
  if (hipblasLtMatrixLayoutCreate(&g->la, ty, K, N, ldw) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&g->lb, ty, K, T, ldx) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&g->lc, ty, N, T, residual ? ldr : ldy) != HIPBLAS_STATUS_SUCCESS ||
      hipblasLtMatrixLayoutCreate(&g->ld, ty, N, T, ldy) != HIPBLAS_STATUS_SUCCESS)
    return JM_ERR_HIP;
  const GemmKey key{dev, bf16 ? 1 : 0, N, T, K, ldw, ldx, residual ? ldr : ldy, ldy, residual};
  std::lock_guard<std::mutex> lock(g_gemm_mu);
  if (!g_handle[dev] && hipblasLtCreate(&g_handle[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_handle[dev] = nullptr;
    return JM_ERR_HIP;
  }
  g->handle = g_handle[dev];
  auto it = g_algos.find(key);
  if (it == g_algos.end()) {
    hipblasLtMatmulPreference_t pref = nullptr;
    if (hipblasLtMatmulPreferenceCreate(&pref) != HIPBLAS_STATUS_SUCCESS) return JM_ERR_HIP;
    hipblasLtMatmulHeuristicResult_t heur[1];
    int found = 0;
    const bool ok = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz,
                                                          sizeof(wsz)) == HIPBLAS_STATUS_SUCCESS &&
                    hipblasLtMatmulAlgoGetHeuristic(g->handle, g->op, g->la, g->lb, g->lc, g->ld, pref, 1, heur,
                                                    &found) == HIPBLAS_STATUS_SUCCESS;
    hipblasLtMatmulPreferenceDestroy(pref);
    if (!ok || found < 1) return JM_ERR_UNSUPPORTED;
    it = g_algos.emplace(key, heur[0].algo).first;
  }
  g->algo = it->second;
  return JM_OK;
}

int gemm_launch(const Gemm& g, const void* X, const void* W, void* Y, const void* res, void* ws, hipStream_t st) {
  const float alpha = 1.0f, beta = g.residual ? 1.0f : 0.0f;
  const void* C = g.residual ? res : Y;
  return hipblasLtMatmul(g.handle, g.op, &alpha, W, g.la, X, g.lb, &beta, C, g.lc, Y, g.ld, &g.algo, ws,
                         (uint64_t)kGemmWorkspace, st) == HIPBLAS_STATUS_SUCCESS
             ? JM_OK
             : JM_ERR_HIP;
}

// ---------------------------------------------------------------------------------------------- the layer

struct LayerPlan {
  jm_mixer_dims md;     // the mixer's dims with x / z strided views of the in_proj output
  int64_t T, C, Dm, esize;
  int64_t off_hn, off_xz, off_y, off_mixer, off_gemm, total;
};

// varlen: a packed batch (d->mixer.batch sequences, d->mixer.seqlen tokens in all)
int layer_plan(const jm_layer_dims* d, bool decode, LayerPlan* p, bool varlen = false) {
  if (!d) return JM_ERR_INVALID_ARG;
  if (d->d_model < 1 || !(d->layer_norm_eps >= 0.0f)) return JM_ERR_INVALID_ARG;
  if (d->d_model % 8 != 0) return JM_ERR_UNSUPPORTED;
  p->md = d->mixer;
  p->md.x_row_stride = 2 * (int64_t)d->mixer.d_inner;
  p->md.z_row_stride = 2 * (int64_t)d->mixer.d_inner;
  const int64_t mws = jm::mixer_workspace_bytes(&p->md, decode, varlen);
  if (mws < 0) return (int)mws;   // the mixer's own validation code
  p->T = varlen ? d->mixer.seqlen : (int64_t)d->mixer.batch * (decode ? 1 : d->mixer.seqlen);
  p->C = d->mixer.d_inner;
  p->Dm = d->d_model;
  p->esize = d->mixer.io_dtype == JM_BF16 ? 2 : 4;
  int64_t off = 0;
  p->off_hn = off;    off += align_up(p->T * p->Dm * p->esize);
  p->off_xz = off;    off += align_up(p->T * 2 * p->C * p->esize);
  p->off_y = off;     off += align_up(p->T * p->C * p->esize);
  p->off_mixer = off; off += align_up(mws);
  p->off_gemm = off;  off += kGemmWorkspace;
  p->total = off;
  return JM_OK;
}

int layer_run(const jm_layer_dims* dims, const jm_layer_weights* lw, const void* x_res, void* out,
              const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
              void* stream, bool decode, const int32_t* slots = nullptr, int pool = 0,
              const int32_t* cu = nullptr) {
  LayerPlan p;
  int s = layer_plan(dims, decode, &p, cu != nullptr);
  if (s != JM_OK) return s;
  if (!lw || !lw->norm_w || !lw->in_proj_w || !lw->out_proj_w) return JM_ERR_INVALID_ARG;
  const void* ptrs[] = {lw->norm_w, lw->in_proj_w, lw->out_proj_w, x_res, out, ws};
  for (const void* q : ptrs)
    if (q && ((uintptr_t)q & 15u) != 0) return JM_ERR_ALIGNMENT;
  if (p.T > 0 && (!x_res || !out)) return JM_ERR_INVALID_ARG;
  if (!conv_out || !h_out || (decode && (!conv_in || !h0))) return JM_ERR_INVALID_ARG;
  if (!ws || (int64_t)ws_bytes < p.total) return JM_ERR_WORKSPACE;
  const bool bf16 = dims->mixer.io_dtype == JM_BF16;
  char* base = (char*)ws;
  void* hn = base + p.off_hn;
  char* xz = base + p.off_xz;
  void* y = base + p.off_y;
  void* mws = base + p.off_mixer;
  void* gws = base + p.off_gemm;
  hipStream_t st = (hipStream_t)stream;
  const size_t mws_bytes = (size_t)(p.off_gemm - p.off_mixer);
  // everything the mixer checks, before the norm and in_proj are enqueued
  if ((s = jm::mixer_validate(&p.md, &lw->mixer, p.T > 0 ? xz : nullptr, p.T > 0 ? xz + p.C * p.esize : nullptr,
                              p.T > 0 ? y : nullptr, conv_in, conv_out, h0, h_out, mws, mws_bytes, decode, slots,
                              pool, cu)) != JM_OK)
    return s;
  if (p.T == 0) {   // no tokens: the mixer copies the states through
    return jm::mixer_run(&p.md, &lw->mixer, nullptr, nullptr, nullptr, conv_in, conv_out, h0, h_out, mws,
                         mws_bytes, stream, decode, slots, pool, cu);
  }
  // A decode-sized batch (at most 256 tokens, bf16) runs both projections on the weight-streaming kernel
  // (gemm_skinny.hip); otherwise both GEMMs are resolved in hipBLASLt (handle, descriptors, algorithm)
  // before anything is enqueued.
  const int sp_in = bf16 ? jm::skinny_gemm_splits((int)p.T, (int)(2 * p.C), (int)p.Dm, kGemmWorkspace) : 0;
  const int sp_out = bf16 ? jm::skinny_gemm_splits((int)p.T, (int)p.Dm, (int)p.C, kGemmWorkspace) : 0;
  Gemm in_proj, out_proj;
  if (!sp_in && (s = gemm_prepare(&in_proj, bf16, p.Dm, p.Dm, 2 * p.C, false, 0, p.T, 2 * p.C, p.Dm)) != JM_OK)
    return s;
  if (!sp_out && (s = gemm_prepare(&out_proj, bf16, p.C, p.C, p.Dm, true, p.Dm, p.T, p.Dm, p.C)) != JM_OK)
    return s;
  (void)hipGetLastError();
  if (bf16)
    hipLaunchKernelGGL(rms_norm_kernel<jm::bf16_t>, dim3((unsigned)p.T), dim3(256), 0, st,
                       (const jm::bf16_t*)x_res, (const jm::bf16_t*)lw->norm_w, (jm::bf16_t*)hn, (int)p.Dm,
                       dims->layer_norm_eps);
  else
    hipLaunchKernelGGL(rms_norm_kernel<float>, dim3((unsigned)p.T), dim3(256), 0, st, (const float*)x_res,
                       (const float*)lw->norm_w, (float*)hn, (int)p.Dm, dims->layer_norm_eps);
  if (hipGetLastError() != hipSuccess) return JM_ERR_HIP;
  if (sp_in) {
    jm::launch_skinny_gemm(hn, p.Dm, lw->in_proj_w, p.Dm, nullptr, 0, xz, 2 * p.C, (int)p.T, (int)(2 * p.C),
                           (int)p.Dm, sp_in, (float*)gws, st);
    if (hipGetLastError() != hipSuccess) return JM_ERR_HIP;
  } else if ((s = gemm_launch(in_proj, hn, lw->in_proj_w, xz, nullptr, gws, st)) != JM_OK) {
    return s;
  }
  if ((s = jm::mixer_run(&p.md, &lw->mixer, xz, xz + p.C * p.esize, y, conv_in, conv_out, h0, h_out, mws,
                         mws_bytes, stream, decode, slots, pool, cu)) != JM_OK)
    return s;
  if (sp_out) {
    jm::launch_skinny_gemm(y, p.C, lw->out_proj_w, p.C, x_res, p.Dm, out, p.Dm, (int)p.T, (int)p.Dm, (int)p.C,
                           sp_out, (float*)gws, st);
    return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
  }
  return gemm_launch(out_proj, y, lw->out_proj_w, out, x_res, gws, st);
}

}  // namespace

extern "C" {

size_t jm_layer_prefill_workspace_size(const jm_layer_dims* dims) {
  LayerPlan p;
  return layer_plan(dims, false, &p) == JM_OK ? (size_t)p.total : 0;
}

size_t jm_layer_decode_workspace_size(const jm_layer_dims* dims) {
  LayerPlan p;
  return layer_plan(dims, true, &p) == JM_OK ? (size_t)p.total : 0;
}

int jm_layer_prefill(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res, void* out,
                     const void* conv_state_in, void* conv_state_out, const float* ssm_state_in,
                     float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return layer_run(dims, weights, x_res, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out,
                   workspace, workspace_bytes, stream, false);
}

int jm_layer_decode_step(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                         void* out, const void* conv_state_in, void* conv_state_out, const float* ssm_state_in,
                         float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return layer_run(dims, weights, x_res, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out,
                   workspace, workspace_bytes, stream, true);
}

int jm_layer_decode_step_slots(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                               void* out, void* conv_state_pool, float* ssm_state_pool, int32_t pool_size,
                               const int32_t* slots, void* workspace, size_t workspace_bytes, void* stream) {
  if (!slots) return JM_ERR_INVALID_ARG;
  return layer_run(dims, weights, x_res, out, conv_state_pool, conv_state_pool, ssm_state_pool, ssm_state_pool,
                   workspace, workspace_bytes, stream, true, slots, pool_size);
}

size_t jm_layer_prefill_varlen_workspace_size(const jm_layer_dims* dims) {
  LayerPlan p;
  return layer_plan(dims, false, &p, true) == JM_OK ? (size_t)p.total : 0;
}

int jm_layer_prefill_varlen(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                            void* out, const int32_t* cu_seqlens, const void* conv_state_in, void* conv_state_out,
                            const float* ssm_state_in, float* ssm_state_out, const int32_t* slots,
                            int32_t pool_size, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cu_seqlens) return JM_ERR_INVALID_ARG;
  return layer_run(dims, weights, x_res, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out,
                   workspace, workspace_bytes, stream, false, slots, pool_size, cu_seqlens);
}

}  // extern "C"
