// C ABI of the gated scan alone (jm_scan.h): the training forward and its backward.  Argument checks,
// workspace plans and the kernel sequences; nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jm_device.h"
#include "jm_launch.h"
#include "jm_scan.h"

namespace {

constexpr int kN = 16;
constexpr int64_t kAlign = 256;
constexpr int kMaxSeqlen = 1 << 21;

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const jm_scan_dims* d) {
  if (!d) return JM_ERR_INVALID_ARG;
  if (d->batch < 1 || d->d_inner < 1 || d->seqlen < 0) return JM_ERR_INVALID_ARG;
  if (d->batch > (1 << 16)) return JM_ERR_UNSUPPORTED;   // sequences index the grid's z axis (at most 65536)
  if (d->seqlen > kMaxSeqlen) return JM_ERR_UNSUPPORTED;
  if (d->io_dtype != JM_F32 && d->io_dtype != JM_BF16) return JM_ERR_UNSUPPORTED;
  if (d->d_state != kN || d->d_inner % 64 != 0) return JM_ERR_UNSUPPORTED;
  return JM_OK;
}

struct FwdPlan {
  int P, Lp;
  int64_t off_loc, off_cin, total;
};

FwdPlan fwd_plan(const jm_scan_dims* d) {
  FwdPlan p;
  const int esize = d->io_dtype == JM_BF16 ? 2 : 4;
  jm::scan_plan(d->batch, d->seqlen, d->d_inner, (int64_t)d->d_inner * esize, &p.P, &p.Lp);
  int64_t off = 0;
  p.off_loc = p.off_cin = -1;
  if (p.P > 1) {
    p.off_loc = off; off += align_up((int64_t)d->batch * p.P * (kN + 1) * d->d_inner * 4);
    p.off_cin = off; off += align_up((int64_t)d->batch * p.P * kN * d->d_inner * 4);
  }
  p.total = off > 0 ? off : kAlign;
  return p;
}

struct BwdPlan {
  int P;
  int64_t off_loc, off_cin, off_bloc, off_gin, off_pA, off_pD, off_pbc, total;
};

BwdPlan bwd_plan(const jm_scan_dims* d) {
  BwdPlan p;
  const int64_t B = d->batch, L = d->seqlen, C = d->d_inner;
  p.P = (int)((L + jm::kBwdPiece - 1) / jm::kBwdPiece);
  const int64_t P = p.P;
  int64_t off = 0;
  p.off_loc = p.off_cin = p.off_bloc = p.off_gin = -1;
  if (P > 1) {
    p.off_loc = off;  off += align_up(B * P * (kN + 1) * C * 4);
    p.off_cin = off;  off += align_up(B * P * kN * C * 4);
    p.off_bloc = off; off += align_up(B * P * (kN + 1) * C * 4);
    p.off_gin = off;  off += align_up(B * P * kN * C * 4);
  }
  p.off_pA = off;  off += align_up(B * P * C * kN * 4);
  p.off_pD = off;  off += align_up(B * P * C * 4);
  p.off_pbc = off; off += align_up((C / 64) * B * L * 2 * kN * 4);
  p.total = off > 0 ? off : kAlign;
  return p;
}

// dst[i] = src ? src[i] : 0 over n floats
__global__ void copy_or_zero_kernel(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float v = src ? src[i] : 0.0f;
    dst[i] = v;
  }
}

void copy_or_zero(const float* src, float* dst, int64_t n, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(copy_or_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, src, dst, n);
}

jm::ScanArgs scan_args(const jm_scan_dims* d, const void* x, const void* delta, const void* z, const float* bc,
                       const void* A_log, const void* D, const float* h0, void* out, float* h_out, int P, int Lp,
                       float* loc, float* cin) {
  jm::ScanArgs a;
  a.xc = x;
  a.delta = delta;
  a.z = z;
  a.z_stride = d->d_inner;
  a.bc = bc;
  a.A_log = A_log;
  a.D = D;
  a.h0 = h0;
  a.out = out;
  a.h_out = h_out;
  a.x = nullptr;
  a.x_stride = 0;
  a.conv_in = nullptr;
  a.conv_out = nullptr;     // the scan alone carries no conv state
  a.loc = loc;
  a.cin = cin;
  a.B = d->batch;
  a.L = d->seqlen;
  a.C = d->d_inner;
  a.P = P;
  a.Lp = Lp;
  a.slots = nullptr;
  a.pool = 0;
  a.cu = nullptr;
  a.nseq = 0;
  a.snap = nullptr;
  a.zoh = 0;
  a.saved = nullptr;
  a.saved_P = 0;
  return a;
}

// Backward pieces of a sequence (the saved states hold one state per piece and sequence).
int64_t bwd_pieces(const jm_scan_dims* d) { return ((int64_t)d->seqlen + jm::kBwdPiece - 1) / jm::kBwdPiece; }

int forward(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
            const void* A_log, const void* D, const float* h0, void* out, float* h_out, float* saved,
            void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_dims(dims);
  if (s != JM_OK) return s;
  const bool any = dims->seqlen > 0;
  if (!A_log || !D || !h_out || (any && (!x || !delta || !z || !bc || !out))) return JM_ERR_INVALID_ARG;
  const void* ptrs[] = {x, delta, z, bc, A_log, D, h0, out, h_out, saved, workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return JM_ERR_ALIGNMENT;
  const FwdPlan p = fwd_plan(dims);
  if (!workspace || (int64_t)workspace_bytes < p.total) return JM_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  (void)hipGetLastError();
  if (!any) {
    copy_or_zero(h0, h_out, (int64_t)dims->batch * dims->d_inner * kN, st);
  } else {
    char* base = (char*)workspace;
    jm::ScanArgs a = scan_args(dims, x, delta, z, bc, A_log, D, h0, out, h_out, p.P, p.Lp,
                               p.off_loc >= 0 ? (float*)(base + p.off_loc) : nullptr,
                               p.off_cin >= 0 ? (float*)(base + p.off_cin) : nullptr);
    a.saved = saved;
    a.saved_P = (int)bwd_pieces(dims);
    jm::launch_scan(dims->io_dtype == JM_BF16, a, st);
  }
  return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
}

}  // namespace

extern "C" {

size_t jm_scan_saved_states_size(const jm_scan_dims* dims) {
  if (check_dims(dims) != JM_OK) return 0;
  return (size_t)((int64_t)dims->batch * bwd_pieces(dims) * kN * dims->d_inner * 4);
}

int jm_scan_forward_train(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                          const void* A_log, const void* D, const float* h0, void* out, float* h_out,
                          float* saved_states, void* workspace, size_t workspace_bytes, void* stream) {
  if (!saved_states && dims && dims->seqlen > 0) return JM_ERR_INVALID_ARG;
  return forward(dims, x, delta, z, bc, A_log, D, h0, out, h_out, saved_states, workspace, workspace_bytes, stream);
}

size_t jm_scan_forward_workspace_size(const jm_scan_dims* dims) {
  if (check_dims(dims) != JM_OK) return 0;
  return (size_t)fwd_plan(dims).total;
}

size_t jm_scan_backward_workspace_size(const jm_scan_dims* dims) {
  if (check_dims(dims) != JM_OK) return 0;
  return (size_t)bwd_plan(dims).total;
}

int jm_scan_forward(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                    const void* A_log, const void* D, const float* h0, void* out, float* h_out,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return forward(dims, x, delta, z, bc, A_log, D, h0, out, h_out, nullptr, workspace, workspace_bytes, stream);
}

int jm_scan_backward(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                     const void* A_log, const void* D, const float* h0, const void* dout, const float* dh_final,
                     const float* saved_states, void* dx, void* ddelta, void* dz, float* dbc, float* dA_log,
                     float* dD, float* dh0, void* workspace, size_t workspace_bytes, void* stream) {
  int s = check_dims(dims);
  if (s != JM_OK) return s;
  const bool any = dims->seqlen > 0;
  if (!A_log || !D || !dA_log || !dD) return JM_ERR_INVALID_ARG;
  if (any && (!x || !delta || !z || !bc || !dout || !dx || !ddelta || !dz || !dbc)) return JM_ERR_INVALID_ARG;
  const void* ptrs[] = {x, delta, z, bc, A_log, D, h0, dout, dh_final, saved_states, dx, ddelta, dz, dbc, dA_log,
                        dD, dh0, workspace};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return JM_ERR_ALIGNMENT;
  const BwdPlan p = bwd_plan(dims);
  if (!workspace || (int64_t)workspace_bytes < p.total) return JM_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const bool bf16 = dims->io_dtype == JM_BF16;
  const int64_t nstate = (int64_t)dims->batch * dims->d_inner * kN;
  (void)hipGetLastError();
  if (!any) {
    copy_or_zero(nullptr, dA_log, (int64_t)dims->d_inner * kN, st);
    copy_or_zero(nullptr, dD, dims->d_inner, st);
    if (dh0) copy_or_zero(dh_final, dh0, nstate, st);
    return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
  }
  char* base = (char*)workspace;
  auto at = [&](int64_t off) { return off >= 0 ? (float*)(base + off) : nullptr; };
  // every piece's incoming state: saved by jm_scan_forward_train, or from the forward's local and carry passes
  // over the backward's pieces
  if (!saved_states) {
    const jm::ScanArgs fa = scan_args(dims, x, delta, z, bc, A_log, D, h0, dx, nullptr, p.P, jm::kBwdPiece,
                                      at(p.off_loc), at(p.off_cin));
    jm::launch_scan_carries(bf16, fa, st);
  }
  jm::BwdArgs a;
  a.xc = x;
  a.delta = delta;
  a.z = z;
  a.dout = dout;
  a.bc = bc;
  a.A_log = A_log;
  a.D = D;
  a.h0 = h0;
  a.dh_final = dh_final;
  a.cin = saved_states ? saved_states : at(p.off_cin);
  a.bloc = at(p.off_bloc);
  a.gin = at(p.off_gin);
  a.pA = at(p.off_pA);
  a.pD = at(p.off_pD);
  a.pbc = at(p.off_pbc);
  a.dxc = dx;
  a.ddelta = ddelta;
  a.dz = dz;
  a.dbc = dbc;
  a.dA_log = dA_log;
  a.dD = dD;
  a.dh0 = dh0;
  a.B = dims->batch;
  a.L = dims->seqlen;
  a.C = dims->d_inner;
  a.P = p.P;
  jm::launch_scan_backward(bf16, a, st);
  return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
}

}  // extern "C"
