// The library's C ABI (jm_mixer.h): argument checks, the execution plan, the workspace layout, and the
// kernel sequence on the caller's stream, for the plain batch, the decode step, state pools (slots) and
// packed variable-length batches.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "jm_launch.h"
#include "jm_mixer.h"

// Device scratch of jm_mixer_decode_step_noalloc: its intermediates live here instead of in a caller's
// workspace.  Each GPU the library runs on holds its own copy until the process ends; every call on a GPU
// shares that GPU's copy.  Host code never uses this name as an address: the address of each device's copy
// comes from hipGetSymbolAddress (static_scratch below).
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kN = 16;       // d_state the kernels are built for
constexpr int kTaps = 4;     // d_conv the kernels are built for
constexpr int kMaxR = 512;   // dt_rank bound of the norm kernel
constexpr int64_t kAlign = 256;
constexpr int kMaxSeqlen = 1 << 21;   // tokens of a prefill call (the conv's grid rows stay within 65536)
constexpr int kMaxBatch = 1 << 16;    // sequences of a call (they index the grid's y / z axes, at most 65536)

// Scan pieces: aim for this many 64-lane waves in the full pass, with pieces of at least kMinPiece tokens.  That
// is more than fit at once (five per SIMD at the full pass's register count, 5120): with more and shorter
// pieces, the workgroups that finish early take more of them.  Measured at 256K tokens: 16384 waves (128
// pieces) 14.7-14.8 ms against 15.3 ms with 6144 (the full pass 6.08-6.18 against 6.48-6.51 ms); 24576 no
// better (the carry pass grows, 58 against 42 us); 5120 and 4096 (one round of five or four waves per SIMD)
// 15.3 and 15.7 ms.  Pieces shorter than 128 tokens (the 4K prefill's 32 pieces) measured slower: 64 tokens
// 337 us, 32 tokens 353 us, against 314-329 us.
constexpr int64_t kScanWaveTarget = 16384;
constexpr int kMinPiece = 128;
// x_proj: split the contraction over channel slices until there are this many workgroups (one per CU).
constexpr int kXprojWgTarget = 256;
// fp32 x_proj (128 x 96 tiles of 4 waves, two resident per CU): split until there are two workgroups per CU,
// so that every CU gets the same number of equal K slices.
constexpr int kXprojF32WgTarget = 512;
// x_proj takes 256-token tiles from this many tokens on (fewer re-reads of W_x; shorter inputs keep 128-token
// tiles, which need half as many channel slices and partial sums to fill the GPU).
constexpr int64_t kXprojTallTokens = 32768;

struct Plan {
  int B, L, C, N, R, W;
  int64_t T;
  bool bf16;
  int esize;
  int splits;    // x_proj channel slices
  bool narrow;   // x_proj in 32-column groups (few tokens)
  bool tall;     // x_proj in 256-token tiles (long inputs)
  bool fused;    // a shape the single-kernel decode step takes (its x_proj slices size the partial sums)
  int P, Lp;     // scan pieces per sequence, tokens per piece
  int64_t xs, zs;
  int nseq;      // packed batches: number of sequences (the plan itself runs B = 1 over L = all tokens)
  int64_t off_xc, off_dbc, off_dln, off_bc, off_delta, off_loc, off_cin, off_snap, off_bar, total;
};

// Optional parts of a call: per-stage events, a state pool (slots), a packed batch (cu_seqlens).
struct Extras {
  bool single = false;   // jm_mixer_decode_step_single_kernel
  void** events = nullptr;
  int n_events = 0;
  const int32_t* slots = nullptr;
  int pool = 0;
  const int32_t* cu = nullptr;
};

int64_t align_up(int64_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int check_dims(const jm_mixer_dims* d, bool decode) {
  if (!d) return JM_ERR_INVALID_ARG;
  if (d->batch < 1 || d->d_inner < 1 || d->dt_rank < 1) return JM_ERR_INVALID_ARG;
  if (d->batch > kMaxBatch) return JM_ERR_UNSUPPORTED;
  if (!decode && d->seqlen < 0) return JM_ERR_INVALID_ARG;
  if (!decode && d->seqlen > kMaxSeqlen) return JM_ERR_UNSUPPORTED;
  if (!(d->norm_eps >= 0.0f)) return JM_ERR_INVALID_ARG;
  if (d->io_dtype != JM_F32 && d->io_dtype != JM_BF16) return JM_ERR_UNSUPPORTED;
  if (d->d_state != kN || d->d_conv != kTaps) return JM_ERR_UNSUPPORTED;
  if (d->discretization != JM_DISC_EULER && d->discretization != JM_DISC_ZOH) return JM_ERR_UNSUPPORTED;
  if (d->reserved != 0) return JM_ERR_INVALID_ARG;
  if (d->d_inner % 64 != 0) return JM_ERR_UNSUPPORTED;
  if (d->dt_rank > kMaxR || d->dt_rank % 8 != 0) return JM_ERR_UNSUPPORTED;
  const int64_t xs = d->x_row_stride ? d->x_row_stride : d->d_inner;
  const int64_t zs = d->z_row_stride ? d->z_row_stride : d->d_inner;
  if (xs < d->d_inner || zs < d->d_inner) return JM_ERR_INVALID_ARG;
  if (xs % 8 != 0 || zs % 8 != 0) return JM_ERR_ALIGNMENT;
  return JM_OK;
}

// varlen: a packed batch of d->batch sequences holding d->seqlen tokens in all, planned as one sequence.
// single: the layout of jm_mixer_decode_step_single_kernel (its partial sums and grid-barrier flags).
Plan make_plan(const jm_mixer_dims* d, bool decode, bool varlen = false, bool single = false) {
  Plan p;
  p.nseq = d->batch;
  p.B = varlen ? 1 : d->batch;
  p.L = decode ? 1 : d->seqlen;
  p.C = d->d_inner;
  p.N = d->d_state;
  p.R = d->dt_rank;
  p.W = p.R + 2 * p.N;
  p.T = (int64_t)p.B * p.L;
  p.bf16 = d->io_dtype == JM_BF16;
  p.esize = p.bf16 ? 2 : 4;
  p.xs = d->x_row_stride ? d->x_row_stride : p.C;
  p.zs = d->z_row_stride ? d->z_row_stride : p.C;

  // x_proj split: channel slices of a multiple of 64, dividing C, until the grid is big enough.  When even
  // the most slices leave the GPU short of workgroups, the narrow column layout multiplies the grid (not for
  // long inputs: their 256-token tiles have no narrow form, and at 32768 tokens or more there are at least 128).
  p.splits = 1;
  p.narrow = false;
  p.tall = p.bf16 && p.T >= kXprojTallTokens;
  if (p.bf16) {
    const int64_t tile = jm::xproj_token_tile(p.tall);
    const int64_t mtiles = (p.T + tile - 1) / tile;
    auto grow = [&](int64_t groups) {
      p.splits = 1;
      while (mtiles * groups * p.splits < kXprojWgTarget && p.splits * 2 <= jm::kMaxXprojSplits &&
             (p.C / 64) % (p.splits * 2) == 0)
        p.splits *= 2;
    };
    grow(jm::xproj_column_groups(p.W, false));
    if (!p.tall && mtiles * jm::xproj_column_groups(p.W, false) * p.splits < kXprojWgTarget) {
      p.narrow = true;
      grow(jm::xproj_column_groups(p.W, true));
    }
  } else {
    const int64_t tiles = jm::gemm_f32_tiles(p.T, p.W);
    while (tiles * p.splits < kXprojF32WgTarget && p.splits * 2 <= jm::kMaxXprojSplits &&
           (p.C / 64) % (p.splits * 2) == 0)
      p.splits *= 2;
  }

  p.fused = single && p.bf16 && p.L == 1 && !varlen && jm::decode_fused_shape_ok(p.B, p.C, p.R);
  const int64_t dbc_slices =
      p.fused && jm::decode_fused_slices(p.C) > p.splits ? jm::decode_fused_slices(p.C) : p.splits;

  // scan pieces
  const int64_t row_bytes = (p.xs > p.zs ? (p.xs > p.C ? p.xs : p.C) : (p.zs > p.C ? p.zs : p.C)) * p.esize;
  jm::scan_plan(p.B, p.L, p.C, row_bytes, &p.P, &p.Lp);

  int64_t off = 0;
  p.off_xc = off;    off += align_up(p.T * p.C * p.esize);
  p.off_dbc = off;   off += align_up(dbc_slices * p.T * p.W * 4);
  p.off_dln = off;   off += align_up(p.T * p.R * p.esize);
  p.off_bc = off;    off += align_up(p.T * 2 * p.N * 4);
  p.off_delta = off; off += align_up(p.T * p.C * p.esize);
  p.off_loc = p.off_cin = p.off_snap = -1;
  if (p.P > 1) {
    p.off_loc = off; off += align_up((int64_t)p.B * p.P * (p.N + 1) * p.C * 4);
    p.off_cin = off; off += align_up((int64_t)p.B * p.P * p.N * p.C * 4);
    if (varlen) {
      p.off_snap = off; off += align_up((int64_t)p.P * p.N * p.C * 4);
    }
  }
  p.off_bar = -1;
  if (p.fused) {
    p.off_bar = off; off += align_up(jm::kDecodeMaxGroups * 8);
  }
  p.total = off > 0 ? off : kAlign;
  return p;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int check_weights(const jm_mixer_weights* w) {
  if (!w) return JM_ERR_INVALID_ARG;
  const void* req[] = {w->conv_w, w->x_proj_w, w->dt_norm_w, w->b_norm_w, w->c_norm_w,
                       w->dt_proj_w, w->dt_proj_b, w->A_log, w->D};
  for (const void* q : req)
    if (!q) return JM_ERR_INVALID_ARG;
  for (const void* q : req)
    if (!aligned16(q)) return JM_ERR_ALIGNMENT;
  if (w->conv_b && !aligned16(w->conv_b)) return JM_ERR_ALIGNMENT;
  return JM_OK;
}

const char* const kStageNames[JM_STAGES] = {"conv_silu", "x_proj", "norm", "dt_proj", "scan_local",
                                            "scan_carry", "scan_full"};

// Records events[i] before stage i when per-stage timing was asked for.
struct StageMarks {
  void** ev;
  hipStream_t st;
  void mark(int i) const {
    if (ev) (void)hipEventRecord((hipEvent_t)ev[i], st);
  }
};

// Every check of a call, before anything is enqueued.
int validate(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
             const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
             bool decode, const int32_t* slots = nullptr, int pool = 0, const int32_t* cu = nullptr,
             bool single = false) {
  int s = check_dims(dims, decode);
  if (s != JM_OK) return s;
  if ((s = check_weights(w)) != JM_OK) return s;
  const Plan p = make_plan(dims, decode, cu != nullptr, single);
  if (!conv_out || !h_out) return JM_ERR_INVALID_ARG;
  if (decode && (!conv_in || !h0)) return JM_ERR_INVALID_ARG;
  if (slots) {   // a state pool: decode or packed prefill, at least one row, int32 indices
    if ((!decode && !cu) || pool < 1) return JM_ERR_INVALID_ARG;
    if (((uintptr_t)slots & 3u) != 0) return JM_ERR_ALIGNMENT;
  }
  if (cu && ((uintptr_t)cu & 3u) != 0) return JM_ERR_ALIGNMENT;
  if (p.L > 0 && (!x || !z || !out)) return JM_ERR_INVALID_ARG;
  const void* ptrs[] = {x, z, out, conv_in, conv_out, h0, h_out, ws};
  for (const void* q : ptrs)
    if (q && !aligned16(q)) return JM_ERR_ALIGNMENT;
  if (!ws || (int64_t)ws_bytes < p.total) return JM_ERR_WORKSPACE;
  return JM_OK;
}

int run(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
        const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
        void* stream, bool decode, const Extras& ex = Extras()) {
  void** events = ex.events;
  const int n_events = ex.n_events;
  const int32_t* slots = ex.slots;
  const int pool = ex.pool;
  const bool varlen = ex.cu != nullptr;
  int s = validate(dims, w, x, z, out, conv_in, conv_out, h0, h_out, ws, ws_bytes, decode, slots, pool, ex.cu,
                   ex.single);
  if (s != JM_OK) return s;
  const Plan p = make_plan(dims, decode, varlen, ex.single);
  const jm::VarSeqs vs{ex.cu, slots, p.nseq, pool};
  if (events) {
    if (n_events < JM_STAGES + 1) return JM_ERR_INVALID_ARG;
    for (int i = 0; i <= JM_STAGES; ++i)
      if (!events[i]) return JM_ERR_INVALID_ARG;
  }

  hipStream_t st = (hipStream_t)stream;
  const StageMarks marks{events, st};
  (void)hipGetLastError();  // clear a stale error so the check below reports this call's launches only
  if (p.L == 0) {
    marks.mark(0);
    if (varlen)   // every sequence is empty: its states carry over
      jm::launch_varlen_states(p.bf16, x, p.xs, conv_in, conv_out, h0, h_out, p.C, 0, vs, st);
    else
      jm::launch_state_passthrough(p.bf16, conv_in, conv_out, h0, h_out, p.B, p.C, st);
    for (int i = 1; i <= JM_STAGES; ++i) marks.mark(i);
    return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
  }
  char* base = (char*)ws;
  void* xc = base + p.off_xc;
  float* dbc = (float*)(base + p.off_dbc);
  void* dln = base + p.off_dln;
  float* bc = (float*)(base + p.off_bc);
  void* delta = base + p.off_delta;

  // one token per sequence: the single-step conv also writes the conv state, so the scan skips it
  const bool step = p.L == 1 && !varlen;
  if (ex.single) {
    // the whole step as one kernel; nothing is enqueued for a shape or device it does not support
    if (!step || !p.fused || !jm::decode_fused_available()) return JM_ERR_UNSUPPORTED;
    marks.mark(0);
    jm::DecodeArgs d;
    d.x = x;
    d.xs = p.xs;
    d.z = z;
    d.zs = p.zs;
    d.conv_w = w->conv_w;
    d.conv_b = w->conv_b;
    d.conv_in = conv_in;
    d.conv_out = conv_out;
    d.x_proj_w = w->x_proj_w;
    d.dt_norm_w = w->dt_norm_w;
    d.b_norm_w = w->b_norm_w;
    d.c_norm_w = w->c_norm_w;
    d.eps = dims->norm_eps;
    d.dt_proj_w = w->dt_proj_w;
    d.dt_proj_b = w->dt_proj_b;
    d.A_log = w->A_log;
    d.D = w->D;
    d.h0 = h0;
    d.h_out = h_out;
    d.out = out;
    d.slots = slots;
    d.pool = pool;
    d.xc = xc;
    d.part = dbc;
    d.dln = dln;
    d.bc = bc;
    d.flags = (uint64_t*)(base + p.off_bar);
    d.B = p.B;
    d.C = p.C;
    d.R = p.R;
    d.zoh = dims->discretization == JM_DISC_ZOH;
    const hipError_t e = jm::launch_decode_fused(d, st);
    for (int i = 1; i <= JM_STAGES; ++i) marks.mark(i);
    return e == hipSuccess && hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
  }
  marks.mark(0);
  // long plain prefills: the conv runs inside x_proj (one read of x; the conv stage is then empty)
  const bool conv_in_xproj = !step && !varlen && p.tall && jm::conv_xproj_fits(p.xs);
  if (step) {
    jm::launch_conv_step(p.bf16, x, p.xs, w->conv_w, w->conv_b, conv_in, xc, conv_out, p.B, p.C, st, slots,
                         pool);
  } else if (!conv_in_xproj) {
    jm::launch_conv_silu(p.bf16, x, p.xs, w->conv_w, w->conv_b, conv_in, xc, p.B, p.L, p.C, st, vs);
    // a packed batch's conv states (and the states of its empty sequences), once the conv has read them
    if (varlen) jm::launch_varlen_states(p.bf16, x, p.xs, conv_in, conv_out, h0, h_out, p.C, p.L, vs, st);
  }
  marks.mark(1);
  if (conv_in_xproj)
    jm::launch_conv_xproj(x, p.xs, w->conv_w, w->conv_b, conv_in, xc, w->x_proj_w, dbc, p.B, p.L, p.W, p.C,
                          p.splits, st);
  else
    jm::launch_xproj(p.bf16, xc, w->x_proj_w, dbc, (int)p.T, p.W, p.C, p.splits, p.narrow, st, p.tall);
  marks.mark(2);
  jm::launch_norm(p.bf16, dbc, p.splits, (int)p.T, p.R, p.N, w->dt_norm_w, w->b_norm_w, w->c_norm_w,
                  dims->norm_eps, dln, bc, st);
  marks.mark(3);
  jm::launch_dtproj(p.bf16, dln, w->dt_proj_w, w->dt_proj_b, delta, (int)p.T, p.C, p.R, st);
  jm::ScanArgs a;
  a.xc = xc;
  a.delta = delta;
  a.z = z;
  a.z_stride = p.zs;
  a.bc = bc;
  a.A_log = w->A_log;
  a.D = w->D;
  a.h0 = h0;
  a.out = out;
  a.h_out = h_out;
  a.x = x;
  a.x_stride = p.xs;
  a.conv_in = conv_in;
  a.conv_out = step || varlen ? nullptr : conv_out;
  a.loc = p.P > 1 ? (float*)(base + p.off_loc) : nullptr;
  a.cin = p.P > 1 ? (float*)(base + p.off_cin) : nullptr;
  a.B = p.B;
  a.L = p.L;
  a.C = p.C;
  a.P = p.P;
  a.Lp = p.Lp;
  a.slots = slots;
  a.pool = pool;
  a.cu = ex.cu;
  a.nseq = p.nseq;
  a.snap = p.off_snap >= 0 ? (float*)(base + p.off_snap) : nullptr;
  a.zoh = dims->discretization == JM_DISC_ZOH;
  a.saved = nullptr;
  a.saved_P = 0;
  // the scan records events[4] (local pass), events[5] (carry pass) and events[6] (full pass)
  jm::launch_scan(p.bf16, a, st, events ? &marks.ev[4] : nullptr);
  marks.mark(JM_STAGES);
  return hipGetLastError() == hipSuccess ? JM_OK : JM_ERR_HIP;
}

// The address of this device's copy of `scratch`, looked up once per device with that device current (the
// first jm_mixer_decode_step_noalloc call on it) and kept for the process's lifetime.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

int static_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return JM_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return JM_ERR_HIP;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return JM_OK;
}

}  // namespace

namespace jm {

void scan_plan(int B, int L, int C, int64_t row_bytes, int* P, int* Lp) {
  const int64_t waves = (int64_t)B * (C / 64);
  const int64_t want = (kScanWaveTarget + waves - 1) / waves;
  int64_t lp = L > 0 ? (L + want - 1) / want : 1;
  if (lp < kMinPiece) lp = kMinPiece;
  // the scan addresses a piece through 32-bit byte offsets: keep each piece's rows under 2 GiB
  const int64_t max_rows = ((int64_t)1 << 31) / row_bytes - 1;
  if (lp > max_rows) lp = max_rows;
  *Lp = (int)(lp < L ? lp : (L > 0 ? L : 1));
  *P = L > 0 ? (int)((L + *Lp - 1) / *Lp) : 1;
}

int64_t mixer_workspace_bytes(const jm_mixer_dims* dims, bool decode, bool varlen) {
  const int s = check_dims(dims, decode);
  if (s != JM_OK) return s;
  return make_plan(dims, decode, varlen).total;
}

int mixer_validate(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
                   const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
                   bool decode, const int32_t* slots, int pool, const int32_t* cu) {
  return validate(dims, w, x, z, out, conv_in, conv_out, h0, h_out, ws, ws_bytes, decode, slots, pool, cu);
}

int mixer_run(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
              const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
              void* stream, bool decode, const int32_t* slots, int pool, const int32_t* cu) {
  Extras ex;
  ex.slots = slots;
  ex.pool = pool;
  ex.cu = cu;
  return run(dims, w, x, z, out, conv_in, conv_out, h0, h_out, ws, ws_bytes, stream, decode, ex);
}

}  // namespace jm

extern "C" {

size_t jm_mixer_prefill_workspace_size(const jm_mixer_dims* dims) {
  if (check_dims(dims, false) != JM_OK) return 0;
  return (size_t)make_plan(dims, false).total;
}

size_t jm_mixer_decode_workspace_size(const jm_mixer_dims* dims) {
  if (check_dims(dims, true) != JM_OK) return 0;
  // also room for jm_mixer_decode_step_single_kernel (its own layout for the shapes it takes)
  const int64_t plain = make_plan(dims, true).total, single = make_plan(dims, true, false, true).total;
  return (size_t)(plain > single ? plain : single);
}

int jm_mixer_prefill(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x, const void* z,
                     void* out, const void* conv_state_in, void* conv_state_out, const float* ssm_state_in,
                     float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, false);
}

int jm_mixer_decode_step(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x, const void* z,
                         void* out, const void* conv_state_in, void* conv_state_out, const float* ssm_state_in,
                         float* ssm_state_out, void* workspace, size_t workspace_bytes, void* stream) {
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, true);
}

int jm_mixer_decode_step_noalloc(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                                 const void* z, void* out, const void* conv_state_in, void* conv_state_out,
                                 const float* ssm_state_in, float* ssm_state_out, void* stream) {
  const int s = check_dims(dims, true);
  if (s != JM_OK) return s;
  if (make_plan(dims, true).total > (int64_t)kStaticScratchBytes) return JM_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const int r = static_scratch(&ws);
  if (r != JM_OK) return r;
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, ws,
             kStaticScratchBytes, stream, true);
}

size_t jm_mixer_decode_noalloc_scratch_limit(void) { return kStaticScratchBytes; }

int jm_mixer_decode_step_slots(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                               const void* z, void* out, void* conv_state_pool, float* ssm_state_pool,
                               int32_t pool_size, const int32_t* slots, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!slots) return JM_ERR_INVALID_ARG;
  Extras ex;
  ex.slots = slots;
  ex.pool = pool_size;
  return run(dims, weights, x, z, out, conv_state_pool, conv_state_pool, ssm_state_pool, ssm_state_pool,
             workspace, workspace_bytes, stream, true, ex);
}

int jm_mixer_decode_step_single_kernel(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                                       const void* z, void* out, const void* conv_state_in, void* conv_state_out,
                                       const float* ssm_state_in, float* ssm_state_out, int32_t pool_size,
                                       const int32_t* slots, void* workspace, size_t workspace_bytes, void* stream) {
  Extras ex;
  ex.single = true;
  if (slots) {   // pools, updated in place
    if (conv_state_out != conv_state_in || ssm_state_out != ssm_state_in) return JM_ERR_INVALID_ARG;
    ex.slots = slots;
    ex.pool = pool_size;
  }
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, true, ex);
}

size_t jm_mixer_prefill_varlen_workspace_size(const jm_mixer_dims* dims) {
  if (check_dims(dims, false) != JM_OK) return 0;
  return (size_t)make_plan(dims, false, true).total;
}

int jm_mixer_prefill_varlen(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                            const void* z, void* out, const int32_t* cu_seqlens, const void* conv_state_in,
                            void* conv_state_out, const float* ssm_state_in, float* ssm_state_out,
                            const int32_t* slots, int32_t pool_size, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!cu_seqlens) return JM_ERR_INVALID_ARG;
  Extras ex;
  ex.cu = cu_seqlens;
  ex.slots = slots;
  ex.pool = pool_size;
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, false, ex);
}

int jm_mixer_prefill_profiled(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                              const void* z, void* out, const void* conv_state_in, void* conv_state_out,
                              const float* ssm_state_in, float* ssm_state_out, void* workspace,
                              size_t workspace_bytes, void* stream, void** events, int n_events) {
  if (!events) return JM_ERR_INVALID_ARG;
  Extras ex;
  ex.events = events;
  ex.n_events = n_events;
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, false, ex);
}

int jm_mixer_decode_step_profiled(const jm_mixer_dims* dims, const jm_mixer_weights* weights, const void* x,
                                  const void* z, void* out, const void* conv_state_in, void* conv_state_out,
                                  const float* ssm_state_in, float* ssm_state_out, void* workspace,
                                  size_t workspace_bytes, void* stream, void** events, int n_events) {
  if (!events) return JM_ERR_INVALID_ARG;
  Extras ex;
  ex.events = events;
  ex.n_events = n_events;
  return run(dims, weights, x, z, out, conv_state_in, conv_state_out, ssm_state_in, ssm_state_out, workspace,
             workspace_bytes, stream, true, ex);
}

const char* jm_stage_name(int stage) { return stage >= 0 && stage < JM_STAGES ? kStageNames[stage] : "?"; }

int jm_mixer_prefill_workspace_layout(const jm_mixer_dims* dims, jm_workspace_layout* layout) {
  if (!layout) return JM_ERR_INVALID_ARG;
  const int s = check_dims(dims, false);
  if (s != JM_OK) return s;
  const Plan p = make_plan(dims, false);
  layout->xc = p.off_xc;
  layout->dbc = p.off_dbc;
  layout->dln = p.off_dln;
  layout->bc = p.off_bc;
  layout->delta = p.off_delta;
  layout->carries = p.off_loc;
  layout->dbc_splits = p.splits;
  layout->scan_chunks = p.P;
  layout->total_bytes = p.total;
  layout->xproj_path = !p.bf16 ? 2 : p.narrow ? 1 : p.tall ? (jm::conv_xproj_fits(p.xs) ? 4 : 3) : 0;
  layout->reserved = 0;
  return JM_OK;
}

const char* jm_status_string(int status) {
  switch (status) {
    case JM_OK: return "ok";
    case JM_ERR_INVALID_ARG: return "invalid argument (NULL required pointer, bad size or stride)";
    case JM_ERR_UNSUPPORTED: return "unsupported dims or dtype (d_state must be 16, d_conv 4, d_inner % 64 == 0, "
                                    "dt_rank a multiple of 8 up to 512)";
    case JM_ERR_ALIGNMENT: return "misaligned pointer (16 bytes required) or row stride (multiple of 8)";
    case JM_ERR_WORKSPACE: return "workspace missing or too small";
    case JM_ERR_HIP: return "HIP runtime error while enqueueing a kernel";
    case JM_ERR_SCRATCH_LIMIT: return "the call needs more than the 32 MiB of device scratch that "
                                      "jm_mixer_decode_step_noalloc has (fewer sequences per call, or use "
                                      "jm_mixer_decode_step with a workspace)";
    default: return "unknown status";
  }
}

}  // extern "C"
