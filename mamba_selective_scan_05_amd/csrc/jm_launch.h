// Host-side launchers of the mixer kernels (internal to the library; the public ABI is jm_mixer.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "jm_mixer.h"

namespace jm {

// A packed batch of variable-length sequences: sequence s holds packed tokens [cu[s], cu[s+1]) (device
// int32 [nseq + 1]); its states are row s of the state tensors, or row slots[s] of pools of `pool` rows
// (slots null: row s).  cu == nullptr: a plain [B, L] batch.
struct VarSeqs {
  const int32_t* cu;
  const int32_t* slots;
  int nseq;
  int pool;
};

// Causal depthwise conv1d (K = 4) + bias + SiLU over [B, L, C] -> xc [B*L, C] (contiguous).  With v.cu the
// input is one packed axis of L tokens (B = 1) and each sequence starts from its own conv state.
void launch_conv_silu(bool bf16, const void* x, int64_t x_stride, const void* conv_w, const void* conv_b,
                      const void* conv_state_in, void* xc, int B, int L, int C, hipStream_t st,
                      const VarSeqs& v = VarSeqs{nullptr, nullptr, 0, 0});

// The same conv + SiLU for the first min(L, 3) tokens of each of the B sequences only (the tokens whose left
// context is the conv state).
void launch_conv_head(bool bf16, const void* x, int64_t x_stride, const void* conv_w, const void* conv_b,
                      const void* conv_state_in, void* xc, int B, int L, int C, hipStream_t st);

// Packed batches, per sequence: conv_state_out = the last K-1 entries of the sequence's extended input
// (x after its conv state), and for an empty sequence ssm_state_out = ssm_state_in (zeros for null).
// Every read of a row precedes its write, so outputs may alias inputs; run it after the conv.
void launch_varlen_states(bool bf16, const void* x, int64_t x_stride, const void* conv_in, void* conv_out,
                          const float* h0, float* h_out, int C, int L, const VarSeqs& v, hipStream_t st);

// One token per sequence (seqlen 1): the same conv + SiLU -> xc [B, C], and the shifted conv state ->
// conv_state_out [B, C, K-1] (may alias conv_state_in; zeros stand in for a NULL conv_state_in).  With
// slots, sequence b's conv state is row slots[b] of pools of `pool` rows; a slot outside [0, pool) runs
// from a zero state and stores none.
void launch_conv_step(bool bf16, const void* x, int64_t x_stride, const void* conv_w, const void* conv_b,
                      const void* conv_state_in, void* xc, void* conv_state_out, int B, int C, hipStream_t st,
                      const int32_t* slots = nullptr, int pool = 0);

// Tokens per x_proj workgroup tile (bf16 path: 128, or 256 in the tall layout for long inputs), and the
// number of column groups (grid z) for N columns in the wide or tall (288 columns per workgroup) or narrow
// (32) layout.
int xproj_token_tile(bool tall = false);
int xproj_column_groups(int N, bool narrow);
// Most channel slices the x_proj contraction may be split over (the norm step adds at most this many).
constexpr int kMaxXprojSplits = 16;

// dbc partial sums: part[s, m, n] = sum over channel slice s of xc[m, k] * w[n, k].
void launch_xproj(bool bf16, const void* xc, const void* w, float* part, int M, int N, int K, int splits,
                  bool narrow, hipStream_t st, bool tall = false);

// bf16, the tall layout, B sequences of L tokens each (not packed): the conv + SiLU of launch_conv_silu
// (xc [B*L, K] written, bit for bit the same) and launch_xproj's partial sums, in one kernel that reads x
// once.  conv_xproj_fits(x_stride) must hold.
bool conv_xproj_fits(int64_t x_stride);
void launch_conv_xproj(const void* x, int64_t x_stride, const void* conv_w, const void* conv_b, const void* conv_in,
                       void* xc, const void* w, float* part, int B, int L, int N, int K, int splits, hipStream_t st);

// Sum the partials in slice order, RMSNorm the dt / B / C slices -> dln [M, R] (io dtype), bc [M, 2N].
void launch_norm(bool bf16, const float* part, int splits, int M, int R, int N, const void* dt_norm_w,
                 const void* b_norm_w, const void* c_norm_w, float eps, void* dln, float* bc, hipStream_t st);

// delta[m, c] = softplus(sum_r dln[m, r] * w[c, r] + b[c])  (io dtype).
void launch_dtproj(bool bf16, const void* dln, const void* w, const void* b, void* delta, int M, int C, int R,
                   hipStream_t st);

struct ScanArgs {
  const void* xc;        // [B*L, C] io dtype
  const void* delta;     // [B*L, C] io dtype
  const void* z;         // [B*L rows, z_stride]
  int64_t z_stride;
  const float* bc;       // [B*L, 2N]
  const void* A_log;     // [C, N]
  const void* D;         // [C]
  const float* h0;       // [B, C, N] or null
  void* out;             // [B*L, C]
  float* h_out;          // [B, C, N]
  const void* x;         // raw input, for the conv state
  int64_t x_stride;
  const void* conv_in;   // [B, C, K-1] or null
  void* conv_out;        // [B, C, K-1], or null when the conv step already wrote the state
  float* loc;            // [B, P, N+1, C]   per-piece local end states and dt sums (P > 1)
  float* cin;            // [B, P, N, C]     per-piece incoming states (P > 1)
  int B, L, C, P, Lp;
  // State pools (decode, or a packed batch): sequence b's SSM state is row slots[b] of h0 / h_out (pools of
  // `pool` rows); a slot outside [0, pool) runs from a zero state and stores nothing.  Null: row b.
  const int32_t* slots;
  int pool;
  // Packed variable-length batch (B = 1, L packed tokens): sequence s holds tokens [cu[s], cu[s+1]) and its
  // SSM state is state row s (or slots[s]); the conv state is written by launch_varlen_states.  snap
  // [P, N, C]: the initial state of the last sequence starting strictly inside a piece and running past it,
  // saved by the local pass for the full pass (which must not read h0 rows other pieces may overwrite).
  const int32_t* cu;
  int nseq;
  float* snap;
  // 1: the input matrix is the exact zero-order hold (exp(dt A) - 1) / A * B instead of dt * B
  int zoh;
  // Training forward (plain batch, dt * B): the state entering every backward piece (tokens 0, kBwdPiece,
  // 2 kBwdPiece, ...) -> saved [B, saved_P, N, C]; null: not saved.
  float* saved;
  int saved_P;
};

// The selective scan with D skip and SiLU(z) gate, split into P pieces of Lp tokens per sequence.
// marks (optional): events recorded before the local pass, the carry pass and the full pass.
void launch_scan(bool bf16, const ScanArgs& a, hipStream_t st, void* const* marks = nullptr);
// Only the local and carry passes (P > 1): every piece's incoming state -> a.cin.
void launch_scan_carries(bool bf16, const ScanArgs& a, hipStream_t st);

// The layer's projections for at most 256 tokens, bf16: Y[m, n] = sum_k X[m, k] W[n, k] (+ R[m, n]), row
// strides ldx / ldw / ldr / ldy in elements (multiples of 8).  skinny_gemm_splits gives the K split for a
// shape (0: the shape is not supported: M > 256, N or K not a multiple of 64), and with it the column-block
// width launch_skinny_gemm uses (128 when a split into whole K slices gives at least 256 workgroups of 128
// columns, else 64); with more than one split the fp32 partial sums take splits * M * N * 4 bytes of `part`,
// within ws_bytes.  R may alias Y.  Pass launch_skinny_gemm the splits skinny_gemm_splits returned for the same
// shape.
int skinny_gemm_splits(int M, int N, int K, int64_t ws_bytes);
void launch_skinny_gemm(const void* X, int64_t ldx, const void* W, int64_t ldw, const void* R, int64_t ldr, void* Y,
                        int64_t ldy, int M, int N, int K, int splits, float* part, hipStream_t st);

// fp32 contractions on the matrix cores: Y[m, n] = sum_k X[m, k] W[n, k] over `splits` equal K slices
// (partial sums at Y + s * M * N), or with bias (splits = 1) softplus(. + bias[n]).  K / splits a multiple of
// 4, X and W 16-byte aligned.  gemm_f32_tiles: the workgroups of one K slice.
int64_t gemm_f32_tiles(int64_t M, int N);
void launch_gemm_f32(const float* X, const float* W, const float* bias, float* Y, int M, int N, int K, int splits,
                     hipStream_t st);

// The one-token step (bf16 I/O) as one cooperative kernel with two grid-wide barriers: conv + SiLU and the
// x_proj partial sums per unit of 32 sequences x 256 channels, the norms per sequence, then dt_proj and the
// state update per unit.  Plain batches and state pools (slots).
// decode_fused_shape_ok: the shapes it takes (d_inner a multiple of 256, dt_rank a multiple of 32 up to 256,
// at most 1024 sequences); decode_fused_available: the current device supports cooperative launches and
// fits the kernel; decode_fused_slices: the x_proj slices it writes (part: slices * B * (R + 2 N) floats).
// xc is written only when a unit cannot stay in LDS (more units than resident workgroups).  Returns the
// launch status.
struct DecodeArgs {
  const void* x;
  int64_t xs;
  const void* z;
  int64_t zs;
  const void* conv_w;
  const void* conv_b;
  const void* conv_in;
  void* conv_out;
  const void* x_proj_w;
  const void* dt_norm_w;
  const void* b_norm_w;
  const void* c_norm_w;
  float eps;
  const void* dt_proj_w;
  const void* dt_proj_b;
  const void* A_log;
  const void* D;
  const float* h0;
  float* h_out;
  void* out;
  const int32_t* slots;
  int pool;
  void* xc;      // [B, C]
  float* part;   // [C / 256, B, R + 2N]
  void* dln;     // [B, R]
  float* bc;     // [B, 2N]
  uint64_t* flags;    // kDecodeMaxGroups flags of the grid barriers (any contents)
  uint64_t launch;    // set by launch_decode_fused
  int B, C, R, zoh;
};
constexpr int kDecodeMaxGroups = 1024;
bool decode_fused_shape_ok(int B, int C, int R);
bool decode_fused_available();
int decode_fused_slices(int C);
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t st);

// Scan pieces for B sequences of L tokens over C channels: about a fixed number of waves in the full pass,
// pieces of at least 128 tokens, each piece's rows (row_bytes apart) under 2 GiB.
void scan_plan(int B, int L, int C, int64_t row_bytes, int* P, int* Lp);

// Backward of the gated scan (training).  Pieces of kBwdPiece tokens; all [B*L, C] tensors contiguous.
constexpr int kBwdPiece = 32;
struct BwdArgs {
  const void* xc;        // [B*L, C] io dtype
  const void* delta;     // [B*L, C]
  const void* z;         // [B*L, C]
  const void* dout;      // [B*L, C]
  const float* bc;       // [B*L, 2N]  B then C
  const void* A_log;     // [C, N]
  const void* D;         // [C]
  const float* h0;       // [B, C, N] or null
  const float* dh_final; // [B, C, N] or null
  const float* cin;      // [B, P, N, C]  incoming states of the pieces (forward carry)
  float* bloc;           // [B, P, N+1, C] backward local records
  float* gin;            // [B, P, N, C]  incoming gradients of the pieces
  float* pA;             // [B*P, C, N]
  float* pD;             // [B*P, C]
  float* pbc;            // [C/64, B*L, 2N]
  void* dxc;             // [B*L, C] io dtype
  void* ddelta;          // [B*L, C]
  void* dz;              // [B*L, C]
  float* dbc;            // [B*L, 2N]
  float* dA_log;         // [C, N]
  float* dD;             // [C]
  float* dh0;            // [B, C, N] or null
  int B, L, C, P;
};
void launch_scan_backward(bool bf16, const BwdArgs& a, hipStream_t st);

// The mixer behind jm_mixer_prefill / jm_mixer_decode_step, for the layer entry points: the workspace bytes
// of a call (a negative jm_status for invalid dims), every check of a call without launching anything, and
// the validated call itself (each a jm_status).
// With slots, the states are pools of `pool` rows indexed by slots[b], as in jm_mixer_decode_step_slots;
// with cu (prefill only), a packed batch as in jm_mixer_prefill_varlen.
int64_t mixer_workspace_bytes(const jm_mixer_dims* dims, bool decode, bool varlen = false);
int mixer_validate(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
                   const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
                   bool decode, const int32_t* slots = nullptr, int pool = 0, const int32_t* cu = nullptr);
int mixer_run(const jm_mixer_dims* dims, const jm_mixer_weights* w, const void* x, const void* z, void* out,
              const void* conv_in, void* conv_out, const float* h0, float* h_out, void* ws, size_t ws_bytes,
              void* stream, bool decode, const int32_t* slots = nullptr, int pool = 0,
              const int32_t* cu = nullptr);

// seqlen == 0: copy the states through (zeros for a NULL input).
void launch_state_passthrough(bool bf16, const void* conv_in, void* conv_out, const float* h0, float* h_out,
                              int B, int C, hipStream_t st);

}  // namespace jm
