/*
 * jm_mixer.h — C ABI of the Jamba Mamba-1 mixer library for AMD MI355X (gfx950).
 *
 * The library computes the part of a Mamba-1 mixer that sits between in_proj and out_proj
 * (TransformerLens, "supported_architectures.jamba", architecture overview: the Mamba-1 mixer is
 * in_proj / conv1d / x_proj / dt_proj / out_proj plus Jamba's dt / B / C RMSNorms on the selective
 * parameters).  Given the two halves x and z of the in_proj output it runs, per token and channel:
 *
 *   1. xc   = SiLU(conv_b + causal depthwise conv1d_K(x))            K = d_conv = 4
 *   2. dbc  = x_proj_w . xc                  -> dt (dt_rank) | B (d_state) | C (d_state)
 *   3. dt, B, C each RMSNorm'ed:  v / sqrt(mean(v^2) + eps) * w
 *   4. delta = softplus(dt_proj_w . dt + dt_proj_b)
 *   5. h_t  = exp(delta_t * A) * h_{t-1} + delta_t * B_t * xc_t,   A = -exp(A_log)
 *      y_t  = C_t . h_t + D * xc_t
 *   6. out  = y * SiLU(z)
 *
 * Steps 4-5 are the selective-scan (S6) discretisation and recurrence of the Jamba Guide
 * (aifetchly blog), section "Inside the Mamba State-Space Layers: Mathematical Mechanics"
 * (discretisation equations and recurrent state update), with B discretised as delta * B as that page
 * does; the A_log convention and the softplus on a biased dt projection follow the same page's
 * SimpleMambaSSM listing.  The dimensions are Jamba v0.1's (llm-architectures-explained, "Jamba v0.1",
 * "Every architecture field": d_inner 8192, state 16, conv kernel 4, dt_rank 256).  The conv bias, the
 * SiLU after the conv, the D skip and the SiLU(z) gate are the mixer's conventional form; the pages do
 * not print them.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or from a torch CUDA tensor), owned by the
 *    caller, and must stay valid until the work enqueued on `stream` has completed.  The library never
 *    allocates or frees device memory and keeps no state between calls; calls are re-entrant, but two
 *    calls that run concurrently need distinct workspaces.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call only enqueues work
 *    and returns; device faults surface at the caller's next synchronisation.
 *  - io_dtype selects the element type of x, z, out, the conv state and every weight: JM_F32 (float) or
 *    JM_BF16 (bfloat16 stored as uint16).  The SSM state is always float32.  In JM_BF16 mode x_proj and
 *    dt_proj run on bf16 matrix cores with fp32 accumulation, xc and delta are kept in bf16, everything
 *    else is fp32 arithmetic; in JM_F32 mode every step is fp32.
 *  - Layouts (row-major, C = d_inner, N = d_state, R = dt_rank, K = d_conv, W = R + 2N):
 *      x, z        [batch, seqlen, row_stride]: element (b, t, c) at (b*seqlen + t)*row_stride + c,
 *                  row_stride = x_row_stride / z_row_stride (0 means C), so x and z may be strided
 *                  views of one in_proj output.
 *      out         [batch, seqlen, C], contiguous.
 *      conv state  [batch, C, K-1]: the K-1 raw inputs preceding the first token, oldest first.
 *      SSM state   [batch, C, N] float32.
 *      conv_w [C, K] (tap K-1 multiplies the current token), conv_b [C], x_proj_w [W, C] with rows
 *      ordered dt | B | C, dt_norm_w [R], b_norm_w [N], c_norm_w [N], dt_proj_w [C, R], dt_proj_b [C],
 *      A_log [C, N], D [C] — all contiguous, in io_dtype.
 *  - Requirements (else an error is returned and nothing is enqueued or written):
 *      discretization a jm_discretization value, d_state == 16, d_conv == 4, d_inner a positive multiple of 64, 1 <= dt_rank <= 512 with
 *      dt_rank % 8 == 0, 1 <= batch <= 65536, 0 <= seqlen <= 2097152 (2^21) for a prefill, row strides >= d_inner
 *      and multiples of 8 elements, every pointer 16-byte aligned (int32 index vectors: 4-byte), and
 *      norm_eps >= 0.
 *  - Errors: every entry point returns JM_OK (0) or a negative jm_status.  Arguments are validated on
 *    the host before anything is enqueued; on an error nothing is launched and no output is written.
 *    NaN / Inf in the inputs propagate and are not reported.  No C++ exception crosses this ABI.
 */
#ifndef JM_MIXER_H
#define JM_MIXER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum jm_status {
  JM_OK = 0,
  JM_ERR_INVALID_ARG = -1,  /* NULL required pointer, non-positive size, stride < d_inner, eps < 0  */
  JM_ERR_UNSUPPORTED = -2,  /* d_state != 16, d_conv != 4, d_inner % 64, dt_rank out of range, dtype */
  JM_ERR_ALIGNMENT = -3,    /* a pointer not 16-byte aligned, or a row stride not a multiple of 8   */
  JM_ERR_WORKSPACE = -4,    /* workspace NULL or smaller than the matching *_workspace_size()       */
  JM_ERR_HIP = -5,          /* the HIP runtime reported an error when enqueueing a kernel           */
  JM_ERR_SCRATCH_LIMIT = -6 /* jm_mixer_decode_step_noalloc: the call exceeds its static scratch     */
};

enum jm_dtype { JM_F32 = 0, JM_BF16 = 1 };

/*
 * The input matrix of the discretised recurrence.  The Jamba Guide's discretisation equation gives the exact
 * zero-order hold (dt A)^-1 (exp(dt A) - I) dt B and, as its approximation, dt B:
 *   JM_DISC_EULER  Bbar = dt * B                        (the default; what the rest of this header describes)
 *   JM_DISC_ZOH    Bbar = (exp(dt * A) - 1) / A * B     (A diagonal; for |dt A| < 1/16 evaluated by its series)
 */
enum jm_discretization { JM_DISC_EULER = 0, JM_DISC_ZOH = 1 };

/* Sizes of one call.  For jm_mixer_decode_step, seqlen is ignored (one token per sequence). */
typedef struct jm_mixer_dims {
  int32_t batch;
  int32_t seqlen;
  int32_t d_inner;
  int32_t d_state;
  int32_t dt_rank;
  int32_t d_conv;
  int32_t io_dtype;      /* enum jm_dtype */
  float norm_eps;        /* epsilon of the three RMSNorms (1e-6 for Jamba) */
  int64_t x_row_stride;  /* elements between consecutive tokens of x; 0 means d_inner */
  int64_t z_row_stride;  /* elements between consecutive tokens of z; 0 means d_inner */
  int32_t discretization; /* enum jm_discretization (0: dt * B) */
  int32_t reserved;       /* must be 0 */
} jm_mixer_dims;

/* Device pointers to the mixer's weights, all in io_dtype.  conv_b may be NULL (zero bias). */
typedef struct jm_mixer_weights {
  const void* conv_w;     /* [C, K]   */
  const void* conv_b;     /* [C]      */
  const void* x_proj_w;   /* [W, C]   */
  const void* dt_norm_w;  /* [R]      */
  const void* b_norm_w;   /* [N]      */
  const void* c_norm_w;   /* [N]      */
  const void* dt_proj_w;  /* [C, R]   */
  const void* dt_proj_b;  /* [C]      */
  const void* A_log;      /* [C, N]   */
  const void* D;          /* [C]      */
} jm_mixer_weights;

/*
 * Bytes of device workspace jm_mixer_prefill needs for these dims (0 if the dims are invalid).
 * The workspace holds the step intermediates (xc, the x_proj output, the normalised dt/B/C, delta)
 * and the per-chunk carries of the scan; it is scratch, its contents on return are unspecified.
 */
size_t jm_mixer_prefill_workspace_size(const jm_mixer_dims* dims);

/*
 * Prefill: run the mixer over `seqlen` tokens of each of `batch` sequences.
 *   x, z            in   [batch, seqlen, row_stride] (see layouts)
 *   out             out  [batch, seqlen, C]
 *   conv_state_in   in   [batch, C, K-1] or NULL (zeros)
 *   conv_state_out  out  [batch, C, K-1]: the last K-1 raw inputs (for seqlen < K-1 it includes entries
 *                        of conv_state_in); may alias conv_state_in.
 *   ssm_state_in    in   [batch, C, N] float32 or NULL (zeros)
 *   ssm_state_out   out  [batch, C, N] float32: the state after the last token; may alias ssm_state_in.
 *   workspace       scratch of at least jm_mixer_prefill_workspace_size(dims) bytes.
 * seqlen == 0 is valid: out is untouched and the states are copied through.
 * Calling it on tokens [0, L1) and then on [L1, L) with the returned states gives the same result as one
 * call on [0, L) up to rounding.
 */
int jm_mixer_prefill(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                     const void* x, const void* z, void* out,
                     const void* conv_state_in, void* conv_state_out,
                     const float* ssm_state_in, float* ssm_state_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace jm_mixer_decode_step (and jm_mixer_decode_step_slots and
 * jm_mixer_decode_step_single_kernel) needs for these dims (0 if invalid). */
size_t jm_mixer_decode_workspace_size(const jm_mixer_dims* dims);

/*
 * Decode step: advance each of `batch` sequences by one token (the prefill definition with seqlen = 1),
 * the generation-time use of the Mamba conv / recurrent cache (TransformerLens
 * "supported_architectures.jamba": generation threads the conv and recurrent states through a cache).
 *   x, z            in   [batch, row_stride]: token t of sequence b at b*row_stride
 *   out             out  [batch, C]
 *   conv_state_in   in   [batch, C, K-1] (required);  conv_state_out out, may alias conv_state_in
 *   ssm_state_in    in   [batch, C, N] float32 (required);  ssm_state_out out, may alias ssm_state_in
 *   workspace       scratch of at least jm_mixer_decode_workspace_size(dims) bytes.
 */
int jm_mixer_decode_step(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                         const void* x, const void* z, void* out,
                         const void* conv_state_in, void* conv_state_out,
                         const float* ssm_state_in, float* ssm_state_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step that allocates nothing, for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).  It is
 * jm_mixer_decode_step with the same kernels and results, except that the intermediates live in a device
 * array inside the library instead of a caller workspace:
 *   - the array holds jm_mixer_decode_noalloc_scratch_limit() bytes (32 MiB) on each GPU the library runs
 *     on, for the lifetime of the process; its address is looked up once per device, on the first call
 *     made with that device current (hipGetSymbolAddress: no allocation);
 *   - a call whose jm_mixer_decode_workspace_size(dims) exceeds the limit returns JM_ERR_SCRATCH_LIMIT with
 *     nothing enqueued (at d_inner 8192, dt_rank 256 in bf16, up to 768 sequences fit);
 *   - every call on one GPU shares that GPU's array and leaves its contents behind; the step needs nothing
 *     in it to start at zero.  Calls that overlap on one GPU (concurrent streams or threads) race on the
 *     array: serialise them, or use jm_mixer_decode_step with one workspace each.
 * Arguments, layouts, aliasing and the other errors are those of jm_mixer_decode_step.
 */
int jm_mixer_decode_step_noalloc(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                                 const void* x, const void* z, void* out,
                                 const void* conv_state_in, void* conv_state_out,
                                 const float* ssm_state_in, float* ssm_state_out, void* stream);

/* Bytes of device scratch jm_mixer_decode_step_noalloc has on each GPU. */
size_t jm_mixer_decode_noalloc_scratch_limit(void);

/*
 * Decode step over a pool of per-sequence states: the decode step above, with sequence b's conv and SSM
 * states kept in row slots[b] of two state pools that the step updates in place.  This is the state
 * layout of a serving engine that batches whichever sequences are generating at the moment (Jamba Guide,
 * aifetchly blog, "Production Engineering: Serving & Hardware Best Practices": serving with continuous
 * batching; TransformerLens "supported_architectures.jamba": generation carries the Mamba conv and
 * recurrent states in a cache), so that a batch can be formed without gathering and scattering states.
 *   x, z, out         as in jm_mixer_decode_step ([batch, row_stride] in, [batch, C] out)
 *   conv_state_pool   in/out [pool_size, C, K-1] in io_dtype
 *   ssm_state_pool    in/out [pool_size, C, N] float32
 *   pool_size         rows in each pool (>= 1)
 *   slots             DEVICE int32 [batch], 4-byte aligned: the pool row of each sequence.  The valid
 *                     entries must be distinct (two sequences on one row race).  An entry outside
 *                     [0, pool_size) — e.g. -1 for a padding entry of the batch — runs from zero states,
 *                     writes its out row and stores no state; it is not an error (the host does not read
 *                     the device's slot values).
 *   workspace         scratch of at least jm_mixer_decode_workspace_size(dims) bytes.
 * Rows of the pools that no valid slot names are left untouched.
 */
int jm_mixer_decode_step_slots(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                               const void* x, const void* z, void* out,
                               void* conv_state_pool, float* ssm_state_pool, int32_t pool_size,
                               const int32_t* slots, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The decode step as a single kernel, the one-token step of the generation loop (TransformerLens
 * "supported_architectures.jamba": generation carries the Mamba conv and recurrent caches from token to
 * token): one cooperative launch with two grid-wide barriers — conv + SiLU and the x_proj partial sums per
 * unit of 32 sequences x 256 channels, then the dt / B / C norms per sequence, then dt_proj, the state update
 * and the gate per unit.
 *   slots == NULL     jm_mixer_decode_step: the same arguments, layouts and aliasing (pool_size ignored).
 *   slots != NULL     jm_mixer_decode_step_slots: conv_state_in / ssm_state_in are the pools of pool_size
 *                     rows, updated in place (conv_state_out and ssm_state_out must equal them, else
 *                     JM_ERR_INVALID_ARG); slot semantics as there.
 *   workspace         at least jm_mixer_decode_workspace_size(dims) bytes, as for jm_mixer_decode_step; its
 *                     contents on entry do not matter (the grid barriers key their flags to the launch).
 * Results agree with jm_mixer_decode_step within the bf16 tolerance (its x_proj is summed over 256-channel
 * slices instead).  Supported: bf16 I/O, d_inner a multiple of 256, dt_rank a multiple of 32 up to 256, at
 * most 1024 sequences, on a device with cooperative launches; anything else returns JM_ERR_UNSUPPORTED with
 * nothing enqueued (there is no fallback to the multi-kernel step).  On MI355X this is slower than
 * jm_mixer_decode_step, which stays the default decode path: a cooperative launch costs ~20 us of dispatch,
 * and each grid barrier ~5-7 us, more than the separate kernels' boundaries.
 */
int jm_mixer_decode_step_single_kernel(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                                       const void* x, const void* z, void* out,
                                       const void* conv_state_in, void* conv_state_out,
                                       const float* ssm_state_in, float* ssm_state_out,
                                       int32_t pool_size, const int32_t* slots,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace jm_mixer_prefill_varlen needs for these dims (0 if the dims are invalid). */
size_t jm_mixer_prefill_varlen_workspace_size(const jm_mixer_dims* dims);

/*
 * Prefill of a packed batch of variable-length sequences, the prefill side of serving with continuous
 * batching (Jamba Guide, aifetchly blog, "Production Engineering: Serving & Hardware Best Practices"):
 * prompts of different lengths run in one call with no padding.  Each sequence gets exactly the result of
 * jm_mixer_prefill on its own tokens and states (up to rounding); no state crosses from one sequence to
 * the next.
 *   dims->batch       number of sequences;  dims->seqlen  total tokens of all of them (the packed length)
 *   x, z              in   [seqlen, row_stride]: the sequences' tokens one after another
 *   out               out  [seqlen, C]
 *   cu_seqlens        DEVICE int32 [batch + 1], 4-byte aligned: sequence s is packed tokens
 *                     [cu_seqlens[s], cu_seqlens[s+1]); cu_seqlens[0] = 0, non-decreasing,
 *                     cu_seqlens[batch] = seqlen.  Empty sequences are allowed (their states carry over).
 *                     The host does not read these values; offsets that break the rules give unspecified
 *                     results, but every access stays inside the buffers described here.
 *   states            slots == NULL: conv_state_* [batch, C, K-1] and ssm_state_* [batch, C, N] float32,
 *                     sequence s at row s.  slots != NULL (DEVICE int32 [batch], 4-byte aligned): pools of
 *                     pool_size rows, sequence s at row slots[s]; the valid entries must be distinct, and an
 *                     entry outside [0, pool_size) runs from zero states and stores none.
 *                     conv_state_in / ssm_state_in may be NULL (zeros); the outputs are required and may
 *                     alias the inputs (in-place update of a state pool).  Rows no sequence names are
 *                     left untouched.
 *   workspace         scratch of at least jm_mixer_prefill_varlen_workspace_size(dims) bytes.
 */
int jm_mixer_prefill_varlen(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                            const void* x, const void* z, void* out, const int32_t* cu_seqlens,
                            const void* conv_state_in, void* conv_state_out,
                            const float* ssm_state_in, float* ssm_state_out,
                            const int32_t* slots, int32_t pool_size,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* jm_status_string(int status);

/*
 * Where jm_mixer_prefill keeps its intermediates inside the workspace (byte offsets; -1 = not kept),
 * for tests that check the steps one by one after a call.  Element types: xc and delta in io_dtype
 * [batch*seqlen, C]; dbc float32 [splits, batch*seqlen, W] (partial sums over `splits` slices of the
 * channels, summed in order); dln in io_dtype [batch*seqlen, R]; bc float32 [batch*seqlen, 2N] (B then C).
 */
typedef struct jm_workspace_layout {
  int64_t xc, dbc, dln, bc, delta, carries;
  int32_t dbc_splits;     /* number of channel slices the x_proj contraction is split over */
  int32_t scan_chunks;    /* number of sequence pieces the scan runs in parallel per channel */
  int64_t total_bytes;
  int32_t xproj_path;     /* x_proj kernel layout: 0: bf16 matrix cores, 128-token x 288-column tiles;
                             1: bf16 matrix cores, 32-column groups (few tokens); 2: fp32 on the matrix cores;
                             3: bf16 matrix cores, 256-token x 288-column tiles (32768 tokens or more);
                             4: as 3, with the conv1d + SiLU computed inside x_proj from x (one read of x,
                                xc still written for the scan; the conv stage of the profiled call is empty) */
  int32_t reserved;
} jm_workspace_layout;

int jm_mixer_prefill_workspace_layout(const jm_mixer_dims* dims, jm_workspace_layout* layout);

/*
 * Per-stage timing, for benchmarks: the same computation as jm_mixer_prefill / jm_mixer_decode_step, with
 * events[i] (hipEvent_t handles created by the caller, passed as void*) recorded on `stream` just before
 * stage i is enqueued and events[JM_STAGES] after the last stage, so hipEventElapsedTime(events[i],
 * events[i+1]) is the time of stage i.  A stage with no work for these dims (e.g. the scan's local and
 * carry passes when the sequence is not split) gets an empty interval.  n_events must be >= JM_STAGES + 1.
 * Stage i is named by jm_stage_name(i).
 */
#define JM_STAGES 7
const char* jm_stage_name(int stage);
int jm_mixer_prefill_profiled(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                              const void* x, const void* z, void* out,
                              const void* conv_state_in, void* conv_state_out,
                              const float* ssm_state_in, float* ssm_state_out,
                              void* workspace, size_t workspace_bytes, void* stream,
                              void** events, int n_events);
int jm_mixer_decode_step_profiled(const jm_mixer_dims* dims, const jm_mixer_weights* weights,
                                  const void* x, const void* z, void* out,
                                  const void* conv_state_in, void* conv_state_out,
                                  const float* ssm_state_in, float* ssm_state_out,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void** events, int n_events);

#ifdef __cplusplus
}
#endif

#endif /* JM_MIXER_H */
