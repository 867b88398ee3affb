/*
 * jm_scan.h — C ABI of the gated selective scan on its own, forward and backward, for training (same library
 * as jm_mixer.h).
 *
 * The scan is the recurrence of the Jamba Guide (aifetchly blog), section "Inside the Mamba State-Space
 * Layers: Mathematical Mechanics" (discretisation equations and recurrent state update), with the mixer's
 * D skip and SiLU(z) gate, exactly as inside jm_mixer_prefill:
 *
 *   A = -exp(A_log),  h_t = exp(delta_t * A) * h_{t-1} + delta_t * B_t * x_t,
 *   y_t = C_t . h_t + D * x_t,  out_t = y_t * SiLU(z_t).
 *
 * The same section notes that training runs the scan over whole sequences at once; training also needs its
 * backward, which the pages do not print: jm_scan_backward is the chain rule through these lines in reverse
 * time (gradients of x, delta, A_log, B, C, D, z and the initial state).
 *
 * Conventions are those of jm_mixer.h (device pointers owned by the caller, `stream` a hipStream_t as void*,
 * no allocation, validation before anything is enqueued, negative jm_status on error).  Layouts (row-major,
 * C = d_inner, N = d_state = 16, T = batch * seqlen tokens, all contiguous):
 *   x (the scan input, the conv output xc), delta, z, out, dout and their gradients: [batch, seqlen, C] in
 *   io_dtype;  bc and dbc: [T, 2N] float32, B_t in columns 0..N-1 and C_t in N..2N-1 (shared by all
 *   channels);  A_log [C, N] and D [C] in io_dtype, their gradients float32;  states [batch, C, N] float32.
 * Requirements: d_state == 16, d_inner a positive multiple of 64, 1 <= batch <= 65536, 0 <= seqlen <= 2^21, every
 * pointer 16-byte aligned.
 */
#ifndef JM_SCAN_H
#define JM_SCAN_H

#include "jm_mixer.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jm_scan_dims {
  int32_t batch;
  int32_t seqlen;
  int32_t d_inner;
  int32_t d_state;
  int32_t io_dtype;   /* enum jm_dtype */
} jm_scan_dims;

/* Bytes of device workspace of each call (0 if the dims are invalid). */
size_t jm_scan_forward_workspace_size(const jm_scan_dims* dims);
size_t jm_scan_backward_workspace_size(const jm_scan_dims* dims);

/*
 * Bytes of the saved states that jm_scan_forward_train writes and jm_scan_backward may read (0 if the dims are
 * invalid): float32 [batch, ceil(seqlen / 32), N, C], entry [b, p, n, c] being state n of channel c entering
 * token 32 p of sequence b.
 */
size_t jm_scan_saved_states_size(const jm_scan_dims* dims);

/*
 * Forward: out [batch, seqlen, C] and the final state h_out [batch, C, N] (required) from x, delta, z, bc,
 * A_log, D and the initial state h0 (NULL: zeros).  h_out may alias h0.
 */
int jm_scan_forward(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                    const void* A_log, const void* D, const float* h0, void* out, float* h_out,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same forward (out and h_out bit for bit as jm_scan_forward), that also writes saved_states (required
 * when seqlen > 0; jm_scan_saved_states_size bytes, owned by the caller) for jm_scan_backward, which then
 * skips recomputing them.  Workspace: jm_scan_forward_workspace_size.
 */
int jm_scan_forward_train(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                          const void* A_log, const void* D, const float* h0, void* out, float* h_out,
                          float* saved_states, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward: the gradients of  sum(dout * out) + sum(dh_final * h_L)  with respect to every input.
 *   inputs   x, delta, z, bc, A_log, D, h0 (NULL: zeros) as given to the forward; dout; dh_final [batch, C, N]
 *            (the gradient arriving at the final state; NULL: zero)
 *   outputs  dx, ddelta, dz [batch, seqlen, C] in io_dtype; dbc [T, 2N] float32; dA_log [C, N] and dD [C]
 *            float32, summed over the batch; dh0 [batch, C, N] float32 (NULL: not computed)
 *   saved_states  what jm_scan_forward_train wrote for these same inputs, or NULL: the backward then
 *            recomputes the states entering its 32-token pieces from x, delta, bc and h0 itself.  Inside each
 *            piece the states are recomputed either way.
 * Outputs must not overlap the inputs.  seqlen == 0 is valid: dA_log = dD = 0 and dh0 = dh_final.
 */
int jm_scan_backward(const jm_scan_dims* dims, const void* x, const void* delta, const void* z, const float* bc,
                     const void* A_log, const void* D, const float* h0, const void* dout, const float* dh_final,
                     const float* saved_states, void* dx, void* ddelta, void* dz, float* dbc, float* dA_log,
                     float* dD, float* dh0, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JM_SCAN_H */
