/*
 * jm_layer.h — C ABI of the whole Jamba Mamba layer around the mixer (same library as jm_mixer.h).
 *
 * One of Jamba's Mamba layers is a pre-norm residual block around the mixer: the neurarch "Jamba" page's
 * Structure table and Exported PyTorch listing put an RMSNorm of width 4096 (nn.RMSNorm(4096)) before each
 * Mamba block and a residual add after it; llm-architectures-explained, "Jamba v0.1", Facts: RMSNorm, pre
 * placement; TransformerLens, "supported_architectures.jamba", architecture overview: pre-norm, mixer,
 * residual, and the mixer's in_proj / conv1d / x_proj / dt_proj / out_proj.  No page prints the norm's
 * epsilon; callers pass it (Jamba's mixer norms use 1e-6).  Per token:
 *
 *   1. hn      = x_res / sqrt(mean(x_res^2) + layer_norm_eps) * norm_w      (width d_model)
 *   2. [x | z] = in_proj_w . hn               in_proj_w [2C, d_model], rows x first, then z; no bias
 *   3. y       = the mixer of jm_mixer.h on x, z (strided views of the in_proj output)
 *   4. out     = x_res + out_proj_w . y       out_proj_w [d_model, C]; no bias
 *
 * Steps 2 and 4 are plain GEMMs and run through hipBLASLt (bf16 operands with fp32 accumulation in
 * JM_BF16 mode, fp32 in JM_F32 mode); step 1 is a HIP kernel; step 3 is the mixer library itself.
 *
 * Conventions are those of jm_mixer.h (device pointers owned by the caller, `stream` a hipStream_t as
 * void*, validation before anything is enqueued, negative jm_status on error).  Additionally:
 *  - x_res and out are [batch, seqlen, d_model] (decode: [batch, d_model]), contiguous, in io_dtype;
 *    out may be the same buffer as x_res (an in-place residual update), but must not partially overlap it.
 *  - d_model must be a positive multiple of 8.  The mixer dims' x_row_stride and z_row_stride are ignored
 *    (the layer sets both to 2 * d_inner).
 *  - The workspace holds hn, the in_proj output, y, the mixer's own workspace and hipBLASLt's; it is
 *    scratch.  The library keeps one hipBLASLt handle per device and a cache of the chosen GEMM
 *    algorithms, both created on first use (host memory, and hipBLASLt's own one-time initialisation).
 *  - Both GEMMs (handle, descriptors, algorithm for the call's shape) are resolved during validation:
 *    JM_ERR_HIP (hipBLASLt set-up failed) and JM_ERR_UNSUPPORTED (no algorithm for the shape) are returned
 *    with nothing enqueued and no state written.  After that only a failed launch (JM_ERR_HIP, as for any
 *    kernel) can end a call early, and then the states may already hold this call's update.
 */
#ifndef JM_LAYER_H
#define JM_LAYER_H

#include "jm_mixer.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct jm_layer_dims {
  jm_mixer_dims mixer;     /* the mixer's sizes (batch, seqlen, d_inner, ...); row strides ignored */
  int32_t d_model;         /* residual width (4096 for Jamba v0.1) */
  float layer_norm_eps;    /* epsilon of the pre-norm (1e-6 for Jamba) */
} jm_layer_dims;

/* Device pointers to the layer's weights, all in io_dtype, contiguous. */
typedef struct jm_layer_weights {
  const void* norm_w;      /* [d_model] */
  const void* in_proj_w;   /* [2 * d_inner, d_model] */
  const void* out_proj_w;  /* [d_model, d_inner] */
  jm_mixer_weights mixer;  /* the mixer's weights (jm_mixer.h) */
} jm_layer_weights;

/* Bytes of device workspace the layer needs for these dims (0 if the dims are invalid). */
size_t jm_layer_prefill_workspace_size(const jm_layer_dims* dims);
size_t jm_layer_decode_workspace_size(const jm_layer_dims* dims);

/*
 * Prefill: the layer over `seqlen` tokens of each of `batch` sequences.
 *   x_res           in   [batch, seqlen, d_model]
 *   out             out  [batch, seqlen, d_model]; may be x_res itself
 *   conv_state_*, ssm_state_*: the mixer's states, exactly as in jm_mixer_prefill
 *   workspace       scratch of at least jm_layer_prefill_workspace_size(dims) bytes
 * seqlen == 0 is valid: out is untouched and the states are copied through.
 */
int jm_layer_prefill(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res, void* out,
                     const void* conv_state_in, void* conv_state_out,
                     const float* ssm_state_in, float* ssm_state_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step: one token per sequence (the prefill definition with seqlen = 1).
 *   x_res, out      [batch, d_model]
 *   states          as in jm_mixer_decode_step (both required; outputs may alias inputs)
 *   workspace       scratch of at least jm_layer_decode_workspace_size(dims) bytes
 */
int jm_layer_decode_step(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                         void* out, const void* conv_state_in, void* conv_state_out,
                         const float* ssm_state_in, float* ssm_state_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step over pools of per-sequence states (serving): jm_layer_decode_step with sequence b's states in
 * row slots[b] of conv_state_pool [pool_size, C, K-1] and ssm_state_pool [pool_size, C, N] float32, updated
 * in place, exactly as in jm_mixer_decode_step_slots (slots: device int32 [batch]; valid entries distinct;
 * an entry outside [0, pool_size) runs from zero states and stores none).
 */
int jm_layer_decode_step_slots(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                               void* out, void* conv_state_pool, float* ssm_state_pool, int32_t pool_size,
                               const int32_t* slots, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill of a packed batch of variable-length sequences (continuous batching): the layer over
 * x_res [seqlen, d_model] holding dims->mixer.batch sequences back to back (dims->mixer.seqlen tokens in
 * all), split by the device offsets cu_seqlens [batch + 1], with states per sequence (or in pools through
 * slots), exactly as in jm_mixer_prefill_varlen.  out [seqlen, d_model] may be x_res itself.  The
 * workspace holds at least jm_layer_prefill_varlen_workspace_size(dims) bytes.
 */
size_t jm_layer_prefill_varlen_workspace_size(const jm_layer_dims* dims);
int jm_layer_prefill_varlen(const jm_layer_dims* dims, const jm_layer_weights* weights, const void* x_res,
                            void* out, const int32_t* cu_seqlens, const void* conv_state_in, void* conv_state_out,
                            const float* ssm_state_in, float* ssm_state_out, const int32_t* slots,
                            int32_t pool_size, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* JM_LAYER_H */
