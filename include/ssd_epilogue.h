/*
 * ssd_epilogue.h -- C ABI of the two element-wise stages next to the SSD layer
 * core in the Mamba-2 block: the gated RMS normalisation of the core's output
 * and the depthwise causal convolution of its inputs. Same conventions as
 * ssd_api.h (device pointers, caller-owned buffers, dense row-major layouts,
 * 16-byte aligned pointers, asynchronous on `stream`, every check on the host
 * before any launch, nothing written on error, deterministic results).
 * `dtype` is the element type of the activation tensors (SSD_F32 or
 * SSD_BF16); weights and biases are fp32; arithmetic is fp32 and outputs are
 * rounded to `dtype` (bf16: round to nearest even).
 */
#ifndef SSD_EPILOGUE_H
#define SSD_EPILOGUE_H

#include "ssd_api.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Gated RMS normalisation, rmsnorm(y) * silu(z) (Qiita "Mamba-2" article,
 * section 4.2, SSD block step 4), over groups of `group` consecutive
 * channels of each token's `dim`-channel feature vector:
 *
 *   out[t, c] = y[t, c] / sqrt(mean_{c' in group(c)} y[t, c']^2 + eps)
 *               * weight[c] * silu(z[t, c]),     silu(v) = v / (1 + exp(-v))
 *
 * group = dim normalises the whole vector (the page's rmsnorm(y) over the
 * layer width); group = headdim normalises each head.
 *   y, z, out  [ntokens, dim]  dtype (e.g. the core's y viewed as [b*T, H*P])
 *   weight     [dim]           fp32
 * out may be y itself (in place); otherwise out must not overlap y, z or
 * weight. Errors: SSD_ERR_NULL (y, z, weight or out NULL), SSD_ERR_SHAPE
 * (ntokens, dim or group < 1, dim % group != 0, or more than 2^26 rows
 * ntokens * dim / group), SSD_ERR_VALUE (eps negative or not finite),
 * SSD_ERR_DTYPE, SSD_ERR_ALIGN, SSD_ERR_ALIAS.
 */
SSD_API ssd_status ssd_gated_rmsnorm(const void *y, const void *z, const float *weight, void *out,
                                     long ntokens, int dim, int group, float eps, ssd_dtype dtype,
                                     void *stream);

#define SSD_CONV_MAX_WIDTH 8

/*
 * Depthwise causal convolution over tokens, channels last (the Mamba block's
 * Conv1d(C, C, K, padding K-1, groups C, bias) trimmed to the first seqlen
 * outputs, then SiLU: youngju.dev "Mamba / selective SSM" page, the Mamba
 * block code):
 *
 *   out[b, t, c] = act(bias[c] + sum_{k=0..K-1} weight[c, k] * x[b, t-(K-1)+k, c])
 *
 * where x before token 0 is init_state (its K-1 tokens, oldest first) or
 * zero. act = SiLU when activation == 1, the identity when 0.
 *   x, out       [batch, seqlen, channels]   dtype
 *   weight       [channels, K] fp32, K = kernel_width in 1 .. SSD_CONV_MAX_WIDTH
 *   bias         [channels] fp32 or NULL (= 0)
 *   init_state   [batch, K-1, channels] dtype or NULL (= zeros)
 *   final_state  [batch, K-1, channels] dtype or NULL: receives the last K-1
 *                tokens of (init_state, x), the state a following call (or
 *                ssd_causal_conv1d_update) continues from. It may be the
 *                init_state buffer itself.
 * out must not overlap any other argument; final_state must not overlap x,
 * out, weight or bias, nor partially overlap init_state. Errors:
 * SSD_ERR_NULL (x, weight or out NULL), SSD_ERR_SHAPE (batch, seqlen or
 * channels < 1, K out of range, or more than 2^31 threads
 * batch * ceil(seqlen / 16) * channels), SSD_ERR_VALUE (activation not 0 or
 * 1), SSD_ERR_DTYPE, SSD_ERR_ALIGN, SSD_ERR_ALIAS.
 */
SSD_API ssd_status ssd_causal_conv1d_fwd(const void *x, const float *weight, const float *bias,
                                         const void *init_state, void *out, void *final_state,
                                         int batch, int seqlen, int channels, int kernel_width,
                                         int activation, ssd_dtype dtype, void *stream);

/*
 * One token of the same convolution in its recurrent form (decode), the
 * state updated in place:
 *   out[b, c] = act(bias[c] + sum_{k<K-1} weight[c, k] * state[b, k, c]
 *                   + weight[c, K-1] * x[b, c])
 *   state[b, :, c] <- (state[b, 1:, c], x[b, c])
 *   state  [batch, K-1, channels] dtype (may be NULL when K == 1)
 *   x, out [batch, channels] dtype
 * A run of calls gives what ssd_causal_conv1d_fwd gives on the concatenated
 * tokens. out must not overlap state, x, weight or bias; state must not
 * overlap x, weight or bias. Errors as for ssd_causal_conv1d_fwd (the thread
 * bound is batch * channels).
 */
SSD_API ssd_status ssd_causal_conv1d_update(void *state, const void *x, const float *weight,
                                            const float *bias, void *out, int batch, int channels,
                                            int kernel_width, int activation, ssd_dtype dtype,
                                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_EPILOGUE_H */
