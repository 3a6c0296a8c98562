/*
 * ssd_backward.h -- C ABI of the backward pass of the SSD layer core: the
 * gradients of ssd_chunk_scan_fwd with respect to all of its inputs, for the
 * training use the pages describe (Qiita "Mamba-2" article, sections 3.3 and
 * 5: the chunked matrix form is what trains fast; youngju.dev "Mamba /
 * selective SSM", "SSDアルゴリズムとチャンク分割": the chunked algorithm, whose
 * steps are differentiated here). Same conventions as ssd_api.h (device
 * pointers, caller-owned buffers and workspace, dense row-major layouts,
 * 16-byte aligned pointers, asynchronous on `stream`, every check on the host
 * before any launch, nothing written on error, deterministic results).
 *
 * Nothing of the forward is kept between the calls: the backward recomputes
 * the in-chunk decays, the chunk states and the states entering each chunk
 * from the inputs (recomputation instead of storing activations). It chooses
 * its own chunk length from headdim and dstate (the largest of 128, 64, 32
 * whose per-chunk tiles fit a compute unit's local memory); the
 * gradients do not depend on it beyond rounding.
 */
#ifndef SSD_BACKWARD_H
#define SSD_BACKWARD_H

#include "ssd_api.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workspace bytes for ssd_chunk_scan_bwd; 0 when the sizes are not supported.
 * Like the forward's query it depends on the current HIP device (its
 * compute-unit count chooses the launches, see below). */
SSD_API size_t ssd_chunk_scan_bwd_workspace(int batch, int seqlen, int nheads, int headdim, int dstate,
                                            int ngroups, ssd_dtype dtype);

/*
 * Which launches ssd_chunk_scan_bwd uses for these sizes on the current HIP
 * device (0 for sizes it rejects): bit 0 set = the recomputation of the chunk
 * states and of the states entering each chunk runs as one walk per (batch
 * row, 64 columns of the flattened (head, headdim) axis), as in the forward
 * (else a chunk-state and a state-passing launch); bit 1 set = the gradients
 * of those states come from the same walk run over the chunks in reverse
 * (else a per-chunk launch and a reverse state-passing launch). The
 * gradients agree up to rounding either way.
 */
SSD_API int ssd_chunk_scan_bwd_fused_walks(int batch, int seqlen, int nheads, int headdim, int dstate,
                                           int ngroups, ssd_dtype dtype);

/*
 * Gradients of the loss L through y = ssd_chunk_scan_fwd(x, dt, A, B, C, D,
 * init_state) and its final_state, given dy = dL/dy and dfinal = dL/dfinal:
 *
 * Forward definition (per batch row b, head h of group g, state column p):
 *   s_t = exp(dt_t A_h) s_{t-1} + dt_t B_t x_t[p],  s_{-1} = init[:, p]
 *   y_t[p] = C_t . s_t + D_h x_t[p],  final[:, p] = s_{T-1}
 * (youngju.dev "Mamba / selective SSM", section "LTIからSelectionへの切り替え").
 *
 * Inputs (as for ssd_chunk_scan_fwd):
 *   x [b,T,H,P], dt [b,T,H], B, C [b,T,G,N]   dtype
 *   A [H] fp32, D [H] fp32 or NULL (= 0), init_state [b,H,N,P] fp32 or NULL (= 0)
 *   dy [b,T,H,P] dtype;  dfinal [b,H,N,P] fp32 or NULL (= 0)
 * Outputs (overwritten, not accumulated):
 *   dx [b,T,H,P], ddt [b,T,H], dB, dC [b,T,G,N]   dtype (summed over the
 *       heads of each group for dB, dC; rounded once at the end)
 *   dA [H] fp32 (summed over b and T)
 *   dD [H] fp32 or NULL (not written); it is sum over b, t, p of dy x
 *   dinit [b,H,N,P] fp32 or NULL (not written)
 *
 * Supported: dtype SSD_BF16, dstate in {32, 64, 128, 256}, headdim in {32,
 * 64, 128} except headdim 128 with dstate 256; others return SSD_ERR_SHAPE.
 * Outputs must not overlap each other, the inputs or the workspace
 * (SSD_ERR_ALIAS). Other errors as for ssd_chunk_scan_fwd: SSD_ERR_NULL (x,
 * dt, A, B, C, dy, dx, ddt, dA, dB or dC NULL), SSD_ERR_DTYPE, SSD_ERR_ALIGN,
 * SSD_ERR_WORKSPACE (workspace NULL or smaller than
 * ssd_chunk_scan_bwd_workspace), SSD_ERR_HIP.
 */
SSD_API ssd_status ssd_chunk_scan_bwd(const void *x, const void *dt, const float *A, const void *B,
                                      const void *C, const float *D, const float *init_state, const void *dy,
                                      const float *dfinal, void *dx, void *ddt, float *dA, void *dB, void *dC,
                                      float *dD, float *dinit, int batch, int seqlen, int nheads, int headdim,
                                      int dstate, int ngroups, ssd_dtype dtype, void *workspace,
                                      size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_BACKWARD_H */
