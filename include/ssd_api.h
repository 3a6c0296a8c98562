/*
 * ssd_api.h -- C ABI of the MI355X (gfx950) selective-state-space layer core.
 *
 * The layer is the multi-head selective SSM with one scalar decay per head
 * (Qiita "Mamba-2" article, sections 4.1-4.2: A = -exp(A_log) is a scalar
 * shared inside a head; B and C are shared by the heads of a group):
 *
 *     abar_t = exp(dt_t * A_h)                                   (discretised A)
 *     h_t    = abar_t * h_{t-1} + (dt_t * B_t) x_t^T             (state, N x P)
 *     y_t    = C_t^T h_t + D_h * x_t
 *
 * (youngju.dev "Mamba / selective SSM", section "LTIからSelectionへの切り替え":
 * abar = exp(dt A), bbar = dt B, h_t = abar h_{t-1} + bbar x_t, y_t = C h_t.)
 *
 * ssd_chunk_scan_fwd evaluates it over a whole sequence chunk by chunk: inside
 * a chunk the masked semiseparable product runs as matrix products, across
 * chunks the state is passed by the recurrence (youngju.dev page, section
 * "SSDアルゴリズムとチャンク分割"; Qiita article, section 4.2, step 3).
 * ssd_state_update is the recurrent single-token mode used for inference
 * (Qiita article, section 3.3; waylandz LLM book ch. 32, section 32.2.4).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers (HIP, gfx950). The caller owns
 *    every buffer, including the forward workspace; the library allocates
 *    nothing and keeps no state between calls.
 *  - Layouts are dense, row-major, last index fastest; no strides:
 *      x, y   [batch, seqlen, nheads, headdim]    (decode: [batch, nheads, headdim])
 *      dt     [batch, seqlen, nheads]             (decode: [batch, nheads])
 *      B, C   [batch, seqlen, ngroups, dstate]    (decode: [batch, ngroups, dstate])
 *      state  [batch, nheads, dstate, headdim]    fp32 (init_state, final_state, state)
 *      A, D   [nheads] fp32
 *    Head h reads group g = h / (nheads / ngroups).
 *  - `dtype` is the element type of x, dt, B, C and y (fp32 or bf16). A, D
 *    and every state are fp32; accumulation is fp32.
 *  - dt is used as given (already positive, e.g. after a softplus); A <= 0 is
 *    the supported domain.
 *  - Every pointer must be 16-byte aligned.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and never synchronise. All argument checks run on the host
 *    before the first launch: on any error nothing is launched, nothing is
 *    written and a status is returned. A launch failure returns SSD_ERR_HIP;
 *    a device-side fault surfaces at the caller's next synchronisation, or,
 *    with SSD_DEBUG=1 in the environment (read once per process), at the
 *    call itself: every entry point that launched work then synchronises its
 *    stream before returning and answers SSD_ERR_HIP if a kernel failed (a
 *    debugging aid: it serialises the caller with the GPU and cannot be used
 *    under stream capture).
 *  - No C++ exception crosses this interface. Results are deterministic
 *    (no atomics): the same inputs give bitwise-identical outputs.
 */
#ifndef SSD_API_H
#define SSD_API_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SSD_API __attribute__((visibility("default")))
#else
#define SSD_API
#endif

/* In C++ the status and dtype enums are declared over int, so that every int
 * value is a valid value of them (a caller may pass any int: unknown values
 * are answered, not undefined). */
#ifdef __cplusplus
#define SSD_ENUM(name) enum name : int
#else
#define SSD_ENUM(name) enum name
#endif

typedef SSD_ENUM(ssd_status) {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,      /* a required pointer is NULL                          */
    SSD_ERR_SHAPE = 2,     /* a dimension is < 1, nheads % ngroups != 0, or a
                              headdim / dstate outside the supported range        */
    SSD_ERR_DTYPE = 3,     /* dtype is not SSD_F32 or SSD_BF16                    */
    SSD_ERR_CHUNK = 4,     /* chunk_len is not one of 16, 32, 64, 128, 256        */
    SSD_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the query's answer   */
    SSD_ERR_HIP = 6,       /* a kernel launch failed                              */
    SSD_ERR_ALIAS = 7,     /* an output overlaps an input it must not overlap     */
    SSD_ERR_ALIGN = 8,     /* a pointer is not 16-byte aligned                    */
    SSD_ERR_VALUE = 9      /* a scalar argument is out of range (eps, activation) */
} ssd_status;

/* Element type of the activations (an unknown value: SSD_ERR_DTYPE). */
typedef SSD_ENUM(ssd_dtype) { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Supported ranges (checked; anything else is SSD_ERR_SHAPE / SSD_ERR_CHUNK):
 *   1 <= headdim <= 256, 1 <= dstate <= 256, chunk_len in {16,32,64,128,256},
 *   batch, seqlen, nheads, ngroups >= 1, nheads % ngroups == 0,
 *   batch <= 65535, ceil(seqlen / chunk_len) <= 65535, and every kernel grid
 *   of the forward pass under 2^32 work-items (for the bf16 matrix-core path
 *   about batch * nchunks * nheads < 2^23, e.g. 8.4M chunk-heads).          */
#define SSD_MAX_HEADDIM 256
#define SSD_MAX_DSTATE 256

/*
 * Bytes of device workspace ssd_chunk_scan_fwd needs for these sizes; 0 when
 * the sizes are invalid. The workspace holds the per-chunk cumulative decay
 * (fp32 [batch, nheads, nchunks, chunk_len], nchunks = ceil(seqlen/chunk_len)),
 * the step sizes widened to fp32 in the same layout, and the states entering
 * each chunk (fp32 [batch, nchunks, nheads, dstate, headdim] on the generic
 * path; on the bf16 matrix-core path bf16, plus the chunk states in fp32 when
 * they are passed by a separate launch, plus the C B^T products of each
 * chunk and a copy of C in the order the matrix-core kernels read it). It
 * carries nothing from one call to the next. `dtype` is an
 * argument because the two paths need different amounts. The answer depends
 * on the current HIP device (its compute-unit count chooses the launches,
 * see ssd_chunk_scan_fwd_fused_states): query on the device that runs the
 * call.
 */
SSD_API size_t ssd_chunk_scan_fwd_workspace(int batch, int seqlen, int nheads, int headdim,
                                    int dstate, int ngroups, int chunk_len, ssd_dtype dtype);

/*
 * Chunked forward over a whole sequence (the SSD algorithm: intra-chunk
 * matrix products plus inter-chunk state passing; youngju.dev page, section
 * "SSDアルゴリズムとチャンク分割"; Qiita article, section 4.2).
 *
 *   x [b,T,H,P], dt [b,T,H], B/C [b,T,G,N] : dtype        (read)
 *   A [H], D [H] fp32                        (read; D may be NULL = no skip term)
 *   init_state [b,H,N,P] fp32                (read; NULL = zero state). It is the
 *                                            state before token 0, so token 0
 *                                            decays it by exp(dt_0 A_h).
 *   y [b,T,H,P] dtype                        (written; rounded to nearest even
 *                                            when dtype is bf16)
 *   final_state [b,H,N,P] fp32               (written; NULL = not produced). The
 *                                            state after token T-1; feeding it as
 *                                            init_state of the next call continues
 *                                            the sequence (youngju.dev page,
 *                                            "状態初期化とシーケンス境界").
 *   workspace / workspace_bytes              (caller-owned scratch, see the query)
 *
 * seqlen need not be a multiple of chunk_len: the last chunk behaves as if
 * padded with dt = 0 tokens, which leave the state unchanged (youngju.dev page,
 * "デバッグチェックリスト": padding tokens get dt = 0). Results do not depend on
 * chunk_len beyond rounding.
 * Aliasing: y must not overlap any input or final_state; final_state may be
 * the same buffer as init_state (in place), but must not partially overlap it.
 */
SSD_API ssd_status ssd_chunk_scan_fwd(const void *x, const void *dt, const float *A, const void *B,
                              const void *C, const float *D, const float *init_state,
                              void *y, float *final_state,
                              int batch, int seqlen, int nheads, int headdim, int dstate,
                              int ngroups, int chunk_len, ssd_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * How ssd_chunk_scan_fwd with these sizes forms the states entering each
 * chunk on the current HIP device: 0 = a chunk-state launch and a separate
 * state-passing launch (also for sizes the call would reject); k >= 1 = one
 * fused launch of walks, each batch row cut into k segments of consecutive
 * chunks (1: whole rows). The results agree up to rounding either way.
 *
 * A walk takes one batch row (or one segment of it) and 64 columns of the
 * flattened (head, headdim) axis (headdim 32: two heads, which must share a
 * B/C group) through its chunks in order with the running state on chip and
 * writes only the bf16 states entering each chunk. It is used for the bf16
 * matrix-core path with dstate 128 or 256 and chunk_len a multiple of 64 when
 * the walks fill the device in one round: between half and all of the
 * compute units, or, at dstate 128 with chunk_len >= 128, up to two per unit.
 * Where whole rows give fewer walks than half the units (a few long rows),
 * each row is cut into k > 1 segments, about one walk per unit; every segment
 * starts from zero, a short recurrence over the segments gives the state
 * entering each one, and the chunk outputs add its decayed contribution (the
 * state handed from chunk to chunk composes associatively; youngju.dev page,
 * "SSDアルゴリズムとチャンク分割"). It reads the device's compute-unit count,
 * so it needs a current HIP device (0 without one).
 */
SSD_API int ssd_chunk_scan_fwd_fused_states(int batch, int seqlen, int nheads, int headdim, int dstate,
                                            int ngroups, int chunk_len, ssd_dtype dtype);

/*
 * The same choice for a device with `compute_units` compute units (no device
 * needed): returns what ssd_chunk_scan_fwd_fused_states returns on such a
 * device, and, when it is above 0, the number of chunks per segment in
 * *seglen (the last segment may have fewer; segment k covers chunks
 * k * seglen .. min(nchunks, (k + 1) * seglen) - 1). *seglen is 0 otherwise;
 * seglen may be NULL. Sizes the forward rejects give 0.
 */
SSD_API int ssd_chunk_scan_fwd_plan(int batch, int seqlen, int nheads, int headdim, int dstate, int ngroups,
                                    int chunk_len, ssd_dtype dtype, int compute_units, int *seglen);

/*
 * Measurement variant of ssd_chunk_scan_fwd: identical computation, and it
 * times its four stages, in launch order: [0] cumulative sums, [1] chunk
 * states, [2] state passing, [3] chunk outputs. stage_events holds 8
 * hipEvent_t handles created by the caller (e.g. with hipEventCreate):
 * stage_events[2 i] and stage_events[2 i + 1] are recorded at the start and
 * the end of stage i's kernel by that kernel's own dispatch
 * (hipExtLaunchKernel), so hipEventElapsedTime on the pair gives the kernel's
 * execution time on `stream`. On the bf16 matrix-core path one launch
 * computes the cumulative sums, the C B^T tiles and the chunk states; stage 0
 * launches nothing there and its two events are recorded back to back. Where
 * ssd_chunk_scan_fwd_fused_states is 1, stage [1] also passes the states
 * between chunks and stage [2] launches nothing the same way; where it is
 * above 1, stage [1] is the segmented walk and stage [2] the recurrence over
 * the segments.
 * stage_events may be NULL (then it is ssd_chunk_scan_fwd). A failed event
 * record returns SSD_ERR_HIP.
 */
SSD_API ssd_status ssd_chunk_scan_fwd_timed(const void *x, const void *dt, const float *A,
                                            const void *B, const void *C, const float *D,
                                            const float *init_state, void *y, float *final_state,
                                            int batch, int seqlen, int nheads, int headdim,
                                            int dstate, int ngroups, int chunk_len,
                                            ssd_dtype dtype, void *workspace,
                                            size_t workspace_bytes, void *stream,
                                            void *const *stage_events);

/*
 * ssd_chunk_scan_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. It allocates nothing and calls no
 * allocating routine; its workspace is a scratch array that the library
 * holds in device memory, SSD_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, for the
 * life of the process (the 130M-shaped layer, batch 8 x 2048 tokens, needs
 * about 36 MiB of it). Sizes whose workspace (ssd_chunk_scan_fwd_workspace)
 * exceeds that return SSD_ERR_WORKSPACE before any launch; every other
 * argument and error is as for ssd_chunk_scan_fwd, and the results are
 * bit-for-bit the same. The first call on a device looks up that device's
 * array (SSD_ERR_HIP if there is no current device). Every call on one GPU
 * uses the same array: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream do
 * not. No byte of the array needs to start at zero.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
SSD_API ssd_status ssd_chunk_scan_fwd_noalloc(const void *x, const void *dt, const float *A, const void *B,
                                              const void *C, const float *D, const float *init_state,
                                              void *y, float *final_state, int batch, int seqlen, int nheads,
                                              int headdim, int dstate, int ngroups, int chunk_len,
                                              ssd_dtype dtype, void *stream);

/*
 * One recurrent step for every (batch row, head), in place on `state`
 * (Qiita article, section 3.3: inference runs as a recurrence with constant
 * memory; waylandz LLM book ch. 32, section 32.2.4, recurrent form):
 *
 *   state [b,H,N,P] fp32 : h <- exp(dt*A_h) h + (dt*B) x^T     (read, written)
 *   x [b,H,P], dt [b,H], B/C [b,G,N] : dtype                   (read)
 *   A [H], D [H] fp32 (D may be NULL)                           (read)
 *   y [b,H,P] dtype : y = C^T h_new + D_h x                     (written)
 *
 * Aliasing: y must not overlap state or any input.
 */
SSD_API ssd_status ssd_state_update(float *state, const void *x, const void *dt, const float *A,
                            const void *B, const void *C, const float *D, void *y,
                            int batch, int nheads, int headdim, int dstate, int ngroups,
                            ssd_dtype dtype, void *stream);

/*
 * Packed variable-length sequences. nseq sequences are packed along one token
 * axis of total_tokens tokens: sequence i is tokens cu_seqlens[i] ..
 * cu_seqlens[i+1] - 1, and each starts from its own initial state, so
 * nothing of one sequence reaches another (youngju.dev "Mamba / selective
 * SSM" page, section "状態初期化とシーケンス境界": the state is set explicitly
 * at the start of every sequence of a batch). The result for sequence i is
 * ssd_chunk_scan_fwd on its tokens alone from init_states[i]:
 *   x, y   [total_tokens, nheads, headdim]        dtype
 *   dt     [total_tokens, nheads]                 dtype
 *   B, C   [total_tokens, ngroups, dstate]        dtype
 *   cu_seqlens   [nseq + 1] int32 DEVICE array, 0 = cu[0] <= cu[1] <= ...
 *                <= cu[nseq] = total_tokens (empty sequences allowed). It is
 *                not read on the host: offsets outside [0, total_tokens] or
 *                decreasing ones are clamped on the device, which keeps every
 *                access in bounds but gives unspecified results.
 *   init_states  [nseq, nheads, dstate, headdim] fp32 or NULL (= zeros)
 *   final_states [nseq, nheads, dstate, headdim] fp32 or NULL; may be the
 *                init_states buffer itself. An empty sequence's final state
 *                is its initial state.
 * Chunks never straddle two sequences: sequence i takes ceil(len_i /
 * chunk_len) chunks, the last one partly filled. Only the bf16 matrix-core
 * configuration is supported (dtype SSD_BF16, dstate in {32, 64, 128, 256},
 * headdim in {32, 64, 128}, chunk_len >= 32); others return SSD_ERR_SHAPE, as
 * does nseq outside 1 .. 65535. Other errors as for ssd_chunk_scan_fwd
 * (cu_seqlens must be 4-byte aligned). The workspace size comes from
 * ssd_chunk_scan_fwd_varlen_workspace (0 when the sizes are not supported).
 */
SSD_API size_t ssd_chunk_scan_fwd_varlen_workspace(int total_tokens, int nseq, int nheads, int headdim,
                                                   int dstate, int ngroups, int chunk_len,
                                                   ssd_dtype dtype);
SSD_API ssd_status ssd_chunk_scan_fwd_varlen(const void *x, const void *dt, const float *A, const void *B,
                                             const void *C, const float *D, const int *cu_seqlens,
                                             const float *init_states, void *y, float *final_states,
                                             int total_tokens, int nseq, int nheads, int headdim,
                                             int dstate, int ngroups, int chunk_len, ssd_dtype dtype,
                                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * How ssd_chunk_scan_fwd_varlen with these sizes forms the states entering
 * each chunk on a device with `compute_units` compute units (no device
 * needed; the call itself reads the current device's count): 0 = a
 * chunk-state launch over every chunk and a recurrence per sequence over its
 * chunks (also for sizes the call rejects); k >= 1 = the fused walks of
 * ssd_chunk_scan_fwd_fused_states over the packed row of chunks: each
 * sequence takes ceil(len / chunk_len) chunk slots (slot
 * floor(cu[i] / chunk_len) + i onwards, ceil(total_tokens / chunk_len) + nseq
 * slots in all, some unused), and the slots are cut into k segments of
 * *seglen consecutive slots (the last may have fewer), one walk per segment
 * and 64 columns, as many as fill the device in one round. A walk restarts
 * from a sequence's initial state at its first chunk (the state never
 * crosses from one sequence into the next) and writes the final state of
 * every sequence that ends inside it; a short recurrence over the segments
 * gives the state entering each one and completes the sequences that cross
 * a segment boundary. seglen may be NULL (*seglen is 0 with the per-chunk
 * path). Used for dstate 128 or 256 and chunk_len a multiple of 64 (headdim
 * 32 needs an even number of heads per group). The results agree up to
 * rounding either way.
 */
SSD_API int ssd_chunk_scan_fwd_varlen_plan(int total_tokens, int nseq, int nheads, int headdim, int dstate,
                                           int ngroups, int chunk_len, ssd_dtype dtype, int compute_units,
                                           int *seglen);

/* Static, NUL-terminated description of a status code. */
SSD_API const char *ssd_status_string(ssd_status status);

#ifdef __cplusplus
}
#endif

#endif /* SSD_API_H */
