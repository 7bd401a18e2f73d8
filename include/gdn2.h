/*
 * gdn2.h -- C ABI of the MI355X (gfx950) Gated DeltaNet-2 chunked prefill
 * forward.
 *
 * The operation (FlashInfer chunk_gated_delta_rule2 documentation, recurrence
 * display equation): for every packed sequence and every value head, with a
 * K x V float32 state S,
 *
 *     S_t    = diag(exp(g_t)) S_{t-1}
 *     vnew_t = w_t * v_t - (beta_t * k_t)^T S_t
 *     S_t   += k_t vnew_t^T
 *     o_t    = scale * q_t^T S_t
 *
 * evaluated in 64-token chunks through the WY form (the chunked evaluation
 * the burn-gdn2 README "Fused CUDA kernels" section and the FlashRT card's
 * 64-token WY chain describe), returning the output and the final state.
 *
 * All entry points are plain C: no exceptions cross the boundary, no C++ or
 * framework types appear in the signatures.
 */
#ifndef GDN2_H
#define GDN2_H

#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

#define GDN2_ABI_VERSION 5

/* Element types a tensor descriptor may carry. */
typedef enum gdn2_dtype {
    GDN2_DTYPE_BF16 = 1, /* bfloat16 */
    GDN2_DTYPE_F32 = 2,  /* IEEE float32 */
    GDN2_DTYPE_I32 = 3,  /* int32 */
    GDN2_DTYPE_F16 = 4,  /* IEEE float16 */
    GDN2_DTYPE_I64 = 5   /* int64 */
} gdn2_dtype;

/*
 * A view of caller-owned memory: `ndim` dimensions of `shape`, element
 * strides in `stride` (row-major contiguous tensors have
 * stride[d] = prod(shape[d+1..ndim-1])). `data` is a DEVICE pointer; it may
 * be NULL only when the tensor has zero elements.
 */
typedef struct gdn2_tensor {
    void *data;
    int32_t dtype; /* gdn2_dtype */
    int32_t ndim;
    int64_t shape[4];
    int64_t stride[4];
} gdn2_tensor;

/* Status codes. 0 is success; every failure is negative. */
enum {
    GDN2_OK = 0,
    GDN2_ERR_NULL_ARG = -1,    /* a required descriptor or pointer is NULL */
    GDN2_ERR_DTYPE = -2,       /* a tensor has the wrong element type */
    GDN2_ERR_SHAPE = -3,       /* ranks or extents disagree */
    GDN2_ERR_HEADS = -4,       /* HV is not a positive multiple of H */
    GDN2_ERR_UNSUPPORTED = -5, /* K or V not 64 or 128 (the backward: K != V), or an option out of range */
    GDN2_ERR_LAYOUT = -6,      /* a tensor's strides or alignment are not accepted */
    GDN2_ERR_ALIAS = -7,       /* an output overlaps an input */
    GDN2_ERR_HIP = -8          /* the HIP runtime reported an error */
};

/*
 * gdn2_chunk_fwd -- enqueue the GDN-2 chunked prefill forward on `stream`.
 *
 * Tensors (T = total packed tokens, N = number of sequences, H = q/k heads,
 * HV = value heads, K = key dim, V = value dim):
 *   q, k           [T, H, K]       bf16 or float16 (the io type: q's type,
 *                                  which k, v, beta, w and out must share)
 *   v, w           [T, HV, V]      io type
 *   g              [T, HV, K]      float32, bf16 or float16, natural-log
 *                                  decay, each value <= 0 and finite
 *                                  (precondition, not checked)
 *   beta           [T, HV, K]      io type (erase gate, taken as given, e.g.
 *                                  in [0, 1] or [0, 2]; not clamped)
 *   initial_state  [N, HV, K, V]   float32 or bf16, K-major (V innermost);
 *                                  V-major [N, HV, V, K] with the
 *                                  state_layout option
 *   cu_seqlens     [N + 1]         int32 or int64, device memory; cu[0] = 0,
 *                                  non-decreasing, cu[N] = T (precondition,
 *                                  not checked on the device)
 *   out            [T, HV, V]      io type, written for every token
 *   final_state    [N, HV, K, V]   float32 or bf16 (rounded to nearest
 *                                  even), layout as initial_state
 *
 * The FlashInfer parameter list names these element types (q, k, v at
 * float16 or bfloat16, beta and w read at q's type, g at float32, bfloat16
 * or float16, states at float32 or bfloat16, int32 or int64 cu_seqlens).
 * Arithmetic is float32 throughout (a bf16 state is widened on load and
 * carried in float32); the MFMA operands are bf16 for either io type.
 *
 * Value head hv reads q/k head hv / (HV / H) (contiguous groups of value
 * heads share one q/k head).
 *
 * Conditioning: each token's transition I - k (beta * k)^T (after the
 * decay; * elementwise) has the eigenvalue 1 - sum_c beta_c k_c^2, and all
 * its other eigenvalues are 1. With unit-norm keys (or qk_l2norm) and beta
 * in [0, 2] that eigenvalue stays within [-1, 1]; beyond that the
 * recurrence itself amplifies every rounding, and no two evaluations of it
 * (this library's or a float64 one) need agree. The accuracy figures of
 * this library hold in the contracting range.
 *
 * Optional arguments (the FlashInfer parameter-list defaults): g NULL means
 * g = 0, beta NULL means beta = 1, w NULL means w = 1, initial_state NULL
 * means a zero state, final_state NULL means the final state is not written,
 * cu_seqlens NULL means one sequence of T tokens (N = 1). scale == 0 means
 * 1/sqrt(K). A descriptor whose `data` is NULL but which has elements is an
 * error (NULL_ARG) for every tensor; an optional tensor is omitted by passing
 * a NULL descriptor pointer.
 *
 * Supported: K and V each 64 or 128, equal or not (the Flash-GDN-2 README,
 * training paragraph: both head dimensions in {64, 128}); any T >= 0,
 * N >= 1, H >= 1, HV a multiple of H. Empty sequences are allowed (their
 * final state equals their initial state).
 *
 * Ownership: the caller owns every buffer. Inputs and initial_state are only
 * read; out and final_state must be preallocated and are fully written. The
 * library keeps no pointer after the call returns. When it splits sequences
 * (see gdn2_chunk_fwd_opts) it takes a stream-ordered workspace of
 * N * HV * nseg * (2 K V + K K) * 4 bytes on `stream` and returns it with
 * hipFreeAsync on the same stream (nseg = segments per sequence, at most
 * ceil(ceil(T / 64) / segment chunks)); if that allocation fails it runs the
 * sequences whole instead. Otherwise it allocates no device memory.
 * Workspaces come from a memory pool the library creates on each device it
 * runs on (hipMemPoolCreate) with an unlimited release threshold: freed
 * workspace stays in that pool for later calls, so the pool holds up to the
 * largest workspace any call has used until the process ends.
 *
 * Layout (GDN2_ERR_LAYOUT otherwise; strides are in elements, as the
 * FlashInfer parameter list has it, only the innermost dimension needs to be
 * contiguous):
 *   q, k, v, g, beta, w, out: the K or V elements of each (token, head) row
 *     contiguous; the token and head strides free, non-negative and
 *     multiples of 16 bytes, with the token stride at least one row (K or V
 *     elements) and under 2^31 / 64 bytes; e.g. q, k, v as views of one
 *     fused [T, 3, H, D] projection. The rows of out must not overlap.
 *   initial_state, final_state, cu_seqlens: row-major contiguous.
 *   Every data pointer is 16-byte aligned.
 *
 * Aliasing: neither output (out, final_state) may overlap any input or the
 * other output; in particular final_state may not alias initial_state
 * (FlashInfer docs, output_state: the incoming state is read while outgoing
 * states are written): GDN2_ERR_ALIAS.
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued; on failure nothing is enqueued, the return value says why and
 * gdn2_last_error() holds a message. Faults inside the kernel (e.g. a
 * cu_seqlens that breaks its precondition) surface at the caller's next
 * synchronisation with the stream.
 *
 * Semantics: asynchronous (returns after enqueueing, does not synchronise);
 * deterministic (no atomics; the same inputs give the same bits); reentrant.
 */
int gdn2_chunk_fwd(const gdn2_tensor *q, const gdn2_tensor *k,
                   const gdn2_tensor *v, const gdn2_tensor *g,
                   const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                   const gdn2_tensor *initial_state,
                   const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                   const gdn2_tensor *final_state, hipStream_t stream);

/* State layouts (gdn2_fwd_options.state_layout). */
enum {
    GDN2_STATE_KV = 0, /* [N, HV, K, V]: V innermost (default) */
    GDN2_STATE_VK = 1  /* [N, HV, V, K]: K innermost, the FlashInfer layout */
};

/*
 * Options of gdn2_chunk_fwd_opts and gdn2_recurrent_fwd_opts. Set
 * `struct_size` to sizeof(gdn2_fwd_options); fields that lie past a smaller
 * struct_size (a caller built against an earlier version; at least the
 * first two fields) take their defaults (0).
 *
 * seq_split_chunks selects how a sequence is walked:
 *    0  automatic: gdn2_split_plan() for this shape and the current
 *       device's compute-unit count decides (what gdn2_chunk_fwd does);
 *   -1  never split: one workgroup walks each (sequence, value head);
 *  > 0  split every sequence into segments of this many 64-token chunks.
 *
 * A split run is the same computation in another order (the chunked WY form
 * is affine in the entering state): a transition pass gives every segment's
 * end state from a zero start and its K x K state transition, a combine
 * chains them into each segment's entering state, and an output pass runs
 * all segments at once. It pays when there are few (sequence, value head)
 * chains for the compute units and they are long (the parallel scan over
 * the sequence that the FlashInfer docs' output_state note alludes to when
 * it speaks of one sequence split across CTAs).
 */
typedef struct gdn2_fwd_options {
    int32_t struct_size;
    int32_t seq_split_chunks; /* chunked entry only; ignored by the recurrent one */
    /* GDN2_STATE_KV or GDN2_STATE_VK: the layout of initial_state and
     * final_state (FlashInfer parameter list: its states are V-major) */
    int32_t state_layout;
    /* 1: normalise every (token, head) row of q and of k to unit L2 norm
     * inside the kernel, x / max(||x||_2, 1e-12) in float32 from the stored
     * values (the FlashInfer use_qk_l2norm_in_kernel flag; the normalisation
     * is that of the Flash-GDN-2 quick start's torch normalize call); 0: q
     * and k are used as given */
    int32_t qk_l2norm;
} gdn2_fwd_options;

/*
 * gdn2_chunk_fwd_opts -- gdn2_chunk_fwd with options (NULL opts = defaults).
 * Same arguments, contract and errors as gdn2_chunk_fwd, plus
 * GDN2_ERR_SHAPE for a bad options struct (struct_size under 8,
 * seq_split_chunks < -1, state_layout or qk_l2norm out of range).
 */
int gdn2_chunk_fwd_opts(const gdn2_tensor *q, const gdn2_tensor *k,
                        const gdn2_tensor *v, const gdn2_tensor *g,
                        const gdn2_tensor *beta, const gdn2_tensor *w,
                        float scale, const gdn2_tensor *initial_state,
                        const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                        const gdn2_tensor *final_state,
                        const gdn2_fwd_options *opts, hipStream_t stream);

/* Bytes of the fixed device array that gdn2_chunk_fwd_noalloc uses (64 MiB). */
#define GDN2_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * gdn2_chunk_fwd_noalloc -- gdn2_chunk_fwd_opts for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, results and errors as
 * gdn2_chunk_fwd_opts; it calls no hipMalloc, hipMallocAsync, hipFree or
 * other allocating routine.
 *
 * Where the split run needs a workspace (N * HV * nseg * (2 K V + K K) * 4
 * bytes, see gdn2_chunk_fwd_opts), it is taken from a static device array of
 * GDN2_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends. Nothing in it needs clearing: every byte a call reads
 * was written earlier in the same call. With seq_split_chunks = 0 the
 * automatic plan lengthens its segments until the workspace fits (whole
 * sequences if none does); an explicit seq_split_chunks whose workspace
 * exceeds the array is rejected with GDN2_ERR_UNSUPPORTED and a message
 * naming both sizes. Device ordinals 0..63.
 *
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (e.g. on two streams without ordering between them) race on it
 * and give undefined results. Calls ordered on one stream are safe.
 */
int gdn2_chunk_fwd_noalloc(const gdn2_tensor *q, const gdn2_tensor *k,
                           const gdn2_tensor *v, const gdn2_tensor *g,
                           const gdn2_tensor *beta, const gdn2_tensor *w,
                           float scale, const gdn2_tensor *initial_state,
                           const gdn2_tensor *cu_seqlens,
                           const gdn2_tensor *out,
                           const gdn2_tensor *final_state,
                           const gdn2_fwd_options *opts, hipStream_t stream);

/*
 * gdn2_recurrent_fwd -- the same operation evaluated token by token: for
 * decode (one new token per sequence) and short spans (a few tokens per
 * sequence, e.g. speculative or chunk-remainder steps), where the WY chunk
 * machinery would waste most of a 64-token chunk. Same tensors, dtypes,
 * defaults, varlen packing and errors as gdn2_chunk_fwd, with one
 * difference: final_state may be the very buffer of initial_state (same
 * data pointer and element type) to update the state in place; any other
 * overlap is GDN2_ERR_ALIAS. The arithmetic is the recurrence step by step
 * in float32 (state, gates, products); only the output (and a bf16 final
 * state) is rounded.
 *
 * Cost: every (sequence, value head) state is read and written once per
 * call (2 * K * V * 4 bytes), plus the tokens' vectors; one workgroup per
 * (sequence, value head, 32 value columns) walks the span in order, so long
 * sequences belong on gdn2_chunk_fwd. Allocates nothing.
 */
int gdn2_recurrent_fwd(const gdn2_tensor *q, const gdn2_tensor *k,
                       const gdn2_tensor *v, const gdn2_tensor *g,
                       const gdn2_tensor *beta, const gdn2_tensor *w,
                       float scale, const gdn2_tensor *initial_state,
                       const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                       const gdn2_tensor *final_state, hipStream_t stream);

/*
 * gdn2_recurrent_fwd_opts -- gdn2_recurrent_fwd with options (NULL opts =
 * defaults): state_layout and qk_l2norm as for gdn2_chunk_fwd_opts;
 * seq_split_chunks is ignored. Errors as gdn2_chunk_fwd_opts.
 */
int gdn2_recurrent_fwd_opts(const gdn2_tensor *q, const gdn2_tensor *k,
                            const gdn2_tensor *v, const gdn2_tensor *g,
                            const gdn2_tensor *beta, const gdn2_tensor *w,
                            float scale, const gdn2_tensor *initial_state,
                            const gdn2_tensor *cu_seqlens,
                            const gdn2_tensor *out,
                            const gdn2_tensor *final_state,
                            const gdn2_fwd_options *opts, hipStream_t stream);

/* The host-side validation of gdn2_recurrent_fwd alone (no device work). */
int gdn2_recurrent_fwd_check(const gdn2_tensor *q, const gdn2_tensor *k,
                             const gdn2_tensor *v, const gdn2_tensor *g,
                             const gdn2_tensor *beta, const gdn2_tensor *w,
                             float scale, const gdn2_tensor *initial_state,
                             const gdn2_tensor *cu_seqlens,
                             const gdn2_tensor *out,
                             const gdn2_tensor *final_state);

/*
 * gdn2_split_plan -- the automatic choice of seq_split_chunks for T packed
 * tokens in N sequences with HV value heads on a device with num_cu compute
 * units: 0 (run whole sequences) or the segment length in chunks. Pure host
 * arithmetic (assumes equal sequence lengths); needs no GPU.
 */
int gdn2_split_plan(int64_t T, int32_t N, int32_t HV, int32_t num_cu);

/*
 * gdn2_chunk_fwd_check -- the host-side argument validation of
 * gdn2_chunk_fwd alone: same arguments (no stream), same return codes, same
 * gdn2_last_error() message. Touches no device memory and makes no HIP call,
 * so it can run on a machine without a GPU.
 */
int gdn2_chunk_fwd_check(const gdn2_tensor *q, const gdn2_tensor *k,
                         const gdn2_tensor *v, const gdn2_tensor *g,
                         const gdn2_tensor *beta, const gdn2_tensor *w,
                         float scale, const gdn2_tensor *initial_state,
                         const gdn2_tensor *cu_seqlens, const gdn2_tensor *out,
                         const gdn2_tensor *final_state);

/*
 * gdn2_chunk_bwd -- enqueue the backward of gdn2_chunk_fwd on `stream`: the
 * gradients of a scalar loss with respect to q, k, v, g, beta, w and the
 * initial state, given its gradients d_out with respect to the output and
 * d_final_state with respect to the final state. It differentiates the same
 * recurrence (FlashInfer chunk_gated_delta_rule2 docs, recurrence display
 * equation) through the same 64-token chunked WY form, so a training step
 * can pair the two calls.
 *
 * Tensors (every one dense, row-major; shapes and roles as in
 * gdn2_chunk_fwd):
 *   q, k [T, H, K], v, w [T, HV, V], beta [T, HV, K]      bf16 or float16, one type (required)
 *   g [T, HV, K]                                           float32, bf16 or float16 (required)
 *   initial_state [N, HV, K, V]                            float32, K-major, or NULL (zero)
 *   cu_seqlens [N + 1]                                     int32 or int64, or NULL (one sequence)
 *   d_out [T, HV, V]                                       q's type (required)
 *   d_final_state [N, HV, K, V]                            float32, or NULL (zero)
 * Outputs (caller-allocated, fully written):
 *   dq, dk [T, H, K]                                       q's type: sums over the value heads that
 *                                                          read each q/k head
 *   dv, dw [T, HV, V], dbeta [T, HV, K]                    q's type
 *   dg [T, HV, K]                                          g's type (gradient of the natural-log g)
 *   d_initial_state [N, HV, K, V]                          float32, or NULL (not written)
 * scale == 0 means 1/sqrt(K). Supported sizes: (K, V) = (64, 64) or
 * (128, 128) (GDN2_ERR_UNSUPPORTED otherwise; the forward also takes K != V).
 *
 * Strong decay: any g <= 0 is supported. A key channel whose running
 * in-chunk sum of g leaves about -83 (120 ln 2) within a chunk cannot use
 * the chunk-start factors e^G and e^-G (the second overflows); such a
 * channel's share of the intra-chunk products is differentiated exactly,
 * per pair of rows with e^(G_r - G_s) <= 1 (burn-gdn2 README, numerical
 * stability), at some extra cost for the chunks that have one.
 *
 * Evaluation: the forward runs again and keeps the state entering every
 * chunk (rounded to bf16) and each chunk's WY quantities (its record); one workgroup
 * per (sequence, value head) carries the state gradient over the chunks in
 * reverse; a chunk-parallel pass forms every gradient; a last pass sums dq
 * and dk over grouped value heads (HV > H). Arithmetic is float32 with bf16
 * MFMA operands, as in the forward.
 *
 * Streams: when every (sequence, value head) chain of the call can be
 * resident at once (more than half of the device's compute units and at
 * most all of them, whole sequences), the longer half of the sequences
 * (by chunk count, ranked on the device) runs its passes on `stream` and
 * the shorter half on a second stream. The library creates that stream
 * per device on first use, at the default priority, and keeps it until
 * the process ends. The work is forked from `stream` and joined back to it
 * with events, so the call is ordered on `stream` like any other. The
 * second stream is never created while `stream` is being captured into a
 * graph (such a call runs on `stream` alone); graph capture of the
 * backward is otherwise untested. Results are bit-identical either way.
 *
 * Ownership and memory: the caller owns every buffer; inputs are only read.
 * A stream-ordered workspace (from the library's pool, see gdn2_chunk_fwd;
 * released with hipFreeAsync on `stream`) of
 *   (T / 64 + N) * HV * (2 * K * V * 2 + 516 * K + 16384) bytes,
 *   plus 2 * T * HV * K * 4 bytes when HV > H (per-value-head dq and dk),
 *   plus N * 4 bytes when the call runs as two groups (each sequence's group)
 * (rounded up per part) holds the checkpoints, the records and partial
 * gradients; if it cannot be allocated the call fails with GDN2_ERR_HIP and
 * enqueues nothing.
 *
 * Errors as gdn2_chunk_fwd: NULL_ARG for a missing required tensor, DTYPE,
 * SHAPE, HEADS, UNSUPPORTED, LAYOUT for a non-dense tensor, ALIAS when an
 * output overlaps an input or another output. Asynchronous, deterministic
 * (no atomics), reentrant.
 */
int gdn2_chunk_bwd(const gdn2_tensor *q, const gdn2_tensor *k,
                   const gdn2_tensor *v, const gdn2_tensor *g,
                   const gdn2_tensor *beta, const gdn2_tensor *w, float scale,
                   const gdn2_tensor *initial_state,
                   const gdn2_tensor *cu_seqlens, const gdn2_tensor *d_out,
                   const gdn2_tensor *d_final_state, const gdn2_tensor *dq,
                   const gdn2_tensor *dk, const gdn2_tensor *dv,
                   const gdn2_tensor *dg, const gdn2_tensor *dbeta,
                   const gdn2_tensor *dw, const gdn2_tensor *d_initial_state,
                   hipStream_t stream);

/* The host-side validation of gdn2_chunk_bwd alone (no device work). */
int gdn2_chunk_bwd_check(const gdn2_tensor *q, const gdn2_tensor *k,
                         const gdn2_tensor *v, const gdn2_tensor *g,
                         const gdn2_tensor *beta, const gdn2_tensor *w,
                         float scale, const gdn2_tensor *initial_state,
                         const gdn2_tensor *cu_seqlens,
                         const gdn2_tensor *d_out,
                         const gdn2_tensor *d_final_state,
                         const gdn2_tensor *dq, const gdn2_tensor *dk,
                         const gdn2_tensor *dv, const gdn2_tensor *dg,
                         const gdn2_tensor *dbeta, const gdn2_tensor *dw,
                         const gdn2_tensor *d_initial_state);

/* Message describing the last failure on the calling thread ("" if none).
 * The string stays valid until the next call on the same thread. */
const char *gdn2_last_error(void);

/* GDN2_ABI_VERSION of the built library. */
int gdn2_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN2_H */
