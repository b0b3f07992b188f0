/*
 * ssd.h -- C ABI of the MI355X (gfx950) Mamba-2 chunked SSD forward pass.
 *
 * The method (page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in
 * NVIDIA CUDA Tile", section "Mamba-2 architecture"): for each batch b and head h,
 *     h_t = exp(A[h] * dt[b,t,h]) * h_{t-1} + dt[b,t,h] * B[b,t,g] x[b,t,h]^T
 *     y[b,t,h] = C[b,t,g]^T h_t + D[h] * x[b,t,h]          (g = h / (nheads/ngroups))
 * evaluated chunk by chunk in three stages: a per-chunk cumulative decay in log2 space
 * (section "Kernel 1: Computing cumulative sums"), chunk-initial states by the jump
 * formula carried across chunks (section "Kernel 2: fwd_pass_state"), and a fused
 * per-chunk output (section "Kernel 3: compute_out").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are dense, row-major (last index fastest), in device memory, and every
 *    pointer must be 16-byte aligned. Layouts:
 *        x        [batch, seqlen, nheads, headdim]        in_dtype
 *        dt       [batch, seqlen, nheads]                 in_dtype
 *        B, C     [batch, seqlen, ngroups, dstate]        in_dtype
 *        A, D     [nheads]                                fp32
 *        h0,final [batch, nheads, headdim, dstate]        fp32 (state stored P x S)
 *        G, dt_t  [batch, nheads, seqlen]                 fp32 (head-major, tokens fastest)
 *        states   [batch, nheads, nchunks, headdim, dstate]   states_dtype
 *        y        [batch, seqlen, nheads, headdim]        out_dtype (fp32 by default)
 *    with nchunks = ceil(seqlen / chunk).
 *  - Lengths: any seqlen >= 0. A last chunk shorter than `chunk` is processed as if it
 *    were padded with zero tokens (dt = 0, x = B = C = 0), which is the page's own padding
 *    (section "Kernel 1: Computing cumulative sums") and leaves the result of every real
 *    token unchanged; only the real tokens' outputs are written. seqlen = 0 is an empty
 *    sequence: nothing is read or written except final_state, which receives h0 (zeros
 *    when h0 is NULL); the tensors with a seqlen extent (and a zero-byte workspace) may
 *    then be NULL.
 *  - Ownership: the caller allocates and frees every buffer, including the workspace.
 *    The library never allocates device memory, keeps no pointer after returning and
 *    holds no global state, so concurrent calls on different buffers are safe. (The one
 *    exception is ssd_forward_noalloc below, which works in a scratch array of its own.)
 *  - Execution: kernels are enqueued on `stream` (a hipStream_t; NULL means the null
 *    stream) and the call returns without synchronising. Outputs are valid once the
 *    caller synchronises that stream. Inputs must not alias outputs.
 *  - Errors: every argument is validated on the host before anything is enqueued; an
 *    invalid call returns a non-zero ssd_status and touches no memory. A failed launch
 *    returns SSD_ERR_HIP. No call aborts the process or throws.
 *  - Supported sizes: chunk in {64, 128, 256}; headdim in {16, 32, 64, 128};
 *    dstate in {16, 32, 64, 128, 256}; nheads a multiple of ngroups; in_dtype and states_dtype in {SSD_F32, SSD_BF16},
 *    except fp32 inputs with bf16 states (SSD_ERR_UNSUPPORTED: it would only lose the
 *    precision the fp32 inputs ask for). Size limits (SSD_ERR_UNSUPPORTED beyond them):
 *    at most 2e9 elements in x and in the chunk states, and below 2 GiB for one chunk's
 *    rows of x or B (chunk * max(nheads*headdim, ngroups*dstate) * 4 bytes) and for one
 *    batch row's decays (nheads * seqlen * 4 bytes).
 */
#ifndef SSD_MI355X_H
#define SSD_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL = 1,        /* a required pointer is NULL */
    SSD_ERR_SHAPE = 2,       /* a size < 1 (seqlen < 0), or nheads % ngroups != 0 */
    SSD_ERR_DTYPE = 3,       /* a dtype code that is neither SSD_F32 nor SSD_BF16 */
    SSD_ERR_UNSUPPORTED = 4, /* chunk, headdim, dstate, dtype pair or size outside the supported sets */
    SSD_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than the size query returns */
    SSD_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
    SSD_ERR_HIP = 7,         /* the HIP runtime reported an error for a launch */
    SSD_ERR_TOO_LARGE = 8    /* ssd_forward_noalloc: the problem needs more scratch than it holds */
} ssd_status;

typedef enum ssd_dtype { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Problem sizes. The names follow the page's kernels: headdim is the per-head size of
 * x (the page's "head size"), dstate the state size, chunk the chunk length. */
typedef struct ssd_shape {
    int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    int32_t in_dtype;     /* dtype of x, dt, B, C */
    int32_t states_dtype; /* dtype of the chunk-initial states (ssd_state_pass output,
                             ssd_chunk_out input, and the forward pass's internal copy) */
    int32_t out_dtype;    /* dtype of y: SSD_F32 (the default to use), or SSD_BF16 for
                             bf16 inputs and bf16 states only. bf16 y is a throughput
                             option: rounding y alone costs ~3e-2 of max|y| / rms(y) */
    int32_t reserved;     /* set to 0 */
} ssd_shape;

/* Human-readable name of a status code (static storage; never NULL). */
const char* ssd_status_string(int status);

/* Host-only check of a shape against the supported sets; enqueues nothing. */
ssd_status ssd_validate_shape(const ssd_shape* shape);

/* Workspace sizes in bytes for ssd_forward and ssd_state_pass (the segmented pair's below).
 * Host-only. */
ssd_status ssd_forward_workspace_bytes(const ssd_shape* shape, size_t* bytes);
ssd_status ssd_state_pass_workspace_bytes(const ssd_shape* shape, size_t* bytes);

/*
 * The plan of the output kernel that ssd_forward launches for a shape (host-only): heads
 * per workgroup, whether the interaction tiles C B^T are built once per workgroup and
 * shared by its heads (1) or rebuilt per head (0), and the matrix-core flops one launch
 * executes (every 16x16 product tile counted at its padded K, the shared tiles once per
 * workgroup). Any output may be NULL. SSD_ERR_UNSUPPORTED for seqlen 0.
 */
ssd_status ssd_chunk_out_plan(const ssd_shape* shape, int32_t* heads_per_workgroup,
                              int32_t* shared_tiles, double* mfma_flops);

/*
 * Stage 1 -- per-chunk cumulative decay (section "Kernel 1: Computing cumulative sums").
 * For token t of chunk c = t / chunk:
 *     G[b,h,t]    = log2(e) * sum_{k = c*chunk .. t} A[h] * dt[b,k,h]   (inclusive, fp32)
 *     dt_t[b,h,t] = dt[b,t,h] widened to fp32
 * Both outputs use the head-major [batch, nheads, seqlen] layout that the page moves
 * decay and dt to for contiguous access (section "Mamba-2 performance optimization",
 * GMEM layout). dt_t may be NULL when only G is wanted.
 */
ssd_status ssd_chunk_cumsum(const ssd_shape* shape, const void* dt, const float* A, float* G,
                            float* dt_t, void* stream);

/*
 * Stage 2 -- chunk-initial states by the jump formula (section "Kernel 2: fwd_pass_state").
 * The state entering chunk c+1 is
 *     S_{c+1} = 2^{G_last} S_c + sum_{j in chunk c} dt_j 2^{G_last - G_j} x_j^T (outer) B_j
 * (stored P x S), starting from S_0 = h0 (zeros when h0 is NULL); G_last is G at the
 * chunk's last (real) token, and the exponent G_last - G_j = log2(e) * sum_{k=j+1}^{last} A dt_k
 * is summed from the chunk's end (hence A is an input), which keeps its rounding error
 * relative to the exponents that dominate the state.
 * Outputs: states[b,h,c] = S_c for every chunk c (states_dtype), and, when final_state
 * is not NULL, final_state[b,h] = S_nchunks in fp32.
 * Inputs: x, B in in_dtype; A fp32 [nheads]; G and dt_t as produced by ssd_chunk_cumsum;
 * h0 fp32. The workspace must hold ssd_state_pass_workspace_bytes bytes.
 * How: where the shape has a segment plan (bf16 inputs and states; see
 * ssd_state_pass_segmented) the chunks are walked by segments with the running states on
 * chip, the states entering the segments are carried, and each recorded state is then
 * completed in place to the true S_c, with the arithmetic ssd_chunk_out_segmented uses for
 * the same sum, so ssd_chunk_cumsum -> ssd_state_pass -> ssd_chunk_out returns the bits
 * ssd_forward returns; otherwise per-chunk increments on the matrix cores and a
 * sequential carry.
 */
ssd_status ssd_state_pass(const ssd_shape* shape, const void* x, const float* A, const void* B,
                          const float* G, const float* dt_t, const float* h0, void* states,
                          float* final_state, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Stage 2 in one kernel, as the page's state kernel does it (section "Kernel 2:
 * fwd_pass_state"): the same outputs as ssd_state_pass (states for every chunk, and the
 * final state when final_state is not NULL) from one sequential pass over the chunks per
 * (batch, head, slice of headdim rows), the running state held on chip; no workspace, and
 * G is not needed (the exponents come from A and dt_t). Built for bf16 inputs, headdim 64
 * or 128, dstate 64, 128 or 256, and seqlen a positive multiple of chunk; other shapes
 * return SSD_ERR_UNSUPPORTED. The fused state operand dt_j 2^{G_last - G_j} x_j enters the
 * matrix cores as a bf16 high/low pair, as in ssd_state_pass. ssd_forward takes this kernel
 * instead of the two-kernel pass for the shapes where it measured faster and the segmented
 * pass below has no plan.
 */
ssd_status ssd_state_scan(const ssd_shape* shape, const void* x, const float* A, const void* B,
                          const float* dt_t, const float* h0, void* states, float* final_state,
                          void* stream);

/*
 * Stage 3 -- fused chunk output (section "Kernel 3: compute_out"). For chunk c, rows i
 * and columns j the chunk's tokens:
 *     y_i = 2^{G_i} C_i^T S_c + sum_{j <= i} 2^{G_i - G_j} (C_i . B_j) dt_j x_j + D[h] x_i
 * The causal mask keeps the diagonal (y_t reads the state after token t). The
 * interaction matrix C B^T never leaves the chip; decays of masked pairs are selected
 * away, never multiplied, so their overflow cannot reach y. y is written in out_dtype.
 * D may be NULL (no skip term).
 */
ssd_status ssd_chunk_out(const ssd_shape* shape, const void* x, const void* B, const void* C,
                         const float* G, const float* dt_t, const void* states, const float* D,
                         void* y, void* stream);

/*
 * Stage 2 by segments, and stage 3 over its output (the linearity of the recurrence of
 * section "Mamba-2 architecture" applied to the state kernel of section "Kernel 2:
 * fwd_pass_state"); the pair ssd_forward runs whenever the shape has a segment plan.
 * The chunks are cut into segments of K consecutive chunks (K and the heads per workgroup
 * are the library's choice for the shape, see ssd_segment_plan). Each segment is walked
 * from a zero state (segment 0 from h0), so what ssd_state_pass_segmented records in
 * seg_relative_states[b,h,c] is NOT the state entering chunk c but that state minus the
 * part carried in from before the chunk's segment; the true state is
 *     S_c = seg_relative_states[b,h,c] + 2^{D_c} S_in(k),   k = c / K,
 *     D_c = sum of G_last over the segment's chunks before c,
 * with S_in(k) the state entering segment k (S_in(0) adds nothing). G and dt_t are
 * ssd_chunk_cumsum's. ssd_state_pass_segmented writes S_in(k) (bf16) and D_c to the
 * workspace, and the final state (fp32) to final_state when it is not NULL; the per-chunk
 * state increments never go to HBM. ssd_chunk_out_segmented then computes y exactly as
 * ssd_chunk_out does from the true states, forming each chunk's S_c (fp32 sum, one bf16
 * rounding) while it stages it; it reads S_in and D_c from the same workspace, which must
 * be passed unchanged between the two calls on the same stream.
 * Built for bf16 inputs with bf16 states (states_dtype SSD_BF16), headdim 64, dstate 64,
 * 128 or 256; other shapes return SSD_ERR_UNSUPPORTED (as do the queries). The workspace
 * must hold ssd_state_pass_segmented_workspace_bytes bytes.
 */
ssd_status ssd_state_pass_segmented_workspace_bytes(const ssd_shape* shape, size_t* bytes);
/* The segment plan the library takes for a shape (host-only): heads per workgroup,
 * chunks per segment K and the number of segments. SSD_ERR_UNSUPPORTED where the shape
 * has no plan (or seqlen is 0). Any of the outputs may be NULL. */
ssd_status ssd_segment_plan(const ssd_shape* shape, int32_t* heads_per_workgroup,
                            int32_t* chunks_per_segment, int32_t* segments);
ssd_status ssd_state_pass_segmented(const ssd_shape* shape, const void* x, const float* A,
                                    const void* B, const float* G, const float* dt_t,
                                    const float* h0, void* seg_relative_states,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    void* stream);
ssd_status ssd_chunk_out_segmented(const ssd_shape* shape, const void* x, const void* B,
                                   const void* C, const float* G, const float* dt_t,
                                   const float* D, const void* seg_relative_states, void* y,
                                   const void* workspace, size_t workspace_bytes, void* stream);

/*
 * The whole forward pass: stage 1, stage 2, stage 3 on one stream. Returns y (out_dtype) and,
 * when final_state is not NULL, the state after the last token (fp32), which may be fed
 * back as the next call's h0 (section "Kernel 2: fwd_pass_state", after the chunk loop).
 * h0 and D may be NULL. The workspace must hold ssd_forward_workspace_bytes bytes.
 */
ssd_status ssd_forward(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* h0, void* y,
                       float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * The whole forward pass without any allocation, for callers that cannot allocate device
 * memory or be handed a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, results and execution as ssd_forward
 * (bitwise: it runs the same kernels), minus the workspace: the intermediates (cumulative
 * decays, state-pass buffers, chunk states) live in a device array of
 * SSD_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs this call on,
 * until the process ends. A problem whose ssd_forward_workspace_bytes exceeds that size
 * returns SSD_ERR_TOO_LARGE before anything is enqueued (256 MiB covers, for example,
 * batch 2 x 16384 tokens x 80 heads at headdim 64, dstate 128, chunk 256).
 * The first call on a device resolves that device's array (hipGetSymbolAddress, which may
 * load the library's code object there); make one call before capturing a graph. Every
 * call on one GPU uses the same array, whose contents persist between calls: calls that
 * overlap on one GPU (on different streams, or from several threads) race and must be
 * serialised by the caller. Nothing in the array needs to start at zero.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
ssd_status ssd_forward_noalloc(const ssd_shape* shape, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* h0, void* y, float* final_state, void* stream);

/*
 * Recurrent decode step (section "Mamba-2 architecture": the recurrent form, which takes
 * one token at a time with a state of fixed size, the form the page names for sequential
 * inference). For each batch b and head h (g = h / (nheads/ngroups)), on the fp32 state
 * that ssd_forward returns as its final state:
 *     state[b,h] <- exp(A[h] dt[b,h]) state[b,h] + dt[b,h] x[b,h]^T (outer) B[b,g]
 *     y[b,h]      = state[b,h] . C[b,g] + D[h] x[b,h]      (reads the updated state)
 * so a prompt prefilled by ssd_forward (final_state) continues here token by token, and
 * a sequence split at any token gives the same result as one pass.
 * Shape: seqlen must be 1 (else SSD_ERR_SHAPE); chunk, states_dtype and out_dtype are not
 * used (the state and y are fp32).
 * Layouts (the [batch, 1, ...] slices of the forward pass's layouts):
 *     x        [batch, nheads, headdim]          in_dtype
 *     dt       [batch, nheads]                   in_dtype
 *     B, C     [batch, ngroups, dstate]          in_dtype
 *     A, D     [nheads]                          fp32 (D may be NULL)
 *     state    [batch, nheads, headdim, dstate]  fp32, read and updated in place
 *     y        [batch, nheads, headdim]          fp32
 * state must not alias any other argument. Errors and execution as for the other entry
 * points (validation before any launch; asynchronous on `stream`).
 */
ssd_status ssd_decode_step(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, float* state, float* y,
                           void* stream);

/*
 * Backward pass: the gradients of sum(dy * y) + sum(dfinal * final_state) with respect to
 * every input of ssd_forward, i.e. reverse-mode differentiation of the recurrence of
 * section "Mamba-2 architecture" (the page publishes no backward; this is the chain rule
 * applied to its forward definition). With Lam_t = dL/dH_t:
 *     Lam_t = dy_t (outer) C_t + exp(A dt_{t+1}) Lam_{t+1}
 *     dx_t = D dy_t + dt_t Lam_t B_t,  dB_t = dt_t Lam_t^T x_t (summed over the group's
 *     heads),  dC_t = H_t^T dy_t (summed likewise),  dD = sum dy . x,  dh0 = dL/dH_{-1},
 *     ddt_t = x_t . Lam_t B_t + A dL/da_t,  dA = sum_t dt_t dL/da_t  (a_t = A dt_t).
 * The forward quantities it needs (cumulative decay, chunk-initial states, final state)
 * are recomputed here, chunk by chunk; states_dtype and out_dtype are not used. Precision:
 * fp32 accumulation throughout. With bf16 inputs (and headdim 64/128, dstate 64/128/256)
 * the per-chunk products run on the matrix cores with every fp32 operand (dy, the decayed
 * interaction weights, the states) entered as a bf16 high/low pair (about 16 significant
 * bits), at a chunk length of the library's choosing (128 or 64 tokens, where the fp32
 * chunk states at that length stay within the size limits; the chunked form is exact for
 * any length, so shape->chunk only sizes the fp32 path); otherwise fp32 VALU arithmetic at
 * shape->chunk. ssd_backward_workspace_bytes accounts for both. dL/da_t is summed over the
 * later tokens of its chunk only, starting from the value at the chunk's end, the inner
 * product of the gradient arriving there with the state there; so its rounding error stays
 * that of one chunk at any seqlen.
 * Inputs: x, dt, B, C in in_dtype and A, D, h0 as for ssd_forward (D and h0 may be NULL);
 * dy [batch, seqlen, nheads, headdim] fp32; dfinal [batch, nheads, headdim, dstate] fp32
 * or NULL (zero). Outputs, all fp32, written in full: dx (x's layout), ddt (dt's layout),
 * dA [nheads], dB and dC (B's layout), dD [nheads] (may be NULL), dh0 (h0's layout, may be
 * NULL). The workspace must hold ssd_backward_workspace_bytes bytes. seqlen = 0: dh0 =
 * dfinal (zeros without), dA = dD = 0, and the seqlen-sized tensors may be NULL.
 */
ssd_status ssd_backward_workspace_bytes(const ssd_shape* shape, size_t* bytes);
ssd_status ssd_backward(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                        const void* B, const void* C, const float* D, const float* h0,
                        const float* dy, const float* dfinal, float* dx, float* ddt, float* dA,
                        float* dB, float* dC, float* dD, float* dh0, void* workspace,
                        size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_MI355X_H */
