// Internal launch interface between the C ABI (ssd_api.cpp) and the kernels.
// Sizes are already validated by the caller; these functions only pick the template
// instance, size the grid and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

enum { kF32 = 0, kBF16 = 1 };

struct Dims {
    int batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
    // chunks of the sequence; the last one holds seqlen - (nchunks - 1) * chunk tokens
    int nchunks() const { return (seqlen + chunk - 1) / chunk; }
};

hipError_t launch_cumsum(int in_dtype, const void* dt, const float* A, float* G, float* dt_t,
                         const Dims& d, hipStream_t stream);

hipError_t launch_chunk_state(int in_dtype, const void* x, const void* Bm, const float* A,
                              const float* dt_t, float* dstate_chunks, const Dims& d,
                              hipStream_t stream);

hipError_t launch_state_carry(int states_dtype, const float* dstate_chunks, const float* G,
                              const float* h0, void* states, float* final_state, const Dims& d,
                              hipStream_t stream);

// Single-pass state kernel, the alternative to chunk_state + state_carry: one workgroup
// per (batch, head, slice of headdim rows) walks the whole sequence with the running state
// in registers. Built for bf16 inputs, headdim 64 or 128, dstate 64, 128 or 256, and a
// sequence of whole chunks (seqlen a positive multiple of the chunk length).
bool state_scan_supported(int in_dtype, const Dims& d);
// Whether the forward pass takes the single-pass kernel for this shape (measured faster).
bool state_scan_preferred(int in_dtype, const Dims& d);
hipError_t launch_state_scan(int states_dtype, const void* x, const void* Bm, const float* A,
                             const float* dt_t, const float* h0, void* states,
                             float* final_state, const Dims& d, hipStream_t stream);

// Segmented state pass (bf16 inputs, bf16 chunk states): workgroups walk runs of
// `chunks` consecutive chunks for blocks of `heads` heads from a zero state (segment 0 from
// h0), recording each chunk's state relative to its segment's start; a small sequential
// kernel carries the states entering each segment and gives the final state. The output
// kernel then adds 2^{dec_in} * seg_in to each recorded state (segments >= 1).
struct SegPlan {
    int heads, chunks, nseg;
};
// Below this log2 decay from a segment's start the factor 2^{D_c} is exactly 0 in fp32
// (even as a denormal), so adding the decayed entering state changes nothing and the
// kernels that form S_c = L_c + 2^{D_c} S_in skip it (and do not read S_in).
constexpr float kSegCut = -160.f;
struct SegBuffers {
    float* seg_end;   // [B, H, nseg, P, S] each segment's end state from its own start
    void* seg_in;     // [B, H, nseg, P, S] bf16 state entering each segment (>= 1)
    float* dec_in;    // [B, H, nC] log2 decay from the segment's start to each chunk's start
    float* dec_seg;   // [B, H, nseg] each segment's total log2 decay
};
bool state_seg_plan(int in_dtype, int states_dtype, const Dims& d, SegPlan* plan);
size_t state_seg_ws_bytes(const Dims& d, const SegPlan& plan);
SegBuffers state_seg_buffers(void* workspace, const Dims& d, const SegPlan& plan);
hipError_t launch_state_seg(const void* x, const void* Bm, const float* A, const float* G,
                            const float* dt_t, const float* h0, void* states,
                            float* final_state, const SegPlan& plan, const SegBuffers& sb,
                            const Dims& d, hipStream_t stream);
// Segment-relative chunk states -> true chunk-initial states, in place (after the carry),
// with the arithmetic of launch_chunk_out_seg's completion (the same bits).
hipError_t launch_seg_correct(void* states, const SegPlan& plan, const SegBuffers& sb,
                              const Dims& d, hipStream_t stream);

// final_state = h0 (zeros when h0 is NULL): the state after an empty sequence.
hipError_t launch_state_init(const float* h0, float* final_state, const Dims& d,
                             hipStream_t stream);

// One recurrent step on a carried fp32 state (in place), y for that token.
hipError_t launch_decode(int in_dtype, const void* x, const void* dt, const float* A,
                         const void* Bm, const void* Cm, const float* D, float* state, float* y,
                         const Dims& d, hipStream_t stream);

// Backward pass: every buffer below is the caller's (the workspace carved up on the host).
struct BwdWorkspace {
    float *G, *dt_t;      // [B, H, L] cumulative decay and dt (fp32)
    float *Hc, *R;        // [B, H, nC, P, S] chunk-initial states; increments, then the
                          // gradient arriving at each chunk's end
    float* fin;           // [B, H, P, S] forward final state
    float *v, *q, *dyx;   // [B, H, L] per-token scalars
    float *dA_bh, *dD_bh; // [B, H]
    float *dBh, *dCh;     // [B, L, H, S] per-head dB, dC (when heads share a group)
    float* anc;           // [B, H, nC, P*S/256] partial sums of <R_c, state after chunk c>
};
struct BwdLaunch {
    const void *x, *dt, *B, *C;
    const float *A, *D, *h0, *dy, *dfinal;
    float *dx, *ddt, *dA, *dB, *dC, *dD, *dh0;
    BwdWorkspace ws;
};
hipError_t launch_backward(int in_dtype, const BwdLaunch& k, const Dims& d, hipStream_t stream);
// Chunk length at which the backward pass runs its matrix-core kernels for this shape (0:
// none; the token walks then run at the caller's chunk length).
int bwd_mfma_chunk(int in_dtype, int P, int S);
// Partial dB, dC rows the backward pass writes per (token, group) before summing them (1:
// it writes dB and dC directly); d.chunk is the backward's chunk length.
int bwd_partials_per_group(int in_dtype, const Dims& d);

// chunk_out's launch plan for a shape: heads per workgroup, shared interaction tiles, the
// matrix-core flops the launch executes and its LDS bytes per workgroup (host-only; SEGC:
// the instance over segment-relative states). False where no instance exists.
struct OutPlan {
    int heads_per_wg;
    bool shared;
    double mfma_flops, lds_bytes;
};
bool chunk_out_plan(int in_dtype, int states_dtype, bool segc, const Dims& d, OutPlan* plan);
hipError_t launch_chunk_out(int in_dtype, int states_dtype, int out_dtype, const void* x,
                            const void* Bm, const void* Cm, const float* G, const float* dt_t,
                            const void* states, const float* D, void* y, const Dims& d,
                            hipStream_t stream);

// The output kernel over segment-relative chunk states (bf16 inputs and states): each
// chunk's state is taken as states[c] + 2^{dec_in[c]} seg_in[c / seg_chunks] for chunks
// past the first segment.
hipError_t launch_chunk_out_seg(int out_dtype, const void* x, const void* Bm, const void* Cm,
                                const float* G, const float* dt_t, const void* states,
                                const void* seg_in, const float* dec_in, int seg_chunks,
                                const float* D, void* y, const Dims& d, hipStream_t stream);

}  // namespace ssd
