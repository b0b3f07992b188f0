// C ABI of the SSD forward pass (declared in include/ssd.h).
//
// Host-side only: argument validation (before anything is enqueued), workspace layout
// and the launch order of the stages on the caller's stream. No device memory is
// allocated here and no synchronisation happens.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "../../include/ssd.h"
#include "ssd_launch.h"

using ssd::Dims;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool one_of(int64_t v, std::initializer_list<int64_t> set) {
    for (int64_t s : set)
        if (v == s) return true;
    return false;
}

size_t esize(int32_t dt) { return dt == SSD_BF16 ? 2 : 4; }

// Chunks of the sequence (the last may be partial; none for an empty sequence).
int64_t nchunks_of(const ssd_shape* s) { return (s->seqlen + s->chunk - 1) / s->chunk; }

ssd_status check_shape(const ssd_shape* s) {
    if (!s) return SSD_ERR_NULL;
    if (s->batch < 1 || s->seqlen < 0 || s->nheads < 1 || s->headdim < 1 || s->dstate < 1 ||
        s->ngroups < 1 || s->chunk < 1)
        return SSD_ERR_SHAPE;
    if (s->nheads % s->ngroups != 0) return SSD_ERR_SHAPE;
    if ((s->in_dtype != SSD_F32 && s->in_dtype != SSD_BF16) ||
        (s->states_dtype != SSD_F32 && s->states_dtype != SSD_BF16) ||
        (s->out_dtype != SSD_F32 && s->out_dtype != SSD_BF16))
        return SSD_ERR_DTYPE;
    if (s->in_dtype == SSD_F32 && s->states_dtype == SSD_BF16) return SSD_ERR_UNSUPPORTED;
    // bf16 y is built for the all-bf16 path only
    if (s->out_dtype == SSD_BF16 && (s->in_dtype != SSD_BF16 || s->states_dtype != SSD_BF16))
        return SSD_ERR_UNSUPPORTED;
    if (!one_of(s->chunk, {64, 128, 256}) || !one_of(s->headdim, {16, 32, 64, 128}) ||
        !one_of(s->dstate, {16, 32, 64, 128, 256}))
        return SSD_ERR_UNSUPPORTED;
    // Element counts handed to a kernel must fit the 31-bit index arithmetic, and the
    // extents the kernels address through buffer descriptors (32-bit byte counts and
    // offsets) must stay below 2 GiB: one chunk's rows of x, y, B, C and their gradients
    // (all heads or groups), and one batch row's decay rows. Each head's chunk state has
    // a descriptor of its own. Larger sizes are rejected rather than overflowed.
    const double states = (double)s->batch * s->nheads * nchunks_of(s) * s->headdim * s->dstate;
    const double xs = (double)s->batch * s->seqlen * s->nheads * s->headdim;
    const double row = (double)std::max(s->nheads * s->headdim, s->ngroups * s->dstate);
    const double chunk_rows = (double)s->chunk * row * 4.0;
    const double per_batch_decay = (double)s->nheads * s->seqlen * 4.0;
    if (states > 2.0e9 || xs > 2.0e9 || chunk_rows >= 2147483648.0 ||
        per_batch_decay >= 2147483648.0)
        return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// Shape check of the decode step: one token, the forward pass's head, group and dtype
// rules; chunk and states_dtype are not used.
ssd_status check_decode_shape(const ssd_shape* s) {
    if (!s) return SSD_ERR_NULL;
    if (s->batch < 1 || s->seqlen != 1 || s->nheads < 1 || s->headdim < 1 || s->dstate < 1 ||
        s->ngroups < 1 || s->nheads % s->ngroups != 0)
        return SSD_ERR_SHAPE;
    if (s->in_dtype != SSD_F32 && s->in_dtype != SSD_BF16) return SSD_ERR_DTYPE;
    if (!one_of(s->headdim, {16, 32, 64, 128}) || !one_of(s->dstate, {16, 32, 64, 128, 256}))
        return SSD_ERR_UNSUPPORTED;
    if ((double)s->batch * s->nheads * s->headdim * s->dstate > 2.0e9) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

Dims dims_of(const ssd_shape* s) {
    Dims d;
    d.batch = (int)s->batch;
    d.seqlen = (int)s->seqlen;
    d.nheads = (int)s->nheads;
    d.headdim = (int)s->headdim;
    d.dstate = (int)s->dstate;
    d.ngroups = (int)s->ngroups;
    d.chunk = (int)s->chunk;
    return d;
}

size_t decay_bytes(const ssd_shape* s) {  // one [batch, nheads, seqlen] fp32 array
    return round_up((size_t)s->batch * s->nheads * s->seqlen * sizeof(float));
}
size_t chunk_states_elems(const ssd_shape* s) {
    return (size_t)s->batch * s->nheads * nchunks_of(s) * s->headdim * s->dstate;
}
size_t pair_ws(const ssd_shape* s) {  // per-chunk state increments, fp32
    return round_up(chunk_states_elems(s) * sizeof(float));
}
// Segment plan of the segmented state pass, when the shape has one.
bool seg_plan_of(const ssd_shape* s, ssd::SegPlan* plan) {
    return s->seqlen > 0 && ssd::state_seg_plan(s->in_dtype, s->states_dtype, dims_of(s), plan);
}
size_t state_seg_ws(const ssd_shape* s) {  // 0 when the shape has no segment plan
    ssd::SegPlan pl;
    return seg_plan_of(s, &pl) ? round_up(ssd::state_seg_ws_bytes(dims_of(s), pl)) : 0;
}
// The state pass's own buffers: the segmented pass's where the shape has a plan, else the
// per-chunk increments.
size_t state_pass_ws(const ssd_shape* s) {
    ssd::SegPlan pl;
    return seg_plan_of(s, &pl) ? state_seg_ws(s) : pair_ws(s);
}
// Forward workspace: G, dt_t, then the state pass's buffers, then the chunk-initial states.
size_t forward_mid_ws(const ssd_shape* s) { return state_pass_ws(s); }
size_t forward_ws(const ssd_shape* s) {
    return 2 * decay_bytes(s) + forward_mid_ws(s) +
           round_up(chunk_states_elems(s) * esize(s->states_dtype));
}

// Backward workspace: the forward quantities it recomputes and its per-token partials.
struct BwdSizes {
    size_t dec, st, fin, tok, bh, part, anc, total;
};
// The shape the backward pass runs at: the caller's, with the chunk length of the
// matrix-core plan when there is one and the recomputed fp32 chunk states at that length
// stay within the size limits (shorter chunks mean more states); otherwise the fp32 token
// walks at the caller's chunk length. The backward keeps fp32 states and y.
ssd_shape bwd_shape(const ssd_shape* s) {
    ssd_shape b = *s;
    b.states_dtype = SSD_F32;
    b.out_dtype = SSD_F32;
    const int t = ssd::bwd_mfma_chunk(s->in_dtype, (int)s->headdim, (int)s->dstate);
    if (t) {
        ssd_shape m = b;
        m.chunk = t;
        if (check_shape(&m) == SSD_OK) b.chunk = t;
    }
    return b;
}

BwdSizes bwd_sizes(const ssd_shape* shape) {
    const ssd_shape bs = bwd_shape(shape);
    const ssd_shape* s = &bs;
    BwdSizes z;
    const size_t BH = (size_t)s->batch * s->nheads;
    z.dec = round_up(BH * s->seqlen * sizeof(float));
    z.st = round_up(chunk_states_elems(s) * sizeof(float));
    z.fin = round_up(BH * s->headdim * s->dstate * sizeof(float));
    z.tok = z.dec;
    z.bh = round_up(BH * sizeof(float));
    // partial dB, dC rows, [B, L, G * parts, S] (none when the kernels write dB, dC directly)
    const int parts = ssd::bwd_partials_per_group(s->in_dtype, dims_of(s));
    z.part = parts > 1 ? round_up((size_t)s->batch * s->seqlen * s->ngroups * parts * s->dstate *
                                  sizeof(float))
                       : 0;
    // per-chunk anchors of the log-decay suffix sums, P*S/256 partials per chunk
    z.anc = round_up(chunk_states_elems(s) / 256 * sizeof(float));
    z.total = s->seqlen == 0 ? 0
                             : 2 * z.dec + 2 * z.st + z.fin + 3 * z.tok + 2 * z.bh + 2 * z.part +
                                   z.anc;
    return z;
}

ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }



#define SSD_REQUIRE(cond, code) \
    do {                        \
        if (!(cond)) return code; \
    } while (0)

}  // namespace

// ssd_forward_noalloc's scratch (see ssd.h): one array per device, each device's address
// resolved once with that device current and kept in g_scratch. On the host `scratch`
// names only a stand-in for the symbol, never a device address, so host code passes the
// resolved pointers to the kernels.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

ssd_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSD_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SSD_OK;
}
}  // namespace

extern "C" {

const char* ssd_status_string(int status) {
    switch (status) {
        case SSD_OK: return "ok";
        case SSD_ERR_NULL: return "a required pointer is NULL";
        case SSD_ERR_SHAPE: return "invalid sizes (a size < 1, seqlen < 0 or nheads % ngroups != 0)";
        case SSD_ERR_DTYPE: return "unknown dtype code";
        case SSD_ERR_UNSUPPORTED: return "chunk, headdim or dstate outside the supported sets";
        case SSD_ERR_WORKSPACE: return "workspace missing or too small";
        case SSD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case SSD_ERR_HIP: return "HIP runtime error";
        case SSD_ERR_TOO_LARGE:
            return "the problem needs more scratch than ssd_forward_noalloc holds "
                   "(SSD_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

ssd_status ssd_validate_shape(const ssd_shape* shape) { return check_shape(shape); }

ssd_status ssd_forward_workspace_bytes(const ssd_shape* shape, size_t* bytes) {
    SSD_REQUIRE(bytes, SSD_ERR_NULL);
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    *bytes = forward_ws(shape);
    return SSD_OK;
}

ssd_status ssd_state_pass_workspace_bytes(const ssd_shape* shape, size_t* bytes) {
    SSD_REQUIRE(bytes, SSD_ERR_NULL);
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    *bytes = state_pass_ws(shape);
    return SSD_OK;
}

ssd_status ssd_state_pass_segmented_workspace_bytes(const ssd_shape* shape, size_t* bytes) {
    SSD_REQUIRE(bytes, SSD_ERR_NULL);
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    ssd::SegPlan pl;
    SSD_REQUIRE(shape->seqlen == 0 || seg_plan_of(shape, &pl), SSD_ERR_UNSUPPORTED);
    *bytes = shape->seqlen == 0 ? 0 : state_seg_ws(shape);
    return SSD_OK;
}

ssd_status ssd_segment_plan(const ssd_shape* shape, int32_t* heads_per_workgroup,
                            int32_t* chunks_per_segment, int32_t* segments) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    ssd::SegPlan pl;
    SSD_REQUIRE(seg_plan_of(shape, &pl), SSD_ERR_UNSUPPORTED);
    if (heads_per_workgroup) *heads_per_workgroup = pl.heads;
    if (chunks_per_segment) *chunks_per_segment = pl.chunks;
    if (segments) *segments = pl.nseg;
    return SSD_OK;
}

ssd_status ssd_chunk_out_plan(const ssd_shape* shape, int32_t* heads_per_workgroup,
                             int32_t* shared_tiles, double* mfma_flops) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    SSD_REQUIRE(shape->seqlen > 0, SSD_ERR_UNSUPPORTED);
    ssd::SegPlan pl;
    ssd::OutPlan op;
    const bool segc = seg_plan_of(shape, &pl);  // the instance ssd_forward launches
    SSD_REQUIRE(ssd::chunk_out_plan(shape->in_dtype, shape->states_dtype, segc, dims_of(shape), &op),
                SSD_ERR_UNSUPPORTED);
    if (heads_per_workgroup) *heads_per_workgroup = op.heads_per_wg;
    if (shared_tiles) *shared_tiles = op.shared ? 1 : 0;
    if (mfma_flops) *mfma_flops = op.mfma_flops;
    return SSD_OK;
}

ssd_status ssd_chunk_cumsum(const ssd_shape* shape, const void* dt, const float* A, float* G,
                            float* dt_t, void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    const bool empty = shape->seqlen == 0;  // nothing to compute
    SSD_REQUIRE(A && (empty || (dt && G)), SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(dt) && aligned16(A) && aligned16(G) && aligned16(dt_t), SSD_ERR_ALIGN);
    if (empty) return SSD_OK;
    return hip_status(ssd::launch_cumsum(shape->in_dtype, dt, A, G, dt_t, dims_of(shape),
                                         (hipStream_t)stream));
}

ssd_status ssd_state_pass(const ssd_shape* shape, const void* x, const float* A, const void* B,
                          const float* G, const float* dt_t, const float* h0, void* states,
                          float* final_state, void* workspace, size_t workspace_bytes,
                          void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    const bool empty = shape->seqlen == 0;  // only the final state (= h0) is written
    SSD_REQUIRE(A && (empty || (x && B && G && dt_t && states)), SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(A) && aligned16(B) && aligned16(G) && aligned16(dt_t) &&
                    aligned16(h0) && aligned16(states) && aligned16(final_state),
                SSD_ERR_ALIGN);
    const size_t need = state_pass_ws(shape);
    SSD_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), SSD_ERR_WORKSPACE);
    SSD_REQUIRE(aligned16(workspace), SSD_ERR_ALIGN);
    const Dims d = dims_of(shape);
    hipStream_t s = (hipStream_t)stream;
    if (empty) return final_state ? hip_status(ssd::launch_state_init(h0, final_state, d, s)) : SSD_OK;
    ssd::SegPlan pl;
    if (seg_plan_of(shape, &pl)) {
        // segmented walk, carry, then the recorded states completed to the true ones
        const ssd::SegBuffers sb = ssd::state_seg_buffers(workspace, d, pl);
        hipError_t e = ssd::launch_state_seg(x, B, A, G, dt_t, h0, states, final_state, pl, sb,
                                             d, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
        return hip_status(ssd::launch_seg_correct(states, pl, sb, d, s));
    }
    float* dS = (float*)workspace;
    hipError_t e = ssd::launch_chunk_state(shape->in_dtype, x, B, A, dt_t, dS, d, s);
    if (e != hipSuccess) return SSD_ERR_HIP;
    return hip_status(ssd::launch_state_carry(shape->states_dtype, dS, G, h0, states,
                                              final_state, d, s));
}

ssd_status ssd_state_pass_segmented(const ssd_shape* shape, const void* x, const float* A,
                                    const void* B, const float* G, const float* dt_t,
                                    const float* h0, void* seg_relative_states,
                                    float* final_state, void* workspace, size_t workspace_bytes,
                                    void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    const bool empty = shape->seqlen == 0;  // only the final state (= h0) is written
    ssd::SegPlan pl;
    SSD_REQUIRE(empty || seg_plan_of(shape, &pl), SSD_ERR_UNSUPPORTED);
    SSD_REQUIRE(A && (empty || (x && B && G && dt_t && seg_relative_states)), SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(A) && aligned16(B) && aligned16(G) && aligned16(dt_t) &&
                    aligned16(h0) && aligned16(seg_relative_states) && aligned16(final_state),
                SSD_ERR_ALIGN);
    const size_t need = empty ? 0 : state_seg_ws(shape);
    SSD_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), SSD_ERR_WORKSPACE);
    SSD_REQUIRE(aligned16(workspace), SSD_ERR_ALIGN);
    const Dims d = dims_of(shape);
    hipStream_t s = (hipStream_t)stream;
    if (empty) return final_state ? hip_status(ssd::launch_state_init(h0, final_state, d, s)) : SSD_OK;
    const ssd::SegBuffers sb = ssd::state_seg_buffers(workspace, d, pl);
    return hip_status(ssd::launch_state_seg(x, B, A, G, dt_t, h0, seg_relative_states,
                                            final_state, pl, sb, d, s));
}

ssd_status ssd_chunk_out_segmented(const ssd_shape* shape, const void* x, const void* B,
                                   const void* C, const float* G, const float* dt_t,
                                   const float* D, const void* seg_relative_states, void* y,
                                   const void* workspace, size_t workspace_bytes, void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    if (shape->seqlen == 0) return SSD_OK;  // empty sequence: no output rows
    ssd::SegPlan pl;
    SSD_REQUIRE(seg_plan_of(shape, &pl), SSD_ERR_UNSUPPORTED);
    SSD_REQUIRE(x && B && C && G && dt_t && seg_relative_states && y, SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(B) && aligned16(C) && aligned16(G) &&
                    aligned16(dt_t) && aligned16(D) && aligned16(seg_relative_states) &&
                    aligned16(y),
                SSD_ERR_ALIGN);
    SSD_REQUIRE(workspace && workspace_bytes >= state_seg_ws(shape), SSD_ERR_WORKSPACE);
    SSD_REQUIRE(aligned16(workspace), SSD_ERR_ALIGN);
    const Dims d = dims_of(shape);
    const ssd::SegBuffers sb = ssd::state_seg_buffers(const_cast<void*>(workspace), d, pl);
    return hip_status(ssd::launch_chunk_out_seg(shape->out_dtype, x, B, C, G, dt_t,
                                                seg_relative_states, sb.seg_in, sb.dec_in,
                                                pl.chunks, D, y, d, (hipStream_t)stream));
}

ssd_status ssd_state_scan(const ssd_shape* shape, const void* x, const float* A, const void* B,
                          const float* dt_t, const float* h0, void* states, float* final_state,
                          void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    const Dims d = dims_of(shape);
    SSD_REQUIRE(ssd::state_scan_supported(shape->in_dtype, d), SSD_ERR_UNSUPPORTED);
    SSD_REQUIRE(x && A && B && dt_t && states, SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(A) && aligned16(B) && aligned16(dt_t) && aligned16(h0) &&
                    aligned16(states) && aligned16(final_state),
                SSD_ERR_ALIGN);
    return hip_status(ssd::launch_state_scan(shape->states_dtype, x, B, A, dt_t, h0, states,
                                             final_state, d, (hipStream_t)stream));
}

ssd_status ssd_chunk_out(const ssd_shape* shape, const void* x, const void* B, const void* C,
                         const float* G, const float* dt_t, const void* states, const float* D,
                         void* y, void* stream) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    if (shape->seqlen == 0) return SSD_OK;  // empty sequence: no output rows
    SSD_REQUIRE(x && B && C && G && dt_t && states && y, SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(B) && aligned16(C) && aligned16(G) &&
                    aligned16(dt_t) && aligned16(states) && aligned16(D) && aligned16(y),
                SSD_ERR_ALIGN);
    return hip_status(ssd::launch_chunk_out(shape->in_dtype, shape->states_dtype,
                                            shape->out_dtype, x, B, C, G,
                                            dt_t, states, D, y, dims_of(shape),
                                            (hipStream_t)stream));
}

// Argument checks of ssd_forward and ssd_forward_noalloc (everything but the workspace).
static ssd_status check_forward_args(const ssd_shape* shape, const void* x, const void* dt,
                                     const float* A, const void* B, const void* C,
                                     const float* D, const float* h0, const void* y,
                                     const float* final_state) {
    ssd_status st = check_shape(shape);
    if (st != SSD_OK) return st;
    const bool empty = shape->seqlen == 0;  // only the final state (= h0) is written
    SSD_REQUIRE(A && (empty || (x && dt && B && C && y)), SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(dt) && aligned16(A) && aligned16(B) && aligned16(C) &&
                    aligned16(D) && aligned16(h0) && aligned16(y) && aligned16(final_state),
                SSD_ERR_ALIGN);
    return SSD_OK;
}

// The forward pass on checked arguments and a workspace of at least forward_ws bytes.
static ssd_status forward_impl(const ssd_shape* shape, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* h0, void* y, float* final_state, void* workspace,
                               void* stream) {
    const bool empty = shape->seqlen == 0;
    const Dims d = dims_of(shape);
    hipStream_t s = (hipStream_t)stream;
    if (empty) return final_state ? hip_status(ssd::launch_state_init(h0, final_state, d, s)) : SSD_OK;
    char* w = (char*)workspace;
    float* G = (float*)w;
    float* dt_t = (float*)(w + decay_bytes(shape));
    void* mid = (void*)(w + 2 * decay_bytes(shape));
    void* states = (void*)(w + 2 * decay_bytes(shape) + forward_mid_ws(shape));
    hipError_t e = ssd::launch_cumsum(shape->in_dtype, dt, A, G, dt_t, d, s);
    if (e != hipSuccess) return SSD_ERR_HIP;
    ssd::SegPlan pl;
    if (seg_plan_of(shape, &pl)) {
        // segment-relative states; the output kernel completes them while staging
        const ssd::SegBuffers sb = ssd::state_seg_buffers(mid, d, pl);
        e = ssd::launch_state_seg(x, B, A, G, dt_t, h0, states, final_state, pl, sb, d, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
        return hip_status(ssd::launch_chunk_out_seg(shape->out_dtype, x, B, C, G, dt_t, states,
                                                    sb.seg_in, sb.dec_in, pl.chunks, D, y, d, s));
    }
    float* dS = (float*)mid;
    if (ssd::state_scan_supported(shape->in_dtype, d) && ssd::state_scan_preferred(shape->in_dtype, d)) {
        e = ssd::launch_state_scan(shape->states_dtype, x, B, A, dt_t, h0, states, final_state, d, s);
    } else {
        e = ssd::launch_chunk_state(shape->in_dtype, x, B, A, dt_t, dS, d, s);
        if (e != hipSuccess) return SSD_ERR_HIP;
        e = ssd::launch_state_carry(shape->states_dtype, dS, G, h0, states, final_state, d, s);
    }
    if (e != hipSuccess) return SSD_ERR_HIP;
    return hip_status(ssd::launch_chunk_out(shape->in_dtype, shape->states_dtype,
                                            shape->out_dtype, x, B, C, G,
                                            dt_t, states, D, y, d, s));
}

ssd_status ssd_forward(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                       const void* B, const void* C, const float* D, const float* h0, void* y,
                       float* final_state, void* workspace, size_t workspace_bytes,
                       void* stream) {
    ssd_status st = check_forward_args(shape, x, dt, A, B, C, D, h0, y, final_state);
    if (st != SSD_OK) return st;
    const size_t need = forward_ws(shape);
    SSD_REQUIRE(workspace_bytes >= need && (need == 0 || workspace), SSD_ERR_WORKSPACE);
    SSD_REQUIRE(aligned16(workspace), SSD_ERR_ALIGN);
    return forward_impl(shape, x, dt, A, B, C, D, h0, y, final_state, workspace, stream);
}

ssd_status ssd_forward_noalloc(const ssd_shape* shape, const void* x, const void* dt,
                               const float* A, const void* B, const void* C, const float* D,
                               const float* h0, void* y, float* final_state, void* stream) {
    ssd_status st = check_forward_args(shape, x, dt, A, B, C, D, h0, y, final_state);
    if (st != SSD_OK) return st;
    SSD_REQUIRE(forward_ws(shape) <= SSD_NOALLOC_SCRATCH_BYTES, SSD_ERR_TOO_LARGE);
    void* ws = nullptr;
    st = scratch_on_current_device(&ws);
    if (st != SSD_OK) return st;
    return forward_impl(shape, x, dt, A, B, C, D, h0, y, final_state, ws, stream);
}

ssd_status ssd_decode_step(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                           const void* B, const void* C, const float* D, float* state, float* y,
                           void* stream) {
    ssd_status st = check_decode_shape(shape);
    if (st != SSD_OK) return st;
    SSD_REQUIRE(x && dt && A && B && C && state && y, SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(dt) && aligned16(A) && aligned16(B) && aligned16(C) &&
                    aligned16(D) && aligned16(state) && aligned16(y),
                SSD_ERR_ALIGN);
    return hip_status(ssd::launch_decode(shape->in_dtype, x, dt, A, B, C, D, state, y,
                                         dims_of(shape), (hipStream_t)stream));
}

// The backward pass computes in fp32 throughout: states_dtype and out_dtype are not used.
static ssd_status check_backward_shape(const ssd_shape* shape) {
    if (!shape) return SSD_ERR_NULL;
    ssd_shape s = *shape;
    s.states_dtype = SSD_F32;
    s.out_dtype = SSD_F32;
    return check_shape(&s);
}

ssd_status ssd_backward_workspace_bytes(const ssd_shape* shape, size_t* bytes) {
    SSD_REQUIRE(bytes, SSD_ERR_NULL);
    ssd_status st = check_backward_shape(shape);
    if (st != SSD_OK) return st;
    *bytes = bwd_sizes(shape).total;
    return SSD_OK;
}

ssd_status ssd_backward(const ssd_shape* shape, const void* x, const void* dt, const float* A,
                        const void* B, const void* C, const float* D, const float* h0,
                        const float* dy, const float* dfinal, float* dx, float* ddt, float* dA,
                        float* dB, float* dC, float* dD, float* dh0, void* workspace,
                        size_t workspace_bytes, void* stream) {
    ssd_status st = check_backward_shape(shape);
    if (st != SSD_OK) return st;
    const bool empty = shape->seqlen == 0;
    SSD_REQUIRE(A && dA && (empty || (x && dt && B && C && dy && dx && ddt && dB && dC)),
                SSD_ERR_NULL);
    SSD_REQUIRE(aligned16(x) && aligned16(dt) && aligned16(A) && aligned16(B) && aligned16(C) &&
                    aligned16(D) && aligned16(h0) && aligned16(dy) && aligned16(dfinal) &&
                    aligned16(dx) && aligned16(ddt) && aligned16(dA) && aligned16(dB) &&
                    aligned16(dC) && aligned16(dD) && aligned16(dh0),
                SSD_ERR_ALIGN);
    const BwdSizes z = bwd_sizes(shape);
    SSD_REQUIRE(workspace_bytes >= z.total && (z.total == 0 || workspace), SSD_ERR_WORKSPACE);
    SSD_REQUIRE(aligned16(workspace), SSD_ERR_ALIGN);
    ssd::BwdLaunch k;
    k.x = x; k.dt = dt; k.B = B; k.C = C; k.A = A; k.D = D; k.h0 = h0; k.dy = dy;
    k.dfinal = dfinal; k.dx = dx; k.ddt = ddt; k.dA = dA; k.dB = dB; k.dC = dC; k.dD = dD;
    k.dh0 = dh0;
    char* w = (char*)workspace;
    auto take = [&](size_t n) {
        float* p = n ? (float*)w : nullptr;
        w += n;
        return p;
    };
    k.ws.G = take(z.dec);
    k.ws.dt_t = take(z.dec);
    k.ws.Hc = take(z.st);
    k.ws.R = take(z.st);
    k.ws.fin = take(z.fin);
    k.ws.v = take(z.tok);
    k.ws.q = take(z.tok);
    k.ws.dyx = take(z.tok);
    k.ws.dA_bh = take(z.bh);
    k.ws.dD_bh = take(z.bh);
    k.ws.dBh = take(z.part);
    k.ws.dCh = take(z.part);
    k.ws.anc = take(z.anc);
    const ssd_shape bs = bwd_shape(shape);
    return hip_status(ssd::launch_backward(shape->in_dtype, k, dims_of(&bs), (hipStream_t)stream));
}

}  // extern "C"
