// Stage 2b: carry the state across chunks.
//
// Page "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA CUDA
// Tile", section "Kernel 2: fwd_pass_state": the state entering each chunk is stored
// before the chunk is applied, the jump S <- 2^{G_last} S + dS_c advances it, and the
// state after the last chunk is the final state. With dS_c precomputed by the matrix
// kernel, what remains is one multiply-add per state element per chunk, sequential in
// the chunk index and independent across the batch*heads*P*S elements: a pure
// streaming kernel bound by HBM bandwidth.
//
// gfx950 mapping: one wave per 256 consecutive state elements of one (batch, head);
// each lane owns 4 elements (16-byte loads), prefetches 8 chunks of dS at a time to
// keep many loads in flight, and writes the chunk-initial states (bf16 or fp32), with
// non-temporal loads and stores (5.8 TB/s at the 2.7B and long shapes, 5.2 without).
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {

// The increments are read once and the states written once here, so both go through
// non-temporal (streaming) accesses that do not displace cached lines.
__device__ __forceinline__ void store4(float* p, f32x4 v) { __builtin_nontemporal_store(v, (f32x4*)p); }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
    bf16x4 o;
    o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
    __builtin_nontemporal_store(o, (bf16x4*)p);
}

template <typename TS>
__global__ __launch_bounds__(64) void state_carry_kernel(const float* __restrict__ dS,
                                                         const float* __restrict__ G,
                                                         const float* __restrict__ h0,
                                                         TS* __restrict__ states,
                                                         float* __restrict__ fin, int L, int T,
                                                         int nC, int PS) {
    const int per_bh = PS / 256;
    const size_t bh = blockIdx.x / per_bh;
    const int e = (blockIdx.x % per_bh) * 256 + threadIdx.x * 4;
    f32x4 hv = f32x4{0.f, 0.f, 0.f, 0.f};
    if (h0) hv = *(const f32x4*)(h0 + bh * PS + e);
    // G at each chunk's last token (the last real one in a partial last chunk, where the
    // zero-padded tokens would leave G unchanged)
    const float* gr = G + bh * L;
    auto g_last = [&](int c) { return gr[min((c + 1) * T, L) - 1]; };
    const float* src = dS + bh * nC * (size_t)PS + e;
    TS* dst = states + bh * nC * (size_t)PS + e;
    constexpr int U = 8;
    for (int c0 = 0; c0 < nC; c0 += U) {
        f32x4 d[U];
        float dec[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < nC) {
                d[u] = __builtin_nontemporal_load((const f32x4*)(src + (size_t)(c0 + u) * PS));
                dec[u] = exp2_fast(g_last(c0 + u));
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < nC) {
                store4(dst + (size_t)(c0 + u) * PS, hv);
                hv = dec[u] * hv + d[u];
            }
        }
    }
    if (fin) *(f32x4*)(fin + bh * PS + e) = hv;
}

// The state after an empty sequence: final = h0 (zeros without h0), 4 floats per thread.
__global__ __launch_bounds__(256) void state_init_kernel(const float* __restrict__ h0,
                                                         float* __restrict__ fin, size_t n4) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) *(f32x4*)(fin + 4 * i) = h0 ? *(const f32x4*)(h0 + 4 * i) : f32x4{0.f, 0.f, 0.f, 0.f};
}

hipError_t launch_state_init(const float* h0, float* fin, const Dims& d, hipStream_t stream) {
    const size_t n4 = (size_t)d.batch * d.nheads * d.headdim * d.dstate / 4;
    state_init_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, stream>>>(h0, fin, n4);
    return hipGetLastError();
}

hipError_t launch_state_carry(int states_dtype, const float* dS, const float* G,
                              const float* h0, void* states, float* fin, const Dims& d,
                              hipStream_t stream) {
    const int PS = d.headdim * d.dstate;  // multiple of 256 for every supported size
    const int nblocks = d.batch * d.nheads * (PS / 256);
    if (states_dtype == kBF16)
        state_carry_kernel<bf16><<<nblocks, 64, 0, stream>>>(
            dS, G, h0, (bf16*)states, fin, d.seqlen, d.chunk, d.nchunks(), PS);
    else
        state_carry_kernel<float><<<nblocks, 64, 0, stream>>>(
            dS, G, h0, (float*)states, fin, d.seqlen, d.chunk, d.nchunks(), PS);
    return hipGetLastError();
}

}  // namespace ssd
